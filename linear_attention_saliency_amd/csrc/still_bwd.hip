// Backward pass of the STILL layer with the routing held fixed: the gradients of
// sum(out * dout) with respect to q, k, v and the NP-Map weights.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h. [P1] section
// "Chunk-Wise并行+延迟选择" and [P4] section Approach use the same chunked layer for
// training, which is what these kernels differentiate.)
//
// With den_i the shared normaliser of query i (softmax terms e^{a_ij} of its SA keys plus
// the linear-attention weights phi(q_i).phi(k_j) of its LA keys), L_i = log den_i, and
// Delta_i = dout_i . out_i:
//   SA pair:  P_ij = e^{a_ij - L_i};  dS_ij = P_ij (dout_i.v_j - Delta_i)
//             dq_i += dS_ij k_j / sqrt(D),  dk_j += dS_ij q_i / sqrt(D),  dv_j += P_ij dout_i
//   LA pair:  g_ij = (dout_i.v_j - Delta_i) e^{-L_i}
//             dphi(q_i) += g_ij phi(k_j),  dphi(k_j) += g_ij phi(q_i),
//             dv_j += e^{-L_i} (phi(q_i).phi(k_j)) dout_i
// LA keys of chunks <= c-2 enter through states: S_c = sum phi(k) v^T and z_c = sum phi(k)
// over their unselected keys for the queries of chunk c, and, for the keys of chunk c,
// R_c = sum e^{-L} phi(q) dout^T and r_c = sum e^{-L} Delta phi(q) over the queries of
// chunks >= c+2. NP-Map phi(x) = |x| m / |m|, m = elu(W x) + 1, is differentiated row by
// row: with m^ = m / |m| and dr = dphi . m^, dm = |x| (dphi - m^ dr) / |m|,
// dz = dm * elu'(Wx), dx = W^T dz + dr x / |x|, dW += dz x^T.
//
// Launch order (one stream):
//   bwd_kprep_kernel     per (chunk, KV head, batch): phi(k), K^T, U_c / u_c, compact rows
//   bwd_scan_fwd_kernel  U_c -> S_c (sum over chunks <= c-2), in place
//   bwd_dq_kernel        per (chunk, one or two query heads, batch): one pass over the keys
//                        gives dq and L_i together (the softmax part against a running reference,
//                        divided by the normaliser at the end), the per-chunk sums behind
//                        R, the q side of dW
//   bwd_rev_seg_kernel / bwd_rev_scan_kernel: R_c = sum over chunks >= c+2 and over the
//                        query group (a segmented scan)
//   bwd_dkv_far_kernel   per (compact rows, query slice, KV head): the selected keys
//                        against the queries of chunks >= their chunk + 2
//   bwd_dkv_local_kernel per (chunk, KV head, batch): keys against the queries of their
//                        own chunk and the next; R_c; the NP-Map backward; dk, dv
//   bwd_dw_part_kernel / bwd_dw_sum_kernel: dW summed over chunks, heads and batch
//
// Instantiated for (head_dim, feat_dim) = (64, 64) in fp32 and bf16 and (128, 128) in bf16,
// chunk 64. Matrix products run on MFMA in the layer's dtype with fp32 accumulation; every
// sum that crosses workgroups goes through fp32 buffers in a fixed order, so the result is
// deterministic.
#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"
#include "still_tile.hpp"

namespace still {

namespace {

// NP-Map forward of one row per lane column, for the row held as B fragments xf (SK):
// m[blk][i] = elu(z) + 1 with z = (W x)[16 blk + 4 grp + i], |x| and 1/|m|. z itself is not
// kept: elu'(z) = min(m, 1) (z > 0 gives m = z + 1 > 1 and slope 1, z <= 0 gives m = e^z <= 1,
// its own slope).
template <int F>
struct NpRow {
  f32x4 m[F / 16];
  float r, inv_nm;
};

// W is [F][D] row-major in memory, or with TILE a Swz<T, D> LDS tile of F rows.
template <typename T, int D, int F, bool TILE = false>
__device__ __forceinline__ void np_forward(NpRow<F>& n, const T* W, const typename Tr<T>::frag (&xf)[D / 32]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int fb = 0; fb < F / 16; ++fb) {
    n.m[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const typename Tr<T>::frag wf = TILE ? Swz<T, D>::load8(W, fb * 16 + r16, ks * 32 + grp * 8)
                                           : Tr<T>::load8(W + (fb * 16 + r16) * D + ks * 32 + grp * 8);
      Tr<T>::mma(n.m[fb], wf, xf[ks]);
    }
  }
  float nm2 = 0.f, xn2 = 0.f;
#pragma unroll
  for (int fb = 0; fb < F / 16; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float zv = n.m[fb][i];
      const float mv = zv > 0.f ? zv + 1.f : __builtin_amdgcn_exp2f(zv * kLog2e);
      n.m[fb][i] = mv;
      nm2 += mv * mv;
    }
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = Tr<T>::to_f(xf[ks][e]);
      xn2 += x * x;
    }
  nm2 = xor_sum_groups(nm2);
  xn2 = xor_sum_groups(xn2);
  n.r = sqrtf(xn2);
  n.inv_nm = 1.0f / sqrtf(nm2);
}

// NP-Map backward for the same row: dphi[blk][i] (feature 16 blk + 4 grp + i) -> dz (in
// place) and dr = dphi . m^. dx = W^T dz + dr x / |x| is formed by the caller.
template <int F>
__device__ __forceinline__ float np_backward(const NpRow<F>& n, f32x4 (&dphi)[F / 16]) {
  float dr = 0.f;
#pragma unroll
  for (int fb = 0; fb < F / 16; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dr += dphi[fb][i] * n.m[fb][i];
  dr = xor_sum_groups(dr) * n.inv_nm;
#pragma unroll
  for (int fb = 0; fb < F / 16; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mh = n.m[fb][i] * n.inv_nm;
      const float dm = n.r * (dphi[fb][i] - mh * dr) * n.inv_nm;
      dphi[fb][i] = dm * fminf(n.m[fb][i], 1.f);
    }
  return dr;
}

// tile[dd][pk_pos(f)] = src[f][dd]: the transpose of a row-major [F][D] matrix (in the
// layer's dtype or fp32), features pk-permuted, into a Swz<T, F> LDS tile of D rows. A
// thread takes the 8 features of one 8-position granule of the permuted order by 8 dims:
// eight 8-element reads of the source, a transpose in registers, eight 8-element LDS
// stores. Neighbouring threads take neighbouring granules of the same dims, so every store
// instruction fills whole rows without bank conflicts.
template <typename T, int D, int F, typename S>
__device__ __forceinline__ void load_pk_transposed(T* lds, const S* src, T* rows = nullptr) {
  constexpr int NG = F / 8;
  for (int it = threadIdx.x; it < NG * (D / 8); it += blockDim.x) {
    const int G = it % NG, dd0 = (it / NG) * 8;
    // position 8 G + 4 hi + r of the permuted order holds feature fb + 16 hi + r
    const int fb = (G / 4) * 32 + (G % 4) * 4;
    typename Tr<T>::frag y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const S* row = src + (fb + (e / 4) * 16 + (e % 4)) * D + dd0;
      typename Tr<T>::frag x;
      if constexpr (sizeof(S) == 4) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(row), hi = *reinterpret_cast<const f32x4*>(row + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = Tr<T>::from_f(lo[j]);
          x[j + 4] = Tr<T>::from_f(hi[j]);
        }
      } else {
        x = Tr<T>::load8(row);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j][e] = x[j];
      // the same 8 elements untransposed, into a Swz<T, D> tile of F rows
      if (rows != nullptr) Swz<T, D>::store8(rows, fb + (e / 4) * 16 + (e % 4), dd0, x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) Swz<T, F>::store8(lds, dd0 + j, 8 * G, y[j]);
  }
}

// W^T with the features pk-permuted, [dim][pk_pos(f)], into a Swz<T, F> LDS tile of D rows
template <typename T, int D, int F>
__device__ __forceinline__ void load_wt(T* lds, const T* W) {
  load_pk_transposed<T, D, F, T>(lds, W);
}

// selection bit mask of complete chunk c from the ascending positions (entries outside
// the chunk are ignored); wave-uniform
__device__ __forceinline__ uint64_t chunk_sel(const int32_t* sel_idx, long long bh, int c, const Dims& d) {
  if (d.topk == 0 || c < 0 || c >= d.nCc) return 0ull;
  const int32_t* p = sel_idx + (bh * d.nCc + c) * d.topk;
  uint64_t m = 0;
  for (int r = 0; r < d.topk; ++r) {
    const int pos = p[r] - 64 * c;
    if (pos >= 0 && pos < 64) m |= 1ull << pos;
  }
  return m;
}

// 1 / sqrt(head_dim)
template <int D>
constexpr float inv_sqrt_d() { return D == 64 ? 0.125f : 0.08838834764831845f; }

}  // namespace

// ---------------------------------------------------------------------------------------
template <typename T, int D, int F>
__global__ __launch_bounds__(256) void bwd_kprep_kernel(BwdArgs a) {
  using TT = Tr<T>;
  constexpr int FPW = F / 64, R = F * D + F;
  __shared__ __attribute__((aligned(16))) T t_k[64 * D];
  __shared__ __attribute__((aligned(16))) T t_v[64 * D];
  __shared__ __attribute__((aligned(16))) T t_vt[D * 64];
  __shared__ __attribute__((aligned(16))) T t_ph[64 * F];  // phi(k) rows, features pk-permuted
  __shared__ float m2part[4 * 64];
  __shared__ float xn2[64];
  __shared__ int selpos[64];  // position of the chunk's selected key of each rank
  const Dims& d = a.d;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int nvalid = min(64, d.T - 64 * c);
  const long long rs = static_cast<long long>(d.Hkv) * D;
  const long long row0 = (static_cast<long long>(b) * d.T + 64LL * c) * d.Hkv + h;
  tile_load<T, D>(t_k, static_cast<const T*>(a.k) + row0 * D, rs, nvalid);
  tile_load<T, D>(t_v, static_cast<const T*>(a.v) + row0 * D, rs, nvalid);
  const uint64_t selm = chunk_sel(a.sel_idx, bh, c, d);
  if (tid < 64 && ((selm >> tid) & 1ull)) selpos[__popcll(selm & ((1ull << tid) - 1ull))] = tid;
  typename TT::frag wf[FPW][D / 32];
  np_map_load_w<T, D, F>(static_cast<const T*>(a.w) + static_cast<long long>(h) * F * D, wf);
  __syncthreads();
  // V^T (keys pk-permuted) into LDS, K^T into memory, 8 positions at a time
  T* ktg = static_cast<T*>(a.kt) + (bh * d.nC + c) * (D * 64);
  for (int e8 = tid; e8 < D * 8; e8 += 256) {
    const int dd = e8 >> 3, p0 = (e8 & 7) * 8;
    typename TT::frag kv, vv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = pk_index(p0 + j);
      kv[j] = t_k[Swz<T, D>::off(row, dd)];
      vv[j] = t_v[Swz<T, D>::off(row, dd)];
    }
    Swz<T, 64>::store8(t_vt, dd, p0, vv);
    TT::store8(ktg + dd * 64 + p0, kv);
  }
  f32x4 phi[4][FPW];
  np_map_rows64<T, D, F>(t_k, 0, wf, m2part, xn2, phi);  // synchronises the workgroup
  T* phk = static_cast<T*>(a.phik) + (bh * d.nC * 64 + 64LL * c) * F;
  T* phkt = static_cast<T*>(a.phikt) + (bh * d.nC + c) * (F * 64);
  float* ust = a.ustate + (bh * d.nC + c) * R;
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi) {
    const int f = (wave * FPW + fi) * 16 + r16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) t_ph[Swz<T, F>::off(kb * 16 + 4 * grp + i, pk_pos(f))] = TT::from_f(phi[kb][fi][i]);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      TT::store8(phkt + f * 64 + 32 * s + 8 * grp, pk_frag<T>(phi[2 * s][fi], phi[2 * s + 1][fi]));
    // U_c = sum over unselected keys of phi(k) v^T, u_c = sum phi(k)
    f32x4 ph[4];
    float zs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kb * 16 + 4 * grp + i;
        const bool la = row < nvalid && !((selm >> row) & 1ull);
        ph[kb][i] = la ? phi[kb][fi][i] : 0.f;
        zs += ph[kb][i];
      }
    zs = xor_sum_groups(zs);
    f32x4 u[D / 16] = {};
    rows_x_acc<T, D / 16>(u, t_vt, ph);  // u[db][i] = U[f][16 db + 4 grp + i]
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(ust + f * D + db * 16 + 4 * grp) = u[db];
    if (grp == 0) ust[F * D + f] = zs;
  }
  __syncthreads();  // the phi(k) rows to memory in 16-byte pieces
  for (int e8 = tid; e8 < 64 * F / 8; e8 += 256) {
    const int row = e8 / (F / 8), col = (e8 % (F / 8)) * 8;
    TT::store8(phk + row * F + col, Swz<T, F>::load8(t_ph, row, col));
  }
  // the selected rows, in position order (compact row c * top_k + rank, as the local-key
  // kernel looks them up), into the compact buffers
  if (c < d.nCc && d.topk > 0) {
    const int nsel = __popcll(selm);
    T* ks = static_cast<T*>(a.ksel) + bh * a.ntiles * 64 * D;
    T* vs = static_cast<T*>(a.vsel) + bh * a.ntiles * 64 * D;
    T* kst = static_cast<T*>(a.kselt) + bh * a.ntiles * (D * 64);
    // rows of K and V: 16-byte granules
    for (int e8 = tid; e8 < d.topk * (D / 8); e8 += 256) {
      const int r = e8 / (D / 8), col = (e8 % (D / 8)) * 8;
      const bool ok = r < nsel;
      const int pos = ok ? selpos[r] : 0;
      const long long n = static_cast<long long>(c) * d.topk + r;
      TT::store8(ks + n * D + col, ok ? Swz<T, D>::load8(t_k, pos, col) : TT::zero());
      TT::store8(vs + n * D + col, ok ? Swz<T, D>::load8(t_v, pos, col) : TT::zero());
    }
    // K^T tiles: the 4 rows of a 4-aligned compact-row group sit at 4 consecutive columns
    // (pk_pos keeps n & 3), so a lane writes one piece of up to 4 elements of one K^T row;
    // rows of a group that belong to a neighbouring chunk are left alone
    const long long n0 = static_cast<long long>(c) * d.topk, g_lo = n0 / 4;
    const int ng = static_cast<int>((n0 + d.topk - 1) / 4 - g_lo) + 1;
    for (int e = tid; e < ng * D; e += 256) {
      const int gi = e % ng, dd = e / ng;
      const long long n4 = 4 * (g_lo + gi);
      typename TT::quad x;
      bool all = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long long r = n4 + j - n0;
        all = all && r >= 0 && r < d.topk;
        x[j] = r >= 0 && r < nsel ? t_k[Swz<T, D>::off(selpos[r], dd)] : TT::from_f(0.f);
      }
      T* dst = kst + ((n4 >> 6) * D + dd) * 64 + pk_pos(static_cast<int>(n4 & 63));
      if (all) {
        *reinterpret_cast<typename TT::quad*>(dst) = x;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long long r = n4 + j - n0;
          if (r >= 0 && r < d.topk) dst[j] = x[j];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// U_c -> S_c = sum over chunks <= c-2, in place; one thread per (b, KV head, element of R)
__global__ __launch_bounds__(256) void bwd_scan_fwd_kernel(float* ust, int nC, int R, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long bh = gid / R, e = gid % R;
  float* p = ust + bh * nC * R + e;
  float acc = 0.f, p1 = 0.f, p2 = 0.f;
  constexpr int U = 8;  // loads of U chunks in flight together
  for (int c0 = 0; c0 < nC; c0 += U) {
    float cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = c0 + u < nC ? p[static_cast<long long>(c0 + u) * R] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nC) {
        acc += p2;
        p[static_cast<long long>(c0 + u) * R] = acc;
      }
      p2 = p1;
      p1 = cur[u];
    }
  }
}

// R_c = sum over chunks >= c+2 of the group's per-chunk sums, as a segmented scan over
// chunks: bwd_rev_seg_kernel sums each segment of kRevSeg chunks (and the group's G records:
// one per query head, or per pair of heads when dq runs two heads per wave),
// bwd_rev_scan_kernel starts from the later segments' total and scans its own segment down.
// One thread per (b, KV head, segment, element of R) in both.
constexpr int kRevSeg = 16;

__global__ __launch_bounds__(256) void bwd_rev_seg_kernel(const float* apart, float* segsum, int nC, int G,
                                                          int Hkv, int nseg, int R, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long e = gid % R, seg = (gid / R) % nseg, bh = gid / (static_cast<long long>(R) * nseg);
  const long long b = bh / Hkv, h = bh % Hkv;
  const long long hq0 = b * Hkv * G + h * G;
  const int c0 = static_cast<int>(seg) * kRevSeg, c1 = min(nC, c0 + kRevSeg);
  float acc = 0.f;
  for (int g = 0; g < G; ++g) {
    const float* p = apart + (hq0 + g) * nC * R + e;
    float x[kRevSeg];
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u) x[u] = c0 + u < c1 ? p[static_cast<long long>(c0 + u) * R] : 0.f;
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u) acc += x[u];
  }
  segsum[gid] = acc;
}

__global__ __launch_bounds__(256) void bwd_rev_scan_kernel(const float* apart, const float* segsum, float* rst,
                                                           int nC, int G, int Hkv, int nseg, int R,
                                                           long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long e = gid % R, seg = (gid / R) % nseg, bh = gid / (static_cast<long long>(R) * nseg);
  const long long b = bh / Hkv, h = bh % Hkv;
  const long long hq0 = b * Hkv * G + h * G;
  const int c0 = static_cast<int>(seg) * kRevSeg, c1 = min(nC, c0 + kRevSeg);
  float acc = 0.f;  // sum over the chunks of later segments
  for (long long s2 = nseg - 1; s2 > seg; --s2) acc += segsum[(bh * nseg + s2) * R + e];
  float x[kRevSeg];
#pragma unroll
  for (int u = 0; u < kRevSeg; ++u) x[u] = 0.f;
  for (int g = 0; g < G; ++g) {
    const float* p = apart + (hq0 + g) * nC * R + e;
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u)
      if (c0 + u < c1) x[u] += p[static_cast<long long>(c0 + u) * R];
  }
  float* r = rst + bh * nC * R + e;
#pragma unroll
  for (int u = kRevSeg - 1; u >= 0; --u) {
    const int c = c0 + u;
    if (c < c1) {
      acc += x[u];  // acc = sum over chunks >= c
      if (c >= 2) r[static_cast<long long>(c - 2) * R] = acc;
    }
  }
  if (seg == nseg - 1) {  // no chunk lies two or more after the last two
    r[static_cast<long long>(nC - 1) * R] = 0.f;
    if (nC >= 2) r[static_cast<long long>(nC - 2) * R] = 0.f;
  }
}

// The same R_c in one pass where one thread per (b, KV head, element of R) already fills the
// GPU: each thread runs down all chunks, with U chunks' loads in flight, so the per-chunk sums
// are read once instead of twice.
__global__ __launch_bounds__(256) void bwd_rev_full_kernel(const float* apart, float* rst, int nC, int G, int Hkv,
                                                           int R, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long e = gid % R, bh = gid / R;
  const long long b = bh / Hkv, h = bh % Hkv;
  const long long hq0 = b * Hkv * G + h * G;
  float* r = rst + bh * nC * R + e;
  constexpr int U = 8;
  float acc = 0.f;  // sum over the chunks >= c
  for (int c0 = nC - 1; c0 >= 0; c0 -= U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = 0.f;
    for (int g = 0; g < G; ++g) {
      const float* p = apart + (hq0 + g) * nC * R + e;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 - u >= 0) x[u] += p[static_cast<long long>(c0 - u) * R];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 - u;
      if (c >= 0) {
        acc += x[u];
        if (c >= 2) r[static_cast<long long>(c - 2) * R] = acc;
      }
    }
  }
  r[static_cast<long long>(nC - 1) * R] = 0.f;  // no chunk lies two or more after the last two
  if (nC >= 2) r[static_cast<long long>(nC - 2) * R] = 0.f;
}

// ---------------------------------------------------------------------------------------
// QH query heads of one KV head per four waves, 16 queries per wave, the wave taking the same
// 16 rows of each of its QH heads, so that every K, V and K^T fragment it reads from LDS
// serves QH products. With NWV = 8 (QH = 1, F = 128) a workgroup takes two heads, one per
// group of four waves: both heads share every staged tile, and each SIMD runs two waves,
// which the registers of two heads per wave would not allow at D = 128.
template <typename T, int D, int F, int QH, int NWV>
__global__ __launch_bounds__(NWV * 64, D == 64 ? (QH == 1 ? 3 : 2) : 1) void bwd_dq_kernel(BwdArgs a) {
  static_assert(NWV == 4 || (NWV == 8 && QH == 1 && F % 128 == 0), "wave layout");
  constexpr int HW = NWV / 4;     // heads side by side (groups of four waves)
  constexpr int HPW = QH * HW;    // query heads per workgroup
  constexpr int NT = NWV * 64;    // threads
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, 64>;
  constexpr int ND = D / 16, NF = F / 16, R = F * D + F;
  constexpr int SLOT = (D > F ? D : F) * 64;  // elements per tile slot
  // tile slots: the compact-key loops double-buffer (K, V, K^T) in slots 0-2 and 3-5; S_c
  // takes slots 0-1 (F x D) after them; the near chunks use K, V, K^T, phi(K), phi(K)^T in
  // slots 0-4; W^T takes slots 0-1 (D x F); the closing products use slots 2-5. W (F x D)
  // stays in a region of its own for the NP-Map forward of every head.
  __shared__ __attribute__((aligned(16))) T lds[6 * SLOT];
  __shared__ __attribute__((aligned(16))) T t_w[F * D];
  __shared__ float s_red[NWV][F];
  T* const t_k = lds;
  T* const t_v = lds + SLOT;
  T* const t_kt = lds + 2 * SLOT;
  T* const t_pk = lds + 3 * SLOT;
  T* const t_pkt = lds + 4 * SLOT;

  const Dims& d = a.d;
  // work index: chunk fastest, then the group of QH query heads, then batch (the heads of one
  // KV head share its compact tiles). Divisions by run-time sizes leave the compiler unsure
  // that these are uniform; telling it keeps the buffer descriptors in scalar registers.
  const int nhg = d.Hq / HPW;
  const int w = xcd_work(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int wq = wave & 3, hsub = __builtin_amdgcn_readfirstlane(wave >> 2);  // rows, group of heads
  const int c = __builtin_amdgcn_readfirstlane(w % d.nC);
  const int hgi = __builtin_amdgcn_readfirstlane((w / d.nC) % nhg);
  const int hqb = hgi * HPW;            // the workgroup's first query head
  const int hq0 = hqb + hsub * QH;      // the wave's first query head
  const int b = __builtin_amdgcn_readfirstlane(w / (d.nC * nhg));
  const int h = hqb / d.G;
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const int qrow = wq * 16 + r16;
  const long long i = 64LL * c + qrow;  // this lane column's query
  const bool qvalid = i < d.T;
  constexpr float isd = inv_sqrt_d<D>();
  const float scale2 = kLog2e * isd;
  const T* W = static_cast<const T*>(a.w) + static_cast<long long>(h) * F * D;

  // the query rows, dout rows and Delta = dout . out of each head (head g at qoff0 + g D)
  const long long qoff0 = ((static_cast<long long>(b) * d.T + i) * d.Hq + hq0) * D;
  frag qf[QH][D / 32], dof[QH][D / 32];
  float delta[QH];
#pragma unroll
  for (int g = 0; g < QH; ++g) {
    const long long qo = qoff0 + g * D;
    delta[g] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[g][ks] = qvalid ? TT::load8(static_cast<const T*>(a.q) + qo + ks * 32 + grp * 8) : TT::zero();
      dof[g][ks] = qvalid ? TT::load8(static_cast<const T*>(a.dout) + qo + ks * 32 + grp * 8) : TT::zero();
      const frag of = qvalid ? TT::load8(static_cast<const T*>(a.out) + qo + ks * 32 + grp * 8) : TT::zero();
#pragma unroll
      for (int e = 0; e < 8; ++e) delta[g] += TT::to_f(dof[g][ks][e]) * TT::to_f(of[e]);
    }
    delta[g] = xor_sum_groups(delta[g]);
  }

  const uint64_t sel_prev = chunk_sel(a.sel_idx, bh, c - 1, d);
  const int nsel_c = c >= 2 ? (c - 1) * d.topk : 0;  // compact rows of chunks <= c-2
  const T* ksel = static_cast<const T*>(a.ksel) + bh * a.ntiles * 64 * D;
  const T* vsel = static_cast<const T*>(a.vsel) + bh * a.ntiles * 64 * D;
  const T* kselt = static_cast<const T*>(a.kselt) + bh * a.ntiles * (D * 64);
  const float* st = a.ustate + (bh * d.nC + c) * R;  // S_c, z_c
  const long long krs = static_cast<long long>(d.Hkv) * D;

  // ---- one pass over the keys. The softmax part of dq accumulates sum 2^{a - m} (dP - Delta) k
  // against a running reference m (log2 units; moved up only when a score passes it by more
  // than kLazy2, the accumulator rescaled then), the linear-attention part of dphi(q)
  // accumulates sum (dP - Delta) phi(k) unscaled, and both are divided by the normaliser
  // once it is known, at the end. Scores are raw q.k, the scale folded into the exponent's fma.
  constexpr float kLazy2 = 8.f;
  float m2[QH], l_lane[QH];  // running reference; this lane's share of the softmax part / 2^m
  f32x4 dqt[QH][ND];
#pragma unroll
  for (int g = 0; g < QH; ++g) {
    m2[g] = -kInf;
    l_lane[g] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) dqt[g][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto rebase = [&](int g, const f32x4 (&sc)[4], const bool (&sa)[4][4], bool masked) {
    float tm = -kInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) tm = (!masked || sa[kb][e]) ? fmaxf(tm, sc[kb][e]) : tm;
    tm = xor_max_groups(tm) * scale2;
    const bool move = tm > m2[g] + kLazy2;  // the same in the four lanes of a query
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float mn = move ? tm : m2[g];
      const float alpha = mn == m2[g] ? 1.f : __builtin_amdgcn_exp2f(m2[g] - mn);
      l_lane[g] *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) dqt[g][db] *= alpha;
      m2[g] = mn;
    }
  };
  // the compact tiles arrive by buffer -> LDS copies, one tile ahead; rows at or beyond
  // nsel_c read as zeros (the copies' range ends there)
  using DmaR = DmaTile<T, D, 64, NWV>;   // 64 rows of D
  using DmaT = DmaTile<T, 64, D, NWV>;   // D rows of 64 (K^T)
  using DmaF = DmaTile<T, F, 64, NWV>;   // 64 rows of F (phi(K))
  using DmaFT = DmaTile<T, 64, F, NWV>;  // F rows of 64 (phi(K)^T)
  DmaR dmr;
  dmr.init(D);
  DmaT dmt;
  dmt.init(64);
  constexpr int ES = static_cast<int>(sizeof(T));
  const int ntc = (nsel_c + 63) / 64;
  const auto rs_k = make_rsrc(ksel, static_cast<uint32_t>(nsel_c * D * ES));
  const auto rs_v = make_rsrc(vsel, static_cast<uint32_t>(nsel_c * D * ES));
  const auto rs_kt = make_rsrc(kselt, static_cast<uint32_t>(ntc * D * 64 * ES));
  auto issue3 = [&](int t) {
    T* const sl = lds + (t & 1) * 3 * SLOT;
    dmr.issue(sl, rs_k, t * 64 * D * ES);
    dmr.issue(sl + SLOT, rs_v, t * 64 * D * ES);
    dmt.issue(sl + 2 * SLOT, rs_kt, t * D * 64 * ES);
  };
  {  // W into its own region, ahead of the first compact tile (copies complete in order)
    DmaTile<T, D, F, NWV> dmw;
    dmw.init(D);
    dmw.issue(t_w, make_rsrc(W, static_cast<uint32_t>(F * D * ES)), 0);
  }
  if (ntc > 0) issue3(0);
  for (int t = 0; t < ntc; ++t) {
    if (t + 1 < ntc) {
      issue3(t + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * DmaR::PER_WAVE + DmaT::PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    lds_sync();
    const int nv = min(64, nsel_c - t * 64);
    const T* const sl = lds + (t & 1) * 3 * SLOT;
    f32x4 s[QH][4], dp[QH][4];
    rows_x_frags<T, D, QH>(s, sl, qf);
    rows_x_frags<T, D, QH>(dp, sl + SLOT, dof);
    bool sa[4][4];
    if (nv == 64) {  // a full tile
#pragma unroll
      for (int g = 0; g < QH; ++g) {
        rebase(g, s[g], sa, false);
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[g][kb][e], scale2, -m2[g]));
            ps += p;
            s[g][kb][e] = p * (dp[g][kb][e] - delta[g]);
          }
        l_lane[g] += ps;
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[kb][e] = kb * 16 + 4 * grp + e < nv;
#pragma unroll
      for (int g = 0; g < QH; ++g) {
        rebase(g, s[g], sa, true);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = sa[kb][e] ? __builtin_amdgcn_exp2f(fmaf(s[g][kb][e], scale2, -m2[g])) : 0.f;
            l_lane[g] += p;
            s[g][kb][e] = p * (dp[g][kb][e] - delta[g]);
          }
      }
    }
    rows_x_accs<T, ND, 64, QH>(dqt, sl + 2 * SLOT, s);
    lds_sync();
  }

  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  lds_sync();  // W is in place, the compact tiles are no longer read

  // dphi(q) starts with the state part S_c dout - Delta z_c (its factor e^{-L}, like that of
  // the near chunks' part, is applied once L is known); S_c is staged in LDS in the operand
  // dtype, which is the rounding its MFMA operands take, and serves every head
  f32x4 dpt[QH][NF];
#pragma unroll
  for (int g = 0; g < QH; ++g)
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) dpt[g][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c >= 2) {
    T* const t_s = lds;  // F rows of D, slots 0-1
    for (int e8 = tid; e8 < F * D / 8; e8 += NT) {
      const int f = e8 / (D / 8), dd = (e8 % (D / 8)) * 8;
      Swz<T, D>::store8(t_s, f, dd, f32_frag<T>(st + f * D + dd));
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < F / 64; ++rb) {
      f32x4 sdo[QH][4];
      rows_x_frags<T, D, QH>(sdo, t_s + rb * 64 * D, dof);
#pragma unroll
      for (int g = 0; g < QH; ++g)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dpt[g][rb * 4 + blk][e] = sdo[g][blk][e] - delta[g] * st[F * D + (rb * 4 + blk) * 16 + 4 * grp + e];
    }
  }

  // phi(q) of each head as operand fragments for the near chunks (the NP-Map forward is
  // recomputed for its backward at the end, which keeps the loops' registers low)
  frag phf[QH][F / 32];
  float dla[QH];  // the linear-attention part of the normaliser
#pragma unroll
  for (int g = 0; g < QH; ++g) {
    NpRow<F> nq;
    np_forward<T, D, F, true>(nq, t_w, qf[g]);
    f32x4 phq[NF];
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) phq[fb][e] = nq.r * nq.m[fb][e] * nq.inv_nm;
#pragma unroll
    for (int s2 = 0; s2 < F / 32; ++s2) phf[g][s2] = pk_frag<T>(phq[2 * s2], phq[2 * s2 + 1]);
    dla[g] = 0.f;
    if (c >= 2) {  // state part: phi(q) . z_c
#pragma unroll
      for (int fb = 0; fb < NF; ++fb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dla[g] += phq[fb][e] * st[F * D + fb * 16 + 4 * grp + e];
    }
  }
  DmaR dkv;  // key and value rows of the input, row stride Hkv * D
  dkv.init(static_cast<int>(krs));
  DmaF dmf;
  dmf.init(F);
  DmaFT dmft;
  dmft.init(64);
  for (int cc = c >= 1 ? c - 1 : 0; cc <= c; ++cc) {
    __syncthreads();
    const long long r0 = (static_cast<long long>(b) * d.T + 64LL * cc) * d.Hkv + h;
    const int nv = min(64, d.T - 64 * cc);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * krs + D) * ES);
    dkv.issue(t_k, make_rsrc(static_cast<const T*>(a.k) + r0 * D, rows_b), 0);
    dkv.issue(t_v, make_rsrc(static_cast<const T*>(a.v) + r0 * D, rows_b), 0);
    dmt.issue(t_kt, make_rsrc(static_cast<const T*>(a.kt) + (bh * d.nC + cc) * D * 64, D * 64 * ES), 0);
    dmf.issue(t_pk, make_rsrc(static_cast<const T*>(a.phik) + (bh * d.nC * 64 + 64LL * cc) * F, 64 * F * ES), 0);
    dmft.issue(t_pkt, make_rsrc(static_cast<const T*>(a.phikt) + (bh * d.nC + cc) * F * 64, F * 64 * ES), 0);
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    lds_sync();
    bool sa[4][4], la[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jr = kb * 16 + 4 * grp + e;
        const int dist = 64 * (c - cc) + qrow - jr;  // i - j
        const bool vis = dist >= 0;
        const bool inwin = dist < d.window;
        const bool sel = cc < c && ((sel_prev >> jr) & 1ull);
        sa[kb][e] = vis && (inwin || sel);
        la[kb][e] = vis && !(inwin || sel);
      }
    // the heads one after the other here (two chunks against the compact loop's many tiles;
    // holding both heads' scores at once would not fit the registers at D = 128)
#pragma unroll
    for (int g = 0; g < QH; ++g) {
      f32x4 s[4], dp[4], lw[4];
      rows_x_frag<T, D>(s, t_k, qf[g]);
      rows_x_frag<T, D>(dp, t_v, dof[g]);
      rows_x_frag<T, F>(lw, t_pk, phf[g]);
      rebase(g, s, sa, true);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = sa[kb][e] ? __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale2, -m2[g])) : 0.f;
          const float gr = dp[kb][e] - delta[g];
          l_lane[g] += p;
          dla[g] += la[kb][e] ? lw[kb][e] : 0.f;
          s[kb][e] = p * gr;
          lw[kb][e] = la[kb][e] ? gr : 0.f;
        }
      rows_x_acc<T, ND>(dqt[g], t_kt, s);
      rows_x_acc<T, NF>(dpt[g], t_pkt, lw);
      __builtin_amdgcn_sched_barrier(0);  // keeps the heads' live ranges apart
    }
  }

  // ---- per head: the normaliser, the NP-Map backward and dq, then what the key side needs:
  // (L, Delta), phi(q) rows and transposed, q^T, dout^T, the per-chunk sums behind R and the
  // q side of dW
  __syncthreads();  // the near tiles are no longer read
  T* const t_wt = lds;  // D x F, slots 0-1
  load_wt<T, D, F>(t_wt, W);
  __syncthreads();
  T* const e_phq = lds + 2 * SLOT;  // e^{-L} phi(q)^T, F rows
  T* const e_do = lds + 3 * SLOT;   // dout^T, D rows
  T* const e_dz = lds + 4 * SLOT;   // dz^T, F rows
  T* const e_q = lds + 5 * SLOT;    // q^T, D rows
  const int pq = pk_pos(qrow);
  // the shares of R and of dW are kept per workgroup (its HPW heads): with four waves the
  // second head adds its share onto the first's (the same thread writes the same elements for
  // both); with eight the sums stay in registers. Either way the reductions over the query
  // heads read 1 / HPW as much.
  const long long gc = (static_cast<long long>(b) * nhg + hgi) * d.nC + c;
  // e-tiles of a head: e^{-L} phi(q)^T (F rows), dout^T (D rows), dz^T (F rows), q^T (D rows).
  // Four waves stage one head in slots 2-5; with eight, the second head takes slots 0-1 and
  // W's region, free once every wave has its dz and dx.
  auto e_tile = [&](int hs, int k) -> T* {  // k: 0 phi(q)^T, 1 dout^T, 2 dz^T, 3 q^T
    return hs == 0 ? lds + (2 + k) * SLOT : (k < 2 ? lds + k * SLOT : t_w + (k - 2) * SLOT);
  };
  static_assert(NWV == 4 || (F * 64 <= SLOT && D * 64 <= SLOT && 2 * SLOT <= F * D), "e-tile room");
  // e^{-L} phi(q) and dz transposed, dout and q transposed into the e-tiles of set hs (the
  // wave's 16 query columns), and this wave's part of the a_c sums over its queries into s_red
  auto stage_tiles = [&](int hs, const f32x4 (&ps4)[NF], const f32x4 (&dz)[NF], const frag (&xq8)[D / 32],
                         const frag (&do8)[D / 32], float dlt) {
    T* const tp = e_tile(hs, 0);
    T* const tdo = e_tile(hs, 1);
    T* const tdz = e_tile(hs, 2);
    T* const tq = e_tile(hs, 3);
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = fb * 16 + 4 * grp + e;
        tp[SW::off(f, pq)] = TT::from_f(ps4[fb][e]);
        tdz[SW::off(f, pq)] = TT::from_f(dz[fb][e]);
      }
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = ks * 32 + grp * 8 + e;
        tdo[SW::off(dd, pq)] = do8[ks][e];
        tq[SW::off(dd, pq)] = xq8[ks][e];
      }
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = xor_sum_16(ps4[fb][e] * dlt);
        if (r16 == 0) s_red[wave][fb * 16 + 4 * grp + e] = v;
      }
  };
  // the staged e-tiles of set hs (query head hq) to memory in 16-byte pieces (every thread)
  auto store_tiles = [&](int hs, int hq) {
    const long long qc = (static_cast<long long>(b) * d.Hq + hq) * d.nC + c;
    T* phqt = static_cast<T*>(a.phiqt) + qc * F * 64;
    T* qt = static_cast<T*>(a.qt) + qc * D * 64;
    T* dot = static_cast<T*>(a.dot) + qc * D * 64;
    for (int idx = tid; idx < F * 8; idx += NT) {
      const int row = idx >> 3, col = (idx & 7) * 8;
      TT::store8(phqt + row * 64 + col, SW::load8(e_tile(hs, 0), row, col));
    }
    for (int idx = tid; idx < D * 8; idx += NT) {
      const int row = idx >> 3, col = (idx & 7) * 8;
      TT::store8(qt + row * 64 + col, SW::load8(e_tile(hs, 3), row, col));
      TT::store8(dot + row * 64 + col, SW::load8(e_tile(hs, 1), row, col));
    }
  };
  float* ap = a.apart + gc * R;
  float* wp = a.dwq + gc * (F * D);
#pragma unroll
  for (int g = 0; g < QH; ++g) {
    const int hq = hq0 + g;
    const long long bhq = static_cast<long long>(b) * d.Hq + hq;
    const long long qoff = qoff0 + g * D;
    const float l = xor_sum_groups(l_lane[g]);
    const float dl = xor_sum_groups(dla[g]);
    float L2;
    if (!qvalid) {
      L2 = kInf;
    } else if (l > 0.f && dl > 0.f) {
      const float ld = log2f(dl);
      const float M = fmaxf(m2[g], ld);
      L2 = M + log2f(l * exp2f(m2[g] - M) + exp2f(ld - M));
    } else if (l > 0.f) {
      L2 = m2[g] + log2f(l);
    } else {
      L2 = dl > 0.f ? log2f(dl) : kInf;  // an empty normaliser: out = 0, no gradient
    }
    const float einv = exp2f(-L2);
    const float sa_scale = l > 0.f ? exp2f(m2[g] - L2) : 0.f;  // 2^m / normaliser
#pragma unroll
    for (int db = 0; db < ND; ++db) dqt[g][db] *= sa_scale;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) dpt[g][fb] *= einv;

    // the head's q rows read again: the loops' copies end there, rather than living on
    // (unpacked for the element stores below) through the loops; dout likewise, further down
    frag xq8[D / 32], do8[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      xq8[ks] = qvalid ? TT::load8(static_cast<const T*>(a.q) + qoff + ks * 32 + grp * 8) : TT::zero();

    // NP-Map backward and dq
    NpRow<F> nq;
    np_forward<T, D, F, true>(nq, t_w, xq8);
    f32x4 ps4[NF];  // e^{-L} phi(q), the factor every key-side use takes
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) ps4[fb][e] = nq.r * nq.m[fb][e] * nq.inv_nm * einv;
    const float dr = np_backward<F>(nq, dpt[g]);  // dpt[g] now holds dz
    f32x4 dxt[ND] = {};
    rows_x_acc<T, ND, F>(dxt, t_wt, dpt[g]);  // dxt[db][e] = (W^T dz)[16 db + 4 grp + e]
    if (qvalid) {
      T* dq = static_cast<T*>(a.dq) + qoff;
      const T* xq = static_cast<const T*>(a.q) + qoff;
      const float xs = nq.r > 0.f ? dr / nq.r : 0.f;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const typename TT::quad x4 = TT::load4(xq + db * 16 + 4 * grp);
        typename TT::quad o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = TT::from_f(dqt[g][db][e] * isd + dxt[db][e] + xs * TT::to_f(x4[e]));
        *reinterpret_cast<typename TT::quad*>(dq + db * 16 + 4 * grp) = o4;
      }
    }

    if (grp == 0) {
      a.ld[(bhq * d.nC * 64 + 64LL * c + qrow) * 2] = L2;
      a.ld[(bhq * d.nC * 64 + 64LL * c + qrow) * 2 + 1] = qvalid ? delta[g] : 0.f;
    }
    // phi(q) rows are stored times e^{-L}, like the transposed tile
    {
      T* phqr = static_cast<T*>(a.phiq) + (bhq * d.nC * 64 + 64LL * c + qrow) * F;
#pragma unroll
      for (int s2 = 0; s2 < F / 32; ++s2) TT::store8(phqr + 32 * s2 + 8 * grp, pk_frag<T>(ps4[2 * s2], ps4[2 * s2 + 1]));
    }
    const float dlt = qvalid ? delta[g] : 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      do8[ks] = qvalid ? TT::load8(static_cast<const T*>(a.dout) + qoff + ks * 32 + grp * 8) : TT::zero();
    if constexpr (NWV == 4) {
      if (g > 0) __syncthreads();  // the previous head's tiles and sums are no longer read
      stage_tiles(0, ps4, dpt[g], xq8, do8, dlt);
      __syncthreads();
      store_tiles(0, hq);
      for (int f = tid; f < F; f += NT) {
        const float v = ((s_red[0][f] + s_red[1][f]) + s_red[2][f]) + s_red[3][f];
        ap[F * D + f] = g > 0 ? ap[F * D + f] + v : v;
      }
      f32x4 acc[F / 64][D / 16];
      tile_x_tile<T, F, D>(acc, e_phq, e_do);  // A_c[f][d] = sum_q e^{-L} phi(q)[f] dout[d]
#pragma unroll
      for (int rb = 0; rb < F / 64; ++rb)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* o = ap + ((wave + 4 * rb) * 16 + 4 * grp + e) * D + cb * 16 + r16;
            *o = g > 0 ? *o + acc[rb][cb][e] : acc[rb][cb][e];
          }
      tile_x_tile<T, F, D>(acc, e_dz, e_q);  // dW[f][d] = sum_q dz[f] q[d]
#pragma unroll
      for (int rb = 0; rb < F / 64; ++rb)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* o = wp + ((wave + 4 * rb) * 16 + 4 * grp + e) * D + cb * 16 + r16;
            *o = g > 0 ? *o + acc[rb][cb][e] : acc[rb][cb][e];
          }
    } else {
      // both heads staged at once, then the block-wide part over the two sets; the products
      // over the staged tiles are split by row block over all eight waves and summed over
      // the heads in registers
      __syncthreads();  // W and W^T are no longer read
      stage_tiles(hsub, ps4, dpt[g], xq8, do8, dlt);
      __syncthreads();
      store_tiles(0, hqb);
      store_tiles(1, hqb + 1);
      float red8 = 0.f;
      if (tid < F) {
#pragma unroll
        for (int w8 = 0; w8 < NWV; ++w8) red8 += s_red[w8][tid];
      }
      constexpr int NRB8 = F / (16 * NWV);
      f32x4 acc_a[NRB8][D / 16], acc_w[NRB8][D / 16];
#pragma unroll
      for (int rb = 0; rb < NRB8; ++rb)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) acc_a[rb][cb] = acc_w[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int rb = 0; rb < NRB8; ++rb)
#pragma unroll
          for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const int row = (wave + NWV * rb) * 16 + r16, col = cb * 16 + r16;
              const int kc = ks * 32 + grp * 8;
              Tr<T>::mma(acc_a[rb][cb], SW::load8(e_tile(hs, 0), row, kc), SW::load8(e_tile(hs, 1), col, kc));
              Tr<T>::mma(acc_w[rb][cb], SW::load8(e_tile(hs, 2), row, kc), SW::load8(e_tile(hs, 3), col, kc));
            }
      if (tid < F) ap[F * D + tid] = red8;
#pragma unroll
      for (int rb = 0; rb < NRB8; ++rb)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int o = ((wave + NWV * rb) * 16 + 4 * grp + e) * D + cb * 16 + r16;
            ap[o] = acc_a[rb][cb][e];
            wp[o] = acc_w[rb][cb][e];
          }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Selected keys against the queries of chunks >= their chunk + 2. A workgroup of eight
// waves takes 128 compact rows (16 per wave) and one of the query slices; it writes fp32
// partial dk, dv (softmax part, before the 1/sqrt(D) of dk). The query-side tiles (q rows,
// dout rows, q^T, dout^T) arrive by buffer -> LDS copies one (chunk, head) step ahead, with
// that step's (L, Delta) prefetched into registers.
template <typename T, int D>
__global__ __launch_bounds__(512, D == 64 ? 2 : 1) void bwd_dkv_far_kernel(BwdArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using DmaR = DmaTile<T, D, 64, 8>;  // 64 rows of D
  using DmaT = DmaTile<T, 64, D, 8>;  // D rows of 64
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int ND = D / 16;
  __shared__ __attribute__((aligned(16))) T lds[2][4][D * 64];  // [buffer][q, dout, q^T, dout^T]
  __shared__ __attribute__((aligned(16))) float s_ld[2][2][64];  // [buffer][L, Delta][query]
  const Dims& d = a.d;
  // work index: row group fastest, then query slice, then (batch, KV head): the row groups
  // of one slice read the same query tiles
  const int ngroups = (a.ntiles + 1) / 2;
  const int w = xcd_work(blockIdx.x, gridDim.x);
  const int grp_id = __builtin_amdgcn_readfirstlane(w % ngroups);
  const int split = __builtin_amdgcn_readfirstlane((w / ngroups) % a.nsplit);
  const long long bh = __builtin_amdgcn_readfirstlane(w / (ngroups * a.nsplit));
  const int b = __builtin_amdgcn_readfirstlane(static_cast<int>(bh / d.Hkv));
  const int h = __builtin_amdgcn_readfirstlane(static_cast<int>(bh % d.Hkv));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const float scale2 = kLog2e * inv_sqrt_d<D>();
  const int nsel = d.nCc * d.topk;
  const int row0 = grp_id * 128;
  const int n = row0 + wave * 16 + r16;  // this lane column's compact row
  const bool nin = n < a.ntiles * 64;     // inside the buffers (rows past nsel are zeros)
  const int ckey = n < nsel ? n / d.topk : 0x3fffffff;
  frag kf[D / 32], vf[D / 32];
  {
    const T* kr = static_cast<const T*>(a.ksel) + (bh * a.ntiles * 64 + n) * D;
    const T* vr = static_cast<const T*>(a.vsel) + (bh * a.ntiles * 64 + n) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      kf[ks] = nin ? TT::load8(kr + ks * 32 + grp * 8) : TT::zero();
      vf[ks] = nin ? TT::load8(vr + ks * 32 + grp * 8) : TT::zero();
    }
  }
  // query chunks: slice `split` of [0, nC) (the same slices for every row group), from the
  // group's first chunk + 2 on; steps run over (chunk, head)
  const int c_lo = row0 / d.topk + 2;
  const int per = (d.nC + a.nsplit - 1) / a.nsplit;
  const int cb0 = max(c_lo, split * per), cb1 = min(d.nC, (split + 1) * per);
  const int nsteps = max(0, cb1 - cb0) * d.G;
  DmaT dma;
  dma.init(64);
  DmaR dmq;
  dmq.init(d.Hq * D);
  const long long hq0 = static_cast<long long>(b) * d.Hq + static_cast<long long>(h) * d.G;  // b*Hq + first head
  auto step_ptrs = [&](int st, long long& qc, long long& r0, int& nv) {
    const int cq = __builtin_amdgcn_readfirstlane(cb0 + st / d.G), g = __builtin_amdgcn_readfirstlane(st % d.G);
    qc = (hq0 + g) * d.nC + cq;
    r0 = ((static_cast<long long>(b) * d.T + 64LL * cq) * d.Hq + h * d.G + g) * D;
    nv = min(64, d.T - 64 * cq);
  };
  auto issue = [&](int st) {
    long long qc, r0;
    int nv;
    step_ptrs(st, qc, r0, nv);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * d.Hq * D + D) * ES);
    T(*dst)[D * 64] = lds[st & 1];
    dmq.issue(dst[0], make_rsrc(static_cast<const T*>(a.q) + r0, rows_b), 0);
    dmq.issue(dst[1], make_rsrc(static_cast<const T*>(a.dout) + r0, rows_b), 0);
    dma.issue(dst[2], make_rsrc(static_cast<const T*>(a.qt) + qc * D * 64, D * 64 * ES), 0);
    dma.issue(dst[3], make_rsrc(static_cast<const T*>(a.dot) + qc * D * 64, D * 64 * ES), 0);
  };
  auto ld_of = [&](int st) {  // this thread's (L, Delta) entry of step st
    long long qc, r0;
    int nv;
    step_ptrs(st, qc, r0, nv);
    return a.ld[qc * 128 + (tid & 127)];
  };
  f32x4 dkt[ND] = {}, dvt[ND] = {};
  float ldn = 0.f;
  if (nsteps > 0) {
    ldn = ld_of(0);
    issue(0);
  }
  for (int st = 0; st < nsteps; ++st) {
    const float ldc = ldn;
    if (st + 1 < nsteps) {
      ldn = ld_of(st + 1);
      issue(st + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * DmaR::PER_WAVE + 2 * DmaT::PER_WAVE + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    if (tid < 128) s_ld[st & 1][tid & 1][tid >> 1] = ldc;
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);  // the copies of the next step stay in flight
    lds_sync();
    const int cq = __builtin_amdgcn_readfirstlane(cb0 + st / d.G);
    const T* tq = lds[st & 1][0];
    const T* tdo = lds[st & 1][1];
    const T* tqt = lds[st & 1][2];
    const T* tdot = lds[st & 1][3];
    f32x4 s[4], dp[4];
    rows_x_frag<T, D>(s, tq, kf);  // s[qb][e] = q[16 qb + 4 grp + e] . k
    rows_x_frag<T, D>(dp, tdo, vf);
    const bool on = cq >= ckey + 2;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 lq = *reinterpret_cast<const f32x4*>(&s_ld[st & 1][0][qb * 16 + 4 * grp]);
      const f32x4 dq4 = *reinterpret_cast<const f32x4*>(&s_ld[st & 1][1][qb * 16 + 4 * grp]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = on ? __builtin_amdgcn_exp2f(fmaf(s[qb][e], scale2, -lq[e])) : 0.f;
        s[qb][e] = p * (dp[qb][e] - dq4[e]);
        dp[qb][e] = p;
      }
    }
    rows_x_acc<T, ND>(dvt, tdot, dp);
    rows_x_acc<T, ND>(dkt, tqt, s);
    lds_sync();
  }
  if (nin) {
    float* out = a.dkvsel + ((static_cast<long long>(split) * d.B * d.Hkv + bh) * a.ntiles * 64 + n) * (2 * D);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      *reinterpret_cast<f32x4*>(out + db * 16 + 4 * grp) = dkt[db];
      *reinterpret_cast<f32x4*>(out + D + db * 16 + 4 * grp) = dvt[db];
    }
  }
}

// ---------------------------------------------------------------------------------------
template <typename T, int D, int F>
__global__ __launch_bounds__(256) void bwd_dkv_local_kernel(BwdArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, 64>;
  using DmaR = DmaTile<T, D, 64, 4>;   // 64 rows of D
  using DmaT = DmaTile<T, 64, D, 4>;   // D rows of 64
  using DmaF = DmaTile<T, F, 64, 4>;   // 64 rows of F
  using DmaFT = DmaTile<T, 64, F, 4>;  // F rows of 64
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int ND = D / 16, NF = F / 16, R = F * D + F;
  constexpr int SLOT = (D > F ? D : F) * 64;
  // per step: q rows, dout rows, q^T, dout^T, phi(q) rows, phi(q)^T of one (head, chunk);
  // after the steps: R^T, R, W, W^T
  constexpr int LDS_ELEMS = 6 * SLOT > 4 * D * F ? 6 * SLOT : 4 * D * F;
  __shared__ __attribute__((aligned(16))) T lds[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float s_ld[2][64];  // [L, Delta][query]
  const Dims& d = a.d;
  // work item (chunk c, record (b, h)). Workgroups go to the eight XCDs in turn, so a
  // one-dimensional grid takes the records in groups of eight (record fastest, then the chunk,
  // then the group): chunks c and c + 1 of a record run on one XCD, one after the other, and
  // the query tiles of chunk c + 1 that both read stay in its L2. Other record counts take the
  // chunks outermost; a grid too large for one dimension is launched as (chunk, h, b).
  int c, h, b;
  {
    const int BHn = d.B * d.Hkv, id = static_cast<int>(blockIdx.x);
    int rec;
    if (gridDim.y != 1 || gridDim.z != 1) {
      c = id;
      rec = static_cast<int>(blockIdx.z) * d.Hkv + static_cast<int>(blockIdx.y);
    } else if (BHn % 8 == 0) {
      const int per = d.nC * 8;
      c = (id % per) / 8;
      rec = (id / per) * 8 + id % 8;
    } else {
      c = id / BHn;
      rec = id % BHn;
    }
    b = rec / d.Hkv;
    h = rec % d.Hkv;
  }
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  constexpr float isd = inv_sqrt_d<D>();
  const float scale2 = kLog2e * isd;
  const int jr = wave * 16 + r16;
  const long long j = 64LL * c + jr;  // this lane column's key
  const bool kvalid = j < d.T;
  const uint64_t selm = chunk_sel(a.sel_idx, bh, c, d);
  const bool selj = (selm >> jr) & 1ull;
  const T* W = static_cast<const T*>(a.w) + static_cast<long long>(h) * F * D;
  const long long koff = ((static_cast<long long>(b) * d.T + j) * d.Hkv + h) * D;
  frag kf[D / 32], vf[D / 32], phk[F / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    kf[ks] = kvalid ? TT::load8(static_cast<const T*>(a.k) + koff + ks * 32 + grp * 8) : TT::zero();
    vf[ks] = kvalid ? TT::load8(static_cast<const T*>(a.v) + koff + ks * 32 + grp * 8) : TT::zero();
  }
#pragma unroll
  for (int s2 = 0; s2 < F / 32; ++s2)
    phk[s2] = TT::load8(static_cast<const T*>(a.phik) + (bh * d.nC * 64 + j) * F + s2 * 32 + grp * 8);
  f32x4 dkt[ND] = {}, dvt[ND] = {}, dpk[NF] = {};
  // steps over (query head g, query chunk cq in {c, c+1}); the tiles arrive by
  // buffer -> LDS copies
  const int ncq = c + 1 < d.nC ? 2 : 1;
  const int nsteps = d.G * ncq;
  DmaR dmq;
  dmq.init(d.Hq * D);
  DmaT dmt;
  dmt.init(64);
  DmaF dmf;
  dmf.init(F);
  DmaFT dmft;
  dmft.init(64);
  for (int st = 0; st < nsteps; ++st) {
    const long long hq = static_cast<long long>(b) * d.Hq + h * d.G + __builtin_amdgcn_readfirstlane(st / ncq);
    const int cq = c + __builtin_amdgcn_readfirstlane(st % ncq);
    const long long qc = hq * d.nC + cq;
    const long long r0 =
        ((static_cast<long long>(b) * d.T + 64LL * cq) * d.Hq + (hq - static_cast<long long>(b) * d.Hq)) * D;
    const int nv = min(64, d.T - 64 * cq);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * d.Hq * D + D) * ES);
    const float ldc = a.ld[qc * 128 + (tid & 127)];
    dmq.issue(lds, make_rsrc(static_cast<const T*>(a.q) + r0, rows_b), 0);
    dmq.issue(lds + SLOT, make_rsrc(static_cast<const T*>(a.dout) + r0, rows_b), 0);
    dmt.issue(lds + 2 * SLOT, make_rsrc(static_cast<const T*>(a.qt) + qc * D * 64, D * 64 * ES), 0);
    dmt.issue(lds + 3 * SLOT, make_rsrc(static_cast<const T*>(a.dot) + qc * D * 64, D * 64 * ES), 0);
    dmf.issue(lds + 4 * SLOT, make_rsrc(static_cast<const T*>(a.phiq) + qc * 64 * F, 64 * F * ES), 0);
    dmft.issue(lds + 5 * SLOT, make_rsrc(static_cast<const T*>(a.phiqt) + qc * F * 64, F * 64 * ES), 0);
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    if (tid < 128) s_ld[tid & 1][tid >> 1] = ldc;
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    lds_sync();
    {
      f32x4 s[4], dp[4], lw[4];
      rows_x_frag<T, D>(s, lds, kf);
      rows_x_frag<T, D>(dp, lds + SLOT, vf);
      rows_x_frag<T, F>(lw, lds + 4 * SLOT, phk);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const f32x4 lq = *reinterpret_cast<const f32x4*>(&s_ld[0][qb * 16 + 4 * grp]);
        const f32x4 dq4 = *reinterpret_cast<const f32x4*>(&s_ld[1][qb * 16 + 4 * grp]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qr = qb * 16 + 4 * grp + e;
          const int dist = 64 * (cq - c) + qr - jr;  // i - j
          const bool vis = dist >= 0;
          const bool inwin = dist < d.window;
          const bool sel = cq > c && selj;
          const bool sa = vis && (inwin || sel);
          const bool la = vis && !(inwin || sel);
          const float p = sa ? __builtin_amdgcn_exp2f(fmaf(s[qb][e], scale2, -lq[e])) : 0.f;
          const float gg = dp[qb][e] - dq4[e];
          s[qb][e] = p * gg;                       // dS
          dp[qb][e] = p + (la ? lw[qb][e] : 0.f);  // weight of v_j in out_i (phi(q) carries e^{-L})
          lw[qb][e] = la ? gg : 0.f;               // g / e^{-L}
        }
      }
      rows_x_acc<T, ND>(dvt, lds + 3 * SLOT, dp);
      rows_x_acc<T, ND>(dkt, lds + 2 * SLOT, s);
      rows_x_acc<T, NF>(dpk, lds + 5 * SLOT, lw);
    }
    lds_sync();
  }
  // The closing products read R_c (rows and transposed), W and W^T from LDS, filled in one
  // phase: R_c from its fp32 record in one read, W by a copy, W^T transposed from memory.
  T* const t_rt = lds;              // R^T, D rows of F (features pk-permuted)
  T* const t_r = lds + D * F;       // R, F rows of D
  T* const t_wr = lds + 2 * D * F;  // W, F rows of D
  T* const t_wt = lds + 3 * D * F;  // W^T, D rows of F (features pk-permuted)
  const bool has_r = c + 2 < d.nC;
  const float* rs = a.rstate + (bh * d.nC + c) * R;
  {
    DmaTile<T, D, F, 4> dmw;
    dmw.init(D);
    dmw.issue(t_wr, make_rsrc(W, static_cast<uint32_t>(F * D * ES)), 0);
  }
  if (has_r) load_pk_transposed<T, D, F, float>(t_rt, rs, t_r);
  load_wt<T, D, F>(t_wt, W);
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  __syncthreads();
  // queries of chunks >= c+2 through R_c, r_c (unselected keys only)
  if (has_r) {
    f32x4 rv[NF];  // (R v)[16 fb + 4 grp + e]
#pragma unroll
    for (int rb = 0; rb < F / 64; ++rb) {
      f32x4 part[4];
      rows_x_frag<T, D>(part, t_r + rb * 64 * D, vf);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) rv[rb * 4 + blk] = part[blk];
    }
    const float on = (kvalid && !selj) ? 1.f : 0.f;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dpk[fb][e] += on * (rv[fb][e] - rs[F * D + fb * 16 + 4 * grp + e]);
    frag pm[F / 32];
#pragma unroll
    for (int s2 = 0; s2 < F / 32; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pm[s2][e] = TT::from_f(on * TT::to_f(phk[s2][e]));
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int s2 = 0; s2 < F / 32; ++s2)
        TT::mma(dvt[db], Swz<T, F>::load8(t_rt, db * 16 + r16, s2 * 32 + grp * 8), pm[s2]);
  }
  // selected keys: the later chunks' softmax part from the compact partials
  if (selj && kvalid) {
    const int32_t* sp = a.sel_idx + (bh * d.nCc + c) * d.topk;
    int rank = 0;
    for (int r = 0; r < d.topk; ++r) rank += (sp[r] - 64 * c) < jr ? 1 : 0;
    const int n = c * d.topk + rank;
    for (int sidx = 0; sidx < a.nsplit; ++sidx) {
      const float* p = a.dkvsel + ((static_cast<long long>(sidx) * d.B * d.Hkv + bh) * a.ntiles * 64 + n) * (2 * D);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        dkt[db] += *reinterpret_cast<const f32x4*>(p + db * 16 + 4 * grp);
        dvt[db] += *reinterpret_cast<const f32x4*>(p + D + db * 16 + 4 * grp);
      }
    }
  }
  // NP-Map backward and dk, dv
  NpRow<F> nk;
  np_forward<T, D, F, true>(nk, t_wr, kf);
  const float dr = np_backward<F>(nk, dpk);  // dpk now holds dz
  f32x4 dxt[ND] = {};
  rows_x_acc<T, ND, F>(dxt, t_wt, dpk);
  if (kvalid) {
    T* dk = static_cast<T*>(a.dk) + koff;
    T* dv = static_cast<T*>(a.dv) + koff;
    const T* xk = static_cast<const T*>(a.k) + koff;
    const float xs = nk.r > 0.f ? dr / nk.r : 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const typename TT::quad x4 = TT::load4(xk + db * 16 + 4 * grp);
      typename TT::quad o4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o4[e] = TT::from_f(dkt[db][e] * isd + dxt[db][e] + xs * TT::to_f(x4[e]));
        v4[e] = TT::from_f(dvt[db][e]);
      }
      *reinterpret_cast<typename TT::quad*>(dk + db * 16 + 4 * grp) = o4;
      *reinterpret_cast<typename TT::quad*>(dv + db * 16 + 4 * grp) = v4;
    }
  }
  // dW (k side) of the chunk: sum over its keys of dz k^T
  __syncthreads();
  T* const t_dz = lds + 2 * SLOT;  // dz^T, F rows of 64 keys
  T* const t_kt = lds + 4 * SLOT;  // K^T, D rows of 64 keys
  const int pj = pk_pos(jr);
#pragma unroll
  for (int fb = 0; fb < NF; ++fb)
#pragma unroll
    for (int e = 0; e < 4; ++e) t_dz[SW::off(fb * 16 + 4 * grp + e, pj)] = TT::from_f(kvalid ? dpk[fb][e] : 0.f);
  tile_load<T, 64, D>(t_kt, static_cast<const T*>(a.kt) + (bh * d.nC + c) * D * 64, 64, D);
  __syncthreads();
  f32x4 acc[F / 64][D / 16];
  tile_x_tile<T, F, D>(acc, t_dz, t_kt);
  float* wp = a.dwk + (bh * d.nC + c) * (F * D);
#pragma unroll
  for (int rb = 0; rb < F / 64; ++rb)
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) wp[((wave + 4 * rb) * 16 + 4 * grp + e) * D + cb * 16 + r16] = acc[rb][cb][e];
}

// ---------------------------------------------------------------------------------------
// dW = sum over batch, chunks and the group's query heads (q side) plus keys (k side):
// gridDim.y slices of the item list, then a fixed-order sum of the slices. A thread takes 4
// neighbouring elements, so that every load of a wave reads 1 KB in one piece.
__global__ __launch_bounds__(256) void bwd_dw_part_kernel(const float* dwq, const float* dwk, float* part, int B,
                                                          int Hkv, int G, int nC, int FD) {
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // over Hkv * F * D
  const int h = e / FD, fd = e % FD;
  const int nq = B * G * nC, nitems = nq + B * nC;
  const int per = (nitems + gridDim.y - 1) / gridDim.y;
  const int i0 = blockIdx.y * per, i1 = min(nitems, i0 + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;  // loads of U items in flight together
  for (int it0 = i0; it0 < i1; it0 += U) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (it < i1) {
        if (it < nq) {
          const int b = it / (G * nC), g = (it / nC) % G, c = it % nC;
          x[u] = *reinterpret_cast<const f32x4*>(dwq + ((static_cast<long long>(b) * Hkv * G + h * G + g) * nC + c) * FD + fd);
        } else {
          const int it2 = it - nq, b = it2 / nC, c = it2 % nC;
          x[u] = *reinterpret_cast<const f32x4*>(dwk + ((static_cast<long long>(b) * Hkv + h) * nC + c) * FD + fd);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += x[u];
  }
  *reinterpret_cast<f32x4*>(part + static_cast<long long>(blockIdx.y) * Hkv * FD + e) = acc;
}

__global__ __launch_bounds__(256) void bwd_dw_sum_kernel(const float* part, float* dw, int n, int nparts) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float acc = 0.f;
  for (int p = 0; p < nparts; ++p) acc += part[static_cast<long long>(p) * n + e];
  dw[e] = acc;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D, int F>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  const Dims& d = a.d;
  constexpr int R = F * D + F;
  hipError_t e;
  auto mark = [&](int k) { return ev ? hipEventRecord(ev[k], s) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  if (a.ntiles > 0) {
    const size_t tb = static_cast<size_t>(d.B) * d.Hkv * a.ntiles * 64 * D * sizeof(T);
    if ((e = launch_fill_zero(a.kselt, tb, s)) != hipSuccess) return e;
    if ((e = launch_fill_zero(a.ksel, tb, s)) != hipSuccess) return e;
    if ((e = launch_fill_zero(a.vsel, tb, s)) != hipSuccess) return e;
  }
  const dim3 gk(d.nC, d.Hkv, d.B);
  hipLaunchKernelGGL((bwd_kprep_kernel<T, D, F>), gk, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
  const long long ne = static_cast<long long>(d.B) * d.Hkv * R;
  const dim3 gs(static_cast<unsigned>((ne + 255) / 256));
  hipLaunchKernelGGL(bwd_scan_fwd_kernel, gs, dim3(256), 0, s, a.ustate, d.nC, R, ne);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  // two query heads per wave where the group splits evenly (bf16: the fp32 operands would
  // double the registers)
  const bool two = bwd_heads_per_wave(sizeof(T) == 2, d.G) == 2;
  const int Gp = two ? d.G / 2 : d.G;  // records of R and dW shares per KV head and chunk
  // (at D = 128 the pair is one head per group of four waves, so that two waves share a SIMD)
  if constexpr (sizeof(T) == 2) {
    if (two) {
      if constexpr (D == 128)
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, F, 1, 8>), dim3(d.nC * (d.Hq / 2) * d.B), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, F, 2, 4>), dim3(d.nC * (d.Hq / 2) * d.B), dim3(256), 0, s, a);
    }
  }
  if (!two) hipLaunchKernelGGL((bwd_dq_kernel<T, D, F, 1, 4>), dim3(d.nC * d.Hq * d.B), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  if (ne >= (1LL << 19)) {  // one thread per (b, KV head, element) fills the GPU
    hipLaunchKernelGGL(bwd_rev_full_kernel, gs, dim3(256), 0, s, a.apart, a.rstate, d.nC, Gp, d.Hkv, R, ne);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(4)) != hipSuccess) return e;
  } else {
    const int nseg = (d.nC + kRevSeg - 1) / kRevSeg;
    const long long nr = ne * nseg;
    const dim3 gr(static_cast<unsigned>((nr + 255) / 256));
    hipLaunchKernelGGL(bwd_rev_seg_kernel, gr, dim3(256), 0, s, a.apart, a.segsum, d.nC, Gp, d.Hkv, nseg, R, nr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_rev_scan_kernel, gr, dim3(256), 0, s, a.apart, a.segsum, a.rstate, d.nC, Gp, d.Hkv, nseg,
                       R, nr);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(4)) != hipSuccess) return e;
  }
  if (a.ntiles > 0) {
    hipLaunchKernelGGL((bwd_dkv_far_kernel<T, D>), dim3((a.ntiles + 1) / 2 * a.nsplit * d.B * d.Hkv), dim3(512), 0, s,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(5)) != hipSuccess) return e;
  {
    const long long items = static_cast<long long>(d.nC) * d.Hkv * d.B;  // one dimension while it fits
    const dim3 gl = items * 256 < (1LL << 32) ? dim3(static_cast<unsigned>(items)) : gk;
    hipLaunchKernelGGL((bwd_dkv_local_kernel<T, D, F>), gl, dim3(256), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(6)) != hipSuccess) return e;
  const int nw = d.Hkv * F * D;
  hipLaunchKernelGGL(bwd_dw_part_kernel, dim3(nw / 1024, a.dw_parts), dim3(256), 0, s, a.dwq, a.dwk, a.dwpart, d.B,
                     d.Hkv, Gp, d.nC, F * D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dw_sum_kernel, dim3((nw + 255) / 256), dim3(256), 0, s, a.dwpart, a.dw, nw, a.dw_parts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(7);
}

int bwd_heads_per_wave(int bf16, int G) { return bf16 && G % 2 == 0 ? 2 : 1; }

bool bwd_shape_supported(int bf16, int D, int F) {
  return (D == 64 && F == 64) || (bf16 && D == 128 && F == 128);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s, hipEvent_t* events) {
  const Dims& d = a.d;
  if (d.bf16 && d.D == 64 && d.DF == 64) return launch_bwd_t<bf16, 64, 64>(a, s, events);
  if (d.bf16 && d.D == 128 && d.DF == 128) return launch_bwd_t<bf16, 128, 128>(a, s, events);
  if (!d.bf16 && d.D == 64 && d.DF == 64) return launch_bwd_t<float, 64, 64>(a, s, events);
  return hipErrorInvalidValue;
}

}  // namespace still

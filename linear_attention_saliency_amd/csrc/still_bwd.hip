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
//   bwd_dq_kernel        per (chunk, query head, batch): one pass over the keys gives dq and
//                        L_i together (the softmax part against a running reference,
//                        divided by the normaliser at the end), the per-chunk sums behind
//                        R, the q side of dW
//   bwd_rev_seg_kernel / bwd_rev_scan_kernel: R_c = sum over chunks >= c+2 and over the
//                        query group (a segmented scan)
//   bwd_dkv_far_kernel   per (compact tile, query split, KV head): the selected keys
//                        against the queries of chunks >= their chunk + 2
//   bwd_dkv_local_kernel per (chunk, KV head, batch): keys against the queries of their
//                        own chunk and the next; R_c; the NP-Map backward; dk, dv
//   bwd_dw_part_kernel / bwd_dw_sum_kernel: dW summed over chunks, heads and batch
//
// Supported: head_dim = feat_dim = 64, chunk 64, fp32 or bf16. Matrix products run on
// MFMA in the layer's dtype with fp32 accumulation; every sum that crosses workgroups
// goes through fp32 buffers in a fixed order, so the result is deterministic.
#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"
#include "still_tile.hpp"

namespace still {

namespace {

constexpr int BD = 64;   // head_dim
constexpr int BF = 64;   // feat_dim
constexpr int BR = BF * BD + BF;

// NP-Map forward of one row per lane column, for the row held as B fragments xf (SK):
// z[blk][i] = (W x)[16 blk + 4 grp + i]; also m = elu(z) + 1, |x| and 1/|m|.
struct NpRow {
  f32x4 z[4];
  f32x4 m[4];
  float r, inv_nm;
};

template <typename T>
__device__ __forceinline__ void np_forward(NpRow& n, const T* W, const typename Tr<T>::frag (&xf)[2]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) {
    n.z[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Tr<T>::mma(n.z[fb], Tr<T>::load8(W + (fb * 16 + r16) * BD + ks * 32 + grp * 8), xf[ks]);
  }
  float nm2 = 0.f, xn2 = 0.f;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float zv = n.z[fb][i];
      const float mv = zv > 0.f ? zv + 1.f : __builtin_amdgcn_exp2f(zv * kLog2e);
      n.m[fb][i] = mv;
      nm2 += mv * mv;
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
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
__device__ __forceinline__ float np_backward(const NpRow& n, f32x4 (&dphi)[4]) {
  float dr = 0.f;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dr += dphi[fb][i] * n.m[fb][i];
  dr = xor_sum_groups(dr) * n.inv_nm;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mh = n.m[fb][i] * n.inv_nm;
      const float dm = n.r * (dphi[fb][i] - mh * dr) * n.inv_nm;
      dphi[fb][i] = dm * (n.z[fb][i] > 0.f ? 1.f : n.m[fb][i]);
    }
  return dr;
}

// W^T with the features pk-permuted, [dim][pk_pos(f)], into an LDS tile
template <typename T>
__device__ __forceinline__ void load_wt(T* lds, const T* W) {
  for (int e = threadIdx.x; e < BF * BD; e += blockDim.x) {
    const int f = e >> 6, dd = e & 63;
    lds[Swz<T, 64>::off(dd, pk_pos(f))] = W[e];
  }
}


// buffers of the local-key kernel's step tiles in bf16 (2: the next step's copies overlap
// this one's work; 1 leaves room for more workgroups per CU)
constexpr int kLocalBuffers = 1;
// query heads per dq workgroup in bf16 when the group size is even (1 or 2)
constexpr int kDqHeads = 1;

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

}  // namespace

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_kprep_kernel(BwdArgs a) {
  using TT = Tr<T>;
  __shared__ __attribute__((aligned(16))) T t_k[64 * 64];
  __shared__ __attribute__((aligned(16))) T t_v[64 * 64];
  __shared__ __attribute__((aligned(16))) T t_vt[64 * 64];
  __shared__ float m2part[4 * 64];
  __shared__ float xn2[64];
  const Dims& d = a.d;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int nvalid = min(64, d.T - 64 * c);
  const long long rs = static_cast<long long>(d.Hkv) * BD;
  const long long row0 = (static_cast<long long>(b) * d.T + 64LL * c) * d.Hkv + h;
  tile_load<T>(t_k, static_cast<const T*>(a.k) + row0 * BD, rs, nvalid);
  tile_load<T>(t_v, static_cast<const T*>(a.v) + row0 * BD, rs, nvalid);
  const uint64_t selm = chunk_sel(a.sel_idx, bh, c, d);
  typename TT::frag wf[1][2];
  np_map_load_w<T, 64, 64>(static_cast<const T*>(a.w) + static_cast<long long>(h) * BF * BD, wf);
  __syncthreads();
  // V^T (keys pk-permuted) into LDS, K^T into memory
  T* ktg = static_cast<T*>(a.kt) + (bh * d.nC + c) * (BD * 64);
  for (int e = tid; e < 64 * 64; e += 256) {
    const int dd = e >> 6, p = e & 63, row = pk_index(p);
    t_vt[Swz<T, 64>::off(dd, p)] = t_v[Swz<T, 64>::off(row, dd)];
    ktg[e] = t_k[Swz<T, 64>::off(row, dd)];
  }
  f32x4 phi[4][1];
  np_map_rows64<T, 64, 64>(t_k, 0, wf, m2part, xn2, phi);  // synchronises the workgroup
  const int f = wave * 16 + r16;
  T* phk = static_cast<T*>(a.phik) + (bh * d.nC * 64 + 64LL * c) * BF;
  T* phkt = static_cast<T*>(a.phikt) + (bh * d.nC + c) * (BF * 64);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) phk[(kb * 16 + 4 * grp + i) * BF + pk_pos(f)] = TT::from_f(phi[kb][0][i]);
#pragma unroll
  for (int s = 0; s < 2; ++s) TT::store8(phkt + f * 64 + 32 * s + 8 * grp, pk_frag<T>(phi[2 * s][0], phi[2 * s + 1][0]));
  // U_c = sum over unselected keys of phi(k) v^T, u_c = sum phi(k)
  f32x4 ph[4];
  float zs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = kb * 16 + 4 * grp + i;
      const bool la = row < nvalid && !((selm >> row) & 1ull);
      ph[kb][i] = la ? phi[kb][0][i] : 0.f;
      zs += ph[kb][i];
    }
  zs = xor_sum_groups(zs);
  f32x4 u[4] = {};
  rows_x_acc<T>(u, t_vt, ph);  // u[db][i] = U[f][16 db + 4 grp + i]
  float* ust = a.ustate + (bh * d.nC + c) * BR;
#pragma unroll
  for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4*>(ust + f * BD + db * 16 + 4 * grp) = u[db];
  if (grp == 0) ust[BF * BD + f] = zs;
  // the selected rows, in chunk order, into the compact buffers
  if (c < d.nCc && d.topk > 0) {
    const int32_t* sp = a.sel_idx + (bh * d.nCc + c) * d.topk;
    T* ks = static_cast<T*>(a.ksel) + bh * a.ntiles * 64 * BD;
    T* vs = static_cast<T*>(a.vsel) + bh * a.ntiles * 64 * BD;
    T* kst = static_cast<T*>(a.kselt) + bh * a.ntiles * (BD * 64);
    for (int e = tid; e < d.topk * 64; e += 256) {
      const int r = e >> 6, dd = e & 63;
      const int pos = sp[r] - 64 * c;
      const bool ok = pos >= 0 && pos < 64;
      const T kv = ok ? t_k[Swz<T, 64>::off(pos, dd)] : TT::from_f(0.f);
      const T vv = ok ? t_v[Swz<T, 64>::off(pos, dd)] : TT::from_f(0.f);
      const int n = c * d.topk + r;
      ks[static_cast<long long>(n) * BD + dd] = kv;
      vs[static_cast<long long>(n) * BD + dd] = vv;
      kst[(static_cast<long long>(n >> 6) * BD + dd) * 64 + pk_pos(n & 63)] = kv;
    }
  }
}

// ---------------------------------------------------------------------------------------
// U_c -> S_c = sum over chunks <= c-2, in place; one thread per (b, KV head, element)
__global__ __launch_bounds__(256) void bwd_scan_fwd_kernel(float* ust, int nC, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long bh = gid / BR, e = gid % BR;
  float* p = ust + bh * nC * BR + e;
  float acc = 0.f, p1 = 0.f, p2 = 0.f;
  constexpr int U = 8;  // loads of U chunks in flight together
  for (int c0 = 0; c0 < nC; c0 += U) {
    float cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = c0 + u < nC ? p[static_cast<long long>(c0 + u) * BR] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nC) {
        acc += p2;
        p[static_cast<long long>(c0 + u) * BR] = acc;
      }
      p2 = p1;
      p1 = cur[u];
    }
  }
}

// R_c = sum over chunks >= c+2 of the group's per-chunk sums, as a segmented scan over
// chunks: bwd_rev_seg_kernel sums each segment of kRevSeg chunks (and the group's heads),
// bwd_rev_scan_kernel starts from the later segments' total and scans its own segment down.
// One thread per (b, KV head, segment, element) in both.
constexpr int kRevSeg = 16;

__global__ __launch_bounds__(256) void bwd_rev_seg_kernel(const float* apart, float* segsum, int nC, int G,
                                                          int Hkv, int nseg, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long e = gid % BR, seg = (gid / BR) % nseg, bh = gid / (BR * nseg);
  const long long b = bh / Hkv, h = bh % Hkv;
  const long long hq0 = b * Hkv * G + h * G;
  const int c0 = static_cast<int>(seg) * kRevSeg, c1 = min(nC, c0 + kRevSeg);
  float acc = 0.f;
  for (int g = 0; g < G; ++g) {
    const float* p = apart + (hq0 + g) * nC * BR + e;
    float x[kRevSeg];
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u) x[u] = c0 + u < c1 ? p[static_cast<long long>(c0 + u) * BR] : 0.f;
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u) acc += x[u];
  }
  segsum[gid] = acc;
}

__global__ __launch_bounds__(256) void bwd_rev_scan_kernel(const float* apart, const float* segsum, float* rst,
                                                           int nC, int G, int Hkv, int nseg, long long n_elems) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n_elems) return;
  const long long e = gid % BR, seg = (gid / BR) % nseg, bh = gid / (BR * nseg);
  const long long b = bh / Hkv, h = bh % Hkv;
  const long long hq0 = b * Hkv * G + h * G;
  const int c0 = static_cast<int>(seg) * kRevSeg, c1 = min(nC, c0 + kRevSeg);
  float acc = 0.f;  // sum over the chunks of later segments
  for (long long s2 = nseg - 1; s2 > seg; --s2) acc += segsum[(bh * nseg + s2) * BR + e];
  float x[kRevSeg];
#pragma unroll
  for (int u = 0; u < kRevSeg; ++u) x[u] = 0.f;
  for (int g = 0; g < G; ++g) {
    const float* p = apart + (hq0 + g) * nC * BR + e;
#pragma unroll
    for (int u = 0; u < kRevSeg; ++u)
      if (c0 + u < c1) x[u] += p[static_cast<long long>(c0 + u) * BR];
  }
  float* r = rst + bh * nC * BR + e;
#pragma unroll
  for (int u = kRevSeg - 1; u >= 0; --u) {
    const int c = c0 + u;
    if (c < c1) {
      acc += x[u];  // acc = sum over chunks >= c
      if (c >= 2) r[static_cast<long long>(c - 2) * BR] = acc;
    }
  }
  if (seg == nseg - 1) {  // no chunk lies two or more after the last two
    r[static_cast<long long>(nC - 1) * BR] = 0.f;
    if (nC >= 2) r[static_cast<long long>(nC - 2) * BR] = 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// NH query heads of one KV head per workgroup (four waves each, 16 queries per wave): the
// key tiles each copy brings serve NH x 64 queries.
template <typename T, int NH>
__global__ __launch_bounds__(256 * NH, NH == 1 ? 3 : 1) void bwd_dq_kernel(BwdArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, 64>;
  constexpr int NSLOT = 4 * NH > 6 ? 4 * NH : 6;
  // tile slots: the compact-key loops double-buffer (K, V, K^T) in slots 0-2 and 3-5; the
  // closing products use slots 4 hs .. 4 hs + 3 for head hs
  __shared__ __attribute__((aligned(16))) T lds[NSLOT][64 * 64];
  __shared__ float s_red[NH][4][64];
  T* const t_k = lds[0];
  T* const t_v = lds[1];
  T* const t_kt = lds[2];
  T* const t_pk = lds[3];
  T* const t_pkt = lds[4];

  const Dims& d = a.d;
  // work index: chunk fastest, then head group, then batch (the heads of one KV head
  // share its compact tiles)
  const int ngrp = d.Hq / NH;
  const int w = xcd_work(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int hs = wave >> 2, wl = wave & 3;  // head slot, wave within the head
  // (divisions by run-time sizes leave the compiler unsure that these are uniform; telling
  // it keeps the buffer descriptors in scalar registers)
  const int c = __builtin_amdgcn_readfirstlane(w % d.nC);
  const int hq = __builtin_amdgcn_readfirstlane(((w / d.nC) % ngrp) * NH + hs);
  const int b = __builtin_amdgcn_readfirstlane(w / (d.nC * ngrp));
  const int h = hq / d.G;
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const long long bhq = static_cast<long long>(b) * d.Hq + hq;
  const int qrow = wl * 16 + r16;
  const long long i = 64LL * c + qrow;  // this lane column's query
  const bool qvalid = i < d.T;
  const float scale2 = kLog2e * 0.125f;  // log2(e) / sqrt(64)
  const T* W = static_cast<const T*>(a.w) + static_cast<long long>(h) * BF * BD;

  // the query row, dout row and Delta = dout . out
  const long long qoff = ((static_cast<long long>(b) * d.T + i) * d.Hq + hq) * BD;
  frag qf[2], dof[2];
  float delta = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    qf[ks] = qvalid ? TT::load8(static_cast<const T*>(a.q) + qoff + ks * 32 + grp * 8) : TT::zero();
    dof[ks] = qvalid ? TT::load8(static_cast<const T*>(a.dout) + qoff + ks * 32 + grp * 8) : TT::zero();
    const frag of = qvalid ? TT::load8(static_cast<const T*>(a.out) + qoff + ks * 32 + grp * 8) : TT::zero();
#pragma unroll
    for (int e = 0; e < 8; ++e) delta += TT::to_f(dof[ks][e]) * TT::to_f(of[e]);
  }
  delta = xor_sum_groups(delta);

  // phi(q): kept as operand fragments through the key loops (the NP-Map forward is
  // recomputed for its backward at the end, which keeps the loops' registers low)
  frag phf[2];
  float dla = 0.f;  // the linear-attention part of the normaliser
  {
    NpRow nq;
    np_forward<T>(nq, W, qf);
    f32x4 phq[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) phq[fb][e] = nq.r * nq.m[fb][e] * nq.inv_nm;
    phf[0] = pk_frag<T>(phq[0], phq[1]);
    phf[1] = pk_frag<T>(phq[2], phq[3]);
    if (c >= 2) {  // state part: phi(q) . z_c
      const float* zc = a.ustate + (bh * d.nC + c) * BR + BF * BD;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dla += phq[fb][e] * zc[fb * 16 + 4 * grp + e];
    }
  }

  const uint64_t sel_prev = chunk_sel(a.sel_idx, bh, c - 1, d);
  const int nsel_c = c >= 2 ? (c - 1) * d.topk : 0;  // compact rows of chunks <= c-2
  const T* ksel = static_cast<const T*>(a.ksel) + bh * a.ntiles * 64 * BD;
  const T* vsel = static_cast<const T*>(a.vsel) + bh * a.ntiles * 64 * BD;
  const T* kselt = static_cast<const T*>(a.kselt) + bh * a.ntiles * (BD * 64);
  const float* st = a.ustate + (bh * d.nC + c) * BR;  // S_c, z_c
  const long long krs = static_cast<long long>(d.Hkv) * BD;


  // ---- one pass over the keys. The softmax part of dq accumulates sum 2^{a - m} (dP - Delta) k
  // against a running reference m (log2 units; moved up only when a score passes it by more
  // than kLazy2, the accumulator rescaled then), the linear-attention part of dphi(q)
  // accumulates sum (dP - Delta) phi(k) unscaled, and both are divided by the normaliser
  // once it is known, at the end. Scores are raw q.k, the scale folded into the exponent's fma.
  constexpr float kLazy2 = 8.f;
  float m2 = -kInf, l_lane = 0.f;  // this lane's share of the softmax part of the normaliser / 2^m
  f32x4 dqt[4] = {}, dpt[4] = {};
  auto rebase = [&](const f32x4 (&sc)[4], const bool (&sa)[4][4], bool masked) {
    float tm = -kInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) tm = (!masked || sa[kb][e]) ? fmaxf(tm, sc[kb][e]) : tm;
    tm = xor_max_groups(tm) * scale2;
    const bool move = tm > m2 + kLazy2;  // the same in the four lanes of a query
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float mn = move ? tm : m2;
      const float alpha = mn == m2 ? 1.f : __builtin_amdgcn_exp2f(m2 - mn);
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) dqt[db] *= alpha;
      m2 = mn;
    }
  };
  // the compact tiles arrive by buffer -> LDS copies, one tile ahead; rows at or beyond
  // nsel_c read as zeros (the copies' range ends there)
  using Dma = DmaTile<T, 64, 64, 4 * NH>;
  Dma dma;
  dma.init(64);
  constexpr int ES = static_cast<int>(sizeof(T));
  const int ntc = (nsel_c + 63) / 64;
  const auto rs_k = make_rsrc(ksel, static_cast<uint32_t>(nsel_c * BD * ES));
  const auto rs_v = make_rsrc(vsel, static_cast<uint32_t>(nsel_c * BD * ES));
  const auto rs_kt = make_rsrc(kselt, static_cast<uint32_t>(ntc * BD * 64 * ES));
  auto issue3 = [&](int t) {
    const int sl = (t & 1) * 3;
    dma.issue(lds[sl], rs_k, t * 64 * BD * ES);
    dma.issue(lds[sl + 1], rs_v, t * 64 * BD * ES);
    dma.issue(lds[sl + 2], rs_kt, t * BD * 64 * ES);
  };
  if (ntc > 0) issue3(0);
  for (int t = 0; t < ntc; ++t) {
    if (t + 1 < ntc) {
      issue3(t + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * Dma::PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    lds_sync();
    const int nv = min(64, nsel_c - t * 64);
    const int sl = (t & 1) * 3;
    f32x4 s[4], dp[4];
    rows_x_frag<T>(s, lds[sl], qf);
    rows_x_frag<T>(dp, lds[sl + 1], dof);
    bool sa[4][4];
    if (nv == 64) {  // a full tile
      rebase(s, sa, false);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale2, -m2));
          ps += p;
          s[kb][e] = p * (dp[kb][e] - delta);
        }
      l_lane += ps;
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[kb][e] = kb * 16 + 4 * grp + e < nv;
      rebase(s, sa, true);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = sa[kb][e] ? __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale2, -m2)) : 0.f;
          l_lane += p;
          s[kb][e] = p * (dp[kb][e] - delta);
        }
    }
    rows_x_acc<T>(dqt, lds[sl + 2], s);
    lds_sync();
  }
  Dma dkv;  // key and value rows of the input, row stride Hkv * D
  dkv.init(static_cast<int>(krs));
  for (int cc = c >= 1 ? c - 1 : 0; cc <= c; ++cc) {
    __syncthreads();
    const long long r0 = (static_cast<long long>(b) * d.T + 64LL * cc) * d.Hkv + h;
    const int nv = min(64, d.T - 64 * cc);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * krs + BD) * ES);
    dkv.issue(t_k, make_rsrc(static_cast<const T*>(a.k) + r0 * BD, rows_b), 0);
    dkv.issue(t_v, make_rsrc(static_cast<const T*>(a.v) + r0 * BD, rows_b), 0);
    dma.issue(t_kt, make_rsrc(static_cast<const T*>(a.kt) + (bh * d.nC + cc) * BD * 64, BD * 64 * ES), 0);
    dma.issue(t_pk, make_rsrc(static_cast<const T*>(a.phik) + (bh * d.nC * 64 + 64LL * cc) * BF, 64 * BF * ES), 0);
    dma.issue(t_pkt, make_rsrc(static_cast<const T*>(a.phikt) + (bh * d.nC + cc) * BF * 64, BF * 64 * ES), 0);
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    lds_sync();
    f32x4 s[4], dp[4], lw[4];
    rows_x_frag<T>(s, t_k, qf);
    rows_x_frag<T>(dp, t_v, dof);
    rows_x_frag<T>(lw, t_pk, phf);
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
    rebase(s, sa, true);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = sa[kb][e] ? __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale2, -m2)) : 0.f;
        const float g = dp[kb][e] - delta;
        l_lane += p;
        dla += la[kb][e] ? lw[kb][e] : 0.f;
        s[kb][e] = p * g;
        lw[kb][e] = la[kb][e] ? g : 0.f;
      }
    rows_x_acc<T>(dqt, t_kt, s);
    rows_x_acc<T>(dpt, t_pkt, lw);
  }
  const float l = xor_sum_groups(l_lane);
  dla = xor_sum_groups(dla);
  float L2;
  if (!qvalid) {
    L2 = kInf;
  } else if (l > 0.f && dla > 0.f) {
    const float ld = log2f(dla);
    const float M = fmaxf(m2, ld);
    L2 = M + log2f(l * exp2f(m2 - M) + exp2f(ld - M));
  } else if (l > 0.f) {
    L2 = m2 + log2f(l);
  } else {
    L2 = dla > 0.f ? log2f(dla) : kInf;  // an empty normaliser: out = 0, no gradient
  }
  const float einv = exp2f(-L2);
  const float sa_scale = l > 0.f ? exp2f(m2 - L2) : 0.f;  // 2^m / normaliser
#pragma unroll
  for (int db = 0; db < 4; ++db) dqt[db] *= sa_scale;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) dpt[fb] *= einv;
  if (c >= 2) {
    // dphi(q) += e^{-L} (S_c dout - Delta z_c)
    f32x4 sdo[4] = {};
    f32rows_x_frag<T>(sdo, st, dof);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dpt[fb][e] += einv * (sdo[fb][e] - delta * st[BF * BD + fb * 16 + 4 * grp + e]);
  }

  // ---- NP-Map backward and dq
  NpRow nq;
  np_forward<T>(nq, W, qf);
  f32x4 phq[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int e = 0; e < 4; ++e) phq[fb][e] = nq.r * nq.m[fb][e] * nq.inv_nm;
  const float dr = np_backward(nq, dpt);  // dpt now holds dz
  __syncthreads();
  load_wt<T>(t_k, W);
  __syncthreads();
  f32x4 dxt[4] = {};
  rows_x_acc<T>(dxt, t_k, dpt);  // dxt[db][e] = (W^T dz)[16 db + 4 grp + e]
  if (qvalid) {
    T* dq = static_cast<T*>(a.dq) + qoff;
    const T* xq = static_cast<const T*>(a.q) + qoff;
    const float xs = nq.r > 0.f ? dr / nq.r : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const typename TT::quad x4 = TT::load4(xq + db * 16 + 4 * grp);
      typename TT::quad o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = TT::from_f(dqt[db][e] * 0.125f + dxt[db][e] + xs * TT::to_f(x4[e]));
      *reinterpret_cast<typename TT::quad*>(dq + db * 16 + 4 * grp) = o4;
    }
  }

  // ---- what the key side needs: (L, Delta), phi(q) rows and transposed, q^T, dout^T
  const long long qc = bhq * d.nC + c;
  if (grp == 0) {
    a.ld[(bhq * d.nC * 64 + 64LL * c + qrow) * 2] = L2;
    a.ld[(bhq * d.nC * 64 + 64LL * c + qrow) * 2 + 1] = qvalid ? delta : 0.f;
  }
  // phi(q) rows and phi(q)^T are stored times e^{-L}, the factor every key-side use takes
  T* phqr = static_cast<T*>(a.phiq) + (bhq * d.nC * 64 + 64LL * c + qrow) * BF;
  {
    f32x4 ps4[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) ps4[fb] = phq[fb] * einv;
    TT::store8(phqr + 8 * grp, pk_frag<T>(ps4[0], ps4[1]));
    TT::store8(phqr + 32 + 8 * grp, pk_frag<T>(ps4[2], ps4[3]));
  }
  T* phqt = static_cast<T*>(a.phiqt) + qc * BF * 64;
  T* qt = static_cast<T*>(a.qt) + qc * BD * 64;
  T* dot = static_cast<T*>(a.dot) + qc * BD * 64;
  const int pq = pk_pos(qrow);
  T* const e_phq = lds[4 * hs];      // e^{-L} phi(q)^T of this head
  T* const e_do = lds[4 * hs + 1];   // dout^T
  T* const e_dz = lds[4 * hs + 2];   // dz^T
  T* const e_q = lds[4 * hs + 3];    // q^T
  __syncthreads();  // slot 0 (W^T) is reused below
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int f = fb * 16 + 4 * grp + e;
      e_phq[SW::off(f, pq)] = TT::from_f(phq[fb][e] * einv);
      e_dz[SW::off(f, pq)] = TT::from_f(dpt[fb][e]);
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dd = ks * 32 + grp * 8 + e;
      e_do[SW::off(dd, pq)] = dof[ks][e];
      e_q[SW::off(dd, pq)] = qf[ks][e];
    }
  // a_c partial: sum over the head's 64 queries of e^{-L} Delta phi(q)
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = xor_sum_16(phq[fb][e] * einv * (qvalid ? delta : 0.f));
      if (r16 == 0) s_red[hs][wl][fb * 16 + 4 * grp + e] = v;
    }
  __syncthreads();
  // the transposed tiles to memory in 16-byte pieces
  for (int idx = tid & 255; idx < 512; idx += 256) {
    const int row = idx >> 3, col = (idx & 7) * 8;
    TT::store8(phqt + row * 64 + col, SW::load8(e_phq, row, col));
    TT::store8(qt + row * 64 + col, SW::load8(e_q, row, col));
    TT::store8(dot + row * 64 + col, SW::load8(e_do, row, col));
  }
  float* ap = a.apart + qc * BR;
  if (wl == 0)
    ap[BF * BD + lane] = ((s_red[hs][0][lane] + s_red[hs][1][lane]) + s_red[hs][2][lane]) + s_red[hs][3][lane];
  f32x4 acc[4];
  tile_x_tile<T>(acc, e_phq, e_do);  // A_c[f][d] = sum_q e^{-L} phi(q)[f] dout[d]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) ap[(wl * 16 + 4 * grp + e) * BD + cb * 16 + r16] = acc[cb][e];
  tile_x_tile<T>(acc, e_dz, e_q);  // dW[f][d] = sum_q dz[f] q[d]
  float* wp = a.dwq + qc * (BF * BD);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) wp[(wl * 16 + 4 * grp + e) * BD + cb * 16 + r16] = acc[cb][e];
}

// ---------------------------------------------------------------------------------------
// Selected keys against the queries of chunks >= their chunk + 2. A workgroup of eight
// waves takes 128 compact rows (16 per wave) and one of gridDim.y slices of the query
// chunks; it writes fp32 partial dk, dv (softmax part, before the 1/sqrt(D) of dk). The
// query-side tiles (q rows, dout rows, q^T, dout^T) arrive by buffer -> LDS copies one
// (chunk, head) step ahead, with that step's (L, Delta) prefetched into registers.
template <typename T>
__global__ __launch_bounds__(512, 2) void bwd_dkv_far_kernel(BwdArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using Dma = DmaTile<T, 64, 64, 8>;
  constexpr int ES = static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(16))) T lds[2][4][64 * 64];  // [buffer][q, dout, q^T, dout^T]
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
  const float scale2 = kLog2e * 0.125f;
  const int nsel = d.nCc * d.topk;
  const int row0 = grp_id * 128;
  const int n = row0 + wave * 16 + r16;  // this lane column's compact row
  const bool nin = n < a.ntiles * 64;     // inside the buffers (rows past nsel are zeros)
  const int ckey = n < nsel ? n / d.topk : 0x3fffffff;
  frag kf[2], vf[2];
  {
    const T* kr = static_cast<const T*>(a.ksel) + (bh * a.ntiles * 64 + n) * BD;
    const T* vr = static_cast<const T*>(a.vsel) + (bh * a.ntiles * 64 + n) * BD;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
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
  Dma dma;
  dma.init(64);
  Dma dmq;
  dmq.init(d.Hq * BD);
  const long long hq0 = static_cast<long long>(b) * d.Hq + static_cast<long long>(h) * d.G;  // b*Hq + first head
  auto step_ptrs = [&](int st, long long& qc, long long& r0, int& nv) {
    const int cq = __builtin_amdgcn_readfirstlane(cb0 + st / d.G), g = __builtin_amdgcn_readfirstlane(st % d.G);
    qc = (hq0 + g) * d.nC + cq;
    r0 = ((static_cast<long long>(b) * d.T + 64LL * cq) * d.Hq + h * d.G + g) * BD;
    nv = min(64, d.T - 64 * cq);
  };
  auto issue = [&](int st) {
    long long qc, r0;
    int nv;
    step_ptrs(st, qc, r0, nv);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * d.Hq * BD + BD) * ES);
    T* dst = lds[st & 1][0];
    dmq.issue(dst, make_rsrc(static_cast<const T*>(a.q) + r0, rows_b), 0);
    dmq.issue(dst + 64 * 64, make_rsrc(static_cast<const T*>(a.dout) + r0, rows_b), 0);
    dma.issue(dst + 2 * 64 * 64, make_rsrc(static_cast<const T*>(a.qt) + qc * BD * 64, BD * 64 * ES), 0);
    dma.issue(dst + 3 * 64 * 64, make_rsrc(static_cast<const T*>(a.dot) + qc * BD * 64, BD * 64 * ES), 0);
  };
  auto ld_of = [&](int st) {  // this thread's (L, Delta) entry of step st
    long long qc, r0;
    int nv;
    step_ptrs(st, qc, r0, nv);
    return a.ld[qc * 128 + (tid & 127)];
  };
  f32x4 dkt[4] = {}, dvt[4] = {};
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
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(4 * Dma::PER_WAVE + 1));
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
    rows_x_frag<T>(s, tq, kf);  // s[qb][e] = q[16 qb + 4 grp + e] . k
    rows_x_frag<T>(dp, tdo, vf);
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
    rows_x_acc<T>(dvt, tdot, dp);
    rows_x_acc<T>(dkt, tqt, s);
    lds_sync();
  }
  if (nin) {
    float* out = a.dkvsel + ((static_cast<long long>(split) * d.B * d.Hkv + bh) * a.ntiles * 64 + n) * (2 * BD);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      *reinterpret_cast<f32x4*>(out + db * 16 + 4 * grp) = dkt[db];
      *reinterpret_cast<f32x4*>(out + BD + db * 16 + 4 * grp) = dvt[db];
    }
  }
}

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dkv_local_kernel(BwdArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, 64>;
  using Dma = DmaTile<T, 64, 64, 4>;
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int NBUF = sizeof(T) == 2 ? kLocalBuffers : 1;
  // per step: q rows, dout rows, q^T, dout^T, phi(q) rows, phi(q)^T of one (head, chunk)
  __shared__ __attribute__((aligned(16))) T lds[NBUF][6][64 * 64];
  __shared__ __attribute__((aligned(16))) float s_ld[NBUF][2][64];  // [buffer][L, Delta][query]
  T* const t_q = lds[0][0];
  T* const t_do = lds[0][1];
  T* const t_qt = lds[0][2];
  const Dims& d = a.d;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const float scale2 = kLog2e * 0.125f;
  const int jr = wave * 16 + r16;
  const long long j = 64LL * c + jr;  // this lane column's key
  const bool kvalid = j < d.T;
  const uint64_t selm = chunk_sel(a.sel_idx, bh, c, d);
  const bool selj = (selm >> jr) & 1ull;
  const T* W = static_cast<const T*>(a.w) + static_cast<long long>(h) * BF * BD;
  const long long koff = ((static_cast<long long>(b) * d.T + j) * d.Hkv + h) * BD;
  frag kf[2], vf[2], phk[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    kf[ks] = kvalid ? TT::load8(static_cast<const T*>(a.k) + koff + ks * 32 + grp * 8) : TT::zero();
    vf[ks] = kvalid ? TT::load8(static_cast<const T*>(a.v) + koff + ks * 32 + grp * 8) : TT::zero();
    phk[ks] = TT::load8(static_cast<const T*>(a.phik) + (bh * d.nC * 64 + j) * BF + ks * 32 + grp * 8);
  }
  f32x4 dkt[4] = {}, dvt[4] = {}, dpk[4] = {};
  // steps over (query head g, query chunk cq in {c, c+1}); the tiles arrive by
  // buffer -> LDS copies, one step ahead when two buffers fit
  const int ncq = c + 1 < d.nC ? 2 : 1;
  const int nsteps = d.G * ncq;
  Dma dma, dmq;
  dma.init(64);
  dmq.init(d.Hq * BD);
  auto step_of = [&](int st, long long& hq, int& cq) {
    hq = static_cast<long long>(b) * d.Hq + h * d.G + __builtin_amdgcn_readfirstlane(st / ncq);  // b*Hq + query head
    cq = c + __builtin_amdgcn_readfirstlane(st % ncq);
  };
  auto issue = [&](int st) {
    long long hq;
    int cq;
    step_of(st, hq, cq);
    const long long qc = hq * d.nC + cq;
    const long long r0 = ((static_cast<long long>(b) * d.T + 64LL * cq) * d.Hq + (hq - static_cast<long long>(b) * d.Hq)) * BD;
    const int nv = min(64, d.T - 64 * cq);
    const uint32_t rows_b = static_cast<uint32_t>(((nv - 1) * d.Hq * BD + BD) * ES);
    T(*dst)[64 * 64] = lds[st % NBUF];
    dmq.issue(dst[0], make_rsrc(static_cast<const T*>(a.q) + r0, rows_b), 0);
    dmq.issue(dst[1], make_rsrc(static_cast<const T*>(a.dout) + r0, rows_b), 0);
    dma.issue(dst[2], make_rsrc(static_cast<const T*>(a.qt) + qc * BD * 64, BD * 64 * ES), 0);
    dma.issue(dst[3], make_rsrc(static_cast<const T*>(a.dot) + qc * BD * 64, BD * 64 * ES), 0);
    dma.issue(dst[4], make_rsrc(static_cast<const T*>(a.phiq) + qc * 64 * BF, 64 * BF * ES), 0);
    dma.issue(dst[5], make_rsrc(static_cast<const T*>(a.phiqt) + qc * BF * 64, BF * 64 * ES), 0);
  };
  auto ld_of = [&](int st) {
    long long hq;
    int cq;
    step_of(st, hq, cq);
    return a.ld[(hq * d.nC + cq) * 128 + (tid & 127)];
  };
  float ldn = ld_of(0);
  if (NBUF == 2) issue(0);
  for (int st = 0; st < nsteps; ++st) {
    const float ldc = ldn;
    if (NBUF == 2) {
      if (st + 1 < nsteps) {
        ldn = ld_of(st + 1);
        issue(st + 1);
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(6 * Dma::PER_WAVE + 1));
      } else {
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      }
    } else {
      issue(st);
      if (st + 1 < nsteps) ldn = ld_of(st + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    if (tid < 128) s_ld[st % NBUF][tid & 1][tid >> 1] = ldc;
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    lds_sync();
    long long hq;
    int cq;
    step_of(st, hq, cq);
    T(*cur)[64 * 64] = lds[st % NBUF];
    {
      f32x4 s[4], dp[4], lw[4];
      rows_x_frag<T>(s, cur[0], kf);
      rows_x_frag<T>(dp, cur[1], vf);
      rows_x_frag<T>(lw, cur[4], phk);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const f32x4 lq = *reinterpret_cast<const f32x4*>(&s_ld[st % NBUF][0][qb * 16 + 4 * grp]);
        const f32x4 dq4 = *reinterpret_cast<const f32x4*>(&s_ld[st % NBUF][1][qb * 16 + 4 * grp]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qr = qb * 16 + 4 * grp + e;
          const int dist = 64 * (cq - c) + qr - jr;  // i - j
          const bool vis = dist >= 0;
          const bool inwin = dist < d.window;
          const bool sel = cq > c && selj;
          const bool sa = vis && (inwin || sel);
          const bool la = vis && !(inwin || sel);
          const float L2 = lq[e], dl = dq4[e];
          const float p = sa ? __builtin_amdgcn_exp2f(fmaf(s[qb][e], scale2, -L2)) : 0.f;
          const float gg = dp[qb][e] - dl;
          s[qb][e] = p * gg;                    // dS
          dp[qb][e] = p + (la ? lw[qb][e] : 0.f);  // weight of v_j in out_i (phi(q) carries e^{-L})
          lw[qb][e] = la ? gg : 0.f;            // g / e^{-L}
        }
      }
      rows_x_acc<T>(dvt, cur[3], dp);
      rows_x_acc<T>(dkt, cur[2], s);
      rows_x_acc<T>(dpk, cur[5], lw);
    }
    lds_sync();
  }
  // queries of chunks >= c+2 through R_c, r_c (unselected keys only)
  if (c + 2 < d.nC) {
    const float* rs = a.rstate + (bh * d.nC + c) * BR;
    f32x4 rv[4] = {};
    f32rows_x_frag<T>(rv, rs, vf);  // (R v)[16 fb + 4 grp + e]
    __syncthreads();
    for (int e = tid; e < BF * BD; e += 256) {  // R^T, features pk-permuted
      const int f = e >> 6, dd = e & 63;
      t_q[SW::off(dd, pk_pos(f))] = TT::from_f(rs[e]);
    }
    __syncthreads();
    const float on = (kvalid && !selj) ? 1.f : 0.f;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dpk[fb][e] += on * (rv[fb][e] - rs[BF * BD + fb * 16 + 4 * grp + e]);
    frag pm[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pm[ks][e] = TT::from_f(on * TT::to_f(phk[ks][e]));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) TT::mma(dvt[db], SW::load8(t_q, db * 16 + r16, ks * 32 + grp * 8), pm[ks]);
  }
  // selected keys: the later chunks' softmax part from the compact partials
  if (selj && kvalid) {
    const int32_t* sp = a.sel_idx + (bh * d.nCc + c) * d.topk;
    int rank = 0;
    for (int r = 0; r < d.topk; ++r) rank += (sp[r] - 64 * c) < jr ? 1 : 0;
    const int n = c * d.topk + rank;
    for (int sidx = 0; sidx < a.nsplit; ++sidx) {
      const float* p = a.dkvsel + ((static_cast<long long>(sidx) * d.B * d.Hkv + bh) * a.ntiles * 64 + n) * (2 * BD);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dkt[db] += *reinterpret_cast<const f32x4*>(p + db * 16 + 4 * grp);
        dvt[db] += *reinterpret_cast<const f32x4*>(p + BD + db * 16 + 4 * grp);
      }
    }
  }
  // NP-Map backward and dk, dv
  NpRow nk;
  np_forward<T>(nk, W, kf);
  const float dr = np_backward(nk, dpk);  // dpk now holds dz
  __syncthreads();
  load_wt<T>(t_q, W);
  __syncthreads();
  f32x4 dxt[4] = {};
  rows_x_acc<T>(dxt, t_q, dpk);
  if (kvalid) {
    T* dk = static_cast<T*>(a.dk) + koff;
    T* dv = static_cast<T*>(a.dv) + koff;
    const T* xk = static_cast<const T*>(a.k) + koff;
    const float xs = nk.r > 0.f ? dr / nk.r : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const typename TT::quad x4 = TT::load4(xk + db * 16 + 4 * grp);
      typename TT::quad o4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o4[e] = TT::from_f(dkt[db][e] * 0.125f + dxt[db][e] + xs * TT::to_f(x4[e]));
        v4[e] = TT::from_f(dvt[db][e]);
      }
      *reinterpret_cast<typename TT::quad*>(dk + db * 16 + 4 * grp) = o4;
      *reinterpret_cast<typename TT::quad*>(dv + db * 16 + 4 * grp) = v4;
    }
  }
  // dW (k side) of the chunk: sum over its keys of dz k^T
  __syncthreads();
  const int pj = pk_pos(jr);
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int e = 0; e < 4; ++e) t_do[SW::off(fb * 16 + 4 * grp + e, pj)] = TT::from_f(kvalid ? dpk[fb][e] : 0.f);
  tile_load<T>(t_qt, static_cast<const T*>(a.kt) + (bh * d.nC + c) * BD * 64, 64, 64);
  __syncthreads();
  f32x4 acc[4];
  tile_x_tile<T>(acc, t_do, t_qt);
  float* wp = a.dwk + (bh * d.nC + c) * (BF * BD);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) wp[(wave * 16 + 4 * grp + e) * BD + cb * 16 + r16] = acc[cb][e];
}

// ---------------------------------------------------------------------------------------
// dW = sum over batch, chunks and the group's query heads (q side) plus keys (k side):
// gridDim.y slices of the item list, then a fixed-order sum of the slices.
__global__ __launch_bounds__(256) void bwd_dw_part_kernel(const float* dwq, const float* dwk, float* part, int B,
                                                          int Hkv, int G, int nC) {
  const int e = blockIdx.x * 256 + threadIdx.x;  // over Hkv * F * D
  const int h = e / (BF * BD), fd = e % (BF * BD);
  const int nq = B * G * nC, nitems = nq + B * nC;
  const int per = (nitems + gridDim.y - 1) / gridDim.y;
  const int i0 = blockIdx.y * per, i1 = min(nitems, i0 + per);
  float acc = 0.f;
  constexpr int U = 8;  // loads of U items in flight together
  for (int it0 = i0; it0 < i1; it0 += U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u;
      x[u] = 0.f;
      if (it < i1) {
        if (it < nq) {
          const int b = it / (G * nC), g = (it / nC) % G, c = it % nC;
          x[u] = dwq[((static_cast<long long>(b) * Hkv * G + h * G + g) * nC + c) * (BF * BD) + fd];
        } else {
          const int it2 = it - nq, b = it2 / nC, c = it2 % nC;
          x[u] = dwk[((static_cast<long long>(b) * Hkv + h) * nC + c) * (BF * BD) + fd];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += x[u];
  }
  part[static_cast<long long>(blockIdx.y) * Hkv * BF * BD + e] = acc;
}

__global__ __launch_bounds__(256) void bwd_dw_sum_kernel(const float* part, float* dw, int n, int nparts) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float acc = 0.f;
  for (int p = 0; p < nparts; ++p) acc += part[static_cast<long long>(p) * n + e];
  dw[e] = acc;
}

// ---------------------------------------------------------------------------------------
template <typename T>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  const Dims& d = a.d;
  hipError_t e;
  auto mark = [&](int k) { return ev ? hipEventRecord(ev[k], s) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  if (a.ntiles > 0) {
    const size_t tb = static_cast<size_t>(d.B) * d.Hkv * a.ntiles * 64 * BD * sizeof(T);
    if ((e = launch_fill_zero(a.kselt, tb, s)) != hipSuccess) return e;
    if ((e = launch_fill_zero(a.ksel, tb, s)) != hipSuccess) return e;
    if ((e = launch_fill_zero(a.vsel, tb, s)) != hipSuccess) return e;
  }
  const dim3 gk(d.nC, d.Hkv, d.B);
  hipLaunchKernelGGL(bwd_kprep_kernel<T>, gk, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
  const long long ne = static_cast<long long>(d.B) * d.Hkv * BR;
  const dim3 gs(static_cast<unsigned>((ne + 255) / 256));
  hipLaunchKernelGGL(bwd_scan_fwd_kernel, gs, dim3(256), 0, s, a.ustate, d.nC, ne);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  if (kDqHeads == 2 && sizeof(T) == 2 && d.G % 2 == 0)
    hipLaunchKernelGGL((bwd_dq_kernel<T, 2>), dim3(d.nC * (d.Hq / 2) * d.B), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, 1>), dim3(d.nC * d.Hq * d.B), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  {
    const int nseg = (d.nC + kRevSeg - 1) / kRevSeg;
    const long long nr = ne * nseg;
    const dim3 gr(static_cast<unsigned>((nr + 255) / 256));
    hipLaunchKernelGGL(bwd_rev_seg_kernel, gr, dim3(256), 0, s, a.apart, a.segsum, d.nC, d.G, d.Hkv, nseg, nr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_rev_scan_kernel, gr, dim3(256), 0, s, a.apart, a.segsum, a.rstate, d.nC, d.G, d.Hkv, nseg,
                       nr);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(4)) != hipSuccess) return e;
  }
  if (a.ntiles > 0) {
    hipLaunchKernelGGL(bwd_dkv_far_kernel<T>, dim3((a.ntiles + 1) / 2 * a.nsplit * d.B * d.Hkv), dim3(512), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(5)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_local_kernel<T>, gk, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(6)) != hipSuccess) return e;
  const int nw = d.Hkv * BF * BD;
  hipLaunchKernelGGL(bwd_dw_part_kernel, dim3(nw / 256, a.dw_parts), dim3(256), 0, s, a.dwq, a.dwk, a.dwpart, d.B,
                     d.Hkv, d.G, d.nC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dw_sum_kernel, dim3((nw + 255) / 256), dim3(256), 0, s, a.dwpart, a.dw, nw, a.dw_parts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(7);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s, hipEvent_t* events) {
  return a.d.bf16 ? launch_bwd_t<bf16>(a, s, events) : launch_bwd_t<float>(a, s, events);
}

}  // namespace still

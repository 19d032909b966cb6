// Per-chunk preparation kernels of the STILL prefill, plus the standalone top-k and
// NP-Map kernels.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h.)
//
// prep_kernel, one workgroup per (chunk c, batch b, routing head rh), four waves; the routing
// head is the KV head (selection per KV head) or a query head (selection per query head), and
// its keys and values are those of KV head h = rh * Gr / G:
//   1. stage the key band of chunks c-L .. c in LDS (L = band_chunks(window));
//   2. Self-Saliency Score of the chunk's 64 tokens for each query head the routing head
//      serves, summed over them in head order ([P1] section "Self-Saliency Score");
//   3. NP-Map of the chunk's keys ([P1] section "Norm-Preserved Feature Map（NP-Map）");
//   4. top-k routing of a complete chunk, ascending positions, and the gather of the
//      selected K/V rows into the compact softmax cache ([P1] section
//      "Chunk-Wise并行+延迟选择"), stored as they are (the consumers scale the
//      fp32 scores);
//   5. the chunk's linear-attention contribution U_c = sum over its unselected keys of
//      phi(k) v^T and u_c = sum phi(k) ([P3] on the fixed-size state of linear attention).
// scan_kernel then turns the U_c into inclusive prefix sums over chunks.
#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"

namespace still {

// Workgroups per CU the registers are sized for: at D = d_f = 64 in bf16 the kernel fits
// in 76 registers, so six share a CU (LDS allows eight) and the 2048 workgroups of a 16K
// layer need few waves of dispatch; at head_dim 128 three (LDS allows four).
template <typename T, int D, int DF, int L>
__global__ __launch_bounds__(256, (D == 64 && DF == 64 && sizeof(T) == 2) ? 6 : (D == 128 ? 3 : 1))
void prep_kernel(PrepArgs a) {
  constexpr int FPW = DF / 64;
  constexpr int V8 = D / 8;
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, D>;

  // key band: chunks c-L .. c and one zero row; bandc (chunks c-1 and c, then the zero row)
  // is also where the gather, the NP-Map of the chunk and the V staging work
  __shared__ __attribute__((aligned(16))) T band[(64 * L + 65) * D];
  T* const bandc = band + 64 * (L - 1) * D;
  __shared__ float s_part[4][64];
  __shared__ float s_acc[64];
  __shared__ float m2part[4 * 64];
  __shared__ float xn2[64];
  __shared__ int selpos[64];
  __shared__ uint64_t s_mask;

  const Dims& d = a.d;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* w = static_cast<const T*>(a.w);
  // work item: (chunk c, (b, routing head) record bh). Workgroups go to the eight XCDs in turn,
  // so a one-dimensional grid takes the records in groups of eight (record fastest, then the
  // chunk, then the group): every chunk of a record runs on the same XCD, right after the
  // chunk before it, whose key rows (the band's chunk c-1) are then still in that XCD's L2.
  // A record count that is not a multiple of 8 takes the chunks outermost; a grid too large
  // for one dimension is launched as (chunks, records).
  const int BHn = d.B * d.Hr;
  int c, bh;
  if (gridDim.y != 1) {
    c = static_cast<int>(blockIdx.x);
    bh = static_cast<int>(blockIdx.y);
  } else if (BHn % 8 == 0) {
    const int per = d.nC * 8, id = static_cast<int>(blockIdx.x);
    c = (id % per) / 8;
    bh = (id / per) * 8 + id % 8;
  } else {
    c = static_cast<int>(blockIdx.x) / BHn;
    bh = static_cast<int>(blockIdx.x) % BHn;
  }
  const int b = bh / d.Hr, rh = bh % d.Hr, h = rh * d.Gr / d.G;
  // phi(K) and V^T depend on the KV head alone: the first routing head of each KV head writes them
  const long long bkv = static_cast<long long>(b) * d.Hkv + h;
  const bool kv_writer = (rh * d.Gr) % d.G == 0;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets addresses stay scalar
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const bool complete = nvalid == kChunk;
  const float scale = kLog2e / sqrtf(static_cast<float>(D));  // saliency logits in log2 units

  // 0. global reads issued up front so their latencies overlap the band and saliency work:
  //    the NP-Map weights and the chunk's V rows
  frag wf[DF / 64][D / 32];
  np_map_load_w<T, D, DF>(w + static_cast<long long>(h) * DF * D, wf);
  constexpr int VPT = 64 * V8 / 256;  // V pieces per thread
  frag vpre[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * 256, row = idx / V8, c8 = idx % V8;
    vpre[i] = row < nvalid ? TT::load8(v + ((b * T_ + t0 + row) * d.Hkv + h) * D + c8 * 8) : TT::zero();
  }

  // 1. key band: row t <-> position t0 - 64 L + t, rows 64 (L - l) .. 64 (L - l) + 63 chunk
  //    c-l, rows 64 L .. 64 L + 63 chunk c, copied straight into LDS (rows outside the
  //    sequence read as zeros); row 64 L + 64 (the position after the chunk, never in a
  //    window) is zero
  {
    const int kvs = d.Hkv * D;
#pragma unroll
    for (int l = L; l >= 1; --l)
      dma_tile<T, D, 64, 4>(band + 64 * (L - l) * D, k + ((b * T_ + (c >= l ? t0 - l * kChunk : t0)) * d.Hkv + h) * D,
                            kvs, c >= l ? 64 : 0);
    dma_tile<T, D, 64, 4>(band + 64 * L * D, k + ((b * T_ + t0) * d.Hkv + h) * D, kvs, nvalid);
    if (tid < V8) SW::store8(band, 64 * L + 64, tid * 8, TT::zero());
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 2. saliency, summed over the group in head order g = 0..G-1
  if (d.window >= 1) {
    for (int g0 = 0; g0 < d.Gr; g0 += 4) {
      const int g = g0 + wave;
      if (g < d.Gr) {
        const int hq = rh * d.Gr + g;
        // queries of block qb (rows past the sequence end read as zeros), one block ahead
        const auto qrs = make_rsrc(q + ((b * T_ + t0) * d.Hq + hq) * D,
                                   static_cast<uint32_t>(((nvalid - 1) * d.Hq + 1) * D * static_cast<int>(sizeof(T))));
        auto qload = [&](int qb, frag (&qf)[D / 32]) {
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks)
            qf[ks] = TT::bload8(qrs, ((qb * 16 + r16) * d.Hq * D + ks * 32 + grp * 8) * static_cast<int>(sizeof(T)), 0);
        };
        frag qcur[D / 32];
        qload(0, qcur);
#pragma unroll 1
        for (int qb = 0; qb < 4; ++qb) {
          frag qf[D / 32];
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) qf[ks] = qcur[ks];
          if (qb < 3) qload(qb + 1, qcur);
          const float sv = saliency_qblock<T, D, L>(band, qf, qb, d.window, t0 - 64 * L + 1, scale, 1, d.score);
          if (grp == 0) s_part[wave][qb * 16 + r16] = sv;
        }
      }
      __syncthreads();
      if (wave == 0) {
        float acc = g0 == 0 ? 0.f : s_acc[lane];
        const int nw = d.Gr - g0 < 4 ? d.Gr - g0 : 4;
        for (int w2 = 0; w2 < nw; ++w2) acc += s_part[w2][lane];
        s_acc[lane] = acc;
      }
      __syncthreads();
    }
    if (tid < nvalid) a.sal[(static_cast<long long>(bh)) * T_ + t0 + tid] = s_acc[tid];
  }

  // 3. NP-Map of the chunk's keys (bandc rows 64..127)
  f32x4 phi[4][FPW];
  np_map_rows64<T, D, DF>(bandc, 64, wf, m2part, xn2, phi);

  // 4. routing of a complete chunk
  const long long nsel_rows = static_cast<long long>(d.nCc) * d.topk;
  if (wave == 0) {
    uint64_t m = 0;
    if (complete && d.topk > 0) {
      if (a.routing_in) {
        uint64_t bit = 0;
        if (lane < d.topk) {
          const long long p = a.routing_in[(static_cast<long long>(bh) * d.nCc + c) * d.topk + lane] - t0;
          if (p >= 0 && p < kChunk) bit = 1ull << p;
        }
        m = or_reduce_u64(bit);
      } else {
        m = topk_mask(s_acc[lane], d.topk);
      }
    }
    // the largest key norm among the selected keys (xn2 holds |k|^2 of the chunk's rows)
    const float kn = wave_max64(((m >> lane) & 1ull) ? xn2[lane] : 0.f);
    const float ka = wave_max64(xn2[lane]);  // every key of the chunk (rows past the end are zero)
    if (lane == 0) {
      s_mask = m;
      a.selmask[static_cast<long long>(bh) * d.nC + c] = m;
      a.kmaxc[static_cast<long long>(bh) * d.nC + c] = sqrtf(kn);
      a.kall[static_cast<long long>(bh) * d.nC + c] = sqrtf(ka);
    }
    if ((m >> lane) & 1ull) {
      const int slot = __popcll(m & ((1ull << lane) - 1ull));
      selpos[slot] = lane;
      if (a.sel_idx) a.sel_idx[(static_cast<long long>(bh) * d.nCc + c) * d.topk + slot] = static_cast<int>(t0 + lane);
    }
  }
  __syncthreads();
  const uint64_t smask = s_mask;
  if (complete && d.topk > 0) {
    const int nsel = __popcll(smask);
    T* ks_ = static_cast<T*>(a.ksel);
    for (int idx = tid; idx < d.topk * V8; idx += 256) {
      const int slot = idx / V8, c8 = idx % V8;
      const long long dst =
          (static_cast<long long>(bh) * a.ntiles_sel * 64 + static_cast<long long>(c) * d.topk + slot) * D + c8 * 8;
      frag kx = TT::zero();
      if (slot < nsel) kx = SW::load8(bandc, 64 + selpos[slot], c8 * 8);  // the chunk's rows are bandc rows 64..127
      TT::store8(ks_ + dst, kx);  // raw rows: the logit scale is applied to the fp32 scores
    }
  }

  // 5. store phi(k) (rounded to T, features permuted by pk_pos); keep the rounded values
  //    of unselected keys for U_c
  T* phik = static_cast<T*>(a.phik);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kb * 16 + 4 * grp + i;
        const int f = (wave * FPW + fi) * 16 + r16;
        const T val = TT::from_f(phi[kb][fi][i]);
        if (row < nvalid && kv_writer) phik[(bkv * T_ + t0 + row) * DF + pk_pos(f)] = val;
        phi[kb][fi][i] = ((smask >> row) & 1ull) ? 0.f : TT::to_f(val);
      }

  // 6. V of the chunk (loaded at the start; zero past the sequence end): stage in LDS over
  //    bandc rows 0..63 once the gather is done with the band, transpose it into bandc rows
  //    64..127 as V^T [d][64] (a Swz<T, 64> tile, keys permuted: position 8*pb + e holds
  //    key 32*(pb/4) + 16*(e/4) + 4*(pb%4) + e%4, the order MFMA operands take), then write
  //    that tile out as vT and the compact transposed copy of the selected rows
  using SV = Swz<T, 64>;
  T* vtl = bandc + 64 * D;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * 256;
    SW::store8(bandc, idx / V8, (idx % V8) * 8, vpre[i]);
  }
  __syncthreads();
  for (int idx = tid; idx < D * 8; idx += 256) {
    const int dd = idx / 8, pb = idx % 8;  // positions 8*pb .. 8*pb+7 of row dd
    frag x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bandc[SW::off(32 * (pb / 4) + 16 * (e / 4) + 4 * (pb % 4) + (e % 4), dd)];
    SV::store8(vtl, dd, pb * 8, x);
  }
  __syncthreads();
  {
    T* vt = static_cast<T*>(a.vT) + (bkv * d.nC + c) * D * 64;
    if (kv_writer)
      for (int idx = tid; idx < D * 8; idx += 256) {
        const int dd = idx / 8, pb = idx % 8;
        TT::store8(vt + dd * 64 + pb * 8, SV::load8(vtl, dd, pb * 8));
      }
    if (complete && d.topk > 0) {
      T* vs = static_cast<T*>(a.vselT) + static_cast<long long>(bh) * a.ntiles_sel * D * 64;
      const int nsel = __popcll(smask);
      // The chunk's compact rows r0 .. r0 + topk - 1, by 4-aligned groups: the 4 rows of a
      // group sit at 4 consecutive columns (pk_pos keeps k & 3), so a lane writes one piece of
      // up to 4 elements of one V^T row, and the lanes of a row are adjacent. Rows of a group
      // that belong to a neighbouring chunk are left alone.
      const long long r0 = static_cast<long long>(c) * d.topk;
      const long long g_lo = r0 / 4;
      const int ng = static_cast<int>((r0 + d.topk - 1) / 4 - g_lo) + 1;
      for (int idx = tid; idx < ng * D; idx += 256) {
        const int gi = idx % ng, dd = idx / ng;
        const long long r4 = 4 * (g_lo + gi);  // first compact row of the group
        typename TT::quad x;
        bool all = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long long slot = r4 + j - r0;
          all = all && slot >= 0 && slot < d.topk;
          x[j] = slot >= 0 && slot < nsel ? bandc[SW::off(selpos[slot], dd)] : TT::from_f(0.f);
        }
        T* dst = vs + ((r4 / 64) * D + dd) * 64 + pk_pos(static_cast<int>(r4 % 64));
        if (all) {
          *reinterpret_cast<typename TT::quad*>(dst) = x;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const long long slot = r4 + j - r0;
            if (slot >= 0 && slot < d.topk) dst[j] = x[j];
          }
        }
      }
      // the last compact tile's unused columns are zero (they meet zero weights)
      const long long n_rows = nsel_rows;
      if (c == d.nCc - 1 && (n_rows % 64) != 0) {
        const long long tl = n_rows / 64;
        const int used = static_cast<int>(n_rows % 64);
        for (int idx = tid; idx < (64 - used) * D; idx += 256) {
          const int col = used + idx / D, dd = idx % D;
          vs[(tl * D + dd) * 64 + pk_pos(col)] = TT::from_f(0.f);
        }
      }
    }
  }

  // 7. U_c = phi_masked^T V_c and u_c, for complete chunks. Stored transposed with the
  //    features permuted, S^T[d][pk_pos(f)], then u[pk_pos(f)]: the layout the attention
  //    kernel feeds to MFMA straight from memory.
  if (!complete) return;  // uniform across the workgroup
  f32x4 u[FPW][D / 16];  // u[fi][db][i] = U[f = (wave*FPW + fi)*16 + 4*grp + i][d = db*16 + r16]
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) u[fi][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    frag pa[FPW];  // A operand: row f, keys of the 32-key slice in accumulator order
#pragma unroll
    for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[fi][e] = TT::from_f(phi[2 * ks + e / 4][fi][e % 4]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      // B operand: column d, the same keys (keys ks*32 + 16*(e/4) + 4*grp + e%4 sit at
      // positions ks*32 + 8*grp + e of the permuted V^T tile)
      const frag vb = SV::load8(vtl, db * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
      for (int fi = 0; fi < FPW; ++fi) TT::mma(u[fi][db], pa[fi], vb);
    }
  }
  T* st = static_cast<T*>(a.states) + (static_cast<long long>(bh) * d.nC + c) * d.R;
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi) {
    const int fb = wave * FPW + fi;
    // features fb*16 + 4*grp + 0..3 sit at 4 consecutive permuted positions
    const int pos = fb / 2 * 32 + 8 * grp + 4 * (fb & 1);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      typename TT::quad qv;
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = TT::from_f(u[fi][db][i]);
      *reinterpret_cast<typename TT::quad*>(st + (db * 16 + r16) * DF + pos) = qv;
    }
    float zs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) zs += phi[kb][fi][i];
    zs = xor_sum_groups(zs);
    if (grp == 0) st[DF * D + pk_pos(fb * 16 + r16)] = TT::from_f(zs);
  }
}

// Inclusive prefix sum of the chunk records over the complete chunks, in place, summed in
// fp32 and stored in the layer's dtype. A workgroup takes 64 32-bit words of the records
// (one per lane: one fp32 or two bf16 elements) of one (b, h) and 8 waves; a round covers
// 8 x SEG chunks, wave w the SEG chunks from SEG w on (SEG = 8, 16 or 32, the smallest that
// covers the sequence in one round, up to 32): each lane loads its SEG words at once (one
// memory round trip per round), scans them in registers, and adds the totals of the earlier
// segments (through LDS) and of the earlier rounds (a running carry). The last block column
// instead reduces the per-chunk selected-key norms to one bound per compact tile (tile t
// holds compact rows 64t .. 64t+63, i.e. chunks 64t/topk .. (64t+63)/topk).
constexpr int kScanWaves = 8;
template <typename T>
__device__ __forceinline__ void unpack_word(uint32_t u, float (&x)[4 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    x[0] = __uint_as_float(u << 16);  // bf16 -> fp32 is exact
    x[1] = __uint_as_float(u & 0xffff0000u);
  } else {
    x[0] = __uint_as_float(u);
  }
}
template <typename T>
__device__ __forceinline__ uint32_t pack_word(const float (&x)[4 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, Tr<T>::from_f(x[0]));
    const uint32_t hi = __builtin_bit_cast(uint16_t, Tr<T>::from_f(x[1]));
    return lo | (hi << 16);
  } else {
    return __float_as_uint(x[0]);
  }
}

template <typename T, int kScanSeg>
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(void* states, int nC, int nCc, int R,
                                                               const float* kmaxc, float* tilemax, int tm_stride,
                                                               int topk) {
  constexpr int EPW = 4 / static_cast<int>(sizeof(T));  // elements per word
  const long long bh = blockIdx.y;
  if (tm_stride > 0 && static_cast<int>(blockIdx.x) == static_cast<int>(gridDim.x) - 1) {
    for (int t = threadIdx.x; t < tm_stride; t += 64 * kScanWaves) {
      const int c0 = 64 * t / topk;
      const int c1 = min((64 * t + 63) / topk, nCc - 1);
      float mx = 0.f;
      for (int cc = c0; cc <= c1; ++cc) mx = fmaxf(mx, kmaxc[bh * nC + cc]);
      tilemax[bh * tm_stride + t] = mx;
    }
    return;
  }
  __shared__ float tot[2][kScanWaves][64 * EPW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int rw = R / EPW;  // words per record (R is even)
  const int wd = blockIdx.x * 64 + lane;
  const bool ok = wd < rw;
  const int rec = R * static_cast<int>(sizeof(T));  // bytes per record
  // the complete chunks' records of this (b, h): reads past them give zeros, writes past
  // them are dropped; lanes past the record (wd >= rw) read but never write
  const auto rs = make_rsrc(static_cast<char*>(states) + bh * nC * rec, static_cast<uint32_t>(nCc) * static_cast<uint32_t>(rec));
  float carry[EPW];
#pragma unroll
  for (int e = 0; e < EPW; ++e) carry[e] = 0.f;
  int par = 0;
  for (int r0 = 0; r0 < nCc; r0 += kScanWaves * kScanSeg, par ^= 1) {
    const int c0 = r0 + wave * kScanSeg;  // this wave's first chunk
    float x[kScanSeg][EPW];
#pragma unroll
    for (int j = 0; j < kScanSeg; ++j)
      unpack_word<T>(__builtin_amdgcn_raw_buffer_load_b32(rs, (c0 + j) * rec + wd * 4, 0, 0), x[j]);
#pragma unroll
    for (int j = 1; j < kScanSeg; ++j)
#pragma unroll
      for (int e = 0; e < EPW; ++e) x[j][e] += x[j - 1][e];
#pragma unroll
    for (int e = 0; e < EPW; ++e) tot[par][wave][lane * EPW + e] = x[kScanSeg - 1][e];
    __syncthreads();
    float before[EPW];
#pragma unroll
    for (int e = 0; e < EPW; ++e) {
      float bsum = carry[e], all = carry[e];
#pragma unroll
      for (int w = 0; w < kScanWaves; ++w) {
        const float t = tot[par][w][lane * EPW + e];
        bsum += w < wave ? t : 0.f;
        all += t;
      }
      before[e] = bsum;
      carry[e] = all;
    }
    if (ok) {
#pragma unroll
      for (int j = 0; j < kScanSeg; ++j) {
        float y[EPW];
#pragma unroll
        for (int e = 0; e < EPW; ++e) y[e] = x[j][e] + before[e];
        __builtin_amdgcn_raw_buffer_store_b32(pack_word<T>(y), rs, (c0 + j) * rec + wd * 4, 0, 0);
      }
    }
  }
}

// Standalone per-chunk top-k: one wave per (complete chunk, batch, KV head).
__global__ __launch_bounds__(64) void topk_kernel(const float* sal, int32_t* sel_idx, int T, int nCc, int topk) {
  const int c = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const uint64_t m = topk_mask(sal[static_cast<long long>(bh) * T + t0 + lane], topk);
  if ((m >> lane) & 1ull) {
    const int slot = __popcll(m & ((1ull << lane) - 1ull));
    sel_idx[(static_cast<long long>(bh) * nCc + c) * topk + slot] = static_cast<int>(t0 + lane);
  }
}

// Standalone NP-Map: one workgroup per (64-row tile of positions, batch, KV head).
template <typename T, int D, int DF>
__global__ __launch_bounds__(256) void feature_map_kernel(Dims d, const void* xv, const void* wv, float* phi_out) {
  constexpr int FPW = DF / 64;
  constexpr int V8 = D / 8;
  using TT = Tr<T>;
  __shared__ __attribute__((aligned(16))) T rows[64 * D];
  __shared__ float m2part[4 * 64];
  __shared__ float xn2[64];
  const T* x = static_cast<const T*>(xv);
  const T* w = static_cast<const T*>(wv);
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const long long T_ = d.T, t0 = static_cast<long long>(c) * 64;
  typename Tr<T>::frag wf[DF / 64][D / 32];
  np_map_load_w<T, D, DF>(w + static_cast<long long>(h) * DF * D, wf);
  for (int idx = tid; idx < 64 * V8; idx += 256) {
    const int row = idx / V8, c8 = idx % V8;
    typename TT::frag val = TT::zero();
    if (t0 + row < T_) val = TT::load8(x + ((b * T_ + t0 + row) * d.Hkv + h) * D + c8 * 8);
    Swz<T, D>::store8(rows, row, c8 * 8, val);
  }
  __syncthreads();
  f32x4 phi[4][FPW];
  np_map_rows64<T, D, DF>(rows, 0, wf, m2part, xn2, phi);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kb * 16 + 4 * grp + i;
        const int f = (wave * FPW + fi) * 16 + r16;
        if (t0 + row < T_) phi_out[((b * T_ + t0 + row) * d.Hkv + h) * DF + f] = phi[kb][fi][i];
      }
}

// ------------------------------------------------------------------------ launchers

template <typename T, int D, int DF>
static hipError_t prep_t(const PrepArgs& a, hipStream_t s) {
  // one dimension (records fastest) while its work-item count fits 32 bits
  const long long items = static_cast<long long>(a.d.nC) * a.d.B * a.d.Hr;
  const dim3 grid = items * 256 < (1LL << 32) ? dim3(static_cast<unsigned>(items)) : dim3(a.d.nC, a.d.B * a.d.Hr);
  static_assert(kMaxBand == 2, "one prep instantiation per band length");
  if (band_chunks(a.d.window) == 1)
    hipLaunchKernelGGL((prep_kernel<T, D, DF, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((prep_kernel<T, D, DF, 2>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int DF>
static hipError_t fmap_t(const Dims& d, const void* x, const void* w, float* phi, hipStream_t s) {
  dim3 grid(d.nC, d.B * d.Hkv);
  hipLaunchKernelGGL((feature_map_kernel<T, D, DF>), grid, dim3(256), 0, s, d, x, w, phi);
  return hipGetLastError();
}

bool shape_supported(int, int D, int DF) { return (D == 64 || D == 128) && (DF == 64 || DF == 128); }

#define STILL_DISPATCH(FN, ...)                                                   \
  do {                                                                            \
    const Dims& dd_ = (DIMS);                                                     \
    if (dd_.bf16) {                                                               \
      if (dd_.D == 64 && dd_.DF == 64) return FN<bf16, 64, 64>(__VA_ARGS__);      \
      if (dd_.D == 64 && dd_.DF == 128) return FN<bf16, 64, 128>(__VA_ARGS__);    \
      if (dd_.D == 128 && dd_.DF == 64) return FN<bf16, 128, 64>(__VA_ARGS__);    \
      if (dd_.D == 128 && dd_.DF == 128) return FN<bf16, 128, 128>(__VA_ARGS__);  \
    } else {                                                                      \
      if (dd_.D == 64 && dd_.DF == 64) return FN<float, 64, 64>(__VA_ARGS__);     \
      if (dd_.D == 64 && dd_.DF == 128) return FN<float, 64, 128>(__VA_ARGS__);   \
      if (dd_.D == 128 && dd_.DF == 64) return FN<float, 128, 64>(__VA_ARGS__);   \
      if (dd_.D == 128 && dd_.DF == 128) return FN<float, 128, 128>(__VA_ARGS__); \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
#define DIMS a.d
  STILL_DISPATCH(prep_t, a, s);
#undef DIMS
}

hipError_t launch_feature_map(const Dims& d, const void* x, const void* w, float* phi, hipStream_t s) {
#define DIMS d
  STILL_DISPATCH(fmap_t, d, x, w, phi, s);
#undef DIMS
}

hipError_t launch_scan(const Dims& d, void* states, const float* kmaxc, float* tilemax, int tm_stride,
                       hipStream_t s) {
  if (d.nCc == 0) return hipSuccess;
  const bool tiles = d.topk > 0 && tm_stride > 0;
  const int words = d.bf16 ? d.R / 2 : d.R;
  dim3 grid((words + 63) / 64 + (tiles ? 1 : 0), d.B * d.Hr);
  const int tms = tiles ? tm_stride : 0, tk = d.topk > 0 ? d.topk : 1;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), 0, s, states, d.nC, d.nCc, d.R, kmaxc, tilemax, tms, tk);
  };
  const int seg = d.nCc <= 8 * kScanWaves ? 8 : d.nCc <= 16 * kScanWaves ? 16 : 32;
  if (d.bf16)
    go(seg == 8 ? scan_kernel<bf16, 8> : seg == 16 ? scan_kernel<bf16, 16> : scan_kernel<bf16, 32>);
  else
    go(seg == 8 ? scan_kernel<float, 8> : seg == 16 ? scan_kernel<float, 16> : scan_kernel<float, 32>);
  return hipGetLastError();
}

hipError_t launch_topk(const Dims& d, const float* sal, int32_t* sel_idx, hipStream_t s) {
  if (d.nCc == 0 || d.topk == 0) return hipSuccess;
  dim3 grid(d.nCc, d.B * d.Hr);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(64), 0, s, sal, sel_idx, d.T, d.nCc, d.topk);
  return hipGetLastError();
}

}  // namespace still

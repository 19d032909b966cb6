// Saliency, per-chunk top-k and NP-Map device routines.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h.)
//
// The prefill kernels and the decode kernel call exactly these functions, so a token's
// saliency (and hence every routing decision) is bit-identical whichever path computed it.
#pragma once

#include "still_common.hpp"

namespace still {

constexpr int kChunk = 64;


// Self-Saliency Score of 16 queries of one query head
// ([P1] section "Self-Saliency Score"; [P4] section Approach).
//
// `band` holds 64 (L + 1) key rows (a Swz<T, D> tile), L = band_chunks(window): band row t is
// the key at position band_pos0 + t, with band_pos0 = chunk_start - 64 L + 1 (rows outside the
// sequence are zero and masked here); it is stored at LDS tile row t + row_base (row_base 0
// or 1, so a tile that starts one position earlier can be used as is).
// Query r of the chunk (its position is chunk_start + r) sits at band row r + 64 L - 1, so
// its window is band rows [r + 64 L - w, r + 64 L - 1]. qf holds the B-operand (SK) fragments
// of the queries qb*16 .. qb*16+15 (lane r16 <-> query qb*16 + r16). The result does not
// depend on L beyond the window's reach (rows outside the window add nothing, and a lane
// holds the same positions whatever L), so every caller gets the same bits.
//
// For query i (logits in log2 units, scale = log2(e)/sqrt(D)): M' = max over the window
// without i, Z' = sum over the window without i of
// e^{a - M'}, and s_i = LSE(W_i) - LSE(W_i \ i) = softplus(a_ii - M' - log Z'), which is
// +inf when i is alone in its window. Returned in every lane of the query's column.
// With score = 1 the routing score is the diagonal logit alone, q_i . k_i / sqrt(D) in
// natural units ([P4] section "Surprising findings": routing by the diagonal attention).
template <typename T, int D, int L = 1>
__device__ __forceinline__ float saliency_qblock(const T* band, const typename Tr<T>::frag (&qf)[D / 32],
                                                 int qb, int window, long long band_pos0, float scale,
                                                 int row_base = 0, int score = 0) {
  constexpr int NJ = 4 * L + 1;  // 16-row key blocks from the query block's window start to its diagonal
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const typename Tr<T>::frag a = Swz<T, D>::load8(band, (qb + j) * 16 + r16 + row_base, ks * 32 + grp * 8);
      Tr<T>::mma(acc[j], a, qf[ks]);
    }
  }
  const int r = qb * 16 + r16;
  const int diag = r + 64 * L - 1;
  if (score == 1) {
    float dr = -kInf;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((qb + j) * 16 + 4 * grp + i == diag) dr = acc[j][i];
    return xor_max_groups(dr) * (1.0f / sqrtf(static_cast<float>(D)));
  }
  // logits in log2 units: scale = log2(e) / sqrt(D)
  if (L == 1 && window == 64 && band_pos0 >= 0) {
    // The window is the 63 rows before the diagonal, all inside the sequence: element (j, i)
    // of the lane's query sits at offset 16 j + e_i from the window's first row, with
    // e_i = 4 grp + i - r16 in [-15, 15]. Blocks 1 and 2 lie inside the window; block 0 holds
    // rows before it (e_i < 0), block 3 the diagonal (e_i = 15) and block 4 the diagonal
    // (e_i = -1) and rows after it (e_i >= 0). Rows outside the window become -inf, so the
    // max and the sum need no further masks (the same values and order as the general path).
    float dr = -kInf, mr = -kInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * grp + i - r16;
      if (e == 15) dr = acc[3][i];
      if (e == -1) dr = acc[4][i];
      if (e < 0) acc[0][i] = -kInf;
      if (e == 15) acc[3][i] = -kInf;
      if (e >= -1) acc[4][i] = -kInf;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mr = fmaxf(mr, acc[j][i]);
    const float mx = xor_max_groups(mr) * scale;  // max of the scaled logits (scale > 0)
    const float dg = xor_max_groups(dr) * scale;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) z += __builtin_amdgcn_exp2f(acc[j][i] * scale - mx);
    z = xor_sum_groups(z);
    const float x = dg - mx - __builtin_amdgcn_logf(z);
    const float sp = fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x)));
    return sp * 0.69314718055994531f;
  }
  const int lo = max(r + 64 * L - window, static_cast<int>(-band_pos0));  // first window row inside the sequence
  float mx = -kInf, dg = -kInf;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (qb + j) * 16 + 4 * grp + i;
      const float a = acc[j][i] * scale;
      if (row == diag) dg = a;
      if (row >= lo && row < diag) mx = fmaxf(mx, a);
    }
  mx = xor_max_groups(mx);
  dg = xor_max_groups(dg);
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (qb + j) * 16 + 4 * grp + i;
      if (row >= lo && row < diag) z += __builtin_amdgcn_exp2f(acc[j][i] * scale - mx);
    }
  z = xor_sum_groups(z);
  // s = ln(1 + 2^x), x = dg - mx - log2 z (log2 units): softplus via exp2 / log2
  if (!(z > 0.f)) return kInf;
  const float x = dg - mx - __builtin_amdgcn_logf(z);
  const float sp = fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x)));
  return sp * 0.69314718055994531f;
}

// Top-k of one chunk ([P1] section "Chunk-Wise并行+延迟选择"): lane p holds the routing
// score of chunk position p (any float but NaN; +inf sorts first). A bitonic sort of the
// 64-bit keys (order-preserving score bits, 63 - p) in descending order leaves rank j in
// lane j; the first topk ranks are returned as a position bit mask. Equal scores sort the
// lower position first. Every lane of the wave must call.
__device__ __forceinline__ uint64_t topk_mask(float s, int topk) {
  const int lane = threadIdx.x & 63;
  // fp32 bits ordered as unsigned integers: negative values flipped, the sign bit set on the rest
  const uint32_t u = __float_as_uint(s);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  uint64_t key = (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(63 - lane);
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(key, j);
      const bool desc = (lane & kk) == 0;
      const bool lower = (lane & j) == 0;
      key = (lower == desc) ? (key > o ? key : o) : (key < o ? key : o);
    }
  const int p = 63 - static_cast<int>(key & 63);
  return or_reduce_u64(lane < topk ? (1ull << p) : 0ull);
}

// NP-Map of 64 rows ([P1] section "Norm-Preserved Feature Map（NP-Map）"; [P4] section
// Approach): phi(x) = |x| m / |m|, m = elu(W_h x) + 1.
//
// rows: rows row0 .. row0+63 of a Swz<T, D> LDS tile. wf: this wave's W_h fragments from
// np_map_load_w. Four waves; wave w owns feature blocks fb = w*FPW + fi (FPW = DF/64). On return
// phi[kb][fi][i] = phi(row kb*16 + 4*grp + i)[feature fb*16 + r16] in fp32.
// Scratch in LDS: m2part[4*64], xn2[64]. Contains two __syncthreads(); all 256 threads
// must call. After it returns no thread reads `rows` again.
// The W_h fragments np_map_rows64 needs (B operand: feature column fb*16 + r16 of wave w's
// feature blocks), loaded ahead of time so their latency can overlap other work.
template <typename T, int D, int DF>
__device__ __forceinline__ void np_map_load_w(const T* Wh, typename Tr<T>::frag (&wf)[DF / 64][D / 32]) {
  constexpr int FPW = DF / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      wf[fi][ks] = Tr<T>::load8(Wh + ((wave * FPW + fi) * 16 + r16) * D + ks * 32 + grp * 8);
}

template <typename T, int D, int DF>
__device__ __forceinline__ void np_map_rows64(const T* rows, int row0, const typename Tr<T>::frag (&wf)[DF / 64][D / 32],
                                              float* m2part, float* xn2, f32x4 (&phi)[4][DF / 64]) {
  constexpr int FPW = DF / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
  {
    // |x|^2 of each row: four lanes per row, D/4 elements each, then a sum over the four
    const int row = tid >> 2, part = tid & 3;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const auto x = Swz<T, D>::load8(rows, row0 + row, part * (D / 4) + j * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = Tr<T>::to_f(x[e]);
        s += v * v;
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) xn2[row] = s;
  }
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const typename Tr<T>::frag a = Swz<T, D>::load8(rows, row0 + kb * 16 + r16, ks * 32 + grp * 8);
        Tr<T>::mma(acc, a, wf[fi][ks]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zv = acc[i];
        acc[i] = zv > 0.f ? zv + 1.f : __builtin_amdgcn_exp2f(zv * kLog2e);  // elu(z) + 1
      }
      phi[kb][fi] = acc;
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p = 0.f;
#pragma unroll
      for (int fi = 0; fi < FPW; ++fi) p += phi[kb][fi][i] * phi[kb][fi][i];
      p = xor_sum_16(p);
      if (r16 == 0) m2part[wave * 64 + kb * 16 + 4 * grp + i] = p;
    }
  __syncthreads();
  // the rescale |x| / |phi(x)| of each row, once per row, left in m2part[0..63]
  if (tid < 64) {
    const float m2 = ((m2part[tid] + m2part[64 + tid]) + m2part[128 + tid]) + m2part[192 + tid];
    m2part[tid] = norm_ratio(xn2[tid], m2);
  }
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = m2part[kb * 16 + 4 * grp + i];
#pragma unroll
      for (int fi = 0; fi < FPW; ++fi) phi[kb][fi][i] *= sc;
    }
}

}  // namespace still

// 64 x 64 tile helpers shared by the backward and the attention-mass kernels (gfx950,
// wave64, 16x16x32 MFMA with the operand conventions of still_common.hpp).
#pragma once

#include "still_common.hpp"
#include "still_layout.hpp"

namespace still {

// index k (0..63) stored at position p = pk_pos(k) of a pk-permuted 64-vector
__device__ __forceinline__ int pk_index(int p) {
  const int s = p & ~31, q = p & 31, g = q >> 3, e = q & 7;
  return s + 16 * (e >> 2) + 4 * g + (e & 3);
}

// Operand fragment from two accumulators (the PK assignment of still_common.hpp): the
// elements 0..3 come from the block of rows 32s..32s+15, 4..7 from rows 32s+16..32s+31.
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag pk_frag(const f32x4& lo, const f32x4& hi) {
  typename Tr<T>::frag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = Tr<T>::from_f(lo[e]);
    f[4 + e] = Tr<T>::from_f(hi[e]);
  }
  return f;
}

// eight consecutive fp32 values as an operand fragment of dtype T
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag f32_frag(const float* p) {
  return pk_frag<T>(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4));
}

// 64 rows of 64 elements from memory (row stride `stride` elements) into a Swz<T, 64> LDS
// tile; rows at or beyond nvalid are zero. All threads of the workgroup call.
template <typename T>
__device__ __forceinline__ void tile_load(T* lds, const T* g, long long stride, int nvalid) {
  for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
    const int row = idx >> 3, col = (idx & 7) * 8;
    const typename Tr<T>::frag x = row < nvalid ? Tr<T>::load8(g + row * stride + col) : Tr<T>::zero();
    Swz<T, 64>::store8(lds, row, col, x);
  }
}

// acc[blk] = tile rows blk*16 + r16 (k = the 64 columns, straight) times the B fragments
template <typename T>
__device__ __forceinline__ void rows_x_frag(f32x4 (&acc)[4], const T* tile, const typename Tr<T>::frag (&bf)[2]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    acc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Tr<T>::mma(acc[blk], Swz<T, 64>::load8(tile, blk * 16 + r16, ks * 32 + grp * 8), bf[ks]);
  }
}

// acc[blk] += tile rows blk*16 + r16 (k = 64 pk-permuted positions) times the PK operand
// built from the accumulators v[0..3] (rows 0..63 of a previous product)
template <typename T>
__device__ __forceinline__ void rows_x_acc(f32x4 (&acc)[4], const T* tile, const f32x4 (&v)[4]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  const typename Tr<T>::frag b0 = pk_frag<T>(v[0], v[1]);
  const typename Tr<T>::frag b1 = pk_frag<T>(v[2], v[3]);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    Tr<T>::mma(acc[blk], Swz<T, 64>::load8(tile, blk * 16 + r16, grp * 8), b0);
    Tr<T>::mma(acc[blk], Swz<T, 64>::load8(tile, blk * 16 + r16, 32 + grp * 8), b1);
  }
}

// acc[blk] += rows blk*16 + r16 of a row-major fp32 [64][64] matrix in memory (k = the 64
// columns, straight) times the B fragments
template <typename T>
__device__ __forceinline__ void f32rows_x_frag(f32x4 (&acc)[4], const float* m, const typename Tr<T>::frag (&bf)[2]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Tr<T>::mma(acc[blk], f32_frag<T>(m + (blk * 16 + r16) * 64 + ks * 32 + grp * 8), bf[ks]);
}

// One 64x64 output of a workgroup-wide product over 64 pk-permuted positions:
// out[row][col] = sum_p A[row][p] B[col][p], A and B Swz<T, 64> tiles. Wave w computes rows
// 16w..16w+15 (w = wave % 4); returns acc[cb][i] = out[16w + 4grp + i][16cb + r16].
template <typename T>
__device__ __forceinline__ void tile_x_tile(f32x4 (&acc)[4], const T* A, const T* B) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4, wave = (threadIdx.x >> 6) & 3;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      Tr<T>::mma(acc[cb], Swz<T, 64>::load8(A, wave * 16 + r16, ks * 32 + grp * 8),
                 Swz<T, 64>::load8(B, cb * 16 + r16, ks * 32 + grp * 8));
  }
}

// s_waitcnt immediate (gfx9 encoding) that waits for vector memory only, until at most n
// operations of this wave are outstanding
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// s_waitcnt immediate that waits for LDS (and scalar memory) only
constexpr int kLgkmWait0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// workgroup barrier; the waits for memory are the caller's, and no LDS access moves across it
__device__ __forceinline__ void lds_sync() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Work index of workgroup L out of n: the hardware deals workgroups to the eight XCDs in
// turn (L on XCD L % 8), so consecutive work indices, which share data, are given to
// workgroups of one XCD and meet in its L2.
__device__ __forceinline__ int xcd_work(int L, int n) {
  const int per = n >> 3, rem = n & 7, x = L & 7, slot = L >> 3;
  return x * per + min(x, rem) + slot;
}

}  // namespace still

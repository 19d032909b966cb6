// Tile helpers shared by the backward and the attention-mass kernels (gfx950, wave64,
// 16x16x32 MFMA with the operand conventions of still_common.hpp): 64-row tiles whose row
// length (head or feature width) is a template parameter, products that read each LDS
// fragment once for several operand sets, and the copy-wait and barrier primitives.
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

// ROWS rows of RL elements from memory (row stride `stride` elements) into a Swz<T, RL> LDS
// tile; rows at or beyond nvalid are zero. All threads of the workgroup call.
template <typename T, int RL = 64, int ROWS = 64>
__device__ __forceinline__ void tile_load(T* lds, const T* g, long long stride, int nvalid) {
  constexpr int PPR = RL / 8;  // 8-element pieces per row
  for (int idx = threadIdx.x; idx < ROWS * PPR; idx += blockDim.x) {
    const int row = idx / PPR, col = (idx % PPR) * 8;
    const typename Tr<T>::frag x = row < nvalid ? Tr<T>::load8(g + row * stride + col) : Tr<T>::zero();
    Swz<T, RL>::store8(lds, row, col, x);
  }
}

// acc[blk] = rows blk*16 + r16 of a 64-row Swz<T, RL> tile (k = its RL columns, straight)
// times the B fragments bf[RL / 32]
template <typename T, int RL = 64>
__device__ __forceinline__ void rows_x_frag(f32x4 (&acc)[4], const T* tile, const typename Tr<T>::frag (&bf)[RL / 32]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    acc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RL / 32; ++ks)
      Tr<T>::mma(acc[blk], Swz<T, RL>::load8(tile, blk * 16 + r16, ks * 32 + grp * 8), bf[ks]);
  }
}

// acc[blk] += rows blk*16 + r16 of an NB*16-row Swz<T, NPOS> tile (k = its NPOS pk-permuted
// positions) times the PK operands built from the accumulators v[NPOS / 16] (rows 0..NPOS-1
// of a previous product)
template <typename T, int NB = 4, int NPOS = 64>
__device__ __forceinline__ void rows_x_acc(f32x4 (&acc)[NB], const T* tile, const f32x4 (&v)[NPOS / 16]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  typename Tr<T>::frag b[NPOS / 32];
#pragma unroll
  for (int s2 = 0; s2 < NPOS / 32; ++s2) b[s2] = pk_frag<T>(v[2 * s2], v[2 * s2 + 1]);
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int s2 = 0; s2 < NPOS / 32; ++s2)
      Tr<T>::mma(acc[blk], Swz<T, NPOS>::load8(tile, blk * 16 + r16, s2 * 32 + grp * 8), b[s2]);
}

// rows_x_frag for NG sets of B fragments at once: acc[g][blk] = rows blk*16 + r16 of the tile
// times bf[g]; every A fragment is read from LDS once and serves all NG sets
template <typename T, int RL, int NG>
__device__ __forceinline__ void rows_x_frags(f32x4 (&acc)[NG][4], const T* tile,
                                             const typename Tr<T>::frag (&bf)[NG][RL / 32]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RL / 32; ++ks) {
      const typename Tr<T>::frag af = Swz<T, RL>::load8(tile, blk * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
      for (int g = 0; g < NG; ++g) Tr<T>::mma(acc[g][blk], af, bf[g][ks]);
    }
  }
}

// rows_x_acc for NG sets of accumulators at once: acc[g][blk] += rows blk*16 + r16 of the
// tile times the PK operands built from v[g]; one LDS read of each A fragment serves all sets
template <typename T, int NB, int NPOS, int NG>
__device__ __forceinline__ void rows_x_accs(f32x4 (&acc)[NG][NB], const T* tile, const f32x4 (&v)[NG][NPOS / 16]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  typename Tr<T>::frag b[NG][NPOS / 32];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int s2 = 0; s2 < NPOS / 32; ++s2) b[g][s2] = pk_frag<T>(v[g][2 * s2], v[g][2 * s2 + 1]);
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int s2 = 0; s2 < NPOS / 32; ++s2) {
      const typename Tr<T>::frag af = Swz<T, NPOS>::load8(tile, blk * 16 + r16, s2 * 32 + grp * 8);
#pragma unroll
      for (int g = 0; g < NG; ++g) Tr<T>::mma(acc[g][blk], af, b[g][s2]);
    }
}

// acc[blk] += rows blk*16 + r16 of a row-major fp32 [NB*16][KC] matrix in memory (k = its KC
// columns, straight) times the B fragments bf[KC / 32]
template <typename T, int NB = 4, int KC = 64>
__device__ __forceinline__ void f32rows_x_frag(f32x4 (&acc)[NB], const float* m, const typename Tr<T>::frag (&bf)[KC / 32]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int ks = 0; ks < KC / 32; ++ks)
      Tr<T>::mma(acc[blk], f32_frag<T>(m + (blk * 16 + r16) * KC + ks * 32 + grp * 8), bf[ks]);
}

// An NR x NC output of a workgroup-wide product over 64 pk-permuted positions:
// out[row][col] = sum_p A[row][p] B[col][p], A (NR rows) and B (NC rows) Swz<T, 64> tiles.
// Wave w (w = wave % 4) computes the row blocks w + 4 rb; returns
// acc[rb][cb][i] = out[16 (w + 4 rb) + 4 grp + i][16 cb + r16].
template <typename T, int NR = 64, int NC = 64>
__device__ __forceinline__ void tile_x_tile(f32x4 (&acc)[NR / 64][NC / 16], const T* A, const T* B) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4, wave = (threadIdx.x >> 6) & 3;
#pragma unroll
  for (int rb = 0; rb < NR / 64; ++rb)
#pragma unroll
    for (int cb = 0; cb < NC / 16; ++cb) {
      acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        Tr<T>::mma(acc[rb][cb], Swz<T, 64>::load8(A, (wave + 4 * rb) * 16 + r16, ks * 32 + grp * 8),
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

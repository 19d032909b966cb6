// Device primitives shared by the STILL kernels (gfx950, wave64).
//
// MFMA convention used everywhere: a "fragment" is 8 elements per lane feeding one
// 16x16x32 contraction step. For lane l, write r16 = l % 16 and grp = l / 16.
//   A operand: row r16 of the 16-row tile, 8 of the 32 k-indices chosen by grp.
//   B operand: column r16 of the 16-column tile, the same 8 k-indices.
//   Accumulator (f32x4): element i holds D[row = 4*grp + i][col = r16].
// Which 8 k-indices a lane group holds only has to agree between A and B, so two
// assignments are used:
//   SK ("straight"):  k = 8*grp + e                        (16-byte contiguous loads)
//   PK ("permuted"):  k = 16*(e/4) + 4*grp + (e%4)          (matches the accumulator
//                     layout of a previous 16x16 product, so a result can be fed back as
//                     an operand without leaving registers)
// bf16 uses one v_mfma_f32_16x16x32_bf16 per step; fp32 uses eight
// v_mfma_f32_16x16x4_f32 (element e of every lane in the e-th instruction), which
// contracts exactly the same index set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace still {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) bf16 bf16x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_huge_valf();

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3); loads through
// it take a 32-bit per-lane offset plus a wave-uniform offset, and read 0 out of range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

template <typename T> struct Tr;

template <> struct Tr<bf16> {
  using frag = bf16x8;
  using quad = bf16x4;
  static __device__ __forceinline__ frag zero() { return frag{}; }
  static __device__ __forceinline__ frag load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static __device__ __forceinline__ quad load4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
  static __device__ __forceinline__ frag bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(frag, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void store8(bf16* p, frag x) { *reinterpret_cast<bf16x8*>(p) = x; }
  static __device__ __forceinline__ frag join(quad lo, quad hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
  static __device__ __forceinline__ bf16 from_f(float x) { return static_cast<bf16>(x); }
};

template <> struct Tr<float> {
  using frag = f32x8;
  using quad = f32x4;
  static __device__ __forceinline__ frag zero() { return frag{}; }
  static __device__ __forceinline__ frag load8(const float* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ quad load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ frag bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ void store8(float* p, frag x) {
    *reinterpret_cast<f32x4*>(p) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    *reinterpret_cast<f32x4*>(p + 4) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ frag join(quad lo, quad hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};

// ---- LDS tiles ----------------------------------------------------------------------
// An LDS tile of rows of RL elements, stored in 16-byte granules whose index is XORed
// with the low bits of the row (granules per row NG; mask 7 for 128-byte rows, 15 for
// 256-byte and longer rows). Sixteen lanes reading one granule column of sixteen rows,
// and lanes writing whole rows, then run at full LDS bandwidth on gfx950 (a padded
// row pitch halves it, an unpadded unswizzled one quarters it: measured).
template <typename T, int RL>
struct Swz {
  static constexpr int EPG = 16 / static_cast<int>(sizeof(T));  // elements per granule
  static constexpr int NG = RL / EPG;                            // granules per row
  static constexpr int MASK = NG >= 16 ? 15 : NG - 1;
  static_assert(RL % EPG == 0 && NG >= 8, "rows must hold at least 8 granules");
  // element offset of (row, col)
  static __device__ __forceinline__ int off(int row, int col) {
    return row * RL + (((col / EPG) ^ (row & MASK)) * EPG) + (col % EPG);
  }
  // 8 consecutive elements starting at a column that is a multiple of 8
  static __device__ __forceinline__ typename Tr<T>::frag load8(const T* base, int row, int col) {
    if constexpr (EPG == 8) {
      return Tr<T>::load8(base + off(row, col));
    } else {
      return Tr<T>::join(Tr<T>::load4(base + off(row, col)), Tr<T>::load4(base + off(row, col + 4)));
    }
  }
  static __device__ __forceinline__ void store8(T* base, int row, int col, const typename Tr<T>::frag& x) {
    if constexpr (EPG == 8) {
      Tr<T>::store8(base + off(row, col), x);
    } else {
      *reinterpret_cast<typename Tr<T>::quad*>(base + off(row, col)) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
      *reinterpret_cast<typename Tr<T>::quad*>(base + off(row, col + 4)) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
    }
  }
};

// Asynchronous copy of a ROWS x RL tile into the Swz<T, RL> LDS tile, straight from memory
// (buffer_load ... lds: no registers hold the data). Row r of the tile is read at byte
// r * gstride * sizeof(T) of the buffer resource, plus a wave-uniform byte offset; reads
// outside the resource's range arrive as zeros. One wave instruction fills 1 KiB of LDS
// (lane l writes byte 16 l), so each lane fetches the granule the swizzle stores in its
// slot. The NW waves of the workgroup split the instructions; the per-lane offsets are
// fixed by the geometry, so init() runs once and issue() is a few scalar ops and the
// copies. The data is visible to the workgroup after s_waitcnt vmcnt and a barrier.
template <typename T, int RL, int ROWS, int NW>
struct DmaTile {
  static constexpr int RB = RL * static_cast<int>(sizeof(T));  // bytes per row
  static constexpr int NGR = RB / 16;                          // 16-byte granules per row
  static constexpr int RPI = 1024 / RB;                        // rows per instruction
  static constexpr int EPG = 16 / static_cast<int>(sizeof(T));
  static constexpr int NINS = ROWS / RPI;                      // instructions per tile
  static constexpr int PER_WAVE = NINS / NW;
  static_assert(RB >= 128 && RB <= 1024 && 1024 % RB == 0 && ROWS % RPI == 0 && NINS % NW == 0, "tile geometry");
  int voff[PER_WAVE];

  __device__ __forceinline__ void init(int gstride) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int row = (wave + i * NW) * RPI + lane / NGR;
      const int g = (lane % NGR) ^ (row & Swz<T, RL>::MASK);
      voff[i] = (row * gstride + g * EPG) * static_cast<int>(sizeof(T));
    }
  }
  __device__ __forceinline__ void issue(T* lds, __amdgpu_buffer_rsrc_t rs, int soff) const {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
#if defined(__HIP_DEVICE_COMPILE__)  // LDS pointers exist only in the device pass
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + (wave + i * NW) * RPI * RL), 16, voff[i], soff, 0, 0);
#else
      (void)lds;
      (void)rs;
      (void)soff;
      (void)wave;
#endif
    }
  }
};

// One-off copy of a tile whose rows at or beyond valid_rows read as zeros.
template <typename T, int RL, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(T* lds, const T* gbase, int gstride, int valid_rows) {
  const uint32_t nrec =
      valid_rows > 0 ? static_cast<uint32_t>(((valid_rows - 1) * gstride + RL) * static_cast<int>(sizeof(T))) : 0u;
  DmaTile<T, RL, ROWS, NW> t;
  t.init(gstride);
  t.issue(lds, make_rsrc(gbase, nrec), 0);
}

// ---- wave64 cross-lane helpers -------------------------------------------------------

// Reductions over the 4 lanes {l, l^16, l^32, l^48} without LDS traffic:
// v_permlane16_swap(x, x) leaves {x[l], x[l^16]} in its two results for every lane l,
// v_permlane32_swap(x, x) leaves {x[l], x[l^32]}; combining the pair reduces one step.
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor_max_groups(float x) { return pair32_max(pair16_max(x)); }

__device__ __forceinline__ float xor_sum_groups(float x) { return pair32_sum(pair16_sum(x)); }

__device__ __forceinline__ float xor_sum_16(float x) {
  // sum over the 16 lanes that share l / 16
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t or_reduce_u64(uint64_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x |= shfl_xor_u64(x, m);
  return x;
}

// Norm ratio sqrt(a) / sqrt(b) with the hardware square root and reciprocal square root
// (about 1 ulp each; the IEEE-exact library forms cost ~40 instructions), 0 if b = 0.
__device__ __forceinline__ float norm_ratio(float a, float b) {
  return b > 0.f ? __builtin_amdgcn_sqrtf(a) * __builtin_amdgcn_rsqf(b) : 0.f;
}

// softplus(x) = log(1 + e^x), stable for any finite x.
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

}  // namespace still

// Head expansion and group reduction for per-query-head routing.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h.)
//
// Routing per query head runs the layer on keys, values and NP-Map weights expanded to one
// copy per query head, so that every query head has its own selection, its own softmax
// cache and its own linear-attention state; the gradients of the copies are then summed
// back over each KV head's group.
#include "still_common.hpp"
#include "still_launch.hpp"

namespace still {

// dst[r][h * G + g][0..inner) = src[r][h][0..inner), in 16-byte pieces; one thread per piece
__global__ __launch_bounds__(256) void expand_heads_kernel(const uint4* src, uint4* dst, long long rows, int Hkv, int G,
                                                           int pieces) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  const long long n = rows * Hkv * G * pieces;
  if (gid >= n) return;
  const int p = static_cast<int>(gid % pieces);
  const long long rest = gid / pieces;
  const int hq = static_cast<int>(rest % (static_cast<long long>(Hkv) * G));
  const long long r = rest / (static_cast<long long>(Hkv) * G);
  dst[gid] = src[(r * Hkv + hq / G) * pieces + p];
}

// dst[r][h][x] = sum over g of src[r][h * G + g][x] (fp32 sums in g order)
template <typename T>
__global__ __launch_bounds__(256) void reduce_heads_kernel(const T* src, T* dst, long long rows, int Hkv, int G,
                                                           int inner) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  const long long n = rows * Hkv * inner;
  if (gid >= n) return;
  const int x = static_cast<int>(gid % inner);
  const long long rh = gid / inner;  // r * Hkv + h
  const T* s = src + rh * G * inner + x;
  float acc = 0.f;
  for (int g = 0; g < G; ++g) acc += Tr<T>::to_f(s[static_cast<long long>(g) * inner]);
  dst[gid] = Tr<T>::from_f(acc);
}

hipError_t launch_expand_heads(const void* src, void* dst, long long rows, int Hkv, int G, long long inner_bytes,
                               hipStream_t s) {
  const int pieces = static_cast<int>(inner_bytes / 16);
  const long long n = rows * Hkv * G * pieces;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_heads_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), rows, Hkv, G, pieces);
  return hipGetLastError();
}

hipError_t launch_reduce_heads(const void* src, void* dst, long long rows, int Hkv, int G, int inner, int elem,
                               hipStream_t s) {
  const long long n = rows * Hkv * inner;
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (elem == 2)
    hipLaunchKernelGGL(reduce_heads_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(src),
                       static_cast<bf16*>(dst), rows, Hkv, G, inner);
  else
    hipLaunchKernelGGL(reduce_heads_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
                       static_cast<float*>(dst), rows, Hkv, G, inner);
  return hipGetLastError();
}

}  // namespace still

// Internal launch interface between the C ABI (still_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace still {

struct Dims {
  int B, T, Hq, Hkv, G, D, DF, window, topk;
  int nC;   // number of chunks, ceil(T / 64)
  int nCc;  // number of complete chunks, T / 64
  int R;    // floats per chunk state record: DF*D (S) + DF (z)
  int bf16; // 1 = bf16 tensors, 0 = fp32
};

struct PrepArgs {
  Dims d;
  const void* q;
  const void* k;
  const void* v;
  const void* w;
  const int32_t* routing_in;  // optional
  float* sal;                 // [B,Hkv,T]
  uint64_t* selmask;          // [B,Hkv,nC]
  int32_t* sel_idx;           // optional [B,Hkv,nCc,topk]
  void* ksel;                 // [B,Hkv,nCc*topk,D]: compact K rows
  void* phik;                // [B,Hkv,T,DF], features permuted by pk_pos
  float* states;              // [B,Hkv,nC,R]
  void* vT;                   // [B,Hkv,nC,D,64]: V of each chunk transposed, keys permuted by pk_pos
  void* vselT;                // [B,Hkv,ntiles_sel,D,64]: compact V rows, same tile layout
  int ntiles_sel;             // ceil(nCc*topk / 64)
};

struct AttnArgs {
  Dims d;
  const void* q;
  const void* k;
  const void* w;
  const uint64_t* selmask;
  const void* ksel;
  const void* vselT;
  const void* vT;
  const void* phik;
  const float* states;  // inclusive prefix over complete chunks
  void* out;
  int ntiles_sel;
  int nw;               // query heads per workgroup (1, 2 or 4)
  int gsplit;           // workgroups per (b, kv head, chunk)
};

hipError_t launch_prep(const PrepArgs& a, hipStream_t s);
hipError_t launch_scan(const Dims& d, float* states, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_topk(const Dims& d, const float* sal, int32_t* sel_idx, hipStream_t s);
hipError_t launch_feature_map(const Dims& d, const void* x, const void* w, float* phi, hipStream_t s);

// true if the (dtype, D, DF) triple has kernel instantiations
bool shape_supported(int bf16, int D, int DF);

}  // namespace still

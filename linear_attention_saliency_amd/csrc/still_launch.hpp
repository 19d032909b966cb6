// Internal launch interface between the C ABI (still_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace still {

struct Dims {
  int B, T, Hq, Hkv, G, D, DF, window, topk;
  // Routing heads: who selects. Per KV head: Hr = Hkv, Gr = G; per query head: Hr = Hq,
  // Gr = 1. Saliency, selection, the compact softmax rows and the linear-attention state are
  // kept per (b, routing head); routing head rh reads KV head rh * Gr / G and serves query
  // heads rh * Gr .. rh * Gr + Gr - 1.
  int Hr, Gr;
  int nC;   // number of chunks, ceil(T / 64)
  int nCc;  // number of complete chunks, T / 64
  int R;    // elements per chunk state record: DF*D (S) + DF (z)
  int bf16; // 1 = bf16 tensors, 0 = fp32
  int score; // routing score: 0 = Self-Saliency Score, 1 = diagonal logit
};

struct PrepArgs {
  Dims d;
  const void* q;
  const void* k;
  const void* v;
  const void* w;
  const int32_t* routing_in;  // optional
  float* sal;                 // [B,Hr,T]
  uint64_t* selmask;          // [B,Hr,nC]
  int32_t* sel_idx;           // optional [B,Hr,nCc,topk]
  void* ksel;                 // [B,Hr,ntiles_sel*64,D]: compact K rows (the selected keys)
  void* phik;                // [B,Hkv,T,DF], features permuted by pk_pos
  void* states;               // [B,Hr,nC,R] in the layer's dtype: S^T [D][DF] with features permuted by
                              // pk_pos, then z [DF] permuted
  void* vT;                   // [B,Hkv,nC,D,64]: V of each chunk transposed, keys permuted by pk_pos
  void* vselT;                // [B,Hr,ntiles_sel,D,64]: compact V rows, same tile layout
  int ntiles_sel;             // compact tiles per (b, KV head): >= ceil(nCc*topk / 64)
  float* kmaxc;               // [B,Hr,nC]: largest |k| among each chunk's selected keys
  float* kall;                // [B,Hr,nC]: largest |k| among all of each chunk's keys
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
  const void* states;   // inclusive prefix over complete chunks (layer dtype)
  void* out;
  int ntiles_sel;
  const float* tilemax; // [B,Hkv,tm_stride]: largest |k| in each compact tile
  const float* kall;    // [B,Hr,nC]: largest |k| among all of each chunk's keys
  int tm_stride;
  int nw;               // query heads per workgroup (1, 2 or 4)
  int gsplit;           // workgroups per (b, kv head, chunk)
};

// Device view of a decode cache (layouts as in still_cache; the compact rows use the
// prefill's tile layout: K rows [B,Hkv,sel_tiles*64,D], V in [B,Hkv,sel_tiles,D,64]).
struct CacheView {
  void* sel_k;
  void* sel_v;
  void* ring_k;    // [B,Hkv,2,64,D], chunk j in slot j % 2
  void* ring_v;
  float* state_s;  // [B,Hkv,DF,D]
  float* state_z;  // [B,Hkv,DF]
  uint64_t* sel_mask;  // [B,Hkv,2]
  float* cur_sal;      // [B,Hkv,64]
  int sel_tiles;       // compact tiles per (b, KV head)
};

// Leaves the cache as decode expects it after a prefill of d.T tokens.
struct ExportArgs {
  Dims d;
  const void* k;
  const void* v;
  const float* sal;        // [B,Hkv,T] group-summed saliency (unused if window = 0)
  const uint64_t* selmask; // [B,Hkv,nC]
  const void* states;      // [B,Hkv,nC,R] inclusive prefix over complete chunks (layer dtype)
  CacheView c;
};

struct DecodeArgs {
  Dims d;               // T unused
  long long pos;        // position of the new token
  int nsel;             // compact rows visible to this token: max(0, chunk - 1) * topk
  int nsplit;           // workgroups per (b, KV head) over the compact rows
  int tiles_per_split;
  const void* q;        // [B,Hq,D]
  const void* k;        // [B,Hkv,D]
  const void* v;
  const void* w;
  void* out;            // [B,Hq,D]
  float* part_ml;       // [B,Hkv,nsplit,G,2]: (max, sum) of each split, log2 units
  float* part_o;        // [B,Hkv,nsplit,G,D]
  CacheView c;
};

// Backward pass with the routing held fixed (head_dim = feat_dim = 64). Workspace buffers,
// per (b, KV head) or per (b, query head); "pk" marks 64-vectors stored pk-permuted.
struct BwdArgs {
  Dims d;
  const void* q;
  const void* k;
  const void* v;
  const void* w;
  const void* out;
  const void* dout;
  const int32_t* sel_idx;  // [B,Hkv,nCc,topk] ascending positions
  void* dq;
  void* dk;
  void* dv;
  float* dw;               // [Hkv,DF,D]
  void* kt;                // [B,Hkv,nC,D,64 pk]: K^T of each chunk
  void* phik;              // [B,Hkv,nC*64,DF pk]: phi(k) rows
  void* phikt;             // [B,Hkv,nC,DF,64 pk]
  float* ustate;           // [B,Hkv,nC,R]: U_c, then S_c = sum over chunks <= c-2
  void* ksel;              // [B,Hkv,ntiles*64,D]: selected K rows in chunk order
  void* vsel;              // [B,Hkv,ntiles*64,D]
  void* kselt;             // [B,Hkv,ntiles,D,64 pk]
  void* qt;                // [B,Hq,nC,D,64 pk]
  void* dot;               // [B,Hq,nC,D,64 pk]
  void* phiq;              // [B,Hq,nC*64,DF pk]: e^{-L} phi(q) rows
  void* phiqt;             // [B,Hq,nC,DF,64 pk]: e^{-L} phi(q)^T
  float* ld;               // [B,Hq,nC*64,2]: (log2 of the normaliser, Delta)
  float* apart;            // [B,Hq,nC,R]: per-chunk sum of e^{-L} phi(q) dout^T, e^{-L} Delta phi(q)
  float* rstate;           // [B,Hkv,nC,R]: R_c, r_c (chunks >= c+2)
  float* segsum;           // [B,Hkv,ceil(nC/16),R]: per-segment sums of the scan behind R
  float* dwq;              // [B,Hq,nC,DF*D]
  float* dwk;              // [B,Hkv,nC,DF*D]
  float* dkvsel;           // [nsplit,B,Hkv,ntiles*64,2,D]
  float* dwpart;           // [dw_parts,Hkv,DF*D]
  int ntiles;              // compact tiles per (b, KV head)
  int nsplit;              // query splits of the compact-key kernel
  int dw_parts;
};

// events: optional, 8 events recorded before each of the seven stages and after the last
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s, hipEvent_t* events);
// (bf16, head_dim, feat_dim) triples the backward kernels are instantiated for
bool bwd_shape_supported(int bf16, int D, int F);
// Query heads per wave in the backward's dq kernel (1 or 2); its shares of R and dW are kept
// per group of that many heads of a KV head.
int bwd_heads_per_wave(int bf16, int G);

// Attention from far-future queries under full causal softmax (head_dim 64).
struct MassArgs {
  Dims d;
  const void* q;
  const void* k;
  float* lse;   // [B,Hq,nC*64]: log2 of each row's causal normaliser (inf past T)
  float* part;  // [nsplit,B,Hkv,T]: per query slice column sums
  float* mass;  // [B,Hkv,T]
  int nsplit;   // query slices
  int per;      // chunks per slice
};

hipError_t launch_mass(const MassArgs& a, hipStream_t s);
hipError_t launch_overlap(const Dims& d, const int32_t* sa, const int32_t* sb, int32_t* out, hipStream_t s);

// Per-query-head routing: dst[r][h*G+g][:] = src[r][h][:] (inner_bytes a multiple of 16),
// and dst[r][h][:] = sum_g src[r][h*G+g][:] (elem 2: bf16, 4: fp32).
hipError_t launch_expand_heads(const void* src, void* dst, long long rows, int Hkv, int G, long long inner_bytes,
                               hipStream_t s);
hipError_t launch_reduce_heads(const void* src, void* dst, long long rows, int Hkv, int G, int inner, int elem,
                               hipStream_t s);

hipError_t launch_prep(const PrepArgs& a, hipStream_t s);
// prefix sums of the chunk records, and the per-tile key-norm bound from kmaxc
hipError_t launch_scan(const Dims& d, void* states, const float* kmaxc, float* tilemax, int tm_stride,
                       hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_topk(const Dims& d, const float* sal, int32_t* sel_idx, hipStream_t s);
hipError_t launch_feature_map(const Dims& d, const void* x, const void* w, float* phi, hipStream_t s);

hipError_t launch_cache_export(const ExportArgs& a, hipStream_t s);
// mid: optional event recorded between the compact-cache kernel and the token kernel
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t mid);
// Bytes of the decode step's file-scope device scratch (the entry point that allocates
// nothing keeps its split partials there), and that scratch's device address on the
// current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// Earlier chunks taken with per-query masks: L = ceil(w / 64), at least 1 (the chunk before
// is always one of them, since its selection is the latest one a query sees). A band of L
// chunks before the query's chunk holds the whole window of every query in it, with the
// window's first key at or after the band's second row, which the saliency's 16-row key
// blocks need. Windows up to kMaxWindow = 2 * 64 (L <= 2) are built.
constexpr int kMaxBand = 2;
constexpr int kMaxWindow = kMaxBand * 64;
__host__ __device__ constexpr int band_chunks(int window) { return window <= 64 ? 1 : (window + 63) / 64; }
static_assert(band_chunks(64) == 1 && band_chunks(65) == 2 && band_chunks(kMaxWindow) == 2, "band length");
hipError_t decode_scratch(void** ptr);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// true if the (dtype, D, DF) triple has kernel instantiations
bool shape_supported(int bf16, int D, int DF);

}  // namespace still

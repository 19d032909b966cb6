// Decode step of the STILL layer and the kernels that build its cache
// ([P1] section "Chunk-Wise并行+延迟选择": routing decided per chunk and used one chunk later,
// so a decoding token never waits for a per-token selection).
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h.)
//
// One new token for every sequence, all at position i = 64c + r. Per (batch b, routing
// head rh: the KV head, or a query head when each query head selects for itself):
//   decode_split_kernel  nsplit workgroups each read a disjoint run of 64-row tiles of the
//                        compact softmax cache (the selected rows of chunks <= c-L-1) and leave
//                        an online-softmax partial (max, sum, unnormalised output, log2 units)
//                        for each of the Gr query heads the routing head serves. This is the only part
//                        whose bytes grow with the context; it is HBM-bound.
//   decode_token_kernel  one workgroup: writes the token into the ring of raw rows (chunks
//                        c-L .. c, L = band_chunks(w)), computes its Self-Saliency Score with the prefill's
//                        routine (so routing is bit-identical to a prefill of the same
//                        tokens), the softmax over the ring keys in the softmax set, the
//                        NP-Map linear-attention term (prefix state plus the ring keys
//                        outside the softmax set), merges all of it with the split partials
//                        under one normaliser and writes the outputs. When the token completes
//                        chunk c it picks that chunk's top_k and folds chunk c-L: the selected
//                        rows are appended to the compact cache, the others are added to the
//                        state (sum phi(k) v^T, sum phi(k)).
// cache_export_kernel leaves a cache as these kernels expect it after a prefill of T tokens.
#include <mutex>

#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"

// Scratch of still_decode_step_noalloc: the split partials, for callers that cannot
// allocate. One copy per GPU, held until the process ends; calls on one GPU share it. In
// host code this name is not a device address: decode_scratch() below looks the address
// up once per device, and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[still::kDecodeScratchBytes];

namespace still {

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

constexpr int kMaxGroup = 16;  // query heads per KV head the decode kernels handle

}  // namespace

// ------------------------------------------------------------------ compact-cache splits

// grid (nsplit, B*Hkv), four waves. Wave w takes tiles t0 + w, t0 + w + 4, ... of the split.
// Per tile (64 keys): S^T = K Q^T on MFMA with the query heads as columns (head g in column
// g, unused columns zero), online softmax per column, O^T += V^T P^T with P fed back from the
// accumulator (PK layout, matching the transposed compact V tiles).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  constexpr int NDB = D / 16;
  __shared__ float red_m[4][16];
  __shared__ float red_l[4][16];
  __shared__ float red_o[4][D][16];

  const Dims& d = a.d;
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));  // logit scale in log2 units
  const int split = blockIdx.x, bh = blockIdx.y;  // bh: the (b, routing head) record
  const int b = bh / d.Hr, rh = bh % d.Hr, G = d.Gr;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int ntiles = (a.nsel + 63) / 64;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(ntiles, t_begin + a.tiles_per_split);

  const T* q = static_cast<const T*>(a.q) + static_cast<long long>(b * d.Hq + rh * G) * D;
  frag qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks] = r16 < G ? TT::load8(q + r16 * D + ks * 32 + grp * 8) : TT::zero();

  const long long tiles = a.c.sel_tiles;
  const T* kbase = static_cast<const T*>(a.c.sel_k) + static_cast<long long>(bh) * tiles * 64 * D;
  const T* vbase = static_cast<const T*>(a.c.sel_v) + static_cast<long long>(bh) * tiles * D * 64;

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -kInf, l = 0.f;

  for (int t = t_begin + wave; t < t_end; t += 4) {
    frag kf[4][D / 32];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kf[j][ks] = TT::load8(kbase + (static_cast<long long>(t) * 64 + j * 16 + r16) * D + ks * 32 + grp * 8);
    frag vf[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        vf[db][ms] = TT::load8(vbase + (static_cast<long long>(t) * D + db * 16 + r16) * 64 + 8 * (4 * ms + grp));
    f32x4 s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) TT::mma(s[j], kf[j][ks], qf[ks]);
    }
    const int valid = a.nsel - t * 64;  // >= 1
    float mx = -kInf;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = j * 16 + 4 * grp + i;
        const float x = key < valid ? s[j][i] * c1 : -kInf;  // logits in log2 units (fp32 scale)
        s[j][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = xor_max_groups(mx);
    const float mn = fmaxf(m, mx);  // finite: every tile holds a valid key
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    frag pf[2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto pb = TT::from_f(__builtin_amdgcn_exp2f(s[j][i] - m));
        l += TT::to_f(pb);
        pf[j >> 1][(j & 1) * 4 + i] = pb;
      }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) TT::mma(o[db], vf[db][ms], pf[ms]);
  }
  l = xor_sum_groups(l);
  if (grp == 0) {
    red_m[wave][r16] = m;
    red_l[wave][r16] = l;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[wave][db * 16 + 4 * grp + i][r16] = o[db][i];
  __syncthreads();

  const long long rec = (static_cast<long long>(bh) * a.nsplit + split) * G;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D, dd = idx % D;
    float M = -kInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][g]);
    float L = 0.f, O = 0.f;
    if (M > -kInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __builtin_amdgcn_exp2f(red_m[w][g] - M);
        L += red_l[w][g] * f;
        O += red_o[w][dd][g] * f;
      }
    }
    a.part_o[(rec + g) * D + dd] = O;
    if (dd == 0) {
      a.part_ml[(rec + g) * 2] = M;
      a.part_ml[(rec + g) * 2 + 1] = L;
    }
  }
}

// ------------------------------------------------------------------------ token kernel

// LDS plan of the token kernel for a ring of NR = BL + 1 chunks (RW = 64 NR ring rows). The
// softmax logits (ex) reuse the phi(K) rows' space: phi(K) is done with before the logits
// are written, and written again only after the last read of the logits.
template <typename T, int D, int DF, int BL>
struct TokLds {
  static constexpr int KP = DF + 1;  // padded phi row (conflict-free column reads)
  static constexpr int RW = 64 * (BL + 1);
  static_assert(kMaxGroup * RW <= 64 * KP, "the logits fit in the phi(K) rows' space");
  // the ring's V rows are staged in LDS where the whole plan fits the CU's 160 KiB, else
  // read from the ring in memory
  static constexpr size_t fixed = (RW + 1) * D * sizeof(T) + kMaxGroup * (D + DF) * 4 + 64 * KP * 4 +
                                  kMaxGroup * RW * 4 + (256 + 64 + 5 * kMaxGroup) * 4;
  static constexpr bool VT_LDS = fixed + RW * D * sizeof(T) <= 160 * 1024;
  static constexpr size_t kt = 0;                                     // Swz<T,D>, RW + 1 rows
  static constexpr size_t vt = kt + (RW + 1) * D * sizeof(T);         // [RW][D] T (VT_LDS)
  static constexpr size_t qs = vt + (VT_LDS ? RW * D * sizeof(T) : 0);  // [16][D] f32
  static constexpr size_t phq = qs + kMaxGroup * D * 4;               // [16][DF]
  static constexpr size_t phk = phq + kMaxGroup * DF * 4;             // [64][KP]
  static constexpr size_t ex = phk;                                   // [16][RW] over phk
  static constexpr size_t wla = phk + 64 * KP * 4;                    // [16][RW]
  static constexpr size_t m2part = wla + kMaxGroup * RW * 4;          // [256]
  static constexpr size_t xn2 = m2part + 256 * 4;                     // [64]
  static constexpr size_t gstat = xn2 + 64 * 4;                       // [5][16]
  static constexpr size_t bytes = gstat + 5 * kMaxGroup * 4;
  static_assert(bytes == fixed + (VT_LDS ? RW * D * sizeof(T) : 0), "layout and budget agree");
  static_assert(bytes <= 160 * 1024, "the token kernel's LDS must fit a CU");
};

// One workgroup per (b, routing head) (a KV head, or a query head when each query head
// selects for itself: then every query head keeps its own ring, compact rows and state). LDS tile row t holds the key at position 64(c-BL) + t:
// rows 64(BL-l) .. 64(BL-l)+63 are chunk c-l (zero when c < l), rows 64 BL .. 64 BL + r
// chunk c up to the new token, the rest zero. Chunk x lives in ring slot x mod (BL + 1).
// Query head g of the routing head is rh*Gr + g.
template <typename T, int D, int DF, int BL>
__global__ __launch_bounds__(256) void decode_token_kernel(DecodeArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SW = Swz<T, D>;
  using L = TokLds<T, D, DF, BL>;
  constexpr int NR = BL + 1, RW = L::RW;
  constexpr int V8 = D / 8;
  constexpr int FPW = DF / 64;
  constexpr int KP = L::KP;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  T* kt = reinterpret_cast<T*>(lds + L::kt);
  T* vt = reinterpret_cast<T*>(lds + L::vt);
  float* qs = reinterpret_cast<float*>(lds + L::qs);
  float* phq = reinterpret_cast<float*>(lds + L::phq);
  float* phk = reinterpret_cast<float*>(lds + L::phk);
  float* wla = reinterpret_cast<float*>(lds + L::wla);
  float* ex = reinterpret_cast<float*>(lds + L::ex);
  float* m2part = reinterpret_cast<float*>(lds + L::m2part);
  float* xn2 = reinterpret_cast<float*>(lds + L::xn2);
  float* gmax = reinterpret_cast<float*>(lds + L::gstat);
  float* gsum = gmax + kMaxGroup;
  float* gden = gsum + kMaxGroup;
  float* gsal = gden + kMaxGroup;
  float* gmisc = gsal + kMaxGroup;  // [0] = group-summed saliency of the new token

  const Dims& d = a.d;
  // bh: the (b, routing head) record; h: its KV head; G: the query heads it serves
  const int bh = blockIdx.x, b = bh / d.Hr, rh = bh % d.Hr, h = rh * d.Gr / d.G, G = d.Gr, w = d.window;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const long long pos = a.pos, c = pos / 64;
  const int r = static_cast<int>(pos % 64);
  auto slot_of = [&](long long ch) { return static_cast<int>(ch % NR); };  // ch >= 0
  const int slot_cur = slot_of(c);
  const float scale = kLog2e / sqrtf(static_cast<float>(D));

  const T* q = static_cast<const T*>(a.q) + static_cast<long long>(b * d.Hq + rh * G) * D;
  const T* knew = static_cast<const T*>(a.k) + static_cast<long long>(b * d.Hkv + h) * D;
  const T* vnew = static_cast<const T*>(a.v) + static_cast<long long>(b * d.Hkv + h) * D;
  const T* wh = static_cast<const T*>(a.w) + static_cast<long long>(h) * DF * D;
  T* ring_k = static_cast<T*>(a.c.ring_k) + static_cast<long long>(bh) * NR * 64 * D;
  T* ring_v = static_cast<T*>(a.c.ring_v) + static_cast<long long>(bh) * NR * 64 * D;
  // selection of band chunk c-l (l = 1 .. BL; none before the sequence)
  uint64_t band_mask[BL + 1];
#pragma unroll
  for (int l = 1; l <= BL; ++l) band_mask[l] = c >= l ? a.c.sel_mask[bh * NR + slot_of(c - l)] : 0ull;
  // element dd of ring row `row` (rows 64(BL-l).. chunk c-l, 64 BL.. chunk c; the new token at
  // row 64 BL + r, later rows zero), from LDS or from the ring in memory
  auto vring = [&](int row, int dd) -> float {
    if constexpr (L::VT_LDS) {
      return TT::to_f(vt[row * D + dd]);
    } else {
      const long long ch = c - BL + row / 64;
      const int p = row % 64;
      if (row < 64 * BL) return ch >= 0 ? TT::to_f(ring_v[(slot_of(ch) * 64 + p) * D + dd]) : 0.f;
      if (p < r) return TT::to_f(ring_v[(slot_cur * 64 + p) * D + dd]);
      return p == r ? TT::to_f(vnew[dd]) : 0.f;
    }
  };

  typename Tr<T>::frag wf[DF / 64][D / 32];  // NP-Map weights, loaded early
  np_map_load_w<T, D, DF>(wh, wf);
  // this thread's share of the prefix state for the read-out of step 5, loaded now so the
  // loads overlap steps 0-4: column dcol of S, features fh*FQ .. fh*FQ + FQ - 1 (the NFH
  // feature slices of a column sit in adjacent lanes); z[tid] for tid < DF
  constexpr int NFH = 256 / D, FQ = DF / NFH;
  const int fh = tid % NFH, dcol = tid / NFH;
  float sreg[FQ];
  {
    const float* S = a.c.state_s + static_cast<long long>(bh) * DF * D;
#pragma unroll
    for (int j = 0; j < FQ; ++j) sreg[j] = S[(fh * FQ + j) * D + dcol];
  }
  const float zreg = tid < DF ? a.c.state_z[static_cast<long long>(bh) * DF + tid] : 0.f;

  // 0. stage the ring (and the new token) in LDS; append the token to the ring. The loads of
  //    up to kBatch pieces per thread are issued before any of them is stored.
  constexpr int NPIECE = (RW + 1) * V8, NIT = (NPIECE + 255) / 256, kBatch = 8;
#pragma unroll
  for (int it0 = 0; it0 < NIT; it0 += kBatch) {
    frag xk[kBatch], xv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = tid + (it0 + j) * 256;
      const int row = idx / V8, c8 = idx % V8;
      const long long ch = c - BL + row / 64;
      const int p = row % 64;
      xk[j] = TT::zero();
      xv[j] = TT::zero();
      if (it0 + j >= NIT || idx >= NPIECE) continue;
      if (row < 64 * BL) {
        if (ch >= 0) {
          xk[j] = TT::load8(ring_k + (slot_of(ch) * 64 + p) * D + c8 * 8);
          xv[j] = TT::load8(ring_v + (slot_of(ch) * 64 + p) * D + c8 * 8);
        }
      } else if (row < RW && p < r) {
        xk[j] = TT::load8(ring_k + (slot_cur * 64 + p) * D + c8 * 8);
        xv[j] = TT::load8(ring_v + (slot_cur * 64 + p) * D + c8 * 8);
      } else if (row < RW && p == r) {
        xk[j] = TT::load8(knew + c8 * 8);
        xv[j] = TT::load8(vnew + c8 * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = tid + (it0 + j) * 256;
      const int row = idx / V8, c8 = idx % V8;
      if (it0 + j >= NIT || idx >= NPIECE) continue;
      if (row < RW && row - 64 * BL == r) {
        TT::store8(ring_k + (slot_cur * 64 + r) * D + c8 * 8, xk[j]);
        TT::store8(ring_v + (slot_cur * 64 + r) * D + c8 * 8, xv[j]);
      }
      SW::store8(kt, row, c8 * 8, xk[j]);
      if constexpr (L::VT_LDS)
        if (row < RW) TT::store8(vt + row * D + c8 * 8, xv[j]);
    }
  }
  for (int idx = tid; idx < G * D; idx += 256) qs[idx] = TT::to_f(q[idx]);
  __syncthreads();

  // 1. Self-Saliency Score of the new token for each query head, summed in head order
  if (w >= 1) {
    for (int g0 = 0; g0 < G; g0 += 4) {
      const int g = g0 + wave;
      if (g < G) {
        frag qf[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          qf[ks] = r16 == (r & 15) ? TT::load8(q + g * D + ks * 32 + grp * 8) : TT::zero();
        const float sv = saliency_qblock<T, D, BL>(kt, qf, r >> 4, w, 64 * c - 64 * BL + 1, scale, 1, d.score);
        if (lane == (r & 15)) gsal[g] = sv;
      }
    }
    __syncthreads();
    if (tid == 0) {
      float acc = 0.f;
      for (int g = 0; g < G; ++g) acc += gsal[g];
      gmisc[0] = acc;
      a.c.cur_sal[bh * 64 + r] = acc;
    }
  }

  // 2. NP-Map of the queries: m = elu(W_h q) + 1, then phi = m |q| / |m|
  for (int idx = tid; idx < G * DF; idx += 256) {
    const int g = idx / DF, f = idx % DF;
    float z = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < V8; ++c8) {  // all of the row's loads in flight together
      const frag wv = TT::load8(wh + f * D + c8 * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) z += TT::to_f(wv[e]) * qs[g * D + c8 * 8 + e];
    }
    phq[idx] = z > 0.f ? z + 1.f : __builtin_amdgcn_exp2f(z * kLog2e);
  }
  __syncthreads();
  for (int g = wave; g < G; g += 4) {
    float m2 = 0.f, q2 = 0.f;
    for (int f = lane; f < DF; f += 64) m2 += phq[g * DF + f] * phq[g * DF + f];
    for (int dd = lane; dd < D; dd += 64) q2 += qs[g * D + dd] * qs[g * D + dd];
    m2 = wave_sum(m2);
    q2 = wave_sum(q2);
    const float sc = norm_ratio(q2, m2);
    for (int f = lane; f < DF; f += 64) phq[g * DF + f] *= sc;
  }

  // 3. linear-attention weights phi(q_g).phi(k_p) of the ring keys outside the softmax set:
  //    chunk c-l (l >= 1) position p: p <= r + 64 l - w and not selected; chunk c position p:
  //    p <= r - w
  for (int part = 0; part <= BL; ++part) {  // ring chunk c - BL + part
    const int l = BL - part;
    const bool any = l >= 1 ? c >= l : (r - w >= 0);
    if (!any) {
      for (int idx = tid; idx < G * 64; idx += 256) wla[(idx / 64) * RW + part * 64 + idx % 64] = 0.f;
      continue;
    }
    f32x4 phi[4][FPW];
    np_map_rows64<T, D, DF>(kt, part * 64, wf, m2part, xn2, phi);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
        for (int i = 0; i < 4; ++i) phk[(kb * 16 + 4 * grp + i) * KP + (wave * FPW + fi) * 16 + r16] = phi[kb][fi][i];
    __syncthreads();
    const uint64_t lmask = l >= 1 ? band_mask[l] : 0ull;
    for (int idx = tid; idx < G * 64; idx += 256) {
      const int g = idx / 64, p = idx % 64;
      const bool la = l >= 1 ? (p <= r + 64 * l - w && !((lmask >> p) & 1ull)) : (p <= r - w);
      float s = 0.f;
      if (la)
        for (int f = 0; f < DF; ++f) s += phk[p * KP + f] * phq[g * DF + f];
      wla[g * RW + part * 64 + p] = s;
    }
    __syncthreads();
  }

  // 4. softmax logits (log2 units) of the ring keys in the softmax set:
  //    chunk c-l position p: p > r + 64 l - w or selected; chunk c position p: r - w < p <= r
  for (int idx = tid; idx < G * RW; idx += 256) {
    const int g = idx / RW, row = idx % RW;
    const int l = BL - row / 64, p = row % 64;
    bool sa;
    if (l >= 1) {
      sa = c >= l && (p > r + 64 * l - w || ((band_mask[l] >> p) & 1ull));
    } else {
      sa = p <= r && p > r - w;
    }
    float x = -kInf;
    if (sa) {
      float s = 0.f;
#pragma unroll 4
      for (int c8 = 0; c8 < V8; ++c8) {
        const frag kx = SW::load8(kt, row, c8 * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += TT::to_f(kx[e]) * qs[g * D + c8 * 8 + e];
      }
      x = s * scale;
    }
    ex[idx] = x;
  }
  __syncthreads();
  for (int g = wave; g < G; g += 4) {
    float xs[NR];
    float mx = -kInf;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      xs[j] = ex[g * RW + 64 * j + lane];
      mx = fmaxf(mx, xs[j]);
    }
    mx = wave_max(mx);
    float es = 0.f, ws = 0.f;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const float e = mx > -kInf ? __builtin_amdgcn_exp2f(xs[j] - mx) : 0.f;
      ex[g * RW + 64 * j + lane] = e;
      es += e;
      ws += wla[g * RW + 64 * j + lane];
    }
    const float l = wave_sum(es);
    const float dl = wave_sum(ws);
    if (lane == 0) {
      gmax[g] = mx;
      gsum[g] = l;
      gden[g] = dl;
    }
  }
  __syncthreads();

  // 5. merge: ring softmax, the linear-attention entry (log-weight log2 D_LA, value N/D_LA)
  //    and the compact-cache partials, one shared normaliser.
  //    First the prefix state's read-out, phi(q_g)^T S and phi(q_g).z: each thread sums its
  //    features of one column, the slices of a column are summed across adjacent lanes
  //    (fixed order), into qs (free after step 4); z goes to m2part, then phi(q_g).z to xn2.
  float* osl = qs;  // [G][D]
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < FQ; ++j) acc += phq[g * DF + fh * FQ + j] * sreg[j];
#pragma unroll
    for (int m = 1; m < NFH; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (fh == 0) osl[g * D + dcol] = acc;
  }
  if (tid < DF) m2part[tid] = zreg;
  __syncthreads();
  for (int g = wave; g < G; g += 4) {
    float x = 0.f;
    for (int f = lane; f < DF; f += 64) x += phq[g * DF + f] * m2part[f];
    x = wave_sum(x);
    if (lane == 0) xn2[g] = x;
  }
  __syncthreads();
  T* out = static_cast<T*>(a.out) + static_cast<long long>(b * d.Hq + rh * G) * D;
  const long long rec0 = static_cast<long long>(bh) * a.nsplit * G;
  const int nsplit = a.nsel > 0 ? a.nsplit : 0;
  constexpr int SB = 8;  // split partials loaded ahead of the ring loop (their latency overlaps it)
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D, dd = idx % D;
    float pm[SB], pl[SB], po[SB];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const long long rec = rec0 + static_cast<long long>(s) * G + g;
      pm[s] = s < nsplit ? a.part_ml[rec * 2] : -kInf;
      pl[s] = s < nsplit ? a.part_ml[rec * 2 + 1] : 0.f;
      po[s] = s < nsplit ? a.part_o[rec * D + dd] : 0.f;
    }
    float osa = 0.f, ola = 0.f;
#pragma unroll 8
    for (int row = 0; row < RW; ++row) {
      const float vv = vring(row, dd);
      osa += ex[g * RW + row] * vv;
      ola += wla[g * RW + row] * vv;
    }
    ola += osl[g * D + dd];
    const float dla = gden[g] + xn2[g];
    const float mla = dla > 0.f ? __log2f(dla) : -kInf;
    float M = fmaxf(gmax[g], mla);
#pragma unroll
    for (int s = 0; s < SB; ++s) M = fmaxf(M, pm[s]);
    for (int s = SB; s < nsplit; ++s) M = fmaxf(M, a.part_ml[(rec0 + s * G + g) * 2]);
    float Lsum = 0.f, O = 0.f;
    if (M > -kInf) {
      if (gmax[g] > -kInf) {
        const float f = __builtin_amdgcn_exp2f(gmax[g] - M);
        Lsum += gsum[g] * f;
        O += osa * f;
      }
      if (dla > 0.f) {
        const float f = __builtin_amdgcn_exp2f(mla - M);
        Lsum += f;
        O += (ola / dla) * f;
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        if (pm[s] > -kInf) {
          const float f = __builtin_amdgcn_exp2f(pm[s] - M);
          Lsum += pl[s] * f;
          O += po[s] * f;
        }
      }
      for (int s = SB; s < nsplit; ++s) {
        const float ms = a.part_ml[(rec0 + s * G + g) * 2];
        if (ms > -kInf) {
          const float f = __builtin_amdgcn_exp2f(ms - M);
          Lsum += a.part_ml[(rec0 + s * G + g) * 2 + 1] * f;
          O += a.part_o[(rec0 + s * G + g) * D + dd] * f;
        }
      }
    }
    out[idx] = TT::from_f(Lsum > 0.f ? O / Lsum : 0.f);
  }

  // 6. chunk completion: top_k of chunk c; fold chunk c-BL (ring rows 0..63), whose slot
  //    the next chunk takes
  if (r != 63) return;  // uniform across the workgroup
  __syncthreads();
  if (wave == 0) {
    uint64_t nm = 0;
    if (d.topk > 0) nm = topk_mask(lane < 63 ? a.c.cur_sal[bh * 64 + lane] : gmisc[0], d.topk);
    if (lane == 0) a.c.sel_mask[bh * NR + slot_cur] = nm;
  }
  if (c < BL) return;
  const uint64_t prev_mask = band_mask[BL];
  {
    const long long tiles = a.c.sel_tiles;
    T* sk = static_cast<T*>(a.c.sel_k) + static_cast<long long>(bh) * tiles * 64 * D;
    T* sv = static_cast<T*>(a.c.sel_v) + static_cast<long long>(bh) * tiles * D * 64;
    const long long row0 = (c - BL) * d.topk;
    for (int idx = tid; idx < 64 * D; idx += 256) {
      const int p = idx / D, dd = idx % D;
      if ((prev_mask >> p) & 1ull) {
        const long long R = row0 + __popcll(prev_mask & ((1ull << p) - 1ull));
        sk[R * D + dd] = kt[SW::off(p, dd)];  // compact rows are the raw keys
        sv[((R / 64) * D + dd) * 64 + pk_pos(static_cast<int>(R % 64))] = TT::from_f(vring(p, dd));
      }
    }
  }
  f32x4 phi[4][FPW];
  np_map_rows64<T, D, DF>(kt, 0, wf, m2part, xn2, phi);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int fi = 0; fi < FPW; ++fi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kb * 16 + 4 * grp + i;
        phk[row * KP + (wave * FPW + fi) * 16 + r16] = ((prev_mask >> row) & 1ull) ? 0.f : phi[kb][fi][i];
      }
  __syncthreads();
  float* Sw = a.c.state_s + static_cast<long long>(bh) * DF * D;
  float* zw = a.c.state_z + static_cast<long long>(bh) * DF;
  for (int idx = tid; idx < DF * D; idx += 256) {
    const int f = idx / D, dd = idx % D;
    float acc = 0.f;
#pragma unroll 8
    for (int p = 0; p < 64; ++p) acc += phk[p * KP + f] * vring(p, dd);
    Sw[idx] += acc;
  }
  for (int f = tid; f < DF; f += 256) {
    float acc = 0.f;
    for (int p = 0; p < 64; ++p) acc += phk[p * KP + f];
    zw[f] += acc;
  }
}

// ---------------------------------------------------------------------- cache export

// One workgroup per (b, routing head): after a prefill of T tokens (chunk cT = T/64 holds the
// next token), put chunks cT-L .. cT into the ring (chunk x in slot x mod (L + 1)), their
// selections and chunk cT's saliencies in place, and the state of the unselected tokens of
// chunks <= cT-L-1 (L = band_chunks(w)). The compact rows were written by the prefill itself.
template <typename T, int D>
__global__ __launch_bounds__(256) void cache_export_kernel(ExportArgs a) {
  using TT = Tr<T>;
  constexpr int V8 = D / 8;
  const Dims& d = a.d;
  const int bh = blockIdx.x, b = bh / d.Hr, rh = bh % d.Hr, h = rh * d.Gr / d.G, tid = threadIdx.x;
  const long long T_ = d.T, cT = T_ / 64;
  const int rT = static_cast<int>(T_ % 64);
  const int BL = band_chunks(d.window), NR = BL + 1;
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* rk = static_cast<T*>(a.c.ring_k) + static_cast<long long>(bh) * NR * 64 * D;
  T* rv = static_cast<T*>(a.c.ring_v) + static_cast<long long>(bh) * NR * 64 * D;
  // the chunk in slot s: the one of cT-L .. cT congruent to s (mod L + 1)
  auto chunk_in = [&](int slot) { return cT - ((cT - slot) % NR + NR) % NR; };
  for (int idx = tid; idx < NR * 64 * V8; idx += 256) {
    const int slot = idx / (64 * V8), row = (idx / V8) % 64, c8 = idx % V8;
    const long long ch = chunk_in(slot);
    const long long p = ch * 64 + row;
    typename TT::frag xk = TT::zero(), xv = TT::zero();
    if (ch >= 0 && p < T_) {
      xk = TT::load8(k + ((b * T_ + p) * d.Hkv + h) * D + c8 * 8);
      xv = TT::load8(v + ((b * T_ + p) * d.Hkv + h) * D + c8 * 8);
    }
    TT::store8(rk + (slot * 64 + row) * D + c8 * 8, xk);
    TT::store8(rv + (slot * 64 + row) * D + c8 * 8, xv);
  }
  if (tid < NR) {
    const long long ch = chunk_in(tid);
    a.c.sel_mask[bh * NR + tid] = (ch >= 0 && ch < d.nCc) ? a.selmask[static_cast<long long>(bh) * d.nC + ch] : 0ull;
  }
  if (tid < 64)
    a.c.cur_sal[bh * 64 + tid] = (d.window >= 1 && tid < rT) ? a.sal[static_cast<long long>(bh) * T_ + cT * 64 + tid] : 0.f;
  // the prefill's records hold S^T[d][pk_pos(f)] and z[pk_pos(f)]; the cache holds S[f][d], z[f]
  const bool has_state = cT >= BL + 1;
  const T* src = static_cast<const T*>(a.states) + (static_cast<long long>(bh) * d.nC + (has_state ? cT - BL - 1 : 0)) * d.R;
  for (int idx = tid; idx < d.R; idx += 256) {
    if (idx < d.DF * D) {
      const int f = idx / D, dd = idx % D;
      a.c.state_s[static_cast<long long>(bh) * d.DF * D + idx] = has_state ? TT::to_f(src[dd * d.DF + pk_pos(f)]) : 0.f;
    } else {
      const int f = idx - d.DF * D;
      a.c.state_z[static_cast<long long>(bh) * d.DF + f] = has_state ? TT::to_f(src[d.DF * D + pk_pos(f)]) : 0.f;
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, long long n16) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<long long>(gridDim.x) * 256)
    p[i] = zero;
}

// ------------------------------------------------------------------------ launchers

template <typename T, int D, int DF>
static hipError_t decode_t(const DecodeArgs& a, hipStream_t s, hipEvent_t mid) {
  const int bhn = a.d.B * a.d.Hr;
  if (a.nsel > 0) {
    hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.nsplit, bhn), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mid) {
    const hipError_t e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  static_assert(kMaxBand == 2, "one token kernel per band length");
  auto go = [&](auto kern, size_t lds) {  // above 64 KiB: opt in (gfx950 has 160 KiB per CU)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(bhn), dim3(256), lds, s, a);
    return hipGetLastError();
  };
  if (band_chunks(a.d.window) == 1) return go(decode_token_kernel<T, D, DF, 1>, TokLds<T, D, DF, 1>::bytes);
  return go(decode_token_kernel<T, D, DF, 2>, TokLds<T, D, DF, 2>::bytes);
}

template <typename T, int D, int DF>
static hipError_t export_t(const ExportArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((cache_export_kernel<T, D>), dim3(a.d.B * a.d.Hr), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define STILL_DISPATCH_D(FN, ...)                                                 \
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t mid) {
#define DIMS a.d
  STILL_DISPATCH_D(decode_t, a, s, mid);
#undef DIMS
}

hipError_t launch_cache_export(const ExportArgs& a, hipStream_t s) {
#define DIMS a.d
  STILL_DISPATCH_D(export_t, a, s);
#undef DIMS
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const long long n16 = static_cast<long long>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const long long blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace still

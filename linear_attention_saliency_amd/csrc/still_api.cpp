// C ABI of the STILL layer: validation, workspace carving and the launch sequence.
// Every check happens before anything is enqueued; the library never allocates.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../include/still.h"
#include "still_launch.hpp"

using still::Dims;

namespace {

// The hipError_t behind the last STILL_ERR_HIP this thread returned (hipSuccess if none).
thread_local hipError_t t_last_hip = hipSuccess;

int fail_hip(hipError_t e) {
  t_last_hip = e;
  return STILL_ERR_HIP;
}

// evaluate a HIP call or launch; on failure keep its error and return STILL_ERR_HIP
#define STILL_HIP(expr)                          \
  do {                                           \
    const hipError_t still_e_ = (expr);          \
    if (still_e_ != hipSuccess) return fail_hip(still_e_); \
  } while (0)

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cfg(const still_config* c, bool use_seq) {
  if (!c) return STILL_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1) return STILL_ERR_INVALID_ARG;
  if (use_seq && c->seq_len < 1) return STILL_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0) return STILL_ERR_INVALID_ARG;
  if (c->dtype != STILL_F32 && c->dtype != STILL_BF16) return STILL_ERR_INVALID_ARG;
  if (c->score != STILL_SCORE_SALIENCY && c->score != STILL_SCORE_DIAG) return STILL_ERR_INVALID_ARG;
  if (c->routing_scope != STILL_ROUTE_PER_KV_HEAD && c->routing_scope != STILL_ROUTE_PER_QUERY_HEAD)
    return STILL_ERR_INVALID_ARG;
  if (c->head_dim < 1 || c->feat_dim < 1 || c->chunk < 1) return STILL_ERR_INVALID_ARG;
  if (c->window < 0 || c->top_k < 0 || c->top_k > c->chunk) return STILL_ERR_INVALID_ARG;
  if (c->window == 0 && c->top_k != 0) return STILL_ERR_INVALID_ARG;
  if (c->chunk != 64 || c->window > still::kMaxWindow) return STILL_ERR_UNSUPPORTED;
  if (!still::shape_supported(c->dtype == STILL_BF16, c->head_dim, c->feat_dim)) return STILL_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(c->batch) * c->n_kv_heads > 65535) return STILL_ERR_UNSUPPORTED;
  if (use_seq) {
    const int64_t n_chunks = (static_cast<int64_t>(c->seq_len) + 63) / 64;
    const int64_t g = c->n_q_heads / c->n_kv_heads;
    const int64_t nw = g < 4 ? g : 4;
    const int64_t gsplit = (g + nw - 1) / nw;
    if (n_chunks * c->batch * c->n_kv_heads * gsplit * 2 > 0x7fffffffLL) return STILL_ERR_UNSUPPORTED;
    // the chunk states of one (b, h) are addressed with 32-bit byte offsets
    const int64_t rec = static_cast<int64_t>(c->head_dim) * c->feat_dim + c->feat_dim;
    if (n_chunks * rec * (c->dtype == STILL_BF16 ? 2 : 4) > 0x7fffffffLL) return STILL_ERR_UNSUPPORTED;
  }
  return STILL_OK;
}

Dims dims_of(const still_config* c) {
  Dims d;
  d.B = c->batch;
  d.T = c->seq_len;
  d.Hq = c->n_q_heads;
  d.Hkv = c->n_kv_heads;
  const bool per_q = c->routing_scope == STILL_ROUTE_PER_QUERY_HEAD;
  d.Hr = per_q ? c->n_q_heads : c->n_kv_heads;
  d.Gr = per_q ? 1 : c->n_q_heads / c->n_kv_heads;
  d.G = c->n_q_heads / c->n_kv_heads;
  d.D = c->head_dim;
  d.DF = c->feat_dim;
  d.window = c->window;
  d.topk = c->top_k;
  d.score = c->score;
  d.nC = (c->seq_len + 63) / 64;
  d.nCc = c->seq_len / 64;
  d.R = c->feat_dim * c->head_dim + c->feat_dim;
  d.bf16 = c->dtype == STILL_BF16 ? 1 : 0;
  return d;
}

size_t elem_bytes(const still_config* c) { return c->dtype == STILL_BF16 ? 2 : 4; }

// Compact tiles per (b, KV head), rounded up to an odd count. The tiles of all (b, KV head)
// pairs sit at this stride, and the workgroups of different pairs read the same tile index
// at about the same time; with an even count (a power of two at the usual sizes) those
// reads meet in the same HBM channels. Measured on the 32 x 64K decode: 258 tiles per pair
// read the compact rows 34% slower than 257.
inline int64_t odd_tiles(int64_t n) { return n > 0 ? (n | 1) : 0; }

struct WsLayout {
  size_t sal, selmask, ksel, vselT, vT, phik, states, kmaxc, kall, tilemax, routing, total;
  int ntiles_sel;
};

WsLayout ws_layout(const still_config* c) {
  const Dims d = dims_of(c);
  const size_t bh = static_cast<size_t>(d.B) * d.Hr;   // routing-head records
  const size_t bkv = static_cast<size_t>(d.B) * d.Hkv;  // KV-head records (V^T and phi(K) tiles)
  const size_t es = elem_bytes(c);
  WsLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.sal = take(bh * d.T * sizeof(float));
  L.selmask = take(bh * d.nC * sizeof(uint64_t));
  L.ntiles_sel = static_cast<int>(odd_tiles((static_cast<int64_t>(d.nCc) * d.topk + 63) / 64));
  L.ksel = take(bh * L.ntiles_sel * 64 * d.D * es);
  L.vselT = take(bh * L.ntiles_sel * 64 * d.D * es);
  L.vT = take(bkv * d.nC * 64 * d.D * es);
  L.phik = take(bkv * d.T * d.DF * es);
  L.states = take(bh * d.nC * d.R * (d.bf16 ? 2 : 4));
  L.kmaxc = take(bh * d.nC * sizeof(float));
  L.kall = take(bh * d.nC * sizeof(float));
  L.tilemax = take(bh * (L.ntiles_sel > 0 ? L.ntiles_sel : 1) * sizeof(float));
  L.routing = take(bh * d.nCc * d.topk * sizeof(int32_t));  // a copy of routing_in, if given
  L.total = off;
  return L;
}

// routing_in (host memory): for every (b, selecting head, complete chunk c), top_k positions
// strictly ascending inside [64 c, 64 c + 63]
bool routing_valid(const still_config* c, const int32_t* r) {
  const int64_t heads = c->routing_scope == STILL_ROUTE_PER_QUERY_HEAD ? c->n_q_heads : c->n_kv_heads;
  const int64_t nCc = c->seq_len / 64, k = c->top_k;
  for (int64_t rec = 0; rec < static_cast<int64_t>(c->batch) * heads * nCc; ++rec) {
    const int64_t lo = (rec % nCc) * 64;
    const int32_t* e = r + rec * k;
    for (int64_t i = 0; i < k; ++i) {
      if (e[i] < lo || e[i] > lo + 63) return false;
      if (i > 0 && e[i] <= e[i - 1]) return false;
    }
  }
  return true;
}

constexpr int kMaxDecodeGroup = 16;  // query heads per KV head the decode kernels handle
static_assert(STILL_DECODE_NOALLOC_SCRATCH_BYTES == still::kDecodeScratchBytes, "the header states the scratch size");

constexpr int kMaxSplit = 64;        // workgroups per (b, KV head) over the compact cache
constexpr int kSplitTarget = 2048;   // aim for this many split workgroups per decode step

struct CacheLayout {
  size_t sel_k, sel_v, ring_k, ring_v, state_s, state_z, sel_mask, cur_sal, total;
  int64_t sel_capacity;  // compact rows per (b, KV head), a multiple of 64
};

CacheLayout cache_layout(const still_config* c, int64_t max_tokens) {
  const Dims d = dims_of(c);
  const size_t bh = static_cast<size_t>(c->batch) * d.Hr;  // routing-head records
  const size_t es = elem_bytes(c);
  const size_t D = c->head_dim, F = c->feat_dim;
  CacheLayout L;
  L.sel_capacity = odd_tiles(((max_tokens / 64) * c->top_k + 63) / 64) * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.sel_k = take(bh * L.sel_capacity * D * es);
  L.sel_v = take(bh * L.sel_capacity * D * es);
  const size_t nr = still::band_chunks(c->window) + 1;  // ring slots: chunks c-L .. c
  L.ring_k = take(bh * nr * 64 * D * es);
  L.ring_v = take(bh * nr * 64 * D * es);
  L.state_s = take(bh * F * D * sizeof(float));
  L.state_z = take(bh * F * sizeof(float));
  L.sel_mask = take(bh * nr * sizeof(uint64_t));
  L.cur_sal = take(bh * 64 * sizeof(float));
  L.total = off;
  return L;
}

int check_cache_cfg(const still_config* c, int64_t max_tokens) {
  const int st = check_cfg(c, false);
  if (st != STILL_OK) return st;
  if (max_tokens < 1 || max_tokens > 0x7fffffffLL) return STILL_ERR_INVALID_ARG;
  if (c->n_q_heads / c->n_kv_heads > kMaxDecodeGroup) return STILL_ERR_UNSUPPORTED;
  return STILL_OK;
}

bool same_layer(const still_config* a, const still_config* b) {
  return a->batch == b->batch && a->n_q_heads == b->n_q_heads && a->n_kv_heads == b->n_kv_heads &&
         a->head_dim == b->head_dim && a->feat_dim == b->feat_dim && a->window == b->window &&
         a->chunk == b->chunk && a->top_k == b->top_k && a->dtype == b->dtype && a->score == b->score &&
         a->routing_scope == b->routing_scope;
}

still::CacheView view_of(const still_cache* c) {
  still::CacheView v;
  v.sel_k = c->sel_k;
  v.sel_v = c->sel_v;
  v.ring_k = c->ring_k;
  v.ring_v = c->ring_v;
  v.state_s = c->state_s;
  v.state_z = c->state_z;
  v.sel_mask = c->sel_mask;
  v.cur_sal = c->cur_saliency;
  v.sel_tiles = static_cast<int>(c->sel_capacity / 64);
  return v;
}

size_t decode_ws_bytes(const still_config* c) {
  const size_t recs = static_cast<size_t>(c->batch) * c->n_kv_heads * kMaxSplit * (c->n_q_heads / c->n_kv_heads);
  return align_up(recs * 2 * sizeof(float)) + align_up(recs * c->head_dim * sizeof(float));
}

// ---- per-query-head routing: the layer on K, V and W_h expanded to one copy per query head
still_config expanded_cfg(const still_config* c) {
  still_config e = *c;
  e.n_kv_heads = c->n_q_heads;
  e.routing_scope = STILL_ROUTE_PER_KV_HEAD;
  return e;
}

struct ExpLayout {
  size_t ek, ev, ew, total;  // expanded K, V, W_h; the inner call's workspace starts at total
};

ExpLayout exp_layout(const still_config* c) {
  const size_t es = c->dtype == STILL_BF16 ? 2 : 4;
  const size_t rows = static_cast<size_t>(c->batch) * c->seq_len;
  ExpLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.ek = take(rows * c->n_q_heads * c->head_dim * es);
  L.ev = take(rows * c->n_q_heads * c->head_dim * es);
  L.ew = take(static_cast<size_t>(c->n_q_heads) * c->feat_dim * c->head_dim * es);
  L.total = off;
  return L;
}

hipError_t expand_kvw(const still_config* c, const void* k, const void* v, const void* w, char* ws, const ExpLayout& L,
                      hipStream_t stream) {
  const long long rows = static_cast<long long>(c->batch) * c->seq_len;
  const int G = c->n_q_heads / c->n_kv_heads;
  const long long es = c->dtype == STILL_BF16 ? 2 : 4;
  hipError_t e;
  if ((e = still::launch_expand_heads(k, ws + L.ek, rows, c->n_kv_heads, G, c->head_dim * es, stream)) != hipSuccess)
    return e;
  if ((e = still::launch_expand_heads(v, ws + L.ev, rows, c->n_kv_heads, G, c->head_dim * es, stream)) != hipSuccess)
    return e;
  return still::launch_expand_heads(w, ws + L.ew, 1, c->n_kv_heads, G,
                                    static_cast<long long>(c->feat_dim) * c->head_dim * es, stream);
}

// ---- backward workspace
struct BwdLayout {
  size_t kt, phik, phikt, ustate, ksel, vsel, kselt, qt, dot, phiq, phiqt, ld, apart, rstate, segsum, dwq, dwk,
      dkvsel, dwpart, total;
  int ntiles, nsplit, dw_parts;
};

int check_bwd_cfg(const still_config* c) {
  const int st = check_cfg(c, true);
  if (st != STILL_OK) return st;
  if (!still::bwd_shape_supported(c->dtype == STILL_BF16, c->head_dim, c->feat_dim)) return STILL_ERR_UNSUPPORTED;
  if (c->window > c->chunk) return STILL_ERR_UNSUPPORTED;  // the backward's band is chunks c-1 and c
  return STILL_OK;
}

BwdLayout bwd_layout(const still_config* c) {
  const Dims d = dims_of(c);
  const size_t bh = static_cast<size_t>(d.B) * d.Hkv, bhq = static_cast<size_t>(d.B) * d.Hq;
  const size_t es = elem_bytes(c), nC = d.nC, D = d.D, F = d.DF, R = d.R;
  BwdLayout L;
  // compact tiles per (b, KV head), odd like the prefill's (the padding tile's row group of
  // the selected-key kernel starts past the last chunk and does no steps)
  L.ntiles = static_cast<int>(odd_tiles((static_cast<int64_t>(d.nCc) * d.topk + 63) / 64));
  const int64_t far_wgs = static_cast<int64_t>(L.ntiles) * d.B * d.Hkv;
  // query slices per row group of the selected-key kernel: about 4096 workgroups in all, so
  // that the long row groups (the early compact rows see every later chunk) are split up,
  // and at most 16 partials for the local-key kernel to add
  L.nsplit = far_wgs > 0 ? static_cast<int>(std::min<int64_t>(16, std::max<int64_t>(1, (4096 + far_wgs - 1) / far_wgs))) : 1;
  const int64_t items = static_cast<int64_t>(d.B) * (d.G + 1) * d.nC;
  L.dw_parts = static_cast<int>(std::min<int64_t>(64, std::max<int64_t>(1, items / 16)));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.kt = take(bh * nC * 64 * D * es);
  L.phik = take(bh * nC * 64 * F * es);
  L.phikt = take(bh * nC * 64 * F * es);
  L.ustate = take(bh * nC * R * 4);
  L.ksel = take(bh * L.ntiles * 64 * D * es);
  L.vsel = take(bh * L.ntiles * 64 * D * es);
  L.kselt = take(bh * L.ntiles * 64 * D * es);
  L.qt = take(bhq * nC * 64 * D * es);
  L.dot = take(bhq * nC * 64 * D * es);
  L.phiq = take(bhq * nC * 64 * F * es);
  L.phiqt = take(bhq * nC * 64 * F * es);
  L.ld = take(bhq * nC * 64 * 2 * 4);
  // the shares of R and dW: one record per group of query heads that a dq wave takes
  const size_t bgq = bhq / static_cast<size_t>(still::bwd_heads_per_wave(c->dtype == STILL_BF16, d.G));
  L.apart = take(bgq * nC * R * 4);
  L.rstate = take(bh * nC * R * 4);
  L.segsum = take(bh * ((nC + 15) / 16) * R * 4);
  L.dwq = take(bgq * nC * F * D * 4);
  L.dwk = take(bh * nC * F * D * 4);
  L.dkvsel = take(static_cast<size_t>(L.nsplit) * bh * L.ntiles * 64 * 2 * D * 4);
  L.dwpart = take(static_cast<size_t>(L.dw_parts) * d.Hkv * F * D * 4);
  L.total = off;
  return L;
}

// ---- future attention mass workspace
constexpr int kMassChunksPerSlice = 16;

struct MassLayout {
  size_t lse, part, total;
  int nsplit, per;
};

MassLayout mass_layout(const still_config* c) {
  const Dims d = dims_of(c);
  MassLayout L;
  L.per = kMassChunksPerSlice;
  L.nsplit = (d.nC + L.per - 1) / L.per;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.lse = take(static_cast<size_t>(d.B) * d.Hq * d.nC * 64 * sizeof(float));
  L.part = take(static_cast<size_t>(L.nsplit) * d.B * d.Hkv * d.T * sizeof(float));
  L.total = off;
  return L;
}

int check_mass_cfg(const still_config* c) {
  const int st = check_cfg(c, true);
  if (st != STILL_OK) return st;
  if (c->head_dim != 64 || c->routing_scope != STILL_ROUTE_PER_KV_HEAD) return STILL_ERR_UNSUPPORTED;
  return STILL_OK;
}

}  // namespace

extern "C" {

const char* still_status_string(int status) {
  switch (status) {
    case STILL_OK: return "ok";
    case STILL_ERR_INVALID_ARG: return "invalid argument";
    case STILL_ERR_UNSUPPORTED: return "unsupported configuration";
    case STILL_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case STILL_ERR_CACHE_FULL: return "decode cache full";
    case STILL_ERR_CACHE_MISMATCH: return "decode cache built for another configuration";
    case STILL_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int still_last_hip_error(void) { return static_cast<int>(t_last_hip); }

int still_timing_event_create(hipEvent_t* out) {
  if (!out) return STILL_ERR_INVALID_ARG;
  STILL_HIP(hipEventCreateWithFlags(out, hipEventReleaseToDevice));
  return STILL_OK;
}

int still_timing_event_destroy(hipEvent_t ev) {
  if (!ev) return STILL_ERR_INVALID_ARG;
  STILL_HIP(hipEventDestroy(ev));
  return STILL_OK;
}

int still_timing_event_record(hipEvent_t ev, hipStream_t stream) {
  if (!ev) return STILL_ERR_INVALID_ARG;
  STILL_HIP(hipEventRecord(ev, stream));
  return STILL_OK;
}

int still_timing_event_elapsed_ms(hipEvent_t start, hipEvent_t end, float* ms) {
  if (!start || !end || !ms) return STILL_ERR_INVALID_ARG;
  STILL_HIP(hipEventElapsedTime(ms, start, end));
  return STILL_OK;
}

size_t still_prefill_workspace_bytes(const still_config* cfg) {
  if (check_cfg(cfg, true) != STILL_OK) return 0;
  return ws_layout(cfg).total;
}

int still_prefill_timed(const still_config* cfg, const void* q, const void* k, const void* v,
                        const void* w_phi, void* out, const int32_t* routing_in,
                        float* saliency_out, int32_t* sel_idx_out, still_cache* cache,
                        void* workspace, size_t ws_bytes, hipStream_t stream,
                        hipEvent_t* events) {
  const int st = check_cfg(cfg, true);
  if (st != STILL_OK) return st;
  if (!q || !k || !v || !w_phi || !out || !workspace) return STILL_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, w_phi, static_cast<const void*>(out), static_cast<const void*>(workspace)})
    if (!aligned(p, 16)) return STILL_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(routing_in), static_cast<const void*>(saliency_out),
                        static_cast<const void*>(sel_idx_out)})
    if (p && !aligned(p, 4)) return STILL_ERR_INVALID_ARG;
  if (saliency_out && cfg->window < 1) return STILL_ERR_INVALID_ARG;
  if (routing_in && cfg->top_k > 0 && !routing_valid(cfg, routing_in)) return STILL_ERR_INVALID_ARG;
  if (cache) {
    if (!same_layer(&cache->cfg, cfg)) return STILL_ERR_CACHE_MISMATCH;
    if (cache->n_tokens != 0) return STILL_ERR_INVALID_ARG;
    if (cfg->seq_len > cache->max_tokens) return STILL_ERR_CACHE_FULL;
  }
  const WsLayout L = ws_layout(cfg);
  if (ws_bytes < L.total) return STILL_ERR_WORKSPACE_TOO_SMALL;

  const Dims d = dims_of(cfg);
  char* ws = static_cast<char*>(workspace);
  still::PrepArgs pa;
  pa.d = d;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.w = w_phi;
  pa.routing_in = nullptr;
  if (routing_in && cfg->top_k > 0 && d.nCc > 0) {  // validated above; the prep kernel reads a device copy
    pa.routing_in = reinterpret_cast<const int32_t*>(ws + L.routing);
    STILL_HIP(hipMemcpyAsync(ws + L.routing, routing_in,
                             static_cast<size_t>(d.B) * d.Hr * d.nCc * d.topk * sizeof(int32_t),
                             hipMemcpyHostToDevice, stream));
  }
  pa.sal = saliency_out ? saliency_out : reinterpret_cast<float*>(ws + L.sal);
  pa.selmask = reinterpret_cast<uint64_t*>(ws + L.selmask);
  pa.sel_idx = sel_idx_out;
  pa.ksel = ws + L.ksel;
  pa.phik = ws + L.phik;
  pa.states = ws + L.states;
  pa.vT = ws + L.vT;
  pa.vselT = ws + L.vselT;
  pa.ntiles_sel = L.ntiles_sel;
  pa.kmaxc = reinterpret_cast<float*>(ws + L.kmaxc);
  pa.kall = reinterpret_cast<float*>(ws + L.kall);
  if (cache && cfg->top_k > 0) {  // the compact rows go straight into the cache
    pa.ksel = cache->sel_k;
    pa.vselT = cache->sel_v;
    pa.ntiles_sel = static_cast<int>(cache->sel_capacity / 64);
  }
  if (events && events[0]) STILL_HIP(hipEventRecord(events[0], stream));
  STILL_HIP(still::launch_prep(pa, stream));
  if (events && events[1]) STILL_HIP(hipEventRecord(events[1], stream));
  float* tilemax = reinterpret_cast<float*>(ws + L.tilemax);
  STILL_HIP(still::launch_scan(d, pa.states, pa.kmaxc, tilemax, L.ntiles_sel, stream));
  if (events && events[2]) STILL_HIP(hipEventRecord(events[2], stream));

  still::AttnArgs aa;
  aa.d = d;
  aa.q = q;
  aa.k = k;
  aa.w = w_phi;
  aa.selmask = pa.selmask;
  aa.ksel = pa.ksel;
  aa.vselT = pa.vselT;
  aa.vT = pa.vT;
  aa.phik = pa.phik;
  aa.states = pa.states;
  aa.out = out;
  aa.ntiles_sel = pa.ntiles_sel;
  aa.tilemax = tilemax;
  aa.kall = pa.kall;
  aa.tm_stride = L.ntiles_sel;
  aa.nw = d.Gr >= 4 ? 4 : (d.Gr == 3 ? 4 : d.Gr);  // query heads per workgroup: 1, 2 or 4
  aa.gsplit = (d.Gr + aa.nw - 1) / aa.nw;
  STILL_HIP(still::launch_attn(aa, stream));
  if (events && events[3]) STILL_HIP(hipEventRecord(events[3], stream));
  if (cache) {
    still::ExportArgs ea;
    ea.d = d;
    ea.k = k;
    ea.v = v;
    ea.sal = pa.sal;
    ea.selmask = pa.selmask;
    ea.states = pa.states;
    ea.c = view_of(cache);
    STILL_HIP(still::launch_cache_export(ea, stream));
    cache->n_tokens = cfg->seq_len;
  }
  return STILL_OK;
}

int still_prefill(const still_config* cfg, const void* q, const void* k, const void* v,
                  const void* w_phi, void* out, const int32_t* routing_in,
                  float* saliency_out, int32_t* sel_idx_out, still_cache* cache,
                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  return still_prefill_timed(cfg, q, k, v, w_phi, out, routing_in, saliency_out, sel_idx_out, cache,
                             workspace, ws_bytes, stream, nullptr);
}

int still_select_topk(const still_config* cfg, const float* saliency, int32_t* sel_idx_out,
                      hipStream_t stream) {
  const int st = check_cfg(cfg, true);
  if (st != STILL_OK) return st;
  if (!saliency || !sel_idx_out || !aligned(saliency, 4) || !aligned(sel_idx_out, 4)) return STILL_ERR_INVALID_ARG;
  const Dims d = dims_of(cfg);
  STILL_HIP(still::launch_topk(d, saliency, sel_idx_out, stream));
  return STILL_OK;
}

int still_feature_map(const still_config* cfg, const void* x, const void* w_phi, float* phi_out,
                      hipStream_t stream) {
  const int st = check_cfg(cfg, true);
  if (st != STILL_OK) return st;
  if (!x || !w_phi || !phi_out || !aligned(x, 16) || !aligned(w_phi, 16) || !aligned(phi_out, 4))
    return STILL_ERR_INVALID_ARG;
  const Dims d = dims_of(cfg);
  STILL_HIP(still::launch_feature_map(d, x, w_phi, phi_out, stream));
  return STILL_OK;
}

size_t still_cache_bytes(const still_config* cfg, int64_t max_tokens) {
  if (check_cache_cfg(cfg, max_tokens) != STILL_OK) return 0;
  return cache_layout(cfg, max_tokens).total;
}

int still_cache_init(const still_config* cfg, int64_t max_tokens, void* dev_buf, size_t bytes,
                     still_cache* out, hipStream_t stream) {
  const int st = check_cache_cfg(cfg, max_tokens);
  if (st != STILL_OK) return st;
  if (!dev_buf || !out || !aligned(dev_buf, 256)) return STILL_ERR_INVALID_ARG;
  const CacheLayout L = cache_layout(cfg, max_tokens);
  if (bytes < L.total) return STILL_ERR_WORKSPACE_TOO_SMALL;
  char* base = static_cast<char*>(dev_buf);
  still_cache c;
  memset(&c, 0, sizeof(c));
  c.cfg = *cfg;
  c.cfg.seq_len = 0;
  c.max_tokens = max_tokens;
  c.n_tokens = 0;
  c.sel_capacity = L.sel_capacity;
  c.sel_k = base + L.sel_k;
  c.sel_v = base + L.sel_v;
  c.ring_k = base + L.ring_k;
  c.ring_v = base + L.ring_v;
  c.state_s = reinterpret_cast<float*>(base + L.state_s);
  c.state_z = reinterpret_cast<float*>(base + L.state_z);
  c.sel_mask = reinterpret_cast<uint64_t*>(base + L.sel_mask);
  c.cur_saliency = reinterpret_cast<float*>(base + L.cur_sal);
  STILL_HIP(still::launch_fill_zero(dev_buf, L.total, stream));
  *out = c;
  return STILL_OK;
}

size_t still_decode_workspace_bytes(const still_config* cfg, int64_t max_tokens) {
  if (check_cache_cfg(cfg, max_tokens) != STILL_OK) return 0;
  return decode_ws_bytes(cfg);
}

}  // extern "C"

namespace {

// Checks of one decode step and its split plan (everything but the scratch of the partials).
int decode_plan(const still_config* cfg, const still_cache* cache, const void* q, const void* k, const void* v,
                const void* w_phi, void* out, still::DecodeArgs& a) {
  const int st = check_cfg(cfg, false);
  if (st != STILL_OK) return st;
  if (!cache || !q || !k || !v || !w_phi || !out) return STILL_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, w_phi, static_cast<const void*>(out)})
    if (!aligned(p, 16)) return STILL_ERR_INVALID_ARG;
  if (!same_layer(&cache->cfg, cfg)) return STILL_ERR_CACHE_MISMATCH;
  if (cfg->n_q_heads / cfg->n_kv_heads > kMaxDecodeGroup) return STILL_ERR_UNSUPPORTED;
  if (cache->n_tokens < 0 || cache->n_tokens >= cache->max_tokens) return STILL_ERR_CACHE_FULL;
  still_config c1 = *cfg;
  c1.seq_len = 1;
  a.d = dims_of(&c1);
  a.pos = cache->n_tokens;
  const int64_t chunk = cache->n_tokens / 64;
  const int bl = still::band_chunks(cfg->window);  // compact rows: chunks <= chunk - bl - 1
  a.nsel = static_cast<int>((chunk >= bl ? chunk - bl : 0) * cfg->top_k);
  const int ntiles = (a.nsel + 63) / 64;
  const int bhn = cfg->batch * a.d.Hr;
  int nsplit = (kSplitTarget + bhn - 1) / bhn;
  if (nsplit > kMaxSplit) nsplit = kMaxSplit;
  if (nsplit > ntiles) nsplit = ntiles;
  if (nsplit < 1) nsplit = 1;
  a.tiles_per_split = (ntiles + nsplit - 1) / nsplit;
  if (a.tiles_per_split < 1) a.tiles_per_split = 1;
  a.nsplit = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (a.nsplit < 1) a.nsplit = 1;
  a.q = q;
  a.k = k;
  a.v = v;
  a.w = w_phi;
  a.out = out;
  a.c = view_of(cache);
  return STILL_OK;
}

}  // namespace

extern "C" {

int still_decode_step_timed(const still_config* cfg, still_cache* cache, const void* q, const void* k,
                            const void* v, const void* w_phi, void* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  still::DecodeArgs a;
  const int st = decode_plan(cfg, cache, q, k, v, w_phi, out, a);
  if (st != STILL_OK) return st;
  if (!workspace || !aligned(workspace, 16)) return STILL_ERR_INVALID_ARG;
  if (ws_bytes < decode_ws_bytes(cfg)) return STILL_ERR_WORKSPACE_TOO_SMALL;
  const size_t recs = static_cast<size_t>(cfg->batch) * cfg->n_kv_heads * kMaxSplit * a.d.G;
  a.part_ml = static_cast<float*>(workspace);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(recs * 2 * sizeof(float)));
  if (events) STILL_HIP(hipEventRecord(events[0], stream));
  STILL_HIP(still::launch_decode(a, stream, events ? events[1] : nullptr));
  if (events) STILL_HIP(hipEventRecord(events[2], stream));
  cache->n_tokens += 1;
  return STILL_OK;
}

int still_decode_step_noalloc(const still_config* cfg, still_cache* cache, const void* q, const void* k,
                              const void* v, const void* w_phi, void* out, hipStream_t stream) {
  still::DecodeArgs a;
  const int st = decode_plan(cfg, cache, q, k, v, w_phi, out, a);
  if (st != STILL_OK) return st;
  // the partials of this call's splits only, at the front of the library's scratch
  const size_t recs = static_cast<size_t>(cfg->batch) * cfg->n_kv_heads * a.nsplit * a.d.G;
  const size_t ml_bytes = align_up(recs * 2 * sizeof(float));
  if (ml_bytes + recs * cfg->head_dim * sizeof(float) > still::kDecodeScratchBytes)
    return STILL_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  STILL_HIP(still::decode_scratch(&scratch));
  a.part_ml = static_cast<float*>(scratch);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(scratch) + ml_bytes);
  STILL_HIP(still::launch_decode(a, stream, nullptr));
  cache->n_tokens += 1;
  return STILL_OK;
}

int still_decode_step(const still_config* cfg, still_cache* cache, const void* q, const void* k,
                      const void* v, const void* w_phi, void* out, void* workspace,
                      size_t ws_bytes, hipStream_t stream) {
  return still_decode_step_timed(cfg, cache, q, k, v, w_phi, out, workspace, ws_bytes, stream, nullptr);
}

// per-query-head backward: after the expanded K, V, W_h, the copies' dk, dv, dW
struct ExpBwdLayout {
  ExpLayout x;
  size_t dk, dv, dw, total;
};

ExpBwdLayout exp_bwd_layout(const still_config* c) {
  ExpBwdLayout L;
  L.x = exp_layout(c);
  const size_t es = c->dtype == STILL_BF16 ? 2 : 4;
  const size_t kv = static_cast<size_t>(c->batch) * c->seq_len * c->n_q_heads * c->head_dim * es;
  size_t off = L.x.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.dk = take(kv);
  L.dv = take(kv);
  L.dw = take(static_cast<size_t>(c->n_q_heads) * c->feat_dim * c->head_dim * sizeof(float));
  L.total = off;
  return L;
}

size_t still_backward_workspace_bytes(const still_config* cfg) {
  if (check_bwd_cfg(cfg) != STILL_OK) return 0;
  if (cfg->routing_scope == STILL_ROUTE_PER_QUERY_HEAD) {
    const still_config e = expanded_cfg(cfg);
    if (check_bwd_cfg(&e) != STILL_OK) return 0;
    return exp_bwd_layout(cfg).total + bwd_layout(&e).total;
  }
  return bwd_layout(cfg).total;
}

int still_backward_timed(const still_config* cfg, const void* q, const void* k, const void* v,
                         const void* w_phi, const void* out, const void* dout, const int32_t* sel_idx,
                         void* dq, void* dk, void* dv, float* dw_phi, void* workspace, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t* events) {
  const int st = check_bwd_cfg(cfg);
  if (st != STILL_OK) return st;
  if (!q || !k || !v || !w_phi || !out || !dout || !dq || !dk || !dv || !dw_phi || !workspace)
    return STILL_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, w_phi, out, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv), static_cast<const void*>(dw_phi),
                        static_cast<const void*>(workspace)})
    if (!aligned(p, 16)) return STILL_ERR_INVALID_ARG;
  if (cfg->top_k > 0 && cfg->seq_len >= 64 && (!sel_idx || !aligned(sel_idx, 4))) return STILL_ERR_INVALID_ARG;
  if (cfg->routing_scope == STILL_ROUTE_PER_QUERY_HEAD) {
    const still_config e = expanded_cfg(cfg);
    const int se = check_bwd_cfg(&e);
    if (se != STILL_OK) return se;
    const ExpBwdLayout X = exp_bwd_layout(cfg);
    if (ws_bytes < X.total + bwd_layout(&e).total) return STILL_ERR_WORKSPACE_TOO_SMALL;
    char* ws = static_cast<char*>(workspace);
    STILL_HIP(expand_kvw(cfg, k, v, w_phi, ws, X.x, stream));
    const int rc = still_backward_timed(&e, q, ws + X.x.ek, ws + X.x.ev, ws + X.x.ew, out, dout, sel_idx, dq, ws + X.dk,
                                        ws + X.dv, reinterpret_cast<float*>(ws + X.dw), ws + X.total,
                                        ws_bytes - X.total, stream, events);
    if (rc != STILL_OK) return rc;
    const long long rows = static_cast<long long>(cfg->batch) * cfg->seq_len;
    const int G = cfg->n_q_heads / cfg->n_kv_heads;
    const int es = cfg->dtype == STILL_BF16 ? 2 : 4;
    STILL_HIP(still::launch_reduce_heads(ws + X.dk, dk, rows, cfg->n_kv_heads, G, cfg->head_dim, es, stream));
    STILL_HIP(still::launch_reduce_heads(ws + X.dv, dv, rows, cfg->n_kv_heads, G, cfg->head_dim, es, stream));
    STILL_HIP(still::launch_reduce_heads(ws + X.dw, dw_phi, 1, cfg->n_kv_heads, G, cfg->feat_dim * cfg->head_dim, 4,
                                         stream));
    return STILL_OK;
  }
  const BwdLayout L = bwd_layout(cfg);
  if (ws_bytes < L.total) return STILL_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  still::BwdArgs a;
  a.d = dims_of(cfg);
  a.q = q;
  a.k = k;
  a.v = v;
  a.w = w_phi;
  a.out = out;
  a.dout = dout;
  a.sel_idx = sel_idx;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = dw_phi;
  a.kt = ws + L.kt;
  a.phik = ws + L.phik;
  a.phikt = ws + L.phikt;
  a.ustate = reinterpret_cast<float*>(ws + L.ustate);
  a.ksel = ws + L.ksel;
  a.vsel = ws + L.vsel;
  a.kselt = ws + L.kselt;
  a.qt = ws + L.qt;
  a.dot = ws + L.dot;
  a.phiq = ws + L.phiq;
  a.phiqt = ws + L.phiqt;
  a.ld = reinterpret_cast<float*>(ws + L.ld);
  a.apart = reinterpret_cast<float*>(ws + L.apart);
  a.rstate = reinterpret_cast<float*>(ws + L.rstate);
  a.segsum = reinterpret_cast<float*>(ws + L.segsum);
  a.dwq = reinterpret_cast<float*>(ws + L.dwq);
  a.dwk = reinterpret_cast<float*>(ws + L.dwk);
  a.dkvsel = reinterpret_cast<float*>(ws + L.dkvsel);
  a.dwpart = reinterpret_cast<float*>(ws + L.dwpart);
  a.ntiles = L.ntiles;
  a.nsplit = L.nsplit;
  a.dw_parts = L.dw_parts;
  STILL_HIP(still::launch_bwd(a, stream, events));
  return STILL_OK;
}

int still_backward(const still_config* cfg, const void* q, const void* k, const void* v, const void* w_phi,
                   const void* out, const void* dout, const int32_t* sel_idx, void* dq, void* dk, void* dv,
                   float* dw_phi, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return still_backward_timed(cfg, q, k, v, w_phi, out, dout, sel_idx, dq, dk, dv, dw_phi, workspace, ws_bytes,
                              stream, nullptr);
}

size_t still_future_attention_mass_workspace_bytes(const still_config* cfg) {
  if (check_mass_cfg(cfg) != STILL_OK) return 0;
  return mass_layout(cfg).total;
}

int still_future_attention_mass(const still_config* cfg, const void* q, const void* k, float* mass_out,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  const int st = check_mass_cfg(cfg);
  if (st != STILL_OK) return st;
  if (!q || !k || !mass_out || !workspace) return STILL_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(mass_out, 4) || !aligned(workspace, 16))
    return STILL_ERR_INVALID_ARG;
  const MassLayout L = mass_layout(cfg);
  if (ws_bytes < L.total) return STILL_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  still::MassArgs a;
  a.d = dims_of(cfg);
  a.q = q;
  a.k = k;
  a.lse = reinterpret_cast<float*>(ws + L.lse);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.mass = mass_out;
  a.nsplit = L.nsplit;
  a.per = L.per;
  STILL_HIP(still::launch_mass(a, stream));
  return STILL_OK;
}

int still_selection_overlap(const still_config* cfg, const int32_t* sel_a, const int32_t* sel_b,
                            int32_t* common_out, hipStream_t stream) {
  const int st = check_cfg(cfg, true);
  if (st != STILL_OK) return st;
  const Dims d = dims_of(cfg);
  if (d.nCc == 0 || d.topk == 0) return STILL_OK;
  if (!sel_a || !sel_b || !common_out || !aligned(sel_a, 4) || !aligned(sel_b, 4) || !aligned(common_out, 4))
    return STILL_ERR_INVALID_ARG;
  STILL_HIP(still::launch_overlap(d, sel_a, sel_b, common_out, stream));
  return STILL_OK;
}

}  // extern "C"

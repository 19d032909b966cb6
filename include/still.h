/*
 * still.h -- C ABI of an MI355X (gfx950) implementation of one STILL intra-layer hybrid
 * attention layer: self-saliency routing, softmax attention over the local window plus
 * the routed tokens, NP-Map linear attention over every other past token, one fused
 * output.
 *
 * Pages that define the operation:
 *   [P1] "仅0.04B！哈工深首创同层混合架构STILL，极低成本线性化LLM" (PaperWeekly repost):
 *        sections "Self-Saliency Score", "Norm-Preserved Feature Map（NP-Map）",
 *        "Chunk-Wise并行+延迟选择", and the paragraph before "STILL三大创新".
 *   [P2] "STILL: Content-Aware Intra-Layer Hybrid Attention Cuts Memory 80%, Speeds
 *        Prefill 83%" (picx.dev), summary and the 机器之心 excerpt.
 *   [P3] "STILL от HIT Shenzhen: гибридное внимание внутри слоя выбирает токены по
 *        содержанию" (news piece), on the fixed-size state of linear attention.
 *   [P4] "STILL: Selecting Tokens for Intra-Layer Hybrid Attention to Linearize LLMs"
 *        (research-map summary), sections Approach and "Surprising findings".
 * The sources under linear_attention_saliency_amd/csrc cite these labels.
 *
 * The pages leave these points open; the library fixes them as follows.
 *   window      W_i = {max(0, i-w+1) .. i}, causal, contains i.
 *   logits      a_ij = q_i . k_j / sqrt(head_dim), for saliency and the softmax branch.
 *   saliency    s_i = KL(no-diagonal window softmax || window softmax) = -log(1 - p_ii),
 *               +inf for a one-token window; per KV head, the G = n_q_heads/n_kv_heads
 *               query heads of the group are summed in order g = 0..G-1 (query head hq
 *               belongs to KV head hq / G).
 *   routing     each complete chunk of `chunk` tokens selects its top_k tokens by s, ties
 *               to the lower position; the selection is used only by later chunks; an
 *               incomplete final chunk is never selected.
 *   partition   key j <= i is in query i's softmax set iff j > i - w, or j lies in an
 *               earlier chunk and was selected; all other keys go to linear attention.
 *   NP-Map      phi(x) = |x| * m / |m|, m = elu(W_h x) + 1 (alpha 1), W_h [feat_dim,
 *               head_dim] per KV head, shared by queries and keys.
 *   output      o_i = (sum_SA e^{a_ij} v_j + sum_LA (phi(q_i).phi(k_j)) v_j)
 *                     / (sum_SA e^{a_ij} + sum_LA phi(q_i).phi(k_j))     (shared normaliser);
 *               0 if the denominator is 0 (only possible with window 0 and q_i = 0).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are device memory owned by the caller, 16-byte aligned, contiguous
 *     in the stated layout, and are not retained after the call returns.
 *   - The library never allocates device memory and never synchronises: all work is
 *     enqueued on `stream`, so results are ready when the stream reaches them.
 *   - Validation errors are returned before anything is enqueued, and no output is
 *     touched. STILL_ERR_HIP means a HIP call or launch failed; outputs are then undefined,
 *     and still_last_hip_error() names the hipError_t.
 *   - There is no shared mutable state (only the per-thread record of the last HIP error):
 *     calls on distinct streams with distinct workspaces and caches may run concurrently.
 *     Calls sharing a workspace or cache must be ordered.
 */
#ifndef STILL_H
#define STILL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, w_phi and out. */
typedef enum still_dtype { STILL_F32 = 0, STILL_BF16 = 1 } still_dtype;

/* Routing score of a token (the value each chunk's top_k is taken on):
 *   STILL_SCORE_SALIENCY  the Self-Saliency Score above ([P1] section "Self-Saliency Score");
 *   STILL_SCORE_DIAG      the diagonal logit alone, s_i = sum_g q_{g,i} . k_i / sqrt(head_dim):
 *                         the pages' ablation that routes by the diagonal attention without
 *                         the rest of the window ([P4] section "Surprising findings"). Routing by the diagonal
 *                         softmax weight p_ii itself would select exactly the saliency's
 *                         tokens, since -log(1 - p_ii) grows with p_ii; the raw logit is the
 *                         reading that differs. */
typedef enum still_score { STILL_SCORE_SALIENCY = 0, STILL_SCORE_DIAG = 1 } still_score;

/* Who selects ([P1] section "Chunk-Wise并行+延迟选择" selects per chunk; the pages do not say
 * per which head):
 *   STILL_ROUTE_PER_KV_HEAD     every KV head selects once, on the sum of its query heads'
 *                               scores; the selection is shared by the group (default);
 *   STILL_ROUTE_PER_QUERY_HEAD  every query head selects on its own score and has its own
 *                               softmax cache and linear-attention state. The library runs
 *                               the layer on keys, values and NP-Map weights expanded to one
 *                               copy per query head (in the workspace) and, in the backward
 *                               pass, sums the copies' gradients over each group. Prefill and
 *                               backward only (no decode cache); saliency_out and sel_idx are
 *                               then per query head ([batch, n_q_heads, ...]). */
typedef enum still_routing_scope { STILL_ROUTE_PER_KV_HEAD = 0, STILL_ROUTE_PER_QUERY_HEAD = 1 } still_routing_scope;

/* Status codes (0 = success). */
enum {
  STILL_OK = 0,
  STILL_ERR_INVALID_ARG = -1,         /* null / misaligned pointer, inconsistent sizes */
  STILL_ERR_UNSUPPORTED = -2,         /* valid layer, but not a shape these kernels cover */
  STILL_ERR_WORKSPACE_TOO_SMALL = -3,
  STILL_ERR_CACHE_FULL = -4,          /* decode cache holds max_tokens tokens already */
  STILL_ERR_CACHE_MISMATCH = -5,      /* cache built for another configuration */
  STILL_ERR_HIP = -6
};

/* Layer configuration. Supported by the kernels: chunk = 64; head_dim in {64, 128};
 * feat_dim in {64, 128}; 0 <= window <= 2 * chunk (a window longer than a chunk reaches into
 * L = ceil(window / chunk) earlier chunks, which the kernels take with per-query masks; a
 * decode cache then holds L + 1 chunks of raw rows); 0 <= top_k <= chunk; top_k = 0 when
 * window = 0; n_q_heads a multiple of n_kv_heads; seq_len >= 1, with the chunk states of
 * one (batch, KV head), ceil(seq_len/64) * (head_dim*feat_dim + feat_dim) elements of the
 * layer's dtype, under 2 GiB (about 16M tokens at 64/64 and 4M at 128/128 in bf16).
 * Both dtypes cover every head_dim / feat_dim pair (fp32 is the reference-precision path). */
typedef struct still_config {
  int32_t batch;
  int32_t seq_len;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t feat_dim;
  int32_t window;
  int32_t chunk;
  int32_t top_k;
  int32_t dtype; /* still_dtype */
  int32_t score; /* still_score; 0 = the Self-Saliency Score */
  int32_t routing_scope; /* still_routing_scope; 0 = per KV head */
} still_config;

/* Decode state for batched token-by-token generation with chunk-delayed selection
 * ([P1] section "Chunk-Wise并行+延迟选择"). A host-side record of device sub-buffers
 * carved from one caller buffer by still_cache_init. Fields are read-only for callers.
 * With c the chunk of the next token: sel_k/sel_v hold the selected rows of chunks
 * <= c-2 in (chunk, position) order (compact row n = chunk * top_k + rank; rows of later
 * chunks may already be present and are not read); ring_k/ring_v hold the raw rows of
 * chunks c-1 and c (chunk j in slot j % 2); state_s/state_z hold the linear-attention
 * state sum phi(k) v^T and sum phi(k) over the unselected tokens of chunks <= c-2.
 * sel_v is stored transposed in tiles of 64 compact rows: element (row n, dim d) is at
 * [((n / 64) * head_dim + d) * 64 + p(n % 64)], where p(j) = (j & ~31) + 8*((j & 15) >> 2)
 * + 4*((j >> 4) & 1) + (j & 3) orders each 32-row slice as the MFMA accumulator holds it.
 * Supported for n_q_heads / n_kv_heads <= 16. */
typedef struct still_cache {
  still_config cfg;     /* configuration the cache was built for (seq_len ignored) */
  int64_t max_tokens;   /* capacity per sequence */
  int64_t n_tokens;     /* tokens held per sequence = position of the next token */
  int64_t sel_capacity; /* compact rows per (batch, KV head), a multiple of 64 */
  void* sel_k;          /* [batch, n_kv_heads, sel_capacity, head_dim] dtype: the selected key
                           rows as given */
  void* sel_v;          /* [batch, n_kv_heads, sel_capacity / 64, head_dim, 64] dtype */
  void* ring_k;         /* [batch, n_kv_heads, 2, chunk, head_dim] dtype */
  void* ring_v;         /* [batch, n_kv_heads, 2, chunk, head_dim] dtype */
  float* state_s;       /* [batch, n_kv_heads, feat_dim, head_dim] fp32 */
  float* state_z;       /* [batch, n_kv_heads, feat_dim] fp32 */
  uint64_t* sel_mask;   /* [batch, n_kv_heads, 2] selection bit masks of ring slots */
  float* cur_saliency;  /* [batch, n_kv_heads, chunk] saliency of the current chunk */
} still_cache;

/* Human-readable name of a status code (static storage). */
const char* still_status_string(int status);

/* The hipError_t (as an int) of the HIP call or launch behind the last STILL_ERR_HIP that any
 * entry point returned on the calling thread; 0 (hipSuccess) if none has. Not cleared by
 * later successful calls. */
int still_last_hip_error(void);

/* Bytes of scratch still_prefill needs for `cfg` (0 if cfg is invalid). */
size_t still_prefill_workspace_bytes(const still_config* cfg);

/* One causal STILL layer over a whole sequence (prefill).
 *   q      [batch, seq_len, n_q_heads, head_dim]   dtype
 *   k, v   [batch, seq_len, n_kv_heads, head_dim]  dtype   (post-RoPE keys/values)
 *   w_phi  [n_kv_heads, feat_dim, head_dim]        dtype   (NP-Map weight per KV head)
 *   out    [batch, seq_len, n_q_heads, head_dim]   dtype   (written, RNE for bf16)
 *   routing_in    optional HOST memory, [batch, n_kv_heads, seq_len/chunk, top_k] int32
 *                 ([batch, n_q_heads, ...] with per-query-head routing): if non-null, these
 *                 positions replace the score's selection (an override for testing the
 *                 attention alone). Every chunk c's top_k entries must be strictly ascending
 *                 and lie in [64 c, 64 c + 63]; otherwise STILL_ERR_INVALID_ARG, before
 *                 anything is enqueued. The array is read during the call and copied into the
 *                 workspace on `stream` (from pageable memory that copy may wait for the
 *                 stream's earlier work); it is not retained.
 *   saliency_out  optional [batch, n_kv_heads, seq_len] fp32: the group-summed saliency
 *                 (requires window >= 1).
 *   sel_idx_out   optional [batch, n_kv_heads, seq_len/chunk, top_k] int32: the selected
 *                 positions of every complete chunk, ascending.
 *   cache         optional: if non-null, a cache from still_cache_init for this layer
 *                 (CACHE_MISMATCH otherwise) with n_tokens == 0 (INVALID_ARG otherwise) and
 *                 max_tokens >= seq_len (CACHE_FULL otherwise); it is left holding the state
 *                 after seq_len tokens, ready for still_decode_step.
 *   workspace     device scratch of at least still_prefill_workspace_bytes(cfg) bytes.
 * Returns STILL_OK or a negative status. */
int still_prefill(const still_config* cfg, const void* q, const void* k, const void* v,
                  const void* w_phi, void* out, const int32_t* routing_in,
                  float* saliency_out, int32_t* sel_idx_out, still_cache* cache,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* still_prefill with timing events: if `events` is non-null it must hold 4 entries, each an
 * event created by the caller or null (not recorded); they are recorded on `stream` before
 * the per-chunk preparation kernel, before the chunk-state scan, before the fused attention
 * kernel and after it, so hipEventElapsedTime between consecutive events gives each kernel's
 * duration. */
int still_prefill_timed(const still_config* cfg, const void* q, const void* k, const void* v,
                        const void* w_phi, void* out, const int32_t* routing_in,
                        float* saliency_out, int32_t* sel_idx_out, still_cache* cache,
                        void* workspace, size_t ws_bytes, hipStream_t stream,
                        hipEvent_t* events);

/* The per-chunk top-k alone: saliency [batch, n_kv_heads, seq_len] fp32 (device) ->
 * sel_idx_out [batch, n_kv_heads, seq_len/chunk, top_k] int32, ascending positions,
 * ties to the lower position ([P1] section "Chunk-Wise并行+延迟选择"). */
int still_select_topk(const still_config* cfg, const float* saliency, int32_t* sel_idx_out,
                      hipStream_t stream);

/* The NP-Map alone ([P1] section "Norm-Preserved Feature Map（NP-Map）"; [P4] section
 * Approach): x [batch, seq_len, n_kv_heads, head_dim] dtype -> phi_out [batch, seq_len,
 * n_kv_heads, feat_dim] fp32, with W_h = w_phi[h]. */
int still_feature_map(const still_config* cfg, const void* x, const void* w_phi,
                      float* phi_out, hipStream_t stream);

/* Bytes of device memory a decode cache of `max_tokens` tokens per sequence needs
 * (0 if the configuration is invalid or unsupported; cfg->seq_len is ignored). */
size_t still_cache_bytes(const still_config* cfg, int64_t max_tokens);

/* Carve a cache from `dev_buf` (256-byte aligned, >= still_cache_bytes bytes, owned by the
 * caller for the cache's lifetime) and clear it on `stream`. Fills *out; n_tokens starts
 * at 0. A cache is filled either by still_prefill (cache argument) or token by token. */
int still_cache_init(const still_config* cfg, int64_t max_tokens, void* dev_buf,
                     size_t bytes, still_cache* out, hipStream_t stream);

/* Bytes of scratch still_decode_step needs for `cfg` and a cache of max_tokens. */
size_t still_decode_workspace_bytes(const still_config* cfg, int64_t max_tokens);

/* One generated token for every sequence of the batch, all at position cache->n_tokens
 * ([P1] section "Chunk-Wise并行+延迟选择": selection delayed to chunk granularity).
 *   q [batch, n_q_heads, head_dim], k/v [batch, n_kv_heads, head_dim], out like q.
 * The token's saliency is accumulated; when it completes its chunk, that chunk's top_k
 * tokens are chosen and the chunk before it is folded: selected rows are appended to the
 * softmax cache, the others join the linear-attention state. cfg->seq_len is ignored.
 * Advances cache->n_tokens by one on success. */
int still_decode_step(const still_config* cfg, still_cache* cache, const void* q,
                      const void* k, const void* v, const void* w_phi, void* out,
                      void* workspace, size_t ws_bytes, hipStream_t stream);

/* still_decode_step with timing events: if `events` is non-null it must hold 3 events
 * created by the caller, recorded before the compact-cache kernel, before the per-token
 * kernel and after it. */
int still_decode_step_timed(const still_config* cfg, still_cache* cache, const void* q,
                            const void* k, const void* v, const void* w_phi, void* out,
                            void* workspace, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t* events);

/* Size of the library's own decode scratch (bytes), the limit of still_decode_step_noalloc. */
#define STILL_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* still_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same step, with no
 * workspace argument. The split partials go to a scratch array the library holds in device
 * memory, one copy per GPU, from the first call on that GPU until the process ends; no HIP
 * allocating routine is called. A call needs 8 * n + 4 * head_dim * n bytes of it (n =
 * batch * n_kv_heads * n_q_heads/n_kv_heads * splits, splits <= 64, chosen as in
 * still_decode_step), at most STILL_DECODE_NOALLOC_SCRATCH_BYTES; a larger step returns
 * STILL_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the 32 x 64K Llama-3.1-8B-shaped
 * decode needs 4.3 MB). Every call on one GPU shares the one scratch: calls that overlap on
 * one GPU (different streams or threads) race, and must be ordered by the caller. Nothing in
 * the scratch has to start at zero (each call writes its partials before reading them).
 * Results are those of still_decode_step. */
int still_decode_step_noalloc(const still_config* cfg, still_cache* cache, const void* q,
                              const void* k, const void* v, const void* w_phi, void* out,
                              hipStream_t stream);

/* Timing events for the *_timed entry points and for callers that time the library's work.
 * They are created with a device-scope release (hipEventReleaseToDevice): recording one
 * between two kernels does not write back and invalidate the caches at system scope, which a
 * default event does and which would slow the kernel that follows and lengthen the measured
 * interval. An elapsed time is valid once the caller has synchronised with the work (device
 * or stream synchronisation); the events order nothing for other devices or the host.
 * Each returns STILL_OK, STILL_ERR_INVALID_ARG for a null pointer, or STILL_ERR_HIP. */
int still_timing_event_create(hipEvent_t* out);
int still_timing_event_destroy(hipEvent_t ev);
int still_timing_event_record(hipEvent_t ev, hipStream_t stream);
int still_timing_event_elapsed_ms(hipEvent_t start, hipEvent_t end, float* ms);

/* Bytes of scratch still_backward needs for `cfg` (0 if cfg is invalid or unsupported). */
size_t still_backward_workspace_bytes(const still_config* cfg);

/* Backward pass of one layer with the routing held fixed: the gradients of sum(out * dout)
 * ([P1] section "Chunk-Wise并行+延迟选择" and [P4] section Approach: the chunked layer is
 * also the training form). The routing is piecewise constant in q and k, so it carries no
 * gradient; it is passed in as the selection the forward pass made.
 *   q, k, v, w_phi  as still_prefill (dtype)
 *   out      [batch, seq_len, n_q_heads, head_dim] dtype: the forward output for these inputs
 *            and this routing (it gives Delta_i = dout_i . out_i)
 *   dout     [batch, seq_len, n_q_heads, head_dim] dtype
 *   sel_idx  [batch, n_kv_heads, seq_len/chunk, top_k] int32 device memory: for every complete
 *            chunk, top_k distinct positions inside that chunk, in any order, as still_prefill's
 *            sel_idx_out writes them (may be null if top_k = 0 or seq_len < chunk). The entries
 *            are not checked (they live on the device); repeated or out-of-chunk entries give
 *            undefined gradients.
 *   dq       like q; dk, dv like k (dtype, written)
 *   dw_phi   [n_kv_heads, feat_dim, head_dim] fp32 (written, not accumulated)
 *   workspace  device scratch of at least still_backward_workspace_bytes(cfg) bytes.
 * Supported for head_dim = feat_dim = 64 (both dtypes) and head_dim = feat_dim = 128 (bf16),
 * window <= chunk; STILL_ERR_UNSUPPORTED otherwise. Every sum runs in a fixed order, so repeated calls give
 * identical bits. Rows whose normaliser is 0 (output
 * 0) get no gradient. Returns STILL_OK or a negative status. */
int still_backward(const still_config* cfg, const void* q, const void* k, const void* v,
                   const void* w_phi, const void* out, const void* dout, const int32_t* sel_idx,
                   void* dq, void* dk, void* dv, float* dw_phi, void* workspace, size_t ws_bytes,
                   hipStream_t stream);

/* still_backward with timing events: if `events` is non-null it must hold 8 events created by
 * the caller, recorded before each of the seven stages (key preparation, linear-attention state
 * scan, dq, reverse state scan, selected keys, local keys, dW reduction) and after the last. */
int still_backward_timed(const still_config* cfg, const void* q, const void* k, const void* v,
                         const void* w_phi, const void* out, const void* dout, const int32_t* sel_idx,
                         void* dq, void* dk, void* dv, float* dw_phi, void* workspace, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t* events);

/* Bytes of scratch still_future_attention_mass needs (0 if cfg is invalid or unsupported). */
size_t still_future_attention_mass_workspace_bytes(const still_config* cfg);

/* Attention each key receives from far-future queries under full causal softmax, the global
 * reference for the routing's local-global consistency ([P2]: the local score is meant to
 * predict whether a token is still attended once it is far history; [P1] section
 * "Self-Saliency Score"). For KV head h and key j:
 *   mass_out[b, h, j] = sum over the group's query heads and over queries i >= j + window of
 *                       softmax_{l <= i}(q_i . k_l / sqrt(head_dim))_j
 *   q [batch, seq_len, n_q_heads, head_dim], k [batch, seq_len, n_kv_heads, head_dim] (dtype);
 *   mass_out [batch, n_kv_heads, seq_len] fp32 (written).
 * Supported for head_dim = 64 (feat_dim and top_k are not used). Sums run in a fixed order. */
int still_future_attention_mass(const still_config* cfg, const void* q, const void* k, float* mass_out,
                                void* workspace, size_t ws_bytes, hipStream_t stream);

/* Tokens two per-chunk selections share: sel_a, sel_b [batch, n_kv_heads, seq_len/chunk,
 * top_k] int32 -> common_out [batch, n_kv_heads, seq_len/chunk] int32 (with still_select_topk
 * on the mass above, the overlap of the routing with the global choice). */
int still_selection_overlap(const still_config* cfg, const int32_t* sel_a, const int32_t* sel_b,
                            int32_t* common_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STILL_H */

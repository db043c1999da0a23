/*
 * prism.h -- C ABI of the MI355X (gfx950) library for token-sparse GQA decode
 * attention with proposal-refined cross-layer index sharing.
 *
 * The operations follow "Prism Attention: Proposal-Refined Index Sharing
 * Mechanism for Efficient LLMs Inference" (arXiv 2610.22985):
 *   - relevance of a cached token to the step's query: Eq. 1 with phi given by
 *     Eq. 9, the maximum over the KV head's group of query heads of <q_j, k_i>
 *     (on the bf16 keys, or on the INT2 keys when the cache carries them);
 *   - exact top-kappa selection: Eq. 2 (anchor / proposal layers);
 *   - refinement inside a candidate pool: Eqs. 5-6 (refined layers), where the
 *     pool is either the union of [i - w, i + w] (clipped to the sequence) over
 *     the anchor layer's selected positions i (window pool), or the anchor
 *     layer's own rho*kappa most relevant tokens (rank-expanded pool, Eq. 4);
 *   - SparseAttn of Algorithm 1: softmax attention of every query head over
 *     its KV head's selected tokens only;
 *   - optional INT2 proposal keys (Section 4.2, Eqs. 7-9), layer roles
 *     (Algorithm 1's proposal / refined partition, the shared layers of
 *     Appendix E) and dense decode over the whole cache.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer unless marked host.  The
 *     caller owns every buffer; the library allocates no device memory and
 *     keeps no state between calls (besides the optional benchmark event
 *     rings and a per-device cache of the compute-unit count).
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without synchronising.  Arguments are validated on the host
 *     before anything is enqueued; an invalid call enqueues nothing.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Selected index sets are token positions in ascending order, without
 *     duplicates; ties in relevance go to the lower position.
 *   - No exception or abort crosses the ABI; failures return a negative
 *     prism_status and prism_last_error() describes the most recent one on
 *     the calling thread.
 *   - Supported shapes: head_dim 128, page_size 64, group size
 *     G = num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}, 1 <= kappa <= 8192,
 *     max_seq_len <= 262144.  Anything else returns PRISM_ERR_UNSUPPORTED.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PRISM_ABI_VERSION 7

#if defined(__GNUC__) || defined(__clang__)
#define PRISM_API __attribute__((visibility("default")))
#else
#define PRISM_API
#endif

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes, kappa out of range ... */
  PRISM_ERR_UNSUPPORTED = -2, /* valid but outside the supported shapes listed above     */
  PRISM_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or smaller than required  */
  PRISM_ERR_HIP = -4          /* no usable GPU, or a HIP call / kernel launch failed     */
} prism_status;

/*
 * Paged KV cache of ONE layer (the historical keys K and values of Section
 * 4.1).  Layout, all row-major:
 *   k_pages, v_pages : bf16 [num_pages][num_kv_heads][page_size][head_dim],
 *                      16-byte aligned; token t of sequence b, KV head g is
 *                      row (t % page_size) of physical page
 *                      block_table[b][t / page_size], head g.
 *   block_table      : int32 [batch][max_pages_per_seq]; only the first
 *                      ceil(seq_lens[b] / page_size) entries of a row are read;
 *                      entries are physical page ids in [0, num_pages).
 *   seq_lens         : int32 [batch]; tokens 0 .. seq_lens[b]-1 are attendable
 *                      (the current token is already in the cache).
 *   k_codes, k_scales: optional INT2 proposal keys ("Prism Attention", Section
 *                      4.2, Eqs. 7-8), both NULL or both set, 16-byte aligned,
 *                      paged exactly like k_pages (same page ids and rows):
 *     k_codes  uint8 [num_pages][num_kv_heads][page_size][32]: the 128 two-bit
 *              codes of a key row.  The code of dimension d = 32 s + 8 u + j
 *              (group s, quarter u, element j, all from 0) is in the row's
 *              little-endian 32-bit word 2 u + s / 2, at bit
 *              2 (4 (s % 2) + j / 2) + 16 (j % 2).
 *     k_scales bf16 [num_pages][num_kv_heads][page_size][4][2]: per group of 32
 *              dimensions, its scale alpha and zero point beta.
 *              The key the row stands for is alpha_s * code + beta_s.
 *   When set, relevance (Eq. 9) at anchor and refined layers is computed from
 *   them instead of k_pages (attention always reads k_pages and v_pages);
 *   prism_quantize_keys writes them.
 *   new_keys     0 <= new_keys <= 64 (every call but prism_quantize_keys
 *                rejects other values), used only with k_codes: the key rows of
 *                positions [max(0, seq_lens[b] - new_keys), seq_lens[b]) of
 *                every sequence and KV head were just appended (a decode step
 *                appends one) and have no codes yet.  prism_score_topk,
 *                prism_refine_topk, prism_decode_layer and
 *                prism_decode_layer_role then write their codes and scales,
 *                exactly as prism_quantize_keys(kv, new_keys, ...) would,
 *                before they score them: inside the scoring kernel, or, for a
 *                shared layer (which scores nothing), in extra workgroups of
 *                its attention launch.  A refined layer writes them whether
 *                or not they are in its pool.  prism_sparse_attn and
 *                prism_dense_attn never read the codes and write none.
 * Host integers: min_seq_len <= seq_lens[b] <= max_seq_len must hold for all b
 * and max_seq_len <= max_pages_per_seq * page_size.  The library cannot check
 * the device arrays; kernels clamp every length and position so that
 * inconsistent contents give wrong results, never out-of-bounds accesses.
 */
typedef struct {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;          /* physical pages in k_pages / v_pages */
  int32_t max_pages_per_seq;
  int32_t max_seq_len;
  int32_t min_seq_len;
  uint8_t* k_codes;           /* optional INT2 codes, see above (NULL: bf16 keys) */
  uint16_t* k_scales;         /* optional INT2 (alpha, beta) per group           */
  int32_t new_keys;           /* trailing positions still without codes          */
} prism_kv_cache;

/*
 * kappa          sparse budget per KV head (Eq. 2); 1 <= kappa <= min_seq_len.
 * anchor_stride  layer l is an anchor (proposal) layer iff l % anchor_stride == 0;
 *                every other layer is refined against the nearest preceding
 *                anchor (the association f of Section 4.1).  >= 1.
 * window         w >= 0 of the window pool [i - w, i + w] (unused when pool_rho >= 1).
 * softmax_scale  logit scale of SparseAttn; 0 selects 1/sqrt(head_dim).
 * pool_rho       0: the refined layers' pool is the window pool.  rho >= 1: it is
 *                the anchor layer's top min(rho * kappa, L) tokens by relevance
 *                (Eq. 4, the rank-expanded pool); the anchor attends its own
 *                top-kappa, which lies inside it.  rho * kappa <= 32768.
 * Query head j belongs to KV head j / G.
 */
typedef struct {
  int32_t num_q_heads;
  int32_t kappa;
  int32_t anchor_stride;
  int32_t window;
  float softmax_scale;
  int32_t pool_rho;
} prism_params;

/* Bytes of device workspace every compute entry point needs for these shapes
 * (0 when the arguments are invalid).  The workspace must be 256-byte aligned;
 * its contents need no initialisation.  Besides scratch it carries one piece
 * of state: the refinement pool that the latest anchor-layer selection
 * (prism_score_topk, or prism_decode_layer at an anchor layer) derived from
 * the set it wrote, which prism_decode_layer's refined layers re-score (the
 * candidate cache of Algorithm 1).  Calls that run concurrently must not share
 * a workspace. */
PRISM_API size_t prism_workspace_size(const prism_kv_cache* kv, const prism_params* params);

/*
 * Anchor (proposal) layer selection: Eq. 9 relevance of EVERY cached token,
 * then the exact top-kappa of Eq. 2, per (sequence, KV head).
 *   q          bf16 [batch][num_q_heads][head_dim], 16-byte aligned.
 *   idx_out    int32 [batch][num_kv_heads][kappa]: ascending positions.
 *   scores_out optional (NULL to skip), float [batch][num_kv_heads][max_seq_len]:
 *              the fp32 relevance of every token (entries past seq_lens[b]
 *              are unspecified).  For checking only; costs an extra copy.
 */
PRISM_API prism_status prism_score_topk(const prism_kv_cache* kv, const uint16_t* q,
                              const prism_params* params, int32_t* idx_out, float* scores_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Refined layer selection (Eqs. 5-6): build the pool from the anchor's set,
 * score only the pool's tokens (Eq. 9), keep the top-kappa.
 *   anchor_idx    int32 [batch][num_kv_heads][kappa]: the anchor layer's sets,
 *                 ascending (as prism_score_topk writes them).  With pool_rho >= 1
 *                 the pool cannot be rebuilt from the set: the call re-scores the
 *                 pool that the latest anchor-layer selection left in the
 *                 workspace, and anchor_idx may be NULL (it is not read).
 *   idx_out       int32 [batch][num_kv_heads][kappa]: ascending positions.
 *   pool_out      optional int32 [batch][num_kv_heads][max_seq_len]: the pool's
 *                 positions, ascending, first pool_len_out[b][g] entries valid.
 *   pool_len_out  optional int32 [batch][num_kv_heads].
 *   pool_scores_out optional float [batch][num_kv_heads][max_seq_len]: fp32
 *                 relevance of pool entry e (same order as pool_out).
 */
PRISM_API prism_status prism_refine_topk(const prism_kv_cache* kv, const uint16_t* q,
                               const prism_params* params, const int32_t* anchor_idx,
                               int32_t* idx_out, int32_t* pool_out, int32_t* pool_len_out,
                               float* pool_scores_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * SparseAttn (Algorithm 1): for every query head j of KV head g,
 *   out[b][j] = sum_{i in idx[b][g]} softmax_i(scale * <q_j, k_i>) * v_i,
 * accumulated in fp32 with an online softmax over splits of the set.
 *   idx   int32 [batch][num_kv_heads][kappa]; entries < 0 are ignored.
 *   out   float [batch][num_q_heads][head_dim].
 */
PRISM_API prism_status prism_sparse_attn(const prism_kv_cache* kv, const uint16_t* q,
                               const prism_params* params, const int32_t* idx, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * One layer of Algorithm 1.  If layer % anchor_stride == 0 the layer is an
 * anchor: select as prism_score_topk, store the set in anchor_idx and its
 * refinement pool in the workspace.  Otherwise the layer is refined as
 * prism_refine_topk would refine it against anchor_idx, re-scoring the pool
 * the nearest preceding anchor layer left in the same workspace: the layers
 * of one decode step share anchor_idx, the workspace and the params (kappa,
 * window and pool_rho bound the pool's size), and calling a refined layer
 * before any anchor layer is the caller's error.  Then SparseAttn over the
 * layer's set into out.
 *   anchor_idx     int32 [batch][num_kv_heads][kappa], state carried between
 *                  the layers of one decode step (written by anchors, read by
 *                  refined layers).
 *   layer_idx_out  optional int32 [batch][num_kv_heads][kappa]: this layer's set.
 *   out            float [batch][num_q_heads][head_dim].
 */
PRISM_API prism_status prism_decode_layer(int32_t layer, const prism_kv_cache* kv, const uint16_t* q,
                                const prism_params* params, int32_t* anchor_idx,
                                int32_t* layer_idx_out, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * prism_decode_layer with the library's own static workspace instead of a
 * caller-owned one, same arguments otherwise.  Allocates nothing: the
 * workspace is a file-scope __device__ array of PRISM_STATIC_WORKSPACE_BYTES
 * (64 MiB) in the library's device code, which every GPU the library runs on
 * holds until the process ends.  The first call on a device resolves the
 * array's device address (hipGetSymbolAddress, which may load the library's
 * code object onto that device): make it outside graph capture.
 *   Returns PRISM_ERR_WORKSPACE, enqueueing nothing, when the shapes need more
 *   workspace than that (prism_workspace_size(kv, params) > 64 MiB), and the
 *   statuses of prism_decode_layer otherwise.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: the layers of a decode step run in order with the same shapes
 * (the anchor layer leaves its pool there for the refined layers), and calls
 * that overlap on one GPU (other streams or threads) race with each other.
 * Nothing in it needs clearing first: the kernels check every counter they
 * read from the workspace and take an exact pass when one is stale.
 */
#define PRISM_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
PRISM_API prism_status prism_decode_layer_noalloc(int32_t layer, const prism_kv_cache* kv,
                                                  const uint16_t* q, const prism_params* params,
                                                  int32_t* anchor_idx, int32_t* layer_idx_out,
                                                  float* out, void* stream);

/*
 * Dense decode attention over every cached token (the FlashAttention-style
 * baseline "Prism Attention" measures against, Tables 6-8): for every query
 * head j of KV head g,
 *   out[b][j] = sum_{i < seq_lens[b]} softmax_i(scale * <q_j, k_i>) * v_i,
 * in fp32 with an online softmax over chunks of the context (at most 128
 * chunks of at least 1024 tokens), merged in chunk order.  params->kappa,
 * window, anchor_stride and pool_rho are validated but not used; the
 * workspace of prism_workspace_size holds the chunk partials (apart from the
 * state the sparse calls carry, which a dense call leaves intact).
 *   out  float [batch][num_q_heads][head_dim].
 */
PRISM_API prism_status prism_dense_attn(const prism_kv_cache* kv, const uint16_t* q,
                                        const prism_params* params, float* out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * INT2 quantization of keys ("Prism Attention", Section 4.2, Eqs. 7-8):
 * group-wise asymmetric 2-bit codes of the key rows of the last num_new
 * positions of every sequence (positions [max(0, seq_lens[b] - num_new),
 * seq_lens[b]), all KV heads; every position when num_new <= 0), read from
 * kv->k_pages through the block table and written to k_codes / k_scales in
 * the layout prism_kv_cache documents.  Per group of 32 dimensions: beta =
 * the minimum, alpha = (max - min) / 3 rounded to the nearest bf16, code = the
 * integer nearest (ties to even) to (k - beta) / alpha, clipped to [0, 3], and
 * 0 when alpha = 0; the subtraction and division are IEEE float32; -0 reads
 * as +0.  Keys must be finite.  It quantizes a prefill's keys (num_new <= 0);
 * a decode step's new keys can instead be left to the layer's own call
 * (prism_kv_cache.new_keys), which saves this launch.  kv->k_codes,
 * kv->k_scales and kv->new_keys are not read.  Rows of other positions are
 * left untouched.
 */
PRISM_API prism_status prism_quantize_keys(const prism_kv_cache* kv, int32_t num_new,
                                           uint8_t* k_codes, uint16_t* k_scales, void* stream);

/*
 * Layer roles of a layer-assignment pattern ("Prism Attention", Algorithm 1's
 * partition into proposal and refined layers; Appendix E, Table 9, for the
 * hybrid with shared layers).
 */
typedef enum {
  PRISM_ROLE_PROPOSAL = 0, /* F: scores the whole cache, keeps its top-kappa and
                              leaves the candidate pool in the workspace          */
  PRISM_ROLE_REFINED = 1,  /* R: re-scores the pool of the nearest preceding F
                              layer and keeps its own top-kappa                   */
  PRISM_ROLE_SHARED = 2    /* S: reuses the set of the nearest preceding F or R
                              layer as it is; no scoring, no selection            */
} prism_layer_role;

/*
 * Role of `layer` in a pattern string of one letter per layer, F, R or S with
 * Table 9's meanings.  table4 != 0 reads the pattern with Table 4's letters,
 * where S marks a refined layer (so S maps to PRISM_ROLE_REFINED and R is not
 * allowed).  Returns the role, or -1 if pattern is NULL, layer lies outside
 * [0, strlen(pattern)), a letter of the pattern is not allowed, or the first
 * letter is not F (every other role needs a preceding proposal layer).  Pure
 * host function; touches no device.
 */
PRISM_API int32_t prism_pattern_role(const char* pattern, int32_t table4, int32_t layer);

/*
 * One layer of a decode step with an explicit role (prism_layer_role):
 *   PRISM_ROLE_PROPOSAL  as an anchor layer of prism_decode_layer: writes its
 *                        top-kappa into set_idx and leaves the refinement pool
 *                        (window or rank-expanded, by params->pool_rho) in the
 *                        workspace;
 *   PRISM_ROLE_REFINED   re-scores the pool the nearest preceding proposal
 *                        layer left in the same workspace, writes its top-kappa
 *                        into set_idx;
 *   PRISM_ROLE_SHARED    reads set_idx (the nearest preceding proposal or
 *                        refined layer's set) and does not change it;
 * then SparseAttn over the layer's set into out.  params->anchor_stride is not
 * used.  The layers of one decode step share set_idx, the workspace and the
 * params; a refined or shared layer before any proposal layer is the caller's
 * error (the results are then undefined, never out-of-bounds accesses).
 *   set_idx  int32 [batch][num_kv_heads][kappa], caller-owned state.
 *   out      float [batch][num_q_heads][head_dim].
 * Returns PRISM_ERR_INVALID_ARG for an unknown role or a NULL set_idx / out.
 */
PRISM_API prism_status prism_decode_layer_role(int32_t role, const prism_kv_cache* kv,
                                               const uint16_t* q, const prism_params* params,
                                               int32_t* set_idx, float* out, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * Optional instrumentation for benchmarks.  Kernel kinds launched by the calls
 * above: */
typedef enum {
  PRISM_KERNEL_ANCHOR_SCORE = 0, /* anchor layer: relevance of every cached token        */
  PRISM_KERNEL_REFINE_SCORE = 1, /* refined layer: relevance of the pool                 */
  PRISM_KERNEL_SELECT = 2,       /* top-kappa of every (sequence, KV head) list          */
  PRISM_KERNEL_ATTENTION = 3,    /* SparseAttn over splits of the set (and, for a layer,
                                    the selection that precedes it)                      */
  PRISM_KERNEL_POOL_BUILD = 4,   /* pool of an anchor set given to prism_refine_topk     */
  PRISM_KERNEL_CLASSIFY = 5,     /* anchor layer, contexts > 16384: marks the entries
                                    above the kappa-th score's coarse bin, lists the bin */
  PRISM_KERNEL_MERGE = 6,        /* merge of the attention splits into out              */
  PRISM_KERNEL_QUANTIZE = 7,     /* INT2 codes of key rows (prism_quantize_keys)         */
  PRISM_KERNEL_DENSE = 8,        /* dense decode attention chunks (prism_dense_attn)     */
  PRISM_KERNEL_KINDS = 9
} prism_kernel_kind;

/*
 * Registers a ring of `count` (start, stop) hipEvent_t pairs for one kernel
 * kind: every later launch of that kind takes the next pair, round robin, and
 * the events are recorded by the dispatch itself at the kernel's start and end
 * on the stream it runs on (hipEventElapsedTime of a pair = that launch's
 * duration).  count 0 (or NULL arrays) switches the kind back to plain
 * launches.  The arrays are copied; the events stay owned by the caller and
 * must outlive their use.  Process-wide setting, not thread-safe: meant for a
 * single benchmarking thread.  Returns PRISM_ERR_INVALID_ARG for a bad kind
 * or a negative count.
 */
PRISM_API prism_status prism_profile_events(int32_t kind, void* const* start_events,
                                            void* const* stop_events, int32_t count);

/* Launches of `kind` that took an event pair since its ring was registered. */
PRISM_API int64_t prism_profile_launches(int32_t kind);

/* Static description of a status code. */
PRISM_API const char* prism_status_string(prism_status status);

/* Message of the most recent failure on the calling thread ("" if none). */
PRISM_API const char* prism_last_error(void);

/* PRISM_ABI_VERSION of the built library. */
PRISM_API int32_t prism_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */

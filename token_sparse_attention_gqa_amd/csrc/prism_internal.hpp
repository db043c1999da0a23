// Internal declarations shared by the library's host API and its kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace prism {

constexpr int kHeadDim = 128;         // elements per K/V row
constexpr int kPageSize = 64;         // tokens per page
constexpr int kSelThreads = 1024;     // threads of a selection workgroup
constexpr int kScoreThreads = 256;    // threads of a relevance workgroup
constexpr int kMaxRankPool = 32768;   // largest rank-expanded pool (rho * kappa)
constexpr int kMaxNewKeys = 64;       // most new keys a call quantizes in its scoring kernel
constexpr int kPoolEntries = 256;     // pool entries scored by one refined-layer workgroup
constexpr int kAttnSplit = 64;        // selected tokens attended by one workgroup
constexpr int kAttnThreads = 256;
constexpr int kMaxKappa = 8192;
constexpr int kMaxSeqLen = 262144;
constexpr int kCoarseBins = 4096;   // anchor-layer score histogram: top 12 bits of the order key
constexpr int kMaxCand = 4096;      // threshold-bin entries an anchor selection ranks exactly
constexpr uint32_t kNoRow = 0xFFFFFFFFu;  // row id of an empty selection slot

// Shapes of one call, resolved and validated on the host.
struct Geometry {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint8_t* k_codes;    // INT2 proposal keys (null: relevance from k_pages)
  uint16_t* k_scales;  // their per-group (alpha, beta), bf16
  int new_keys;        // trailing positions whose codes the scoring kernels write first
  int batch;
  int hkv;          // KV heads
  int hq;           // query heads
  int group;        // hq / hkv
  int num_pages;    // physical pages in the cache arrays
  int max_pages;    // block_table row length
  int max_seq_len;
  int n_cap;        // per-problem list capacity: max_seq_len rounded up to 64
  int kappa;
  int window;
  int pool_rho;     // 0: window pool; >= 1: rank-expanded pool of pool_rho * kappa tokens
  int splits;       // attention splits per problem
  size_t page_stride;  // elements per physical page: hkv * page * head_dim
  __host__ __device__ int problems() const { return batch * hkv; }
};

// Carved workspace regions (device pointers).  A row id r addresses the K/V
// row at element offset r * head_dim of a layer's page array.
struct Workspace {
  uint32_t* ghist;        // [P][kCoarseBins] anchor-layer score histogram, left at zero
                          //     by its last reader and checked by the selection
  uint32_t* cand_cnt;     // [P][W] threshold-bin entries found by classify workgroup w
                          //     (W = workgroups per problem), written by every pass
  int32_t* sel_meta;      // [P][4] threshold bin, entries above it, entries in it
  uint32_t* cand_key;     // [P][W][2048] order keys of the threshold-bin entries, per
  int32_t* cand_idx;      // [P][W][2048] classify workgroup; their list indices
  uint32_t* gbits;        // [P][n_cap / 32] marks of the entries above the threshold bin
  float* scores;          // [P][n_cap] relevance in list order
  int32_t* pool_pos;      // [P][n_cap] refinement pool: positions, ascending
  uint32_t* pool_row;     // [P][n_cap] refinement pool: row ids
  int32_t* pool_len;      // [P]
  uint32_t* sel_row;      // [P][kappa] row ids of the latest selection
  int32_t* idx_tmp;       // [P][kappa]
  int32_t* sel_ent;       // [P][kappa] pool indices of a deferred selection (rank order)
  float* part_o;          // [P][splits][G][head_dim]
  float* part_ml;         // [P][splits][G][2]  (max logit, sum of exponentials)
  float* dense_o;         // [P][dense splits][G][head_dim]: dense decode partials
  float* dense_ml;        // [P][dense splits][G][2]
  // a second classification of the anchor list, made in the same pass as the
  // first (the rank-expanded pool's, beside the anchor set's): as above
  uint32_t* cand_cnt2;    // [P][W]
  int32_t* sel_meta2;     // [P][4]
  uint32_t* cand_key2;    // [P][W][2048]
  int32_t* cand_idx2;     // [P][W][2048]
  uint32_t* gbits2;       // [P][n_cap / 32]
};

// Kernel kinds, numbered as prism_kernel_kind in prism.h.
enum KernelKind {
  kAnchorScore = 0,
  kRefineScore,
  kSelect,
  kAttention,
  kPoolBuild,
  kClassify,
  kMerge,
  kQuantize,
  kDense,
  kKernelKinds
};

// Benchmark instrumentation: per kind, a ring of (start, stop) events that the
// dispatch of each launch records.
bool set_profile_events(int kind, void* const* starts, void* const* stops, int count);
int64_t profile_launches(int kind);

size_t workspace_bytes(const Geometry& g);
Workspace carve_workspace(void* base, const Geometry& g);

// Anchor layer: relevance of every cached token, top-kappa into out (and out2),
// the selection's row ids, and the refinement pool of the selected set.
hipError_t launch_anchor(const Geometry& g, const Workspace& w, const uint16_t* q, int32_t* out,
                         int32_t* out2, hipStream_t s);
// Refinement pool of an anchor set given in device memory.
hipError_t launch_pool_build(const Geometry& g, const Workspace& w, const int32_t* anchor_idx,
                             hipStream_t s);
// Refined layer over the workspace's pool: relevance of the pool, top-kappa
// into out, and the selection's row ids; with `defer`, only the set's pool
// indices (Workspace::sel_ent) and out is not written.
hipError_t launch_refine(const Geometry& g, const Workspace& w, const uint16_t* q, int32_t* out,
                         hipStream_t s, bool defer = false);
// Anchor layer of a decode step: scoring, selection, the refinement pool and
// SparseAttn.  anchor_idx receives the set (and layer_idx, if not null).
hipError_t launch_anchor_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, int32_t* anchor_idx, int32_t* layer_idx, float* out,
                                hipStream_t s);
// Refined layer of a decode step: pool scoring, then selection and SparseAttn
// (pools of at most 8192 entries are selected inside the attention kernel).
// layer_idx (nullable) receives the layer's set.
// Anchor layer with the rank-expanded pool: scoring, classification of long
// lists for rho*kappa, the pool and the anchor set (out, out2, row ids).
hipError_t launch_anchor_rank(const Geometry& g, const Workspace& w, const uint16_t* q,
                              int32_t* out, int32_t* out2, hipStream_t s);
// Anchor layer of a decode step with the rank-expanded pool: the anchor set
// (into anchor_idx and layer_idx, if not null), the pool in the workspace, and
// SparseAttn over the set into out.
hipError_t launch_anchor_rank_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                     float scale, int32_t* anchor_idx, int32_t* layer_idx,
                                     float* out, hipStream_t s);
hipError_t launch_refine_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, int32_t* layer_idx, float* out, hipStream_t s);
// INT2 codes and scales of the keys of the last num_new positions of every
// sequence (every position if num_new <= 0), from k_pages.
hipError_t launch_quantize(const Geometry& g, int num_new, uint8_t* codes, uint16_t* scales,
                           hipStream_t s);
// Dense decode attention over every cached token into out [B][Hq][D].
hipError_t launch_dense(const Geometry& g, const Workspace& w, const uint16_t* q, float scale,
                        float* out, hipStream_t s);
// SparseAttn into out [B][Hq][D] over the set `idx` (positions), or, with
// use_sel_rows, over the row ids the latest selection left in the workspace.
// quantize_new: the same launch also writes the codes of g.new_keys new keys
// (for a layer that scores nothing).
hipError_t launch_attention(const Geometry& g, const Workspace& w, const uint16_t* q,
                            const int32_t* idx, bool use_sel_rows, float scale, float* out,
                            hipStream_t s, bool quantize_new = false);
// SparseAttn over the pool indices a deferred refined selection left in the
// workspace; pos_out (nullable) receives the set's positions.
hipError_t launch_attention_entries(const Geometry& g, const Workspace& w, const uint16_t* q,
                                    int32_t* pos_out, float scale, float* out, hipStream_t s);

}  // namespace prism

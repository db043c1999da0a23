// Internal declarations shared by the library's host API and its kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace prism {

constexpr int kHeadDim = 128;       // elements per K/V row
constexpr int kPageSize = 64;       // tokens per page
constexpr int kHistBits = 12;       // leading key bits histogrammed by the scoring kernel
constexpr int kHistBins = 1 << kHistBits;
constexpr int kScoreChunk = 1024;   // list entries scored by one workgroup
constexpr int kAttnSplit = 64;      // selected tokens attended by one workgroup
constexpr int kSelectCap = 4096;    // threshold-bin candidates the select kernel holds in LDS
constexpr int kMaxKappa = 8192;
constexpr int kMaxSeqLen = 524288;

// Shapes of one call, resolved and validated on the host.
struct Geometry {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
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
  int splits;       // attention splits per problem
  size_t page_stride;  // elements per physical page: hkv * page * head_dim
  int problems() const { return batch * hkv; }
};

// Carved workspace regions (device pointers).
struct Workspace {
  uint32_t* hist;     // [P][kHistBins]
  float* scores;      // [P][n_cap] relevance in list order
  int32_t* pool_pos;  // [P][n_cap] positions of a refined layer's pool
  int32_t* pool_len;  // [P]
  int32_t* idx_tmp;   // [P][kappa]
  float* part_o;      // [P][splits][G][head_dim]
  float* part_ml;     // [P][splits][G][2]  (running max, sum of exponentials)
};

// Kernel kinds, numbered as prism_kernel_kind in prism.h.
enum KernelKind { kAnchorScore = 0, kPoolScore, kSelect, kAttention, kCombine, kPoolPlan,
                  kHistReset, kKernelKinds };

// Benchmark instrumentation: per kind, a ring of (start, stop) events that the
// dispatch of each launch records.
bool set_profile_events(int kind, void* const* starts, void* const* stops, int count);
int64_t profile_launches(int kind);

size_t workspace_bytes(const Geometry& g);
Workspace carve_workspace(void* base, const Geometry& g);

hipError_t launch_zero_hist(const Geometry& g, const Workspace& w, hipStream_t s);
hipError_t launch_pool_plan(const Geometry& g, const Workspace& w, const int32_t* anchor_idx,
                            hipStream_t s);
hipError_t launch_score(const Geometry& g, const Workspace& w, const uint16_t* q, bool pool,
                        hipStream_t s);
hipError_t launch_select(const Geometry& g, const Workspace& w, bool pool, int32_t* out,
                         int32_t* out2, hipStream_t s);
hipError_t launch_attention(const Geometry& g, const Workspace& w, const uint16_t* q,
                            const int32_t* idx, float scale, float* out, hipStream_t s);

}  // namespace prism

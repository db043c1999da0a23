// Host side of the C ABI declared in include/prism.h: argument validation,
// workspace carving and the order in which kernels are enqueued.
#include "prism.h"
#include "prism_internal.hpp"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

// Workspace of prism_decode_layer_noalloc: one copy per GPU, in this file's
// device code, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory):
// scratch_address() gives the current device's copy.
static __device__ __align__(256) uint8_t scratch[PRISM_STATIC_WORKSPACE_BYTES];

namespace {

using prism::Geometry;
using prism::Workspace;

thread_local std::string g_last_error;

prism_status fail(prism_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

#define PRISM_TRY(expr)                 \
  do {                                  \
    const prism_status _s = (expr);     \
    if (_s != PRISM_OK) return _s;      \
  } while (0)

// Validates the cache description alone (the fields every call reads).
prism_status resolve_cache(const prism_kv_cache* kv) {
  if (!kv) return fail(PRISM_ERR_INVALID_ARG, "kv cache must not be NULL");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table || !kv->seq_lens)
    return fail(PRISM_ERR_INVALID_ARG, "k_pages, v_pages, block_table and seq_lens must not be NULL");
  if (kv->batch < 1 || kv->num_kv_heads < 1)
    return fail(PRISM_ERR_INVALID_ARG, "batch and num_kv_heads must be >= 1");
  if (kv->head_dim != prism::kHeadDim) return fail(PRISM_ERR_UNSUPPORTED, "head_dim must be 128");
  if (kv->page_size != prism::kPageSize) return fail(PRISM_ERR_UNSUPPORTED, "page_size must be 64");
  if (kv->num_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(PRISM_ERR_INVALID_ARG, "num_pages and max_pages_per_seq must be >= 1");
  if (kv->max_seq_len < 1 || kv->min_seq_len < 1 || kv->min_seq_len > kv->max_seq_len)
    return fail(PRISM_ERR_INVALID_ARG, "need 1 <= min_seq_len <= max_seq_len");
  if ((int64_t)kv->max_seq_len > (int64_t)kv->max_pages_per_seq * kv->page_size)
    return fail(PRISM_ERR_INVALID_ARG, "max_seq_len exceeds max_pages_per_seq * page_size");
  if (kv->max_seq_len > prism::kMaxSeqLen)
    return fail(PRISM_ERR_UNSUPPORTED, "max_seq_len above 262144");
  if ((int64_t)kv->batch * kv->num_kv_heads > (1 << 22))
    return fail(PRISM_ERR_UNSUPPORTED, "batch * heads too large");
  if ((int64_t)kv->num_pages * kv->num_kv_heads * kv->page_size > (int64_t)UINT32_MAX)
    return fail(PRISM_ERR_UNSUPPORTED, "num_pages * num_kv_heads * page_size above 2^32 rows");
  if (!aligned(kv->k_pages, 16) || !aligned(kv->v_pages, 16))
    return fail(PRISM_ERR_INVALID_ARG, "k_pages and v_pages must be 16-byte aligned");
  if (!aligned(kv->block_table, 4) || !aligned(kv->seq_lens, 4))
    return fail(PRISM_ERR_INVALID_ARG, "block_table and seq_lens must be 4-byte aligned");
  if ((kv->k_codes == nullptr) != (kv->k_scales == nullptr))
    return fail(PRISM_ERR_INVALID_ARG, "k_codes and k_scales must both be set or both be NULL");
  if (!aligned(kv->k_codes, 16) || !aligned(kv->k_scales, 16))
    return fail(PRISM_ERR_INVALID_ARG, "k_codes and k_scales must be 16-byte aligned");
  return PRISM_OK;
}

void fill_cache(const prism_kv_cache* kv, Geometry* g) {
  g->k_pages = kv->k_pages;
  g->v_pages = kv->v_pages;
  g->block_table = kv->block_table;
  g->seq_lens = kv->seq_lens;
  g->k_codes = kv->k_codes;
  g->k_scales = kv->k_scales;
  g->new_keys = kv->k_codes ? kv->new_keys : 0;
  g->batch = kv->batch;
  g->hkv = kv->num_kv_heads;
  g->num_pages = kv->num_pages;
  g->max_pages = kv->max_pages_per_seq;
  g->max_seq_len = kv->max_seq_len;
  g->n_cap = (kv->max_seq_len + 63) / 64 * 64;
  g->page_stride = (size_t)kv->num_kv_heads * prism::kPageSize * prism::kHeadDim;
}

// Validates the cache description and parameters and fills the geometry.
prism_status resolve(const prism_kv_cache* kv, const prism_params* p, Geometry* g) {
  if (!kv || !p) return fail(PRISM_ERR_INVALID_ARG, "kv cache and params must not be NULL");
  PRISM_TRY(resolve_cache(kv));
  if (kv->new_keys < 0) return fail(PRISM_ERR_INVALID_ARG, "new_keys must be >= 0");
  if (kv->new_keys > prism::kMaxNewKeys)
    return fail(PRISM_ERR_UNSUPPORTED, "new_keys above 64 (quantize with prism_quantize_keys)");
  if (p->num_q_heads < 1) return fail(PRISM_ERR_INVALID_ARG, "num_q_heads must be >= 1");
  if (p->num_q_heads % kv->num_kv_heads != 0)
    return fail(PRISM_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  const int G = p->num_q_heads / kv->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PRISM_ERR_UNSUPPORTED, "group size num_q_heads/num_kv_heads must be 1, 2, 4, 8 or 16");
  if ((int64_t)kv->batch * p->num_q_heads > (1 << 24))
    return fail(PRISM_ERR_UNSUPPORTED, "batch * heads too large");
  if (p->kappa < 1 || p->kappa > kv->min_seq_len)
    return fail(PRISM_ERR_INVALID_ARG, "need 1 <= kappa <= min_seq_len");
  if (p->kappa > prism::kMaxKappa) return fail(PRISM_ERR_UNSUPPORTED, "kappa above 8192");
  if (p->window < 0) return fail(PRISM_ERR_INVALID_ARG, "window must be >= 0");
  if (p->pool_rho < 0) return fail(PRISM_ERR_INVALID_ARG, "pool_rho must be >= 0");
  if ((int64_t)p->pool_rho * p->kappa > prism::kMaxRankPool)
    return fail(PRISM_ERR_UNSUPPORTED, "pool_rho * kappa above 32768");
  if (p->anchor_stride < 1) return fail(PRISM_ERR_INVALID_ARG, "anchor_stride must be >= 1");
  if (!std::isfinite(p->softmax_scale))
    return fail(PRISM_ERR_INVALID_ARG, "softmax_scale must be finite");

  fill_cache(kv, g);
  g->hq = p->num_q_heads;
  g->group = G;
  g->kappa = p->kappa;
  g->window = p->window;
  g->pool_rho = p->pool_rho;
  g->splits = (p->kappa + prism::kAttnSplit - 1) / prism::kAttnSplit;
  return PRISM_OK;
}

prism_status check_q(const uint16_t* q) {
  if (!q) return fail(PRISM_ERR_INVALID_ARG, "q must not be NULL");
  if (!aligned(q, 16)) return fail(PRISM_ERR_INVALID_ARG, "q must be 16-byte aligned");
  return PRISM_OK;
}

prism_status check_ws(const Geometry& g, void* ws, size_t bytes) {
  const size_t need = prism::workspace_bytes(g);
  if (!ws) return fail(PRISM_ERR_WORKSPACE, "workspace must not be NULL");
  if (!aligned(ws, 256)) return fail(PRISM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < need)
    return fail(PRISM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                         " bytes, got " + std::to_string(bytes));
  return PRISM_OK;
}

// A usable device must be current; also clears any stale runtime error so that
// launch errors reported afterwards are this call's own.
prism_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return fail(PRISM_ERR_HIP, std::string("no HIP device available: ") +
                                   (e != hipSuccess ? hipGetErrorString(e) : "device count is 0"));
  }
  (void)hipGetLastError();
  return PRISM_OK;
}

prism_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return PRISM_OK;
  return fail(PRISM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

float resolve_scale(const prism_params* p) {
  return p->softmax_scale != 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)prism::kHeadDim);
}


prism_status run_anchor(const Geometry& g, const Workspace& w, const uint16_t* q, int32_t* out,
                        int32_t* out2, hipStream_t s) {
  return hip_check(prism::launch_anchor(g, w, q, out, out2, s), "anchor selection launch");
}

// Device address of the current device's `scratch`, resolved once per device
// (with that device current) by hipGetSymbolAddress and kept.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

prism_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PRISM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PRISM_ERR_UNSUPPORTED, "static workspace: device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || !p)
      return fail(PRISM_ERR_HIP, std::string("static workspace address: ") +
                                     (es != hipSuccess ? hipGetErrorString(es) : "null"));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PRISM_OK;
}

prism_status copy_rows(void* dst, size_t dst_row, const void* src, size_t src_row, size_t row,
                       size_t rows, hipStream_t s, const char* what) {
  return hip_check(hipMemcpy2DAsync(dst, dst_row, src, src_row, row, rows,
                                    hipMemcpyDeviceToDevice, s),
                   what);
}

}  // namespace

extern "C" {

size_t prism_workspace_size(const prism_kv_cache* kv, const prism_params* params) {
  Geometry g;
  if (resolve(kv, params, &g) != PRISM_OK) return 0;
  return prism::workspace_bytes(g);
}

prism_status prism_score_topk(const prism_kv_cache* kv, const uint16_t* q,
                              const prism_params* params, int32_t* idx_out, float* scores_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (!idx_out) return fail(PRISM_ERR_INVALID_ARG, "idx_out must not be NULL");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace w = prism::carve_workspace(workspace, g);
  if (g.pool_rho >= 1)
    PRISM_TRY(hip_check(prism::launch_anchor_rank(g, w, q, idx_out, nullptr, s),
                        "anchor selection launch"));
  else
    PRISM_TRY(run_anchor(g, w, q, idx_out, nullptr, s));
  if (scores_out)
    PRISM_TRY(copy_rows(scores_out, (size_t)g.max_seq_len * 4, w.scores, (size_t)g.n_cap * 4,
                        (size_t)g.max_seq_len * 4, (size_t)g.problems(), s, "scores copy"));
  return PRISM_OK;
}

prism_status prism_refine_topk(const prism_kv_cache* kv, const uint16_t* q,
                               const prism_params* params, const int32_t* anchor_idx,
                               int32_t* idx_out, int32_t* pool_out, int32_t* pool_len_out,
                               float* pool_scores_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (!idx_out) return fail(PRISM_ERR_INVALID_ARG, "idx_out must not be NULL");
  if (!anchor_idx && g.pool_rho < 1)
    return fail(PRISM_ERR_INVALID_ARG, "anchor_idx must not be NULL for the window pool");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace w = prism::carve_workspace(workspace, g);
  if (g.pool_rho < 1)  // the rank-expanded pool is the one the anchor selection left
    PRISM_TRY(hip_check(prism::launch_pool_build(g, w, anchor_idx, s), "pool build launch"));
  PRISM_TRY(hip_check(prism::launch_refine(g, w, q, idx_out, s), "refined selection launch"));
  const size_t rowb = (size_t)g.max_seq_len * 4, caprow = (size_t)g.n_cap * 4;
  if (pool_out)
    PRISM_TRY(copy_rows(pool_out, rowb, w.pool_pos, caprow, rowb, g.problems(), s, "pool copy"));
  if (pool_scores_out)
    PRISM_TRY(copy_rows(pool_scores_out, rowb, w.scores, caprow, rowb, g.problems(), s,
                        "pool scores copy"));
  if (pool_len_out)
    PRISM_TRY(hip_check(hipMemcpyAsync(pool_len_out, w.pool_len, (size_t)g.problems() * 4,
                                       hipMemcpyDeviceToDevice, s),
                        "pool length copy"));
  return PRISM_OK;
}

prism_status prism_sparse_attn(const prism_kv_cache* kv, const uint16_t* q,
                               const prism_params* params, const int32_t* idx, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (!idx || !out) return fail(PRISM_ERR_INVALID_ARG, "idx and out must not be NULL");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace w = prism::carve_workspace(workspace, g);
  return hip_check(prism::launch_attention(g, w, q, idx, false, resolve_scale(params), out, s),
                   "attention launch");
}

prism_status prism_decode_layer(int32_t layer, const prism_kv_cache* kv, const uint16_t* q,
                                const prism_params* params, int32_t* anchor_idx,
                                int32_t* layer_idx_out, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (layer < 0) return fail(PRISM_ERR_INVALID_ARG, "layer must be >= 0");
  if (!anchor_idx || !out) return fail(PRISM_ERR_INVALID_ARG, "anchor_idx and out must not be NULL");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace w = prism::carve_workspace(workspace, g);
  if (layer % params->anchor_stride == 0) {
    if (g.pool_rho >= 1)
      return hip_check(prism::launch_anchor_rank_attend(g, w, q, resolve_scale(params),
                                                        anchor_idx, layer_idx_out, out, s),
                       "anchor layer launch");
    return hip_check(prism::launch_anchor_attend(g, w, q, resolve_scale(params), anchor_idx,
                                                 layer_idx_out, out, s),
                     "anchor layer launch");
  }
  return hip_check(
      prism::launch_refine_attend(g, w, q, resolve_scale(params), layer_idx_out, out, s),
      "refined layer launch");
}

prism_status prism_decode_layer_noalloc(int32_t layer, const prism_kv_cache* kv,
                                        const uint16_t* q, const prism_params* params,
                                        int32_t* anchor_idx, int32_t* layer_idx_out, float* out,
                                        void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (layer < 0) return fail(PRISM_ERR_INVALID_ARG, "layer must be >= 0");
  if (!anchor_idx || !out) return fail(PRISM_ERR_INVALID_ARG, "anchor_idx and out must not be NULL");
  const size_t need = prism::workspace_bytes(g);
  if (need > PRISM_STATIC_WORKSPACE_BYTES)
    return fail(PRISM_ERR_WORKSPACE,
                "these shapes need " + std::to_string(need) +
                    " bytes of workspace; the static workspace holds " +
                    std::to_string(PRISM_STATIC_WORKSPACE_BYTES) +
                    " (use prism_decode_layer with a caller-owned workspace)");
  PRISM_TRY(check_device());
  void* ws = nullptr;
  PRISM_TRY(scratch_address(&ws));
  return prism_decode_layer(layer, kv, q, params, anchor_idx, layer_idx_out, out, ws,
                            PRISM_STATIC_WORKSPACE_BYTES, stream);
}

prism_status prism_dense_attn(const prism_kv_cache* kv, const uint16_t* q,
                              const prism_params* params, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (!out) return fail(PRISM_ERR_INVALID_ARG, "out must not be NULL");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  const Workspace w = prism::carve_workspace(workspace, g);
  return hip_check(prism::launch_dense(g, w, q, resolve_scale(params), out,
                                       static_cast<hipStream_t>(stream)),
                   "dense attention launch");
}

prism_status prism_quantize_keys(const prism_kv_cache* kv, int32_t num_new, uint8_t* k_codes,
                                 uint16_t* k_scales, void* stream) {
  if (!kv) return fail(PRISM_ERR_INVALID_ARG, "kv cache must not be NULL");
  // kv->k_codes, kv->k_scales and kv->new_keys are not read here: validate the
  // rest of the description without them
  prism_kv_cache c = *kv;
  c.k_codes = nullptr;
  c.k_scales = nullptr;
  PRISM_TRY(resolve_cache(&c));
  if (!k_codes || !k_scales)
    return fail(PRISM_ERR_INVALID_ARG, "k_codes and k_scales must not be NULL");
  if (!aligned(k_codes, 16) || !aligned(k_scales, 16))
    return fail(PRISM_ERR_INVALID_ARG, "k_codes and k_scales must be 16-byte aligned");
  PRISM_TRY(check_device());
  Geometry g{};
  fill_cache(&c, &g);
  return hip_check(prism::launch_quantize(g, num_new, k_codes, k_scales,
                                          static_cast<hipStream_t>(stream)),
                   "quantize launch");
}

int32_t prism_pattern_role(const char* pattern, int32_t table4, int32_t layer) {
  if (!pattern || layer < 0) return -1;
  int32_t n = 0, role = -1;
  for (const char* c = pattern; *c; ++c, ++n) {
    int32_t r;
    switch (*c) {
      case 'F': r = PRISM_ROLE_PROPOSAL; break;
      case 'R': if (table4) return -1; r = PRISM_ROLE_REFINED; break;
      case 'S': r = table4 ? PRISM_ROLE_REFINED : PRISM_ROLE_SHARED; break;
      default: return -1;
    }
    if (n == 0 && r != PRISM_ROLE_PROPOSAL) return -1;
    if (n == layer) role = r;
  }
  return role;
}

prism_status prism_decode_layer_role(int32_t role, const prism_kv_cache* kv, const uint16_t* q,
                                     const prism_params* params, int32_t* set_idx, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  PRISM_TRY(resolve(kv, params, &g));
  PRISM_TRY(check_q(q));
  if (role != PRISM_ROLE_PROPOSAL && role != PRISM_ROLE_REFINED && role != PRISM_ROLE_SHARED)
    return fail(PRISM_ERR_INVALID_ARG, "role must be PRISM_ROLE_PROPOSAL, _REFINED or _SHARED");
  if (!set_idx || !out) return fail(PRISM_ERR_INVALID_ARG, "set_idx and out must not be NULL");
  PRISM_TRY(check_ws(g, workspace, workspace_bytes));
  PRISM_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Workspace w = prism::carve_workspace(workspace, g);
  const float scale = resolve_scale(params);
  switch (role) {
    case PRISM_ROLE_PROPOSAL:
      if (g.pool_rho >= 1)
        return hip_check(prism::launch_anchor_rank_attend(g, w, q, scale, set_idx, nullptr, out, s),
                         "proposal layer launch");
      return hip_check(prism::launch_anchor_attend(g, w, q, scale, set_idx, nullptr, out, s),
                       "proposal layer launch");
    case PRISM_ROLE_REFINED:
      return hip_check(prism::launch_refine_attend(g, w, q, scale, set_idx, out, s),
                       "refined layer launch");
    default:  // nothing here scores the new keys: the attention launch writes their codes
      return hip_check(prism::launch_attention(g, w, q, set_idx, false, scale, out, s, true),
                       "shared layer attention launch");
  }
}

prism_status prism_profile_events(int32_t kind, void* const* start_events,
                                  void* const* stop_events, int32_t count) {
  if (!prism::set_profile_events(kind, start_events, stop_events, count))
    return fail(PRISM_ERR_INVALID_ARG, "bad kernel kind or negative count");
  return PRISM_OK;
}

int64_t prism_profile_launches(int32_t kind) { return prism::profile_launches(kind); }

const char* prism_status_string(prism_status status) {
  // read as an integer: a C caller may pass any int, and a value outside the
  // enumeration must not be loaded as the enum type
  int32_t v;
  std::memcpy(&v, &status, sizeof v);
  switch (v) {
    case PRISM_OK: return "ok";
    case PRISM_ERR_INVALID_ARG: return "invalid argument";
    case PRISM_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case PRISM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PRISM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* prism_last_error(void) { return g_last_error.c_str(); }

int32_t prism_abi_version(void) { return PRISM_ABI_VERSION; }

}  // extern "C"

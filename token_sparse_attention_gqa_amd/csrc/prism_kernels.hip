// HIP kernels for gfx950 (CDNA4): token-sparse GQA decode attention with
// proposal-refined cross-layer index sharing ("Prism Attention", arXiv
// 2610.22985).
//
// One decode layer (prism_decode_layer, groups of up to 8 query heads):
//   anchor layer   score_anchor_kernel  relevance of every cached token (Eq. 9
//                                       with Eq. 1) and a coarse histogram of
//                                       the scores;
//                  classify_kernel      (contexts > kSmall) marks the entries
//                                       above the bin of the kappa-th score and
//                                       lists the bin's own entries;
//                  anchor_attn_kernel   top-kappa (Eq. 2), the refinement pool
//                                       (the +-w windows of the set), and
//                                       SparseAttn of Algorithm 1 over one
//                                       split of the set per workgroup;
//   refined layer  score_pool_kernel    relevance of the pool's tokens (Eq. 5);
//                  refine_attn_kernel   top-kappa of the pool (Eq. 6) and
//                                       SparseAttn over one split;
//   both           merge_kernel         the splits merged into the output.
// Grids the fused kernels do not fit at once (many problems, large kappa)
// use fewer, wider splits: refine_attn_multi_kernel (pools up to kSmall),
// refine_attn_multi_long_kernel (longer pools, after classify_kernel) and
// anchor_rank_multi_kernel (the rank-expanded pool's anchor layer), each
// selecting in every split and attending 256-2048 ranks with all sixteen
// waves.  The single-step entry points and the remaining shapes use
// select_kernel, pool_build_kernel and attn_kernel instead.  Options:
//   rank-expanded pool (Eq. 4)  rank_pool_kernel: the anchor's top rho*kappa
//                               as the pool, its top-kappa as the anchor set;
//   INT2 proposal keys (Eqs. 7-9) quantize_kernel, score_anchor_int2_kernel,
//                               score_pool_int2_kernel;
//   dense decode                dense_attn_kernel over every cached token.
#include "prism_internal.hpp"

#include <hip/hip_ext.h>

#include <cmath>
#include <vector>

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = kSelThreads;
constexpr int kSmall = 16384;   // lists up to this length are selected with every key in registers
constexpr int kSmallPer = kSmall / kSelThreads;  // 16 consecutive entries per thread
constexpr int kRegMarks = 2 * kSmall;  // fused refined kernel: pools held 32 keys per thread
static_assert(kMaxRankPool <= kRegMarks, "a rank-expanded pool is selected from registers");
constexpr int kSample = 8192;   // most entries of a longer list sampled to bracket the kappa-th key
constexpr int kCand = 4096;     // bracketed candidates held in LDS
constexpr int kPassUnroll = 4;  // 16-byte loads in flight per thread in the list pass
constexpr int kPoolPer = kMaxKappa / NT;  // anchor entries per thread in the pool build
constexpr int kClsThreads = 256;
constexpr int kClsEntries = 8192;         // anchor-list entries classified by one workgroup
constexpr int kClsCap = 2048;             // threshold-bin entries one classify workgroup keeps
constexpr int kClsSlots = kMaxSeqLen / kClsEntries;  // classify workgroups of the longest list
static_assert(kClsSlots <= 32, "candidate region starts fit sm.ured");
// classify workgroups (candidate regions) per problem
__host__ __device__ inline int cls_regions(const Geometry& g) {
  return (g.n_cap + kClsEntries - 1) / kClsEntries;
}
constexpr int kFusedSplit = 128;          // selected tokens attended by one fused workgroup
constexpr int kPoolHistChunks = 4;        // pool chunks per workgroup when pool scoring counts bins
constexpr int kFusedAnchorLen = 6144 * 32;  // contexts whose nonzero mark words fit sm.hist
static_assert(kMaxCand <= kCand, "candidates of the threshold bin fit the LDS candidate buffer");
static_assert(kMaxKappa <= 2 * kCand, "pool-build run offsets fit the LDS candidate buffer");

// Monotone map of a float to uint32: a > b  <=>  key(a) > key(b); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose order_key is k (-0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Workgroup barrier for LDS communication only: waits for the workgroup's LDS
// accesses, not for its global loads and stores still in flight (the
// compiler's __syncthreads waits for every memory access of the workgroup).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int seq_len_of(const Geometry& g, int b) {
  return clampi(g.seq_lens[b], 0, g.max_seq_len);
}

__device__ __forceinline__ int phys_page(const Geometry& g, int b, int logical) {
  return clampi(g.block_table[(size_t)b * g.max_pages + logical], 0, g.num_pages - 1);
}

// Row id of token `pos` of sequence b, KV head h: its row in the page array.
__device__ __forceinline__ uint32_t row_id_of_page(const Geometry& g, int page, int h, int pos) {
  return (uint32_t)page * (uint32_t)(g.hkv * kPageSize) + (uint32_t)(h * kPageSize) +
         (uint32_t)(pos & (kPageSize - 1));
}
__device__ __forceinline__ uint32_t row_id(const Geometry& g, int b, int h, int pos) {
  return row_id_of_page(g, phys_page(g, b, pos >> 6), h, pos);
}

// Workgroup -> (problem, index within problem).  Dispatch places workgroup i
// on XCD i % 8; when the problem count allows, all workgroups of a problem
// land on one XCD so that its scores stay in that XCD's L2.
__device__ __forceinline__ void map_block(int bid, int P, int W, int* p, int* w) {
  if ((P & 7) == 0) {
    const int x = bid & 7, s = bid >> 3;
    *p = x + 8 * (s / W);
    *w = s % W;
  } else {
    *p = bid / W;
    *w = bid % W;
  }
}

// max(v[l], v[l ^ 16]) and max(v[l], v[l ^ 32]) for every lane l, by the
// VALU row swaps (v_permlane16_swap / v_permlane32_swap with the value as both
// operands: each lane receives its partner's value in one of the two results).
// The larger of two scores in one v_max_f32: fmaxf first canonicalises each
// operand that comes from a lane swap (two more instructions), which scores
// (finite, or -inf for masked entries) never need.
__device__ __forceinline__ float max_score(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_score(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t xor16_or(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] | r[1];
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_score(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// MFMA A-operand fragment of the group's query heads.  Lane l holds head
// (l % 16) (zero when >= G) and, for step s, the 16-byte chunk g4 + 4s of the
// head dimension, g4 = l / 16.  Key fragments use the same chunk order, so the
// four steps together contract over all 128 dimensions.
template <int G>
__device__ __forceinline__ void load_q_frag(const uint16_t* q, const Geometry& g, int b, int kvh,
                                            int lane, u32x4 (&qf)[4]) {
  const int j = lane & 15, g4 = lane >> 4;
  if (j < G) {
    const u32x4* qrow =
        reinterpret_cast<const u32x4*>(q + ((size_t)b * g.hq + kvh * G + j) * kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = qrow[g4 + 4 * s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = u32x4{0u, 0u, 0u, 0u};
  }
}

// 16 tokens x G heads of <q_j, k_i>: D[i][j] lands in lane (j + 16*(i/4)),
// register i % 4.
__device__ __forceinline__ f32x4 qk_tile(const u32x4 (&qf)[4], const u32x4 (&kf)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[s]),
                                                  __builtin_bit_cast(bf16x8, kf[s]), acc, 0, 0,
                                                  0);
  return acc;
}

// Max over the group's heads of a qk_tile; valid in lanes 0..15 (token = lane).
template <int G>
__device__ __forceinline__ float group_max(const f32x4& acc, int g4) {
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * g4 + r < G) m = fmaxf(m, acc[r]);
  if (G > 4) m = xor16_max(m);
  if (G > 8) m = xor32_max(m);
  return m;
}

// Lane movement inside a wave by DPP (GCN/CDNA controls): row_shr:n moves
// lane i - n of the same 16-lane row to lane i; row_bcast:15 sends lane 15 of
// each row to the next row, row_bcast:31 lane 31 to rows 2 and 3; quad_perm
// permutes inside groups of four lanes.  Lanes with no source (or a row left
// out by the row mask) get `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;  // quad_perm [1,0,3,2] and [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;             // lane 7 - i of each 8-lane half row
constexpr int kRowMirror = 0x140;                 // lane 15 - i of each 16-lane row
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;  // rotate right in a row

// Inclusive scan of an associative op over the wave (ident: its identity);
// lane 63 ends with the result over all 64 lanes.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t ident, Op op) {
  v = op(v, dpp<kRowShr1, 0xf>(ident, v));
  v = op(v, dpp<kRowShr2, 0xf>(ident, v));
  v = op(v, dpp<kRowShr4, 0xf>(ident, v));
  v = op(v, dpp<kRowShr8, 0xf>(ident, v));
  v = op(v, dpp<kRowBcast15, 0xa>(ident, v));
  v = op(v, dpp<kRowBcast31, 0xc>(ident, v));
  return v;
}
__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t r = wave_scan(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float(lane63(r));
}
__device__ __forceinline__ float wave_sum(float v) {
  const uint32_t r = wave_scan(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float(lane63(r));
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  return (int)wave_scan((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  return lane63(wave_scan(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); }));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }));
}

// Exclusive prefix sum over the T threads of the block; *total gets the sum.
// tmp: at least T/64 ints of LDS.  Contains barriers: call uniformly.
template <int T>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = T / 64;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int inc = wave_incl_scan(v);
  lds_barrier();  // earlier readers of tmp are done
  if (lane == 63) tmp[w] = inc;
  lds_barrier();
  const int x = lane < NW ? tmp[lane] : 0;
  const int xi = wave_incl_scan(x);
  *total = __builtin_amdgcn_readlane(xi, NW - 1);
  return __builtin_amdgcn_readlane(xi - x, w) + inc - v;
}

struct Bin {
  int bin, above, count;
};

// One wave: in a histogram of NB bins, the bin holding the need-th largest
// element (1-based, counting down from the top bin), the count of higher bins
// and the bin's own count; bin = -1 if the histogram holds fewer than need.
// Lane l owns NB/64 consecutive bins; their sums (read in a rotated order that
// keeps the lanes on distinct LDS banks) are scanned across the wave, then the
// owning lane's bins are scanned across the wave, one bin per lane.  Result is
// uniform over the wave.
template <int NB>
__device__ Bin wave_find_bin(const uint32_t* h, int need) {
  constexpr int R = NB / 64;
  const int lane = threadIdx.x & 63;
  const int top = NB - 1 - R * lane;
  int sum = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) sum += (int)h[top - ((r + lane) & (R - 1))];
  const int incl = wave_incl_scan(sum);
  const int excl = incl - sum;
  const unsigned long long hit = __ballot(excl < need && incl >= need);
  if (!hit) return Bin{-1, 0, 0};
  const int src = __ffsll((unsigned long long)hit) - 1;
  const int base = __builtin_amdgcn_readlane(excl, src);
  const int src_top = NB - 1 - R * src;
  const int c = lane < R ? (int)h[src_top - lane] : 0;
  const int inc2 = wave_incl_scan(c) + base;
  const unsigned long long hit2 = __ballot(lane < R && inc2 >= need);
  const int k = __ffsll((unsigned long long)hit2) - 1;
  return Bin{src_top - k, __builtin_amdgcn_readlane(inc2 - c, k), __builtin_amdgcn_readlane(c, k)};
}

// ---------------------------------------------------------------------------
// Relevance
// ---------------------------------------------------------------------------

// Sum over each group of 8 lanes (lanes 8k .. 8k + 7); every lane of the group
// receives the same value.
__device__ __forceinline__ float group8_sum(float v) {
  v += __uint_as_float(dpp<kRowHalfMirror, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kQuadXor2, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kQuadXor1, 0xf>(0u, __float_as_uint(v)));
  return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// Anchor layer: workgroup w of problem p scores tokens [w * E, +E) of the cache,
// E = 256 kPages tokens (kPages whole pages per wave; fewer for caches too short
// to give every compute unit four workgroups of 1024 tokens).  The
// workgroup also counts its scores by coarse bin (top 12 bits of the order
// key) in LDS and adds the counts to the problem's histogram in the workspace,
// which the selection uses to find the bin holding the kappa-th score.
//
// Groups of up to 8 query heads score on the VALU: 8 lanes share a key row,
// each lane taking the 16-byte chunks `part` and `part + 8`, so one load
// instruction of the wave reads 8 rows x 128 contiguous bytes (whole cache
// lines; operand fragments for the matrix cores would read 16 rows x 64 bytes
// per instruction, which streams from HBM measurably slower).  Each lane forms
// bf16 pair products with the group's query chunks (v_dot2), the 8 lanes of a
// row sum their partials, and the maximum over the heads is the relevance.
// Larger groups use the matrix cores (four MFMAs per 16 tokens).
// Adds a scoring workgroup's LDS histogram to its problem's histogram in
// device memory, two adjacent bins per 64-bit atomic (a bin's total is at most
// the context length, far below 2^32, so the low half never carries into the
// high one).  Every workgroup of a problem flushes at about the same time, and
// the atomics on one problem's bins serialise: half as many of them made INT2
// anchor scoring on the 4 x 128K GQA-8 workload 9 us faster per launch.
__device__ __forceinline__ void flush_hist(const uint32_t* lh, uint32_t* gh) {
  unsigned long long* g2 = reinterpret_cast<unsigned long long*>(gh);
  for (int i = threadIdx.x; i < kCoarseBins / 2; i += kScoreThreads) {
    const unsigned long long c =
        (unsigned long long)lh[2 * i] | ((unsigned long long)lh[2 * i + 1] << 32);
    if (c) atomicAdd(g2 + i, c);
  }
}

template <int G, int kPages>
__global__ __launch_bounds__(kScoreThreads) void score_anchor_kernel(Geometry g, Workspace ws,
                                                                     const uint16_t* __restrict__ q,
                                                                     int wgs) {
  constexpr int kEntries = 4 * kPages * kPageSize;  // tokens of one workgroup, whole pages per wave
  __shared__ uint32_t lh[kCoarseBins];
  int p, w;
  map_block(blockIdx.x, g.problems(), wgs, &p, &w);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int n = seq_len_of(g, b);
  if (w * kEntries >= n) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wbase = w * kEntries + wave * (kEntries / 4);
  for (int i = threadIdx.x; i < kCoarseBins; i += kScoreThreads) lh[i] = 0u;
  lds_barrier();
  if (wbase < n) {
    float* sc = ws.scores + (size_t)p * g.n_cap;
    const int last_page = (n - 1) >> 6;
    const size_t head = (size_t)kvh * kPageSize * kHeadDim;
    size_t page_off[kPages];
#pragma unroll
    for (int r = 0; r < kPages; ++r)
      page_off[r] = (size_t)phys_page(g, b, min((wbase >> 6) + r, last_page)) * g.page_stride + head;
    if constexpr (G <= 8) {
      const int part = lane & 7, rs = lane >> 3;
      uint32_t qv[G][8];  // head h: chunk `part` in [0, 4), chunk `part + 8` in [4, 8)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const u32x4* qrow =
            reinterpret_cast<const u32x4*>(q + ((size_t)b * g.hq + kvh * G + h) * kHeadDim);
        const u32x4 x0 = qrow[part], x1 = qrow[part + 8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qv[h][i] = x0[i];
          qv[h][4 + i] = x1[i];
        }
      }
      // Half a page (4 groups of 8 rows) per step, three buffers: the loads of
      // the next two half pages are in flight during the current one's
      // arithmetic (the scheduling barriers keep the compiler from moving them).
      u32x4 kb[3][4][2];
#pragma unroll
      for (int r = 0; r < 2 * kPages + 2; ++r) {
        if (r < 2 * kPages) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4* row = reinterpret_cast<const u32x4*>(
                g.k_pages + page_off[r >> 1] + (size_t)((((r & 1) * 4 + u) * 8 + rs) * kHeadDim));
            kb[r % 3][u][0] = __builtin_nontemporal_load(row + part);
            kb[r % 3][u][1] = __builtin_nontemporal_load(row + part + 8);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (r >= 2) {
          const int rp = r - 2;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4 k0 = kb[rp % 3][u][0], k1 = kb[rp % 3][u][1];
            float m = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float a = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i) a = dot2_bf16(qv[h][i], k0[i], a);
#pragma unroll
              for (int i = 0; i < 4; ++i) a = dot2_bf16(qv[h][4 + i], k1[i], a);
              m = fmaxf(m, group8_sum(a));
            }
            const int e = wbase + rp * 32 + u * 8 + rs;
            if (part == 0 && e < n) {
              sc[e] = m;
              atomicAdd(&lh[order_key(m) >> 20], 1u);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const int j = lane & 15, g4 = lane >> 4;
      u32x4 qf[4];
      load_q_frag<G>(q, g, b, kvh, lane, qf);
      // One page (4 tiles of 16 tokens) per step, double-buffered: the next page's
      // 16 loads are issued before the current page's MFMAs (the scheduling
      // barriers keep the compiler from interleaving them back into a few loads
      // in flight).  Addresses stay offsets from the kernel-argument base so the
      // loads remain global loads.
      u32x4 kb[2][4][4];
#pragma unroll
      for (int r = 0; r < kPages + 1; ++r) {
        if (r < kPages) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4* row = reinterpret_cast<const u32x4*>(
                g.k_pages + page_off[r] + (size_t)((u * 16 + j) * kHeadDim));
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
              kb[r & 1][u][s4] = __builtin_nontemporal_load(row + g4 + 4 * s4);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (r > 0) {
          const int rp = r - 1;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float m = group_max<G>(qk_tile(qf, kb[rp & 1][u]), g4);
            const int e = wbase + rp * 64 + u * 16 + j;
            if (g4 == 0 && e < n) {
              sc[e] = m;
              atomicAdd(&lh[order_key(m) >> 20], 1u);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  lds_barrier();
  flush_hist(lh, ws.ghist + (size_t)p * kCoarseBins);
}

// Refined layer: workgroup w of problem p scores pool entries
// [w * chunks * kPoolEntries, +chunks * kPoolEntries) from the pool's row ids,
// 64 per wave and chunk; the key rows are read and combined as in anchor
// scoring (VALU for groups of up to 8 heads, 8 lanes per row; matrix cores for
// larger groups).  With `hist`, pools longer than kSmall are also counted per
// coarse bin, as in anchor scoring, for the classification that follows
// (several chunks per workgroup amortise the LDS histogram).
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_pool_kernel(Geometry g, Workspace ws,
                                                                   const uint16_t* __restrict__ q,
                                                                   int wgs, int chunks, int hist) {
  __shared__ uint32_t lh[kCoarseBins];
  int p, w;
  map_block(blockIdx.x, g.problems(), wgs, &p, &w);
  const int n = clampi(ws.pool_len[p], 0, g.n_cap);
  const int base = w * chunks * kPoolEntries;
  if (base >= n) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool counted = hist != 0 && n > kSmall;  // uniform over the workgroup
  if (counted) {
    for (int i = threadIdx.x; i < kCoarseBins; i += kScoreThreads) lh[i] = 0u;
    lds_barrier();
  }
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const uint32_t* prow = ws.pool_row + (size_t)p * g.n_cap;
  float* sc = ws.scores + (size_t)p * g.n_cap;
  const uint32_t max_row = (uint32_t)g.num_pages * (uint32_t)(g.hkv * kPageSize) - 1u;
  if constexpr (G <= 8) {
    const int part = lane & 7, rs = lane >> 3;
    constexpr int kGroups = kPoolEntries / 4 / 8;  // 8 groups of 8 rows per wave
    uint32_t qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const u32x4* qrow =
          reinterpret_cast<const u32x4*>(q + ((size_t)b * g.hq + kvh * G + h) * kHeadDim);
      const u32x4 x0 = qrow[part], x1 = qrow[part + 8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[h][i] = x0[i];
        qv[h][4 + i] = x1[i];
      }
    }
    // row ids one chunk ahead: the next chunk's are loaded behind the current
    // chunk's keys, so only the first chunk waits for its row ids
    uint32_t rid[kGroups];
    {
      const int wb0 = base + wave * (kPoolEntries / 4);
#pragma unroll
      for (int u = 0; u < kGroups; ++u) rid[u] = prow[min(wb0 + u * 8 + rs, n - 1)];
    }
    for (int c = 0; c < chunks; ++c) {
      const int wbase = base + c * kPoolEntries + wave * (kPoolEntries / 4);
      if (wbase >= n) break;  // uniform over the wave
      u32x4 kb[kGroups][2];
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        const u32x4* row =
            reinterpret_cast<const u32x4*>(g.k_pages + (size_t)min(rid[u], max_row) * kHeadDim);
        kb[u][0] = __builtin_nontemporal_load(row + part);
        kb[u][1] = __builtin_nontemporal_load(row + part + 8);
      }
      {
        const int wn = wbase + kPoolEntries;  // clamped into the pool: in bounds
#pragma unroll
        for (int u = 0; u < kGroups; ++u) rid[u] = prow[min(wn + u * 8 + rs, n - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        float m = -INFINITY;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) a = dot2_bf16(qv[h][i], kb[u][0][i], a);
#pragma unroll
          for (int i = 0; i < 4; ++i) a = dot2_bf16(qv[h][4 + i], kb[u][1][i], a);
          m = fmaxf(m, group8_sum(a));
        }
        const int e = wbase + u * 8 + rs;
        if (part == 0 && e < n) {
          sc[e] = m;
          if (counted) atomicAdd(&lh[order_key(m) >> 20], 1u);
        }
      }
    }
  } else {
    const int j = lane & 15, g4 = lane >> 4;
    u32x4 qf[4];
    load_q_frag<G>(q, g, b, kvh, lane, qf);
    constexpr int kTiles = kPoolEntries / 4 / 16;
    for (int c = 0; c < chunks; ++c) {
      const int wbase = base + c * kPoolEntries + wave * (kPoolEntries / 4);
      if (wbase >= n) break;  // uniform over the wave
      uint32_t rid[kTiles];
#pragma unroll
      for (int u = 0; u < kTiles; ++u) rid[u] = prow[min(wbase + u * 16 + j, n - 1)];
      u32x4 kf[kTiles][4];
#pragma unroll
      for (int u = 0; u < kTiles; ++u) {
        const u32x4* row =
            reinterpret_cast<const u32x4*>(g.k_pages + (size_t)min(rid[u], max_row) * kHeadDim);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) kf[u][s4] = __builtin_nontemporal_load(row + g4 + 4 * s4);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kTiles; ++u) {
        const float m = group_max<G>(qk_tile(qf, kf[u]), g4);
        const int e = wbase + u * 16 + j;
        if (g4 == 0 && e < n) {
          sc[e] = m;
          if (counted) atomicAdd(&lh[order_key(m) >> 20], 1u);
        }
      }
    }
  }
  if (counted) {
    lds_barrier();
    flush_hist(lh, ws.ghist + (size_t)p * kCoarseBins);
  }
}

// ---------------------------------------------------------------------------
// INT2 proposal keys ("Prism Attention", Section 4.2, Eqs. 7-9)
// ---------------------------------------------------------------------------
// A token's key is stored as 128 two-bit codes (32 bytes) and, per group of 32
// dimensions, a bf16 scale alpha and zero point beta (16 bytes), in arrays
// paged exactly like K, so a row id addresses both.  Code of dimension d =
// 32 s + 8 u + j (group s, lane quarter u, element j): 32-bit word 2u + s/2 of
// the token's eight, bit 2 t + 16 (j % 2) with t = 4 (s % 2) + j / 2.  The
// MFMA B-operand fragment of lane quarter u for group s is then word 2u + s/2,
// whose element pairs (j, j + 1) sit 16 bits apart: one shift and one mask put
// a pair into both halves of a bf16x2 register.

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {  // nearest, ties to even
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eq. 8 on one key row, by one whole wave (every lane active).  Lane l holds
// dimensions 2l and 2l + 1, so a group of 32 dimensions is one 16-lane row of
// the wave.  Per group: beta = min, alpha = (max - min) / 3 rounded to bf16,
// code = the nearest integer (ties to even) to (k - beta) / alpha clipped to
// [0, 3], 0 when alpha = 0; the subtraction and division are IEEE float32 (the
// oracle takes the same decisions in the same precision).  -0 is read as +0.
// quantize_kernel applies it to the keys of positions [max(0, L - num_new), L)
// of every (sequence, KV head) (num_new <= 0: every position), 16 rows per
// wave; the scoring kernels apply it to a decode step's new keys before they
// score them (Geometry::new_keys).  x: the row's 32-bit word `lane`.
// Code of one element: rint(fl(d / alpha)) clipped to [0, 3], ties to even
// (d = v - min >= 0, alpha > 0).  The quotient from the approximate reciprocal
// ra (int2_recip) is within a few ulp of fl(d / alpha), so it rounds the same
// way unless it lies within 1e-5 of a half-integer; only then, or when ra is
// NaN, is the IEEE quotient taken.
__device__ __forceinline__ float int2_recip(float alpha) {
  // far from 1 the reciprocal could leave the normal range: every element then
  // takes the IEEE quotient
  return (alpha >= 0x1p-100f && alpha <= 0x1p100f) ? __builtin_amdgcn_rcpf(alpha)
                                                   : __builtin_nanf("");
}
__device__ __forceinline__ uint32_t int2_code(float d, float alpha, float ra) {
  const float q = d * ra;
  float r = rintf(q);
  if (!(fabsf(q - r) <= 0.49999f)) r = rintf(__fdiv_rn(d, alpha));
  return (uint32_t)__builtin_amdgcn_fmed3f(r, 0.f, 3.f);
}

__device__ __forceinline__ void quantize_value(uint32_t x, size_t row, int lane,
                                               uint8_t* __restrict__ codes,
                                               uint16_t* __restrict__ scales) {
  const float v0 = __uint_as_float(x << 16) + 0.0f;
  const float v1 = __uint_as_float(x & 0xFFFF0000u) + 0.0f;
  // min and max over the 16-lane row (quad, half row, row; every lane gets
  // both), on order-preserving integer keys: integer min and max take their
  // DPP operand directly, with no float canonicalisation in between
  const uint32_t k0 = order_key(v0), k1 = order_key(v1);
  uint32_t kn = min(k0, k1), kx = max(k0, k1);
  kn = min(kn, dpp<kQuadXor1, 0xf>(0xFFFFFFFFu, kn));  // old = the identity: one DPP op each
  kx = max(kx, dpp<kQuadXor1, 0xf>(0u, kx));
  kn = min(kn, dpp<kQuadXor2, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kQuadXor2, 0xf>(0u, kx));
  kn = min(kn, dpp<kRowHalfMirror, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kRowHalfMirror, 0xf>(0u, kx));
  kn = min(kn, dpp<kRowMirror, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kRowMirror, 0xf>(0u, kx));
  const float mn = key_value(kn), mx = key_value(kx);
  const uint32_t ab = f32_to_bf16_bits(__fdiv_rn(mx - mn, 3.0f));
  const float alpha = __uint_as_float(ab << 16);
  uint32_t c0 = 0u, c1 = 0u;
  if (alpha != 0.f) {
    const float ra = int2_recip(alpha);
    c0 = int2_code(v0 - mn, alpha, ra);
    c1 = int2_code(v1 - mn, alpha, ra);
  }
  // dimensions 2l, 2l + 1: group s = l / 16, quarter u = (l % 16) / 4, elements
  // j = 2 (l % 4) and j + 1 -> word 2u + s/2, bits 2 (4 (s % 2) + l % 4) (+ 16)
  const int s4 = lane >> 4;
  uint32_t wd = (c0 | (c1 << 16)) << (2 * (4 * (s4 & 1) + (lane & 3)));
  wd |= dpp<kQuadXor1, 0xf>(wd, wd);
  wd |= dpp<kQuadXor2, 0xf>(wd, wd);
  wd = xor16_or(wd);  // groups 2m and 2m + 1 share a word
  if ((lane & 3) == 0 && (s4 & 1) == 0)
    reinterpret_cast<uint32_t*>(codes + row * (kHeadDim / 4))[2 * ((lane & 15) >> 2) + (s4 >> 1)] =
        wd;
  if ((lane & 15) == 0)  // alpha in the low half, beta in the high half
    reinterpret_cast<uint32_t*>(scales)[row * 4 + s4] = ab | (__float_as_uint(mn) & 0xFFFF0000u);
}

// The same for a row read here (lane l: dimensions 2l, 2l + 1).
__device__ __forceinline__ void quantize_row(const Geometry& g, size_t row, int lane,
                                             uint8_t* __restrict__ codes,
                                             uint16_t* __restrict__ scales) {
  quantize_value(reinterpret_cast<const uint32_t*>(g.k_pages + row * kHeadDim)[lane], row, lane,
                 codes, scales);
}

// Positions [lo, hi) of sequence b, KV head kvh, one wave per position.  Every
// wave of the workgroup calls it (the loop bound is uniform over a wave).
__device__ __forceinline__ void quantize_positions(const Geometry& g, int b, int kvh, int lo,
                                                   int hi, int lane, int wave, int waves) {
  for (int pos = lo + wave; pos < hi; pos += waves)
    quantize_row(g, (size_t)row_id(g, b, kvh, pos), lane, g.k_codes, g.k_scales);
}

// Prefill: a wave quantizes kQuantRows consecutive positions, two rows per
// pass (lanes 0-31 the first, 32-63 the second, four dimensions per lane, so
// a 32-dimension group is 8 lanes), all rows loaded before the first pass.
// Per pass: the group's min and max over its 8 lanes (integer keys, DPP), then
// alpha, the codes, and the code bits OR-combined across the 4 lanes that
// share a 32-bit code word; the same codes and scales quantize_value writes.
constexpr int kQuantRows = 16;
__device__ __forceinline__ void quantize_pair(uint32_t w0, uint32_t w1, size_t row, int lq,
                                              bool live, uint8_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales) {
  // dimensions 4 lq .. 4 lq + 3: group s = lq / 8; quarter u = (lq % 8) / 2;
  // elements j = 4 (lq % 2) + e -> word 2u + s/2, bits 2t (+ 2), (+ 16), t =
  // 4 (s % 2) + 2 (lq % 2)
  const float v0 = __uint_as_float(w0 << 16) + 0.0f;
  const float v1 = __uint_as_float(w0 & 0xFFFF0000u) + 0.0f;
  const float v2 = __uint_as_float(w1 << 16) + 0.0f;
  const float v3 = __uint_as_float(w1 & 0xFFFF0000u) + 0.0f;
  uint32_t kn = order_key(fminf(fminf(v0, v1), fminf(v2, v3)));
  uint32_t kx = order_key(fmaxf(fmaxf(v0, v1), fmaxf(v2, v3)));
  kn = min(kn, dpp<kQuadXor1, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kQuadXor1, 0xf>(0u, kx));
  kn = min(kn, dpp<kQuadXor2, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kQuadXor2, 0xf>(0u, kx));
  kn = min(kn, dpp<kRowHalfMirror, 0xf>(0xFFFFFFFFu, kn));
  kx = max(kx, dpp<kRowHalfMirror, 0xf>(0u, kx));
  const float mn = key_value(kn), mx = key_value(kx);
  const uint32_t ab = f32_to_bf16_bits(__fdiv_rn(mx - mn, 3.0f));
  const float alpha = __uint_as_float(ab << 16);
  uint32_t c0 = 0u, c1 = 0u, c2 = 0u, c3 = 0u;
  if (alpha != 0.f) {
    const float ra = int2_recip(alpha);
    c0 = int2_code(v0 - mn, alpha, ra);
    c1 = int2_code(v1 - mn, alpha, ra);
    c2 = int2_code(v2 - mn, alpha, ra);
    c3 = int2_code(v3 - mn, alpha, ra);
  }
  const int s = lq >> 3;
  uint32_t wd = (c0 | (c1 << 16) | (c2 << 2) | (c3 << 18)) << (2 * (4 * (s & 1) + 2 * (lq & 1)));
  wd |= dpp<kQuadXor1, 0xf>(0u, wd);
  wd |= dpp<kRowRor8, 0xf>(0u, wd);  // groups 2m and 2m + 1 share a word
  if (live && (lq & 1) == 0 && (s & 1) == 0)
    reinterpret_cast<uint32_t*>(codes + row * (kHeadDim / 4))[2 * ((lq & 7) >> 1) + (s >> 1)] = wd;
  if (live && (lq & 7) == 0)  // alpha in the low half, beta in the high half
    reinterpret_cast<uint32_t*>(scales)[row * 4 + s] = ab | (__float_as_uint(mn) & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void quantize_kernel(Geometry g, int num_new, int chunks,
                                                       uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int p = blockIdx.x / chunks, c = blockIdx.x - p * chunks;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int n = seq_len_of(g, b);
  const int first = (num_new > 0 && num_new < n) ? n - num_new : 0;
  const int pos0 = first + (c * 4 + wv) * kQuantRows;
  if (pos0 >= n) return;  // uniform over the wave
  const int h = lane >> 5, lq = lane & 31;
  // the wave's positions lie in one page unless its range starts unaligned
  const int plast = min(pos0 + kQuantRows - 1, n - 1);
  const bool one_page = (pos0 >> 6) == (plast >> 6);
  const uint32_t row0 = row_id(g, b, kvh, pos0);
  constexpr int kPairs = kQuantRows / 2;
  uint32_t rows[kPairs];
  u32x2 x[kPairs];
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int pos = min(pos0 + 2 * i + h, n - 1);
    rows[i] = one_page ? row0 + (uint32_t)(pos - pos0) : row_id(g, b, kvh, pos);
    x[i] = reinterpret_cast<const u32x2*>(g.k_pages + (size_t)rows[i] * kHeadDim)[lq];
  }
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    // both halves run every pass (a DPP row lies inside one half); a half
    // past the sequence's end stores nothing
    quantize_pair(x[i][0], x[i][1], rows[i], lq, pos0 + 2 * i + h < n, codes, scales);
  }
}

// The group's query heads as MFMA A operands against INT2 keys.  A tile is 16
// rows (head h, quantization group m) = row 4 (h mod 4) + m, block diagonal
// over the four group steps: at step s, row (h, m) holds q_h's dimensions of
// group s when m = s and zeros otherwise.  The B operand of step s is the
// token's group-s codes c widened to the bf16 value 2 + c / 2 (exact), so the
// accumulator of row (h, m) is 2 Q_hm + D_hm / 2 with D_hm = sum over group m
// of q c and Q_hm = the sum of q over group m, and
//   <q_h, k-hat> = sum_m alpha_m D_hm + beta_m Q_hm
//               = sum_m alpha_m (2 acc_hm - 4 Q_hm) + beta_m Q_hm.
// Output lane (token j, quarter g4) holds rows 4 g4 + m: head 4t + g4 of tile t.
// (a & m) | c in one VALU instruction.  The compiler keeps the two constants
// as literals of a VOP2 AND and a VOP2 OR (VOP3 takes no literal on gfx9);
// with the mask in a scalar register and c in a vector register the VOP3
// form does both, one instruction of the INT2 operand build per code dword.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

template <int G>
struct Int2Query {
  static constexpr int kTiles = (4 * G + 15) / 16;
  u32x4 a[kTiles][4];
  float qs[kTiles][4];   // Q of the output lane's head, per group
  float nq4[kTiles][4];  // -4 Q

  __device__ __forceinline__ void load(const uint16_t* q, const Geometry& g, int b, int kvh,
                                       int lane) {
    const int r = lane & 15, g4 = lane >> 4;
    const uint16_t* qb = q + ((size_t)b * g.hq + (size_t)kvh * G) * kHeadDim;
    const u32x4 twos = {0x40004000u, 0x40004000u, 0x40004000u, 0x40004000u};  // bf16 2.0
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int h = 4 * t + r / 4, m = r % 4;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (h < G) x = reinterpret_cast<const u32x4*>(qb + (size_t)h * kHeadDim)[4 * m + g4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) a[t][s4] = (m == s4) ? x : u32x4{0u, 0u, 0u, 0u};
      // the same contraction against code 0 (every B element 2.0) gives 2 Q_hm
      // in the accumulator layout the scores use
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[t][s4]),
                                                      __builtin_bit_cast(bf16x8, twos), acc, 0, 0,
                                                      0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qs[t][i] = 0.5f * acc[i];
        nq4[t][i] = -2.f * acc[i];
      }
    }
  }

  // Relevance of the lane's token (max over the group's heads), valid in every
  // lane of the token's column.  codes: the lane quarter's two code words;
  // scl: the token's (alpha, beta) pairs.
  __device__ __forceinline__ float score(u32x2 codes, u32x4 scl, int g4) const {
    u32x4 bf[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const uint32_t wd = codes[s4 >> 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * (s4 & 1) + i;
        const uint32_t sh = t <= 2 ? (wd << (5 - 2 * t)) : (wd >> (2 * t - 5));
        bf[s4][i] = and_or(sh, 0x00600060u, 0x40004000u);
      }
    }
    float best = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[t][s4]),
                                                      __builtin_bit_cast(bf16x8, bf[s4]), acc, 0,
                                                      0, 0);
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float alpha = __uint_as_float(scl[i] << 16);
        const float beta = __uint_as_float(scl[i] & 0xFFFF0000u);
        v = fmaf(alpha, fmaf(2.f, acc[i], nq4[t][i]), fmaf(beta, qs[t][i], v));
      }
      if (4 * t + g4 < G) best = fmaxf(best, v);
    }
    if (G > 1) best = xor16_max(best);
    if (G > 2) best = xor32_max(best);
    return best;
  }
};

// Anchor-layer relevance from INT2 keys: the score list and the coarse
// histogram are those of score_anchor_kernel.  A workgroup scores
// kInt2Entries tokens; each wave takes a quarter of them in rounds of two
// pages (per 16-token tile a lane reads its quarter's 8 bytes of codes and the
// token's 16 bytes of scales), four MFMAs per tile and 16-row tile of (head,
// group) rows.  A round's loads are not prefetched during the previous round:
// at 104 registers four waves share a SIMD, and the waves' interleaving hides
// the loads better than a second buffer at two waves per SIMD did (21 against
// 23.6 us at 128K).
constexpr int kInt2Entries = 1024;
constexpr int kInt2RoundPages = 2;
constexpr int kInt2Rounds = kInt2Entries / 4 / kPageSize / kInt2RoundPages;

template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_anchor_int2_kernel(
    Geometry g, Workspace ws, const uint16_t* __restrict__ q, int wgs) {
  __shared__ uint32_t lh[kCoarseBins];
  int p, w;
  map_block(blockIdx.x, g.problems(), wgs, &p, &w);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int n = seq_len_of(g, b);
  if (w * kInt2Entries >= n) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kRoundTokens = kInt2RoundPages * kPageSize;
  const int wbase = w * kInt2Entries + wave * (kInt2Entries / 4);
  for (int i = threadIdx.x; i < kCoarseBins; i += kScoreThreads) lh[i] = 0u;
  // the step's new keys inside this workgroup's range get their codes first
  const int qlo = max(max(n - g.new_keys, 0), w * kInt2Entries);
  const int qhi = min(n, (w + 1) * kInt2Entries);
  if (g.new_keys > 0 && qlo < qhi) {  // uniform over the workgroup
    quantize_positions(g, b, kvh, qlo, qhi, lane, wave, kScoreThreads / 64);
    __syncthreads();  // the rows' stores before any wave loads them
  } else {
    lds_barrier();
  }
  if (wbase < n) {
    float* sc = ws.scores + (size_t)p * g.n_cap;
    const int last_page = (n - 1) >> 6;
    const int rounds = min(kInt2Rounds, (n - wbase + kRoundTokens - 1) / kRoundTokens);
    const int j = lane & 15, g4 = lane >> 4;
    Int2Query<G> qq;
    qq.load(q, g, b, kvh, lane);
    const u32x2* cbase = reinterpret_cast<const u32x2*>(g.k_codes);
    const u32x4* sbase = reinterpret_cast<const u32x4*>(g.k_scales);
    auto fetch = [&](int r, u32x2 (&cr)[kInt2RoundPages][4], u32x4 (&sr)[kInt2RoundPages][4]) {
#pragma unroll
      for (int pg = 0; pg < kInt2RoundPages; ++pg) {
        const int lp = min((wbase >> 6) + r * kInt2RoundPages + pg, last_page);
        const size_t row0 = (size_t)row_id_of_page(g, phys_page(g, b, lp), kvh, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const size_t row = row0 + u * 16 + j;
          cr[pg][u] = __builtin_nontemporal_load(cbase + row * 4 + g4);
          sr[pg][u] = __builtin_nontemporal_load(sbase + row);
        }
      }
    };
#pragma unroll
    for (int r = 0; r < kInt2Rounds; ++r) {
      if (r >= rounds) break;  // uniform over the wave
      u32x2 cb[kInt2RoundPages][4];
      u32x4 sb[kInt2RoundPages][4];
      fetch(r, cb, sb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pg = 0; pg < kInt2RoundPages; ++pg) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float m = qq.score(cb[pg][u], sb[pg][u], g4);
          const int e = wbase + r * kRoundTokens + pg * 64 + u * 16 + j;
          if (g4 == 0 && e < n) {
            sc[e] = m;
            atomicAdd(&lh[order_key(m) >> 20], 1u);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();
  flush_hist(lh, ws.ghist + (size_t)p * kCoarseBins);
}

// Refined-layer relevance from INT2 keys over the pool's row ids; work split,
// scores and optional histogram as in score_pool_kernel.
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_pool_int2_kernel(
    Geometry g, Workspace ws, const uint16_t* __restrict__ q, int wgs, int chunks, int hist) {
  __shared__ uint32_t lh[kCoarseBins];
  int p, w;
  map_block(blockIdx.x, g.problems(), wgs, &p, &w);
  const int n = clampi(ws.pool_len[p], 0, g.n_cap);
  const int base = w * chunks * kPoolEntries;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  if (g.new_keys > 0 && (base < n || (w == 0 && n == 0))) {  // uniform over the workgroup
    // The step's new keys that can be among this workgroup's entries get
    // their codes before it loads any.  Pool positions ascend, so new keys
    // can only be the pool's last new_keys entries; the workgroup holding the
    // last entry (workgroup 0 if the pool is empty) takes every new key, so
    // those outside the pool are written as well.
    const int L = seq_len_of(g, b);
    int lo = max(L - g.new_keys, 0), hi = L;
    if (base < n) {
      const int last = min(base + chunks * kPoolEntries, n) - 1;
      if (last < n - g.new_keys) {
        hi = lo;  // every entry here precedes the new keys
      } else if (last < n - 1) {
        const int32_t* ppos = ws.pool_pos + (size_t)p * g.n_cap;
        lo = max(lo, ppos[base]);
        hi = min(hi, clampi(ppos[last], -1, L - 1) + 1);
      }
    }
    if (lo < hi) {
      quantize_positions(g, b, kvh, lo, hi, lane, wave, kScoreThreads / 64);
      __syncthreads();  // the rows' stores before any wave loads them
    }
  }
  if (base >= n) return;  // uniform over the workgroup
  const bool counted = hist != 0 && n > kSmall;  // uniform over the workgroup
  if (counted) {
    for (int i = threadIdx.x; i < kCoarseBins; i += kScoreThreads) lh[i] = 0u;
    lds_barrier();
  }
  const uint32_t* prow = ws.pool_row + (size_t)p * g.n_cap;
  float* sc = ws.scores + (size_t)p * g.n_cap;
  const uint32_t max_row = (uint32_t)g.num_pages * (uint32_t)(g.hkv * kPageSize) - 1u;
  const int j = lane & 15, g4 = lane >> 4;
  Int2Query<G> qq;
  qq.load(q, g, b, kvh, lane);
  const u32x2* cbase = reinterpret_cast<const u32x2*>(g.k_codes);
  const u32x4* sbase = reinterpret_cast<const u32x4*>(g.k_scales);
  constexpr int kTiles = kPoolEntries / 4 / 16;
  for (int c = 0; c < chunks; ++c) {
    const int wbase = base + c * kPoolEntries + wave * (kPoolEntries / 4);
    if (wbase >= n) break;  // uniform over the wave
    u32x2 cb[kTiles];
    u32x4 sb[kTiles];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      const size_t row = min(prow[min(wbase + u * 16 + j, n - 1)], max_row);
      cb[u] = __builtin_nontemporal_load(cbase + row * 4 + g4);
      sb[u] = __builtin_nontemporal_load(sbase + row);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      const float m = qq.score(cb[u], sb[u], g4);
      const int e = wbase + u * 16 + j;
      if (g4 == 0 && e < n) {
        sc[e] = m;
        if (counted) atomicAdd(&lh[order_key(m) >> 20], 1u);
      }
    }
  }
  if (counted) {
    lds_barrier();
    flush_hist(lh, ws.ghist + (size_t)p * kCoarseBins);
  }
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
constexpr int kMaxPages = kMaxSeqLen / kPageSize;

constexpr int kPairMax = 256;  // bucket entries ranked against each other directly

struct SelectSmem {
  int32_t bt[kMaxPages];              // the sequence's block table row (physical pages)
  alignas(16) uint32_t bitmap[kMaxSeqLen / 32];  // selection marks in list order
  uint32_t hist[4096 + 1024 + 1024];  // bucket histogram / three radix levels
  uint32_t cbuf[2 * kCand];           // list keys / sample keys / candidate keys and indices
  int32_t apos[kMaxKappa];            // the emitted set, for the pool build
  uint32_t pair[kPairMax];            // keys of the threshold bucket
  uint32_t ured[32];                  // per-wave minima and maxima
  int tmp[NT / 64 + 1];
  int res[9];
  int cnt[2];
};

struct SelList {
  const float* sc;       // relevance in list order
  const int32_t* plist;  // list index -> position (null: identity)
  const uint32_t* prow;  // list index -> row id (null: from the block table)
  int n, K, b, kvh;
  int32_t* o1;
  int32_t* o2;
  uint32_t* srow;
  int32_t* ent;          // if set: the set's list indices only (rank order), nothing else
};

__device__ __forceinline__ void emit_at(const Geometry& g, const SelList& c, int e, int pos,
                                        uint32_t row, int o, SelectSmem& sm) {
  if (c.ent) {
    c.ent[o] = e;
    return;
  }
  c.o1[o] = pos;
  if (c.o2) c.o2[o] = pos;
  c.srow[o] = row;
  sm.apos[o] = pos;
}

__device__ __forceinline__ void emit_entry(const Geometry& g, const SelList& c, int e, int o,
                                           SelectSmem& sm) {
  if (c.ent) {
    c.ent[o] = e;
    return;
  }
  const int pos = c.plist ? c.plist[e] : e;
  const uint32_t row = c.prow ? c.prow[e] : row_id_of_page(g, sm.bt[pos >> 6], c.kvh, pos);
  emit_at(g, c, e, pos, row, o, sm);
}

__device__ __forceinline__ void emit_empty(const SelList& c, int o, SelectSmem& sm) {
  if (c.ent) {
    c.ent[o] = -1;
    return;
  }
  c.o1[o] = -1;
  if (c.o2) c.o2[o] = -1;
  c.srow[o] = kNoRow;
  sm.apos[o] = -1;
}

// Wave 0 finds a bin and publishes it in sm.res[slot..slot+2]; all threads
// read it after the barrier.
template <int NB, typename Sm>
__device__ Bin find_publish(const uint32_t* h, int need, Sm& sm, int slot) {
  if (threadIdx.x < 64) {
    const Bin r = wave_find_bin<NB>(h, need);
    if (threadIdx.x == 0) {
      sm.res[slot] = r.bin;
      sm.res[slot + 1] = r.above;
      sm.res[slot + 2] = r.count;
    }
  }
  lds_barrier();
  return Bin{sm.res[slot], sm.res[slot + 1], sm.res[slot + 2]};
}

// The bin of a 4096-bin histogram holding the need-th largest entry (counted
// down from the top bin), with the count of higher bins and its own count;
// bin = -1 if the histogram holds fewer than need.  Thread t owns bins
// 4092 - 4t .. 4095 - 4t, so an exclusive scan in thread order counts from the
// top.  Uniform over the block; contains barriers.
template <typename Sm>
__device__ Bin block_find_top(const uint32_t* h, int need, Sm& sm) {
  static_assert(NT * 4 == 4096, "four bins per thread");
  const int t = threadIdx.x;
  const u32x4 c4 = *reinterpret_cast<const u32x4*>(h + 4092 - 4 * t);
  const int sum = (int)(c4[0] + c4[1] + c4[2] + c4[3]);
  if (t == 0) {
    sm.res[3] = -1;
    sm.res[4] = 0;
    sm.res[5] = 0;
  }
  int tot;
  const int above = block_excl_scan<NT>(sum, sm.tmp, &tot);
  if (above < need && need <= above + sum) {
    int a = above, k = 3, cnt = (int)c4[3];
    if (need > a + (int)c4[3]) {
      a += (int)c4[3];
      k = 2;
      cnt = (int)c4[2];
      if (need > a + (int)c4[2]) {
        a += (int)c4[2];
        k = 1;
        cnt = (int)c4[1];
        if (need > a + (int)c4[1]) {
          a += (int)c4[1];
          k = 0;
          cnt = (int)c4[0];
        }
      }
    }
    sm.res[3] = 4092 - 4 * t + k;
    sm.res[4] = a;
    sm.res[5] = cnt;
  }
  lds_barrier();
  return Bin{sm.res[3], sm.res[4], sm.res[5]};
}

// Threshold of a selection: T is the need-th largest key; need_eq entries
// equal to T are taken (lowest list index first) out of eq_total equal to T.
struct Thresh {
  uint32_t T;
  int need_eq, eq_total;
};

// The need-th largest of the keys the block holds in registers: thread t
// holds key[0 .. nv) (nv <= R); 1 <= need <= total count.
//
// Scores are binned into 4096 equal-width buckets between the smallest and
// the largest score.  The map score -> bucket is monotone (each rounding step
// of (s - lo) * (4096 / range) is), so a higher bucket holds only higher
// scores.  The bucket holding the need-th largest is found from the top; if it
// holds at most kPairMax entries they are ranked against each other (four
// threads per entry).  A larger bucket (scores concentrated far inside their
// range), a zero range or a non-finite range falls back to an exact
// 12/10/10-bit radix over the keys.
template <int R, typename Sm>
__device__ __forceinline__ Thresh find_threshold(const uint32_t (&key)[R], int nv, int need, Sm& sm) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i < nv) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  kmin = wave_min_u(kmin);
  kmax = wave_max_u(kmax);
  if (lane == 0) {
    sm.ured[wave] = kmin;
    sm.ured[16 + wave] = kmax;
  }
  for (int i = t; i < 4096; i += NT) sm.hist[i] = 0u;
  if (t == 0) sm.cnt[0] = 0;
  lds_barrier();
  kmin = wave_min_u(lane < NT / 64 ? sm.ured[lane] : 0xFFFFFFFFu);
  kmax = wave_max_u(lane < NT / 64 ? sm.ured[16 + lane] : 0u);
  const float lo = key_value(kmin);
  const float range = key_value(kmax) - lo;
  const float inv = 4096.f / range;
  if (range > 0.f && range <= 3.0e38f && inv <= 3.0e38f) {
    int bk[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
      bk[i] = i < nv ? clampi((int)((key_value(key[i]) - lo) * inv), 0, 4095) : -1;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (bk[i] >= 0) atomicAdd(&sm.hist[bk[i]], 1u);
    lds_barrier();
    const Bin B = block_find_top(sm.hist, need, sm);
    if (B.bin >= 0 && B.count <= kPairMax) {
      // gather the bucket's keys: one LDS atomic per wave
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < R; ++i) cnt += bk[i] == B.bin ? 1 : 0;
      const int inc = wave_incl_scan(cnt);
      const int wtot = (int)lane63((uint32_t)inc);
      if (wtot) {
        int off = 0;
        if (lane == 0) off = atomicAdd(&sm.cnt[0], wtot);
        int slot = __builtin_amdgcn_readfirstlane(off) + inc - cnt;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (bk[i] == B.bin) {
            if (slot < kPairMax) sm.pair[slot] = key[i];
            ++slot;
          }
        }
      }
      lds_barrier();
      const int pc = min(B.count, kPairMax);
      const int need_b = need - B.above;
      const int x = t >> 2, part = t & 3;
      int gt = 0, ge = 0;
      uint32_t kx = 0u;
      if (x < pc) {
        kx = sm.pair[x];
        for (int y = part; y < pc; y += 4) {
          const uint32_t ky = sm.pair[y];
          gt += ky > kx ? 1 : 0;
          ge += ky >= kx ? 1 : 0;
        }
      }
      gt += (int)dpp<kQuadXor1, 0xf>(0u, (uint32_t)gt);
      ge += (int)dpp<kQuadXor1, 0xf>(0u, (uint32_t)ge);
      gt += (int)dpp<kQuadXor2, 0xf>(0u, (uint32_t)gt);
      ge += (int)dpp<kQuadXor2, 0xf>(0u, (uint32_t)ge);
      if (x < pc && part == 0 && gt < need_b && need_b <= ge) {
        sm.res[0] = (int)kx;  // every thread that writes writes the same values
        sm.res[1] = need_b - gt;
        sm.res[2] = ge - gt;
      }
      lds_barrier();
      return Thresh{(uint32_t)sm.res[0], sm.res[1], sm.res[2]};
    }
  }
  // exact radix over the keys
  uint32_t* h1 = sm.hist;
  uint32_t* h2 = sm.hist + 4096;
  uint32_t* h3 = sm.hist + 5120;
  lds_barrier();
  for (int i = t; i < 6144; i += NT) sm.hist[i] = 0u;
  lds_barrier();
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nv) atomicAdd(&h1[key[i] >> 20], 1u);
  lds_barrier();
  const Bin a = find_publish<4096>(h1, need, sm, 0);
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nv && (int)(key[i] >> 20) == a.bin) atomicAdd(&h2[(key[i] >> 10) & 1023u], 1u);
  lds_barrier();
  const Bin bb = find_publish<1024>(h2, need - a.above, sm, 3);
  const uint32_t pre = ((uint32_t)a.bin << 10) | (uint32_t)bb.bin;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nv && (key[i] >> 10) == pre) atomicAdd(&h3[key[i] & 1023u], 1u);
  lds_barrier();
  const Bin cc = find_publish<1024>(h3, need - a.above - bb.above, sm, 6);
  return Thresh{(pre << 10) | (uint32_t)cc.bin, need - a.above - bb.above - cc.above, cc.count};
}

// Which of a thread's R consecutive list entries (keys in registers, valid
// for i < nv) belong to the top-K of the n-entry list: bit i of the result.
// Ties at the threshold go to the lowest list indices (thread order is list
// order).  Contains barriers: call uniformly.
template <int R, typename Sm>
__device__ __forceinline__ uint32_t top_k_mask(const uint32_t (&key)[R], int nv, int n, int K, Sm& sm) {
  static_assert(R <= 32, "one mask bit per entry");
  if (n <= K) return nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);
  const Thresh th = find_threshold<R>(key, nv, K, sm);
  uint32_t take = 0u;
  if (th.eq_total == th.need_eq) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < nv && key[i] >= th.T) take |= 1u << i;
  } else {  // more entries equal T than needed: the lowest list indices win
    int my_eq = 0;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < nv && key[i] == th.T) ++my_eq;
    int tot;
    int r = block_excl_scan<NT>(my_eq, sm.tmp, &tot);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (i < nv && key[i] > th.T) take |= 1u << i;
      if (i < nv && key[i] == th.T) {
        if (r < th.need_eq) take |= 1u << i;
        ++r;
      }
    }
  }
  return take;
}

// Loads R consecutive 32-bit entries starting at e0 (a multiple of R below the
// row's capacity, a multiple of 64) as R / 4 vector loads.
template <int R, typename T>
__device__ __forceinline__ void load_run(const T* base, int e0, uint32_t (&v)[R]) {
#pragma unroll
  for (int k = 0; k < R / 4; ++k) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(base + e0 + 4 * k);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[4 * k + i] = x[i];
  }
}

// Lists of at most kSmall entries.  Thread t holds entries R t .. R t + R - 1
// (keys, and for a pool their positions and row ids, all loaded up front), so
// counts scanned in thread order give ascending output positions directly.
template <int R>
__device__ __forceinline__ void select_small(const Geometry& g, const SelList& c, SelectSmem& sm) {
  const int t = threadIdx.x;
  const int e0 = R * t;
  const int nv = clampi(c.n - e0, 0, R);  // valid entries of this thread
  const int ea = e0 < c.n ? e0 : 0;       // entries past n are loaded but not used
  uint32_t key[R], pl[R], pr[R];
  load_run<R>(c.sc, ea, key);
  if (c.plist) {
    load_run<R>(c.plist, ea, pl);
    load_run<R>(c.prow, ea, pr);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) key[i] = order_key(__uint_as_float(key[i]));
  const uint32_t take = top_k_mask<R>(key, nv, c.n, c.K, sm);
  int total;
  int o = block_excl_scan<NT>(__popc(take), sm.tmp, &total);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (take & (1u << i)) {
      if (o < c.K) {
        const int pos = c.plist ? (int)pl[i] : e0 + i;
        const uint32_t row = c.prow ? pr[i] : row_id_of_page(g, sm.bt[pos >> 6], c.kvh, pos);
        emit_at(g, c, e0 + i, pos, row, o, sm);
      }
      ++o;
    }
  }
  for (int o2 = total + t; o2 < c.K; o2 += NT) emit_empty(c, o2, sm);
}

// Emission of the entries marked in the LDS bitmap, in list order (ascending
// positions), in two steps.  Compaction into an LDS list in rank order
// (sm.cbuf, free once the marks are final): wave v owns a contiguous range of
// bitmap words, 64 per step, one word per lane; a wave scan of the words'
// bit counts gives each word its first rank, and each lane writes its word's
// marks one after another (a step costs its densest word's count, so runs of
// dense words share steps and the cost stays near the number of marks).  Then
// thread t emits ranks t, t + NT, ... from the list, so the outputs leave as
// coalesced stores and the loads of a pool's positions and row ids (when not
// deferred) are all in flight together.
__device__ __forceinline__ void emit_bitmap(const Geometry& g, const SelList& c, SelectSmem& sm) {
  static_assert(2 * kCand >= kMaxKappa, "the compacted set fits sm.cbuf");
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int words = (c.n + 31) >> 5;
  const int wpw = ((words + NW - 1) / NW + 63) & ~63;  // words per wave, whole steps
  const int wlo = min(words, wave * wpw), whi = min(words, wlo + wpw);
  int cnt = 0;
  for (int i = wlo + lane; i < whi; i += 64) cnt += __popc(sm.bitmap[i]);
  cnt = (int)lane63((uint32_t)wave_incl_scan(cnt));
  lds_barrier();  // earlier readers of sm.tmp are done
  if (lane == 0) sm.tmp[wave] = cnt;
  lds_barrier();
  int o = 0, total = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    o += x < wave ? sm.tmp[x] : 0;
    total += sm.tmp[x];
  }
  int32_t* const lst = reinterpret_cast<int32_t*>(sm.cbuf);
  for (int base = wlo; base < whi && o < c.K; base += 64) {  // uniform over the wave
    const int wi = base + lane;
    uint32_t m = wi < whi ? sm.bitmap[wi] : 0u;
    const int n1 = __popc(m);
    const int inc = wave_incl_scan(n1);
    int r = o + inc - n1;
    o += (int)lane63((uint32_t)inc);
    const int stop = min(c.K, r + n1);
    for (; r < stop; ++r) {
      lst[r] = wi * 32 + (__ffs(m) - 1);
      m &= m - 1u;
    }
  }
  const int lim = min(total, c.K);
  lds_barrier();
  constexpr int PER = kMaxKappa / NT;
  if (c.ent) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int r = t + k * NT;
      if (r < c.K) c.ent[r] = r < lim ? lst[r] : -1;
    }
    return;
  }
  int pos[PER];
  uint32_t row[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {  // every load first
    const int r = t + k * NT;
    const int e = r < lim ? lst[r] : 0;
    pos[k] = c.plist ? c.plist[e] : e;
    row[k] = c.prow ? c.prow[e] : 0u;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int r = t + k * NT;
    if (r < lim) {
      const uint32_t rw = c.prow ? row[k] : row_id_of_page(g, sm.bt[pos[k] >> 6], c.kvh, pos[k]);
      emit_at(g, c, lst[r], pos[k], rw, r, sm);
    } else if (r < c.K) {
      emit_empty(c, r, sm);
    }
  }
}

// Longer lists.  A strided sample of at most kSample keys brackets the K-th
// largest key between two sample order statistics [klo, khi] (+-4 sigma of the
// sample count plus slack).  One pass over the list marks entries above khi
// in the bitmap and gathers the entries inside the bracket into LDS, where
// the exact K-th key T is found.  If the bracket misses or overflows, an exact
// radix runs over the whole list instead.  The bitmap, read in order, gives
// ascending positions; entries equal to T are taken lowest list index first.
template <typename Sm>
__device__ __forceinline__ void select_large_marks(const SelList& c, Sm& sm) {
  const int t = threadIdx.x, lane = t & 63;
  const int n = c.n, K = c.K;
  uint32_t* h1 = sm.hist;
  uint32_t* h2 = sm.hist + 4096;
  uint32_t* h3 = sm.hist + 5120;
  uint32_t* const ckey = sm.cbuf;
  int32_t* const cidx = reinterpret_cast<int32_t*>(sm.cbuf + kCand);

  const int S = (n + kSample - 1) / kSample;
  const int ns = (n + S - 1) / S;
  const float ks = (float)K * (float)ns / (float)n;
  const int d = (int)ceilf(4.f * sqrtf(ks * (1.f - ks / (float)ns))) + 16;
  const int r_hi = (int)floorf(ks) - d, r_lo = (int)ceilf(ks) + d;

  uint32_t khi = 0xFFFFFFFFu, klo = 0u;
  {
    constexpr int RS = kSample / NT;
    uint32_t key[RS];
#pragma unroll
    for (int u = 0; u < RS; ++u) {
      const int i = u * NT + t;
      key[u] = order_key(c.sc[(size_t)(i < ns ? i : 0) * S]);
    }
    const int nvs = clampi((ns - t + NT - 1) / NT, 0, RS);  // sample u*NT + t exists iff u < nvs
    if (r_hi >= 1) khi = find_threshold<RS>(key, nvs, r_hi, sm).T;
    if (r_lo <= ns) klo = find_threshold<RS>(key, nvs, r_lo, sm).T;
  }
  if (t == 0) {
    sm.cnt[0] = 0;
    sm.cnt[1] = 0;
  }
  lds_barrier();

  // --- one pass over the list: lanes hold 4 consecutive entries; the bitmap
  //     words of a wave's 256 entries are built from ballots, and bracket
  //     entries are appended with one LDS atomic per wave and round ----------------
  int above = 0;  // uniform over the wave
  const int wave = t >> 6;
  for (int base = 0; base < n; base += 4 * NT * kPassUnroll) {
    u32x4 raw[kPassUnroll];
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      const int e0 = base + u * 4 * NT + 4 * t;
      raw[u] = *reinterpret_cast<const u32x4*>(c.sc + (e0 < n ? e0 : 0));
    }
    uint32_t cand = 0u;  // bit 4u + q4: entry inside the bracket
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      const int e0 = base + u * 4 * NT + 4 * t;
      unsigned long long mh[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t key = order_key(__uint_as_float(raw[u][q4]));
        const bool ok = e0 + q4 < n;
        const bool hi = ok && key > khi;
        cand |= (ok && !hi && key >= klo) ? 1u << (4 * u + q4) : 0u;
        mh[q4] = __ballot(hi);
        above += __popcll(mh[q4]);
      }
      // word k of the wave's 256 entries holds lanes 8k .. 8k+7: bit 4i + q4 is
      // bit 8k + i of mask q4
      const int first = base + u * 4 * NT + 256 * wave + 32 * lane;
      if (lane < 8 && first < n) {
        uint32_t word = 0u;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint32_t x = (uint32_t)(mh[q4] >> (8 * lane)) & 0xFFu;
          x = (x | (x << 12)) & 0x000F000Fu;
          x = (x | (x << 6)) & 0x03030303u;
          x = (x | (x << 3)) & 0x11111111u;
          word |= x << q4;
        }
        sm.bitmap[first >> 5] = word;
      }
    }
    const int cnt = __popc(cand);
    const int inc = wave_incl_scan(cnt);
    const int wtot = (int)lane63((uint32_t)inc);
    if (wtot) {
      int off = 0;
      if (lane == 0) off = atomicAdd(&sm.cnt[0], wtot);
      int slot = __builtin_amdgcn_readfirstlane(off) + inc - cnt;
#pragma unroll
      for (int u = 0; u < kPassUnroll; ++u) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if (cand & (1u << (4 * u + q4))) {
            if (slot < kCand) {
              ckey[slot] = order_key(__uint_as_float(raw[u][q4]));
              cidx[slot] = base + u * 4 * NT + 4 * t + q4;
            }
            ++slot;
          }
        }
      }
    }
  }
  if (lane == 0) atomicAdd(&sm.cnt[1], above);
  lds_barrier();
  const int ncand = sm.cnt[0];
  const int need = K - sm.cnt[1];
  lds_barrier();  // every thread has read the counters before they are reused

  if (need >= 1 && need <= ncand && ncand <= kCand) {
    constexpr int RC = kCand / NT;
    uint32_t ck[RC];
#pragma unroll
    for (int u = 0; u < RC; ++u) ck[u] = ckey[min(u * NT + t, kCand - 1)];
    const int nvc = clampi((ncand - t + NT - 1) / NT, 0, RC);
    const Thresh th = find_threshold<RC>(ck, nvc, need, sm);
    for (int i = t; i < ncand; i += NT) {
      const uint32_t key = ckey[i];
      const int e = cidx[i];
      bool take = key > th.T;
      if (key == th.T) {
        if (th.eq_total == th.need_eq) {
          take = true;
        } else {  // rank among equal keys by list index
          int rank = 0;
          for (int i2 = 0; i2 < ncand; ++i2) rank += (ckey[i2] == th.T && cidx[i2] < e) ? 1 : 0;
          take = rank < th.need_eq;
        }
      }
      if (take) atomicOr(&sm.bitmap[e >> 5], 1u << (e & 31));
    }
  } else {
    // exact radix over the whole list
    for (int i = t; i < 6144; i += NT) sm.hist[i] = 0u;
    lds_barrier();
    for (int e = t; e < n; e += NT) atomicAdd(&h1[order_key(c.sc[e]) >> 20], 1u);
    lds_barrier();
    const Bin a = find_publish<4096>(h1, K, sm, 0);
    for (int e = t; e < n; e += NT) {
      const uint32_t key = order_key(c.sc[e]);
      if ((int)(key >> 20) == a.bin) atomicAdd(&h2[(key >> 10) & 1023u], 1u);
    }
    lds_barrier();
    const Bin bb = find_publish<1024>(h2, K - a.above, sm, 3);
    const uint32_t pre = ((uint32_t)a.bin << 10) | (uint32_t)bb.bin;
    for (int e = t; e < n; e += NT) {
      const uint32_t key = order_key(c.sc[e]);
      if ((key >> 10) == pre) atomicAdd(&h3[key & 1023u], 1u);
    }
    lds_barrier();
    const Bin cc = find_publish<1024>(h3, K - a.above - bb.above, sm, 6);
    const uint32_t T = (pre << 10) | (uint32_t)cc.bin;
    const int need_eq = K - a.above - bb.above - cc.above;
    int run = 0;  // equal keys in earlier chunks
    for (int base = 0; base < n; base += NT) {
      const int e = base + t;
      const bool valid = e < n;
      const uint32_t key = valid ? order_key(c.sc[e]) : 0u;
      const bool eq = valid && key == T;
      int tot;
      const int r = block_excl_scan<NT>(eq ? 1 : 0, sm.tmp, &tot);
      const bool take = valid && (key > T || (eq && run + r < need_eq));
      const unsigned long long m = __ballot(take);
      if (lane == 0 && e < n) sm.bitmap[e >> 5] = (uint32_t)m;
      if (lane == 32 && e < n) sm.bitmap[e >> 5] = (uint32_t)(m >> 32);
      run += tot;
    }
  }
  lds_barrier();
}

// Leaves the problem's coarse histogram zero for the next anchor layer (called
// by one workgroup once nothing reads it).  The classify workgroups' candidate
// counts need no reset: every pass writes each count it uses.
__device__ __forceinline__ void reset_selection_counters(const Workspace& ws, int p) {
  uint32_t* gh = ws.ghist + (size_t)p * kCoarseBins;
  for (int i = threadIdx.x; i < kCoarseBins; i += blockDim.x) gh[i] = 0u;
}

// The second classification (the rank-expanded pool's, made in the same
// classify pass as the anchor set's) as the workspace view classified_marks reads.
__device__ __forceinline__ Workspace second_class(const Workspace& ws) {
  Workspace w = ws;
  w.gbits = ws.gbits2;
  w.cand_key = ws.cand_key2;
  w.cand_idx = ws.cand_idx2;
  w.sel_meta = ws.sel_meta2;
  w.cand_cnt = ws.cand_cnt2;
  return w;
}

// Anchor lists longer than kSmall, after the classify kernel: the entries
// above the threshold bin are marked in the workspace bitmap, and the bin's own
// entries (the candidates) are listed with their keys.  The candidates are
// ranked here (directly against each other when there are at most kPairMax,
// else by a threshold search); if the bin held more than kMaxCand of them, an
// exact radix over the whole list runs instead.
template <typename Sm>
__device__ __forceinline__ void classified_marks(const Geometry& g, const Workspace& ws, int p, const SelList& c,
                                 Sm& sm) {
  const int t = threadIdx.x, lane = t & 63;
  const int n = c.n, K = c.K;
  const int words = (n + 31) >> 5;
  const uint32_t* gb = ws.gbits + (size_t)p * (g.n_cap >> 5);
  int marks = 0;
  {
    constexpr int PER = kMaxSeqLen / 32 / NT;  // all of a thread's words loaded at once
    uint32_t m[PER];
    const int last = (g.n_cap >> 5) - 1;  // inside the problem's row: loads need no branch
#pragma unroll
    for (int k = 0; k < PER; ++k) m[k] = gb[min(t + k * NT, last)];
#pragma unroll
    for (int k = 0; k < PER; ++k) m[k] = t + k * NT < words ? m[k] : 0u;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (t + k * NT < words) sm.bitmap[t + k * NT] = m[k];
      marks += __popc(m[k]);
    }
  }
  block_excl_scan<NT>(marks, sm.tmp, &marks);
  const int above = ws.sel_meta[4 * p + 1];
  const int in_bin = ws.sel_meta[4 * p + 2];
  const int need = K - above;
  uint32_t* const ckey = sm.cbuf;
  int32_t* const cidx = reinterpret_cast<int32_t*>(sm.cbuf + kCand);
  // the classify workgroups' candidate regions, gathered into LDS in region
  // order: the counts (at most kClsSlots) are loaded at once and scanned by
  // wave 0 into region starts (sm.ured, free here), then every thread copies
  // up to kMaxCand / NT candidates, all loads issued before any store.  A
  // region that overflowed makes the pass inconsistent (ncand = -1).
  const int regions = (n + kClsEntries - 1) / kClsEntries;
  const int W = cls_regions(g);
  const uint32_t* gk = ws.cand_key + (size_t)p * W * kClsCap;
  const int32_t* gi = ws.cand_idx + (size_t)p * W * kClsCap;
  if (t < 64) {
    // counts are read unsigned and clamped: a classification this call did not
    // make (the rank pool's at rho = 1) leaves arbitrary workspace bytes, and
    // the region starts must stay monotone and each within its region
    const uint32_t cu = t < regions ? ws.cand_cnt[(size_t)p * W + t] : 0u;
    const int c = (int)min(cu, (uint32_t)kClsCap + 1u);
    const int cs = min(c, kClsCap);
    const int inc = wave_incl_scan(cs);
    if (t < regions) sm.ured[t] = (uint32_t)(inc - cs);
    const bool ovf = __ballot(c > kClsCap) != 0ull;
    if (t == 63) {
      sm.res[0] = inc;
      sm.res[1] = ovf ? 1 : 0;
    }
  }
  lds_barrier();
  const int stored = sm.res[0];
  const int ncand = sm.res[1] ? -1 : stored;
  {
    constexpr int CU = kMaxCand / NT;
    uint32_t kk[CU];
    int32_t ii[CU];
    int dst[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int i = t + NT * u;
      dst[u] = -1;
      if (i < min(stored, kMaxCand)) {
        int lo = 0, hi = regions - 1;  // the last region starting at or before i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if ((int)sm.ured[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        const size_t src = (size_t)lo * kClsCap + (size_t)(i - (int)sm.ured[lo]);
        kk[u] = gk[src];
        ii[u] = gi[src];
        dst[u] = i;
      }
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      if (dst[u] >= 0) {
        ckey[dst[u]] = kk[u];
        cidx[dst[u]] = ii[u];
      }
    }
  }
  lds_barrier();
  // the classify pass must agree with itself: as many marks as entries above the
  // threshold bin and as many candidates as entries in it (a histogram left
  // over from an earlier call, e.g. in a fresh workspace, fails this)
  if (marks == above && ncand == in_bin && need >= 1 && need <= ncand && ncand <= kPairMax) {
    // few candidates (the usual case): each one's rank among them, four
    // threads per candidate: candidates with a larger key, or an equal key and
    // a lower list index, come first
    const int x = t >> 2, part = t & 3;
    uint32_t kx = 0u;
    int ix = 0, r = 0;
    if (x < ncand) {
      kx = ckey[x];
      ix = cidx[x];
      for (int y = part; y < ncand; y += 4) {
        const uint32_t ky = ckey[y];
        r += (ky > kx || (ky == kx && cidx[y] < ix)) ? 1 : 0;
      }
    }
    r += (int)dpp<kQuadXor1, 0xf>(0u, (uint32_t)r);
    r += (int)dpp<kQuadXor2, 0xf>(0u, (uint32_t)r);
    if (x < ncand && part == 0 && r < need) {
      const int e = clampi(ix, 0, n - 1);
      atomicOr(&sm.bitmap[e >> 5], 1u << (e & 31));
    }
  } else if (marks == above && ncand == in_bin && need >= 1 && need <= ncand &&
             ncand <= kMaxCand) {
    constexpr int RC = kMaxCand / NT;
    uint32_t ck[RC];
    int32_t ci[RC];
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      const int i = u * NT + t;
      ck[u] = ckey[i];
      ci[u] = cidx[i];
    }
    const int nvc = clampi((ncand - t + NT - 1) / NT, 0, RC);
    const Thresh th = find_threshold<RC>(ck, nvc, need, sm);  // its barriers order the LDS writes
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      if (u < nvc) {
        const int e = clampi(ci[u], 0, n - 1);
        bool take = ck[u] > th.T;
        if (ck[u] == th.T) {
          if (th.eq_total == th.need_eq) {
            take = true;
          } else {  // rank among equal keys by list index
            int rank = 0;
            for (int i2 = 0; i2 < ncand; ++i2) rank += (ckey[i2] == th.T && cidx[i2] < ci[u]) ? 1 : 0;
            take = rank < th.need_eq;
          }
        }
        if (take) atomicOr(&sm.bitmap[e >> 5], 1u << (e & 31));
      }
    }
  } else {
    // More candidates than LDS holds (a wide threshold bin, as when ranking
    // rho * kappa of a long list), but every one stored in its region: a
    // radix select over the candidates' next 10 and last 10 key bits, read
    // from the regions.  Equal keys at the threshold beyond those needed are
    // ranked by list index in LDS; more than kPairMax of them fall back to
    // the exact radix over the whole list below, as does an inconsistent or
    // overflowing classification.
    bool whole_list = true;
    if (marks == above && ncand == in_bin && need >= 1 && need <= ncand) {
      auto cand = [&](int i, uint32_t* key, int32_t* idx) {
        int lo = 0, hi = regions - 1;  // the last region starting at or before i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if ((int)sm.ured[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        const size_t src = (size_t)lo * kClsCap + (size_t)(i - (int)sm.ured[lo]);
        *key = gk[src];
        *idx = gi[src];
      };
      uint32_t* h2 = sm.hist;
      uint32_t* h3 = sm.hist + 1024;
      for (int i = t; i < 2048; i += NT) sm.hist[i] = 0u;
      if (t == 0) sm.cnt[0] = 0;
      lds_barrier();
      for (int i = t; i < ncand; i += NT) {
        uint32_t k;
        int32_t x;
        cand(i, &k, &x);
        atomicAdd(&h2[(k >> 10) & 1023u], 1u);
      }
      lds_barrier();
      const Bin bb = find_publish<1024>(h2, need, sm, 3);
      for (int i = t; i < ncand; i += NT) {
        uint32_t k;
        int32_t x;
        cand(i, &k, &x);
        if ((int)((k >> 10) & 1023u) == bb.bin) atomicAdd(&h3[k & 1023u], 1u);
      }
      lds_barrier();
      const Bin cc = find_publish<1024>(h3, need - bb.above, sm, 6);
      const uint32_t T = ((uint32_t)ws.sel_meta[4 * p] << 20) | ((uint32_t)bb.bin << 10) |
                         (uint32_t)cc.bin;
      const int need_eq = need - bb.above - cc.above;
      if (bb.bin >= 0 && cc.bin >= 0 && need_eq >= 1 &&
          (need_eq == cc.count || cc.count <= kPairMax)) {  // uniform over the workgroup
        whole_list = false;
        if (need_eq != cc.count) {  // the equal keys' list indices, for their ranks
          for (int i = t; i < ncand; i += NT) {
            uint32_t k;
            int32_t x;
            cand(i, &k, &x);
            if (k == T) {
              const int slot = atomicAdd(&sm.cnt[0], 1);
              if (slot < kPairMax) sm.pair[slot] = (uint32_t)x;
            }
          }
          lds_barrier();
        }
        const int ne = min(cc.count, kPairMax);
        for (int i = t; i < ncand; i += NT) {
          uint32_t k;
          int32_t x;
          cand(i, &k, &x);
          bool take = k > T;
          if (k == T) {
            if (need_eq == cc.count) {
              take = true;
            } else {
              int rank = 0;
              for (int y = 0; y < ne; ++y) rank += (int)sm.pair[y] < x ? 1 : 0;
              take = rank < need_eq;
            }
          }
          if (take) {
            const int e = clampi(x, 0, n - 1);
            atomicOr(&sm.bitmap[e >> 5], 1u << (e & 31));
          }
        }
      }
    }
    if (whole_list) {  // exact radix over the whole list
      uint32_t* h1 = sm.hist;
      uint32_t* h2 = sm.hist + 4096;
      uint32_t* h3 = sm.hist + 5120;
      lds_barrier();  // earlier readers of sm.hist are done
      for (int i = t; i < 6144; i += NT) sm.hist[i] = 0u;
      lds_barrier();
      for (int e = t; e < n; e += NT) atomicAdd(&h1[order_key(c.sc[e]) >> 20], 1u);
      lds_barrier();
      const Bin a = find_publish<4096>(h1, K, sm, 0);
      for (int e = t; e < n; e += NT) {
        const uint32_t key = order_key(c.sc[e]);
        if ((int)(key >> 20) == a.bin) atomicAdd(&h2[(key >> 10) & 1023u], 1u);
      }
      lds_barrier();
      const Bin bb = find_publish<1024>(h2, K - a.above, sm, 3);
      const uint32_t pre = ((uint32_t)a.bin << 10) | (uint32_t)bb.bin;
      for (int e = t; e < n; e += NT) {
        const uint32_t key = order_key(c.sc[e]);
        if ((key >> 10) == pre) atomicAdd(&h3[key & 1023u], 1u);
      }
      lds_barrier();
      const Bin cc = find_publish<1024>(h3, K - a.above - bb.above, sm, 6);
      const uint32_t T = (pre << 10) | (uint32_t)cc.bin;
      const int need_eq = K - a.above - bb.above - cc.above;
      int run = 0;  // equal keys in earlier chunks
      for (int base = 0; base < n; base += NT) {
        const int e = base + t;
        const bool valid = e < n;
        const uint32_t key = valid ? order_key(c.sc[e]) : 0u;
        const bool eq = valid && key == T;
        int tot;
        const int r = block_excl_scan<NT>(eq ? 1 : 0, sm.tmp, &tot);
        const bool take = valid && (key > T || (eq && run + r < need_eq));
        const unsigned long long m = __ballot(take);
        if (lane == 0 && e < n) sm.bitmap[e >> 5] = (uint32_t)m;
        if (lane == 32 && e < n) sm.bitmap[e >> 5] = (uint32_t)(m >> 32);
        run += tot;
      }
    }
  }
  lds_barrier();
}

__device__ __forceinline__ void select_classified(const Geometry& g, const Workspace& ws, int p, const SelList& c,
                                  SelectSmem& sm) {
  classified_marks(g, ws, p, c, sm);
  emit_bitmap(g, c, sm);
}

// Refinement pool of one (sequence, KV head) from its ascending anchor set:
// the union of [a_k - w, a_k + w] clipped to [0, L) is the disjoint union over
// k of the runs [max(lo_k, hi_{k-1} + 1), hi_k] (all windows have one width, so
// run k adds exactly what run k-1 did not cover).  Run lengths are scanned
// into offsets (kept in LDS); then each thread fills 8 consecutive pool
// entries per round: a binary search over the offsets finds the run of the
// first one, and positions and row ids leave as 32-byte stores.  sm.apos holds
// the anchor set, sm.bt the sequence's block table.
template <typename Sm>
__device__ __forceinline__ void build_pool(const Geometry& g, const Workspace& ws, int p, int kvh,
                                           int L, Sm& sm, int slice = 0, int slices = 1) {
  const int K = g.kappa, t = threadIdx.x;
  const int win = min(g.window, L);
  int32_t* const off = reinterpret_cast<int32_t*>(sm.cbuf);  // [K] run offsets
  auto run_of = [&](int k, int* start) -> int {                // length and start of run k
    const int ai = sm.apos[k];
    *start = 0;
    if (ai < 0 || ai >= L) return 0;
    const int prev = k > 0 ? sm.apos[k - 1] : -1;
    const int lo = max(ai - win, 0), hi = min(ai + win, L - 1);
    const int prev_hi = (prev >= 0 && prev < L) ? min(prev + win, L - 1) : -1;
    *start = max(lo, prev_hi + 1);
    return max(0, hi - *start + 1);
  };
  const int per = (K + NT - 1) / NT;
  const int j0 = min(K, t * per), j1 = min(K, j0 + per);
  int lens[kPoolPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) {
    int st;
    lens[i] = j0 + i < j1 ? run_of(j0 + i, &st) : 0;
    sum += lens[i];
  }
  int total;
  int e = block_excl_scan<NT>(sum, sm.tmp, &total);
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) {
    if (j0 + i < j1) off[j0 + i] = e;
    e += lens[i];
  }
  const int n = min(total, g.n_cap);
  if (t == 0 && slice == 0) ws.pool_len[p] = n;
  lds_barrier();
  int32_t* pp = ws.pool_pos + (size_t)p * g.n_cap;
  uint32_t* pr = ws.pool_row + (size_t)p * g.n_cap;
  // this call's share of the entries: [s_lo, s_hi), ends at multiples of 8 (or n)
  const int per8 = ((n + slices - 1) / slices + 7) & ~7;
  const int s_lo = min(n, slice * per8), s_hi = min(n, s_lo + per8);
  for (int o0 = s_lo + 8 * t; o0 < s_hi; o0 += 8 * NT) {
    int lo = 0, hi = K - 1;  // the last run k with off[k] <= o0 (it is not empty)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= o0) lo = mid;
      else hi = mid - 1;
    }
    int k = lo, st;
    run_of(k, &st);
    u32x4 pv[2], rv[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = o0 + i;
      uint32_t ps = 0u, rw = 0u;
      if (o < s_hi) {
        while (k + 1 < K && off[k + 1] <= o) run_of(++k, &st);
        ps = (uint32_t)(st + (o - off[k]));
        rw = row_id_of_page(g, sm.bt[ps >> 6], kvh, (int)ps);
      }
      pv[i >> 2][i & 3] = ps;
      rv[i >> 2][i & 3] = rw;
    }
    // n_cap is a multiple of 64, so the 8 entries stay inside the problem's row
    *reinterpret_cast<u32x4*>(pp + o0) = pv[0];
    *reinterpret_cast<u32x4*>(pp + o0 + 4) = pv[1];
    *reinterpret_cast<u32x4*>(pr + o0) = rv[0];
    *reinterpret_cast<u32x4*>(pr + o0 + 4) = rv[1];
  }
}

// Loads the block table row of sequence b (its first ceil(L/64) entries,
// clamped to physical pages) into LDS.
__device__ __forceinline__ void load_bt(const Geometry& g, int b, int L, int32_t* bt) {
  constexpr int PER = kMaxPages / NT;  // every thread's loads go out before its stores
  const int np = (L + kPageSize - 1) / kPageSize;
  int v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * NT;
    v[k] = i < np ? phys_page(g, b, i) : 0;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < np) bt[i] = v[k];
  }
}

// Top-kappa of one (sequence, KV head) per workgroup (an anchor layer's pool is
// built by pool_build_kernel next).  Leaves the problem's coarse histogram at
// zero.
template <bool POOL>
__global__ __launch_bounds__(NT) void select_kernel(Geometry g, Workspace ws,
                                                    int32_t* __restrict__ out,
                                                    int32_t* __restrict__ out2, int defer) {
  __shared__ SelectSmem sm;
  const int p = blockIdx.x, b = p / g.hkv, kvh = p - b * g.hkv;
  const int L = seq_len_of(g, b);
  const int K = g.kappa;
  if (!POOL) {
    load_bt(g, b, L, sm.bt);
    lds_barrier();
  }
  SelList c;
  c.sc = ws.scores + (size_t)p * g.n_cap;
  c.plist = POOL ? ws.pool_pos + (size_t)p * g.n_cap : nullptr;
  c.prow = POOL ? ws.pool_row + (size_t)p * g.n_cap : nullptr;
  c.n = POOL ? clampi(ws.pool_len[p], 0, g.n_cap) : L;
  c.K = K;
  c.b = b;
  c.kvh = kvh;
  c.o1 = out ? out + (size_t)p * K : nullptr;
  c.o2 = out2 ? out2 + (size_t)p * K : nullptr;
  c.srow = ws.sel_row + (size_t)p * K;
  // deferred (a pool, for attn_kernel's entry mode): only the set's pool
  // indices leave this kernel; the attention's many workgroups look up the
  // positions and row ids, instead of this one workgroup gathering them
  c.ent = (POOL && defer) ? ws.sel_ent + (size_t)p * K : nullptr;
  if (c.n <= K) {
    for (int e = threadIdx.x; e < K; e += NT) {
      if (e < c.n) emit_entry(g, c, e, e, sm);
      else emit_empty(c, e, sm);
    }
  } else if (c.n <= kSmall / 2) {
    select_small<kSmallPer / 2>(g, c, sm);
  } else if (c.n <= kSmall) {
    select_small<kSmallPer>(g, c, sm);
  } else {  // after classify_kernel (with `pool` at a refined layer)
    select_classified(g, ws, p, c, sm);
  }
  reset_selection_counters(ws, p);
}

// Pool of an anchor set given in device memory: workgroup w of a problem
// writes slice w of the pool's entries (every workgroup scans the same run
// lengths).  One workgroup per problem would write the pool of a long context
// (over 100K entries at 128K tokens with w = 64) alone.
struct PoolSmem {
  int32_t bt[kMaxPages];
  int32_t apos[kMaxKappa];
  uint32_t cbuf[kMaxKappa];  // run offsets
  int tmp[NT / 64 + 1];
};

__global__ __launch_bounds__(NT) void pool_build_kernel(Geometry g, Workspace ws,
                                                        const int32_t* __restrict__ anchor,
                                                        int slices) {
  __shared__ PoolSmem sm;
  const int p = blockIdx.x / slices, w = blockIdx.x - p * slices;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int L = seq_len_of(g, b);
  const int32_t* a = anchor + (size_t)p * g.kappa;
  load_bt(g, b, L, sm.bt);
  {
    constexpr int PER = kMaxKappa / NT;
    int32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x + k * NT;
      v[k] = i < g.kappa ? a[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < g.kappa) sm.apos[i] = v[k];
    }
  }
  lds_barrier();
  build_pool(g, ws, p, kvh, L, sm, w, slices);
}

// One classification of workgroup w's list entries (raw, from base) for the
// `need` largest, into the workspace view wv: the bin holding the need-th score
// (found from the problem's coarse histogram, h: this thread's 16 bins; every
// workgroup finds the same bin and workgroup 0 records it with the counts of
// entries above it and in it), marks of the entries above that bin in wv.gbits
// and the bin's own entries, with their keys, appended to wv's candidate list.
// Contains barriers: call uniformly.
constexpr int kClsU = kClsEntries / (4 * kClsThreads);
constexpr int kClsBPT = kCoarseBins / kClsThreads;  // 16 bins per thread
__device__ void classify_into(const Geometry& g, const Workspace& wv, int p, int w, int base,
                              int n, int need, const u32x4 (&raw)[kClsU],
                              const u32x4 (&h)[kClsBPT / 4], int* tmp, int* res) {
  constexpr int U = kClsU, BPT = kClsBPT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  lds_barrier();  // readers of res from an earlier call are done
  int sum = 0;
#pragma unroll
  for (int k = 0; k < BPT / 4; ++k) sum += (int)(h[k][0] + h[k][1] + h[k][2] + h[k][3]);
  if (t == 0) {
    res[0] = -1;
    res[1] = 0;
    res[2] = 0;
  }
  int tot;
  const int above_t = block_excl_scan<kClsThreads>(sum, tmp, &tot);
  if (above_t < need && need <= above_t + sum) {
    int a = above_t, bin = -1, cnt = 0;
#pragma unroll
    for (int k = BPT / 4 - 1; k >= 0; --k) {
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const int hc = (int)h[k][q];
        if (bin < 0) {
          if (need <= a + hc) {
            bin = kCoarseBins - BPT * (t + 1) + 4 * k + q;
            cnt = hc;
          } else {
            a += hc;
          }
        }
      }
    }
    res[0] = bin;
    res[1] = a;
    res[2] = cnt;
  }
  lds_barrier();
  const int bstar = res[0];
  if (w == 0 && t == 0) {
    wv.sel_meta[4 * p] = bstar;
    wv.sel_meta[4 * p + 1] = res[1];
    wv.sel_meta[4 * p + 2] = res[2];
  }
  if (bstar < 0) {  // the histogram disagrees with the list: the selection falls back
    if (t == 0) wv.cand_cnt[(size_t)p * cls_regions(g) + w] = 0u;
    return;
  }

  uint32_t* gb = wv.gbits + (size_t)p * (g.n_cap >> 5);
  uint32_t cand = 0u;  // bit 4u + q4: entry in the threshold bin
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e0 = base + u * 4 * kClsThreads + 4 * t;
    unsigned long long mh[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int bin = (int)(order_key(__uint_as_float(raw[u][q4])) >> 20);
      const bool ok = e0 + q4 < n;
      cand |= (ok && bin == bstar) ? 1u << (4 * u + q4) : 0u;
      mh[q4] = __ballot(ok && bin > bstar);
    }
    // word k of the wave's 256 entries holds lanes 8k .. 8k+7: bit 4i + q4 is
    // bit 8k + i of mask q4
    const int first = base + u * 4 * kClsThreads + 256 * wave + 32 * lane;
    if (lane < 8 && first < n) {
      uint32_t word = 0u;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint32_t x = (uint32_t)(mh[q4] >> (8 * lane)) & 0xFFu;
        x = (x | (x << 12)) & 0x000F000Fu;
        x = (x | (x << 6)) & 0x03030303u;
        x = (x | (x << 3)) & 0x11111111u;
        word |= x << q4;
      }
      gb[first >> 5] = word;
    }
  }
  // the bin's entries go to this workgroup's own candidate region, in thread
  // order (no counter shared between workgroups); its count goes beside it
  const int cnt = __popc(cand);
  const int inc = wave_incl_scan(cnt);
  if (lane == 63) tmp[wave] = inc;
  lds_barrier();
  int before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < kClsThreads / 64; ++x) {
    const int c = tmp[x];
    before += x < wave ? c : 0;
    total += c;
  }
  const int W = cls_regions(g);
  if (t == 0) wv.cand_cnt[(size_t)p * W + w] = (uint32_t)total;
  if (cnt) {
    int slot = before + inc - cnt;
    uint32_t* ck = wv.cand_key + ((size_t)p * W + w) * kClsCap;
    int32_t* ci = wv.cand_idx + ((size_t)p * W + w) * kClsCap;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (cand & (1u << (4 * u + q4))) {
          if (slot < kClsCap) {
            ck[slot] = order_key(__uint_as_float(raw[u][q4]));
            ci[slot] = base + u * 4 * kClsThreads + 4 * t + q4;
          }
          ++slot;
        }
      }
    }
  }
}

// Lists longer than kSmall (the cache at an anchor layer, the pool at a refined
// layer with `pool`), of which the need_k largest are wanted (kappa, or the
// size of a rank-expanded pool): workgroup w of problem p takes list entries
// [w * kClsEntries, +kClsEntries) and classifies them for need_k into the
// workspace (classify_into); with need2 > need_k (an anchor list whose rank
// pool is also wanted) a second time for need2 into the second classification.
__global__ __launch_bounds__(kClsThreads) void classify_kernel(Geometry g, Workspace ws, int wgs,
                                                               int pool, int need_k, int need2) {
  __shared__ int tmp[kClsThreads / 64];
  __shared__ int res[3];
  int p, w;
  map_block(blockIdx.x, g.problems(), wgs, &p, &w);
  const int b = p / g.hkv;
  const int n = pool ? clampi(ws.pool_len[p], 0, g.n_cap) : seq_len_of(g, b);
  const int base = w * kClsEntries;
  const int need = min(need_k, n);  // entries to select: kappa, or the rank pool's size
  if (n <= kSmall || n <= need || base >= n) return;  // uniform over the workgroup
  const int t = threadIdx.x;
  const float* sc = ws.scores + (size_t)p * g.n_cap;
  u32x4 raw[kClsU];
#pragma unroll
  for (int u = 0; u < kClsU; ++u) {
    const int e0 = base + u * 4 * kClsThreads + 4 * t;
    raw[u] = *reinterpret_cast<const u32x4*>(sc + (e0 < n ? e0 : 0));
  }
  // thread t holds bins 4080 - 16t .. 4095 - 16t; scanned in thread order the
  // counts run down from the top bin
  const uint32_t* gh = ws.ghist + (size_t)p * kCoarseBins + kCoarseBins - kClsBPT * (t + 1);
  u32x4 h[kClsBPT / 4];
#pragma unroll
  for (int k = 0; k < kClsBPT / 4; ++k) h[k] = reinterpret_cast<const u32x4*>(gh)[k];
  classify_into(g, ws, p, w, base, n, need, raw, h, tmp, res);
  if (need2 > need_k && n > need2)  // uniform over the workgroup
    classify_into(g, second_class(ws), p, w, base, n, need2, raw, h, tmp, res);
}

// ---------------------------------------------------------------------------
// SparseAttn over one split of kAttnSplit selected tokens of one (sequence, KV
// head), all G query heads.  Each wave takes 16 tokens: logits by MFMA as in
// scoring (lane j + 16 i4 holds token j for heads 4 i4 .. 4 i4 + 3), softmax
// statistics over the wave's tokens inside 16-lane rows, the probabilities
// through the wave's own LDS rows into the V accumulation (two dimensions per
// lane).  One barrier combines the waves into the split's statistics (max
// logit, sum of exponentials) and unnormalised output, which go to the
// workspace; merge_kernel, launched next, merges the splits in split order.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kRowRor8, 0xf>(0u, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kRowRor4, 0xf>(0u, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kRowRor2, 0xf>(0u, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kRowRor1, 0xf>(0u, __float_as_uint(v))));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __uint_as_float(dpp<kRowRor8, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kRowRor4, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kRowRor2, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<kRowRor1, 0xf>(0u, __float_as_uint(v)));
  return v;
}

static_assert(kAttnSplit == 64 && kAttnThreads == 256, "the smallest split: one 16-token tile per wave");
constexpr int kMergeBatch = 32;  // splits whose partials one merge round loads at once
constexpr int kMaxSplits = kMaxKappa / kAttnSplit;  // splits of the smallest split size
constexpr int kDenseMinChunk = 1024;  // dense decode: tokens per workgroup (more above 128K)

// Dense decode splits a context into at most kMaxSplits chunks of whole
// 64-token multiples (16 tokens per wave step, four waves).
__host__ __device__ inline int dense_splits(const Geometry& g) {
  const int sp = (g.n_cap + kDenseMinChunk - 1) / kDenseMinChunk;
  return sp < 1 ? 1 : (sp > kMaxSplits ? kMaxSplits : sp);
}
__host__ __device__ inline int dense_chunk(const Geometry& g) {
  const int sp = dense_splits(g);
  return ((g.n_cap + sp - 1) / sp + 63) / 64 * 64;
}

template <int G>
constexpr int prob_stride() { return G < 4 ? 4 : G; }

// One wave's share of SparseAttn: 16 tokens (row ids; `valid` false masks a
// token).  Leaves the wave's softmax statistics for heads 4 g4 + r in m[r],
// l[r] (lanes 16 g4 .. 16 g4 + 15 agree) and the unnormalised output of every
// head for dimensions 2 lane, 2 lane + 1 in o0, o1.  pw: the wave's own
// [16][prob_stride<G>] rows of LDS.
// The K and V of a wave's 16 tokens: the K fragments of the lane's token
// (lane % 16) and, per token jj, the V dimensions 2 lane, 2 lane + 1.
struct KvTile {
  u32x4 kf[4];
  uint32_t vv[16];
};

__device__ __forceinline__ void load_kv_tile(const Geometry& g, uint32_t row, int lane,
                                             KvTile& t) {
  const int g4 = lane >> 4;
  const u32x4* krow = reinterpret_cast<const u32x4*>(g.k_pages + (size_t)row * kHeadDim);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) t.kf[s4] = krow[g4 + 4 * s4];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const uint32_t rj = (uint32_t)__builtin_amdgcn_readlane((int)row, jj);
    t.vv[jj] = reinterpret_cast<const uint32_t*>(g.v_pages + (size_t)rj * kHeadDim)[lane];
  }
}

template <int G>
__device__ __forceinline__ void attend_tile(const KvTile& t, const u32x4 (&qf)[4], bool valid,
                                            float scale, float* pw, float (&m)[4],
                                            float (&l)[4], float (&o0)[G], float (&o1)[G]);

template <int G>
__device__ __forceinline__ void wave_attend(const Geometry& g, const uint16_t* q, int b, int kvh,
                                            uint32_t row, bool valid, float scale, float* pw,
                                            float (&m)[4], float (&l)[4], float (&o0)[G],
                                            float (&o1)[G]) {
  const int lane = threadIdx.x & 63;
  KvTile t;
  load_kv_tile(g, row, lane, t);
  u32x4 qf[4];
  load_q_frag<G>(q, g, b, kvh, lane, qf);
  attend_tile<G>(t, qf, valid, scale, pw, m, l, o0, o1);
}

template <int G>
__device__ __forceinline__ void attend_tile(const KvTile& t, const u32x4 (&qf)[4], bool valid,
                                            float scale, float* pw, float (&m)[4],
                                            float (&l)[4], float (&o0)[G], float (&o1)[G]) {
  constexpr int GP = prob_stride<G>();
  const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
  const f32x4 acc = qk_tile(qf, t.kf);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float z = valid ? acc[r] * scale : -INFINITY;
    m[r] = row16_max(z);
    const float e = (z == -INFINITY) ? 0.f : __expf(z - m[r]);
    l[r] = row16_sum(e);
    if (4 * g4 + r < G) pw[j * GP + 4 * g4 + r] = e;
  }
  // pw rows are written and read by this wave only: LDS keeps a wave's
  // accesses in order; this keeps the compiler from reordering them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < G; ++i) o0[i] = o1[i] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float v0 = __uint_as_float(t.vv[jj] << 16);
    const float v1 = __uint_as_float(t.vv[jj] & 0xffff0000u);
#pragma unroll
    for (int i4 = 0; i4 < GP / 4; ++i4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&pw[jj * GP + 4 * i4]);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * i4 + r < G) {
          o0[4 * i4 + r] += wv[r] * v0;
          o1[4 * i4 + r] += wv[r] * v1;
        }
      }
    }
  }
}

// One 16-token tile folded into a wave's running softmax state (online
// softmax): Mrow[r], Lrow[r] the running maximum logit and sum of exponentials
// of head 4 g4 + r (the 16 lanes of row g4 agree), O0[i], O1[i] head i's
// unnormalised output for dimensions 2 lane, 2 lane + 1.  The tile's
// probabilities are taken against the updated maximum and the output is
// rescaled once per tile, so no per-tile partial is kept.
template <int G>
__device__ __forceinline__ void attend_tile_online(const KvTile& t, const u32x4 (&qf)[4],
                                                   bool valid, float scale, float* pw,
                                                   float (&Mrow)[4], float (&Lrow)[4],
                                                   float (&O0)[G], float (&O1)[G]) {
  constexpr int GP = prob_stride<G>();
  const int lane = threadIdx.x & 63, j = lane & 15, g4 = lane >> 4;
  const f32x4 acc = qk_tile(qf, t.kf);
  float fr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float z = valid ? acc[r] * scale : -INFINITY;
    const float Mn = fmaxf(Mrow[r], row16_max(z));
    fr[r] = (Mrow[r] == -INFINITY) ? 0.f : __expf(Mrow[r] - Mn);
    const float e = (z == -INFINITY) ? 0.f : __expf(z - Mn);
    Lrow[r] = Lrow[r] * fr[r] + row16_sum(e);
    Mrow[r] = Mn;
    if (4 * g4 + r < G) pw[j * GP + 4 * g4 + r] = e;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fr[i & 3]), 16 * (i >> 2)));
    O0[i] *= f;
    O1[i] *= f;
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float v0 = __uint_as_float(t.vv[jj] << 16);
    const float v1 = __uint_as_float(t.vv[jj] & 0xffff0000u);
#pragma unroll
    for (int i4 = 0; i4 < GP / 4; ++i4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&pw[jj * GP + 4 * i4]);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * i4 + r < G) {
          O0[4 * i4 + r] += wv[r] * v0;
          O1[4 * i4 + r] += wv[r] * v1;
        }
      }
    }
  }
}

// The block's split of SparseAttn from its NW waves' results (wo, wml, filled
// and synchronised by the caller), rescaled to a common maximum: the
// unnormalised output [G][128] and (max, sum) [G][2] of split s of problem p,
// stored to the workspace for merge_kernel.
template <int G, int NW, int T>
__device__ __forceinline__ void store_split(const Workspace& ws, int p, int s, int splits,
                            float (*wo)[G][kHeadDim], float (*wml)[G][2]) {
  float* po = ws.part_o + ((size_t)p * splits + s) * G * kHeadDim;
  float* pm = ws.part_ml + ((size_t)p * splits + s) * G * 2;
  for (int o = threadIdx.x; o < G * kHeadDim; o += T) {
    const int i = o / kHeadDim, d = o - i * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wml[w][i][0]);
    float a = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = wml[w][i][0];
        const float f = (mw == -INFINITY) ? 0.f : __expf(mw - M);
        a += wo[w][i][d] * f;
        L += wml[w][i][1] * f;
      }
    }
    po[o] = a;
    if (d == 0) {
      pm[2 * i] = M;
      pm[2 * i + 1] = L;
    }
  }
}

// Merge of the splits of SparseAttn, one workgroup per (problem, query head),
// one output dimension per thread: the maximum M over the splits' maxima,
// every split's weight exp(m - M), and out = sum of weighted outputs / sum of
// weighted sums, accumulated in split order (so the result does not depend on
// the order in which splits finished).  The partials come from the attention
// kernel just before it in the stream (the kernel boundary makes them
// visible; they are read back from L2, not through the device coherence
// point).  With `reset`, the problem's selection counters are cleared for the
// next anchor layer (every split has read them by now).
template <int G>
__global__ __launch_bounds__(kHeadDim) void merge_kernel(Geometry g, Workspace ws, int splits,
                                                         float* __restrict__ out, int reset) {
  __shared__ float sm_m[kMaxSplits], sm_l[kMaxSplits], sm_w[kMaxSplits];
  __shared__ float sm_sum;
  int p, i;
  map_block(blockIdx.x, g.problems(), G, &p, &i);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int d = threadIdx.x, lane = d & 63, wave = d >> 6;
  const float* pob = ws.part_o + (size_t)p * splits * G * kHeadDim + i * kHeadDim + d;
  const float* pml = ws.part_ml + (size_t)p * splits * G * 2 + i * 2;
  constexpr size_t so = (size_t)G * kHeadDim;  // split stride of the outputs
  // unconditional loads (indices clamped; surplus values get no weight) keep
  // the first batch free of branches
  float pv[kMergeBatch];
#pragma unroll
  for (int x = 0; x < kMergeBatch; ++x) pv[x] = pob[(size_t)min(x, splits - 1) * so];
  for (int x = d; x < splits; x += kHeadDim) {
    sm_m[x] = pml[(size_t)x * G * 2];
    sm_l[x] = pml[(size_t)x * G * 2 + 1];
  }
  lds_barrier();
  if (wave == 0) {
    float M = -INFINITY;
    for (int x = lane; x < splits; x += 64) M = fmaxf(M, sm_m[x]);
    M = wave_max(M);
    float l = 0.f;
    for (int x = lane; x < splits; x += 64) {
      const float mx = sm_m[x];
      const float f = (mx == -INFINITY) ? 0.f : __expf(mx - M);
      sm_w[x] = f;
      l += sm_l[x] * f;
    }
    l = wave_sum(l);
    if (lane == 0) sm_sum = l;
  }
  lds_barrier();
  float a = 0.f;
  for (int x0 = 0; x0 < splits; x0 += kMergeBatch) {
    if (x0 > 0) {
#pragma unroll
      for (int x = 0; x < kMergeBatch; ++x) pv[x] = pob[(size_t)min(x0 + x, splits - 1) * so];
    }
#pragma unroll
    for (int x = 0; x < kMergeBatch; ++x)
      if (x0 + x < splits) a += pv[x] * sm_w[x0 + x];
  }
  const float L = sm_sum;
  out[((size_t)b * g.hq + kvh * G + i) * kHeadDim + d] = L > 0.f ? a / L : 0.f;
  if (reset && i == 0) reset_selection_counters(ws, p);
}

// SparseAttn over a given set (positions in idx), over the row ids the latest
// selection left in the workspace, or over a deferred selection's pool
// indices: workgroup s of a problem takes set entries [s * kSetSplit,
// (s + 1) * kSetSplit), one 16-token tile per wave, and stores one split for
// merge_kernel.  Eight waves per workgroup: a 128-token split halves the
// partials the merge reads against 64-token splits, and the loads of each
// wave's tile are still all in flight at once (1.1% of the 4 x 128K GQA-8
// step).
constexpr int kSetPositions = 0;  // attn_kernel's set: positions in idx
constexpr int kSetRows = 1;       // row ids the latest selection left (Workspace::sel_row)
constexpr int kSetEntries = 2;    // pool indices of a deferred selection (Workspace::sel_ent)
constexpr int kSetWaves = 8;
constexpr int kSetSplit = 16 * kSetWaves;  // set entries of one workgroup
static_assert(kSetSplit >= kAttnSplit, "the workspace holds partials of kAttnSplit-token splits");

template <int G, int MODE>
__global__ __launch_bounds__(64 * kSetWaves) void attn_kernel(Geometry g, Workspace ws,
                                                              const uint16_t* __restrict__ q,
                                                              const int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ pos_out,
                                                              float scale, int splits) {
  constexpr int NW = kSetWaves;
  __shared__ float wo[NW][G][kHeadDim];
  __shared__ float wml[NW][G][2];
  __shared__ __attribute__((aligned(16))) float pw[NW][16 * prob_stride<G>()];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (blockIdx.x >= (unsigned)(g.problems() * splits)) {  // uniform over the workgroup
    // one workgroup per problem past the attention's grid (a shared layer's
    // launch): the step's new keys get their codes, as no kernel of the layer
    // scores them
    const int pq = blockIdx.x - g.problems() * splits;
    const int bq = pq / g.hkv, L = seq_len_of(g, bq);
    quantize_positions(g, bq, pq - bq * g.hkv, max(L - g.new_keys, 0), L, lane, wave, NW);
    return;
  }
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int j = lane & 15;
  const uint32_t max_row = (uint32_t)g.num_pages * (uint32_t)(g.hkv * kPageSize) - 1u;
  const int L = seq_len_of(g, b);
  const int first = s * kSetSplit + wave * 16;  // this wave's first set entry
  const int ti = first + j;
  uint32_t row;
  bool valid;
  if (MODE == kSetRows) {
    const uint32_t r = ti < g.kappa ? ws.sel_row[(size_t)p * g.kappa + ti] : kNoRow;
    valid = r <= max_row;
    row = valid ? r : 0u;
  } else if (MODE == kSetEntries) {
    // pool index -> row id and position; the set's positions go to pos_out
    const int n = clampi(ws.pool_len[p], 0, g.n_cap);
    const int e = ti < g.kappa ? ws.sel_ent[(size_t)p * g.kappa + ti] : -1;
    const bool ok = e >= 0 && e < n;
    const size_t pe = (size_t)p * g.n_cap + (ok ? e : 0);
    const uint32_t r = ws.pool_row[pe];
    valid = ok && r <= max_row;
    row = valid ? r : 0u;
    if (pos_out && lane < 16 && ti < g.kappa)
      pos_out[(size_t)p * g.kappa + ti] = valid ? ws.pool_pos[pe] : -1;
  } else {
    const int pos = ti < g.kappa ? idx[(size_t)p * g.kappa + ti] : -1;
    valid = pos >= 0 && pos < L;
    row = row_id(g, b, kvh, valid ? pos : 0);
  }
  float Mr[G], Lr[G], O0[G], O1[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    Mr[i] = -INFINITY;
    Lr[i] = 0.f;
    O0[i] = O1[i] = 0.f;
  }
  if (first < g.kappa) {  // uniform over the wave
    u32x4 qf[4];
    load_q_frag<G>(q, g, b, kvh, lane, qf);
    KvTile kt;
    load_kv_tile(g, row, lane, kt);
    float m[4], l[4];
    attend_tile<G>(kt, qf, valid, scale, pw[wave], m, l, O0, O1);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      Mr[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m[i & 3]), 16 * (i >> 2)));
      Lr[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l[i & 3]), 16 * (i >> 2)));
    }
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    wo[wave][i][2 * lane] = O0[i];
    wo[wave][i][2 * lane + 1] = O1[i];
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      wml[wave][i][0] = Mr[i];
      wml[wave][i][1] = Lr[i];
    }
  }
  lds_barrier();
  store_split<G, NW, 64 * kSetWaves>(ws, p, s, splits, wo, wml);
}

// Dense decode attention (every cached token; the FlashAttention-style
// baseline of the paper's Tables 6-8): workgroup s of problem p takes tokens
// [s * chunk, (s + 1) * chunk), each wave a quarter of them in 16-token
// steps with the next step's K and V in flight; a wave keeps running softmax
// statistics per head (the step's maximum and sum from the same code as
// SparseAttn, rescaled to the running maximum) and its unnormalised output,
// and the workgroup stores one split for merge_kernel.  ws carries the dense
// partials (dense_o, dense_ml) in place of the sparse ones.
template <int G>
__global__ __launch_bounds__(kAttnThreads) void dense_attn_kernel(Geometry g, Workspace ws,
                                                                  const uint16_t* __restrict__ q,
                                                                  int splits, int chunk,
                                                                  float scale) {
  constexpr int NW = kAttnThreads / 64;
  __shared__ float wo[NW][G][kHeadDim];
  __shared__ float wml[NW][G][2];
  __shared__ __attribute__((aligned(16))) float pw[NW][16 * prob_stride<G>()];
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15;
  const int L = seq_len_of(g, b);
  const int per_wave = chunk / NW;  // a multiple of 16
  const int start = s * chunk + wave * per_wave;
  const int steps = clampi((min(L, start + per_wave) - start + 15) / 16, 0, per_wave / 16);
  float Mr[G], Lr[G], O0[G], O1[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    Mr[i] = -INFINITY;
    Lr[i] = 0.f;
    O0[i] = O1[i] = 0.f;
  }
  if (steps > 0) {  // uniform over the wave
    u32x4 qf[4];
    load_q_frag<G>(q, g, b, kvh, lane, qf);
    auto row_of = [&](int k) {
      const int pos = min(start + 16 * k + j, L - 1);
      return row_id(g, b, kvh, pos);
    };
    auto step = [&](const KvTile& t, int k) {
      float m[4], l[4], o0[G], o1[G];
      attend_tile<G>(t, qf, start + 16 * k + j < L, scale, pw[wave], m, l, o0, o1);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m[i & 3]), 16 * (i >> 2)));
        const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l[i & 3]), 16 * (i >> 2)));
        const float Mn = fmaxf(Mr[i], mh);
        const float fa = (Mr[i] == -INFINITY) ? 0.f : __expf(Mr[i] - Mn);
        const float fb = (mh == -INFINITY) ? 0.f : __expf(mh - Mn);
        Lr[i] = Lr[i] * fa + lh * fb;
        O0[i] = O0[i] * fa + o0[i] * fb;
        O1[i] = O1[i] * fa + o1[i] * fb;
        Mr[i] = Mn;
      }
    };
    KvTile t0, t1;
    load_kv_tile(g, row_of(0), lane, t0);
    for (int k = 0; k < steps; k += 2) {
      if (k + 1 < steps) load_kv_tile(g, row_of(k + 1), lane, t1);
      __builtin_amdgcn_sched_barrier(0);
      step(t0, k);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < steps) {
        if (k + 2 < steps) load_kv_tile(g, row_of(k + 2), lane, t0);
        __builtin_amdgcn_sched_barrier(0);
        step(t1, k + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    wo[wave][i][2 * lane] = O0[i];
    wo[wave][i][2 * lane + 1] = O1[i];
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      wml[wave][i][0] = Mr[i];
      wml[wave][i][1] = Lr[i];
    }
  }
  lds_barrier();
  store_split<G, NW, kAttnThreads>(ws, p, s, splits, wo, wml);
}

// Refined layer of a decode step: the selection and SparseAttn in one kernel.
// Workgroup s of problem p selects the pool's top-kappa itself (every split's
// workgroup reaches the same set: same keys, same order) and attends its ranks
// [s * SP, (s + 1) * SP) of the ascending set, 16 per wave (SP = 64 when the
// grid of 64-token splits still fits the device at once, else 128);
// layer_idx, if given, receives those ranks' positions.  Pools of at most
// kSmall entries are selected in registers; up to kRegMarks entries also from
// registers (32 keys per thread) into marks in an LDS bitmap; longer ones by
// the sampled bracket and one pass over the pool (marks in the bitmap), both
// in an out-of-line function.  The REG32 instantiation (caches of at most
// kRegMarks tokens) selects pools above kSmall / 2 entries from 32 keys per
// thread inline and has no out-of-line path.
template <int G, int SP>
struct FusedSmem {
  uint32_t hist[4096 + 1024 + 1024];
  uint32_t pair[kPairMax];
  uint32_t ured[32];
  int tmp[NT / 64 + 1];
  int res[9];
  int cnt[2];
  uint32_t bitmap[kMaxSeqLen / 32];  // pools longer than kSmall: selection marks
  uint32_t cbuf[2 * kCand];
  uint32_t srow[SP];
  float wo[SP / 16][G][kHeadDim];
  float wml[SP / 16][G][2];
  float pw[SP / 16][16 * prob_stride<G>()] __attribute__((aligned(16)));
};

// The selection step of refine_attn_kernel: every thread holds R consecutive
// pool entries (R n_threads >= n); the block finds the pool's top-kappa and
// keeps the row ids of ranks [r0, r0 + span) in sm.srow (and writes their
// positions to layer_idx).  Returns the size of the selected set.
template <int R, typename Sm>
__device__ int fused_select_slice(const Geometry& g, const Workspace& ws, int p, int n, int r0,
                                  int span, int32_t* layer_idx, Sm& sm) {
  const int t = threadIdx.x, K = g.kappa;
  const int e0 = R * t;
  const int nv = clampi(n - e0, 0, R);
  const int ea = e0 < n ? e0 : 0;
  const size_t base = (size_t)p * g.n_cap;
  uint32_t key[R], pr[R], pl[R];
  load_run<R>(ws.scores + base, ea, key);
  load_run<R>(ws.pool_row + base, ea, pr);
  if (layer_idx) load_run<R>(ws.pool_pos + base, ea, pl);
#pragma unroll
  for (int i = 0; i < R; ++i) key[i] = order_key(__uint_as_float(key[i]));
  const uint32_t take = top_k_mask<R>(key, nv, n, K, sm);
  int total;
  int o = block_excl_scan<NT>(__popc(take), sm.tmp, &total);
  const int rend = min(K, r0 + span);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (take & (1u << i)) {
      if (o >= r0 && o < rend) {
        sm.srow[o - r0] = pr[i];
        if (layer_idx) layer_idx[(size_t)p * K + o] = (int32_t)pl[i];
      }
      ++o;
    }
  }
  if (layer_idx)
    for (int o2 = max(total, r0) + t; o2 < rend; o2 += NT) layer_idx[(size_t)p * K + o2] = -1;
  lds_barrier();
  return total;
}

// Ranks [r0, r0 + span) of the entries marked in sm.bitmap (marks in list
// order, so ranks are ascending positions): their row ids go to sm.srow and
// their positions to layer_idx.  Returns the number of marked entries.
template <typename Sm>
__device__ __forceinline__ int slice_from_marks(const SelList& c, int p, int r0, int span,
                                                int32_t* layer_idx, Sm& sm) {
  const int t = threadIdx.x, K = c.K;
  const int words = (c.n + 31) >> 5;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = min(words, t * wpt), w1 = min(words, w0 + wpt);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(sm.bitmap[i]);
  int total;
  int o = block_excl_scan<NT>(cnt, sm.tmp, &total);
  const int rend = min(K, r0 + span);
  if (o < rend && o + cnt > r0) {
    for (int i = w0; i < w1 && o < rend; ++i) {
      uint32_t m = sm.bitmap[i];
      while (m && o < rend) {
        const int e = i * 32 + (__ffs(m) - 1);
        m &= m - 1u;
        if (o >= r0) {
          sm.srow[o - r0] = c.prow[e];
          if (layer_idx) layer_idx[(size_t)p * K + o] = c.plist[e];
        }
        ++o;
      }
    }
  }
  if (layer_idx)
    for (int o2 = max(total, r0) + t; o2 < rend; o2 += NT) layer_idx[(size_t)p * K + o2] = -1;
  lds_barrier();
  return total;
}

// The selection step of refine_attn_kernel for pools longer than kSmall, kept
// out of line (plain pointer and integer arguments) so that the common path
// stays small: up to kRegMarks entries from 32 keys per thread (each thread's
// mask is one bitmap word), longer pools by the sampled bracket and one pass.
// Returns the size of the selected set; sm.srow receives the split's rows.
template <typename Sm>
__device__ __attribute__((noinline)) int long_pool_slice(const float* sc, const int32_t* plist,
                                                        const uint32_t* prow, int n, int n_cap,
                                                        int K, int p, int r0, int span,
                                                        int32_t* layer_idx, Sm* smp) {
  Sm& sm = *smp;
  const int t = threadIdx.x;
  SelList c;
  c.sc = sc;
  c.plist = plist;
  c.prow = prow;
  c.n = n;
  c.K = K;
  c.b = 0;
  c.kvh = 0;
  c.o1 = c.o2 = nullptr;
  c.srow = nullptr;
  c.ent = nullptr;
  if (n <= kRegMarks) {
    constexpr int R = kRegMarks / NT;
    static_assert(R == 32, "one bitmap word per thread");
    const int e0 = R * t;
    uint32_t key[R];
    load_run<R>(sc, min(e0, n_cap - R), key);  // n_cap is a multiple of 64
#pragma unroll
    for (int i = 0; i < R; ++i) key[i] = order_key(__uint_as_float(key[i]));
    const uint32_t take = top_k_mask<R>(key, clampi(n - e0, 0, R), n, K, sm);
    if (e0 < n) sm.bitmap[t] = take;
    lds_barrier();
  } else {
    select_large_marks(c, sm);
  }
  return slice_from_marks(c, p, r0, span, layer_idx, sm);
}

template <int G, int SP, bool REG32 = false>
__global__ __launch_bounds__(NT) void refine_attn_kernel(Geometry g, Workspace ws,
                                                         const uint16_t* __restrict__ q,
                                                         float scale,
                                                         int32_t* __restrict__ layer_idx) {
  constexpr int NW = SP / 16;  // waves that attend, 16 tokens each
  static_assert(NW >= 1 && NW <= NT / 64, "attending waves fit the workgroup");
  __shared__ FusedSmem<G, SP> sm;
  const int K = g.kappa;
  const int splits = (K + SP - 1) / SP;
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  const int n = clampi(ws.pool_len[p], 0, g.n_cap);
  const int r0 = s * SP;  // first rank of this split
  const int myr = r0 + wave * 16 + j;
  uint32_t row = 0u;
  bool valid = false;
  if (REG32 && n <= kSmall / 2) {  // uniform over the workgroup
    const int total = fused_select_slice<kSmallPer / 2>(g, ws, p, n, r0, SP, layer_idx, sm);
    valid = myr < min(total, K);
    row = valid && wave < NW ? sm.srow[wave * 16 + j] : 0u;
  } else if constexpr (REG32) {
    // caches of at most kRegMarks tokens (the launch's choice): pools above
    // kSmall / 2 entries are selected from 32 keys per thread, inline, with no
    // call frame; the split's rows and positions are read from the pool by
    // rank
    const size_t base = (size_t)p * g.n_cap;
    constexpr int R = kRegMarks / NT;
    const int e0 = R * t, m = min(n, kRegMarks);
    uint32_t key[R];
    load_run<R>(ws.scores + base, min(e0, g.n_cap - R), key);  // n_cap is a multiple of 64
#pragma unroll
    for (int i = 0; i < R; ++i) key[i] = order_key(__uint_as_float(key[i]));
    const uint32_t take = top_k_mask<R>(key, clampi(m - e0, 0, R), m, K, sm);
    if (e0 < m) sm.bitmap[t] = take;
    lds_barrier();
    SelList c;
    c.sc = ws.scores + base;
    c.plist = ws.pool_pos + base;
    c.prow = ws.pool_row + base;
    c.n = m;
    c.K = K;
    c.b = b;
    c.kvh = kvh;
    c.o1 = c.o2 = nullptr;
    c.srow = nullptr;
    c.ent = nullptr;
    const int total = slice_from_marks(c, p, r0, SP, layer_idx, sm);
    valid = myr < min(total, K);
    row = valid && wave < NW ? sm.srow[wave * 16 + j] : 0u;
  } else if (n <= kSmall) {  // uniform over the workgroup
    int total;
    if (n <= kSmall / 2)
      total = fused_select_slice<kSmallPer / 2>(g, ws, p, n, r0, SP, layer_idx, sm);
    else
      total = fused_select_slice<kSmallPer>(g, ws, p, n, r0, SP, layer_idx, sm);
    valid = myr < min(total, K);
    row = valid && wave < NW ? sm.srow[wave * 16 + j] : 0u;
  } else {
    const size_t base = (size_t)p * g.n_cap;
    const int total = long_pool_slice(ws.scores + base, ws.pool_pos + base, ws.pool_row + base, n,
                                      g.n_cap, K, p, r0, SP, layer_idx, &sm);
    valid = myr < min(total, K);
    row = valid && wave < NW ? sm.srow[wave * 16 + j] : 0u;
  }
  const uint32_t max_row = (uint32_t)g.num_pages * (uint32_t)(g.hkv * kPageSize) - 1u;
  valid = valid && row <= max_row;
  if (!valid) row = 0u;

  if (wave < NW) {  // uniform over the wave
    float m[4], l[4], o0[G], o1[G];
    wave_attend<G>(g, q, b, kvh, row, valid, scale, sm.pw[wave], m, l, o0, o1);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      sm.wo[wave][i][2 * lane] = o0[i];
      sm.wo[wave][i][2 * lane + 1] = o1[i];
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g4 + r < G) {
          sm.wml[wave][4 * g4 + r][0] = m[r];
          sm.wml[wave][4 * g4 + r][1] = l[r];
        }
      }
    }
  }
  lds_barrier();
  store_split<G, NW, NT>(ws, p, s, splits, sm.wo, sm.wml);
}

// The attention phase shared by the multi-tile kernels: wave w attends tiles
// w, w + 16, w + 32, ... of the workgroup's `lim` ranks (row ids in srow),
// then the waves' results are combined and stored as split s.  Contains
// barriers; after the first one the helper overwrites the LDS behind wo / wml,
// so the caller must no longer need it.
template <int G, typename Sm>
__device__ __forceinline__ void multi_attend_store(const Geometry& g, const Workspace& ws,
                                                   const uint16_t* q, float scale, int p, int s,
                                                   int splits, int lim, int tiles, Sm& sm) {
  constexpr int NW = NT / 64;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15;
  const uint32_t max_row = (uint32_t)g.num_pages * (uint32_t)(g.hkv * kPageSize) - 1u;
  const int steps = clampi((lim - 16 * wave + 16 * NW - 1) / (16 * NW), 0, tiles);
  float Mrow[4], Lrow[4], O0[G], O1[G];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    Mrow[r] = -INFINITY;
    Lrow[r] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < G; ++i) O0[i] = O1[i] = 0.f;
  if (steps > 0) {  // uniform over the wave
    u32x4 qf[4];
    load_q_frag<G>(q, g, b, kvh, lane, qf);
    for (int k = 0; k < steps; ++k) {
      const int r = 16 * (k * NW + wave) + j;
      const uint32_t row = r < lim ? sm.srow[r] : 0u;
      const bool valid = r < lim && row <= max_row;
      KvTile t0;
      load_kv_tile(g, valid ? row : 0u, lane, t0);
      attend_tile_online<G>(t0, qf, valid, scale, sm.pw[wave], Mrow, Lrow, O0, O1);
    }
  }
  lds_barrier();  // every wave is past its last read of the selection's LDS
#pragma unroll
  for (int i = 0; i < G; ++i) {
    sm.wo[wave][i][2 * lane] = O0[i];
    sm.wo[wave][i][2 * lane + 1] = O1[i];
  }
  if (j == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * (lane >> 4) + r < G) {
        sm.wml[wave][4 * (lane >> 4) + r][0] = Mrow[r];
        sm.wml[wave][4 * (lane >> 4) + r][1] = Lrow[r];
      }
    }
  }
  lds_barrier();
  store_split<G, NW, NT>(ws, p, s, splits, sm.wo, sm.wml);
}

// Refined layer of grids that the fused kernel's one workgroup per 64 or 128
// selected tokens would not fit at once (many (sequence, KV head) problems,
// or a large kappa), for pools of at most kSmall entries: `splits` workgroups
// per problem, each selecting the pool's top-kappa from keys in registers as
// refine_attn_kernel does (every split reaches the same set), then attending
// its 256 * tiles consecutive ranks of the set with all sixteen waves, each
// wave a strided run of 16-token tiles, one tile's K and V in flight at a time
// (sixteen waves per compute unit keep enough loads outstanding; a second
// buffer would not fit 128 registers at G = 8), each folded into running
// softmax statistics per head (attend_tile_online).  The waves' results are
// combined in the workgroup and stored as one split for merge_kernel.  The
// selection's LDS is reused for the waves' results once the set's rows are in
// sm.srow.
constexpr int kMultiMaxTiles = 8;                 // 16-token tiles per wave at most
constexpr int kMultiMaxSpan = 16 * NT / 64 * kMultiMaxTiles;  // ranks per workgroup at most

template <int G>
struct MultiSmem {
  union {
    struct {
      uint32_t hist[4096 + 1024 + 1024];
      uint32_t pair[kPairMax];
      uint32_t ured[32];
      int tmp[NT / 64 + 1];
      int res[9];
      int cnt[2];
    };
    struct {
      float wo[NT / 64][G][kHeadDim];
      float wml[NT / 64][G][2];
    };
  };
  uint32_t srow[kMultiMaxSpan];
  float pw[NT / 64][16 * prob_stride<G>()] __attribute__((aligned(16)));
};

template <int G>
__global__ __launch_bounds__(NT) void refine_attn_multi_kernel(Geometry g, Workspace ws,
                                                               const uint16_t* __restrict__ q,
                                                               float scale,
                                                               int32_t* __restrict__ layer_idx,
                                                               int tiles) {
  constexpr int NW = NT / 64;
  __shared__ MultiSmem<G> sm;
  const int K = g.kappa;
  tiles = clampi(tiles, 1, kMultiMaxTiles);
  const int span = 16 * NW * tiles;  // ranks of one workgroup
  const int splits = (K + span - 1) / span;
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  // the launch takes this kernel only for pools of at most kSmall entries;
  // a longer length in the workspace is clamped (a wrong set, never an access
  // beyond the pool)
  const int n = min(clampi(ws.pool_len[p], 0, g.n_cap), kSmall);
  const int r0 = s * span;
  int total;
  if (n <= kSmall / 2)
    total = fused_select_slice<kSmallPer / 2>(g, ws, p, n, r0, span, layer_idx, sm);
  else
    total = fused_select_slice<kSmallPer>(g, ws, p, n, r0, span, layer_idx, sm);
  // ranks of this split that hold a token
  multi_attend_store<G>(g, ws, q, scale, p, s, splits, min(min(total, K) - r0, span), tiles, sm);
}

// ---------------------------------------------------------------------------
// Anchor layer of a decode step: the selection, the refinement pool and
// SparseAttn in one kernel (after scoring and, for contexts longer than
// kSmall, classification).  Every split's workgroup rebuilds the selection as
// a bitmap over the cache (same inputs, same set), takes the marked entries'
// ranks, predecessors and run offsets from block scans, writes its rank slice
// of the anchor set and of the window pool, and attends that slice (16 tokens
// per wave); merge_kernel, launched next, merges the splits.  The rank-pool
// instantiation (RANK) writes no window pool: one extra workgroup per problem
// writes the rank-expanded pool instead (anchor_rank_emit).
// ---------------------------------------------------------------------------

// The pool in position order from the marks in sm.bitmap over a list of L
// entries: positions and row ids to the workspace and its length; with kStage
// also the positions in rank order to sm.apos when the pool has at most
// kMaxKappa entries (returns whether they went there).  Long lists emit by
// rank: every word's first rank in sm.hist, then thread t places ranks
// [R t, R t + R), a binary search finding the word of its first rank and a walk
// forward through the marks, so every thread does the same small amount of
// work whatever the clustering of the marks (a thread owning full mark words
// would otherwise emit 128 entries while most emit none).  Contains barriers.
template <bool kStage, typename Sm>
__device__ __forceinline__ bool emit_pool(const Geometry& g, const Workspace& ws, int p, int kvh, int L, Sm& sm,
                          int* pool_n_out) {
  const int t = threadIdx.x;
  const size_t base = (size_t)p * g.n_cap;
  const int words = (L + 31) >> 5;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = min(words, t * wpt), w1 = min(words, w0 + wpt);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(sm.bitmap[i]);
  int pool_n;
  int o = block_excl_scan<NT>(cnt, sm.tmp, &pool_n);
  int32_t* pp = ws.pool_pos + base;
  uint32_t* pr = ws.pool_row + base;
  constexpr int kListWords = 4096 + 1024 + 1024;  // sm.hist, free until the caller's next phase
  const bool staged = kStage && pool_n <= kMaxKappa;  // uniform over the workgroup
  const bool balanced = pool_n <= kMaxKappa && words > 2 * NT && words <= kListWords;
  if (balanced) {
    uint32_t* const wb = sm.hist;
    for (int i = w0; i < w1; ++i) {
      wb[i] = (uint32_t)o;
      o += __popc(sm.bitmap[i]);
    }
    lds_barrier();
    constexpr int R = kMaxKappa / NT;
    const int r0 = R * t;
    if (r0 < pool_n) {
      int lo = 0, hi = words;  // first word whose base exceeds r0, minus one
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)wb[mid] <= r0) lo = mid + 1;
        else hi = mid;
      }
      int wi = lo - 1;
      uint32_t mk = sm.bitmap[wi];
      for (int k = r0 - (int)wb[wi]; k > 0; --k) mk &= mk - 1u;
      for (int i = 0; i < R && r0 + i < pool_n; ++i) {
        while (mk == 0u) mk = sm.bitmap[++wi];
        const int a = wi * 32 + (__ffs(mk) - 1);
        mk &= mk - 1u;
        if constexpr (kStage) sm.apos[r0 + i] = a;
        pp[r0 + i] = a;
        pr[r0 + i] = row_id_of_page(g, sm.bt[a >> 6], kvh, a);
      }
    }
  } else {  // a few words per thread: each thread emits its own words' marks
    for (int i = w0; i < w1; ++i) {
      uint32_t mk = sm.bitmap[i];
      while (mk) {
        const int e = i * 32 + (__ffs(mk) - 1);
        mk &= mk - 1u;
        if (o < g.n_cap) {
          pp[o] = e;
          pr[o] = row_id_of_page(g, sm.bt[e >> 6], kvh, e);
          if constexpr (kStage) {
            if (staged) sm.apos[o] = e;
          }
        }
        ++o;
      }
    }
  }
  if (t == 0) ws.pool_len[p] = min(pool_n, g.n_cap);
  if (staged || balanced) lds_barrier();  // sm.apos complete; sm.hist free again
  *pool_n_out = pool_n;
  return staged;
}

template <int G>
struct AnchorSmem {
  int32_t bt[kMaxPages];
  uint32_t bitmap[kMaxSeqLen / 32];
  uint32_t cbuf[2 * kCand];
  uint32_t hist[4096 + 1024 + 1024];
  uint32_t pair[kPairMax];
  uint32_t ured[32];
  int tmp[NT / 64 + 1];
  int res[9];
  int cnt[2];
  uint32_t srow[kFusedSplit];
  int32_t spos[kFusedSplit];  // the split's anchors: positions and pool-run starts
  int32_t sst[kFusedSplit];
  float wo[kFusedSplit / 16][G][kHeadDim];
  float wml[kFusedSplit / 16][G][2];
  float pw[kFusedSplit / 16][16 * prob_stride<G>()] __attribute__((aligned(16)));
};

// Marks of a list of at most kSmall entries from the keys in registers.
template <int R, typename Sm>
__device__ __forceinline__ void small_marks(const float* sc, int n, int K, Sm& sm) {
  const int t = threadIdx.x;
  const int words = (n + 31) >> 5;
  for (int i = t; i < words; i += NT) sm.bitmap[i] = 0u;
  const int e0 = R * t;
  const int nv = clampi(n - e0, 0, R);
  uint32_t key[R];
  load_run<R>(sc, e0 < n ? e0 : 0, key);
#pragma unroll
  for (int i = 0; i < R; ++i) key[i] = order_key(__uint_as_float(key[i]));
  const uint32_t take = top_k_mask<R>(key, nv, n, K, sm);  // its barriers order the zeroing
  if (take) atomicOr(&sm.bitmap[e0 >> 5], take << (e0 & 31));
  lds_barrier();
}

// Rank-expanded pool (Eq. 4) beside the fused anchor kernel's attention: one
// extra workgroup per problem marks the cache's top rho*kappa (from the second
// classification) and writes the pool in position order (only in the kernel's
// rank-pool instantiation, so the window-pool one is left as it is).
template <bool REG32 = false, typename Sm>
__device__ __forceinline__ void anchor_rank_emit(const Geometry& g, const Workspace& ws, int pe,
                                                 Sm& sm) {
  const int be = pe / g.hkv, kvhe = pe - be * g.hkv;
  const int ne = seq_len_of(g, be);
  const int m = min(g.pool_rho * g.kappa, ne);
  load_bt(g, be, ne, sm.bt);
  const float* sce = ws.scores + (size_t)pe * g.n_cap;
  if (m >= ne) {
    for (int i = threadIdx.x; i < ((ne + 31) >> 5); i += NT)
      sm.bitmap[i] = (32 * i + 32 <= ne) ? 0xFFFFFFFFu : ((1u << (ne & 31)) - 1u);
    lds_barrier();
  } else if (ne <= kSmall / 2) {
    small_marks<kSmallPer / 2>(sce, ne, m, sm);
  } else if (ne <= kSmall) {
    small_marks<kSmallPer>(sce, ne, m, sm);
  } else if (REG32) {  // caches of at most kRegMarks tokens: no classification
    small_marks<kRegMarks / NT>(sce, ne, m, sm);
  } else {
    SelList c;
    c.sc = sce;
    c.plist = nullptr;
    c.prow = nullptr;
    c.n = ne;
    c.K = m;
    c.b = be;
    c.kvh = kvhe;
    c.o1 = c.o2 = nullptr;
    c.srow = nullptr;
    c.ent = nullptr;
    classified_marks(g, second_class(ws), pe, c, sm);
  }
  int pool_n;
  emit_pool<false>(g, ws, pe, kvhe, ne, sm, &pool_n);
}

template <int G, bool RANK, bool REG32 = false>
__global__ __launch_bounds__(NT) void anchor_attn_kernel(Geometry g, Workspace ws,
                                                         const uint16_t* __restrict__ q,
                                                         float scale,
                                                         int32_t* __restrict__ anchor_idx,
                                                         int32_t* __restrict__ layer_idx) {
  constexpr int NW = kFusedSplit / 16;
  static_assert(NW < NT / 64, "waves left over to write the pool during the attention");
  __shared__ AnchorSmem<G> sm;
  const int K = g.kappa;
  const int splits = (K + kFusedSplit - 1) / kFusedSplit;
  if constexpr (RANK) {
    if ((int)blockIdx.x >= g.problems() * splits) {  // uniform over the workgroup
      anchor_rank_emit<REG32>(g, ws, (int)blockIdx.x - g.problems() * splits, sm);
      return;
    }
  }
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  const int n = seq_len_of(g, b);
  const int r0 = s * kFusedSplit;
  load_bt(g, b, n, sm.bt);

  // the selection as marks over the list
  if (n <= K) {
    for (int i = t; i < ((n + 31) >> 5); i += NT)
      sm.bitmap[i] = (32 * i + 32 <= n) ? 0xFFFFFFFFu : ((1u << (n & 31)) - 1u);
    lds_barrier();
  } else if (n <= kSmall / 2) {
    small_marks<kSmallPer / 2>(ws.scores + (size_t)p * g.n_cap, n, K, sm);
  } else if (n <= kSmall) {
    small_marks<kSmallPer>(ws.scores + (size_t)p * g.n_cap, n, K, sm);
  } else if (REG32) {  // caches of at most kRegMarks tokens: no classification
    small_marks<kRegMarks / NT>(ws.scores + (size_t)p * g.n_cap, n, K, sm);
  } else {
    SelList c;
    c.sc = ws.scores + (size_t)p * g.n_cap;
    c.plist = nullptr;
    c.prow = nullptr;
    c.n = n;
    c.K = K;
    c.b = b;
    c.kvh = kvh;
    c.o1 = c.o2 = nullptr;
    c.srow = nullptr;
    c.ent = nullptr;
    classified_marks(g, ws, p, c, sm);
  }

  // --- the anchor set from the marks ----------------------------------------
  // 1. the nonzero words in order, each with the rank of its first mark, as a
  //    list in sm.hist (word index << 14 | rank, ranks clamped to 16383)
  const int words = (n + 31) >> 5;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = min(words, t * wpt), w1 = min(words, w0 + wpt);
  int cnt = 0, nz = 0;
  for (int i = w0; i < w1; ++i) {
    const uint32_t m = sm.bitmap[i];
    cnt += __popc(m);
    nz += m ? 1 : 0;
  }
  int total, nz_total;
  int rank = block_excl_scan<NT>(cnt, sm.tmp, &total);
  int slot = block_excl_scan<NT>(nz, sm.tmp, &nz_total);
  uint32_t* const wl = sm.hist;
  for (int i = w0; i < w1; ++i) {
    const uint32_t m = sm.bitmap[i];
    if (m) {
      wl[slot++] = ((uint32_t)i << 14) | (uint32_t)min(rank, 16383);
      rank += __popc(m);
    }
  }
  lds_barrier();
  // 2. one lane per bit of two listed words at a time: the mark's rank,
  //    position and predecessor give its pool run; run lengths go to lens[rank]
  //    and the slice's anchors (position, run start) to spos / sst
  const int kt = min(total, K);  // anchors
  const int rend = min(K, r0 + kFusedSplit);
  int32_t* const lens = reinterpret_cast<int32_t*>(sm.cbuf);  // [K]: run lengths, then offsets
  const int win = RANK ? 0 : min(g.window, n);  // rank pool: written by the extra workgroups
  for (int x = 2 * wave; x < nz_total; x += 2 * (NT / 64)) {
    const int idx = x + (lane >> 5), bit = lane & 31;
    if (idx < nz_total) {
      const uint32_t e = wl[idx];
      const int wi = (int)(e >> 14), base = (int)(e & 16383u);
      const uint32_t m = sm.bitmap[wi];
      if ((m >> bit) & 1u) {
        const uint32_t below = m & ((1u << bit) - 1u);
        const int r = base + __popc(below);
        int pv = -1;
        if (below) {
          pv = wi * 32 + 31 - __clz(below);
        } else if (idx > 0) {
          const int wp = (int)(wl[idx - 1] >> 14);
          pv = wp * 32 + 31 - __clz(sm.bitmap[wp]);
        }
        const int a = wi * 32 + bit;
        const int lo = max(a - win, 0), hi = min(a + win, n - 1);
        const int phi = pv >= 0 ? min(pv + win, n - 1) : -1;
        const int st = max(lo, phi + 1);
        if (r < kt) lens[r] = max(0, hi - st + 1);
        if (r >= r0 && r < rend) {
          sm.spos[r - r0] = a;
          sm.sst[r - r0] = st;
        }
      }
    }
  }
  lds_barrier();
  // 3. run offsets in rank order
  const int per = (K + NT - 1) / NT;
  const int k0 = min(kt, t * per), k1 = min(kt, k0 + per);
  int sum = 0;
  for (int k = k0; k < k1; ++k) sum += lens[k];
  int pool_n;
  int off = block_excl_scan<NT>(sum, sm.tmp, &pool_n);
  for (int k = k0; k < k1; ++k) {
    const int l = lens[k];
    lens[k] = off;
    off += l;
  }
  lds_barrier();
  // 4. this split's ranks: row ids for the attention below, the anchor set
  for (int k = t; k < rend - r0; k += NT) {
    const int r = r0 + k;
    int a = -1;
    if (r < kt) {
      a = sm.spos[k];
      sm.srow[k] = row_id_of_page(g, sm.bt[a >> 6], kvh, a);
    }
    if (anchor_idx) anchor_idx[(size_t)p * K + r] = a;
    if (layer_idx) layer_idx[(size_t)p * K + r] = a;
  }
  lds_barrier();  // srow, lens and sst are complete

  const int myr = r0 + wave * 16 + j;
  bool valid = wave < NW && myr < min(total, K);
  uint32_t row = valid ? sm.srow[wave * 16 + j] : 0u;
  if (wave < NW) {  // uniform over the wave
    float m[4], l[4], o0v[G], o1v[G];
    wave_attend<G>(g, q, b, kvh, row, valid, scale, sm.pw[wave], m, l, o0v, o1v);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      sm.wo[wave][i][2 * lane] = o0v[i];
      sm.wo[wave][i][2 * lane + 1] = o1v[i];
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g4 + r < G) {
          sm.wml[wave][4 * g4 + r][0] = m[r];
          sm.wml[wave][4 * g4 + r][1] = l[r];
        }
      }
    }
  } else if (!RANK) {
    // 5. meanwhile the other waves write this split's part of the pool: 8
    //    consecutive entries per thread, the run of the first found by binary
    //    search over the slice's offsets
    const int tp = t - NW * 64;  // thread index among the pool-writing waves
    constexpr int TP = NT - NW * 64;
    int32_t* pp = ws.pool_pos + (size_t)p * g.n_cap;
    uint32_t* prw = ws.pool_row + (size_t)p * g.n_cap;
    if (r0 < kt) {
      const int re = min(rend, kt);
      const int ob = lens[r0];
      const int oe = min(re < kt ? lens[re] : pool_n, g.n_cap);
      for (int o = ob + 8 * tp; o < oe; o += 8 * TP) {
        int lo = r0, hi = re - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (lens[mid] <= o) lo = mid;
          else hi = mid - 1;
        }
        int k = lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int oi = o + i;
          if (oi < oe) {
            while (k + 1 < re && lens[k + 1] <= oi) ++k;
            const int ps = sm.sst[k - r0] + (oi - lens[k]);
            pp[oi] = ps;
            prw[oi] = row_id_of_page(g, sm.bt[ps >> 6], kvh, ps);
          }
        }
      }
    }
    if (s == 0 && tp == 0) ws.pool_len[p] = min(pool_n, g.n_cap);
  }
  lds_barrier();
  store_split<G, NW, NT>(ws, p, s, splits, sm.wo, sm.wml);
}

// Anchor layer with the rank-expanded pool on grids that the fused anchor
// kernel's one workgroup per 128 selected tokens would not fit (many
// problems, a large kappa): every split's workgroup marks the top-kappa over
// the cache as anchor_attn_kernel does (same inputs, same set), takes the
// positions of its 256 * tiles ranks of the set from the marks, and attends
// them with all sixteen waves in 16-token tiles with running softmax
// statistics (as refine_attn_multi_kernel); one extra workgroup per problem
// writes the rank-expanded pool meanwhile (anchor_rank_emit).  merge_kernel,
// launched next, merges the splits and clears the selection counters.
template <int G>
struct AnchorMultiSmem {
  int32_t bt[kMaxPages];
  uint32_t bitmap[kMaxSeqLen / 32];
  union {
    struct {  // the selection
      uint32_t cbuf[2 * kCand];
      uint32_t hist[4096 + 1024 + 1024];
      uint32_t pair[kPairMax];
      uint32_t ured[32];
      int tmp[NT / 64 + 1];
      int res[9];
      int cnt[2];
    };
    struct {  // the waves' results, after the selection
      float wo[NT / 64][G][kHeadDim];
      float wml[NT / 64][G][2];
    };
  };
  uint32_t srow[kMultiMaxSpan];
  int32_t spos[kMultiMaxSpan];
  float pw[NT / 64][16 * prob_stride<G>()] __attribute__((aligned(16)));
};

// The selection step of the multi-tile kernels over a list of c.n entries
// (scores c.sc; lists longer than kSmall after classify_kernel), as the fused
// anchor kernel makes it: the top-c.K as marks in sm.bitmap, the nonzero mark
// words in order with the rank of their first mark, then the list indices of
// ranks [r0, r0 + span) in sm.spos.  Returns the number of marked entries.
// Contains barriers; lists up to kFusedAnchorLen entries.
template <typename Sm>
__device__ __forceinline__ int multi_select_slice(const Geometry& g, const Workspace& ws, int p,
                                                  const SelList& c, int r0, int span, Sm& sm) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = c.n, K = c.K;
  if (n <= K) {
    for (int i = t; i < ((n + 31) >> 5); i += NT)
      sm.bitmap[i] = (32 * i + 32 <= n) ? 0xFFFFFFFFu : ((1u << (n & 31)) - 1u);
    lds_barrier();
  } else if (n <= kSmall / 2) {
    small_marks<kSmallPer / 2>(c.sc, n, K, sm);
  } else if (n <= kSmall) {
    small_marks<kSmallPer>(c.sc, n, K, sm);
  } else {
    classified_marks(g, ws, p, c, sm);
  }
  const int words = (n + 31) >> 5;
  const int wpt = (words + NT - 1) / NT;
  const int w0 = min(words, t * wpt), w1 = min(words, w0 + wpt);
  int cnt = 0, nz = 0;
  for (int i = w0; i < w1; ++i) {
    const uint32_t m = sm.bitmap[i];
    cnt += __popc(m);
    nz += m ? 1 : 0;
  }
  int total, nz_total;
  int rank = block_excl_scan<NT>(cnt, sm.tmp, &total);
  int slot = block_excl_scan<NT>(nz, sm.tmp, &nz_total);
  uint32_t* const wl = sm.hist;  // word index << 14 | rank of its first mark
  for (int i = w0; i < w1; ++i) {
    const uint32_t m = sm.bitmap[i];
    if (m) {
      wl[slot++] = ((uint32_t)i << 14) | (uint32_t)min(rank, 16383);
      rank += __popc(m);
    }
  }
  lds_barrier();
  // one lane per bit of two listed words at a time
  const int rend = min(K, r0 + span);
  for (int x = 2 * wave; x < nz_total; x += 2 * (NT / 64)) {
    const int idx = x + (lane >> 5), bit = lane & 31;
    if (idx < nz_total) {
      const uint32_t e = wl[idx];
      const int wi = (int)(e >> 14), base = (int)(e & 16383u);
      const uint32_t m = sm.bitmap[wi];
      if ((m >> bit) & 1u) {
        const int r = base + __popc(m & ((1u << bit) - 1u));
        if (r >= r0 && r < rend) sm.spos[r - r0] = wi * 32 + bit;
      }
    }
  }
  lds_barrier();
  return total;
}

template <int G>
__global__ __launch_bounds__(NT) void anchor_rank_multi_kernel(Geometry g, Workspace ws,
                                                               const uint16_t* __restrict__ q,
                                                               float scale,
                                                               int32_t* __restrict__ anchor_idx,
                                                               int32_t* __restrict__ layer_idx,
                                                               int tiles) {
  __shared__ AnchorMultiSmem<G> sm;
  const int K = g.kappa;
  tiles = clampi(tiles, 1, kMultiMaxTiles);
  const int span = 16 * (NT / 64) * tiles;
  const int splits = (K + span - 1) / span;
  if ((int)blockIdx.x >= g.problems() * splits) {  // uniform over the workgroup
    anchor_rank_emit(g, ws, (int)blockIdx.x - g.problems() * splits, sm);
    return;
  }
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int t = threadIdx.x;
  const int n = seq_len_of(g, b);
  const int r0 = s * span;
  load_bt(g, b, n, sm.bt);
  SelList c;
  c.sc = ws.scores + (size_t)p * g.n_cap;
  c.plist = nullptr;
  c.prow = nullptr;
  c.n = n;
  c.K = K;
  c.b = b;
  c.kvh = kvh;
  c.o1 = c.o2 = nullptr;
  c.srow = nullptr;
  c.ent = nullptr;
  const int total = multi_select_slice(g, ws, p, c, r0, span, sm);
  const int rend = min(K, r0 + span);
  // this split's ranks: row ids for the attention, the anchor set
  const int kt = min(total, K);
  for (int k = t; k < rend - r0; k += NT) {
    const int r = r0 + k;
    int a = -1;
    if (r < kt) {
      a = clampi(sm.spos[k], 0, n - 1);
      sm.srow[k] = row_id_of_page(g, sm.bt[a >> 6], kvh, a);
    }
    if (anchor_idx) anchor_idx[(size_t)p * K + r] = a;
    if (layer_idx) layer_idx[(size_t)p * K + r] = a;
  }
  lds_barrier();
  multi_attend_store<G>(g, ws, q, scale, p, s, splits, min(kt - r0, span), tiles, sm);
}

// Refined layer of grids the fused kernel does not fit, for pools that can
// hold more than kSmall entries (scored with coarse counts and classified
// first): the multi-tile kernels' selection over the pool's list (its scores
// in pool order and the pool's classification), this split's ranks resolved
// to row ids and positions through the pool, then the multi-tile attention.
// merge_kernel, launched next, clears the counters the classification used.
template <int G>
__global__ __launch_bounds__(NT) void refine_attn_multi_long_kernel(
    Geometry g, Workspace ws, const uint16_t* __restrict__ q, float scale,
    int32_t* __restrict__ layer_idx, int tiles) {
  __shared__ AnchorMultiSmem<G> sm;
  const int K = g.kappa;
  tiles = clampi(tiles, 1, kMultiMaxTiles);
  const int span = 16 * (NT / 64) * tiles;
  const int splits = (K + span - 1) / span;
  int p, s;
  map_block(blockIdx.x, g.problems(), splits, &p, &s);
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int t = threadIdx.x;
  const size_t base = (size_t)p * g.n_cap;
  SelList c;
  c.sc = ws.scores + base;
  c.plist = ws.pool_pos + base;
  c.prow = ws.pool_row + base;
  c.n = min(clampi(ws.pool_len[p], 0, g.n_cap), kFusedAnchorLen);
  c.K = K;
  c.b = b;
  c.kvh = kvh;
  c.o1 = c.o2 = nullptr;
  c.srow = nullptr;
  c.ent = nullptr;
  const int r0 = s * span;
  const int total = multi_select_slice(g, ws, p, c, r0, span, sm);
  const int rend = min(K, r0 + span);
  const int kt = min(total, K);
  for (int k = t; k < rend - r0; k += NT) {
    const int r = r0 + k;
    int a = -1;
    if (r < kt) {
      const int e = clampi(sm.spos[k], 0, c.n - 1);
      a = c.plist[e];
      sm.srow[k] = c.prow[e];
    }
    if (layer_idx) layer_idx[(size_t)p * K + r] = a;
  }
  lds_barrier();
  multi_attend_store<G>(g, ws, q, scale, p, s, splits, min(kt - r0, span), tiles, sm);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Anchor layer with the rank-expanded pool (Eq. 4): the pool that the refined
// layers re-score is the anchor's own top rho*kappa tokens, and the anchor
// attends its top-kappa, which lies inside that pool.  One workgroup per
// problem, after scoring (and, for lists longer than kSmall, classification
// with rho*kappa wanted): the pool's marks over the cache, the pool in
// position order (positions, row ids, length), then the top-kappa of the
// pool's scores as the anchor set (positions to out / out2, row ids for the
// attention).  Leaves the selection counters at zero.
// ---------------------------------------------------------------------------
template <int R>
__device__ __forceinline__ void select_in_pool(const Geometry& g, const Workspace& ws, int p, int kvh, int m,
                               int32_t* out, int32_t* out2, SelectSmem& sm, bool pos_in_lds) {
  const int t = threadIdx.x, K = g.kappa;
  const size_t base = (size_t)p * g.n_cap;
  const int e0 = R * t;
  const int nv = clampi(m - e0, 0, R);
  uint32_t pos[R], key[R];
  if (pos_in_lds) {  // the pool's positions in rank order are in sm.apos
#pragma unroll
    for (int i = 0; i < R; ++i) pos[i] = i < nv ? (uint32_t)sm.apos[e0 + i] : 0u;
  } else {
    load_run<R>(ws.pool_pos + base, min(e0, g.n_cap - R), pos);  // n_cap is a multiple of 64
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int e = clampi((int)pos[i], 0, g.n_cap - 1);
    key[i] = i < nv ? order_key(ws.scores[base + e]) : 0u;
  }
  const uint32_t take = top_k_mask<R>(key, nv, m, K, sm);
  int total;
  int o = block_excl_scan<NT>(__popc(take), sm.tmp, &total);
  int32_t* o1 = out + (size_t)p * K;
  int32_t* o2 = out2 ? out2 + (size_t)p * K : nullptr;
  uint32_t* sr = ws.sel_row + (size_t)p * K;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (take & (1u << i)) {
      if (o < K) {
        const int ps = clampi((int)pos[i], 0, kMaxSeqLen - 1);
        o1[o] = ps;
        if (o2) o2[o] = ps;
        sr[o] = row_id_of_page(g, sm.bt[ps >> 6], kvh, ps);
      }
      ++o;
    }
  }
  for (int o3 = total + t; o3 < K; o3 += NT) {
    o1[o3] = -1;
    if (o2) o2[o3] = -1;
    sr[o3] = kNoRow;
  }
}

__global__ __launch_bounds__(NT) void rank_pool_kernel(Geometry g, Workspace ws,
                                                       int32_t* __restrict__ out,
                                                       int32_t* __restrict__ out2) {
  __shared__ SelectSmem sm;
  const int p = blockIdx.x, b = p / g.hkv, kvh = p - b * g.hkv;
  const int t = threadIdx.x;
  const int L = seq_len_of(g, b);
  const int m = min(g.pool_rho * g.kappa, L);  // the pool's size
  const size_t base = (size_t)p * g.n_cap;
  load_bt(g, b, L, sm.bt);
  // 1. the pool's marks: the m largest scores of the cache
  SelList c;
  c.sc = ws.scores + base;
  c.plist = nullptr;
  c.prow = nullptr;
  c.n = L;
  c.K = m;
  c.b = b;
  c.kvh = kvh;
  c.o1 = c.o2 = nullptr;
  c.srow = nullptr;
  c.ent = nullptr;
  if (m >= L) {
    for (int i = t; i < ((L + 31) >> 5); i += NT)
      sm.bitmap[i] = (32 * i + 32 <= L) ? 0xFFFFFFFFu : ((1u << (L & 31)) - 1u);
    lds_barrier();
  } else if (L <= kSmall / 2) {
    small_marks<kSmallPer / 2>(c.sc, L, m, sm);
  } else if (L <= kSmall) {
    small_marks<kSmallPer>(c.sc, L, m, sm);
  } else {
    classified_marks(g, ws, p, c, sm);  // after classify_kernel with need m
  }
  // 2. the pool in position order (positions also in sm.apos when it fits)
  int pool_n;
  const bool in_lds = emit_pool<true>(g, ws, p, kvh, L, sm, &pool_n);
  if (!in_lds) __syncthreads();  // the pool's global stores are visible to the whole workgroup
  // 3. the anchor set: the top-kappa of the pool
  const int mm = min(pool_n, kRegMarks);
  if (mm <= kSmall / 2) select_in_pool<kSmallPer / 2>(g, ws, p, kvh, mm, out, out2, sm, in_lds);
  else if (mm <= kSmall) select_in_pool<kSmallPer>(g, ws, p, kvh, mm, out, out2, sm, in_lds);
  else select_in_pool<kRegMarks / NT>(g, ws, p, kvh, mm, out, out2, sm, in_lds);
  reset_selection_counters(ws, p);
}

struct ProfileRing {
  std::vector<hipEvent_t> starts, stops;
  int64_t launches = 0;
};
ProfileRing g_profile[kKernelKinds];

// Launches `kernel`; if its kind has an event ring, the dispatch records the
// ring's next pair at kernel start and end.
template <typename... KArgs, typename... Args>
void launch(int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
            Args... args) {
  ProfileRing& r = g_profile[kind];
  if (!r.starts.empty()) {
    const size_t i = (size_t)(r.launches++ % (int64_t)r.starts.size());
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, r.starts[i], r.stops[i], 0,
                          static_cast<KArgs>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<KArgs>(args)...);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
  }
  return cus[dev];
}

// The fused anchor / refined kernels repeat the selection in every attention
// workgroup of a (sequence, KV head); that costs nothing while all of them run
// at once (one workgroup of 1024 threads per compute unit), but multiplies
// when the grid needs several rounds.  Larger grids select once per problem,
// then attend.
bool fused_fits(const Geometry& g) {
  const long long wgs = (long long)g.problems() * ((g.kappa + kFusedSplit - 1) / kFusedSplit);
  return g.group <= 8 && wgs <= (long long)device_cus();
}

// Tokens per workgroup of the fused refined kernel: 64 when that grid still
// fits the device at once (each workgroup then gathers half the rows, and the
// repeated selection runs on compute units that would idle; 128K planted
// workload: 0.828 against 0.859 ms per step), else kFusedSplit.
int refine_split(const Geometry& g) {
  return (long long)g.problems() * ((g.kappa + 63) / 64) <= (long long)device_cus() ? 64
                                                                                    : kFusedSplit;
}

template <int G>
void launch_anchor_score_g(const Geometry& g, const Workspace& w, const uint16_t* q,
                           hipStream_t s) {
  if (g.k_codes) {
    const int wgs = (g.n_cap + kInt2Entries - 1) / kInt2Entries;
    launch(kAnchorScore, score_anchor_int2_kernel<G>, dim3(g.problems() * wgs),
           dim3(kScoreThreads), s, g, w, q, wgs);
  } else {
    // pages per wave: the largest of 4, 2, 1 that still gives every compute
    // unit four workgroups
    const long long four_per_cu = 4LL * std::max(device_cus(), 1);
    int pages = 4;
    while (pages > 1 && (long long)g.problems() * ((g.n_cap + 256 * pages - 1) / (256 * pages)) <
                            four_per_cu)
      pages >>= 1;
    const int wgs = (g.n_cap + 256 * pages - 1) / (256 * pages);
    const dim3 grid(g.problems() * wgs), block(kScoreThreads);
    if (pages == 4)
      launch(kAnchorScore, score_anchor_kernel<G, 4>, grid, block, s, g, w, q, wgs);
    else if (pages == 2)
      launch(kAnchorScore, score_anchor_kernel<G, 2>, grid, block, s, g, w, q, wgs);
    else
      launch(kAnchorScore, score_anchor_kernel<G, 1>, grid, block, s, g, w, q, wgs);
  }
}

// Bound of a refinement pool's length: min(n_cap, kappa (2w + 1)) for the
// window pool, min(n_cap, rho kappa) for the rank-expanded one.
int pool_cap(const Geometry& g) {
  return (int)std::min<long long>(g.n_cap, g.pool_rho >= 1
                                               ? (long long)g.pool_rho * g.kappa
                                               : (long long)g.kappa * (2LL * g.window + 1));
}

// Tiles per wave of refine_attn_multi_kernel at a refined layer whose grid
// the fused kernel does not fit: the fewest (up to kMultiMaxTiles) whose grid
// of problems x ceil(kappa / (256 tiles)) workgroups fits the device at once;
// 0 (the per-problem path) when none does, for groups above 8, and when the
// pool can hold more than kSmall entries.
int multi_tiles(const Geometry& g) {
  if (g.group > 8 || pool_cap(g) > kSmall) return 0;
  for (int tl = 1; tl <= kMultiMaxTiles; ++tl) {
    const int span = 16 * (NT / 64) * tl;
    if ((long long)g.problems() * ((g.kappa + span - 1) / span) <= (long long)device_cus())
      return tl;
  }
  return 0;
}

template <int G>
void launch_pool_score_g(const Geometry& g, const Workspace& w, const uint16_t* q, bool hist,
                         hipStream_t s) {
  const int chunks = hist ? kPoolHistChunks : 1;
  const int per_wg = chunks * kPoolEntries;
  const int wgs = (pool_cap(g) + per_wg - 1) / per_wg;
  if (g.k_codes)
    launch(kRefineScore, score_pool_int2_kernel<G>, dim3(g.problems() * wgs), dim3(kScoreThreads),
           s, g, w, q, wgs, chunks, hist ? 1 : 0);
  else
    launch(kRefineScore, score_pool_kernel<G>, dim3(g.problems() * wgs), dim3(kScoreThreads), s,
           g, w, q, wgs, chunks, hist ? 1 : 0);
}

template <int G>
void launch_merge_g(const Geometry& g, const Workspace& w, int splits, float* out, bool reset,
                    hipStream_t s) {
  launch(kMerge, merge_kernel<G>, dim3(g.problems() * G), dim3(kHeadDim), s, g, w, splits, out,
         reset ? 1 : 0);
}

template <int G, int MODE>
void launch_attention_g(const Geometry& g, const Workspace& w, const uint16_t* q,
                        const int32_t* idx, int32_t* pos_out, float scale, float* out,
                        bool quantize_new, hipStream_t s) {
  const int extra = quantize_new && g.k_codes && g.new_keys > 0 ? g.problems() : 0;
  const int splits = (g.kappa + kSetSplit - 1) / kSetSplit;
  launch(kAttention, attn_kernel<G, MODE>, dim3(g.problems() * splits + extra),
         dim3(64 * kSetWaves), s, g, w, q, idx, pos_out, scale, splits);
  launch_merge_g<G>(g, w, splits, out, false, s);
}

#define PRISM_BY_GROUP(FN, ...)                      \
  switch (g.group) {                                 \
    case 1: FN<1>(__VA_ARGS__); break;               \
    case 2: FN<2>(__VA_ARGS__); break;               \
    case 4: FN<4>(__VA_ARGS__); break;               \
    case 8: FN<8>(__VA_ARGS__); break;               \
    case 16: FN<16>(__VA_ARGS__); break;             \
    default: return hipErrorInvalidValue;            \
  }

}  // namespace

bool set_profile_events(int kind, void* const* starts, void* const* stops, int count) {
  if (kind < 0 || kind >= kKernelKinds || count < 0) return false;
  ProfileRing& r = g_profile[kind];
  r.starts.clear();
  r.stops.clear();
  r.launches = 0;
  if (count == 0 || !starts || !stops) return true;
  for (int i = 0; i < count; ++i) {
    r.starts.push_back(static_cast<hipEvent_t>(starts[i]));
    r.stops.push_back(static_cast<hipEvent_t>(stops[i]));
  }
  return true;
}

int64_t profile_launches(int kind) {
  if (kind < 0 || kind >= kKernelKinds) return -1;
  return g_profile[kind].launches;
}

// Workspace regions in carve order: {bytes, alignment padding applied}.
size_t workspace_bytes(const Geometry& g) {
  const size_t P = (size_t)g.problems();
  size_t o = 0;
  const size_t W = (size_t)cls_regions(g);
  o += align256(P * kCoarseBins * 4);                            // ghist
  o += align256(P * W * 4);                                      // cand_cnt
  o += align256(P * W * 4);                                      // cand_cnt2
  o += align256(P * 4 * 4);                                      // sel_meta
  o += align256(P * W * kClsCap * 4);                            // cand_key
  o += align256(P * W * kClsCap * 4);                            // cand_idx
  o += align256(P * (size_t)(g.n_cap / 32) * 4);                 // gbits
  o += align256(P * (size_t)g.n_cap * 4);                        // scores
  o += align256(P * (size_t)g.n_cap * 4);                        // pool_pos
  o += align256(P * (size_t)g.n_cap * 4);                        // pool_row
  o += align256(P * 4);                                          // pool_len
  o += align256(P * (size_t)g.kappa * 4);                        // sel_row
  o += align256(P * (size_t)g.kappa * 4);                        // idx_tmp
  o += align256(P * (size_t)g.kappa * 4);                        // sel_ent
  o += align256(P * (size_t)g.splits * g.group * kHeadDim * 4);  // part_o
  o += align256(P * (size_t)g.splits * g.group * 2 * 4);         // part_ml
  o += align256(P * (size_t)dense_splits(g) * g.group * kHeadDim * 4);  // dense_o
  o += align256(P * (size_t)dense_splits(g) * g.group * 2 * 4);         // dense_ml
  o += align256(P * 4 * 4);                                      // sel_meta2
  o += align256(P * W * kClsCap * 4);                            // cand_key2
  o += align256(P * W * kClsCap * 4);                            // cand_idx2
  o += align256(P * (size_t)(g.n_cap / 32) * 4);                 // gbits2
  return o;
}

Workspace carve_workspace(void* base, const Geometry& g) {
  const size_t P = (size_t)g.problems();
  char* c = static_cast<char*>(base);
  Workspace w;
  const size_t W = (size_t)cls_regions(g);
  w.ghist = reinterpret_cast<uint32_t*>(c);
  c += align256(P * kCoarseBins * 4);
  w.cand_cnt = reinterpret_cast<uint32_t*>(c);
  c += align256(P * W * 4);
  w.cand_cnt2 = reinterpret_cast<uint32_t*>(c);
  c += align256(P * W * 4);
  w.sel_meta = reinterpret_cast<int32_t*>(c);
  c += align256(P * 4 * 4);
  w.cand_key = reinterpret_cast<uint32_t*>(c);
  c += align256(P * W * kClsCap * 4);
  w.cand_idx = reinterpret_cast<int32_t*>(c);
  c += align256(P * W * kClsCap * 4);
  w.gbits = reinterpret_cast<uint32_t*>(c);
  c += align256(P * (size_t)(g.n_cap / 32) * 4);
  w.scores = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)g.n_cap * 4);
  w.pool_pos = reinterpret_cast<int32_t*>(c);
  c += align256(P * (size_t)g.n_cap * 4);
  w.pool_row = reinterpret_cast<uint32_t*>(c);
  c += align256(P * (size_t)g.n_cap * 4);
  w.pool_len = reinterpret_cast<int32_t*>(c);
  c += align256(P * 4);
  w.sel_row = reinterpret_cast<uint32_t*>(c);
  c += align256(P * (size_t)g.kappa * 4);
  w.idx_tmp = reinterpret_cast<int32_t*>(c);
  c += align256(P * (size_t)g.kappa * 4);
  w.sel_ent = reinterpret_cast<int32_t*>(c);
  c += align256(P * (size_t)g.kappa * 4);
  w.part_o = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)g.splits * g.group * kHeadDim * 4);
  w.part_ml = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)g.splits * g.group * 2 * 4);
  w.dense_o = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)dense_splits(g) * g.group * kHeadDim * 4);
  w.dense_ml = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)dense_splits(g) * g.group * 2 * 4);
  w.sel_meta2 = reinterpret_cast<int32_t*>(c);
  c += align256(P * 4 * 4);
  w.cand_key2 = reinterpret_cast<uint32_t*>(c);
  c += align256(P * W * kClsCap * 4);
  w.cand_idx2 = reinterpret_cast<int32_t*>(c);
  c += align256(P * W * kClsCap * 4);
  w.gbits2 = reinterpret_cast<uint32_t*>(c);
  return w;
}

// Anchor layer: score every cached token (filling the coarse histogram),
// classify lists longer than kSmall over many workgroups, then select per
// problem (and build the pool).  The histogram is zero from its last reader
// (each selection clears it); in a fresh or reused workspace it holds other
// bytes, and then the classification disagrees with itself and the selection
// runs its exact fallback once.
hipError_t launch_anchor(const Geometry& g, const Workspace& w, const uint16_t* q, int32_t* out,
                         int32_t* out2, hipStream_t s) {
  PRISM_BY_GROUP(launch_anchor_score_g, g, w, q, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.max_seq_len > kSmall && g.max_seq_len > g.kappa) {
    const int wgs = (g.n_cap + kClsEntries - 1) / kClsEntries;
    launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w, wgs,
           0, g.kappa, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  launch(kSelect, select_kernel<false>, dim3(g.problems()), dim3(NT), s, g, w, out, out2, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pool_build(g, w, out, s);  // the pool of the set just written to out
}

hipError_t launch_anchor_rank(const Geometry& g, const Workspace& w, const uint16_t* q,
                              int32_t* out, int32_t* out2, hipStream_t s) {
  PRISM_BY_GROUP(launch_anchor_score_g, g, w, q, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long m = (long long)g.pool_rho * g.kappa;
  if (g.max_seq_len > kSmall && g.max_seq_len > m) {
    const int wgs = (g.n_cap + kClsEntries - 1) / kClsEntries;
    launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w, wgs,
           0, (int)m, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  launch(kSelect, rank_pool_kernel, dim3(g.problems()), dim3(NT), s, g, w, out, out2);
  return hipGetLastError();
}

template <int G>
void launch_anchor_attn_g(const Geometry& g, const Workspace& w, const uint16_t* q, float scale,
                          float* out, int32_t* anchor_idx, int32_t* layer_idx, bool rank,
                          hipStream_t s) {
  const int splits = (g.kappa + kFusedSplit - 1) / kFusedSplit;
  const dim3 block(NT);
  // contexts of at most kRegMarks tokens are selected from keys in registers
  // (no classification launched before)
  const bool reg32 = g.max_seq_len <= kRegMarks;
  if (rank) {
    const dim3 grid(g.problems() * (splits + 1));
    if (reg32)
      launch(kAttention, anchor_attn_kernel<G, true, true>, grid, block, s, g, w, q, scale,
             anchor_idx, layer_idx);
    else
      launch(kAttention, anchor_attn_kernel<G, true>, grid, block, s, g, w, q, scale, anchor_idx,
             layer_idx);
  } else {
    const dim3 grid(g.problems() * splits);
    if (reg32)
      launch(kAttention, anchor_attn_kernel<G, false, true>, grid, block, s, g, w, q, scale,
             anchor_idx, layer_idx);
    else
      launch(kAttention, anchor_attn_kernel<G, false>, grid, block, s, g, w, q, scale, anchor_idx,
             layer_idx);
  }
  launch_merge_g<G>(g, w, splits, out, true, s);
}

// Tiles per wave of anchor_rank_multi_kernel at a rank-pool anchor layer
// whose grid the fused anchor kernel does not fit: the fewest (up to
// kMultiMaxTiles) whose grid of problems x (ceil(kappa / (256 tiles)) + 1)
// workgroups fits the device at once, if that still gives every problem two
// or more attention workgroups; else 0 (the per-problem rank kernel, then
// the attention over many workgroups), also for groups above 8 and for
// contexts whose nonzero mark words exceed the word list.  With one split a
// single compute unit would gather all kappa rows of its problem (batched
// 16 x 8K-64K workload, kappa = 1024: 3.26 against 3.23 ms per step).
int anchor_multi_tiles(const Geometry& g) {
  if (g.group > 8 || g.max_seq_len > kFusedAnchorLen) return 0;
  for (int tl = 1; tl <= kMultiMaxTiles; ++tl) {
    const int span = 16 * (NT / 64) * tl;
    const int splits = (g.kappa + span - 1) / span;
    if ((long long)g.problems() * (splits + 1) <= (long long)device_cus())
      return splits >= 2 ? tl : 0;
  }
  return 0;
}

template <int G>
void launch_anchor_rank_multi_g(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, float* out, int32_t* anchor_idx, int32_t* layer_idx,
                                int tiles, hipStream_t s) {
  const int span = 16 * (NT / 64) * tiles;
  const int splits = (g.kappa + span - 1) / span;
  launch(kAttention, anchor_rank_multi_kernel<G>, dim3(g.problems() * (splits + 1)), dim3(NT), s,
         g, w, q, scale, anchor_idx, layer_idx, tiles);
  launch_merge_g<G>(g, w, splits, out, true, s);
}

hipError_t launch_anchor_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, int32_t* anchor_idx, int32_t* layer_idx, float* out,
                                hipStream_t s) {
  // the fused kernel's LDS holds up to 8 heads and lists up to kFusedAnchorLen
  // nonzero mark words; otherwise select, then attend
  if (!fused_fits(g) || g.max_seq_len > kFusedAnchorLen) {
    hipError_t e = launch_anchor(g, w, q, anchor_idx, layer_idx, s);
    if (e != hipSuccess) return e;
    return launch_attention(g, w, q, nullptr, true, scale, out, s);
  }
  // The histogram and candidate counter are zero from the previous anchor
  // layer (the selection checks its own consistency, so a fresh workspace only
  // takes the exact fallback once).
  PRISM_BY_GROUP(launch_anchor_score_g, g, w, q, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.max_seq_len > kRegMarks && g.max_seq_len > g.kappa) {
    const int wgs = (g.n_cap + kClsEntries - 1) / kClsEntries;
    launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w, wgs,
           0, g.kappa, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (g.group) {
    case 1: launch_anchor_attn_g<1>(g, w, q, scale, out, anchor_idx, layer_idx, false, s); break;
    case 2: launch_anchor_attn_g<2>(g, w, q, scale, out, anchor_idx, layer_idx, false, s); break;
    case 4: launch_anchor_attn_g<4>(g, w, q, scale, out, anchor_idx, layer_idx, false, s); break;
    case 8: launch_anchor_attn_g<8>(g, w, q, scale, out, anchor_idx, layer_idx, false, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Anchor layer with the rank-expanded pool.  When the fused anchor kernel's
// grid, with one more workgroup per problem, fits the device: scoring, one
// classify pass for both kappa (the anchor set) and rho*kappa (the pool), the
// fused kernel (its attention workgroups select and attend the anchor set as
// for the window pool; the extra workgroups write the pool meanwhile), the
// merge.  Otherwise the per-problem rank kernel, then the attention.
hipError_t launch_anchor_rank_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                     float scale, int32_t* anchor_idx, int32_t* layer_idx,
                                     float* out, hipStream_t s) {
  const long long splits = (g.kappa + kFusedSplit - 1) / kFusedSplit;
  const bool fits = g.group <= 8 && g.max_seq_len <= kFusedAnchorLen &&
                    (long long)g.problems() * (splits + 1) <= (long long)device_cus();
  const int tiles = fits ? 0 : anchor_multi_tiles(g);
  if (!fits && tiles == 0) {
    hipError_t e = launch_anchor_rank(g, w, q, anchor_idx, layer_idx, s);
    if (e != hipSuccess) return e;
    return launch_attention(g, w, q, nullptr, true, scale, out, s);
  }
  PRISM_BY_GROUP(launch_anchor_score_g, g, w, q, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long m = (long long)g.pool_rho * g.kappa;
  // the fused kernel selects contexts of at most kRegMarks tokens from keys in
  // registers; the multi-tile kernel selects from the classification
  if (g.max_seq_len > (tiles > 0 ? kSmall : kRegMarks) && g.max_seq_len > g.kappa) {
    const int wgs = (g.n_cap + kClsEntries - 1) / kClsEntries;
    launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w, wgs,
           0, g.kappa, g.max_seq_len > m ? (int)m : 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tiles > 0) {  // groups of at most 8 heads
#define PRISM_RANK_MULTI(G) \
  launch_anchor_rank_multi_g<G>(g, w, q, scale, out, anchor_idx, layer_idx, tiles, s); break;
    switch (g.group) {
      case 1: PRISM_RANK_MULTI(1)
      case 2: PRISM_RANK_MULTI(2)
      case 4: PRISM_RANK_MULTI(4)
      case 8: PRISM_RANK_MULTI(8)
      default: return hipErrorInvalidValue;
    }
#undef PRISM_RANK_MULTI
    return hipGetLastError();
  }
  switch (g.group) {
    case 1: launch_anchor_attn_g<1>(g, w, q, scale, out, anchor_idx, layer_idx, true, s); break;
    case 2: launch_anchor_attn_g<2>(g, w, q, scale, out, anchor_idx, layer_idx, true, s); break;
    case 4: launch_anchor_attn_g<4>(g, w, q, scale, out, anchor_idx, layer_idx, true, s); break;
    case 8: launch_anchor_attn_g<8>(g, w, q, scale, out, anchor_idx, layer_idx, true, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pool_build(const Geometry& g, const Workspace& w, const int32_t* anchor_idx,
                             hipStream_t s) {
  const int slices = std::max(1, (pool_cap(g) + 8 * NT - 1) / (8 * NT));  // 8 entries per thread
  launch(kPoolBuild, pool_build_kernel, dim3(g.problems() * slices), dim3(NT), s, g, w,
         anchor_idx, slices);
  return hipGetLastError();
}

// Refined layer without the fused kernel: score the pool (counting pools longer
// than kSmall per coarse bin), classify those pools over many workgroups, then
// select per problem.  The pool's length is known on the device only; its
// bound decides whether classification can be needed, and sizes the grids.
hipError_t launch_refine(const Geometry& g, const Workspace& w, const uint16_t* q, int32_t* out,
                         hipStream_t s, bool defer) {
  const int bound = pool_cap(g);
  const bool classify = bound > kSmall && bound > g.kappa;
  PRISM_BY_GROUP(launch_pool_score_g, g, w, q, classify, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (classify) {
    const int wgs = (bound + kClsEntries - 1) / kClsEntries;
    launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w, wgs,
           1, g.kappa, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  launch(kSelect, select_kernel<true>, dim3(g.problems()), dim3(NT), s, g, w, out,
         static_cast<int32_t*>(nullptr), defer ? 1 : 0);
  return hipGetLastError();
}

template <int G>
void launch_refine_attn_g(const Geometry& g, const Workspace& w, const uint16_t* q, float scale,
                          float* out, int32_t* layer_idx, hipStream_t s) {
  if (!fused_fits(g)) {  // the caller checked multi_tiles(g) > 0
    const int tiles = multi_tiles(g);
    const int span = 16 * (NT / 64) * tiles;
    const int splits = (g.kappa + span - 1) / span;
    launch(kAttention, refine_attn_multi_kernel<G>, dim3(g.problems() * splits), dim3(NT), s, g,
           w, q, scale, layer_idx, tiles);
    launch_merge_g<G>(g, w, splits, out, false, s);
    return;
  }
  const int sp = refine_split(g);
  const int splits = (g.kappa + sp - 1) / sp;
  // caches of at most kRegMarks tokens select every pool from registers in
  // the kernel itself: the out-of-line path for longer pools, and its call
  // frame, are then not compiled in (the 32K workload, whose unstructured
  // pools cover most of the cache, takes it on every refined layer)
  const bool reg32 = g.n_cap <= kRegMarks;
  const dim3 grid(g.problems() * splits), block(NT);
  if (sp == 64) {
    if (reg32)
      launch(kAttention, refine_attn_kernel<G, 64, true>, grid, block, s, g, w, q, scale, layer_idx);
    else
      launch(kAttention, refine_attn_kernel<G, 64>, grid, block, s, g, w, q, scale, layer_idx);
  } else {
    if (reg32)
      launch(kAttention, refine_attn_kernel<G, kFusedSplit, true>, grid, block, s, g, w, q, scale,
             layer_idx);
    else
      launch(kAttention, refine_attn_kernel<G, kFusedSplit>, grid, block, s, g, w, q, scale,
             layer_idx);
  }
  launch_merge_g<G>(g, w, splits, out, false, s);
}

// Tiles per wave of refine_attn_multi_long_kernel at a refined layer whose
// grid the fused kernel does not fit and whose pool can exceed kSmall
// entries: the fewest (up to kMultiMaxTiles) whose grid of problems x
// ceil(kappa / (256 tiles)) workgroups fits the device, if that leaves two or
// more workgroups per problem; else 0 (selection once per problem), also for
// groups above 8 and pools longer than the multi-tile selection's word list.
int multi_long_tiles(const Geometry& g) {
  if (g.group > 8 || g.max_seq_len > kFusedAnchorLen || pool_cap(g) <= kSmall) return 0;
  for (int tl = 1; tl <= kMultiMaxTiles; ++tl) {
    const int span = 16 * (NT / 64) * tl;
    const int splits = (g.kappa + span - 1) / span;
    if ((long long)g.problems() * splits <= (long long)device_cus()) return splits >= 2 ? tl : 0;
  }
  return 0;
}

template <int G>
void launch_refine_multi_long_g(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, float* out, int32_t* layer_idx, int tiles,
                                hipStream_t s) {
  const int span = 16 * (NT / 64) * tiles;
  const int splits = (g.kappa + span - 1) / span;
  launch(kAttention, refine_attn_multi_long_kernel<G>, dim3(g.problems() * splits), dim3(NT), s,
         g, w, q, scale, layer_idx, tiles);
  launch_merge_g<G>(g, w, splits, out, true, s);
}

hipError_t launch_refine_attend(const Geometry& g, const Workspace& w, const uint16_t* q,
                                float scale, int32_t* layer_idx, float* out, hipStream_t s) {
  const int long_tiles = fused_fits(g) ? 0 : multi_long_tiles(g);
  if (long_tiles > 0) {
    // pools scored with coarse counts and classified over many workgroups,
    // then selected and attended in the multi-tile kernel
    const int bound = pool_cap(g);
    const bool classify = bound > g.kappa;  // bound > kSmall here
    PRISM_BY_GROUP(launch_pool_score_g, g, w, q, classify, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (classify) {
      const int wgs = (bound + kClsEntries - 1) / kClsEntries;
      launch(kClassify, classify_kernel, dim3(g.problems() * wgs), dim3(kClsThreads), s, g, w,
             wgs, 1, g.kappa, 0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
#define PRISM_LONG_MULTI(G) \
  launch_refine_multi_long_g<G>(g, w, q, scale, out, layer_idx, long_tiles, s); break;
    switch (g.group) {
      case 1: PRISM_LONG_MULTI(1)
      case 2: PRISM_LONG_MULTI(2)
      case 4: PRISM_LONG_MULTI(4)
      case 8: PRISM_LONG_MULTI(8)
      default: return hipErrorInvalidValue;
    }
#undef PRISM_LONG_MULTI
    return hipGetLastError();
  }
  if (!fused_fits(g) && multi_tiles(g) == 0) {
    // select once per problem (pool indices only), then attend
    hipError_t e = launch_refine(g, w, q, nullptr, s, true);
    if (e != hipSuccess) return e;
    return launch_attention_entries(g, w, q, layer_idx, scale, out, s);
  }
  PRISM_BY_GROUP(launch_pool_score_g, g, w, q, false, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (g.group) {
    case 1: launch_refine_attn_g<1>(g, w, q, scale, out, layer_idx, s); break;
    case 2: launch_refine_attn_g<2>(g, w, q, scale, out, layer_idx, s); break;
    case 4: launch_refine_attn_g<4>(g, w, q, scale, out, layer_idx, s); break;
    case 8: launch_refine_attn_g<8>(g, w, q, scale, out, layer_idx, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dense(const Geometry& g, const Workspace& w, const uint16_t* q, float scale,
                        float* out, hipStream_t s) {
  const int splits = dense_splits(g), chunk = dense_chunk(g);
  Workspace wd = w;
  wd.part_o = w.dense_o;
  wd.part_ml = w.dense_ml;
#define PRISM_DENSE(G)                                                                          \
  launch(kDense, dense_attn_kernel<G>, dim3(g.problems() * splits), dim3(kAttnThreads), s, g, wd, \
         q, splits, chunk, scale);                                                              \
  launch_merge_g<G>(g, wd, splits, out, false, s);                                              \
  break;
  switch (g.group) {
    case 1: PRISM_DENSE(1)
    case 2: PRISM_DENSE(2)
    case 4: PRISM_DENSE(4)
    case 8: PRISM_DENSE(8)
    case 16: PRISM_DENSE(16)
    default: return hipErrorInvalidValue;
  }
#undef PRISM_DENSE
  return hipGetLastError();
}

hipError_t launch_quantize(const Geometry& g, int num_new, uint8_t* codes, uint16_t* scales,
                           hipStream_t s) {
  const int range = (num_new > 0 && num_new < g.max_seq_len) ? num_new : g.max_seq_len;
  const int chunks = (range + 4 * kQuantRows - 1) / (4 * kQuantRows);  // four waves per workgroup
  launch(kQuantize, quantize_kernel, dim3(g.problems() * chunks), dim3(256), s, g, num_new, chunks,
         codes, scales);
  return hipGetLastError();
}

hipError_t launch_attention(const Geometry& g, const Workspace& w, const uint16_t* q,
                            const int32_t* idx, bool use_sel_rows, float scale, float* out,
                            hipStream_t s, bool quantize_new) {
#define PRISM_ATTN(MODE)                                                                    \
  switch (g.group) {                                                                        \
    case 1: launch_attention_g<1, MODE>(g, w, q, idx, nullptr, scale, out, quantize_new, s); break; \
    case 2: launch_attention_g<2, MODE>(g, w, q, idx, nullptr, scale, out, quantize_new, s); break; \
    case 4: launch_attention_g<4, MODE>(g, w, q, idx, nullptr, scale, out, quantize_new, s); break; \
    case 8: launch_attention_g<8, MODE>(g, w, q, idx, nullptr, scale, out, quantize_new, s); break; \
    case 16: launch_attention_g<16, MODE>(g, w, q, idx, nullptr, scale, out, quantize_new, s); break; \
    default: return hipErrorInvalidValue;                                                    \
  }
  if (use_sel_rows) {
    PRISM_ATTN(kSetRows)
  } else {
    PRISM_ATTN(kSetPositions)
  }
#undef PRISM_ATTN
  return hipGetLastError();
}

hipError_t launch_attention_entries(const Geometry& g, const Workspace& w, const uint16_t* q,
                                    int32_t* pos_out, float scale, float* out, hipStream_t s) {
  switch (g.group) {
    case 1: launch_attention_g<1, kSetEntries>(g, w, q, nullptr, pos_out, scale, out, false, s); break;
    case 2: launch_attention_g<2, kSetEntries>(g, w, q, nullptr, pos_out, scale, out, false, s); break;
    case 4: launch_attention_g<4, kSetEntries>(g, w, q, nullptr, pos_out, scale, out, false, s); break;
    case 8: launch_attention_g<8, kSetEntries>(g, w, q, nullptr, pos_out, scale, out, false, s); break;
    case 16: launch_attention_g<16, kSetEntries>(g, w, q, nullptr, pos_out, scale, out, false, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace prism

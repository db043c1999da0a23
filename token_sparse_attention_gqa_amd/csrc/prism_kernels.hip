// HIP kernels for gfx950 (CDNA4): token-sparse GQA decode attention with
// proposal-refined cross-layer index sharing ("Prism Attention", arXiv
// 2610.22985).
//
//   score_kernel      relevance (Eq. 9 / Eq. 1) of every entry of a token list
//                     (all cached tokens at an anchor layer, the refinement pool
//                     at a refined layer) with one MFMA per 16 tokens x 32 dims,
//                     plus a 4096-bin histogram of the scores' leading bits.
//   pool_plan_kernel  the refined layer's pool: union of [i-w, i+w] over the
//                     anchor's ascending set, as disjoint runs, flattened.
//   select_kernel     exact top-kappa (Eq. 2 / Eq. 6) by radix select on
//                     order-preserving 32-bit keys; lower position wins ties.
//   attn_kernel       SparseAttn of Algorithm 1 over one split of the set,
//   combine_kernel    and the fixed-order merge of the splits.
#include "prism_internal.hpp"

#include <hip/hip_ext.h>

#include <cmath>
#include <vector>

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;

// Monotone map of a float to uint32: a > b  <=>  key(a) > key(b); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ __forceinline__ int seq_len_of(const Geometry& g, int b) {
  return clampi(g.seq_lens[b], 0, g.max_seq_len);
}

// Element offset of token `pos` of sequence b, KV head h in the paged cache.
__device__ __forceinline__ size_t row_offset(const Geometry& g, int b, int h, int pos) {
  int page = g.block_table[(size_t)b * g.max_pages + (pos >> 6)];
  page = clampi(page, 0, g.num_pages - 1);
  return (size_t)page * g.page_stride + ((size_t)h * kPageSize + (pos & (kPageSize - 1))) * kHeadDim;
}

// MFMA A-operand fragment of the group's query heads.  Lane l holds head
// (l % 16) (zero when >= G) and, for step s, the 16-byte chunk g4 + 4s of the
// head dimension, g4 = l / 16.  The key fragments use the same chunk order, so
// the four steps together contract over all 128 dimensions.
template <int G>
__device__ __forceinline__ void load_q_frag(const uint16_t* q, const Geometry& g, int b, int kvh,
                                            int lane, u32x4 (&qf)[4]) {
  const int j = lane & 15, g4 = lane >> 4;
  if (j < G) {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(q + ((size_t)b * g.hq + kvh * G + j) * kHeadDim);
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
                                                  __builtin_bit_cast(bf16x8, kf[s]), acc, 0, 0, 0);
  return acc;
}

// Max over the group's heads of a qk_tile; valid in lanes 0..15 (token = lane).
template <int G>
__device__ __forceinline__ float group_max(const f32x4& acc, int g4) {
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * g4 + r < G) m = fmaxf(m, acc[r]);
  if (G > 4) m = fmaxf(m, __shfl_xor(m, 16));
  if (G > 8) m = fmaxf(m, __shfl_xor(m, 32));
  return m;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix sum over the NT threads of the block; *total gets the sum.
// tmp: at least NT/64 + 1 ints of LDS.  Contains barriers: call uniformly.
template <int NT>
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int x = lane < NW ? tmp[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < NW) tmp[lane] = xi - x;
    if (lane == NW - 1) tmp[NW] = xi;
  }
  __syncthreads();
  const int r = tmp[w] + inc - v;
  *total = tmp[NW];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Histogram reset (anchor layers; the pool plan resets it for refined layers)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_hist_kernel(uint32_t* hist) {
  uint32_t* h = hist + (size_t)blockIdx.x * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0u;
}

// ---------------------------------------------------------------------------
// Refined-layer pool.  With the anchor set ascending and every window of equal
// width, the union of [a_k - w, a_k + w] is the disjoint union over k of
// [max(lo_k, hi_{k-1} + 1), hi_k]: run k only adds what run k-1 did not cover.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pool_plan_kernel(Geometry g, Workspace ws,
                                                        const int32_t* __restrict__ anchor) {
  extern __shared__ int32_t plan[];  // run start [kappa], then run offset [kappa]
  __shared__ int tmp[8];
  const int p = blockIdx.x, b = p / g.hkv, t = threadIdx.x;
  const int K = g.kappa;
  int32_t* st = plan;
  int32_t* off = plan + K;
  const int L = seq_len_of(g, b);
  const int w = g.window < L ? g.window : L;

  uint32_t* h = ws.hist + (size_t)p * kHistBins;
  for (int i = t; i < kHistBins; i += 256) h[i] = 0u;

  const int32_t* a = anchor + (size_t)p * K;
  const int per = (K + 255) / 256;
  const int k0 = min(K, t * per), k1 = min(K, k0 + per);
  int sum = 0;
  for (int k = k0; k < k1; ++k) {
    const int ai = a[k];
    int s0 = 0, len = 0;
    if (ai >= 0 && ai < L) {
      const int lo = max(ai - w, 0), hi = min(ai + w, L - 1);
      int prev_hi = -1;
      if (k > 0) {
        const int ap = a[k - 1];
        if (ap >= 0 && ap < L) prev_hi = min(ap + w, L - 1);
      }
      s0 = max(lo, prev_hi + 1);
      len = max(0, hi - s0 + 1);
    }
    st[k] = s0;
    off[k] = len;
    sum += len;
  }
  int total;
  int ex = block_excl_scan<256>(sum, tmp, &total);
  for (int k = k0; k < k1; ++k) {
    const int len = off[k];
    off[k] = ex;
    ex += len;
  }
  const int n = min(total, g.n_cap);
  if (t == 0) ws.pool_len[p] = n;
  __syncthreads();
  int32_t* out = ws.pool_pos + (size_t)p * g.n_cap;
  for (int e = t; e < n; e += 256) {
    int lo = 0, hi = K - 1;  // largest k with off[k] <= e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= e) lo = mid; else hi = mid - 1;
    }
    out[e] = st[lo] + (e - off[lo]);
  }
}

// ---------------------------------------------------------------------------
// Relevance of a token list (Eq. 9).  One workgroup scores kScoreChunk list
// entries of one (sequence, KV head); each wave takes 256 of them as 16 tiles of
// 16 tokens.  Per tile every lane issues four 16-byte loads (the 64-byte
// quarter-rows of 16 consecutive tokens) and the wave issues four MFMAs.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void score_kernel(Geometry g, Workspace ws,
                                                    const uint16_t* __restrict__ q, int chunks,
                                                    int pool) {
  __shared__ uint32_t lhist[kHistBins];
  const int p = blockIdx.x / chunks;
  const int chunk = blockIdx.x - p * chunks;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int L = seq_len_of(g, b);
  const int n = pool ? clampi(ws.pool_len[p], 0, g.n_cap) : L;
  const int begin = chunk * kScoreChunk;
  if (L <= 0 || begin >= n) return;  // uniform over the workgroup
  const int end = min(n, begin + kScoreChunk);

  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  u32x4 qf[4];
  load_q_frag<G>(q, g, b, kvh, lane, qf);
  __syncthreads();

  const int32_t* plist = ws.pool_pos + (size_t)p * g.n_cap;
  float* out = ws.scores + (size_t)p * g.n_cap;
  const int wbegin = begin + wave * (kScoreChunk / 4);
#pragma unroll 1
  for (int t0 = 0; t0 < 16; t0 += 4) {
    u32x4 kf[4][4];
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      e[u] = wbegin + (t0 + u) * 16 + j;
      const int es = min(e[u], end - 1);
      const int pos = clampi(pool ? plist[es] : es, 0, L - 1);
      const u32x4* row = reinterpret_cast<const u32x4*>(g.k_pages + row_offset(g, b, kvh, pos));
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[u][s] = __builtin_nontemporal_load(row + g4 + 4 * s);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float m = group_max<G>(qk_tile(qf, kf[u]), g4);
      if (g4 == 0 && e[u] < end) {
        out[e[u]] = m;
        atomicAdd(&lhist[order_key(m) >> (32 - kHistBits)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)p * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// In a histogram of NB bins, the bin holding the need-th largest element
// (1-based, counting down from the top bin).  res = {bin, count strictly above,
// count in bin}; res[0] stays -1 if the histogram holds fewer than need.
template <int NB>
__device__ void find_bin(const uint32_t* h, int need, int* res, int* tmp) {
  constexpr int R = NB / kSelThreads;
  const int t = threadIdx.x;
  if (t == 0) res[0] = -1;
  int c[R];
  int sum = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    c[r] = (int)h[NB - 1 - (R * t + r)];
    sum += c[r];
  }
  int total;
  const int excl = block_excl_scan<kSelThreads>(sum, tmp, &total);
  if (excl < need && excl + sum >= need) {
    int acc = excl;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (acc + c[r] >= need) {
        res[0] = NB - 1 - (R * t + r);
        res[1] = acc;
        res[2] = c[r];
        break;
      }
      acc += c[r];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Exact top-kappa of one (sequence, KV head) list.  The scoring kernel's
// histogram gives the bin of the kappa-th largest key; one pass over the list
// marks every entry of a higher bin in an LDS bitmap and gathers the threshold
// bin into LDS; two 10-bit radix levels there give the exact kappa-th key T.
// Entries equal to T are taken lowest list index first (list order is position
// order).  The bitmap, read in order, gives ascending positions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_kernel(Geometry g, Workspace ws, int pool,
                                                             int32_t* __restrict__ out,
                                                             int32_t* __restrict__ out2) {
  extern __shared__ uint32_t bitmap[];
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t ckey[kSelectCap];
  __shared__ int32_t cidx[kSelectCap];
  __shared__ int tmp[kSelThreads / 64 + 1];
  __shared__ int res[4];
  __shared__ int ccount;

  const int p = blockIdx.x, b = p / g.hkv, t = threadIdx.x;
  const int K = g.kappa;
  const int L = seq_len_of(g, b);
  const int n = pool ? clampi(ws.pool_len[p], 0, g.n_cap) : L;
  int32_t* o1 = out + (size_t)p * K;
  int32_t* o2 = out2 ? out2 + (size_t)p * K : nullptr;
  const int32_t* plist = ws.pool_pos + (size_t)p * g.n_cap;

  if (n <= K) {  // everything is selected (n == kappa for consistent inputs)
    for (int e = t; e < K; e += kSelThreads) {
      const int v = e < n ? (pool ? plist[e] : e) : -1;
      o1[e] = v;
      if (o2) o2[e] = v;
    }
    return;
  }

  const float* sc = ws.scores + (size_t)p * g.n_cap;
  const int words = (n + 31) >> 5;
  for (int i = t; i < words; i += kSelThreads) bitmap[i] = 0u;
  for (int i = t; i < kHistBins; i += kSelThreads) h[i] = ws.hist[(size_t)p * kHistBins + i];
  if (t == 0) ccount = 0;
  __syncthreads();

  find_bin<kHistBins>(h, K, res, tmp);
  const int tbin = res[0], need1 = K - res[1], inbin = res[2];
  if (tbin < 0) {  // histogram inconsistent with the list: only on corrupted workspace
    for (int e = t; e < K; e += kSelThreads) {
      o1[e] = -1;
      if (o2) o2[e] = -1;
    }
    return;
  }
  const bool fast = inbin <= kSelectCap;

  // Pass 1: lanes hold 4 consecutive entries, 8 lanes one 32-bit bitmap word.
  for (int base = 0; base < n; base += 4 * kSelThreads) {
    const int e0 = base + 4 * t;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (e0 < n) raw = *reinterpret_cast<const u32x4*>(sc + e0);
    uint32_t nib = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + c;
      if (e < n) {
        const uint32_t key = order_key(__uint_as_float(raw[c]));
        const int bin = (int)(key >> (32 - kHistBits));
        if (bin > tbin) {
          nib |= 1u << c;
        } else if (bin == tbin && fast) {
          const int slot = atomicAdd(&ccount, 1);
          if (slot < kSelectCap) {
            ckey[slot] = key;
            cidx[slot] = e;
          }
        }
      }
    }
    uint32_t word = nib << (4 * (t & 7));
    word |= __shfl_xor(word, 1);
    word |= __shfl_xor(word, 2);
    word |= __shfl_xor(word, 4);
    if ((t & 7) == 0 && e0 < n) bitmap[e0 >> 5] = word;
  }
  __syncthreads();

  uint32_t T;
  int need_eq, count_eq;
  if (fast) {
    const int nc = min(ccount, kSelectCap);
    for (int i = t; i < 1024; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (int c = t; c < nc; c += kSelThreads) atomicAdd(&h[(ckey[c] >> 10) & 1023u], 1u);
    __syncthreads();
    find_bin<1024>(h, need1, res, tmp);
    const uint32_t dA = (uint32_t)res[0];
    const int need2 = need1 - res[1];
    for (int i = t; i < 1024; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (int c = t; c < nc; c += kSelThreads)
      if (((ckey[c] >> 10) & 1023u) == dA) atomicAdd(&h[ckey[c] & 1023u], 1u);
    __syncthreads();
    find_bin<1024>(h, need2, res, tmp);
    T = ((uint32_t)tbin << 20) | (dA << 10) | (uint32_t)res[0];
    need_eq = need2 - res[1];
    count_eq = res[2];
    for (int c = t; c < nc; c += kSelThreads) {
      const uint32_t key = ckey[c];
      const int e = cidx[c];
      bool take = key > T;
      if (key == T) {
        if (count_eq == need_eq) {
          take = true;
        } else {  // rank among equal keys by list index
          int rank = 0;
          for (int c2 = 0; c2 < nc; ++c2) rank += (ckey[c2] == T && cidx[c2] < e) ? 1 : 0;
          take = rank < need_eq;
        }
      }
      if (take) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
  } else {
    // Threshold bin too large for LDS: resolve the low 20 bits over the list.
    for (int i = t; i < 1024; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (int e = t; e < n; e += kSelThreads) {
      const uint32_t key = order_key(sc[e]);
      if ((int)(key >> 20) == tbin) atomicAdd(&h[(key >> 10) & 1023u], 1u);
    }
    __syncthreads();
    find_bin<1024>(h, need1, res, tmp);
    const uint32_t prefix = ((uint32_t)tbin << 10) | (uint32_t)res[0];
    const int need2 = need1 - res[1];
    for (int i = t; i < 1024; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (int e = t; e < n; e += kSelThreads) {
      const uint32_t key = order_key(sc[e]);
      if ((key >> 10) == prefix) atomicAdd(&h[key & 1023u], 1u);
    }
    __syncthreads();
    find_bin<1024>(h, need2, res, tmp);
    T = (prefix << 10) | (uint32_t)res[0];
    need_eq = need2 - res[1];
    count_eq = res[2];
    int run = 0;  // equal keys seen in earlier chunks
    for (int base = 0; base < n; base += kSelThreads) {
      const int e = base + t;
      const bool valid = e < n;
      const uint32_t key = valid ? order_key(sc[e]) : 0u;
      const bool gt = valid && key > T && (int)(key >> 20) == tbin;
      const bool eq = valid && key == T;
      int tot;
      const int r = block_excl_scan<kSelThreads>(eq ? 1 : 0, tmp, &tot);
      if (gt || (eq && run + r < need_eq)) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
      run += tot;
    }
  }
  (void)count_eq;
  __syncthreads();

  // Emission in bitmap order = ascending position.
  const int wpt = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(words, t * wpt), w1 = min(words, w0 + wpt);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(bitmap[i]);
  int total;
  int o = block_excl_scan<kSelThreads>(cnt, tmp, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t m = bitmap[i];
    while (m) {
      const int e = i * 32 + (__ffs(m) - 1);
      m &= m - 1u;
      if (o < K) {
        const int v = pool ? plist[e] : e;
        o1[o] = v;
        if (o2) o2[o] = v;
      }
      ++o;
    }
  }
  for (int e = total + t; e < K; e += kSelThreads) {
    o1[e] = -1;
    if (o2) o2[e] = -1;
  }
}

// ---------------------------------------------------------------------------
// SparseAttn over one split of kAttnSplit selected tokens of one (sequence,
// KV head), all G query heads.  Logits by MFMA as in scoring; the split's
// softmax statistics (max, sum of exponentials) and unnormalised output are
// written for the combine kernel.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void attn_kernel(Geometry g, Workspace ws,
                                                   const uint16_t* __restrict__ q,
                                                   const int32_t* __restrict__ idx, float scale) {
  __shared__ float lg[G][kAttnSplit];
  __shared__ float red[4][G][kHeadDim];
  __shared__ float sm[G], sl[G];
  const int splits = g.splits;
  const int p = blockIdx.x / splits, s = blockIdx.x - p * splits;
  const int b = p / g.hkv, kvh = p - b * g.hkv;
  const int L = seq_len_of(g, b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4;

  const int t = s * kAttnSplit + wave * 16 + j;
  int pos = t < g.kappa ? idx[(size_t)p * g.kappa + t] : -1;
  const bool valid = pos >= 0 && pos < L;
  if (!valid) pos = 0;
  const size_t roff = row_offset(g, b, kvh, pos);

  u32x4 kf[4];
  const u32x4* krow = reinterpret_cast<const u32x4*>(g.k_pages + roff);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) kf[s4] = krow[g4 + 4 * s4];
  uint32_t vv[16];
  const uint32_t lo = (uint32_t)roff, hi = (uint32_t)(roff >> 32);
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const size_t o = (size_t)(uint32_t)__shfl((int)lo, jj) |
                     ((size_t)(uint32_t)__shfl((int)hi, jj) << 32);
    vv[jj] = reinterpret_cast<const uint32_t*>(g.v_pages + o)[lane];
  }
  u32x4 qf[4];
  load_q_frag<G>(q, g, b, kvh, lane, qf);

  const f32x4 acc = qk_tile(qf, kf);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * g4 + r;
    if (i < G) lg[i][wave * 16 + j] = valid ? acc[r] * scale : -INFINITY;
  }
  __syncthreads();
  for (int i = wave; i < G; i += 4) {
    const float z = lg[i][lane];
    const float m = wave_max(z);
    const float e = (z == -INFINITY) ? 0.f : __expf(z - m);
    const float l = wave_sum(e);
    lg[i][lane] = e;
    if (lane == 0) {
      sm[i] = m;
      sl[i] = l;
    }
  }
  __syncthreads();
  float o0[G], o1[G];
#pragma unroll
  for (int i = 0; i < G; ++i) o0[i] = o1[i] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float v0 = __uint_as_float(vv[jj] << 16);
    const float v1 = __uint_as_float(vv[jj] & 0xffff0000u);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float pw = lg[i][wave * 16 + jj];
      o0[i] += pw * v0;
      o1[i] += pw * v1;
    }
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    red[wave][i][2 * lane] = o0[i];
    red[wave][i][2 * lane + 1] = o1[i];
  }
  __syncthreads();
  float* po = ws.part_o + ((size_t)p * splits + s) * G * kHeadDim;
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int i = o / kHeadDim, d = o - i * kHeadDim;
    po[o] = (red[0][i][d] + red[1][i][d]) + (red[2][i][d] + red[3][i][d]);
  }
  if (threadIdx.x < G) {
    float* pm = ws.part_ml + (((size_t)p * splits + s) * G + threadIdx.x) * 2;
    pm[0] = sm[threadIdx.x];
    pm[1] = sl[threadIdx.x];
  }
}

// Merge of the splits in split order (deterministic, no float atomics).
template <int G>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(Geometry g, Workspace ws, float* out) {
  const int bq = blockIdx.x, b = bq / g.hq, h = bq - b * g.hq;
  const int kvh = h / G, i = h - kvh * G;
  const int p = b * g.hkv + kvh, d = threadIdx.x, splits = g.splits;
  const float* pml = ws.part_ml + (size_t)p * splits * G * 2;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pml[(s * G + i) * 2]);
  float lsum = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float ms = pml[(s * G + i) * 2];
      if (ms == -INFINITY) continue;
      const float f = __expf(ms - M);
      lsum += pml[(s * G + i) * 2 + 1] * f;
      o += ws.part_o[(((size_t)p * splits + s) * G + i) * kHeadDim + d] * f;
    }
  }
  out[((size_t)b * g.hq + h) * kHeadDim + d] = lsum > 0.f ? o / lsum : 0.f;
}

size_t select_lds_bytes(const Geometry& g) { return (size_t)(g.n_cap / 32) * sizeof(uint32_t); }

}  // namespace

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
namespace {

struct ProfileRing {
  std::vector<hipEvent_t> starts, stops;
  int64_t launches = 0;
};
ProfileRing g_profile[kKernelKinds];

// Launches `kernel`; if the kind has an event ring, the dispatch records the
// ring's next pair at kernel start and end.
template <typename... KArgs, typename... Args>
void launch(int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
            Args... args) {
  ProfileRing& r = g_profile[kind];
  if (!r.starts.empty()) {
    const size_t i = (size_t)(r.launches++ % (int64_t)r.starts.size());
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, r.starts[i], r.stops[i], 0,
                          static_cast<KArgs>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
  }
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

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(const Geometry& g) {
  const size_t P = (size_t)g.problems();
  size_t o = 0;
  o += align256(P * kHistBins * 4);
  o += align256(P * (size_t)g.n_cap * 4);
  o += align256(P * (size_t)g.n_cap * 4);
  o += align256(P * 4);
  o += align256(P * (size_t)g.kappa * 4);
  o += align256(P * (size_t)g.splits * g.group * kHeadDim * 4);
  o += align256(P * (size_t)g.splits * g.group * 2 * 4);
  return o;
}

Workspace carve_workspace(void* base, const Geometry& g) {
  const size_t P = (size_t)g.problems();
  char* c = static_cast<char*>(base);
  Workspace w;
  w.hist = reinterpret_cast<uint32_t*>(c);
  c += align256(P * kHistBins * 4);
  w.scores = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)g.n_cap * 4);
  w.pool_pos = reinterpret_cast<int32_t*>(c);
  c += align256(P * (size_t)g.n_cap * 4);
  w.pool_len = reinterpret_cast<int32_t*>(c);
  c += align256(P * 4);
  w.idx_tmp = reinterpret_cast<int32_t*>(c);
  c += align256(P * (size_t)g.kappa * 4);
  w.part_o = reinterpret_cast<float*>(c);
  c += align256(P * (size_t)g.splits * g.group * kHeadDim * 4);
  w.part_ml = reinterpret_cast<float*>(c);
  return w;
}

hipError_t launch_zero_hist(const Geometry& g, const Workspace& w, hipStream_t s) {
  launch(kHistReset, zero_hist_kernel, dim3(g.problems()), dim3(256), 0, s, w.hist);
  return hipGetLastError();
}

hipError_t launch_pool_plan(const Geometry& g, const Workspace& w, const int32_t* anchor_idx,
                            hipStream_t s) {
  const size_t lds = (size_t)2 * g.kappa * sizeof(int32_t);
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(pool_plan_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)((size_t)2 * kMaxKappa * sizeof(int32_t)));
    attr_done = true;
  }
  launch(kPoolPlan, pool_plan_kernel, dim3(g.problems()), dim3(256), lds, s, g, w, anchor_idx);
  return hipGetLastError();
}

template <int G>
static void launch_score_g(const Geometry& g, const Workspace& w, const uint16_t* q, bool pool,
                           hipStream_t s) {
  const int chunks = (g.n_cap + kScoreChunk - 1) / kScoreChunk;
  launch(pool ? kPoolScore : kAnchorScore, score_kernel<G>, dim3(g.problems() * chunks), dim3(256),
         0, s, g, w, q, chunks, pool ? 1 : 0);
}

hipError_t launch_score(const Geometry& g, const Workspace& w, const uint16_t* q, bool pool,
                        hipStream_t s) {
  switch (g.group) {
    case 1: launch_score_g<1>(g, w, q, pool, s); break;
    case 2: launch_score_g<2>(g, w, q, pool, s); break;
    case 4: launch_score_g<4>(g, w, q, pool, s); break;
    case 8: launch_score_g<8>(g, w, q, pool, s); break;
    case 16: launch_score_g<16>(g, w, q, pool, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select(const Geometry& g, const Workspace& w, bool pool, int32_t* out,
                         int32_t* out2, hipStream_t s) {
  const size_t lds = select_lds_bytes(g);
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)((size_t)kMaxSeqLen / 32 * sizeof(uint32_t)));
    attr_done = true;
  }
  launch(kSelect, select_kernel, dim3(g.problems()), dim3(kSelThreads), lds, s, g, w, pool ? 1 : 0,
         out, out2);
  return hipGetLastError();
}

template <int G>
static void launch_attention_g(const Geometry& g, const Workspace& w, const uint16_t* q,
                               const int32_t* idx, float scale, float* out, hipStream_t s) {
  launch(kAttention, attn_kernel<G>, dim3(g.problems() * g.splits), dim3(256), 0, s, g, w, q, idx,
         scale);
  launch(kCombine, combine_kernel<G>, dim3(g.batch * g.hq), dim3(kHeadDim), 0, s, g, w, out);
}

hipError_t launch_attention(const Geometry& g, const Workspace& w, const uint16_t* q,
                            const int32_t* idx, float scale, float* out, hipStream_t s) {
  switch (g.group) {
    case 1: launch_attention_g<1>(g, w, q, idx, scale, out, s); break;
    case 2: launch_attention_g<2>(g, w, q, idx, scale, out, s); break;
    case 4: launch_attention_g<4>(g, w, q, idx, scale, out, s); break;
    case 8: launch_attention_g<8>(g, w, q, idx, scale, out, s); break;
    case 16: launch_attention_g<16>(g, w, q, idx, scale, out, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace prism

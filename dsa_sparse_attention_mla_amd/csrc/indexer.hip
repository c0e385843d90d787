// DSA indexer with a running top-k ("Sparse prefill for GLM", section "Blocked
// top-k": keys are scored a block at a time and folded into a running top-k
// list, so the full batch x heads x L x N score tensor is never built).
//
// Score (the pages print none; the library uses)
//     s[i, n] = sum_h w[i, h] * ReLU(q[i, h, :] . k[n, :]),   visible iff n <= N - L + i,
// and the result is the EXACT top-k set of the canonical fp64 score (dot products
// summed in ascending dim order, head terms added in ascending head order, no
// fused multiply-add), ties to the lower key index.
//
// Pipeline, all on the caller's stream:
//  1. key_norm_partial:   per-block max of ||k_n|| (squares summed in fp64, so no
//                         bf16 key overflows or underflows it).
//  2. query_eps:          eps_i, a rigorous bound on |s_hat - s| for the fp32
//                         MFMA score s_hat, from sum_h |w_h| ||q_h|| * max_n ||k_n||.
//  3. one score kernel, both with 32x32x16 bf16 MFMA scores for 32 heads and the
//     ReLU, weight and head sum in registers; only candidates leave the chip:
//     score_list (long contexts: every query of a group sees at least 8 * SAMPLE
//                         keys): the workgroup scores S keys (SAMPLE, or
//                         SAMPLE_SMALL where the lists have room for the looser
//                         start) spread over the visible range, fixes each query's
//                         threshold just below
//                         the sample's expected k-th largest, streams its key split
//                         and appends every key at or above the threshold to the
//                         query's list in memory (no list on chip, no compaction).
//     score_filter (short contexts): every wave owns one query and keeps a
//                         candidate list in LDS of all keys with
//                         s_hat >= tau - band(tau), tau = the running k-th largest
//                         s_hat (found by an in-LDS radix select whenever the list
//                         fills up), i.e. a running top-k folded tile by tile.
//  4. select_refine:      per query, T = k-th largest s_hat among candidates, after
//                         a coverage check (every split's threshold at most
//                         T - band: the lists then hold the whole top-k).
//                         s_hat > T + band: in. s_hat < T - band: out. The keys in
//                         between are re-scored canonically in fp64 and ranked by
//                         (s desc, index asc) to fill the rest.
//  5. exact_fallback:     rows that failed the coverage check or whose lists
//                         overflowed (huge ties, a sampled threshold set badly), and
//                         rows whose magnitudes could overflow the fp32 scores (eps
//                         = +inf), are solved from the canonical fp64 score of every
//                         visible key.
// Output rows are in ascending key order, padded with -1.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int ID = 128;                 // indexer head dim
constexpr int IH = 32;                  // indexer heads
constexpr int TK = 256;                 // keys per tile of the score kernel
constexpr int IDX_STAGE = TK * ID * 2;  // the LDS key stage: 256 keys x 256 B (swizzled, unpadded)
constexpr int QPB = 4;                  // queries per workgroup
constexpr int IDX_NW = 8;               // waves per score workgroup: 2 per query
constexpr int SAMPLE = 2048;            // keys scored up front to start the filter threshold
constexpr int SAMPLE_SMALL = 1024;      // the list kernel's smaller sample, where its lists have room
constexpr int RANK_WORDS = 4096;        // bitmap words for ordering the output (131072 keys per window)
static_assert(RANK_WORDS * 4 >= 64 * IH * 8, "band dots alias the word-prefix table");
constexpr int BAND_CAP = 256;           // band entries re-scored and ranked in select_refine
constexpr int BIN_CAP = 1024;           // entries of the threshold bin ranked in select_refine
constexpr int SR_T = 512;               // threads of a select_refine workgroup (one query)
constexpr int SR_W = SR_T / 64;         // its waves
constexpr int SR_J = 24;                // candidates per thread (in registers) in select_refine
constexpr int SR_MAX = SR_J * SR_T;     // candidates per query select_refine holds
constexpr int NORM_BLOCKS = 1024;
constexpr int FB_ROWS = 256;            // block size of the fallback kernel
constexpr int FB_BLOCKS = 256;          // fallback workgroups: one per compute unit
#ifndef FB_CHUNK
#define FB_CHUNK 16                     // key dims converted to fp64 at a time in the fallback
#endif
static_assert(FB_CHUNK % 8 == 0 && ID % FB_CHUNK == 0, "whole 16-byte key loads per chunk");
}  // namespace

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Half-width of the uncertainty band around a threshold t (of either sign): 2*eps
// plus a few ulps of t for the fp32 evaluation of t +- 2*eps. Its slope in t is
// below 1 in magnitude, so t1 <= t2 implies t1 - band(t1) <= t2 - band(t2).
__device__ __forceinline__ float band_halfwidth(float eps, float t) {
  return 2.0f * eps * 1.001f + fabsf(t) * 4.8e-7f;
}

// ---------------------------------------------------------------- 1. key norms
__global__ __launch_bounds__(256) void key_norm_partial_kernel(const uint16_t* __restrict__ k, int N,
                                                               float* __restrict__ partial) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid >> 4, l16 = tid & 15;   // 16 keys per pass, 16 lanes per key
  constexpr int U = 8;                        // passes in flight per thread
  double mx = 0.0;                            // largest squared norm of this thread's keys
  const int stride = gridDim.x * 16;
  for (int n0 = blockIdx.x * 16 + sub; n0 < N; n0 += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * stride;
      v[u] = n < N ? *(const u32x4*)(k + (size_t)n * ID + 8 * l16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = bf_bits2f((uint16_t)(v[u][e] & 0xFFFFu)), b = bf_bits2f((uint16_t)(v[u][e] >> 16));
        acc = __fma_rn(a, a, acc);
        acc = __fma_rn(b, b, acc);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
      mx = fmax(mx, acc);
    }
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) mx = fmax(mx, __shfl_xor(mx, off));
  // the norm, rounded up into fp32 (+inf past its range)
  if (lane == 0) red[wave] = (float)(sqrt(mx) * (1.0 + 0x1p-20));
  __syncthreads();
  if (tid == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------- 2. eps per query
// |fl(q.k) - q.k| <= gamma_128 * sum|q_c k_c| <= gamma_128 ||q|| ||k|| (any order,
// round-to-nearest or toward zero: u = 2^-23); the ReLU is 1-Lipschitz; the
// weight product and the 32-term head sum add (u + gamma_32) * sum_h |w_h| |d_h|
// (weights of either sign).
// The constant below is that sum (1.92e-5) with a 30% margin. The norms are
// summed in fp64, so they neither overflow nor underflow for any bf16 input; an
// absolute term covers fp32 results below the normal range, which the matrix unit
// may flush (at most 2^-126 per product, partial sum or weighted head term:
// below 2^-117 * (sum_h |w_h| + 1) per score).
// Inputs whose fp32 score could overflow (max_h ||q_h|| max ||k|| or
// sum_h |w_h| ||q_h|| max ||k|| at or past 2^120, or non-finite) get eps = +inf,
// which sends the query to the exact fallback.
__global__ __launch_bounds__(64) void query_eps_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                       const float* __restrict__ partial, int nparts, int L,
                                                       float* __restrict__ eps) {
  const int i = blockIdx.x, lane = threadIdx.x;
  float km = 0.f;                                 // max_n ||k_n|| (rounded up)
  {
    // all of this lane's partial maxima in flight at once (nparts = NORM_BLOCKS)
    constexpr int PPL = NORM_BLOCKS / 64;
    float pv[PPL];
#pragma unroll
    for (int x = 0; x < PPL; ++x) pv[x] = lane + 64 * x < nparts ? partial[lane + 64 * x] : 0.f;
#pragma unroll
    for (int x = 0; x < PPL; ++x) km = fmaxf(km, pv[x]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) km = fmaxf(km, __shfl_xor(km, off));
  if (km != km) km = INFINITY;                    // (a NaN partial cannot occur; be safe)
  double contrib = 0.0, qn = 0.0, aw = 0.0;      // |w_h| ||q_h||, ||q_h||, |w_h|
  if (lane < IH) {
    const uint16_t* qh = q + ((size_t)i * IH + lane) * ID;
    u32x4 v[ID / 8];
#pragma unroll
    for (int c = 0; c < ID / 8; ++c) v[c] = *(const u32x4*)(qh + 8 * c);
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < ID / 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = bf_bits2f((uint16_t)(v[c][e] & 0xFFFFu)), b = bf_bits2f((uint16_t)(v[c][e] >> 16));
        acc = __fma_rn(a, a, acc);
        acc = __fma_rn(b, b, acc);
      }
    qn = sqrt(acc) * (1.0 + 0x1p-20);
    aw = fabs((double)w[(size_t)i * IH + lane]);
    contrib = aw * qn;
  }
  double qmax = qn;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    contrib += __shfl_xor(contrib, off);
    aw += __shfl_xor(aw, off);
    qmax = fmax(qmax, __shfl_xor(qmax, off));
  }
  if (lane == 0) {
    const double kmd = km, bound = contrib * kmd;
    const bool safe = bound < 0x1p120 && qmax * kmd < 0x1p120;   // false for +inf and NaN too
    eps[i] = safe ? (float)(2.5e-5 * bound * 1.0002) + (float)((aw + 1.0) * 0x1p-117) + 1e-30f : INFINITY;
  }
}

// ---------------------------------------------------------------- 3. score + running candidates
// Wave-wide reduction with an associative, commutative op, every lane getting the
// result: DPP exchanges within each row of 16 lanes (xor 1, xor 2, half-row mirror,
// row mirror), then the permlane swaps across rows 16 and 32 lanes apart. All VALU:
// no LDS round trips.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_bits(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(b[0], b[1]);
}
__device__ __forceinline__ float wave_max(float x) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(x), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_min(float x) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(x), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ int wave_sum_int(int x) {
  return (int)wave_reduce_bits((uint32_t)x, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_bits(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce_bits(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Bucket of x in a 256-bin linear histogram over [mn, mx]; non-decreasing in x.
__device__ __forceinline__ int lin_bucket(float x, float mn, float inv_w) {
  const float f = fminf(fmaxf((x - mn) * inv_w, 0.f), 255.f);   // fmaxf also maps NaN to 0
  return (int)f;
}

// Given a 256-bin histogram (higher bin = larger values), find the bin B holding
// the need-th largest entry: returns B and the number of entries in bins above B.
// Executed by one wave (lane = 0..63, 4 bins per lane).
__device__ __forceinline__ void wave_find_bin(const int* hist, int need, int lane, int& bin, int& above_bin) {
  const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const int own = h0 + h1 + h2 + h3;
  int suf = own;  // inclusive suffix sum over lanes (higher lanes hold higher bins)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_down(suf, off);
    if (lane + off < 64) suf += v;
  }
  const int above = suf - own;
  const bool here = above < need && suf >= need;
  int digit = 0, above_d = 0;
  if (here) {
    int acc = above;
    if (acc + h3 >= need) { digit = 4 * lane + 3; above_d = acc; }
    else { acc += h3;
      if (acc + h2 >= need) { digit = 4 * lane + 2; above_d = acc; }
      else { acc += h2;
        if (acc + h1 >= need) { digit = 4 * lane + 1; above_d = acc; }
        else { acc += h1; digit = 4 * lane; above_d = acc; } } }
  }
  const unsigned long long bm = __ballot(here);
  const int src = __ffsll((long long)bm) - 1;
  bin = __shfl(digit, src);
  above_bin = __shfl(above_d, src);
}

// Block-wide helpers for the 512-thread score workgroup.
__device__ __forceinline__ float block512_max(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_max(x);
  if (lane == 0) red[wave] = x;
  lds_barrier();
  float r = red[0];
#pragma unroll
  for (int v = 1; v < IDX_NW; ++v) r = fmaxf(r, red[v]);
  lds_barrier();
  return r;
}
__device__ __forceinline__ float block512_min(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_min(x);
  if (lane == 0) red[wave] = x;
  lds_barrier();
  float r = red[0];
#pragma unroll
  for (int v = 1; v < IDX_NW; ++v) r = fminf(r, red[v]);
  lds_barrier();
  return r;
}

// Threshold update and in-place compaction of the candidate lists of the queries
// flagged in `mine`, all queries at once. A query's list has two segments, owned by
// its two waves: the front wave (kh = 0) keeps its entries at [0, n0), the back wave
// (kh = 1) at [CAPS - n1, CAPS). Each wave scans only its own segment; partial
// results (min / max, the shared 256-bin linear histogram, the minimum inside the
// bin of the k-th largest) meet in LDS at three workgroup barriers that every wave
// takes. tau = that minimum is a lower bound of the list's k-th largest score; each
// wave then keeps its entries with score >= max(old threshold, tau - band(tau)),
// compacting them toward its own end (a destination never passes the entry being
// read, so the in-place moves are safe). Returns this wave's new segment count.
// The caller guarantees that a flagged list holds at least k entries.
template <typename Off, int CAPS, int NQ = QPB>
__device__ int pair_compact(float* cs, Off* co, int mycnt, int kh, bool mine, int k, float eps, float& thr,
                            int* hq, float* red, bool compact = true) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, partner = wave ^ NQ;
  auto seg = [&](int e) { return kh == 0 ? e : CAPS - 1 - e; };
  if (mine) {
    float mx = -INFINITY, mn = INFINITY;
    for (int e = lane; e < mycnt; e += 64) {
      const float v = cs[seg(e)];
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
    mx = wave_max(mx);
    mn = wave_min(mn);
    if (lane == 0) {
      red[2 * wave] = mx;
      red[2 * wave + 1] = mn;
    }
    if (kh == 0)
      for (int b = lane; b < 256; b += 64) hq[b] = 0;
  }
  lds_barrier();
  float qmx = -INFINITY, qmn = INFINITY;
  if (mine) {
    qmx = fmaxf(red[2 * wave], red[2 * partner]);
    qmn = fminf(red[2 * wave + 1], red[2 * partner + 1]);
  }
  const bool spread = qmx > qmn;
  const float inv_w = spread ? 256.0f / (qmx - qmn) : 0.f;
  if (mine && spread)
    for (int e = lane; e < mycnt; e += 64) atomicAdd(&hq[lin_bucket(cs[seg(e)], qmn, inv_w)], 1);
  lds_barrier();
  if (mine && spread) {
    int bin, above;
    wave_find_bin(hq, k, lane, bin, above);   // both waves of the query find the same bin
    float tb = INFINITY;
    for (int e = lane; e < mycnt; e += 64) {
      const float v = cs[seg(e)];
      if (lin_bucket(v, qmn, inv_w) == bin) tb = fminf(tb, v);
    }
    tb = wave_min(tb);
    if (lane == 0) red[2 * wave] = tb;
  }
  lds_barrier();
  if (!mine) return mycnt;
  const float tau = spread ? fminf(red[2 * wave], red[2 * partner]) : qmn;
  thr = fmaxf(thr, tau - band_halfwidth(eps, tau));
  if (!compact) return mycnt;
  int outc = 0;
  for (int c0 = 0; c0 < mycnt; c0 += 64) {
    const int e = c0 + lane;
    const bool in = e < mycnt;
    const int ps = seg(in ? e : c0);
    const float v = cs[ps];
    const Off id = co[ps];
    const bool keep = in && v >= thr;
    const unsigned long long bm = __ballot(keep);
    if (keep) {
      const int dst = seg(outc + __popcll(bm & ((1ull << lane) - 1ull)));
      cs[dst] = v;
      co[dst] = id;
    }
    outc += __popcll(bm);
  }
  return outc;
}

// Largest candidate capacity per query that fits the LDS next to the key stage.
template <typename Off>
struct FilterCap {
  static constexpr int value =
      (int)(((163840 - IDX_STAGE - QPB * 256 * 4 - 8 * QPB * 4 - 2 * IDX_NW * 4) / (QPB * (4 + sizeof(Off)))) / 64 * 64);
};

// Key tiles (256 keys x 256 B) are fetched into registers one tile ahead of use
// (eight 16-byte loads per thread) and written into the single LDS stage once
// every wave has finished reading the previous tile. Within the stage, key r's
// 16-byte chunk c sits at chunk slot r*16 + (c ^ (r & 15)), so the 32 keys one
// MFMA operand read touches fall in distinct banks.
// Eight waves: wave w scores query w%4 against keys [128h, 128h+128) of every
// tile, h = w/4, as four independent 32-key MFMA chains (two pairs), so two
// waves share each SIMD with plenty of independent work between barriers.
// A query's two waves append survivors (score, key offset within the split) to
// the query's LDS list from opposite ends, each tracking its own count. When a
// list nears capacity at a tile boundary, the whole workgroup recomputes that
// query's threshold from the list and compacts it.
template <typename Off>
__global__ __launch_bounds__(64 * IDX_NW) void score_filter_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ eps_in, int L, int N, int topk, int span, int nsplit, int cap,
    float* __restrict__ cand_s, int* __restrict__ cand_i, int* __restrict__ cand_n, float* __restrict__ cand_t) {
  constexpr int CAPS = FilterCap<Off>::value;
  constexpr int PER_WAVE = TK / 2;      // keys per wave per tile (128)
  constexpr int MARGIN = 2 * PER_WAVE + 64;   // room for one tile's appends plus slack
  constexpr int CPT = TK * 16 / 512;    // 16-byte chunks per thread per tile (8)
  __shared__ __attribute__((aligned(16))) unsigned char stage[IDX_STAGE];
  __shared__ float cs_all[QPB * CAPS];
  __shared__ Off co_all[QPB * CAPS];
  __shared__ int hist[QPB * 256];
  __shared__ __attribute__((aligned(16))) int qlo[QPB];   // entries at the low end, written by wave h=0
  __shared__ __attribute__((aligned(16))) int qhi[QPB];   // entries at the high end, written by wave h=1
  __shared__ __attribute__((aligned(16))) int qovf[QPB];
  __shared__ float qthr[QPB];
  __shared__ float qeps[QPB];
  __shared__ float red[2 * IDX_NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave & (QPB - 1), kh = wave / QPB;
  const int split = blockIdx.y;
  const int n_lo = split * span;
  const int i = blockIdx.x * QPB + qi;
  const bool active = i < L;
  const int ii = active ? i : L - 1;
  const int p = N - L + ii;
  const int ilast = min(L - 1, (int)blockIdx.x * QPB + QPB - 1);
  const int n_hi = min(min(N, n_lo + span), N - L + ilast + 1);
  float* cs = cs_all + qi * CAPS;      // cap (<= CAPS) is the list capacity the refine step sizes for
  Off* co = co_all + qi * CAPS;

  bf16x8 qa[ID / 16];
  {
    const uint16_t* qrow = q + ((size_t)ii * IH + (lane & 31)) * ID + 8 * (lane >> 5);
#pragma unroll
    for (int kc = 0; kc < ID / 16; ++kc) qa[kc] = *(const bf16x8*)(qrow + 16 * kc);
  }
  float wr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wr[j] = w[(size_t)ii * IH + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)];
  // Consume the fragments and weights here, so their loads are known complete before the
  // tile loop; otherwise the loop's merged wait state would drain the key prefetch.
#pragma unroll
  for (int kc = 0; kc < ID / 16; ++kc) asm volatile("" ::"v"(qa[kc]));
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(wr[j]));
  if (tid < QPB) {
    qlo[tid] = 0;
    qhi[tid] = 0;
    qovf[tid] = 0;
    qthr[tid] = -INFINITY;
    qeps[tid] = eps_in[min((int)blockIdx.x * QPB + tid, L - 1)];
  }
  int mycnt = 0;                        // this wave's entries in its segment (uniform)

  // thread tid fetches chunk slots tid + 512u (u < CPT) of a tile: key r = slot / 16,
  // chunk c = (slot % 16) ^ (r % 16), stored at the slot. Every fetch issues all its
  // loads, also past the last tile (clamped rows, never staged), so the number of
  // outstanding loads is the same on every path and the compiler's waits stay exact.
  u32x4 pf[CPT];
  auto fetch = [&](int t) {
    const int n0 = n_lo + t * TK;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int slot = tid + 512 * u;
      const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
      const int n = min(n0 + r, n_hi - 1);
      pf[u] = *(const u32x4*)(k + (size_t)n * ID + c * 8);
    }
  };
  auto stage_in = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) *(u32x4*)(stage + (tid + 512 * u) * 16) = pf[u];
  };

  // two 32-key MFMA chains: scores of keys r0 + lane (lanes < 32) and r0 + 32 + (lane - 32)
  auto score_pair = [&](int r0) -> float {
    const int ra = r0 + (lane & 31), rb = ra + 32;
    bf16x8 ka[ID / 16], kb[ID / 16];
#pragma unroll
    for (int kc = 0; kc < ID / 16; ++kc) {
      const int c = 2 * kc + (lane >> 5);
      ka[kc] = *(const bf16x8*)(stage + ra * 256 + ((c ^ (ra & 15)) * 16));
      kb[kc] = *(const bf16x8*)(stage + rb * 256 + ((c ^ (rb & 15)) * 16));
    }
    f32x16 acca = {}, accb = {};
#pragma unroll
    for (int kc = 0; kc < ID / 16; ++kc) {
      acca = mfma32x32x16(qa[kc], ka[kc], acca);
      accb = mfma32x32x16(qa[kc], kb[kc], accb);
    }
    // ReLU as an integer max on the bit pattern (exact for every non-NaN float, -0 -> +0),
    // then the weighted head sums
    float pa = 0.f, pb = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      pa = fmaf(wr[j], __int_as_float(max(__float_as_int(acca[j]), 0)), pa);
      pb = fmaf(wr[j], __int_as_float(max(__float_as_int(accb[j]), 0)), pb);
    }
    // lanes l and l^32 hold the two head halves of one key: lanes < 32 get key l of the
    // first chain (pa), lanes >= 32 key l-32 of the second (pb)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  };

  // Sampling prologue. SAMPLE keys spread evenly over the keys that every query of
  // the group sees are scored first; each query's threshold starts just below the
  // r-th largest sample score, r six standard deviations above the expected number
  // of sample keys in the top-k. That start is an estimate, not a bound: the refine
  // step checks that every list covers the band around the final k-th score and
  // sends the query to the exact fallback otherwise. With few visible keys the
  // threshold starts at -inf, a bound by construction.
  {
    const int nv_min = min(N, N - L + (int)blockIdx.x * QPB + 1);
    const float mean = (float)topk * SAMPLE / (float)max(nv_min, 1);
    if (nv_min >= 8 * SAMPLE && mean <= SAMPLE / 8 && SAMPLE <= cap) {
      const int rk = min(SAMPLE / 2, (int)ceilf(mean + 6.f * sqrtf(mean) + 8.f));
      for (int t = 0; t < SAMPLE / TK; ++t) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int slot = tid + 512 * u;
          const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
          const int n = (int)((long long)(t * TK + r) * nv_min / SAMPLE);
          pf[u] = *(const u32x4*)(k + (size_t)n * ID + c * 8);
        }
        lds_barrier();                  // previous sample tile fully read
        stage_in();
        lds_barrier();
        const int r0 = PER_WAVE * kh;
        const float sv0 = score_pair(r0), sv1 = score_pair(r0 + 64);
        if (active) {                   // every score goes to the list; key ids are not needed
          cs[kh == 0 ? mycnt + lane : CAPS - 1 - (mycnt + lane)] = sv0;
          cs[kh == 0 ? mycnt + 64 + lane : CAPS - 65 - (mycnt + lane)] = sv1;
          mycnt += 128;
        }
      }
      lds_barrier();
      float thr_q = -INFINITY;
      pair_compact<Off, CAPS>(cs, co, mycnt, kh, active, rk, qeps[qi], thr_q, hist + qi * 256, red, false);
      mycnt = 0;
      if (active && kh == 0 && lane == 0) qthr[qi] = thr_q;
      lds_barrier();
    }
  }

  const int ntiles = n_hi > n_lo ? (n_hi - n_lo + TK - 1) / TK : 0;
  if (ntiles > 0) {
    fetch(0);
    stage_in();
    fetch(1);
  }
  for (int t = 0; t < ntiles; ++t) {
    const int n0 = n_lo + t * TK;
    // Barrier 1 publishes tile t and the previous tile's appends and counts; until
    // barrier 2 no count changes except inside the cooperative compaction, which
    // publishes them only after barriers every wave reaches, so all waves take the
    // same decisions. After barrier 2 the stage is free: survivors are appended,
    // tile t+1 moves in from registers and the registers fetch tile t+2.
    lds_barrier();
    const int4 vlo = *(const int4*)qlo, vhi = *(const int4*)qhi, vov = *(const int4*)qovf;
    const int need = ((vlo.x + vhi.x > cap - MARGIN) && !vov.x) | (((vlo.y + vhi.y > cap - MARGIN) && !vov.y) << 1) |
                     (((vlo.z + vhi.z > cap - MARGIN) && !vov.z) << 2) | (((vlo.w + vhi.w > cap - MARGIN) && !vov.w) << 3);
    bool ovf_now = false;
    if (need) {
      const bool mine = (need >> qi) & 1;
      float thr_q = qthr[qi];
      const int newc = pair_compact<Off, CAPS>(cs, co, mycnt, kh, mine, topk, qeps[qi], thr_q, hist + qi * 256, red);
      if (mine) {
        mycnt = newc;
        if (lane == 0) {
          if (kh == 0) {
            qlo[qi] = newc;
            qthr[qi] = thr_q;
          } else {
            qhi[qi] = newc;
          }
        }
      }
      lds_barrier();
      if (mine) {
        ovf_now = qlo[qi] + qhi[qi] > cap - MARGIN;
        if (kh == 0 && lane == 0) qovf[qi] = ovf_now;
      }
    }
    const float thr = qthr[qi];
    const bool ovf = ovf_now || qovf[qi] != 0;

    const int r0 = PER_WAVE * kh;
    const float sv0 = score_pair(r0);
    const float sv1 = score_pair(r0 + 64);
    const int key0 = n0 + r0 + lane, key1 = key0 + 64;
    const bool keep0 = active && !ovf && key0 < n_hi && key0 <= p && sv0 >= thr;
    const bool keep1 = active && !ovf && key1 < n_hi && key1 <= p && sv1 >= thr;
    lds_barrier();
    const unsigned long long bm0 = __ballot(keep0), bm1 = __ballot(keep1);
    if (bm0 | bm1) {
      const int b0 = __popcll(bm0);
      const int before0 = __popcll(bm0 & ((1ull << lane) - 1ull));
      const int before1 = b0 + __popcll(bm1 & ((1ull << lane) - 1ull));
      if (keep0) {
        const int pos = kh == 0 ? mycnt + before0 : CAPS - 1 - (mycnt + before0);
        cs[pos] = sv0;
        co[pos] = (Off)(key0 - n_lo);
      }
      if (keep1) {
        const int pos = kh == 0 ? mycnt + before1 : CAPS - 1 - (mycnt + before1);
        cs[pos] = sv1;
        co[pos] = (Off)(key1 - n_lo);
      }
      mycnt += b0 + __popcll(bm1);
      if (lane == 0) {
        if (kh == 0) qlo[qi] = mycnt;
        else qhi[qi] = mycnt;
      }
    }
    if (t + 1 < ntiles) stage_in();
    fetch(t + 2);
  }
  lds_barrier();
  if (active) {
    const size_t slot = (size_t)i * nsplit + split;
    const int lo = qlo[qi], hi = qhi[qi], cnt = lo + hi;
    for (int e = lane + 64 * kh; e < cnt; e += 64 * (IDX_NW / QPB)) {
      const int ps = e < lo ? e : CAPS - hi + (e - lo);
      cand_s[slot * cap + e] = cs[ps];
      cand_i[slot * cap + e] = n_lo + (int)co[ps];
    }
    if (kh == 0 && lane == 0) {
      cand_n[slot] = qovf[qi] ? -1 : cnt;
      cand_t[slot] = qthr[qi];
    }
  }
}

// ---------------------------------------------------------------- 3b. score + filter, global lists
// Variant of the score kernel for contexts long enough for the sampled start
// (every query of the launch sees at least 8 * SAMPLE keys). The threshold is
// fixed after the sampling prologue, so no list has to be kept on chip: each wave
// stages its survivors (score, key) in a small LDS buffer and moves them to the
// query's list in global memory when the buffer is half full (one LDS atomic per
// flush for the positions). That frees the LDS for a ring of four key stages
// filled by direct global-to-LDS loads three 128-key tiles ahead. Sixteen waves
// (two per query, eight queries) share each tile, so one tile load feeds twice
// as many MFMAs as with four queries, and with at most 128 VGPRs per wave the one
// workgroup per compute unit still keeps four waves on every SIMD. A list that
// would exceed its capacity marks the query for the exact fallback.
// Stage rows are 272 bytes (a key's 256 plus 16 of padding): the 16 rows one
// quarter of an MFMA operand read touches then start 68 banks apart and cover all
// 64 banks, and every operand address is a per-lane base plus an immediate.
namespace {
constexpr int GQ = 8;                                    // queries per workgroup
constexpr int GW = 2 * GQ;                               // waves: two per query
constexpr int GT = 128;                                  // keys per tile
constexpr int G_ROW = ID * 2 + 16;                       // LDS bytes per key row
constexpr int G_STAGE = GT * G_ROW;                      // 34816 B
constexpr int G_NST = 4;                                 // ring stages (G_NST - 1 tiles in flight)
constexpr int G_LOADS = G_STAGE / 1024;                  // 1 KB direct loads per tile (one per wave instruction)
constexpr int G_CB = 128;                                // staged survivors per wave
static_assert(G_LOADS * 1024 == G_STAGE, "tile loads cover the stage");
static_assert(G_LOADS > 2 * GW && G_LOADS <= 3 * GW, "every wave issues two or three loads per tile");
static_assert(SAMPLE * GQ * 4 <= 2 * G_STAGE && SAMPLE_SMALL <= SAMPLE, "sample scores fit two stages");
static_assert(G_NST >= 4, "the sampling prologue takes two stages for tiles and two for scores");
static_assert(GQ * 256 <= GW * G_CB, "the prologue's histograms fit the staging buffer");
static_assert(G_CB >= 128, "a half-full buffer still takes a whole tile of survivors");
}  // namespace


template <int S>
__global__ __launch_bounds__(64 * GW) __attribute__((amdgpu_waves_per_eu(4, 4))) void score_list_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ eps_in, int L, int N, int topk, int span, int nsplit, int cap,
    float* __restrict__ cand_s, int* __restrict__ cand_i, int* __restrict__ cand_n, float* __restrict__ cand_t) {
  __shared__ __attribute__((aligned(1024))) unsigned char stage[G_NST * G_STAGE];
  // staged survivors: wave v's scores (as bits) at [v G_CB, v G_CB + G_CB), its keys
  // GW * G_CB words further; the sampling prologue keeps its histograms here
  __shared__ __attribute__((aligned(16))) int cbuf[2 * GW * G_CB];
  __shared__ int qcnt[GQ];
  __shared__ int qovf[GQ];
  __shared__ float red[2 * GW];
  int* const hist = cbuf;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = wave & (GQ - 1), kh = wave / GQ;
  const int split = blockIdx.y;
  const int n_lo = split * span;
  const int i = blockIdx.x * GQ + qi;
  const bool active = i < L;
  const int ii = active ? i : L - 1;
  const int p = N - L + ii;
  const int ilast = min(L - 1, (int)blockIdx.x * GQ + GQ - 1);
  const int n_hi = min(min(N, n_lo + span), N - L + ilast + 1);
  const uint32_t lds_stage = (uint32_t)(uintptr_t)(DSA_LDS void*)&stage[0];

  bf16x8 qa[ID / 16];
  {
    const uint16_t* qrow = q + ((size_t)ii * IH + (lane & 31)) * ID + 8 * (lane >> 5);
#pragma unroll
    for (int kc = 0; kc < ID / 16; ++kc) qa[kc] = *(const bf16x8*)(qrow + 16 * kc);
  }
  float wr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wr[j] = w[(size_t)ii * IH + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)];
#pragma unroll
  for (int kc = 0; kc < ID / 16; ++kc) asm volatile("" ::"v"(qa[kc]));
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(wr[j]));
  if (tid < GQ) {
    qcnt[tid] = 0;
    qovf[tid] = 0;
  }

  // Tile loads: load j (0 <= j < G_LOADS) fills stage bytes [1024 j, 1024 j + 1024);
  // wave w issues loads w, w + GW and, for w < G_LOADS - 2 GW, w + 2 GW. Lane l of
  // load j writes row (1024 j + 16 l) / G_ROW, 16-byte chunk ((1024 j + 16 l) % G_ROW) / 16;
  // chunk 16 is the padding, for which the lane loads chunk 15 again.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool third = wave_u < G_LOADS - 2 * GW;
  int lrow[3], lchk[3];
  uint32_t voff[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int pos = 1024 * (wave + GW * u) + 16 * lane;
    lrow[u] = pos / G_ROW;
    lchk[u] = min((pos % G_ROW) / 16, 15);
    voff[u] = (uint32_t)(lrow[u] * (ID * 2) + lchk[u] * 16);
  }
  // rows mapped to arbitrary keys (sampled tiles, the clamped last tile)
  auto dma_tile = [&](auto key_of, int st) {
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (u < 2 || third)
        dma16(k + (size_t)key_of(lrow[u]) * ID + lchk[u] * 8,
              lds_stage + st * G_STAGE + 1024 * (wave_u + GW * u));
  };
  // rows n0 .. n0 + GT - 1
  auto dma_run = [&](int n0, int st) {
    const unsigned char* base = (const unsigned char*)k + (size_t)n0 * (ID * 2);
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (u < 2 || third) dma16s(base, voff[u], lds_stage + st * G_STAGE + 1024 * (wave_u + GW * u));
  };

  // Scores of keys r0 + lane (this query), r0 = 64 kh, of a stage: chains a (lanes
  // < 32 get keys r0 .. r0+31) and b (lanes >= 32 get r0+32 .. r0+63), with
  // accumulators acc_a and acc_b. Phase A runs the eight chain-a MFMAs, phase B the
  // chain-b ones; the VALU work that turns accumulators into weighted ReLU sums is
  // interleaved with the other phase's MFMAs: the chain-a sums with phase B of the
  // same tile, the chain-b sums with phase A of the next tile (the accumulators of
  // both chains stay live), so no MFMA waits for them. Fragments are read two
  // k-steps ahead.
  const int lane_rd = (lane & 31) * G_ROW + (lane >> 5) * 16 + kh * 64 * G_ROW;
  constexpr int KS = ID / 16;           // k-steps per chain
  f32x16 acc_a, acc_b = {};
  // the empty asm pins the running sum at this point of the instruction stream
  auto relu_w = [&](const f32x16& c, int j, float p) {
    p = fmaf(wr[j], __int_as_float(max(__float_as_int(c[j]), 0)), p);
    asm volatile("" : "+v"(p));
    return p;
  };
  // One k-step: the MFMA, the fragment read two k-steps ahead and the two VALU
  // sums of this step; the scheduling barrier after each step keeps the compiler
  // from gathering the VALU work in one place.
  // phase A on stage st; meanwhile the chain-b sums of the previous tile (pb)
  auto phase_a = [&](int st) -> float {
    const unsigned char* ba = stage + st * G_STAGE + lane_rd;
    bf16x8 f0 = *(const bf16x8*)(ba), f1 = *(const bf16x8*)(ba + 32);
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) {
      const bf16x8 x = (kc & 1) ? f1 : f0;
      acc_a = mfma32x32x16(qa[kc], x, kc ? acc_a : f32x16{});
      p0 = relu_w(acc_b, 2 * kc, p0);
      if (kc + 2 < KS) {
        if (kc & 1) f1 = *(const bf16x8*)(ba + 32 * (kc + 2));
        else f0 = *(const bf16x8*)(ba + 32 * (kc + 2));
      }
      p1 = relu_w(acc_b, 2 * kc + 1, p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    return p0 + p1;
  };
  // phase B on stage st; meanwhile the chain-a sums of this tile (pa)
  auto phase_b = [&](int st) -> float {
    const unsigned char* ba = stage + st * G_STAGE + lane_rd + 32 * G_ROW;
    bf16x8 f0 = *(const bf16x8*)(ba), f1 = *(const bf16x8*)(ba + 32);
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) {
      const bf16x8 x = (kc & 1) ? f1 : f0;
      acc_b = mfma32x32x16(qa[kc], x, kc ? acc_b : f32x16{});
      p0 = relu_w(acc_a, 2 * kc, p0);
      if (kc + 2 < KS) {
        if (kc & 1) f1 = *(const bf16x8*)(ba + 32 * (kc + 2));
        else f0 = *(const bf16x8*)(ba + 32 * (kc + 2));
      }
      p1 = relu_w(acc_a, 2 * kc + 1, p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    return p0 + p1;
  };
  // chain-b sums alone (after the last tile)
  auto tail_b = [&]() -> float {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      p0 = relu_w(acc_b, j, p0);
      p1 = relu_w(acc_b, j + 1, p1);
    }
    return p0 + p1;
  };
  // lanes < 32 hold chain a's half of the heads (and lanes >= 32 chain b's) for key
  // lane % 32 of each chain; the swap gives every lane both halves of its own key
  auto combine = [&](float pa, float pb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  };

  // Sampling prologue: S keys spread evenly over the keys every query of the
  // group sees; the start threshold sits just below the rk-th largest sample score
  // (see score_filter_kernel). Sample tiles alternate between stages 0 and 1, one
  // tile ahead; the scores go to stages 2-3 as two segments per query (front wave
  // from the start, back wave from the end), the layout the threshold search shares
  // with the list compaction.
  float thr = -INFINITY;
  {
    const int nv_min = min(N, N - L + (int)blockIdx.x * GQ + 1);
    const float mean = (float)topk * S / (float)max(nv_min, 1);
    if (nv_min >= 8 * S && mean <= S / 8) {
      const int rk = min(S / 2, (int)ceilf(mean + 6.f * sqrtf(mean) + 8.f));
      float* ss = (float*)(stage + 2 * G_STAGE) + qi * S;
      auto sample_tile = [&](int t) {
        dma_tile([&](int r) { return (int)((long long)(t * GT + r) * nv_min / S); }, t & 1);
      };
      // pipelined like the main loop: the chain-b sums of tile t - 1 run under the
      // chain-a MFMAs of tile t, so tile t - 1's scores are stored during tile t
      auto store_sample = [&](int t, float sv) {
        const int e = t * 64 + lane;
        if (active) ss[kh == 0 ? e : S - 1 - e] = sv;
      };
      sample_tile(0);
      float pa = 0.f;
      for (int t = 0; t < S / GT; ++t) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();                  // tile t landed; every wave is done with tile t - 1
        if (t + 1 < S / GT) sample_tile(t + 1);
        const float pb = phase_a(t & 1);   // + chain-b sums of tile t - 1
        if (t > 0) store_sample(t - 1, combine(pa, pb));
        pa = phase_b(t & 1);               // + chain-a sums of tile t
      }
      store_sample(S / GT - 1, combine(pa, tail_b()));
      float thr_q = -INFINITY;
      pair_compact<float, S, GQ>(ss, (float*)nullptr, S / 2, kh, active, rk, eps_in[ii], thr_q,
                                      hist + qi * 256, red, false);
      thr = thr_q;
      lds_barrier();                    // scores and histograms read before the ring reuses them
    }
  }

  const size_t slot = (size_t)ii * nsplit + split;
  float* ls = cand_s + slot * cap;
  int* li = cand_i + slot * cap;
  const int ntiles = n_hi > n_lo ? (n_hi - n_lo + GT - 1) / GT : 0;
  // rows past n_hi are loaded but masked; only a tile running past the end of the key
  // array clamps its rows
  auto dma_main = [&](int t, int st) {
    const int n0 = n_lo + t * GT;
    if (n0 + GT <= N) dma_run(n0, st);
    else dma_tile([=](int r) { return min(n0 + r, N - 1); }, st);
  };
  int* const my_s = cbuf + wave * G_CB;
  int* const my_i = cbuf + (GW + wave) * G_CB;
  // a key of this wave is kept when key <= lim and its score reaches thr
  const int lim = active ? min(n_hi - 1, p) : -1;
  int cnt = 0;                          // staged survivors of this wave (wave-uniform)
  auto flush = [&]() {
    wave_sync();
    int base = 0;
    if (lane == 0) base = atomicAdd(&qcnt[qi], cnt);
    base = __shfl(base, 0);
    for (int e = lane; e < cnt; e += 64) {
      const int pos = base + e;
      if (pos < cap) {
        ls[pos] = __int_as_float(my_s[e]);
        li[pos] = my_i[e];
      } else {
        qovf[qi] = 1;
      }
    }
    cnt = 0;
  };
  // Tiles are issued G_NST - 1 ahead (the last tile is loaded again into the spare
  // stages near the end, so the number of loads in flight is always the same);
  // stage t % G_NST holds tile t. The wait at the top of iteration t leaves the
  // loads of tiles t+1 .. t+G_NST-2 in flight, unless survivors were flushed in the
  // previous iteration: then everything is drained, stores included.
  if (ntiles > 0)
    for (int s = 0; s < G_NST - 1; ++s) dma_main(min(s, ntiles - 1), s);
  // survivors of tile t (score sv of key n_lo + t GT + 64 kh + lane)
  auto stage_keep = [&](int t, float sv, bool valid) {
    const int key = n_lo + t * GT + 64 * kh + lane;
    const bool keep = valid && key <= lim && sv >= thr;
    const unsigned long long bm = __ballot(keep);
    if (keep) {
      const int e = cnt + (int)__popcll(bm & ((1ull << lane) - 1ull));
      my_s[e] = __float_as_int(sv);
      my_i[e] = key;
    }
    cnt += (int)__popcll(bm);
    const bool fl = cnt > G_CB - 64;
    if (fl) flush();
    return fl;
  };
  bool flushed = false;
  float pa = 0.f;                       // chain-a sums of the previous tile
  for (int t = 0; t < ntiles; ++t) {
    if (flushed) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (third) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((G_NST - 2) * 3) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((G_NST - 2) * 2) : "memory");
    lds_barrier();                      // tile t landed; every wave is done with tile t - 1
    // the MFMAs go first when several waves of a SIMD are ready; the VALU work of
    // the others fills in behind them
    __builtin_amdgcn_s_setprio(1);
    const float pb = phase_a(t % G_NST);   // + chain-b sums of tile t - 1
    __builtin_amdgcn_s_setprio(0);
    // Between the two phases, while the other waves of the SIMD keep its matrix pipe
    // busy: the survivors of tile t - 1 (nothing is kept at t = 0, whose
    // previous-tile sums are zeros) and the loads of tile t + G_NST - 1.
    flushed = stage_keep(t - 1, combine(pa, pb), t > 0);
    dma_main(min(t + G_NST - 1, ntiles - 1), (t + G_NST - 1) % G_NST);
    __builtin_amdgcn_s_setprio(1);
    pa = phase_b(t % G_NST);               // + chain-a sums of tile t
    __builtin_amdgcn_s_setprio(0);
  }
  if (ntiles > 0) stage_keep(ntiles - 1, combine(pa, tail_b()), true);
  if (cnt > 0) flush();
  // no load may still be writing the LDS when the workgroup ends (the ring's last
  // loads repeat the final tile and are never waited for in the loop)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();                        // every flush of the group has taken its positions
  if (active && kh == 0 && lane == 0) {
    cand_n[slot] = qovf[qi] ? -1 : qcnt[qi];
    cand_t[slot] = thr;
  }
}

// ---------------------------------------------------------------- 4. select + band refine
// One workgroup (SR_T = 512 threads, eight waves) per query: every phase is a short
// latency-bound step, so more waves per query shorten each of them. The query's
// candidates (the concatenated split lists, M <= SR_MAX) sit in registers: thread t
// holds entries t + SR_T j, j < SR_J, with per-thread bit masks for "kept" and "in
// the band". The LDS holds only the histograms, the band, the staged query and the
// rank bitmap (about 54 KB); at 128 VGPRs two workgroups share a compute unit.
//   1. tk = the exact topk-th largest candidate score (linear histogram over
//      [min, max], then an exact rank count inside the bin that holds it);
//   2. scores above tk + band are kept, scores in [tk - band, tk + band] form the
//      band, whose keys get canonical fp64 scores; the best (topk - #above) of them
//      by (fp64 score desc, key asc) are kept;
//   3. kept keys are written in ascending order: a bitmap over a window of keys and
//      prefix popcounts give every kept key its output slot.
namespace {
constexpr int Q_ROW = ID + 8;           // staged query row, in bf16 (16 B of padding)
constexpr int DH_ROW = IH + 1;          // per-key head dots, in doubles (8 B of padding)

struct RefineLds {
  uint32_t bitmap[RANK_WORDS];                         // kept keys of the window; band key rows while re-scoring
  union {
    int wpre[RANK_WORDS];                              // kept keys before each bitmap word
    double dh[64 * DH_ROW];                            // head dots of a band batch
  } u;
  uint16_t qrow[IH * Q_ROW];
  float wrow[IH];
  double bscore[BAND_CAP];
  int bkey[BAND_CAP];
  float bval[BAND_CAP];
  float binv[BIN_CAP];
  unsigned char bsel[BAND_CAP];
  int hist[4][256];                                    // 256-bin histograms; waves w and w + 4 share one
  int misc[12 + 2 * SR_W];                             // 0-3 selection, 4.. output prefix, then per-wave max, min
  float red[SR_W];
};
// a band batch of 64 fp32 key rows spans the bitmap and the union after it
static_assert(offsetof(RefineLds, u) == sizeof(uint32_t) * RANK_WORDS, "the union follows the bitmap");
static_assert(64 * ID * 4 <= sizeof(uint32_t) * RANK_WORDS + sizeof(RefineLds::u), "a band batch fits");
static_assert(BAND_CAP <= SR_T, "one thread per band slot in the emit");
constexpr int MISC_PRE = 4, MISC_MX = 4 + SR_W, MISC_MN = 4 + 2 * SR_W;
static_assert(sizeof(RefineLds) <= 80 * 1024, "two refine workgroups per compute unit");
}  // namespace

// Canonical fp64 scores of up to 64 band keys whose rows are staged in LDS as
// fp32 (krows, 512 B each; bf16 -> fp32 is exact, so each key value is widened once
// when staged instead of once per head): lane l32 of 32-lane group g (G = SR_T / 32
// groups) owns head l32 and keys g, g+G, ... (64 / G independent chains). d_h is summed over dims in
// ascending order; the head terms are then added in ascending head order by one
// lane per key. A bf16 x bf16 product is exact in fp64, so the fused multiply-add
// rounds exactly as a product followed by a sum; the weight products are rounded
// separately.
// fp64 product rounded on its own: the weight products of the canonical score are
// not exact, and a fused multiply-add formed from a product and the following sum
// would round once instead of twice.
__device__ __forceinline__ double dmul_rounded(double a, double b) {
  double p;
  asm volatile("v_mul_f64 %0, %1, %2" : "=v"(p) : "v"(a), "v"(b));
  return p;
}

__device__ void canonical_scores_batch(const uint16_t* qrow_lds, const float* krows, int nkeys,
                                       const float* wrow, double* dh, double* out) {
  constexpr int G = SR_T / 32, KPT = 64 / G;         // 32-lane groups, keys per thread
  const int tid = threadIdx.x, g = tid >> 5, l32 = tid & 31;
  const uint16_t* qh = qrow_lds + l32 * Q_ROW;
  double d[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) d[j] = 0.0;
  // chains whose rows lie past the batch for both groups of a wave are skipped: the
  // wave runs its first kn chains, kn = #{j : 2 w + G j < nkeys}
  auto chains = [&](auto KN) __attribute__((always_inline)) {
    constexpr int kn = decltype(KN)::value;
    for (int c = 0; c < ID / 4; ++c) {
      const uint2 qv = *(const uint2*)(qh + 4 * c);
      f32x4 kv[kn];
#pragma unroll
      for (int j = 0; j < kn; ++j) kv[j] = *(const f32x4*)(krows + (size_t)(g + G * j) * ID + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t qw = (e >> 1) ? qv.y : qv.x;
        const double qd = (double)bf_bits2f((uint16_t)((qw >> (16 * (e & 1))) & 0xFFFFu));
#pragma unroll
        for (int j = 0; j < kn; ++j) d[j] = __fma_rn(qd, (double)kv[j][e], d[j]);
      }
    }
  };
  static_assert(KPT == 4, "one specialisation per chain count");
  const int g0 = 2 * (tid >> 6);
  const int kn = nkeys > g0 ? min(KPT, (nkeys - g0 + G - 1) / G) : 0;
  switch (kn) {
    case 4: chains(std::integral_constant<int, 4>{}); break;
    case 3: chains(std::integral_constant<int, 3>{}); break;
    case 2: chains(std::integral_constant<int, 2>{}); break;
    case 1: chains(std::integral_constant<int, 1>{}); break;
    default: break;
  }
  __syncthreads();                      // the head dots overwrite the tail of the key rows
#pragma unroll
  for (int j = 0; j < KPT; ++j) dh[(g + G * j) * DH_ROW + l32] = d[j];
  __syncthreads();
  if (tid < nkeys) {
    // the weight products do not depend on the running sum: eight are formed at a
    // time, then added in ascending head order
    double sc = 0.0;
#pragma unroll
    for (int h0 = 0; h0 < IH; h0 += 8) {
      double pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double v = dh[tid * DH_ROW + h0 + e];
        pr[e] = dmul_rounded((double)wrow[h0 + e], v > 0.0 ? v : 0.0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sc = sc + pr[e];
    }
    out[tid] = sc;
  }
  __syncthreads();
}

// Order-preserving map of a float to an unsigned integer (for -0 < +0 it does not
// matter: both are scored alike).
__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(SR_T, 4) void select_refine_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ eps_in, int L, int N, int topk, int nsplit, int cap,
    const float* __restrict__ cand_s, const int* __restrict__ cand_i, const int* __restrict__ cand_n,
    const float* __restrict__ cand_t, int* __restrict__ fb_flag, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  __shared__ __attribute__((aligned(16))) RefineLds sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.x;
  const int p = N - L + i;
  const int nv = min(N, p + 1);
  int32_t* orow = idx_out + (size_t)i * topk;
  float* srow = score_out ? score_out + (size_t)i * topk : nullptr;
  // magnitudes past the range the fp32 scores are safe in (eps = +inf): exact fallback
  if (!(eps_in[i] < INFINITY)) {
    if (tid == 0) fb_flag[i] = 1;
    return;
  }

  // ---- candidates into registers. Split sp's list fills slots [pre4[sp], pre4[sp] +
  // cnt rounded up to 4); thread t loads slot groups t + SR_T u (4 slots each, one
  // 16-byte load of scores and one of keys). Unused slots hold key -1.
  int cnt[4] = {0, 0, 0, 0}, pre4[5] = {0, 0, 0, 0, 0};
  bool overflow = nsplit > 4;
  int M = 0;
  for (int sp = 0; sp < nsplit && sp < 4; ++sp) {
    cnt[sp] = cand_n[(size_t)i * nsplit + sp];
    if (cnt[sp] < 0) overflow = true;
    M += max(cnt[sp], 0);
    pre4[sp + 1] = pre4[sp] + (max(cnt[sp], 0) + 3) / 4 * 4;
  }
  const int M4 = pre4[min(nsplit, 4)];
  for (int sp = min(nsplit, 4) + 1; sp < 5; ++sp) pre4[sp] = INT_MAX;   // no slot maps past the last split
  if (overflow || M4 > SR_MAX) {
    if (tid == 0) fb_flag[i] = 1;
    return;
  }
  constexpr int SR_U = SR_J / 4;
  // slot groups of this wave that hold anything: those below M4 / 4
  const int uw = min(SR_U, (M4 / 4 - wave * 64 + SR_T - 1) / SR_T);
  float sc[SR_J];
  int ky[SR_J];
#pragma unroll
  for (int u = 0; u < SR_U; ++u) {
    float4 s4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int4 k4 = {-1, -1, -1, -1};
    if (u < uw) {
      const int slot = 4 * (tid + SR_T * u);
      if (slot < M4) {
        const int sp = (slot >= pre4[1]) + (slot >= pre4[2]) + (slot >= pre4[3]);
        const int off = slot - pre4[sp];
        const size_t o = ((size_t)i * nsplit + sp) * cap + off;   // cap is a multiple of 64
        s4 = *(const float4*)(cand_s + o);
        k4 = *(const int4*)(cand_i + o);
        if (off + 1 > cnt[sp]) k4.x = -1;
        if (off + 2 > cnt[sp]) k4.y = -1;
        if (off + 3 > cnt[sp]) k4.z = -1;
        if (off + 4 > cnt[sp]) k4.w = -1;
      }
    }
    sc[4 * u] = s4.x; sc[4 * u + 1] = s4.y; sc[4 * u + 2] = s4.z; sc[4 * u + 3] = s4.w;
    ky[4 * u] = k4.x; ky[4 * u + 1] = k4.y; ky[4 * u + 2] = k4.z; ky[4 * u + 3] = k4.w;
  }
  const int jw = 4 * uw;                // register slots of this wave that may hold entries
  uint64_t kept = 0;

  const float eps = eps_in[i];
  // Each split's list holds every key scoring at least that split's final filter
  // threshold; the selection below is exact only if every threshold lies at or
  // below the band around the k-th score (always true for thresholds derived from
  // the lists themselves, to be checked for the sampled start).
  float thr_max = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) thr_max = fmaxf(thr_max, cand_t[(size_t)i * nsplit + sp]);
  int nb = 0;                           // band entries (slots [0, nb) of the LDS band arrays)
  if (nv <= topk) {
    // every visible key must be in the lists: only an untouched threshold guarantees it
    if (thr_max > -INFINITY) {
      if (tid == 0) fb_flag[i] = 1;
      return;
    }
#pragma unroll
    for (int j = 0; j < SR_J; ++j)
      if (j < jw && ky[j] >= 0) kept |= 1ull << j;
  } else {
    // fewer candidates than topk: a sampled start threshold was set too high
    if (M < topk) {
      if (tid == 0) fb_flag[i] = 1;
      return;
    }
    // ---- 1. tk, the topk-th largest score: a 256-bin histogram linear in the
    // order-preserving integer image of the scores (so a heavy low tail spreads over
    // many bins), narrowed by further 8-bit digits while the bin that holds it is
    // too full, then an exact rank count inside that bin
    uint32_t umx = 0u, umn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < SR_J; ++j)
      if (j < jw && ky[j] >= 0) {
        const uint32_t u = ord_bits(sc[j]);
        umx = max(umx, u);
        umn = min(umn, u);
      }
    umx = wave_max_u32(umx);
    umn = wave_min_u32(umn);
    if (lane == 0) {
      sm.misc[MISC_MX + wave] = (int)umx;
      sm.misc[MISC_MN + wave] = (int)umn;
    }
    for (int x = tid; x < 4 * 256; x += SR_T) (&sm.hist[0][0])[x] = 0;
    if (tid == 0) sm.misc[2] = 0;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < SR_W; ++x) {
      umx = max(umx, (uint32_t)sm.misc[MISC_MX + x]);
      umn = min(umn, (uint32_t)sm.misc[MISC_MN + x]);
    }
    // bin = (u - umn) >> shift with (umx - umn) >> shift < 256
    const uint32_t span = umx - umn;
    const int shift = span < 256u ? 0 : 32 - __clz((int)(span >> 8)) ;
    float tk;
    if (span == 0u) {
      // all scores equal
      tk = __uint_as_float((umx & 0x80000000u) ? (umx & 0x7FFFFFFFu) : ~umx);
    } else {
      // Radix descent: the entries still in play are those with (d >> hi_sh) == sel,
      // d = ord_bits - umn; each level histograms the next digit (d >> sh) - (sel <<
      // (hi_sh - sh)) of those entries and keeps the bin of the need-th largest. The
      // first level covers the whole span; further levels of 8 bits run only while
      // the bin holds more entries than the exact rank step takes.
      int sh = shift, hi_sh = 32, need = topk, cnt = 0;
      uint64_t sel = 0;
      for (;;) {
        const uint64_t base = sel << (hi_sh - sh);
#pragma unroll
        for (int j = 0; j < SR_J; ++j)
          if (j < jw && ky[j] >= 0) {
            const uint64_t d = ord_bits(sc[j]) - umn;
            if ((d >> hi_sh) == sel) atomicAdd(&sm.hist[wave & 3][(int)((d >> sh) - base)], 1);
          }
        __syncthreads();
        if (tid < 256) sm.hist[0][tid] += sm.hist[1][tid] + sm.hist[2][tid] + sm.hist[3][tid];
        __syncthreads();
        if (wave == 0) {
          int bin, above;
          wave_find_bin(sm.hist[0], need, lane, bin, above);
          if (lane == 0) {
            sm.misc[0] = bin;
            sm.misc[1] = above;
          }
        }
        __syncthreads();
        const int bin = sm.misc[0];
        need -= sm.misc[1];
        cnt = sm.hist[0][bin];
        sel = base + (uint64_t)bin;
        hi_sh = sh;
        if (cnt <= BIN_CAP || sh == 0) break;
        sh = sh >= 8 ? sh - 8 : 0;
        __syncthreads();                  // every thread has read the histogram
        for (int x = tid; x < 4 * 256; x += SR_T) (&sm.hist[0][0])[x] = 0;
        __syncthreads();
      }
      if (cnt > BIN_CAP) {
        // sh == 0: every entry of the bin has the same bit pattern
        const uint32_t ub = umn + (uint32_t)sel;
        tk = __uint_as_float((ub & 0x80000000u) ? (ub & 0x7FFFFFFFu) : ~ub);
      } else {
#pragma unroll
        for (int j = 0; j < SR_J; ++j)
          if (j < jw && ky[j] >= 0 && (((uint64_t)(ord_bits(sc[j]) - umn)) >> hi_sh) == sel) {
            const int slot = atomicAdd(&sm.misc[2], 1);
            if (slot < BIN_CAP) sm.binv[slot] = sc[j];
          }
        __syncthreads();
        const int nbin = sm.misc[2];
        // the need-th largest inside the bin: the largest v with #{u >= v} >= need
        float best = -INFINITY;
        for (int e = tid; e < nbin; e += SR_T) {
          const float v = sm.binv[e];
          int c = 0, f = 0;
          for (; f + 4 <= nbin; f += 4) {
            const float4 u = *(const float4*)&sm.binv[f];
            c += (u.x >= v) + (u.y >= v) + (u.z >= v) + (u.w >= v);
          }
          for (; f < nbin; ++f) c += sm.binv[f] >= v;
          if (c >= need) best = fmaxf(best, v);
        }
        best = wave_max(best);
        if (lane == 0) sm.red[wave] = best;
        __syncthreads();
        tk = sm.red[0];
#pragma unroll
        for (int x = 1; x < SR_W; ++x) tk = fmaxf(tk, sm.red[x]);
      }
    }
    const float hw = band_halfwidth(eps, tk);
    const float hi = tk + hw, lo = tk - hw;
    if (thr_max > lo) {
      if (tid == 0) fb_flag[i] = 1;
      return;
    }
    // ---- 2. above the band: kept; inside: band slots (key and fp32 score)
    if (tid == 0) {
      sm.misc[2] = 0;
      sm.misc[3] = 0;
    }
    __syncthreads();
    int my_in = 0;
#pragma unroll
    for (int j = 0; j < SR_J; ++j) {
      if (j < jw) {
        const bool ok = ky[j] >= 0;
        const bool isin = ok && sc[j] > hi, isband = ok && !isin && sc[j] >= lo;
        if (isin) kept |= 1ull << j;
        my_in += isin;
        const unsigned long long bb = __ballot(isband);
        if (bb) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&sm.misc[3], (int)__popcll(bb));
          base = __shfl(base, 0);
          if (isband) {
            const int b = base + (int)__popcll(bb & ((1ull << lane) - 1ull));
            if (b < BAND_CAP) {
              sm.bkey[b] = ky[j];
              sm.bval[b] = sc[j];
            }
          }
        }
      }
    }
    my_in = wave_sum_int(my_in);
    if (lane == 0) atomicAdd(&sm.misc[2], my_in);
    __syncthreads();
    const int n_in = sm.misc[2];
    nb = sm.misc[3];
    const int need_band = topk - n_in;
    if (nb > BAND_CAP || need_band < 0 || need_band > nb) {
      if (tid == 0) fb_flag[i] = 1;
      return;
    }
    if (nb > 0) {
      for (int e = tid; e < IH * ID / 8; e += SR_T) {
        const int h = e / (ID / 8), c = e % (ID / 8);
        *(u32x4*)(sm.qrow + h * Q_ROW + 8 * c) = *(const u32x4*)(q + (size_t)i * IH * ID + 8 * e);
      }
      if (tid < IH) sm.wrow[tid] = w[(size_t)i * IH + tid];
      float* krows = (float*)sm.bitmap;                 // 64 rows x 512 B, over the bitmap and the union
      for (int b0 = 0; b0 < nb; b0 += 64) {
        const int nk = min(64, nb - b0);
        for (int x = tid; x < 64 * (ID / 8); x += SR_T) {  // row r, chunk c; missing rows repeat row 0
          const int r = x >> 4, c = x & 15;
          const int n = sm.bkey[b0 + (r < nk ? r : 0)];
          const u32x4 v = *(const u32x4*)(k + (size_t)n * ID + 8 * c);
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] = __uint_as_float(v[e] << 16);
            lo[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
            hi[2 * e] = __uint_as_float(v[2 + e] << 16);
            hi[2 * e + 1] = __uint_as_float(v[2 + e] & 0xFFFF0000u);
          }
          *(f32x4*)(krows + r * ID + 8 * c) = lo;
          *(f32x4*)(krows + r * ID + 8 * c + 4) = hi;
        }
        __syncthreads();
        canonical_scores_batch(sm.qrow, krows, nk, sm.wrow, sm.u.dh, sm.bscore + b0);
      }
      // rank by (fp64 score desc, key asc); the best need_band are kept. Up to 64
      // entries, thread (b, part) counts the entries o = part, part + SR_W, ... that
      // precede entry b, and the partial counts of the waves meet in LDS (the
      // histograms are free by now)
      if (nb <= 64) {
        const int b = tid & 63, part = tid >> 6;
        int r = 0;
        if (b < nb) {
          const double s0 = sm.bscore[b];
          const int key = sm.bkey[b];
#pragma unroll
          for (int m = 0; m < 64 / SR_W; ++m) {
            const int o = part + SR_W * m;
            if (o < nb) {
              const double so = sm.bscore[o];
              r += (so > s0) || (so == s0 && sm.bkey[o] < key);
            }
          }
        }
        int* cnts = &sm.hist[0][0];
        cnts[64 * part + b] = r;
        __syncthreads();
        if (tid < nb) {
          int rank = 0;
#pragma unroll
          for (int x = 0; x < SR_W; ++x) rank += cnts[64 * x + tid];
          sm.bsel[tid] = rank < need_band;
        }
      } else
      for (int b = tid; b < nb; b += SR_T) {
        const double s0 = sm.bscore[b];
        const int key = sm.bkey[b];
        int r = 0, o = 0;
        for (; o + 4 <= nb; o += 4) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const double so = sm.bscore[o + x];
            r += (so > s0) || (so == s0 && sm.bkey[o + x] < key);
          }
        }
        for (; o < nb; ++o) {
          const double so = sm.bscore[o];
          r += (so > s0) || (so == s0 && sm.bkey[o] < key);
        }
        sm.bsel[b] = r < need_band;
      }
    }
  }
  if (tid == 0) fb_flag[i] = 0;

  // ---- 3. kept keys in ascending order, one window of RANK_WORDS * 32 keys at a time:
  // the kept candidates in registers plus the selected band slots (thread b owns slot b)
  const bool band_kept = tid < nb && sm.bsel[tid];
  const int bk = tid < nb ? sm.bkey[tid] : -1;
  int done = 0;
  for (int w0 = 0; w0 < N; w0 += RANK_WORDS * 32) {
    auto in_win = [&](int key) { return key >= w0 && key < w0 + RANK_WORDS * 32; };
    __syncthreads();                    // the band rows (or the last window) are no longer read
    for (int x = tid; x < RANK_WORDS / 4; x += SR_T) ((u32x4*)sm.bitmap)[x] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SR_J; ++j)
      if (((kept >> j) & 1) && in_win(ky[j])) atomicOr(&sm.bitmap[(ky[j] - w0) >> 5], 1u << ((ky[j] - w0) & 31));
    if (band_kept && in_win(bk)) atomicOr(&sm.bitmap[(bk - w0) >> 5], 1u << ((bk - w0) & 31));
    __syncthreads();
    constexpr int WPT = RANK_WORDS / SR_T;       // consecutive words per thread
    u32x4 wv[WPT / 4];
    int own = 0;
#pragma unroll
    for (int x = 0; x < WPT / 4; ++x) {
      wv[x] = ((const u32x4*)sm.bitmap)[tid * (WPT / 4) + x];
      own += __popc(wv[x][0]) + __popc(wv[x][1]) + __popc(wv[x][2]) + __popc(wv[x][3]);
    }
    int incl = own;                              // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) sm.misc[MISC_PRE + wave] = incl;
    __syncthreads();
    int run = incl - own;
    for (int x = 0; x < wave; ++x) run += sm.misc[MISC_PRE + x];
#pragma unroll
    for (int x = 0; x < WPT / 4; ++x) {
      u32x4 pre;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        pre[y] = (uint32_t)run;
        run += __popc(wv[x][y]);
      }
      ((u32x4*)sm.u.wpre)[tid * (WPT / 4) + x] = pre;
    }
    int total = 0;
#pragma unroll
    for (int x = 0; x < SR_W; ++x) total += sm.misc[MISC_PRE + x];
    __syncthreads();
    auto emit = [&](int key, float v) {
      const int word = (key - w0) >> 5, bit = (key - w0) & 31;
      const int pos = done + sm.u.wpre[word] + __popc(sm.bitmap[word] & ((1u << bit) - 1u));
      if (pos < topk) {
        orow[pos] = key;
        if (srow) srow[pos] = v;
      }
    };
#pragma unroll
    for (int j = 0; j < SR_J; ++j)
      if (((kept >> j) & 1) && in_win(ky[j])) emit(ky[j], sc[j]);
    if (band_kept && in_win(bk)) emit(bk, sm.bval[tid]);
    done += total;
  }
  for (int e = done + tid; e < topk; e += SR_T) {
    orow[e] = -1;
    if (srow) srow[e] = -INFINITY;
  }
}

// ---------------------------------------------------------------- 5. exact fallback
// One workgroup per flagged row at a time (one workgroup per compute unit); the
// canonical fp64 score of every visible key goes to a per-workgroup scratch row,
// then an exact 64-bit radix select finds the k-th largest value and a stable scan
// emits the set. A thread scores one key at a time: the 32 head dots advance
// together over 32-dim chunks of the key (converted to fp64 once per chunk), with
// the query in LDS as fp64 and read by all lanes at once. A product of two bf16
// values is exact in fp64, so each fused multiply-add rounds exactly as the
// canonical product-then-sum; dims are added in ascending order per head, and the
// weighted head terms (products of an fp32 weight and an fp64 dot, not exact) are
// rounded separately and added in ascending head order.
__global__ __launch_bounds__(FB_ROWS) void exact_fallback_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w, int L, int N,
    int topk, const int* __restrict__ fb_flag, double* __restrict__ scratch, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  __shared__ double qd[IH * ID];
  __shared__ float wrow[IH];
  __shared__ int hist[256];
  __shared__ int misc[4];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double* sc = scratch + (size_t)blockIdx.x * N;
  // this block's rows i = blockIdx.x + gridDim.x e: all flags read at once first, so a
  // launch with no flagged row costs one load round trip
  int any = 0;
  for (int e = tid; (int)blockIdx.x + (int)gridDim.x * e < L; e += FB_ROWS) any |= fb_flag[blockIdx.x + gridDim.x * e];
  if (!__syncthreads_or(any)) return;
  for (int i = blockIdx.x; i < L; i += gridDim.x) {
    if (fb_flag[i] == 0) continue;
    const int nv = min(N, N - L + i + 1);
    __syncthreads();
    for (int e = tid; e < IH * ID; e += FB_ROWS) qd[e] = (double)bf_bits2f(q[(size_t)i * IH * ID + e]);
    if (tid < IH) wrow[tid] = w[(size_t)i * IH + tid];
    __syncthreads();
    // two keys per thread (n and n + FB_ROWS): every query value read from LDS feeds
    // four multiply-adds
    for (int n = tid; n < nv; n += 2 * FB_ROWS) {
      const int n2 = n + FB_ROWS < nv ? n + FB_ROWS : n;     // past the end: key n again, not stored
      const u32x4* kr0 = (const u32x4*)(k + (size_t)n * ID);
      const u32x4* kr1 = (const u32x4*)(k + (size_t)n2 * ID);
      double d0[IH], d1[IH];
#pragma unroll
      for (int h = 0; h < IH; ++h) d0[h] = d1[h] = 0.0;
      // 16-dim chunks: the 64 head dots, the chunk of both keys in fp64 and the query
      // reads stay within the vector registers (32-dim chunks spilled); the next
      // chunk's key loads are in flight while this one is multiplied
      u32x4 kn0[FB_CHUNK / 8], kn1[FB_CHUNK / 8];
#pragma unroll
      for (int x = 0; x < FB_CHUNK / 8; ++x) {
        kn0[x] = kr0[x];
        kn1[x] = kr1[x];
      }
#pragma unroll
      for (int c0 = 0; c0 < ID; c0 += FB_CHUNK) {
        u32x4 kw0[FB_CHUNK / 8], kw1[FB_CHUNK / 8];
#pragma unroll
        for (int x = 0; x < FB_CHUNK / 8; ++x) {
          kw0[x] = kn0[x];
          kw1[x] = kn1[x];
        }
        if (c0 + FB_CHUNK < ID) {
#pragma unroll
          for (int x = 0; x < FB_CHUNK / 8; ++x) {
            kn0[x] = kr0[(c0 + FB_CHUNK) / 8 + x];
            kn1[x] = kr1[(c0 + FB_CHUNK) / 8 + x];
          }
        }
        double kd0[FB_CHUNK], kd1[FB_CHUNK];
#pragma unroll
        for (int e = 0; e < FB_CHUNK; ++e) {
          const uint32_t w0 = kw0[e / 8][(e % 8) / 2], w1 = kw1[e / 8][(e % 8) / 2];
          kd0[e] = (double)bf_bits2f((uint16_t)((e & 1) ? (w0 >> 16) : (w0 & 0xFFFFu)));
          kd1[e] = (double)bf_bits2f((uint16_t)((e & 1) ? (w1 >> 16) : (w1 & 0xFFFFu)));
        }
        const double* qc = qd + c0;
#pragma unroll
        for (int h = 0; h < IH; ++h)
#pragma unroll
          for (int e = 0; e < FB_CHUNK; e += 2) {
            const double2 qq = *(const double2*)(qc + h * ID + e);
            d0[h] = __builtin_fma(qq.x, kd0[e], d0[h]);
            d1[h] = __builtin_fma(qq.x, kd1[e], d1[h]);
            d0[h] = __builtin_fma(qq.y, kd0[e + 1], d0[h]);
            d1[h] = __builtin_fma(qq.y, kd1[e + 1], d1[h]);
          }
      }
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int h = 0; h < IH; ++h) {
        s0 = s0 + dmul_rounded((double)wrow[h], d0[h] > 0.0 ? d0[h] : 0.0);
        s1 = s1 + dmul_rounded((double)wrow[h], d1[h] > 0.0 ? d1[h] : 0.0);
      }
      sc[n] = s0 + 0.0;                 // -0 -> +0: one bit pattern per value
      if (n + FB_ROWS < nv) sc[n + FB_ROWS] = s1 + 0.0;
    }
    __syncthreads();
    const int kk = min(topk, nv);
    // exact k-th largest by 8-bit digits of the order-preserving image of the bit
    // pattern (weights of either sign give scores of either sign)
    auto ord64 = [](double d) -> unsigned long long {
      const unsigned long long u = (unsigned long long)__double_as_longlong(d);
      return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    };
    unsigned long long prefix = 0, pmask = 0;
    int need = kk;
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      // lanes of a wave that share the first active lane's digit add once (a row of
      // equal scores would otherwise put every lane's atomic on one bin)
      for (int n0 = 0; n0 < nv; n0 += FB_ROWS) {
        const int n = n0 + tid;
        const unsigned long long u = n < nv ? ord64(sc[n]) : 0ull;
        const bool act = n < nv && (u & pmask) == prefix;
        const int dig = (int)((u >> shift) & 255ull);
        const unsigned long long am = __ballot(act);
        if (am) {
          const int first = __ffsll((long long)am) - 1;
          const int d0 = __shfl(dig, first);
          const unsigned long long same = __ballot(act && dig == d0);
          if (lane == first) atomicAdd(&hist[d0], (int)__popcll(same));
          if (act && dig != d0) atomicAdd(&hist[dig], 1);
        }
      }
      __syncthreads();
      if (tid < 64) {
        const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const int own = h0 + h1 + h2 + h3;
        int suf = own;
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_down(suf, off);
          if (lane + off < 64) suf += v;
        }
        const int above = suf - own;
        if (above < need && suf >= need) {
          int acc = above, digit, above_d;
          if (acc + h3 >= need) { digit = 4 * lane + 3; above_d = acc; }
          else { acc += h3;
            if (acc + h2 >= need) { digit = 4 * lane + 2; above_d = acc; }
            else { acc += h2;
              if (acc + h1 >= need) { digit = 4 * lane + 1; above_d = acc; }
              else { acc += h1; digit = 4 * lane; above_d = acc; } } }
          misc[0] = digit;
          misc[1] = above_d;
        }
      }
      __syncthreads();
      prefix |= (unsigned long long)misc[0] << shift;
      pmask |= 255ull << shift;
      need -= misc[1];
      __syncthreads();
    }
    const double kth = __longlong_as_double((long long)((prefix >> 63) ? (prefix & 0x7FFFFFFFFFFFFFFFull) : ~prefix));
    // keys with s > kth are in; of those equal to kth, the `need` lowest indices are in
    int base = 0, eq_taken = 0;
    int32_t* orow = idx_out + (size_t)i * topk;
    float* srow = score_out ? score_out + (size_t)i * topk : nullptr;
    for (int c0 = 0; c0 < nv; c0 += FB_ROWS) {
      const int n = c0 + tid;
      const double s = n < nv ? sc[n] : -INFINITY;
      const bool gt = n < nv && s > kth;
      const bool eq = n < nv && s == kth;
      const unsigned long long meq = __ballot(eq);
      if (lane == 0) wave_tot[wave] = __popcll(meq);
      __syncthreads();
      int eq_before = eq_taken;
      for (int x = 0; x < wave; ++x) eq_before += wave_tot[x];
      eq_before += __popcll(meq & ((1ull << lane) - 1ull));
      const int eq_all = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
      __syncthreads();
      const bool keep = gt || (eq && eq_before < need);
      const unsigned long long mk = __ballot(keep);
      if (lane == 0) wave_tot[wave] = __popcll(mk);
      __syncthreads();
      int off = base;
      for (int x = 0; x < wave; ++x) off += wave_tot[x];
      if (keep) {
        const int pos = off + __popcll(mk & ((1ull << lane) - 1ull));
        if (pos < topk) {
          orow[pos] = n;
          if (srow) srow[pos] = (float)s;
        }
      }
      base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
      eq_taken += eq_all;
      __syncthreads();
    }
    for (int e = base + tid; e < topk; e += FB_ROWS) {
      orow[e] = -1;
      if (srow) srow[e] = -INFINITY;
    }
  }
}

// ---------------------------------------------------------------- host side
IndexerPlan indexer_plan(int L, int N, int topk, int block) {
  IndexerPlan pl;
  const int groups = L > 0 ? (L + QPB - 1) / QPB : 1;
  int ns = (256 + groups - 1) / groups;
  const int blk = block > 0 ? block : 4096;
  const int max_by_n = (N + blk - 1) / blk;
  ns = ns < 1 ? 1 : ns;
  ns = ns > 3 ? 3 : ns;                 // the refine kernel holds nsplit * cap candidates in LDS
  ns = ns > max_by_n ? max_by_n : ns;
  if (ns < 1) ns = 1;
  // 16-bit key offsets (and a 4-stage ring) when every split spans at most 65536 keys
  const int ns16 = (N + 65535) / 65536;
  if (ns16 <= 3 && ns < ns16) ns = ns16;
  int span = (N + ns - 1) / ns;
  span = (span + TK - 1) / TK * TK;
  pl.nsplit = ns;
  pl.span = span;
  pl.small_off = span <= 65536;
  pl.nstage = 1;
  // candidate capacity: what the LDS holds after the ring, per query, in multiples of 64
  pl.cap = pl.small_off ? FilterCap<uint16_t>::value : FilterCap<int>::value;
  // the refine kernel holds nsplit * cap candidates (SR_MAX at most, in registers)
  const int cap_sel = SR_MAX / ns / 64 * 64;
  if (pl.cap > cap_sel) pl.cap = cap_sel;
  {
    // Long contexts use the global-list kernel, whose lists live in memory and are
    // bounded only by what the refine kernel holds (cap_sel per split). It is chosen
    // when every query group gets the sampled start and the expected candidate count,
    // k + 6 sqrt(k nv / S) + 8 nv / S (the keys above the rk-th largest of S samples),
    // stays under 60% of that capacity; a list that still overflows costs its query
    // the exact fallback.
    const int nv0 = L > 0 ? std::min(N, N - L + 1) : N;
    const double mean = (double)topk * SAMPLE / std::max(nv0, 1);
    auto expect_of = [&](int S) { return topk + 6.0 * std::sqrt((double)topk * nv0 / S) + 8.0 * nv0 / S; };
    const double expect = expect_of(SAMPLE);
    auto fits = [&](int n_s, int c_sel) {
      return L > 0 && nv0 >= 8 * SAMPLE && mean <= SAMPLE / 8 && SAMPLE <= c_sel &&
             expect <= 0.6 * (double)n_s * c_sel;
    };
    pl.global_lists = fits(ns, cap_sel);
    if (pl.global_lists) {
      pl.cap = cap_sel;
      // The list kernel takes GQ queries per workgroup: more splits (up to the four
      // the refine kernel merges) until the launch has a workgroup per compute unit.
      const int lgroups = (L + GQ - 1) / GQ;
      int ns_l = (256 + lgroups - 1) / lgroups;
      ns_l = std::min(std::min(ns_l, 4), max_by_n);
      const int cap_l = SR_MAX / std::max(ns_l, 1) / 64 * 64;
      if (ns_l > ns && fits(ns_l, cap_l)) {
        ns = ns_l;
        span = ((N + ns - 1) / ns + TK - 1) / TK * TK;
        pl.nsplit = ns;
        pl.span = span;
        pl.small_off = span <= 65536;
        pl.cap = cap_l;
      }
      // Every key split of a group scores the same sample, so a smaller one shortens
      // the prologue; its start is looser (more candidates: a list past its capacity
      // costs the query the exact fallback), so it is taken only when even its
      // expected count leaves the lists at most 40% full.
      pl.sample = expect_of(SAMPLE_SMALL) <= 0.4 * (double)ns * pl.cap ? SAMPLE_SMALL : SAMPLE;
    }
  }
  pl.fb_blocks = L < FB_BLOCKS ? L : FB_BLOCKS;
  if (pl.fb_blocks < 1) pl.fb_blocks = 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  pl.off_partial = take(sizeof(float) * NORM_BLOCKS);
  pl.off_eps = take(sizeof(float) * (size_t)L);
  pl.off_cand_n = take(sizeof(int) * (size_t)L * ns);
  pl.off_cand_t = take(sizeof(float) * (size_t)L * ns);
  pl.off_fb = take(sizeof(int) * (size_t)L);
  pl.off_cand_s = take(sizeof(float) * (size_t)L * ns * pl.cap);
  pl.off_cand_i = take(sizeof(int) * (size_t)L * ns * pl.cap);
  // the fallback's scratch rows reuse the candidate lists, which select_refine has
  // consumed by the time the fallback runs (same stream)
  pl.off_scratch = pl.off_cand_s;
  {
    const size_t scratch_end = pl.off_scratch + (sizeof(double) * (size_t)pl.fb_blocks * N + 255) / 256 * 256;
    if (scratch_end > off) off = scratch_end;
  }
  pl.ws_bytes = off;
  pl.filter_lds = 0;                    // all LDS of the score and refine kernels is static
  pl.select_lds = 0;
  return pl;
}

hipError_t launch_indexer(const IndexerPlan& pl, const uint16_t* q, const uint16_t* k, const float* w, int L, int N,
                          int topk, int32_t* idx_out, float* score_out, void* ws, hipStream_t stream) {
  unsigned char* base = (unsigned char*)ws;
  float* partial = (float*)(base + pl.off_partial);
  float* eps = (float*)(base + pl.off_eps);
  int* cand_n = (int*)(base + pl.off_cand_n);
  float* cand_t = (float*)(base + pl.off_cand_t);
  int* fb = (int*)(base + pl.off_fb);
  float* cand_s = (float*)(base + pl.off_cand_s);
  int* cand_i = (int*)(base + pl.off_cand_i);
  double* scratch = (double*)(base + pl.off_scratch);
  {
    KernelTrace kt("key_norm_partial", stream);
    hipLaunchKernelGGL(key_norm_partial_kernel, dim3(NORM_BLOCKS), dim3(256), 0, stream, k, N, partial);
  }
  {
    KernelTrace kt("query_eps", stream);
    hipLaunchKernelGGL(query_eps_kernel, dim3(L), dim3(64), 0, stream, q, w, partial, NORM_BLOCKS, L, eps);
  }
  {
    KernelTrace kt("indexer_score_filter", stream);
    const dim3 grid((L + QPB - 1) / QPB, pl.nsplit), block(64 * IDX_NW);
    if (pl.global_lists)
      hipLaunchKernelGGL(pl.sample == SAMPLE_SMALL ? score_list_kernel<SAMPLE_SMALL> : score_list_kernel<SAMPLE>,
                         dim3((L + GQ - 1) / GQ, pl.nsplit), dim3(64 * GW), 0, stream, q, k, w, eps, L, N, topk,
                         pl.span, pl.nsplit, pl.cap, cand_s, cand_i, cand_n, cand_t);
    else if (pl.small_off)
      hipLaunchKernelGGL((score_filter_kernel<uint16_t>), grid, block, 0, stream, q, k, w, eps, L, N,
                         topk, pl.span, pl.nsplit, pl.cap, cand_s, cand_i, cand_n, cand_t);
    else
      hipLaunchKernelGGL((score_filter_kernel<int>), grid, block, 0, stream, q, k, w, eps, L, N, topk,
                         pl.span, pl.nsplit, pl.cap, cand_s, cand_i, cand_n, cand_t);
  }
  {
    KernelTrace kt("indexer_select_refine", stream);
    hipLaunchKernelGGL(select_refine_kernel, dim3(L), dim3(SR_T), 0, stream, q, k, w, eps, L, N, topk,
                       pl.nsplit, pl.cap, cand_s, cand_i, cand_n, cand_t, fb, idx_out, score_out);
  }
  {
    KernelTrace kt("indexer_exact_fallback", stream);
    hipLaunchKernelGGL(exact_fallback_kernel, dim3(pl.fb_blocks), dim3(FB_ROWS), 0, stream, q, k, w, L, N, topk, fb,
                       scratch, idx_out, score_out);
  }
  return hipGetLastError();
}

}  // namespace dsa

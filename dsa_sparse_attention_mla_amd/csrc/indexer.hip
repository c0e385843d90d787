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
//  1. key_norm_partial:   per-block max of ||k_n||^2 (fp32).
//  2. query_eps:          eps_i, a rigorous bound on |s_hat - s| for the fp32
//                         MFMA score s_hat, from sum_h w_h ||q_h|| * max_n ||k_n||.
//  3. score_filter:       32x32x16 bf16 MFMA scores for 32 heads; ReLU, weight and
//                         head sum in registers; every wave owns one query and keeps
//                         a candidate list in LDS of all keys with
//                         s_hat >= tau - band(tau), tau = the running k-th largest
//                         s_hat (found by an in-LDS radix select whenever the list
//                         fills up). Only candidates leave the chip.
//  4. select_refine:      per query, T = k-th largest s_hat among candidates.
//                         s_hat > T + band: in. s_hat < T - band: out. The keys in
//                         between are re-scored canonically in fp64 and ranked by
//                         (s desc, index asc) to fill the rest.
//  5. exact_fallback:     rows whose candidates overflowed (huge ties) are solved
//                         from the canonical fp64 score of every visible key.
// Output rows are in ascending key order, padded with -1.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int ID = 128;                 // indexer head dim
constexpr int IH = 32;                  // indexer heads
constexpr int TK = 64;                  // keys per tile
constexpr int IDX_STAGE = TK * ID * 2;  // one ring stage: 64 keys x 256 B (swizzled, unpadded)
constexpr int IDX_NSTAGE = 3;           // ring stages
constexpr int IDX_AHEAD = IDX_NSTAGE - 1;
constexpr int QPB = 4;                  // queries per workgroup, one per wave
constexpr int RANK_CAP = 1024;          // band entries ranked in select_refine
constexpr int NORM_BLOCKS = 256;
constexpr int FB_ROWS = 256;            // block size of the fallback kernel
}  // namespace

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Half-width of the uncertainty band around a threshold t (t >= 0): 2*eps plus
// a few ulps of t for the fp32 evaluation of t +- 2*eps. Increasing in t with
// slope < 1, so t1 <= t2 implies t1 - band(t1) <= t2 - band(t2).
__device__ __forceinline__ float band_halfwidth(float eps, float t) {
  return 2.0f * eps * 1.001f + fabsf(t) * 4.8e-7f;
}

// ---------------------------------------------------------------- 1. key norms
__global__ __launch_bounds__(256) void key_norm_partial_kernel(const uint16_t* __restrict__ k, int N,
                                                               float* __restrict__ partial) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid >> 4, l16 = tid & 15;   // 16 keys per pass, 16 lanes per key
  float mx = 0.f;
  for (int n = blockIdx.x * 16 + sub; n < N; n += gridDim.x * 16) {
    const u32x4 v = *(const u32x4*)(k + (size_t)n * ID + 8 * l16);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf_bits2f((uint16_t)(v[e] & 0xFFFFu)), b = bf_bits2f((uint16_t)(v[e] >> 16));
      acc += a * a + b * b;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
    mx = fmaxf(mx, acc);
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (tid == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------- 2. eps per query
// |fl(q.k) - q.k| <= gamma_128 * sum|q_c k_c| <= gamma_128 ||q|| ||k|| (any order,
// round-to-nearest or toward zero: u = 2^-23); the ReLU is 1-Lipschitz; the
// weight product and the 32-term head sum add (u + gamma_32) * sum_h w_h |d_h|.
// The constant below is that sum (1.92e-5) with a 30% margin for the fp32
// evaluation of the norms.
__global__ __launch_bounds__(64) void query_eps_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                       const float* __restrict__ partial, int nparts, int L,
                                                       float* __restrict__ eps) {
  const int i = blockIdx.x, lane = threadIdx.x;
  float km = 0.f;
  for (int b = lane; b < nparts; b += 64) km = fmaxf(km, partial[b]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) km = fmaxf(km, __shfl_xor(km, off));
  float contrib = 0.f;
  if (lane < IH) {
    const uint16_t* qh = q + ((size_t)i * IH + lane) * ID;
    float acc = 0.f;
    for (int c = 0; c < ID; ++c) {
      const float a = bf_bits2f(qh[c]);
      acc += a * a;
    }
    contrib = w[(size_t)i * IH + lane] * sqrtf(acc);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) contrib += __shfl_xor(contrib, off);
  if (lane == 0) eps[i] = 2.5e-5f * contrib * sqrtf(km * 1.0001f) * 1.0001f + 1e-30f;
}

// ---------------------------------------------------------------- 3. score + running candidates
// Wave-level radix select of the k-th largest non-negative float among n entries.
__device__ float wave_kth_largest(const float* vals, int n, int k, int* hist, int lane) {
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hist[b] = 0;
    wave_sync();
    for (int e = lane; e < n; e += 64) {
      const uint32_t u = __float_as_uint(vals[e]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    wave_sync();
    const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const int own = h0 + h1 + h2 + h3;
    int suf = own;  // inclusive suffix sum over lanes (higher lanes hold higher digits)
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
    digit = __shfl(digit, src);
    above_d = __shfl(above_d, src);
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    need -= above_d;
    wave_sync();
  }
  return __uint_as_float(prefix);
}

// Wait until at most n of this wave's vector-memory operations are outstanding.
__device__ __forceinline__ void idx_wait_vm(int n) {
  if (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}

// Keys stream through a ring of LDS stages filled by direct global->LDS loads,
// AHEAD tiles ahead of use. Within a stage, key r's 16-byte chunk c sits at chunk
// slot r*16 + (c ^ (r & 15)), so the 32 keys one MFMA operand read touches fall
// in distinct banks.
__global__ __launch_bounds__(256) void score_filter_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ eps_in, int L, int N, int topk, int span, int nsplit, int cap,
    float* __restrict__ cand_s, int* __restrict__ cand_i, int* __restrict__ cand_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  unsigned char* ring = dyn;                                          // [NSTAGE][TK*256]
  float* cs_all = (float*)(dyn + IDX_NSTAGE * IDX_STAGE);             // [QPB][cap]
  int* ci_all = (int*)(cs_all + QPB * cap);                           // [QPB][cap]
  int* hist_all = ci_all + QPB * cap;                                 // [QPB][256]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.y;
  const int n_lo = split * span;
  const int i = blockIdx.x * QPB + wave;
  const bool active = i < L;
  const int ii = active ? i : L - 1;
  const int p = N - L + ii;
  const int ilast = min(L - 1, (int)blockIdx.x * QPB + QPB - 1);
  const int n_hi = min(min(N, n_lo + span), N - L + ilast + 1);
  float* cs = cs_all + wave * cap;
  int* ci = ci_all + wave * cap;
  int* hist = hist_all + wave * 256;

  bf16x8 qa[ID / 16];
  {
    const uint16_t* qrow = q + ((size_t)ii * IH + (lane & 31)) * ID + 8 * (lane >> 5);
#pragma unroll
    for (int kc = 0; kc < ID / 16; ++kc) qa[kc] = *(const bf16x8*)(qrow + 16 * kc);
  }
  float wr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wr[j] = w[(size_t)ii * IH + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)];
  const float eps = eps_in[ii];
  float thr = -INFINITY;
  int cnt = 0;
  bool ovf = false;

  // 16 wave instructions of 64 x 16 B fill one stage; wave w issues blocks w, w+4, w+8, w+12
  auto issue_tile = [&](int n0, int s) {
    unsigned char* st = ring + s * IDX_STAGE;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int blk = wave + 4 * u;
      const int slot = blk * 64 + lane;
      const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
      const int n = min(n0 + r, n_hi - 1);          // keys past the range fetch a harmless row
      __builtin_amdgcn_global_load_lds((const void*)(k + (size_t)n * ID + c * 8),
                                       (DSA_LDS void*)(st + blk * 1024), 16, 0, 0);
    }
  };

  const int ntiles = n_hi > n_lo ? (n_hi - n_lo + TK - 1) / TK : 0;
  for (int t = 0; t < IDX_AHEAD && t < ntiles; ++t) issue_tile(n_lo + t * TK, t % IDX_NSTAGE);
  for (int t = 0; t < ntiles; ++t) {
    const int s = t % IDX_NSTAGE;
    const int n0 = n_lo + t * TK;
    idx_wait_vm(min(t + IDX_AHEAD - 1, ntiles - 1) - t);
    __syncthreads();
    if (t + IDX_AHEAD < ntiles) issue_tile(n0 + IDX_AHEAD * TK, (t + IDX_AHEAD) % IDX_NSTAGE);
    const unsigned char* st = ring + s * IDX_STAGE;
    float tot[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 acc = {};
      const int r = 32 * sub + (lane & 31);
      const unsigned char* kp = st + r * 256;
#pragma unroll
      for (int kc = 0; kc < ID / 16; ++kc) {
        const int c = (2 * kc + (lane >> 5)) ^ (r & 15);
        acc = mfma32x32x16(qa[kc], *(const bf16x8*)(kp + c * 16), acc);
      }
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) part = fmaf(wr[j], fmaxf(acc[j], 0.f), part);
      tot[sub] = part + __shfl_xor(part, 32);
    }
    if (active && !ovf) {
      const float sv = lane < 32 ? tot[0] : tot[1];
      const int key = n0 + lane;
      const bool keep = key < n_hi && key <= p && sv >= thr;
      const unsigned long long bm = __ballot(keep);
      if (keep) {
        const int pos = cnt + __popcll(bm & ((1ull << lane) - 1ull));
        cs[pos] = sv;
        ci[pos] = key;
      }
      cnt += __popcll(bm);
      if (cnt > cap - 64) {
        wave_sync();
        const float tau = wave_kth_largest(cs, cnt, topk, hist, lane);
        thr = fmaxf(thr, tau - band_halfwidth(eps, tau));
        int newc = 0;
        for (int base = 0; base < cnt; base += 64) {
          const int e = base + lane;
          const bool in = e < cnt;
          const float v = in ? cs[e] : 0.f;
          const int id = in ? ci[e] : 0;
          const bool kp2 = in && v >= thr;
          const unsigned long long m2 = __ballot(kp2);
          wave_sync();
          if (kp2) {
            const int pos = newc + __popcll(m2 & ((1ull << lane) - 1ull));
            cs[pos] = v;
            ci[pos] = id;
          }
          newc += __popcll(m2);
          wave_sync();
        }
        cnt = newc;
        if (cnt > cap - 64) ovf = true;
      }
    }
  }
  if (active) {
    const size_t slot = (size_t)i * nsplit + split;
    wave_sync();
    for (int e = lane; e < cnt; e += 64) {
      cand_s[slot * cap + e] = cs[e];
      cand_i[slot * cap + e] = ci[e];
    }
    if (lane == 0) cand_n[slot] = ovf ? -1 : cnt;
  }
}

// ---------------------------------------------------------------- 4. select + band refine
// Block-level (256 threads) radix select of the k-th largest non-negative float.
__device__ float block_kth_largest(const float* vals, int n, int k, int* hist, int* bcast) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int e = tid; e < n; e += 256) {
      const uint32_t u = __float_as_uint(vals[e]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      const int lane = tid;
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int own = h0 + h1 + h2 + h3;
      int suf = own;
#pragma unroll
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
        bcast[0] = digit;
        bcast[1] = above_d;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    pmask |= 255u << shift;
    need -= bcast[1];
    __syncthreads();
  }
  return __uint_as_float(prefix);
}

// Canonical fp64 score of key n for query i, computed by 32 lanes (one head
// each): d_h summed over dims in ascending order, then the head terms added in
// ascending head order. Every product and sum is a separate IEEE operation.
__device__ double canonical_score_32lanes(const uint16_t* qrow_lds, const uint16_t* __restrict__ k,
                                          const float* __restrict__ wrow, int n, int l32, int src_base) {
  const uint16_t* kr = k + (size_t)n * ID;
  const uint16_t* qh = qrow_lds + l32 * ID;
  double d = 0.0;
  for (int c = 0; c < ID; c += 8) {
    const u32x4 kv = *(const u32x4*)(kr + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t kb = (uint16_t)((kv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      d = __dadd_rn(d, __dmul_rn((double)bf_bits2f(qh[c + e]), (double)bf_bits2f(kb)));
    }
  }
  double s = 0.0;
  for (int h = 0; h < IH; ++h) {
    const double dh = __shfl(d, src_base + h);
    s = __dadd_rn(s, __dmul_rn((double)wrow[h], dh > 0.0 ? dh : 0.0));
  }
  return s;
}

__global__ __launch_bounds__(256) void select_refine_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ eps_in, int L, int N, int topk, int nsplit, int cap,
    const float* __restrict__ cand_s, const int* __restrict__ cand_i, const int* __restrict__ cand_n,
    int* __restrict__ fb_flag, int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  const int M_cap = nsplit * cap;
  float* vs = (float*)dyn;                       // [M_cap] candidate scores
  int* vi = (int*)(vs + M_cap);                  // [M_cap] candidate keys
  unsigned char* cls = (unsigned char*)(vi + M_cap);   // [M_cap] 0 out, 1 in, 2 band
  short* bid = (short*)(cls + ((M_cap + 15) & ~15));   // [M_cap] band id
  double* bscore = (double*)(bid + ((M_cap + 7) & ~7)); // [RANK_CAP]
  int* bkey = (int*)(bscore + RANK_CAP);          // [RANK_CAP]
  unsigned char* bsel = (unsigned char*)(bkey + RANK_CAP);  // [RANK_CAP]
  uint16_t* qrow = (uint16_t*)(bsel + RANK_CAP);  // [IH*ID]
  int* hist = (int*)(qrow + IH * ID);             // [256]
  int* misc = hist + 256;                         // [8]
  int* wave_tot = misc + 8;                       // [4]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.x;
  const int p = N - L + i;
  const int nv = min(N, p + 1);
  int32_t* orow = idx_out + (size_t)i * topk;
  float* srow = score_out ? score_out + (size_t)i * topk : nullptr;

  // gather candidate lists (ascending key order within and across splits)
  int M = 0;
  bool overflow = false;
  for (int sp = 0; sp < nsplit; ++sp) {
    const int c = cand_n[(size_t)i * nsplit + sp];
    if (c < 0) { overflow = true; break; }
    const float* src_s = cand_s + ((size_t)i * nsplit + sp) * cap;
    const int* src_i = cand_i + ((size_t)i * nsplit + sp) * cap;
    for (int e = tid; e < c; e += 256) { vs[M + e] = src_s[e]; vi[M + e] = src_i[e]; }
    M += c;
  }
  if (overflow) {
    if (tid == 0) fb_flag[i] = 1;
    return;
  }
  if (tid == 0) fb_flag[i] = 0;
  __syncthreads();

  const float eps = eps_in[i];
  int need_band = 0;
  float tk = 0.f;
  if (nv <= topk) {
    // every visible key is in the list (the filter threshold never rose)
    for (int e = tid; e < M; e += 256) cls[e] = 1;
  } else {
    tk = block_kth_largest(vs, M, topk, hist, misc);
    const float hw = band_halfwidth(eps, tk);
    const float hi = tk + hw, lo = tk - hw;
    if (tid == 0) { misc[2] = 0; misc[3] = 0; }
    __syncthreads();
    for (int e = tid; e < M; e += 256) {
      const float v = vs[e];
      unsigned char c = 0;
      if (v > hi) { c = 1; atomicAdd(&misc[2], 1); }
      else if (v >= lo) {
        c = 2;
        const int b = atomicAdd(&misc[3], 1);
        if (b < RANK_CAP) { bid[e] = (short)b; bkey[b] = vi[e]; }
      }
      cls[e] = c;
    }
    __syncthreads();
    const int n_in = misc[2], nb = misc[3];
    need_band = topk - n_in;
    if (nb > RANK_CAP || need_band < 0 || need_band > nb) {
      if (tid == 0) fb_flag[i] = 1;
      return;
    }
    // stage the query (bf16) for the canonical re-score
    for (int e = tid; e < IH * ID / 8; e += 256)
      *(u32x4*)(qrow + 8 * e) = *(const u32x4*)(q + (size_t)i * IH * ID + 8 * e);
    __syncthreads();
    const float* wrow = w + (size_t)i * IH;
    const int half = lane >> 5, l32 = lane & 31;
    for (int b0 = wave * 2; b0 < nb; b0 += 8) {
      const int b = b0 + half;
      const int n = b < nb ? bkey[b] : bkey[0];
      const double s = canonical_score_32lanes(qrow, k, wrow, n, l32, half * 32);
      if (b < nb && l32 == 0) bscore[b] = s;
    }
    __syncthreads();
    for (int b = tid; b < nb; b += 256) {
      const double s = bscore[b];
      const int key = bkey[b];
      int r = 0;
      for (int o = 0; o < nb; ++o) {
        const double so = bscore[o];
        r += (so > s) || (so == s && bkey[o] < key);
      }
      bsel[b] = r < need_band;
    }
    __syncthreads();
  }

  // stable compaction of kept candidates, in candidate (= ascending key) order
  int base = 0;
  for (int c0 = 0; c0 < M; c0 += 256) {
    const int e = c0 + tid;
    bool keep = false;
    if (e < M) keep = cls[e] == 1 || (cls[e] == 2 && bsel[bid[e]]);
    const unsigned long long bm = __ballot(keep);
    if (lane == 0) wave_tot[wave] = __popcll(bm);
    __syncthreads();
    int off = base;
    for (int x = 0; x < wave; ++x) off += wave_tot[x];
    if (keep) {
      const int pos = off + __popcll(bm & ((1ull << lane) - 1ull));
      if (pos < topk) {
        orow[pos] = vi[e];
        if (srow) srow[pos] = vs[e];
      }
    }
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  for (int e = base + tid; e < topk; e += 256) {
    orow[e] = -1;
    if (srow) srow[e] = -INFINITY;
  }
}

// ---------------------------------------------------------------- 5. exact fallback
// One workgroup per flagged row at a time; the canonical fp64 score of every
// visible key goes to a per-workgroup scratch row, then an exact 64-bit radix
// select finds the k-th largest value and a stable scan emits the set.
__global__ __launch_bounds__(FB_ROWS) void exact_fallback_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w, int L, int N,
    int topk, const int* __restrict__ fb_flag, double* __restrict__ scratch, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  __shared__ uint16_t qrow[IH * ID];
  __shared__ float wrow[IH];
  __shared__ int hist[256];
  __shared__ int misc[4];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double* sc = scratch + (size_t)blockIdx.x * N;
  for (int i = blockIdx.x; i < L; i += gridDim.x) {
    if (fb_flag[i] == 0) continue;
    const int nv = min(N, N - L + i + 1);
    __syncthreads();
    for (int e = tid; e < IH * ID; e += FB_ROWS) qrow[e] = q[(size_t)i * IH * ID + e];
    if (tid < IH) wrow[tid] = w[(size_t)i * IH + tid];
    __syncthreads();
    for (int n = tid; n < nv; n += FB_ROWS) {
      const uint16_t* kr = k + (size_t)n * ID;
      double s = 0.0;
      for (int h = 0; h < IH; ++h) {
        double d = 0.0;
        for (int c = 0; c < ID; ++c) d = __dadd_rn(d, __dmul_rn((double)bf_bits2f(qrow[h * ID + c]), (double)bf_bits2f(kr[c])));
        s = __dadd_rn(s, __dmul_rn((double)wrow[h], d > 0.0 ? d : 0.0));
      }
      sc[n] = s;
    }
    __syncthreads();
    const int kk = min(topk, nv);
    // exact k-th largest of non-negative doubles by 8-bit digits of the bit pattern
    unsigned long long prefix = 0, pmask = 0;
    int need = kk;
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int n = tid; n < nv; n += FB_ROWS) {
        const unsigned long long u = (unsigned long long)__double_as_longlong(sc[n]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255ull], 1);
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
    const double kth = __longlong_as_double((long long)prefix);
    // keys with s > kth are in; of those equal to kth, the `need` lowest indices are in
    int base = 0, eq_taken = 0;
    int32_t* orow = idx_out + (size_t)i * topk;
    float* srow = score_out ? score_out + (size_t)i * topk : nullptr;
    for (int c0 = 0; c0 < nv; c0 += FB_ROWS) {
      const int n = c0 + tid;
      const double s = n < nv ? sc[n] : -1.0;
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
  int span = (N + ns - 1) / ns;
  span = (span + TK - 1) / TK * TK;
  pl.nsplit = ns;
  pl.span = span;
  pl.cap = 3456;                        // (160 KiB - ring - histograms) / (4 queries x 8 B)
  pl.fb_blocks = L < 32 ? L : 32;
  if (pl.fb_blocks < 1) pl.fb_blocks = 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  pl.off_partial = take(sizeof(float) * NORM_BLOCKS);
  pl.off_eps = take(sizeof(float) * (size_t)L);
  pl.off_cand_n = take(sizeof(int) * (size_t)L * ns);
  pl.off_fb = take(sizeof(int) * (size_t)L);
  pl.off_cand_s = take(sizeof(float) * (size_t)L * ns * pl.cap);
  pl.off_cand_i = take(sizeof(int) * (size_t)L * ns * pl.cap);
  pl.off_scratch = take(sizeof(double) * (size_t)pl.fb_blocks * N);
  pl.ws_bytes = off;
  pl.filter_lds = IDX_NSTAGE * IDX_STAGE + QPB * pl.cap * 8 + QPB * 256 * 4;
  const size_t M = (size_t)ns * pl.cap;
  pl.select_lds = M * 4 + M * 4 + ((M + 15) & ~(size_t)15) + ((M + 7) & ~(size_t)7) * 2 + RANK_CAP * 8 + RANK_CAP * 4 +
                  RANK_CAP + IH * ID * 2 + 256 * 4 + 8 * 4 + 4 * 4;
  return pl;
}

hipError_t launch_indexer(const IndexerPlan& pl, const uint16_t* q, const uint16_t* k, const float* w, int L, int N,
                          int topk, int32_t* idx_out, float* score_out, void* ws, hipStream_t stream) {
  unsigned char* base = (unsigned char*)ws;
  float* partial = (float*)(base + pl.off_partial);
  float* eps = (float*)(base + pl.off_eps);
  int* cand_n = (int*)(base + pl.off_cand_n);
  int* fb = (int*)(base + pl.off_fb);
  float* cand_s = (float*)(base + pl.off_cand_s);
  int* cand_i = (int*)(base + pl.off_cand_i);
  double* scratch = (double*)(base + pl.off_scratch);
  hipError_t e;
  static bool attr_set = false;
  if (!attr_set) {
    e = hipFuncSetAttribute((const void*)score_filter_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)select_refine_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
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
    hipLaunchKernelGGL(score_filter_kernel, dim3((L + QPB - 1) / QPB, pl.nsplit), dim3(256), pl.filter_lds, stream, q,
                       k, w, eps, L, N, topk, pl.span, pl.nsplit, pl.cap, cand_s, cand_i, cand_n);
  }
  {
    KernelTrace kt("indexer_select_refine", stream);
    hipLaunchKernelGGL(select_refine_kernel, dim3(L), dim3(256), pl.select_lds, stream, q, k, w, eps, L, N, topk,
                       pl.nsplit, pl.cap, cand_s, cand_i, cand_n, fb, idx_out, score_out);
  }
  {
    KernelTrace kt("indexer_exact_fallback", stream);
    hipLaunchKernelGGL(exact_fallback_kernel, dim3(pl.fb_blocks), dim3(FB_ROWS), 0, stream, q, k, w, L, N, topk, fb,
                       scratch, idx_out, score_out);
  }
  return hipGetLastError();
}

}  // namespace dsa

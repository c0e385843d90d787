// Dense absorbed MLA prefill over a contiguous joined latent+rope cache, and the
// same attention under each query's top-k selection bitmap.
//
//  * Dense: "Sparse prefill for GLM", section "Sparse attention" -- attention in
//    the absorbed latent space over one 576-wide row per position (512 latent +
//    64 rope) that all heads share, the value being the latent part of the row;
//    every key up to the query's causal limit is visited.
//  * Masked: same page, section "The dense mask" -- the path the sparse one
//    replaces: every visible key is visited and only the keys the query's top-k
//    selection marks in a bitmap get weight.
//
// Work decomposition (gfx950). All heads of all queries read the same rows, so a
// workgroup takes 128 (query, head) rows -- two queries of 64 heads -- and every
// staged key tile feeds all of them. Four waves, one per SIMD (512 registers each);
// wave w owns 32 rows, the 32 columns of 32x32x16 bf16 MFMAs, and does all of their
// work:
//   S^T[32 keys x 32 rows] = K_tile[32 x 576] . Q^T[576 x 32]   (36 k-steps; Q^T in
//                                                  vector registers, K from LDS)
//   softmax per column (a column's 32 keys sit in lanes l and l + 32)
//   O^T[512 x 32] += V_tile^T[512 x 32 keys] . P^T[32 keys x 32]  (16 dim blocks x 2
//                                                  k-steps; V^T by transpose reads)
// Every operand fragment read from LDS (1 KB) feeds a 32-cycle MFMA, so at full MFMA
// rate the CU reads 128 bytes of LDS per clock, half of what it can deliver.
// Registers: O^T takes all 256 accumulation registers; the score accumulators must
// then live in vector registers, so the score MFMAs are issued through inline
// assembly with vector-register operands (the compiler would place every MFMA result
// in the accumulation registers and shuffle O^T to make room), with the wait states
// the ISA requires before a vector instruction may read an MFMA result written in
// explicitly. Q^T (144 registers), both score tiles and the operand prefetch fill the
// vector registers.
// Each wave overlaps its own work: the 36 score MFMAs of tile t+1 run while the
// vector unit turns the scores of tile t into bf16 weights, then the 32 value MFMAs
// of tile t run while it forms the exponent arguments of tile t+1. Key tiles arrive
// by direct global->LDS loads into a ring of four stages, issued three tiles ahead
// between the value MFMAs; one barrier per tile.
// Softmax reference: softmax does not depend on the number subtracted before the
// exponential, and weights up to 2^64 (or down to 2^-64 of the row's largest) lose
// nothing in fp32/bf16, so a row's weights are taken against the maximum of its first
// tile and never rescaled; the row's true maximum is tracked on the side. If it ends
// more than 64 (log2 units) above or below the reference, the whole row block runs
// again with the true maximum as reference (inputs with such score ranges only).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int D = 576;                  // joined row: 512 latent + 64 rope
constexpr int DV = 512;                 // value = latent part of the row
constexpr int T = 32;                   // keys per tile
constexpr int ROWCH = D * 2 / 16 + 1;   // 16-byte chunks per padded LDS row (72 + 1)
constexpr int ROWB = ROWCH * 16;        // 1168 bytes
constexpr int NCH = T * ROWCH;          // chunks of a stage's rows (2336)
constexpr int NLD = (NCH + 63) / 64;    // 1 KB direct loads per stage (37; the last one half)
constexpr int STAGE = NLD * 1024;       // 37888 bytes per stage: 32 rows and the tail of the last load
constexpr int NST = 4;                  // stages: tile t (values), t+1 (scores), t+2 and t+3 landing
constexpr int NWV = 4;                  // waves, one per SIMD
constexpr int LPW = (NLD + NWV - 1) / NWV;   // loads per wave per tile (10; spare ones go to a dump area)
constexpr int KS = D / 16;              // 32x32x16 k-steps of the score (36)
constexpr int NDB = DV / 32;            // 32-dim value blocks (16)
constexpr int ROWS = 32 * NWV;          // (query, head) rows per workgroup (128)
constexpr int PDK = 5;                  // K fragment reads in flight
constexpr int PDV = 3;                  // V^T fragments (two transpose reads each) in flight
constexpr float SPAN = 64.f;            // largest |log2| of a weight relative to the row's largest one
constexpr size_t DUMP_OFF = (size_t)NST * STAGE;          // 1 KB target of the spare loads
constexpr size_t MASK_OFF = DUMP_OFF + 1024;               // [NST][waves][2] selection words
constexpr size_t FLAG_OFF = MASK_OFF + NST * NWV * 2 * 4;  // [waves] second-pass votes
constexpr size_t LDS_BYTES = FLAG_OFF + NWV * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");

// Score accumulator row c = 4m + e (m < 8, e < 4) holds tile row krow(c) =
// m%4 + 4e + 16(m/4): the four rows one transpose read of V^T covers are then four
// apart, and with 1168-byte rows both that read and the K fragment read (32 rows at
// one column) run without bank conflicts (measured with the conflict counter).
__device__ __forceinline__ int krow(int c) { return ((c >> 2) & 3) + 4 * (c & 3) + 16 * (c >> 4); }
// Tile row of element j (of 16) of lane half `up` of a score accumulator (its row is
// c = 8 (j/4) + 4 up + j%4).
__device__ __forceinline__ int key_of_elem(int j, int up) { return up + 2 * ((j >> 2) & 1) + 4 * (j & 3) + 16 * (j >> 3); }

// 4-byte direct global->LDS load: lane l writes LDS bytes [m0 + 4 l, m0 + 4 l + 4).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// Score MFMAs with the accumulator in vector registers. The leading s_nop covers a
// vector instruction that may have written an A/B operand just before.
__device__ __forceinline__ void score_mfma_first(f32x16& s, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma(f32x16& s, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
// After the last score MFMA of a tile: more wait states than an XDL result needs
// before a vector instruction reads or overwrites it.
__device__ __forceinline__ void score_settle(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// Elements 8 h .. 8 h + 7 of a score tile as bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_half(const f32x16& x, int h) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 v = h ? __builtin_shufflevector(x, x, 8, 9, 10, 11, 12, 13, 14, 15)
                    : __builtin_shufflevector(x, x, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_convertvector(v, bf16x8);
}

// Sum of the eight bf16 values of v in fp32 added to acc: dot products with (1, 1)
// pairs. The pairs are taken with a vector shuffle (taking them through a 32-bit
// reinterpretation of the packed vector is miscompiled by the current compiler: every
// pair becomes the first).
__device__ __forceinline__ float sum8_dot(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}
}  // namespace

// MASKED: weight only the keys the row's query has set in its selection bitmap
// (mask [B][L][ceil(N/32)] words, bit n%32 of word n/32 for key n).
template <bool MASKED>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(1, 1))) void absorbed_dense_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint32_t* __restrict__ mask,
    uint16_t* __restrict__ out, int L, int N, int H, int causal, float scale_log2) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, up = lane >> 5;                // MFMA column (row of the wave), lane half
  const int b = blockIdx.y;
  const int nrows = L * H;
  const int r0 = blockIdx.x * ROWS;
  const int row = r0 + 32 * wave + l32;                     // this lane's (query, head) row
  const bool row_ok = row < nrows;
  const int qi = (row_ok ? row : nrows - 1) / H, hd = (row_ok ? row : nrows - 1) % H;
  const int lim = causal ? N - L + qi : N - 1;              // last key this row sees
  // keys the workgroup visits: up to the limit of its last row
  const int qlast = (min(nrows, r0 + ROWS) - 1) / H;
  const int count = causal ? N - L + qlast + 1 : N;
  const int ntiles = (count + T - 1) / T;
  // the wave's smallest limit (rows ascend with the column; lane 0 of a wave past the
  // last row takes the last row's)
  const int lim_min = __builtin_amdgcn_readfirstlane(lim);
  const uint16_t* kvb = kv + (size_t)b * N * D;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(DSA_LDS void*)lds;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // ---- tile loads: stage chunk c (16 bytes) is chunk c % ROWCH of row c / ROWCH (71
  // data chunks and the padding, which loads the row's last data chunk again; chunks
  // past the 32 rows load row 31 into the stage's tail); load j (1 KB) covers chunks
  // 64 j .. 64 j + 63 and wave w issues loads w, w + 4, ...; the spare loads past the
  // 37th go to a dump area, so every wave issues the same number of loads per tile and
  // the waits below are exact. Rows past the last key repeat it (their scores are
  // masked).
  static_assert(NLD <= NWV * LPW, "every load has a wave");
  // selection words of this wave's (at most two) queries: lanes 0 and 1
  const int qw0 = min(r0 + 32 * wave, nrows - 1) / H;
  const int qw1 = min(r0 + 32 * wave + 31, nrows - 1) / H;
  const int W = (N + 31) / 32;
  const uint32_t* mrow = MASKED ? mask + ((size_t)b * L + (lane == 0 ? qw0 : qw1)) * W : nullptr;
  // Byte offset of this lane's chunk of load slot s within a whole tile, fixed for the
  // kernel; a tile with fewer key rows clamps it to the last chunk of its last key row.
  uint32_t soff[LPW];
#pragma unroll
  for (int s = 0; s < LPW; ++s) {
    const int c = 64 * (NWV * s + wave_u) + lane, r = c / ROWCH;
    soff[s] = (uint32_t)(min(r, T - 1) * D * 2 + 16 * min(c - r * ROWCH, D * 2 / 16 - 1));
  }
  // Tile t's loads go to stage st. Every step issues one tile's loads, also past the
  // last tile (then the last tile again, into a stage nobody reads), so the number of
  // loads in flight is the same on every path; no branch, no per-load arithmetic but a
  // minimum.
  auto load_part = [&](int t, int st, int s) {
    const int rlim = min(count - 1 - t * T, T - 1);         // last row of the tile that is a key
    const void* base = uniform_ptr(kvb + (size_t)t * T * D);
    const int j = NWV * s + wave_u;
    const uint32_t dst = j < NLD ? lds0 + st * STAGE + 1024 * j : lds0 + (uint32_t)DUMP_OFF;
    dma16s(base, min(soff[s], (uint32_t)(rlim * D * 2 + 16 * (D * 2 / 16 - 1))), dst);
  };
  auto load_mask = [&](int t, int st) {
    if constexpr (MASKED) {
      if (lane < 2) dma4(mrow + t, lds0 + (uint32_t)(MASK_OFF + (st * NWV + wave_u) * 8));
    }
  };
  auto load_tile = [&](int t, int st) {
#pragma unroll
    for (int s = 0; s < LPW; ++s) load_part(t, st, s);
    load_mask(t, st);
  };
  constexpr int LPT = LPW + (MASKED ? 1 : 0);              // loads per wave per tile
  // wait until at most n tiles' loads of this wave are in flight
  auto wait_tiles = [&](int n) {
    if (n >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT) : "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPT) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- Q^T fragments: lane (up, l32) holds row l32, dims 16 kc + 8 up .. +8
  bf16x8 qt[KS];
  {
    const uint16_t* qrow = q + (((size_t)b * L + qi) * H + hd) * D + 8 * up;
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) qt[kc] = *(const bf16x8*)(qrow + 16 * kc);
    if (!row_ok) {
#pragma unroll
      for (int kc = 0; kc < KS; ++kc) qt[kc] = bf16x8{};
    }
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) asm volatile("" ::"v"(qt[kc]));   // loads complete before the tile loop
  }

  // ---- operand addresses. K fragment: lane (up, l32) reads tile row krow(l32) (its
  // accumulator row), dims 16 kc + 8 up. V^T: lane (G = lane/16, j = lane%16) points at
  // tile row G/2 + 4 (j/4) (+16 ks, +2 for the upper four k entries) and value dim
  // 16 (G%2) + 4 (j%4) (+32 per block); the read returns value dim 16 (G%2) + j of the
  // four rows its lane groups point at, which are the tile rows of score accumulator
  // rows 16 ks + 4 up + e and 16 ks + 8 + 4 up + e, so the packed weights serve as the
  // B operand as they stand.
  const int kofs = krow(l32) * ROWB + 16 * up;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int voff = ((g16 >> 1) + 4 * (j16 >> 2)) * ROWB + (16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
  auto kbase = [&](int t) {
    int sofs = (t % NST) * STAGE + kofs;
    asm volatile("" : "+v"(sofs));
    return (DSA_LDS const unsigned char*)lds + sofs;
  };
  auto vbase = [&](int t) {
    int vsofs = (t % NST) * STAGE + voff;
    asm volatile("" : "+v"(vsofs));
    return (DSA_LDS const unsigned char*)lds + vsofs;
  };
  auto kfrag = [&](DSA_LDS const unsigned char* kp, int kc) { return *(DSA_LDS const bf16x8*)(kp + 32 * kc); };
  // value MFMA i (< 32): block i / 2, k-step i % 2
  auto vfrag = [&](DSA_LDS const unsigned char* vb, int i) {
    const int db = i >> 1, ks = i & 1;
    return join_bf16x8(lds_read_tr16(vb + (16 * ks) * ROWB + 64 * db), lds_read_tr16(vb + (16 * ks + 2) * ROWB + 64 * db));
  };
  // all 36 score MFMAs of a tile in one chain (used outside the pipelined loop)
  auto scores = [&](int t, f32x16& s) {
    DSA_LDS const unsigned char* kp = kbase(t);
    bf16x8 f[PDK];
#pragma unroll
    for (int i = 0; i < PDK; ++i) f[i] = kfrag(kp, i);
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) {
      if (kc == 0) score_mfma_first(s, f[0], qt[0]);
      else score_mfma(s, f[kc % PDK], qt[kc]);
      if (kc + PDK < KS) f[kc % PDK] = kfrag(kp, kc + PDK);
    }
    score_settle(s);
  };
  // exponent arguments of a raw score tile against the reference (in place), masked
  // keys at -inf; the lane's running maximum of them goes to mx.
  // EDGE: the tile reaches past the smallest causal limit of the wave's rows.
  auto exponents = [&](int t, f32x16& s, float mref, float& mx, auto edge) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = fmaf(s[j], scale_log2, -mref);
    if constexpr (MASKED || decltype(edge)::value) {
      uint32_t word = 0xFFFFFFFFu;
      if constexpr (MASKED) {
        const uint32_t* mw = (const uint32_t*)(lds + MASK_OFF + ((t % NST) * NWV + wave) * 8);
        word = qi == qw0 ? mw[0] : mw[1];
      }
      const int lt = lim - t * T;                           // last visible tile row
      const uint32_t vis = lt >= T - 1 ? 0xFFFFFFFFu : (lt < 0 ? 0u : (2u << lt) - 1u);
      word = (word & vis) >> up;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = ((word >> key_of_elem(j, 0)) & 1u) ? s[j] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[j]);
  };
  auto pair_max = [](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };

  typedef std::integral_constant<bool, false> no_edge;
  typedef std::integral_constant<bool, true> edge;
  typedef std::integral_constant<bool, false> more;
  typedef std::integral_constant<bool, true> last;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float lsum = 0.f;                                         // this lane's share of the row's sum
  if (ntiles > 0) {
    // reference for the first pass: the maximum of the first tile (0 if it has no key)
    load_tile(0, 0);
    load_tile(min(1, ntiles - 1), 1);
    load_tile(min(2, ntiles - 1), 2);
    wait_tiles(2);
    lds_barrier();
    float mref;
    {
      f32x16 s0;
      scores(0, s0);
      float mx = -INFINITY;
      exponents(0, s0, 0.f, mx, edge());
      mx = pair_max(mx);
      mref = mx == -INFINITY ? 0.f : mx;
    }
    // iterations whose next tile lies wholly below the wave's smallest causal limit,
    // then the rest with masking
    const int nfull = min(ntiles, max(0, (lim_min + 1) / T - 1));
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
      float mx = -INFINITY;                                 // running maximum of the exponent arguments
      if (pass) {                                           // again from tile 0, against the true maximum
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
        lsum = 0.f;
        lds_barrier();
        load_tile(0, 0);
        load_tile(min(1, ntiles - 1), 1);
        load_tile(min(2, ntiles - 1), 2);
        wait_tiles(2);
        lds_barrier();
      }
      f32x16 c;
      scores(0, c);
      exponents(0, c, mref, mx, edge());
      // one tile: the weights of tile t are formed under the score MFMAs of tile t+1,
      // the exponent arguments of tile t+1 under the value MFMAs of tile t (LAST: tile
      // t is the last one, no scores follow). Every MFMA sits in a block of its own
      // with the LDS read a fixed distance ahead and its share of the other work; the
      // blocks are fenced, so the reads stay ahead and the vector work stays spread.
      auto step = [&](int t, auto edge_t, auto last_t) {
        constexpr bool LAST = decltype(last_t)::value;
        wait_tiles(1);                                      // tile t+1 landed (t+2 may be in flight)
        lds_barrier();                                      // ... for every wave; stage t-1 is free
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pk0, pk1;
        f32x16 n;
        DSA_LDS const unsigned char* vb = vbase(t);
        bf16x8 vf[PDV];
        if constexpr (!LAST) {
          DSA_LDS const unsigned char* kp = kbase(t + 1);
          bf16x8 f[PDK];
#pragma unroll
          for (int i = 0; i < PDK; ++i) f[i] = kfrag(kp, i);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kc = 0; kc < KS; ++kc) {
            if (kc == 0) score_mfma_first(n, f[0], qt[0]);
            else score_mfma(n, f[kc % PDK], qt[kc]);
            if (kc + PDK < KS) f[kc % PDK] = kfrag(kp, kc + PDK);
            if (kc < 8) {
              c[2 * kc] = exp2_fast(c[2 * kc]);
              c[2 * kc + 1] = exp2_fast(c[2 * kc + 1]);
            }
            if (kc == 8) pk0 = pack_half(c, 0);
            if (kc == 9) pk1 = pack_half(c, 1);
            if (kc == 10) lsum = sum8_dot(pk1, sum8_dot(pk0, lsum));
            // the first value fragments of tile t, under the last score MFMAs
            if (kc >= KS - PDV) vf[kc - (KS - PDV)] = vfrag(vb, kc - (KS - PDV));
            __builtin_amdgcn_sched_barrier(0);
          }
          score_settle(n);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) c[j] = exp2_fast(c[j]);
          pk0 = pack_half(c, 0);
          pk1 = pack_half(c, 1);
          lsum = sum8_dot(pk1, sum8_dot(pk0, lsum));
#pragma unroll
          for (int i = 0; i < PDV; ++i) vf[i] = vfrag(vb, i);
        }
        __builtin_amdgcn_sched_barrier(0);
        // value MFMAs of tile t; the loads of tile t+3 (stage t-1, free since the
        // barrier) and the exponent arguments of tile t+1 ride between them
        const int tl = min(t + 3, ntiles - 1), sl = (t + 3) % NST;
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
          o[i >> 1] = mfma32x32x16(vf[i % PDV], (i & 1) ? pk1 : pk0, o[i >> 1]);
          if (i + PDV < 2 * NDB) vf[i % PDV] = vfrag(vb, i + PDV);
          if (i % 2 == 1 && i / 2 < LPW) load_part(tl, sl, i / 2);
          if (i == 2 * LPW + 1) load_mask(tl, sl);
          if constexpr (!LAST) {
            if (i == 3) exponents(t + 1, n, mref, mx, edge_t);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!LAST) c = n;
      };
      int t = 0;
      for (; t < min(nfull, ntiles - 1); ++t) step(t, no_edge(), more());
      for (; t < ntiles - 1; ++t) step(t, edge(), more());
      step(t, edge(), last());
      // the spare loads of the last steps land before a second pass reloads the
      // stages, or the workgroup ends
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // the row's largest exponent argument: within SPAN of the reference, or a second
      // pass against the row's true maximum
      mx = pair_max(mx);
      const bool redo = mx != -INFINITY && (mx > SPAN || mx < -SPAN);
      // the decision is the workgroup's (every wave takes the same number of barriers)
      if (pass) break;
      int* votes = (int*)(lds + FLAG_OFF);
      if (lane == 0) votes[wave] = __ballot(redo) != 0;
      lds_barrier();
      int any = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) any |= votes[w];
      if (!any) break;
      if (redo) mref += mx;
    }
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      lsum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }

  if (!row_ok) return;
  // O^T element j of block db: value dim 32 db + 8 (j/4) + 4 up + j%4 of this lane's row
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = out + (((size_t)b * L + qi) * H + hd) * DV + 4 * up;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]} * inv;
      *(bf16x4*)(orow + 32 * db + 8 * g) = __builtin_convertvector(v, bf16x4);
    }
}

// Dense (mask == nullptr) or masked dense absorbed attention for all L queries of each
// batch entry. H is any positive count (rows are flattened (query, head) pairs).
hipError_t launch_absorbed_dense(const uint16_t* q, const uint16_t* kv, const uint32_t* mask, uint16_t* out, int B,
                                 int L, int N, int H, int causal, float scale, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)absorbed_dense_kernel<false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)absorbed_dense_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const long long rows = (long long)L * H;
  dim3 grid((unsigned)((rows + ROWS - 1) / ROWS), B), block(64 * NWV);
  if (mask) {
    KernelTrace kt("masked_dense_attn", stream);
    hipLaunchKernelGGL(absorbed_dense_kernel<true>, grid, block, LDS_BYTES, stream, q, kv, mask, out, L, N, H, causal,
                       scale_log2);
  } else {
    KernelTrace kt("absorbed_dense_attn", stream);
    hipLaunchKernelGGL(absorbed_dense_kernel<false>, grid, block, LDS_BYTES, stream, q, kv, mask, out, L, N, H,
                       causal, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace dsa

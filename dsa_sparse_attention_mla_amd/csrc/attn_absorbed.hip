// Absorbed (latent-space) MLA attention over joined 576-wide latent+rope rows.
//
// One kernel serves two calls:
//  * sparse prefill: each query attends only to the rows its index list names,
//    gathered from the cache ("Sparse prefill for GLM", section "Sparse
//    attention": joined latent+rope rows, all heads share the gathered block,
//    absorbed attention whose value is the latent part of the row), and
//  * one split of a paged decode step (the rows of a sequence's page list).
// Dense and masked dense absorbed prefill, where a cache tile is shared by many
// queries, have a kernel of their own (attn_absorbed_dense.hip).
//
// Work decomposition (gfx950): one workgroup per query and 64-head group, 8
// waves, with the 32x32x16 bf16 MFMA so that every operand fragment read from LDS
// serves 32 heads. Waves 0-3 score: wave w contracts half w/2 (288 dims) of the
// 576-wide score for head group w%2 (32 heads): partial S^T[32 keys x 32 heads] =
// K_tile[:, half] . Q^T[half] (K fragments from LDS, Q^T fragments in registers),
// written to LDS. Waves 4-7 produce output: wave 4+w owns value half w/2 (256 dims)
// of head group w%2; it sums the two partial scores of a tile in a fixed order (so
// both output waves of a group run the identical online softmax; a head is one MFMA
// column, its running max and sum live in the two lanes owning the column) and
// accumulates O^T[256 dims x 32 heads] += V_tile^T[half] . P^T (V^T fragments by
// transpose reads from LDS, P^T already in the operand layout in registers).
// The two roles are pipelined one tile apart: while the output waves consume the
// scores of tile t, the score waves compute those of tile t+1, and the rows of tile
// t+2 are written into the third LDS stage, so one barrier per tile suffices. Waves
// w and w+4 share a SIMD: one score and one output wave each. Each role runs its own
// loop, so its registers (Q^T for scoring, the 256x32 accumulator for output) do not
// add up. All 64 heads share every gathered row, which is read from HBM once.
// Row fetch (score waves only, so the output waves' critical path has none of it):
// each tile's rows are loaded into registers two tiles ahead of staging (nine
// 16-byte loads per thread, eight threads per row) and written to their LDS stage;
// the index list of a segment of up to 2048 keys is staged in LDS first, so a row
// address never waits on an index load.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int D = 576;                  // joined row: 512 latent + 64 rope
constexpr int DV = 512;                 // value = latent part of the row
constexpr int T = 32;                   // keys per tile
constexpr int CH = D * 2 / 16;          // 16-byte chunks per row (72)
constexpr int ROWCH = CH + 1;           // padded LDS row, in chunks (bank spread)
constexpr int ROWB = ROWCH * 16;        // 1168 bytes
constexpr int STAGE = T * ROWB;         // 37376 bytes per LDS stage
constexpr int NST = 3;                  // LDS stages: tiles t (output), t+1 (scores), t+2 (filling)
constexpr int FPR = 8;                  // score-wave threads per tile row in the row fetch
constexpr int CPT = CH / FPR;           // 16-byte chunks per fetching thread per tile (9)
constexpr int PF = 2;                   // tiles in flight in the fetching threads' registers
constexpr int SEG = 2048;               // index entries staged per segment
constexpr int KST = D / 2 / 16;         // 32x32x16 k-steps per score half (18)
// Score accumulator row c = 4m + e (m < 8, e < 4) holds tile row krow(c) =
// m%4 + 4e + 16(m/4): the four rows one transpose read of V^T covers are then four
// apart, 144 bytes of bank offset each with 1168-byte rows, so a 32-lane read
// touches every bank once, and the 16 rows of a K fragment read stay distinct.
__device__ __forceinline__ int krow(int c) { return ((c >> 2) & 3) + 4 * (c & 3) + 16 * (c >> 4); }
constexpr int NW = 8;                   // waves per workgroup: 4 scoring, 4 producing output
constexpr int DH = DV / 2;              // value dims per output wave (256)
constexpr int NDB = DH / 32;            // 32-row value blocks per output wave (8)
constexpr float SLACK = 8.f;            // log2 of the largest unnormalised softmax weight
constexpr int XCH_TILE = 4 * 4 * 64 * 16;   // partial scores of a tile: 4 score waves x 16 floats x 64 lanes
constexpr size_t LDS_BYTES = NST * (size_t)STAGE + SEG * 4 + 16 + 2 * XCH_TILE;
static_assert(T * FPR == 256 && CPT * FPR == CH, "the score waves fetch whole tiles");
static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
}  // namespace

// MODE: 1 sparse (gathered index lists), 3 paged decode split (one query per sequence; workgroup x gathers
// keys [x*spl, x*spl + spl) of the sequence's row list and writes its unnormalised
// partial output with the running max and sum, merged afterwards).
template <int MODE>
__global__ __launch_bounds__(64 * NW) void absorbed_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ mask, uint16_t* __restrict__ out, int L, int N, int H, int topk, int q0, int causal,
    float scale_log2, const int32_t* __restrict__ seqlens, float* __restrict__ part, int spl, int psz) {
  static_assert(MODE == 1 || MODE == 3, "rows come from an index list");
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  unsigned char* ring = dyn;                                // [NST][STAGE]
  int* sidx = (int*)(dyn + NST * (size_t)STAGE);            // [SEG]
  uint32_t* smask = (uint32_t*)(sidx + SEG);                // [NST] valid keys of the staged tile (bit r = row r)
  f32x4* xch = (f32x4*)((unsigned char*)smask + 16);        // [2 tile parities][4 score waves][4][64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, up = lane >> 5;
  const int b = blockIdx.y;
  const int i = MODE == 3 ? 0 : q0 + blockIdx.x;
  const bool score_wave = wave < 4;
  const int hg = wave & 1;
  const int half = (wave >> 1) & 1;                         // score half, or value half of an output wave
  const int head = blockIdx.z * 64 + 32 * hg + l32;
  const bool head_ok = head < H;
  int count = topk;
  // (topk is the row-list length here; a sequence length past it is clamped to it)
  if constexpr (MODE == 3) count = max(0, min(spl, min(seqlens[b], topk) - (int)blockIdx.x * spl));
  // paged decode: rows are physical rows of the page pool (N of them), shared by all sequences
  const uint16_t* kvb = kv + (MODE == 3 ? (size_t)0 : (size_t)b * N * D);
  // sparse: the query's index list; paged decode: the sequence's page table row
  // (topk = max_pages * page_size there)
  const int32_t* irow = MODE == 1 ? idx + ((size_t)b * L + i) * topk : idx + (size_t)b * (topk / psz);

  // Tile rows (score waves, tid < 256): thread tid handles row tid / 8 of the tile and
  // its 16-byte columns tid % 8 + 8 u, so a thread looks up one key per tile and its
  // loads and LDS writes are one base plus immediates.
  const int frow = (tid & 255) >> 3, fcol = tid & 7;
  auto key_of = [&](int t, int r, int seg_base, int seg_cnt) -> int {
    const int slot = t * T + r;
    if (slot >= seg_cnt) return -1;
    return sidx[slot];
  };
  // Every fetching thread issues CPT loads for every fetch, also past the last tile
  // (those read row 0 and are never staged), so the number of outstanding loads is the
  // same on every path and the compiler's waits stay exact.
  auto fetch = [&](int t, u32x4 (&dst)[CPT], int seg_base, int seg_cnt) {
    const int key = key_of(t, frow, seg_base, seg_cnt);
    const uint16_t* rp = kvb + (size_t)(key >= 0 ? key : 0) * D + 8 * fcol;   // invalid: row 0, masked
#pragma unroll
    for (int u = 0; u < CPT; ++u) dst[u] = *(const u32x4*)(rp + 64 * u);
  };
  auto stage_in = [&](int t, int st_i, const u32x4 (&src)[CPT], int seg_base, int seg_cnt) {
    unsigned char* st = ring + (size_t)st_i * STAGE + frow * ROWB + 16 * fcol;
#pragma unroll
    for (int u = 0; u < CPT; ++u) *(u32x4*)(st + 128 * u) = src[u];
    if (wave == 0) {
      const bool v = lane < T && key_of(t, lane, seg_base, seg_cnt) >= 0;
      const unsigned long long bm = __ballot(v);
      if (lane == 0) smask[st_i] = (uint32_t)bm;
    }
  };
  // Index list of a segment into LDS (all of this thread's index loads in flight
  // before any is used).
  auto segment_indices = [&](int seg_base, int seg_cnt) {
    lds_barrier();                                 // the previous segment's indices and stages are no longer read
    {
      constexpr int PER = SEG / (64 * NW);
      int xs[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 64 * NW * u;
        if constexpr (MODE == 3) {
          // position n of the sequence lives in row n % page_size of page table[n / page_size]
          const int n = (int)blockIdx.x * spl + seg_base + e;
          const int pg = e < seg_cnt ? irow[n / psz] : -1;
          xs[u] = pg >= 0 && pg < N / psz ? pg * psz + n % psz : -1;
        } else {
          xs[u] = e < seg_cnt ? irow[seg_base + e] : -1;
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 64 * NW * u;
        if (e < seg_cnt) sidx[e] = (xs[u] >= 0 && xs[u] < N) ? xs[u] : -1;
      }
      lds_barrier();
    }
  };

  const int nseg = count > 0 ? (count + SEG - 1) / SEG : 0;

  if (score_wave) {
    // ---------------------------------------------------------------- scoring
    // Q^T fragments: lane (up, l32) holds head l32 of the group, dims 288 half +
    // 16 kc + 8 up .. +8 (zero for heads past H)
    bf16x8 qt[KST];
    {
      const uint16_t* qrow = q + (((size_t)b * L + i) * H + (head_ok ? head : 0)) * D + 288 * half + 8 * up;
#pragma unroll
      for (int kc = 0; kc < KST; ++kc) {
        bf16x8 v = {};
        if (head_ok) v = *(const bf16x8*)(qrow + 16 * kc);
        qt[kc] = v;
      }
      // Consume the fragments here, so their loads are known complete before the tile
      // loop; otherwise the loop's merged wait state would drain the row prefetch.
#pragma unroll
      for (int kc = 0; kc < KST; ++kc) asm volatile("" ::"v"(qt[kc]));
    }
    // lane (up, l32) reads K fragments of tile row krow(l32): accumulator row l32
    const int kofs = krow(l32) * ROWB + 576 * half + 16 * up;
    auto score_tile = [&](int t) {
      const unsigned char* kp = ring + (size_t)(t % NST) * STAGE + kofs;
      f32x16 sc = {};
      // K fragments in two batches of nine reads, each issued before its MFMAs
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 kf[KST / 2];
#pragma unroll
        for (int kc = 0; kc < KST / 2; ++kc) kf[kc] = *(const bf16x8*)(kp + 32 * (KST / 2 * h2 + kc));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < KST / 2; ++kc) sc = mfma32x32x16(kf[kc], qt[KST / 2 * h2 + kc], sc);
      }
      f32x4* xw = xch + (size_t)(((t & 1) * 4 + wave) * 4) * 64;
#pragma unroll
      for (int c = 0; c < 4; ++c) xw[c * 64 + lane] = f32x4{sc[4 * c], sc[4 * c + 1], sc[4 * c + 2], sc[4 * c + 3]};
    };
    u32x4 pf[PF][CPT];
    // tile t: scores of t+1, then tile t+2 from register slot t%2 into its stage (its
    // last readers worked on tile t-1, before this tile's barrier) and the slot
    // refetches t+4
    auto step = [&](int t, u32x4 (&slot)[CPT], int ntiles, int seg_base, int seg_cnt) {
      lds_barrier();                               // scores of t, rows of t+1 published
      if (t + 1 < ntiles) score_tile(t + 1);
      if (t + 2 < ntiles) stage_in(t + 2, (t + 2) % NST, slot, seg_base, seg_cnt);
      fetch(t + 2 + PF, slot, seg_base, seg_cnt);
    };
    for (int seg = 0; seg < nseg; ++seg) {
      const int seg_base = seg * SEG;
      const int seg_cnt = min(SEG, count - seg_base);
      const int ntiles = (seg_cnt + T - 1) / T;
      segment_indices(seg_base, seg_cnt);
      // tiles 0 and 1 staged, 2 and 3 in registers, scores of 0
      fetch(0, pf[0], seg_base, seg_cnt);
      fetch(1, pf[1], seg_base, seg_cnt);
      if (ntiles > 0) stage_in(0, 0, pf[0], seg_base, seg_cnt);
      if (ntiles > 1) stage_in(1, 1, pf[1], seg_base, seg_cnt);
      fetch(2, pf[0], seg_base, seg_cnt);
      fetch(3, pf[1], seg_base, seg_cnt);
      lds_barrier();
      if (ntiles > 0) score_tile(0);
      for (int t = 0; t < ntiles; t += 2) {
        step(t, pf[0], ntiles, seg_base, seg_cnt);
        if (t + 1 < ntiles) step(t + 1, pf[1], ntiles, seg_base, seg_cnt);
      }
    }
    return;
  }

  // ---------------------------------------------------------------- output
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;                          // per head (lane column)
  // V^T operand by transpose reads: lane (G = lane/16, j = lane%16) points at tile row
  // G/2 + 4 (j/4) (+16 ks, +2 for the upper four k entries) and value dim 256 half +
  // 16 (G%2) + 4 (j%4); the read returns dims 256 half + 16 (G%2) + j (= lane % 32) of
  // the four rows its lane groups point at. Those are tile rows krow(c) of the score
  // accumulator rows c = 16 ks + 4 up + e and 16 ks + 8 + 4 up + e (e < 4): k entry
  // 8 up + e of k-step ks follows the accumulator's row order, so the packed weights
  // serve as the B operand unchanged.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int voff = ((g16 >> 1) + 4 * (j16 >> 2)) * ROWB + (DH * half + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
  auto output_tile = [&](int t) {
    const int s3 = t % NST;
    // the first batch of V^T fragments does not depend on the scores: read it now,
    // under the softmax
    // (decode: the stage offset is made opaque, so the compiler keeps one address
    // register and folds every read's constant into the instruction instead of
    // strength-reducing sixteen addresses across the loop; the prefill gather was
    // measured no faster that way, even slower with uncorrelated index lists, and
    // keeps the compiler's form)
    int sofs = s3 * STAGE;
    if constexpr (MODE == 3) asm volatile("" : "+s"(sofs));
    DSA_LDS const unsigned char* vb = (DSA_LDS const unsigned char*)dyn + sofs + voff;
    bf16x8 vf0[NDB / 2][2];
#pragma unroll
    for (int d = 0; d < NDB / 2; ++d)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vf0[d][ks] = join_bf16x8(lds_read_tr16(vb + (16 * ks) * ROWB + 64 * d),
                                 lds_read_tr16(vb + (16 * ks + 2) * ROWB + 64 * d));
    // S = part0 + part1, in that order in both output waves of the group
    const f32x4* x0 = xch + (size_t)(((t & 1) * 4 + hg) * 4) * 64;         // score wave hg: half 0
    const f32x4* x1 = xch + (size_t)(((t & 1) * 4 + 2 + hg) * 4) * 64;     // score wave 2 + hg: half 1
    // valid keys of the tile; element j sits in accumulator row c = 8 (j/4) + 4 up + j%4,
    // tile row krow(c) = up + 2 ((j/4)%2) + 16 (j/8) + 4 (j%4). With all
    // 32 keys valid and a positive scale (the usual tile) the scale goes into the
    // exponent's fused multiply-add; otherwise scores are scaled and masked first.
    const uint32_t vmask = smask[s3];
    float sv[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 a0 = x0[c * 64 + lane], a1 = x1[c * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[4 * c + e] = a0[e] + a1[e];
    }
    const bool plain = vmask == 0xFFFFFFFFu && scale_log2 > 0.f;
    float mul = scale_log2;
    if (!plain) {
      const uint32_t vm = vmask >> up;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        sv[j] = ((vm >> (2 * ((j >> 2) & 1) + 16 * (j >> 3) + 4 * (j & 3))) & 1u) ? sv[j] * scale_log2 : -INFINITY;
      mul = 1.f;
    }
    float tmax = sv[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, sv[j]);
    tmax *= mul;
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    // The reference max moves only when a score exceeds it by more than 2^SLACK (or
    // on the first valid key): softmax does not depend on the reference, and weights
    // up to 2^SLACK lose nothing in bf16 / fp32, so the output rescale is rare.
    const bool bump = tmax - m > SLACK;
    const float mnew = bump ? tmax : m;
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pv[e] = exp2_fast(fmaf(sv[e], mul, -mref));
    // The normaliser sums the bf16-rounded weights the value product uses, so the
    // output is an exact convex combination of those weights (a dominant key gives
    // back its value row, whatever the rounding of its weight).
    const bf16x8 pk0 = pack_bf16x8(pv), pk1 = pack_bf16x8(pv + 8);
    float psum = sum_bf16x8(pk0) + sum_bf16x8(pk1);
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
      psum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (__ballot(bump)) {
      const float alpha = bump ? exp2_fast(m - mref) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    lsum += psum;
    m = mnew;
    // P^T operand of k-step ks: this lane's weights of keys 16 ks + 4 up + (0..3) and
    // 16 ks + 8 + 4 up + (0..3), exactly pk0 (ks = 0) and pk1 (ks = 1).
    const bf16x8 pt0 = pk0, pt1 = pk1;
    // value product in two batches of four 32-dim blocks; the second batch's eight
    // transpose-read pairs are issued before its MFMAs
#pragma unroll
    for (int d = 0; d < NDB / 2; ++d)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o[d] = mfma32x32x16(vf0[d][ks], ks ? pt1 : pt0, o[d]);
    {
      bf16x8 vf[NDB / 2][2];
#pragma unroll
      for (int d = 0; d < NDB / 2; ++d)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int db = NDB / 2 + d;
          vf[d][ks] = join_bf16x8(lds_read_tr16(vb + (16 * ks) * ROWB + 64 * db),
                                  lds_read_tr16(vb + (16 * ks + 2) * ROWB + 64 * db));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < NDB / 2; ++d)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o[NDB / 2 + d] = mfma32x32x16(vf[d][ks], ks ? pt1 : pt0, o[NDB / 2 + d]);
    }
  };
  for (int seg = 0; seg < nseg; ++seg) {
    const int seg_base = seg * SEG;
    const int seg_cnt = min(SEG, count - seg_base);
    const int ntiles = (seg_cnt + T - 1) / T;
    segment_indices(seg_base, seg_cnt);
    lds_barrier();                                 // tiles 0 and 1 staged, scores of 0 under way
    for (int t = 0; t < ntiles; ++t) {
      lds_barrier();                               // scores of t, rows of t+1 published
      output_tile(t);
    }
  }

  if (!head_ok) return;
  // O^T element j of block db: dim 256 half + 32 db + 8 (j/4) + 4 up + j%4 of head `head`
  if constexpr (MODE == 3) {
    // partial record of (sequence b, split x, head): 512 unnormalised output values,
    // then the running max (log2 units) and sum
    float* rec = part + (((size_t)b * gridDim.x + blockIdx.x) * H + head) * (DV + 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(rec + DH * half + 32 * db + 8 * g + 4 * up) =
            f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    if (half == 0 && up == 0) {
      rec[DV] = m;
      rec[DV + 1] = lsum;
    }
    return;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = out + (((size_t)b * L + i) * H + head) * DV + DH * half + 4 * up;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]} * inv;
      *(bf16x4*)(orow + 32 * db + 8 * g) = __builtin_convertvector(v, bf16x4);
    }
}

// One workgroup per (query, batch): the query's selection bitmap (bit n of word n/32
// set when its index list names key n, entries outside [0, N) ignored), built in LDS
// a chunk of words at a time and written out whole.
__global__ __launch_bounds__(256) void mask_rows_kernel(const int32_t* __restrict__ idx, int L, int N, int topk,
                                                        uint32_t* __restrict__ mask) {
  constexpr int CW = 8192;                  // words per chunk (32 KB of LDS)
  __shared__ uint32_t words[CW];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int W = (N + 31) / 32;
  const int32_t* irow = idx + ((size_t)b * L + i) * topk;
  uint32_t* mrow = mask + ((size_t)b * L + i) * W;
  for (int c0 = 0; c0 < W; c0 += CW) {
    const int cw = min(CW, W - c0);
    for (int e = tid; e < cw; e += 256) words[e] = 0u;
    __syncthreads();
    for (int t = tid; t < topk; t += 256) {
      const int n = irow[t];
      const int wd = n >> 5;
      if (n >= 0 && n < N && wd >= c0 && wd < c0 + cw) atomicOr(&words[wd - c0], 1u << (n & 31));
    }
    __syncthreads();
    for (int e = tid; e < cw; e += 256) mrow[c0 + e] = words[e];
    __syncthreads();
  }
}

// Merge of the split partials of one (sequence, head): out = sum_x 2^(m_x - M) O_x /
// sum_x 2^(m_x - M) l_x with M the largest split max; splits without a visible key
// (m = -inf) contribute nothing; a sequence with none gets zeros. The maxima and sums
// of all splits are reduced by the whole workgroup first; the weights of 256 splits
// at a time then go through LDS and each thread accumulates its two output dims with
// eight split records in flight.
__device__ __forceinline__ float block_reduce256(float v, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  __syncthreads();                                  // earlier readers of red are done
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part, int nsplit, int H,
                                                             uint16_t* __restrict__ out) {
  __shared__ float wsh[256];
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* base = part + ((size_t)b * nsplit * H + h) * (DV + 2);
  const size_t stride = (size_t)H * (DV + 2);
  float mloc = -INFINITY;
  for (int x = tid; x < nsplit; x += 256) mloc = fmaxf(mloc, base[x * stride + DV]);
  const float M = block_reduce256(mloc, true, red);
  float dl = 0.f;
  if (M != -INFINITY)
    for (int x = tid; x < nsplit; x += 256) {
      const float mx = base[x * stride + DV];
      if (mx != -INFINITY) dl += exp2_fast(mx - M) * base[x * stride + DV + 1];
    }
  const float den = block_reduce256(dl, false, red);
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 acc = {0.f, 0.f};
  if (M != -INFINITY)
    for (int c = 0; c < nsplit; c += 256) {
      __syncthreads();                              // the previous chunk's weights are consumed
      const int x = c + tid;
      float w = 0.f;
      if (x < nsplit) {
        const float mx = base[(size_t)x * stride + DV];
        w = mx == -INFINITY ? 0.f : exp2_fast(mx - M);
      }
      wsh[tid] = w;
      __syncthreads();
      const int n = min(256, nsplit - c);
      const float* col = base + (size_t)c * stride + 2 * tid;
      int u = 0;
      for (; u + 8 <= n; u += 8) {
        f32x2 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = *(const f32x2*)(col + (size_t)(u + k) * stride);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += wsh[u + k] * v[k];
      }
      for (; u < n; ++u) acc += wsh[u] * *(const f32x2*)(col + (size_t)u * stride);
    }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = acc * inv;
  *(bf16x2*)(out + ((size_t)b * H + h) * DV + 2 * tid) = __builtin_convertvector(v, bf16x2);
}

hipError_t launch_paged_decode(const uint16_t* q, const uint16_t* kv_pages, const int32_t* page_table,
                               const int32_t* seqlens, int B, int H, int num_pages, int page_size, int max_pages,
                               int spl, int nsplit, float* part, uint16_t* out, float scale, hipStream_t stream) {
  const int maxlen = max_pages * page_size;
  hipError_t e = launch_absorbed_attn(3, q, kv_pages, page_table, nullptr, nullptr, B, 1, num_pages * page_size, H,
                                      maxlen, 0, nsplit, 0, scale, stream, seqlens, part, spl, page_size);
  if (e != hipSuccess) return e;
  KernelTrace kt("decode_combine", stream);
  hipLaunchKernelGGL(decode_combine_kernel, dim3(H, B), dim3(DV / 2), 0, stream, part, nsplit, H, out);
  return hipGetLastError();
}

// Fixed device scratch for the decode entry point that allocates nothing: the split
// partials live here instead of in a caller workspace. Each device that loads the
// library holds its own copy until the process ends. In host code the name is only a
// stand-in for the symbol: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_mask_rows(const int32_t* idx, int B, int L, int N, int topk, uint32_t* mask, hipStream_t stream) {
  KernelTrace kt("mask_rows", stream);
  hipLaunchKernelGGL(mask_rows_kernel, dim3(L, B), dim3(256), 0, stream, idx, L, N, topk, mask);
  return hipGetLastError();
}

// Launch over queries [q0, q0 + nq) of a chunk of L queries. H must be a multiple of 16;
// a workgroup covers 64 heads (grid z walks head groups).
hipError_t launch_absorbed_attn(int mode, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                const uint32_t* mask, uint16_t* out, int B, int L, int N, int H, int topk, int q0,
                                int nq, int causal, float scale, hipStream_t stream, const int32_t* seqlens,
                                float* part, int spl, int psz) {
  static bool attr_set = false;
  if (!attr_set) {
    const void* fns[2] = {(const void*)absorbed_attn_kernel<1>, (const void*)absorbed_attn_kernel<3>};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nq, B, (H + 63) / 64), block(64 * NW);
  if (mode != 1 && mode != 3) return hipErrorInvalidValue;
  KernelTrace kt(mode == 1 ? "sparse_attn" : "paged_decode_attn", stream);
#define DSA_LAUNCH_ABS(M)                                                                                    \
  hipLaunchKernelGGL((absorbed_attn_kernel<M>), grid, block, LDS_BYTES, stream, q, kv, idx, mask, out, L, N, H, \
                     topk, q0, causal, scale_log2, seqlens, part, spl, psz)
  if (mode == 1) DSA_LAUNCH_ABS(1);
  else DSA_LAUNCH_ABS(3);
#undef DSA_LAUNCH_ABS
  return hipGetLastError();
}

}  // namespace dsa

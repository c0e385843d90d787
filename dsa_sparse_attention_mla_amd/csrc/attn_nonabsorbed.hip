// Non-absorbed MLA prefill: per head, the score is the sum of a 128-dim
// contraction against that head's key and a 64-dim contraction against a rope
// key shared by every head, followed by softmax and the 128-dim value product
// (Fornax part 5, "Apple M3 vs M5 kernels", section "What the kernel has to
// compute").
//
// Both contractions go into ONE MFMA accumulator: the LDS key row of a tile is
// [K_nope(head) | K_rope] (192 entries), the query fragment is [Q_nope | Q_rope],
// so S^T = K_row . Q^T is a single 192-deep contraction.
//
// fp32 path (the correctness configuration): one workgroup per (head, 16 queries),
// one 16x16 MFMA column block. Its four waves take the key blocks of 16 in turn
// (wave w: blocks w, w + 4, ...), each with its own online softmax, and merge their
// (max, sum, output) through LDS in wave order at the end, so the longest query
// block's chain of MFMAs is a quarter of its keys. 16x16x4 fp32 MFMA throughout.
// The bf16 path is described with its kernel below.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int DN = 128, DR = 64, DQK = DN + DR, DVN = 128;
static_assert(DVN == DN, "K_nope and V rows share one address formula");
constexpr int F_QB = 16;                          // queries per workgroup
constexpr int F_KB = 16;                          // keys per block
constexpr int F_KROW = DQK * 4 + 16;              // LDS row [K_nope | K_rope] + pad (784 B)
constexpr int F_VROW = DVN * 4 + 16;              // LDS V row + pad (528 B)
constexpr int F_BLK = F_KB * (F_KROW + F_VROW);   // one key block in LDS
constexpr int F_ROWCH = (DQK + DVN) * 4 / 16;     // 16-byte chunks of one key's K and V rows
constexpr int F_PER = 4 * F_KB * F_ROWCH / 256;   // chunks per thread for a round of four blocks
constexpr int F_OROW = DVN + 4;                   // merge record row (floats)
static_assert(4 * F_KB * F_ROWCH % 256 == 0, "whole chunks per thread");
static_assert((128 + 4 * F_QB * F_OROW) * 4 <= 4 * F_BLK, "merge records fit the staging area");
}  // namespace

__global__ __launch_bounds__(256) void nonabsorbed_f32_kernel(
    const float* __restrict__ qn, const float* __restrict__ qr, const float* __restrict__ kn,
    const float* __restrict__ kr, const float* __restrict__ vv, float* __restrict__ out, int L, int N, int H,
    int causal, float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * F_BLK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qt = gridDim.x - 1 - blockIdx.x;        // longest rows first
  const int i0 = qt * F_QB, i = i0 + c16;           // this lane's query (MFMA column)
  const bool qvalid = i < L;
  const int p = N - L + i;                          // its causal limit
  const int count = causal ? N - L + min(L - 1, i0 + F_QB - 1) + 1 : N;
  const int nkb = (count + F_KB - 1) / F_KB, nround = (nkb + 3) / 4;
  const float* knb = kn + (size_t)b * N * H * DN;
  const float* krb = kr + (size_t)b * N * DR;
  const float* vb = vv + (size_t)b * N * H * DVN;

  // Query fragments (B operand): column = query, k = dims 4 kc + g of [Q_nope | Q_rope].
  float qf[DQK / 4];
  {
    const int ii = qvalid ? i : 0;
    const float* pn = qn + (((size_t)b * L + ii) * H + h) * DN + g;
    const float* pr = qr + (((size_t)b * L + ii) * H + h) * DR + g;
#pragma unroll
    for (int kc = 0; kc < DQK / 4; ++kc) qf[kc] = kc < DN / 4 ? pn[4 * kc] : pr[4 * (kc - DN / 4)];
  }
  f32x4 o[DVN / 16];
#pragma unroll
  for (int db = 0; db < DVN / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // A round stages blocks 4 rd .. 4 rd + 3 (one per wave) through registers: chunk c
  // is block c / (F_KB F_ROWCH), key row r of it, 16-byte chunk w of that key's
  // [K_nope | K_rope | V]; keys past the visible range load zeros.
  u32x4 stg[F_PER];
  auto load_round = [&](int rd) {
#pragma unroll
    for (int u = 0; u < F_PER; ++u) {
      const int c = tid + 256 * u, kq = c / (F_KB * F_ROWCH), rem = c - kq * (F_KB * F_ROWCH);
      const int r = rem / F_ROWCH, w = rem - r * F_ROWCH;
      const int key = (4 * rd + kq) * F_KB + r;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (key < count) {
        const float* src = w < DN / 4 ? knb + ((size_t)key * H + h) * DN + 4 * w
                         : w < DQK / 4 ? krb + (size_t)key * DR + 4 * (w - DN / 4)
                                       : vb + ((size_t)key * H + h) * DVN + 4 * (w - DQK / 4);
        val = *(const u32x4*)src;
      }
      stg[u] = val;
    }
  };
  auto store_round = [&]() {
#pragma unroll
    for (int u = 0; u < F_PER; ++u) {
      const int c = tid + 256 * u, kq = c / (F_KB * F_ROWCH), rem = c - kq * (F_KB * F_ROWCH);
      const int r = rem / F_ROWCH, w = rem - r * F_ROWCH;
      unsigned char* blk = smem + kq * F_BLK;
      unsigned char* dst = w < DQK / 4 ? blk + r * F_KROW + 16 * w : blk + F_KB * F_KROW + r * F_VROW + 16 * (w - DQK / 4);
      *(u32x4*)dst = stg[u];
    }
  };

  if (nround > 0) {
    load_round(0);
    store_round();
  }
  __syncthreads();
  for (int rd = 0; rd < nround; ++rd) {
    if (rd + 1 < nround) load_round(rd + 1);
    const int kb = 4 * rd + wave;                   // this wave's key block
    if (kb < nkb) {
      const unsigned char* ks = smem + wave * F_BLK;
      const unsigned char* vs = ks + F_KB * F_KROW;
      // S^T (16 keys x 16 queries): lane holds query c16, keys 4 g + j of the block
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* rowp = (const float*)(ks + c16 * F_KROW) + g;
#pragma unroll
      for (int kc = 0; kc < DQK / 4; ++kc) sacc = mfma16x16x4f32(rowp[4 * kc], qf[kc], sacc);
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kb * F_KB + 4 * g + j;
        const bool v = key < count && (!causal || key <= p);
        x[j] = v ? sacc[j] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[j]);
      }
      tmax = group4_max(tmax);
      const float mnew = fmaxf(m, tmax);
      float pv[4];
      float alpha = 1.f, psum = 0.f;
      if (mnew == -INFINITY) {
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[j] = 0.f;
      } else {
        alpha = exp2_fast(m - mnew);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[j] = exp2_fast(x[j] - mnew);
          psum += pv[j];
        }
      }
      psum = group4_sum(psum);
      lsum = lsum * alpha + psum;
      m = mnew;
      // O^T += V^T P^T: MFMA j covers keys 4 g' + j of the lane groups g'; its B
      // operand is this lane's own weight
#pragma unroll
      for (int db = 0; db < DVN / 16; ++db) {
        o[db] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = ((const float*)(vs + (4 * g + j) * F_VROW))[16 * db + c16];
          o[db] = mfma16x16x4f32(a, pv[j], o[db]);
        }
      }
    }
    __syncthreads();                                // every wave is done with this round's blocks
    if (rd + 1 < nround) {
      store_round();
      __syncthreads();
    }
  }

  // Merge: wave w's record is its max and sum per query and its 16 x 128 partial
  // output; wave w then finishes dims 32 w .. 32 w + 31 of the 16 queries.
  float* rec = (float*)smem;
  if (g == 0) {
    rec[wave * F_QB + c16] = m;
    rec[64 + wave * F_QB + c16] = lsum;
  }
  float* orec = rec + 128 + (wave * F_QB + c16) * F_OROW + 4 * g;
#pragma unroll
  for (int db = 0; db < DVN / 16; ++db) *(f32x4*)(orec + 16 * db) = o[db];
  __syncthreads();
  float mw[4], mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = rec[w * F_QB + c16];
    mx = fmaxf(mx, mw[w]);
  }
  float wt[4], lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = mx == -INFINITY ? 0.f : exp2_fast(mw[w] - mx);
    lt += rec[64 + w * F_QB + c16] * wt[w];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int db = 2 * wave + e;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += *(const f32x4*)(rec + 128 + (w * F_QB + c16) * F_OROW + 16 * db + 4 * g) * wt[w];
      *(f32x4*)(out + (((size_t)b * L + i) * H + h) * DVN + 16 * db + 4 * g) = acc * inv;
    }
  }
}

// bf16 path.
//
// Work: a query tile is 128 queries of one head. Causal tiles grow linearly
// with their index, so each workgroup runs the pair (tile p, tile nq-1-p) back
// to back: every workgroup carries the same work, and with one workgroup per
// compute unit none of them idles at the end.
//
// Workgroup: 8 / NBLK waves. A wave owns NBLK blocks of 32 queries (the 32 columns
// of 32x32x16 MFMAs) and one key half of every 64-key step; the two waves of a
// query group (halves 0 and 1) merge their (max, sum, output) through LDS at the
// end of the tile. With two blocks a wave reads each K and V^T fragment from LDS
// once for two MFMAs.
//
// Per step and block: S^T (32 keys x 32 queries) = K_row . Q^T in 12 MFMAs over
// the 192-deep [K_nope | K_rope] row; lanes l and l+32 hold the 32 scores of one
// query. P^T rounded to bf16 is the B operand of O^T += V^T . P^T (8 MFMAs, V^T
// read with LDS transpose reads in the key order of the S^T accumulator layout).
//
// Software pipeline: step t issues the MFMAs of S(t+1) and of P(t-1) V while its
// vector instructions turn S(t) into the weights P(t), so the exponentials of a
// wave run under its own matrix work. The output rescale of a moved maximum is
// applied after the value MFMAs of the step.
//
// K and V stream through two-stage LDS rings by direct global->LDS loads issued a
// step ahead (K(t+2) and V(t) at the top of step t): one barrier per step.
#ifndef NB_NBLK
#define NB_NBLK 1
#endif
#ifndef NB_VALU_PER_MFMA
#define NB_VALU_PER_MFMA 4
#endif
namespace {
constexpr int NB_QT = 128;                              // queries per tile
constexpr int NB_KT = 64;                               // keys per step
constexpr int NB_NROW = DN * 2 + 16;                    // LDS K_nope row + pad (272 B)
constexpr int NB_RROW = DR * 2 + 16;                    // LDS K_rope row + pad (144 B)
constexpr int NB_VROW = DVN * 2 + 64;                   // LDS V row + pad: rows 16 banks apart, transpose reads conflict-free
constexpr int NB_NCH = NB_NROW / 16, NB_RCH = NB_RROW / 16, NB_VCH = NB_VROW / 16;  // 16-byte chunks per row
constexpr int NB_KSTAGE = NB_KT * (NB_NROW + NB_RROW);  // K_nope rows, then K_rope rows
constexpr int NB_VSTAGE = NB_KT * NB_VROW;
constexpr int NB_DN = NB_KT * NB_NROW / 1024;           // 1 KB direct loads per step: K_nope
constexpr int NB_DK = NB_DN + NB_KT * NB_RROW / 1024;   // K_nope + K_rope
constexpr int NB_DV = NB_KT * NB_VROW / 1024;           // V
constexpr int NB_LDS = 2 * NB_KSTAGE + 2 * NB_VSTAGE;
constexpr float NB_SLACK = 8.f;                         // log2 of the largest unnormalised weight
constexpr int NB_XREC = 2 + 2 * 16;                     // merge record per lane and block: m, l, two output blocks
static_assert(NB_KT * NB_NROW % 1024 == 0 && NB_KT * NB_RROW % 1024 == 0 && NB_KT * NB_VROW % 1024 == 0,
              "rows fill whole 1 KB loads");
static_assert(8 * NB_XREC * 64 * 4 <= NB_LDS, "merge area fits the rings");
}  // namespace

// Combine lanes l and l^32 (the two row halves of a 32x32 accumulator column).
// Both lanes see the operands in the same order, so they agree bit for bit.
__device__ __forceinline__ float half_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int NBLK>
__global__ __launch_bounds__(512 / NBLK) __attribute__((amdgpu_waves_per_eu(2 / NBLK, 2 / NBLK))) void
nonabsorbed_bf16_kernel(const uint16_t* __restrict__ qn, const uint16_t* __restrict__ qr,
                        const uint16_t* __restrict__ kn, const uint16_t* __restrict__ kr,
                        const uint16_t* __restrict__ vv, uint16_t* __restrict__ out, int L, int N, int H, int nq,
                        int causal, float scale_log2) {
  constexpr int QG = 4 / NBLK;                  // query groups per tile
  constexpr int NW = 2 * QG;                    // waves
  constexpr int KSLOT = (NB_DK + NW - 1) / NW, VSLOT = (NB_DV + NW - 1) / NW;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NB_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int qg = wave % QG, kh = wave / QG;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int pair = blockIdx.x / H, h = blockIdx.x - pair * H, b = blockIdx.y;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(DSA_LDS void*)&smem[0];
  // With a positive scale, masks and maxima work on raw scores and the scale goes
  // into the exponent's fused multiply-add; otherwise scores are scaled first.
  const bool pos = scale_log2 > 0.f;
  const float mul = pos ? scale_log2 : 1.f;

  // Direct loads of one step. K load j (j < NB_DK) fills K-stage bytes
  // [1024 j, 1024 j + 1024), lane l chunk 64 j + l of the K_nope rows (NB_NCH
  // chunks per key, the last one padding) for j < NB_DN, else of the K_rope rows;
  // V load v fills chunk 64 v + l of the V rows (NB_VCH chunks per key, the last
  // four padding). A padding chunk loads the row's last data chunk again; rows past
  // the last key repeat it (their scores are masked). Wave w issues K loads w,
  // w + NW, ... and V loads w, w + NW, ...
  const size_t nstride = (size_t)H * DN * 2, vstride = (size_t)H * DVN * 2;
  constexpr int rstride = DR * 2;
  const unsigned char* kn_b = (const unsigned char*)kn + (size_t)b * N * nstride + (size_t)h * DN * 2;
  const unsigned char* kr_b = (const unsigned char*)kr + (size_t)b * N * rstride;
  const unsigned char* v_b = (const unsigned char*)vv + (size_t)b * N * vstride + (size_t)h * DVN * 2;
  // (the empty asm keeps the row arithmetic of the rare clamped tile where it is used)
  auto k_off = [&](int j, int rmax) __attribute__((always_inline)) -> uint32_t {
    int l = lane;
    asm volatile("" : "+v"(l));
    if (j < NB_DN) {
      const int c = 64 * j + l, r = min(c / NB_NCH, rmax), u = min(c % NB_NCH, DN * 2 / 16 - 1);
      return (uint32_t)(r * nstride) + 16 * u;
    }
    const int c = 64 * (j - NB_DN) + l, r = min(c / NB_RCH, rmax), u = min(c % NB_RCH, DR * 2 / 16 - 1);
    return (uint32_t)(r * rstride) + 16 * u;
  };
  auto v_off = [&](int v, int rmax) __attribute__((always_inline)) -> uint32_t {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int c = 64 * v + l, r = min(c / NB_VCH, rmax), u = min(c % NB_VCH, DVN * 2 / 16 - 1);
    return (uint32_t)(r * vstride) + 16 * u;
  };
  uint32_t ko[KSLOT], vo[VSLOT];
#pragma unroll
  for (int s = 0; s < KSLOT; ++s) ko[s] = k_off(min(NW * s + wave_u, NB_DK - 1), NB_KT - 1);
#pragma unroll
  for (int s = 0; s < VSLOT; ++s) vo[s] = v_off(min(NW * s + wave_u, NB_DV - 1), NB_KT - 1);
  // (the empty asm makes the scalar address arithmetic of a call local to it, so the
  // compiler does not keep every slot's addresses live across the loop)
  auto issue_k = [&](int tile, int st) __attribute__((always_inline)) {
    int wu = wave_u;
    asm volatile("" : "+s"(wu));
    const int key0 = tile * NB_KT, rmax = N - 1 - key0;
    const unsigned char* nb = kn_b + (size_t)key0 * nstride;
    const unsigned char* rb = kr_b + (size_t)key0 * rstride;
    const uint32_t dst = lds0 + st * NB_KSTAGE;
#pragma unroll
    for (int s = 0; s < KSLOT; ++s) {
      const int j = NW * s + wu;
      if (j < NB_DK)
        dma16s(uniform_ptr(j < NB_DN ? nb : rb), rmax >= NB_KT - 1 ? ko[s] : k_off(j, rmax), dst + 1024 * j);
    }
  };
  auto issue_v = [&](int tile, int st) __attribute__((always_inline)) {
    int wu = wave_u;
    asm volatile("" : "+s"(wu));
    const int key0 = tile * NB_KT, rmax = N - 1 - key0;
    const unsigned char* vb = v_b + (size_t)key0 * vstride;
    const uint32_t dst = lds0 + 2 * NB_KSTAGE + st * NB_VSTAGE;
#pragma unroll
    for (int s = 0; s < VSLOT; ++s) {
      const int v = NW * s + wu;
      if (v < NB_DV) dma16s(uniform_ptr(vb), rmax >= NB_KT - 1 ? vo[s] : v_off(v, rmax), dst + 1024 * v);
    }
  };

  // LDS fragment addresses. K (A operand of S^T): row = key 32 kh + col of the
  // step, k = dims 16 kk + 8 g + e. V^T (A operand of O^T): lane points at key
  // 32 kh + 16 ks + 4 g + (lane%16)/4 (+8 for the upper four k entries), dims
  // 32 db + 16 ((lane/16)%2) + 4 (lane%4).
  const int krow = 32 * kh + col;
  const uint32_t ka_n = krow * NB_NROW + 16 * g, ka_r = NB_KT * NB_NROW + krow * NB_RROW + 16 * g;
  const uint32_t va = 2 * NB_KSTAGE + (32 * kh + 4 * g + ((lane & 15) >> 2)) * NB_VROW +
                      2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  auto kfrag = [&](int st, int kk) __attribute__((always_inline)) {
    return *(const bf16x8*)(smem + st * NB_KSTAGE + (kk < DN / 16 ? ka_n + 32 * kk : ka_r + 32 * (kk - DN / 16)));
  };
  auto vfrag = [&](int st, int ks, int db) __attribute__((always_inline)) {
    const unsigned char* p = smem + va + st * NB_VSTAGE + 16 * ks * NB_VROW + 64 * db;
    return join_bf16x8(lds_read_tr16(p), lds_read_tr16(p + 8 * NB_VROW));
  };

  const int npass = (nq - 1 - pair == pair) ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = pass == 0 ? pair : nq - 1 - pair;
    const int i0 = qt * NB_QT, iw = i0 + 32 * NBLK * qg;
    const int count = causal ? N - L + min(L - 1, i0 + NB_QT - 1) + 1 : N;
    const int ntiles = (count + NB_KT - 1) / NB_KT;
    const int plim = causal ? N - L + iw : N - 1;          // keys up to plim are visible to every query of the wave
    int qi[NBLK], p[NBLK];
    bf16x8 qf[NBLK][DQK / 16];
#pragma unroll
    for (int x = 0; x < NBLK; ++x) {
      qi[x] = iw + 32 * x + col;
      p[x] = causal ? N - L + qi[x] : N - 1;                // last visible key of this lane's query
      // Query fragments (B operand): column = query, k = dims 16kk + 8g + e of [Q_nope | Q_rope].
      const size_t qrow = ((size_t)b * L + (qi[x] < L ? qi[x] : 0)) * H + h;
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk)
        qf[x][kk] = kk < DN / 16 ? *(const bf16x8*)(qn + qrow * DN + 16 * kk + 8 * g)
                                 : *(const bf16x8*)(qr + qrow * DR + 16 * (kk - DN / 16) + 8 * g);
    }
    f32x16 o[NBLK][DVN / 32];
#pragma unroll
    for (int x = 0; x < NBLK; ++x)
#pragma unroll
      for (int db = 0; db < DVN / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[x][db][j] = 0.f;
    float m[NBLK], lsum[NBLK];
#pragma unroll
    for (int x = 0; x < NBLK; ++x) {
      m[x] = -INFINITY;
      lsum[x] = 0.f;
    }
    f32x16 s0[NBLK], s1[NBLK];
    bf16x8 p0[NBLK][2], p1[NBLK][2];

    // S of every block from K stage st; K fragments are read three k-steps ahead
    auto scores = [&](int st, f32x16 (&sn)[NBLK]) __attribute__((always_inline)) {
      bf16x8 kf[3];
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) kf[kk] = kfrag(st, kk);
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk) {
        const bf16x8 a = kf[kk % 3];
#pragma unroll
        for (int x = 0; x < NBLK; ++x) sn[x] = mfma32x32x16(a, qf[x][kk], kk ? sn[x] : f32x16{});
        if (kk + 3 < DQK / 16) kf[kk % 3] = kfrag(st, kk + 3);
      }
    };
    // One pipeline step t: S(t+1) if DS, softmax of S(t) if DSM, P(t-1) V if DPV.
    auto iter = [&](auto DS, auto DSM, auto DPV, int t, f32x16 (&sc)[NBLK], f32x16 (&sn)[NBLK],
                    const bf16x8 (&pp)[NBLK][2], bf16x8 (&pc)[NBLK][2]) __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // this wave's loads of K(t+1) and V(t-1) landed
      lds_barrier();                                       // everyone's landed; stages of K(t), V(t-2) free
      if (DS && t + 2 < ntiles) issue_k(t + 2, t & 1);
      if (DSM) issue_v(t, t & 1);
      bool bump[NBLK];
      float alpha[NBLK];
#pragma unroll
      for (int x = 0; x < NBLK; ++x) {
        bump[x] = false;
        alpha[x] = 1.f;
      }
      if (DSM) {
        // keys 32 kh + 8 (j/4) + 4 g + j%4 of the step: mask what lies past the query's
        // limit (diagonal and last steps), scale first for a non-positive scale
        const int k0 = t * NB_KT + 32 * kh;
        if (k0 + 31 > plim || !pos) {
#pragma unroll
          for (int x = 0; x < NBLK; ++x)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const float v = pos ? sc[x][j] : sc[x][j] * scale_log2;
              sc[x][j] = k0 + 8 * (j >> 2) + 4 * g + (j & 3) <= p[x] ? v : -INFINITY;
            }
        }
      }
      if (DS) scores((t + 1) & 1, sn);
      if (DPV) {
        const int st = (t - 1) & 1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < DVN / 32; ++db) {
            const bf16x8 vf = vfrag(st, ks, db);
#pragma unroll
            for (int x = 0; x < NBLK; ++x) o[x][db] = mfma32x32x16(vf, pp[x][ks], o[x][db]);
          }
      }
      if (DSM) {
#pragma unroll
        for (int x = 0; x < NBLK; ++x) {
          float tmax = sc[x][0];
#pragma unroll
          for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, sc[x][j]);
          tmax = half_max(tmax);
          // The reference max moves only when the new scores exceed it by more than
          // 2^NB_SLACK (or on the first visible key): softmax does not depend on the
          // reference, and weights up to 2^NB_SLACK are exact enough in bf16 / fp32.
          bump[x] = (tmax - m[x]) * mul > NB_SLACK;
          const float mnew = bump[x] ? tmax : m[x];
          const float mref = mnew == -INFINITY ? 0.f : mnew;
          const float nb = -mref * mul;
          float pv[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) pv[j] = exp2_fast(fmaf(sc[x][j], mul, nb));
          float ps[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ps[e] = (pv[4 * e] + pv[4 * e + 1]) + (pv[4 * e + 2] + pv[4 * e + 3]);
          const float psum = half_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
          alpha[x] = bump[x] ? exp2_fast((m[x] - mref) * mul) : 1.f;
          lsum[x] = lsum[x] * alpha[x] + psum;
          m[x] = mnew;
          pc[x][0] = pack_bf16x8(pv);
          pc[x][1] = pack_bf16x8(pv + 8);
        }
      }
      // Interleave for the steady-state step: every MFMA is followed by a few
      // vector instructions of the softmax, and the LDS reads run ahead of the
      // MFMAs that use them (K fragments three k-steps, V^T fragments two).
      if constexpr (std::is_same<decltype(DS), std::true_type>::value &&
                    std::is_same<decltype(DSM), std::true_type>::value &&
                    std::is_same<decltype(DPV), std::true_type>::value) {
        constexpr int VPM = NB_VALU_PER_MFMA;
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int kk = 0; kk < DQK / 16; ++kk) {
#pragma unroll
          for (int x = 0; x < NBLK; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
          if (kk + 3 < DQK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (kk == DQK / 16 - 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        }
#pragma unroll
        for (int i = 0; i < DVN / 16; ++i) {
#pragma unroll
          for (int x = 0; x < NBLK; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
          if (i + 2 < DVN / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      // rescale after the value MFMAs of P(t-1), before those of P(t)
      bool any = false;
#pragma unroll
      for (int x = 0; x < NBLK; ++x) any = any || bump[x];
      if (DSM && __ballot(any)) {
#pragma unroll
        for (int x = 0; x < NBLK; ++x)
#pragma unroll
          for (int db = 0; db < DVN / 32; ++db) o[x][db] *= alpha[x];
      }
    };
    // Even steps read S from s0 and write P to p0, odd steps s1 and p1; the loop
    // runs steps in pairs, so every buffer role is fixed at compile time.
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    if (ntiles > 0) {
      issue_k(0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (ntiles > 1) issue_k(1, 1);
      scores(0, s0);
      iter(ntiles > 1, yes, no, 0, s0, s1, p1, p0);
      int t = 1;
      for (; t + 2 < ntiles; t += 2) {
        iter(yes, yes, yes, t, s1, s0, p0, p1);
        iter(yes, yes, yes, t + 1, s0, s1, p1, p0);
      }
      // t is odd here and steps t .. ntiles remain (at most three)
      if (t < ntiles) {
        iter(t + 1 < ntiles, yes, yes, t, s1, s0, p0, p1);
        if (t + 1 < ntiles) {
          iter(no, yes, yes, t + 1, s0, s1, p1, p0);
          iter(no, no, yes, t + 2, s1, s0, p0, p1);
        } else {
          iter(no, no, yes, t + 1, s0, s1, p1, p0);
        }
      } else {
        iter(no, no, yes, t, s1, s0, p0, p1);
      }
    }

    // Merge the two key halves: each wave hands over the output blocks it does
    // not write (half 0 writes dims 0-63, half 1 dims 64-127) with its m and l.
    lds_barrier();                                         // every wave is done with the rings
    float* xw = (float*)smem + wave * NBLK * NB_XREC * 64 + lane;
#pragma unroll
    for (int x = 0; x < NBLK; ++x) {
      float* xr = xw + NB_XREC * x * 64;
      xr[0] = m[x];
      xr[64] = lsum[x];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        xr[(2 + j) * 64] = o[x][kh == 0 ? 2 : 0][j];
        xr[(18 + j) * 64] = o[x][kh == 0 ? 3 : 1][j];
      }
    }
    lds_barrier();
#pragma unroll
    for (int x = 0; x < NBLK; ++x) {
      const float* xp = (const float*)smem + ((wave + QG) % NW) * NBLK * NB_XREC * 64 + NB_XREC * x * 64 + lane;
      const float m2 = xp[0], l2 = xp[64];
      const float mx = fmaxf(m[x], m2);
      const float a1 = mx == -INFINITY ? 0.f : exp2_fast((m[x] - mx) * mul);
      const float a2 = mx == -INFINITY ? 0.f : exp2_fast((m2 - mx) * mul);
      const float lt = lsum[x] * a1 + l2 * a2;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (qi[x] < L) {
        uint16_t* op = out + (((size_t)b * L + qi[x]) * H + h) * DVN + 4 * g;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int db = 2 * kh + e;
          const f32x16 mine = kh == 0 ? o[x][e] : o[x][2 + e];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            f32x4 v4;
#pragma unroll
            for (int q = 0; q < 4; ++q) v4[q] = (mine[4 * jj + q] * a1 + xp[(2 + 16 * e + 4 * jj + q) * 64] * a2) * inv;
            *(bf16x4*)(op + 32 * db + 8 * jj) = __builtin_convertvector(v4, bf16x4);
          }
        }
      }
    }
    lds_barrier();
  }
}


hipError_t launch_nonabsorbed_attn(bool bf16, const void* qn, const void* qr, const void* kn, const void* kr,
                                   const void* v, void* out, int B, int L, int N, int H, int causal, float scale,
                                   hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  if (bf16) {
    const int nq = (L + NB_QT - 1) / NB_QT;
    dim3 grid((nq + 1) / 2 * H, B), block(64 * 8 / NB_NBLK);
    KernelTrace kt("nonabsorbed_attn_bf16", stream);
    hipLaunchKernelGGL(nonabsorbed_bf16_kernel<NB_NBLK>, grid, block, 0, stream, (const uint16_t*)qn, (const uint16_t*)qr,
                       (const uint16_t*)kn, (const uint16_t*)kr, (const uint16_t*)v, (uint16_t*)out, L, N, H, nq,
                       causal, scale_log2);
    return hipGetLastError();
  }
  dim3 grid((L + F_QB - 1) / F_QB, H, B), block(256);
  KernelTrace kt("nonabsorbed_attn_f32", stream);
  hipLaunchKernelGGL(nonabsorbed_f32_kernel, grid, block, 0, stream, (const float*)qn, (const float*)qr,
                     (const float*)kn, (const float*)kr, (const float*)v, (float*)out, L, N, H, causal, scale_log2);
  return hipGetLastError();
}

}  // namespace dsa

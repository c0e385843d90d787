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
// Decomposition: one workgroup per (head, 64 queries); each of its 4 waves owns
// 16 queries (one MFMA column each). Keys stream through LDS in tiles of 32,
// double-buffered. The causal limit of the workgroup's last query bounds the
// key loop; per-lane masks handle the diagonal.
//
// bf16 path: 16x16x32 bf16 MFMA; P is rounded to bf16 for the value product,
// accumulation is fp32. fp32 path: 16x16x4 fp32 MFMA throughout.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int DN = 128, DR = 64, DQK = DN + DR, DVN = 128;
static_assert(DVN == DN, "K_nope and V rows share one address formula");
constexpr int T = 32;
}  // namespace

template <bool BF16>
struct NonAbsTraits {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int KN_CH = DN * ESZ / 16;        // 16-byte chunks from K_nope
  static constexpr int KR_CH = DR * ESZ / 16;        // from K_rope
  static constexpr int K_CH = KN_CH + KR_CH;
  static constexpr int V_CH = DVN * ESZ / 16;
  static constexpr int ROW_CH = K_CH + V_CH;
  static constexpr int KROWB = K_CH * 16 + 16;       // padded LDS strides
  static constexpr int VROWB = V_CH * 16 + 16;
  static constexpr int STAGE = T * (KROWB + VROWB);
};

template <bool BF16>
__global__ __launch_bounds__(256) void nonabsorbed_attn_kernel(
    const void* __restrict__ qn_, const void* __restrict__ qr_, const void* __restrict__ kn_,
    const void* __restrict__ kr_, const void* __restrict__ v_, void* __restrict__ out_, int L, int N, int H,
    int causal, float scale_log2) {
  using Tr = NonAbsTraits<BF16>;
  constexpr int ESZ = Tr::ESZ;
  constexpr int NT = 256;
  constexpr int PER = (T * Tr::ROW_CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][Tr::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.y, b = blockIdx.z;
  // longest rows first: the last query tile is launched first
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int i0 = qt * 64;
  const int i = i0 + wave * 16 + c16;              // this lane's query (column)
  const bool qvalid = i < L;
  const int p = N - L + i;                          // its causal limit
  const int wg_last = min(L - 1, i0 + 63);
  const int count = causal ? (N - L + wg_last + 1) : N;

  const unsigned char* qn = (const unsigned char*)qn_;
  const unsigned char* qr = (const unsigned char*)qr_;
  const unsigned char* kn = (const unsigned char*)kn_ + (size_t)b * N * H * DN * ESZ;
  const unsigned char* kr = (const unsigned char*)kr_ + (size_t)b * N * DR * ESZ;
  const unsigned char* vv = (const unsigned char*)v_ + (size_t)b * N * H * DVN * ESZ;

  // Query fragments (B operand): column = query, k = dims of [Q_nope | Q_rope].
  constexpr int QREG = BF16 ? DQK / 32 : DQK / 4;
  bf16x8 qb[BF16 ? QREG : 1];
  float qf[BF16 ? 1 : QREG];
  {
    const int ii = qvalid ? i : 0;
    const size_t qoff_n = (((size_t)b * L + ii) * H + h) * DN;
    const size_t qoff_r = (((size_t)b * L + ii) * H + h) * DR;
    if constexpr (BF16) {
      const uint16_t* pn = (const uint16_t*)qn + qoff_n + 8 * g;
      const uint16_t* pr = (const uint16_t*)qr + qoff_r + 8 * g;
#pragma unroll
      for (int kc = 0; kc < QREG; ++kc) qb[kc] = kc < DN / 32 ? *(const bf16x8*)(pn + 32 * kc) : *(const bf16x8*)(pr + 32 * (kc - DN / 32));
    } else {
      const float* pn = (const float*)qn + qoff_n + g;
      const float* pr = (const float*)qr + qoff_r + g;
#pragma unroll
      for (int kc = 0; kc < QREG; ++kc) qf[kc] = kc < DN / 4 ? pn[4 * kc] : pr[4 * (kc - DN / 4)];
    }
  }
  f32x4 o[DVN / 16];
#pragma unroll
  for (int db = 0; db < DVN / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  u32x4 stg[PER];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      if (c < T * Tr::ROW_CH) {
        const int r = c / Tr::ROW_CH, w = c - r * Tr::ROW_CH;
        const int key = t * T + r;
        u32x4 val = u32x4{0u, 0u, 0u, 0u};
        if (key < count) {
          const unsigned char* src;
          if (w < Tr::KN_CH) src = kn + (((size_t)key * H + h) * DN) * ESZ + w * 16;
          else if (w < Tr::K_CH) src = kr + ((size_t)key * DR) * ESZ + (w - Tr::KN_CH) * 16;
          else src = vv + (((size_t)key * H + h) * DVN) * ESZ + (w - Tr::K_CH) * 16;
          val = *(const u32x4*)src;
        }
        stg[u] = val;
      }
    }
  };
  auto store_tile = [&](int s) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      if (c < T * Tr::ROW_CH) {
        const int r = c / Tr::ROW_CH, w = c - r * Tr::ROW_CH;
        unsigned char* dst = w < Tr::K_CH ? smem[s] + r * Tr::KROWB + w * 16
                                          : smem[s] + T * Tr::KROWB + r * Tr::VROWB + (w - Tr::K_CH) * 16;
        *(u32x4*)dst = stg[u];
      }
    }
  };

  const int ntiles = (count + T - 1) / T;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int s = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const unsigned char* ks = smem[s];
    const unsigned char* vs = smem[s] + T * Tr::KROWB;

    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        const unsigned char* rowp = ks + (16 * kb + c16) * Tr::KROWB + 16 * g;
#pragma unroll
        for (int kc = 0; kc < QREG; ++kc) sacc[kb] = mfma16x16x32(*(const bf16x8*)(rowp + 64 * kc), qb[kc], sacc[kb]);
      } else {
        const float* rowp = (const float*)(ks + (16 * kb + c16) * Tr::KROWB) + g;
#pragma unroll
        for (int kc = 0; kc < QREG; ++kc) sacc[kb] = mfma16x16x4f32(rowp[4 * kc], qf[kc], sacc[kb]);
      }
    }
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = t * T + 16 * kb + 4 * g + j;
        const bool v = key < count && (!causal || key <= p);
        const float xv = v ? sacc[kb][j] * scale_log2 : -INFINITY;
        x[kb * 4 + j] = xv;
        tmax = fmaxf(tmax, xv);
      }
    tmax = group4_max(tmax);
    const float mnew = fmaxf(m, tmax);
    float pv[8];
    float alpha = 1.f, psum = 0.f;
    if (mnew == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
    } else {
      alpha = exp2_fast(m - mnew);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = exp2_fast(x[e] - mnew);
        psum += pv[e];
      }
    }
    psum = group4_sum(psum);
    lsum = lsum * alpha + psum;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DVN / 16; ++db) o[db] *= alpha;
    if constexpr (BF16) {
      const bf16x8 pk = pack_bf16x8(pv);
      const unsigned char* vb = vs + (4 * g + (c16 >> 2)) * Tr::VROWB + 8 * (c16 & 3);
#pragma unroll
      for (int db = 0; db < DVN / 16; ++db) {
        const short4v lo = lds_read_tr16(vb + 32 * db);
        const short4v hi = lds_read_tr16(vb + 16 * Tr::VROWB + 32 * db);
        o[db] = mfma16x16x32(join_bf16x8(lo, hi), pk, o[db]);
      }
    } else {
      // MFMA (kb, j) covers keys 16kb + 4g' + j for lane groups g'; its B operand is this lane's own p.
#pragma unroll
      for (int db = 0; db < DVN / 16; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = ((const float*)(vs + (16 * kb + 4 * g + j) * Tr::VROWB))[16 * db + c16];
            o[db] = mfma16x16x4f32(a, pv[kb * 4 + j], o[db]);
          }
    }
    if (t + 1 < ntiles) store_tile(s ^ 1);
    __syncthreads();
  }

  if (qvalid) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const size_t ooff = (((size_t)b * L + i) * H + h) * DVN + 4 * g;
#pragma unroll
    for (int db = 0; db < DVN / 16; ++db) {
      if constexpr (BF16) {
        uint2 w;
        w.x = (uint32_t)f2bf_bits(o[db][0] * inv) | ((uint32_t)f2bf_bits(o[db][1] * inv) << 16);
        w.y = (uint32_t)f2bf_bits(o[db][2] * inv) | ((uint32_t)f2bf_bits(o[db][3] * inv) << 16);
        *(uint2*)((uint16_t*)out_ + ooff + 16 * db) = w;
      } else {
        *(f32x4*)((float*)out_ + ooff + 16 * db) = o[db] * inv;
      }
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
// Workgroup: 8 waves. Wave w owns queries 32*(w%4) .. +31 of the tile (the 32
// columns of 32x32x16 MFMAs) and key half w/4 of every 64-key step, so the two
// waves of a query group split the keys and merge their (max, sum, output)
// through LDS at the end of the tile.
//
// Keys stream through two LDS stages; the next step is loaded into registers
// while the current one is consumed, then stored to the other stage: one
// barrier per step.
//
// Per step and wave: S^T (32 keys x 32 queries) = K_row . Q^T in 12 MFMAs over
// the 192-deep [K_nope | K_rope] row; lanes l and l+32 hold the 32 scores of one
// query; P^T rounded to bf16 is the B operand of O^T += V^T . P^T (8 MFMAs, V^T
// read with LDS transpose reads in the key order of the S^T accumulator layout).
namespace {
constexpr int NB_T = 32;                               // keys per wave per step
constexpr int NB_KT = 2 * NB_T;                        // keys per step
constexpr int NB_KROW = DQK * 2 + 16;                  // LDS K row: [K_nope(h) | K_rope] + pad
constexpr int NB_VROW = DVN * 2 + 64;                  // LDS V row + pad: rows 16 banks apart, transpose reads conflict-free
constexpr int NB_KREG = NB_KT * NB_KROW;
constexpr int NB_STAGE = NB_KREG + NB_KT * NB_VROW;
constexpr int NB_NW = 8;
constexpr int NB_RCH = (DQK + DVN) * 2 / 16;           // 16-byte chunks per key: 16 K_nope, 8 K_rope, 16 V
constexpr int NB_PER = NB_KT * NB_RCH / (NB_NW * 64);  // chunks per thread per step
constexpr int NB_QT = 128;
constexpr float NB_SLACK = 8.f;                        // log2 of the largest unnormalised weight
constexpr int NB_XCH = 2 + 2 * 16;                     // merge record per lane: m, l, two output blocks
static_assert(NB_KT * NB_RCH % (NB_NW * 64) == 0, "step chunks must divide the workgroup");
static_assert(NB_NW * NB_XCH * 64 * 4 <= 2 * NB_STAGE, "merge area fits the stages");
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

__global__ __launch_bounds__(512) void nonabsorbed_bf16_kernel(
    const uint16_t* __restrict__ qn, const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vv, uint16_t* __restrict__ out, int L, int N,
    int H, int nq, int causal, float scale_log2) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * NB_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int qg = wave & 3, half = wave >> 2;
  const int pair = blockIdx.x / H, h = blockIdx.x - pair * H, b = blockIdx.y;
  const size_t kb0 = (size_t)b * N;
  const float sl = scale_log2;

  // Loads of one step (64 keys): loads 0-1 take K_nope (16 lanes per 256-byte
  // row, keys tid/16 and 32 + tid/16), load 2 K_rope (8 lanes per 128-byte row,
  // key tid/8), loads 3-4 V like K_nope. Keys past the context repeat the last
  // key (their scores are masked).
  static_assert(NB_PER == 5 && NB_KT == 64 && NB_NW * 64 == 512, "load map assumes 64 keys x 512 threads");
  const int r16 = tid >> 4, c16b = (tid & 15) * 16, r8 = tid >> 3, c8b = (tid & 7) * 16;
  const unsigned char* kn_b = (const unsigned char*)kn + (size_t)h * DN * 2 + c16b;
  const unsigned char* kr_b = (const unsigned char*)kr + c8b;
  const unsigned char* v_b = (const unsigned char*)vv + (size_t)h * DVN * 2 + c16b;
  const size_t kstride = (size_t)H * DN * 2;
  auto fetch = [&](u32x4 (&pf)[NB_PER], int t) {
    const int kt = t * NB_KT;
    const size_t ka = kb0 + min(kt + r16, N - 1), kb = kb0 + min(kt + 32 + r16, N - 1);
    const size_t kc = kb0 + min(kt + r8, N - 1);
    pf[0] = *(const u32x4*)(kn_b + ka * kstride);
    pf[1] = *(const u32x4*)(kn_b + kb * kstride);
    pf[2] = *(const u32x4*)(kr_b + kc * (DR * 2));
    pf[3] = *(const u32x4*)(v_b + ka * kstride);
    pf[4] = *(const u32x4*)(v_b + kb * kstride);
  };
  const int ldk0 = r16 * NB_KROW + c16b, ldk1 = (32 + r16) * NB_KROW + c16b;
  const int ldr = r8 * NB_KROW + DN * 2 + c8b;
  const int ldv0 = NB_KREG + r16 * NB_VROW + c16b, ldv1 = NB_KREG + (32 + r16) * NB_VROW + c16b;
  auto stage_in = [&](const u32x4 (&pf)[NB_PER], int st) {
    unsigned char* sb = smem + st * NB_STAGE;
    *(u32x4*)(sb + ldk0) = pf[0];
    *(u32x4*)(sb + ldk1) = pf[1];
    *(u32x4*)(sb + ldr) = pf[2];
    *(u32x4*)(sb + ldv0) = pf[3];
    *(u32x4*)(sb + ldv1) = pf[4];
  };

  const int npass = (nq - 1 - pair == pair) ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    const int qt = pass == 0 ? pair : nq - 1 - pair;
    const int i0 = qt * NB_QT, iw = i0 + 32 * qg, i = iw + col;
    const bool qvalid = i < L;
    const int p = causal ? N - L + i : N - 1;             // last visible key of this lane's query
    const int count = causal ? N - L + min(L - 1, i0 + NB_QT - 1) + 1 : N;
    const int wcount = iw >= L ? 0 : (causal ? N - L + min(L - 1, iw + 31) + 1 : N);
    const int wsafe = causal ? N - L + iw : N;            // keys below this are visible to all queries of the wave
    const int ntiles = (count + NB_KT - 1) / NB_KT;

    // Query fragments (B operand): column = query, k = dims 16kk + 8g + e of [Q_nope | Q_rope].
    bf16x8 qb[DQK / 16];
    {
      const size_t qrow = ((size_t)b * L + (qvalid ? i : 0)) * H + h;
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk)
        qb[kk] = kk < DN / 16 ? *(const bf16x8*)(qn + qrow * DN + 16 * kk + 8 * g)
                              : *(const bf16x8*)(qr + qrow * DR + 16 * (kk - DN / 16) + 8 * g);
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk) asm volatile("" ::"v"(qb[kk]));
    }
    f32x16 o[DVN / 32];
#pragma unroll
    for (int db = 0; db < DVN / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    // Steps alternate between LDS stages 0 and 1; the next step's rows are
    // loaded into registers while this one is consumed.
    auto step = [&](int t, int st) {
      const int k0 = t * NB_KT + NB_T * half;
      if (k0 >= wcount) return;
      const unsigned char* ks = smem + st * NB_STAGE + NB_T * half * NB_KROW;
      const unsigned char* vs = smem + st * NB_STAGE + NB_KREG + NB_T * half * NB_VROW;
      f32x16 sacc;
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
      const unsigned char* kp = ks + col * NB_KROW + 16 * g;
      // K fragments rotate through four registers so that four LDS reads are in
      // flight ahead of the MFMA chain
      bf16x8 kf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[kk] = *(const bf16x8*)(kp + 32 * kk);
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk) {
        sacc = mfma32x32x16(kf[kk & 3], qb[kk], sacc);
        if (kk + 4 < DQK / 16) kf[kk & 3] = *(const bf16x8*)(kp + 32 * (kk + 4));
      }
      // schedule: 4 LDS reads, then (MFMA, LDS read) x 8, then the last 4 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int kk = 0; kk < DQK / 16 - 4; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // this lane holds keys k0 + 8*(j/4) + 4g + j%4 of query i
      if (k0 + NB_T - 1 >= wsafe) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (k0 + 8 * (j >> 2) + 4 * g + (j & 3) > p) sacc[j] = -INFINITY;
      }
      float tmax = sacc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, sacc[j]);
      tmax = half_max(tmax);
      // The reference max m moves only when the new scores exceed it by more than
      // 2^NB_SLACK (or on the first visible key): softmax does not depend on the
      // reference, and weights up to 2^NB_SLACK are exact enough in bf16 / fp32.
      // The output rescale then happens a few times per query instead of most steps.
      const bool bump = (tmax - m) * sl > NB_SLACK;
      const float mnew = bump ? tmax : m;
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float nb = -mref * sl;
      float pv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pv[j] = exp2_fast(fmaf(sacc[j], sl, nb));
      // the normaliser sums the bf16-rounded weights the value product uses
      bf16x8 pk[2];
      pk[0] = pack_bf16x8(pv);
      pk[1] = pack_bf16x8(pv + 8);
      const float psum = half_sum(sum_bf16x8(pk[0]) + sum_bf16x8(pk[1]));
      if (__ballot(bump)) {
        const float alpha = bump ? exp2_fast((m - mref) * sl) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DVN / 32; ++db) o[db] *= alpha;
      }
      lsum += psum;
      m = mnew;
      // V^T fragment: lane points at key 16ks + 4g + (lane%16)/4 (+8 for the upper
      // four k entries), dims 32db + 16*((lane/16)%2) + 4*(lane%4).
      const unsigned char* vb = vs + (4 * g + ((lane & 15) >> 2)) * NB_VROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int db = 0; db < DVN / 32; ++db) {
          const short4v lo = lds_read_tr16(vb + 16 * ks2 * NB_VROW + 64 * db);
          const short4v hi = lds_read_tr16(vb + (16 * ks2 + 8) * NB_VROW + 64 * db);
          o[db] = mfma32x32x16(join_bf16x8(lo, hi), pk[ks2], o[db]);
        }
    };

    u32x4 pf[NB_PER];
    fetch(pf, 0);
    stage_in(pf, 0);
    lds_barrier();
    for (int t = 0; t < ntiles; ++t) {
      fetch(pf, min(t + 1, ntiles - 1));
      step(t, t & 1);
      stage_in(pf, (t + 1) & 1);
      lds_barrier();
    }

    // Merge the two key halves: each wave hands over the output blocks it does
    // not write (half 0 writes dims 0-63, half 1 dims 64-127) with its m and l.
    float* xw = (float*)smem + wave * NB_XCH * 64 + lane;
    xw[0] = m;
    xw[64] = lsum;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      xw[(2 + j) * 64] = o[half == 0 ? 2 : 0][j];
      xw[(18 + j) * 64] = o[half == 0 ? 3 : 1][j];
    }
    lds_barrier();
    const float* xp = (const float*)smem + (wave ^ 4) * NB_XCH * 64 + lane;
    const float m2 = xp[0], l2 = xp[64];
    const float mx = fmaxf(m, m2);
    const float a1 = mx == -INFINITY ? 0.f : exp2_fast((m - mx) * sl);
    const float a2 = mx == -INFINITY ? 0.f : exp2_fast((m2 - mx) * sl);
    const float lt = lsum * a1 + l2 * a2;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid) {
      uint16_t* op = out + (((size_t)b * L + i) * H + h) * DVN + 4 * g;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int db = 2 * half + e;
        const f32x16 mine = half == 0 ? o[e] : o[2 + e];
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
    lds_barrier();
  }
}

hipError_t launch_nonabsorbed_attn(bool bf16, const void* qn, const void* qr, const void* kn, const void* kr,
                                   const void* v, void* out, int B, int L, int N, int H, int causal, float scale,
                                   hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  if (bf16) {
    const int nq = (L + NB_QT - 1) / NB_QT;
    dim3 grid((nq + 1) / 2 * H, B), block(512);
    KernelTrace kt("nonabsorbed_attn_bf16", stream);
    hipLaunchKernelGGL(nonabsorbed_bf16_kernel, grid, block, 0, stream, (const uint16_t*)qn, (const uint16_t*)qr,
                       (const uint16_t*)kn, (const uint16_t*)kr, (const uint16_t*)v, (uint16_t*)out, L, N, H, nq,
                       causal, scale_log2);
    return hipGetLastError();
  }
  dim3 grid((L + 63) / 64, H, B), block(256);
  KernelTrace kt("nonabsorbed_attn_f32", stream);
  hipLaunchKernelGGL((nonabsorbed_attn_kernel<false>), grid, block, 0, stream, qn, qr, kn, kr, v, out, L, N, H, causal, scale_log2);
  return hipGetLastError();
}

}  // namespace dsa

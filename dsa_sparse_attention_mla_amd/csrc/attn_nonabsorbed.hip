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
      alpha = exp2f(m - mnew);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = exp2f(x[e] - mnew);
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

hipError_t launch_nonabsorbed_attn(bool bf16, const void* qn, const void* qr, const void* kn, const void* kr,
                                   const void* v, void* out, int B, int L, int N, int H, int causal, float scale,
                                   hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((L + 63) / 64, H, B), block(256);
  KernelTrace kt(bf16 ? "nonabsorbed_attn_bf16" : "nonabsorbed_attn_f32", stream);
  if (bf16)
    hipLaunchKernelGGL((nonabsorbed_attn_kernel<true>), grid, block, 0, stream, qn, qr, kn, kr, v, out, L, N, H, causal, scale_log2);
  else
    hipLaunchKernelGGL((nonabsorbed_attn_kernel<false>), grid, block, 0, stream, qn, qr, kn, kr, v, out, L, N, H, causal, scale_log2);
  return hipGetLastError();
}

}  // namespace dsa

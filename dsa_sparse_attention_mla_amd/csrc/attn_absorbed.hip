// Absorbed (latent-space) MLA attention over joined 576-wide latent+rope rows.
//
// One kernel serves two calls:
//  * dense absorbed prefill (keys 0..p_i of a contiguous cache, bottom-right
//    causal), and
//  * sparse prefill: each query attends only to the rows its index list names,
//    gathered from the cache ("Sparse prefill for GLM", section "Sparse
//    attention": joined latent+rope rows, all heads share the gathered block,
//    absorbed attention whose value is the latent part of the row).
//
// Work decomposition (gfx950): one workgroup per query; its waves each own 16
// heads, so the 64 heads of a query share every gathered row, which is read
// from HBM once into LDS and reused by all waves. Per tile of 32 keys:
//   S^T[32 keys x 16 heads] = K_tile . Q^T     (16x16x32 bf16 MFMA, K from LDS,
//                                              Q fragments held in registers)
//   online softmax per head (a head is one MFMA column, so its running max and
//   sum live in the lane that owns the column, reduced across the 4 lane groups)
//   O^T[512 x 16 heads] += V_tile^T . P^T      (P^T is the softmax output in the
//                                              exact register layout the MFMA B
//                                              operand wants; V^T comes from LDS
//                                              by transpose reads)
// Tiles are double-buffered: the next tile's rows are fetched into registers
// while the current one is multiplied.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {
constexpr int D = 576;                  // joined row: 512 latent + 64 rope
constexpr int DV = 512;                 // value = latent part of the row
constexpr int T = 32;                   // keys per tile
constexpr int ROWB = D * 2 + 16;        // padded LDS row stride in bytes
constexpr int CH = D * 2 / 16;          // 16-byte chunks per row (72)
constexpr int KC = D / 32;              // MFMA k-steps over the row (18)
constexpr int NDB = DV / 16;            // 16-wide value blocks (32)
constexpr int STAGE = T * ROWB;
}  // namespace

template <bool SPARSE, int NW>
__global__ __launch_bounds__(64 * NW) void absorbed_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, int L, int N, int H, int topk, int q0, int causal, float scale_log2) {
  constexpr int NT = 64 * NW;
  constexpr int PER = (T * CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][STAGE];
  __shared__ int svalid[2][T];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.y;
  const int i = q0 + blockIdx.x;
  // a wave whose 16 heads lie beyond H (H not a multiple of 16*NW) computes on a
  // clamped copy and stores nothing; it still helps fetch the shared rows
  const bool wave_active = (blockIdx.z * NW + wave) * 16 < H;
  const int head = wave_active ? (blockIdx.z * NW + wave) * 16 + c16 : c16;
  const int p = N - L + i;
  const int count = SPARSE ? topk : (causal ? p + 1 : N);
  const uint16_t* kvb = kv + (size_t)b * N * D;
  const int32_t* irow = SPARSE ? idx + ((size_t)b * L + i) * topk : nullptr;

  bf16x8 qf[KC];
  {
    const uint16_t* qrow = q + (((size_t)b * L + i) * H + head) * D + 8 * g;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const bf16x8*)(qrow + 32 * kc);
  }
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  auto key_of = [&](int t, int r) -> int {
    const int slot = t * T + r;
    if (slot >= count) return -1;
    if (SPARSE) {
      const int x = irow[slot];
      return (x >= 0 && x < N) ? x : -1;
    }
    return slot;
  };
  u32x4 stg[PER];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      if (c < T * CH) {
        const int r = c / CH, col = c - r * CH;
        const int key = key_of(t, r);
        stg[u] = key >= 0 ? *(const u32x4*)(kvb + (size_t)key * D + col * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int t, int s) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      if (c < T * CH) {
        const int r = c / CH, col = c - r * CH;
        *(u32x4*)(smem[s] + r * ROWB + col * 16) = stg[u];
      }
    }
    if (tid < T) svalid[s][tid] = key_of(t, tid) >= 0;
  };

  const int ntiles = (count + T - 1) / T;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int s = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const unsigned char* rowp = smem[s] + (16 * kb + c16) * ROWB + 16 * g;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) sacc[kb] = mfma16x16x32(*(const bf16x8*)(rowp + 64 * kc), qf[kc], sacc[kb]);
    }
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool v = svalid[s][16 * kb + 4 * g + j] != 0;
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
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    const bf16x8 pk = pack_bf16x8(pv);
    // V^T operand: lane (g, c16) points at row 4g + c16/4 (and 16 + that), columns 4*(c16%4)
    const unsigned char* vb = smem[s] + (4 * g + (c16 >> 2)) * ROWB + 8 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const short4v lo = lds_read_tr16(vb + 32 * db);
      const short4v hi = lds_read_tr16(vb + 16 * ROWB + 32 * db);
      o[db] = mfma16x16x32(join_bf16x8(lo, hi), pk, o[db]);
    }
    if (t + 1 < ntiles) store_tile(t + 1, s ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = out + (((size_t)b * L + i) * H + head) * DV + 4 * g;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    uint2 w;
    w.x = (uint32_t)f2bf_bits(o[db][0] * inv) | ((uint32_t)f2bf_bits(o[db][1] * inv) << 16);
    w.y = (uint32_t)f2bf_bits(o[db][2] * inv) | ((uint32_t)f2bf_bits(o[db][3] * inv) << 16);
    *(uint2*)(orow + 16 * db) = w;
  }
}

// Launch over queries [q0, q0 + nq) of a chunk of L queries. H must be a multiple of 16;
// a workgroup covers 64 heads (grid z walks head groups).
hipError_t launch_absorbed_attn(bool sparse, const uint16_t* q, const uint16_t* kv, const int32_t* idx, uint16_t* out,
                                int B, int L, int N, int H, int topk, int q0, int nq, int causal, float scale,
                                hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nq, B, (H + 63) / 64), block(256);
  KernelTrace kt(sparse ? "sparse_attn" : "absorbed_dense_attn", stream);
  if (sparse)
    hipLaunchKernelGGL((absorbed_attn_kernel<true, 4>), grid, block, 0, stream, q, kv, idx, out, L, N, H, topk, q0, causal, scale_log2);
  else
    hipLaunchKernelGGL((absorbed_attn_kernel<false, 4>), grid, block, 0, stream, q, kv, idx, out, L, N, H, topk, q0, causal, scale_log2);
  return hipGetLastError();
}

}  // namespace dsa

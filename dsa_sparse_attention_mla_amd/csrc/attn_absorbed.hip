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
// Work decomposition (gfx950): one workgroup per query and 64-head group, 8
// waves. Wave w owns the 16 heads of head group w%4 and one half h = w/4 of the
// row: it contracts dims [288h, 288h+288) of the 576-wide score and accumulates
// value dims [256h, 256h+256). All 64 heads share every gathered row, which is
// read from HBM once into LDS. Per tile of 32 keys:
//   partial S^T[32 keys x 16 heads] = K_tile[:, half] . Q^T[half]
//                        (16x16x32 bf16 MFMA, K from LDS, Q fragments in registers)
//   the two halves swap partials through LDS; both form S = part0 + part1 in the
//   same order, so both run the identical online softmax per head (a head is one
//   MFMA column: its running max and sum live in the lane owning the column,
//   reduced across the 4 lane groups)
//   O^T[256 x 16 heads] += V_tile^T[half] . P^T
//                        (P^T is the softmax output in the exact register layout
//                        the MFMA B operand wants; V^T comes from LDS by transpose
//                        reads)
// Splitting the row between two waves halves the per-wave registers (Q 36, O 64
// VGPRs), which lets two waves share a SIMD and keep LDS reads in flight.
// Row fetch: a ring of 3 LDS stages filled by direct global->LDS 16-byte loads
// (no register staging), issued 2 tiles ahead of use; the index list of a
// segment of up to 2048 keys is staged in LDS first, so a row address never
// waits on an index load.
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
constexpr int BLK = 64;                 // chunks per direct-to-LDS wave instruction
constexpr int NBLK = (T * ROWCH + BLK - 1) / BLK;   // 37 instructions per tile
constexpr int STAGE = NBLK * BLK * 16;  // 37888 bytes per ring stage
constexpr int NSTAGE = 3;               // ring depth
constexpr int AHEAD = NSTAGE - 1;       // tiles in flight beyond the current one
constexpr int SEG = 2048;               // index entries staged per segment
constexpr int KCH = D / 32 / 2;         // MFMA k-steps per half row (9)
constexpr int NDBH = DV / 16 / 2;       // 16-wide value blocks per half (16)
constexpr int NW = 8;                   // waves per workgroup: 4 head groups x 2 row halves
constexpr int XCH_BYTES = NW * 64 * 32; // partial-score exchange: 8 floats per lane
constexpr size_t LDS_BYTES = (size_t)NSTAGE * STAGE + SEG * 4 + NSTAGE * T * 4 + XCH_BYTES;
}  // namespace

// Wait until at most n of this wave's vector-memory operations are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

template <bool SPARSE>
__global__ __launch_bounds__(64 * NW) void absorbed_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, int L, int N, int H, int topk, int q0, int causal, float scale_log2) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  unsigned char* ring = dyn;
  int* sidx = (int*)(dyn + (size_t)NSTAGE * STAGE);
  int* sflag = sidx + SEG;                                  // [NSTAGE][T]
  f32x4* xch = (f32x4*)(sflag + NSTAGE * T);                // [NW][2][64] partial scores

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.y;
  const int i = q0 + blockIdx.x;
  // a wave whose 16 heads lie beyond H computes on a clamped copy and stores nothing
  const int hg = wave & 3, half = wave >> 2;
  const bool wave_active = (blockIdx.z * 4 + hg) * 16 < H;
  const int head = wave_active ? (blockIdx.z * 4 + hg) * 16 + c16 : c16;
  const int p = N - L + i;
  const int count = SPARSE ? topk : (causal ? p + 1 : N);
  const uint16_t* kvb = kv + (size_t)b * N * D;
  const int32_t* irow = SPARSE ? idx + ((size_t)b * L + i) * topk : nullptr;
  const int nblk_w = wave < NBLK % NW ? NBLK / NW + 1 : NBLK / NW;   // 5 or 4 instructions per tile

  bf16x8 qf[KCH];
  {
    const uint16_t* qrow = q + (((size_t)b * L + i) * H + head) * D + 288 * half + 8 * g;
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) qf[kc] = *(const bf16x8*)(qrow + 32 * kc);
  }
  f32x4 o[NDBH];
#pragma unroll
  for (int db = 0; db < NDBH; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // Issue the direct-to-LDS loads of tile t (keys seg_base + 32t ...) into ring stage s.
  auto issue_tile = [&](int t, int s, int seg_base, int seg_cnt) {
    unsigned char* st = ring + (size_t)s * STAGE;
    for (int u = 0; u < nblk_w; ++u) {
      const int blk = wave + NW * u;
      const int pch = blk * BLK + lane;             // chunk slot within the stage
      const int r = pch / ROWCH, cpos = pch - r * ROWCH;
      int key = -1;
      if (r < T) {
        const int slot = t * T + r;
        if (slot < seg_cnt) key = SPARSE ? sidx[slot] : seg_base + slot;
        if (cpos == 0) sflag[s * T + r] = key >= 0;
      }
      const int c = (r < T && cpos < CH) ? cpos : 0;   // padding slots fetch a harmless chunk
      const uint16_t* src = kvb + (size_t)(key >= 0 ? key : 0) * D + c * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (DSA_LDS void*)(st + blk * BLK * 16), 16, 0, 0);
    }
  };

  const int nseg = count > 0 ? (SPARSE ? (count + SEG - 1) / SEG : 1) : 0;
  for (int seg = 0; seg < nseg; ++seg) {
    const int seg_base = SPARSE ? seg * SEG : 0;
    const int seg_cnt = SPARSE ? min(SEG, count - seg_base) : count;
    if (SPARSE) {
      lds_barrier();                               // the previous segment's indices are no longer read
      for (int e = tid; e < seg_cnt; e += 64 * NW) {
        const int x = irow[seg_base + e];
        sidx[e] = (x >= 0 && x < N) ? x : -1;
      }
      lds_barrier();
    }
    const int ntiles = (seg_cnt + T - 1) / T;
    for (int t = 0; t < AHEAD && t < ntiles; ++t) issue_tile(t, t % NSTAGE, seg_base, seg_cnt);

    for (int t = 0; t < ntiles; ++t) {
      const int s = t % NSTAGE;
      const int after = min(t + AHEAD - 1, ntiles - 1) - t;   // tiles issued after tile t
      wait_vm(after * nblk_w);
      lds_barrier();                               // tile t is in LDS; stage of tile t-1 is free
      if (t + AHEAD < ntiles) issue_tile(t + AHEAD, (t + AHEAD) % NSTAGE, seg_base, seg_cnt);

      const unsigned char* st = ring + (size_t)s * STAGE;
      f32x4 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* rowp = st + (16 * kb + c16) * ROWB + 576 * half + 16 * g;
#pragma unroll
        for (int kc = 0; kc < KCH; ++kc) sacc[kb] = mfma16x16x32(*(const bf16x8*)(rowp + 64 * kc), qf[kc], sacc[kb]);
      }
      // swap partial scores with the other half of this head group; both sum in the same order
      xch[(wave * 2 + 0) * 64 + lane] = sacc[0];
      xch[(wave * 2 + 1) * 64 + lane] = sacc[1];
      lds_barrier();
      {
        const int pw = wave ^ 4;
        const f32x4 o0 = xch[(pw * 2 + 0) * 64 + lane], o1 = xch[(pw * 2 + 1) * 64 + lane];
        sacc[0] = half == 0 ? sacc[0] + o0 : o0 + sacc[0];
        sacc[1] = half == 0 ? sacc[1] + o1 : o1 + sacc[1];
      }
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool v = sflag[s * T + 16 * kb + 4 * g + j] != 0;
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
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDBH; ++db) o[db] *= alpha;
      }
      const bf16x8 pk = pack_bf16x8(pv);
      // V^T operand: lane (g, c16) points at row 4g + c16/4 (and 16 + that), columns 4*(c16%4)
      const unsigned char* vb = st + (4 * g + (c16 >> 2)) * ROWB + 512 * half + 8 * (c16 & 3);
#pragma unroll
      for (int db = 0; db < NDBH; ++db) {
        const short4v lo = lds_read_tr16(vb + 32 * db);
        const short4v hi = lds_read_tr16(vb + 16 * ROWB + 32 * db);
        o[db] = mfma16x16x32(join_bf16x8(lo, hi), pk, o[db]);
      }
    }
  }

  if (!wave_active) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = out + (((size_t)b * L + i) * H + head) * DV + 256 * half + 4 * g;
#pragma unroll
  for (int db = 0; db < NDBH; ++db) {
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
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)absorbed_attn_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)absorbed_attn_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nq, B, (H + 63) / 64), block(64 * NW);
  KernelTrace kt(sparse ? "sparse_attn" : "absorbed_dense_attn", stream);
  if (sparse)
    hipLaunchKernelGGL((absorbed_attn_kernel<true>), grid, block, LDS_BYTES, stream, q, kv, idx, out, L, N, H, topk,
                       q0, causal, scale_log2);
  else
    hipLaunchKernelGGL((absorbed_attn_kernel<false>), grid, block, LDS_BYTES, stream, q, kv, idx, out, L, N, H, topk,
                       q0, causal, scale_log2);
  return hipGetLastError();
}

}  // namespace dsa

// Absorbed (latent-space) MLA attention over joined 576-wide latent+rope rows.
//
// One kernel serves three calls:
//  * dense absorbed prefill (keys 0..p_i of a contiguous cache, bottom-right
//    causal),
//  * sparse prefill: each query attends only to the rows its index list names,
//    gathered from the cache ("Sparse prefill for GLM", section "Sparse
//    attention": joined latent+rope rows, all heads share the gathered block,
//    absorbed attention whose value is the latent part of the row), and
//  * masked dense prefill, the path the sparse one replaces (same page, section
//    "The dense mask"): every visible key is visited and only the keys the
//    query's top-k selection marks in a bitmap get weight.
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
// Row fetch: each tile's rows are loaded into registers PF tiles ahead of use
// (five 16-byte loads per thread at most) and written to one of two LDS stages
// just before they are needed; the tile loop is unrolled PF times so every
// register slot is static and the compiler waits only for the loads it must.
// The index list of a segment of up to 4096 keys is staged in LDS first, so a
// row address never waits on an index load.
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
constexpr int STAGE = T * ROWB;         // 37376 bytes per LDS stage (two stages)
constexpr int PF = 2;                   // tiles in flight in registers
constexpr int CPT = (T * CH + 511) / 512;   // 16-byte chunks per thread per tile (5)
constexpr int SEG = 4096;               // index entries staged per segment
constexpr int KCH = D / 32 / 2;         // MFMA k-steps per half row (9)
constexpr int NDBH = DV / 16 / 2;       // 16-wide value blocks per half (16)
constexpr int NW = 8;                   // waves per workgroup: 4 head groups x 2 row halves
constexpr float SLACK = 8.f;            // log2 of the largest unnormalised softmax weight
constexpr int XCH_BYTES = NW * 64 * 32; // partial-score exchange: 8 floats per lane
constexpr size_t LDS_BYTES = 2 * (size_t)STAGE + SEG * 4 + 2 * T * 4 + XCH_BYTES;
}  // namespace

// MODE: 0 dense (every visible key), 1 sparse (gathered index lists), 2 masked
// dense (every visible key, weighted only where the query's selection bitmap has
// its bit set), 3 paged decode split (one query per sequence; workgroup x gathers
// keys [x*spl, x*spl + spl) of the sequence's row list and writes its unnormalised
// partial output with the running max and sum, merged afterwards).
template <int MODE>
__global__ __launch_bounds__(64 * NW) void absorbed_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ mask, uint16_t* __restrict__ out, int L, int N, int H, int topk, int q0, int causal,
    float scale_log2, const int32_t* __restrict__ seqlens, float* __restrict__ part, int spl) {
  constexpr bool SPARSE = MODE == 1 || MODE == 3;   // rows come from an index list
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  unsigned char* ring = dyn;                                // [2][STAGE]
  int* sidx = (int*)(dyn + 2 * (size_t)STAGE);              // [SEG]
  int* sflag = sidx + SEG;                                  // [2][T]
  f32x4* xch = (f32x4*)(sflag + 2 * T);                     // [NW][2][64] partial scores

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.y;
  const int i = MODE == 3 ? 0 : q0 + blockIdx.x;
  const int hg = wave & 3, half = wave >> 2;
  const bool wave_active = (blockIdx.z * 4 + hg) * 16 < H;
  const int head = wave_active ? (blockIdx.z * 4 + hg) * 16 + c16 : c16;
  const int p = N - L + i;
  int count = MODE == 1 ? topk : (causal ? p + 1 : N);
  // (topk is the row-list length here; a sequence length past it is clamped to it)
  if constexpr (MODE == 3) count = max(0, min(spl, min(seqlens[b], topk) - (int)blockIdx.x * spl));
  // paged decode: rows are physical rows of the page pool (N of them), shared by all sequences
  const uint16_t* kvb = kv + (MODE == 3 ? (size_t)0 : (size_t)b * N * D);
  const int32_t* irow = MODE == 1   ? idx + ((size_t)b * L + i) * topk
                        : MODE == 3 ? idx + (size_t)b * topk + (size_t)blockIdx.x * spl
                                    : nullptr;
  const uint32_t* mrow = MODE == 2 ? mask + ((size_t)b * L + i) * ((N + 31) / 32) : nullptr;

  bf16x8 qf[KCH];
  {
    const uint16_t* qrow = q + (((size_t)b * L + i) * H + head) * D + 288 * half + 8 * g;
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) qf[kc] = *(const bf16x8*)(qrow + 32 * kc);
    // Consume the fragments here, so their loads are known complete before the tile loop;
    // otherwise the loop's merged wait state would drain the row prefetch every tile.
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) asm volatile("" ::"v"(qf[kc]));
  }
  f32x4 o[NDBH];
#pragma unroll
  for (int db = 0; db < NDBH; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // chunk u of this thread in a tile: c = tid + 512u (c < 32*72): row c/72, 16-byte column c%72
  auto key_of = [&](int t, int r, int seg_base, int seg_cnt) -> int {
    const int slot = t * T + r;
    if (slot >= seg_cnt) return -1;
    return SPARSE ? sidx[slot] : seg_base + slot;
  };
  // Every thread issues CPT loads for every fetch, also past the tile's chunks and past
  // the last tile (those read row 0 and are never staged), so the number of outstanding
  // loads is the same on every path and the compiler's waits stay exact.
  auto fetch = [&](int t, u32x4 (&dst)[CPT], int seg_base, int seg_cnt) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = min(tid + 512 * u, T * CH - 1);
      const int r = c / CH, col = c - r * CH;
      const int key = key_of(t, r, seg_base, seg_cnt);
      dst[u] = *(const u32x4*)(kvb + (size_t)(key >= 0 ? key : 0) * D + col * 8);   // invalid: row 0, masked
    }
  };
  auto stage_in = [&](int t, int st_i, const u32x4 (&src)[CPT], int seg_base, int seg_cnt) {
    unsigned char* st = ring + (size_t)st_i * STAGE;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 512 * u;
      if (c < T * CH) {
        const int r = c / CH, col = c - r * CH;
        *(u32x4*)(st + r * ROWB + col * 16) = src[u];
      }
    }
    if (tid < T) {
      bool v = key_of(t, tid, seg_base, seg_cnt) >= 0;
      if constexpr (MODE == 2) v = v && ((mrow[(seg_base + t * T) / 32] >> tid) & 1u);
      sflag[st_i * T + tid] = v;
    }
  };
  u32x4 pf[PF][CPT];

  // One tile. Barrier 1 publishes tile t; the partial-score exchange needs barrier 2.
  // After the value product (stage t%2 and the exchange buffer fully read by this
  // wave; every wave has passed barrier 2, so the other stage is free) tile t+1
  // moves from its register slot into the other stage and the slot refetches t+1+PF.
  auto body = [&](int t, u32x4 (&slot)[CPT], int ntiles, int seg_base, int seg_cnt) {
    lds_barrier();
    const int s = t & 1;
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
    // The reference max moves only when a score exceeds it by more than 2^SLACK (or
    // on the first valid key): softmax does not depend on the reference, and weights
    // up to 2^SLACK lose nothing in bf16 / fp32, so the output rescale is rare.
    const bool bump = tmax - m > SLACK;
    const float mnew = bump ? tmax : m;
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(x[e] - mref);
    // The normaliser sums the bf16-rounded weights the value product uses, so the
    // output is an exact convex combination of those weights (a dominant key gives
    // back its value row, whatever the rounding of its weight).
    const bf16x8 pk = pack_bf16x8(pv);
    const float psum = group4_sum(sum_bf16x8(pk));
    if (__ballot(bump)) {
      const float alpha = bump ? exp2_fast(m - mref) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDBH; ++db) o[db] *= alpha;
    }
    lsum += psum;
    m = mnew;
    // V^T operand: lane (g, c16) points at row 4g + c16/4 (and 16 + that), columns 4*(c16%4)
    const unsigned char* vb = st + (4 * g + (c16 >> 2)) * ROWB + 512 * half + 8 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < NDBH; ++db) {
      const short4v lo = lds_read_tr16(vb + 32 * db);
      const short4v hi = lds_read_tr16(vb + 16 * ROWB + 32 * db);
      o[db] = mfma16x16x32(join_bf16x8(lo, hi), pk, o[db]);
    }
    if (t + 1 < ntiles) stage_in(t + 1, (t + 1) & 1, slot, seg_base, seg_cnt);
    fetch(t + 1 + PF, slot, seg_base, seg_cnt);
  };

  const int nseg = count > 0 ? (SPARSE ? (count + SEG - 1) / SEG : 1) : 0;
  for (int seg = 0; seg < nseg; ++seg) {
    const int seg_base = SPARSE ? seg * SEG : 0;
    const int seg_cnt = SPARSE ? min(SEG, count - seg_base) : count;
    if (SPARSE) {
      lds_barrier();                               // the previous segment's indices are no longer read
      // all of this thread's index loads in flight before any is used
      constexpr int PER = SEG / (64 * NW);
      int xs[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 64 * NW * u;
        xs[u] = e < seg_cnt ? irow[seg_base + e] : -1;
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 64 * NW * u;
        if (e < seg_cnt) sidx[e] = (xs[u] >= 0 && xs[u] < N) ? xs[u] : -1;
      }
      lds_barrier();
    }
    const int ntiles = (seg_cnt + T - 1) / T;
#pragma unroll
    for (int t = 0; t < PF; ++t) fetch(t, pf[t], seg_base, seg_cnt);
    if (ntiles > 0) stage_in(0, 0, pf[0], seg_base, seg_cnt);
    fetch(PF, pf[0], seg_base, seg_cnt);
    // tile t+1 sits in register slot (t+1) % PF
    static_assert(PF == 2, "the unrolled tile loop below assumes two register slots");
    for (int t0 = 0; t0 < ntiles; t0 += PF) {
      body(t0, pf[1], ntiles, seg_base, seg_cnt);
      if (t0 + 1 < ntiles) body(t0 + 1, pf[0], ntiles, seg_base, seg_cnt);
    }
  }

  if (!wave_active) return;
  if constexpr (MODE == 3) {
    // partial record of (sequence b, split x, head): 512 unnormalised output values,
    // then the running max (log2 units) and sum
    float* rec = part + (((size_t)b * gridDim.x + blockIdx.x) * H + head) * (DV + 2);
#pragma unroll
    for (int db = 0; db < NDBH; ++db) *(f32x4*)(rec + 256 * half + 16 * db + 4 * g) = o[db];
    if (half == 0 && g == 0) {
      rec[DV] = m;
      rec[DV + 1] = lsum;
    }
    return;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = out + (((size_t)b * L + i) * H + head) * DV + 256 * half + 4 * g;
#pragma unroll
  for (int db = 0; db < NDBH; ++db) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *(bf16x4*)(orow + 16 * db) = __builtin_convertvector(o[db] * inv, bf16x4);
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

// Row list of each sequence of a paged cache: entry n < seq_len is the physical row
// page_table[b][n / page_size] * page_size + n % page_size (rows addressed one at a
// time, so a tile never has to sit inside one page); -1 past the sequence, for a page
// id outside the pool, or a position past the table.
__global__ __launch_bounds__(256) void paged_rows_kernel(const int32_t* __restrict__ page_table,
                                                         const int32_t* __restrict__ seqlens, int max_pages,
                                                         int page_size, int num_pages, int32_t* __restrict__ rows) {
  const int b = blockIdx.y;
  const int maxlen = max_pages * page_size;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= maxlen) return;
  const int len = seqlens[b];
  int r = -1;
  if (n < len) {
    const int pg = page_table[(size_t)b * max_pages + n / page_size];
    if (pg >= 0 && pg < num_pages) r = pg * page_size + n % page_size;
  }
  rows[(size_t)b * maxlen + n] = r;
}

// Merge of the split partials of one (sequence, head): out = sum_x 2^(m_x - M) O_x /
// sum_x 2^(m_x - M) l_x with M the largest split max; splits without a visible key
// (m = -inf) contribute nothing; a sequence with none gets zeros.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part, int nsplit, int H,
                                                             uint16_t* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* base = part + ((size_t)b * nsplit * H + h) * (DV + 2);
  const size_t stride = (size_t)H * (DV + 2);
  float M = -INFINITY;
  for (int x = 0; x < nsplit; ++x) M = fmaxf(M, base[x * stride + DV]);
  float acc0 = 0.f, acc1 = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int x = 0; x < nsplit; ++x) {
      const float* rec = base + x * stride;
      const float mx = rec[DV];
      const float wgt = mx == -INFINITY ? 0.f : exp2_fast(mx - M);
      den += wgt * rec[DV + 1];
      acc0 += wgt * rec[2 * tid];
      acc1 += wgt * rec[2 * tid + 1];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {acc0 * inv, acc1 * inv};
  *(bf16x2*)(out + ((size_t)b * H + h) * DV + 2 * tid) = __builtin_convertvector(v, bf16x2);
}

hipError_t launch_paged_decode(const uint16_t* q, const uint16_t* kv_pages, const int32_t* page_table,
                               const int32_t* seqlens, int B, int H, int num_pages, int page_size, int max_pages,
                               int spl, int nsplit, int32_t* rows, float* part, uint16_t* out, float scale,
                               hipStream_t stream) {
  const int maxlen = max_pages * page_size;
  {
    KernelTrace kt("paged_rows", stream);
    hipLaunchKernelGGL(paged_rows_kernel, dim3((maxlen + 255) / 256, B), dim3(256), 0, stream, page_table, seqlens,
                       max_pages, page_size, num_pages, rows);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_absorbed_attn(3, q, kv_pages, rows, nullptr, nullptr, B, 1, num_pages * page_size, H, maxlen, 0, nsplit,
                           0, scale, stream, seqlens, part, spl);
  if (e != hipSuccess) return e;
  KernelTrace kt("decode_combine", stream);
  hipLaunchKernelGGL(decode_combine_kernel, dim3(H, B), dim3(DV / 2), 0, stream, part, nsplit, H, out);
  return hipGetLastError();
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
                                float* part, int spl) {
  static bool attr_set = false;
  if (!attr_set) {
    const void* fns[4] = {(const void*)absorbed_attn_kernel<0>, (const void*)absorbed_attn_kernel<1>,
                          (const void*)absorbed_attn_kernel<2>, (const void*)absorbed_attn_kernel<3>};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nq, B, (H + 63) / 64), block(64 * NW);
  static const char* names[4] = {"absorbed_dense_attn", "sparse_attn", "masked_dense_attn", "paged_decode_attn"};
  KernelTrace kt(names[mode], stream);
#define DSA_LAUNCH_ABS(M)                                                                                    \
  hipLaunchKernelGGL((absorbed_attn_kernel<M>), grid, block, LDS_BYTES, stream, q, kv, idx, mask, out, L, N, H, \
                     topk, q0, causal, scale_log2, seqlens, part, spl)
  switch (mode) {
    case 1: DSA_LAUNCH_ABS(1); break;
    case 2: DSA_LAUNCH_ABS(2); break;
    case 3: DSA_LAUNCH_ABS(3); break;
    default: DSA_LAUNCH_ABS(0); break;
  }
#undef DSA_LAUNCH_ABS
  return hipGetLastError();
}

}  // namespace dsa

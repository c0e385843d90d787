// C ABI of libdsa_mla.so: host-side validation, device check and launch.
// The contract of every entry point is documented in include/dsa_mla.h.
#include "../../include/dsa_mla.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_arch_mu;
int g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The current device must be gfx950; the answer is cached per device.
int check_arch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return DSA_MLA_ARCH;
  }
  if (dev < kMaxDevices) {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_state[dev] == 1) return DSA_MLA_OK;
    if (g_arch_state[dev] == 2) return DSA_MLA_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return DSA_MLA_ARCH;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                  (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
  if (dev < kMaxDevices) {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    g_arch_state[dev] = ok ? 1 : 2;
  }
  return ok ? DSA_MLA_OK : DSA_MLA_ARCH;
}

// Shared workspace protocol. Returns -1 to continue with the launch, or a status to return.
int workspace_step(size_t need, void* ws, size_t* ws_bytes) {
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return DSA_MLA_OK;
  }
  if (need == 0) return -1;
  if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < need) return DSA_MLA_WORKSPACE;
  if (!aligned16(ws)) return DSA_MLA_INVALID_ARG;
  return -1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DSA_MLA_OK : DSA_MLA_HIP; }

// Argument checks shared by both decode entry points.
int decode_check(int B, int H, int num_pages, int page_size, int max_pages, const void* q, const void* kv_pages,
                 const int32_t* page_table, const int32_t* seq_lens, float scale, const void* out) {
  if (B < 0 || H < 1 || num_pages < 1 || page_size < 1 || max_pages < 1) return DSA_MLA_INVALID_ARG;
  if ((long long)num_pages * page_size > INT32_MAX || (long long)max_pages * page_size > INT32_MAX)
    return DSA_MLA_INVALID_ARG;
  if (!std::isfinite(scale)) return DSA_MLA_INVALID_ARG;
  if (q == nullptr || kv_pages == nullptr || page_table == nullptr || seq_lens == nullptr || out == nullptr)
    return DSA_MLA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_pages) || !aligned4(page_table) || !aligned4(seq_lens) || !aligned16(out))
    return DSA_MLA_INVALID_ARG;
  if (H % 16 != 0) return DSA_MLA_UNSUPPORTED;
  return DSA_MLA_OK;
}

// Split of the decode keys: a multiple of 32 keys, 256 .. 4096, aiming at one workgroup
// per compute unit (256; one round of workgroups, since one fills a CU's LDS).
struct DecodePlan {
  int spl, nsplit;
  size_t part_bytes;   // split partials: B * nsplit * H records of 512 outputs + max + sum
};
DecodePlan decode_plan(int B, int H, int max_pages, int page_size) {
  const int maxlen = max_pages * page_size;
  long long spl = ((long long)B * maxlen + 255) / 256;
  spl = (spl + 31) / 32 * 32;
  spl = spl < 256 ? 256 : (spl > 4096 ? 4096 : spl);
  DecodePlan p;
  p.spl = (int)spl;
  p.nsplit = (int)((maxlen + spl - 1) / spl);
  p.part_bytes = (size_t)B * p.nsplit * H * (512 + 2) * 4;
  return p;
}

}  // namespace

extern "C" {

int dsa_mla_abi_version(void) { return 1; }

const char* dsa_mla_status_string(int s) {
  switch (s) {
    case DSA_MLA_OK: return "ok";
    case DSA_MLA_INVALID_ARG: return "invalid argument";
    case DSA_MLA_UNSUPPORTED: return "unsupported configuration";
    case DSA_MLA_ARCH: return "device is not gfx950";
    case DSA_MLA_WORKSPACE: return "workspace missing or too small";
    case DSA_MLA_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int mla_prefill_dense(int mode, int dtype, int B, int L, int N, int H, const void* q, const void* q_rope,
                      const void* k, const void* k_rope, const void* v, void* out, float scale, int causal, void* ws,
                      size_t* ws_bytes, void* stream) {
  if (mode != DSA_MLA_MODE_NONABSORBED && mode != DSA_MLA_MODE_ABSORBED) return DSA_MLA_INVALID_ARG;
  if (dtype != DSA_MLA_F32 && dtype != DSA_MLA_BF16) return DSA_MLA_INVALID_ARG;
  if (B < 0 || L < 0 || N < 0 || H < 1) return DSA_MLA_INVALID_ARG;
  if (causal != 0 && causal != 1) return DSA_MLA_INVALID_ARG;
  if (causal && L > N) return DSA_MLA_INVALID_ARG;
  if (!std::isfinite(scale)) return DSA_MLA_INVALID_ARG;
  if (q == nullptr || k == nullptr || out == nullptr) return DSA_MLA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(out)) return DSA_MLA_INVALID_ARG;
  if (mode == DSA_MLA_MODE_NONABSORBED) {
    if (q_rope == nullptr || k_rope == nullptr || v == nullptr) return DSA_MLA_INVALID_ARG;
    if (!aligned16(q_rope) || !aligned16(k_rope) || !aligned16(v)) return DSA_MLA_INVALID_ARG;
    if (H > 65535) return DSA_MLA_UNSUPPORTED;    // heads index a grid dimension; tile offsets are 32-bit
  } else {
    if (q_rope != nullptr || k_rope != nullptr || v != nullptr) return DSA_MLA_INVALID_ARG;
    if (dtype != DSA_MLA_BF16) return DSA_MLA_UNSUPPORTED;
    if (H % 16 != 0) return DSA_MLA_UNSUPPORTED;
    if ((long long)L * H > INT32_MAX) return DSA_MLA_UNSUPPORTED;   // (query, head) rows are 32-bit
  }
  const int wsr = workspace_step(0, ws, ws_bytes);
  if (wsr >= 0) return wsr;
  if (B == 0 || L == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  hipStream_t st = (hipStream_t)stream;
  if (mode == DSA_MLA_MODE_NONABSORBED)
    return hip_status(dsa::launch_nonabsorbed_attn(dtype == DSA_MLA_BF16, q, q_rope, k, k_rope, v, out, B, L, N, H,
                                                   causal, scale, st));
  return hip_status(dsa::launch_absorbed_dense((const uint16_t*)q, (const uint16_t*)k, nullptr, (uint16_t*)out, B, L, N,
                                               H, causal, scale, st));
}

int dsa_indexer_topk(int B, int L, int N, int Hi, int Di, const void* q_idx, const void* k_idx, const float* w,
                     int topk, int block, int32_t* idx_out, float* score_out, void* ws, size_t* ws_bytes,
                     void* stream) {
  if (B < 0 || L < 0 || N < 1 || Hi < 1 || Di < 1 || topk < 1 || block < 1) return DSA_MLA_INVALID_ARG;
  if (L > N) return DSA_MLA_INVALID_ARG;
  if (q_idx == nullptr || k_idx == nullptr || w == nullptr || idx_out == nullptr) return DSA_MLA_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned4(w) || !aligned4(idx_out) ||
      (score_out != nullptr && !aligned4(score_out)))
    return DSA_MLA_INVALID_ARG;
  if (Hi != 32 || Di != 128 || topk > 2560) return DSA_MLA_UNSUPPORTED;
  const dsa::IndexerPlan pl = dsa::indexer_plan(L, N, topk, block);
  const int wsr = workspace_step(pl.ws_bytes, ws, ws_bytes);
  if (wsr >= 0) return wsr;
  if (B == 0 || L == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  // batch entries run one after another on the stream, sharing the workspace
  for (int b = 0; b < B; ++b) {
    const hipError_t e = dsa::launch_indexer(
        pl, (const uint16_t*)q_idx + (size_t)b * L * Hi * Di, (const uint16_t*)k_idx + (size_t)b * N * Di,
        w + (size_t)b * L * Hi, L, N, topk, idx_out + (size_t)b * L * topk,
        score_out ? score_out + (size_t)b * L * topk : nullptr, ws, (hipStream_t)stream);
    if (e != hipSuccess) return DSA_MLA_HIP;
  }
  return DSA_MLA_OK;
}

int mla_prefill_sparse(int B, int L, int N, int H, const void* q, const void* kv, const int32_t* idx, int topk,
                       float scale, int query_block, void* out, void* ws, size_t* ws_bytes, void* stream) {
  if (B < 0 || L < 0 || N < 1 || H < 1 || topk < 1) return DSA_MLA_INVALID_ARG;
  if (query_block < 1 || query_block > 1024) return DSA_MLA_INVALID_ARG;
  if (!std::isfinite(scale)) return DSA_MLA_INVALID_ARG;
  if (q == nullptr || kv == nullptr || idx == nullptr || out == nullptr) return DSA_MLA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv) || !aligned4(idx) || !aligned16(out)) return DSA_MLA_INVALID_ARG;
  if (H % 16 != 0) return DSA_MLA_UNSUPPORTED;
  const int wsr = workspace_step(0, ws, ws_bytes);
  if (wsr >= 0) return wsr;
  if (B == 0 || L == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  for (int q0 = 0; q0 < L; q0 += query_block) {
    const int nq = L - q0 < query_block ? L - q0 : query_block;
    const hipError_t e = dsa::launch_absorbed_attn(1, (const uint16_t*)q, (const uint16_t*)kv, idx, nullptr, (uint16_t*)out,
                                                   B, L, N, H, topk, q0, nq, 0, scale, (hipStream_t)stream);
    if (e != hipSuccess) return DSA_MLA_HIP;
  }
  return DSA_MLA_OK;
}

int mla_prefill_masked(int B, int L, int N, int H, const void* q, const void* kv, const int32_t* idx, int topk,
                       float scale, void* out, void* ws, size_t* ws_bytes, void* stream) {
  if (B < 0 || L < 0 || N < 1 || H < 1 || topk < 1) return DSA_MLA_INVALID_ARG;
  if (L > N) return DSA_MLA_INVALID_ARG;
  if (!std::isfinite(scale)) return DSA_MLA_INVALID_ARG;
  if (q == nullptr || kv == nullptr || idx == nullptr || out == nullptr) return DSA_MLA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv) || !aligned4(idx) || !aligned16(out)) return DSA_MLA_INVALID_ARG;
  if (H % 16 != 0) return DSA_MLA_UNSUPPORTED;
  if ((long long)L * H > INT32_MAX) return DSA_MLA_UNSUPPORTED;     // (query, head) rows are 32-bit
  const size_t words = (size_t)B * L * (size_t)((N + 31) / 32);
  const int wsr = workspace_step(words * 4, ws, ws_bytes);
  if (wsr >= 0) return wsr;
  if (B == 0 || L == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  uint32_t* mask = (uint32_t*)ws;
  hipError_t e = dsa::launch_mask_rows(idx, B, L, N, topk, mask, (hipStream_t)stream);
  if (e != hipSuccess) return DSA_MLA_HIP;
  e = dsa::launch_absorbed_dense((const uint16_t*)q, (const uint16_t*)kv, mask, (uint16_t*)out, B, L, N, H, 1, scale,
                                 (hipStream_t)stream);
  return hip_status(e);
}

int mla_decode_paged(int B, int H, int num_pages, int page_size, int max_pages, const void* q, const void* kv_pages,
                     const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, void* ws,
                     size_t* ws_bytes, void* stream) {
  const int v = decode_check(B, H, num_pages, page_size, max_pages, q, kv_pages, page_table, seq_lens, scale, out);
  if (v != DSA_MLA_OK) return v;
  const DecodePlan dp = decode_plan(B, H, max_pages, page_size);
  const int wsr = workspace_step(dp.part_bytes, ws, ws_bytes);
  if (wsr >= 0) return wsr;
  if (B == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  return hip_status(dsa::launch_paged_decode((const uint16_t*)q, (const uint16_t*)kv_pages, page_table, seq_lens, B,
                                             H, num_pages, page_size, max_pages, dp.spl, dp.nsplit, (float*)ws,
                                             (uint16_t*)out, scale, (hipStream_t)stream));
}

int mla_decode_paged_noalloc(int B, int H, int num_pages, int page_size, int max_pages, const void* q,
                             const void* kv_pages, const int32_t* page_table, const int32_t* seq_lens, float scale,
                             void* out, void* stream) {
  const int v = decode_check(B, H, num_pages, page_size, max_pages, q, kv_pages, page_table, seq_lens, scale, out);
  if (v != DSA_MLA_OK) return v;
  const DecodePlan dp = decode_plan(B, H, max_pages, page_size);
  if (dp.part_bytes > dsa::kDecodeScratchBytes) return DSA_MLA_WORKSPACE;
  if (B == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  void* part = nullptr;
  if (dsa::decode_scratch(&part) != hipSuccess || part == nullptr) {
    (void)hipGetLastError();
    return DSA_MLA_HIP;
  }
  return hip_status(dsa::launch_paged_decode((const uint16_t*)q, (const uint16_t*)kv_pages, page_table, seq_lens, B,
                                             H, num_pages, page_size, max_pages, dp.spl, dp.nsplit, (float*)part,
                                             (uint16_t*)out, scale, (hipStream_t)stream));
}

size_t mla_decode_paged_noalloc_capacity(void) { return dsa::kDecodeScratchBytes; }

int dsa_mla_probe_mfma(int grid, int iters, long long* cycles, long long* wall, float* sink, int* wall_khz,
                       void* stream) {
  if (grid < 1 || grid > 65535 || iters < 1 || cycles == nullptr || wall == nullptr || sink == nullptr)
    return DSA_MLA_INVALID_ARG;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  if (wall_khz != nullptr) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return DSA_MLA_HIP;
    *wall_khz = khz;
  }
  return hip_status(dsa::launch_mfma_burn(grid, iters, cycles, wall, sink, (hipStream_t)stream));
}

int dsa_mla_probe_stream(int mode, const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if ((mode != 0 && mode != 1) || grid < 1 || grid > 65535 || bytes % 64 != 0) return DSA_MLA_INVALID_ARG;
  if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return DSA_MLA_INVALID_ARG;
  if (bytes == 0) return DSA_MLA_OK;
  const int a = check_arch();
  if (a != DSA_MLA_OK) return a;
  return hip_status(dsa::launch_stream(mode, src, dst, bytes, grid, (hipStream_t)stream));
}

}  // extern "C"

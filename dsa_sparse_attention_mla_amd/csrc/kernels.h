// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// RAII scope that brackets one kernel launch with HIP events when tracing is on
// (see dsa_mla_trace_enable); a no-op otherwise.
class KernelTrace {
 public:
  KernelTrace(const char* name, hipStream_t s);
  ~KernelTrace();
  KernelTrace(const KernelTrace&) = delete;
  KernelTrace& operator=(const KernelTrace&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  void* a_;
};

// mode 1: sparse prefill over index lists; mode 3: one split of a paged decode step
hipError_t launch_absorbed_attn(int mode, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                const uint32_t* mask, uint16_t* out, int B, int L, int N, int H, int topk, int q0,
                                int nq, int causal, float scale, hipStream_t stream, const int32_t* seqlens = nullptr,
                                float* part = nullptr, int spl = 0, int psz = 1);
hipError_t launch_absorbed_dense(const uint16_t* q, const uint16_t* kv, const uint32_t* mask, uint16_t* out, int B,
                                 int L, int N, int H, int causal, float scale, hipStream_t stream);
hipError_t launch_paged_decode(const uint16_t* q, const uint16_t* kv_pages, const int32_t* page_table,
                               const int32_t* seqlens, int B, int H, int num_pages, int page_size, int max_pages,
                               int spl, int nsplit, float* part, uint16_t* out, float scale, hipStream_t stream);
// Size of the fixed decode scratch (split partials of the no-allocation decode call).
constexpr size_t kDecodeScratchBytes = (size_t)40 << 20;
// Device address of that scratch on the current device (looked up once per device).
hipError_t decode_scratch(void** ptr);
hipError_t launch_mfma_burn(int grid, int iters, long long* cycles, long long* wall, float* sink,
                            hipStream_t stream);
hipError_t launch_stream(int mode, const void* src, void* dst, size_t bytes, int grid, hipStream_t stream);
hipError_t launch_mask_rows(const int32_t* idx, int B, int L, int N, int topk, uint32_t* mask, hipStream_t stream);

hipError_t launch_nonabsorbed_attn(bool bf16, const void* qn, const void* qr, const void* kn, const void* kr,
                                   const void* v, void* out, int B, int L, int N, int H, int causal, float scale,
                                   hipStream_t stream);

struct IndexerPlan {
  int nsplit = 1, span = 0, cap = 0, fb_blocks = 1, nstage = 3;
  bool small_off = false;   // candidate keys stored as 16-bit offsets within the split
  bool global_lists = false;  // long context: sampled start, candidate lists written straight to memory
  int sample = 0;             // keys the list kernel samples for its start threshold
  size_t off_partial = 0, off_eps = 0, off_cand_n = 0, off_cand_t = 0, off_fb = 0, off_cand_s = 0, off_cand_i = 0, off_scratch = 0;
  size_t ws_bytes = 0, filter_lds = 0, select_lds = 0;
};
IndexerPlan indexer_plan(int L, int N, int topk, int block);
hipError_t launch_indexer(const IndexerPlan& pl, const uint16_t* q, const uint16_t* k, const float* w, int L, int N,
                          int topk, int32_t* idx_out, float* score_out, void* ws, hipStream_t stream);

}  // namespace dsa

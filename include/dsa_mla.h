/*
 * dsa_mla.h -- C ABI of libdsa_mla.so: MLA prefill and DeepSeek-sparse-attention
 * (DSA) prefill on AMD Instinct MI355X (gfx950).
 *
 * Five calls:
 *   mla_prefill_dense   dense causal MLA prefill, non-absorbed or absorbed
 *   dsa_indexer_topk    indexer scores fused with a running top-k selection
 *   mla_prefill_sparse  absorbed attention over each query's gathered top-k rows
 *   mla_prefill_masked  dense absorbed attention under each query's top-k mask
 *                       (the path the sparse call replaces; the gated case)
 *   mla_decode_paged    one decode step (L = 1) of absorbed attention over a
 *                       paged joined cache
 *   mla_decode_paged_noalloc  the same step with the library's fixed scratch
 *                       instead of a workspace (for callers that cannot allocate)
 *
 * Conventions shared by all calls
 * -------------------------------
 * Return value: a dsa_mla_status code; 0 means the work was enqueued.
 * Validation: every argument check runs on the host before anything is
 *   launched; a call that returns an error has launched nothing and left every
 *   output untouched. No call prints, throws or allocates device memory.
 * Process-wide state: the library keeps a per-device record of the device
 *   check, the tracing switch and its pending event records (diagnostics, see
 *   dsa_mla_trace_enable), and, per device, the fixed scratch array of
 *   mla_decode_paged_noalloc with its looked-up device address. All of it is
 *   guarded by locks; nothing else persists between calls.
 * Memory: every tensor argument is a DEVICE pointer of the current device (the
 *   one kernels are launched on), owned by the caller,
 *   contiguous row-major in the layout stated per call, with a 16-byte aligned
 *   base. Inputs are only read; outputs are fully overwritten.
 * bf16: passed as 16-bit storage (the upper half of an IEEE fp32). Arithmetic
 *   accumulates in fp32; outputs have the input dtype.
 * Causality: the L queries of a chunk are the LAST L positions of an
 *   N-position context: query i sits at position N - L + i and sees key n iff
 *   n <= N - L + i. For L = N this is the usual j <= i rule.
 * Workspace: ws == NULL together with a non-NULL ws_bytes is a size query: the
 *   call stores the required byte count in *ws_bytes, returns DSA_MLA_OK and
 *   launches nothing. Otherwise, if the call needs workspace, ws must be a
 *   device buffer of at least the queried size, given in *ws_bytes (256-byte
 *   alignment recommended). A call that needs none may pass ws_bytes == NULL.
 *   The workspace holds no state between calls.
 * Streams: `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *   on it and the call returns without synchronising; a device-side fault
 *   surfaces at the caller's next synchronisation.
 * Device: the current HIP device must be gfx950, otherwise DSA_MLA_ARCH
 *   (dispatch checks the chip before launching, so no device ever receives a
 *   kernel it cannot run; Fornax part 5 "Apple M3 vs M5 kernels", section
 *   "Dispatch has to know the chip").
 * Threads: calls are re-entrant; calls on different streams may overlap.
 */
#ifndef DSA_MLA_H
#define DSA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_mla_status {
  DSA_MLA_OK = 0,
  DSA_MLA_INVALID_ARG = 1,   /* NULL pointer, bad size/enum, misaligned pointer, L > N when causal */
  DSA_MLA_UNSUPPORTED = 2,   /* valid request outside what the kernels implement (dims, dtype, B) */
  DSA_MLA_ARCH = 3,          /* no HIP device, or the current device is not gfx950 */
  DSA_MLA_WORKSPACE = 4,     /* workspace missing or smaller than required */
  DSA_MLA_HIP = 5            /* the HIP runtime reported an error while launching */
} dsa_mla_status;

enum { DSA_MLA_MODE_NONABSORBED = 0, DSA_MLA_MODE_ABSORBED = 1 };
enum { DSA_MLA_F32 = 0, DSA_MLA_BF16 = 1 };

/*
 * mla_prefill_dense -- dense causal (or full) MLA prefill.
 *
 * mode DSA_MLA_MODE_NONABSORBED (Fornax part 5 "Apple M3 vs M5 kernels",
 * section "What the kernel has to compute"): per head h,
 *   score[i,j] = scale * (q[i,h,:] . k[j,h,:]  +  q_rope[i,h,:] . k_rope[j,:])
 *   out[i,h,:] = softmax_j(score[i,:]) . v[:,h,:]
 * with the rope key shared by all heads.
 *   q      [B,L,H,128]   q_rope [B,L,H,64]
 *   k      [B,N,H,128]   k_rope [B,N,64]     v [B,N,H,128]
 *   out    [B,L,H,128]
 *   dtype DSA_MLA_F32 or DSA_MLA_BF16 (all tensors the same dtype); H <= 65535.
 *
 * mode DSA_MLA_MODE_ABSORBED ("Sparse prefill for GLM", section "Sparse
 * attention": attention in the absorbed latent space over one joined
 * latent+rope row per position, shared by all heads):
 *   score[i,j] = scale * q[i,h,:] . kv[j,:]          out[i,h,:] = softmax . kv[:, 0:512]
 *   q  [B,L,H,576] (512 latent then 64 rope)  k = kv [B,N,576]  out [B,L,H,512]
 *   q_rope, k_rope and v must be NULL. dtype must be DSA_MLA_BF16; H a multiple of 16;
 *   L * H < 2^31 (DSA_MLA_UNSUPPORTED otherwise).
 *
 * causal: 1 = bottom-right causal (see above; needs L <= N), 0 = every key.
 * B >= 1 is allowed. B == 0 or L == 0 is a no-op. A query that sees no key
 * (only possible with N == 0, non-causal) gets a zero row. No workspace.
 */
int mla_prefill_dense(int mode, int dtype, int B, int L, int N, int H,
                      const void* q, const void* q_rope, const void* k, const void* k_rope, const void* v,
                      void* out, float scale, int causal, void* ws, size_t* ws_bytes, void* stream);

/*
 * dsa_indexer_topk -- indexer top-k ("Sparse prefill for GLM", section
 * "Blocked top-k": keys are scored a block at a time and folded into a running
 * top-k list; the full batch x heads x L x N score tensor is never built).
 *
 *   s[b,i,n] = sum_h w[b,i,h] * ReLU(q_idx[b,i,h,:] . k_idx[b,n,:])     for n <= N - L + i
 *   q_idx [B,L,Hi,Di] bf16   k_idx [B,N,Di] bf16   w [B,L,Hi] fp32   idx_out [B,L,topk] int32
 *
 * The result is the EXACT top-k set of the canonical score (dot products in
 * fp64 summed over dims in ascending order, head terms added in ascending head
 * order, every operation separately rounded), ties to the lower key index.
 * This holds for any finite inputs: queries whose magnitudes could overflow the
 * fp32 filter scores are resolved by the exact fp64 path. (NaN or infinite inputs
 * have no canonical score; their result is unspecified.)
 * Rows are written in ascending key order; a row with fewer than topk visible
 * keys holds all of them followed by -1. score_out (nullable) [B,L,topk] fp32
 * receives the fp32 MFMA score of each returned key (-inf on padding).
 * `block` (>= 1; the pages use 4096) is the folding granularity of the key
 * sweep and never changes the result.
 * Supported: B >= 1 (batch entries run one after another and share the
 * workspace), Hi == 32, Di == 128, 1 <= topk <= 2560, 0 <= L <= N.
 * Needs workspace (query its size first; it does not depend on B).
 */
int dsa_indexer_topk(int B, int L, int N, int Hi, int Di, const void* q_idx, const void* k_idx, const float* w,
                     int topk, int block, int32_t* idx_out, float* score_out, void* ws, size_t* ws_bytes,
                     void* stream);

/*
 * mla_prefill_sparse -- sparse absorbed MLA prefill ("Sparse prefill for GLM",
 * section "Sparse attention": the joined 576-wide row of every chosen key is
 * gathered, all heads share the gathered block, attention runs in absorbed
 * latent space; chunks longer than the query block are split into blocks).
 *
 *   score[b,i,h,t] = scale * q[b,i,h,:] . kv[b,idx[b,i,t],:]   over t with idx[b,i,t] valid
 *   out[b,i,h,:]   = softmax_t(score) . kv[b,idx[b,i,t], 0:512]
 *   q [B,L,H,576] bf16   kv [B,N,576] bf16   idx [B,L,topk] int32   out [B,L,H,512] bf16
 *
 * Index entries outside [0, N) (-1 in particular) are skipped; a row with no
 * valid entry gets zeros. Indices are not re-masked for causality. A repeated
 * index counts once per occurrence. query_block (1..1024) splits the L queries
 * into launches of at most that many; the output does not depend on it.
 * Supported: B >= 1 (the pages' limit of one sequence, section "Limits and what
 * to do", is lifted here), H a multiple of 16. No workspace.
 */
int mla_prefill_sparse(int B, int L, int N, int H, const void* q, const void* kv, const int32_t* idx, int topk,
                       float scale, int query_block, void* out, void* ws, size_t* ws_bytes, void* stream);

/*
 * mla_prefill_masked -- dense absorbed MLA prefill under each query's top-k
 * selection ("Sparse prefill for GLM", section "The dense mask": before the
 * sparse path, the indexer's choice became a boolean mask with one row per query
 * and one column per key, and attention ran over every key with the unselected
 * ones masked out; section "When it runs": calls the gate turns away still take
 * this path).
 *
 *   score[b,i,h,n] = scale * q[b,i,h,:] . kv[b,n,:]   for n <= N-L+i named in idx[b,i,:]
 *   out[b,i,h,:]   = softmax_n(score) . kv[b,n,0:512]
 *   q [B,L,H,576] bf16   kv [B,N,576] bf16   idx [B,L,topk] int32   out [B,L,H,512] bf16
 *
 * Index entries outside [0, N) are ignored, a repeated index selects its key
 * once, and a selected key past the causal limit stays masked. Every visible
 * key is visited: this is the dense cost the sparse call removes. A row with no
 * selected visible key gets zeros. Supported: B >= 1, 0 <= L <= N, H a multiple
 * of 16, L * H < 2^31. Needs workspace: B*L*ceil(N/32) 32-bit words for the selection bitmaps
 * (query its size with ws == NULL); the bitmaps are rebuilt on every call.
 */
int mla_prefill_masked(int B, int L, int N, int H, const void* q, const void* kv, const int32_t* idx, int topk,
                       float scale, void* out, void* ws, size_t* ws_bytes, void* stream);

/*
 * mla_decode_paged -- one decode step of absorbed MLA over a paged joined cache
 * ("Sparse prefill for GLM", section "When it runs": decode keeps the dense
 * absorbed path, also after a sparse prefill; "Apple M3 vs M5 kernels", section
 * "Paged KV: alignment follows the tile": every row is addressed on its own
 * through the page table, so no tile has to sit inside one page).
 *
 *   row(b, n)   = kv_pages[page_table[b, n / page_size], n % page_size, :]   n < seq_lens[b]
 *   score[b,h,n] = scale * q[b,h,:] . row(b, n)
 *   out[b,h,:]   = softmax_n(score) . row(b, n)[0:512]
 *   q [B,H,576] bf16   kv_pages [num_pages,page_size,576] bf16
 *   page_table [B,max_pages] int32   seq_lens [B] int32   out [B,H,512] bf16
 *
 * The new token's key is already in the cache: the query sees all seq_lens[b]
 * rows. A length past max_pages*page_size is clamped to it; a page id outside
 * [0, num_pages) makes its rows count as absent; a sequence without rows gets
 * zeros. The keys are split across workgroups and the partial results merged
 * (flash-decoding style). Supported: B >= 0, H a multiple of 16. Needs
 * workspace: the split partials, B * nsplit * H * 514 floats (query its size
 * with ws == NULL).
 */
int mla_decode_paged(int B, int H, int num_pages, int page_size, int max_pages, const void* q, const void* kv_pages,
                     const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, void* ws,
                     size_t* ws_bytes, void* stream);

/*
 * mla_decode_paged_noalloc -- mla_decode_paged for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. It takes no workspace: the split partials go to a fixed scratch
 * array of mla_decode_paged_noalloc_capacity() bytes (40 MiB) that the library holds
 * on every device it runs on until the process ends. Same arguments, layouts,
 * kernels and result as mla_decode_paged; a call whose partials,
 * B * nsplit * H * 514 * 4 bytes (nsplit as in mla_decode_paged: about 256 / B
 * splits per sequence, fewer for short caches), would not fit returns
 * DSA_MLA_WORKSPACE and launches nothing. At H = 64 this admits, e.g., 8 sequences
 * of 131072 keys or up to about 1.3M cached keys in all. Every record the combine
 * reads is written by the same call, so nothing needs clearing between calls. All
 * calls on one device share its scratch: calls that overlap in time on one device
 * (different streams, or different threads without ordering) race and must not be
 * issued.
 */
int mla_decode_paged_noalloc(int B, int H, int num_pages, int page_size, int max_pages, const void* q,
                             const void* kv_pages, const int32_t* page_table, const int32_t* seq_lens, float scale,
                             void* out, void* stream);
size_t mla_decode_paged_noalloc_capacity(void);

/*
 * Per-kernel timing (diagnostics). dsa_mla_trace_enable(1) makes every later
 * kernel launch of the library record a HIP event pair on its launch stream;
 * it returns the previous setting. dsa_mla_trace_collect waits for the
 * recorded events, and for each distinct kernel name (at most max_kernels)
 * writes the name (NUL-terminated, 32 bytes per entry) into `names`, the
 * launch count into `counts` and the summed event time in milliseconds into
 * `total_ms`; any of the three may be NULL. It clears the record and returns
 * the number of distinct kernels seen.
 */
int dsa_mla_trace_enable(int on);
int dsa_mla_trace_collect(int max_kernels, char* names, int* counts, double* total_ms);

/*
 * Measurement probes (diagnostics, not part of the attention path): the ceilings
 * the kernels above are measured against on the running GPU, next to the data
 * sheet's peaks.
 *
 * dsa_mla_probe_mfma launches `grid` workgroups of four waves (one per SIMD when
 * grid is a multiple of the compute-unit count); every wave runs `iters` rounds
 * of eight independent 32x32x16 bf16 MFMAs (32768 FLOP each) on register
 * operands. Per wave w of workgroup g, cycles[4g + w] receives the shader-clock
 * cycles of its loop and wall[4g + w] the ticks of the constant-rate wall clock
 * over the same loop; sink[256 g + thread] receives a sum of the results.
 * cycles, wall and sink are device buffers of 4 grid, 4 grid and 256 grid
 * elements, owned by the caller. *wall_khz (host, may be NULL) receives the
 * wall clock's rate in kHz. Total work: grid * 4 * iters * 8 * 32768 FLOP; the
 * ratio cycles / wall gives the shader clock under full matrix load.
 *
 * dsa_mla_probe_stream moves `bytes` (a multiple of 64) through HBM with
 * 16-byte-per-lane loads over a grid of `grid` workgroups of 256 threads:
 * mode 0 copies src to dst (bytes read and bytes written), mode 1 only reads src
 * (non-temporal loads, eight per thread in flight) and writes one 32-bit word per
 * thread (dst: 1024 grid bytes). src and dst are
 * 16-byte-aligned device buffers owned by the caller.
 *
 * Both return DSA_MLA_INVALID_ARG for out-of-range arguments before launching.
 */
int dsa_mla_probe_mfma(int grid, int iters, long long* cycles, long long* wall, float* sink, int* wall_khz,
                       void* stream);
int dsa_mla_probe_stream(int mode, const void* src, void* dst, size_t bytes, int grid, void* stream);

/* Short English name of a status code (static storage). */
const char* dsa_mla_status_string(int status);

/* ABI version of this header (increments on incompatible changes). */
int dsa_mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_MLA_H */

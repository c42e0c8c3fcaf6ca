/*
 * fa.h -- C ABI of the MI355X (gfx950) attention forward library (libfa.so).
 *
 * The operation is the fused attention forward pass
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * computed tile by tile with an online (running max / running sum) softmax, in
 * the two workloads the pages turn on:
 *
 *  - prefill over microbatches with grouped-query heads ("CUDA: fix FA
 *    occupancy, optimize tile kernel", llama.cpp: opening paragraph -- tile FA
 *    kernel, KQ accumulators compressed to 16-bit before the second product, the
 *    GQA optimisation -- and the "Performance changes" microbatch sweep);
 *  - paged-KV decode, including MLA where K and V are one compressed-KV matrix
 *    ("perf: FlashAttention-3 style MLA PageAttention", FlashInfer: change list
 *    item 4, and "Results" for batch x seq_len x 64 heads at page_size = 1).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates no device memory and keeps no pointer after a call returns.
 *  - Layouts are fixed, row-major, last index fastest; there are no strides.
 *  - Every call validates its arguments on the host first. A negative status
 *    means nothing was enqueued. Status 0 means the kernels were enqueued on
 *    `stream` (0 = the default stream); the call does not synchronise, so a
 *    fault inside a kernel surfaces at the caller's next synchronisation.
 *  - The mask is none (causal = 0) or causal aligned bottom-right: query i of
 *    Sq sits at absolute position Skv - Sq + i and sees keys j <= Skv - Sq + i.
 *    With Sq = Skv this is ordinary lower-triangular causal attention. A query
 *    with no visible key (Sq > Skv, or an empty sequence) gets O = 0 and
 *    lse = -infinity.
 *  - Grouped-query heads: query head h reads K/V head h / (Hq / Hkv).
 *  - lse (optional, may be NULL) is the natural-log log-sum-exp of the scaled
 *    scores of a row, in fp32.
 *  - Tensor base pointers must be 16-byte aligned (lse, page tables and
 *    sequence lengths: 4-byte aligned).
 *  - Calls on one stream are ordered; calls that share a workspace must not
 *    run concurrently on different streams.
 *  - With the environment variable FA_LOG=1 (read once per process) every
 *    compute call that passes validation prints the plan it launches (compute
 *    units planned for, workgroup shape, head pack, key splits, workspace
 *    bytes) as one "fa_log ..." line on stderr.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_BF16 = 0, FA_FP16 = 1, FA_FP32 = 2 } fa_dtype;

/* Paged KV pool layouts.
 *  FA_KV_SPLIT:      pool [num_pages, 2 (K, V), Hkv, page_size, D]; D_qk == D_v.
 *  FA_KV_MLA_SHARED: pool [num_pages, page_size, D_qk]; one row per token that is
 *                    both the key (all D_qk columns, [ckv | kpe]) and the value
 *                    (its first D_v columns, ckv). Hkv must be 1.
 * Token t of sequence b is in page page_table[b * max_pages_per_seq + t / page_size]
 * at slot t % page_size. */
typedef enum { FA_KV_SPLIT = 0, FA_KV_MLA_SHARED = 1 } fa_kv_layout;

enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  FA_ERR_UNSUPPORTED = -3, /* head size / dtype combination not built */
  FA_ERR_ALIGN = -4,       /* a base pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = -5,   /* workspace smaller than the plan needs */
  FA_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCRATCH = -7      /* a no-alloc call's split plan exceeds the static scratch */
};

/*
 * Prefill attention, bf16 in and bf16 out.
 * Passage: "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp), opening
 * paragraph (the tile FlashAttention kernel, grouped-query heads) and its
 * "Performance changes" table (prompt processing in microbatches of 16 to
 * 16384 queries, each call attending to every earlier key: causal, aligned
 * bottom-right).
 *   q, o [B, Sq, Hq, D]; k, v [B, Skv, Hkv, D]   (bf16)
 *   D in {64, 128}; Hq % Hkv == 0; B, Hq, Hkv, D >= 1; Sq, Skv >= 0.
 *   scale multiplies Q K^T (usually 1/sqrt(D)).
 * Never splits the keys and needs no workspace. Same as fa_prefill_ex with
 * in_dtype = out_dtype = FA_BF16, lse = NULL and no workspace.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN (nothing
 * enqueued); FA_ERR_HIP if the launch failed.
 */
int fa_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
               int Sq, int Skv, int D, int causal, float scale, hipStream_t stream);

/*
 * Prefill attention, full form: input and output types, the log-sum-exp, and
 * key splits merged by a log-sum-exp combine.
 * Passage: "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp), opening
 * paragraph (enough blocks in flight to occupy the GPU; the KQ values rounded
 * to 16 bits before the second product) for the operation; splitting a
 * reduction over several workers and merging the parts afterwards follows the
 * dk-split of "perf(kernels): speed up linear-attention prefill ~2.6x"
 * (hip-ep), Summary, here applied to key ranges.
 *   in_dtype  FA_BF16 or FA_FP16 (q, k, v)
 *   out_dtype FA_BF16, FA_FP16 or FA_FP32 (o)
 *   lse       [B, Hq, Sq] fp32, or NULL
 *   workspace device memory for split-KV partial results, or NULL. With NULL
 *             the keys are never split. Otherwise the launch planner may split
 *             the keys of long rows over several workgroups and merge the parts
 *             with a log-sum-exp combine kernel; workspace_bytes must then be at
 *             least fa_prefill_workspace_size(..., out_dtype) for the same
 *             shape, or the call fails with FA_ERR_WORKSPACE. The workspace
 *             holds no state between calls. Per split it holds a normalised
 *             partial output (in out_dtype) and an fp32 log-sum-exp per row.
 * Errors as fa_prefill, plus FA_ERR_WORKSPACE (and FA_ERR_ALIGN for a
 * workspace that is not 16-byte aligned).
 */
int fa_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                  fa_dtype in_dtype, fa_dtype out_dtype, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * Prefill attention with an explicit additive mask:
 *     O = softmax(scale * Q K^T + M) V        (and the causal rule if causal)
 * Passage: "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp), opening
 * paragraph: the KQ mask is an input of the FlashAttention kernels, and its
 * reads count as memory traffic that the grouped-query optimisation reduces.
 *   mask               element (b, i, j) at mask[b * mask_batch_stride +
 *                      i * mask_stride + j], in in_dtype; finite or -inf (-inf
 *                      hides the key; a row whose keys are all hidden gives
 *                      o = 0 and lse = -inf). mask_batch_stride 0 shares one
 *                      [Sq, Skv] mask over the batch.
 *   mask_stride        elements between rows: a multiple of 8 and at least Skv
 *                      rounded up to 8 (the kernel copies keys in groups of 8;
 *                      entries past Skv are read but never used); Sq *
 *                      mask_stride at most 2^30 (FA_ERR_SHAPE otherwise)
 *   mask_batch_stride  0, or elements between batch entries (a multiple of 8)
 * The mask pointer must be 16-byte aligned (FA_ERR_ALIGN otherwise, also for a
 * stride that is not a multiple of 8); a null mask is FA_ERR_NULL. Every other
 * argument is as for fa_prefill_ex.
 */
int fa_prefill_mask(const void* q, const void* k, const void* v, const void* mask,
                    int64_t mask_stride, int64_t mask_batch_stride, void* o, float* lse, int B,
                    int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                    fa_dtype in_dtype, fa_dtype out_dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of workspace the planner may use for this prefill shape and output
 * type (0 if it never splits it): per split, the partial rows in out_dtype and
 * an fp32 log-sum-exp per row.
 * Passage: the occupancy rule of "CUDA: fix FA occupancy, optimize tile
 * kernel" (llama.cpp), opening paragraph -- the keys are split until the grid
 * fills the GPU's compute units.
 * Host function: planned for the compute units of the current device
 * (hipDeviceGetAttribute; 256 when no device can be queried). Environment
 * variables: FA_PREFILL_SPLITS forces a split count (tuning), FA_NUM_CUS sets
 * the compute units planned for. Returns 0 for an invalid shape or type.
 */
size_t fa_prefill_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                                 fa_dtype out_dtype);

/*
 * Paged-KV decode: one query token per sequence, attending to every cached
 * token of its sequence (no mask).
 * Passage: "perf: FlashAttention-3 style MLA PageAttention" (FlashInfer):
 * "Results" (decode over a page table, batch x seq_len x 64 heads at
 * page_size = 1, measured in GB/s) and change list item 4 (MLA keeps one
 * compressed-KV matrix that serves as both K and V: FA_KV_MLA_SHARED).
 *   q           [B, Hq, D_qk]  (dtype)
 *   kv_pool     see fa_kv_layout (dtype)
 *   page_table  [B, max_pages_per_seq] int32 page ids (entries past a sequence's
 *               last page are never read)
 *   seq_lens    [B] int32, each in [0, max_seq_len] (device memory); values are
 *               clamped to that range on the device
 *   num_pages   pages in kv_pool (>= 1). A page id outside [0, num_pages) is
 *               never dereferenced: its tokens read as zero keys and values
 *               (a wrong table gives wrong numbers, not a memory fault).
 *   o           [B, Hq, D_v] (dtype)
 *   lse         [B, Hq] fp32, or NULL
 *   (D_qk, D_v) (128, 128) with FA_KV_SPLIT, (576, 512) with FA_KV_MLA_SHARED
 *   page_size   >= 1; max_pages_per_seq * page_size >= max_seq_len; with
 *               FA_KV_SPLIT one page (2 * Hkv * page_size * 128 * 2 bytes)
 *               must be smaller than 2 GiB (FA_ERR_SHAPE otherwise)
 *   max_seq_len host-side upper bound of seq_lens (sizes the grid)
 *   num_splits  0 = let the planner choose; n >= 1 asks for n key splits per
 *               sequence (clamped to what the shape allows)
 *   dtype       FA_BF16 or FA_FP16
 *   workspace   partial results of split-KV, or NULL (then num_splits is 1):
 *               per split a normalised partial output (in dtype) and an fp32
 *               log-sum-exp per row; at least fa_decode_workspace_size(...)
 *               bytes for the same arguments (FA_ERR_WORKSPACE otherwise)
 * Pool slots that no token of a sequence owns (tail slots, spare pages) are
 * never read as data, so they may hold anything, NaN included.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN,
 * FA_ERR_WORKSPACE (nothing enqueued); FA_ERR_HIP if a launch failed.
 */
int fa_decode_paged(const void* q, const void* kv_pool, const int32_t* page_table,
                    const int32_t* seq_lens, int num_pages, void* o, float* lse, int B, int Hq,
                    int Hkv, int D_qk, int D_v, int page_size, int max_pages_per_seq,
                    int max_seq_len, fa_kv_layout layout, float scale, int num_splits,
                    fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged decode of Sq new tokens per sequence (speculative or chunked decode):
 * the Sq queries of sequence b are its last Sq tokens, token i at position
 * seq_lens[b] - Sq + i, and each sees the cached tokens up to its own position
 * (causal, bottom-right, as in fa_prefill). With Sq = 1 this is
 * fa_decode_paged.
 * Passage: "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp), opening
 * paragraph: the grouped-query optimisation reads each K/V row once for a
 * group of query heads, which pays for small batches of more than one token.
 * Here the query tokens of a sequence and the query heads of a K/V group are
 * packed into the MFMA rows together, so each K/V row is read once per
 * (sequence, K/V head). The paged gather is that of fa_decode_paged.
 *   q   [B, Sq, Hq, D_qk]; o [B, Sq, Hq, D_v]; lse [B, Hq, Sq] fp32 or NULL
 *   Sq  1 .. 64 (FA_ERR_SHAPE otherwise)
 * Both pool layouts. A row whose position is negative (seq_lens[b] < Sq)
 * sees no key: o = 0, lse = -inf. Every other argument and error is as for
 * fa_decode_paged; the workspace size comes from fa_decode_multi_workspace_size.
 */
int fa_decode_paged_multi(const void* q, const void* kv_pool, const int32_t* page_table,
                          const int32_t* seq_lens, int num_pages, void* o, float* lse,
                          int B, int Sq, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                          int max_pages_per_seq, int max_seq_len, fa_kv_layout layout,
                          float scale, int num_splits, fa_dtype dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace fa_decode_paged_multi may use (0 if it would not split).
 * Passage: the occupancy rule of "CUDA: fix FA occupancy, optimize tile kernel"
 * (llama.cpp), opening paragraph: sequences too short to fill the compute
 * units are split over key ranges. Host function, planned for the current
 * device as fa_prefill_workspace_size is; 0 for an invalid shape. */
size_t fa_decode_multi_workspace_size(int B, int Sq, int Hq, int Hkv, int D_qk, int D_v,
                                      int page_size, int max_seq_len, fa_kv_layout layout,
                                      int num_splits);

/* Bytes of workspace fa_decode_paged may use for this shape and split request
 * (0 if it would not split). Passage and planning as for
 * fa_decode_multi_workspace_size; 0 for an invalid shape. */
size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                                int max_seq_len, fa_kv_layout layout, int num_splits);

/* The number of key splits fa_decode_paged would use with a workspace (>= 1).
 * Passage as for fa_decode_multi_workspace_size. Host function, planned for
 * the compute units of the current device (FA_NUM_CUS overrides them). */
int fa_decode_num_splits(int B, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                         int max_seq_len, fa_kv_layout layout, int num_splits);

/*
 * Paged decode that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, plan, kernels and
 * results as fa_decode_paged with a workspace, except that the split-KV
 * partials go to a static device buffer the library owns: 32 MiB per GPU
 * (FA_DECODE_NOALLOC_SCRATCH_BYTES), held until the process ends. A plan whose
 * partials (splits x B x Hq x (2 D_v + 4) bytes) exceed it fails with
 * FA_ERR_SCRATCH before anything is enqueued; num_splits can then ask for
 * fewer. The call makes no hipMalloc / hipFree and no allocating library call;
 * its first call on a device looks up that device's copy of the buffer.
 * Every call on one GPU shares the buffer: calls that overlap on one GPU (on
 * different streams without ordering) race on it; calls ordered on one stream
 * do not. Errors: those of fa_decode_paged (without FA_ERR_WORKSPACE), plus
 * FA_ERR_SCRATCH, and FA_ERR_HIP if the buffer's address cannot be looked up.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fa_decode_paged_noalloc(const void* q, const void* kv_pool, const int32_t* page_table,
                            const int32_t* seq_lens, int num_pages, void* o, float* lse, int B,
                            int Hq, int Hkv, int D_qk, int D_v, int page_size,
                            int max_pages_per_seq, int max_seq_len, fa_kv_layout layout,
                            float scale, int num_splits, fa_dtype dtype, hipStream_t stream);

/* Static text for a status code. */
const char* fa_strerror(int status);

/* Library version, e.g. "0.1.0". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

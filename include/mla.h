/*
 * mla.h - C ABI of libmla.so: multi-head latent attention (MLA) decode over a
 * paged latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation (sabi-mla-vllm, opening paragraph and "What the plugin does";
 * vLLM pull request 55543, description and the review of its equivalence
 * test): every cached token holds one 576-value row per layer, a 512-wide
 * latent followed by one shared 64-wide rotary key.  An absorbed query per
 * head, cat(q_latent[512], q_pe[64]), scores every row of its request's
 * context, s_t = softmax_scale * <q, row_t> over all 576 values; the softmax
 * runs over the cache tokens; the output is the softmax-weighted sum of the
 * 512-wide latents, returned with the natural-log log-sum-exp of the scores.
 *
 * Paging: a request's token t lives in slot
 *     block_table[b * block_table_stride + t / page_size] * page_size + t % page_size
 * and the row starts at byte slot * row_bytes.  All slot and byte offsets are
 * formed in 64-bit arithmetic (sabi-mla-vllm, "B300 fix (0.2.0)": a 32-bit
 * element offset wraps at slot 2^31 / 576 = 3,728,270).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers on the current HIP device, row-major,
 *    contiguous; every pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    are asynchronous on that stream, never synchronise the device and never
 *    read device memory from the host.
 *  - The caller owns all memory.  The library allocates nothing and keeps no
 *    state beyond a per-device cache of the architecture check (and of the
 *    device's compute-unit count) and a thread-local message.
 *  - Arguments are validated on the host before any launch.  On error the call
 *    returns a nonzero MLA_ERR_* code, launches nothing and records a message
 *    (mla_last_error_message) naming the offending argument.  Nothing aborts,
 *    throws or prints.
 *  - Conditions that cannot be checked without reading device memory are
 *    preconditions: block-table entries inside the context must lie in
 *    [0, num_pages), and 0 <= seq_lens[b] <= block_table_stride * page_size.
 *    Entries past a request's last page are never read (may hold -1).  A wrong
 *    offset reads the wrong memory and then faults (sabi-mla-vllm, "B300 fix
 *    (0.2.0)": correct first token, then garbage, then an illegal memory
 *    access), so the library also comes as a checked build (libmla_checked.so,
 *    same ABI) whose kernels test both preconditions before forming an address.
 *
 * Per-call options of every decode entry point (the two arguments before `stream`)
 *  - flags: MLA_FLAG_* bits, 0 for the defaults; unknown bits are MLA_ERR_SHAPE.
 *      MLA_FLAG_CACHED_ROWS: plain loads of the cache rows instead of the default
 *      non-temporal (streaming) ones.  Results are bit-identical either way.  The
 *      default suits rows read once per step: whole 128-byte lines per load
 *      instruction with the non-temporal hint stream faster (long context, random
 *      pages: bf16 rows 211 -> 189 us per decode, fp8 rows 147 -> 136 us on
 *      MI355X) but stay out of the caches; plain loads suit batches whose requests
 *      share pages within a step (prefix sharing), whose repeated rows then hit in
 *      the L2 / last-level cache.  (The rank-768 decode reads 64-byte row segments
 *      and always uses plain loads.)
 *  - check_status: NULL, or (checked build only) a device int32 the caller zeroes
 *      beforehand.  A checked build's kernels OR MLA_CHECK_* bits into it when a
 *      precondition fails, and then read page 0 in place of an out-of-pool block id
 *      and clamp a length into [0, block_table_stride * page_size], so that no read
 *      leaves the cache or the block table; nothing traps.  The release build
 *      refuses a non-NULL check_status with MLA_ERR_SHAPE (it checks nothing).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

#if defined(__GNUC__) || defined(__clang__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL                            */
  MLA_ERR_SHAPE = 2,     /* a size or count is out of range                       */
  MLA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                      */
  MLA_ERR_WORKSPACE = 4, /* workspace missing or smaller than required            */
  MLA_ERR_ARCH = 5,      /* the current device is not gfx950                      */
  MLA_ERR_HIP = 6        /* a HIP runtime call or kernel launch failed            */
};

enum {
  MLA_CACHE_BF16_576 = 0, /* 576 bf16 values, 1152 bytes per row                  */
  MLA_CACHE_FP8_656 = 1   /* 512 e4m3 codes, 4 fp32 block scales, 64 bf16 = 656 B */
};

/* Decode option bits (the flags argument). */
enum { MLA_FLAG_CACHED_ROWS = 1 };

/* Bits a checked build ORs into *check_status. */
enum {
  MLA_CHECK_BLOCK_ID = 1, /* a block-table entry a context uses lies outside [0, num_pages) */
  MLA_CHECK_SEQ_LEN = 2   /* seq_lens[b] < 0 or > block_table_stride * page_size          */
};

enum { MLA_LATENT = 512, MLA_ROPE = 64, MLA_ROW = 576, MLA_MAX_HEADS = 16, MLA_MAX_Q_LEN = 16,
       MLA_MAX_QUERY_ROWS = 64, MLA_MAX_BALANCED_BATCH = 1024, MLA_MAX_SPARSE_TOKENS = 1 << 20,
       MLA_MAX_SPARSE_TOPK = 1 << 24 };

/* Bytes of workspace mla_decode_bf16 / mla_decode_fp8_656 need for num_splits
 * partitions: num_splits * batch * num_heads * (512 + 1) * 4 rounded up to 256,
 * or 0 when num_splits == 1.  Returns 0 for invalid arguments. */
MLA_API size_t mla_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t num_splits);

/* Decode over a bf16 cache (MLA_CACHE_BF16_576).
 *
 * q            bf16 [batch][num_heads][576], absorbed queries (latent part first).
 * kv_cache     bf16 [num_pages][page_size][576].
 * num_pages    pages in the pool (>= 1); page_size tokens per page (>= 1).
 * block_table  int32 [batch][block_table_stride]; physical page of each logical page.
 * seq_lens     int32 [batch]; context length of each request (0 allowed).
 * num_heads    1..16.  softmax_scale: finite float, applied to the fp32 scores.
 * num_splits   1..65535.  Each request's pages are cut into partitions of
 *              c = ceil(block_table_stride / num_splits) whole pages (the same c for
 *              every request, so short requests use fewer partitions and the rest are
 *              empty); each partition returns (out, lse) for its tokens and, when
 *              num_splits > 1, a second kernel merges them by log-sum-exp (vLLM pull
 *              request 55543: the partial-result merge contract with (0, -inf) as the
 *              neutral element).  The result does not depend on num_splits beyond
 *              rounding.  When batch x num_splits exceeds the device's compute units
 *              (and batch <= 1024), the workgroups take the non-empty partitions first.
 *              Merged here, empty partitions write no partial; kept (out == lse ==
 *              NULL), every partition's partial is written.
 * out          fp32 [batch][num_heads][512]: softmax-weighted latent sum.
 * lse          fp32 [batch][num_heads]: natural-log log-sum-exp of the scaled scores.
 *              A request with seq_lens == 0 gets out = +0.0 and lse = -inf.
 * workspace    device scratch of at least mla_decode_workspace_size() bytes when
 *              num_splits > 1 (may be NULL otherwise); holds the partials
 *              [num_splits][batch][num_heads][512] then [num_splits][batch][num_heads].
 *              Passing out == lse == NULL with num_splits > 1 stops there: the
 *              partials stay in the workspace for the caller to merge later (for
 *              example after exchanging them with other devices) with mla_merge_lse.
 */
MLA_API int mla_decode_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                    int32_t page_size, float softmax_scale, int32_t num_splits,
                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                    uint32_t flags, int32_t* check_status, void* stream);

/* mla_decode_bf16 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments, kernels and
 * results as mla_decode_bf16 without workspace / workspace_bytes.  The split partials go to a
 * scratch array of MLA_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on each device it
 * runs on until the process ends (part of the loaded code object; nothing is allocated per call).
 * num_splits is limited by it: mla_decode_workspace_size(batch, num_heads, num_splits) must not
 * exceed MLA_NOALLOC_SCRATCH_BYTES (MLA_ERR_WORKSPACE otherwise; the long-context batch of 4
 * requests x 16 heads at 64 splits needs 8.4 MB).  out and lse are required (the partials are
 * not handed out).  Every call on a device shares that device's scratch: calls that overlap on
 * one GPU (different streams, or threads without ordering) race and must be serialised by the
 * caller.  Nothing in the scratch needs to start at any value.  No hipMalloc, hipFree or other
 * allocating call is made. */
enum { MLA_NOALLOC_SCRATCH_BYTES = 16 << 20 };
MLA_API int mla_decode_bf16_noalloc(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                    int32_t page_size, float softmax_scale, int32_t num_splits,
                                    float* out, float* lse, uint32_t flags, int32_t* check_status,
                                    void* stream);

/* Decode over an fp8 cache (MLA_CACHE_FP8_656).  Same arguments and results as
 * mla_decode_bf16; kv_cache is uint8 [num_pages][page_size][656], each row
 * [0,512) OCP e4m3fn codes, [512,528) four little-endian fp32 scales (scale k
 * multiplies latent values [128k, 128k+128)), [528,656) 64 bf16 rope values
 * (vLLM pull request 55543, description: the 656-byte fp8_ds_mla row with
 * per-128-block scales and bf16 rope bytes; the byte order is this library's
 * reading, as the page lists the parts but not their order).  Latent values are
 * code * scale, exact; q is used in bf16 as given. */
MLA_API int mla_decode_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                       const int32_t* block_table, int64_t block_table_stride,
                       const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                       int32_t page_size, float softmax_scale, int32_t num_splits,
                       float* out, float* lse, void* workspace, size_t workspace_bytes,
                       uint32_t flags, int32_t* check_status, void* stream);

/* Batch-balanced decode: the same results as mla_decode_bf16 / mla_decode_fp8_656
 * (single-token queries), with the work cut across the whole batch instead of per
 * request.  The split-KV partition with log-sum-exp merge (vLLM pull request 55543: the
 * partial-result merge contract) is applied to the batch's concatenated context: the
 * requests' tokens, request after request, each non-empty request preceded by a fixed
 * allowance for the start-up of a segment, are cut into num_workgroups equal ranges (fewer
 * when the batch is smaller); a workgroup decodes every request segment its range meets
 * into a partial (out, lse), and a merge kernel combines each request's partials.  Every
 * workgroup gets the same cost whatever the length mix, so a ragged batch finishes in one
 * balanced wave instead of a tail of long requests.  Two launches, no host synchronisation.
 *
 * batch           1..MLA_MAX_BALANCED_BATCH (1024).
 * num_workgroups  0..65535; 0 = one per compute unit of the current device (256 on MI355X),
 *                 the intended use.
 * workspace       device scratch of at least mla_decode_balanced_workspace_size(batch,
 *                 num_heads, num_workgroups) bytes, 16-byte aligned: int64 range
 *                 bounds [batch + 1], then up to batch + num_workgroups - 1 partials.
 *                 (The size function resolves num_workgroups = 0 the same way; it
 *                 returns 0 when there is no usable device.)
 * The decode reads seq_lens on the device (no host synchronisation); a request with
 * seq_lens == 0 gets (+0.0, -inf).  Passing out == lse == NULL stops after the decode
 * kernel: the partials stay in the workspace and mla_merge_lse_balanced combines them
 * later.  Every other argument, result and error as mla_decode_bf16 / mla_decode_fp8_656. */
MLA_API size_t mla_decode_balanced_workspace_size(int32_t batch, int32_t num_heads, int32_t num_workgroups);
MLA_API int mla_decode_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                     const int32_t* block_table, int64_t block_table_stride,
                                     const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                     int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                     float* out, float* lse, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, int32_t* check_status, void* stream);
/* Batch-balanced NoPE-512 decode: the schedule of mla_decode_balanced_* with the scores of
 * mla_decode_nope_bf16 / mla_decode_nope_fp8_656 (q bf16 [batch][num_heads][512], the rows'
 * rope part never read).  Arguments, workspace, results and errors as mla_decode_balanced_*. */
MLA_API int mla_decode_balanced_nope_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                          const int32_t* block_table, int64_t block_table_stride,
                                          const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                          int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                                          uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_balanced_nope_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                             const int32_t* block_table, int64_t block_table_stride,
                                             const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                             int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                                             uint32_t flags, int32_t* check_status, void* stream);

/* Merge step of the batch-balanced decode: combines each request's partials left in the
 * workspace by a mla_decode_balanced_* call made with out == lse == NULL and the same
 * batch, num_heads and num_workgroups (the log-sum-exp merge contract of vLLM pull request
 * 55543).  out fp32 [batch][num_heads][512], lse fp32 [batch][num_heads]; a request with
 * no token gets (+0.0, -inf).  After mla_decode_mtp_balanced_* pass num_heads' = q_len *
 * num_heads (1..MLA_MAX_QUERY_ROWS): the query rows of a request act as its heads.  Errors
 * as mla_merge_lse; MLA_ERR_WORKSPACE if workspace_bytes is below
 * mla_decode_balanced_workspace_size(). */
MLA_API int mla_merge_lse_balanced(const void* workspace, size_t workspace_bytes, int32_t batch,
                                   int32_t num_heads, int32_t num_workgroups, float* out, float* lse,
                                   void* stream);
MLA_API int mla_decode_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                        const int32_t* block_table, int64_t block_table_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                        int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                        float* out, float* lse, void* workspace, size_t workspace_bytes,
                                        uint32_t flags, int32_t* check_status, void* stream);

/* NoPE-512 decode: layers without a rotary part (vLLM pull request 55543, description
 * of the NoPE-512 change: such layers keep the 576-value / 656-byte row, store zeros in
 * its rope part and pad q_pe with zeros, so the rope part adds nothing to any score).
 * Here the padding is not needed: q is bf16 [batch][num_heads][512] and the scores use
 * the 512 latent values only, s_t = softmax_scale * <q, latent_t>.  The rows' rope part
 * never enters a score and may hold anything (non-finite values included).  A bf16 row
 * costs 1,024 bytes of HBM traffic instead of 1,152; fp8 rows are streamed whole (656
 * bytes: the 528 bytes a score uses are not contiguous across rows, and whole-line
 * streaming of the full rows measured faster than reading the pieces).  kv_cache, every other
 * argument, the results and the errors are those of mla_decode_bf16 / mla_decode_fp8_656. */
MLA_API int mla_decode_nope_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                 const int32_t* block_table, int64_t block_table_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                 int32_t page_size, float softmax_scale, int32_t num_splits,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_nope_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                    int32_t page_size, float softmax_scale, int32_t num_splits,
                                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                                    uint32_t flags, int32_t* check_status, void* stream);

/* Decode over per-query index lists (sparse MLA: vLLM pull request 55543 serves the
 * NoPE-512 layers through the FlashMLA sparse backend, where an indexer picks for every
 * query token the cache slots it attends to; its ragged mixed-batch test gives lists with
 * 0, 1 or some valid entries followed by -1).  Query token t attends to the slots listed in
 * indices[t][0 .. topk): s_j = softmax_scale * <q_t, row(indices[t][j])> over the valid
 * entries j, softmax over them, out = sum p_j latent(indices[t][j]).
 * q           bf16 [num_tokens][num_heads][576] (_nope_: [num_tokens][num_heads][512], the
 *             scores over the 512 latent values only, as mla_decode_nope_*).
 * kv_cache    num_slots rows of 1,152 bytes (bf16 576) or 656 bytes (fp8_656), slot after
 *             slot: a paged pool seen as its slots (slot = page * page_size + offset).
 * num_slots   rows in kv_cache, >= 1.  Row offsets are formed in 64 bits (slot * row bytes),
 *             so slots above 3,728,270 (where a 32-bit element offset of a 576-value row
 *             wraps) are addressed like any other.
 * indices     int32 [num_tokens][topk], row-major.  An entry in [0, num_slots) selects that
 *             slot (a slot listed twice counts twice); a negative entry (-1 in the lists'
 *             padding, but anywhere in a list) selects nothing.  A query whose list selects
 *             nothing gets (+0.0, -inf), the neutral partial of the merge contract.  Entries
 *             >= num_slots break the precondition: the release build reads outside the cache;
 *             the checked build reads slot 0 instead and sets MLA_CHECK_BLOCK_ID.
 * topk        entries per list, 1..MLA_MAX_SPARSE_TOPK.    num_tokens  1..MLA_MAX_SPARSE_TOKENS.
 * num_heads   1..MLA_MAX_HEADS.
 * num_splits  1..65535: each list is cut into num_splits parts of ceil(topk / num_splits)
 *             entries (trailing parts may be empty), decoded by separate workgroups and
 *             merged by log-sum-exp; a workspace of mla_decode_workspace_size(num_tokens,
 *             num_heads, num_splits) bytes is needed when num_splits > 1.
 * out, lse    fp32 [num_tokens][num_heads][512] and [num_tokens][num_heads] (natural log).
 *             out == lse == NULL with num_splits > 1 stops after the decode kernel: the
 *             partials stay in the workspace ([num_splits][num_tokens][num_heads][512], then
 *             [num_splits][num_tokens][num_heads]; every partition writes one, an empty one
 *             (+0, -inf)) for mla_merge_lse.
 * flags, check_status, stream, the errors and the rounding as mla_decode_bf16 /
 * mla_decode_fp8_656. */
MLA_API int mla_decode_sparse_bf16(const void* q, const void* kv_cache, int64_t num_slots,
                                   const int32_t* indices, int32_t topk, int32_t num_tokens, int32_t num_heads,
                                   float softmax_scale, int32_t num_splits, float* out, float* lse,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   int32_t* check_status, void* stream);
MLA_API int mla_decode_sparse_fp8_656(const void* q, const void* kv_cache, int64_t num_slots,
                                      const int32_t* indices, int32_t topk, int32_t num_tokens, int32_t num_heads,
                                      float softmax_scale, int32_t num_splits, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, uint32_t flags,
                                      int32_t* check_status, void* stream);
MLA_API int mla_decode_sparse_nope_bf16(const void* q, const void* kv_cache, int64_t num_slots,
                                        const int32_t* indices, int32_t topk, int32_t num_tokens, int32_t num_heads,
                                        float softmax_scale, int32_t num_splits, float* out, float* lse,
                                        void* workspace, size_t workspace_bytes, uint32_t flags,
                                        int32_t* check_status, void* stream);
MLA_API int mla_decode_sparse_nope_fp8_656(const void* q, const void* kv_cache, int64_t num_slots,
                                           const int32_t* indices, int32_t topk, int32_t num_tokens, int32_t num_heads,
                                           float softmax_scale, int32_t num_splits, float* out, float* lse,
                                           void* workspace, size_t workspace_bytes, uint32_t flags,
                                           int32_t* check_status, void* stream);

/* Multi-token verify decode (speculative decoding): q_len query tokens per request, the
 * last q_len positions of its sequence, scored against the cache in one pass that reads
 * every row once per request (qwen-mla-vllm, "16 GB GPUs": a verify step reading the latent
 * cache once per request instead of once per draft token).  Causal: seq_lens[b] = L counts
 * the q_len new tokens, whose rows must already be in the cache, and query i (0-based)
 * attends to tokens 0 .. L - q_len + i; a query that sees no token (L < q_len) gets
 * (+0, -inf).  The mask is this library's reading; the pages do not spell it out.
 * q      bf16 [batch][q_len][num_heads][576]
 * out    fp32 [batch][q_len][num_heads][512];  lse fp32 [batch][q_len][num_heads]
 * q_len  1..MLA_MAX_Q_LEN with q_len * num_heads <= MLA_MAX_QUERY_ROWS (64); q_len = 1 is
 *        mla_decode_bf16 / mla_decode_fp8_656.
 * The workspace is sized as for num_heads' = q_len * num_heads
 * (mla_decode_workspace_size(batch, q_len * num_heads, num_splits)); partials and
 * mla_merge_lse treat the q_len * num_heads query rows of a request as its heads.
 * Every other argument, result and error as mla_decode_bf16 / mla_decode_fp8_656. */
MLA_API int mla_decode_mtp_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                const int32_t* block_table, int64_t block_table_stride,
                                const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t num_heads,
                                int32_t page_size, float softmax_scale, int32_t num_splits,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_mtp_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                   const int32_t* block_table, int64_t block_table_stride,
                                   const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                   int32_t num_heads, int32_t page_size, float softmax_scale,
                                   int32_t num_splits, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream);

/* Batch-balanced verify decode: the results of mla_decode_mtp_bf16 / mla_decode_mtp_fp8_656
 * (q_len query tokens per request, the same causal reading) with the schedule of
 * mla_decode_balanced_* (the batch's tokens cut into num_workgroups equal-cost ranges across
 * request boundaries, each range's partials merged by log-sum-exp), so a ragged batch of
 * verify steps finishes in one balanced wave.  The cache is still read once per request
 * range, for all q_len query tokens.
 * workspace  at least mla_decode_balanced_workspace_size(batch, q_len * num_heads,
 *            num_workgroups) bytes: a partial slot holds the q_len * num_heads query rows
 *            of its request.  Passing out == lse == NULL leaves the partials there for
 *            mla_merge_lse_balanced(..., q_len * num_heads, num_workgroups, ...).
 * q, out, lse, q_len as mla_decode_mtp_*; batch, num_workgroups and every other argument,
 * result and error as mla_decode_balanced_*. */
MLA_API int mla_decode_mtp_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                         const int32_t* block_table, int64_t block_table_stride,
                                         const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                         int32_t num_heads, int32_t page_size, float softmax_scale,
                                         int32_t num_workgroups, float* out, float* lse, void* workspace,
                                         size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_mtp_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                            const int32_t* block_table, int64_t block_table_stride,
                                            const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                            int32_t num_heads, int32_t page_size, float softmax_scale,
                                            int32_t num_workgroups, float* out, float* lse, void* workspace,
                                            size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream);

/* Decode step with the cache write folded in: the results of mla_cache_write of the step's
 * new rows followed by mla_decode_mtp_* (per-request partitions) or mla_decode_mtp_balanced_*
 * (batch-balanced), in one launch of the decode (plus its merge).  The cache write and the
 * decode read the same rows (vLLM pull request 55543: the cache-write step stores the new
 * token's latent ++ rotary key row, which the decode then attends to); here the partition
 * whose token range holds a new row's position stores that row before it reads any row, so
 * no separate cache-write kernel runs (this library's arrangement, not the pages').
 * new_latent bf16 [batch][q_len][512], new_k_pe bf16 [batch][q_len][64] or NULL (rope part
 *            written as zeros); new_slots int64 [batch][q_len], negative = not written.
 *            New row i of request b is context position seq_lens[b] - q_len + i; rows whose
 *            position is negative (seq_lens[b] < q_len) are not written.
 * kv_cache   written (the new rows, encoded as mla_cache_write encodes them) and read.
 * Precondition (as for the separate calls): new_slots[b][i] is the slot the block table gives
 * for that position, page_id * page_size + position % page_size, and the slots are distinct;
 * the checked build leaves a row unwritten, and reports MLA_CHECK_BLOCK_ID, when its slot lies
 * outside [0, num_pages * page_size) or differs from that slot.  q_len 1..MLA_MAX_Q_LEN
 * (q_len = 1: the single-token decode).
 * mla_decode_append_*: every other argument, result and error as mla_decode_mtp_*;
 * mla_decode_append_balanced_*: as mla_decode_mtp_balanced_* (num_workgroups, workspace,
 * out == lse == NULL for the partials). */
MLA_API int mla_decode_append_bf16(const void* q, const void* new_latent, const void* new_k_pe,
                                   const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                   const int32_t* block_table, int64_t block_table_stride,
                                   const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t num_heads,
                                   int32_t page_size, float softmax_scale, int32_t num_splits, float* out,
                                   float* lse, void* workspace, size_t workspace_bytes, uint32_t flags,
                                   int32_t* check_status, void* stream);
MLA_API int mla_decode_append_fp8_656(const void* q, const void* new_latent, const void* new_k_pe,
                                      const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                      const int32_t* block_table, int64_t block_table_stride,
                                      const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t num_heads,
                                      int32_t page_size, float softmax_scale, int32_t num_splits, float* out,
                                      float* lse, void* workspace, size_t workspace_bytes, uint32_t flags,
                                      int32_t* check_status, void* stream);
MLA_API int mla_decode_append_balanced_bf16(const void* q, const void* new_latent, const void* new_k_pe,
                                            const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                            const int32_t* block_table, int64_t block_table_stride,
                                            const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                            int32_t num_heads, int32_t page_size, float softmax_scale,
                                            int32_t num_workgroups, float* out, float* lse, void* workspace,
                                            size_t workspace_bytes, uint32_t flags, int32_t* check_status,
                                            void* stream);
MLA_API int mla_decode_append_balanced_fp8_656(const void* q, const void* new_latent, const void* new_k_pe,
                                               const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                               const int32_t* block_table, int64_t block_table_stride,
                                               const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                               int32_t num_heads, int32_t page_size, float softmax_scale,
                                               int32_t num_workgroups, float* out, float* lse, void* workspace,
                                               size_t workspace_bytes, uint32_t flags, int32_t* check_status,
                                               void* stream);

/* Other latent geometries (qwen-mla-vllm: per-layer latent ranks 256 / 768 / 1792 with a small
 * rotary tail, "How it works"; GLA-g2, the latent split into two head groups, opening section).
 * The row layouts are this library's reading; the pages give none.
 *
 * mla_decode_rank256_bf16: a rank-256 layer.  kv_cache bf16 [num_pages][page_size][320] (256
 * latent values, then 64 rope values), q bf16 [batch][num_heads][320], out fp32
 * [batch][num_heads][256]; scores over all 320 values, output the weighted latent sum.
 *
 * mla_decode_gla2_bf16 / mla_decode_gla2_fp8_656: GLA-g2 on the 576-value / 656-byte row.
 * num_heads even; heads [0, H/2) use latent values [0, 256), heads [H/2, H) use [256, 512),
 * both groups share the 64 rope values.  q bf16 [batch][num_heads][320] (the head's group
 * latent part, then its rope part); out fp32 [batch][num_heads][256], the weighted sum of the
 * group's latent values.  The row is read once for both groups.
 *
 * Every other argument, result and error as mla_decode_bf16; the partials left in the
 * workspace (out == lse == NULL) are 256 wide: merge them with mla_merge_lse_width(.., 256, ..).
 *
 * mla_decode_rank768_bf16 / mla_decode_rank1792_bf16: rank-768 / rank-1792 layers.  kv_cache
 * bf16 [num_pages][page_size][D + 64] (D latent values, then 64 rope values), q bf16
 * [batch][num_heads][D + 64], out fp32 [batch][num_heads][D], D = 768 / 1792; scores over all
 * D + 64 values.  The workspace (num_splits > 1) is mla_decode_rank_workspace_size(batch,
 * num_heads, num_splits, D) bytes: partials [num_splits][batch][num_heads][D] then
 * [num_splits][batch][num_heads]; merge left partials with mla_merge_lse_width(.., D, ..).
 * One pass (the pages' own kernels take two for 1792, where one does not fit their shared
 * memory). */
MLA_API int mla_decode_rank256_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                    int32_t page_size, float softmax_scale, int32_t num_splits,
                                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                                    uint32_t flags, int32_t* check_status, void* stream);
MLA_API size_t mla_decode_rank_workspace_size(int32_t batch, int32_t num_heads, int32_t num_splits,
                                              int32_t latent_rank);
MLA_API int mla_decode_rank768_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                    int32_t page_size, float softmax_scale, int32_t num_splits,
                                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                                    uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_rank1792_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                     const int32_t* block_table, int64_t block_table_stride,
                                     const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                     int32_t page_size, float softmax_scale, int32_t num_splits,
                                     float* out, float* lse, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_gla2_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                 const int32_t* block_table, int64_t block_table_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                 int32_t page_size, float softmax_scale, int32_t num_splits,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_gla2_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                    int32_t page_size, float softmax_scale, int32_t num_splits,
                                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                                    uint32_t flags, int32_t* check_status, void* stream);

/* GLA-g2 heads under the batch-balanced schedule (ragged batches): q bf16
 * [batch][num_heads][320], out fp32 [batch][num_heads][256], lse [batch][num_heads], head groups
 * and rows as mla_decode_gla2_*; num_workgroups, the workspace
 * (mla_decode_balanced_workspace_size(batch, num_heads, num_workgroups) bytes) and the schedule as
 * mla_decode_balanced_*.  out and lse are required: these calls always merge their own partials
 * (whose rows are 256 values wide), so there is no partials-only form.  flags, check_status,
 * stream and the errors as mla_decode_bf16. */
MLA_API int mla_decode_gla2_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages,
                                          const int32_t* block_table, int64_t block_table_stride,
                                          const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                          int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                                          uint32_t flags, int32_t* check_status, void* stream);
MLA_API int mla_decode_gla2_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                             const int32_t* block_table, int64_t block_table_stride,
                                             const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                             int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                                             uint32_t flags, int32_t* check_status, void* stream);

/* mla_merge_lse for partial rows of `width` values (256, 512, 768 or 1792): part_out fp32
 * [num_splits][batch][num_rows][width], part_lse [num_splits][batch][num_rows], out
 * [batch][num_rows][width], lse [batch][num_rows]; same formula and NaN / empty rules. */
MLA_API int mla_merge_lse_width(const float* part_out, const float* part_lse, int32_t num_splits,
                                int32_t batch, int32_t num_rows, int32_t width, float* out,
                                float* lse, void* stream);

/* Merge num_splits partial results over disjoint token sets (vLLM pull request
 * 55543: partial (o, lse) pairs merge by log-sum-exp; a partition with no
 * tokens is (0, -inf)).
 * part_out fp32 [num_splits][batch][num_heads][512], part_lse fp32 [num_splits][batch][num_heads].
 * out fp32 [batch][num_heads][512], lse fp32 [batch][num_heads]:
 *   M = max_p lse_p; if M = -inf: out = 0, lse = -inf;
 *   else w_p = exp(lse_p - M), lse = M + ln sum_p w_p, out = sum_p w_p out_p / sum_p w_p.
 * out/lse must not overlap the partials. */
MLA_API int mla_merge_lse(const float* part_out, const float* part_lse, int32_t num_splits,
                  int32_t batch, int32_t num_heads, float* out, float* lse, void* stream);

/* Write new tokens' rows into the cache (the cache-write step of vLLM pull
 * request 55543, which concatenates the latent and the 64-wide rotary key into
 * the row at each token's slot).
 * latent bf16 [num_tokens][512]; k_pe bf16 [num_tokens][64], or NULL for a NoPE layer:
 * the rope part of each row is then written as zeros (+0.0 bf16 values);
 * slot_mapping int64 [num_tokens], slot of each token; negative = skip the token.
 * kv_cache: num_slots rows in cache_format; slots must be < num_slots and distinct
 * (two tokens writing one slot race).
 * MLA_CACHE_BF16_576: row = latent ++ k_pe, copied bit for bit.
 * MLA_CACHE_FP8_656: per 128-value block a = max|x|, s = a / 448 (fp32, IEEE
 *   division), codes = e4m3fn(x / s) rounded to nearest-even and saturated at
 *   +-448, sign kept; a block with a == 0 stores s = 0 and codes 0x00; then the
 *   four scales and k_pe as bf16.  A block holding a NaN or an infinity stores the
 *   quiet NaN scale 0x7FC00000 and 128 codes 0x7F (e4m3fn NaN), so every value of
 *   that block decodes to NaN and a score that uses it is NaN (this library's
 *   reading: the pages cover finite latents only; the bf16 row keeps such values
 *   as they are). */
MLA_API int mla_cache_write(const void* latent, const void* k_pe, const int64_t* slot_mapping,
                    int32_t num_tokens, void* kv_cache, int32_t cache_format,
                    int64_t num_slots, void* stream);

/* Context gather for prefill (the int64 cache gather of sabi-mla-vllm, "B300 fix (0.2.0)",
 * and the fp8 context-gather-and-upconvert path of vLLM pull request 55543, which reads
 * 656-byte rows into a workspace 576 values wide).  Writes bf16 [total_rows][576]:
 *   out row cu_rows[b] + j = token seq_starts[b] + j of request b, j < cu_rows[b+1] - cu_rows[b]
 * read through the block table with 64-bit slot and byte offsets.  MLA_CACHE_BF16_576: the
 * row as stored.  MLA_CACHE_FP8_656: each latent value is bf16(fl32(code * scale)), the
 * float32 product rounded to nearest even and then to bf16, nearest even (this library's
 * reading; the pages name the operation, not its rounding); rope values as stored.
 * cu_rows    int64 [batch + 1], cu_rows[0] = 0, non-decreasing, cu_rows[batch] = total_rows.
 * seq_starts int32 [batch], first context position to gather per request, or NULL for 0.
 * total_rows passed by the caller (the library never reads device memory on the host),
 *            0 .. 2^32.
 * Preconditions (not checkable without reading device memory): the cu_rows layout above;
 * seq_starts[b] + rows of b <= block_table_stride * page_size; the block-table entries
 * those tokens use lie in [0, num_pages).  total_rows == 0 launches nothing.
 * check_status: as for the decodes (NULL in the release build); a checked build tests
 * every block id the gather uses (MLA_CHECK_BLOCK_ID) and seq_starts[b] + rows of b
 * against block_table_stride * page_size (MLA_CHECK_SEQ_LEN; the rows past that bound
 * are then written as zeros). */
MLA_API int mla_gather_context(const void* kv_cache, int32_t cache_format, int64_t num_pages,
                               int32_t page_size, const int32_t* block_table,
                               int64_t block_table_stride, const int64_t* cu_rows,
                               const int32_t* seq_starts, int32_t batch, int64_t total_rows,
                               void* out, int32_t* check_status, void* stream);

/* 1 for the checked build (libmla_checked.so), 0 for the release build (libmla.so). */
MLA_API int mla_checked_build(void);

/* The preconditions of the decodes, tested on the host over host copies of the block table
 * and the lengths (the test the checked build's kernels make on the device, for callers that
 * hold the tables on the host before uploading them): returns the MLA_CHECK_* bits that hold
 * (0 when every context lies inside the pool and the table), or -MLA_ERR_NULL /
 * -MLA_ERR_SHAPE for missing or out-of-range arguments.  Token t of request b uses entry
 * block_table[b * block_table_stride + t / page_size] for t < seq_lens[b]; entries past a
 * request's context are not looked at.  q_len and the schedule do not change the
 * preconditions. */
MLA_API int mla_check_preconditions_host(const int32_t* block_table, int64_t block_table_stride,
                                         const int32_t* seq_lens, int32_t batch, int32_t page_size,
                                         int64_t num_pages);

MLA_API const char* mla_status_string(int status);
/* Message describing the last failed call on this thread ("" if none). */
MLA_API const char* mla_last_error_message(void);
MLA_API int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */

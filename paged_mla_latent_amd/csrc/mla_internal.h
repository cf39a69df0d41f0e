// Internal launch interface between the C ABI (mla_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

struct DecodeParams {
  const uint16_t* q;           // bf16 [B][q_len][H][576] ([..][512] for the NoPE kernels)
  const uint8_t* cache;        // rows of row_bytes bytes
  const int32_t* block_table;  // [B][bt_stride]
  int64_t bt_stride;
  const int32_t* seq_lens;     // [B]
  int batch;
  int heads;
  int q_len;                   // query tokens per request (1 = plain decode)
  int page_size;
  int num_splits;
  float scale_log2;            // softmax_scale * log2(e)
  float* out;                  // [B][q_len][H][512]  (num_splits == 1)
  float* lse;                  // [B][q_len][H]
  float* part_out;             // [S][B][q_len][H][512] (num_splits > 1)
  float* part_lse;             // [S][B][q_len][H]
  int64_t* cu;                 // batch-balanced mode: cost-axis starts v [B + 1], stored by the decode
  int compact;                 // per-request mode: map workgroups onto the non-empty partitions first
  int skip_empty;              // per-request split mode: empty partitions write no partial (the
                               // merge counts each request's non-empty partitions itself)
  int stream_rows;             // non-temporal row loads (no MLA_FLAG_CACHED_ROWS)
  int64_t num_pages;           // pages in the pool (checked build: block ids are tested against it)
  int32_t* check_status;       // checked build: MLA_CHECK_* bits are ORed in here (may be NULL)
  // The step's new rows, written by the decode itself before it reads them (NULL: none).  New
  // row i of request b (index b * q_len + i) is context position L_b - q_len + i.
  const uint16_t* new_latent = nullptr;  // bf16 [B][q_len][512]
  const uint16_t* new_k_pe = nullptr;    // bf16 [B][q_len][64], or NULL: rope part written as zeros
  const int64_t* new_slots = nullptr;    // int64 [B][q_len]: slot of each new row; negative = not written
  uint8_t* cache_w = nullptr;            // the cache again, writable (set with new_latent)
};

// ------------------------------------------------------------------------------------
// Preconditions of the decodes (mla.h): every block id a context uses lies in [0, num_pages)
// and 0 <= L <= block_table_stride * page_size.  The release build trusts them; the checked
// build (-DMLA_CHECKED) tests them on the device before forming any address: an out-of-pool
// block id reads page 0 instead and a length outside the range is clamped into it, so no read
// leaves the cache or the block table, and the failed test's bit goes to *check_status.  The
// host helper mla_check_preconditions_host applies the same predicates.
// ------------------------------------------------------------------------------------
#ifdef MLA_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif
constexpr uint32_t kCheckBlockId = 1;  // MLA_CHECK_BLOCK_ID
constexpr uint32_t kCheckSeqLen = 2;   // MLA_CHECK_SEQ_LEN

__host__ __device__ __forceinline__ bool page_in_pool(int64_t page, int64_t num_pages) {
  return page >= 0 && page < num_pages;
}
__host__ __device__ __forceinline__ bool len_in_table(int64_t L, int64_t bt_stride, int64_t page_size) {
  return L >= 0 && L <= bt_stride * page_size;
}

// Checked build: page 0 in place of a block id outside the pool, and the bit in `bad`.
__device__ __forceinline__ int32_t checked_page(int32_t page, int64_t num_pages, uint32_t& bad) {
  if constexpr (kChecked) {
    const bool ok = page_in_pool(page, num_pages);
    bad |= ok ? 0u : kCheckBlockId;
    return ok ? page : 0;
  } else {
    return page;
  }
}

// Checked build: a context length clamped into [0, bt_stride * page_size], and the bit in `bad`.
__device__ __forceinline__ int64_t checked_len(int64_t L, int64_t bt_stride, int64_t page_size, uint32_t& bad) {
  if constexpr (kChecked) {
    const bool ok = len_in_table(L, bt_stride, page_size);
    bad |= ok ? 0u : kCheckSeqLen;
    return L < 0 ? 0 : (ok ? L : bt_stride * page_size);
  } else {
    return L;
  }
}

// Checked build: ORs the wave's `bad` bits into *status (one atomic per wave, only when a
// test failed).  Called from wave-uniform control flow with every lane active.
__device__ __forceinline__ void report_checks(uint32_t bad, int32_t* status) {
  if constexpr (kChecked) {
    uint32_t any = 0;
    if (__builtin_amdgcn_ballot_w64((bad & kCheckBlockId) != 0)) any |= kCheckBlockId;
    if (__builtin_amdgcn_ballot_w64((bad & kCheckSeqLen) != 0)) any |= kCheckSeqLen;
    if (any != 0 && status != nullptr && (threadIdx.x & 63) == 0) atomicOr(status, (int32_t)any);
  }
}

// Tokens [t0, t1) of one request.
struct Range {
  int64_t t0, t1;
};

// Partition s of a request of L tokens: whole pages, c = ceil(W / S) pages per partition,
// W = the block table's width (the most pages any request may use).  Every request's
// partitions have the same size, so a batch of ragged lengths balances: short requests
// use fewer (non-empty) partitions instead of smaller ones.
__device__ __forceinline__ Range partition(int64_t L, int ps, int S, int s, int64_t W) {
  const int64_t P = (L + ps - 1) / ps;
  int64_t c = (W + S - 1) / S;
  if (c < 1) c = 1;
  const int64_t p0 = min(P, (int64_t)s * c);
  const int64_t p1 = min(P, (int64_t)(s + 1) * c);
  return {min(L, p0 * ps), min(L, p1 * ps)};
}

// Non-empty partitions of a request of L tokens under the rule above: ceil(ceil(L / ps) / c),
// kept within [0, S] so that a length past the block table (a broken precondition) can
// never index a partial beyond the workspace.
__device__ __forceinline__ int counted_partitions(int64_t L, int ps, int64_t W, int S) {
  const int64_t c = max((W + S - 1) / S, (int64_t)1);
  const int64_t n = ((max(L, (int64_t)0) + ps - 1) / ps + c - 1) / c;
  return (int)min(n, (int64_t)S);
}

// Batch-balanced mode: at most kMaxBalancedBatch requests; each non-empty request adds
// kSegmentCost positions to the cost axis, and workgroup w of W takes axis positions
// [flat_begin(V, W, w), flat_begin(V, W, w + 1)), V = the axis length.
constexpr int kMaxBalancedBatch = 1024;
constexpr int64_t kSegmentCost = 512;
// The single-token kernels that also write the step's new rows charge each non-empty request
// kAppendTail more positions after its last token (tokenless, like the start-up allowance): the
// segment that holds a request's newest row waits one more trip to memory for its store before
// its first row load, and the workgroups meeting a request's end are given that much less work
// (fp8_ragged 93.0 -> 91.8 us per step, high_slot 492.1 -> 491.4 us).  The verify steps take no
// tail: with one, the fp8 verify step measured 3 us slower.
constexpr int64_t kAppendTail = 64;
__device__ __forceinline__ int64_t flat_begin(int64_t N, int64_t W, int64_t w) {
  return (N / W) * w + ((N % W) * w) / W;  // floor(w N / W) without 64-bit overflow
}

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_nope_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_nope_fp8(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_rank256_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_gla2_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_rank768_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_rank1792_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_gla2_fp8(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_sparse(const DecodeParams& p, int fp8, int nope, hipStream_t stream);
hipError_t launch_decode_flat_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_nope_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_nope_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_gla2(const DecodeParams& p, int fp8, int num_workgroups, hipStream_t stream);
hipError_t launch_merge_flat(const float* part_out, const float* part_lse, const int64_t* cu, int batch, int heads,
                             int num_workgroups, float* out, float* lse, hipStream_t stream, int width = kLatent);
hipError_t launch_gather(const uint8_t* cache, int fp8, int64_t num_pages, const int32_t* block_table,
                         int64_t bt_stride, const int64_t* cu_rows, const int32_t* seq_starts, int batch,
                         int page_size, int64_t total_rows, uint16_t* out, int32_t* check_status,
                         hipStream_t stream);
hipError_t launch_merge(const float* part_out, const float* part_lse, int num_splits, int batch,
                        int heads, float* out, float* lse, hipStream_t stream, int width = kLatent);
// Merge of the per-request split decode when empty partitions left no partial: request b's
// non-empty partitions are the first ceil(ceil(L_b / page_size) / c) ones, c = ceil(bt_stride /
// num_splits) pages (the partition rule of the decode).
hipError_t launch_merge_counted(const float* part_out, const float* part_lse, int num_splits, int batch,
                                int rows_per_request, int width, const int32_t* seq_lens, int page_size,
                                int64_t bt_stride, float* out, float* lse, hipStream_t stream);
hipError_t launch_cache_write(const uint16_t* latent, const uint16_t* k_pe, const int64_t* slots,
                              int num_tokens, uint8_t* cache, int fp8, hipStream_t stream);

}  // namespace mla

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
  int stream_rows;             // non-temporal row loads (MLA_ROW_LOADS_STREAMING)
};

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

// Batch-balanced mode: at most kMaxBalancedBatch requests; each non-empty request adds
// kSegmentCost positions to the cost axis, and workgroup w of W takes axis positions
// [flat_begin(V, W, w), flat_begin(V, W, w + 1)), V = the axis length.
constexpr int kMaxBalancedBatch = 1024;
constexpr int64_t kSegmentCost = 512;
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
hipError_t launch_decode_flat_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_nope_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_decode_flat_nope_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream);
hipError_t launch_merge_flat(const float* part_out, const float* part_lse, const int64_t* cu, int batch, int heads,
                             int num_workgroups, float* out, float* lse, hipStream_t stream);
hipError_t launch_gather(const uint8_t* cache, int fp8, const int32_t* block_table, int64_t bt_stride,
                         const int64_t* cu_rows, const int32_t* seq_starts, int batch, int page_size,
                         int64_t total_rows, uint16_t* out, hipStream_t stream);
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

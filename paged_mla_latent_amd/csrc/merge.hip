// Log-sum-exp merge of partial decode results (vLLM pull request 55543: partial
// (out, lse) pairs over disjoint token sets combine by log-sum-exp, with (0, -inf)
// as the neutral element of an empty partition).
//
//   M = max_p lse_p;  M = -inf  ->  (0, -inf)
//   w_p = exp(lse_p - M);  lse = M + ln sum_p w_p;  out = sum_p w_p out_p / sum_p w_p
//
// A NaN partial makes the result NaN (as the definition does), also when every other
// partition is empty.
//
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kGroups = 8;    // partial streams per workgroup
constexpr int kCols = 32;     // float4 columns per workgroup (128 output values)

// Merges the `count` partials of one output row (row bh of `out`), partial i at row
// base + i * stride of part_out / part_lse.
__device__ __forceinline__ void merge_row(const float* __restrict__ part_out, const float* __restrict__ part_lse,
                                          int count, int64_t base, int64_t stride, int width, int64_t bh,
                                          float* __restrict__ out, float* __restrict__ lse) {
  __shared__ f32x4 acc_s[kGroups][kCols];
  __shared__ float w_s[kGroups];
  __shared__ float m_s[kGroups * kCols / 64];
  __shared__ float n_s[kGroups * kCols / 64];
  const int col = blockIdx.y * kCols + (threadIdx.x % kCols);
  const int grp = threadIdx.x / kCols;
  // This lane's first kPre partials (rows and LSEs) are requested before M is known: they do
  // not depend on it, so their loads travel with the LSE loads below instead of after them.
  constexpr int kPre = 8;
  const float* src = part_out + base * width + 4 * col;
  f32x4 pre[kPre];
  float pre_lse[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int p = grp + i * kGroups;
    pre[i] = p < count ? *(const f32x4*)(src + (int64_t)p * stride * width) : f32x4{0.f, 0.f, 0.f, 0.f};
    pre_lse[i] = p < count ? part_lse[base + p * stride] : -INFINITY;
  }
  // M = max_p lse_p: every lane loads a strided share (independent loads), then a
  // wave reduction and a reduction over the waves through LDS.
  // fmaxf skips NaN, so NaN partials are counted apart and force M = NaN.
  float M = -INFINITY;
  float nan = 0.f;
  for (int p = threadIdx.x; p < count; p += kGroups * kCols) {
    const float x = part_lse[base + p * stride];
    M = fmaxf(M, x);
    nan = (x != x) ? 1.f : nan;
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    M = fmaxf(M, __shfl_xor(M, mask, 64));
    nan = fmaxf(nan, __shfl_xor(nan, mask, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    m_s[threadIdx.x >> 6] = M;
    n_s[threadIdx.x >> 6] = nan;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kGroups * kCols / 64; ++w) {
    M = fmaxf(M, m_s[w]);
    nan = fmaxf(nan, n_s[w]);
  }
  if (nan != 0.f) M = __builtin_nanf("");
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      if (grp + i * kGroups < count) {
        const float w = __expf(pre_lse[i] - M);
        W += w;
        acc += w * pre[i];
      }
    }
#pragma unroll 4
    for (int p = grp + kPre * kGroups; p < count; p += kGroups) {
      const float w = __expf(part_lse[base + p * stride] - M);
      W += w;
      acc += w * *(const f32x4*)(src + (int64_t)p * stride * width);
    }
  }
  acc_s[grp][threadIdx.x % kCols] = acc;
  if (threadIdx.x % kCols == 0) w_s[grp] = W;
  __syncthreads();
  if (grp != 0) return;
  W = 0.f;
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    W += w_s[g];
    acc += acc_s[g][threadIdx.x];
  }
  if (M != -INFINITY) acc *= 1.0f / W;
  *(f32x4*)(out + bh * width + 4 * col) = acc;
  if (blockIdx.y == 0 && threadIdx.x == 0) lse[bh] = (M == -INFINITY) ? -INFINITY : M + __logf(W);
}

// grid = (batch * heads, width / 128): workgroup (bh, y) merges columns [128y, 128y + 128)
// of row bh (width = 512 for the latent rows, 256 for the rank-256 / GLA-g2 outputs).
// Lane t owns float4 column t % 32 and partials p = t / 32, t / 32 + 8, ...; the eight
// partial streams are then summed through LDS.  Partial p of row bh: row p * rows + bh.
__global__ __launch_bounds__(kGroups * kCols) void merge_kernel(const float* __restrict__ part_out,
                                                               const float* __restrict__ part_lse, int S,
                                                               int64_t rows, int width, float* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  merge_row(part_out, part_lse, S, bh, rows, width, bh, out, lse);
}

// Per-request split decode whose empty partitions wrote nothing: row bh of request b =
// bh / rows_per_request merges partials s = 0 .. n_b - 1 (row s * rows + bh), n_b = the number
// of non-empty partitions of b under the decode's partition rule; n_b = 0 gives (0, -inf).
__global__ __launch_bounds__(kGroups * kCols) void merge_counted_kernel(const float* __restrict__ part_out,
                                                                       const float* __restrict__ part_lse, int S,
                                                                       int64_t rows, int rows_per_request, int width,
                                                                       const int32_t* __restrict__ seq_lens,
                                                                       int page_size, int64_t bt_stride,
                                                                       float* __restrict__ out,
                                                                       float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const int n = counted_partitions(seq_lens[bh / rows_per_request], page_size, bt_stride, S);
  merge_row(part_out, part_lse, n, bh, rows, width, bh, out, lse);
}

// Merge of one output row by one 64-lane wavefront, for rows with few partials: lane l owns
// float4 columns l, l + 64, ... (NV of them: width = 256 NV) of every partial; every lane reads
// the partials' LSEs; partials are taken four at a time with their loads issued together.  No
// LDS, no barrier.  Partial i of the row: row first + i * stride of part_out / part_lse.
constexpr int kRowBatch = 4;
template <int NV>
__device__ __forceinline__ void merge_row_wave(const float* __restrict__ part_out, const float* __restrict__ part_lse,
                                               int count, int64_t first, int64_t stride, int64_t bh,
                                               float* __restrict__ out, float* __restrict__ lse) {
  constexpr int kWidth = 256 * NV;
  const int lane = threadIdx.x & 63;
  // M = max_p lse_p; fmaxf skips NaN, so a NaN partial forces M = NaN.
  float M = -INFINITY;
  bool nan = false;
  for (int p0 = 0; p0 < count; p0 += kRowBatch) {
    float x[kRowBatch];
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) x[i] = p0 + i < count ? part_lse[first + (int64_t)(p0 + i) * stride] : -INFINITY;
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      M = fmaxf(M, x[i]);
      nan = nan || x[i] != x[i];
    }
  }
  if (nan) M = __builtin_nanf("");
  f32x4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int p0 = 0; p0 < count; p0 += kRowBatch) {
      float w[kRowBatch];
      f32x4 val[kRowBatch][NV];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) {
        const bool in = p0 + i < count;
        const int64_t row = first + (int64_t)(in ? p0 + i : p0) * stride;  // a valid row either way
        const f32x4* src = (const f32x4*)(part_out + row * kWidth) + lane;
        w[i] = in ? part_lse[row] : -INFINITY;
#pragma unroll
        for (int v = 0; v < NV; ++v) val[i][v] = src[64 * v];
      }
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) {
        if (p0 + i >= count) continue;
        const float e = __expf(w[i] - M);
        wsum += e;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += e * val[i][v];
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] *= 1.0f / wsum;
  }
  f32x4* dst = (f32x4*)(out + bh * kWidth) + lane;
#pragma unroll
  for (int v = 0; v < NV; ++v) dst[64 * v] = acc[v];
  if (lane == 0) lse[bh] = (M == -INFINITY) ? -INFINITY : M + __logf(wsum);
}

// Per-request merges with at most kFewSplits partials per row: one row per 64-lane workgroup
// (merge_row_wave); counted (empty partitions wrote nothing) or all S partials.
constexpr int kFewSplits = 16;
template <int NV, bool kCounted>
__global__ __launch_bounds__(64) void merge_few_kernel(const float* __restrict__ part_out,
                                                       const float* __restrict__ part_lse, int S, int64_t rows,
                                                       int rows_per_request, const int32_t* __restrict__ seq_lens,
                                                       int page_size, int64_t bt_stride, float* __restrict__ out,
                                                       float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  int n = S;
  if constexpr (kCounted) n = counted_partitions(seq_lens[bh / rows_per_request], page_size, bt_stride, S);
  merge_row_wave<NV>(part_out, part_lse, n, bh, rows, bh, out, lse);
}

// Batch-balanced mode: request b's partials are the slots b + w for the workgroups w whose
// cost-axis ranges meet [cu[b], cu[b + 1]) (the axis the decode stored); row h of slot q is row
// q * heads + h.  A request has one or two partials here (a handful for the longest): one row
// per 64-lane workgroup (merge_row_wave).
template <int NV>
__global__ __launch_bounds__(64) void merge_flat_kernel(const float* __restrict__ part_out,
                                                        const float* __restrict__ part_lse,
                                                        const int64_t* __restrict__ cu, int batch, int heads,
                                                        int num_workgroups, float* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / heads), h = (int)(bh % heads);
  const int64_t N = cu[batch], c0 = cu[b], c1 = cu[b + 1];
  const int64_t W = min((int64_t)num_workgroups, N);  // the workgroups that took part
  int count = 0;
  int64_t first = 0;
  if (c1 > c0) {
    // The workgroup whose range holds axis position x < N: the largest w with
    // floor(w N / W) <= x, i.e. w N < (x + 1) W, i.e. w = floor(((x + 1) W - 1) / N).
    // (x + 1) W < 2^41 * 2^16 fits in 64 bits.
    auto owner = [&](int64_t x) -> int64_t { return ((x + 1) * W - 1) / N; };
    const int64_t w0 = owner(c0), w1 = owner(c1 - 1);
    first = ((int64_t)b + w0) * heads + h;
    count = (int)(w1 - w0 + 1);
  }
  merge_row_wave<NV>(part_out, part_lse, count, first, heads, bh, out, lse);
}

template <bool kCounted>
hipError_t launch_few(const float* part_out, const float* part_lse, int S, int64_t rows, int rows_per_request,
                      int width, const int32_t* seq_lens, int page_size, int64_t bt_stride, float* out, float* lse,
                      hipStream_t stream) {
  const dim3 grid((unsigned)rows), block(64);
  switch (width) {
    case 256:
      hipLaunchKernelGGL((merge_few_kernel<1, kCounted>), grid, block, 0, stream, part_out, part_lse, S, rows,
                         rows_per_request, seq_lens, page_size, bt_stride, out, lse);
      break;
    case 768:
      hipLaunchKernelGGL((merge_few_kernel<3, kCounted>), grid, block, 0, stream, part_out, part_lse, S, rows,
                         rows_per_request, seq_lens, page_size, bt_stride, out, lse);
      break;
    case 1792:
      hipLaunchKernelGGL((merge_few_kernel<7, kCounted>), grid, block, 0, stream, part_out, part_lse, S, rows,
                         rows_per_request, seq_lens, page_size, bt_stride, out, lse);
      break;
    default:
      hipLaunchKernelGGL((merge_few_kernel<2, kCounted>), grid, block, 0, stream, part_out, part_lse, S, rows,
                         rows_per_request, seq_lens, page_size, bt_stride, out, lse);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_flat(const float* part_out, const float* part_lse, const int64_t* cu, int batch, int heads,
                             int num_workgroups, float* out, float* lse, hipStream_t stream, int width) {
  const int64_t rows = (int64_t)batch * heads;
  if (width == 256)
    hipLaunchKernelGGL(merge_flat_kernel<1>, dim3((unsigned)rows), dim3(64), 0, stream, part_out, part_lse, cu, batch,
                       heads, num_workgroups, out, lse);
  else
    hipLaunchKernelGGL(merge_flat_kernel<kLatent / 256>, dim3((unsigned)rows), dim3(64), 0, stream, part_out, part_lse,
                       cu, batch, heads, num_workgroups, out, lse);
  return hipGetLastError();
}

hipError_t launch_merge_counted(const float* part_out, const float* part_lse, int num_splits, int batch,
                                int rows_per_request, int width, const int32_t* seq_lens, int page_size,
                                int64_t bt_stride, float* out, float* lse, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * rows_per_request;
  if (num_splits <= kFewSplits)
    return launch_few<true>(part_out, part_lse, num_splits, rows, rows_per_request, width, seq_lens, page_size,
                            bt_stride, out, lse, stream);
  hipLaunchKernelGGL(merge_counted_kernel, dim3((unsigned)rows, (unsigned)(width / (4 * kCols))),
                     dim3(kGroups * kCols), 0, stream, part_out, part_lse, num_splits, rows, rows_per_request, width,
                     seq_lens, page_size, bt_stride, out, lse);
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_out, const float* part_lse, int num_splits, int batch,
                        int heads, float* out, float* lse, hipStream_t stream, int width) {
  const int64_t rows = (int64_t)batch * heads;
  if (num_splits <= kFewSplits)
    return launch_few<false>(part_out, part_lse, num_splits, rows, 1, width, nullptr, 1, 1, out, lse, stream);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows, (unsigned)(width / (4 * kCols))), dim3(kGroups * kCols), 0,
                     stream, part_out, part_lse, num_splits, rows, width, out, lse);
  return hipGetLastError();
}

}  // namespace mla

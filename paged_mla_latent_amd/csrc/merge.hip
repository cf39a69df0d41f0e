// Log-sum-exp merge of partial decode results (vLLM pull request 55543: partial
// (out, lse) pairs over disjoint token sets combine by log-sum-exp, with (0, -inf)
// as the neutral element of an empty partition).
//
//   M = max_p lse_p;  M = -inf  ->  (0, -inf)
//   w_p = exp(lse_p - M);  lse = M + ln sum_p w_p;  out = sum_p w_p out_p / sum_p w_p
//
// One workgroup of 128 lanes per (request, head); each lane owns 4 of the 512
// latent columns, so every partial row is read once with 16-byte loads.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_out,
                                                    const float* __restrict__ part_lse, int S,
                                                    int64_t rows, float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  float M = -INFINITY;
  for (int p = 0; p < S; ++p) M = fmaxf(M, part_lse[p * rows + bh]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  if (M != -INFINITY) {
    const float* src = part_out + bh * kLatent + 4 * t;
    int p = 0;
    for (; p + 4 <= S; p += 4) {
      float w[4];
      f32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = __expf(part_lse[(p + i) * rows + bh] - M);
        v[i] = *(const f32x4*)(src + (int64_t)(p + i) * rows * kLatent);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        W += w[i];
        acc += w[i] * v[i];
      }
    }
    for (; p < S; ++p) {
      const float w = __expf(part_lse[p * rows + bh] - M);
      W += w;
      acc += w * *(const f32x4*)(src + (int64_t)p * rows * kLatent);
    }
    acc *= 1.0f / W;
  }
  *(f32x4*)(out + bh * kLatent + 4 * t) = acc;
  if (t == 0) lse[bh] = (M == -INFINITY) ? -INFINITY : M + __logf(W);
}

}  // namespace

hipError_t launch_merge(const float* part_out, const float* part_lse, int num_splits, int batch,
                        int heads, float* out, float* lse, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * heads;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows), dim3(128), 0, stream, part_out, part_lse,
                     num_splits, rows, out, lse);
  return hipGetLastError();
}

}  // namespace mla

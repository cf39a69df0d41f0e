// Cache write: the row of each new token, latent[512] ++ k_pe[64], goes to its slot
// (vLLM pull request 55543: the cache-write step concatenates the latent and the
// 64-wide rotary key into the 576-wide / 656-byte row).
//
// One wavefront per token; the row encodings (bf16 copy, fp8 block quantisation) are those of
// cache_rows.h.  Byte offsets are slot * row_bytes in 64-bit arithmetic.  A token's inputs are
// requested before its slot is known (the slot only decides whether and where the row goes), so
// the two loads travel together.
#include "cache_rows.h"
#include "mla_internal.h"

namespace mla {
namespace {

template <bool kFp8>
__device__ __forceinline__ void write_token(const uint16_t* __restrict__ latent, const uint16_t* __restrict__ k_pe,
                                            const int64_t* __restrict__ slots, int T, uint8_t* __restrict__ cache) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= T) return;
  const RowIn in = load_row(latent + (int64_t)tok * kLatent, k_pe == nullptr ? nullptr : k_pe + (int64_t)tok * kRope,
                            lane);
  const int64_t slot = slots[tok];
  if (slot < 0) return;
  if constexpr (kFp8) {
    store_row_fp8(in, cache + slot * (int64_t)kRowBytesFp8, lane);
  } else {
    store_row_bf16(in, cache + slot * (int64_t)kRowBytesBf16, lane);
  }
}

__global__ __launch_bounds__(256) void cache_write_bf16(const uint16_t* __restrict__ latent,
                                                        const uint16_t* __restrict__ k_pe,
                                                        const int64_t* __restrict__ slots, int T,
                                                        uint8_t* __restrict__ cache) {
  write_token<false>(latent, k_pe, slots, T, cache);
}

__global__ __launch_bounds__(256) void cache_write_fp8(const uint16_t* __restrict__ latent,
                                                       const uint16_t* __restrict__ k_pe,
                                                       const int64_t* __restrict__ slots, int T,
                                                       uint8_t* __restrict__ cache) {
  write_token<true>(latent, k_pe, slots, T, cache);
}

}  // namespace

hipError_t launch_cache_write(const uint16_t* latent, const uint16_t* k_pe, const int64_t* slots,
                              int num_tokens, uint8_t* cache, int fp8, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((num_tokens + 3) / 4));
  if (fp8)
    hipLaunchKernelGGL(cache_write_fp8, grid, dim3(256), 0, stream, latent, k_pe, slots, num_tokens, cache);
  else
    hipLaunchKernelGGL(cache_write_bf16, grid, dim3(256), 0, stream, latent, k_pe, slots, num_tokens, cache);
  return hipGetLastError();
}

}  // namespace mla

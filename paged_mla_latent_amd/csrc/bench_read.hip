// Streaming-read reference kernel of libmla_bench.so (a measurement helper, not part of the
// decode path): every 16-byte word of a buffer read once, workgroup w reading the contiguous
// range [w * per, (w + 1) * per) of words, four loads in flight per thread, the words XORed so
// that no load is dead.  Contiguous ranges per workgroup read faster than a grid-stride walk
// on MI355X (2 GiB, non-temporal: about 7.0 TB/s against 6.2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 4;

template <bool kNonTemporal>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (kNonTemporal) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool kNonTemporal>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf, uint64_t words,
                                                               uint64_t per, uint32_t* __restrict__ sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * per;
  const uint64_t end = begin + per < words ? begin + per : words;
  uint64_t i = begin + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = load16<kNonTemporal>(buf + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
  }
  for (; i < end; i += kThreads) acc ^= load16<kNonTemporal>(buf + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if ((threadIdx.x & 63) == 0) sink[4 * blockIdx.x + (threadIdx.x >> 6)] = x;
}

}  // namespace

extern "C" int mla_bench_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t num_workgroups,
                                     int32_t nontemporal, void* stream) {
  if (buf == nullptr || sink == nullptr) return 1;
  if (bytes < 16 || bytes % 16 != 0 || num_workgroups < 1 || num_workgroups > 65535) return 2;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return 3;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  const uint64_t words = bytes / 16;
  const uint64_t per = (words + num_workgroups - 1) / num_workgroups;  // trailing workgroups may get none
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(num_workgroups), dim3(kThreads), 0, s, p, words, per, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(num_workgroups), dim3(kThreads), 0, s, p, words, per, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

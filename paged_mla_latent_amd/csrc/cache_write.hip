// Cache write: the row of each new token, latent[512] ++ k_pe[64], goes to its slot
// (vLLM pull request 55543: the cache-write step concatenates the latent and the
// 64-wide rotary key into the 576-wide / 656-byte row).
//
// One wavefront per token.  Byte offsets are slot * row_bytes in 64-bit arithmetic.
//  bf16: 1152 bytes copied bit for bit (64 lanes x 16 B latent, 8 lanes x 16 B rope).
//  fp8 (656 bytes): lane l owns latent values 8l..8l+7; the 16 lanes of block k = l/16
//    reduce a = max|x| (fp32, exact), s = a / 448 (IEEE division), each code is
//    e4m3fn(x / s) rounded to nearest-even.  The quotient is clamped to +-448 before
//    the hardware conversion, which rounds to nearest-even but does not saturate; a
//    block with a == 0 stores s = 0 and zero codes.  A block holding a NaN or an infinity
//    stores the NaN scale 0x7FC00000 and the NaN code 0x7F for all 128 values, so that it
//    decodes to NaN (a quotient by an infinite or NaN scale would otherwise turn into
//    plausible finite codes).  Bytes: [0,512) codes, [512,528) scales (little-endian fp32),
//    [528,656) k_pe as bf16.
// k_pe == nullptr (a NoPE layer): the rope part is written as zeros.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// 16 bytes (8 bf16 values) of token tok's rope part for lane < 8; zeros without k_pe.
__device__ __forceinline__ u32x4 rope16(const uint16_t* __restrict__ k_pe, int tok, int lane) {
  if (k_pe == nullptr) return u32x4{0u, 0u, 0u, 0u};
  return *(const u32x4*)(k_pe + (int64_t)tok * kRope + 8 * lane);
}

__global__ __launch_bounds__(256) void cache_write_bf16(const uint16_t* __restrict__ latent,
                                                        const uint16_t* __restrict__ k_pe,
                                                        const int64_t* __restrict__ slots, int T,
                                                        uint8_t* __restrict__ cache) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= T) return;
  const int64_t slot = slots[tok];
  if (slot < 0) return;
  uint8_t* row = cache + slot * (int64_t)kRowBytesBf16;
  // Whole 128-byte lines in and out, each touched once: non-temporal both ways.
  __builtin_nontemporal_store(__builtin_nontemporal_load((const u32x4*)(latent + (int64_t)tok * kLatent + 8 * lane)),
                              (u32x4*)(row + 16 * lane));
  if (lane < 8) __builtin_nontemporal_store(rope16(k_pe, tok, lane), (u32x4*)(row + 1024 + 16 * lane));
}

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__global__ __launch_bounds__(256) void cache_write_fp8(const uint16_t* __restrict__ latent,
                                                       const uint16_t* __restrict__ k_pe,
                                                       const int64_t* __restrict__ slots, int T,
                                                       uint8_t* __restrict__ cache) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= T) return;
  const int64_t slot = slots[tok];
  if (slot < 0) return;
  uint8_t* row = cache + slot * (int64_t)kRowBytesFp8;

  const u32x4 raw = *(const u32x4*)(latent + (int64_t)tok * kLatent + 8 * lane);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_float(raw[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_float(raw[i] >> 16);
  }
  float a = 0.f;
  int nonfinite = 0;  // a NaN or an infinity among this lane's values
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a = fmaxf(a, fabsf(x[i]));
    nonfinite |= (raw[i / 2] >> (16 * (i & 1)) & 0x7F80u) == 0x7F80u ? 1 : 0;  // exponent all ones
  }
#pragma unroll
  for (int mask = 8; mask >= 1; mask >>= 1) {
    a = fmaxf(a, __shfl_xor(a, mask, 64));
    nonfinite |= __shfl_xor(nonfinite, mask, 64);
  }
  float s = a / 448.0f;
  u32x2 codes = {0u, 0u};
  if (nonfinite) {
    s = __uint_as_float(0x7FC00000u);
    codes = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
  } else if (s != 0.f) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[i] / s, -448.0f), 448.0f);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w], y[4 * w + 1], 0, false);
      codes[w] = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w + 2], y[4 * w + 3], v, true);
    }
  }
  *(u32x2*)(row + 8 * lane) = codes;
  if ((lane & 15) == 0) *(float*)(row + 512 + 4 * (lane >> 4)) = s;
  if (lane < 8) *(u32x4*)(row + 528 + 16 * lane) = rope16(k_pe, tok, lane);
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

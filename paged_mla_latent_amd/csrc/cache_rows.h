// Encoding of one token's cache row, shared by the cache-write kernels and the decodes that
// append the step's new rows themselves (vLLM pull request 55543: the cache-write step
// concatenates the latent and the 64-wide rotary key into the 576-value / 656-byte row).
//
// One wavefront handles one row.  Lane l holds latent values 8l .. 8l + 7 and, for l < 8, rope
// values 8l .. 8l + 7 (RowIn, loaded by load_row); store_row_* writes the row's bytes at the
// row's address (64-bit slot * row bytes, formed by the caller).
//  bf16 (1,152 bytes): latent ++ k_pe, bit for bit.
//  fp8 (656 bytes): the 16 lanes of block k = l / 16 reduce a = max|x| (fp32, exact),
//    s = a / 448 (IEEE division), each code is e4m3fn(x / s) rounded to nearest-even.  The
//    quotient is clamped to +-448 before the hardware conversion, which rounds to nearest-even
//    but does not saturate; a block with a == 0 stores s = 0 and zero codes.  A block holding a
//    NaN or an infinity stores the NaN scale 0x7FC00000 and the NaN code 0x7F for all 128
//    values, so that it decodes to NaN (a quotient by an infinite or NaN scale would otherwise
//    turn into plausible finite codes).  Bytes: [0,512) codes, [512,528) scales (little-endian
//    fp32), [528,656) k_pe as bf16.
// k_pe == nullptr (a NoPE layer): the rope part is written as zeros.
#pragma once

#include "mla_device.h"

namespace mla {

struct RowIn {
  u32x4 lat;   // latent values 8l .. 8l + 7 (bf16 bits)
  u32x4 rope;  // lanes l < 8: rope values 8l .. 8l + 7; zeros without k_pe
};

// The inputs of one row: latent_row bf16 [512], k_pe_row bf16 [64] or nullptr.  Both are read
// once, as whole 128-byte lines: non-temporal.
__device__ __forceinline__ RowIn load_row(const uint16_t* __restrict__ latent_row, const uint16_t* __restrict__ k_pe_row,
                                          int lane) {
  RowIn in;
  in.lat = __builtin_nontemporal_load((const u32x4*)(latent_row + 8 * lane));
  in.rope = u32x4{0u, 0u, 0u, 0u};
  if (k_pe_row != nullptr && lane < 8) in.rope = *(const u32x4*)(k_pe_row + 8 * lane);
  return in;
}

// bf16 row: whole 128-byte lines out, each written once: non-temporal.
__device__ __forceinline__ void store_row_bf16(const RowIn& in, uint8_t* __restrict__ row, int lane) {
  __builtin_nontemporal_store(in.lat, (u32x4*)(row + 16 * lane));
  if (lane < 8) __builtin_nontemporal_store(in.rope, (u32x4*)(row + 1024 + 16 * lane));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp8 row (the block quantisation above).
__device__ __forceinline__ void store_row_fp8(const RowIn& in, uint8_t* __restrict__ row, int lane) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_float(in.lat[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_float(in.lat[i] >> 16);
  }
  float a = 0.f;
  int nonfinite = 0;  // a NaN or an infinity among this lane's values
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a = fmaxf(a, fabsf(x[i]));
    nonfinite |= (in.lat[i / 2] >> (16 * (i & 1)) & 0x7F80u) == 0x7F80u ? 1 : 0;  // exponent all ones
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
  if (lane < 8) *(u32x4*)(row + 528 + 16 * lane) = in.rope;
}

}  // namespace mla

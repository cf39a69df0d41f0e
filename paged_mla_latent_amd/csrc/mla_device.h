// Device-side helpers shared by the gfx950 kernels of libmla.
//
// Lane layouts used below (CDNA4 matrix cores, 64-lane wavefronts):
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[l%16][8*(l/16) + 0..7]
//                             B: lane l holds B[8*(l/16) + 0..7][l%16]
//                             D: lane l holds D[4*(l/16) + 0..3][l%16]
//   v_mfma_f32_16x16x16_bf16  same with 4 K values per lane: A[l%16][4*(l/16) + 0..3]
//   ds_read_b64_tr_b16        within each group of 16 lanes, output lane i gets
//                             element (i & 3) of the 4-element chunks addressed by
//                             lanes (i >> 2) + 4*v, v = 0..3
//   ds_read_b64_tr_b8         within each group of 16 lanes, output lane i gets byte
//                             (i & 7) of the 8-byte chunks addressed by lanes
//                             (i >> 3) + 2*v, v = 0..7 (byte v of the result)
//   global_load_lds (16 B)    lane l writes LDS[base + 16*l]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kRow = kLatent + kRope;  // 576 values
constexpr int kRowBytesBf16 = 2 * kRow;  // 1152
constexpr int kRowBytesFp8 = 656;        // 512 codes + 16 scale bytes + 128 rope bytes
constexpr int kMaxHeads = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// Wait until at most N vector-memory operations of this wave are outstanding.
// The "memory" clobber keeps LDS reads of DMA'd data below the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS void*)p;
}

// 16-byte global -> LDS copy (global_load_lds_dwordx4); lane l lands at lds_addr + 16 * l.
// lds_addr must be wave-uniform.  Written as inline assembly so that the compiler does
// not treat every later LDS read as a possible reader of this DMA and wait for it:
// completion is tracked explicitly with wait_vmcnt<>() before the data is read.  The
// compiler's own vmcnt waits stay correct because these loads only add younger
// entries to the in-order vector-memory counter.  M0 is written here; on gfx950 the
// compiler does not keep values in M0 across code that uses no M0-based instruction.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_addr)
               : "memory");
}

// The same copy with the non-temporal hint (streaming data, read once): measured on this part
// at 6.8 TB/s against 6.1 TB/s without it when every instruction reads whole 128-byte lines,
// and slower than without it when an instruction reads only half of each line it touches
// (the other half then comes from HBM again instead of the L2).
__device__ __forceinline__ void dma16_nt(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gsrc), "s"(lds_addr)
               : "memory");
}

// 4-byte global -> LDS copy (global_load_lds_dword); lane l lands at lds_addr + 4 * l.
__device__ __forceinline__ void dma4(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(lds_addr)
               : "memory");
}

// Softmax rescale of the output accumulators, O *= alpha, for a rare wave-uniform branch (the
// running maximum settles early).  Every accumulator is pinned to the matrix-core registers
// (AGPRs) before and after by empty volatile asm, which also keeps the branch from being
// executed speculatively.  Without the pin the compiler carries O around the tile loop in ordinary
// VGPRs, where the multiply happens, and copies all of it into AGPRs and back around every
// batch of MFMAs; executed unconditionally with alpha = 1 the multiply would cost 128 VALU
// instructions per tile.
template <int N>
__device__ __forceinline__ void scale_acc(f32x4 (&O)[N], float alpha) {
#pragma unroll
  for (int u = 0; u < N; ++u) asm volatile("" : "+a"(O[u]));  // the copies out stay in the branch
#pragma unroll
  for (int u = 0; u < N; ++u) O[u] *= alpha;
#pragma unroll
  for (int u = 0; u < N; ++u) asm volatile("" : "+a"(O[u]));
}

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr8(const void* lds_addr) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)lds_addr);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)lds_addr);
  return __builtin_bit_cast(u32x2, v);
}

// Two floats -> packed bf16 pair (round to nearest even), lo in bits [15:0].
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Values of lane l and lane l ^ 16 (row swap within 32-lane halves), and of lane l and
// lane l ^ 32, via the gfx950 permlane swaps (VALU, no LDS round trip).  Each returns the
// pair; callers combine the two symmetrically.
__device__ __forceinline__ f32x2 pair_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 pair_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float max_over_rows(float v) {
  f32x2 a = pair_xor16(v);
  v = fmaxf(a[0], a[1]);
  a = pair_xor32(v);
  return fmaxf(a[0], a[1]);
}
__device__ __forceinline__ float sum_over_rows(float v) {
  f32x2 a = pair_xor16(v);
  v = a[0] + a[1];
  a = pair_xor32(v);
  return a[0] + a[1];
}

// ------------------------------------------------------------------------------------
// Chunk layout of a tile in LDS (rank-768 rows, and the bf16 tiles that fp8 tiles are
// widened into for the multi-token loop).  A tile is 16 tokens x C chunks of 16 bytes (C = 72
// for a 576-value bf16 row).  DMA instruction j fills
// chunk positions 64j .. 64j+63, lane L landing at 64j + L; lane L = 4t + v fetches chunk
// 4j + (v ^ h(t)) of token t, so each group of four lanes reads 64 contiguous bytes of one
// row (the coalesced form: four lanes per row segment measured 6% faster than one lane per
// row).  Chunk c of token t therefore sits at
//     P(t, c) = 64 * (c >> 2) + 4 * t + ((c & 3) ^ h(t)),   h(t) = bit-swap of t >> 2,
// and both read patterns are bank-conflict free: the QK reads (one chunk of all 16 tokens:
// 4 * (t & 3) + ((c & 3) ^ h(t)) covers 16 banks groups) and the transposing PV reads (8
// tokens x 2 adjacent chunks per 32 lanes: tokens t and t + 4 use opposite chunk pairs).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ int swz(int t) { return (((t >> 2) & 1) << 1) | ((t >> 3) & 1); }
__device__ __forceinline__ int chunk_pos(int t, int c) { return 64 * (c >> 2) + 4 * t + ((c & 3) ^ swz(t)); }

// ------------------------------------------------------------------------------------
// Line layout of a bf16 tile (rows whose byte length is a multiple of 128).  DMA instruction
// j reads line j >> 1 (chunks 8 (j >> 1) .. + 7) of tokens 8 (j & 1) .. + 7: lane L = 8 t' + v
// fetches chunk 8 (j >> 1) + (v ^ s(t')) of token 8 (j & 1) + t', so every instruction reads
// eight whole 128-byte lines (the form the non-temporal hint needs).  Chunk c of token t sits at
//     Q(t, c) = 64 (2 (c >> 3) + (t >> 3)) + 8 (t & 7) + ((c & 7) ^ s(t & 7)),
//     s(t) = 2 (t & 3) + ((t >> 2) & 1)   (a permutation of 0 .. 7),
// and chunks c and c + 8a of a token lie 128a positions (2,048a bytes) apart.  QK reads (one
// chunk of tokens 0 .. 7, then of 8 .. 15) meet eight distinct 16-byte bank groups since s is a
// permutation; the transposing PV reads of 16 lanes (tokens 4i .. 4i + 3, two adjacent chunks
// 2r, 2r + 1 each) meet eight distinct ones since s(t) >> 1 differs across any four tokens 4i ..
// 4i + 3.  (LDS probe, 4 waves: 118-121 B/clk for the QK pattern, 89-97 for the PV pattern.)
// ------------------------------------------------------------------------------------
__device__ __forceinline__ int line_swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ int line_pos(int t, int c) {
  return 64 * (2 * (c >> 3) + (t >> 3)) + 8 * (t & 7) + ((c & 7) ^ line_swz(t & 7));
}

}  // namespace mla

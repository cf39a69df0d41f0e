// Context gather for prefill: cached rows of each request, read through the block table
// with 64-bit slot and byte offsets (sabi-mla-vllm, "B300 fix (0.2.0)": prefill gathers the
// cache with int64 indices), written as contiguous 576-value bf16 rows (vLLM pull request
// 55543, commit on the context-gather path: 656-byte rows read into a workspace 576 wide).
//
//   output row cu_rows[b] + j  =  token seq_starts[b] + j of request b
//   bf16 cache: the row as stored;  fp8 cache: latent value bf16(fl32(code * scale)),
//   rope values as stored.
//
// A wavefront copies a few consecutive output rows (4 bf16 / 8 fp8 rows, about 5 KB): its
// first lanes resolve the source of one row each (request by binary search over cu_rows,
// page, 64-bit byte offset), then the rows stream through the whole wavefront, every row's
// loads issued before the first store.  Few rows per wavefront keep many wavefronts in
// flight per compute unit, so the lookups of some overlap the copies of others (32 rows per
// wavefront, eight in flight, ran 13 % (bf16) and 19 % (fp8) slower on MI355X).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// Rows per wavefront (one row address per lane below it), all in flight at once.
template <bool kFp8>
constexpr int kRowsPerWave = kFp8 ? 8 : 4;
constexpr int kWavesPerGroup = 4;

template <bool kFp8>
__global__ __launch_bounds__(kWavesPerGroup * 64, 4) void gather_kernel(const uint8_t* __restrict__ cache,
                                                                     const int32_t* __restrict__ block_table,
                                                                     int64_t bt_stride,
                                                                     const int64_t* __restrict__ cu_rows,
                                                                     const int32_t* __restrict__ seq_starts,
                                                                     int batch, int page_size, int64_t total_rows,
                                                                     uint16_t* __restrict__ out, int64_t num_pages,
                                                                     int32_t* check_status) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  constexpr int kRows = kRowsPerWave<kFp8>;
  const int64_t r0 = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * kRows;
  if (r0 >= total_rows) return;
  constexpr int kRowBytes = kFp8 ? kRowBytesFp8 : kRowBytesBf16;

  // Lane j < kRows resolves row r0 + j: its request (binary search over cu_rows; every lane
  // runs the same number of steps), token, page and byte offset, all in 64-bit.  The
  // lookups of the wavefront's rows run in parallel instead of one dependent chain per row.
  constexpr int64_t kZeroRow = -2;  // checked build: a token past the block table, written as zeros
  int64_t my_off = -1;
  uint32_t bad = 0;  // checked build: MLA_CHECK_* bits of this lane's row
  {
    const int64_t r = r0 + lane;
    if (lane < kRows && r < total_rows) {
      int lo = 0, hi = batch;  // invariant: cu_rows[lo] <= r < cu_rows[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_rows[mid] <= r) lo = mid; else hi = mid;
      }
      const int64_t t = (seq_starts ? (int64_t)seq_starts[lo] : 0) + (r - cu_rows[lo]);
      if (kChecked && !len_in_table(t + 1, bt_stride, page_size)) {
        bad |= kCheckSeqLen;
        my_off = kZeroRow;
      } else {
        const int64_t page = checked_page(block_table[(int64_t)lo * bt_stride + t / page_size], num_pages, bad);
        my_off = (page * page_size + t % page_size) * (int64_t)kRowBytes;
      }
    }
  }
  report_checks(bad, check_status);
  auto row_off = [&](int j) -> int64_t {  // wave-uniform offset of row r0 + j (-1: none)
    const uint32_t lo32 = __builtin_amdgcn_readlane((uint32_t)my_off, j);
    const uint32_t hi32 = __builtin_amdgcn_readlane((uint32_t)((uint64_t)my_off >> 32), j);
    return (int64_t)(((uint64_t)hi32 << 32) | lo32);
  };

  {
    int64_t off[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) off[i] = row_off(i);
    if constexpr (kChecked) {
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (off[i] != kZeroRow) continue;
        uint16_t* o = out + (r0 + i) * kRow;
        *(u32x4*)(o + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
        if (lane < 8) *(u32x4*)(o + kLatent + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (!kFp8) {
      u32x4 lat[kRows], pe[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (off[i] < 0) continue;
        lat[i] = __builtin_nontemporal_load((const u32x4*)(cache + off[i] + 16 * lane));
        if (lane < 8) pe[i] = __builtin_nontemporal_load((const u32x4*)(cache + off[i] + 1024 + 16 * lane));
      }
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (off[i] < 0) continue;
        uint16_t* o = out + (r0 + i) * kRow;
        __builtin_nontemporal_store(lat[i], (u32x4*)(o + 8 * lane));
        if (lane < 8) __builtin_nontemporal_store(pe[i], (u32x4*)(o + kLatent + 8 * lane));
      }
    } else {
      // lane l: codes 8l .. 8l+7 of block l / 16; lanes 0..7: 16 rope bytes each.
      u32x2 codes[kRows];
      float scale[kRows];
      u32x4 pe[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (off[i] < 0) continue;
        codes[i] = *(const u32x2*)(cache + off[i] + 8 * lane);
        scale[i] = *(const float*)(cache + off[i] + 512 + 4 * (lane >> 4));
        if (lane < 8) pe[i] = *(const u32x4*)(cache + off[i] + 528 + 16 * lane);
      }
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (off[i] < 0) continue;
        float v[8];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes[i][w], 1.0f, false);  // exact
          const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes[i][w], 1.0f, true);
          v[4 * w + 0] = a[0] * scale[i];  // IEEE float32 multiply
          v[4 * w + 1] = a[1] * scale[i];
          v[4 * w + 2] = c[0] * scale[i];
          v[4 * w + 3] = c[1] * scale[i];
        }
        const u32x4 packed = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                              pack_bf16(v[6], v[7])};
        uint16_t* o = out + (r0 + i) * kRow;
        __builtin_nontemporal_store(packed, (u32x4*)(o + 8 * lane));
        if (lane < 8) __builtin_nontemporal_store(pe[i], (u32x4*)(o + kLatent + 8 * lane));
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* cache, int fp8, int64_t num_pages, const int32_t* block_table,
                         int64_t bt_stride, const int64_t* cu_rows, const int32_t* seq_starts, int batch,
                         int page_size, int64_t total_rows, uint16_t* out, int32_t* check_status,
                         hipStream_t stream) {
  if (total_rows == 0) return hipSuccess;
  const int64_t rows_per_group = (int64_t)(fp8 ? kRowsPerWave<true> : kRowsPerWave<false>) * kWavesPerGroup;
  const dim3 grid((unsigned)((total_rows + rows_per_group - 1) / rows_per_group));
  if (fp8)
    hipLaunchKernelGGL(gather_kernel<true>, grid, dim3(kWavesPerGroup * 64), 0, stream, cache, block_table,
                       bt_stride, cu_rows, seq_starts, batch, page_size, total_rows, out, num_pages,
                       check_status);
  else
    hipLaunchKernelGGL(gather_kernel<false>, grid, dim3(kWavesPerGroup * 64), 0, stream, cache, block_table,
                       bt_stride, cu_rows, seq_starts, batch, page_size, total_rows, out, num_pages,
                       check_status);
  return hipGetLastError();
}

}  // namespace mla

// Paged MLA latent decode kernels for gfx950 (bf16 1152-byte rows and fp8 656-byte rows).
//
// What is computed (sabi-mla-vllm, opening paragraph; vLLM pull request 55543,
// review of the equivalence test): for request b and head h,
//   s_t = scale * <q[b,h,0:576], row_t[0:576]> over the tokens t of the context,
//   out[b,h] = sum_t softmax(s)_t * row_t[0:512],  lse[b,h] = ln sum_t exp(s_t),
// with row_t reached through the block table in 64-bit byte offsets (sabi-mla-vllm,
// "B300 fix (0.2.0)").  Long contexts are cut into page-aligned partitions that each
// return (out, lse); a merge kernel combines them by log-sum-exp.
//
// Mapping onto CDNA4:
//  * grid = (partition, request); 4 waves per workgroup; each wave streams its own
//    16-token tiles (tiles wave, wave+4, ...) and keeps its own online-softmax state,
//    so the main loop has no workgroup barrier.  The 4 states merge through LDS at
//    the end.
//  * Rows go HBM -> LDS with 16-byte direct-to-LDS loads (no VGPR round trip), double
//    buffered per wave; the page lookup for tile k+1 is issued before tile k's loads
//    so that issuing k+1 never waits for k's data.
//  * All 16 heads share every row, so QK^T is a real 16 x 16 x 576 contraction per
//    tile (v_mfma_f32_16x16x32_bf16, rows as A, q^T as B) and PV a 512 x 16 x 16 one
//    (v_mfma_f32_16x16x16_bf16, rows^T as A via ds_read_b64_tr_b16, P^T as B).  The
//    QK output layout (lane = head, 4 tokens per lane) is exactly PV's B operand.
//  * Online softmax in the log2 domain with a lazy rescale: the running max moves
//    only when a tile's max exceeds it by more than 8, so probabilities stay <= 2^8
//    and the 128-register accumulator is rescaled a handful of times per partition.
//  * fp8 rows: codes widen to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1);
//    each 128-value block's scale multiplies that block's partial score (fp32) and is
//    folded into P for that block's PV, so no dequantised value is ever rounded.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;

struct Range {
  int64_t t0, t1;
};

// Partition s of a request of L tokens: whole pages, ceil(P / S) pages per partition.
__device__ __forceinline__ Range partition(int64_t L, int ps, int S, int s) {
  const int64_t P = (L + ps - 1) / ps;
  int64_t c = (P + S - 1) / S;
  if (c < 1) c = 1;
  const int64_t p0 = min(P, (int64_t)s * c);
  const int64_t p1 = min(P, (int64_t)(s + 1) * c);
  return {min(L, p0 * ps), min(L, p1 * ps)};
}

// ------------------------------------------------------------------------------------
// bf16 rows: a tile is 16 tokens x 72 chunks of 16 bytes.  Chunk c of token t sits at
// chunk position 16*c + (t ^ 8*(c & 1)).  QK reads (fixed c, all 16 tokens) and the
// transposing PV reads (8 tokens x 2 chunks per 32 lanes) are both bank-conflict free,
// and DMA instruction j (positions 64j..64j+63) makes lane L fetch chunk 4j + L/16 of
// token (L & 15) ^ 8*((L >> 4) & 1): one token per lane per tile.
// ------------------------------------------------------------------------------------
struct Bf16Rows {
  static constexpr int kRowBytes = kRowBytesBf16;
  static constexpr int kDmaOps = 18;
  static constexpr int kTileBytes = kTile * kRowBytes;  // 18,432
  static constexpr int kAcc = 32;                       // 16x16 output tiles per head group

  struct Aux {};

  __device__ static __forceinline__ int dma_token(int lane) { return (lane & 15) ^ (8 * ((lane >> 4) & 1)); }

  __device__ static __forceinline__ void issue(const uint8_t* row, uint32_t dst, int lane) {
    const uint8_t* src = row + 16 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < kDmaOps; ++j) dma16(src + 64 * j, dst + 1024 * j);
  }

  __device__ static __forceinline__ f32x4 qk(const uint8_t* buf, int m, int g, const u32x4* qf, Aux&) {
    const uint8_t* base = buf + 256 * g + 16 * (m ^ (8 * (g & 1)));
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 18; ++j) s = mfma_16x16x32(*(const u32x4*)(base + 1024 * j), qf[j], s);
    return s;
  }

  __device__ static __forceinline__ void pv(const uint8_t* buf, int m, int g, const float (&p)[4],
                                            const Aux&, f32x4 (&O)[kAcc]) {
    const u32x2 pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
    const int t = 4 * g + (m >> 2);
    const int cc = (m >> 1) & 1;
    const uint8_t* base = buf + 16 * (16 * cc + (t ^ (8 * cc))) + 8 * (m & 1);
#pragma unroll
    for (int u = 0; u < kAcc; ++u) O[u] = mfma_16x16x16(lds_read_tr16(base + 512 * u), pb, O[u]);
  }

  // Accumulator u holds, for head m, d = 16u + 4g + r in element r.
  __device__ static __forceinline__ void store(const f32x4 (&O)[kAcc], float* row, int g) {
#pragma unroll
    for (int u = 0; u < kAcc; ++u) *(f32x4*)(row + 16 * u + 4 * g) = O[u];
  }
};

// ------------------------------------------------------------------------------------
// fp8 656-byte rows: 41 chunks of 16 bytes per token (32 code chunks, 1 scale chunk,
// 8 rope chunks).  Chunk c of token t sits at position 16*c + (t ^ (c & 3)); DMA
// instruction j makes lane L fetch chunk 4j + L/16 of token (L & 15) ^ (L >> 4).  The
// eleventh instruction only has 16 real chunks; its other lanes re-read an in-row chunk
// into padding, so every access stays inside the row.
// ------------------------------------------------------------------------------------
struct Fp8Rows {
  static constexpr int kRowBytes = kRowBytesFp8;
  static constexpr int kDmaOps = 11;
  static constexpr int kTileBytes = kDmaOps * 1024;  // 10,496 used + padding
  static constexpr int kAcc = 32;

  struct Aux {
    f32x4 sc[4];  // sc[r][k]: scale of block k of token 4g + r
  };

  __device__ static __forceinline__ int dma_token(int lane) { return (lane & 15) ^ (lane >> 4); }

  __device__ static __forceinline__ void issue(const uint8_t* row, uint32_t dst, int lane) {
    const uint8_t* src = row + 16 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 10; ++j) dma16(src + 64 * j, dst + 1024 * j);
    dma16(row + 16 * 40, dst + 1024 * 10);  // chunk 40 for lanes 0..15; padding for the rest
  }

  __device__ static __forceinline__ u32x4 widen8(u32x2 codes) {
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], 1.0f, true));
    return r;
  }

  __device__ static __forceinline__ f32x4 qk(const uint8_t* buf, int m, int g, const u32x4* qf, Aux& aux) {
#pragma unroll
    for (int r = 0; r < 4; ++r) aux.sc[r] = *(const f32x4*)(buf + 16 * (16 * 32 + 4 * g + r));
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * k + jj;
        const int c = 2 * j + (g >> 1);
        const u32x2 codes = *(const u32x2*)(buf + 16 * (16 * c + (m ^ (c & 3))) + 8 * (g & 1));
        sk = mfma_16x16x32(widen8(codes), qf[j], sk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += aux.sc[r][k] * sk[r];
    }
    f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jr = 0; jr < 2; ++jr) {
      const int c = 33 + 4 * jr + g;
      sr = mfma_16x16x32(*(const u32x4*)(buf + 16 * (16 * c + (m ^ (c & 3)))), qf[16 + jr], sr);
    }
    return s + sr;
  }

  __device__ static __forceinline__ void pv(const uint8_t* buf, int m, int g, const float (&p)[4],
                                            const Aux& aux, f32x4 (&O)[kAcc]) {
    u32x2 pb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      pb[k] = u32x2{pack_bf16(p[0] * aux.sc[0][k], p[1] * aux.sc[1][k]),
                    pack_bf16(p[2] * aux.sc[2][k], p[3] * aux.sc[3][k])};
    const int q = m >> 2;  // chunk c = 4i + q, so c & 3 == q
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 4 * i + q;
        const uint32_t w = *(const uint32_t*)(buf + 16 * (16 * c + ((4 * g + r) ^ q)) + 4 * (m & 3));
        lo[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
        hi[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
      }
      // lo[r] = (x[r][0], x[r][1]), hi[r] = (x[r][2], x[r][3]) with x[r][e] = row(4g+r)[64i + 4m + e].
      // A operand e needs (x[0][e], x[1][e], x[2][e], x[3][e]).
      const u32x2 a0 = {__builtin_amdgcn_perm(lo[1], lo[0], 0x05040100u), __builtin_amdgcn_perm(lo[3], lo[2], 0x05040100u)};
      const u32x2 a1 = {__builtin_amdgcn_perm(lo[1], lo[0], 0x07060302u), __builtin_amdgcn_perm(lo[3], lo[2], 0x07060302u)};
      const u32x2 a2 = {__builtin_amdgcn_perm(hi[1], hi[0], 0x05040100u), __builtin_amdgcn_perm(hi[3], hi[2], 0x05040100u)};
      const u32x2 a3 = {__builtin_amdgcn_perm(hi[1], hi[0], 0x07060302u), __builtin_amdgcn_perm(hi[3], hi[2], 0x07060302u)};
      const u32x2 b = pb[i >> 1];
      O[4 * i + 0] = mfma_16x16x16(a0, b, O[4 * i + 0]);
      O[4 * i + 1] = mfma_16x16x16(a1, b, O[4 * i + 1]);
      O[4 * i + 2] = mfma_16x16x16(a2, b, O[4 * i + 2]);
      O[4 * i + 3] = mfma_16x16x16(a3, b, O[4 * i + 3]);
    }
  }

  // Accumulator 4i + e holds, for head m, d = 64i + 16g + 4r + e in element r.
  __device__ static __forceinline__ void store(const f32x4 (&O)[kAcc], float* row, int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4*)(row + 64 * i + 16 * g + 4 * r) =
            f32x4{O[4 * i + 0][r], O[4 * i + 1][r], O[4 * i + 2][r], O[4 * i + 3][r]};
  }
};

constexpr int kRedStride = kLatent + 4;  // padded per-head row of the cross-wave merge
constexpr int kRedBytes = kWaves * kMaxHeads * kRedStride * 4 + 2 * kWaves * kMaxHeads * 4;

// Per wave: two tile buffers, then (after all waves' buffers) 512 bytes of page-id slots.
template <class Fmt>
constexpr int smem_bytes() {
  return kWaves * 2 * Fmt::kTileBytes + kWaves * 512 > kRedBytes ? kWaves * 2 * Fmt::kTileBytes + kWaves * 512
                                                                 : kRedBytes;
}

template <class Fmt>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<Fmt>()];

  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int g = lane >> 4;

  const int64_t L = p.seq_lens[b];
  const Range rg = partition(L, p.page_size, p.num_splits, s);
  const int n = (int)(rg.t1 - rg.t0);
  const int ntiles = (n + kTile - 1) / kTile;

  // q as the B operand of the QK MFMA: lane (head m, slice g) holds q[m][32j + 8g .. +8].
  u32x4 qf[18];
  {
#pragma unroll
    for (int j = 0; j < 18; ++j) qf[j] = u32x4{0u, 0u, 0u, 0u};
    if (m < p.heads) {
      const uint16_t* qrow = p.q + ((int64_t)b * p.heads + m) * kRow + 8 * g;
#pragma unroll
      for (int j = 0; j < 18; ++j) qf[j] = *(const u32x4*)(qrow + 32 * j);
    }
    // Consume q here so the compiler's waits for these loads land before the
    // pipeline: inside it, a compiler-generated vmcnt wait would also wait for the
    // hand-counted row DMAs in flight.
#pragma unroll
    for (int j = 0; j < 18; ++j) asm volatile("" ::"v"(qf[j]));
  }

  float m_run = -INFINITY;  // running max (log2 domain) for head m
  float l_run = 0.f;        // this lane's share of the softmax denominator
  f32x4 O[Fmt::kAcc];
#pragma unroll
  for (int u = 0; u < Fmt::kAcc; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const uint32_t ps = (uint32_t)p.page_size;
  const int my_tok = Fmt::dma_token(lane);
  uint8_t* wbuf = smem + wave * 2 * Fmt::kTileBytes;
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_offset(wbuf));

  // Token this lane fetches in tile k, clamped into the partition (ragged tail).
  // Tokens and page indices fit in 32 bits (seq_lens are int32).
  const uint32_t t0 = (uint32_t)rg.t0;
  const uint32_t tlast = (uint32_t)(rg.t1 - 1);
  auto lane_token = [&](int k) -> uint32_t {
    const uint32_t t = t0 + (uint32_t)k * kTile + (uint32_t)my_tok;
    return t > tlast ? tlast : t;
  };
  // Page ids travel HBM -> LDS by DMA as well (one 4-byte entry per lane, lane l's own
  // token), two tiles ahead of use, so that no compiler-visible load sits in the loop:
  // the only vector-memory operations are these DMAs, whose completion is counted by
  // hand.  The slot for the tile issued in pipeline step i is pslot[i & 1].
  uint8_t* pslot = smem + kWaves * 2 * Fmt::kTileBytes + wave * 512;
  const uint32_t plds = __builtin_amdgcn_readfirstlane(lds_offset(pslot));
  auto fetch_page = [&](int k, uint32_t slot) {
    const uint32_t pi = lane_token(k) / ps;
    dma4(bt + pi, slot);
  };
  auto row_of = [&](uint32_t tok, int32_t page) -> const uint8_t* {
    const uint32_t within = tok % ps;
    const int64_t slot = (int64_t)page * (int64_t)ps + (int64_t)within;
    return p.cache + slot * (int64_t)Fmt::kRowBytes;
  };
  auto read_page = [&](const uint8_t* slot) -> int32_t { return *(const int32_t*)(slot + 4 * lane); };

  // One tile of work: QK^T, online softmax, PV on the tile in `buf`.
  auto compute = [&](const uint8_t* buf, int k) {
    typename Fmt::Aux aux;
    const f32x4 raw = Fmt::qk(buf, m, g, qf, aux);
    const int valid = n - k * kTile;
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = (4 * g + r < valid) ? raw[r] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const bool grow = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < Fmt::kAcc; ++u) O[u] *= alpha;
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sc[r] - m_run);
      l_run += pr[r];
    }
    Fmt::pv(buf, m, g, pr, aux, O);
  };

  // Software pipeline over this wave's tiles k = wave, wave + 4, ...: tile k+4 is in
  // flight while tile k is computed.  The page id of the tile after next is loaded
  // before the next tile's row loads are issued, so consuming it never waits on them.
  // Pipeline step i computes tile k = wave + 4i while tile k + 4 streams in; the page
  // ids of tile k + 8 are fetched before tile k + 4's rows are issued.
  int k = wave;
  int it = 0;
  if (k < ntiles) {
    fetch_page(k, plds + 256);
    wait_vmcnt<0>();
    const int32_t page0 = read_page(pslot + 256);
    fetch_page(min(k + kWaves, ntiles - 1), plds);
    Fmt::issue(row_of(lane_token(k), page0), wlds, lane);
    for (; k + kWaves < ntiles; k += kWaves, ++it) {
      const int kn = k + kWaves;
      wait_vmcnt<Fmt::kDmaOps>();  // page ids of tile kn have landed; tile k may be in flight
      const int32_t page_n = read_page(pslot + 256 * (it & 1));
      fetch_page(min(kn + kWaves, ntiles - 1), plds + 256 * ((it + 1) & 1));
      Fmt::issue(row_of(lane_token(kn), page_n), wlds + ((it + 1) & 1) * Fmt::kTileBytes, lane);
      wait_vmcnt<Fmt::kDmaOps + 1>();  // tile k has landed
      compute(wbuf + (it & 1) * Fmt::kTileBytes, k);
    }
    wait_vmcnt<0>();
    compute(wbuf + (it & 1) * Fmt::kTileBytes, k);
  }

  // ---- merge the waves' states through LDS ---------------------------------------
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
  __syncthreads();
  float* red = (float*)smem;
  float* red_m = red + kWaves * kMaxHeads * kRedStride;
  float* red_l = red_m + kWaves * kMaxHeads;
  Fmt::store(O, red + (wave * kMaxHeads + m) * kRedStride, g);
  if (g == 0) {
    red_m[wave * kMaxHeads + m] = m_run;
    red_l[wave * kMaxHeads + m] = l_run;
  }
  __syncthreads();

  const int H = p.heads;
  const bool split = p.num_splits > 1;
  const int64_t row_bh = (int64_t)b * H;
  float* out = split ? p.part_out + ((int64_t)s * p.batch * H + row_bh) * kLatent : p.out + row_bh * kLatent;
  float* lse = split ? p.part_lse + (int64_t)s * p.batch * H + row_bh : p.lse + row_bh;
  for (int idx = threadIdx.x; idx < H * (kLatent / 4); idx += kWaves * 64) {
    const int h = idx / (kLatent / 4);
    const int d4 = idx % (kLatent / 4);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * kMaxHeads + h]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(red_m[w * kMaxHeads + h] - M);
        lsum += f * red_l[w * kMaxHeads + h];
        o += f * *(const f32x4*)(red + (w * kMaxHeads + h) * kRedStride + 4 * d4);
      }
      o *= 1.0f / lsum;
    }
    *(f32x4*)(out + (int64_t)h * kLatent + 4 * d4) = o;
    if (d4 == 0) lse[h] = (M == -INFINITY) ? -INFINITY : (M + fast_log2(lsum)) * 0.69314718055994530942f;
  }
}

template <class Fmt>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)p.batch);
  hipLaunchKernelGGL(decode_kernel<Fmt>, grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) { return launch<Bf16Rows>(p, stream); }
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream) { return launch<Fp8Rows>(p, stream); }

}  // namespace mla

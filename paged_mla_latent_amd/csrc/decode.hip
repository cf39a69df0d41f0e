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
//  * Two schedules share one per-segment routine (decode_segment): decode_kernel, grid
//    (request, partition) with equal page-aligned partitions (dispatched non-empty first when
//    the grid exceeds the compute units), and decode_flat_kernel, the batch-balanced schedule
//    that cuts the whole batch's tokens into equal ranges across request boundaries (both for
//    single-token and multi-token verify queries).
//  * 4 waves per workgroup; each wave streams its own 16-token tiles (tiles wave, wave+4,
//    ...) and keeps its own online-softmax state, so the single-token loop has no
//    workgroup barrier.  The 4 states merge through LDS at the end.  Multi-token verify
//    steps with more than 16 query rows share each step's four tiles between the waves
//    (one barrier per step), each wave scoring them for its 16-row group.
//  * Rows go HBM -> LDS with 16-byte direct-to-LDS loads (no VGPR round trip), two or three
//    buffers per wave; the page ids travel by DMA as well, ahead of the rows that need
//    them, and completion is counted by hand, so no compiler-inserted wait stalls the loop.
//    Every instruction reads whole 128-byte lines, so the loads can carry the
//    non-temporal hint: bf16 rows in the line layout, fp8 rows (not line-aligned) as
//    row-major tiles, 16 consecutive rows of a page read as one run.
//  * All 16 heads share every row, so QK^T is a real 16 x 16 x 576 contraction per
//    tile (v_mfma_f32_16x16x32_bf16, rows as A, q^T as B) and PV a 512 x 16 x 16 one
//    (v_mfma_f32_16x16x16_bf16, rows^T as A via ds_read_b64_tr_b16, P^T as B; two tiles
//    per 16x16x32 instruction where a wave holds several).  The QK output layout (lane =
//    head, 4 tokens per lane) is exactly PV's B operand.
//  * Online softmax in the log2 domain with a lazy rescale: the running max moves
//    only when a tile's max exceeds it by more than 8, so probabilities stay <= 2^8
//    and the 128-register accumulator is rescaled a handful of times per partition.  The
//    accumulator and the q fragments stay in the matrix-core registers (AGPRs).
//  * fp8 rows: codes widen to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1);
//    each 128-value block's scale multiplies that block's partial score (fp32) and is
//    folded into P for that block's PV, so no dequantised value is ever rounded.
#include <type_traits>

#include "cache_rows.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;

// A row of zeros (as long as the longest row, 1,152 bytes) that index-list decodes load in place
// of a negative entry: its score is masked, and its values (zeros, not whatever slot 0 holds,
// which may be non-finite) add nothing to the output.  Never written.
__device__ __align__(256) uint8_t g_zero_row[1152];

// Rows of kLat latent values followed by 64 rope values, bf16.  kLat = 512, kRopeDim = 64:
// the 576-value row.  kRopeDim = 0 (NoPE-512 layers): only the 512 latent values (the
// first 1,024 bytes of each row) are loaded and scored.  kLat = 256: rank-256 layers,
// 320-value (640-byte) rows.
template <int kLat, int kRopeDim>
struct Bf16Rows {
  static_assert(kRopeDim == 64 || kRopeDim == 0, "rope part: 64 values or none");
  static_assert(kLat == 512 || (kLat == 256 && kRopeDim == 64), "latent widths 512 and 256");
  static constexpr int kLatent = kLat;
  static constexpr int kRowBytes = 2 * (kLat + 64);     // rows are stored with their rope part
  static constexpr int kQDim = kLat + kRopeDim;         // query values per head
  static constexpr int kQSteps = kQDim / 32;            // QK K-steps of 32 values
  static constexpr int kDmaOps = kQDim * 2 / 64;        // 18; 16 without rope; 10 at rank 256
  static constexpr int kBufs = 2;  // tiles per wave resident in LDS (2 x 4 x 18 KB)
  static constexpr int kTileBytes = kDmaOps * 1024;     // 18,432 / 16,384 / 10,240
  static constexpr int kAcc = kLat / 16;                // 16x16 output tiles per row group

  struct Aux {};
  static constexpr bool kFlatTile = false;

  // Tiles in the line layout (line_pos): lane L fetches tokens L >> 3 and 8 + (L >> 3) of a
  // tile, whole 128-byte lines, with the non-temporal hint unless cached loads were asked for.
  static constexpr int kTokensPerLane = 2;
  __device__ static __forceinline__ int fetch_token(int lane, int i) { return (lane >> 3) + 8 * i; }

  __device__ static __forceinline__ void issue(const uint8_t* const (&rows)[2], uint32_t dst, int lane, bool nt) {
    const int cv = 16 * ((lane & 7) ^ line_swz(lane >> 3));
    if (nt) {
#pragma unroll
      for (int j = 0; j < kDmaOps; ++j) dma16_nt(rows[j & 1] + 128 * (j >> 1) + cv, dst + 1024 * j);
    } else {
#pragma unroll
      for (int j = 0; j < kDmaOps; ++j) dma16(rows[j & 1] + 128 * (j >> 1) + cv, dst + 1024 * j);
    }
  }
  // Instruction j of issue() alone.
  __device__ static __forceinline__ void issue_one(const uint8_t* const (&rows)[2], uint32_t dst, int lane, bool nt,
                                                   int j) {
    const int cv = 16 * ((lane & 7) ^ line_swz(lane >> 3));
    if (nt) dma16_nt(rows[j & 1] + 128 * (j >> 1) + cv, dst + 1024 * j);
    else dma16(rows[j & 1] + 128 * (j >> 1) + cv, dst + 1024 * j);
  }

  // K-step j reads chunk 4j + g of token m (the A operand: token m, values 32j + 8g ..), at
  // line_pos(m, 4 (j & 1) + g) + 128 (j >> 1).
  __device__ static __forceinline__ f32x4 qk(const uint8_t* buf, int m, int g, const u32x4* qf, Aux&) {
    const uint8_t* base0 = buf + 16 * line_pos(m, g);
    const uint8_t* base1 = buf + 16 * line_pos(m, 4 + g);
    // Two independent accumulation chains halve the dependent-MFMA latency.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int j = 0; j < kQSteps; j += 2) {
      s0 = mfma_16x16x32(*(const u32x4*)(base0 + 1024 * j), qf[j], s0);
      s1 = mfma_16x16x32(*(const u32x4*)(base1 + 1024 * j), qf[j + 1], s1);
    }
    return s0 + s1;
  }

  // 16-wide column group u: lane (m, g) addresses token 4g + (m >> 2), values
  // 16u + 4(m & 3) .. +4, i.e. chunk 2u + ((m >> 1) & 1), half m & 1: at
  // line_pos(t, 2 (u & 3) + ((m >> 1) & 1)) + 128 (u >> 2).
  __device__ static __forceinline__ void pv_bases(const uint8_t* buf, int m, int g, const uint8_t* (&b)[4]) {
    const int t = 4 * g + (m >> 2);
    const int cc = (m >> 1) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = buf + 16 * line_pos(t, 2 * r + cc) + 8 * (m & 1);
  }
  __device__ static __forceinline__ void pv(const uint8_t* buf, int m, int g, const float (&p)[4],
                                            const Aux&, f32x4 (&O)[kAcc]) {
    const u32x2 pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
    const uint8_t* b[4];
    pv_bases(buf, m, g, b);
#pragma unroll
    for (int u = 0; u < kAcc; ++u) O[u] = mfma_16x16x16(lds_read_tr16(b[u & 3] + 2048 * (u >> 2)), pb, O[u]);
  }

  // PV over two tiles at once with the 32-deep MFMA (the 16-deep one takes as many cycles for
  // half the work): K slots 8g .. 8g + 3 carry tokens 4g .. 4g + 3 of tile a, slots 8g + 4 ..
  // 8g + 7 the same tokens of tile b, in both operands, so no lane exchanges values.
  __device__ static __forceinline__ void pv2(const uint8_t* bufa, const uint8_t* bufb, int m, int g,
                                             const float (&pa)[4], const float (&pb)[4], const Aux&, const Aux&,
                                             f32x4 (&O)[kAcc]) {
    const u32x4 p8 = {pack_bf16(pa[0], pa[1]), pack_bf16(pa[2], pa[3]), pack_bf16(pb[0], pb[1]),
                      pack_bf16(pb[2], pb[3])};
    const uint8_t* ba[4];
    pv_bases(bufa, m, g, ba);
    const int db = (int)(bufb - bufa);
#pragma unroll
    for (int u = 0; u < kAcc; ++u) {
      const uint8_t* a = ba[u & 3] + 2048 * (u >> 2);
      const u32x2 x = lds_read_tr16(a), y = lds_read_tr16(a + db);
      O[u] = mfma_16x16x32(u32x4{x[0], x[1], y[0], y[1]}, p8, O[u]);
    }
  }

  // Accumulator u holds, for head m, d = 16u + 4g + r in element r.
  __device__ static __forceinline__ void store(const f32x4 (&O)[kAcc], float* row, int g) {
#pragma unroll
    for (int u = 0; u < kAcc; ++u) *(f32x4*)(row + 16 * u + 4 * g) = O[u];
  }
};

// ------------------------------------------------------------------------------------
// fp8 656-byte rows: 41 chunks per token (32 code chunks, 1 scale chunk, 8 rope chunks).
// With rope the tile is row-major, the layout the 16 rows have in their page (token t's byte
// b at 656 t + b, 10,496 bytes): DMA instruction j fetches tile bytes [1024 j, 1024 j + 1024),
// lane L the chunk 64 j + L; the eleventh holds the last 16 chunks, which lanes L and L + 16,
// L + 32, L + 48 fetch alike (the spares land in padding).  When the 16 tokens are consecutive
// slots of one page, an instruction reads eight whole 128-byte lines of one contiguous run,
// the form the non-temporal hint needs; otherwise (a tile that crosses a page or holds the
// partition's clamped tail) each lane finds the token of every chunk it fetches.  Reads stay
// bank-conflict free: token bases 656 t fall on 16 distinct 16-byte bank groups (656 = 144 mod
// 256, 144 t / 16 a permutation of 0 .. 15).  Without rope (kRopeDim = 0) the scores use the
// first 528 bytes of each row, but the whole rows are streamed all the same: those 528-byte
// pieces are not contiguous across rows, and whole-line streaming of the full rows measured
// faster than half-line plain loads of the pieces; the rope bytes land in LDS unused.
// kTrim (NoPE index lists, whose rows are fetched one by one anyway): only the first 528 bytes
// of each row are fetched, the tile holds 528-byte rows (9 instructions, 9 KB), and the LDS
// that frees holds a fourth tile per wave.
// ------------------------------------------------------------------------------------
template <int kRopeDim, bool kTrim = false>
struct Fp8Rows {
  static_assert(kRopeDim == 64 || kRopeDim == 0, "rope part: 64 values or none");
  static_assert(!kTrim || kRopeDim == 0, "trimmed rows: no rope part");
  static constexpr int kLatent = 512;
  static constexpr int kRowBytes = kRowBytesFp8;                   // row stride in the cache
  static constexpr int kSpan = kTrim ? kLatent + 16 : kRowBytes;  // bytes of a row in a tile
  static constexpr int kQDim = kLatent + kRopeDim;
  static constexpr int kQSteps = kQDim / 32;
  static constexpr int kDmaOps = (16 * kSpan + 1023) / 1024;  // 11 instructions per tile (trimmed: 9)
  static constexpr int kBufs = kTrim ? 4 : 3;  // tiles per wave with one row group (3 x 4 x 11 KB)
  static constexpr int kTileBytes = kDmaOps * 1024;  // used bytes + padding
  static constexpr int kAcc = 32;

  struct Aux {
    f32x4 sc[4];  // sc[r][k]: scale of block k of token 4g + r
  };

  static constexpr bool kFlatTile = true;        // row-major tiles
  static constexpr int kChunks = kSpan / 16;  // 41 chunks of 16 bytes per row (trimmed: 33)
  static_assert(16 * kChunks == 64 * (kDmaOps - 1) + 16, "the last instruction: 16 chunks");

  // Byte offset of chunk c of token t in a tile.
  __device__ static __forceinline__ int pos(int t, int c) { return t * kSpan + 16 * c; }

  // The tile chunk lane L fetches in instruction j, and its token.
  __device__ static __forceinline__ int tile_chunk(int lane, int j) {
    return 64 * j + (j == kDmaOps - 1 ? (lane & 15) : lane);
  }
  static constexpr int kTokensPerLane = kDmaOps;
  __device__ static __forceinline__ int fetch_token(int lane, int j) { return tile_chunk(lane, j) / kChunks; }

  // Row-major tile fetched row by row: row_of(j) is the row of token fetch_token(lane, j),
  // found as each instruction is issued (a lane's rows are not all held at once).
  template <class RowOf>
  __device__ static __forceinline__ void issue_rows(RowOf&& row_of, uint32_t dst, int lane, bool nt) {
#pragma unroll
    for (int j = 0; j < kDmaOps; ++j) {
      const uint8_t* src = row_of(j) + 16 * (tile_chunk(lane, j) % kChunks);
      if (nt) dma16_nt(src, dst + 1024 * j); else dma16(src, dst + 1024 * j);
    }
  }

  // Row-major tile whose 16 rows are consecutive slots from `tile` on.
  __device__ static __forceinline__ void issue_contiguous(const uint8_t* tile, uint32_t dst, int lane, bool nt) {
    static_assert(!kTrim, "a trimmed tile is fetched row by row");
    if (nt) {
#pragma unroll
      for (int j = 0; j < kDmaOps; ++j) dma16_nt(tile + 16 * tile_chunk(lane, j), dst + 1024 * j);
    } else {
#pragma unroll
      for (int j = 0; j < kDmaOps; ++j) dma16(tile + 16 * tile_chunk(lane, j), dst + 1024 * j);
    }
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
    for (int r = 0; r < 4; ++r) aux.sc[r] = *(const f32x4*)(buf + pos(4 * g + r, 32));
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * k + jj;  // codes 32j + 8g .. +8: chunk 2j + (g >> 1), half g & 1
        const int c = 2 * j + (g >> 1);
        const u32x2 codes = *(const u32x2*)(buf + pos(m, c) + 8 * (g & 1));
        sk = mfma_16x16x32(widen8(codes), qf[j], sk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += aux.sc[r][k] * sk[r];
    }
    if constexpr (kRopeDim == 0) {
      return s;
    } else {
      f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jr = 0; jr < 2; ++jr)
        sr = mfma_16x16x32(*(const u32x4*)(buf + pos(m, 33 + 4 * jr + g)), qf[16 + jr], sr);
      return s + sr;
    }
  }

  // P of the 4 tokens of this lane, with each latent block's scale folded in.
  __device__ static __forceinline__ void scaled_p(const float (&p)[4], const Aux& aux, u32x2 (&pb)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      pb[k] = u32x2{pack_bf16(p[0] * aux.sc[0][k], p[1] * aux.sc[1][k]),
                    pack_bf16(p[2] * aux.sc[2][k], p[3] * aux.sc[3][k])};
  }

  // PV operands by transposing LDS reads (ds_read_b64_tr_b8): lane 16g + 2v + h addresses
  // bytes 8h .. 8h + 7 of one chunk (16 codes: a 16-column block) of one row, and lane 16g + i
  // then holds column i of the eight (row, chunk) pairs of its lane group, one byte each, in
  // the order v = 0 .. 7.  Two 4-token halves of that, widened exactly (two codes per
  // instruction), are the A operands of two 16 x 16 x 16 products, or one 16 x 16 x 32.
  // Accumulator u holds, for head m, d = 16u + 4g + r in element r (the bf16 layout).
  __device__ static __forceinline__ u32x4 widen_tr8(u32x2 w) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true))};
  }

  // One tile: lane group g reads tokens 4g .. 4g + 3 of chunks 2c' and 2c' + 1 (v < 4 and
  // v >= 4), so one read serves the products of two column blocks.
  __device__ static __forceinline__ void pv(const uint8_t* buf, int m, int g, const float (&p)[4],
                                            const Aux& aux, f32x4 (&O)[kAcc]) {
    u32x2 pb[4];
    scaled_p(p, aux, pb);
    const int v = m >> 1, h = m & 1;
    const uint8_t* src = buf + 8 * h;
    const int t = 4 * g + (v & 3);
#pragma unroll
    for (int c2 = 0; c2 < kAcc / 2; ++c2) {
      const u32x4 a = widen_tr8(lds_read_tr8(src + pos(t, 2 * c2 + (v >> 2))));
      const u32x2 b = pb[c2 >> 2];  // chunks 2c2, 2c2 + 1 lie in 128-value block c2 / 4
      O[2 * c2] = mfma_16x16x16(u32x2{a[0], a[1]}, b, O[2 * c2]);
      O[2 * c2 + 1] = mfma_16x16x16(u32x2{a[2], a[3]}, b, O[2 * c2 + 1]);
    }
  }

  // Two tiles with the 32-deep MFMA: K slots 8g .. 8g + 3 are tile a's tokens 4g .. 4g + 3,
  // slots 8g + 4 .. 8g + 7 tile b's, in both operands (lanes v < 4 read tile a, v >= 4 tile b).
  __device__ static __forceinline__ void pv2(const uint8_t* bufa, const uint8_t* bufb, int m, int g,
                                             const float (&pa)[4], const float (&pb)[4], const Aux& auxa,
                                             const Aux& auxb, f32x4 (&O)[kAcc]) {
    u32x2 qa[4], qb[4];
    scaled_p(pa, auxa, qa);
    scaled_p(pb, auxb, qb);
    const int v = m >> 1, h = m & 1;
    const uint8_t* src = (v < 4 ? bufa : bufb) + 8 * h;
    const int t = 4 * g + (v & 3);
#pragma unroll
    for (int c = 0; c < kAcc; ++c) {
      const u32x4 p8 = {qa[c >> 3][0], qa[c >> 3][1], qb[c >> 3][0], qb[c >> 3][1]};
      O[c] = mfma_16x16x32(widen_tr8(lds_read_tr8(src + pos(t, c))), p8, O[c]);
    }
  }

  __device__ static __forceinline__ void store(const f32x4 (&O)[kAcc], float* row, int g) {
#pragma unroll
    for (int u = 0; u < kAcc; ++u) *(f32x4*)(row + 16 * u + 4 * g) = O[u];
  }
};

// fp8 tiles widened once into bf16 tiles in LDS, for the multi-token loop where every wave
// scores every tile of a step for its own query rows: each wave converts the tile it loaded
// (codes to bf16 exactly, rope copied, block scales kept apart) and all waves then read bf16
// tiles with the 576-value row's layout.  The block scales still multiply the partial scores
// in fp32 and are folded into P, so no dequantised value is rounded.
struct Fp8Conv {
  static constexpr int kLatent = 512;
  static constexpr int kTileBytes = 18 * 1024;          // the 576-value bf16 tile
  static constexpr int kSlotBytes = kTileBytes + 256;   // + 16 tokens x 4 fp32 block scales
  static constexpr int kAcc = 32;
  using Aux = Fp8Rows<64>::Aux;

  // Wave-wide: the raw fp8 tile (Fp8Rows<64>, row-major) at `raw` into the bf16 tile at `conv`.
  __device__ static __forceinline__ void convert(const uint8_t* raw, uint8_t* conv, int lane) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // 16 tokens x 32 code chunks, 8 per lane
      const int q = lane + 64 * j;
      const int tk = q >> 5, c = q & 31;  // token, chunk of 16 codes (latent values 16c ..)
      const u32x4 codes = *(const u32x4*)(raw + Fp8Rows<64>::pos(tk, c));
      uint32_t v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], 1.0f, false));
        v[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], 1.0f, true));
      }
      *(u32x4*)(conv + 16 * chunk_pos(tk, 2 * c)) = u32x4{v[0], v[1], v[2], v[3]};
      *(u32x4*)(conv + 16 * chunk_pos(tk, 2 * c + 1)) = u32x4{v[4], v[5], v[6], v[7]};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 16 tokens x 8 rope chunks
      const int q = lane + 64 * j;
      const int tk = q >> 3, r = q & 7;
      *(u32x4*)(conv + 16 * chunk_pos(tk, 64 + r)) = *(const u32x4*)(raw + Fp8Rows<64>::pos(tk, 33 + r));
    }
    if (lane < 16) *(u32x4*)(conv + kTileBytes + 16 * lane) = *(const u32x4*)(raw + Fp8Rows<64>::pos(lane, 32));
  }

  __device__ static __forceinline__ f32x4 qk(const uint8_t* buf, int m, int g, const u32x4* qf, Aux& aux) {
#pragma unroll
    for (int r = 0; r < 4; ++r) aux.sc[r] = *(const f32x4*)(buf + kTileBytes + 16 * (4 * g + r));
    const uint8_t* base = buf + 16 * chunk_pos(m, g);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sk = mfma_16x16x32(*(const u32x4*)(base + 1024 * (4 * k + jj)), qf[4 * k + jj], sk);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += aux.sc[r][k] * sk[r];
    }
    f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jr = 0; jr < 2; ++jr) sr = mfma_16x16x32(*(const u32x4*)(base + 1024 * (16 + jr)), qf[16 + jr], sr);
    return s + sr;
  }

  // Two tiles per 32-deep MFMA as in Bf16Rows::pv2; column group u belongs to latent block u / 8,
  // whose scale is folded into P.
  __device__ static __forceinline__ void pv2(const uint8_t* bufa, const uint8_t* bufb, int m, int g,
                                             const float (&pa)[4], const float (&pb)[4], const Aux& auxa,
                                             const Aux& auxb, f32x4 (&O)[kAcc]) {
    u32x4 p8[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      p8[k] = u32x4{pack_bf16(pa[0] * auxa.sc[0][k], pa[1] * auxa.sc[1][k]),
                    pack_bf16(pa[2] * auxa.sc[2][k], pa[3] * auxa.sc[3][k]),
                    pack_bf16(pb[0] * auxb.sc[0][k], pb[1] * auxb.sc[1][k]),
                    pack_bf16(pb[2] * auxb.sc[2][k], pb[3] * auxb.sc[3][k])};
    const int t = 4 * g + (m >> 2);
    const int cc = (m >> 1) & 1;
    const int o0 = 16 * chunk_pos(t, cc) + 8 * (m & 1);
    const int o1 = 16 * chunk_pos(t, 2 + cc) + 8 * (m & 1);
#pragma unroll
    for (int u = 0; u < kAcc; u += 2) {
      const u32x2 a0 = lds_read_tr16(bufa + o0 + 512 * u), b0 = lds_read_tr16(bufb + o0 + 512 * u);
      const u32x2 a1 = lds_read_tr16(bufa + o1 + 512 * u), b1 = lds_read_tr16(bufb + o1 + 512 * u);
      O[u] = mfma_16x16x32(u32x4{a0[0], a0[1], b0[0], b0[1]}, p8[u >> 3], O[u]);
      O[u + 1] = mfma_16x16x32(u32x4{a1[0], a1[1], b1[0], b1[1]}, p8[u >> 3], O[u + 1]);
    }
  }

  // Accumulator u holds, for head m, d = 16u + 4g + r in element r (the bf16 layout).
  __device__ static __forceinline__ void store(const f32x4 (&O)[kAcc], float* row, int g) {
#pragma unroll
    for (int u = 0; u < kAcc; ++u) *(f32x4*)(row + 16 * u + 4 * g) = O[u];
  }
};

template <class Fmt, int G>
constexpr bool kConvTiles = G > 1 && std::is_same<Fmt, Fp8Rows<64>>::value;

constexpr int kRedStride = kLatent + 4;  // padded per-head row of the cross-wave merge
constexpr int kRedBytes = kWaves * kMaxHeads * kRedStride * 4 + 2 * kWaves * kMaxHeads * 4;

// Per wave: kBufs tile buffers, then (after all waves' buffers) kBufs 256-byte page-id slots.
template <class Fmt>
constexpr int pipe_bytes() {
  // row-major tiles add NB - 1 page-id slots per wave for the first tiles (the last bytes)
  return kWaves * Fmt::kBufs * (Fmt::kTileBytes + 256) + (Fmt::kFlatTile ? kWaves * (Fmt::kBufs - 1) * 256 : 0);
}
template <class Fmt>
constexpr int smem_bytes() {
  return pipe_bytes<Fmt>() > kRedBytes ? pipe_bytes<Fmt>() : kRedBytes;
}

// Merges the four waves' softmax states through LDS and writes this segment's R query rows
// of out ([R][kOut]) and lse ([R]).  Row group gg's states are held by the waves w with
// w % G == gg.
template <class TF, int G, bool kGla2, int kOut>
__device__ __forceinline__ void finish_rows(uint8_t* smem, const f32x4 (&O)[TF::kAcc], float m_run, float l_run,
                                            int R, int H, float* out, float* lse) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  l_run = sum_over_rows(l_run);
  __syncthreads();
  float* red = (float*)smem;
  float* red_m = red + kWaves * kMaxHeads * kRedStride;
  float* red_l = red_m + kWaves * kMaxHeads;
  TF::store(O, red + (wave * kMaxHeads + m) * kRedStride, g);
  if (g == 0) {
    red_m[wave * kMaxHeads + m] = m_run;
    red_l[wave * kMaxHeads + m] = l_run;
  }
  __syncthreads();

  // Thread t merges row r = t / 16 (+ 16 per pass) at float4 columns t % 16 + 16 j: the row's
  // weights are formed once, every LDS read of a pass is independent of the others (no chain
  // of waits), and 16 lanes store 256 contiguous bytes of a row.  Row r's states are those of
  // the kWaves / G waves gg + G i, gg = r / 16, taken in that order.
  constexpr int kPer = kWaves / G;        // waves holding a row group's states
  constexpr int kCols = kOut / 4 / 16;    // float4 columns per thread and row
  const int t = threadIdx.x;
  for (int r = t / 16; r < R; r += kWaves * 64 / 16) {
    const int gg = r / 16;
    const int mm = r % 16;
    // first O column of this row's output (GLA-g2: its head group's half)
    const int c0 = kGla2 ? ((r % H) >= H / 2 ? 256 : 0) : 0;
    float mw[kPer], lw[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      mw[i] = red_m[(gg + G * i) * kMaxHeads + mm];
      lw[i] = red_l[(gg + G * i) * kMaxHeads + mm];
    }
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) M = fmaxf(M, mw[i]);
    const bool live = M != -INFINITY;
    float f[kPer];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      f[i] = live ? fast_exp2(mw[i] - M) : 0.f;
      // No finite score: the running maxima ignore NaN scores, but the sums do not: they are 0
      // for an empty partition, giving (+0, -inf), and NaN when every score was NaN.
      lsum += live ? f[i] * lw[i] : lw[i];
    }
    // a NaN score anywhere made lsum NaN: NaN out
    const float scale = live ? 1.0f / lsum : lsum;
    const float* src = red + (gg * kMaxHeads + mm) * kRedStride + c0 + 4 * (t % 16);
    float* dst = out + (int64_t)r * kOut + 4 * (t % 16);
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (live) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) o += f[i] * *(const f32x4*)(src + G * i * kMaxHeads * kRedStride + 64 * j);
      }
      o *= scale;
      *(f32x4*)(dst + 64 * j) = o;
    }
    if (t % 16 == 0) lse[r] = (M == -INFINITY) ? -INFINITY + lsum : (M + fast_log2(lsum)) * 0.69314718055994530942f;
  }
}

// Query rows.  A launch decodes R = q_len x heads query rows per request (q_len > 1: the
// query tokens of a speculative-decoding verify step, query i of a request with L tokens
// seeing tokens 0 .. L - q_len + i).  Row r = i * heads + h.  The rows are cut into G
// groups of 16 (one MFMA N-tile each):
//  * G = 1 (R <= 16): every wave streams its own tiles k = wave, wave + 4, ... and scores
//    them for all rows; the four waves' states are merged at the end (no barrier).
//  * G = 2 or 4: every wave still streams its own tiles, but a workgroup barrier per step
//    makes the step's four tiles visible to all waves, and wave w scores tiles
//    G(w/G) .. G(w/G) + G - 1 of the step for row group w % G.  The cache is read once
//    per request whatever q_len is; the arithmetic per byte grows with G.
// kGla2: GLA-g2 heads.  Head h of H belongs to group gh = h / (H / 2) and scores latent
// values [256 gh, 256 gh + 256) plus the shared rope: q holds 320 values per head (group
// latent, rope), scattered into a 576-wide fragment that is zero outside the group, and
// the output of each head is its group's 256 columns.  The row is read once for both
// groups; the MFMA work is that of the 576-wide decode.
// kSparse (single-token decodes only): the block table is a per-query list of cache slots
// (page size 1) whose negative entries select nothing: such a token is loaded from slot 0 and
// masked out of the scores (a 16-bit validity mask per tile, taken when the tile's slots are read).
// ------------------------------------------------------------------------------------
// The step's new rows, written by the decode (the cache-write step fused into the launch).  New
// row i of request b is context position L - q_len + i; the segment whose token range holds a
// position writes that row, and no other workgroup reads it.  Its inputs are requested at the
// segment's start, beside the q loads (append_begin); the stores go out just before the
// segment's first row load, are waited for (vmcnt 0: the vector-memory counter does not order
// stores against loads) and a barrier orders them before every wave's row loads
// (append_end), which then read the new rows from this XCD's L2.  Wave w writes the segment's
// new rows w, w + 4, ...; only segments that hold new rows pay the extra round trip.
// ------------------------------------------------------------------------------------
struct AppendRows {
  int64_t lo = 0;  // position of the segment's first new row
  int count = 0;   // new rows in the segment (workgroup-uniform)
  int64_t slot = -1;
  RowIn in;        // this wave's first row's inputs
};

template <class Fmt>
__device__ __forceinline__ AppendRows append_begin(const DecodeParams& p, int b, int64_t L, int64_t t0, int64_t t1,
                                                   int wave, int lane) {
  AppendRows a;
  if constexpr (Fmt::kLatent == kLatent) {
    if (p.new_latent == nullptr) return a;
    const int64_t base = L - p.q_len;  // position of new row 0
    const int64_t lo = base > t0 ? base : t0, hi = L < t1 ? L : t1;
    if (lo >= hi) return a;
    a.lo = lo;
    a.count = (int)(hi - lo);
    if (wave < a.count) {
      const int64_t tok = (int64_t)b * p.q_len + (lo + wave - base);
      a.slot = p.new_slots[tok];
      a.in = load_row(p.new_latent + tok * kLatent, p.new_k_pe == nullptr ? nullptr : p.new_k_pe + tok * kRope, lane);
    }
  }
  return a;
}

template <class Fmt>
__device__ __forceinline__ void append_end(const DecodeParams& p, int b, int64_t L, const AppendRows& a, int wave,
                                           int lane, uint32_t& bad) {
  if constexpr (Fmt::kLatent == kLatent) {
    if (a.count == 0) return;
    constexpr bool kFp8 = Fmt::kRowBytes == kRowBytesFp8;
    const int64_t base = L - p.q_len;
    const int64_t slots = p.num_pages * (int64_t)p.page_size;
    for (int j = wave; j < a.count; j += kWaves) {
      int64_t slot = a.slot;
      RowIn in = a.in;
      if (j != wave) {  // rows past the first four (q_len > 4)
        const int64_t tok = (int64_t)b * p.q_len + (a.lo + j - base);
        slot = p.new_slots[tok];
        in = load_row(p.new_latent + tok * kLatent, p.new_k_pe == nullptr ? nullptr : p.new_k_pe + tok * kRope, lane);
      }
      if (slot < 0) continue;
      if constexpr (kChecked) {
        // a row outside the pool, or not at the slot the block table gives its position: not written
        const int64_t pos = a.lo + j;
        const int32_t pg = p.block_table[(int64_t)b * p.bt_stride + pos / p.page_size];
        if (slot >= slots || slot != (int64_t)pg * p.page_size + pos % p.page_size) {
          bad |= kCheckBlockId;
          continue;
        }
      }
      if constexpr (kFp8) {
        store_row_fp8(in, p.cache_w + slot * (int64_t)kRowBytesFp8, lane);
      } else {
        store_row_bf16(in, p.cache_w + slot * (int64_t)kRowBytesBf16, lane);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
}

template <class Fmt, int G, bool kGla2, bool kSparse = false, bool kAppend = false>
__device__ __forceinline__ void decode_segment(const DecodeParams& p, uint8_t* smem, int b, int64_t L,
                                               int64_t t0_abs, int64_t t1_abs, float* out, float* lse) {
  static_assert(!kSparse || (G == 1 && !kGla2), "index lists: single-token queries");
  static_assert(G == 1 || G == 2 || G == 4, "row groups per workgroup");
  static_assert(!kGla2 || (Fmt::kLatent == 512 && Fmt::kQDim == 576), "GLA-g2 on the 576-value row");
  constexpr int kOut = kGla2 ? 256 : Fmt::kLatent;  // output values per query row
  // fp8 rows in the multi-token loop: tiles widened once per step into bf16 (Fp8Conv).
  constexpr bool kConv = kConvTiles<Fmt, G>;
  using TF = typename std::conditional<kConv, Fp8Conv, Fmt>::type;  // layout the scores read
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int m = lane & 15;
  const int g = lane >> 4;

  // Tokens [t0_abs, t1_abs) of request b, whose context holds L tokens (a partition of it,
  // or a segment of a workgroup's share of the batch).
  const Range rg = {t0_abs, t1_abs};
  const int n = (int)(rg.t1 - rg.t0);
  const int ntiles = (n + kTile - 1) / kTile;

  const int H = p.heads;
  const int R = p.q_len * H;                     // query rows of a request
  const int row = 16 * (G == 1 ? 0 : wave % G) + m;  // this lane's query row
  // This lane's row sees the tokens before `lim` (absolute); as an offset into the
  // partition, clamped to its end.
  const int64_t lim = L - p.q_len + 1 + (row < R ? row / H : 0);
  const int n_vis = (int)(min(rg.t1, lim) - rg.t0);
  // the step's new rows in this segment (kernels of the append calls only)
  AppendRows app;
  if constexpr (kAppend) app = append_begin<Fmt>(p, b, L, rg.t0, rg.t1, wave, lane);

  // q as the B operand of the QK MFMA: lane (row m, slice g) holds q[row][32j + 8g .. +8].
  constexpr int QS = Fmt::kQSteps;
  u32x4 qf[QS];
  {
#pragma unroll
    for (int j = 0; j < QS; ++j) qf[j] = u32x4{0u, 0u, 0u, 0u};
    if (row < R) {
      if constexpr (kGla2) {
        // 320 values per head: group latent [0, 256) then rope [256, 320).
        const int gh = (row % H) >= H / 2 ? 1 : 0;
        const uint16_t* qrow = p.q + ((int64_t)b * R + row) * 320 + 8 * g;
#pragma unroll
        for (int j = 0; j < QS; ++j) {
          if (j >= 16)
            qf[j] = *(const u32x4*)(qrow + 256 + 32 * (j - 16));
          else if (j / 8 == gh)
            qf[j] = *(const u32x4*)(qrow + 32 * (j - 8 * gh));
        }
      } else {
        const uint16_t* qrow = p.q + ((int64_t)b * R + row) * Fmt::kQDim + 8 * g;
#pragma unroll
        for (int j = 0; j < QS; ++j) qf[j] = *(const u32x4*)(qrow + 32 * j);
      }
    }
  }

  float m_run = -INFINITY;  // running max (log2 domain) of this lane's row
  float l_run = 0.f;        // this lane's share of the softmax denominator
  f32x4 O[Fmt::kAcc];
#pragma unroll
  for (int u = 0; u < Fmt::kAcc; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const uint32_t ps = (uint32_t)p.page_size;
  uint32_t bad = 0;  // checked build: MLA_CHECK_* bits of the block ids this lane used
  // A block id (with index lists: a slot) as used for an address.
  auto page_id = [&](int32_t id) -> int32_t {
    if constexpr (kSparse) {
      return id < 0 ? -1 : checked_page(id, p.num_pages, bad);
    } else {
      return checked_page(id, p.num_pages, bad);
    }
  };
  // Address of the row at offset `off` of page `pg` (index lists: a negative entry is the zero row).
  auto row_addr = [&](int32_t pg, uint32_t off) -> const uint8_t* {
    const uint8_t* a = p.cache + ((int64_t)pg * (int64_t)ps + (int64_t)off) * (int64_t)Fmt::kRowBytes;
    if constexpr (kSparse) a = pg < 0 ? g_zero_row : a;
    return a;
  };
  // Index lists: which of a tile's 16 slots are valid (bit T for token T), kept per tile buffer
  // in vmask (16 bits per buffer).
  uint64_t vmask = ~(uint64_t)0;
  auto set_mask = [&](int buf, bool ok) {
    if constexpr (kSparse) {
      const uint64_t bits = (uint64_t)__builtin_amdgcn_ballot_w64(ok && lane < kTile) & 0xFFFFu;
      vmask = (vmask & ~((uint64_t)0xFFFF << (16 * buf))) | (bits << (16 * buf));
    }
  };
  const int my_tok = lane >> 2;  // the token whose page id this lane fetches
  constexpr int TPL = Fmt::kTokensPerLane;  // the tokens whose rows this lane fetches
  // Tile buffers per wave: Fmt::kBufs for one row group; the shared-tile loop of G > 1 is
  // written for two.
  constexpr int NB = G == 1 ? Fmt::kBufs : 2;
  constexpr int NR = kConv ? 1 : NB;  // raw tile buffers per wave (one when tiles are widened)
  uint8_t* wbuf = smem + wave * NR * Fmt::kTileBytes;
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_offset(wbuf));

  // Token this lane fetches in tile k, clamped into the partition (ragged tail).
  // Tokens and page indices fit in 32 bits (seq_lens are int32).
  const uint32_t t0 = (uint32_t)rg.t0;
  const uint32_t tlast = (uint32_t)(rg.t1 - 1);
  auto clamp_token = [&](int k, int within) -> uint32_t {
    const uint32_t t = t0 + (uint32_t)k * kTile + (uint32_t)within;
    return t > tlast ? tlast : t;
  };
  auto lane_token = [&](int k) -> uint32_t { return clamp_token(k, my_tok); };
  // Page ids travel HBM -> LDS by DMA as well (one 4-byte entry per lane: lane l holds the
  // page of token l >> 2, so token T's entry is at byte 16T), well ahead of use, so that no
  // compiler-visible load sits in the loop: the only vector-memory operations are these DMAs,
  // whose completion is counted by hand.
  uint8_t* pslot = smem + kWaves * NR * Fmt::kTileBytes + wave * NB * 256;
  const uint32_t plds = __builtin_amdgcn_readfirstlane(lds_offset(pslot));
  // widened tiles, one slot per wave, after the raw tiles and page-id slots
  uint8_t* conv = smem + kWaves * NR * Fmt::kTileBytes + kWaves * NB * 256;
  static_assert(!kConv || kWaves * (Fmt::kTileBytes + NB * 256 + Fp8Conv::kSlotBytes) <= smem_bytes<Fmt>(),
                "widened tiles fit in the workgroup's LDS");
  auto fetch_page = [&](int k, uint32_t slot) {
    const uint32_t pi = lane_token(k) / ps;
    dma4(bt + pi, slot);
  };
  // The rows this lane fetches in tile k, from their pages.
  using Pages = int32_t[TPL];
  auto issue_tile = [&](int k, const Pages& page, uint32_t dst) {
    if constexpr (!Fmt::kFlatTile) {
      const uint8_t* rows[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const uint32_t tok = clamp_token(k, Fmt::fetch_token(lane, i));
        rows[i] = row_addr(page[i], tok % ps);
      }
      Fmt::issue(rows, dst, lane, p.stream_rows != 0);
    }
  };
  auto read_pages = [&](const uint8_t* slot, Pages& page) {
#pragma unroll
    for (int i = 0; i < TPL; ++i)
      page[i] = page_id(*(const int32_t*)(slot + 16 * Fmt::fetch_token(lane, i)));
  };
  // Row-major tiles (Fmt::kFlatTile) take their page ids from a page-id slot in LDS (token T's
  // page at byte 16T): a tile of 16 consecutive slots of one page is fetched as one run (a single
  // page id, read by every lane alike); any other tile row by row, each lane looking up the page
  // of every token it fetches from.  Tokens past the partition are clamped to its last one.
  auto issue_tile_flat = [&](int k, const uint8_t* pids, uint32_t dst) {
    if constexpr (Fmt::kFlatTile) {
      // the tile's first token; a tile past the partition (G > 1) is its last token, 16 times
      const uint32_t a = __builtin_amdgcn_readfirstlane(min(t0 + (uint32_t)k * kTile, tlast));
      const uint32_t q0 = __builtin_amdgcn_readfirstlane(a % ps);  // its slot in its page (uniform)
      const bool nt = p.stream_rows != 0;
      bool whole = false;  // (index lists: never one run)
      if constexpr (!kSparse) whole = a + (kTile - 1) <= tlast && q0 + kTile <= ps;
      if (whole) {
        if constexpr (!kSparse) {
          const int32_t pg = __builtin_amdgcn_readfirstlane(page_id(*(const int32_t*)pids));
          Fmt::issue_contiguous(p.cache + ((int64_t)pg * ps + q0) * Fmt::kRowBytes, dst, lane, nt);
        }
      } else {
        auto row_of = [&](int i) -> const uint8_t* {
          const uint32_t T = (uint32_t)Fmt::fetch_token(lane, i);
          uint32_t off = q0 + min(T, tlast - a);  // slot of the clamped token, before wrapping
          off = ps >= (uint32_t)kTile ? (off >= ps ? off - ps : off) : off % ps;
          return row_addr(page_id(*(const int32_t*)(pids + 16 * T)), off);
        };
        Fmt::issue_rows(row_of, dst, lane, nt);
      }
    }
  };

  // One tile of work: QK^T, online softmax, PV on tile k (partition-relative) in `buf`.
  // Tokens at or past this lane's visibility limit, or past the partition, get p = 0.
  auto compute = [&](const uint8_t* buf, int k, int cur) {
    typename Fmt::Aux aux;
    const f32x4 raw = Fmt::qk(buf, m, g, qf, aux);
    const int valid = n_vis - k * kTile;
    const uint32_t tm = kSparse ? (uint32_t)(vmask >> (16 * cur)) : 0xFFFFu;  // the tile's valid slots
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = (4 * g + r < valid) && (!kSparse || ((tm >> (4 * g + r)) & 1u));
      sc[r] = in ? raw[r] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    mx = max_over_rows(mx);
    const bool grow = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // Rows that do not grow keep alpha = 1 (exp2(m_run - m_run) would be NaN for a row
      // that has seen no visible token, m_run = -inf).
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
      scale_acc(O, alpha);
      m_run = m_new;
    }
    // A row that has seen no visible token yet keeps m_run = -inf: its masked scores
    // must give exp2(-inf) = 0, not exp2(-inf - -inf) = NaN.
    const float m_base = m_run == -INFINITY ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sc[r] - m_base);
      l_run += pr[r];
    }
    Fmt::pv(buf, m, g, pr, aux, O);
  };

  // The G tiles u0 .. u0 + G - 1 of step i for this lane's row group (G > 1), GB at a time
  // (fp8 rows keep 16 block scales per tile between QK and PV, so four fp8 tiles at once
  // would spill).  Tiles past the partition hold finite rows and score -inf.
  constexpr int GB = (G == 4 && sizeof(typename TF::Aux) > 16) ? 2 : G;
  auto tile_of = [&](int i, int u) -> const uint8_t* {
    return kConv ? conv + u * Fp8Conv::kSlotBytes : smem + (u * NB + (i & 1)) * Fmt::kTileBytes;
  };
  auto compute_tiles = [&](int i, int u0) {
    typename TF::Aux aux[GB];
    f32x4 raw[GB];
#pragma unroll
    for (int v = 0; v < GB; ++v) raw[v] = TF::qk(tile_of(i, u0 + v), m, g, qf, aux[v]);
    float sc[GB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < GB; ++v) {
      const int valid = n_vis - (kWaves * i + u0 + v) * kTile;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[v][r] = (4 * g + r < valid) ? raw[v][r] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[v][r]);
      }
    }
    mx = max_over_rows(mx);
    const bool grow = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
      scale_acc(O, alpha);
      m_run = m_new;
    }
    const float m_base = m_run == -INFINITY ? 0.f : m_run;
    float pr[GB][4];
#pragma unroll
    for (int v = 0; v < GB; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[v][r] = fast_exp2(sc[v][r] - m_base);
        l_run += pr[v][r];
      }
    // PV two tiles at a time (GB is even)
#pragma unroll
    for (int v = 0; v < GB; v += 2)
      TF::pv2(tile_of(i, u0 + v), tile_of(i, u0 + v + 1), m, g, pr[v], pr[v + 1], aux[v], aux[v + 1], O);
  };
  auto compute_step = [&](int i, int u0) {
#pragma unroll
    for (int h = 0; h < G; h += GB) compute_tiles(i, u0 + h);
  };

  constexpr int D = Fmt::kDmaOps;
  int k = wave;
  // G > 1: every wave loads a tile even where its tile lies past the partition (the
  // partition's last rows again, clamped by lane_token), so that every buffer of a step holds
  // finite rows and the step's tiles can be scored without a branch per tile.
  const bool first_tiles = G == 1 ? k < ntiles : ntiles > 0;
  if constexpr (Fmt::kFlatTile) {
    // The first NB-1 tiles' page ids go to LDS by DMA as well (slots after the pipeline's),
    // awaited before any row is requested, so the queue order below is the loop's.
    uint8_t* xslot = smem + smem_bytes<Fmt>() - kWaves * (NB - 1) * 256 + wave * (NB - 1) * 256;
    const uint32_t xlds = __builtin_amdgcn_readfirstlane(lds_offset(xslot));
    if (first_tiles) {
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) fetch_page(min(k + kWaves * t, ntiles - 1), xlds + 256 * t);
    }
#pragma unroll
    for (int j = 0; j < QS; ++j) asm volatile("" : "+a"(qf[j]));
    if constexpr (kAppend) append_end<Fmt>(p, b, L, app, wave, lane, bad);
    wait_vmcnt<0>();
    if (first_tiles) {
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) {
        fetch_page(min(k + kWaves * (t + NB - 1), ntiles - 1), plds + 256 * t);
        if constexpr (kSparse) set_mask(t, *(const int32_t*)(xslot + 256 * t + 16 * (lane & (kTile - 1))) >= 0);
        if (G > 1 || k + kWaves * t < ntiles)
          issue_tile_flat(k + kWaves * t, xslot + 256 * t, wlds + t * Fmt::kTileBytes);
      }
    }
  } else {
    // The first NB-1 tiles' page ids are ordinary loads issued with the q loads; all are
    // consumed here, so the compiler's waits for them land before the pipeline (inside it
    // a compiler-generated vmcnt wait would also wait for the hand-counted DMAs).  The q
    // fragments move to the matrix-core registers (AGPRs, beside O), which MFMA reads as
    // directly as VGPRs: that leaves about 70 more VGPRs to the compiler's schedule.
    int32_t page_first[NB - 1][TPL];
#pragma unroll
    for (int t = 0; t < NB - 1; ++t)
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        page_first[t][i] = (G == 1 ? k + kWaves * t < ntiles : ntiles > 0)
                               ? page_id(bt[clamp_token(k + kWaves * t, Fmt::fetch_token(lane, i)) / ps])
                               : 0;
    if constexpr (kSparse) {
#pragma unroll
      for (int t = 0; t < NB - 1; ++t)
        set_mask(t, k + kWaves * t < ntiles && lane < kTile && bt[clamp_token(k + kWaves * t, lane) / ps] >= 0);
    }
#pragma unroll
    for (int j = 0; j < QS; ++j) asm volatile("" : "+a"(qf[j]));
#pragma unroll
    for (int t = 0; t < NB - 1; ++t)
#pragma unroll
      for (int i = 0; i < TPL; ++i) asm volatile("" ::"v"(page_first[t][i]));
    if constexpr (kAppend) append_end<Fmt>(p, b, L, app, wave, lane, bad);
    if (first_tiles) {
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) {
        fetch_page(min(k + kWaves * (t + NB - 1), ntiles - 1), plds + 256 * t);
        if (G > 1 || k + kWaves * t < ntiles) issue_tile(k + kWaves * t, page_first[t], wlds + t * Fmt::kTileBytes);
      }
    }
  }

  if constexpr (G == 1) {
    // Software pipeline over this wave's tiles k = wave, wave + 4, ...  With NB = kBufs
    // buffers, step i computes tile k while tiles k + 4 .. k + 4(NB - 1) stream in.  The
    // vector-memory queue is kept in this order (completion is in order):
    //     ... PID(k + 4(NB-1))  DMA(k)  PID(k + 4NB)  DMA(k + 4)  ...
    // where PID(t) is the 4-byte page-id DMA of tile t and DMA(t) its D row DMAs.  Step i
    // first waits until PID(k + 4(NB-1)) has landed (at most (NB-1)D + NB-2 younger ops),
    // issues PID(k + 8(NB-1)) and DMA(k + 4(NB-1)), then waits until DMA(k) has landed (at
    // most (NB-1)(D+1) younger ops).  The steady loop runs only while tile k + 4(NB-1)
    // exists, so every counted op is really issued; page-id fetches past the end re-read
    // the last tile's entries.  The last NB-1 tiles drain under a full wait.
    if (k < ntiles) {
      int cur = 0;  // buffer / page-id slot of tile k (step index mod NB)
      for (; k + kWaves * (NB - 1) < ntiles; k += kWaves) {
        const int ahead = cur == 0 ? NB - 1 : cur - 1;  // (cur + NB - 1) mod NB
        wait_vmcnt<(NB - 1) * D + (NB - 2)>();  // page ids of tile k + 4(NB-1) have landed
        if constexpr (kSparse) set_mask(ahead, *(const int32_t*)(pslot + 256 * cur + 16 * (lane & (kTile - 1))) >= 0);
        if constexpr (Fmt::kFlatTile) {
          fetch_page(min(k + kWaves * 2 * (NB - 1), ntiles - 1), plds + 256 * ahead);
          issue_tile_flat(k + kWaves * (NB - 1), pslot + 256 * cur, wlds + ahead * Fmt::kTileBytes);
        } else {
          Pages page_n;
          read_pages(pslot + 256 * cur, page_n);
          fetch_page(min(k + kWaves * 2 * (NB - 1), ntiles - 1), plds + 256 * ahead);
          issue_tile(k + kWaves * (NB - 1), page_n, wlds + ahead * Fmt::kTileBytes);
        }
        wait_vmcnt<(NB - 1) * (D + 1)>();  // tile k has landed
        compute(wbuf + cur * Fmt::kTileBytes, k, cur);
        cur = cur + 1 == NB ? 0 : cur + 1;
      }
      wait_vmcnt<0>();
      for (; k < ntiles; k += kWaves) {
        compute(wbuf + cur * Fmt::kTileBytes, k, cur);
        cur = cur + 1 == NB ? 0 : cur + 1;
      }
    }
  } else {
    static_assert(NB == 2, "the shared-tile pipeline is written for two buffers per wave");
    // Step i: every wave waits for its own tile 4i + wave (and the page ids of its next
    // one), the barrier makes all four tiles of the step visible and tells every wave that
    // the others are done with step i-1, whose buffers the next tiles then overwrite.
    // (A second barrier that lets the next loads start before this wait was measured
    // slower: the step is bound by its compute and the barrier, not by load depth.)
    //   The G tiles a wave scores per step are processed together: the scores of all G
    // first (independent MFMA chains), one running-max update over the step's 16 G tokens,
    // then the G PV products.  With one wave per SIMD, per-tile processing left the MFMA
    // pipe idle on each tile's dependent chain (scores -> max -> exp -> PV).
    const int nsteps = (ntiles + kWaves - 1) / kWaves;
    const int u0 = G * (wave / G);  // first tile of a step this wave scores
#pragma unroll 1
    for (int i = 0; i < nsteps; ++i) {
      wait_vmcnt<0>();
      __syncthreads();
      // Widened tiles: each wave converts the tile it loaded; its raw buffer is then free for
      // the next step's tile, and a second barrier publishes the four bf16 tiles.  (The first
      // barrier also tells every wave that the others are done with step i - 1's tiles.)
      if constexpr (kConv) Fp8Conv::convert(wbuf, conv + wave * Fp8Conv::kSlotBytes, lane);
      if (i + 1 < nsteps) {
        // this wave's tile of step i + 1, clamped to the partition's last tile
        const int kn = min(kWaves * (i + 1) + wave, ntiles - 1);
        const uint32_t dst = wlds + (kConv ? 0 : ((i + 1) & 1) * Fmt::kTileBytes);
        if constexpr (Fmt::kFlatTile) {
          fetch_page(min(kn + kWaves, ntiles - 1), plds + 256 * ((i + 1) & 1));
          issue_tile_flat(kn, pslot + 256 * (i & 1), dst);
        } else {
          Pages page_n;
          read_pages(pslot + 256 * (i & 1), page_n);
          fetch_page(min(kn + kWaves, ntiles - 1), plds + 256 * ((i + 1) & 1));
          issue_tile(kn, page_n, dst);
        }
      }
      if constexpr (kConv) __syncthreads();
      compute_step(i, u0);
    }
  }

  finish_rows<TF, G, kGla2, kOut>(smem, O, m_run, l_run, R, H, out, lse);
  report_checks(bad, p.check_status);
}

// ------------------------------------------------------------------------------------
// Verify steps with 33..64 query rows (q_len x heads, four 16-row groups): the scores are
// split by row group and the PV by output columns.
//
// Each wave still streams its own tiles (wave w loads tile 4i + w of step i) and scores the
// step's four tiles for its row group w (QK reads every tile once per row group: the A operand
// of a 16-row group).  The PV is split the other way: wave w accumulates output columns
// [128w, 128w + 128) of all 64 query rows (4 row groups x 8 column tiles = 32 accumulators, the
// same 128 registers as one row group x 512 columns), so every column tile of a tile is read
// from LDS once per step instead of once per row group (PV LDS reads per tile: 16 KB instead
// of 64 KB).  The probabilities reach the other waves through LDS: bf16 rows exchange them as
// the bf16 pairs the PV MFMA consumes; fp8 rows exchange them in fp32, because wave w folds the
// scale of its own 128-value block (block w) into P before the one bf16 rounding, and reads
// that block's codes straight from the raw 656-byte tile (no widened copy in LDS).  A softmax
// rescale of row group r (rare: the running maximum moves in steps of at least 2^8) travels the
// same way: its owner wave publishes alpha for its rows and a flag, and every wave scales its
// accumulators of that row group before adding the step.
//
// fp8 rows score with the K dimension split as well: the waves pair up by row half (waves 2h
// and 2h + 1 own row groups 2h and 2h + 1) and each wave of a pair takes one half of the row
// (latent blocks 2k and 2k + 1 and rope values [32k, 32k + 32) for wave 2h + k) for both row
// groups of its half.  A code is then widened once per row half instead of once per row group,
// and each wave reads half of every tile for its scores.  The partial scores of the partner's
// row group go through LDS (in the slot that then carries that row group's P), a barrier, and
// every owner adds them to its own partial: three barriers per step instead of two.
//
// Per step: each wave waits for its own tile, a barrier makes the four tiles (and the end of
// the previous step) visible, the next tiles are requested, the owner waves score (fp8: the
// pairs exchange partial scores), rescale and publish P, a barrier, then every wave reads the
// four row groups' P and accumulates its columns.  The owner of row group r keeps its running
// maximum and sum; the epilogue publishes them and every wave writes its columns of every row.
// ------------------------------------------------------------------------------------
template <class Fmt>
struct ColSplit {
  static constexpr bool kFp8 = std::is_same<Fmt, Fp8Rows<64>>::value;
  static_assert(kFp8 || std::is_same<Fmt, Bf16Rows<512, 64>>::value, "576-value rows");
  static constexpr int kNB = kFp8 ? 3 : 2;  // tiles per wave resident: 3 x 4 x 11 KB / 2 x 4 x 18 KB
  static constexpr int kTiles = kWaves * kNB * Fmt::kTileBytes;
  static constexpr int kPids = kWaves * kNB * 256;
  static constexpr int kXslots = Fmt::kFlatTile ? kWaves * (kNB - 1) * 256 : 0;
  // P of a step: bf16, [row group][tile pair][lane] u32x4 (8 KB); fp8, fp32 [row group][tile][lane]
  // f32x4 (16 KB).
  static constexpr int kPex = kFp8 ? 4 * 4 * 64 * 16 : 4 * 2 * 64 * 16;
  static constexpr int kAlpha = 4 * 16 * 4 + 16;  // alpha [row group][row], then 4 flags
  // fp8: the step's block scales transposed, [2 steps][tile][block][token] fp32
  static constexpr int kScales = kFp8 ? 2 * 4 * 4 * 16 * 4 : 0;
  static constexpr int kBytes = kTiles + kPids + kXslots + kPex + kAlpha + kScales;
  static_assert(kBytes <= 160 * 1024, "column-split verify step fits in the LDS");
};

// bf16 scores of one 16-row group over four tiles: raw[v] = A(tile v) x q^T, as Bf16Rows::qk
// computes them, with the four tiles' MFMA chains interleaved K-step by K-step.  between(j) runs
// after K-step j's four MFMAs are issued: the next tile's loads go out one instruction per
// K-step there, spread over the MFMAs, instead of holding all four waves in a burst of
// vector-memory instructions right after the step's barrier.
template <class Fmt, class Between>
__device__ __forceinline__ void score_tiles(const uint8_t* t0, const uint8_t* t1, const uint8_t* t2,
                                            const uint8_t* t3, int m, int g, const u32x4* qf, f32x4 (&raw)[4],
                                            Between&& between) {
  static_assert(!Fmt::kFlatTile, "bf16 line-layout tiles");
  const uint8_t* const tile[4] = {t0, t1, t2, t3};
  // line layout: K-step j reads chunk 4 (j & 1) + g of token m, plus 128 (j >> 1) chunks
  const int o0 = 16 * line_pos(m, g), o1 = 16 * line_pos(m, 4 + g);
#pragma unroll
  for (int v = 0; v < 4; ++v) raw[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  // K-step j's four A operands in a[j % 3], read two K-steps ahead (eight reads in flight: with
  // one wave per SIMD, fewer leave the LDS latency exposed before the MFMAs)
  auto read = [&](int j, u32x4 (&dst)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[v] = *(const u32x4*)(tile[v] + ((j & 1) ? o1 : o0) + 1024 * (j & ~1));
  };
  u32x4 a[3][4];
  read(0, a[0]);
  read(1, a[1]);
#pragma unroll
  for (int j = 0; j < Fmt::kQSteps; ++j) {
    if (j + 2 < Fmt::kQSteps) read(j + 2, a[(j + 2) % 3]);
#pragma unroll
    for (int v = 0; v < 4; ++v) raw[v] = mfma_16x16x32(a[j % 3][v], qf[j], raw[v]);
    between(j);
  }
}

// fp8 partial scores of two 16-row groups (own, partner) over four tiles and one half of the
// row: latent blocks 2 kh and 2 kh + 1 (each block's partial scaled by its block scale, from the
// transposed table sct) plus rope values [32 kh, 32 kh + 32).  qo / qp: the own / partner rows'
// q fragments, [0, 8) the half's eight latent K-steps, [8] its rope K-step.  Each widened code
// feeds both row groups' MFMAs.  A block's LDS reads (16 code fragments, its 4 scale vectors;
// block 1 also the rope) are all issued before its first MFMA, so that one LDS latency is
// exposed per block instead of one per read.  between() runs after block 0's MFMAs are issued
// (the next tile's loads are requested there, while those MFMAs execute; spread a few at a time
// over the K-steps instead, as the bf16 scores do, they measured slower here).
template <class Between>
__device__ __forceinline__ void score_tiles_half(const uint8_t* const (&tile)[4], const uint8_t* sct, int m, int g,
                                                 int kh, const u32x4* qo, const u32x4* qp, f32x4 (&po)[4],
                                                 f32x4 (&pp)[4], Between&& between) {
  using F = Fp8Rows<64>;
#pragma unroll
  for (int v = 0; v < 4; ++v) po[v] = pp[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 rope[4];
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const int k = 2 * kh + bk;  // latent block
    u32x2 codes[4][4];          // [K-step jj][tile v]: codes 32j + 8g .. + 8 of token m
    f32x4 sc[4];                // [tile v]: block k's scales of tokens 4g .. 4g + 3
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 4 * k + jj;  // chunk 2j + (g >> 1), half g & 1
        codes[jj][v] = *(const u32x2*)(tile[v] + F::pos(m, 2 * j + (g >> 1)) + 8 * (g & 1));
      }
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = *(const f32x4*)(sct + (16 * (4 * v + k) + 4 * g) * 4);
    if (bk == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) rope[v] = *(const u32x4*)(tile[v] + F::pos(m, 33 + 4 * kh + g));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 so[4], sp[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) so[v] = sp[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 a = F::widen8(codes[jj][v]);
        so[v] = mfma_16x16x32(a, qo[4 * bk + jj], so[v]);
        sp[v] = mfma_16x16x32(a, qp[4 * bk + jj], sp[v]);
      }
    // Widen the next operand while the current one's two MFMAs run (the matrix core and the
    // vector ALU work side by side only when the instruction stream alternates them): one
    // MFMA, then two vector instructions.  Pairs of MFMAs between groups of four measured about
    // 1.4 % slower on the whole verify step.
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    if (bk == 0) {
      __builtin_amdgcn_sched_barrier(0);
      between();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        po[v][r] += sc[v][r] * so[v][r];
        pp[v][r] += sc[v][r] * sp[v][r];
      }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    po[v] = mfma_16x16x32(rope[v], qo[8], po[v]);
    pp[v] = mfma_16x16x32(rope[v], qp[8], pp[v]);
  }
}

template <class Fmt, bool kAppend = false>
__device__ __forceinline__ void decode_segment_cs(const DecodeParams& p, uint8_t* smem, int b, int64_t L,
                                                  int64_t t0_abs, int64_t t1_abs, float* out, float* lse) {
  using CS = ColSplit<Fmt>;
  constexpr int NB = CS::kNB;
  constexpr int D = Fmt::kDmaOps;
  constexpr int QS = Fmt::kQSteps;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // = this wave's row group
  const int m = lane & 15;
  const int g = lane >> 4;

  const Range rg = {t0_abs, t1_abs};
  const int n = (int)(rg.t1 - rg.t0);
  const int ntiles = (n + kTile - 1) / kTile;
  const int nsteps = (ntiles + kWaves - 1) / kWaves;

  const int H = p.heads;
  const int R = p.q_len * H;
  const int row = 16 * wave + m;  // this lane's query row in the scores (row group = wave)
  const int64_t lim = L - p.q_len + 1 + (row < R ? row / H : 0);
  const int n_vis = (int)(min(rg.t1, lim) - rg.t0);
  AppendRows app;  // the step's new rows in this segment (kernels of the append calls only)
  if constexpr (kAppend) app = append_begin<Fmt>(p, b, L, rg.t0, rg.t1, wave, lane);

  // q as the B operand of the QK MFMA: lane (row m, slice g) holds q[row][32j + 8g .. + 8].  bf16:
  // the own row group's 18 K-steps.  fp8: [0, 9) the own row group's, [9, 18) the partner row
  // group's K-steps of this wave's half of the row (8 latent, then 1 rope).
  [[maybe_unused]] const int kh = wave & 1;  // fp8: this wave's half of the row
  u32x4 qf[QS];
#pragma unroll
  for (int j = 0; j < QS; ++j) qf[j] = u32x4{0u, 0u, 0u, 0u};
  if constexpr (CS::kFp8) {
    static_assert(QS == 18, "two row groups x (8 + 1) K-steps");
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int rr = 16 * (c == 0 ? wave : (wave ^ 1)) + m;
      if (rr < R) {
        const uint16_t* qrow = p.q + ((int64_t)b * R + rr) * Fmt::kQDim + 8 * g;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) qf[9 * c + jj] = *(const u32x4*)(qrow + 32 * (8 * kh + jj));
        qf[9 * c + 8] = *(const u32x4*)(qrow + 512 + 32 * kh);
      }
    }
  } else if (row < R) {
    const uint16_t* qrow = p.q + ((int64_t)b * R + row) * Fmt::kQDim + 8 * g;
#pragma unroll
    for (int j = 0; j < QS; ++j) qf[j] = *(const u32x4*)(qrow + 32 * j);
  }

  float m_run = -INFINITY;  // row group `wave`: running max (log2 domain) of row m
  float l_run = 0.f;        // and this lane's share of its sum
  f32x4 O[32];              // O[8 r + c]: row group r, columns 128 wave + 16 c + 4 g .. + 3, row m
#pragma unroll
  for (int u = 0; u < 32; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* pex = smem + CS::kTiles + CS::kPids + CS::kXslots;
  float* alpha_s = (float*)(pex + CS::kPex);
  int32_t* flag_s = (int32_t*)(alpha_s + 64);
  uint8_t* sct_base = pex + CS::kPex + CS::kAlpha;  // fp8 block scales, two steps

  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const uint32_t ps = (uint32_t)p.page_size;
  uint32_t bad = 0;
  const int my_tok = lane >> 2;
  constexpr int TPL = Fmt::kTokensPerLane;
  uint8_t* wbuf = smem + wave * NB * Fmt::kTileBytes;
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_offset(wbuf));
  uint8_t* pslot = smem + CS::kTiles + wave * NB * 256;
  const uint32_t plds = __builtin_amdgcn_readfirstlane(lds_offset(pslot));
  const uint32_t t0 = (uint32_t)rg.t0;
  const uint32_t tlast = (uint32_t)(rg.t1 - 1);
  auto clamp_token = [&](int k, int within) -> uint32_t {
    const uint32_t t = t0 + (uint32_t)k * kTile + (uint32_t)within;
    return t > tlast ? tlast : t;
  };
  // This wave's tile of step i (past the partition: its last tile, loaded again).
  auto tile_of_step = [&](int i) -> int { return min(kWaves * i + wave, ntiles - 1); };
  auto fetch_page = [&](int k, uint32_t slot_lds) { dma4(bt + clamp_token(k, my_tok) / ps, slot_lds); };
  using Pages = int32_t[TPL];
  auto issue_tile = [&](int k, const Pages& page, uint32_t dst) {
    if constexpr (!Fmt::kFlatTile) {
      const uint8_t* rows[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const uint32_t tok = clamp_token(k, Fmt::fetch_token(lane, i));
        rows[i] = p.cache + ((int64_t)page[i] * (int64_t)ps + (int64_t)(tok % ps)) * (int64_t)Fmt::kRowBytes;
      }
      Fmt::issue(rows, dst, lane, p.stream_rows != 0);
    }
  };
  auto read_pages = [&](const uint8_t* slot, Pages& page) {
#pragma unroll
    for (int i = 0; i < TPL; ++i)
      page[i] = checked_page(*(const int32_t*)(slot + 16 * Fmt::fetch_token(lane, i)), p.num_pages, bad);
  };
  auto issue_tile_flat = [&](int k, const uint8_t* pids, uint32_t dst) {
    if constexpr (Fmt::kFlatTile) {
      const uint32_t a = __builtin_amdgcn_readfirstlane(min(t0 + (uint32_t)k * kTile, tlast));
      const uint32_t q0 = __builtin_amdgcn_readfirstlane(a % ps);
      const bool nt = p.stream_rows != 0;
      if (a + (kTile - 1) <= tlast && q0 + kTile <= ps) {
        const int32_t pg = __builtin_amdgcn_readfirstlane(checked_page(*(const int32_t*)pids, p.num_pages, bad));
        Fmt::issue_contiguous(p.cache + ((int64_t)pg * ps + q0) * Fmt::kRowBytes, dst, lane, nt);
      } else {
        auto row_of = [&](int i) -> const uint8_t* {
          const uint32_t T = (uint32_t)Fmt::fetch_token(lane, i);
          uint32_t off = q0 + min(T, tlast - a);
          off = ps >= (uint32_t)kTile ? (off >= ps ? off - ps : off) : off % ps;
          const int32_t pg = checked_page(*(const int32_t*)(pids + 16 * T), p.num_pages, bad);
          return p.cache + ((int64_t)pg * ps + off) * Fmt::kRowBytes;
        };
        Fmt::issue_rows(row_of, dst, lane, nt);
      }
    }
  };
  // Page ids of step s land in slot s % NB; this wave's tile of step s in buffer s % NB.
  // Queue per wave: PID(NB - 1) DMA(0) PID(NB) DMA(1) ... ; step i then issues PID(i + 2NB - 2)
  // and DMA(i + NB - 1), so the ops younger than DMA(i) at the start of step i are those of
  // steps i - NB + 2 .. i - 1: (NB - 2)(D + 1) of them when those steps issued.
  auto slot_lds = [&](int s) { return plds + 256 * (uint32_t)(s % NB); };
  auto buf_lds = [&](int s) { return wlds + (uint32_t)(s % NB) * Fmt::kTileBytes; };
  if (nsteps > 0) {
    if constexpr (Fmt::kFlatTile) {
      uint8_t* xslot = smem + CS::kTiles + CS::kPids + wave * (NB - 1) * 256;
      const uint32_t xlds = __builtin_amdgcn_readfirstlane(lds_offset(xslot));
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) fetch_page(tile_of_step(t), xlds + 256 * t);
#pragma unroll
      for (int j = 0; j < QS; ++j) asm volatile("" : "+a"(qf[j]));
      if constexpr (kAppend) append_end<Fmt>(p, b, L, app, wave, lane, bad);
      wait_vmcnt<0>();
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) {
        fetch_page(tile_of_step(t + NB - 1), slot_lds(t + NB - 1));
        issue_tile_flat(tile_of_step(t), xslot + 256 * t, buf_lds(t));
      }
    } else {
      int32_t page_first[NB - 1][TPL];
#pragma unroll
      for (int t = 0; t < NB - 1; ++t)
#pragma unroll
        for (int i = 0; i < TPL; ++i)
          page_first[t][i] =
              checked_page(bt[clamp_token(tile_of_step(t), Fmt::fetch_token(lane, i)) / ps], p.num_pages, bad);
#pragma unroll
      for (int j = 0; j < QS; ++j) asm volatile("" : "+a"(qf[j]));
#pragma unroll
      for (int t = 0; t < NB - 1; ++t)
#pragma unroll
        for (int i = 0; i < TPL; ++i) asm volatile("" ::"v"(page_first[t][i]));
      if constexpr (kAppend) append_end<Fmt>(p, b, L, app, wave, lane, bad);
#pragma unroll
      for (int t = 0; t < NB - 1; ++t) {
        fetch_page(tile_of_step(t + NB - 1), slot_lds(t + NB - 1));
        issue_tile(tile_of_step(t), page_first[t], buf_lds(t));
      }
    }
  }

  const uint8_t* tiles = smem;
  auto tile_ptr = [&](int i, int u) -> const uint8_t* { return tiles + (u * NB + i % NB) * Fmt::kTileBytes; };

#pragma unroll 1
  for (int i = 0; i < nsteps; ++i) {
    // this wave's tile of step i has landed (and with it the page ids of step i + NB - 1)
    if (i == 0 || i + NB - 2 < nsteps) wait_vmcnt<(NB - 2) * (D + 1)>();
    else wait_vmcnt<0>();
    uint8_t* sct = sct_base + (i & 1) * (4 * 4 * 16 * 4);
    if constexpr (CS::kFp8) {
      // this wave's tile has landed: its 16 tokens x 4 block scales, transposed to [block][token]
      const int t = lane >> 2, k = lane & 3;
      ((float*)sct)[16 * (4 * wave + k) + t] = *(const float*)(tile_ptr(i, wave) + Fmt::pos(t, 32) + 4 * k);
    }
    __syncthreads();  // the step's four tiles are visible; every wave is done with step i - 1
    // The next tiles: into buffer (i - 1) % NB, free since the barrier, requested while the
    // scores' MFMAs execute (a burst of vector-memory instructions right after the barrier held
    // all four waves for about a microsecond per step).  bf16: the page ids of a later step and
    // the rows' addresses now, the row loads one instruction per K-step of the scores.
    const bool have_next = i + NB - 1 < nsteps;
    const uint8_t* next_rows[TPL];
    if constexpr (!CS::kFp8) {
      if (have_next) {
        const int s = i + NB - 1;
        fetch_page(tile_of_step(min(s + NB - 1, nsteps - 1)), slot_lds(s + NB - 1));
        Pages page_n;
        read_pages(pslot + 256 * (s % NB), page_n);
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
          const uint32_t tok = clamp_token(tile_of_step(s), Fmt::fetch_token(lane, t));
          next_rows[t] = p.cache + ((int64_t)page_n[t] * (int64_t)ps + (int64_t)(tok % ps)) * (int64_t)Fmt::kRowBytes;
        }
      }
    }
    // bf16: one row-load instruction after each K-step of the scores; the scores come in three
    // copies (streaming loads, cached loads, no next tile) chosen once per step, so that no
    // K-step branches.
    auto dma_nt = [&](int j) {
      if constexpr (!CS::kFp8) Fmt::issue_one(next_rows, buf_lds(i + NB - 1), lane, true, j);
    };
    auto dma_cached = [&](int j) {
      if constexpr (!CS::kFp8) Fmt::issue_one(next_rows, buf_lds(i + NB - 1), lane, false, j);
    };
    auto dma_none = [&](int) {};
    // fp8: the whole tile between the two halves of the scores.
    auto issue_next_fp8 = [&]() {
      if constexpr (CS::kFp8) {
        if (have_next) {
          const int s = i + NB - 1;
          fetch_page(tile_of_step(min(s + NB - 1, nsteps - 1)), slot_lds(s + NB - 1));
          issue_tile_flat(tile_of_step(s), pslot + 256 * (s % NB), buf_lds(s));
        }
      }
    };

    // ---- scores of row group `wave` over the step's four tiles, online softmax, P out.
    // The four tiles are four independent MFMA chains advanced one K-step at a time, so that
    // the LDS reads of the next K-steps can be in flight while a K-step's MFMAs run.
    f32x4 raw[4];
    if constexpr (CS::kFp8) {
      const uint8_t* const tl[4] = {tile_ptr(i, 0), tile_ptr(i, 1), tile_ptr(i, 2), tile_ptr(i, 3)};
      f32x4 part[4];  // the partner row group's partial scores
      score_tiles_half(tl, sct, m, g, kh, qf, qf + 9, raw, part, issue_next_fp8);
      // the partner's partial goes to its row group's slot (where its P goes next); ours arrives
      f32x4* xo = (f32x4*)pex + ((wave ^ 1) * 4) * 64 + lane;
#pragma unroll
      for (int v = 0; v < 4; ++v) xo[64 * v] = part[v];
      __syncthreads();
      const f32x4* xi = (const f32x4*)pex + (wave * 4) * 64 + lane;
#pragma unroll
      for (int v = 0; v < 4; ++v) raw[v] += xi[64 * v];
    } else {
      if (!have_next)
        score_tiles<Fmt>(tile_ptr(i, 0), tile_ptr(i, 1), tile_ptr(i, 2), tile_ptr(i, 3), m, g, qf, raw, dma_none);
      else if (p.stream_rows != 0)
        score_tiles<Fmt>(tile_ptr(i, 0), tile_ptr(i, 1), tile_ptr(i, 2), tile_ptr(i, 3), m, g, qf, raw, dma_nt);
      else
        score_tiles<Fmt>(tile_ptr(i, 0), tile_ptr(i, 1), tile_ptr(i, 2), tile_ptr(i, 3), m, g, qf, raw, dma_cached);
    }
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int valid = n_vis - (kWaves * i + v) * kTile;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[v][r] = (4 * g + r < valid) ? raw[v][r] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[v][r]);
      }
    }
    mx = max_over_rows(mx);
    const bool grow = mx > m_run + kRescaleThreshold;
    const bool any_grow = __builtin_amdgcn_ballot_w64(grow) != 0;
    if (any_grow) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
      m_run = m_new;
      if (g == 0) alpha_s[16 * wave + m] = alpha;
    }
    if (lane == 0) flag_s[wave] = any_grow ? 1 : 0;
    const float m_base = m_run == -INFINITY ? 0.f : m_run;
    float pr[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[v][r] = fast_exp2(sc[v][r] - m_base);
        l_run += pr[v][r];
      }
    if constexpr (CS::kFp8) {
      f32x4* dst = (f32x4*)pex + (wave * 4) * 64 + lane;
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[64 * v] = f32x4{pr[v][0], pr[v][1], pr[v][2], pr[v][3]};
    } else {
      u32x4* dst = (u32x4*)pex + (wave * 2) * 64 + lane;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        dst[64 * j] = u32x4{pack_bf16(pr[2 * j][0], pr[2 * j][1]), pack_bf16(pr[2 * j][2], pr[2 * j][3]),
                            pack_bf16(pr[2 * j + 1][0], pr[2 * j + 1][1]), pack_bf16(pr[2 * j + 1][2], pr[2 * j + 1][3])};
    }
    __syncthreads();  // P, alpha and the flags of all four row groups are visible

    // ---- rescales, then PV over this wave's columns for all four row groups
    const u32x4 fl = *(const u32x4*)flag_s;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (__builtin_amdgcn_readfirstlane(fl[r]) != 0) {
        const float a = alpha_s[16 * r + m];
        f32x4(&Or)[8] = *reinterpret_cast<f32x4(*)[8]>(&O[8 * r]);
        scale_acc(Or, a);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* ta = tile_ptr(i, 2 * j);
      const uint8_t* tb = tile_ptr(i, 2 * j + 1);
      if constexpr (CS::kFp8) {
        // All LDS reads of the tile pair first (one exposed latency): the scales of block `wave`
        // for this lane's tokens 4g .. 4g + 3 of tiles a and b, the four row groups' P, and the
        // codes of block `wave` (A operand: lanes v < 4 read tile a, v >= 4 tile b, as
        // Fp8Rows::pv2 does).
        const f32x4 sa = *(const f32x4*)(sct + (16 * (4 * (2 * j) + wave) + 4 * g) * 4);
        const f32x4 sb = *(const f32x4*)(sct + (16 * (4 * (2 * j + 1) + wave) + 4 * g) * 4);
        f32x4 pa[4], pb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pa[r] = ((const f32x4*)pex)[(r * 4 + 2 * j) * 64 + lane];
          pb[r] = ((const f32x4*)pex)[(r * 4 + 2 * j + 1) * 64 + lane];
        }
        const int v = m >> 1, h = m & 1;
        const uint8_t* src = (v < 4 ? ta : tb) + 8 * h + Fmt::pos(4 * g + (v & 3), 8 * wave);
        u32x2 cw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) cw[c] = lds_read_tr8(src + 16 * c);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 bp[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bp[r] = u32x4{pack_bf16(pa[r][0] * sa[0], pa[r][1] * sa[1]), pack_bf16(pa[r][2] * sa[2], pa[r][3] * sa[3]),
                        pack_bf16(pb[r][0] * sb[0], pb[r][1] * sb[1]), pack_bf16(pb[r][2] * sb[2], pb[r][3] * sb[3])};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 a = Fmt::widen_tr8(cw[c]);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[8 * r + c] = mfma_16x16x32(a, bp[r], O[8 * r + c]);
        }
        // P products and the first operand, then the MFMAs one at a time, each beside one
        // vector instruction (the next operand's widening)
        __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        }
      } else {
        u32x4 bp[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) bp[r] = ((const u32x4*)pex)[(r * 2 + j) * 64 + lane];
        const uint8_t* ba[4];
        Fmt::pv_bases(ta, m, g, ba);
        const int db = (int)(tb - ta);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          // global column tile 8 wave + c: base (c & 3), plus 2048 (2 wave + (c >> 2))
          const uint8_t* a0 = ba[c & 3] + 2048 * (2 * wave + (c >> 2));
          const u32x2 x = lds_read_tr16(a0), y = lds_read_tr16(a0 + db);
          const u32x4 a = {x[0], x[1], y[0], y[1]};
#pragma unroll
          for (int r = 0; r < 4; ++r) O[8 * r + c] = mfma_16x16x32(a, bp[r], O[8 * r + c]);
        }
      }
    }
  }

  // ---- epilogue: the owners publish (max, sum) of their rows; every wave writes its columns
  const float l_row = sum_over_rows(l_run);
  __syncthreads();  // every wave is done with the last step's P
  float* fin = (float*)pex;  // [row group][row]: max, then sum
  if (g == 0) {
    fin[16 * wave + m] = m_run;
    fin[64 + 16 * wave + m] = l_row;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 16 * r + m;
    const float M = fin[rr], l = fin[64 + rr];
    if (rr < R) {
      // no finite score: (+0, -inf), or NaN when every score was NaN (the sum is then NaN)
      const float f = M == -INFINITY ? 0.f : 1.0f / l;
      float* orow = out + (int64_t)rr * kLatent + 128 * wave + 4 * g;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f32x4 o = M == -INFINITY ? f32x4{l * 0.f, l * 0.f, l * 0.f, l * 0.f} : O[8 * r + c] * f;
        *(f32x4*)(orow + 16 * c) = o;
      }
      if (wave == 0 && g == 0)
        lse[rr] = (M == -INFINITY) ? -INFINITY + l : (M + fast_log2(l)) * 0.69314718055994530942f;
    }
  }
  report_checks(bad, p.check_status);
}

// Rows that take the column-split verify step (four row groups).
template <class Fmt, int G>
constexpr bool kColSplit = G == 4 && (std::is_same<Fmt, Bf16Rows<512, 64>>::value ||
                                      std::is_same<Fmt, Fp8Rows<64>>::value);

template <class Fmt, int G>
constexpr int kernel_smem_bytes() {
  if constexpr (kColSplit<Fmt, G>) {
    return ColSplit<Fmt>::kBytes > smem_bytes<Fmt>() ? ColSplit<Fmt>::kBytes : smem_bytes<Fmt>();
  } else {
    return smem_bytes<Fmt>();
  }
}

template <class Fmt, int G, bool kGla2, bool kAppend>
__device__ __forceinline__ void decode_rows(const DecodeParams& p, uint8_t* smem, int b, int64_t L, int64_t t0,
                                            int64_t t1, float* out, float* lse) {
  if constexpr (kColSplit<Fmt, G>) {
    static_assert(!kGla2, "GLA-g2 decodes one row group");
    decode_segment_cs<Fmt, kAppend>(p, smem, b, L, t0, t1, out, lse);
  } else {
    decode_segment<Fmt, G, kGla2, false, kAppend>(p, smem, b, L, t0, t1, out, lse);
  }
}

// Rows whose kernels also come in the form that writes the step's new rows (the append calls):
// the 576-value rows with their rope part.
template <class Fmt>
constexpr bool kAppendable = std::is_same<Fmt, Bf16Rows<512, 64>>::value || std::is_same<Fmt, Fp8Rows<64>>::value;

// Prefix sums over the requests of a batch of B <= kMaxBalancedBatch: out[0] = 0, out[b + 1] =
// out[b] + value(b).  Thread t takes requests 4t .. 4t + 3; the 256 sums are scanned with wave
// shuffles and a pass over the four wave totals (in `scratch`, kWaves values).  Ends with a
// workgroup barrier, so `out` is visible to every thread.
template <typename T, class F>
__device__ __forceinline__ void scan_requests(int B, F value, T* out, T* scratch) {
  constexpr int kPer = kMaxBalancedBatch / (kWaves * 64);
  const int t = threadIdx.x;
  T c[kPer];
  T sum = 0;
  // value() of an index clamped into [0, B) for every i, so that the loads behind it are issued
  // together (under a branch per i the compiler waited for each load in turn); the surplus
  // ones are then dropped.  value() may be called more than once for B - 1.
#pragma unroll
  for (int i = 0; i < kPer; ++i) c[i] = value(min(kPer * t + i, B - 1));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (kPer * t + i >= B) c[i] = T(0);
    sum += c[i];
  }
  T incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_up(incl, d, 64);
    if ((t & 63) >= d) incl += o;
  }
  if ((t & 63) == 63) scratch[t >> 6] = incl;
  __syncthreads();
  T run = incl - sum;
  for (int w = 0; w < (t >> 6); ++w) run += scratch[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kPer * t + i;
    if (b < B) {
      run += c[i];
      out[b + 1] = run;
    }
  }
  if (t == 0) out[0] = 0;
  __syncthreads();
}

// The b with pre[b] <= x < pre[b + 1] (pre non-decreasing, pre[0] <= x < pre[B]).
template <typename T>
__device__ __forceinline__ int find_request(const T* pre, int B, T x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Per-request partitions: grid (request, partition).  Without compaction the grid is
// partition-major (all requests' first partitions are dispatched first, then the second
// ones, ...).  With p.compact (a grid larger than one workgroup per compute unit, batch <=
// kMaxBalancedBatch) every workgroup first counts the batch's non-empty partitions in LDS and
// the dispatch index w is mapped onto them: workgroups 0 .. E - 1 take the E non-empty
// partitions (request-major), the rest write the empty ones' (0, -inf), so no non-empty
// partition waits behind empty ones for a compute unit.  The partial slots (s, b) and the
// merge are the same either way.
template <class Fmt, int G, bool kGla2 = false, bool kAppend = false>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kernel_smem_bytes<Fmt, G>()];
  constexpr int kOut = kGla2 ? 256 : Fmt::kLatent;
  int b = blockIdx.x;
  int s = blockIdx.y;
  int64_t L;
  uint32_t lbad = 0;  // checked build: a length outside [0, bt_stride * page_size]
  if (p.compact) {
    // Scratch in the tile memory, which the pipeline only uses after this prologue.
    static_assert(smem_bytes<Fmt>() >= (3 * kMaxBalancedBatch + 2 + 2 * kWaves) * 4, "compaction scratch");
    int32_t* len_s = (int32_t*)smem + 2 * kWaves;
    int32_t* full_s = len_s + kMaxBalancedBatch;       // prefix of non-empty partition counts
    int32_t* empty_s = full_s + kMaxBalancedBatch + 1;  // prefix of empty partition counts
    const int B = p.batch, S = p.num_splits;
    auto nonempty = [&](int r) -> int32_t {
      const int32_t Lr = (int32_t)checked_len(p.seq_lens[r], p.bt_stride, p.page_size, lbad);
      len_s[r] = Lr;
      return counted_partitions(Lr, p.page_size, p.bt_stride, S);
    };
    scan_requests<int32_t>(B, nonempty, full_s, (int32_t*)smem);
    scan_requests<int32_t>(
        B, [&](int r) -> int32_t { return S - (full_s[r + 1] - full_s[r]); }, empty_s, (int32_t*)smem + kWaves);
    report_checks(lbad, p.check_status);
    const int32_t w = (int32_t)(blockIdx.y * gridDim.x + blockIdx.x);
    const int32_t E = full_s[B];
    if (w >= E && p.skip_empty) return;  // an empty partition: nothing to write (uniform)
    if (w < E) {
      b = find_request(full_s, B, w);
      s = w - full_s[b];
    } else {
      const int32_t k = w - E;
      b = find_request(empty_s, B, k);
      s = (full_s[b + 1] - full_s[b]) + (k - empty_s[b]);
    }
    L = len_s[b];
    __syncthreads();  // the scratch is tile memory from here on
  } else {
    L = checked_len(p.seq_lens[b], p.bt_stride, p.page_size, lbad);
    report_checks(lbad, p.check_status);
  }
  const Range rg = partition(L, p.page_size, p.num_splits, s, p.bt_stride);
  if (p.skip_empty && rg.t0 >= rg.t1) return;  // empty partition, no partial (uniform)
  const int R = p.q_len * p.heads;
  const int64_t row_b = (int64_t)b * R;
  const bool split = p.num_splits > 1;
  float* out = split ? p.part_out + ((int64_t)s * p.batch * R + row_b) * kOut : p.out + row_b * kOut;
  float* lse = split ? p.part_lse + (int64_t)s * p.batch * R + row_b : p.lse + row_b;
  decode_rows<Fmt, G, kGla2, kAppend>(p, smem, b, L, rg.t0, rg.t1, out, lse);
}

// Decode over per-query index lists: grid (query token, partition).  Query t attends to the
// cache slots indices[t][0 .. topk) (p.block_table with row stride p.bt_stride = topk, read as
// a block table of page size 1); a negative entry selects nothing.  Every query's list has the
// same length topk, split into p.num_splits equal parts; each partition writes its partial,
// empty or not (a partition whose entries are all negative gives (0, -inf) like an empty one).
template <class Fmt>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_sparse_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<Fmt>()];
  const int b = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t L = p.bt_stride;
  const Range rg = partition(L, 1, p.num_splits, s, L);
  const int R = p.heads;
  const int64_t row_b = (int64_t)b * R;
  const bool split = p.num_splits > 1;
  float* out = split ? p.part_out + ((int64_t)s * p.batch * R + row_b) * Fmt::kLatent : p.out + row_b * Fmt::kLatent;
  float* lse = split ? p.part_lse + (int64_t)s * p.batch * R + row_b : p.lse + row_b;
  decode_segment<Fmt, 1, false, true>(p, smem, b, L, rg.t0, rg.t1, out, lse);
}

// Batch-balanced decode.  The batch's requests are laid end to end on a cost axis: request
// b occupies [v[b], v[b + 1]) with v[b + 1] - v[b] = kSegmentCost + L_b for L_b > 0 (0 for
// an empty request), its tokens at the last L_b positions; the first kSegmentCost stand
// for the start-up of a segment (first loads in flight, epilogue), measured at about as
// long as streaming that many rows.  (The single-token kernels that write the step's new
// rows add kAppendTail tokenless positions after the tokens, for the wait on those stores.)  The axis, of length V = v[B], is cut into W =
// min(gridDim.x, V) equal ranges [floor(wV/W), floor((w+1)V/W)); workgroup w decodes the
// tokens of every request its range meets (possibly none, when the range lies in a
// request's start-up part) into partial slot b + w (unique: along the axis, b or w grows at
// every segment start), so request b's partials are the slots b + w_first(b) .. b +
// w_last(b), at most B + W - 1 slots in all.  Every workgroup scans seq_lens into v itself
// (no planning launch, no dependent global reads before its first tile); workgroup 0 also
// stores v for the merge.  A slot holds the R = q_len x heads query rows of its request (G row
// groups of 16, as in decode_kernel).
// LDS of the axis v [kMaxBalancedBatch + 1] (and the scan's per-wave totals) when it is kept apart
// from the tile memory for the whole launch.
constexpr int kAxisBytes = (kWaves + kMaxBalancedBatch + 1) * 8;
template <class Fmt, int G>
constexpr bool kAxisApart = kernel_smem_bytes<Fmt, G>() + kAxisBytes <= 160 * 1024;

template <class Fmt, int G, bool kGla2 = false, bool kAppend = false>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_flat_kernel(DecodeParams p) {
  constexpr int kOut = kGla2 ? 256 : Fmt::kLatent;  // output values per query row
  constexpr int kTileMem = kernel_smem_bytes<Fmt, G>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[kTileMem + (kAxisApart<Fmt, G> ? kAxisBytes : 0)];
  // The grid size lives in another line of the kernel arguments than the fields read first: read
  // it here, with them, rather than after the scan, where its load would wait out a trip to
  // memory before the workgroup can find its range.
  const uint32_t grid_w = gridDim.x;
  asm volatile("" ::"s"(grid_w));
  const int B = p.batch;
  uint32_t lbad = 0;  // checked build: a length outside [0, bt_stride * page_size]
  constexpr int64_t kTail = (kAppend && G == 1) ? kAppendTail : 0;  // see kAppendTail
  auto cost = [&](int r) -> int64_t {
    const int64_t L = checked_len(p.seq_lens[r], p.bt_stride, p.page_size, lbad);
    return L > 0 ? L + kSegmentCost + kTail : 0;
  };
  // The axis v [B + 1] is scanned into LDS; each workgroup then keeps the start of its first
  // request and walks forward from there.  Where the LDS has room the axis stays apart from the
  // tile memory and the walk reads the next request's end from it; otherwise it is scanned into
  // the tile memory (used by the segments only after the scan) and the walk reads the lengths
  // again.
  static_assert(kTileMem >= kAxisBytes, "axis scratch");
  int64_t* axis = (int64_t*)(smem + (kAxisApart<Fmt, G> ? kTileMem : 0));
  int64_t* v_s = axis + kWaves;
  scan_requests<int64_t>(B, cost, v_s, axis);
  report_checks(lbad, p.check_status);
  if (blockIdx.x == 0)
    for (int b = threadIdx.x; b <= B; b += kWaves * 64) p.cu[b] = v_s[b];

  const int64_t V = v_s[B];
  const int64_t W = min((int64_t)grid_w, V);
  const int64_t w = blockIdx.x;
  if (w >= W) return;  // uniform over the workgroup
  const int64_t lo = flat_begin(V, W, w), hi = flat_begin(V, W, w + 1);
  int bl = 0, bh = B;  // v[bl] <= lo < v[bh]
  while (bh - bl > 1) {
    const int mid = (bl + bh) >> 1;
    if (v_s[mid] <= lo) bl = mid; else bh = mid;
  }
  int64_t v0 = v_s[bl];
  __syncthreads();  // the scratch is tile memory from here on
  const int R = p.q_len * p.heads;
  for (int b = bl; b < B; ++b) {
    const int64_t v1 = kAxisApart<Fmt, G> ? v_s[b + 1] : v0 + cost(b);
    if (v0 >= hi) break;
    if (v1 <= lo || v1 == v0) {  // empty requests have no partial
      v0 = v1;
      continue;
    }
    const int64_t s0 = v0 + kSegmentCost;  // axis position of token 0
    const int64_t L = v1 - s0 - kTail;
    // Token boundaries fall on multiples of 16 (a tile), so that the tiles of a segment start
    // where a page's tiles do; both workgroups that share a boundary round it alike.
    auto on_tile = [&](int64_t t) -> int64_t { return t >= L ? L : t & ~(int64_t)(kTile - 1); };
    const int64_t t0 = on_tile(max(lo, s0) - s0);
    const int64_t t1 = on_tile(max(min(hi, v1) - s0, (int64_t)0));  // 0: the range holds start-up only
    const int64_t slot = (int64_t)b + w;
    decode_rows<Fmt, G, kGla2, kAppend>(p, smem, b, L, t0, max(t0, t1), p.part_out + slot * R * kOut,
                               p.part_lse + slot * R);
    __syncthreads();  // the epilogue's LDS reads finish before the next segment's loads land
    v0 = v1;
  }
}

template <class Fmt, bool kAppend>
hipError_t launch_rows(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.batch, (unsigned)p.num_splits);
  const int R = p.q_len * p.heads;
  if (R <= 16)
    hipLaunchKernelGGL((decode_kernel<Fmt, 1, false, kAppend>), grid, dim3(kWaves * 64), 0, stream, p);
  else if (R <= 32)
    hipLaunchKernelGGL((decode_kernel<Fmt, 2, false, kAppend>), grid, dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<Fmt, 4, false, kAppend>), grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

// The per-request launch; with the step's new rows (p.new_latent) the kernels that write them.
template <class Fmt>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  if constexpr (kAppendable<Fmt>) {
    if (p.new_latent != nullptr) return launch_rows<Fmt, true>(p, stream);
  }
  if (p.new_latent != nullptr) return hipErrorInvalidValue;
  return launch_rows<Fmt, false>(p, stream);
}

// Balanced launches: one row group per 16 of the R = q_len x heads query rows (kMaxG = 1: the
// single-token geometries).
template <class Fmt, int kMaxG, bool kAppend>
hipError_t launch_flat_rows(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  const int R = p.q_len * p.heads;
  const dim3 grid((unsigned)num_workgroups), block(kWaves * 64);
  if (kMaxG == 1 || R <= 16)
    hipLaunchKernelGGL((decode_flat_kernel<Fmt, 1, false, kAppend>), grid, block, 0, stream, p);
  else if (R <= 32)
    hipLaunchKernelGGL((decode_flat_kernel<Fmt, kMaxG >= 2 ? 2 : 1, false, kAppend>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_flat_kernel<Fmt, kMaxG, false, kAppend>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <class Fmt, int kMaxG>
hipError_t launch_flat(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  if constexpr (kAppendable<Fmt>) {
    if (p.new_latent != nullptr) return launch_flat_rows<Fmt, kMaxG, true>(p, num_workgroups, stream);
  }
  if (p.new_latent != nullptr) return hipErrorInvalidValue;
  return launch_flat_rows<Fmt, kMaxG, false>(p, num_workgroups, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  return launch<Bf16Rows<512, 64>>(p, stream);
}
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream) { return launch<Fp8Rows<64>>(p, stream); }
hipError_t launch_decode_nope_bf16(const DecodeParams& p, hipStream_t stream) {
  return launch<Bf16Rows<512, 0>>(p, stream);
}
// Single-token decodes of the other geometries (at most 16 query rows: one row group).
hipError_t launch_decode_rank256_bf16(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<Bf16Rows<256, 64>, 1>), dim3((unsigned)p.batch, (unsigned)p.num_splits),
                     dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}
hipError_t launch_decode_gla2_bf16(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<Bf16Rows<512, 64>, 1, true>), dim3((unsigned)p.batch, (unsigned)p.num_splits),
                     dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}
hipError_t launch_decode_gla2_fp8(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<Fp8Rows<64>, 1, true>), dim3((unsigned)p.batch, (unsigned)p.num_splits),
                     dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}
hipError_t launch_decode_flat_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  return launch_flat<Bf16Rows<512, 64>, 4>(p, num_workgroups, stream);
}
hipError_t launch_decode_flat_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  return launch_flat<Fp8Rows<64>, 4>(p, num_workgroups, stream);
}
hipError_t launch_decode_flat_nope_bf16(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  return launch_flat<Bf16Rows<512, 0>, 1>(p, num_workgroups, stream);
}
hipError_t launch_decode_flat_nope_fp8(const DecodeParams& p, int num_workgroups, hipStream_t stream) {
  return launch_flat<Fp8Rows<0>, 1>(p, num_workgroups, stream);
}
// GLA-g2 heads under the batch-balanced schedule (one row group; 256-value partial rows).
hipError_t launch_decode_flat_gla2(const DecodeParams& p, int fp8, int num_workgroups, hipStream_t stream) {
  const dim3 grid((unsigned)num_workgroups), block(kWaves * 64);
  if (fp8)
    hipLaunchKernelGGL((decode_flat_kernel<Fp8Rows<64>, 1, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_flat_kernel<Bf16Rows<512, 64>, 1, true>), grid, block, 0, stream, p);
  return hipGetLastError();
}
hipError_t launch_decode_nope_fp8(const DecodeParams& p, hipStream_t stream) {
  return launch<Fp8Rows<0>>(p, stream);
}
// Index-list decodes: p.batch query tokens of at most 16 heads, p.q_len = 1, p.page_size = 1,
// p.bt_stride = topk.  Formats 0 bf16, 1 fp8 656-byte rows; nope: scores over the latent only.
hipError_t launch_decode_sparse(const DecodeParams& p, int fp8, int nope, hipStream_t stream) {
  const dim3 grid((unsigned)p.batch, (unsigned)p.num_splits), block(kWaves * 64);
  if (!fp8 && !nope)
    hipLaunchKernelGGL((decode_sparse_kernel<Bf16Rows<512, 64>>), grid, block, 0, stream, p);
  else if (!fp8)
    hipLaunchKernelGGL((decode_sparse_kernel<Bf16Rows<512, 0>>), grid, block, 0, stream, p);
  else if (!nope)
    hipLaunchKernelGGL((decode_sparse_kernel<Fp8Rows<64>>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_sparse_kernel<Fp8Rows<0, true>>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla

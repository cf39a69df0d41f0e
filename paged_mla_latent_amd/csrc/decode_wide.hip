// Decode over wide latent rows: rank-768 and rank-1792 layers (qwen-mla-vllm, "How it
// works": per-layer latent ranks 256 / 768 / 1792 with a small rotary tail).  Row: kLat
// latent values then 64 rope values, bf16; q [B][H][kLat + 64]; out [B][H][kLat].
//
//   s_t = scale * <q[b,h], row_t>  over all kLat + 64 values,
//   out[b,h] = sum_t softmax(s)_t * row_t[0:kLat],  lse[b,h] = ln sum_t exp(s_t)
//
// A 16-token tile is 26 KB (768) or 58 KB (1792), and a 16-head output tile over kLat
// columns would need kLat / 4 accumulator registers per lane, so the per-wave tiles of the
// 512-wide kernel do not fit.  Here the four waves of a workgroup share every tile and split
// both contractions:
//  * QK: wave w owns K-steps [j0(w), j1(w)) of the row (32 values each) and also fetches
//    exactly the row bytes of those K-steps, so its partial scores need only its own loads.
//    Rank 1792 (kLine): tiles in the line layout of mla_device.h, DMA instruction 2l + h
//    carrying 128-byte line l of tokens 8h .. 8h + 7 (whole lines, non-temporal unless cached
//    loads were asked for), a wave owning whole lines (7, 7, 7, 8 of 29).  Rank 768: tiles
//    in the chunk layout, DMA instruction j carrying the 64 bytes of K-step j of all 16
//    tokens (6, 6, 7, 7 K-steps); split into whole lines (3, 3, 3, 4 of 13) the widest slice
//    delays every step's barrier, measured 5 % slower than the streaming hint gains.
//    The four partial 16 x 16 score tiles are summed through LDS after one
//    workgroup barrier per tile; every wave sums them in the same order, so all waves hold
//    identical scores and softmax state.
//  * PV: wave w accumulates output columns [w kLat / 4, (w + 1) kLat / 4) (48 or 112
//    accumulator registers per lane) and writes them itself; no cross-wave merge.
// The pages' kernels take two passes for rank 1792 where one pass does not fit their
// shared memory; with this split one pass fits in 129 KB of LDS.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;

template <int kLat>
struct Wide {
  static_assert(kLat == 768 || kLat == 1792, "wide latent ranks");
  static constexpr int kQDim = kLat + 64;             // values per row and per query head
  static constexpr int kRowBytes = 2 * kQDim;         // 1,664 / 3,712
  static constexpr int kOps = kQDim / 32;             // DMA instructions = QK K-steps per tile: 26 / 58
  static constexpr int kLines = kOps / 2;             // 128-byte lines per row: 13 / 29
  static constexpr bool kLine = kLat == 1792;         // line layout and whole-line wave slices
  static constexpr int kTileBytes = kOps * 1024;      // 26,624 / 59,392
  static constexpr int kBufs = kLat == 768 ? 4 : 2;   // shared tiles resident: 104 / 116 KB (5 for 768: slower)
  static constexpr int kColGroups = kLat / 64;        // 16-column groups per wave: 12 / 28
  // K-steps of the widest wave slice: 7 (rank 768) / 16 (rank 1792, whole lines); the others
  // have one (768) or two (1792) fewer.
  static constexpr int kMaxSteps = kLine ? 2 * ((kLines + 3) / 4) : (kOps + 3) / 4;
  static constexpr int kSlack = kLine ? 2 : 1;
  static constexpr int kPidBytes = kWaves * kBufs * 256;
  static constexpr int kXchBytes = 2 * kWaves * 64 * 16;  // double-buffered partial scores
  static constexpr int kSmem = kBufs * kTileBytes + kPidBytes + kXchBytes;
  __device__ static constexpr int j0(int w) { return kLine ? 2 * ((kLines * w) >> 2) : (kOps * w) >> 2; }
};

// vmcnt wait with a count that depends on the wave's slice width (wave-uniform branch).
template <int kBig, int kSmall>
__device__ __forceinline__ void wait_vmcnt_for(bool big) {
  if (big)
    wait_vmcnt<kBig>();
  else
    wait_vmcnt<kSmall>();
}

template <int kLat>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_wide_kernel(DecodeParams p) {
  using Wd = Wide<kLat>;
  constexpr int NB = Wd::kBufs;
  constexpr int QS = Wd::kMaxSteps;
  constexpr int NU = Wd::kColGroups;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Wd::kSmem];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;  // head of this lane in the score / output tiles
  const int g = lane >> 4;  // token group of this lane (tokens 4g .. 4g + 3)
  const int b = blockIdx.x;
  const int s = blockIdx.y;
  const int H = p.heads;

  uint32_t bad = 0;  // checked build: MLA_CHECK_* bits of this lane's length and block ids
  const int64_t L = checked_len(p.seq_lens[b], p.bt_stride, p.page_size, bad);
  report_checks(bad, p.check_status);
  const Range rg = partition(L, p.page_size, p.num_splits, s, p.bt_stride);
  const int n = (int)(rg.t1 - rg.t0);
  const int ntiles = (n + kTile - 1) / kTile;
  if (p.skip_empty && n == 0) return;  // empty partition: no partial (the merge counts)

  const int j0 = Wd::j0(wave), j1 = Wd::j0(wave + 1);
  const int nj = j1 - j0;  // QS or QS - kSlack
  const bool big = nj == QS;

  // q as the B operand of the QK MFMA for this wave's K-steps: qf[i] = q[m][32 (j0 + i) + 8g ..].
  u32x4 qf[QS];
#pragma unroll
  for (int i = 0; i < QS; ++i) qf[i] = u32x4{0u, 0u, 0u, 0u};
  if (m < H) {
    const uint16_t* qrow = p.q + ((int64_t)b * H + m) * Wd::kQDim + 8 * g;
#pragma unroll
    for (int i = 0; i < QS; ++i)
      if (i < nj) qf[i] = *(const u32x4*)(qrow + 32 * (j0 + i));
  }

  float m_run = -INFINITY;  // running max (log2 domain) of head m; the same in every wave
  float l_run = 0.f;        // this lane's share (tokens 4g .. 4g + 3 of each tile) of the sum
  f32x4 O[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const uint32_t ps = (uint32_t)p.page_size;
  // Page ids: lane l fetches the page of token l >> 2 (token T's entry at byte 16T of a slot).
  // Rows, line layout: lane l fetches tokens l >> 3 and 8 + (l >> 3), chunk (l & 7) ^
  // line_swz(l >> 3) of each line; chunk layout: token l >> 2, chunk (l & 3) ^ swz(l >> 2) of
  // each 64-byte segment.
  constexpr int TPL = Wd::kLine ? 2 : 1;
  const int my_tok = lane >> 2;
  const int row_tok = Wd::kLine ? lane >> 3 : lane >> 2;
  const uint32_t t0 = (uint32_t)rg.t0;
  const uint32_t tlast = (uint32_t)(rg.t1 - 1);
  auto clamp_token = [&](int k, int within) -> uint32_t {  // clamped into the partition (ragged tail)
    const uint32_t t = t0 + (uint32_t)k * kTile + (uint32_t)within;
    return t > tlast ? tlast : t;
  };
  auto lane_token = [&](int k) -> uint32_t { return clamp_token(k, my_tok); };
  const uint32_t tiles_lds = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  uint8_t* pslot = smem + NB * Wd::kTileBytes + wave * NB * 256;
  const uint32_t plds = __builtin_amdgcn_readfirstlane(lds_offset(pslot));
  f32x4* xch = (f32x4*)(smem + NB * Wd::kTileBytes + Wd::kPidBytes);

  auto fetch_page = [&](int k, int slot) { dma4(bt + lane_token(k) / ps, plds + 256 * slot); };
  // This wave's DMA instructions (K-steps j0 .. j1 - 1) of tile k into buffer `buf`; page[h] is
  // the page of token row_tok + 8h.  Line layout: instruction j reads line j >> 1 of token
  // half j & 1 (j0 is even).
  const int cv = Wd::kLine ? 16 * ((lane & 7) ^ line_swz(row_tok)) : 16 * ((lane & 3) ^ swz(row_tok));
  auto issue = [&](int k, const int32_t (&page)[TPL], int buf) {
    const uint8_t* src[TPL];
#pragma unroll
    for (int h = 0; h < TPL; ++h) {
      const uint32_t tok = clamp_token(k, row_tok + 8 * h);
      const int64_t slot = (int64_t)page[h] * (int64_t)ps + (int64_t)(tok % ps);
      src[h] = p.cache + slot * (int64_t)Wd::kRowBytes + cv;
    }
    const uint32_t dst = tiles_lds + buf * Wd::kTileBytes;
    if constexpr (Wd::kLine) {
      if (p.stream_rows) {
#pragma unroll
        for (int i = 0; i < QS; ++i)
          if (i < nj) dma16_nt(src[i & 1] + 64 * (j0 + i - (i & 1)), dst + 1024 * (j0 + i));
      } else {
#pragma unroll
        for (int i = 0; i < QS; ++i)
          if (i < nj) dma16(src[i & 1] + 64 * (j0 + i - (i & 1)), dst + 1024 * (j0 + i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < QS; ++i)
        if (i < nj) dma16(src[0] + 64 * (j0 + i), dst + 1024 * (j0 + i));
    }
  };
  auto read_pages = [&](int slot, int32_t (&page)[TPL]) {
#pragma unroll
    for (int h = 0; h < TPL; ++h)
      page[h] = checked_page(*(const int32_t*)(pslot + 256 * slot + 16 * (row_tok + 8 * h)), p.num_pages, bad);
  };
  // Chunk c of token t in a tile: line_pos or chunk_pos.
  auto pos = [&](int tk, int c) { return Wd::kLine ? line_pos(tk, c) : chunk_pos(tk, c); };

  // Partial scores of tile buffer `buf` over this wave's K-steps, into the exchange slot.
  // K-step j = j0 + i reads chunk 4j + g of token m: line layout (j0 even) at
  // line_pos(m, 4 (j & 1) + g) + 128 (j >> 1), chunk layout at chunk_pos(m, g) + 64 j.
  auto qk_partial = [&](int buf, int k) {
    const uint8_t* tile = smem + buf * Wd::kTileBytes + 1024 * j0;
    const uint8_t* base0 = tile + 16 * pos(m, g);
    const uint8_t* base1 = Wd::kLine ? tile + 16 * line_pos(m, 4 + g) : base0 + 1024;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int i = 0; i < QS; i += 2) {
      if (i < nj) s0 = mfma_16x16x32(*(const u32x4*)(base0 + 1024 * i), qf[i], s0);
      if (i + 1 < nj) s1 = mfma_16x16x32(*(const u32x4*)(base1 + 1024 * i), qf[i + 1], s1);
    }
    xch[((k & 1) * kWaves + wave) * 64 + lane] = s0 + s1;
  };

  // After the barrier: full scores, online softmax, PV over this wave's columns.
  auto finish_tile = [&](int buf, int k) {
    const f32x4* x = xch + (k & 1) * kWaves * 64 + lane;
    const f32x4 raw = ((x[0] + x[64]) + x[128]) + x[192];  // fixed order: identical in every wave
    const int valid = n - k * kTile;
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = (4 * g + r < valid) ? raw[r] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[r]);
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
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sc[r] - m_base);
      l_run += pr[r];
    }
    // PV: column group u of this wave is global group wave * NU + u (values 16 (.) .. +16, chunks
    // 2 (.) + {0, 1}); NU is a multiple of 4, so group u sits at pos(t, 2 (u & 3) + cc) +
    // 128 (wave NU / 4 + (u >> 2)) in either layout.
    const u32x2 pb = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
    const int t = 4 * g + (m >> 2);
    const int cc = (m >> 1) & 1;
    const uint8_t* tile = smem + buf * Wd::kTileBytes + 2048 * (wave * NU / 4) + 8 * (m & 1);
    const uint8_t* bs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bs[r] = tile + 16 * pos(t, 2 * r + cc);
#pragma unroll
    for (int u = 0; u < NU; ++u) O[u] = mfma_16x16x16(lds_read_tr16(bs[u & 3] + 2048 * (u >> 2)), pb, O[u]);
  };

  // Pipeline over the shared tiles i = 0, 1, ...  Step i issues the page ids of tile
  // i + 2(NB - 1) and this wave's DMAs of tile i + NB - 1, so each wave's queue reads
  //     ... PID(i + NB - 1) DMA(i) PID(i + NB) DMA(i + 1) ...
  // and the wait for DMA(i) (at most (NB - 2)(nj + 1) younger operations) also covers the
  // page ids the step consumes.  A barrier per step makes tile i (loaded in four slices) and
  // its partial scores visible to every wave, and tells every wave that the others are done
  // with tile i - 1, whose buffer the step's DMAs then overwrite.
  int32_t page_first[NB - 1][TPL];
#pragma unroll
  for (int t = 0; t < NB - 1; ++t)
#pragma unroll
    for (int h = 0; h < TPL; ++h)
      page_first[t][h] = (t < ntiles) ? checked_page(bt[clamp_token(t, row_tok + 8 * h) / ps], p.num_pages, bad) : 0;
#pragma unroll
  for (int i = 0; i < QS; ++i) asm volatile("" : "+a"(qf[i]));
#pragma unroll
  for (int t = 0; t < NB - 1; ++t)
#pragma unroll
    for (int h = 0; h < TPL; ++h) asm volatile("" ::"v"(page_first[t][h]));
  int i = 0;
  if (ntiles > 0) {
#pragma unroll
    for (int t = 0; t < NB - 1; ++t) {
      fetch_page(min(t + NB - 1, ntiles - 1), (t + NB - 1) % NB);
      if (t < ntiles) issue(t, page_first[t], t);
    }
#pragma unroll 1
    for (; i + NB - 1 < ntiles; ++i) {
      wait_vmcnt_for<(NB - 2) * (QS + 1), (NB - 2) * (QS + 1 - Wd::kSlack)>(big);  // slices of QS or QS - kSlack
      const int cur = i % NB;
      qk_partial(cur, i);
      __syncthreads();
      const int ahead = (i + NB - 1) % NB;
      int32_t page_n[TPL];
      read_pages(ahead, page_n);
      fetch_page(min(i + 2 * (NB - 1), ntiles - 1), (i + 2 * (NB - 1)) % NB);
      issue(i + NB - 1, page_n, ahead);
      finish_tile(cur, i);
    }
    wait_vmcnt<0>();
#pragma unroll 1
    for (; i < ntiles; ++i) {
      const int cur = i % NB;
      qk_partial(cur, i);
      __syncthreads();
      finish_tile(cur, i);
    }
  }

  // Finalize this wave's columns: out = O / l, lse = ln sum; no token: (+0, -inf); a NaN
  // score anywhere: NaN (the running max ignores NaN, the sum does not).
  const float l = sum_over_rows(l_run);
  const bool split = p.num_splits > 1;
  const int64_t row = (split ? ((int64_t)s * p.batch + b) : (int64_t)b) * H + m;
  float* out = (split ? p.part_out : p.out) + row * kLat + wave * (kLat / 4);
  float* lse = (split ? p.part_lse : p.lse) + row;
  const float f = m_run == -INFINITY ? l : 1.0f / l;
  if (m < H) {
#pragma unroll
    for (int u = 0; u < NU; ++u) *(f32x4*)(out + 16 * u + 4 * g) = O[u] * f;
    if (wave == 0 && g == 0)
      *lse = m_run == -INFINITY ? -INFINITY + l : (m_run + fast_log2(l)) * 0.69314718055994530942f;
  }
  report_checks(bad & kCheckBlockId, p.check_status);
}

}  // namespace

hipError_t launch_decode_rank768_bf16(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_wide_kernel<768>, dim3((unsigned)p.batch, (unsigned)p.num_splits), dim3(kWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}
hipError_t launch_decode_rank1792_bf16(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_wide_kernel<1792>, dim3((unsigned)p.batch, (unsigned)p.num_splits), dim3(kWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace mla

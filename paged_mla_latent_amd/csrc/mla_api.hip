// C ABI of libmla.so (declared in include/mla.h): host-side argument validation,
// device-architecture check and kernel launches.  No allocation, no synchronisation.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local char g_message[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_message, sizeof(g_message), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, -1 other; and of the
// compute-unit count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(MLA_ERR_ARCH, "no usable HIP device (hipGetDevice: %s)", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(MLA_ERR_ARCH, "device index %d exceeds %d", dev, kMaxDevices);
  int state = g_arch[dev].load(std::memory_order_acquire);  // pairs with the release below
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MLA_ERR_ARCH, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch[dev].store(state, std::memory_order_release);  // g_cus is visible once g_arch is
    if (state < 0)
      return fail(MLA_ERR_ARCH, "device %d is %s; this library is built for gfx950 (MI355X) only", dev,
                  prop.gcnArchName);
  }
  if (state < 0) return fail(MLA_ERR_ARCH, "device %d is not gfx950 (MI355X)", dev);
  return MLA_OK;
}

// Compute units of the current device (after check_device succeeded).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  return g_cus[dev].load(std::memory_order_relaxed);
}

// The per-call options of the decodes: known flag bits only; check_status only in the
// checked build (the release build tests nothing and must not pretend to).
int check_options(const char* fn, uint32_t flags, const int32_t* check_status) {
  if (flags & ~(uint32_t)MLA_FLAG_CACHED_ROWS)
    return fail(MLA_ERR_SHAPE, "%s: unknown flag bits 0x%x", fn, flags & ~(uint32_t)MLA_FLAG_CACHED_ROWS);
  if (check_status) {
    if (!mla::kChecked)
      return fail(MLA_ERR_SHAPE, "%s: check_status needs the checked build (libmla_checked.so)", fn);
    if ((reinterpret_cast<uintptr_t>(check_status) & 3u) != 0)
      return fail(MLA_ERR_ALIGN, "%s: check_status must be 4-byte aligned", fn);
  }
  return MLA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Partials [splits][batch][rows][width] then [splits][batch][rows] fp32.
size_t workspace_bytes_for(int64_t batch, int64_t heads, int64_t splits, int64_t width = MLA_LATENT) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)splits * (size_t)batch * (size_t)heads;
  const size_t bytes = n * (size_t)(width + 1) * sizeof(float) + 64;  // + lse alignment slack
  return (bytes + 255) & ~(size_t)255;
}

// Scratch of mla_decode_bf16_noalloc: the split partials of one call, one copy per device,
// held until the process ends.  Its name is a host-side stand-in, never a device address:
// host code uses only the per-device address from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static_assert(kNoAllocScratchBytes == (size_t)MLA_NOALLOC_SCRATCH_BYTES, "scratch size in mla.h");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's scratch, looked up once per device with that device
// current.  No allocation: the array is part of the loaded code object.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_ARCH, "mla_decode_bf16_noalloc: no usable HIP device (%s)", hipGetErrorString(e));
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return fail(MLA_ERR_HIP, "mla_decode_bf16_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MLA_OK;
}

// Kinds of decode: row format and whether the rope part takes part in the scores.
enum DecodeKind {
  kBf16 = 0, kFp8 = 1, kNopeBf16 = 2, kNopeFp8 = 3, kRank256Bf16 = 4, kGla2Bf16 = 5, kGla2Fp8 = 6,
  kRank768Bf16 = 7, kRank1792Bf16 = 8
};

// The step's new rows of the mla_decode_append_* calls (the cache write fused into the decode).
struct AppendArgs {
  const void* new_latent;
  const void* new_k_pe;
  const int64_t* new_slots;
  void* kv_cache;
};

int check_append(const char* fn, const AppendArgs* app) {
  if (!app) return MLA_OK;
  if (!app->new_latent) return fail(MLA_ERR_NULL, "%s: new_latent is NULL", fn);
  if (!app->new_slots) return fail(MLA_ERR_NULL, "%s: new_slots is NULL", fn);
  if (!aligned16(app->new_latent) || !aligned16(app->new_k_pe) || !aligned16(app->new_slots))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  return MLA_OK;
}

void set_append(mla::DecodeParams& p, const AppendArgs* app) {
  if (!app) return;
  p.new_latent = static_cast<const uint16_t*>(app->new_latent);
  p.new_k_pe = static_cast<const uint16_t*>(app->new_k_pe);
  p.new_slots = app->new_slots;
  p.cache_w = static_cast<uint8_t*>(app->kv_cache);
}

int decode_common(int kind, int32_t q_len, const void* q, const void* kv_cache, int64_t num_pages,
                  const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                  int32_t batch, int32_t num_heads, int32_t page_size, float softmax_scale,
                  int32_t num_splits, float* out, float* lse, void* workspace, size_t workspace_bytes,
                  uint32_t flags, int32_t* check_status, void* stream, bool use_scratch = false,
                  const AppendArgs* app = nullptr) {
  static const char* const kNames[] = {"mla_decode_bf16",         "mla_decode_fp8_656",
                                       "mla_decode_nope_bf16",    "mla_decode_nope_fp8_656",
                                       "mla_decode_rank256_bf16", "mla_decode_gla2_bf16",
                                       "mla_decode_gla2_fp8_656", "mla_decode_rank768_bf16",
                                       "mla_decode_rank1792_bf16"};
  const bool gla = kind == kGla2Bf16 || kind == kGla2Fp8;
  const bool wide = kind == kRank768Bf16 || kind == kRank1792Bf16;
  const int out_width = (kind == kRank256Bf16 || gla) ? 256
                        : kind == kRank768Bf16        ? 768
                        : kind == kRank1792Bf16       ? 1792
                                                      : MLA_LATENT;
  const char* fn = use_scratch ? "mla_decode_bf16_noalloc"
                   : app         ? (kind == kBf16 ? "mla_decode_append_bf16" : "mla_decode_append_fp8_656")
                   : q_len == 1  ? kNames[kind]
                                 : (kind == kBf16 ? "mla_decode_mtp_bf16" : "mla_decode_mtp_fp8_656");
  if (int rc0 = check_options(fn, flags, check_status)) return rc0;
  if (int rc0 = check_append(fn, app)) return rc0;
  if (!q) return fail(MLA_ERR_NULL, "%s: q is NULL", fn);
  if (!kv_cache) return fail(MLA_ERR_NULL, "%s: kv_cache is NULL", fn);
  if (!block_table) return fail(MLA_ERR_NULL, "%s: block_table is NULL", fn);
  if (!seq_lens) return fail(MLA_ERR_NULL, "%s: seq_lens is NULL", fn);
  // out == lse == NULL with num_splits > 1 leaves the partials in the workspace (no merge).
  const bool partials_only = !out && !lse && num_splits > 1 && !use_scratch;
  if (!out && !partials_only) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse && !partials_only) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (batch < 1 || batch > 65535) return fail(MLA_ERR_SHAPE, "%s: batch=%d outside [1, 65535]", fn, batch);
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d outside [1, %d]", fn, num_heads, MLA_MAX_HEADS);
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN)
    return fail(MLA_ERR_SHAPE, "%s: q_len=%d outside [1, %d]", fn, q_len, MLA_MAX_Q_LEN);
  if (gla && num_heads % 2)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d must be even (two head groups)", fn, num_heads);
  if (q_len * num_heads > MLA_MAX_QUERY_ROWS)
    return fail(MLA_ERR_SHAPE, "%s: q_len * num_heads = %d exceeds %d", fn, q_len * num_heads, MLA_MAX_QUERY_ROWS);
  if (page_size < 1) return fail(MLA_ERR_SHAPE, "%s: page_size=%d must be >= 1", fn, page_size);
  if (num_pages < 1) return fail(MLA_ERR_SHAPE, "%s: num_pages=%lld must be >= 1", fn, (long long)num_pages);
  if (block_table_stride < 1)
    return fail(MLA_ERR_SHAPE, "%s: block_table_stride=%lld must be >= 1", fn, (long long)block_table_stride);
  if (block_table_stride > ((int64_t)1 << 31) / page_size + 1)
    return fail(MLA_ERR_SHAPE, "%s: block_table_stride * page_size exceeds the int32 token range", fn);
  if (num_splits < 1 || num_splits > 65535)
    return fail(MLA_ERR_SHAPE, "%s: num_splits=%d outside [1, 65535]", fn, num_splits);
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_SHAPE, "%s: softmax_scale is not finite", fn);
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(block_table) || !aligned16(seq_lens) ||
      !aligned16(out) || !aligned16(lse))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  float* part_out = nullptr;
  float* part_lse = nullptr;
  if (num_splits > 1 && use_scratch) {
    // the library's per-device scratch stands in for the workspace
    const size_t need = workspace_bytes_for(batch, num_heads, num_splits);
    if (need > kNoAllocScratchBytes)
      return fail(MLA_ERR_WORKSPACE,
                  "%s: %d splits x %d requests x %d heads need %zu bytes of partials, more than the %zu-byte "
                  "scratch; use mla_decode_bf16 with a workspace",
                  fn, num_splits, batch, num_heads, need, kNoAllocScratchBytes);
    int rc = check_device();
    if (rc != MLA_OK) return rc;
    rc = scratch_address(&workspace);
    if (rc != MLA_OK) return rc;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (num_splits > 1) {
    // the 256-wide outputs keep the 512-wide workspace size of the first ABI version
    const size_t need = workspace_bytes_for(batch, (int64_t)q_len * num_heads, num_splits, wide ? out_width : MLA_LATENT);
    if (!workspace) return fail(MLA_ERR_WORKSPACE, "%s: num_splits=%d needs a workspace", fn, num_splits);
    if (!aligned16(workspace)) return fail(MLA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
    part_out = static_cast<float*>(workspace);
    part_lse = part_out + (size_t)num_splits * batch * q_len * num_heads * out_width;
  }
  int rc = check_device();
  if (rc != MLA_OK) return rc;

  mla::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.cache = static_cast<const uint8_t*>(kv_cache);
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.heads = num_heads;
  p.q_len = q_len;
  p.page_size = page_size;
  p.num_splits = num_splits;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.out = out;
  p.lse = lse;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.cu = nullptr;
  // More workgroups than compute units: put the non-empty partitions first (see decode_kernel).
  p.compact = batch <= MLA_MAX_BALANCED_BATCH && (int64_t)batch * num_splits > device_cus();
  // Merged here: empty partitions need not leave the (0, -inf) partial that a caller's own merge
  // of the workspace would read.
  p.skip_empty = num_splits > 1 && !partials_only;
  p.stream_rows = (flags & MLA_FLAG_CACHED_ROWS) == 0;
  p.num_pages = num_pages;
  p.check_status = check_status;
  set_append(p, app);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t launched;
  switch (kind) {
    case kBf16: launched = mla::launch_decode_bf16(p, s); break;
    case kFp8: launched = mla::launch_decode_fp8(p, s); break;
    case kNopeBf16: launched = mla::launch_decode_nope_bf16(p, s); break;
    case kNopeFp8: launched = mla::launch_decode_nope_fp8(p, s); break;
    case kRank256Bf16: launched = mla::launch_decode_rank256_bf16(p, s); break;
    case kGla2Bf16: launched = mla::launch_decode_gla2_bf16(p, s); break;
    case kRank768Bf16: launched = mla::launch_decode_rank768_bf16(p, s); break;
    case kRank1792Bf16: launched = mla::launch_decode_rank1792_bf16(p, s); break;
    default: launched = mla::launch_decode_gla2_fp8(p, s); break;
  }
  rc = hip_status(launched, fn);
  if (rc != MLA_OK || num_splits == 1 || partials_only) return rc;
  return hip_status(mla::launch_merge_counted(part_out, part_lse, num_splits, batch, q_len * num_heads, out_width,
                                              seq_lens, page_size, block_table_stride, out, lse, s),
                    "mla_merge_lse (after decode)");
}

// Batch-balanced workspace: int64 prefix sums [batch + 1] (padded to 256 bytes), then
// batch + W - 1 partial slots of [heads][512] fp32 and their [heads] lse.
size_t balanced_cu_bytes(int64_t batch) { return ((size_t)(batch + 1) * sizeof(int64_t) + 255) & ~(size_t)255; }
size_t balanced_bytes_for(int64_t batch, int64_t heads, int64_t workgroups) {
  const size_t slots = (size_t)(batch + workgroups - 1);
  const size_t bytes = balanced_cu_bytes(batch) + slots * (size_t)heads * (MLA_LATENT + 1) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

struct BalancedWorkspace {
  int64_t* cu;
  float* part_out;
  float* part_lse;
};
BalancedWorkspace balanced_layout(void* workspace, int64_t batch, int64_t heads, int64_t workgroups) {
  BalancedWorkspace w;
  w.cu = static_cast<int64_t*>(workspace);
  w.part_out = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + balanced_cu_bytes(batch));
  w.part_lse = w.part_out + (size_t)(batch + workgroups - 1) * heads * MLA_LATENT;
  return w;
}

// mtp (kinds kBf16 / kFp8 only): the verify step of mla_decode_mtp_*, a slot holding the
// q_len x num_heads query rows of its request; otherwise q_len = 1.
int decode_balanced(int kind, bool mtp, int32_t q_len, const void* q, const void* kv_cache, int64_t num_pages,
                    const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                    int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_workgroups, float* out,
                    float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status,
                    void* stream, const AppendArgs* app = nullptr) {
  static const char* const kNames[] = {"mla_decode_balanced_bf16", "mla_decode_balanced_fp8_656",
                                       "mla_decode_balanced_nope_bf16", "mla_decode_balanced_nope_fp8_656"};
  static const char* const kMtpNames[] = {"mla_decode_mtp_balanced_bf16", "mla_decode_mtp_balanced_fp8_656"};
  const bool gla = kind == kGla2Bf16 || kind == kGla2Fp8;
  const char* fn = gla   ? (kind == kGla2Fp8 ? "mla_decode_gla2_balanced_fp8_656" : "mla_decode_gla2_balanced_bf16")
                   : app ? (kind == kFp8 ? "mla_decode_append_balanced_fp8_656" : "mla_decode_append_balanced_bf16")
                   : mtp ? kMtpNames[kind == kFp8]
                         : kNames[kind];
  if (int rc0 = check_options(fn, flags, check_status)) return rc0;
  if (int rc0 = check_append(fn, app)) return rc0;
  if (!q) return fail(MLA_ERR_NULL, "%s: q is NULL", fn);
  if (!kv_cache) return fail(MLA_ERR_NULL, "%s: kv_cache is NULL", fn);
  if (!block_table) return fail(MLA_ERR_NULL, "%s: block_table is NULL", fn);
  if (!seq_lens) return fail(MLA_ERR_NULL, "%s: seq_lens is NULL", fn);
  // out == lse == NULL leaves the partials in the workspace for mla_merge_lse_balanced (not for
  // GLA-g2 heads, whose 256-value partial rows that merge does not take).
  const bool partials_only = !out && !lse && !gla;
  if (!out && !partials_only) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse && !partials_only) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (batch < 1 || batch > MLA_MAX_BALANCED_BATCH)
    return fail(MLA_ERR_SHAPE, "%s: batch=%d outside [1, %d]", fn, batch, MLA_MAX_BALANCED_BATCH);
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d outside [1, %d]", fn, num_heads, MLA_MAX_HEADS);
  if (gla && num_heads % 2)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d must be even (two head groups)", fn, num_heads);
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN)
    return fail(MLA_ERR_SHAPE, "%s: q_len=%d outside [1, %d]", fn, q_len, MLA_MAX_Q_LEN);
  if (q_len * num_heads > MLA_MAX_QUERY_ROWS)
    return fail(MLA_ERR_SHAPE, "%s: q_len * num_heads = %d exceeds %d", fn, q_len * num_heads, MLA_MAX_QUERY_ROWS);
  if (page_size < 1) return fail(MLA_ERR_SHAPE, "%s: page_size=%d must be >= 1", fn, page_size);
  if (num_pages < 1) return fail(MLA_ERR_SHAPE, "%s: num_pages=%lld must be >= 1", fn, (long long)num_pages);
  if (block_table_stride < 1)
    return fail(MLA_ERR_SHAPE, "%s: block_table_stride=%lld must be >= 1", fn, (long long)block_table_stride);
  if (block_table_stride > ((int64_t)1 << 31) / page_size + 1)
    return fail(MLA_ERR_SHAPE, "%s: block_table_stride * page_size exceeds the int32 token range", fn);
  if (num_workgroups < 0 || num_workgroups > 65535)
    return fail(MLA_ERR_SHAPE, "%s: num_workgroups=%d outside [0, 65535]", fn, num_workgroups);
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_SHAPE, "%s: softmax_scale is not finite", fn);
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(block_table) || !aligned16(seq_lens) ||
      !aligned16(out) || !aligned16(lse))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  const int32_t rows = q_len * num_heads;  // query rows per request
  if (!workspace) return fail(MLA_ERR_WORKSPACE, "%s: a workspace is required", fn);
  if (!aligned16(workspace)) return fail(MLA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  // The workspace size depends on the workgroup count; 0 (one per compute unit) is resolved
  // from the device first.
  auto size_ok = [&]() -> int {
    const size_t need = balanced_bytes_for(batch, rows, num_workgroups);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
    return MLA_OK;
  };
  int rc = num_workgroups > 0 ? size_ok() : MLA_OK;
  if (rc != MLA_OK) return rc;
  rc = check_device();
  if (rc != MLA_OK) return rc;
  if (num_workgroups == 0) {
    num_workgroups = device_cus();
    if (num_workgroups < 1) return fail(MLA_ERR_HIP, "%s: the device reports no compute units", fn);
    rc = size_ok();
    if (rc != MLA_OK) return rc;
  }

  BalancedWorkspace ws = balanced_layout(workspace, batch, rows, num_workgroups);
  mla::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.cache = static_cast<const uint8_t*>(kv_cache);
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.heads = num_heads;
  p.q_len = q_len;
  p.page_size = page_size;
  p.num_splits = 1;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.out = nullptr;
  p.lse = nullptr;
  p.part_out = ws.part_out;
  p.part_lse = ws.part_lse;
  p.cu = ws.cu;
  p.compact = 0;
  p.skip_empty = 0;
  p.stream_rows = (flags & MLA_FLAG_CACHED_ROWS) == 0;
  p.num_pages = num_pages;
  p.check_status = check_status;
  set_append(p, app);
  static_assert(MLA_MAX_BALANCED_BATCH == mla::kMaxBalancedBatch, "batch limit of the balanced kernels");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t launched;
  switch (kind) {
    case kBf16: launched = mla::launch_decode_flat_bf16(p, num_workgroups, s); break;
    case kFp8: launched = mla::launch_decode_flat_fp8(p, num_workgroups, s); break;
    case kNopeBf16: launched = mla::launch_decode_flat_nope_bf16(p, num_workgroups, s); break;
    case kNopeFp8: launched = mla::launch_decode_flat_nope_fp8(p, num_workgroups, s); break;
    default: launched = mla::launch_decode_flat_gla2(p, kind == kGla2Fp8, num_workgroups, s); break;
  }
  rc = hip_status(launched, fn);
  if (rc != MLA_OK || partials_only) return rc;
  return hip_status(
      mla::launch_merge_flat(ws.part_out, ws.part_lse, ws.cu, batch, rows, num_workgroups, out, lse, s,
                             gla ? 256 : MLA_LATENT),
      "mla_merge_lse_balanced (after balanced decode)");
}

// Decode over per-query index lists (mla_decode_sparse_*): fp8 selects the 656-byte rows, nope
// the scores over the latent only.
int decode_sparse_common(int fp8, int nope, const void* q, const void* kv_cache, int64_t num_slots,
                         const int32_t* indices, int32_t topk, int32_t num_tokens, int32_t num_heads,
                         float softmax_scale, int32_t num_splits, float* out, float* lse, void* workspace,
                         size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  static const char* const kNames[2][2] = {{"mla_decode_sparse_bf16", "mla_decode_sparse_nope_bf16"},
                                           {"mla_decode_sparse_fp8_656", "mla_decode_sparse_nope_fp8_656"}};
  const char* fn = kNames[fp8][nope];
  if (int rc0 = check_options(fn, flags, check_status)) return rc0;
  if (!q) return fail(MLA_ERR_NULL, "%s: q is NULL", fn);
  if (!kv_cache) return fail(MLA_ERR_NULL, "%s: kv_cache is NULL", fn);
  if (!indices) return fail(MLA_ERR_NULL, "%s: indices is NULL", fn);
  // out == lse == NULL with num_splits > 1 leaves the partials in the workspace (no merge).
  const bool partials_only = !out && !lse && num_splits > 1;
  if (!out && !partials_only) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse && !partials_only) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (num_tokens < 1 || num_tokens > MLA_MAX_SPARSE_TOKENS)
    return fail(MLA_ERR_SHAPE, "%s: num_tokens=%d outside [1, %d]", fn, num_tokens, (int)MLA_MAX_SPARSE_TOKENS);
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d outside [1, %d]", fn, num_heads, MLA_MAX_HEADS);
  if (topk < 1 || topk > MLA_MAX_SPARSE_TOPK)
    return fail(MLA_ERR_SHAPE, "%s: topk=%d outside [1, %d]", fn, topk, (int)MLA_MAX_SPARSE_TOPK);
  if (num_slots < 1) return fail(MLA_ERR_SHAPE, "%s: num_slots=%lld must be >= 1", fn, (long long)num_slots);
  if (num_splits < 1 || num_splits > 65535)
    return fail(MLA_ERR_SHAPE, "%s: num_splits=%d outside [1, 65535]", fn, num_splits);
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_SHAPE, "%s: softmax_scale is not finite", fn);
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(indices) || !aligned16(out) || !aligned16(lse))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  float* part_out = nullptr;
  float* part_lse = nullptr;
  if (num_splits > 1) {
    const size_t need = workspace_bytes_for(num_tokens, num_heads, num_splits);
    if (!workspace) return fail(MLA_ERR_WORKSPACE, "%s: num_splits=%d needs a workspace", fn, num_splits);
    if (!aligned16(workspace)) return fail(MLA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
    part_out = static_cast<float*>(workspace);
    part_lse = part_out + (size_t)num_splits * num_tokens * num_heads * MLA_LATENT;
  }
  int rc = check_device();
  if (rc != MLA_OK) return rc;

  mla::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.cache = static_cast<const uint8_t*>(kv_cache);
  p.block_table = indices;  // a block table of page size 1: one slot per entry
  p.bt_stride = topk;
  p.seq_lens = nullptr;
  p.batch = num_tokens;
  p.heads = num_heads;
  p.q_len = 1;
  p.page_size = 1;
  p.num_splits = num_splits;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  p.out = out;
  p.lse = lse;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.cu = nullptr;
  p.compact = 0;
  p.skip_empty = 0;
  p.stream_rows = (flags & MLA_FLAG_CACHED_ROWS) == 0;
  p.num_pages = num_slots;
  p.check_status = check_status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = hip_status(mla::launch_decode_sparse(p, fp8, nope, s), fn);
  if (rc != MLA_OK || num_splits == 1 || partials_only) return rc;
  return hip_status(mla::launch_merge(part_out, part_lse, num_splits, num_tokens, num_heads, out, lse, s),
                    "mla_merge_lse (after sparse decode)");
}

}  // namespace

extern "C" {

int mla_decode_bf16_noalloc(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                            int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                            int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                            uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kBf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch, num_heads,
                       page_size, softmax_scale, num_splits, out, lse, nullptr, 0, flags, check_status, stream,
                       /*use_scratch=*/true);
}

#define MLA_SPARSE_ENTRY(NAME, FP8, NOPE)                                                                   \
  int NAME(const void* q, const void* kv_cache, int64_t num_slots, const int32_t* indices, int32_t topk,     \
           int32_t num_tokens, int32_t num_heads, float softmax_scale, int32_t num_splits, float* out,       \
           float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status,      \
           void* stream) {                                                                                  \
    return decode_sparse_common(FP8, NOPE, q, kv_cache, num_slots, indices, topk, num_tokens, num_heads,    \
                                softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags,     \
                                check_status, stream);                                                      \
  }
MLA_SPARSE_ENTRY(mla_decode_sparse_bf16, 0, 0)
MLA_SPARSE_ENTRY(mla_decode_sparse_fp8_656, 1, 0)
MLA_SPARSE_ENTRY(mla_decode_sparse_nope_bf16, 0, 1)
MLA_SPARSE_ENTRY(mla_decode_sparse_nope_fp8_656, 1, 1)
#undef MLA_SPARSE_ENTRY

size_t mla_decode_balanced_workspace_size(int32_t batch, int32_t num_heads, int32_t num_workgroups) {
  if (batch < 1 || num_heads < 1 || num_workgroups < 0) return 0;
  if (num_workgroups == 0) {
    if (check_device() != MLA_OK) return 0;
    num_workgroups = device_cus();
    if (num_workgroups < 1) return 0;
  }
  return balanced_bytes_for(batch, num_heads, num_workgroups);
}

int mla_decode_gla2_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                  int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                                  int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                  float* out, float* lse, void* workspace, size_t workspace_bytes, uint32_t flags,
                                  int32_t* check_status, void* stream) {
  return decode_balanced(kGla2Bf16, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens,
                         batch, num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace,
                         workspace_bytes, flags, check_status, stream);
}

int mla_decode_gla2_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                     const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                                     int32_t batch, int32_t num_heads, int32_t page_size, float softmax_scale,
                                     int32_t num_workgroups, float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kGla2Fp8, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens,
                         batch, num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace,
                         workspace_bytes, flags, check_status, stream);
}

int mla_decode_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                             int32_t page_size, float softmax_scale, int32_t num_workgroups, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kBf16, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

int mla_decode_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                                int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                float* out, float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kFp8, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

int mla_decode_balanced_nope_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                  int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                                  int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                  float* out, float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kNopeBf16, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

int mla_decode_balanced_nope_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                     const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                                     int32_t batch, int32_t num_heads, int32_t page_size, float softmax_scale,
                                     int32_t num_workgroups, float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kNopeFp8, false, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

int mla_decode_mtp_balanced_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                 int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                                 int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_workgroups,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kBf16, true, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

int mla_decode_mtp_balanced_fp8_656(const void* q, const void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                                    int32_t batch, int32_t q_len, int32_t num_heads, int32_t page_size,
                                    float softmax_scale, int32_t num_workgroups, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_balanced(kFp8, true, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                         num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace, workspace_bytes,
                         flags, check_status, stream);
}

size_t mla_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t num_splits) {
  if (batch < 1 || num_heads < 1 || num_splits < 1) return 0;
  return workspace_bytes_for(batch, num_heads, num_splits);
}

size_t mla_decode_rank_workspace_size(int32_t batch, int32_t num_heads, int32_t num_splits, int32_t latent_rank) {
  if (batch < 1 || num_heads < 1 || num_splits < 1) return 0;
  if (latent_rank != 768 && latent_rank != 1792) return 0;
  return workspace_bytes_for(batch, num_heads, num_splits, latent_rank);
}

int mla_decode_rank768_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                            int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                            int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kRank768Bf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_rank1792_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                             int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kRank1792Bf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                    int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                    int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                    void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kBf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch, num_heads,
                       page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_fp8_656(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                       int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                       int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kFp8, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch, num_heads,
                       page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_nope_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                         int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                         int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                         void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kNopeBf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_nope_fp8_656(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                            int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                            int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kNopeFp8, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_mtp_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                        int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                        int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_splits, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kBf16, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_mtp_fp8_656(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                           int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                           int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_splits, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kFp8, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_append_bf16(const void* q, const void* new_latent, const void* new_k_pe, const int64_t* new_slots,
                           void* kv_cache, int64_t num_pages, const int32_t* block_table, int64_t block_table_stride,
                           const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t num_heads, int32_t page_size,
                           float softmax_scale, int32_t num_splits, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  const AppendArgs app = {new_latent, new_k_pe, new_slots, kv_cache};
  return decode_common(kBf16, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags,
                       check_status, stream, false, &app);
}

int mla_decode_append_fp8_656(const void* q, const void* new_latent, const void* new_k_pe, const int64_t* new_slots,
                              void* kv_cache, int64_t num_pages, const int32_t* block_table,
                              int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                              int32_t num_heads, int32_t page_size, float softmax_scale, int32_t num_splits,
                              float* out, float* lse, void* workspace, size_t workspace_bytes, uint32_t flags,
                              int32_t* check_status, void* stream) {
  const AppendArgs app = {new_latent, new_k_pe, new_slots, kv_cache};
  return decode_common(kFp8, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags,
                       check_status, stream, false, &app);
}

int mla_decode_append_balanced_bf16(const void* q, const void* new_latent, const void* new_k_pe,
                                    const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                    const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                                    int32_t batch, int32_t q_len, int32_t num_heads, int32_t page_size,
                                    float softmax_scale, int32_t num_workgroups, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status,
                                    void* stream) {
  const AppendArgs app = {new_latent, new_k_pe, new_slots, kv_cache};
  return decode_balanced(kBf16, q_len > 1, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens,
                         batch, num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace,
                         workspace_bytes, flags, check_status, stream, &app);
}

int mla_decode_append_balanced_fp8_656(const void* q, const void* new_latent, const void* new_k_pe,
                                       const int64_t* new_slots, void* kv_cache, int64_t num_pages,
                                       const int32_t* block_table, int64_t block_table_stride,
                                       const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t num_heads,
                                       int32_t page_size, float softmax_scale, int32_t num_workgroups, float* out,
                                       float* lse, void* workspace, size_t workspace_bytes, uint32_t flags,
                                       int32_t* check_status, void* stream) {
  const AppendArgs app = {new_latent, new_k_pe, new_slots, kv_cache};
  return decode_balanced(kFp8, q_len > 1, q_len, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens,
                         batch, num_heads, page_size, softmax_scale, num_workgroups, out, lse, workspace,
                         workspace_bytes, flags, check_status, stream, &app);
}

int mla_decode_rank256_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                            int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                            int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kRank256Bf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_gla2_bf16(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                         int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                         int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                         void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kGla2Bf16, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_decode_gla2_fp8_656(const void* q, const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                            int64_t block_table_stride, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                            int32_t page_size, float softmax_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, uint32_t flags, int32_t* check_status, void* stream) {
  return decode_common(kGla2Fp8, 1, q, kv_cache, num_pages, block_table, block_table_stride, seq_lens, batch,
                       num_heads, page_size, softmax_scale, num_splits, out, lse, workspace, workspace_bytes, flags, check_status, stream);
}

int mla_merge_lse_balanced(const void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_heads,
                           int32_t num_workgroups, float* out, float* lse, void* stream) {
  const char* fn = "mla_merge_lse_balanced";
  if (!workspace) return fail(MLA_ERR_NULL, "%s: workspace is NULL", fn);
  if (!out) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (batch < 1 || batch > MLA_MAX_BALANCED_BATCH)
    return fail(MLA_ERR_SHAPE, "%s: batch=%d outside [1, %d]", fn, batch, MLA_MAX_BALANCED_BATCH);
  // num_heads: the query rows of a request (q_len * num_heads after a verify-step decode)
  if (num_heads < 1 || num_heads > MLA_MAX_QUERY_ROWS)
    return fail(MLA_ERR_SHAPE, "%s: num_heads=%d outside [1, %d]", fn, num_heads, MLA_MAX_QUERY_ROWS);
  if (num_workgroups < 0 || num_workgroups > 65535)
    return fail(MLA_ERR_SHAPE, "%s: num_workgroups=%d outside [0, 65535]", fn, num_workgroups);
  if (!aligned16(workspace) || !aligned16(out) || !aligned16(lse))
    return fail(MLA_ERR_ALIGN, "%s: workspace, out and lse must be 16-byte aligned", fn);
  if (num_workgroups > 0 && workspace_bytes < balanced_bytes_for(batch, num_heads, num_workgroups))
    return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes,
                balanced_bytes_for(batch, num_heads, num_workgroups));
  int rc = check_device();
  if (rc != MLA_OK) return rc;
  if (num_workgroups == 0) {
    num_workgroups = device_cus();
    if (num_workgroups < 1) return fail(MLA_ERR_HIP, "%s: the device reports no compute units", fn);
    const size_t need = balanced_bytes_for(batch, num_heads, num_workgroups);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
  }
  BalancedWorkspace ws = balanced_layout(const_cast<void*>(workspace), batch, num_heads, num_workgroups);
  return hip_status(mla::launch_merge_flat(ws.part_out, ws.part_lse, ws.cu, batch, num_heads, num_workgroups, out,
                                           lse, static_cast<hipStream_t>(stream)),
                    fn);
}

int mla_merge_lse_width(const float* part_out, const float* part_lse, int32_t num_splits, int32_t batch,
                        int32_t num_rows, int32_t width, float* out, float* lse, void* stream) {
  const char* fn = "mla_merge_lse_width";
  if (width != 256 && width != 512 && width != 768 && width != 1792)
    return fail(MLA_ERR_SHAPE, "%s: width=%d must be 256, 512, 768 or 1792", fn, width);
  if (!part_out) return fail(MLA_ERR_NULL, "%s: part_out is NULL", fn);
  if (!part_lse) return fail(MLA_ERR_NULL, "%s: part_lse is NULL", fn);
  if (!out) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (num_splits < 1 || num_splits > 65536)
    return fail(MLA_ERR_SHAPE, "%s: num_splits=%d outside [1, 65536]", fn, num_splits);
  if (batch < 1) return fail(MLA_ERR_SHAPE, "%s: batch=%d must be >= 1", fn, batch);
  if (num_rows < 1) return fail(MLA_ERR_SHAPE, "%s: num_rows=%d must be >= 1", fn, num_rows);
  if ((int64_t)batch * num_rows > 0x7FFFFFFF) return fail(MLA_ERR_SHAPE, "%s: batch * num_rows too large", fn);
  if (!aligned16(part_out) || !aligned16(out))
    return fail(MLA_ERR_ALIGN, "%s: part_out and out must be 16-byte aligned", fn);
  int rc = check_device();
  if (rc != MLA_OK) return rc;
  return hip_status(mla::launch_merge(part_out, part_lse, num_splits, batch, num_rows, out, lse,
                                      static_cast<hipStream_t>(stream), width),
                    fn);
}

int mla_merge_lse(const float* part_out, const float* part_lse, int32_t num_splits, int32_t batch,
                  int32_t num_heads, float* out, float* lse, void* stream) {
  const char* fn = "mla_merge_lse";
  if (!part_out) return fail(MLA_ERR_NULL, "%s: part_out is NULL", fn);
  if (!part_lse) return fail(MLA_ERR_NULL, "%s: part_lse is NULL", fn);
  if (!out) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!lse) return fail(MLA_ERR_NULL, "%s: lse is NULL", fn);
  if (num_splits < 1 || num_splits > 65536)
    return fail(MLA_ERR_SHAPE, "%s: num_splits=%d outside [1, 65536]", fn, num_splits);
  if (batch < 1) return fail(MLA_ERR_SHAPE, "%s: batch=%d must be >= 1", fn, batch);
  if (num_heads < 1) return fail(MLA_ERR_SHAPE, "%s: num_heads=%d must be >= 1", fn, num_heads);
  if ((int64_t)batch * num_heads > 0x7FFFFFFF) return fail(MLA_ERR_SHAPE, "%s: batch * num_heads too large", fn);
  if (!aligned16(part_out) || !aligned16(out))
    return fail(MLA_ERR_ALIGN, "%s: part_out and out must be 16-byte aligned", fn);
  int rc = check_device();
  if (rc != MLA_OK) return rc;
  return hip_status(mla::launch_merge(part_out, part_lse, num_splits, batch, num_heads, out, lse,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

int mla_cache_write(const void* latent, const void* k_pe, const int64_t* slot_mapping, int32_t num_tokens,
                    void* kv_cache, int32_t cache_format, int64_t num_slots, void* stream) {
  const char* fn = "mla_cache_write";
  if (num_tokens < 0) return fail(MLA_ERR_SHAPE, "%s: num_tokens=%d is negative", fn, num_tokens);
  if (cache_format != MLA_CACHE_BF16_576 && cache_format != MLA_CACHE_FP8_656)
    return fail(MLA_ERR_SHAPE, "%s: cache_format=%d unknown", fn, cache_format);
  if (num_slots < 1) return fail(MLA_ERR_SHAPE, "%s: num_slots=%lld must be >= 1", fn, (long long)num_slots);
  if (num_tokens == 0) return MLA_OK;
  if (!latent) return fail(MLA_ERR_NULL, "%s: latent is NULL", fn);
  if (!slot_mapping) return fail(MLA_ERR_NULL, "%s: slot_mapping is NULL", fn);
  if (!kv_cache) return fail(MLA_ERR_NULL, "%s: kv_cache is NULL", fn);
  if (!aligned16(latent) || !aligned16(k_pe) || !aligned16(slot_mapping) || !aligned16(kv_cache))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  int rc = check_device();
  if (rc != MLA_OK) return rc;
  return hip_status(mla::launch_cache_write(static_cast<const uint16_t*>(latent), static_cast<const uint16_t*>(k_pe),
                                            slot_mapping, num_tokens, static_cast<uint8_t*>(kv_cache),
                                            cache_format == MLA_CACHE_FP8_656, static_cast<hipStream_t>(stream)),
                    fn);
}

int mla_gather_context(const void* kv_cache, int32_t cache_format, int64_t num_pages, int32_t page_size,
                       const int32_t* block_table, int64_t block_table_stride, const int64_t* cu_rows,
                       const int32_t* seq_starts, int32_t batch, int64_t total_rows, void* out,
                       int32_t* check_status, void* stream) {
  const char* fn = "mla_gather_context";
  if (int rc0 = check_options(fn, 0, check_status)) return rc0;
  if (cache_format != MLA_CACHE_BF16_576 && cache_format != MLA_CACHE_FP8_656)
    return fail(MLA_ERR_SHAPE, "%s: cache_format=%d unknown", fn, cache_format);
  if (total_rows < 0) return fail(MLA_ERR_SHAPE, "%s: total_rows=%lld is negative", fn, (long long)total_rows);
  if (total_rows > ((int64_t)1 << 32))  // bf16 output alone would be 4.9 TB; keeps the grid below 2^31
    return fail(MLA_ERR_SHAPE, "%s: total_rows=%lld exceeds 2^32", fn, (long long)total_rows);
  if (batch < 1) return fail(MLA_ERR_SHAPE, "%s: batch=%d must be >= 1", fn, batch);
  if (num_pages < 1) return fail(MLA_ERR_SHAPE, "%s: num_pages=%lld must be >= 1", fn, (long long)num_pages);
  if (page_size < 1) return fail(MLA_ERR_SHAPE, "%s: page_size=%d must be >= 1", fn, page_size);
  if (block_table_stride < 1)
    return fail(MLA_ERR_SHAPE, "%s: block_table_stride=%lld must be >= 1", fn, (long long)block_table_stride);
  if (total_rows == 0) return MLA_OK;
  if (!kv_cache) return fail(MLA_ERR_NULL, "%s: kv_cache is NULL", fn);
  if (!block_table) return fail(MLA_ERR_NULL, "%s: block_table is NULL", fn);
  if (!cu_rows) return fail(MLA_ERR_NULL, "%s: cu_rows is NULL", fn);
  if (!out) return fail(MLA_ERR_NULL, "%s: out is NULL", fn);
  if (!aligned16(kv_cache) || !aligned16(block_table) || !aligned16(cu_rows) || !aligned16(seq_starts) ||
      !aligned16(out))
    return fail(MLA_ERR_ALIGN, "%s: every tensor pointer must be 16-byte aligned", fn);
  int rc = check_device();
  if (rc != MLA_OK) return rc;
  return hip_status(mla::launch_gather(static_cast<const uint8_t*>(kv_cache), cache_format == MLA_CACHE_FP8_656,
                                       num_pages, block_table, block_table_stride, cu_rows, seq_starts, batch,
                                       page_size, total_rows, static_cast<uint16_t*>(out), check_status,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_ARCH: return "MLA_ERR_ARCH";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error_message(void) { return g_message; }

int mla_abi_version(void) { return MLA_ABI_VERSION; }

int mla_checked_build(void) { return mla::kChecked ? 1 : 0; }

int mla_check_preconditions_host(const int32_t* block_table, int64_t block_table_stride, const int32_t* seq_lens,
                                 int32_t batch, int32_t page_size, int64_t num_pages) {
  const char* fn = "mla_check_preconditions_host";
  if (!block_table || !seq_lens) {
    fail(MLA_ERR_NULL, "%s: block_table and seq_lens are required", fn);
    return -MLA_ERR_NULL;
  }
  if (batch < 0 || page_size < 1 || block_table_stride < 1 || num_pages < 0) {
    fail(MLA_ERR_SHAPE, "%s: batch=%d, page_size=%d, block_table_stride=%lld, num_pages=%lld out of range", fn,
         batch, page_size, (long long)block_table_stride, (long long)num_pages);
    return -MLA_ERR_SHAPE;
  }
  int bits = 0;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t L = seq_lens[b];
    if (!mla::len_in_table(L, block_table_stride, page_size)) {
      bits |= MLA_CHECK_SEQ_LEN;
      L = L < 0 ? 0 : block_table_stride * page_size;
    }
    const int64_t pages = (L + page_size - 1) / page_size;  // the entries the context uses
    const int32_t* row = block_table + (int64_t)b * block_table_stride;
    for (int64_t j = 0; j < pages; ++j)
      if (!mla::page_in_pool(row[j], num_pages)) bits |= MLA_CHECK_BLOCK_ID;
  }
  return bits;
}

}  // extern "C"

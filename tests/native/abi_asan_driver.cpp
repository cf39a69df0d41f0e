// Host-side driver for the AddressSanitizer build of the C ABI (tests/test_abi_asan.py).
//
// Runs without a GPU: every call either fails host-side validation or stops at the device
// check (MLA_ERR_ARCH), so only the library's host code runs, under ASan.  Exits 0 when every
// expectation holds; prints the first failure otherwise.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "mla.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (last message: %s)\n", what, mla_last_error_message());
    ++failures;
  }
}

// A 16-byte aligned stand-in pointer that is never dereferenced.
void* const P = reinterpret_cast<void*>(0x1000);
void* const MIS = reinterpret_cast<void*>(0x1008);

using DecodeFn = int (*)(const void*, const void*, int64_t, const int32_t*, int64_t, const int32_t*, int32_t,
                         int32_t, int32_t, float, int32_t, float*, float*, void*, size_t, uint32_t, int32_t*,
                         void*);

struct Args {
  const void* q = P;
  const void* kv = P;
  int64_t pages = 10;
  const int32_t* bt = static_cast<const int32_t*>(P);
  int64_t stride = 4;
  const int32_t* lens = static_cast<const int32_t*>(P);
  int32_t batch = 2, heads = 16, ps = 64;
  float scale = 0.07f;
  int32_t splits = 1;
  float* out = static_cast<float*>(P);
  float* lse = static_cast<float*>(P);
  void* ws = P;
  size_t ws_bytes = size_t(1) << 30;
  uint32_t flags = 0;
  int32_t* status = nullptr;
};

int call(DecodeFn f, const Args& a) {
  return f(a.q, a.kv, a.pages, a.bt, a.stride, a.lens, a.batch, a.heads, a.ps, a.scale, a.splits, a.out, a.lse,
           a.ws, a.ws_bytes, a.flags, a.status, nullptr);
}

// The preconditions written out on their own: the reference for mla_check_preconditions_host.
int reference_bits(const std::vector<int32_t>& bt, int64_t stride, const std::vector<int32_t>& lens, int32_t ps,
                   int64_t pages) {
  int bits = 0;
  for (size_t b = 0; b < lens.size(); ++b) {
    int64_t L = lens[b];
    if (L < 0 || L > stride * ps) {
      bits |= MLA_CHECK_SEQ_LEN;
      L = L < 0 ? 0 : stride * ps;
    }
    for (int64_t t = 0; t < L; ++t) {
      const int32_t page = bt[b * stride + t / ps];
      if (page < 0 || page >= pages) bits |= MLA_CHECK_BLOCK_ID;
    }
  }
  return bits;
}

}  // namespace

int main() {
  const std::pair<const char*, DecodeFn> decoders[] = {
      {"mla_decode_bf16", mla_decode_bf16},
      {"mla_decode_fp8_656", mla_decode_fp8_656},
      {"mla_decode_nope_bf16", mla_decode_nope_bf16},
      {"mla_decode_nope_fp8_656", mla_decode_nope_fp8_656},
      {"mla_decode_rank256_bf16", mla_decode_rank256_bf16},
      {"mla_decode_rank768_bf16", mla_decode_rank768_bf16},
      {"mla_decode_rank1792_bf16", mla_decode_rank1792_bf16},
      {"mla_decode_gla2_bf16", mla_decode_gla2_bf16},
      {"mla_decode_gla2_fp8_656", mla_decode_gla2_fp8_656},
      {"mla_decode_balanced_bf16", mla_decode_balanced_bf16},
      {"mla_decode_balanced_fp8_656", mla_decode_balanced_fp8_656},
      {"mla_decode_balanced_nope_bf16", mla_decode_balanced_nope_bf16},
      {"mla_decode_balanced_nope_fp8_656", mla_decode_balanced_nope_fp8_656},
      {"mla_decode_gla2_balanced_bf16", mla_decode_gla2_balanced_bf16},
      {"mla_decode_gla2_balanced_fp8_656", mla_decode_gla2_balanced_fp8_656},
  };
  for (const auto& d : decoders) {
    Args a;
    expect(call(d.second, a) == MLA_ERR_ARCH, d.first);  // valid: only the device is missing
    Args n = a;
    n.q = nullptr;
    expect(call(d.second, n) == MLA_ERR_NULL && std::strstr(mla_last_error_message(), d.first), "null q");
    Args s = a;
    s.heads = 17;
    expect(call(d.second, s) == MLA_ERR_SHAPE, "num_heads 17");
    s = a;
    s.ps = 0;
    expect(call(d.second, s) == MLA_ERR_SHAPE, "page_size 0");
    s = a;
    s.stride = int64_t(1) << 40;
    expect(call(d.second, s) == MLA_ERR_SHAPE, "stride past int32 tokens");
    s = a;
    s.flags = 0xFFFFFFFEu;
    expect(call(d.second, s) == MLA_ERR_SHAPE, "unknown flags");
    s = a;
    s.status = static_cast<int32_t*>(P);
    expect(call(d.second, s) == (mla_checked_build() ? MLA_ERR_ARCH : MLA_ERR_SHAPE), "status word");
    s = a;
    s.out = static_cast<float*>(MIS);
    expect(call(d.second, s) == MLA_ERR_ALIGN, "misaligned out");
    s = a;
    s.scale = 1.0f / 0.0f;
    expect(call(d.second, s) == MLA_ERR_SHAPE, "infinite scale");
  }
  // workspace sizes, including the largest shapes the validation admits
  expect(mla_decode_workspace_size(65535, 16, 65535) > 0, "largest workspace size");
  expect(mla_decode_workspace_size(0, 16, 4) == 0, "empty batch");
  expect(mla_decode_balanced_workspace_size(1024, 64, 65535) > 0, "largest balanced workspace");
  expect(mla_decode_rank_workspace_size(4, 16, 8, 1000) == 0, "unknown rank");
  // merges, cache write, gather
  expect(mla_merge_lse(nullptr, static_cast<float*>(P), 2, 1, 1, static_cast<float*>(P), static_cast<float*>(P),
                       nullptr) == MLA_ERR_NULL, "merge null");
  expect(mla_merge_lse_width(static_cast<float*>(P), static_cast<float*>(P), 2, 1, 4, 384, static_cast<float*>(P),
                             static_cast<float*>(P), nullptr) == MLA_ERR_SHAPE, "merge width");
  expect(mla_merge_lse_balanced(P, 1, 4, 16, 256, static_cast<float*>(P), static_cast<float*>(P), nullptr) ==
             MLA_ERR_WORKSPACE, "balanced merge workspace");
  expect(mla_cache_write(P, P, static_cast<const int64_t*>(P), -1, P, 0, 10, nullptr) == MLA_ERR_SHAPE, "write count");
  expect(mla_cache_write(nullptr, nullptr, nullptr, 0, nullptr, 0, 10, nullptr) == MLA_OK, "write nothing");
  expect(mla_gather_context(P, 0, 10, 16, static_cast<const int32_t*>(P), 4, static_cast<const int64_t*>(P),
                            nullptr, 2, int64_t(1) << 40, P, nullptr, nullptr) == MLA_ERR_SHAPE, "gather rows");
  expect(mla_decode_bf16_noalloc(P, P, 10, static_cast<const int32_t*>(P), 4, static_cast<const int32_t*>(P), 4, 16,
                                 64, 0.07f, 200, static_cast<float*>(P), static_cast<float*>(P), 0, nullptr,
                                 nullptr) == MLA_ERR_WORKSPACE, "noalloc scratch limit");
  // index-list decodes: the longest name in every message, the largest workspace the checks admit
  for (auto fn : {mla_decode_sparse_bf16, mla_decode_sparse_fp8_656, mla_decode_sparse_nope_bf16,
                  mla_decode_sparse_nope_fp8_656}) {
    const int32_t* idx = static_cast<const int32_t*>(P);
    float* f = static_cast<float*>(P);
    expect(fn(nullptr, P, 100, idx, 64, 3, 16, 0.07f, 1, f, f, nullptr, 0, 0, nullptr, nullptr) == MLA_ERR_NULL,
           "sparse null q");
    expect(fn(P, P, 100, idx, 0, 3, 16, 0.07f, 1, f, f, nullptr, 0, 0, nullptr, nullptr) == MLA_ERR_SHAPE,
           "sparse topk");
    expect(fn(P, P, 100, idx, MLA_MAX_SPARSE_TOPK + 1, 3, 16, 0.07f, 1, f, f, nullptr, 0, 0, nullptr, nullptr) ==
               MLA_ERR_SHAPE, "sparse topk above the limit");
    expect(fn(P, P, 100, idx, 64, MLA_MAX_SPARSE_TOKENS, 16, 0.07f, 65535, f, f, P, 1, 0, nullptr, nullptr) ==
               MLA_ERR_WORKSPACE, "sparse largest workspace");
  }
  // decodes that write the step's new rows: the longest names, a missing new_slots, a NULL new_k_pe
  for (auto fn : {mla_decode_append_bf16, mla_decode_append_fp8_656, mla_decode_append_balanced_bf16,
                  mla_decode_append_balanced_fp8_656}) {
    const int32_t* i32 = static_cast<const int32_t*>(P);
    const int64_t* slots = static_cast<const int64_t*>(P);
    float* f = static_cast<float*>(P);
    expect(fn(P, P, nullptr, slots, P, 10, i32, 4, i32, 2, 4, 16, 64, 0.07f, 1, f, f, P, 1 << 30, 0, nullptr,
              nullptr) == MLA_ERR_ARCH, "append valid without k_pe");
    expect(fn(P, P, P, nullptr, P, 10, i32, 4, i32, 2, 4, 16, 64, 0.07f, 1, f, f, P, 1 << 30, 0, nullptr,
              nullptr) == MLA_ERR_NULL && std::strstr(mla_last_error_message(), "new_slots"), "append null slots");
    expect(fn(P, P, P, slots, P, 10, i32, 4, i32, 2, 17, 4, 64, 0.07f, 1, f, f, P, 1 << 30, 0, nullptr,
              nullptr) == MLA_ERR_SHAPE, "append q_len 17");
  }
  for (int st = -3; st < 10; ++st) expect(std::strlen(mla_status_string(st)) > 0, "status string");

  // the host precondition check against the reference on random tables (ragged, with -1 tails,
  // ids past the pool, lengths past the table)
  std::mt19937 rng(7);
  for (int trial = 0; trial < 2000; ++trial) {
    const int32_t batch = 1 + rng() % 9, ps = 1 + rng() % 70;
    const int64_t stride = 1 + rng() % 12, pages = 1 + rng() % 40;
    std::vector<int32_t> bt(batch * stride), lens(batch);
    for (auto& v : bt) v = int32_t(rng() % (pages + 3)) - 2;
    for (auto& v : lens) v = int32_t(rng() % (stride * ps + 20)) - 5;
    const int got = mla_check_preconditions_host(bt.data(), stride, lens.data(), batch, ps, pages);
    if (got != reference_bits(bt, stride, lens, ps, pages)) {
      expect(false, "host precondition check");
      break;
    }
  }
  expect(mla_check_preconditions_host(nullptr, 4, nullptr, 1, 16, 10) == -MLA_ERR_NULL, "host check null");

  // the message is per thread
  Args bad;
  bad.heads = 99;
  call(mla_decode_bf16, bad);
  const std::string mine = mla_last_error_message();
  std::string theirs = "unset";
  std::thread t([&] { theirs = mla_last_error_message(); Args b2; b2.ps = 0; call(mla_decode_bf16, b2); });
  t.join();
  expect(theirs.empty() && mine == mla_last_error_message(), "thread-local message");

  if (failures == 0) std::printf("abi_asan_driver: all checks passed\n");
  return failures == 0 ? 0 : 1;
}

// abi_check.cpp — driver for the AddressSanitizer / UndefinedBehaviorSanitizer
// build of the library's host code (test infrastructure).  It calls every
// entry point of include/attn.h with arguments that the host-side validation
// rejects (so no GPU is touched), the workspace-size queries, and the kernel
// timing session without launches, and checks the status codes and that
// attn_last_error() names the entry point.
#include <cstdio>
#include <cstring>

#include "attn.h"

static int bad = 0;

static void expect(int got, int want, const char* fn, const char* what) {
  if (got != want) {
    std::printf("FAIL %s %s: status %d, want %d\n", fn, what, got, want);
    ++bad;
  } else if (want != ATTN_OK && std::strstr(attn_last_error(), fn) == nullptr) {
    std::printf("FAIL %s %s: error text '%s'\n", fn, what, attn_last_error());
    ++bad;
  }
}

int main() {
  void* F = reinterpret_cast<void*>(0x1000);  // never dereferenced
  const float* Fm = static_cast<const float*>(F);
  const int* Fi = static_cast<const int*>(F);
  float* Fl = static_cast<float*>(F);
  // attn_fwd
  expect(attn_fwd(nullptr, F, F, F, nullptr, 1, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "null q");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 0, 64, 0, 0.125f, 0.f, 1, nullptr),
         ATTN_ERR_EMPTY_KV, "attn_fwd", "Skv 0");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 6, 4, 8, 8, 64, 0, 0.125f, 0.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "Hq % Hkv");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 8, 63, 0, 0.125f, 10000.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "odd D with RoPE");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 8, 64, 2, 0.125f, 0.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "causal 2");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 8, 64, 0, -1.f, 0.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "scale");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 9, nullptr),
         ATTN_ERR_INVALID, "attn_fwd", "dtype");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 8, 8, 256, 0, 0.125f, 0.f, 1, nullptr),
         ATTN_ERR_UNSUPPORTED, "attn_fwd", "D 256");
  expect(attn_fwd(F, F, F, F, nullptr, 1, 4, 2, 9, 8, 64, 1, 0.125f, 10000.f, 1, nullptr),
         ATTN_ERR_UNSUPPORTED, "attn_fwd", "RoPE with Sq > Skv");
  // attn_fwd_masked
  expect(attn_fwd_masked(F, F, F, nullptr, 0, 0, 8, F, nullptr, 1, 4, 2, 8, 8, 64, 0, 0.125f,
                         0.f, 1, nullptr),
         ATTN_ERR_INVALID, "attn_fwd_masked", "null mask");
  expect(attn_fwd_masked(F, F, F, Fm, 0, -1, 8, F, nullptr, 1, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 1,
                         nullptr),
         ATTN_ERR_INVALID, "attn_fwd_masked", "negative stride");
  expect(attn_fwd_masked(F, F, F, Fm, 0, 0, 8, F, nullptr, 0, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 1,
                         nullptr),
         ATTN_ERR_INVALID, "attn_fwd_masked", "B 0");
  // attn_bwd
  expect(attn_bwd(F, F, F, F, F, Fm, F, F, F, 1, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 0, nullptr,
                  nullptr),
         ATTN_ERR_UNSUPPORTED, "attn_bwd", "fp32");
  expect(attn_bwd(nullptr, F, F, F, F, Fm, F, F, F, 1, 4, 2, 8, 8, 64, 0, 0.125f, 0.f, 1,
                  nullptr, nullptr),
         ATTN_ERR_INVALID, "attn_bwd", "null q");
  expect(attn_bwd(F, F, F, F, F, Fm, F, F, F, 1, 4, 2, 8, 0, 64, 0, 0.125f, 0.f, 1, nullptr,
                  nullptr),
         ATTN_ERR_EMPTY_KV, "attn_bwd", "Skv 0");
  // decode
  expect(attn_decode_splitkv(F, F, F, Fi, F, 2, 8, 2, 128, 0, 0.088f, 64, nullptr, nullptr,
                             nullptr),
         ATTN_ERR_INVALID, "attn_decode_splitkv", "0 splits");
  expect(attn_decode_splitkv(F, F, F, Fi, F, 2, 8, 2, 128, 65, 0.088f, 64, nullptr, nullptr,
                             nullptr),
         ATTN_ERR_INVALID, "attn_decode_splitkv", "65 splits");
  expect(attn_decode_splitkv(F, F, F, nullptr, F, 2, 8, 2, 128, 4, 0.088f, 64, nullptr, nullptr,
                             nullptr),
         ATTN_ERR_INVALID, "attn_decode_splitkv", "null seqlens");
  expect(attn_decode_splitkv(F, F, F, Fi, F, 2, 8, 2, 80, 4, 0.088f, 64, Fl, nullptr, nullptr),
         ATTN_ERR_UNSUPPORTED, "attn_decode_splitkv", "D 80");
  // prefill against a cache
  expect(attn_prefill_kvcache(F, F, F, F, F, Fi, F, nullptr, 1, 4, 2, 65, 64, 64, 1, 0.125f,
                              0.f, nullptr),
         ATTN_ERR_INVALID, "attn_prefill_kvcache", "Sq > max_seqlen");
  expect(attn_prefill_kvcache(F, F, F, F, F, nullptr, F, nullptr, 1, 4, 2, 8, 64, 64, 1, 0.125f,
                              0.f, nullptr),
         ATTN_ERR_INVALID, "attn_prefill_kvcache", "null cache_lens");
  expect(attn_prefill_kvcache(F, F, F, F, F, Fi, F, nullptr, 1, 4, 2, 8, 40, 64, 1, 0.125f, 0.f,
                              nullptr),
         ATTN_ERR_UNSUPPORTED, "attn_prefill_kvcache", "D 40");
  // rope_apply
  expect(rope_apply(F, 1, 4, 2, 7, 0, 10000.f, 1, nullptr), ATTN_ERR_INVALID, "rope_apply",
         "odd D");
  expect(rope_apply(F, 1, 4, 2, 8, -1, 10000.f, 1, nullptr), ATTN_ERR_INVALID, "rope_apply",
         "negative offset");
  expect(rope_apply(F, 1, 4, 2, 512, 0, 10000.f, 1, nullptr), ATTN_ERR_UNSUPPORTED,
         "rope_apply", "D 512");
  expect(rope_apply(nullptr, 1, 4, 2, 8, 0, 10000.f, 1, nullptr), ATTN_ERR_INVALID, "rope_apply",
         "null x");
  // workspace queries
  if (attn_decode_workspace_bytes(2, 8, 128, 16) == 0 || attn_decode_workspace_bytes(0, 8, 128, 16) != 0 ||
      attn_bwd_workspace_bytes(1, 4, 2, 64, 64, 64, 10000.f) == 0 ||
      attn_bwd_workspace_bytes(1, 4, 2, 0, 64, 64, 0.f) != 0) {
    std::printf("FAIL workspace queries\n");
    ++bad;
  }
  // timing session without launches
  int n = -1;
  expect(attn_profile_end(nullptr, 0, nullptr), ATTN_ERR_INVALID, "attn_profile_end", "null n");
  expect(attn_profile_begin(), ATTN_OK, "attn_profile_begin", "begin");
  float ms[4];
  expect(attn_profile_end(ms, 4, &n), ATTN_OK, "attn_profile_end", "end");
  if (n != 0) {
    std::printf("FAIL attn_profile_end: %d launches recorded without a call\n", n);
    ++bad;
  }
  std::printf("library host-code sanitizer driver: %s\n", bad ? "FAILED" : "ok");
  return bad != 0;
}

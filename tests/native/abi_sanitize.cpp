// Host-side checks of libfb's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py).  Runs without a
// GPU: every call below returns before any device work (argument, config and
// option checks; the missing device at allocation).  Exit status 0 when every
// return code is the documented one.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fb.h"

static int failures = 0;

static void expect(const char* what, fb_status got, fb_status want) {
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d (%s)\n", what, got, want, fb_last_error());
    ++failures;
  }
}

static fb_config good() {
  fb_config c;
  c.batch = 2;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.block_size = 32;
  c.max_prefix = 4096;
  c.dtype = FB_BF16;
  c.softmax_scale = 0.0f;
  return c;
}

int main() {
  fb_cache* h = nullptr;
  struct Bad {
    const char* what;
    void (*edit)(fb_config&);
    fb_status code;
  } bad[] = {
      {"dtype", [](fb_config& c) { c.dtype = 5; }, FB_E_DTYPE},
      {"batch 0", [](fb_config& c) { c.batch = 0; }, FB_E_SHAPE},
      {"batch big", [](fb_config& c) { c.batch = FB_MAX_BATCH + 1; }, FB_E_SHAPE},
      {"heads", [](fb_config& c) { c.n_q_heads = 7; }, FB_E_SHAPE},
      {"kv heads 0", [](fb_config& c) { c.n_kv_heads = 0; }, FB_E_SHAPE},
      {"q heads big", [](fb_config& c) { c.n_q_heads = FB_MAX_HEADS + 2; }, FB_E_SHAPE},
      {"block 0", [](fb_config& c) { c.block_size = 0; }, FB_E_SHAPE},
      {"block huge", [](fb_config& c) { c.block_size = 1 << 21; }, FB_E_SHAPE},
      {"max_prefix", [](fb_config& c) { c.max_prefix = -5; }, FB_E_SHAPE},
      {"head_dim", [](fb_config& c) { c.head_dim = 96; }, FB_E_UNSUPPORTED},
      {"scale nan", [](fb_config& c) { c.softmax_scale = std::numeric_limits<float>::quiet_NaN(); }, FB_E_ARG},
      {"scale inf", [](fb_config& c) { c.softmax_scale = std::numeric_limits<float>::infinity(); }, FB_E_ARG},
      {"rows", [](fb_config& c) { c.n_q_heads = 256; c.n_kv_heads = 1; c.block_size = 1 << 20; }, FB_E_SHAPE},
  };
  for (const Bad& b : bad) {
    fb_config c = good();
    b.edit(c);
    h = nullptr;
    expect(b.what, fb_cache_alloc(&c, &h), b.code);
    if (h != nullptr) ++failures;
    if (std::strlen(fb_last_error()) == 0) ++failures;
  }
  fb_config c = good();
  expect("alloc null cfg", fb_cache_alloc(nullptr, &h), FB_E_ARG);
  expect("alloc null out", fb_cache_alloc(&c, nullptr), FB_E_ARG);
  expect("alloc_ex null out", fb_cache_alloc_ex(&c, nullptr, nullptr), FB_E_ARG);
  fb_cache_opts o{};
  o.struct_size = 2;
  expect("opts size", fb_cache_alloc_ex(&c, &o, &h), FB_E_ARG);
  o.struct_size = sizeof o;
  o.kv_splits = 65;
  expect("opts splits", fb_cache_alloc_ex(&c, &o, &h), FB_E_ARG);
  // a caller whose struct ends before kv_splits: the bytes behind it are not read
  struct {
    uint32_t struct_size;
  } short_opts = {4};
  expect("short opts, no device", fb_cache_alloc_ex(&c, reinterpret_cast<const fb_cache_opts*>(&short_opts), &h),
         FB_E_HIP);
  expect("no device", fb_cache_alloc(&c, &h), FB_E_HIP);
  if (h != nullptr) ++failures;

  expect("free null", fb_cache_free(nullptr), FB_OK);
  if (std::strlen(fb_last_error()) != 0) ++failures;
  expect("reset null", fb_cache_reset(nullptr, nullptr), FB_E_ARG);
  expect("external null", fb_external_attn(nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr), FB_E_ARG);
  expect("internal null", fb_internal_attn_merge(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), FB_E_ARG);
  fb_policy_args pa{FB_POLICY_TAU, 4, 0.0f, nullptr};
  expect("step null", fb_step(nullptr, &pa, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr), FB_E_ARG);
  fb_step_opts so{sizeof(fb_step_opts), nullptr};
  expect("step_ex null", fb_step_ex(nullptr, &pa, &so, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr),
         FB_E_ARG);
  expect("sparse null",
         fb_step_sparse(nullptr, &pa, &so, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr),
         FB_E_ARG);
  char buf[16];
  expect("read null", fb_cache_read(nullptr, 0, buf, sizeof buf, nullptr), FB_E_ARG);
  expect("info null", fb_cache_info(nullptr, nullptr, nullptr), FB_E_ARG);
  expect("profile null", fb_profile_enable(nullptr, 1), FB_E_ARG);
  expect("profile read null", fb_profile_read(nullptr, nullptr), FB_E_ARG);
  std::printf("%d failures\n", failures);
  return failures == 0 ? 0 : 1;
}

// Host-only driver for the sanitizer test: exercises every argument check of the C ABI
// that returns before any HIP call, plus a few thousand random and extreme configs, so that
// AddressSanitizer / UndefinedBehaviorSanitizer see the validation paths (size arithmetic
// on untrusted int32 fields, message formatting). Exit status 0 = every expectation held.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "moe_verify.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static moe_verify_config base() {
  moe_verify_config c{};
  c.hidden = 1280; c.n_routed = 64; c.top_k = 6; c.n_shared = 2; c.inter = 896; c.n_layers = 12;
  c.vocab = 129280; c.wdtype = MOE_BF16; c.rms_eps = 1e-6f; c.max_positions = 128;
  return c;
}

int main() {
  // valid configs
  moe_verify_config c = base();
  EXPECT(moe_verify_check_config(&c) == MOE_OK);
  EXPECT(std::strlen(moe_verify_last_error()) == 0);
  c.max_positions = 36992; c.vocab = 0;
  EXPECT(moe_verify_check_config(&c) == MOE_OK);
  // invalid ones, each with a message
  EXPECT(moe_verify_check_config(nullptr) == MOE_EINVAL);
  const int32_t bad[] = {0, -1, INT_MIN, INT_MAX, 7, 65, 100000};
  for (int field = 0; field < 8; ++field)
    for (int32_t v : bad) {
      moe_verify_config b = base();
      int32_t* f[] = {&b.hidden, &b.n_routed, &b.top_k, &b.n_shared, &b.inter, &b.n_layers, &b.vocab, &b.max_positions};
      *f[field] = v;
      const int rc = moe_verify_check_config(&b);
      EXPECT(rc == MOE_OK || rc == MOE_EINVAL || rc == MOE_EUNSUPPORTED);
      if (rc != MOE_OK) EXPECT(std::strlen(moe_verify_last_error()) > 0);
    }
  // random configs, including sizes whose products overflow 32 bits
  std::mt19937 rng(1234);
  std::uniform_int_distribution<int32_t> any(INT_MIN, INT_MAX);
  std::uniform_int_distribution<int32_t> small(-4, 70000);
  for (int i = 0; i < 4000; ++i) {
    moe_verify_config r{};
    auto pick = [&]() { return (i & 1) ? any(rng) : small(rng); };
    r.hidden = pick(); r.n_routed = pick() & 127; r.top_k = pick() & 127; r.n_shared = pick() & 15;
    r.inter = pick(); r.n_layers = pick() & 63; r.vocab = pick(); r.wdtype = pick() & 1;
    r.rms_eps = 1e-6f; r.max_positions = pick();
    const int rc = moe_verify_check_config(&r);
    EXPECT(rc == MOE_OK || rc == MOE_EINVAL || rc == MOE_EUNSUPPORTED);
    for (int j = 0; j < 4; ++j) {
      const int rs = moe_verify_check_step(&r, pick(), pick() & 255, j & 1, (j >> 1) & 1, 1);
      EXPECT(rs == MOE_OK || rs == MOE_EINVAL || rs == MOE_EUNSUPPORTED);
    }
  }
  // step arguments
  c = base();
  EXPECT(moe_verify_check_step(&c, 32, 3, 1, 1, 0) == MOE_OK);
  EXPECT(moe_verify_check_step(&c, INT_MAX, INT_MAX, 1, 1, 0) == MOE_EINVAL);
  EXPECT(moe_verify_check_step(&c, 1, INT_MAX, 1, 1, 0) == MOE_EINVAL);  // K + 1 must not wrap
  EXPECT(moe_verify_check_step(&c, INT_MAX, 0, 1, 1, 0) == MOE_EINVAL);
  EXPECT(moe_verify_check_step(&c, 0, 3, 1, 1, 0) == MOE_EINVAL);
  EXPECT(moe_verify_check_step(&c, 1, -1, 1, 1, 0) == MOE_EINVAL);
  // entry points that must refuse before touching the device
  moe_verify_ctx* ctx = reinterpret_cast<moe_verify_ctx*>(0x1);
  EXPECT(moe_verify_init(&c, nullptr, nullptr, &ctx) == MOE_EINVAL);
  EXPECT(ctx == nullptr);
  EXPECT(moe_verify_init(nullptr, nullptr, nullptr, nullptr) == MOE_EINVAL);
  moe_verify_weights w{};
  EXPECT(moe_verify_init(&c, &w, nullptr, &ctx) == MOE_EINVAL);
  w.router_w = reinterpret_cast<const void*>(0x11);
  w.w_gate = w.w_up = w.w_down = w.lm_head = reinterpret_cast<const void*>(0x10);
  EXPECT(moe_verify_init(&c, &w, nullptr, &ctx) == MOE_EINVAL);  // misaligned
  const float* hp = reinterpret_cast<const float*>(0x100);
  int32_t* ip = reinterpret_cast<int32_t*>(0x100);
  EXPECT(moe_verify_step(nullptr, hp, 1, 3, ip, nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_step_static(nullptr, hp, 1, 3, ip, nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_step_mixed(nullptr, hp, 4, 1, 3, ip, nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_debug_layer(nullptr, 0, hp, 4, nullptr, nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_debug_head(nullptr, hp, 4, ip, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_debug_plan(nullptr, ip, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_profile(nullptr, 1) == MOE_EINVAL);
  EXPECT(moe_verify_profile_read(nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_verify_expert_counts(nullptr, ip) == MOE_EINVAL);
  moe_draft_weights dw{};
  EXPECT(moe_draft_init(nullptr, &dw, nullptr) == MOE_EINVAL);
  EXPECT(moe_draft_step(nullptr, hp, ip, ip, 1, 3, 3, ip, nullptr) == MOE_EINVAL);
  EXPECT(accept_greedy(ip, ip, 0, 3, ip, ip, nullptr) == MOE_EINVAL);
  EXPECT(accept_greedy(ip, ip, 1, -1, ip, ip, nullptr) == MOE_EINVAL);
  EXPECT(accept_greedy(nullptr, ip, 1, 3, ip, ip, nullptr) == MOE_EINVAL);
  EXPECT(accept_greedy(ip, ip, 1, 3, nullptr, ip, nullptr) == MOE_EINVAL);
  moe_verify_destroy(nullptr);
  std::printf("host checks: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}

// host_abi_check.cpp -- drives the library's host code (plan, layout,
// argument checks, stage names) with no GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; built and run by
// tests/test_sanitizers.py against an instrumented build of the host
// translation unit).  Every call here returns before any kernel launch.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe_decode.h"

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "line %d: %s failed\n", __LINE__, #c);   \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static moe_decode_desc desc(int H, int E, int k, int I, int Is, int rows, int act, int ef, int routing,
                            uint32_t flags) {
  moe_decode_desc d;
  std::memset(&d, 0, sizeof d);
  d.hidden = H; d.num_experts = E; d.top_k = k; d.inter = I; d.shared_inter = Is;
  d.max_rows = rows; d.act_fmt = act; d.expert_fmt = ef; d.routing = routing; d.flags = flags;
  d.routed_scaling_factor = 1.0f; d.norm_eps = 1e-6f;
  return d;
}

// A weights struct whose pointers are non-null and aligned (never dereferenced).
static moe_decode_weights fake_weights() {
  moe_decode_weights w;
  const void *p = reinterpret_cast<const void *>(uintptr_t(4096));
  const uint64_t *t = reinterpret_cast<const uint64_t *>(uintptr_t(4096));
  w.router_w = p; w.expert_bias = reinterpret_cast<const float *>(p);
  w.gate_w = w.up_w = w.down_w = w.gate_s = w.up_s = w.down_s = w.gate_b = w.up_b = w.down_b = t;
  w.sh_gate_w = w.sh_up_w = w.sh_down_w = w.sh_gate_vec = p;
  w.gate_scale2 = w.up_scale2 = w.down_scale2 = reinterpret_cast<const float *>(p);
  w.pre_norm_w = w.router_norm_w = p;
  return w;
}

static void plan_case(const moe_decode_desc &d, bool want_ok) {
  moe_decode_plan_t *plan = nullptr;
  size_t ws = 0;
  const moe_status st = moe_decode_plan(&d, &plan, &ws);
  EXPECT((st == MOE_OK) == want_ok);
  if (st != MOE_OK) {
    EXPECT(plan == nullptr);
    EXPECT(std::strlen(moe_decode_last_error()) > 0);
    return;
  }
  moe_decode_ws_layout L;
  EXPECT(moe_decode_workspace_layout(plan, &L) == MOE_OK);
  EXPECT(L.total == ws && ws % 256 == 0);
  const int32_t n = moe_decode_num_stages(plan);
  EXPECT(n >= 3 && n <= 6);
  for (int32_t i = -1; i <= n; ++i) (void)moe_decode_stage_name(plan, i);
  // Argument checks: all fail before any launch.
  moe_decode_weights w = fake_weights();
  void *dev = reinterpret_cast<void *>(uintptr_t(1) << 20);
  EXPECT(moe_decode_forward(plan, &w, dev, 0, dev, nullptr, nullptr, dev, ws, nullptr) == MOE_EINVAL);
  EXPECT(moe_decode_forward(plan, &w, dev, d.max_rows + 1, dev, nullptr, nullptr, dev, ws, nullptr) == MOE_EINVAL);
  EXPECT(moe_decode_forward(plan, nullptr, dev, 1, dev, nullptr, nullptr, dev, ws, nullptr) == MOE_EINVAL);
  EXPECT(moe_decode_forward(plan, &w, nullptr, 1, dev, nullptr, nullptr, dev, ws, nullptr) == MOE_EINVAL);
  EXPECT(moe_decode_forward(plan, &w, dev, 1, dev, nullptr, nullptr, dev, ws - 256, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_decode_forward(plan, &w, dev, 1, dev, nullptr, nullptr,
                            reinterpret_cast<char *>(dev) + 16, ws, nullptr) == MOE_EWORKSPACE);
  void *ev[12] = {dev, dev, dev, dev, dev, dev, dev, dev, dev, dev, dev, dev};
  EXPECT(moe_decode_forward_timed(plan, &w, dev, 1, dev, nullptr, nullptr, dev, ws, nullptr, ev, 2 * n + 1) ==
         MOE_EINVAL);
  EXPECT(moe_decode_forward_noalloc(plan, &w, dev, 0, dev, nullptr, nullptr, nullptr) != MOE_OK);
  w.router_w = nullptr;
  EXPECT(moe_decode_forward(plan, &w, dev, 1, dev, nullptr, nullptr, dev, ws, nullptr) == MOE_EINVAL);
  moe_decode_plan_destroy(plan);
}

int main() {
  EXPECT(std::strlen(moe_decode_version()) > 0);
  EXPECT(moe_decode_plan(nullptr, nullptr, nullptr) == MOE_EINVAL);
  const int fmts[6] = {MOE_F32, MOE_BF16, MOE_AFF4_G64, MOE_MXFP4_B32, MOE_NVFP4_B16, MOE_FP8_B128};
  for (int act = MOE_F32; act <= MOE_BF16; ++act)
    for (int ef : fmts)
      for (int routing = MOE_ROUTE_SOFTMAX; routing <= MOE_ROUTE_SQRTSOFTPLUS; ++routing)
        for (uint32_t flags : {0u, 1u | 4u | 8u, 2u | 4u | 32u | 64u, 1u | 128u | 16u}) {
          for (int rows : {1, 8, 32}) {
            plan_case(desc(2048, 256, 8, 512, 512, rows, act, ef, routing, flags), true);
            plan_case(desc(5120, 16, 1, 8192, 8192, rows, act, ef, routing, flags), true);
          }
          // The grouped path: bf16 activations with bf16, 4-bit or fp8 experts.
          const bool grouped = act == MOE_BF16 && ef != MOE_F32;
          plan_case(desc(2048, 128, 8, 768, 512, 256, act, ef, routing, flags), grouped);
        }
  // Malformed and unsupported descriptors.
  plan_case(desc(0, 8, 2, 64, 0, 1, MOE_BF16, MOE_BF16, 0, 0), false);
  plan_case(desc(64, 257, 2, 64, 0, 1, MOE_BF16, MOE_BF16, 0, 0), false);
  plan_case(desc(64, 8, 17, 64, 0, 1, MOE_BF16, MOE_BF16, 0, 0), false);
  plan_case(desc(64, 8, 2, 64, 0, 257, MOE_BF16, MOE_BF16, 0, 0), false);
  plan_case(desc(64, 8, 2, 64, 0, 1, MOE_BF16, 7, 0, 0), false);
  plan_case(desc(64, 8, 2, 64, 0, 1, MOE_BF16, MOE_BF16, 9, 0), false);
  plan_case(desc(64, 8, 2, 64, 0, 1, MOE_BF16, MOE_BF16, 0, 1u << 12), false);
  plan_case(desc(64, 8, 2, 64, 0, 1, MOE_BF16, MOE_FP8_B128, 0, 0), false);          // 64 is not a multiple of 128
  plan_case(desc(128, 8, 2, 96, 0, 1, MOE_BF16, MOE_AFF4_G64, 0, 0), false);        // aff4 needs multiples of 64
  plan_case(desc(2048, 8, 2, 1 << 19, 0, 1, MOE_BF16, MOE_BF16, 0, 0), false);      // a projection past 2 GiB
  plan_case(desc(64, 8, 2, 64, 0, 1, MOE_BF16, MOE_BF16, 0, MOE_SHARED_GATED), false);
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}

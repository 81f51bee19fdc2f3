// Host-side driver of the C ABI for an AddressSanitizer build: every entry point is called
// with arguments its host validation rejects, plus the pure host queries (defaults, parameter
// counts, capacities, workspace sizes, messages) over many configurations. No call here
// reaches a HIP call, so the driver runs without a GPU; any out-of-bounds access or
// use-after-free in the host code aborts it with a sanitizer report.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_mi355x.h"

static int g_failures = 0;

#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
              moe_last_error_message());                                        \
      ++g_failures;                                                             \
    }                                                                           \
  } while (0)

static moe_config_t base_config(int64_t d, int32_t E, int32_t k, int64_t h, int64_t L) {
  moe_config_t c;
  moe_config_default(&c);
  c.d_model = d;
  c.num_experts = E;
  c.top_k = k;
  c.hidden_size = h;
  c.latent_dim = L;
  return c;
}

int main(void) {
  void* fake = reinterpret_cast<void*>(0x10000);  // never dereferenced: every call fails first
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  for (int st = -1; st <= 6; ++st) EXPECT(strlen(moe_status_string(static_cast<moe_status_t>(st))) > 0);
  EXPECT(moe_config_default(nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(strlen(moe_last_error_message()) > 0);
  EXPECT(moe_config_validate(nullptr) == MOE_ERR_INVALID_ARG);

  // host queries over a grid of shapes (the workload shapes among them)
  const int64_t ds[] = {64, 256, 2048, 4096};
  const int32_t Es[] = {1, 8, 64, 256, 896, 1024};
  const int32_t ks[] = {1, 2, 8, 16};
  const int64_t Ts[] = {0, 1, 3, 64, 1000, 8192, 32768};
  for (int64_t d : ds)
    for (int32_t E : Es)
      for (int32_t k : ks) {
        if (k > E) continue;
        for (int64_t L : {int64_t(0), d / 4 >= 64 ? d / 4 : int64_t(0)}) {
          moe_config_t c = base_config(d, E, k, 128, L);
          EXPECT(moe_config_validate(&c) == MOE_OK);
          int64_t tot = 0, act = 0;
          EXPECT(moe_num_params(&c, &tot, &act) == MOE_OK && tot >= act && act > 0);
          EXPECT(moe_num_params(&c, nullptr, nullptr) == MOE_OK);
          for (int64_t T : Ts) {
            // shapes whose bf16 operands pass 4 GiB are refused with a message
            size_t ws = 0;
            moe_status_t st = moe_workspace_size(&c, T, &ws);
            EXPECT(st == MOE_OK || (st == MOE_ERR_UNSUPPORTED && strlen(moe_last_error_message()) > 0));
            for (float cf : {0.0f, 0.5f, 1.25f, 1e-6f, 7.0f}) {
              c.capacity_factor = cf;
              int64_t cap = -1;
              st = moe_expert_capacity(&c, T, &cap);
              EXPECT((st == MOE_OK && cap >= 0) || st == MOE_ERR_UNSUPPORTED);
            }
            c.capacity_factor = 0.f;
            size_t bws = 0;
            moe_experts_backward_workspace_size(&c, T, &bws);
          }
        }
      }

  // configurations the validation rejects, each with its message
  moe_config_t c = base_config(2048, 64, 8, 1024, 0);
  moe_config_t bad = c;
  bad.top_k = 65;
  EXPECT(moe_config_validate(&bad) != MOE_OK);
  bad = c;
  bad.struct_size = 8;
  EXPECT(moe_config_validate(&bad) == MOE_ERR_INVALID_ARG);
  bad = c;
  bad.num_experts = 2048;
  bad.top_k = 2;
  EXPECT(moe_config_validate(&bad) == MOE_ERR_UNSUPPORTED);
  bad = c;
  bad.gating_function = 7;
  EXPECT(moe_config_validate(&bad) != MOE_OK);
  bad = c;
  bad.capacity_factor = -1.f;
  EXPECT(moe_config_validate(&bad) == MOE_ERR_INVALID_ARG);
  bad = c;
  bad.hidden_size = 96;
  EXPECT(moe_config_validate(&bad) == MOE_ERR_UNSUPPORTED);
  size_t ws = 0;
  EXPECT(moe_workspace_size(&c, -1, &ws) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, int64_t(1) << 28, &ws) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, 8, nullptr) == MOE_ERR_INVALID_ARG);

  // whole-layer and stage entry points: missing pointers, short workspaces
  moe_weights_t w;
  memset(&w, 0, sizeof w);
  const int64_t T = 128;
  EXPECT(moe_forward(&c, nullptr, T, fake, fake, nullptr, fake, size_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_forward(&c, &w, T, fake, fake, nullptr, fake, size_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
  w.router_weight = static_cast<const float*>(fake);
  w.w1 = fake;
  w.w2 = fake;
  EXPECT(moe_forward(&c, &w, T, nullptr, fake, nullptr, fake, size_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_size(&c, T, &ws) == MOE_OK);
  EXPECT(moe_forward(&c, &w, T, fake, fake, nullptr, fake, ws - 1, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_forward(&c, &w, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == MOE_OK);
  EXPECT(moe_forward_noalloc(&c, &w, 8192, fake, fake, nullptr, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_forward_noalloc(&c, &w, T, nullptr, fake, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_forward_noalloc(nullptr, &w, T, fake, fake, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  moe_routing_t r;
  memset(&r, 0, sizeof r);
  EXPECT(moe_router_forward(&c, &w, T, fake, &r, fake, ws, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_router_forward(&c, &w, T, fake, nullptr, fake, ws, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_from_scores(&c, T, static_cast<const float*>(fake), nullptr, nullptr,
                               static_cast<float*>(fake), nullptr) == MOE_ERR_INVALID_ARG);
  int32_t* ip = static_cast<int32_t*>(fake);
  EXPECT(moe_permute(&c, T, ip, ip, ip, ip, ip, fake, 16, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_permute(&c, T, ip, nullptr, ip, ip, ip, fake, ws, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_latent_down(&c, &w, T, fake, fake, nullptr, 0, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_latent_up(&c, &w, T, fake, fake, nullptr, 0, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_experts_forward(&c, &w, T, fake, ip, ip, fake, fake, 16, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_combine(&c, &w, T, fake, nullptr, fake, nullptr) == MOE_ERR_INVALID_ARG);
  moe_config_t lat = base_config(4096, 896, 8, 512, 1024);
  EXPECT(moe_forward(&lat, &w, T, fake, fake, nullptr, fake, size_t(1) << 40, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(strstr(moe_last_error_message(), "down_proj") != nullptr);

  // backward
  float* fp = static_cast<float*>(fake);
  size_t bws = 0;
  EXPECT(moe_experts_backward_workspace_size(&c, T, &bws) == MOE_OK);
  EXPECT(moe_experts_backward(&c, &w, T, fake, ip, ip, fake, fake, fake, fake, fake, fake, fake, bws - 1,
                              nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(moe_experts_backward(&c, &w, T, nullptr, ip, ip, fake, fake, fake, fake, fake, fake, fake, bws,
                              nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_backward(&c, T, fake, fp, nullptr, fake, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_backward(&lat, T, fake, fp, fake, fake, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);

  // balancing state, quantiser, calibration
  int64_t* lp = static_cast<int64_t*>(fake);
  double* dp = static_cast<double*>(fake);
  for (int32_t E : {0, -1, 1025}) {
    EXPECT(moe_accumulate_expert_counts(E, ip, lp, nullptr) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_load_imbalance(E, lp, dp, nullptr) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_score_bias_update(E, 0.1f, lp, fp, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  }
  EXPECT(moe_score_bias_update(8, 1.f / 0.f, lp, fp, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  uint8_t* up = static_cast<uint8_t*>(fake);
  EXPECT(moe_mx_quantize(4, 48, fake, up, up, nullptr) != MOE_OK);
  EXPECT(moe_mx_quantize(4, 64, nullptr, up, up, nullptr) == MOE_ERR_INVALID_ARG);
  int64_t waves = 0;
  double flops = 0;
  EXPECT(moe_calibrate_mfma_bf16(0, fp, &waves, &flops, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_calibrate_mfma_mxfp8(10, fp, nullptr, &flops, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_calibrate_copy(fake, fake, 24, nullptr) == MOE_ERR_INVALID_ARG);

  if (g_failures) {
    fprintf(stderr, "%d checks failed\n", g_failures);
    return 1;
  }
  printf("abi host driver: all checks passed\n");
  return 0;
}

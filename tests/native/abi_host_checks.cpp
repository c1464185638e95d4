// Host-side checks of the C ABI, built with the address and undefined-
// behaviour sanitizers on the host code (tests/test_abi_sanitized.py builds
// and runs it; no GPU is needed): every host-only function on ordinary and
// edge inputs, every workspace-size function, and the validation path of
// every device entry point with invalid arguments (the pointers are never
// dereferenced: validation fails before anything is launched).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fam.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

int main() {
  void* const fake = reinterpret_cast<void*>(static_cast<uintptr_t>(0x1000));   // never dereferenced
  float* const ffake = static_cast<float*>(fake);
  int32_t* const ifake = static_cast<int32_t*>(fake);
  int64_t* const lfake = static_cast<int64_t*>(fake);
  double* const dfake = static_cast<double*>(fake);

  // status strings and the error text
  for (int st = -2; st < 10; ++st) EXPECT(fam_status_string(static_cast<fam_status>(st)) != nullptr);
  EXPECT(std::strcmp(fam_status_string(FAM_ERR_TIMEOUT), "FAM_ERR_TIMEOUT") == 0);
  EXPECT(fam_last_error() != nullptr);

  // budget plan
  {
    const int64_t budgets[6] = {0, 3, 12, 50, 5000, 100};
    int64_t kept[6], offsets[7];
    EXPECT(evict_plan(6, 100, budgets, 4, 8, kept, offsets) == FAM_OK);
    EXPECT(kept[0] == 12 && kept[2] == 12 && kept[3] == 50 && kept[4] == 100 && offsets[6] == 12 + 12 + 12 + 50 + 100 + 100);
    EXPECT(evict_plan(0, 100, nullptr, 4, 8, nullptr, offsets) == FAM_OK && offsets[0] == 0);
    EXPECT(evict_plan(6, 0, budgets, 4, 8, kept, offsets) == FAM_ERR_INVALID_ARG);
    const int64_t neg[1] = {-1};
    EXPECT(evict_plan(1, 10, neg, 1, 1, kept, offsets) == FAM_ERR_INVALID_ARG);
    EXPECT(evict_plan(2, 10, budgets, -1, 1, kept, offsets) == FAM_ERR_INVALID_ARG);
  }
  // ratios to budgets
  {
    const double r[3] = {0.15, 0.0, 1.2};
    int64_t b[3];
    EXPECT(fam_budgets_from_ratios(3, r, 131072, b) == FAM_OK && b[0] == 19660 && b[1] == 0 && b[2] == 157286);
    const double bad[2] = {0.1, NAN};
    EXPECT(fam_budgets_from_ratios(2, bad, 100, b) == FAM_ERR_INVALID_ARG);
    const double huge[1] = {1e300};
    EXPECT(fam_budgets_from_ratios(1, huge, 100, b) == FAM_ERR_INVALID_ARG);
    EXPECT(fam_budgets_from_ratios(0, nullptr, 100, nullptr) == FAM_OK);
  }
  // Soft-TopK: sums to k, and edge inputs
  {
    std::vector<double> x(257), out(257);
    for (int i = 0; i < 257; ++i) x[i] = std::sin(0.37 * i) * 3.0;
    for (double k : {1.0, 2.5, 100.0, 256.0}) {
      for (double tau : {1e-3, 0.5, 10.0}) {
        EXPECT(fam_soft_topk(x.data(), 257, k, tau, out.data()) == FAM_OK);
        double s = 0;
        for (double v : out) s += v;
        EXPECT(std::fabs(s - k) < 1e-6 * (1 + k));
      }
    }
    const double one[1] = {2.0};
    double o1[1];
    EXPECT(fam_soft_topk(one, 1, 0.5, 1.0, o1) == FAM_OK && std::fabs(o1[0] - 0.5) < 1e-12);
    EXPECT(fam_soft_topk(x.data(), 257, 0.0, 1.0, out.data()) == FAM_ERR_INVALID_ARG);
    EXPECT(fam_soft_topk(x.data(), 257, 258.0, 1.0, out.data()) == FAM_ERR_INVALID_ARG);
    EXPECT(fam_soft_topk(x.data(), 257, 2.0, 0.0, out.data()) == FAM_ERR_INVALID_ARG);
    EXPECT(fam_soft_topk(nullptr, 3, 1.0, 1.0, out.data()) == FAM_ERR_INVALID_ARG);
  }
  // workspace sizes, including invalid sizes (0) and large ones
  EXPECT(evict_select_workspace_size(-1, 10, 0, 0) == 0);
  EXPECT(evict_select_workspace_size(64, (1 << 20) + 516, 4, 512) > 0);
  EXPECT(fam_mass_workspace_size(1, 32, 8, 131072) == (size_t)32 * 8 * 131072 * 4);
  EXPECT(fam_mass_per_head_workspace_size(1, 32, 8, 131072) > 0);
  EXPECT(fam_compute_workspace_size(1, 32, 8, 4096, 131072) > 0);
  EXPECT(kv_compact_inplace_workspace_size(-5) == 0 && kv_compact_inplace_workspace_size(1000) > 0);
  EXPECT(fam_rank_order_workspace_size(8, 131072) > 0);
  EXPECT(fam_eviction_cost_workspace_size(8, 131072) > 0);
  EXPECT(fam_eviction_cost_ratio_workspace_size(8, 131072) > 0);
  EXPECT(fam_topk_cutoff_workspace_size(8, 300000) > 0 && fam_topk_cutoff_workspace_size(8, (1 << 20) + 1) == 0);
  EXPECT(fam_key_norm_parts(131072) == 64);

  // validation of the device entry points (nothing is launched)
  EXPECT(fam_compute(fake, fake, FAM_BF16, 1, 3, 2, 100, 128, 0, 0, 128, 0, 0, 128, 0, 0.f, ffake, ffake,
                     nullptr, 0, nullptr) == FAM_ERR_INVALID_ARG);                 // Hq % Hkv
  EXPECT(fam_compute(fake, fake, FAM_BF16, 1, 4, 2, 100, 96, 0, 0, 96, 0, 0, 96, 0, 0.f, ffake, ffake,
                     nullptr, 0, nullptr) == FAM_ERR_UNSUPPORTED);                 // head dim
  EXPECT(fam_compute(fake, fake, FAM_BF16, 1, 4, 2, 100, 128, 4 * 100 * 128, 100 * 128, 128,
                     2 * 100 * 128, 100 * 128, 128, -1, 0.f, ffake, ffake, nullptr, 0, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_lse(fake, fake, FAM_FP16, 1, 4, 2, 100, 128, 0, 0, 128, 0, 0, 128, NAN, nullptr, ffake, nullptr)
         != FAM_OK);
  EXPECT(fam_key_norms(fake, static_cast<fam_dtype>(9), 1, 2, 100, 128, 0, 0, 128, ffake, nullptr) == FAM_ERR_UNSUPPORTED);
  EXPECT(fam_mass(fake, fake, ffake, FAM_BF16, 1, 4, 2, 100, 128, 0, 0, 128, 0, 0, 128, 0, 0.f, nullptr, nullptr, 0,
                  nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_mass_per_head(fake, fake, ffake, FAM_BF16, 1, 4, 2, 100, 64, 0, 0, 64, 0, 0, 64, -2, 0.f, ffake, nullptr,
                           0, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_kvpop_target(ffake, 1, 4, 3, 100, 8, 0.f, FAM_AGG_MAX, ffake, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_compute_chunk(fake, fake, FAM_BF16, 1, 4, 2, 200, 100, 128, 0, 0, 128, 0, 0, 128, 0, 0.f, ffake, ffake,
                           nullptr, 0, nullptr) == FAM_ERR_INVALID_ARG);           // Sq > Sk
  {
    const int64_t b[2] = {10, 10};
    const size_t ws = evict_select_workspace_size(2, 100, 4, 4);
    EXPECT(evict_select(ffake, 99, 2, 100, b, 4, 4, ifake, lfake, fake, ws, nullptr) == FAM_ERR_INVALID_ARG);
    EXPECT(evict_select(ffake, 100, 2, 100, b, 4, 4, ifake, lfake, fake, ws - 1, nullptr) == FAM_ERR_WORKSPACE);
    EXPECT(evict_select(ffake, (1 << 20) + 9, 2, (1 << 20) + 9, b, 4, 4, ifake, lfake, fake, 1u << 30, nullptr) ==
           FAM_ERR_UNSUPPORTED);
    EXPECT(evict_select_noalloc(ffake, 100, 2, 100, b, -1, 4, ifake, lfake, nullptr) == FAM_ERR_INVALID_ARG);
    EXPECT(evict_select(ffake, 100, 0, 100, nullptr, 4, 4, ifake, lfake, nullptr, 0, nullptr) == FAM_OK);
    const size_t mws = fam_mass_workspace_size(1, 4, 2, 8192), sws = evict_select_workspace_size(2, 8192, 4, 64);
    EXPECT(fam_mass_select(fake, fake, ffake, FAM_BF16, 1, 4, 2, 8192, 128, 0, 8192 * 128, 128, 0, 8192 * 128, 128,
                           4, 0.f, ffake, fake, mws, b, 4, 64, ifake, lfake, fake, sws, nullptr) ==
           FAM_ERR_INVALID_ARG);                                                     // overlapping workspaces
    EXPECT(fam_mass_select(fake, fake, ffake, FAM_BF16, 1, 4, 2, 8192, 128, 0, 8192 * 128, 128, 0, 8192 * 128, 128,
                           4, 0.f, ffake, fake, mws, b, 4, 64, ifake, lfake, nullptr, 0, nullptr) ==
           FAM_ERR_WORKSPACE);
    EXPECT(evict_select_prepare(ffake, 8192, 2, 8192, 4, 64, fake, sws - 1, nullptr) == FAM_ERR_WORKSPACE);
    EXPECT(evict_select_prepare(nullptr, 8192, 2, 8192, 4, 64, fake, sws, nullptr) == FAM_ERR_INVALID_ARG);
    EXPECT(evict_select_prepare(ffake, 8192, 0, 8192, 4, 64, nullptr, 0, nullptr) == FAM_OK);
    EXPECT(evict_select_prepared(ffake, 8192, 2, 8192, b, 4, 64, nullptr, lfake, fake, sws, nullptr) ==
           FAM_ERR_INVALID_ARG);
    EXPECT(fam_mass_prepare_select(fake, fake, ffake, FAM_BF16, 1, 4, 2, 8192, 128, 0, 8192 * 128, 128, 0,
                                   8192 * 128, 128, 4, 0.f, ffake, fake, mws, 4, 64, fake, sws, nullptr) ==
           FAM_ERR_INVALID_ARG);                                                     // overlapping workspaces
  }
  EXPECT(kv_compact(fake, fake, 4, 2, 100, 128, 0, 128, 0, 128, ifake, lfake, 10, fake, fake, nullptr) ==
         FAM_ERR_UNSUPPORTED);
  EXPECT(kv_append(fake, fake, 2, 2, 10, 128, 0, 128, 0, 128, fake, fake, 0, 128, 0, 128, 100, 95, nullptr, 0, 0,
                   nullptr) == FAM_ERR_INVALID_ARG);                                 // rows beyond the capacity
  EXPECT(kv_compact_inplace(fake, fake, 2, 2, 100, 128, 100 * 128, 128, 100 * 128, 128, ifake, lfake, 10, nullptr,
                            0, fake, 0, nullptr) == FAM_ERR_WORKSPACE);
  EXPECT(kv_compact_inplace_status(nullptr, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_rank_order(ffake, 99, 2, 100, ifake, fake, 1 << 20, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_eviction_cost(ffake, 100, ifake, 2, 100, nullptr, fake, 64, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(fam_eviction_cost_ratio(ffake, 100, ffake, 100, 2, 100, dfake, fake, 8, nullptr) == FAM_ERR_WORKSPACE);
  EXPECT(fam_retention_overlap(ifake, lfake, ifake, lfake, 2, (1 << 28) + 1, lfake, nullptr) == FAM_ERR_UNSUPPORTED);
  EXPECT(fam_topk_cutoff(ifake, 2, 100, -1, 8, 10, ifake, fake, 1 << 20, nullptr) == FAM_ERR_INVALID_ARG);
  EXPECT(std::strlen(fam_last_error()) > 0);

  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  else std::printf("all host checks passed\n");
  return failures ? 1 : 0;
}

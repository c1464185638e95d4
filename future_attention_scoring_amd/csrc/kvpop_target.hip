// KVpop supervision target from per-query-head future mass (gfx950).
//
// KVpop, "Defining Future Attention Utility" (worked example) and the
// appendix ("Alternative Aggregation Methods"): key j can be seen by
// N_j = max(1, S - (j + W)) future queries; the mean future mass is the mass
// over N_j, the target is log(eps + mean), and the g query heads of a KV head
// are aggregated by the maximum of their logs or, alternatively, by the mean
// in probability space before the log.
//
// One thread per output element, consecutive threads on consecutive keys
// (coalesced g loads of 4 bytes each and one store). Bound: HBM; the work is
// O(B * Hq * S) and tiny next to the passes that produce mass_q.
#include <math.h>

#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void target_kernel(TargetArgs p) {
  const int g = p.Hq / p.Hkv;
  const int64_t n = (int64_t)p.B * p.Hkv * p.S;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
    const int j = (int)(e % p.S);
    const int64_t bh = e / p.S;
    const int b = (int)(bh / p.Hkv), h = (int)(bh % p.Hkv);
    const int64_t unseen = (int64_t)j + p.W;
    const float count = unseen < p.S ? (float)(p.S - unseen) : 1.f;
    const float* m = p.mass_q + ((int64_t)b * p.Hq + (int64_t)h * g) * p.S + j;
    float r;
    if (p.mean) {
      float sum = 0.f;
      for (int gi = 0; gi < g; ++gi) sum += m[(int64_t)gi * p.S];
      r = logf(p.eps + sum / (count * (float)g));
    } else {
      r = -kInf;
      for (int gi = 0; gi < g; ++gi) r = fmaxf(r, logf(p.eps + m[(int64_t)gi * p.S] / count));
    }
    p.target[e] = r;
  }
}

}  // namespace

hipError_t launch_target(const TargetArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.S;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(target_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

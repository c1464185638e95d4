// KVpop supervision target from per-query-head future mass (gfx950).
//
// KVpop, "Defining Future Attention Utility" (worked example) and the
// appendix ("Alternative Aggregation Methods"): key j can be seen by
// N_j = max(1, S - (j + W)) future queries; the mean future mass is the mass
// over N_j, the target is log(eps + mean), and the g query heads of a KV head
// are aggregated by the maximum of their logs or, alternatively, by the mean
// in probability space before the log.
//
// Four consecutive keys per thread (16-byte loads of the g query heads' rows,
// all in flight, and one 16-byte store) when S is a multiple of 4 and the
// rows are 16-byte aligned; one key per thread otherwise. The group size is
// a template parameter for the usual GQA groups, so the g loads are
// unrolled. The maximum of the logs is taken as the log of the largest
// mass: x -> log(eps + x / N_j) is non-decreasing, so both give the same
// value, with one log instead of g. Bound: HBM; the work is O(B * Hq * S)
// and tiny next to the passes that produce mass_q.
#include <math.h>

#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float target_of(float agg, float count, float eps, int g, bool mean) {
  return mean ? logf(eps + agg / (count * (float)g)) : logf(eps + agg / count);
}

__device__ __forceinline__ float count_of(int64_t j, const TargetArgs& p) {
  const int64_t unseen = j + p.W;
  return unseen < p.S ? (float)(p.S - unseen) : 1.f;
}

// G > 0: the group size as a constant; G == 0: a runtime group size.
template <int G, bool VEC>
__global__ __launch_bounds__(kThreads) void target_kernel(TargetArgs p) {
  const int g = G > 0 ? G : p.Hq / p.Hkv;
  constexpr int V = VEC ? 4 : 1;           // keys per thread
  const int64_t per_row = p.S / V;         // S % V == 0 when VEC
  const int64_t n = (int64_t)p.B * p.Hkv * per_row;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
    const int64_t bh = e / per_row;
    const int64_t j0 = (e - bh * per_row) * V;
    const int b = (int)(bh / p.Hkv), h = (int)(bh % p.Hkv);
    const float* m = p.mass_q + ((int64_t)b * p.Hq + (int64_t)h * g) * p.S + j0;
    float agg[V];
#pragma unroll
    for (int v = 0; v < V; ++v) agg[v] = p.mean ? 0.f : -kInf;
    if constexpr (G > 0) {
      float x[G][V];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        if constexpr (VEC) {
          const float4 t = *reinterpret_cast<const float4*>(m + (int64_t)gi * p.S);
          x[gi][0] = t.x, x[gi][1] = t.y, x[gi][2] = t.z, x[gi][3] = t.w;
        } else {
          x[gi][0] = m[(int64_t)gi * p.S];
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int v = 0; v < V; ++v) agg[v] = p.mean ? agg[v] + x[gi][v] : fmaxf(agg[v], x[gi][v]);
    } else {
      for (int gi = 0; gi < g; ++gi) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const float x = m[(int64_t)gi * p.S + v];
          agg[v] = p.mean ? agg[v] + x : fmaxf(agg[v], x);
        }
      }
    }
    float r[V];
#pragma unroll
    for (int v = 0; v < V; ++v) r[v] = target_of(agg[v], count_of(j0 + v, p), p.eps, g, p.mean != 0);
    float* out = p.target + bh * p.S + j0;
    if constexpr (VEC) *reinterpret_cast<float4*>(out) = float4{r[0], r[1], r[2], r[3]};
    else out[0] = r[0];
  }
}

template <int G, bool VEC>
void launch_target_t(const TargetArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Hkv * (a.S / (VEC ? 4 : 1));
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL((target_kernel<G, VEC>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <bool VEC>
void launch_target_g(const TargetArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: launch_target_t<1, VEC>(a, s); break;
    case 2: launch_target_t<2, VEC>(a, s); break;
    case 4: launch_target_t<4, VEC>(a, s); break;
    case 8: launch_target_t<8, VEC>(a, s); break;
    default: launch_target_t<0, VEC>(a, s); break;
  }
}

}  // namespace

hipError_t launch_target(const TargetArgs& a, hipStream_t s) {
  const bool vec = a.S % 4 == 0 && (reinterpret_cast<uintptr_t>(a.mass_q) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.target) & 15u) == 0;
  if (vec) launch_target_g<true>(a, s);
  else launch_target_g<false>(a, s);
  return hipGetLastError();
}

}  // namespace fam

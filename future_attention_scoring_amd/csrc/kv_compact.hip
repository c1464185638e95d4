// Gather of kept K/V rows into a new packed cache (gfx950).
//
// KVP (section 4.1, A.2: physical tensor compaction) and the pruning blog
// ("What we did": the retained entries are copied into a new cache tensor).
//
// The output rows r = 0 .. total_rows-1 are split into blocks of 64 rows.
// A row of d two-byte elements is d/8 16-byte chunks; a wave moves 64 such
// chunks per instruction (4 rows for d = 128), reading one contiguous source
// row per group of lanes and writing fully contiguous output. Each thread
// issues all of its loads before its stores. The head of an output row comes
// from the offsets: a block binary-searches its first row once and then walks
// forward, since rows are ordered by head.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;

template <int CPR>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs p) {
  constexpr int ROWS_PER_PASS = kThreads / CPR;
  constexpr int PASSES = kRowsPerBlock / ROWS_PER_PASS;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
  const int64_t rend = min(p.total_rows, r0 + kRowsPerBlock);
  const int tid = threadIdx.x;
  const int ch = tid % CPR;

  // last head h with offsets[h] <= r0
  int lo = 0, hi = p.H - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.offsets[mid] <= r0) lo = mid; else hi = mid - 1;
  }
  int h = lo;

  u32x4_t kv[PASSES], vv[PASSES];
  int64_t rows[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = r0 + tid / CPR + (int64_t)i * ROWS_PER_PASS;
    rows[i] = r;
    kv[i] = zero16();
    vv[i] = zero16();
    if (r < rend) {
      while (h + 1 < p.H && r >= p.offsets[h + 1]) ++h;
      const int src = p.idx[r];
      if (src >= 0 && src < p.S) {
        kv[i] = load16(p.k + h * p.k_sh + (int64_t)src * p.k_ss + ch * 8);
        vv[i] = load16(p.v + h * p.v_sh + (int64_t)src * p.v_ss + ch * 8);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    if (rows[i] < rend) {
      store16(p.k_new + rows[i] * p.d + ch * 8, kv[i]);
      store16(p.v_new + rows[i] * p.d + ch * 8, vv[i]);
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const int64_t blocks = (a.total_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int cpr = a.d / 8;
  switch (cpr) {
    case 8: hipLaunchKernelGGL(compact_kernel<8>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL(compact_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL(compact_kernel<32>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fam

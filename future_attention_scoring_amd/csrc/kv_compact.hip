// Gather of kept K/V rows into a new packed cache (gfx950).
//
// KVP (section 4.1, A.2: physical tensor compaction) and the pruning blog
// ("What we did": the retained entries are copied into a new cache tensor).
//
// The output rows r = 0 .. total_rows-1 are split into blocks of 64 rows.
// A row of d two-byte elements is d/8 16-byte chunks; a wave moves 64 such
// chunks per instruction (4 rows for d = 128), reading one contiguous source
// row per group of lanes and writing fully contiguous output. Each thread
// issues all of its loads before its stores.
//
// The head of an output row comes from the offsets. With fewer than 256
// heads, a block stages all of offsets[0..H] in LDS in the same memory round
// trip as its idx loads and searches there; otherwise it binary-searches the
// global offsets. Every byte is touched once, so loads and stores carry the
// non-temporal hint: on this chip that keeps the gather at the same rate
// whether or not the caches hold dirty data from earlier kernels.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;

__device__ __forceinline__ u32x4_t load16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void store16_nt(uint16_t* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

template <int CPR>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs p) {
  constexpr int ROWS_PER_PASS = kThreads / CPR;
  constexpr int PASSES = kRowsPerBlock / ROWS_PER_PASS;
  __shared__ int64_t offs[kThreads];
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
  const int64_t rend = min(p.total_rows, r0 + kRowsPerBlock);
  const int tid = threadIdx.x;
  const int ch = tid % CPR;
  const bool lds_heads = p.H < kThreads;  // offsets[0 .. H] fit in LDS
  if (lds_heads && tid <= p.H) offs[tid] = p.offsets[tid];
  int src[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = r0 + tid / CPR + (int64_t)i * ROWS_PER_PASS;
    src[i] = r < rend ? p.idx[r] : -1;
  }
  __syncthreads();

  // last head h with offsets[h] <= this thread's first row
  const int64_t rfirst = r0 + tid / CPR;
  int lo = 0, hi = p.H - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((lds_heads ? offs[mid] : p.offsets[mid]) <= rfirst) lo = mid;
    else hi = mid - 1;
  }
  int h = lo;

  // the head of every row first; then all loads of the thread in flight at
  // once, unconditional (a row without a valid source reads row 0 of its
  // head and is written as zeros), so that no load waits for another
  int hs[PASSES];
  bool ok[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = rfirst + (int64_t)i * ROWS_PER_PASS;
    if (r < rend)
      while (h + 1 < p.H && r >= (lds_heads ? offs[h + 1] : p.offsets[h + 1])) ++h;
    hs[i] = h;
    ok[i] = r < rend && src[i] >= 0 && src[i] < p.S;
  }
  u32x4_t kv[PASSES], vv[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t row = ok[i] ? src[i] : 0;
    kv[i] = load16_nt(p.k + hs[i] * p.k_sh + row * p.k_ss + ch * 8);
    vv[i] = load16_nt(p.v + hs[i] * p.v_sh + row * p.v_ss + ch * 8);
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    kv[i] = ok[i] ? kv[i] : zero16();
    vv[i] = ok[i] ? vv[i] : zero16();
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = rfirst + (int64_t)i * ROWS_PER_PASS;
    if (r < rend) {
      store16_nt(p.k_new + r * p.d + ch * 8, kv[i]);
      store16_nt(p.v_new + r * p.d + ch * 8, vv[i]);
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

// Static cache regions: appending a chunk's rows and compacting in place
// (gfx950).
//
// KVP (section 4: long contexts are prefilled chunk by chunk and compressed
// after each chunk with physical tensor compaction) and the pruning blog
// (conclusion: a static cache can keep a fixed region per head and overwrite
// old entries in place instead of copying into a new tensor).
//
// Append. One 16-byte piece per thread and pass over (head, row, piece);
// every head's rows row0 .. row0+n-1 are written, and optionally their
// positions pos0 .. pos0+n-1.
//
// In-place compaction. Head h keeps the rows idx[offsets[h] + r] (ascending,
// as evict_select writes them) and moves row idx[...+r] to row r. Ascending
// indices satisfy idx[r] >= r, so a sweep in increasing r is safe as long as
// every row is read before it is overwritten. The kept rows of all heads
// (output index g = offsets[h] + r) are cut into passes that the whole grid
// takes in order: in a pass every workgroup loads the source rows of its
// share into registers, the grid meets at one grid-wide barrier (a
// cooperative launch keeps every workgroup resident), and then every
// workgroup stores. Within a head, the rows a pass writes lie before every
// source of later passes (sources satisfy idx[r] >= r), and every source a
// pass reads lies at or after its first output row, hence after every row
// an earlier pass wrote; inside a pass the barrier puts all reads before all
// writes. So one barrier per pass suffices. Rows with idx[r] = r stay where
// they are and cost nothing.
#include <hip/hip_cooperative_groups.h>

#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kInplaceThreads = 512;
constexpr int kInplaceUnroll = 8;   // rows per thread and pass (loads in flight: 2 x 8)

template <int CPR>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs p) {
  const int h = blockIdx.y;
  const int64_t pieces = (int64_t)p.n * CPR;
  const int64_t stride = (int64_t)gridDim.x * kAppendThreads;
  for (int64_t e = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x; e < pieces; e += stride) {
    const int r = (int)(e / CPR), ch = (int)(e % CPR);
    const u32x4_t kv = load16(p.k_src + h * p.ks_sh + (int64_t)r * p.ks_ss + ch * 8);
    const u32x4_t vv = load16(p.v_src + h * p.vs_sh + (int64_t)r * p.vs_ss + ch * 8);
    store16(p.k + h * p.k_sh + (int64_t)(p.row0 + r) * p.k_ss + ch * 8, kv);
    store16(p.v + h * p.v_sh + (int64_t)(p.row0 + r) * p.v_ss + ch * 8, vv);
    if (p.pos && ch == 0) p.pos[h * p.pos_sh + p.row0 + r] = p.pos0 + r;
  }
}

template <int CPR>
__global__ __launch_bounds__(kInplaceThreads) void inplace_kernel(InplaceArgs p) {
  constexpr int RPP = kInplaceThreads / CPR;   // rows per workgroup and row pass
  constexpr int U = kInplaceUnroll;
  constexpr int ROWS_PER_WG = RPP * U;
  __shared__ int64_t offs[kInplaceThreads];
  const int tid = threadIdx.x, ch = tid % CPR, rr = tid / CPR;
  const bool lds_heads = p.H < kInplaceThreads;   // offsets[0 .. H] fit in LDS
  if (lds_heads && tid <= p.H) offs[tid] = p.offsets[tid];
  __syncthreads();
  auto off_at = [&](int i) { return lds_heads ? offs[i] : p.offsets[i]; };
  const int64_t per_pass = (int64_t)ROWS_PER_WG * gridDim.x;
  cooperative_groups::grid_group grid = cooperative_groups::this_grid();

  for (int64_t base = 0; base < p.total; base += per_pass) {   // uniform across the grid
    const int64_t g0 = base + (int64_t)blockIdx.x * ROWS_PER_WG + rr;
    // the head of this thread's first row (last h with offsets[h] <= g0)
    int h = 0;
    if (g0 < p.total) {
      int lo = 0, hi = p.H - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off_at(mid) <= g0) lo = mid;
        else hi = mid - 1;
      }
      h = lo;
    }
    u32x4_t kv[U], vv[U];
    int hd[U], row[U], pv[U];   // destination head and row (row -1: nothing to store)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + (int64_t)u * RPP;
      kv[u] = zero16();
      vv[u] = zero16();
      pv[u] = -1;
      row[u] = -1;
      hd[u] = 0;
      if (g < p.total) {
        while (h + 1 < p.H && g >= off_at(h + 1)) ++h;
        const int64_t r = g - off_at(h);
        const int src = p.idx[g];
        if (r >= 0 && r < p.S && src != r) {
          hd[u] = h;
          row[u] = (int)r;
          if (src >= 0 && src < p.S) {
            kv[u] = load16(p.k + h * p.k_sh + (int64_t)src * p.k_ss + ch * 8);
            vv[u] = load16(p.v + h * p.v_sh + (int64_t)src * p.v_ss + ch * 8);
            if (p.pos && ch == 0) pv[u] = p.pos[h * p.pos_sh + src];
          }
        }
      }
    }
    // every load of the pass has returned, in every workgroup, before any store
    __builtin_amdgcn_s_waitcnt(0);
    grid.sync();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (row[u] < 0) continue;
      const int64_t hh = hd[u], r = row[u];
      store16(p.k + hh * p.k_sh + r * p.k_ss + ch * 8, kv[u]);
      store16(p.v + hh * p.v_sh + r * p.v_ss + ch * 8, vv[u]);
      if (p.pos && ch == 0) p.pos[hh * p.pos_sh + r] = pv[u];
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n == 0 || a.H == 0) return hipSuccess;
  const int cpr = a.d / 8;
  const int64_t pieces = (int64_t)a.n * cpr;
  int64_t bx = (pieces + kAppendThreads - 1) / kAppendThreads;
  if (bx > 4096) bx = 4096;
  if (a.H > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)bx, (unsigned)a.H);
  switch (cpr) {
    case 8: hipLaunchKernelGGL(append_kernel<8>, grid, dim3(kAppendThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL(append_kernel<16>, grid, dim3(kAppendThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL(append_kernel<32>, grid, dim3(kAppendThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int CPR>
hipError_t launch_inplace_t(const InplaceArgs& a, hipStream_t s) {
  constexpr int rows_per_wg = kInplaceThreads / CPR * kInplaceUnroll;
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, inplace_kernel<CPR>, kInplaceThreads, 0);
  if (e != hipSuccess) return e;
  if (!coop || per_cu < 1 || cus < 1) return hipErrorNotSupported;
  const int64_t need = (a.total + rows_per_wg - 1) / rows_per_wg;
  const int64_t resident = (int64_t)per_cu * cus;
  const unsigned grid = (unsigned)(need < resident ? need : resident);
  InplaceArgs args = a;
  void* params[] = {&args};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(inplace_kernel<CPR>), dim3(grid),
                                 dim3(kInplaceThreads), params, 0, s);
  return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_compact_inplace(const InplaceArgs& a, hipStream_t s) {
  if (a.H == 0 || a.total <= 0) return hipSuccess;
  switch (a.d / 8) {
    case 8: return launch_inplace_t<8>(a, s);
    case 16: return launch_inplace_t<16>(a, s);
    case 32: return launch_inplace_t<32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fam

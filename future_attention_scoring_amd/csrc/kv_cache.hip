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
// indices satisfy idx[r] >= r, so a forward sweep is safe: one workgroup per
// head walks its output rows in tiles, loads every source row of a tile into
// registers, waits for all of those loads across the workgroup, and only then
// stores the tile. A tile's sources lie at or after the tile's first row,
// hence after every row an earlier tile wrote, and the stores of a tile go to
// rows that later tiles never read (their sources lie at or after their own
// first row). Rows with idx[r] = r stay where they are and cost nothing.
// The sweep of one head is sequential by construction; heads run in
// parallel, so the kernel is latency-bound for a few heads and approaches
// the per-CU copy rate for many.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kInplaceThreads = 512;
constexpr int kInplaceUnroll = 8;   // row passes per tile (loads in flight per thread: 2 x 8)

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
  constexpr int RPP = kInplaceThreads / CPR;   // rows per pass
  constexpr int U = kInplaceUnroll;
  constexpr int TILE = RPP * U;
  const int h = blockIdx.x;
  const int64_t base = p.offsets[h];
  const int64_t kept = p.offsets[h + 1] - base;
  const int n = (int)(kept < p.S ? (kept > 0 ? kept : 0) : p.S);   // never past the region
  const int tid = threadIdx.x, ch = tid % CPR, rr = tid / CPR;
  uint16_t* kh = p.k + h * p.k_sh;
  uint16_t* vh = p.v + h * p.v_sh;
  int32_t* ph = p.pos ? p.pos + h * p.pos_sh : nullptr;

  for (int t0 = 0; t0 < n; t0 += TILE) {   // uniform across the workgroup
    u32x4_t kv[U], vv[U];
    int src[U], pv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = t0 + u * RPP + rr;
      src[u] = r < n ? p.idx[base + r] : r;
      kv[u] = zero16();
      vv[u] = zero16();
      pv[u] = -1;
      if (src[u] != r && src[u] >= 0 && src[u] < p.S) {
        kv[u] = load16(kh + (int64_t)src[u] * p.k_ss + ch * 8);
        vv[u] = load16(vh + (int64_t)src[u] * p.v_ss + ch * 8);
        if (ph && ch == 0) pv[u] = ph[src[u]];
      }
    }
    // every load of the tile has returned before any store of the tile
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = t0 + u * RPP + rr;
      if (src[u] != r) {   // r < n here (rows past n carry src = r)
        store16(kh + (int64_t)r * p.k_ss + ch * 8, kv[u]);
        store16(vh + (int64_t)r * p.v_ss + ch * 8, vv[u]);
        if (ph && ch == 0) ph[r] = pv[u];
      }
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

hipError_t launch_compact_inplace(const InplaceArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const int cpr = a.d / 8;
  switch (cpr) {
    case 8: hipLaunchKernelGGL(inplace_kernel<8>, dim3((unsigned)a.H), dim3(kInplaceThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL(inplace_kernel<16>, dim3((unsigned)a.H), dim3(kInplaceThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL(inplace_kernel<32>, dim3((unsigned)a.H), dim3(kInplaceThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fam

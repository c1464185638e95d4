// Static cache regions: appending a chunk's rows and compacting in place
// (gfx950).
//
// KVP (section 4: long contexts are prefilled chunk by chunk and compressed
// after each chunk with physical tensor compaction) and the pruning blog
// (conclusion: a static cache can keep a fixed region per head and overwrite
// old entries in place instead of copying into a new tensor).
//
// Append. Four 16-byte pieces of (row, piece) per thread, all loads in
// flight, grid (pieces / 1024, heads); every head's rows row0 .. row0+n-1
// are written, and optionally their positions pos0 .. pos0+n-1.
//
// In-place compaction. Head h keeps the rows idx[offsets[h] + r] (ascending,
// as evict_select writes them) and moves row idx[...+r] to row r. Every read
// wants a row's original contents, so the only hazard is a row overwritten
// before its reader has read it. The kept rows of all heads (output index
// g = offsets[h] + r) are cut into chunks of R rows; a workgroup takes the
// next chunk by ticket (an atomic counter, so tickets follow start order),
// loads its source rows into registers, raises its chunk's flag, waits for
// the flags of the earlier chunks that may read its output rows, and stores.
//   * Which chunks read my rows: ascending indices give idx[r] >= r, and the
//     shift idx[r] - r never decreases along a head, so it is at most the
//     head's last shift D. Rows a.. of head h are read only by outputs r' >=
//     a - D of that head, all in chunks from the one holding row a - D up to
//     mine. Rows of a later head inside my chunk are read only from my own
//     chunk (outputs never lie after their sources), which the workgroup
//     orders itself (all loads, a barrier, then the stores).
//   * No deadlock and no residency requirement: a chunk waits only for
//     chunks with smaller tickets, whose workgroups have already started and
//     themselves wait only for smaller tickets.
//   * No fences: a flag is raised after the chunk's loads have returned
//     their data, and the stores that depend on it are issued after the flag
//     is seen; nothing written in the launch is ever read in it.
// The tickets and flags live in a caller workspace that a fill kernel clears
// first. Rows with idx[r] = r stay where they are and cost nothing. Indices
// that are not ascending give unspecified row contents but never an access
// out of bounds, and every wait still ends (it only involves earlier
// tickets).
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendPer = 4;   // pieces per thread
constexpr int kInplaceThreads = 512;
constexpr int kInplaceUnroll = 8;   // rows per thread and chunk (loads in flight: 2 x 8)

template <int CPR>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs p) {
  // kAppendPer pieces per thread, kAppendThreads apart, all loads in flight
  // (clamped pieces past the end are loaded and not stored)
  const int h = blockIdx.y;
  const int64_t pieces = (int64_t)p.n * CPR;
  const int64_t e0 = (int64_t)blockIdx.x * kAppendThreads * kAppendPer + threadIdx.x;
  u32x4_t kv[kAppendPer], vv[kAppendPer];
#pragma unroll
  for (int u = 0; u < kAppendPer; ++u) {
    const int64_t e = e0 + (int64_t)u * kAppendThreads;
    const int64_t ec = e < pieces ? e : pieces - 1;
    const int r = (int)(ec / CPR), ch = (int)(ec % CPR);
    kv[u] = load16(p.k_src + h * p.ks_sh + (int64_t)r * p.ks_ss + ch * 8);
    vv[u] = load16(p.v_src + h * p.vs_sh + (int64_t)r * p.vs_ss + ch * 8);
  }
#pragma unroll
  for (int u = 0; u < kAppendPer; ++u) {
    const int64_t e = e0 + (int64_t)u * kAppendThreads;
    if (e < pieces) {
      const int r = (int)(e / CPR), ch = (int)(e % CPR);
      store16(p.k + h * p.k_sh + (int64_t)(p.row0 + r) * p.k_ss + ch * 8, kv[u]);
      store16(p.v + h * p.v_sh + (int64_t)(p.row0 + r) * p.v_ss + ch * 8, vv[u]);
      if (p.pos && ch == 0) p.pos[h * p.pos_sh + p.row0 + r] = p.pos0 + r;
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) w[i] = 0u;
}

template <int CPR>
__global__ __launch_bounds__(kInplaceThreads) void inplace_kernel(InplaceArgs p) {
  constexpr int RPP = kInplaceThreads / CPR;   // rows per row pass of the workgroup
  constexpr int U = kInplaceUnroll;
  constexpr int R = RPP * U;                   // rows per chunk
  static_assert(R >= kInplaceMinChunkRows, "workspace sized for chunks of at least kInplaceMinChunkRows");
  __shared__ int64_t offs[kInplaceThreads];
  __shared__ int sh_ticket, sh_umin, sh_gave_up;
  const int tid = threadIdx.x, ch = tid % CPR, rr = tid / CPR;
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t* ticket = p.ws;
  uint32_t* flags = p.ws + kInplaceFlags0;
  const bool lds_heads = p.H < kInplaceThreads;   // offsets[0 .. H] fit in LDS
  if (lds_heads && tid <= p.H) offs[tid] = p.offsets[tid];
  if (tid == 0) sh_ticket = (int)__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  auto off_at = [&](int i) { return lds_heads ? offs[i] : p.offsets[i]; };
  const int t = sh_ticket;
  const int64_t c0 = (int64_t)t * R;   // first output of the chunk (c0 < total by the grid size)

  // the head of the chunk's first row (last h with offsets[h] <= c0), and of
  // this thread's first row
  auto head_of = [&](int64_t g) {
    int lo = 0, hi = p.H - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off_at(mid) <= g) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  if (tid == 0) {
    // earliest chunk that may read rows of the first head from row a on
    const int h0 = head_of(c0);
    const int64_t o0 = off_at(h0), e0 = off_at(h0 + 1) < p.total ? off_at(h0 + 1) : p.total;
    const int64_t a = c0 - o0;
    int64_t shift = e0 > o0 ? (int64_t)p.idx[e0 - 1] - (e0 - 1 - o0) : 0;   // the head's last shift
    shift = shift < 0 ? 0 : shift;
    const int64_t lo_row = a > shift ? a - shift : 0;
    sh_umin = (int)((o0 + lo_row) / R);
  }
  // Loads are issued unconditionally at clamped, in-bounds addresses (so that
  // no branch writes a register a load is still filling, which would stall
  // every row on the previous one); what is stored is decided at the end.
  const int64_t g0 = c0 + rr;
  int h = head_of(g0 < p.total ? g0 : p.total - 1);
  int hd[U], row[U], src[U];   // head, destination row (-1: nothing to store), source row (-1: zero row)
  // heads first (loops over the offsets), then all index loads in flight
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + (int64_t)u * RPP;
    const int64_t gc = g < p.total ? g : p.total - 1;
    while (h + 1 < p.H && gc >= off_at(h + 1)) ++h;
    hd[u] = h;
    const int64_t r = gc - off_at(h);
    row[u] = (g < p.total && r >= 0 && r < p.S) ? (int)r : -1;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + (int64_t)u * RPP;
    src[u] = p.idx[g < p.total ? g : p.total - 1];
  }
  u32x4_t kv[U], vv[U];
  int pv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool in = src[u] >= 0 && src[u] < p.S;
    if (row[u] == src[u]) row[u] = -1;   // stays where it is
    if (!in) src[u] = -1;
    const int64_t sr = in ? src[u] : 0;
    kv[u] = load16(p.k + hd[u] * p.k_sh + sr * p.k_ss + ch * 8);
    vv[u] = load16(p.v + hd[u] * p.v_sh + sr * p.v_ss + ch * 8);
    pv[u] = p.pos ? p.pos[hd[u] * p.pos_sh + sr] : 0;
  }
  // every load of the chunk has returned its data: raise the chunk's flag
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) __hip_atomic_store(flags + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // wait for the earlier chunks that may read this chunk's output rows; a
  // wait that runs out of polls leaves the chunk's rows unwritten and counts
  // the chunk in the error word (the bound is never reached in practice)
  if (wave == 0) {
    bool gave_up = false;
    for (int u0 = sh_umin; u0 < t && !gave_up; u0 += 64) {
      const int u = u0 + lane;
      bool pending = u < t;
      for (int spin = 0; spin < p.spin_limit && __any(pending); ++spin) {
        if (pending) pending = __hip_atomic_load(flags + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
        if (__any(pending)) __builtin_amdgcn_s_sleep(1);
      }
      gave_up = __any(pending);
    }
    if (lane == 0) {
      sh_gave_up = gave_up ? 1 : 0;
      if (gave_up) __hip_atomic_fetch_add(p.ws + kInplaceErrorWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (sh_gave_up) return;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (row[u] < 0) continue;
    const int64_t hh = hd[u], r = row[u];
    const bool zero = src[u] < 0;   // an index outside the region: zero row, position -1
    store16(p.k + hh * p.k_sh + r * p.k_ss + ch * 8, zero ? zero16() : kv[u]);
    store16(p.v + hh * p.v_sh + r * p.v_ss + ch * 8, zero ? zero16() : vv[u]);
    if (p.pos && ch == 0) p.pos[hh * p.pos_sh + r] = zero ? -1 : pv[u];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n == 0 || a.H == 0) return hipSuccess;
  const int cpr = a.d / 8;
  const int64_t pieces = (int64_t)a.n * cpr;
  const int64_t bx = (pieces + kAppendThreads * kAppendPer - 1) / (kAppendThreads * kAppendPer);
  if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
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
  constexpr int rows_per_chunk = kInplaceThreads / CPR * kInplaceUnroll;
  const int64_t chunks = (a.total + rows_per_chunk - 1) / rows_per_chunk;
  if (chunks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int64_t words = kInplaceFlags0 + chunks;
  const int64_t fb = (words + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(fb < 1024 ? fb : 1024)), dim3(256), 0, s, a.ws, words);
  hipLaunchKernelGGL(inplace_kernel<CPR>, dim3((unsigned)chunks), dim3(kInplaceThreads), 0, s, a);
  return hipGetLastError();
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

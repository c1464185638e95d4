// Ranking-quality measures of per-head scores (gfx950).
//
// KVP (section 3: the top-b entries of a ranking form the cache for every
// budget b, so eviction is ranking; 3.1.1: a ranking is scored by the
// future-attention importance of the entries it evicts, accumulated over all
// budgets as a cost-versus-budget area and normalised by the same area of
// the optimal ranking). KVpop (Figure 7: top-k retention recall, the share
// of the teacher's kept set that another scorer's kept set also holds under
// the same budget).
//
// rank_count / rank_place: order[h, r] is the position of the r-th best
// entry of head h (score descending, ties to the lower position, -0 equal to
// +0, NaN last). A stable least-significant-digit radix sort of the
// complemented order key, 8 bits per pass, between two buffers of (key,
// position) pairs in the workspace; the first pass reads the scores and the
// last writes only positions. Each pass is three launches: rank_count writes
// the digit counts of every (4096-entry tile, head), rank_scan turns them
// into each tile's first slot per digit (one exclusive scan per head over
// the digit-major counts), and rank_place ranks each entry among the tile's
// entries with its digit (eight wave ballots, the wave's running count of
// the digit, a per-digit prefix over the waves) and scatters it, keeping the
// order of equal digits.
//
// cost_kernel: cost[h] = sum_r (r + 1) * importance[h, order[h, r]], which
// equals the sum over budgets b = 0 .. n of the importance evicted at b
// (the entry ranked r is evicted for the r + 1 budgets b <= r). One
// workgroup per block of 4096 entries of a head (all gathers of a thread in
// flight) writes an fp64 partial sum; cost_reduce_kernel adds a head's
// partials in block order, so the result is deterministic.
//
// overlap_kernel: common[h] = |set(a_h) & set(b_h)| for two kept-index lists
// per head, with a bitmap of the head's positions in LDS (per window of
// 262144 positions).
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kRankThreads = 256;
constexpr int kRankWaves = kRankThreads / 64;
constexpr int kDigits = 256;
constexpr int kRankSteps = 16;                          // 64-lane steps per wave and tile
constexpr int kRankTile = kRankThreads * kRankSteps;    // 4096 entries

// Lanes of the wave whose digit equals this lane's (among the lanes in `live`).
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool live) {
  uint64_t peers = __ballot(live);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  return peers;
}

// Keys and positions of the entries e0 + j * stride (j < kRankSteps) at pass
// `pass` (pass 0 reads the scores). Entries past n are read at n - 1 (the
// callers mark them invalid); the pass branch sits outside the loads, so
// all of them are in flight at once.
__device__ __forceinline__ void rank_entries(const RankArgs& p, int h, int pass, int e0, int stride,
                                             uint32_t (&key)[kRankSteps], uint32_t (&pos)[kRankSteps]) {
  if (pass == 0) {
    const float* sc = p.scores + h * p.row_stride;
#pragma unroll
    for (int j = 0; j < kRankSteps; ++j) {
      const int e = e0 + j * stride;
      key[j] = ~order_key(sc[e < p.n ? e : p.n - 1]);
      pos[j] = (uint32_t)e;
    }
  } else {
    const u32x2_t* src = static_cast<const u32x2_t*>(p.ws) + ((int64_t)((pass & 1) ? 0 : p.H) + h) * p.n;
#pragma unroll
    for (int j = 0; j < kRankSteps; ++j) {
      const int e = e0 + j * stride;
      const u32x2_t kv = src[e < p.n ? e : p.n - 1];
      key[j] = kv.x;
      pos[j] = kv.y;
    }
  }
}

__device__ __forceinline__ int* rank_hist(const RankArgs& p, int h) {
  int* base = reinterpret_cast<int*>(static_cast<u32x2_t*>(p.ws) + (int64_t)2 * p.H * p.n);
  return base + (int64_t)h * kDigits * p.ntiles;   // [H][256 digits][ntiles]
}

// Pass `pass`: digit counts of one tile of one head.
// tile_major: counts stored [tile][digit] (read by a fused rank_place)
// instead of [digit][tile] (read by rank_scan).
__global__ __launch_bounds__(kRankThreads) void rank_count(RankArgs p, int pass, int tile_major) {
  __shared__ int cnt[kDigits];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int shift = 8 * pass;
  if (threadIdx.x < kDigits) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int e0 = tile * kRankTile;
  uint32_t key[kRankSteps], pos[kRankSteps];
  rank_entries(p, h, pass, e0 + (int)threadIdx.x, kRankThreads, key, pos);
#pragma unroll
  for (int j = 0; j < kRankSteps; ++j)
    if (e0 + j * kRankThreads + (int)threadIdx.x < p.n) atomicAdd(&cnt[(key[j] >> shift) & 255u], 1);
  __syncthreads();
  if (threadIdx.x < kDigits)
    rank_hist(p, h)[tile_major ? (int64_t)tile * kDigits + threadIdx.x : (int64_t)threadIdx.x * p.ntiles + tile] =
        cnt[threadIdx.x];
}

// Pass `pass`: the counts of every (digit, tile) of a head, digit-major,
// become exclusive offsets in place: the slots before a tile's entries of a
// digit hold every smaller digit and that digit's entries of earlier tiles.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void rank_scan(RankArgs p) {
  __shared__ int sh[kScanThreads / 64];
  int* hist = rank_hist(p, blockIdx.x);
  const int64_t n = (int64_t)kDigits * p.ntiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;   // entries of the chunks before
  for (int64_t c0 = 0; c0 < n; c0 += kScanThreads * 16) {   // uniform across the workgroup
    const int64_t i0 = c0 + (int64_t)threadIdx.x * 16;
    int c[16], sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      c[j] = i0 + j < n ? hist[i0 + j] : 0;
      sum += c[j];
    }
    const int incl = wave_scan(sum);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    int run = carry + incl - sum, all = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      run += w < wave ? sh[w] : 0;
      all += sh[w];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (i0 + j < n) hist[i0 + j] = run;
      run += c[j];
    }
    carry += all;
    __syncthreads();
  }
}

// Pass `pass`: place one tile's entries after the slots rank_scan reserved;
// inside the tile, (wave, step, lane) order is entry order, so equal digits
// keep their order and the sort is stable.
// FUSED: rank_scan did not run, the digit counts are raw and tile-major; with at most
// kFusedTiles tiles a head, every workgroup forms its own first slots: digit
// d's slot = entries of smaller digits in all tiles + entries of digit d in
// earlier tiles (one exclusive scan over the digits).
constexpr int kFusedTiles = 64;
template <bool FUSED>
__global__ __launch_bounds__(kRankThreads) void rank_place(RankArgs p, int pass) {
  __shared__ int base[kDigits];                // this tile's first slot per digit
  __shared__ int wcnt[kRankWaves][kDigits];    // per wave: running count, then exclusive prefix
  __shared__ int ssh[kRankWaves];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int shift = 8 * pass;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  if constexpr (FUSED) {
    const int* cnt = rank_hist(p, h) + tid;   // digit tid of every tile: [tile][digit], coalesced
    int c[kFusedTiles];
#pragma unroll
    for (int t = 0; t < kFusedTiles; ++t) c[t] = cnt[(t < p.ntiles ? t : p.ntiles - 1) * kDigits];   // all in flight
    int all = 0, before = 0;
#pragma unroll
    for (int t = 0; t < kFusedTiles; ++t) {
      all += t < p.ntiles ? c[t] : 0;
      before += t < tile ? c[t] : 0;
    }
    // exclusive scan of the digit totals over the 256 threads
    const int incl = wave_scan(all);
    if (lane == 63) ssh[wave] = incl;
    __syncthreads();
    int prev = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) prev += w < wave ? ssh[w] : 0;
    base[tid] = prev + incl - all + before;
  } else {
    base[tid] = rank_hist(p, h)[(int64_t)tid * p.ntiles + tile];
  }
#pragma unroll
  for (int w = 0; w < kRankWaves; ++w) wcnt[w][tid] = 0;
  __syncthreads();

  uint32_t key[kRankSteps], pos[kRankSteps], dg[kRankSteps];
  int rank[kRankSteps];
  const int e0 = tile * kRankTile + wave * 64 * kRankSteps;
  // every load of the thread in flight: clamped entries, no branch between
  // the loads (entries past n are marked invalid below)
  rank_entries(p, h, pass, e0 + lane, 64, key, pos);
#pragma unroll
  for (int st = 0; st < kRankSteps; ++st) {
    const bool valid = e0 + st * 64 + lane < p.n;
    const uint32_t d = (key[st] >> shift) & 255u;
    const uint64_t peers = digit_peers(d, valid);
    const uint64_t bef = peers & below;
    // all lanes of a digit read the wave's count before its first lane adds
    // the step's lanes (LDS operations of a wave run in order)
    const int seen = valid ? wcnt[wave][d] : 0;
    rank[st] = valid ? seen + (int)__popcll(bef) : -1;
    dg[st] = d;
    if (valid && bef == 0ull) wcnt[wave][d] = seen + (int)__popcll(peers);
  }
  __syncthreads();
  if (tid < kDigits) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  u32x2_t* dst = static_cast<u32x2_t*>(p.ws) + ((int64_t)((pass & 1) ? p.H : 0) + h) * p.n;
  int32_t* out = p.order + (int64_t)h * p.n;
#pragma unroll
  for (int st = 0; st < kRankSteps; ++st) {
    if (rank[st] < 0) continue;
    const int at = base[dg[st]] + wcnt[wave][dg[st]] + rank[st];
    if (pass == 3) out[at] = (int32_t)pos[st];
    else dst[at] = u32x2_t{key[st], pos[st]};
  }
}

constexpr int kCostThreads = 256;
constexpr int kCostPer = kCostBlock / kCostThreads;   // entries per thread, all gathers in flight
static_assert(kCostPer * kCostThreads == kCostBlock, "cost block");

// Partial sum of (r + 1) * importance[order[r]] over one block of entries of
// one head, in fp64 with a fixed reduction order.
__global__ __launch_bounds__(kCostThreads) void cost_kernel(CostArgs p) {
  __shared__ double red[kCostThreads / 64];
  const int blk = blockIdx.x, h = blockIdx.y;
  const float* imp = p.importance + h * p.row_stride;
  const int32_t* ord = p.order + (int64_t)h * p.n;
  const int r0 = blk * kCostBlock + threadIdx.x;
  int j[kCostPer];
  float x[kCostPer];
#pragma unroll
  for (int u = 0; u < kCostPer; ++u) {   // clamped entries: no branch between the loads
    const int r = r0 + u * kCostThreads;
    j[u] = ord[r < p.n ? r : p.n - 1];
  }
#pragma unroll
  for (int u = 0; u < kCostPer; ++u) x[u] = imp[j[u] >= 0 && j[u] < p.n ? j[u] : 0];
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kCostPer; ++u) {
    const int r = r0 + u * kCostThreads;
    const bool ok = r < p.n && j[u] >= 0 && j[u] < p.n;
    acc = fma((double)(r + 1), ok ? (double)x[u] : 0.0, acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kCostThreads / 64; ++w) t += red[w];
    p.part[(int64_t)h * gridDim.x + blk] = t;
  }
}

// cost[h] = the sum of the head's block partial sums, in block order.
__global__ __launch_bounds__(64) void cost_reduce_kernel(CostArgs p, int nb) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= p.H) return;
  const double* part = p.part + (int64_t)h * nb;
  double t = 0.0;
  for (int b = 0; b < nb; ++b) t += part[b];
  p.cost[h] = t;
}

// KVP's normalised cost: each head's two costs summed from their block
// partial sums in block order (the same sums cost_reduce_kernel forms), then
// their quotient; 1 where both are 0 (no importance to evict at any budget:
// every ranking is optimal).
__global__ __launch_bounds__(64) void cost_ratio_kernel(const double* part, const double* part_opt, int H,
                                                        int nb, double* ratio) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= H) return;
  double c = 0.0, c_opt = 0.0;
  for (int b = 0; b < nb; ++b) {
    c += part[(int64_t)h * nb + b];
    c_opt += part_opt[(int64_t)h * nb + b];
  }
  ratio[h] = (c == 0.0 && c_opt == 0.0) ? 1.0 : c / c_opt;
}

constexpr int kOverlapThreads = 1024;

constexpr int kOverlapBatch = 8;   // list entries per thread and batch
__global__ __launch_bounds__(kOverlapThreads) void overlap_kernel(OverlapArgs p) {
  extern __shared__ uint32_t bits[];
  __shared__ int64_t part[kOverlapThreads / 64];
  const int h = blockIdx.x;
  const int64_t a0 = p.off_a[h], a1 = p.off_a[h + 1];
  const int64_t b0 = p.off_b[h], b1 = p.off_b[h + 1];
  int64_t cnt = 0;
  // windows of kOverlapWindow positions, one bitmap in LDS each (one window
  // up to 262144 positions; longer heads re-read both lists per window)
  for (int w0 = 0; w0 < p.S; w0 += kOverlapWindow) {
    const int wn = p.S - w0 < kOverlapWindow ? p.S - w0 : kOverlapWindow;
    const int words = (wn + 31) / 32;
    for (int w = threadIdx.x; w < words; w += kOverlapThreads) bits[w] = 0u;
    __syncthreads();
    // batches of kOverlapBatch entries per thread, all loads in flight
    // (clamped indices; entries past the list are dropped after the loads)
    for (int64_t i0 = a0 + threadIdx.x; i0 < a1; i0 += (int64_t)kOverlapThreads * kOverlapBatch) {
      int x[kOverlapBatch];
#pragma unroll
      for (int u = 0; u < kOverlapBatch; ++u) {
        const int64_t i = i0 + (int64_t)u * kOverlapThreads;
        x[u] = p.idx_a[i < a1 ? i : a1 - 1];
      }
#pragma unroll
      for (int u = 0; u < kOverlapBatch; ++u) {
        const int y = x[u] - w0;
        if (i0 + (int64_t)u * kOverlapThreads < a1 && x[u] >= w0 && y < wn)
          atomicOr(&bits[y >> 5], 1u << (y & 31));
      }
    }
    __syncthreads();
    for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (int64_t)kOverlapThreads * kOverlapBatch) {
      int x[kOverlapBatch];
#pragma unroll
      for (int u = 0; u < kOverlapBatch; ++u) {
        const int64_t i = i0 + (int64_t)u * kOverlapThreads;
        x[u] = p.idx_b[i < b1 ? i : b1 - 1];
      }
#pragma unroll
      for (int u = 0; u < kOverlapBatch; ++u) {
        const int y = x[u] - w0;
        if (i0 + (int64_t)u * kOverlapThreads < b1 && x[u] >= w0 && y < wn && ((bits[y >> 5] >> (y & 31)) & 1u)) {
          // count each position of b once: clear it after the first hit
          const uint32_t old = atomicAnd(&bits[y >> 5], ~(1u << (y & 31)));
          if ((old >> (y & 31)) & 1u) ++cnt;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t t = 0;
    for (int w = 0; w < kOverlapThreads / 64; ++w) t += part[w];
    p.common[h] = t;
  }
}

}  // namespace

hipError_t launch_rank(const RankArgs& a, hipStream_t s) {
  if (a.H == 0 || a.n == 0) return hipSuccess;
  const dim3 grid((unsigned)a.ntiles, (unsigned)a.H);
  const bool fused = a.ntiles <= kFusedTiles;   // the place launch forms its own slots
  for (int pass = 0; pass < 4; ++pass) {
    hipLaunchKernelGGL(rank_count, grid, dim3(kRankThreads), 0, s, a, pass, fused ? 1 : 0);
    if (fused) {
      hipLaunchKernelGGL(rank_place<true>, grid, dim3(kRankThreads), 0, s, a, pass);
    } else {
      hipLaunchKernelGGL(rank_scan, dim3((unsigned)a.H), dim3(kScanThreads), 0, s, a);
      hipLaunchKernelGGL(rank_place<false>, grid, dim3(kRankThreads), 0, s, a, pass);
    }
  }
  return hipGetLastError();
}

hipError_t launch_cost(const CostArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const int nb = cost_blocks(a.n);
  if (nb > 0) hipLaunchKernelGGL(cost_kernel, dim3((unsigned)nb, (unsigned)a.H), dim3(kCostThreads), 0, s, a);
  hipLaunchKernelGGL(cost_reduce_kernel, dim3((unsigned)((a.H + 63) / 64)), dim3(64), 0, s, a, nb);
  return hipGetLastError();
}

hipError_t launch_cost_ratio(const RankArgs& rank_scores, const RankArgs& rank_imp, const CostArgs& cost,
                             double* part_opt, double* ratio, hipStream_t s) {
  if (cost.H == 0) return hipSuccess;
  const int nb = cost_blocks(cost.n);
  hipError_t e = launch_rank(rank_scores, s);
  if (e != hipSuccess) return e;
  if (nb > 0) hipLaunchKernelGGL(cost_kernel, dim3((unsigned)nb, (unsigned)cost.H), dim3(kCostThreads), 0, s, cost);
  e = launch_rank(rank_imp, s);   // overwrites the order once the first costs are formed (stream order)
  if (e != hipSuccess) return e;
  CostArgs opt = cost;
  opt.part = part_opt;
  if (nb > 0) hipLaunchKernelGGL(cost_kernel, dim3((unsigned)nb, (unsigned)cost.H), dim3(kCostThreads), 0, s, opt);
  hipLaunchKernelGGL(cost_ratio_kernel, dim3((unsigned)((cost.H + 63) / 64)), dim3(64), 0, s, cost.part, part_opt,
                     cost.H, nb, ratio);
  return hipGetLastError();
}

hipError_t launch_overlap(const OverlapArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const int window = a.S < kOverlapWindow ? a.S : kOverlapWindow;
  const size_t lds = (size_t)((window + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)a.H), dim3(kOverlapThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace fam

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
// rank_kernel: order[h, r] is the position of the r-th best entry of head h
// (score descending, ties to the lower position, -0 equal to +0, NaN last).
// One workgroup per head runs a stable least-significant-digit radix sort on
// the complemented order key, 8 bits per pass, between two buffers of (key,
// position) pairs in the workspace; the first pass reads the scores and the
// last writes only positions. A pass counts its digits over the whole head
// (LDS atomics), scans the 256 counts into bases, then walks the head in
// tiles of 4096 entries in order. Inside a tile an entry's rank among the
// entries with its digit comes from eight wave ballots (the lanes that share
// its digit), the wave's running count of that digit, and a per-digit prefix
// over the 16 waves, so the scatter keeps the order of equal digits and the
// sort is stable.
//
// cost_kernel: cost[h] = sum_r (r + 1) * importance[h, order[h, r]], which
// equals the sum over budgets b = 0 .. n of the importance evicted at b
// (the entry ranked r is evicted for the r + 1 budgets b <= r). fp64
// partial sums in a fixed order, so the result is deterministic.
//
// overlap_kernel: common[h] = |set(a_h) & set(b_h)| for two kept-index lists
// per head, with a bitmap of the head's positions in LDS.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / 64;
constexpr int kDigits = 256;
constexpr int kRankSteps = 4;                           // 64-lane steps per wave and tile
constexpr int kRankTile = kRankThreads * kRankSteps;

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

__global__ __launch_bounds__(kRankThreads) void rank_kernel(RankArgs p) {
  __shared__ int base[kDigits];                // digit counts, then running offsets
  __shared__ int next[kDigits];                // counts of the pass's digit
  __shared__ int wcnt[kRankWaves][kDigits];    // per wave: count, then exclusive prefix
  const int h = blockIdx.x;
  const int n = p.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = p.scores + h * p.row_stride;
  u32x2_t* buf0 = static_cast<u32x2_t*>(p.ws) + (int64_t)h * n;
  u32x2_t* buf1 = static_cast<u32x2_t*>(p.ws) + ((int64_t)p.H + h) * n;
  int32_t* out = p.order + (int64_t)h * n;
  const uint64_t below = (1ull << lane) - 1ull;

  if (tid < kDigits) {
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) wcnt[w][tid] = 0;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    const u32x2_t* src = pass == 1 || pass == 3 ? buf0 : buf1;   // pass 0 reads the scores
    u32x2_t* dst = pass == 0 || pass == 2 ? buf0 : buf1;         // pass 3 writes positions
    if (tid < kDigits) next[tid] = 0;
    __syncthreads();
    for (int e = tid; e < n; e += kRankThreads) {
      const uint32_t key = pass == 0 ? ~order_key(srow[e]) : src[e].x;
      atomicAdd(&next[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    // exclusive scan of the 256 digit counts (wave 0, four digits per lane)
    if (wave == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = next[4 * lane + i];
        sum += c[i];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      int run = incl - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[4 * lane + i] = run;
        run += c[i];
      }
    }
    __syncthreads();

    // Tiles of kRankTile entries; wave w takes the contiguous 256 entries
    // t0 + 256 w .. in four 64-lane steps, so (wave, step, lane) order is
    // entry order. A step ranks its lanes among the wave's earlier entries of
    // the same digit (the wave's running count in LDS plus the lanes below
    // with that digit); after the tile a per-digit prefix over the waves
    // gives every entry its place.
    for (int t0 = 0; t0 < n; t0 += kRankTile) {   // uniform across the workgroup
      uint32_t key[kRankSteps], pos[kRankSteps], dg[kRankSteps];
      int rank[kRankSteps];
#pragma unroll
      for (int st = 0; st < kRankSteps; ++st) {
        const int e = t0 + wave * 64 * kRankSteps + st * 64 + lane;
        key[st] = 0;
        pos[st] = 0;
        if (e < n) {
          if (pass == 0) {
            key[st] = ~order_key(srow[e]);
            pos[st] = (uint32_t)e;
          } else {
            const u32x2_t kv = src[e];
            key[st] = kv.x;
            pos[st] = kv.y;
          }
        }
      }
#pragma unroll
      for (int st = 0; st < kRankSteps; ++st) {
        const int e = t0 + wave * 64 * kRankSteps + st * 64 + lane;
        const bool valid = e < n;
        const uint32_t d = (key[st] >> shift) & 255u;
        const uint64_t peers = digit_peers(d, valid);
        const uint64_t before = peers & below;
        // all lanes of a digit read the wave's count before its first lane
        // adds the step's lanes (LDS operations of a wave run in order)
        const int seen = valid ? wcnt[wave][d] : 0;
        rank[st] = valid ? seen + (int)__popcll(before) : -1;
        dg[st] = d;
        if (valid && before == 0ull) wcnt[wave][d] = seen + (int)__popcll(peers);
      }
      __syncthreads();
      int total = 0;
      if (tid < kDigits) {
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) {
          const int c = wcnt[w][tid];
          wcnt[w][tid] = total;
          total += c;
        }
      }
      __syncthreads();
#pragma unroll
      for (int st = 0; st < kRankSteps; ++st) {
        if (rank[st] < 0) continue;
        const int at = base[dg[st]] + wcnt[wave][dg[st]] + rank[st];
        if (pass == 3) out[at] = (int32_t)pos[st];
        else dst[at] = u32x2_t{key[st], pos[st]};
      }
      __syncthreads();
      if (tid < kDigits) {
        base[tid] += total;
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) wcnt[w][tid] = 0;
      }
      __syncthreads();
    }
  }
}

constexpr int kCostThreads = 1024;
constexpr int kCostUnroll = 4;   // gathers in flight per thread

__global__ __launch_bounds__(kCostThreads) void cost_kernel(CostArgs p) {
  __shared__ double part[kCostThreads];
  const int h = blockIdx.x;
  const float* imp = p.importance + h * p.row_stride;
  const int32_t* ord = p.order + (int64_t)h * p.n;
  double acc = 0.0;
  for (int r0 = threadIdx.x; r0 < p.n; r0 += kCostThreads * kCostUnroll) {
    int j[kCostUnroll];
    float x[kCostUnroll];
#pragma unroll
    for (int u = 0; u < kCostUnroll; ++u) {
      const int r = r0 + u * kCostThreads;
      j[u] = r < p.n ? ord[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kCostUnroll; ++u) x[u] = (j[u] >= 0 && j[u] < p.n) ? imp[j[u]] : 0.f;
#pragma unroll
    for (int u = 0; u < kCostUnroll; ++u)
      acc = fma((double)(r0 + u * kCostThreads + 1), (double)x[u], acc);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kCostThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.cost[h] = part[0];
}

constexpr int kOverlapThreads = 1024;

__global__ __launch_bounds__(kOverlapThreads) void overlap_kernel(OverlapArgs p) {
  extern __shared__ uint32_t bits[];
  __shared__ int64_t part[kOverlapThreads / 64];
  const int h = blockIdx.x;
  const int words = (p.S + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kOverlapThreads) bits[w] = 0u;
  __syncthreads();
  for (int64_t i = p.off_a[h] + threadIdx.x; i < p.off_a[h + 1]; i += kOverlapThreads) {
    const int x = p.idx_a[i];
    if (x >= 0 && x < p.S) atomicOr(&bits[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  int64_t cnt = 0;
  for (int64_t i = p.off_b[h] + threadIdx.x; i < p.off_b[h + 1]; i += kOverlapThreads) {
    const int x = p.idx_b[i];
    if (x >= 0 && x < p.S && ((bits[x >> 5] >> (x & 31)) & 1u)) {
      // count each position of b once: clear it after the first hit
      const uint32_t old = atomicAnd(&bits[x >> 5], ~(1u << (x & 31)));
      if ((old >> (x & 31)) & 1u) ++cnt;
    }
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
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)a.H), dim3(kRankThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cost(const CostArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  hipLaunchKernelGGL(cost_kernel, dim3((unsigned)a.H), dim3(kCostThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_overlap(const OverlapArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const size_t lds = (size_t)((a.S + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)a.H), dim3(kOverlapThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace fam

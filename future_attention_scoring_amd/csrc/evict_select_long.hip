// Per-head top-k selection for heads beyond 131072 candidates (gfx950): the
// same selection as evict_select.hip's three launches (whose per-chunk
// register and LDS arrays stop at 33 chunks a head), in one launch after a
// small fill, for up to 2^20 candidates a head (long contexts such as LKV's
// 262k+ tokens).
//
// KVpop ("The KVpop Scoring Module", Figure 1): sinks and the protected
// window are always kept; the rest of the budget goes to the best-scored
// long-range tokens. KVP (section 3): the cache is the top of a ranking.
// Ties are broken towards the lower position, -0.0 equals +0.0 and NaN ranks
// below every number, so exactly one kept set is correct.
//
// Keys. A score maps to an order-preserving u32 key (NaN -> 1; 0 is reserved
// for "not a candidate"). The chosen set is the n_choose largest keys, equal
// keys taken by ascending position.
//
// Rounds. A head's candidates are cut into chunks of 4096 positions, one
// workgroup per chunk, every thread holding 16 consecutive keys in registers
// for the whole launch. The key is resolved 12, 12 and 8 bits at a time:
//   round r (1..3): every chunk adds the histogram of level r's key field
//     over its keys that match the levels decided so far into the head's
//     histogram (agent-scope atomics), and reports its count of keys above
//     the decided prefix and its count matching it. The chunk that arrives
//     last at the head's round counter resolves the round: it finds the bin
//     holding the needed key, publishes it with a flag, and the others,
//     waiting on the flag, go on with the next level;
//   when the needed keys fill their bin exactly (the usual case at level 2
//     or 3 on continuous scores) the next round's resolver only turns the
//     chunks' counts into output bases; after level 3 the remaining keys are
//     all equal and the lowest positions win: the counts of the chunks
//     (which are in position order) tell which chunk takes how many of them.
// Every chunk then writes its chosen positions in ascending order with one
// block scan. Chunk 0 also writes the sinks, the window and the offsets.
//
// Cross-workgroup data travels only through agent-scope atomic operations
// (adds, loads and stores), and a chunk arrives at a counter only after its
// own contributions have completed (s_waitcnt), so no cache writeback or
// invalidation is needed. The waits assume that all workgroups of the launch
// can be resident together: the host sizes each launch to the device's
// occupancy, one workgroup a CU to spare (more heads run as further
// launches). Every wait is bounded; a wait that runs out of polls counts
// itself in the workspace's error word and its workgroup exits, leaving its
// outputs unwritten.
//
// Measured at 131072 candidates x 8 heads this path costs about as much as
// the three launches (each round is a chain of agent-scope atomic round
// trips and block scans), and more at 120000 x 56 heads, so it serves only
// the heads the three launches cannot take.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

#include <atomic>

namespace fam {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kSelectChunk / kThreads;   // 16 consecutive positions
constexpr int kBins = 4096;                           // levels 1 and 2: 12 key bits each
constexpr int kBins3 = 256;                           // level 3: the last 8 key bits
constexpr int kBinsPerThread = kBins / kThreads;      // 16
constexpr int kSpinLimit = 1 << 22;                   // polls per wait (a bound; waits end long before)

// Per head slot of the workspace, in 32-bit words. The first kClear words
// (histograms, counters, flags, decisions) are cleared by the fill kernel
// before the selection launch.
constexpr int kRounds = 4;
constexpr int kHist1 = 0;                        // [4096] level-1 counts
constexpr int kHist2 = kHist1 + kBins;           // [4096] level-2 counts
constexpr int kHist3 = kHist2 + kBins;           // [256]  level-3 counts
constexpr int kArrive = kHist3 + kBins3;         // [4] arrivals per round
constexpr int kFlag = kArrive + kRounds;         // [4] round resolved
constexpr int kCtl = kFlag + kRounds;            // [8] the decisions
constexpr int kClear = kCtl + 8;
constexpr int kA = kClear;                       // [chunks] keys above the decided prefix
constexpr int kM = kA + kSelectLongMaxChunks;        // [chunks] keys matching it
constexpr int kBase = kM + kSelectLongMaxChunks;     // [chunks] output base of the chunk's chosen keys
constexpr int kSlotWords = (kBase + kSelectLongMaxChunks + 63) & ~63;
constexpr int kHeaderWords = kSelectLongHeaderWords; // word 0: error count (cleared by the first fill)
static_assert(kSlotWords <= kSelectLongSlotWordsMax, "slot layout exceeds the stated bound");

// Decision words.
constexpr int kCtlBin = 0;       // [3] bins decided at levels 1..3
constexpr int kCtlNeed = 3;      // keys still needed among those matching the decided prefix
constexpr int kCtlWhole = 4;     // 1: the needed keys fill the last decided bin
constexpr int kCtlFinal = 5;     // 1: bases published
constexpr int kCtlCstar = 6;     // split: chunks before cstar take all their equal keys,
constexpr int kCtlRstar = 7;     //        chunk cstar the first rstar

__device__ __forceinline__ uint32_t ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__host__ __device__ inline int chunks_of(const SelectArgs& p) {
  const int a0 = p.c0 & ~3;
  const int n = (p.c1 - a0 + kSelectChunk - 1) / kSelectChunk;
  return n < 1 ? 1 : n;
}

// Keys of positions base + 16*tid + i (0 outside the candidate range).
// Interior chunks of 16-byte aligned rows issue four 16-byte loads. So do the
// edge chunks of such rows when they hold a multiple of 4 scores: a piece of
// 4 positions then lies wholly inside the row or wholly past its end, and a
// piece past it loads the row's last piece (in bounds) and is masked like
// every position outside the candidates.
__device__ __forceinline__ void load_chunk(const SelectArgs& p, const float* row, int base,
                                           uint32_t (&k)[kPerThread]) {
  const int first = base + kPerThread * (int)threadIdx.x;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (aligned && (base < p.c0 || base + kSelectChunk > p.c1) && (p.S & 3) == 0) {
    f32x4_t f[kPerThread / 4];
#pragma unroll
    for (int it = 0; it < kPerThread / 4; ++it)
      f[it] = *reinterpret_cast<const f32x4_t*>(row + min(first + 4 * it, p.S - 4));
#pragma unroll
    for (int it = 0; it < kPerThread / 4; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int at = first + 4 * it + c;
        k[4 * it + c] = (at >= p.c0 && at < p.c1) ? order_key(f[it][c]) : 0u;
      }
    return;
  }
  if (aligned && base >= p.c0 && base + kSelectChunk <= p.c1) {
    f32x4_t f[kPerThread / 4];
#pragma unroll
    for (int it = 0; it < kPerThread / 4; ++it)
      f[it] = *reinterpret_cast<const f32x4_t*>(row + first + 4 * it);
#pragma unroll
    for (int it = 0; it < kPerThread / 4; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) k[4 * it + c] = order_key(f[it][c]);
    return;
  }
  // edge chunks of other rows: every load reads a clamped in-range position, then masks
  float f[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) f[i] = row[min(max(first + i, p.c0), p.c1 - 1)];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    k[i] = (first + i >= p.c0 && first + i < p.c1) ? order_key(f[i]) : 0u;
}

// Inclusive prefix sum over the workgroup's threads; `total` receives the sum.
__device__ int block_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan(v);
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int s = sh[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

// Shared state of one workgroup.
struct Lds {
  uint32_t hist[kBins];
  int sh[kThreads / 64];
  uint32_t ctl[8];
  int last;   // this workgroup arrived last (arrive)
  int ok;     // the wait ended with the flag set (wait_round)
};

// This workgroup's contributions are complete; arrive at the head's counter
// of round r. Returns true for the last chunk to arrive.
__device__ bool arrive(uint32_t* slot, int r, int nchunk, Lds& s) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(slot + kArrive + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.last = t == (uint32_t)(nchunk - 1) ? 1 : 0;
  }
  __syncthreads();
  return s.last != 0;
}

// Publish round r: the decisions (already stored) are complete, then the flag.
__device__ void publish(uint32_t* slot, int r) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) st(slot + kFlag + r, 1u);
}

// Wait for round r's flag; false if the wait ran out of polls.
__device__ bool wait_round(uint32_t* slot, int r, uint32_t* err, Lds& s) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (ld(slot + kFlag + r) == 0u && spins < kSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
    }
    const bool ok = spins < kSpinLimit || ld(slot + kFlag + r) != 0u;
    if (!ok) add(err, 1u);
    s.ok = ok ? 1 : 0;
  }
  __syncthreads();
  return s.ok != 0;
}

// The decisions, read once by thread 0 and shared.
__device__ void read_ctl(const uint32_t* slot, Lds& s) {
  if (threadIdx.x < 8) s.ctl[threadIdx.x] = ld(slot + kCtl + threadIdx.x);
  __syncthreads();
}

// Resolver of a level: over the head's histogram of nb bins (nb / 256 per
// thread), the bin b holding the need-th largest key: the keys in bins above
// b number fewer than need, with b's they reach it. Stores the bin, the
// keys still needed inside it and whether they fill it.
__device__ void resolve_level(uint32_t* slot, const uint32_t* hist, int nb, int level, uint32_t need, Lds& s) {
  const int per = nb >= kThreads ? nb / kThreads : ((int)threadIdx.x < nb ? 1 : 0);
  uint32_t h[kBinsPerThread];
  int local = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    h[j] = j < per ? ld(hist + threadIdx.x * per + j) : 0u;
    local += (int)h[j];
  }
  int total;
  const int incl = block_scan(local, s.sh, total);
  uint32_t run = (uint32_t)(total - incl);   // keys in the bins of higher threads
  for (int j = per - 1; j >= 0; --j) {
    if (run < need && need <= run + h[j]) {
      const uint32_t left = need - run;
      st(slot + kCtl + kCtlBin + (level - 1), (uint32_t)(threadIdx.x * per + j));
      st(slot + kCtl + kCtlNeed, left);
      st(slot + kCtl + kCtlWhole, left == h[j] ? 1u : 0u);
    }
    run += h[j];
  }
}

// Resolver of the last round: every chunk's output base. take(c, m) is the
// number of chunk c's m matching keys it keeps.
template <typename F>
__device__ void resolve_bases(uint32_t* slot, int nchunk, F take, Lds& s) {
  // thread t holds chunks t and t + kThreads (at most 512 chunks a head): the
  // first set precedes the second in chunk order, so each set is scanned
  // on its own and the second starts after the first's total
  uint32_t n0 = 0, n1 = 0;
  const int ca = threadIdx.x, cb = threadIdx.x + kThreads;
  if (ca < nchunk) n0 = ld(slot + kA + ca) + take(ca, ld(slot + kM + ca));
  if (cb < nchunk) n1 = ld(slot + kA + cb) + take(cb, ld(slot + kM + cb));
  int t0, t1;
  const int i0 = block_scan((int)n0, s.sh, t0);
  const int i1 = block_scan((int)n1, s.sh, t1);
  if (ca < nchunk) st(slot + kBase + ca, (uint32_t)(i0 - (int)n0));
  if (cb < nchunk) st(slot + kBase + cb, (uint32_t)(t0 + i1 - (int)n1));
  if (threadIdx.x == 0) st(slot + kCtl + kCtlFinal, 1u);
}

// Resolver of the last round when the needed keys do not fill their bin:
// after level 3 the matching keys are equal, so the lowest positions win,
// chunk by chunk in order until `need` are taken.
__device__ void resolve_split(uint32_t* slot, int nchunk, uint32_t need, Lds& s) {
  uint32_t m0 = 0, m1 = 0;
  const int ca = threadIdx.x, cb = threadIdx.x + kThreads;
  if (ca < nchunk) m0 = ld(slot + kM + ca);
  if (cb < nchunk) m1 = ld(slot + kM + cb);
  int t0, t1;
  const int i0 = block_scan((int)m0, s.sh, t0);
  const int i1 = block_scan((int)m1, s.sh, t1);
  const uint32_t before0 = (uint32_t)(i0 - (int)m0), before1 = (uint32_t)t0 + (uint32_t)(i1 - (int)m1);
  if (ca < nchunk && before0 < need && need <= before0 + m0) {
    st(slot + kCtl + kCtlCstar, (uint32_t)ca);
    st(slot + kCtl + kCtlRstar, need - before0);
  }
  if (cb < nchunk && before1 < need && need <= before1 + m1) {
    st(slot + kCtl + kCtlCstar, (uint32_t)cb);
    st(slot + kCtl + kCtlRstar, need - before1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t cs = ld(slot + kCtl + kCtlCstar), rs = ld(slot + kCtl + kCtlRstar);
  resolve_bases(slot, nchunk, [&](int c, uint32_t m) { return (uint32_t)c < cs ? m : (uint32_t)c == cs ? rs : 0u; },
                s);
}

__global__ __launch_bounds__(256) void lsel_fill(uint32_t* ws, int slots, int clear_header) {
  const int64_t n = (int64_t)slots * kClear;
  uint32_t* base = ws + kHeaderWords;
  if (clear_header && blockIdx.x == 0 && threadIdx.x < kHeaderWords) ws[threadIdx.x] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t sl = i / kClear, w = i - sl * kClear;
    base[sl * kSlotWords + w] = 0u;
  }
}

__global__ __launch_bounds__(kThreads) void lsel_rounds(SelectArgs p) {
  __shared__ Lds s;
  const int nchunk = chunks_of(p);
  const int hl = blockIdx.x / nchunk, w = blockIdx.x - hl * nchunk;
  if (hl >= p.nheads) return;
  const int h = p.head0 + hl;
  const uint32_t n_choose = (uint32_t)p.n_choose[hl];
  const int c0 = p.c0, c1 = p.c1, S = p.S;
  int32_t* dst = p.idx + p.out_off[hl];
  const int a0 = c0 & ~3;
  const int base = a0 + w * kSelectChunk;
  uint32_t* err = static_cast<uint32_t*>(p.ws);
  uint32_t* slot = err + kHeaderWords + (size_t)hl * kSlotWords;

  if (w == 0) {
    if (threadIdx.x == 0) {
      p.offsets_dev[h] = p.out_off[hl];
      if (h == p.H - 1) p.offsets_dev[p.H] = p.total;
    }
    for (int i = threadIdx.x; i < c0; i += kThreads) dst[i] = i;
    for (int i = c1 + threadIdx.x; i < S; i += kThreads) dst[c0 + (int)n_choose + (i - c1)] = i;
  }
  if (n_choose == 0) return;
  if (n_choose == (uint32_t)(c1 - c0)) {   // every candidate is kept
    for (int i = max(base, c0) + threadIdx.x; i < min(c1, base + kSelectChunk); i += kThreads) dst[i] = i;
    return;
  }

  const float* row = p.scores + (int64_t)h * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
  uint32_t match = 0;   // bit i: key i matches the decided prefix
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) match |= (k[i] != 0u ? 1u : 0u) << i;
  uint32_t above = 0;   // bit i: key i lies above the decided prefix (chosen)
  uint32_t need = n_choose;
  bool whole = false;

  int r = 0;
  bool final_ = false;
#pragma unroll 1
  for (; r < kRounds; ++r) {
    // (a) the previous round's decision narrows the matching keys
    if (r > 0) {
      const int sft = r == 1 ? 20 : r == 2 ? 8 : 0;   // the field of level r
      const uint32_t msk = r == 3 ? 0xffu : 0xfffu;
      const uint32_t b = s.ctl[kCtlBin + r - 1];
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const uint32_t f = (k[i] >> sft) & msk;
        const uint32_t bit = match & (1u << i);
        above |= f > b ? bit : 0u;
        match &= f == b ? ~0u : ~bit;
      }
      int tot;
      block_scan((__popc(above) << 16) | __popc(match), s.sh, tot);   // both counts <= 4096
      if (threadIdx.x == 0) {
        st(slot + kA + w, (uint32_t)tot >> 16);
        st(slot + kM + w, (uint32_t)tot & 0xffffu);
      }
    }
    // (b) the histogram of the next level over the matching keys
    const int lev = r + 1;
    const bool hist_round = !whole && lev <= 3;
    const int nb = lev == 3 ? kBins3 : kBins;
    uint32_t* gh = slot + (lev == 1 ? kHist1 : lev == 2 ? kHist2 : kHist3);
    if (hist_round) {
      const int sft = lev == 1 ? 20 : lev == 2 ? 8 : 0;
      const uint32_t msk = lev == 3 ? 0xffu : 0xfffu;
#pragma unroll 1
      for (int i = threadIdx.x; i < nb; i += kThreads) s.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if ((match >> i) & 1u) atomicAdd(&s.hist[(k[i] >> sft) & msk], 1u);
      __syncthreads();
#pragma unroll 1
      for (int b = threadIdx.x; b < nb; b += kThreads)
        if (s.hist[b] != 0u) add(gh + b, s.hist[b]);
    }
    // (c) arrive; the last chunk resolves the round
    if (arrive(slot, r, nchunk, s)) {
      if (hist_round) {
        resolve_level(slot, gh, nb, lev, need, s);
      } else if (whole) {
        resolve_bases(slot, nchunk, [](int, uint32_t m) { return m; }, s);
      } else {
        resolve_split(slot, nchunk, need, s);
      }
      publish(slot, r);
    } else if (!wait_round(slot, r, err, s)) {
      return;
    }
    read_ctl(slot, s);
    if (s.ctl[kCtlFinal]) {
      final_ = true;
      break;
    }
    need = s.ctl[kCtlNeed];
    whole = s.ctl[kCtlWhole] != 0u;
  }
  if (!final_) {   // every last round publishes bases; only a broken decision gets here
    if (threadIdx.x == 0) add(err, 1u);
    return;
  }

  // chosen: every key above the decided prefix, and the matching keys the
  // decision takes (all of them, or the first rstar of chunk cstar)
  uint32_t sel = above;
  if (s.ctl[kCtlWhole] != 0u || r < 3) {
    sel |= match;
  } else {
    const uint32_t cs = s.ctl[kCtlCstar], rs = s.ctl[kCtlRstar];
    if ((uint32_t)w < cs) {
      sel |= match;
    } else if ((uint32_t)w == cs) {
      int tot;
      const int incl = block_scan(__popc(match), s.sh, tot);
      int rank = incl - __popc(match);
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        if ((match >> i) & 1u) {
          if ((uint32_t)rank < rs) sel |= 1u << i;
          ++rank;
        }
      }
    }
  }
  const uint32_t out_base = ld(slot + kBase + w);
  const int n_mine = __popc(sel);
  int total;
  int o = c0 + (int)out_base + block_scan(n_mine, s.sh, total) - n_mine;
  const int out_end = c0 + (int)n_choose;
  const int first = base + kPerThread * (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    if (((sel >> i) & 1u) && o >= c0 && o < out_end) dst[o] = first + i;
    o += (int)((sel >> i) & 1u);
  }
}

// Workgroups of lsel_rounds the device holds at once (per device, computed
// once): a launch of more would not be resident together.
int resident_capacity() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap > 0) return cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lsel_rounds, kThreads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cap = (per_cu > 1 ? per_cu - 1 : per_cu) * cus;   // one workgroup a CU to spare
  cache[dev].store(cap, std::memory_order_relaxed);
  return cap;
}

}  // namespace

size_t select_long_workspace_bytes(int slots) {
  return 4 * ((size_t)kHeaderWords + (size_t)slots * kSlotWords);
}

int select_long_batch_heads(int nchunk) {
  const int cap = resident_capacity();
  if (cap <= 0 || nchunk > cap) return 0;
  const int n = cap / nchunk;
  return n < kSelectBatch ? n : kSelectBatch;
}

hipError_t launch_select_long(const SelectArgs& a, hipStream_t s, bool first_batch) {
  const int nchunk = chunks_of(a);
  const int fb = (a.nheads * kClear + 255) / 256;
  hipLaunchKernelGGL(lsel_fill, dim3((unsigned)(fb < 1024 ? fb : 1024)), dim3(256), 0, s,
                     static_cast<uint32_t*>(a.ws), a.nheads, first_batch ? 1 : 0);
  hipLaunchKernelGGL(lsel_rounds, dim3((unsigned)(a.nheads * nchunk)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

// Per-head top-k selection with forced sinks and recent window (gfx950).
//
// KVpop ("The KVpop Scoring Module", Figure 1): sinks and the protected
// window are always kept; the rest of the budget goes to the best-scored
// long-range tokens. KVP (section 3): the cache is the top of a ranking.
// Ties are broken towards the lower position, -0.0 equals +0.0 and NaN ranks
// below every number, so exactly one kept set is correct.
//
// Keys. A score maps to an order-preserving u32 key (NaN -> 1; 0 is reserved
// for "not a candidate"). A candidate's composite is (key << 32 | ~position):
// composites are distinct, and the chosen set is the n_choose largest.
//
// Three launches over (chunk, head) workgroups. A chunk is 4096 candidate
// positions of one head; thread t holds positions 16t .. 16t+15 of it in
// registers. Workgroups exchange data only across launch boundaries (a
// device-scope fence per workgroup costs more than a launch on this chip),
// and each launch issues its global loads together, so that it costs about
// one memory round trip:
//   1. hist:    per chunk, an LDS histogram of key bits 31..22 (level 1),
//               stored as descending cumulative counts (u16 per bin).
//   2. collect: every chunk sums the head's level-1 counts and finds the bin
//               b1 holding the n_choose-th composite, counts its keys above
//               and inside b1, and writes its keys inside b1 to a list
//               grouped by key bits 21..12 (level 2, descending; a counting
//               sort in LDS) with its cumulative level-2 counts beside it.
//   3. scatter: every chunk sums the level-2 counts (bin b2), gathers the few
//               (b1, b2) entries of all chunks, picks the exact threshold
//               composite among them, derives every chunk's chosen count and
//               hence its own output base, and writes its chosen positions
//               in ascending order. The resolution is repeated per chunk on
//               L2-resident data instead of costing another launch. Chunk 0
//               also writes the sinks, the window and the offsets.
// A bin that is taken whole needs no further level.
// Output per head: sinks, then the chosen candidates, then the window.
// When the scores are masses whose split parts the mass pass has just
// written, launch 1 is sel_hist_reduce instead: it adds the parts (the mass
// pass's own reduction) and builds the histograms from the sums in registers.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kSelectChunk / kThreads;  // 16 consecutive positions
constexpr int kBins = 1024;                          // per histogram level (10 key bits)
constexpr int kBinsPerThread = kBins / kThreads;     // 4 bins = one 8-byte u16 group
constexpr int kRadixBins = 2048;                     // exact pick: 11 bits per pass
constexpr int kMaxChunks = (kSelectMaxCandidates + 3) / kSelectChunk + 1;
constexpr int kLdsList = 1024;  // (b1, b2) entries held in LDS (more are read from the lists in L2);
                                 // 8 KB keeps the scatter launch at four workgroups per CU
constexpr int kRankMax = 128;   // up to this many, rank them by direct comparison


__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - pos);
}
__device__ __forceinline__ uint32_t comp_pos(uint64_t v) { return 0xffffffffu - (uint32_t)v; }
__device__ __forceinline__ uint32_t key_top(uint32_t k) { return k >> 22; }
__device__ __forceinline__ uint32_t key_mid(uint32_t k) { return (k >> 12) & 1023u; }

// Workspace of one launch: per head slot, per chunk.
struct Ws {
  uint64_t* list;   // [slots][nchunk][kSelectChunk] composites inside b1, mid bits descending
  uint16_t* cum1;   // [slots][nchunk][kBins] # keys with top bits >= bin
  uint16_t* cum2;   // [slots][nchunk][kBins] # keys inside b1 with mid bits >= bin
  int* cnt;         // [slots][nchunk][2]: # keys above b1, # inside b1
  int* st;          // [slots][4]: b1, keys still needed from b1, whole-bin flag
};

__host__ __device__ inline size_t ws_bytes(int slots, int nchunk) {
  const size_t nh = slots, nc = nchunk;
  return nh * nc * kSelectChunk * sizeof(uint64_t) + 2 * nh * nc * kBins * sizeof(uint16_t) +
         nh * nc * 2 * sizeof(int) + nh * 4 * sizeof(int);
}

__device__ __forceinline__ Ws ws_of(const SelectArgs& p) {
  Ws w;
  const size_t nh = p.slots, nc = p.nchunk;
  char* base = static_cast<char*>(p.ws);
  w.list = reinterpret_cast<uint64_t*>(base);
  base += nh * nc * kSelectChunk * sizeof(uint64_t);
  w.cum1 = reinterpret_cast<uint16_t*>(base);
  base += nh * nc * kBins * sizeof(uint16_t);
  w.cum2 = reinterpret_cast<uint16_t*>(base);
  base += nh * nc * kBins * sizeof(uint16_t);
  w.cnt = reinterpret_cast<int*>(base);
  base += nh * nc * 2 * sizeof(int);
  w.st = reinterpret_cast<int*>(base);
  return w;
}

__device__ __forceinline__ int chunks_of(const SelectArgs& p) {
  const int a0 = p.c0 & ~3;
  return max(1, (p.c1 - a0 + kSelectChunk - 1) / kSelectChunk);
}

// Workgroup -> (chunk w, head slot hl). Consecutive workgroup ids go to
// consecutive XCDs (round robin over kXcds), so all chunks of a head are
// placed on one XCD: the head's scores, histograms and lists then stay in
// that XCD's L2 across the three launches. Returns false for the padding
// workgroups of a last, partial group of heads.
constexpr int kXcds = 8;
__device__ __forceinline__ bool wg_coords(const SelectArgs& p, int& w, int& hl) {
  const int id = blockIdx.x, x = id % kXcds, j = id / kXcds;
  const int grp = j / p.nchunk;
  w = j - grp * p.nchunk;
  hl = x + kXcds * grp;
  return hl < p.nheads;
}

// No candidate or every candidate is chosen: only the scatter launch works.
__device__ __forceinline__ bool trivial_head(const SelectArgs& p, int n_choose) {
  return n_choose == 0 || n_choose == p.c1 - p.c0;
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
  if (aligned && (p.S & 3) == 0) {
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
  // edge chunks of other rows: every load reads a clamped in-range position, then masks
  float f[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) f[i] = row[min(max(first + i, p.c0), p.c1 - 1)];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    k[i] = (first + i >= p.c0 && first + i < p.c1) ? order_key(f[i]) : 0u;
}

// Inclusive prefix sum over the NT threads of the workgroup; `total`
// receives the sum. `sh` holds NT / 64 ints.
template <int NT = kThreads>
__device__ int block_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan(v);
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = sh[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

// Wave 0 computes out[c] = sum_{c' < c} val(c') for c < n <= 64 and out[n] =
// the total, all loads issued at once. The caller synchronises afterwards.
template <typename F>
__device__ __forceinline__ void wave0_exclusive_scan(int n, F val, int* out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int x = lane < n ? val(lane) : 0;
    const int v = wave_scan(x);
    if (lane < n) out[lane] = v - x;
    if (lane == 63) out[n] = v;
  }
}

// This thread's kBins / NT bins of an LDS histogram as descending inclusive
// cumulative counts: cum[j] = # elements in bins >= (kBins / NT) * tid + j.
template <int NT = kThreads>
__device__ __forceinline__ void descending_cum(const uint32_t* hist, int* sh,
                                               uint32_t (&cum)[kBins / NT]) {
  constexpr int kB = kBins / NT;
  uint32_t h[kB];
  int local = 0;
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    h[j] = hist[kB * threadIdx.x + j];
    local += (int)h[j];
  }
  int total;
  const int incl = block_scan<NT>(local, sh, total);
  uint32_t run = (uint32_t)(total - incl);
#pragma unroll
  for (int j = kB - 1; j >= 0; --j) {
    run += h[j];
    cum[j] = run;
  }
}

// This thread's 4 counts (each <= kSelectChunk) as packed u16 at dst.
__device__ __forceinline__ void store_u16x4(uint16_t* dst, const uint32_t (&v)[kBinsPerThread]) {
  u32x2_t r;
#pragma unroll
  for (int q = 0; q < 2; ++q) r[q] = (v[2 * q] & 0xffffu) | (v[2 * q + 1] << 16);
  *reinterpret_cast<u32x2_t*>(dst + kBinsPerThread * threadIdx.x) = r;
}

__device__ __forceinline__ uint32_t u16_at(u32x2_t v, int j) {
  const uint32_t word = j < 2 ? v[0] : v[1];
  return (j & 1) ? word >> 16 : word & 0xffffu;
}

// Every chunk's packed u16 counts of this thread's 4 bins, all loads in flight.
__device__ __forceinline__ void load_cums(const uint16_t* src, int nchunk_h,
                                          u32x2_t (&v)[kMaxChunks]) {
  src += kBinsPerThread * threadIdx.x;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    v[c] = c < nchunk_h ? *reinterpret_cast<const u32x2_t*>(src + (size_t)c * kBins)
                        : u32x2_t{0u, 0u};
}

__device__ __forceinline__ void sum_cums(const u32x2_t (&v)[kMaxChunks],
                                         uint32_t (&acc)[kBinsPerThread]) {
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) acc[j] = 0u;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      acc[2 * q] += v[c][q] & 0xffffu;
      acc[2 * q + 1] += v[c][q] >> 16;
    }
}

// Given the head's descending cumulative counts of this thread's bins (staged
// through `cum`, kBins + 1 entries of LDS), find the bin b with
// cum[b] >= need > cum[b + 1]: out3 = {b, cum[b + 1], cum[b] - cum[b + 1]}.
__device__ void find_cum_bin(const uint32_t (&acc)[kBinsPerThread], uint32_t* cum, int need,
                             int* out3) {
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) cum[kBinsPerThread * threadIdx.x + j] = acc[j];
  if (threadIdx.x == 0) cum[kBins] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    const int b = kBinsPerThread * threadIdx.x + j;
    const uint32_t hi = cum[b], lo = cum[b + 1];
    if (hi >= (uint32_t)need && lo < (uint32_t)need) {
      out3[0] = b;
      out3[1] = (int)lo;
      out3[2] = (int)(hi - lo);
    }
  }
  __syncthreads();
}

// Over an LDS histogram of nb bins (nb a multiple of 256), find the bin that
// holds the need-th largest element: out3 = {bin, count above it, count in it}.
__device__ void find_bin(const uint32_t* hist, int nb, int need, int* sh, int* out3) {
  const int bpt = nb / kThreads;
  int local = 0;
  for (int j = 0; j < bpt; ++j) local += (int)hist[threadIdx.x * bpt + j];
  int total;
  const int incl = block_scan(local, sh, total);
  int above = total - incl;
  for (int j = bpt - 1; j >= 0; --j) {
    const int bin = threadIdx.x * bpt + j;
    const int c = (int)hist[bin];
    if (above < need && need <= above + c) {
      out3[0] = bin;
      out3[1] = above;
      out3[2] = c;
    }
    above += c;
  }
  __syncthreads();
}

// The need-th largest of n distinct composites whose top 20 bits are equal;
// fetch(g) returns entry g (from LDS or from the global lists). Small sets
// rank every entry by direct comparison and return the entry itself; larger
// ones run a radix select over the low 44 bits (4 x 11) and return those
// bits.
template <typename F>
__device__ uint64_t pick_threshold(int n, int need, F fetch, uint32_t* hist, int* sh, int* res,
                                   uint64_t* sh_thr) {
  if (n <= kRankMax) {
    for (int g = threadIdx.x; g < n; g += kThreads) {
      const uint64_t x = fetch(g);
      int r = 0;
      for (int j = 0; j < n; ++j) r += fetch(j) > x ? 1 : 0;
      if (r == need - 1) *sh_thr = x;
    }
    __syncthreads();
    return *sh_thr;
  }
  uint64_t prefix = 0, pmask = 0;
  int rem = need;
  const uint64_t lowmask = (1ull << 44) - 1;
  for (int lev = 0; lev < 4; ++lev) {
    const int sft = 33 - 11 * lev;
    constexpr int nb = kRadixBins;
    for (int i = threadIdx.x; i < nb; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int g0 = threadIdx.x; g0 < n; g0 += kThreads * 8) {
      uint64_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int g = g0 + j * kThreads;
        v[j] = g < n ? fetch(g) : 0ull;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t x = v[j] & lowmask;
        if (g0 + j * kThreads < n && (x & pmask) == prefix)
          atomicAdd(&hist[(x >> sft) & (uint64_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    find_bin(hist, nb, rem, sh, res);
    rem -= res[1];
    prefix |= (uint64_t)res[0] << sft;
    pmask |= (uint64_t)(nb - 1) << sft;
    __syncthreads();
  }
  return prefix;
}

// ---------------------------------------------------------------- launch 1
__device__ __forceinline__ void hist_phase(const SelectArgs& p) {
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[8];
  int w, hl;
  if (!wg_coords(p, w, hl)) return;
  if (trivial_head(p, p.n_choose[hl])) return;
  const int base = (p.c0 & ~3) + w * kSelectChunk;
  const float* row = p.scores + (int64_t)(p.head0 + hl) * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (k[i] != 0u) atomicAdd(&hist[key_top(k[i])], 1u);
  __syncthreads();
  uint32_t cum[kBinsPerThread];
  descending_cum(hist, sh, cum);
  store_u16x4(ws_of(p).cum1 + ((size_t)hl * p.nchunk + w) * kBins, cum);
}

// ---------------------------------------------------------------- launch 2
__device__ __forceinline__ void collect_phase(const SelectArgs& p) {
  __shared__ uint32_t hist[kBins];     // level-2 histogram, then bucket cursors
  __shared__ uint32_t cum[kBins + 1];  // the head's level-1 cumulative counts
  __shared__ int sh[8];
  __shared__ int res[3];

  int w, hl;
  if (!wg_coords(p, w, hl)) return;
  const int n_choose = p.n_choose[hl];
  if (trivial_head(p, n_choose)) return;
  const int base = (p.c0 & ~3) + w * kSelectChunk;
  const int nchunk_h = chunks_of(p);
  const Ws ws = ws_of(p);
  const float* row = p.scores + (int64_t)(p.head0 + hl) * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);

  // level 1: the head's bin b1
  {
    u32x2_t v[kMaxChunks];
    load_cums(ws.cum1 + (size_t)hl * p.nchunk * kBins, nchunk_h, v);
    uint32_t acc[kBinsPerThread];
    sum_cums(v, acc);
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
    find_cum_bin(acc, cum, n_choose, res);
  }
  const uint32_t b1 = (uint32_t)res[0];
  const int need1 = n_choose - res[1];
  const bool whole1 = need1 == res[2];
  if (w == 0 && threadIdx.x == 0) {
    int* st = ws.st + hl * 4;
    st[0] = (int)b1;
    st[1] = need1;
    st[2] = whole1 ? 1 : 0;
  }

  // this chunk: keys above b1, keys inside b1 and their level-2 histogram
  int packed = 0;  // (# above) << 16 | # inside, each <= 4096
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const bool valid = k[i] != 0u;
    packed += (valid && key_top(k[i]) > b1) ? (1 << 16) : 0;
    const bool in = valid && key_top(k[i]) == b1;
    packed += in ? 1 : 0;
    if (!whole1 && in) atomicAdd(&hist[key_mid(k[i])], 1u);
  }
  int total;
  block_scan(packed, sh, total);  // (its barriers also order the LDS atomics)
  if (!whole1) {
    // cumulative level-2 counts; bucket b starts after the keys with mid > b
    uint32_t c2[kBinsPerThread];
    descending_cum(hist, sh, c2);
    store_u16x4(ws.cum2 + ((size_t)hl * p.nchunk + w) * kBins, c2);
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) {
      const int b = kBinsPerThread * threadIdx.x + j;
      hist[b] = c2[j] - hist[b];
    }
    __syncthreads();
    uint64_t* list = ws.list + ((size_t)hl * p.nchunk + w) * kSelectChunk;
    const uint32_t first = (uint32_t)(base + kPerThread * (int)threadIdx.x);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      if (k[i] != 0u && key_top(k[i]) == b1) {
        const uint32_t slot = atomicAdd(&hist[key_mid(k[i])], 1u);
        list[slot] = composite(k[i], first + i);
      }
    }
  }
  if (threadIdx.x == 0) {
    int* c = ws.cnt + ((size_t)hl * p.nchunk + w) * 2;
    c[0] = total >> 16;
    c[1] = total & 0xffff;
  }
}

// ---------------------------------------------------------------- launch 3
__device__ __forceinline__ void scatter_phase(const SelectArgs& p) {
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t cum[kBins + 1];
  __shared__ uint64_t lst[kLdsList];
  __shared__ int sh[8];
  __shared__ int res[3];
  __shared__ uint64_t sh_thr;
  __shared__ int a1[kMaxChunks], i1[kMaxChunks], a2[kMaxChunks], hi2[kMaxChunks];
  __shared__ int goff[kMaxChunks + 1], choff[kMaxChunks + 1];
  __shared__ uint32_t chosen[kMaxChunks];

  int w, hl;
  if (!wg_coords(p, w, hl)) return;
  const int h = p.head0 + hl;
  const int n_choose = p.n_choose[hl];
  const int c0 = p.c0, c1 = p.c1, S = p.S;
  int32_t* dst = p.idx + p.out_off[hl];
  const int a0 = c0 & ~3;
  const int base = a0 + w * kSelectChunk;

  if (w == 0) {
    if (threadIdx.x == 0) {
      p.offsets_dev[h] = p.out_off[hl];
      if (h == p.H - 1) p.offsets_dev[p.H] = p.total;
    }
    for (int i = threadIdx.x; i < c0; i += kThreads) dst[i] = i;
    for (int i = c1 + threadIdx.x; i < S; i += kThreads) dst[c0 + n_choose + (i - c1)] = i;
  }
  if (n_choose == 0) return;
  if (n_choose == c1 - c0) {  // every candidate is kept
    for (int i = max(base, c0) + threadIdx.x; i < min(c1, base + kSelectChunk); i += kThreads)
      dst[i] = i;
    return;
  }
  const int nchunk_h = chunks_of(p);
  const Ws ws = ws_of(p);
  const float* row = p.scores + (int64_t)h * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
  // level-2 counts are loaded with everything else; unused if b1 is whole
  const uint16_t* cum2 = ws.cum2 + (size_t)hl * p.nchunk * kBins;
  u32x2_t v[kMaxChunks];
  load_cums(cum2, nchunk_h, v);
  const int* cnt = ws.cnt + (size_t)hl * p.nchunk * 2;
  for (int c = threadIdx.x; c < nchunk_h; c += kThreads) {
    a1[c] = cnt[2 * c];
    i1[c] = cnt[2 * c + 1];
  }
  const int* st = ws.st + hl * 4;
  const uint32_t b1 = (uint32_t)st[0];
  const int need1 = st[1];
  const bool whole1 = st[2] != 0;
  __syncthreads();

  bool whole2 = true;
  uint32_t b2 = 0;
  uint64_t thr = 0;  // inside (b1, b2), chosen iff composite >= thr
  if (whole1) {
    for (int c = threadIdx.x; c < nchunk_h; c += kThreads) chosen[c] = a1[c] + i1[c];
  } else {
    {
      uint32_t acc[kBinsPerThread];
      sum_cums(v, acc);
      find_cum_bin(acc, cum, need1, res);
    }
    b2 = (uint32_t)res[0];
    const int need2 = need1 - res[1];
    const int in_b2 = res[2];
    whole2 = need2 == in_b2;
    // per chunk: # inside b1 with mid >= b2 (hi2) and > b2 (a2), taken from
    // the registers of the threads that own bins b2 and b2 + 1
    if ((int)threadIdx.x == (int)(b2 / kBinsPerThread)) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nchunk_h) hi2[c] = (int)u16_at(v[c], (int)(b2 % kBinsPerThread));
    }
    if (b2 + 1 < (uint32_t)kBins) {
      if ((int)threadIdx.x == (int)((b2 + 1) / kBinsPerThread)) {
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
          if (c < nchunk_h) a2[c] = (int)u16_at(v[c], (int)((b2 + 1) % kBinsPerThread));
      }
    } else {
      for (int c = threadIdx.x; c < nchunk_h; c += kThreads) a2[c] = 0;
    }
    __syncthreads();
    if (whole2) {
      for (int c = threadIdx.x; c < nchunk_h; c += kThreads) chosen[c] = a1[c] + hi2[c];
    } else {
      wave0_exclusive_scan(nchunk_h, [&](int c) { return hi2[c] - a2[c]; }, goff);
      __syncthreads();
      const uint64_t* lists = ws.list + (size_t)hl * p.nchunk * kSelectChunk;
      // entry g of the concatenated (b1, b2) runs of the chunk lists
      auto global_entry = [&](int g) {
        int lo = 0, hi = nchunk_h - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (goff[mid] <= g) lo = mid;
          else hi = mid - 1;
        }
        return lists[(size_t)lo * kSelectChunk + a2[lo] + (g - goff[lo])];
      };
      const bool in_lds = in_b2 <= kLdsList;
      if (in_lds) {
        for (int g = threadIdx.x; g < in_b2; g += kThreads) lst[g] = global_entry(g);
        __syncthreads();
      }
      auto fetch = [&](int g) { return in_lds ? lst[g] : global_entry(g); };
      const uint64_t t = pick_threshold(in_b2, need2, fetch, hist, sh, res, &sh_thr);
      thr = in_b2 <= kRankMax ? t : (((uint64_t)b1 << 54) | ((uint64_t)b2 << 44) | t);
      for (int c = threadIdx.x; c < nchunk_h; c += kThreads) chosen[c] = a1[c] + a2[c];
      __syncthreads();
      for (int g = threadIdx.x; g < in_b2; g += kThreads) {
        const uint64_t e = fetch(g);
        if (e >= thr) atomicAdd(&chosen[(comp_pos(e) - (uint32_t)a0) / kSelectChunk], 1u);
      }
    }
  }
  __syncthreads();
  wave0_exclusive_scan(nchunk_h, [&](int c) { return (int)chosen[c]; }, choff);
  __syncthreads();

  // ordered write of this chunk's chosen positions
  const int out_end = c0 + n_choose;
  const uint32_t first = (uint32_t)(base + kPerThread * (int)threadIdx.x);
  uint32_t sel = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t key = k[i];
    bool s = key != 0u && key_top(key) > b1;
    if (key != 0u && key_top(key) == b1) {
      const uint32_t d2 = key_mid(key);
      if (whole1 || d2 > b2) s = true;
      else if (d2 == b2) s = whole2 || composite(key, first + i) >= thr;
    }
    sel |= (s ? 1u : 0u) << i;
  }
  const int n_mine = __popc(sel);
  int total;
  int o = c0 + choff[w] + block_scan(n_mine, sh, total) - n_mine;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    if (((sel >> i) & 1u) && o < out_end) dst[o] = (int32_t)(first + i);
    o += (int)((sel >> i) & 1u);
  }
}

// ---------------------------------------------------------------- launch 1, fed by the mass pass
// When the scores are the key masses whose partial sums the mass pass left
// in `part` ([nsplit][H * S], the slices of a [H, S] output), this launch
// replaces the mass pass's reduction and the first select launch: each chunk
// adds its positions' slices in split order (the order, and so the bits, of
// the plain reduction), writes the masses, and builds its level-1 histogram
// from the sums still in registers. Workgroups past the select grid reduce
// the positions no chunk covers (before the first chunk, after the last).
constexpr int kReduceBatch = 8;     // slices in flight per thread
constexpr int kReduceThreads = 256; // threads per chunk (16 positions each)

__device__ __forceinline__ float reduce_one(const float* part, int64_t n, int nsplit, int64_t e) {
  float acc = 0.f;
  for (int k0 = 0; k0 < nsplit; k0 += kReduceBatch) {
    float v[kReduceBatch];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) v[j] = part[(int64_t)min(k0 + j, nsplit - 1) * n + e];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j)
      if (k0 + j < nsplit) acc = k0 + j == 0 ? v[j] : acc + v[j];
  }
  return acc;
}

template <int NT>
__global__ __launch_bounds__(NT) void sel_hist_reduce(SelectArgs p, const float* part, float* mass,
                                                      int nsplit, int ngrid) {
  constexpr int PT = kSelectChunk / NT;   // consecutive positions per thread
  constexpr int BPT = kBins / NT;         // histogram bins per thread
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[NT / 64];
  const int S = p.S;
  const int64_t n = (int64_t)p.H * S;
  const int a0 = p.c0 & ~3;
  if ((int)blockIdx.x >= ngrid) {
    const int64_t after = (int64_t)a0 + (int64_t)p.nchunk * kSelectChunk;
    const int64_t per_head = a0 + (S > after ? S - after : 0);
    const int64_t nout = (int64_t)p.H * per_head;
    const int64_t stride = (int64_t)(gridDim.x - ngrid) * NT;
    for (int64_t e = (int64_t)(blockIdx.x - ngrid) * NT + threadIdx.x; e < nout; e += stride) {
      const int64_t h = e / per_head, j = e - h * per_head;
      const int64_t at = h * S + (j < a0 ? j : after + (j - a0));
      mass[at] = reduce_one(part, n, nsplit, at);
    }
    return;
  }
  int w, hl;
  if (!wg_coords(p, w, hl)) return;
  const int base = a0 + w * kSelectChunk;
  const int64_t row = (int64_t)hl * S;
  // piece q of this thread holds positions piece(q) .. piece(q) + 3; the
  // pieces of a wave's 16-byte load lie side by side (1 KB in a row), which
  // the histogram allows (it does not care which thread holds a position)
  auto piece = [&](int q) { return base + 4 * (int)threadIdx.x + 4 * NT * q; };
  auto pos = [&](int i) { return piece(i >> 2) + (i & 3); };
  float acc[PT];
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(part) | reinterpret_cast<uintptr_t>(mass)) & 15u) == 0 &&
                      (S & 3) == 0;
  if (vec_ok) {
    // rows of a multiple of 4: a piece lies wholly inside the row or wholly
    // past its end; pieces past it load the row's last piece (in bounds) and
    // are neither stored nor counted
    for (int k0 = 0; k0 < nsplit; k0 += kReduceBatch) {
      f32x4_t v[kReduceBatch][PT / 4];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        const float* src = part + (int64_t)min(k0 + j, nsplit - 1) * n + row;
#pragma unroll
        for (int q = 0; q < PT / 4; ++q) v[j][q] = *reinterpret_cast<const f32x4_t*>(src + min(piece(q), S - 4));
      }
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j)
        if (k0 + j < nsplit) {
#pragma unroll
          for (int q = 0; q < PT / 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              acc[4 * q + c] = k0 + j == 0 ? v[j][q][c] : acc[4 * q + c] + v[j][q][c];
        }
    }
#pragma unroll
    for (int q = 0; q < PT / 4; ++q)
      if (piece(q) < S)
        *reinterpret_cast<f32x4_t*>(mass + row + piece(q)) =
            f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  } else {
    // unaligned rows: positions clamped into the row, stores masked
#pragma unroll
    for (int i = 0; i < PT; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < nsplit; k0 += kReduceBatch) {
      float v[kReduceBatch][PT];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        const float* src = part + (int64_t)min(k0 + j, nsplit - 1) * n + row;
#pragma unroll
        for (int i = 0; i < PT; ++i) v[j][i] = src[min(pos(i), S - 1)];
      }
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j)
        if (k0 + j < nsplit) {
#pragma unroll
          for (int i = 0; i < PT; ++i) acc[i] = k0 + j == 0 ? v[j][i] : acc[i] + v[j][i];
        }
    }
#pragma unroll
    for (int i = 0; i < PT; ++i)
      if (pos(i) < S) mass[row + pos(i)] = acc[i];
  }
  if (trivial_head(p, p.n_choose[hl])) return;
  for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (pos(i) >= p.c0 && pos(i) < p.c1) atomicAdd(&hist[key_top(order_key(acc[i]))], 1u);
  __syncthreads();
  uint32_t cum[BPT];
  descending_cum<NT>(hist, sh, cum);
  // this thread's BPT counts (each <= kSelectChunk) as packed u16
  uint16_t* dst = ws_of(p).cum1 + ((size_t)hl * p.nchunk + w) * kBins + BPT * threadIdx.x;
  uint32_t r[BPT / 2];
#pragma unroll
  for (int q = 0; q < BPT / 2; ++q) r[q] = (cum[2 * q] & 0xffffu) | (cum[2 * q + 1] << 16);
  if constexpr (BPT == 4) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{r[0], r[1]};
  else *reinterpret_cast<uint32_t*>(dst) = r[0];
}

__global__ __launch_bounds__(kThreads) void sel_hist(SelectArgs p) { hist_phase(p); }
__global__ __launch_bounds__(kThreads) void sel_collect(SelectArgs p) { collect_phase(p); }
__global__ __launch_bounds__(kThreads) void sel_scatter(SelectArgs p) { scatter_phase(p); }

// One chunk a head: every phase reads only what its own workgroup wrote in
// the phase before, so the three run in one launch, separated by barriers
// (which also make the workgroup's global writes visible to all its threads).
__global__ __launch_bounds__(kThreads) void sel_one(SelectArgs p) {
  hist_phase(p);
  __syncthreads();
  collect_phase(p);
  __syncthreads();
  scatter_phase(p);
}

}  // namespace

size_t select_workspace_bytes(int slots, int nchunk) { return ws_bytes(slots, nchunk); }

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int groups = (a.nheads + kXcds - 1) / kXcds;
  const dim3 grid(kXcds * a.nchunk * groups);
  // heads that keep all their candidates or none need no threshold: when
  // every head is such, the last launch alone writes the lists
  bool all_trivial = true;
  for (int i = 0; i < a.nheads; ++i)
    if (a.n_choose[i] != 0 && a.n_choose[i] != a.c1 - a.c0) all_trivial = false;
  if (all_trivial) {
    hipLaunchKernelGGL(sel_scatter, grid, dim3(kThreads), 0, s, a);
  } else if (a.nchunk == 1) {   // every head one chunk: one launch
    hipLaunchKernelGGL(sel_one, grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(sel_hist, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(sel_collect, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(sel_scatter, grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_select_hist(const SelectArgs& a, hipStream_t s) {
  const int groups = (a.nheads + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(sel_hist, dim3(kXcds * a.nchunk * groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_hist_reduce(const SelectArgs& a, const float* part, int nsplit, hipStream_t s) {
  const int groups = (a.nheads + kXcds - 1) / kXcds;
  const int ngrid = kXcds * a.nchunk * groups;
  const int a0 = a.c0 & ~3;
  const int64_t after = (int64_t)a0 + (int64_t)a.nchunk * kSelectChunk;
  const int64_t nout = (int64_t)a.H * (a0 + (a.S > after ? a.S - after : 0));
  const int64_t blocks = (nout + kReduceThreads - 1) / kReduceThreads;
  const int64_t extra = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(sel_hist_reduce<kReduceThreads>, dim3((unsigned)(ngrid + extra)), dim3(kReduceThreads), 0, s,
                     a, part, const_cast<float*>(a.scores), nsplit, ngrid);
  return hipGetLastError();
}

hipError_t launch_select_prepared(const SelectArgs& a, hipStream_t s) {
  const int groups = (a.nheads + kXcds - 1) / kXcds;
  const dim3 grid(kXcds * a.nchunk * groups);
  bool all_trivial = true;
  for (int i = 0; i < a.nheads; ++i)
    if (a.n_choose[i] != 0 && a.n_choose[i] != a.c1 - a.c0) all_trivial = false;
  if (!all_trivial) hipLaunchKernelGGL(sel_collect, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(sel_scatter, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_from_parts(const SelectArgs& a, const float* part, int nsplit,
                                    hipStream_t s) {
  const hipError_t e = launch_select_hist_reduce(a, part, nsplit, s);
  return e != hipSuccess ? e : launch_select_prepared(a, s);
}

}  // namespace fam

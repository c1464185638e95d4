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
// Three launches over (chunk, head) workgroups; a chunk is 4096 candidate
// positions of one head, 16 per thread in registers:
//   1. hist:    per chunk, an LDS histogram of key bits 31..21 (level 1).
//   2. collect: every chunk sums the head's level-1 histograms and finds the
//               bin b1 holding the n_choose-th composite; it counts its keys
//               above b1, lists the composites of its keys inside b1, and
//               builds their histogram of key bits 20..10 (level 2).
//   3. finish:  every chunk sums the level-2 histograms (bin b2), walks the
//               head's b1 lists once to count, per chunk, the entries above
//               (b1, b2) and to gather those equal to it into LDS, runs an
//               exact radix select over the gathered composites, derives
//               every chunk's chosen count and hence its output base, and
//               writes its chosen positions in ascending order. Chunk 0 also
//               writes the sinks, the window and the offsets.
// A whole bin that is taken needs no further level. If the (b1, b2) entries
// do not fit in LDS, the exact select streams the b1 lists instead.
// Output per head: sinks, then the chosen candidates, then the window.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kSelectChunk / kThreads;  // 16
constexpr int kIters = kPerThread / 4;               // float4 loads per thread
constexpr int kBins = 2048;
constexpr int kMaxChunks = (kSelectMaxCandidates + 3) / kSelectChunk + 1;
constexpr int kLdsList = 8192;                       // (b1, b2) entries held in LDS

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - pos);
}
__device__ __forceinline__ uint32_t comp_pos(uint64_t v) { return 0xffffffffu - (uint32_t)v; }
__device__ __forceinline__ uint32_t comp_d2(uint64_t v) { return (uint32_t)(v >> 42) & 2047u; }

// Workspace of one launch: per head slot, per chunk.
struct Ws {
  uint64_t* list;   // [slots][nchunk][kSelectChunk] composites of the keys inside bin b1
  uint16_t* hist1;  // [slots][nchunk][kBins]
  uint16_t* hist2;  // [slots][nchunk][kBins]
  int* cnt;         // [slots][nchunk][2]: (# inside b1, # above b1)
  int* state;       // [slots][4]: b1, need (inside b1), # inside b1, whole-bin flag
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
  w.hist1 = reinterpret_cast<uint16_t*>(base);
  base += nh * nc * kBins * sizeof(uint16_t);
  w.hist2 = reinterpret_cast<uint16_t*>(base);
  base += nh * nc * kBins * sizeof(uint16_t);
  w.cnt = reinterpret_cast<int*>(base);
  base += nh * nc * 2 * sizeof(int);
  w.state = reinterpret_cast<int*>(base);
  return w;
}

// Keys of this thread's 16 positions: pos(i) = base + (i/4)*1024 + 4*tid + i%4.
// Interior chunks issue their four 16-byte loads back to back.
__device__ __forceinline__ void load_chunk(const SelectArgs& p, const float* row, int base,
                                           uint32_t (&k)[kPerThread]) {
  const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (vec_ok && base >= p.c0 && base + kSelectChunk <= p.c1) {
    f32x4_t f[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it)
      f[it] = *reinterpret_cast<const f32x4_t*>(row + base + it * (4 * kThreads) + 4 * threadIdx.x);
#pragma unroll
    for (int it = 0; it < kIters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) k[4 * it + c] = order_key(f[it][c]);
    return;
  }
  // edge chunk: every load reads a clamped in-range position, then masks
  float f[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int q = base + (i / 4) * (4 * kThreads) + 4 * (int)threadIdx.x + (i % 4);
    f[i] = row[min(max(q, p.c0), p.c1 - 1)];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int q = base + (i / 4) * (4 * kThreads) + 4 * (int)threadIdx.x + (i % 4);
    k[i] = (q >= p.c0 && q < p.c1) ? order_key(f[i]) : 0u;
  }
}

// LDS counter increment with the lanes that share the first active lane's
// slot combined into one atomic (scores cluster, so a few slots take most
// of the increments and same-address atomics would serialise).
__device__ __forceinline__ void agg_inc(uint32_t* cnt, uint32_t slot, bool valid) {
  const uint64_t vmask = __ballot(valid);
  if (vmask == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)vmask) - 1;
  const uint32_t ls = __shfl(slot, leader);
  const bool same = valid && slot == ls;
  const uint64_t smask = __ballot(same);
  if (same) {
    if (lane == leader) atomicAdd(&cnt[ls], (uint32_t)__popcll(smask));
  } else if (valid) {
    atomicAdd(&cnt[slot], 1u);
  }
}

__device__ __forceinline__ int chunk_pos(int base, int i) {
  return base + (i / 4) * (4 * kThreads) + 4 * (int)threadIdx.x + (i % 4);
}

// Inclusive prefix sum over the 256 threads; `total` receives the sum.
__device__ int block_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
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

// Wave 0 computes out[c] = sum_{c' < c} val(c') for c < n <= 64 and out[n] =
// the total (all loads issued at once). The caller synchronises afterwards.
template <typename F>
__device__ __forceinline__ void wave0_exclusive_scan(int n, F val, int* out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int v = lane < n ? val(lane) : 0;
    const int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d);
      if (lane >= d) v += t;
    }
    if (lane < n) out[lane] = v - x;
    if (lane == 63) out[n] = v;
  }
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

// Sum of the head's per-chunk u16 histograms into LDS (8 loads in flight).
__device__ void sum_hists(const uint16_t* src, int nchunk_h, uint32_t* hist) {
  constexpr int BPT = kBins / kThreads;  // 8 bins = one 16-byte load per chunk
  uint32_t acc[BPT] = {};
  src += threadIdx.x * BPT;
  for (int w0 = 0; w0 < nchunk_h; w0 += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = w0 + j < nchunk_h ? *reinterpret_cast<const u32x4_t*>(src + (size_t)(w0 + j) * kBins)
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += v[j][q] & 0xffffu;
        acc[2 * q + 1] += v[j][q] >> 16;
      }
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) hist[threadIdx.x * BPT + j] = acc[j];
  __syncthreads();
}

__device__ __forceinline__ void store_hist(const uint32_t* hist, uint16_t* dst) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) dst[i] = (uint16_t)hist[i];
}

__device__ __forceinline__ int chunks_of(const SelectArgs& p) {
  const int a0 = p.c0 & ~3;
  return max(1, (p.c1 - a0 + kSelectChunk - 1) / kSelectChunk);
}

// ---------------------------------------------------------------- launch 1
__global__ __launch_bounds__(kThreads) void sel_hist(SelectArgs p) {
  __shared__ uint32_t hist[kBins];
  const int hl = blockIdx.y, w = blockIdx.x;
  const int n_choose = p.n_choose[hl];
  if (n_choose == 0 || n_choose == p.c1 - p.c0) return;
  const int base = (p.c0 & ~3) + w * kSelectChunk;
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
  __syncthreads();
  const float* row = p.scores + (int64_t)(p.head0 + hl) * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) agg_inc(hist, k[i] >> 21, k[i] != 0u);
  __syncthreads();
  const Ws ws = ws_of(p);
  store_hist(hist, ws.hist1 + ((size_t)hl * p.nchunk + w) * kBins);
}

// ---------------------------------------------------------------- launch 2
__global__ __launch_bounds__(kThreads) void sel_collect(SelectArgs p) {
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[8];
  __shared__ int res[3];
  __shared__ int n_list;
  const int hl = blockIdx.y, w = blockIdx.x;
  const int n_choose = p.n_choose[hl];
  if (n_choose == 0 || n_choose == p.c1 - p.c0) return;
  const int base = (p.c0 & ~3) + w * kSelectChunk;
  const int nchunk_h = chunks_of(p);
  const Ws ws = ws_of(p);
  sum_hists(ws.hist1 + (size_t)hl * p.nchunk * kBins, nchunk_h, hist);
  find_bin(hist, kBins, n_choose, sh, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int need = n_choose - res[1];
  const int in_b1 = res[2];
  const bool whole = need == in_b1;
  if (w == 0 && threadIdx.x == 0) {
    int* st = ws.state + hl * 4;
    st[0] = (int)b1;
    st[1] = need;
    st[2] = in_b1;
    st[3] = whole ? 1 : 0;
  }
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
  if (threadIdx.x == 0) n_list = 0;
  __syncthreads();
  const float* row = p.scores + (int64_t)(p.head0 + hl) * p.row_stride;
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
  uint64_t* list = ws.list + ((size_t)hl * p.nchunk + w) * kSelectChunk;
  int above = 0;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const uint32_t top = k[i] >> 21;
    above += (k[i] != 0u && top > b1) ? 1 : 0;
    const bool in = k[i] != 0u && top == b1;
    // one list-slot atomic per wave
    const uint64_t m = __ballot(in);
    const int leader = m != 0 ? __ffsll((unsigned long long)m) - 1 : 0;
    int slot0 = 0;
    if (m != 0 && lane == leader) slot0 = atomicAdd(&n_list, __popcll(m));
    slot0 = __shfl(slot0, leader);
    if (in && !whole) {
      const int slot = slot0 + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      list[slot] = composite(k[i], (uint32_t)chunk_pos(base, i));
    }
    if (!whole) agg_inc(hist, (k[i] >> 10) & 2047u, in);
  }
  int total;
  block_scan(above, sh, total);  // (its barriers also order the LDS atomics)
  if (!whole) store_hist(hist, ws.hist2 + ((size_t)hl * p.nchunk + w) * kBins);
  if (threadIdx.x == 0) {
    int* c = ws.cnt + ((size_t)hl * p.nchunk + w) * 2;
    c[0] = n_list;
    c[1] = total;
  }
}

// ---------------------------------------------------------------- launch 3
__global__ __launch_bounds__(kThreads) void sel_finish(SelectArgs p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t lst[kLdsList];
  __shared__ int sh[8];
  __shared__ int res[3];
  __shared__ int list_off[kMaxChunks + 1];
  __shared__ uint32_t chunk_sel[kMaxChunks];
  __shared__ int chunk_off[kMaxChunks + 1];
  __shared__ int n_lds;

  const int hl = blockIdx.y, w = blockIdx.x;
  const int h = p.head0 + hl;
  const int n_choose = p.n_choose[hl];
  const int c0 = p.c0, c1 = p.c1, S = p.S;
  int32_t* dst = p.idx + p.out_off[hl];
  const int a0 = c0 & ~3;
  const int nchunk_h = chunks_of(p);
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

  const Ws ws = ws_of(p);
  const int* st = ws.state + hl * 4;
  const uint32_t b1 = (uint32_t)st[0];
  const int need1 = st[1];
  const bool whole1 = st[3] != 0;
  const float* row = p.scores + (int64_t)h * p.row_stride;
  const int* cnt = ws.cnt + (size_t)hl * p.nchunk * 2;

  for (int c = threadIdx.x; c < nchunk_h; c += kThreads) chunk_sel[c] = (uint32_t)cnt[2 * c + 1];
  wave0_exclusive_scan(nchunk_h, [&](int c) { return cnt[2 * c]; }, list_off);
  if (threadIdx.x == 0) n_lds = 0;
  __syncthreads();

  uint32_t b2 = 0;
  bool whole2 = true;
  uint64_t thr = 0;  // inside (b1, b2), chosen iff composite >= thr
  if (whole1) {
    for (int c = threadIdx.x; c < nchunk_h; c += kThreads) chunk_sel[c] += (uint32_t)cnt[2 * c];
    __syncthreads();
  } else {
    const int n_b1 = list_off[nchunk_h];
    const uint64_t* lists = ws.list + (size_t)hl * p.nchunk * kSelectChunk;
    // entry g (< n_b1) of the concatenated b1 lists; `c` is a chunk hint that
    // only moves forward (each thread visits increasing g)
    auto entry = [&](int g, int& c) {
      while (c + 1 < nchunk_h && list_off[c + 1] <= g) ++c;
      return lists[(size_t)c * kSelectChunk + (g - list_off[c])];
    };
    sum_hists(ws.hist2 + (size_t)hl * p.nchunk * kBins, nchunk_h, hist);
    find_bin(hist, kBins, need1, sh, res);
    b2 = (uint32_t)res[0];
    const int need2 = need1 - res[1];
    const int in_b2 = res[2];
    whole2 = need2 == in_b2;
    const bool in_lds = in_b2 <= kLdsList;
    // one walk over the b1 entries: per-chunk counts above b2 (and, for a
    // whole b2, inside it); the b2 entries go to LDS
    {
      int ch = 0;
      for (int g0 = threadIdx.x; g0 < n_b1 + (kThreads * 8 - 1) - (n_b1 + kThreads * 8 - 1) % (kThreads * 8) ; g0 += kThreads * 8) {
        uint64_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = g0 + j * kThreads;
          v[j] = g < n_b1 ? entry(g, ch) : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = g0 + j * kThreads;
          const bool ok = g < n_b1;
          const uint32_t d2 = comp_d2(v[j]);
          const uint32_t c = ok ? (comp_pos(v[j]) - (uint32_t)a0) / kSelectChunk : 0u;
          agg_inc(chunk_sel, c, ok && (d2 > b2 || (d2 == b2 && whole2)));
          if (ok && d2 == b2 && !whole2 && in_lds) {
            const int slot = atomicAdd(&n_lds, 1);
            if (slot < kLdsList) lst[slot] = v[j];
          }
        }
      }
    }
    __syncthreads();
    if (!whole2) {
      // radix select of the need2-th largest composite among the (b1, b2)
      // entries, over its low 42 bits (key bits 9..0, inverted position):
      // 11 + 11 + 11 + 9 bits
      const int n = in_lds ? min(n_lds, kLdsList) : n_b1;
      uint64_t prefix = 0, pmask = 0;
      int rem = need2;
      const uint64_t lowmask = (1ull << 42) - 1;
      for (int lev = 0; lev < 4; ++lev) {
        const int sft = lev < 3 ? 31 - 11 * lev : 0;
        const int nb = lev < 3 ? 2048 : 512;
        for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
        __syncthreads();
        int ch = 0;
        for (int g0 = threadIdx.x; g0 < n; g0 += kThreads * 8) {
          uint64_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int g = g0 + j * kThreads;
            v[j] = g < n ? (in_lds ? lst[g] : entry(g, ch)) : 0ull;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int g = g0 + j * kThreads;
            const uint64_t x = v[j] & lowmask;
            if (g < n && (in_lds || comp_d2(v[j]) == b2) && (x & pmask) == prefix)
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
      thr = ((uint64_t)b1 << 53) | ((uint64_t)b2 << 42) | prefix;
      // chosen (b1, b2) entries per chunk
      int ch = 0;
      for (int g = threadIdx.x; g < n; g += kThreads) {
        const uint64_t v = in_lds ? lst[g] : entry(g, ch);
        if ((in_lds || comp_d2(v) == b2) && v >= thr)
          atomicAdd(&chunk_sel[(comp_pos(v) - (uint32_t)a0) / kSelectChunk], 1u);
      }
      __syncthreads();
    }
  }
  wave0_exclusive_scan(nchunk_h, [&](int c) { return (int)chunk_sel[c]; }, chunk_off);
  __syncthreads();

  // ordered write of this chunk's chosen positions
  uint32_t k[kPerThread];
  load_chunk(p, row, base, k);
  int out = c0 + chunk_off[w];
  const int out_end = c0 + n_choose;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    bool sel[4];
    int n_mine = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t key = k[4 * it + c];
      const uint32_t top = key >> 21, d2 = (key >> 10) & 2047u;
      bool s = key != 0u && top > b1;
      if (key != 0u && top == b1) {
        if (whole1 || d2 > b2) s = true;
        else if (d2 == b2) s = whole2 || composite(key, (uint32_t)chunk_pos(base, 4 * it + c)) >= thr;
      }
      sel[c] = s;
      n_mine += s;
    }
    int total;
    const int incl = block_scan(n_mine, sh, total);
    int o = out + incl - n_mine;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (sel[c] && o < out_end) dst[o] = chunk_pos(base, 4 * it + c);
      o += sel[c];
    }
    out += total;
  }
}

}  // namespace

size_t select_workspace_bytes(int slots, int nchunk) { return ws_bytes(slots, nchunk); }

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const dim3 grid(a.nchunk, a.nheads);
  hipLaunchKernelGGL(sel_hist, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(sel_collect, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(sel_finish, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

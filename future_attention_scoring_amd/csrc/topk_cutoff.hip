// Running top-k cut-off over static ranks (gfx950).
//
// KVpop ("Delayed Memory Scoring", "Efficient Online Pruning" and Algorithm
// 2): tokens carry a static rank (1 = best); the budget is (s, w, k); at
// query q the token t = q - w leaves the protected window and joins the
// eligible set E(q) if it is not a sink (t >= s); tau_q stays -1 until
// |E(q)| >= k and is then the rank of the k-th best eligible token (0 when
// k = 0), so that the sparse attention keeps the sinks, the window and the
// eligible tokens with rank <= tau_q.
//
// The page keeps E(q) in a Fenwick tree, inserts one token per query and
// finds tau_q by binary lifting: a sequential sweep. Here tau_q is read as
// what it is, the k-th smallest value of the positions [s, q - w] of the
// per-position rank sequence, and every query is answered independently
// from a wavelet matrix of that sequence:
//   * level l holds one bit per position (bit L-1-l of the values, most
//     significant first) with per-word prefix counts of ones, and the next
//     level's sequence is the stable partition of this one by that bit
//     (zeros first);
//   * a query walks the L levels with its range [lo, hi): if the zeros in
//     the range number at least k it follows them, otherwise it counts them
//     off, sets the bit and follows the ones. Two counts per level.
// Build: a fill kernel clears the per-tile counts of ones; wt_ranks
// inverts fam_rank_order's order into a rank per position and counts, per
// 1024-position tile, the ones of the first level (LDS histogram, one
// atomic per touched tile). Then one launch per level (wt_level), one
// workgroup per tile: the tile's ones come first from the counts of the
// earlier tiles, so the kernel writes the bit words and the word counts and
// moves every value to its place in the next level at once; the zeros of the
// next level come first, and their number is known in advance, because the
// values are the ranks - 1, a permutation of 0 .. S-1. While moving, it
// counts the next level's ones per destination tile: a tile's zeros land in
// at most two consecutive tiles and its ones in at most two, so four
// counters in LDS and four atomics per workgroup. Then wt_query answers all
// queries of all heads at once.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kWtThreads = 256;
constexpr int kWtPer = kCutoffTile / kWtThreads;   // positions per thread and tile
constexpr int kWtTileWords = kCutoffTile / 32;     // 32 words
constexpr int kWtRanksPer = 16;                    // order entries per thread in wt_ranks
constexpr int kWtMaxTiles = kCutoffMaxS / kCutoffTile;

struct WtLayout {
  uint32_t* tile1;   // [L][H][ntiles] ones per tile of each level
  int32_t* seq[2];   // [H][S] value sequences of the levels (ping-pong)
  u32x2_t* wc;       // [H][L][nw] {bit word, ones before the word}: one 8-byte load per rank
};

__device__ __forceinline__ WtLayout wt_layout(const CutoffArgs& p) {
  WtLayout w;
  const size_t hs = (size_t)p.H * p.S;
  w.tile1 = reinterpret_cast<uint32_t*>(p.ws);
  w.seq[0] = reinterpret_cast<int32_t*>(w.tile1 + (size_t)p.L * p.H * p.ntiles);
  w.seq[1] = w.seq[0] + hs;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w.seq[1] + hs);
  w.wc = reinterpret_cast<u32x2_t*>((a + 7) & ~(uintptr_t)7);   // 8-byte aligned (the size has the slack)
  return w;
}

__global__ __launch_bounds__(256) void wt_fill_kernel(uint32_t* w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) w[i] = 0u;
}

// Ranks of a block of 4096 order entries of head blockIdx.y, and the first
// level's ones (bit L-1 of rank - 1) per tile of the positions they land on.
__global__ __launch_bounds__(256) void wt_ranks(CutoffArgs p) {
  __shared__ uint32_t hist[kWtMaxTiles];
  const WtLayout w = wt_layout(p);
  const int h = blockIdx.y, tid = threadIdx.x;
  for (int b = tid; b < p.ntiles; b += 256) hist[b] = 0u;
  __syncthreads();
  int pos[kWtRanksPer];   // all loads in flight (clamped index, no branch between them)
#pragma unroll
  for (int j = 0; j < kWtRanksPer; ++j) {
    const int r = (blockIdx.x * kWtRanksPer + j) * 256 + tid;
    pos[j] = p.order[(int64_t)h * p.S + (r < p.S ? r : p.S - 1)];
  }
#pragma unroll
  for (int j = 0; j < kWtRanksPer; ++j) {
    const int r = (blockIdx.x * kWtRanksPer + j) * 256 + tid;
    if (r < p.S && pos[j] >= 0 && pos[j] < p.S) {
      p.rank[(int64_t)h * p.S + pos[j]] = r + 1;
      if ((r >> (p.L - 1)) & 1) atomicAdd(&hist[pos[j] / kCutoffTile], 1u);
    }
  }
  __syncthreads();
  uint32_t* t1 = w.tile1 + (size_t)h * p.ntiles;   // level 0
  for (int b = tid; b < p.ntiles; b += 256)
    if (hist[b]) __hip_atomic_fetch_add(t1 + b, hist[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// How many of 0 .. S-1 have bit b set.
__device__ __forceinline__ int ones_below(int S, int b) {
  const int period = 2 << b, half = 1 << b;
  const int rest = S % period;
  return (S / period) * half + (rest > half ? rest - half : 0);
}

// One level for one tile of one head: bit words, word counts, and the stable
// partition by the level's bit into the next level's sequence, counting the
// next level's ones per destination tile.
__global__ __launch_bounds__(kWtThreads) void wt_level(CutoffArgs p, int l) {
  __shared__ uint32_t wl[kWtTileWords];
  __shared__ uint32_t cl[kWtTileWords];
  __shared__ uint32_t nxt[4];      // next level's ones: zeros' two tiles, then ones' two tiles
  __shared__ int sh_before, sh_total;
  const WtLayout w = wt_layout(p);
  const int tile = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int shift = p.L - 1 - l;
  u32x2_t* wc = w.wc + ((size_t)h * p.L + l) * p.nw;
  const uint32_t* t1 = w.tile1 + ((size_t)l * p.H + h) * p.ntiles;

  // ones of the head before this tile and in all (wave 0), with the values
  // of the tile in flight
  // the level's sequence and the next one (explicit selects: a runtime index
  // into the pointer pair would put it in memory and serialise the loads)
  const int32_t* cur = l == 0 ? p.rank + (int64_t)h * p.S : ((l & 1) ? w.seq[1] : w.seq[0]) + (int64_t)h * p.S;
  const int off = l == 0 ? 1 : 0;   // level 0 holds rank = value + 1
  int v[kWtPer];
#pragma unroll
  for (int j = 0; j < kWtPer; ++j) {
    const int i = tile * kCutoffTile + wave * (kCutoffTile / 4) + j * 64 + lane;
    v[j] = cur[i < p.S ? i : p.S - 1] - off;   // clamped: no branch between the loads
  }
  if (wave == 0) {
    int before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < kWtMaxTiles / 64; ++u) {
      const int b = lane + 64 * u;
      const int c = b < p.ntiles ? (int)t1[b] : 0;
      total += c;
      before += b < tile ? c : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      before += __shfl_xor(before, o);
      total += __shfl_xor(total, o);
    }
    if (lane == 0) {
      sh_before = before;
      sh_total = total;
    }
    if (lane < 4) nxt[lane] = 0u;
  }
  // wave `wave` covers positions tile*1024 + wave*256 + j*64 + lane
  bool bit[kWtPer];
#pragma unroll
  for (int j = 0; j < kWtPer; ++j) {
    const int i = tile * kCutoffTile + wave * (kCutoffTile / 4) + j * 64 + lane;
    bit[j] = i < p.S && ((v[j] >> shift) & 1);
    const uint64_t m = __ballot(bit[j]);
    if (lane == 0) {
      wl[wave * 8 + j * 2] = (uint32_t)m;
      wl[wave * 8 + j * 2 + 1] = (uint32_t)(m >> 32);
    }
  }
  __syncthreads();
  const int before = sh_before;
  // word counts of the tile: exclusive scan of the 32 words' ones
  if (wave == 0 && lane < kWtTileWords) {
    const uint32_t word = wl[lane];
    const int pc = __popc(word);
    int incl = pc;
#pragma unroll
    for (int o = 1; o < kWtTileWords; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    cl[lane] = (uint32_t)(incl - pc);
    wc[tile * kWtTileWords + lane] = u32x2_t{word, (uint32_t)(before + incl - pc)};
    if (tile == p.ntiles - 1 && lane == 0) {   // terminal entry: rank1(S) and the level's ones
      wc[p.nw - 1] = u32x2_t{0u, (uint32_t)sh_total};
    }
  }
  if (l + 1 == p.L) return;   // the last level needs no next sequence
  __syncthreads();
  const int zeros = p.S - ones_below(p.S, shift);
  const int nshift = shift - 1;   // the next level's bit
  const int tz = (tile * kCutoffTile - before) / kCutoffTile;   // first tile of the zeros' run
  const int to = (zeros + before) / kCutoffTile;                 // first tile of the ones' run
  int32_t* next = (((l + 1) & 1) ? w.seq[1] : w.seq[0]) + (int64_t)h * p.S;
#pragma unroll
  for (int j = 0; j < kWtPer; ++j) {
    const int i = tile * kCutoffTile + wave * (kCutoffTile / 4) + j * 64 + lane;
    int slot = -1;
    if (i < p.S) {
      const int lw = wave * 8 + j * 2 + (lane >> 5);
      const int ob = before + (int)cl[lw] + __popc(wl[lw] & ((1u << (i & 31)) - 1u));
      int dst = bit[j] ? zeros + ob : i - ob;
      dst = dst < 0 ? 0 : (dst >= p.S ? p.S - 1 : dst);   // only a non-permutation can leave [0, S)
      next[dst] = v[j];
      const int rel = dst / kCutoffTile - (bit[j] ? to : tz);
      if (((v[j] >> nshift) & 1) && rel >= 0 && rel < 2) slot = (bit[j] ? 2 : 0) + rel;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = __popcll(__ballot(slot == s));
      if (lane == 0 && c) atomicAdd(&nxt[s], (uint32_t)c);
    }
  }
  __syncthreads();
  if (tid < 4 && nxt[tid]) {
    const int dt = (tid < 2 ? tz : to) + (tid & 1);
    uint32_t* t1n = w.tile1 + ((size_t)(l + 1) * p.H + h) * p.ntiles;
    if (dt < p.ntiles) __hip_atomic_fetch_add(t1n + dt, nxt[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// rank1 of a level at position i (0 <= i <= S): the ones before i
__device__ __forceinline__ int wt_rank1(const u32x2_t* wc, int i) {
  const u32x2_t e = wc[i >> 5];
  return (int)e.y + __popc(e.x & ((1u << (i & 31)) - 1u));
}

__global__ __launch_bounds__(256) void wt_query(CutoffArgs p) {
  const WtLayout w = wt_layout(p);
  const int64_t n = (int64_t)p.H * p.S;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += stride) {
    const int h = (int)(e / p.S), q = (int)(e - (int64_t)h * p.S);
    const int hi0 = q - p.w + 1;                   // E(q) = positions [sinks, q - w]
    const int m = hi0 - p.sinks;                   // |E(q)| (negative: none)
    int out;
    if (p.k == 0) {
      out = 0;
    } else if (m < p.k) {
      out = -1;
    } else {
      int lo = p.sinks, hi = hi0, k = p.k, val = 0;
      for (int l = 0; l < p.L; ++l) {
        const u32x2_t* wc = w.wc + ((size_t)h * p.L + l) * p.nw;
        const int o_lo = wt_rank1(wc, lo), o_hi = wt_rank1(wc, hi);
        const int z = (hi - lo) - (o_hi - o_lo);
        if (k <= z) {
          lo -= o_lo;
          hi -= o_hi;
        } else {
          k -= z;
          val |= 1 << (p.L - 1 - l);
          const int zeros = p.S - ones_below(p.S, p.L - 1 - l);   // the level's zeros come first (as placed)
          lo = min(zeros + o_lo, p.S);   // the clamp only acts on a non-permutation order
          hi = min(zeros + o_hi, p.S);
        }
      }
      out = val + 1;
    }
    p.tau[e] = out;
  }
}

}  // namespace

hipError_t launch_cutoff(const CutoffArgs& a0, hipStream_t s) {
  if (a0.H == 0) return hipSuccess;
  CutoffArgs a = a0;
  const int64_t n = (int64_t)a.H * a.S;
  // with k = 0, or fewer than k eligible tokens at the last query, every
  // answer is 0 or -1 and no matrix is needed
  if (a.k > 0 && (int64_t)a.sinks + a.w + a.k - 1 < a.S) {
    const int64_t ncount = (int64_t)a.L * a.H * a.ntiles;
    const int64_t fb = (ncount + 255) / 256;
    hipLaunchKernelGGL(wt_fill_kernel, dim3((unsigned)(fb < 2048 ? fb : 2048)), dim3(256), 0, s,
                       static_cast<uint32_t*>(a.ws), ncount);
    const int rb = (a.S + kWtRanksPer * 256 - 1) / (kWtRanksPer * 256);
    hipLaunchKernelGGL(wt_ranks, dim3((unsigned)rb, (unsigned)a.H), dim3(256), 0, s, a);
    for (int l = 0; l < a.L; ++l)
      hipLaunchKernelGGL(wt_level, dim3((unsigned)a.ntiles, (unsigned)a.H), dim3(kWtThreads), 0, s, a, l);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (n + 255) / 256;
  const unsigned gq = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(wt_query, dim3(gq), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

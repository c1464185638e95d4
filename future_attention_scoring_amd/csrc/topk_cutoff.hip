// Running top-k cut-off over static ranks (gfx950).
//
// KVpop ("Delayed Memory Scoring" and "Efficient Online Pruning"): tokens
// carry a static rank (1 = best); at query q the token t = q - w leaves the
// protected window and becomes eligible, and the cut-off tau_q is the rank of
// the k-th best eligible token, so that the sparse attention keeps the sinks,
// the window and the eligible tokens with rank <= tau_q. With fewer than k
// eligible tokens tau_q = S (every eligible token passes); with k = 0,
// tau_q = 0.
//
// The page keeps the eligible ranks in a Fenwick tree, inserts one token per
// query and finds tau_q by binary lifting: a sequential sweep. Here tau_q is
// read as what it is, the k-th smallest value of the prefix of length
// q - w + 1 of the per-position rank sequence, and every query is answered
// independently from a wavelet matrix of that sequence:
//   * level l holds one bit per position (bit L-1-l of the values, most
//     significant first) with per-word prefix counts of ones, and the next
//     level's sequence is the stable partition of this one by that bit
//     (zeros first);
//   * a query walks the L levels with its prefix [lo, hi): if the zeros in
//     the range number at least k it follows them, otherwise it counts them
//     off, sets the bit and follows the ones. Two counts per level.
// Build: ranks_kernel inverts fam_rank_order's order into a rank per
// position; per level, wt_bits writes the bit words and each 4096-position
// tile's count of ones, and wt_scatter adds the tile prefix to the word
// counts and moves every value to its place in the next level. Then
// wt_query answers all queries of all heads at once.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kWtThreads = 256;
constexpr int kWtPer = 16;                         // positions per thread and tile
constexpr int kWtTile = kWtThreads * kWtPer;       // 4096 positions
constexpr int kWtTileWords = kWtTile / 32;         // 128 words

__global__ __launch_bounds__(256) void ranks_kernel(const int32_t* order, int32_t* rank, int H, int S) {
  const int64_t n = (int64_t)H * S;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const int64_t h = i / S;
    const int r = (int)(i - h * S);
    const int pos = order[i];
    if (pos >= 0 && pos < S) rank[h * S + pos] = r + 1;
  }
}

struct WtLayout {
  int32_t* seq[2];   // [H][S] value sequences of the levels (ping-pong)
  uint32_t* words;   // [H][L][nw] bit words
  uint32_t* cnt;     // [H][L][nw] ones before each word
  int32_t* tile1;    // [H][ntiles] ones per tile of the current level
};

__device__ __forceinline__ WtLayout wt_layout(const CutoffArgs& p) {
  WtLayout w;
  char* b = reinterpret_cast<char*>(p.ws);
  const size_t hs = (size_t)p.H * p.S;
  w.seq[0] = reinterpret_cast<int32_t*>(b);
  w.seq[1] = w.seq[0] + hs;
  w.words = reinterpret_cast<uint32_t*>(w.seq[1] + hs);
  w.cnt = w.words + (size_t)p.H * p.L * p.nw;
  w.tile1 = reinterpret_cast<int32_t*>(w.cnt + (size_t)p.H * p.L * p.nw);
  return w;
}

// value of position i at level l (0 .. S-1; level 0 reads the ranks)
__device__ __forceinline__ int wt_value(const CutoffArgs& p, const WtLayout& w, int h, int l, int i) {
  return l == 0 ? p.rank[(int64_t)h * p.S + i] - 1 : w.seq[l & 1][(int64_t)h * p.S + i];
}

// Level l: bit words of the tile and its count of ones.
__global__ __launch_bounds__(kWtThreads) void wt_bits(CutoffArgs p, int l) {
  __shared__ int red[kWtThreads / 64];
  const int tile = blockIdx.x, h = blockIdx.y;
  const WtLayout w = wt_layout(p);
  const int shift = p.L - 1 - l;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* words = w.words + ((size_t)h * p.L + l) * p.nw;
  int ones = 0;
#pragma unroll 4
  for (int j = 0; j < kWtPer; ++j) {
    // wave `wave` covers positions tile*4096 + wave*1024 + j*64 + lane
    const int i = tile * kWtTile + wave * (kWtTile / 4) + j * 64 + lane;
    const bool bit = i < p.S && ((wt_value(p, w, h, l, i) >> shift) & 1);
    const uint64_t m = __ballot(bit);
    // lanes 0 and 32 store the wave's two words (positions past S are 0)
    if ((lane & 31) == 0) words[i >> 5] = (uint32_t)(lane == 0 ? m : (m >> 32));
    ones += lane == 0 ? __popcll(m) : 0;
  }
  if (lane == 0) red[wave] = ones;
  __syncthreads();
  if (threadIdx.x == 0) w.tile1[(size_t)h * p.ntiles + tile] = red[0] + red[1] + red[2] + red[3];
}

// Level l: word counts (tile prefix added) and the stable partition by the
// level's bit into the next level's sequence.
__global__ __launch_bounds__(kWtThreads) void wt_scatter(CutoffArgs p, int l) {
  __shared__ uint32_t wl[kWtTileWords];
  __shared__ uint32_t cl[kWtTileWords];
  __shared__ int sh[2];
  const int tile = blockIdx.x, h = blockIdx.y;
  const WtLayout w = wt_layout(p);
  const int shift = p.L - 1 - l;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t* words = w.words + ((size_t)h * p.L + l) * p.nw;
  uint32_t* cnt = w.cnt + ((size_t)h * p.L + l) * p.nw;
  const int32_t* t1 = w.tile1 + (size_t)h * p.ntiles;
  // ones before this tile and in total (at most 64 tiles)
  if (wave == 0) {
    const int a = lane < p.ntiles ? t1[lane] : 0;
    int before = lane < tile ? a : 0, all = a;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      before += __shfl_xor(before, o);
      all += __shfl_xor(all, o);
    }
    if (lane == 0) {
      sh[0] = before;
      sh[1] = all;
    }
  }
  // the tile's words and their exclusive prefix counts (wave 0: 2 per lane)
  const int w0 = tile * kWtTileWords;
  if (wave == 0) {
    const uint32_t a = words[w0 + 2 * lane];
    const uint32_t b = words[w0 + 2 * lane + 1];
    const int pa = __popc(a), pb = __popc(b);
    int incl = pa + pb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int ex = incl - pa - pb;
    wl[2 * lane] = a;
    wl[2 * lane + 1] = b;
    cl[2 * lane] = (uint32_t)ex;
    cl[2 * lane + 1] = (uint32_t)(ex + pa);
  }
  __syncthreads();
  const int before = sh[0];
  const int zeros = p.S - sh[1];
  for (int j = threadIdx.x; j < kWtTileWords; j += kWtThreads) cnt[w0 + j] = (uint32_t)before + cl[j];
  if (tile == p.ntiles - 1 && threadIdx.x == 0) {   // terminal entry: rank1(S) and the level's ones
    uint32_t* wr = w.words + ((size_t)h * p.L + l) * p.nw;
    wr[p.nw - 1] = 0u;
    cnt[p.nw - 1] = (uint32_t)sh[1];
  }
  if (l + 1 == p.L) return;   // the last level needs no next sequence
  int32_t* next = w.seq[(l + 1) & 1] + (int64_t)h * p.S;
#pragma unroll 4
  for (int j = 0; j < kWtPer; ++j) {
    const int i = tile * kWtTile + wave * (kWtTile / 4) + j * 64 + lane;
    if (i < p.S) {
      const int v = wt_value(p, w, h, l, i);
      const int lw = (i >> 5) - w0;
      const int ones = before + (int)cl[lw] + __popc(wl[lw] & ((1u << (i & 31)) - 1u));
      next[((v >> shift) & 1) ? zeros + ones : i - ones] = v;
    }
  }
}

// rank1 of level words/counts at position i (0 <= i <= S)
__device__ __forceinline__ int wt_rank1(const uint32_t* words, const uint32_t* cnt, int i) {
  const int wi = i >> 5;
  return (int)cnt[wi] + __popc(words[wi] & ((1u << (i & 31)) - 1u));
}

__global__ __launch_bounds__(256) void wt_query(CutoffArgs p) {
  const WtLayout w = wt_layout(p);
  const int64_t n = (int64_t)p.H * p.S;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += stride) {
    const int h = (int)(e / p.S), q = (int)(e - (int64_t)h * p.S);
    const int m = q - p.w + 1;   // eligible prefix length
    int out;
    if (p.k == 0) {
      out = 0;
    } else if (m < p.k) {
      out = p.S;
    } else {
      int lo = 0, hi = m, k = p.k, val = 0;
      for (int l = 0; l < p.L; ++l) {
        const uint32_t* words = w.words + ((size_t)h * p.L + l) * p.nw;
        const uint32_t* cnt = w.cnt + ((size_t)h * p.L + l) * p.nw;
        const int o_lo = wt_rank1(words, cnt, lo), o_hi = wt_rank1(words, cnt, hi);
        const int z = (hi - lo) - (o_hi - o_lo);
        if (k <= z) {
          lo -= o_lo;
          hi -= o_hi;
        } else {
          k -= z;
          val |= 1 << (p.L - 1 - l);
          const int zeros = p.S - (int)cnt[p.nw - 1];   // the level's zeros come first
          lo = zeros + o_lo;
          hi = zeros + o_hi;
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
  const int64_t blocks = (n + 255) / 256;
  const unsigned gq = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(ranks_kernel, dim3(gq < 4096 ? gq : 4096), dim3(256), 0, s, a.order, a.rank, a.H, a.S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.k > 0 && a.w < a.S) {   // otherwise every answer is 0 or S
    const dim3 grid((unsigned)a.ntiles, (unsigned)a.H);
    for (int l = 0; l < a.L; ++l) {
      hipLaunchKernelGGL(wt_bits, grid, dim3(kWtThreads), 0, s, a, l);
      hipLaunchKernelGGL(wt_scatter, grid, dim3(kWtThreads), 0, s, a, l);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(wt_query, dim3(gq), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

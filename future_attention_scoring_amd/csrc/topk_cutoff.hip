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
// The page keeps the eligible ranks in a Fenwick tree and finds tau_q by
// binary lifting. Here the same values come from a sweep whose steps are
// amortised O(1): the eligible set only grows, so once it holds k tokens the
// k-th smallest rank can only fall. When a token whose rank is below the
// current cut-off arrives, the cut-off moves to the largest present rank
// below it, found by scanning a bitset of the present ranks downwards; over
// a head the scans cover at most S/32 words plus one word per move. The
// bitset (S bits) lives in LDS.
//
// ranks_kernel: rank[h, order[h, r]] = r + 1 (the inverse of the order that
// fam_rank_order writes). cutoff_kernel: one workgroup per head; all threads
// stage the ranks of the next chunk of 2048 newly eligible tokens in LDS and
// store the previous chunk's cut-offs, while wave 0 runs the sweep on
// wave-uniform values (scalar registers and branches).
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kCutThreads = 256;
constexpr int kCutChunk = 2048;                       // queries per staged chunk
constexpr int kCutWords = kCutoffMaxS / 32;           // bitset words

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

__global__ __launch_bounds__(kCutThreads) void cutoff_kernel(CutoffArgs p) {
  __shared__ uint32_t bits[kCutWords];          // bit r-1 set: rank r is eligible
  __shared__ __attribute__((aligned(16))) int32_t rk[2][kCutChunk];   // ranks of the tokens that become eligible
  __shared__ __attribute__((aligned(16))) int32_t tau[kCutChunk];     // cut-offs of the chunk's queries
  const int h = blockIdx.x;
  const int S = p.S, w = p.w, k = p.k;
  const int tid = threadIdx.x;
  const int32_t* rank = p.rank + (int64_t)h * S;
  int32_t* out = p.tau + (int64_t)h * S;
  const int words = (S + 31) / 32;
  for (int i = tid; i < words; i += kCutThreads) bits[i] = 0u;
  // ranks of the tokens that become eligible at queries q0 .. q0+kCutChunk-1
  auto stage = [&](int q0, int buf) {
    for (int i = tid; i < kCutChunk; i += kCutThreads) {
      const int t = q0 + i - w;
      rk[buf][i] = (q0 + i < S && t >= 0) ? rank[t] : 0;
    }
  };
  stage(0, 0);
  __syncthreads();

  // sweep state (wave 0, uniform across its lanes)
  int count = 0;       // eligible tokens so far
  int cut = S;         // current cut-off once count >= k
  int maxr = 0;        // largest eligible rank while count < k
  const int nchunks = (S + kCutChunk - 1) / kCutChunk;
  for (int c = 0; c < nchunks; ++c) {   // uniform across the workgroup
    const int q0 = c * kCutChunk;
    if (c + 1 < nchunks) stage(q0 + kCutChunk, (c + 1) & 1);
    if (tid < 64) {
      // wave 0 runs the sweep on wave-uniform values (scalar registers and
      // branches); lane 0 writes
      const int nq4 = (min(kCutChunk, S - q0) + 3) & ~3;
      const int4* rk4 = reinterpret_cast<const int4*>(rk[c & 1]);
      for (int i = 0; i < nq4; i += 4) {
        const int4 cur = rk4[i >> 2];
        const int rr[4] = {__builtin_amdgcn_readfirstlane(cur.x), __builtin_amdgcn_readfirstlane(cur.y),
                           __builtin_amdgcn_readfirstlane(cur.z), __builtin_amdgcn_readfirstlane(cur.w)};
        int out4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = rr[j];
          if (k > 0 && r >= 1 && r <= S) {
            const int bi = r - 1;
            if (tid == 0) atomicOr(&bits[bi >> 5], 1u << (bi & 31));
            ++count;
            if (count <= k) {
              maxr = max(maxr, r);
              if (count == k) cut = maxr;
            } else if (r < cut) {
              // the old k-th best drops out: the largest present rank below it
              int b = cut - 2;   // bit index of rank cut - 1
              uint32_t word = __builtin_amdgcn_readfirstlane(bits[b >> 5]) & (0xffffffffu >> (31 - (b & 31)));
              while (word == 0u) {
                b = (b & ~31) - 1;
                word = __builtin_amdgcn_readfirstlane(bits[b >> 5]);
              }
              cut = ((b & ~31) | (31 - __builtin_clz(word))) + 1;
            }
          }
          out4[j] = k == 0 ? 0 : (count >= k ? cut : S);
        }
        if (tid == 0) *reinterpret_cast<int4*>(&tau[i]) = int4{out4[0], out4[1], out4[2], out4[3]};
      }
    }
    __syncthreads();
    for (int i = tid; i < kCutChunk && q0 + i < S; i += kCutThreads) out[q0 + i] = tau[i];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_cutoff(const CutoffArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const int64_t n = (int64_t)a.H * a.S;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(ranks_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     a.order, a.rank, a.H, a.S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cutoff_kernel, dim3((unsigned)a.H), dim3(kCutThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

// Per-head top-k selection with forced sinks and recent window (gfx950).
//
// KVpop ("The KVpop Scoring Module", Figure 1): sinks and the protected
// window are always kept; the rest of the budget goes to the best-scored
// long-range tokens. KVP (section 3): the cache is the top of a ranking.
// Ties are broken towards the lower position, -0.0 equals +0.0 and NaN ranks
// below every number, so exactly one kept set is correct.
//
// One workgroup of 1024 threads handles one head:
//   1. fp32 scores map to order-preserving u32 keys (NaN -> 1; 0 is reserved
//      for "not a candidate");
//   2. a radix select over 11 + 11 + 10 key bits finds the threshold: LDS
//      histograms of the keys that still match the chosen prefix, a block
//      scan over the bins from the top, and an early exit as soon as a whole
//      bin is taken;
//   3. each wave owns a contiguous run of candidate rows; per-wave counts of
//      keys above the threshold and equal to it give every wave its output
//      base and its share of the tied keys (lowest positions first);
//   4. a last pass writes the kept positions in ascending order, ranking
//      selected entries inside each 256-position row with ballots.
// Scores are streamed from memory on every pass (a head's scores stay in L2).
// Output per head: sinks, then the chosen candidates, then the window.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRow = 256;  // positions per wave row (4 per lane)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void load_keys(const float* row, bool vec_ok, int pos, int c0, int c1,
                                          uint32_t (&k)[4]) {
  if (vec_ok && pos >= c0 && pos + 3 < c1) {
    const f32x4_t f = *reinterpret_cast<const f32x4_t*>(row + pos);
    k[0] = order_key(f[0]);
    k[1] = order_key(f[1]);
    k[2] = order_key(f[2]);
    k[3] = order_key(f[3]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = pos + c;
      k[c] = (q >= c0 && q < c1) ? order_key(row[q]) : 0u;
    }
  }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ int below_me(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 1024 threads; `total` receives the sum.
__device__ int block_incl_scan(int v, int* sh_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  if (lane == 63) sh_wave[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = sh_wave[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs p) {
  __shared__ uint32_t hist[2048];
  __shared__ int sh_wave[kWaves];
  __shared__ int sh_state[3];
  __shared__ int sh_gt[kWaves], sh_eq[kWaves], sh_selbase[kWaves], sh_eqbase[kWaves];

  const int hl = blockIdx.x;
  const int h = p.head0 + hl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = p.S, c0 = p.c0, c1 = p.c1;
  const int n_choose = p.n_choose[hl];
  const float* row = p.scores + (int64_t)h * p.row_stride;
  int32_t* dst = p.idx + p.out_off[hl];

  if (tid == 0) {
    p.offsets_dev[h] = p.out_off[hl];
    if (h == p.H - 1) p.offsets_dev[p.H] = p.total;
  }
  for (int i = tid; i < c0; i += kThreads) dst[i] = i;
  for (int i = c1 + tid; i < S; i += kThreads) dst[c0 + n_choose + (i - c1)] = i;
  if (n_choose == 0) return;
  if (n_choose == c1 - c0) {
    for (int i = c0 + tid; i < c1; i += kThreads) dst[i] = i;
    return;
  }

  // candidate rows: 256 positions each from a0; wave w owns rows [rw0, rw1)
  const int a0 = c0 & ~3;
  const int nrows = (c1 - a0 + kRow - 1) / kRow;
  const int rpw = (nrows + kWaves - 1) / kWaves;
  const int rw0 = min(nrows, wave * rpw), rw1 = min(nrows, rw0 + rpw);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;

  // ---- radix select of the n_choose-th largest key ----
  uint32_t prefix = 0, pmask = 0;
  int need = n_choose;
  uint32_t t_gt = 0, t_eq = 0;  // selected: key > t_gt, or key == t_eq within the first need_eq
  int need_eq = 0;
  bool resolved = false;
#pragma unroll 1
  for (int level = 0; level < 3 && !resolved; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int nb = level == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int r = rw0; r < rw1; ++r) {
      uint32_t k[4];
      load_keys(row, vec_ok, a0 + r * kRow + 4 * lane, c0, c1, k);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (k[c] != 0u && (k[c] & pmask) == prefix)
          atomicAdd(&hist[(k[c] >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // bins owned by this thread: [tid*bpt, tid*bpt + bpt)
    const int bpt = nb / kThreads;
    int local = 0;
    for (int j = 0; j < bpt; ++j) local += (int)hist[tid * bpt + j];
    int total;
    const int incl = block_incl_scan(local, sh_wave, total);
    int above = total - incl;  // keys in bins after this thread's bins
    for (int j = bpt - 1; j >= 0; --j) {
      const int bin = tid * bpt + j;
      const int cnt = (int)hist[bin];
      if (above < need && need <= above + cnt) {
        sh_state[0] = bin;
        sh_state[1] = above;
        sh_state[2] = cnt;
      }
      above += cnt;
    }
    __syncthreads();
    const int bin = sh_state[0], cnt_above = sh_state[1], cnt_bin = sh_state[2];
    __syncthreads();
    need -= cnt_above;
    prefix |= (uint32_t)bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    if (need == cnt_bin) {  // the whole bin is taken: keep every key >= prefix
      t_gt = prefix == 0u ? 0u : prefix - 1u;
      resolved = true;
    }
  }
  if (!resolved) {  // prefix is now the full threshold key
    t_gt = prefix;
    t_eq = prefix;
    need_eq = need;
  }

  // ---- per-wave counts and output bases ----
  int gt = 0, eq = 0;
  for (int r = rw0; r < rw1; ++r) {
    uint32_t k[4];
    load_keys(row, vec_ok, a0 + r * kRow + 4 * lane, c0, c1, k);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gt += k[c] > t_gt;
      eq += need_eq > 0 && k[c] == t_eq;
    }
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) {
    sh_gt[wave] = gt;
    sh_eq[wave] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    int eq_base = 0, sel_base = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int ties = min(max(need_eq - eq_base, 0), sh_eq[w]);
      sh_eqbase[w] = eq_base;
      sh_selbase[w] = sel_base;
      eq_base += sh_eq[w];
      sel_base += sh_gt[w] + ties;
    }
  }
  __syncthreads();

  // ---- ordered write of the chosen candidates ----
  int eq_run = sh_eqbase[wave];
  int out = c0 + sh_selbase[wave];
  for (int r = rw0; r < rw1; ++r) {
    const int pos = a0 + r * kRow + 4 * lane;
    uint32_t k[4];
    load_keys(row, vec_ok, pos, c0, c1, k);
    bool sel[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sel[c] = k[c] > t_gt;
    if (need_eq > 0) {
      bool is_eq[4];
      int eq_before = 0, eq_row = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        is_eq[c] = k[c] == t_eq;
        const uint64_t m = __ballot(is_eq[c]);
        eq_before += below_me(m);
        eq_row += __popcll(m);
      }
      int rank = eq_run + eq_before;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (is_eq[c]) {
          sel[c] = sel[c] || rank < need_eq;
          ++rank;
        }
      }
      eq_run += eq_row;
    }
    int sel_before = 0, sel_row = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = __ballot(sel[c]);
      sel_before += below_me(m);
      sel_row += __popcll(m);
    }
    int o = out + sel_before;
    const int o_end = c0 + n_choose;  // never write past this head's chosen block
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (sel[c] && o < o_end) dst[o] = pos + c;
      o += sel[c];
    }
    out += sel_row;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.nheads), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fam

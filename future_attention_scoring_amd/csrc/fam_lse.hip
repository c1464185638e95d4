// First pass: causal row log-sum-exp on bf16/fp16 MFMA (gfx950).
//
// KVpop ("Delayed Memory Scoring"): the normaliser of query i sums exp(logit)
// over the keys j <= i. Here each query's normaliser is formed over key tiles,
// in base 2 internally, and stored as a natural log. The Sq query rows are the
// last Sq of the S key positions (row r at position S - Sq + r): Sq = S is the
// full causal square, Sq < S the queries of a chunk over a cache that holds
// the earlier keys.
//
// Work decomposition
//   * A "row unit" is 64 consecutive query positions of one query head. The
//     units of one (batch, KV head) are ordered by position, latest first, and
//     a workgroup of 4 waves takes 4 consecutive units, so the query heads of
//     a GQA group (or neighbouring position blocks when the group is smaller
//     than 4) share every K tile the workgroup stages.
//   * Each wave keeps its 64 queries' Q fragments in registers as the MFMA B
//     operand and computes S^T = K_tile * Q^T, so every accumulator column is
//     one query and the reduction over keys stays inside a lane (the two
//     half-waves hold disjoint key rows and are merged once at the end).
//   * K tiles of 64 keys are double-buffered through LDS with a 16-byte row
//     pad (conflict-free ds_read_b128 of the A fragments).
//   * Workgroups are numbered latest-position-first (the longest causal rows
//     start first) and with the (batch, KV head) index fastest, so with eight
//     KV heads each XCD works on a single head's K.
//
// Shift of the exponentials. Any per-row shift M gives the same normaliser,
// M + log2(sum_j exp2(c*s_ij - M)), as long as the terms neither overflow nor
// all vanish. Two forms are used:
//   * running maximum (the standard online form): exact for any input;
//   * fixed bound (when the caller provides key norms): by Cauchy-Schwarz,
//     c*s_ij <= M_i = c * |q_i| * max_j |k_j|, so no term exceeds one and the
//     per-term maximum and rescaling disappear from the inner loop. If the
//     bound is so loose that some row's sum falls below 2^-80 (then terms that
//     underflow could matter), the workgroup repeats its sweep with the
//     running maximum. A sum of at least 2^-80 over at most 2^28 terms leaves
//     the underflowed part below 2^-98 of it.
//
// Key-range split. A chunk's few thousand queries (or a short sequence) give
// fewer workgroups than the chip holds at once. Since the bounded form's
// shift does not depend on the keys seen, the partial sums of disjoint key
// ranges simply add: the host may split every workgroup's key tiles over
// nks workgroups, each writing its rows' partial sums (and split 0 the
// shift) to a workspace. A second launch of the running-maximum kernel adds
// them in split order and writes the normalisers; a workgroup with a loose
// row repeats the whole sweep with the running maximum, exactly as above.
#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 64;
constexpr int kKeyTile = 64;
constexpr float kMinBoundSum = 0x1p-80f;
constexpr int kReadAhead = 2;   // bounded pass: A-fragment reads ahead of their MFMAs (KS >= 4)

// Causal and ragged-tile mask of a 32x32 block (keys on rows, queries on columns).
__device__ __forceinline__ void mask_block(f32x16_t& acc, int kb, int qblock, int S, int lane) {
  const int qrow = qblock + (lane & 31);
  if (kb + 31 > qblock || kb + 32 > S) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kb + acc_row(v, lane);
      if (key > qrow || key >= S) acc[v] = -kInf;
    }
  }
}

__device__ __forceinline__ void online_update(f32x16_t acc, int kb, int qblock, int S,
                                              int lane, float c, float& m, float& l) {
  mask_block(acc, kb, qblock, S, lane);
  float mx = acc[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = fmaxf(mx, acc[v]);
  const float m_new = fmaxf(m, mx * c);
  const float m_use = m_new == -kInf ? 0.f : m_new;
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(acc[v], c, -m_use));
  l = fmaf(l, fast_exp2(m - m_use), sum16(e));
  m = m_new;
}

__device__ __forceinline__ void bound_update(f32x16_t acc, int kb, int qblock, int S,
                                             int lane, float c, float M, float& l) {
  mask_block(acc, kb, qblock, S, lane);
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(acc[v], c, -M));
  l += sum16(e);
}

// Maximum of |k_j|^2 over one part of the keys of one (batch, KV head).
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void knorm_kernel(LseArgs p, int chunk) {
  constexpr int CPR = D / 8;             // 16-byte pieces per key row
  constexpr int KPP = kThreads / CPR;    // keys per pass of the workgroup
  constexpr int U = 8;                   // passes in flight
  __shared__ float red[kWaves];
  const int part = blockIdx.x % p.nkn, bh = blockIdx.x / p.nkn;
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  const uint16_t* kbase = p.k + b * p.k_sb + h * p.k_sh;
  const int j0 = part * chunk, j1 = min(p.S, j0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, piece = tid % CPR;
  float mx = 0.f;
  for (int base = j0; base < j1; base += KPP * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * KPP + tid / CPR;
      v[u] = j < j1 ? load16(kbase + (int64_t)j * p.k_ss + piece * 8) : zero16();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float ss = sumsq8<T>(v[u]);
#pragma unroll
      for (int o = CPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      mx = fmaxf(mx, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) p.knorm[(int64_t)bh * p.nkn + part] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int D, typename T, bool BOUND, bool SPLIT>
__global__ __launch_bounds__(kThreads, 3) void lse_kernel(LseArgs p, int npb) {
  static_assert(BOUND || !SPLIT, "only the bounded form splits the key range");
  constexpr int PITCH = D + 8;                 // LDS row pitch in elements
  constexpr int KS = D / 16;                   // MFMA k-steps per 32x32 block
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][kKeyTile * PITCH];

  const int nbh = p.B * p.Hkv;
  const int nks = SPLIT ? p.nks : 1;   // key-range splits of this launch
  const int bh = blockIdx.x % nbh;
  const int split = (blockIdx.x / nbh) % nks;
  const int slot = (blockIdx.x / nbh) / nks;
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  // the wave index is uniform over the wave: kept in a scalar register, so that
  // the per-wave window and causal tests below are scalar work
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  const int unit = slot * kWaves + wave;
  const bool active = unit < npb * p.g;
  const int pb = npb - 1 - (active ? unit / p.g : 0);
  const int qh = h * p.g + (active ? unit % p.g : 0);
  const int q0 = pb * kRowsPerWave;   // first query row of this wave
  const int off = p.S - p.Sq;         // position of query row 0
  const int qp0 = off + q0;           // position of the wave's first query row

  // the workgroup's first unit holds its latest positions
  const int pb_top = npb - 1 - (slot * kWaves) / p.g;
  const int kend = min(p.S, off + (pb_top + 1) * kRowsPerWave);
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;

  const uint16_t* qbase = p.q + b * p.q_sb + qh * p.q_sh;
  const uint16_t* kbase = p.k + b * p.k_sb + h * p.k_sh;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  const int64_t row0 = ((int64_t)b * p.Hq + qh) * p.Sq + q0;   // this wave's first row

  if constexpr (!BOUND) {
    if (p.part) {
      // second launch of a split bounded sweep: add the partial sums (split
      // order), and sweep again with the running maximum only if some row
      // of the workgroup came out loose
      const int row = q0 + lane;
      int loose = 0;
      if (active && row < p.Sq) {
        float L = 0.f;
        for (int sp = 0; sp < p.nks; ++sp) L += p.part[sp * rows + row0 + lane];
        const float M = p.part[p.nks * rows + row0 + lane];
        if (L < kMinBoundSum) loose = 1;
        else p.lse[row0 + lane] = (M + fast_log2(L)) * kLn2;
      }
      if (!__syncthreads_or(loose)) return;
    }
  }

  u32x4_t qf[2][KS];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int row = q0 + 32 * blk + col;
    const bool ok = active && row < p.Sq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[blk][ks] = ok ? load16(qbase + (int64_t)row * p.q_ss + ks * 16 + half * 8) : zero16();
  }

  // K tiles go from global memory straight into LDS (gfx950's
  // global_load_lds_dwordx4: lane l of a wave instruction fills the 16 bytes
  // at the LDS base + 16 l), so they hold no registers while in flight. The
  // padded tile is NCH chunks of 64 such slots; slot s is key s / SPR, 16-byte
  // column s % SPR, and the pad column re-reads the row's last 16 bytes.
  // Wave w loads chunks w, w + 4, ...; the last chunk goes to a wave that
  // changes with the tile. Offsets are bytes inside a tile (the host refuses
  // row strides above 2^24 elements, so 64 rows span less than 2^31 bytes);
  // the ragged last tile clamps its keys (keys >= S are masked in the update).
  constexpr int SPR = PITCH / 8;
  constexpr int NCH = kKeyTile * SPR / 64;
  constexpr int NPW = NCH / 4;
  static_assert(kKeyTile * SPR % 64 == 0 && NCH % 4 == 1, "chunks of the padded tile");
  uint32_t koff[NPW + 1];
#pragma unroll
  for (int j = 0; j <= NPW; ++j) {
    const int s = (j < NPW ? wave + 4 * j : NCH - 1) * 64 + lane;
    koff[j] = (uint32_t)((s / SPR) * (int)p.k_ss + min(s % SPR, SPR - 2) * 8) * 2u;
  }
  const uint32_t sk_lds = (uint32_t)(uintptr_t)(lds_void*)&sk[0][0];
  auto load_tile = [&](int t, int buf) {
    const int r0 = t * kKeyTile;
    const int xw = t & 3;   // the wave that loads the last chunk
    const uint16_t* tile = kbase + (int64_t)r0 * p.k_ss;   // uniform
    const uint32_t lb = sk_lds + (uint32_t)(buf * kKeyTile * PITCH * 2);
    if (r0 + kKeyTile <= p.S) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) dma16(tile, koff[j], lb + (uint32_t)((wave + 4 * j) * 1024));
      if (wave == xw) dma16(tile, koff[NPW], lb + (uint32_t)((NCH - 1) * 1024));
    } else {
#pragma unroll
      for (int j = 0; j <= NPW; ++j) {
        if (j < NPW || wave == xw) {
          const int ch = j < NPW ? wave + 4 * j : NCH - 1;
          const int s = ch * 64 + lane;
          const int key = min(s / SPR, p.S - 1 - r0);   // >= 0: r0 < S
          dma16(tile, (uint32_t)(key * (int)p.k_ss + min(s % SPR, SPR - 2) * 8) * 2u,
                lb + (uint32_t)(ch * 1024));
        }
      }
    }
  };
  // the tile's direct loads have landed in LDS (before the barrier that
  // publishes it)
  auto wait_tile = [&]() { __builtin_amdgcn_s_waitcnt(kWaitVm0); };

  float* lse_row = p.lse + row0;
  bool done = false;

  if constexpr (BOUND) {
    // row bounds from |q_i| (this wave's registers) and the head's max |k|^2
    float kk = lane < p.nkn ? p.knorm[(int64_t)bh * p.nkn + lane] : 0.f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kk = fmaxf(kk, __shfl_xor(kk, o));
    float M[2], l[2] = {0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float qq = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qq += sumsq8<T>(qf[blk][ks]);
      qq += __shfl_xor(qq, 32);
      M[blk] = p.c * sqrtf(qq * kk);
    }
    // this workgroup's share of the key tiles
    const int t0 = (int)((int64_t)ntiles * split / nks), t1 = (int)((int64_t)ntiles * (split + 1) / nks);
    if (t0 < t1) {
      load_tile(t0, 0);
      wait_tile();
    }
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      const bool more = t + 1 < t1;
      if (more) load_tile(t + 1, (t + 1 - t0) & 1);
      const uint16_t* buf = sk[(t - t0) & 1];
#pragma unroll
      for (int kk2 = 0; kk2 < kKeyTile / 32; ++kk2) {
        const int kb = t * kKeyTile + 32 * kk2;
        if (active && kb <= qp0 + 63 && kb < p.S) {
          f32x16_t acc0 = {}, acc1 = {};
          // the wave's MFMA block at raised priority: its matrix work issues
          // while the other waves of the SIMD are in their exp/sum phase
          __builtin_amdgcn_s_setprio(1);
          // the A fragments are read kReadAhead k-steps ahead of their MFMAs:
          // the first kReadAhead reads, then per k-step two MFMAs and the
          // read kReadAhead steps ahead, then the last MFMAs (without the
          // scheduling groups the compiler waits for each read just before
          // its MFMAs)
          u32x4_t af[KS];
#pragma unroll
          for (int ks = 0; ks < kReadAhead; ++ks)
            af[ks] = *reinterpret_cast<const u32x4_t*>(&buf[(32 * kk2 + col) * PITCH + ks * 16 + half * 8]);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + kReadAhead < KS)
              af[ks + kReadAhead] = *reinterpret_cast<const u32x4_t*>(
                  &buf[(32 * kk2 + col) * PITCH + (ks + kReadAhead) * 16 + half * 8]);
            acc0 = Mma<T>::run(af[ks], qf[0][ks], acc0);
            acc1 = Mma<T>::run(af[ks], qf[1][ks], acc1);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);   // DS reads
#pragma unroll
          for (int ks = 0; ks < KS - kReadAhead; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * kReadAhead, 0);
          __builtin_amdgcn_s_setprio(0);
          bound_update(acc0, kb, qp0, p.S, lane, p.c, M[0], l[0]);
          bound_update(acc1, kb, qp0 + 32, p.S, lane, p.c, M[1], l[1]);
        }
      }
      if (more) wait_tile();
      __syncthreads();
    }
    if constexpr (SPLIT) {   // partial sums and the shift; the second launch finishes
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float Lp = l[blk] + __shfl_xor(l[blk], 32);
        const int row = q0 + 32 * blk + col;
        if (active && half == 0 && row < p.Sq) {
          p.part[split * rows + row0 + 32 * blk + col] = Lp;
          if (split == 0) p.part[nks * rows + row0 + 32 * blk + col] = M[blk];
        }
      }
      return;
    }
    float L[2];
    int loose = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      L[blk] = l[blk] + __shfl_xor(l[blk], 32);
      const int row = q0 + 32 * blk + col;
      if (active && row < p.Sq && L[blk] < kMinBoundSum) loose = 1;
    }
    if (!__syncthreads_or(loose)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int row = q0 + 32 * blk + col;
        if (active && half == 0 && row < p.Sq)
          lse_row[32 * blk + col] = (M[blk] + fast_log2(L[blk])) * kLn2;
      }
      done = true;
    }
  }
  if (done) return;

  // running maximum: the plain form, or the repeat of a loose bound
  float m[2] = {-kInf, -kInf}, l[2] = {0.f, 0.f};
  load_tile(0, 0);
  wait_tile();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1, (t + 1) & 1);
    const uint16_t* buf = sk[t & 1];
#pragma unroll
    for (int kk = 0; kk < kKeyTile / 32; ++kk) {
      const int kb = t * kKeyTile + 32 * kk;
      if (active && kb <= qp0 + 63 && kb < p.S) {
        f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              &buf[(32 * kk + col) * PITCH + ks * 16 + half * 8]);
          acc0 = Mma<T>::run(a, qf[0][ks], acc0);
          acc1 = Mma<T>::run(a, qf[1][ks], acc1);
        }
        online_update(acc0, kb, qp0, p.S, lane, p.c, m[0], l[0]);
        online_update(acc1, kb, qp0 + 32, p.S, lane, p.c, m[1], l[1]);
      }
    }
    if (more) wait_tile();
    __syncthreads();
  }

#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float mo = __shfl_xor(m[blk], 32);
    const float lo = __shfl_xor(l[blk], 32);
    const float Mx = fmaxf(m[blk], mo);
    const float Mu = Mx == -kInf ? 0.f : Mx;
    const float L = l[blk] * fast_exp2(m[blk] - Mu) + lo * fast_exp2(mo - Mu);
    const int row = q0 + 32 * blk + col;
    if (active && half == 0 && row < p.Sq) lse_row[32 * blk + col] = (Mx + fast_log2(L)) * kLn2;
  }
}

template <int D, typename T>
hipError_t launch_lse_t(const LseArgs& a, hipStream_t s) {
  const int npb = (a.Sq + kRowsPerWave - 1) / kRowsPerWave;
  const int slots = (npb * a.g + kWaves - 1) / kWaves;
  const int64_t grid = (int64_t)slots * a.B * a.Hkv;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.knorm && a.nks > 1 && a.part) {
    if (grid * a.nks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((lse_kernel<D, T, true, true>), dim3((unsigned)(grid * a.nks)), dim3(kThreads), 0, s, a, npb);
    hipLaunchKernelGGL((lse_kernel<D, T, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, npb);
  } else if (a.knorm) {
    hipLaunchKernelGGL((lse_kernel<D, T, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, npb);
  } else {
    LseArgs b = a;
    b.part = nullptr;
    hipLaunchKernelGGL((lse_kernel<D, T, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, b, npb);
  }
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_knorm_t(const LseArgs& a, hipStream_t s) {
  const int chunk = (a.S + a.nkn - 1) / a.nkn;
  const int64_t grid = (int64_t)a.nkn * a.B * a.Hkv;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((knorm_kernel<D, T>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse(const LseArgs& a, Elem e, hipStream_t s) {
  if (a.d == 128) return e == Elem::kBf16 ? launch_lse_t<128, Bf16>(a, s) : launch_lse_t<128, Fp16>(a, s);
  return e == Elem::kBf16 ? launch_lse_t<64, Bf16>(a, s) : launch_lse_t<64, Fp16>(a, s);
}

hipError_t launch_knorm(const LseArgs& a, Elem e, hipStream_t s) {
  if (a.d == 128) return e == Elem::kBf16 ? launch_knorm_t<128, Bf16>(a, s) : launch_knorm_t<128, Fp16>(a, s);
  return e == Elem::kBf16 ? launch_knorm_t<64, Bf16>(a, s) : launch_knorm_t<64, Fp16>(a, s);
}

}  // namespace fam

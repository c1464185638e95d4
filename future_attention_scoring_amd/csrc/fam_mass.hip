// Second pass: key-major future-attention mass on bf16/fp16 MFMA (gfx950).
//
// KVpop ("Defining Future Attention Utility", Figure 2 "Transposed
// Attention", and the appendix on the transposed pass): the mass of key j is
// the sum, over the query heads of its GQA group and over queries i >= j + W,
// of exp(logit_ij - LSE_i). The page obtains it by swapping the roles of
// queries and keys in an attention call; here the same sum is formed directly
// as register column sums, which needs no running maximum because every term
// exp(logit - LSE) is at most one. The Sq query rows are the last Sq of the S
// key positions (row r at position S - Sq + r), so a chunk's queries can score
// the keys of a cache that also holds earlier positions.
//
// Work decomposition
//   * A workgroup owns 256 consecutive keys of one (batch, KV head); each of
//     its 4 waves keeps 64 keys' K fragments in registers as the MFMA B
//     operand and computes S = Q_tile * K^T, so every accumulator column is
//     one key and the column sum over queries stays inside a lane (the two
//     half-waves hold disjoint query rows and are added once at the end).
//   * The workgroup walks the 64-row query tiles i >= j0 + W of every query
//     head of the group, latest tile first. Each (tile, head) step stages 64
//     query rows and, per row, -L/c (the normaliser in base-2 units over the
//     scale c, where the row's accumulators start) in double-buffered LDS;
//     the rows go from global memory straight into LDS (a uniform tile base
//     plus one 32-bit offset per chunk and lane), the next step's while the
//     current one computes.
//   * Only band steps (those that contain some i < j + W) evaluate the window
//     predicate. Keys that no query can reach (j > S - 1 - W) get exactly 0.
//   * Per-step partial sums are added into a mid-level accumulator that is
//     folded into the total every 8 steps, which bounds the fp32 summation
//     error independently of S.
//   * Workgroups are numbered earliest-key-first (the longest columns start
//     first) with the (batch, KV head) index fastest, so with eight KV heads
//     every XCD works on one head.
//   * Short sequences give too few (and very unequal) key blocks to fill the
//     chip, so the host may split each key block's steps over nsplit
//     workgroups; their partial sums go to a caller workspace and a second
//     launch adds them in split order (deterministic).
//   * Long sequences split by ranges of query rows instead: split s of every
//     key block takes the tiles [s * R, (s + 1) * R) and the workgroups run
//     range-major, latest range first. Workgroups at different key positions
//     would otherwise stream different query tiles at the same time, and the
//     caches would not hold them; within a range they share a few MB of Q.
//     The per-query-head mode splits the same way, one partial slice per
//     query head.
#include <type_traits>

#include "fam_device.hpp"
#include "fam_kernels.hpp"

namespace fam {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = 64;
constexpr int kKeysPerWG = kKeysPerWave * kWaves;
static_assert(kKeysPerWG == kMassKeysPerWG, "host and kernel key-block size");
constexpr int kQTile = 64;   // query rows per staged step (two 32-row MFMA blocks)
constexpr int kReadAhead = 2;   // A-fragment reads issued this many k-steps ahead
static_assert(kQTile == kMassQTile, "host and kernel query-tile size");

// The accumulator of a block starts at -L_i / c for its query row i, so that
// after the MFMAs it holds s - L_i / c and each term is exp2(c * acc): one
// multiply per element, and the normalisers need no registers beside the
// accumulators once the MFMAs have started. (The rounding of -L_i / c and of
// the accumulation is scaled back down by c: about |L_i| * 2^-21 in the
// exponent, i.e. a relative error near 1e-5 at most per term.)
//
// Sum of exp2(c * acc) over one 32x32 block, no window predicate.
__device__ __forceinline__ float block_sum_full(const f32x16_t& acc, float c) {
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(acc[v] * c);
  return sum16(e);
}

// Same with the window predicate i >= j + W.
__device__ __forceinline__ float block_sum_band(const f32x16_t& acc, int i0, int jk, int W, int lane,
                                                float c) {
  if (i0 + 31 < jk + W) return 0.f;
  float e[16];
  const int j = jk + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float x = fast_exp2(acc[v] * c);
    e[v] = i0 + acc_row(v, lane) < j + W ? 0.f : x;
  }
  return sum16(e);
}


// PER_HEAD: the steps run head-major (all tiles of one query head, then the
// next) and each query head's column sums go to mass_q [B, Hq, S] when its
// last tile is done; otherwise the steps interleave the heads tile by tile
// and the group sum goes to mass [B, Hkv, S].
template <int D, typename T, bool PER_HEAD>
__global__ __launch_bounds__(kThreads, 3) void mass_kernel(MassArgs p) {
  constexpr int PITCH = D + 8;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][kQTile * PITCH];
  __shared__ __attribute__((aligned(16))) float sl[2][kQTile];

  const int nbh = p.B * p.Hkv;
  const int bh = blockIdx.x % nbh;
  const int rest = blockIdx.x / nbh;
  // range mode numbers the workgroups range-major, latest range first, so
  // that the workgroups resident together read the same query tiles
  const int rtiles = p.range_tiles;
  const int nkb_all = (p.S + kKeysPerWG - 1) / kKeysPerWG;
  const int split = rtiles > 0 ? p.nsplit - 1 - rest / nkb_all : (PER_HEAD ? 0 : rest % p.nsplit);
  const int kbi = rtiles > 0 ? rest % nkb_all : (PER_HEAD ? rest : rest / p.nsplit);
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  // the wave index is uniform over the wave: kept in a scalar register, so that
  // the per-wave window and causal tests below are scalar work
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;

  const int j0 = kbi * kKeysPerWG;
  const int jw = j0 + wave * kKeysPerWave;

  // PER_HEAD: query head gi's column sums go to mass_q, or in range mode to
  // its slice of the partial sums [nsplit][B][Hq][S]
  auto head_dst = [&](int gi) {
    const int64_t row = (int64_t)b * p.Hq + h * p.g + gi;
    return rtiles > 0 ? p.part + ((int64_t)split * p.B * p.Hq + row) * p.S : p.mass_q + row * p.S;
  };
  // query row r (position off + r) sees key j iff r >= j + Wr; the block's
  // future queries lie in the tiles [t_first, t_last)
  const int Wr = p.W - (p.S - p.Sq);
  const int i_first = max(0, j0 + Wr);
  const int t_first = i_first / kQTile;
  const int t_last = (p.Sq + kQTile - 1) / kQTile;
  // range mode: the tiles [split * rtiles, (split + 1) * rtiles) of this
  // workgroup's range that hold future queries of the block, [r_lo, r_hi)
  const int r_lo = rtiles > 0 ? max(t_first, split * rtiles) : t_first;
  const int r_hi = rtiles > 0 ? min(t_last, (split + 1) * rtiles) : t_last;

  const uint16_t* kbase = p.k + b * p.k_sb + h * p.k_sh;
  u32x4_t kf[2][KS];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int key = jw + 32 * blk + col;
    const bool ok = key < p.S && r_lo < r_hi;   // an empty range only writes zeros
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[blk][ks] = ok ? load16(kbase + (int64_t)key * p.k_ss + ks * 16 + half * 8) : zero16();
  }
  // wait for the K fragments here, once: otherwise the compiler's wait
  // analysis keeps them pending across the loop's back edge and waits for
  // every load in flight (the next step's Q tile included) before each step's
  // first MFMA
  __builtin_amdgcn_s_waitcnt(0);

  float top[2] = {0.f, 0.f}, mid[2] = {0.f, 0.f};
  // this wave's column sums (the two half-waves added) into dst[key]
  auto write_cols = [&](float* dst) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float tot = top[blk] + mid[blk];
      tot += __shfl_xor(tot, 32);
      const int key = jw + 32 * blk + col;
      if (half == 0 && key < p.S) dst[key] = tot;
    }
  };
  if (i_first < p.Sq) {
    const int g = p.g;
    const int t0 = t_first;
    const int t1 = t_last;
    const int ntiles = t1 - t0;
    const int nsteps = ntiles * g;
    // tiles t >= t_full have every row r >= j0 + 255 + Wr: no predicate needed
    const int t_full = (max(0, j0 + kKeysPerWG - 1 + Wr) + kQTile - 1) / kQTile;
    // PER_HEAD walks the tiles [r_lo, r_hi) (all of [t0, t1) outside range
    // mode) once per query head
    const int ntw = r_hi - r_lo;
    const int nfull_h = PER_HEAD ? max(0, r_hi - max(t_full, r_lo))   // per query head
                                 : max(0, t1 - max(t_full, t0));
    // step u = sq * D + sr with D = ntw (PER_HEAD: sq the query head, sr the
    // tile counted from the latest) or D = g (sq the tile counted from the
    // latest, sr the query head); the loop keeps the pair (sq, sr) and steps
    // it instead of dividing every step
    auto tile_at = [&](int sq_, int sr_) { return PER_HEAD ? r_hi - 1 - sr_ : t1 - 1 - sq_; };
    auto head_at = [&](int sq_, int sr_) { return PER_HEAD ? sq_ : sr_; };

    const uint16_t* qgroup = p.q + b * p.q_sb + (int64_t)(h * g) * p.q_sh;
    const float* lgroup = p.lse + ((int64_t)b * p.Hq + h * g) * p.Sq;
    // The Q tile goes from global memory straight into LDS (gfx950's
    // global_load_lds_dwordx4: lane l of a wave instruction fills the 16
    // bytes at the LDS base + 16 l), so it holds no registers while in
    // flight. The padded tile is NCH chunks of 64 such slots; slot s is row
    // s / SPR, 16-byte column s % SPR, and the pad column re-reads the row's
    // last 16 bytes. Wave w loads chunks w, w + 4, ...; the last chunk goes to
    // a wave that changes with the step. Offsets are bytes inside a tile: the
    // host refuses row strides above 2^24 elements, so 64 rows span less than
    // 2^31 bytes.
    constexpr int SPR = PITCH / 8;
    constexpr int NCH = kQTile * SPR / 64;
    constexpr int NPW = NCH / 4;
    static_assert(kQTile * SPR % 64 == 0 && NCH % 4 == 1, "chunks of the padded tile");
    uint32_t qoff[NPW + 1];   // bytes
#pragma unroll
    for (int j = 0; j <= NPW; ++j) {
      const int s = (j < NPW ? wave + 4 * j : NCH - 1) * 64 + lane;
      qoff[j] = (uint32_t)((s / SPR) * (int)p.q_ss + min(s % SPR, SPR - 2) * 8) * 2u;
    }
    const uint32_t sq_lds = (uint32_t)(uintptr_t)(lds_void*)&sq[0][0];
    auto dma = [&](const uint16_t* tile, uint32_t off, int buf, int chunk) {
      dma16(tile, off, sq_lds + (uint32_t)(buf * kQTile * PITCH * 2 + chunk * 1024));
    };
    // the step's 64 normalisers are loaded and staged by one wave, lw, which
    // rotates with the step so that no SIMD carries that work every step
    float lst = 0.f;
    bool lrow_ok = true;
    const float nlc = -kLog2e / p.c;   // accumulator start = lse * nlc
    auto load_step = [&](int sq_, int sr_, int lw, int buf) {
      const int t = tile_at(sq_, sr_);
      const int gi = head_at(sq_, sr_);
      const int r0 = t * kQTile;
      const int xw = (lw + 2) & 3;   // the wave that loads the last chunk
      const uint16_t* tile = qgroup + gi * p.q_sh + (int64_t)r0 * p.q_ss;   // uniform
      if (r0 + kQTile <= p.Sq) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) dma(tile, qoff[j], buf, wave + 4 * j);
        if (wave == xw) dma(tile, qoff[NPW], buf, NCH - 1);
      } else {  // ragged last tile: rows past Sq re-read row Sq - 1 (their normaliser is -inf)
#pragma unroll
        for (int j = 0; j <= NPW; ++j) {
          if (j < NPW || wave == xw) {
            const int ch = j < NPW ? wave + 4 * j : NCH - 1;
            const int s = ch * 64 + lane;
            const int row = min(s / SPR, p.Sq - 1 - r0);   // >= 0: r0 < Sq
            dma(tile, (uint32_t)(row * (int)p.q_ss + min(s % SPR, SPR - 2) * 8) * 2u, buf, ch);
          }
        }
      }
      if (wave == lw) {
        const int row = r0 + lane;
        // the loaded value is not used until the store, so that this wave
        // does not wait for the step's loads here
        lst = lgroup[(int64_t)gi * p.Sq + min(row, p.Sq - 1)];
        lrow_ok = row < p.Sq;
      }
    };
    auto store_step = [&](int buf, int lw) {
      if (wave == lw) {
        // the slot's address is formed here from the lane index (an opaque
        // copy, so that it is not hoisted out of the loop into a spilled register)
        int t = lane;
        asm volatile("" : "+v"(t));
        sl[buf][t] = lrow_ok ? lst * nlc : -kInf;   // the accumulators' start (rows past Sq: -inf)
      }
      // the tile's direct loads have landed in LDS before the barrier that follows
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    };

    // this workgroup's share of the key block's steps: its range's tiles, or
    // an even share of all steps
    int u_begin = PER_HEAD ? 0 : (int)((int64_t)nsteps * split / p.nsplit);
    int u_end = PER_HEAD ? max(0, ntw) * g : (int)((int64_t)nsteps * (split + 1) / p.nsplit);
    if (!PER_HEAD && rtiles > 0) {
      u_begin = r_lo < r_hi ? (t1 - r_hi) * g : 0;
      u_end = r_lo < r_hi ? (t1 - r_lo) * g : 0;
    }
    const int nsr = PER_HEAD ? ntw : g;   // D above
    int cq = 0, cr = 0;   // (sq, sr) of step u
    if (u_begin < u_end) {   // then nsr >= 1
      cq = u_begin / nsr;
      cr = u_begin - cq * nsr;
      load_step(cq, cr, u_begin & 3, u_begin & 1);
      store_step(u_begin & 1, u_begin & 3);
      __syncthreads();
    }
    for (int u = u_begin; u < u_end; ++u) {
      const bool more = u + 1 < u_end;
      int nq = cq, nr = cr + 1;   // (sq, sr) of step u + 1
      if (nr == nsr) {
        nr = 0;
        ++nq;
      }
      if (more) load_step(nq, nr, (u + 1) & 3, (u + 1) & 1);
      const int buf = u & 1;
      const int i0t = tile_at(cq, cr) * kQTile;
      const bool full = PER_HEAD ? cr < nfull_h : u < nfull_h * g;
      // the step's two 32-row blocks, instantiated for full steps (no
      // window tests at all) and for band steps; one uniform branch a step
      auto blocks = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
        for (int rb = 0; rb < kQTile / 32; ++rb) {
          const int i0 = i0t + 32 * rb;
          if (FULL || i0 + 31 >= jw + Wr) {
            float lv[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&sl[buf][32 * rb + 8 * r4 + 4 * half]);
              lv[4 * r4 + 0] = x[0];
              lv[4 * r4 + 1] = x[1];
              lv[4 * r4 + 2] = x[2];
              lv[4 * r4 + 3] = x[3];
            }
            f32x16_t acc0, acc1;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc0[v] = lv[v];
            acc1 = acc0;
            // the A fragments are read kReadAhead k-steps ahead of their MFMAs:
            // the normaliser reads and the first kReadAhead fragment reads,
            // then per k-step two MFMAs and the read kReadAhead steps ahead,
            // then the last MFMAs (left to itself the compiler reads one step
            // ahead)
            u32x4_t af[KS];
#pragma unroll
            for (int ks = 0; ks < kReadAhead; ++ks)
              af[ks] = *reinterpret_cast<const u32x4_t*>(&sq[buf][(32 * rb + col) * PITCH + ks * 16 + half * 8]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              if (ks + kReadAhead < KS)
                af[ks + kReadAhead] = *reinterpret_cast<const u32x4_t*>(
                    &sq[buf][(32 * rb + col) * PITCH + (ks + kReadAhead) * 16 + half * 8]);
              acc0 = Mma<T>::run(af[ks], kf[0][ks], acc0);
              acc1 = Mma<T>::run(af[ks], kf[1][ks], acc1);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4 + kReadAhead, 0);   // DS reads
#pragma unroll
            for (int ks = 0; ks < KS - kReadAhead; ++ks) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMAs
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * kReadAhead, 0);
            if constexpr (FULL) {
              mid[0] += block_sum_full(acc0, p.c);
              mid[1] += block_sum_full(acc1, p.c);
              // keep the next block's reads and MFMAs from being scheduled
              // into this block's exps (that raises the register peak)
              __builtin_amdgcn_sched_barrier(0);
            } else {
              mid[0] += block_sum_band(acc0, i0, jw, Wr, lane, p.c);
              mid[1] += block_sum_band(acc1, i0, jw + 32, Wr, lane, p.c);
            }
          }
        }
      };
      if (full) blocks(std::true_type{});
      else blocks(std::false_type{});
      if ((u & 7) == 7) {
        top[0] += mid[0];
        top[1] += mid[1];
        mid[0] = 0.f;
        mid[1] = 0.f;
      }
      if (PER_HEAD && cr == ntw - 1) {  // this query head is complete
        write_cols(head_dst(cq));
        top[0] = top[1] = mid[0] = mid[1] = 0.f;
      }
      if (more) store_step((u + 1) & 1, (u + 1) & 3);
      __syncthreads();
      cq = nq;
      cr = nr;
    }
  }

  if (!PER_HEAD) {
    write_cols(p.nsplit > 1 ? p.part + ((int64_t)split * nbh + bh) * p.S
                            : p.mass + ((int64_t)b * p.Hkv + h) * p.S);
  } else if (i_first >= p.Sq || r_lo >= r_hi) {  // no future query here: every head's part is 0
    for (int gi = 0; gi < p.g; ++gi) write_cols(head_dst(gi));
  }
}

// mass = sum over the splits of the partial column sums, in split order.
// The slices' loads go out kBatch at a time and are added in split order,
// so a thread waits for a few round trips instead of one per slice.
__global__ __launch_bounds__(kThreads) void mass_reduce_kernel(const float* part, float* mass,
                                                               int64_t n, int nsplit) {
  constexpr int kBatch = 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
    float acc = 0.f;
    for (int k0 = 0; k0 < nsplit; k0 += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = part[(int64_t)min(k0 + j, nsplit - 1) * n + e];   // in bounds, used only if k0 + j < nsplit
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (k0 + j < nsplit) acc = k0 + j == 0 ? v[j] : acc + v[j];
    }
    mass[e] = acc;
  }
}

template <int D, typename T>
hipError_t launch_mass_t(const MassArgs& a, hipStream_t s, bool reduce) {
  const int nkb = (a.S + kKeysPerWG - 1) / kKeysPerWG;
  const bool per_head = a.mass_q != nullptr;
  // per-query-head mass splits only in range mode
  const int nsplit = per_head && a.range_tiles == 0 ? 1 : a.nsplit;
  const int64_t grid = (int64_t)nkb * nsplit * a.B * a.Hkv;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (per_head)
    hipLaunchKernelGGL((mass_kernel<D, T, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mass_kernel<D, T, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  if (nsplit > 1 && reduce) {
    const int64_t n = (int64_t)a.B * (per_head ? a.Hq : a.Hkv) * a.S;
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(mass_reduce_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(kThreads), 0, s, a.part, per_head ? a.mass_q : a.mass, n, nsplit);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mass(const MassArgs& a, Elem e, hipStream_t s, bool reduce) {
  if (a.d == 128)
    return e == Elem::kBf16 ? launch_mass_t<128, Bf16>(a, s, reduce) : launch_mass_t<128, Fp16>(a, s, reduce);
  return e == Elem::kBf16 ? launch_mass_t<64, Bf16>(a, s, reduce) : launch_mass_t<64, Fp16>(a, s, reduce);
}

}  // namespace fam

// Launch interfaces between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fam {

enum class Elem { kBf16, kFp16 };

// Query rows and key rows. The S keys sit at positions 0 .. S-1 and the Sq
// query rows (Sq <= S) at positions S - Sq .. S - 1 (the queries of the last
// Sq positions; Sq = S is the full causal square).

// Causal row log-sum-exp (first pass).
struct LseArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* lse;  // [B, Hq, Sq]
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int B, Hq, Hkv, S, d, g;
  int Sq;
  float c;  // scale * log2(e)
  // Key-norm bound: knorm[(b * Hkv + h) * nkn + p] is the largest |k_j|^2
  // over key range p of that KV head (written by launch_knorm). Null selects
  // the running-maximum form of the first pass.
  float* knorm;
  int nkn;
  // Key-range split of the bounded form (nks > 1, knorm set): workgroup
  // split s sums its share of the key tiles and writes the row's partial sum
  // to part[s * R + row] (R = B * Hq * Sq rows); split 0 also writes the
  // row's shift M to part[nks * R + row]. A second launch adds the partial
  // sums and repeats the sweep with the running maximum where the bound
  // turned out loose. part holds (nks + 1) * R floats.
  float* part;
  int nks;
};
constexpr int kNormParts = 64;   // partial key-norm maxima per (batch, KV head)
constexpr int kLseMaxSplits = 8; // key-range splits of the bounded first pass
hipError_t launch_knorm(const LseArgs& a, Elem e, hipStream_t s);
hipError_t launch_lse(const LseArgs& a, Elem e, hipStream_t s);

// Key-major future-attention mass (second pass).
struct MassArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* lse;  // [B, Hq, Sq]
  float* mass;       // [B, Hkv, S]
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int B, Hq, Hkv, S, d, g, W;
  int Sq;
  float c;  // scale * log2(e)
  float* mass_q;  // non-null: per-query-head mass [B, Hq, S] instead of `mass`
  // Split of each key block's query tiles over nsplit workgroups (group-sum
  // mode only): with nsplit > 1 the partial sums go to part [nsplit, B*Hkv*S]
  // and a reduction adds them into `mass` in a fixed order.
  float* part;
  int nsplit;
  // Range mode (range_tiles > 0): split s owns the query tiles
  // [s * range_tiles, (s + 1) * range_tiles) of every key block instead of an
  // even share of the block's steps. In per-query-head mode (the only split
  // it has) the parts are [nsplit, B*Hq*S] and the reduction writes mass_q.
  int range_tiles;
};
constexpr int kMassKeysPerWG = 256;   // keys owned by one mass-pass workgroup
constexpr int kMassQTile = 64;        // query rows per mass-pass step
constexpr int kMassRangeTiles = 64;   // query tiles per range in range mode
constexpr int kMassRangeMinS = 65536; // range mode from this many keys on
constexpr int kMassMaxRanges = 128;   // at most this many ranges (partial slices)
// With reduce == false and nsplit > 1 the partial sums stay in `part` and
// the caller launches their reduction (the select launches that read them).
hipError_t launch_mass(const MassArgs& a, Elem e, hipStream_t s, bool reduce = true);

// KVpop supervision target from per-query-head mass.
struct TargetArgs {
  const float* mass_q;  // [B, Hq, S]
  float* target;        // [B, Hkv, S]
  int B, Hq, Hkv, S, W;
  float eps;
  int mean;             // 0: max over the group of the logs; 1: log of the group mean
};
hipError_t launch_target(const TargetArgs& a, hipStream_t s);

// Per-head selection. Heads are launched in batches of up to kSelectBatch
// whose plan travels in the kernel arguments; each head's candidates are
// split into chunks of kSelectChunk positions. Up to kSelectMaxCandidates a
// head: three launches (evict_select.hip); beyond, up to
// kSelectLongMaxCandidates: one round-based launch (evict_select_long.hip).
constexpr int kSelectBatch = 64;
constexpr int kSelectChunk = 4096;
constexpr int kSelectMaxCandidates = 131072;
constexpr int kSelectLongMaxCandidates = 1 << 20;
constexpr int kSelectLongMaxChunks = kSelectLongMaxCandidates / kSelectChunk + 1;   // chunks start 4-aligned
constexpr int kSelectLongSlotWordsMax = 10240;   // long-path workspace words per head slot (at most)
constexpr int kSelectLongHeaderWords = 64;
struct SelectArgs {
  const float* scores;
  int64_t row_stride;
  int32_t* idx;
  int64_t* offsets_dev;
  void* ws;            // workspace of select_workspace_bytes(slots, nchunk) (or the long path's)
  int64_t total;       // offsets[H]
  int S, H;
  int c0, c1;          // candidates are positions [c0, c1)
  int head0, nheads;   // heads [head0, head0 + nheads) in this launch
  int slots, nchunk;   // workspace head slots (>= nheads) and chunks per head
  int64_t out_off[kSelectBatch];
  int32_t n_choose[kSelectBatch];
};
size_t select_workspace_bytes(int slots, int nchunk);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
// The select launches over scores that are the mass pass's output, fed by its
// partial sums part [nsplit][H * S]: the first launch adds the slices (the
// reduction the mass pass would otherwise run) and builds the histograms.
// Requires head0 == 0, nheads == H <= kSelectBatch, row_stride == S, more
// than one chunk a head, at most kSelectMaxCandidates candidates and a head
// that is not trivial; `a.scores` is the mass the launches write and read.
hipError_t launch_select_from_parts(const SelectArgs& a, const float* part, int nsplit, hipStream_t s);
// The select split in two for callers that build the first histograms
// ahead of the budgets: launch_select_hist is the first launch alone (every
// head with n_choose set so that none is skipped), launch_select_hist_reduce
// the first launch of launch_select_from_parts alone, and
// launch_select_prepared the launches after it (the last alone when every
// head is empty or whole). The same conditions as launch_select_from_parts
// apply, except that every head may be trivial.
hipError_t launch_select_hist(const SelectArgs& a, hipStream_t s);
hipError_t launch_select_hist_reduce(const SelectArgs& a, const float* part, int nsplit, hipStream_t s);
hipError_t launch_select_prepared(const SelectArgs& a, hipStream_t s);
size_t select_long_workspace_bytes(int slots);
// Heads per long-path launch for heads of nchunk chunks (0: the device holds fewer).
int select_long_batch_heads(int nchunk);
hipError_t launch_select_long(const SelectArgs& a, hipStream_t s, bool first_batch);

// Row gather of K and V into packed caches.
struct CompactArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_sh, k_ss, v_sh, v_ss;
  const int32_t* idx;
  const int64_t* offsets;
  int64_t total_rows;
  uint16_t* k_new;
  uint16_t* v_new;
  int H, S, d;
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

// Per-head cache regions (H regions with a head stride, rows of d elements):
// append rows at row0, or move rows idx[offsets[h] + r] to row r in place.
struct AppendArgs {
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t ks_sh, ks_ss, vs_sh, vs_ss;
  uint16_t* k;
  uint16_t* v;
  int64_t k_sh, k_ss, v_sh, v_ss;
  int32_t* pos;  // optional [H] rows of pos_sh: pos[row0 + r] = pos0 + r
  int64_t pos_sh;
  int H, n, d, row0, pos0;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

struct InplaceArgs {
  uint16_t* k;
  uint16_t* v;
  int64_t k_sh, k_ss, v_sh, v_ss;
  const int32_t* idx;
  const int64_t* offsets;
  int32_t* pos;  // optional, moved with the rows
  int64_t pos_sh;
  int64_t total; // offsets[H]: kept rows over all heads
  int H, S, d;   // S: rows per head region
  uint32_t* ws;  // ticket counter, error word, then one flag per chunk from word kInplaceFlags0
  int spin_limit;   // polls per flag batch before a chunk gives up (and reports it)
};
constexpr int kInplaceErrorWord = 1;        // chunks whose wait gave up (their rows are not written)
constexpr int kInplaceFlags0 = 32;          // words before the first chunk flag
constexpr int kInplaceSpinLimit = 1 << 22;  // default bound on the polls (waits end long before)
constexpr int kInplaceMinChunkRows = 128;   // rows per chunk at d = 256 (more for smaller d)
inline size_t inplace_workspace_bytes(int64_t total) {
  return 4 * (size_t)(kInplaceFlags0 + (total + kInplaceMinChunkRows - 1) / kInplaceMinChunkRows);
}
hipError_t launch_compact_inplace(const InplaceArgs& a, hipStream_t s);

// Ranking measures: stable per-head order by score, the eviction cost of an
// order summed over budgets, and the overlap of two kept sets.
struct RankArgs {
  const float* scores;
  int64_t row_stride;
  int32_t* order;  // [H, n]
  void* ws;        // rank_workspace_bytes(H, n): two (key, position) buffers, digit counts
  int H, n;
  int ntiles;      // 4096-entry tiles per head
};
inline int rank_tiles(int n) { return (n + 4095) / 4096; }
inline size_t rank_workspace_bytes(int H, int n) {
  return (size_t)16 * H * n + (size_t)4 * H * 256 * rank_tiles(n);
}
hipError_t launch_rank(const RankArgs& a, hipStream_t s);

struct CostArgs {
  const float* importance;
  int64_t row_stride;
  const int32_t* order;  // [H, n]
  double* cost;          // [H]
  double* part;          // [H][cost_blocks(n)] workspace: partial sums per block of entries
  int H, n;
};
constexpr int kCostBlock = 4096;   // entries per workgroup
inline int cost_blocks(int n) { return (n + kCostBlock - 1) / kCostBlock; }
hipError_t launch_cost(const CostArgs& a, hipStream_t s);
// Both rankings' orders into cost.order (scores first, then importance), the
// two costs' block partial sums into cost.part and part_opt, and the ratio.
hipError_t launch_cost_ratio(const RankArgs& rank_scores, const RankArgs& rank_imp, const CostArgs& cost,
                             double* part_opt, double* ratio, hipStream_t s);

struct OverlapArgs {
  const int32_t* idx_a;
  const int64_t* off_a;
  const int32_t* idx_b;
  const int64_t* off_b;
  int64_t* common;  // [H]
  int H, S;
};
constexpr int kOverlapWindow = 1 << 18;  // positions per LDS bitmap (32 KiB)
constexpr int kOverlapMaxS = 1 << 28;    // longer heads take several windows
hipError_t launch_overlap(const OverlapArgs& a, hipStream_t s);

// Running top-k cut-off over static ranks.
struct CutoffArgs {
  const int32_t* order;  // [H, S] positions best first (fam_rank_order)
  int32_t* rank;         // [H, S] workspace: rank of every position
  int32_t* tau;          // [H, S] out
  void* ws;              // wavelet matrix (cutoff_workspace_bytes after rank)
  int H, S, sinks, w, k; // the budget (sinks, window, long-range tokens)
  int L, nw, ntiles;     // levels, words per level (with a terminal word), 1024-position tiles
};
constexpr int kCutoffMaxS = 1 << 20;  // at most 1024 tiles of 1024 positions
constexpr int kCutoffTile = 1024;
// Levels (bits of a rank - 1), words per level and tiles for S positions, and
// the workspace bytes after the ranks: per-tile counts of ones [L][H][ntiles],
// two level sequences [H][S], and (bit word, word count) pairs [H][L][nw].
inline void cutoff_shape(int S, int& L, int& nw, int& ntiles) {
  L = 1;
  while ((1 << L) < S) ++L;
  ntiles = (S + kCutoffTile - 1) / kCutoffTile;
  nw = ntiles * (kCutoffTile / 32) + 1;
}
inline size_t cutoff_workspace_bytes(int H, int S) {
  int L, nw, ntiles;
  cutoff_shape(S, L, nw, ntiles);
  // + 8: slack to align the interleaved (word, count) pairs to 8 bytes
  return 4 * ((size_t)L * H * ntiles + (size_t)2 * H * S + (size_t)2 * H * L * nw) + 8;
}
hipError_t launch_cutoff(const CutoffArgs& a, hipStream_t s);

}  // namespace fam

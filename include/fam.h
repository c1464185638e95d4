/*
 * fam.h -- future-attention mass and budgeted KV-cache eviction on gfx950.
 *
 * C ABI of libfam.so. Every entry point takes plain pointers and sizes.
 * Device pointers are HIP device memory on the current device; `stream` is a
 * hipStream_t passed as void* (NULL means the default stream).
 *
 * Conventions shared by every entry point
 *   - Strides are in elements. The last (head-dim) axis is contiguous.
 *   - The library never allocates or frees device memory and keeps no state
 *     between calls, apart from loaded code objects, a thread-local error
 *     string and two per-device values read once (the address of
 *     evict_select_noalloc's static scratch array, which the code object
 *     holds on every GPU it is loaded on, and the long select path's count
 *     of resident workgroups). The caller owns every other buffer.
 *   - Device entry points only enqueue work on `stream` and return; they do
 *     not synchronise (except under the FAM_SYNC_CHECK debug switch below,
 *     and kv_compact_inplace_status, which exists to wait). Outputs are valid
 *     once the caller has synchronised the stream.
 *   - All arguments are validated before anything is launched. On failure an
 *     entry point returns a non-zero fam_status, launches nothing and leaves
 *     every output untouched; fam_last_error() then describes the failure.
 *   - No C++ exception and no abort crosses this boundary.
 *
 * Debug switches (environment variables, read on every call)
 *   FAM_SYNC_CHECK=1  every device entry point synchronises its stream after
 *                     its launches and reports a fault of the enqueued work
 *                     (FAM_ERR_HIP) or an incomplete in-place compaction
 *                     (FAM_ERR_TIMEOUT) as its own status. Off by default.
 *   FAM_INPLACE_SPIN_LIMIT=n  lowers the bound on the polls of
 *                     kv_compact_inplace's waits (for tests of the timeout
 *                     path; 0 makes every wait give up at once).
 *
 * Sources (titles and sections of the pages this library implements)
 *   [KVpop]  "KVpop - Key-Value Cache Compression with Predictive Online
 *            Pruning" (paperglide summary)
 *   [KVP]    "Learning to Evict from Key-Value Cache" (paperlayer summary)
 *   [LKV]    "LKV: End-to-End Learning of Head-wise Budgets and Token
 *            Selection for LLM KV Cache Eviction" (picx summary)
 *   [Blog]   "How much KV cache can you prune before quality degrades?"
 *            (bilalrana.com)
 */
#ifndef FAM_H
#define FAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAM_OK = 0,
  FAM_ERR_INVALID_ARG = 1, /* a size, stride, pointer or budget is invalid   */
  FAM_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype...) */
  FAM_ERR_WORKSPACE = 3,   /* the workspace is missing or too small          */
  FAM_ERR_HIP = 4,         /* the HIP runtime reported an error at launch    */
  FAM_ERR_TIMEOUT = 5      /* a bounded wait inside a kernel gave up; the
                              outputs of that call are incomplete            */
} fam_status;

typedef enum {
  FAM_BF16 = 0, /* bfloat16 */
  FAM_FP16 = 1  /* IEEE binary16 */
} fam_dtype;

/* Human-readable name of a status code (static storage). */
const char* fam_status_string(fam_status status);

/* Detail of the last failure on the calling thread ("" if none). The pointer
 * stays valid until the next call into the library on this thread. */
const char* fam_last_error(void);

/* ------------------------------------------------------------------------
 * fam_key_norms -- partial maxima of the squared key norms.
 *
 * Not a quantity of the pages: an input of fam_lse's bounded form (below).
 * Per (batch, KV head), the keys are split into P = fam_key_norm_parts(S)
 * consecutive ranges of ceil(S / P) keys and
 *
 *   knorm[b, h, p] = max over keys j of range p of sum_e k[b,h,j,e]^2   (fp32)
 *
 * (0 for an empty range).
 *
 *   k      device, [B, Hkv, S, d] of `dtype`, strides (k_sb, k_sh, k_ss)
 *   knorm  device out, [B, Hkv, P] fp32, contiguous, fully overwritten
 * Requirements and errors as for fam_lse (for the k side).
 * ---------------------------------------------------------------------- */
int fam_key_norm_parts(int S);
fam_status fam_key_norms(const void* k, fam_dtype dtype, int B, int Hkv, int S, int d,
                         int64_t k_sb, int64_t k_sh, int64_t k_ss,
                         float* knorm, void* stream);

/* ------------------------------------------------------------------------
 * fam_lse -- causal row log-sum-exp (first pass).
 *
 * [KVpop] "Delayed Memory Scoring": the normaliser of query i is the log of
 * the sum of exp(logit) over the keys it may attend to; under causal masking
 * these are keys j <= i, the query's own position included.
 *
 *   lse[b, qh, i] = log( sum_{j <= i} exp(scale * <q[b,qh,i,:], k[b,qh/g,j,:]>) )
 *
 * natural log, fp32, with g = Hq / Hkv (query head qh reads KV head qh / g).
 *
 *   q      device, [B, Hq, S, d] of `dtype`, strides (q_sb, q_sh, q_ss)
 *   k      device, [B, Hkv, S, d] of `dtype`, strides (k_sb, k_sh, k_ss)
 *   scale  softmax scale; a value <= 0 selects 1/sqrt(d)
 *   knorm  device, [B, Hkv, fam_key_norm_parts(S)] fp32 from fam_key_norms
 *          on this k, or NULL. With it, each row's exponentials are shifted
 *          by the Cauchy-Schwarz bound scale * |q_i| * max_j |k_j| instead of
 *          a running maximum (faster; a workgroup whose bound is too loose
 *          repeats its rows with the running maximum). The result is the
 *          same up to fp32 rounding.
 *   lse    device out, [B, Hq, S] fp32, contiguous, fully overwritten
 *
 * Requirements: B, Hq, Hkv, S >= 1; Hq % Hkv == 0; d in {64, 128};
 * q and k 16-byte aligned with row strides (q_ss, k_ss) multiples of 8
 * elements and at most 2^24 elements; every stride >= 0 and the tensors
 * addressable with them.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED (d, dtype), FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_lse(const void* q, const void* k, fam_dtype dtype,
                   int B, int Hq, int Hkv, int S, int d,
                   int64_t q_sb, int64_t q_sh, int64_t q_ss,
                   int64_t k_sb, int64_t k_sh, int64_t k_ss,
                   float scale, const float* knorm, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * fam_mass -- per-KV-head future-attention mass (second, key-major pass).
 *
 * [KVpop] "Defining Future Attention Utility" and Figure 2 ("Transposed
 * Attention"): the utility of key j is the attention it receives from queries
 * that arrive after it has left the protected window of W recent tokens,
 * i.e. from queries i >= j + W; transposing queries and keys turns that
 * column sum into a row sum. [KVpop] "Delayed Memory Scoring" and the
 * appendix on the transposed pass: subtract each query's normaliser from its
 * logits. The query heads of a GQA group are summed.
 *
 *   mass[b, h, j] = sum_{qh : qh / g == h} sum_{i = j + W}^{S - 1}
 *                   exp(scale * <q[b,qh,i,:], k[b,h,j,:]> - lse[b,qh,i])
 *
 * Keys j > S - 1 - W get exactly 0. No S x S map is formed.
 *
 *   lse    device, [B, Hq, S] fp32 contiguous (normally fam_lse's output)
 *   W      protected recent window, W >= 0 (W >= S makes every mass 0)
 *   mass   device out, [B, Hkv, S] fp32, contiguous, fully overwritten
 *   workspace, workspace_bytes
 *          optional device scratch (16-byte aligned, owned by the caller,
 *          contents irrelevant on entry and unspecified on return). With
 *          fam_mass_workspace_size(B, Hq, Hkv, S) bytes, each key block's
 *          queries are split over several workgroups whose parts are added
 *          in a fixed order (same result up to fp32 rounding;
 *          deterministic): short sequences split to fill the chip; from
 *          65536 keys on (up to 524288 query rows) every range of 4096
 *          query rows gets its own workgroup per key block, so that
 *          workgroups running together read the same queries. With fewer
 *          bytes the long-sequence ranges give way to the short-sequence
 *          splits, as many as fit; NULL: no splits. Calls sharing a
 *          workspace must be ordered on one stream.
 *   other arguments and requirements as for fam_lse, except that a positive
 *   scale with scale * log2(e) < 2^-100 returns FAM_ERR_UNSUPPORTED (the
 *   pass starts each row's accumulators at -lse / scale in base-2 units;
 *   the same holds for fam_mass_per_head, fam_compute and fam_compute_chunk).
 * ---------------------------------------------------------------------- */
fam_status fam_mass(const void* q, const void* k, const float* lse, fam_dtype dtype,
                    int B, int Hq, int Hkv, int S, int d,
                    int64_t q_sb, int64_t q_sh, int64_t q_ss,
                    int64_t k_sb, int64_t k_sh, int64_t k_ss,
                    int W, float scale, float* mass,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fam_mass uses for these sizes: splits * B * Hkv * S
 * floats (0 when the pass does not split, or for invalid sizes). */
size_t fam_mass_workspace_size(int B, int Hq, int Hkv, int S);

/* ------------------------------------------------------------------------
 * fam_mass_per_head -- the future-attention mass of each query head.
 *
 * [KVpop] "Defining Future Attention Utility" (worked example: the future
 * attention of each query head is kept separately before aggregation) and
 * the appendix on the transposed pass:
 *
 *   mass_q[b, qh, j] = sum_{i = j + W}^{S - 1}
 *                      exp(scale * <q[b,qh,i,:], k[b,qh/g,j,:]> - lse[b,qh,i])
 *
 * so that fam_mass's output is the sum of mass_q over each group. Keys
 * j > S - 1 - W get exactly 0.
 *
 *   mass_q  device out, [B, Hq, S] fp32, contiguous, fully overwritten
 *   workspace, workspace_bytes
 *           optional device scratch (16-byte aligned, owned by the caller,
 *           contents irrelevant on entry and unspecified on return). With
 *           fam_mass_per_head_workspace_size(B, Hq, Hkv, S) bytes (non-zero
 *           from 65536 keys on), every range of 4096 query rows gets its own
 *           workgroup per key block, as in fam_mass, and a second launch
 *           adds the ranges' parts in a fixed order (same result up to fp32
 *           rounding; deterministic). NULL or fewer bytes: no split. Calls
 *           sharing a workspace must be ordered on one stream.
 *   other arguments, requirements and errors as for fam_mass.
 * ---------------------------------------------------------------------- */
fam_status fam_mass_per_head(const void* q, const void* k, const float* lse, fam_dtype dtype,
                             int B, int Hq, int Hkv, int S, int d,
                             int64_t q_sb, int64_t q_sh, int64_t q_ss,
                             int64_t k_sb, int64_t k_sh, int64_t k_ss,
                             int W, float scale, float* mass_q,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fam_mass_per_head uses for these sizes: ranges * B * Hq
 * * S floats (0 when it does not split, or for invalid sizes). */
size_t fam_mass_per_head_workspace_size(int B, int Hq, int Hkv, int S);

/* ------------------------------------------------------------------------
 * fam_kvpop_target -- KVpop's supervision target from per-head mass.
 *
 * [KVpop] "Defining Future Attention Utility" (count normalisation and the
 * log of the mean future mass, max over the query heads of a KV head) and
 * the appendix "Alternative Aggregation Methods" (mean in probability space
 * before the log). With N_j = max(1, S - (j + W)) and g = Hq / Hkv:
 *
 *   FAM_AGG_MAX:  target[b,h,j] = max_{qh in group h} log(eps + mass_q[b,qh,j] / N_j)
 *   FAM_AGG_MEAN: target[b,h,j] = log(eps + (sum_{qh in group h} mass_q[b,qh,j]) / (g N_j))
 *
 * With eps = 0 a key with zero mass gets -inf.
 *
 *   mass_q  device, [B, Hq, S] fp32 contiguous (normally fam_mass_per_head's)
 *   W       protected window (>= 0), as used for mass_q
 *   eps     >= 0, finite
 *   target  device out, [B, Hkv, S] fp32, contiguous, fully overwritten
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
typedef enum { FAM_AGG_MAX = 0, FAM_AGG_MEAN = 1 } fam_aggregate;
fam_status fam_kvpop_target(const float* mass_q, int B, int Hq, int Hkv, int S, int W, float eps,
                            fam_aggregate aggregate, float* target, void* stream);

/* fam_compute -- fam_key_norms, fam_lse (bounded form) and fam_mass on the
 * same stream. The key-norm partial maxima are kept in the first entries of
 * `mass` until the mass pass overwrites it. The optional workspace (16-byte
 * aligned, caller-owned, contents irrelevant on entry and unspecified on
 * return) serves both passes in turn: when the query rows are too few to fill
 * the chip, the first pass splits every row's key range over several
 * workgroups, adds their partial sums in a fixed order and repeats the sweep
 * with the running maximum for any workgroup whose bound came out loose; the
 * mass pass then splits as in fam_mass. fam_compute_workspace_size gives the
 * bytes for all splits; fewer bytes (or NULL) mean fewer (or no) splits, with
 * the same results up to fp32 rounding. */
fam_status fam_compute(const void* q, const void* k, fam_dtype dtype,
                       int B, int Hq, int Hkv, int S, int d,
                       int64_t q_sb, int64_t q_sh, int64_t q_ss,
                       int64_t k_sb, int64_t k_sh, int64_t k_ss,
                       int W, float scale, float* lse, float* mass,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * fam_compute_chunk -- the scores of one chunk of a chunked prefill over a
 * cache that already holds (a compacted subset of) the earlier keys.
 *
 * [KVP] section 4 ("Evaluation") and 4.1: long contexts are prefilled chunk
 * by chunk and the cache is compressed after each chunk to the budget, with
 * physical compaction. [KVpop] "Delayed Memory Scoring": the normalisers are
 * those of the sparse (retained-key) attention the model actually runs, and
 * the target is the mass a key receives from queries at least W positions
 * later.
 *
 * The Sk keys k[b, h, 0 .. Sk-1] are the cache rows and the Sq queries are
 * the last Sq of them: query row r sits at cache row Sk - Sq + r. Causality
 * and the window are taken in that row order:
 *
 *   lse[b, qh, r]  = log sum_{j <= Sk - Sq + r} exp(scale <q[b,qh,r,:], k[b,qh/g,j,:]>)
 *   mass[b, h, j]  = sum_{qh in group h} sum_{r : Sk - Sq + r >= j + W}
 *                    exp(scale <q[b,qh,r,:], k[b,h,j,:]> - lse[b,qh,r])
 *
 * For a compacted cache this equals the same sums taken over original
 * positions whenever the last W rows before the chunk hold the W positions
 * just before it (the recent window that every compression keeps; any
 * cache that was never compressed qualifies): the chunk's keys are its own
 * last Sq rows, every earlier row lies before the chunk, and only the
 * window rows can be less than W positions before a chunk query. With
 * Sq == Sk this is fam_compute.
 *
 *   q     device, [B, Hq, Sq, d], strides (q_sb, q_sh, q_ss): the chunk's queries
 *   k     device, [B, Hkv, Sk, d], strides (k_sb, k_sh, k_ss): the cache rows,
 *         the chunk's own keys last
 *   lse   device out, [B, Hq, Sq] fp32, contiguous, fully overwritten
 *   mass  device out, [B, Hkv, Sk] fp32, contiguous, fully overwritten
 *         (rows j > Sk - 1 - W get exactly 0)
 *   workspace  as for fam_compute, sized fam_compute_workspace_size(B, Hq, Hkv, Sq, Sk)
 * Requirements: 1 <= Sq <= Sk; otherwise as for fam_compute.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_compute_chunk(const void* q, const void* k, fam_dtype dtype,
                             int B, int Hq, int Hkv, int Sq, int Sk, int d,
                             int64_t q_sb, int64_t q_sh, int64_t q_ss,
                             int64_t k_sb, int64_t k_sh, int64_t k_ss,
                             int W, float scale, float* lse, float* mass,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fam_compute (Sq == Sk == S) and fam_compute_chunk use
 * for these sizes: the larger of the first pass's split partial sums
 * ((splits + 1) floats per query row) and the mass pass's split parts
 * (splits * B * Hkv * Sk floats, the splits chosen for Sq query rows as in
 * fam_mass). 0 when neither pass splits, or for invalid sizes. */
size_t fam_compute_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk);

/* ------------------------------------------------------------------------
 * evict_plan -- host-only budget plan (no device work).
 *
 * [KVpop] "The KVpop Scoring Module" / Figure 1: the sinks and the recent
 * window are always kept and the rest of the per-head budget goes to the
 * best-scored long-range tokens; [KVP] A.2 and [Blog] "What we did" keep
 * the first and the newest tokens the same way.
 *
 * The forced set is F = [0, min(sinks, S)) U [max(0, S - recent), S). A
 * budget is the total number of rows a head keeps, forced rows included:
 *   kept[h]    = min(S, max(budgets[h], |F|))
 *   offsets[0] = 0, offsets[h + 1] = offsets[h] + kept[h]
 *
 *   budgets  host, [H] int64, each >= 0
 *   kept     host out, [H] int64 (may be NULL)
 *   offsets  host out, [H + 1] int64 (may be NULL)
 * Errors: FAM_ERR_INVALID_ARG (H < 0, S < 1, sinks/recent < 0, a negative
 * budget, budgets NULL with H > 0).
 * ---------------------------------------------------------------------- */
fam_status evict_plan(int H, int S, const int64_t* budgets, int sinks, int recent,
                      int64_t* kept, int64_t* offsets);

/* ------------------------------------------------------------------------
 * fam_soft_topk -- host-only, LKV's closed-form Soft-TopK (fp64).
 *
 * [LKV] "The Differentiable Soft-TopK Operator": ST_k(x; tau) has entries in
 * (0, 1) that sum to k, keeps the order of x and ignores a constant shift;
 * the page prints its threshold lambda in closed form. The mask is read as
 * the Laplace CDF of x_i / tau - lambda (1 - e^-u / 2 for u >= 0, e^u / 2
 * below), which makes the printed lambda exactly the root that sums to k.
 * [LKV] "LKV-H: Learning Global Budget Allocation": a model's per-head
 * retention ratios are ST of the flattened head scores with k = the mean
 * ratio times the number of heads; fam_budgets_from_ratios then floors
 * r * t.
 *
 *   x    host, [n] finite scores;  out  host out, [n] fp64 masks
 *   k    0 < k < n;  tau > 0 (finite)
 * Errors: FAM_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
fam_status fam_soft_topk(const double* x, int n, double k, double tau, double* out);

/* ------------------------------------------------------------------------
 * fam_budgets_from_ratios -- host-only, b[h] = floor(ratios[h] * t).
 *
 * [LKV] "LKV-H: Learning Global Budget Allocation": a head's discrete budget
 * at length t is the floor of its frozen retention ratio times t. The
 * product is formed in double precision.
 *   ratios   host, [H] double, each finite and >= 0
 *   budgets  host out, [H] int64
 * Errors: FAM_ERR_INVALID_ARG (negative or non-finite ratio, overflow).
 * ---------------------------------------------------------------------- */
fam_status fam_budgets_from_ratios(int H, const double* ratios, int64_t t, int64_t* budgets);

/* ------------------------------------------------------------------------
 * evict_select -- per-head top-k selection with forced sinks and window.
 *
 * [KVP] section 3: the top-b entries of a ranking form the cache and the
 * lowest-ranked entries are evicted. [KVpop] "The KVpop Scoring Module":
 * sinks + window + top-k of the remaining tokens. Among the candidates
 * C = [min(sinks,S), max(min(sinks,S), S - recent)) the kept[h] - |F|
 * best are chosen by score descending; equal scores go to the lower
 * position; -0.0 equals +0.0; NaN ranks below every number.
 *
 *   scores      device, [H, S] fp32, row stride `score_row_stride` (>= S when
 *               H > 1)
 *   budgets     host, [H] int64 (as for evict_plan)
 *   idx         device out, [offsets[H]] int32: for each head h, the kept
 *               positions in ascending order at idx[offsets[h] ...]
 *   offsets_dev device out, [H + 1] int64: the offsets of evict_plan
 *   workspace   device scratch of at least
 *               evict_select_workspace_size(H, S, sinks, recent) bytes,
 *               16-byte aligned, owned by the caller; its contents on entry
 *               do not matter and on return are unspecified. Calls that
 *               share a workspace must be ordered on one stream.
 *
 * Requirements: H >= 0, 1 <= S; every head's candidate count (S minus the
 * forced rows) at most 2^20 (up to 131072 in three launches over chunks of
 * 4096 candidates; beyond, one round-based launch after a fill, which waits
 * across its workgroups and sizes each launch to the workgroups the device
 * holds at once). H == 0 is a no-op (nothing is written).
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED (too many candidates),
 * FAM_ERR_WORKSPACE (missing or too small workspace), FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status evict_select(const float* scores, int64_t score_row_stride, int H, int S,
                        const int64_t* budgets, int sinks, int recent,
                        int32_t* idx, int64_t* offsets_dev,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace evict_select needs for these sizes (host-only;
 * 0 for invalid sizes). */
size_t evict_select_workspace_size(int H, int S, int sinks, int recent);

/* ------------------------------------------------------------------------
 * fam_mass_select -- fam_mass, then evict_select on its output.
 *
 * [KVpop] "Defining Future Attention Utility" (the mass of each key) and
 * "The KVpop Scoring Module" / Figure 1 (sinks + window + the best-scored
 * rest): the budgeted selection runs on the masses just computed. The
 * results are those of
 *
 *   fam_mass(q, k, lse, ..., W, scale, mass, mass_workspace, ...);
 *   evict_select(mass, S, B * Hkv, S, budgets, sinks, recent, idx,
 *                offsets_dev, select_workspace, ...);
 *
 * bit for bit (mass, idx and offsets_dev), with one launch fewer when the
 * mass pass splits (a mass_workspace of fam_mass_workspace_size bytes), the
 * heads B * Hkv number at most 64, each head has at most 131072 candidates
 * in more than one chunk of 4096, and some head keeps part of its
 * candidates: the launch that adds the mass pass's partial sums then also
 * builds the selection's first histograms, from the sums in registers.
 * Otherwise the two calls run one after the other.
 *
 *   arguments as for fam_mass (q ... mass_workspace_bytes) and for
 *   evict_select (budgets ... select_workspace_bytes), with H = B * Hkv
 *   heads of S scores (the mass rows); mass, idx, offsets_dev and the two
 *   workspaces must not overlap (overlapping workspaces are refused).
 * Errors: those of fam_mass and evict_select; nothing is launched when an
 * argument is refused.
 * ---------------------------------------------------------------------- */
fam_status fam_mass_select(const void* q, const void* k, const float* lse, fam_dtype dtype,
                           int B, int Hq, int Hkv, int S, int d,
                           int64_t q_sb, int64_t q_sh, int64_t q_ss,
                           int64_t k_sb, int64_t k_sh, int64_t k_ss,
                           int W, float scale, float* mass,
                           void* mass_workspace, size_t mass_workspace_bytes,
                           const int64_t* budgets, int sinks, int recent,
                           int32_t* idx, int64_t* offsets_dev,
                           void* select_workspace, size_t select_workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * evict_select_prepare / evict_select_prepared / fam_mass_prepare_select --
 * evict_select split at the part that does not depend on the budgets.
 *
 * [KVP] section 3 (the cache holds the top b of one ranking, for every
 * budget b) and [Blog] "What we did" (one score set evicted at several cache
 * budgets): the selection's first histograms depend only on the scores, so
 * they can be built once, ahead of the budgets, and serve every later
 * selection on the same scores.
 *
 *   evict_select_prepare(scores, row_stride, H, S, sinks, recent,
 *                        workspace, ...)
 *       builds those histograms in `workspace` (evict_select's workspace of
 *       evict_select_workspace_size(H, S, sinks, recent) bytes);
 *   fam_mass_prepare_select(<fam_mass's arguments>, sinks, recent,
 *                           select_workspace, ...)
 *       is fam_mass (same mass, bit for bit) that also builds them for its
 *       own output, in the launch that adds the mass pass's partial sums
 *       when the pass splits (a mass_workspace of fam_mass_workspace_size
 *       bytes), so without a launch of their own;
 *   evict_select_prepared(<evict_select's arguments>)
 *       is evict_select (same idx and offsets_dev, bit for bit) without the
 *       histogram launch, on a workspace that one of the two calls above
 *       prepared for these scores, H, S, sinks and recent, and that nothing
 *       has written since; it may be called any number of times, with any
 *       budgets.
 * The split applies when there are H <= 64 heads whose at most 131072
 * candidates span more than one chunk of 4096 positions (chunks start at the
 * first candidate rounded down to a multiple of 4); for other sizes the
 * preparing calls build nothing
 * (fam_mass_prepare_select is then fam_mass) and evict_select_prepared is
 * evict_select. A workspace not prepared for these scores gives an
 * unspecified selection.
 *
 * Arguments: as for evict_select, fam_mass and fam_mass_select; the select
 *   workspace must not overlap the mass workspace (refused).
 * Errors: those of evict_select and fam_mass; nothing is launched when an
 *   argument is refused.
 * ---------------------------------------------------------------------- */
fam_status evict_select_prepare(const float* scores, int64_t score_row_stride, int H, int S,
                                int sinks, int recent, void* workspace, size_t workspace_bytes,
                                void* stream);

fam_status evict_select_prepared(const float* scores, int64_t score_row_stride, int H, int S,
                                 const int64_t* budgets, int sinks, int recent,
                                 int32_t* idx, int64_t* offsets_dev,
                                 void* workspace, size_t workspace_bytes, void* stream);

fam_status fam_mass_prepare_select(const void* q, const void* k, const float* lse, fam_dtype dtype,
                                   int B, int Hq, int Hkv, int S, int d,
                                   int64_t q_sb, int64_t q_sh, int64_t q_ss,
                                   int64_t k_sb, int64_t k_sh, int64_t k_ss,
                                   int W, float scale, float* mass,
                                   void* mass_workspace, size_t mass_workspace_bytes,
                                   int sinks, int recent,
                                   void* select_workspace, size_t select_workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * evict_select_noalloc -- evict_select for callers that cannot allocate.
 *
 * For callers that may not allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same selection, with the same results bit for bit, as evict_select,
 * whose workspace here is a static device array of
 * FAM_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU holds from the library's
 * first use on it until the process ends. The call allocates nothing and
 * calls no allocating routine; the caller still passes every input and
 * output. Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams without ordering) race and give
 * unspecified results; calls ordered on one stream are safe. What must
 * start cleared is cleared by the call's own kernels. On its first call on
 * a device the library looks up and keeps the array's address there (with
 * a per-device occupancy figure, the only state it keeps besides the error
 * string).
 *
 * Arguments, outputs and errors as evict_select, without the workspace;
 * FAM_ERR_UNSUPPORTED when evict_select_workspace_size(H, S, sinks, recent)
 * exceeds FAM_NOALLOC_SCRATCH_BYTES (e.g. 64 heads of 131072 candidates;
 * 8 such heads, 56 heads of 120000, and heads beyond 131072 candidates fit).
 * ---------------------------------------------------------------------- */
#define FAM_NOALLOC_SCRATCH_BYTES (64u << 20)
fam_status evict_select_noalloc(const float* scores, int64_t score_row_stride, int H, int S,
                                const int64_t* budgets, int sinks, int recent,
                                int32_t* idx, int64_t* offsets_dev, void* stream);

/* ------------------------------------------------------------------------
 * kv_compact -- gather kept K and V rows into a new packed cache.
 *
 * [KVP] section 4.1 and A.2 (physical tensor compaction) and [Blog]
 * "What we did" (the retained entries are copied into a new cache tensor).
 *
 *   k_new[r, :] = k[h, idx[r], :],  v_new[r, :] = v[h, idx[r], :]
 *   for offsets_dev[h] <= r < offsets_dev[h + 1]; a bit copy.
 *
 *   k, v         device, [H, S, d] of `elem_bytes`-byte elements, strides
 *                (k_sh, k_ss) and (v_sh, v_ss) in elements
 *   idx          device, [total_rows] int32, normally evict_select's output
 *   offsets_dev  device, [H + 1] int64, non-decreasing, offsets_dev[0] = 0,
 *                offsets_dev[H] = total_rows
 *   k_new, v_new device out, [total_rows, d] contiguous
 *
 * Requirements: elem_bytes == 2; d * 2 a multiple of 16; k, v, k_new, v_new
 * 16-byte aligned; row strides multiples of 8 elements. An index outside
 * [0, S) yields a zero row instead of a read out of bounds.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status kv_compact(const void* k, const void* v, int elem_bytes, int H, int S, int d,
                      int64_t k_sh, int64_t k_ss, int64_t v_sh, int64_t v_ss,
                      const int32_t* idx, const int64_t* offsets_dev, int64_t total_rows,
                      void* k_new, void* v_new, void* stream);

/* ------------------------------------------------------------------------
 * kv_append -- copy a chunk's K and V rows into per-head cache regions.
 *
 * [KVP] section 4 (chunked prefill) and [Blog] conclusion (a static cache
 * reserves a fixed region per head): the chunk's rows follow the rows the
 * cache already holds.
 *
 *   k_cache[h, row0 + r, :] = k_src[h, r, :],  v_cache likewise,
 *   pos[h * pos_sh + row0 + r] = pos0 + r      (when pos is not NULL)
 *   for 0 <= h < H, 0 <= r < n; a bit copy.
 *
 *   k_src, v_src      device, [H, n, d], strides (ks_sh, ks_ss), (vs_sh, vs_ss)
 *   k_cache, v_cache  device in/out, [H, capacity, d], strides (kc_sh, kc_ss),
 *                     (vc_sh, vc_ss); only rows row0 .. row0+n-1 are written
 *   pos               optional device in/out int32, head stride pos_sh >= capacity
 * Requirements: elem_bytes == 2; d in {64, 128, 256}; row0 + n <= capacity;
 * H <= 65535; pointers 16-byte aligned (pos 4-byte); strides multiples of 8
 * elements. Source and cache rows must not overlap.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status kv_append(const void* k_src, const void* v_src, int elem_bytes, int H, int n, int d,
                     int64_t ks_sh, int64_t ks_ss, int64_t vs_sh, int64_t vs_ss,
                     void* k_cache, void* v_cache, int64_t kc_sh, int64_t kc_ss,
                     int64_t vc_sh, int64_t vc_ss, int capacity, int row0,
                     int32_t* pos, int64_t pos_sh, int pos0, void* stream);

/* ------------------------------------------------------------------------
 * kv_compact_inplace -- keep the selected rows of each head's cache region,
 * moved to its first rows, without a second cache.
 *
 * [Blog] conclusion (a ring or static cache can overwrite old entries in
 * place instead of copying into a new tensor) and [KVP] 4.1 (physical
 * compaction).
 *
 *   for each head h and 0 <= r < n_h = offsets_dev[h + 1] - offsets_dev[h]:
 *     row r of head h  <-  row idx[offsets_dev[h] + r] of head h (K, V, pos)
 *
 * Rows n_h and beyond keep stale contents. The rows of a head must be
 * ascending (as evict_select writes them); then idx[...+r] >= r, and the
 * kept rows are moved in chunks, each written only after the chunks that
 * read its rows have loaded them (no grid-wide barrier, no cooperative
 * launch). Unsorted indices give unspecified row contents (never an access
 * out of bounds, never a wait that does not end); an index outside [0, S)
 * yields a zero row and position -1; rows r >= S (offsets that do not fit
 * the region) are skipped.
 *
 *   k, v         device in/out, [H, S, d], strides (k_sh, k_ss), (v_sh, v_ss)
 *   idx          device, [total_rows] int32 (evict_select's output)
 *   offsets_dev  device, [H + 1] int64, non-decreasing, offsets_dev[0] = 0,
 *                offsets_dev[H] = total_rows
 *   total_rows   host copy of offsets_dev[H], <= H * S
 *   pos          optional device in/out int32 [H, S] with head stride pos_sh,
 *                moved with the rows
 *   workspace    device scratch of kv_compact_inplace_workspace_size(total_rows)
 *                bytes (4-byte aligned, caller-owned, contents irrelevant on
 *                entry and unspecified on return): the chunk tickets and
 *                flags, cleared by the call itself. Calls sharing a
 *                workspace must be ordered on one stream.
 * Requirements: elem_bytes == 2; d in {64, 128, 256}; k, v 16-byte aligned;
 * strides multiples of 8 elements; pos 4-byte aligned with pos_sh >= S.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_WORKSPACE,
 * FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status kv_compact_inplace(void* k, void* v, int elem_bytes, int H, int S, int d,
                              int64_t k_sh, int64_t k_ss, int64_t v_sh, int64_t v_ss,
                              const int32_t* idx, const int64_t* offsets_dev,
                              int64_t total_rows, int32_t* pos, int64_t pos_sh,
                              void* workspace, size_t workspace_bytes, void* stream);

/* kv_compact_inplace_status -- whether the last kv_compact_inplace on this
 * workspace moved every row. Waits for `stream` (the one the compaction was
 * enqueued on) and reads the workspace's error word: FAM_OK, or
 * FAM_ERR_TIMEOUT if a chunk's bounded wait for the chunks reading its rows
 * gave up, in which case that chunk's rows were left unwritten (the other
 * chunks are complete). The only synchronising call of the library. */
fam_status kv_compact_inplace_status(const void* workspace, void* stream);

/* Bytes of workspace kv_compact_inplace needs for total_rows kept rows (about
 * one byte per 32 rows; 0 for total_rows < 0). */
size_t kv_compact_inplace_workspace_size(int64_t total_rows);

/* ------------------------------------------------------------------------
 * fam_rank_order -- each head's entries ordered best first.
 *
 * [KVP] section 3: a ranking's top-b entries form the cache for every budget
 * b. The order is by score descending; ties go to the lower position, -0.0
 * equals +0.0 and NaN ranks below every number (NaNs by position), as in
 * evict_select.
 *
 *   order[h * n + r] = position (0 .. n-1) of the r-th best entry of row h
 *
 *   scores     device, [H] rows of n fp32 with row stride row_stride (>= n
 *              when H > 1)
 *   order      device out, [H, n] int32, fully overwritten
 *   workspace  device scratch of fam_rank_order_workspace_size(H, n) bytes
 *              (16 * H * n, plus 1 KiB per head and 4096 entries for digit
 *              counts), 8-byte aligned, owned by the caller; contents
 *              irrelevant on entry and unspecified on return
 * A stable radix sort, 4 passes of 3 launches over 4096-entry tiles.
 * Requirements: H <= 65535.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED (n > 2^28),
 * FAM_ERR_WORKSPACE, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_rank_order(const float* scores, int64_t row_stride, int H, int n, int32_t* order,
                          void* workspace, size_t workspace_bytes, void* stream);
size_t fam_rank_order_workspace_size(int H, int n);

/* ------------------------------------------------------------------------
 * fam_eviction_cost -- the importance a ranking evicts, summed over budgets.
 *
 * [KVP] 3.1.1: a ranking is scored by the future-attention importance of the
 * entries it evicts across cache budgets (a cost-versus-budget area under
 * the curve), normalised by the same area of the optimal ranking (the order
 * of the importance itself). With order from fam_rank_order:
 *
 *   cost[h] = sum_{b=0}^{n} sum_{r >= b} importance[h, order[h, r]]
 *           = sum_r (r + 1) * importance[h, order[h, r]]
 *
 * and the normalised cost is cost / cost_optimal, where cost_optimal uses
 * the order of importance (it is >= 1 for non-negative importance and
 * equals 1 exactly for an optimal order).
 *
 *   importance  device, [H] rows of n fp32, row stride row_stride (>= n when
 *               H > 1)
 *   order       device, [H, n] int32 (entries outside [0, n) are skipped)
 *   cost        device out, [H] fp64 (sums in fp64, fixed order: per block
 *               of 4096 entries, then the blocks in order)
 *   workspace   device scratch of fam_eviction_cost_workspace_size(H, n)
 *               bytes (one fp64 partial sum per head and block), 8-byte
 *               aligned, owned by the caller; may be NULL when that is 0
 * Requirements: H <= 65535.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_WORKSPACE,
 * FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_eviction_cost(const float* importance, int64_t row_stride, const int32_t* order,
                             int H, int n, double* cost, void* workspace, size_t workspace_bytes,
                             void* stream);
size_t fam_eviction_cost_workspace_size(int H, int n);

/* ------------------------------------------------------------------------
 * fam_eviction_cost_ratio -- KVP's normalised eviction cost of a scorer.
 *
 * [KVP] 3.1.1: the cost-versus-budget area of the importance a ranking
 * evicts, normalised by the cost of the optimal ranking. Per head h:
 *
 *   ratio[h] = cost(importance, order of scores) / cost(importance, order
 *              of importance)
 *
 * with cost and order exactly as fam_eviction_cost and fam_rank_order
 * define them (the two costs are bit-identical to what those calls return).
 * The ratio is >= 1 for non-negative importance and 1 for an optimal
 * order. Where both costs are 0 (no importance anywhere) the ratio is 1:
 * every ranking is optimal; otherwise it is the plain IEEE quotient (so a
 * zero optimal cost against a non-zero cost, possible only with negative
 * importance, gives an infinity).
 *
 *   scores      device, [H] rows of n fp32 (the scorer), row stride
 *               scores_row_stride (>= n when H > 1)
 *   importance  device, [H] rows of n fp32 (e.g. future-attention mass),
 *               row stride importance_row_stride (>= n when H > 1)
 *   ratio       device out, [H] fp64
 *   workspace   device scratch of fam_eviction_cost_ratio_workspace_size(H,
 *               n) bytes (rank-order scratch, one order [H, n] int32 and two
 *               sets of per-block partial sums), 8-byte aligned, owned by the
 *               caller; contents irrelevant on entry
 * Requirements: H <= 65535.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_WORKSPACE,
 * FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_eviction_cost_ratio(const float* scores, int64_t scores_row_stride, const float* importance,
                                   int64_t importance_row_stride, int H, int n, double* ratio,
                                   void* workspace, size_t workspace_bytes, void* stream);
size_t fam_eviction_cost_ratio_workspace_size(int H, int n);

/* ------------------------------------------------------------------------
 * fam_retention_overlap -- entries two kept sets share, per head.
 *
 * [KVpop] Figure 7: top-k retention recall is the fraction of the teacher's
 * kept set (the top of the future-attention mass) that another scorer also
 * keeps under the same budget. With kept lists a (the teacher's) and b:
 *
 *   common[h] = | {idx_a[offsets_a[h] ..]} & {idx_b[offsets_b[h] ..]} |
 *
 * and the recall of head h is common[h] / |set of a_h|. Duplicates count
 * once; indices outside [0, S) are ignored.
 *
 *   idx_a, idx_b          device int32 kept positions (e.g. evict_select's)
 *   offsets_a, offsets_b  device [H + 1] int64, non-decreasing
 *   common                device out, [H] int64
 * Requirements: S <= 2^28 (a bitmap of 262144 positions in LDS per pass;
 * longer heads take one pass per 262144 positions).
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_retention_overlap(const int32_t* idx_a, const int64_t* offsets_a,
                                 const int32_t* idx_b, const int64_t* offsets_b, int H, int S,
                                 int64_t* common, void* stream);

/* ------------------------------------------------------------------------
 * fam_topk_cutoff -- the running top-k cut-off of a sparse prefill mask.
 *
 * [KVpop] "Delayed Memory Scoring", "Efficient Online Pruning" and
 * Algorithm 2 (running top-k cutoff computation for one KV head): tokens
 * are pre-sorted by a static priority score (rank 1 = best); the budget is
 * (s, w, k); at query q the token t = q - w leaves the protected window and
 * becomes eligible if it is not a sink (t >= s); tau_q starts at -1 and,
 * once at least k tokens are eligible, is the rank of the k-th best
 * eligible token. The attention then keeps the sinks, the window and the
 * eligible tokens with rank <= tau_q. The page finds tau_q with a Fenwick
 * tree, one insertion per query; this answers every query independently
 * from a wavelet matrix of the per-position ranks (tau_q is the k-th
 * smallest value of a range of that sequence).
 *
 *   E(q)      = positions t with sinks <= t <= q - w
 *   tau[h, q] = -1 if |E(q)| < k; otherwise 0 if k == 0, else the k-th
 *               smallest rank among the positions in E(q) of head h
 *
 *   order      device, [H, S] int32 positions best first (fam_rank_order's
 *              output: every position exactly once; any other content gives
 *              unspecified cut-offs, never an access out of bounds)
 *   sinks, w, k  the budget: sink tokens, window, long-range tokens
 *   tau        device out, [H, S] int32, fully overwritten
 *   workspace  device scratch of fam_topk_cutoff_workspace_size(H, S) bytes
 *              (the ranks, two level sequences, the bit words and counts
 *              of ceil(log2 S) levels and per-tile counts of ones: about 16
 *              bytes per entry at S = 131072), 4-byte aligned, owned by the
 *              caller, contents irrelevant on entry
 * Requirements: S <= 1048576; H <= 65535; sinks, w, k >= 0.
 * Errors: FAM_ERR_INVALID_ARG, FAM_ERR_UNSUPPORTED, FAM_ERR_WORKSPACE,
 * FAM_ERR_HIP.
 * ---------------------------------------------------------------------- */
fam_status fam_topk_cutoff(const int32_t* order, int H, int S, int sinks, int w, int k, int32_t* tau,
                           void* workspace, size_t workspace_bytes, void* stream);
size_t fam_topk_cutoff_workspace_size(int H, int S);

#ifdef __cplusplus
}
#endif

#endif /* FAM_H */

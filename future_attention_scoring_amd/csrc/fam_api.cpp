// C ABI of libfam.so: argument validation, the host-side budget plan and
// kernel dispatch. Nothing here allocates device memory; nothing synchronises
// except the FAM_SYNC_CHECK debug switch and kv_compact_inplace_status.
#include "fam.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fam_kernels.hpp"

namespace {

thread_local std::string g_error;

fam_status fail(fam_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

fam_status ok() {
  g_error.clear();
  return FAM_OK;
}

fam_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FAM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// FAM_SYNC_CHECK (debug switch, read on every call): set to anything but
// "" or "0", every device entry point synchronises its stream after its
// launches, so that a fault in the work it enqueued is reported by that call.
bool sync_check() {
  const char* v = std::getenv("FAM_SYNC_CHECK");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

// The status of a call whose launches returned e: under FAM_SYNC_CHECK also
// the outcome of the enqueued work.
fam_status launched(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess || !sync_check()) return hip_status(e, what);
  e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(FAM_ERR_HIP, "%s (sync check): %s", what, hipGetErrorString(e));
  return ok();
}

// The bits of an enum argument as an int: a C caller may pass any value, and
// loading an out-of-range value as the C++ enum type would be undefined.
template <typename E>
int enum_bits(const E* e) {
  static_assert(sizeof(E) == sizeof(int), "enums of the ABI are int-sized");
  int v;
  std::memcpy(&v, e, sizeof v);
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxSeq = 1 << 28;
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

// S keys; Sq query rows at the last Sq positions (Sq = 0 stands for Sq = S).
struct ScoreShape {
  int B, Hq, Hkv, S, d;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss;
  int Sq;
  int rows() const { return Sq > 0 ? Sq : S; }
};

fam_status check_scores(const void* q, const void* k, int dtype, const ScoreShape& s) {
  if (!q || !k) return fail(FAM_ERR_INVALID_ARG, "q and k must be non-null");
  if (dtype != FAM_BF16 && dtype != FAM_FP16)
    return fail(FAM_ERR_UNSUPPORTED, "dtype %d is not bf16 or fp16", dtype);
  if (s.B < 1 || s.Hq < 1 || s.Hkv < 1 || s.S < 1)
    return fail(FAM_ERR_INVALID_ARG, "B, Hq, Hkv and S must be >= 1 (got %d, %d, %d, %d)",
                s.B, s.Hq, s.Hkv, s.S);
  if (s.S > kMaxSeq) return fail(FAM_ERR_UNSUPPORTED, "S = %d exceeds %d", s.S, kMaxSeq);
  if (s.Sq < 0 || s.Sq > s.S)
    return fail(FAM_ERR_INVALID_ARG, "query rows Sq = %d must be in [1, Sk = %d]", s.Sq, s.S);
  if (s.Hq % s.Hkv != 0)
    return fail(FAM_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", s.Hq, s.Hkv);
  if (s.d != 64 && s.d != 128) return fail(FAM_ERR_UNSUPPORTED, "head dim %d (need 64 or 128)", s.d);
  const int64_t st[6] = {s.q_sb, s.q_sh, s.q_ss, s.k_sb, s.k_sh, s.k_ss};
  for (int i = 0; i < 6; ++i) {
    if (st[i] < 0) return fail(FAM_ERR_INVALID_ARG, "strides must be >= 0");
    if (st[i] % 8 != 0)
      return fail(FAM_ERR_INVALID_ARG, "strides must be multiples of 8 elements (16 bytes)");
  }
  if (!aligned16(q) || !aligned16(k)) return fail(FAM_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  // the kernels address a 64-row tile with 32-bit offsets
  if (s.q_ss > kMaxRowStride || s.k_ss > kMaxRowStride)
    return fail(FAM_ERR_UNSUPPORTED, "row strides above %lld elements", (long long)kMaxRowStride);
  return FAM_OK;
}

float resolve_scale(float scale, int d) {
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)d);
  return (float)(sc * 1.4426950408889634);  // base-2 logits inside the kernels
}

// Arguments of the first pass and of the key-norm pass; with `knorm` non-null
// the row shift is the Cauchy-Schwarz bound built from the key-norm partial
// maxima stored there ([B * Hkv][nkn] floats).
// The mass pass starts its accumulators at -L/c (c = scale * log2 e); below
// c = 2^-100 that quotient could overflow. Such a scale is refused by every
// entry point that runs the mass pass.
fam_status check_mass_scale(float scale, int d) {
  if (!std::isfinite(scale)) return fail(FAM_ERR_INVALID_ARG, "scale must be finite");
  const float c = resolve_scale(scale, d);
  if (!(c >= 0x1p-100f))
    return fail(FAM_ERR_UNSUPPORTED, "scale %g is below what the mass pass supports (scale * log2(e) >= 2^-100)",
                (double)scale);
  return FAM_OK;
}

fam::LseArgs lse_args(const void* q, const void* k, const ScoreShape& s, float scale, float* lse,
                      float* knorm) {
  fam::LseArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.lse = lse;
  a.q_sb = s.q_sb, a.q_sh = s.q_sh, a.q_ss = s.q_ss;
  a.k_sb = s.k_sb, a.k_sh = s.k_sh, a.k_ss = s.k_ss;
  a.B = s.B, a.Hq = s.Hq, a.Hkv = s.Hkv, a.S = s.S, a.d = s.d, a.g = s.Hq / s.Hkv;
  a.Sq = s.rows();
  a.c = resolve_scale(scale, s.d);
  a.knorm = knorm;
  a.nkn = knorm ? fam_key_norm_parts(s.S) : 0;
  a.part = nullptr;
  a.nks = 1;
  return a;
}

// Arguments of the mass pass (group sum into `mass` with nsplit splits, or
// per query head into `mass_q`).
fam::MassArgs mass_args(const void* q, const void* k, const float* lse, const ScoreShape& s, int W,
                        float scale, float* mass, float* mass_q, float* part, int nsplit) {
  fam::MassArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.lse = lse;
  a.mass = mass;
  a.q_sb = s.q_sb, a.q_sh = s.q_sh, a.q_ss = s.q_ss;
  a.k_sb = s.k_sb, a.k_sh = s.k_sh, a.k_ss = s.k_ss;
  a.B = s.B, a.Hq = s.Hq, a.Hkv = s.Hkv, a.S = s.S, a.d = s.d, a.g = s.Hq / s.Hkv;
  a.W = W < s.S ? W : s.S;
  a.Sq = s.rows();
  a.c = resolve_scale(scale, s.d);
  a.mass_q = mass_q;
  a.part = part;
  a.nsplit = nsplit;
  return a;
}

// Splits of the mass pass: aim at >= 3072 workgroups (three per CU on 256
// CUs, with room for the uneven column lengths), at most 16.
int mass_splits(int B, int Hkv, int S) {
  const int64_t wgs = (int64_t)((S + fam::kMassKeysPerWG - 1) / fam::kMassKeysPerWG) * B * Hkv;
  const int64_t n = (3072 + wgs - 1) / wgs;
  return (int)(n < 1 ? 1 : (n > 16 ? 16 : n));
}

// Key-range splits of the bounded first pass: aim at >= 3072 workgroups (as
// for the mass pass), at most kLseMaxSplits, and at least 16 key tiles of 64
// per split for the longest rows.
int lse_splits(const ScoreShape& s) {
  const int64_t npb = ((int64_t)s.rows() + 63) / 64;
  const int64_t wgs = (npb * (s.Hq / s.Hkv) + 3) / 4 * s.B * s.Hkv;
  int64_t n = (3072 + wgs - 1) / wgs;
  const int64_t by_tiles = ((int64_t)s.S + 63) / 64 / 16;
  if (n > by_tiles) n = by_tiles;
  if (n > fam::kLseMaxSplits) n = fam::kLseMaxSplits;
  return (int)(n < 1 ? 1 : n);
}

// Bytes of the first pass's split partial sums: nks + 1 floats per row.
size_t lse_split_bytes(const ScoreShape& s, int nks) {
  return nks > 1 ? (size_t)(nks + 1) * s.B * s.Hq * s.rows() * sizeof(float) : 0;
}

fam::Elem elem_of(int dt) { return dt == FAM_BF16 ? fam::Elem::kBf16 : fam::Elem::kFp16; }

// Partial slices of the group-sum mass pass. From kMassRangeMinS keys on
// (while at most kMassMaxRanges ranges cover the query rows and the grid of
// key blocks x ranges x B x Hkv workgroups fits one launch) split s owns
// the query tiles [s * R, (s + 1) * R), R = kMassRangeTiles: the workgroups
// resident together then read the same few MB of Q, which stay in cache,
// instead of each re-reading its own share from HBM. Shorter sequences
// divide each key block's steps evenly over mass_splits workgroups.
struct MassPlan {
  int nsplit;
  int range_tiles;   // 0: even shares
};
MassPlan mass_plan(const ScoreShape& s) {
  if (s.S >= fam::kMassRangeMinS) {
    const int64_t nt = ((int64_t)s.rows() + fam::kMassQTile - 1) / fam::kMassQTile;
    const int64_t nr = (nt + fam::kMassRangeTiles - 1) / fam::kMassRangeTiles;
    const int64_t nkb = ((int64_t)s.S + fam::kMassKeysPerWG - 1) / fam::kMassKeysPerWG;
    if (nr > 1 && nr <= fam::kMassMaxRanges && nkb * nr * s.B * s.Hkv <= 0x7fffffff)
      return {(int)nr, fam::kMassRangeTiles};
  }
  return {mass_splits(s.B, s.Hkv, s.S), 0};
}

// Bytes of the mass pass's partial slices: nsplit * B * Hkv * S floats.
size_t mass_split_bytes(const ScoreShape& s, int nsplit) {
  return nsplit > 1 ? (size_t)nsplit * s.B * s.Hkv * s.S * sizeof(float) : 0;
}

// Bytes of the per-query-head mass pass's range slices: nsplit * B * Hq * S floats.
size_t per_head_split_bytes(const ScoreShape& s, int nsplit) {
  return nsplit > 1 ? (size_t)nsplit * s.B * s.Hq * s.S * sizeof(float) : 0;
}

// Group-sum mass pass on a validated shape: as many splits as wanted and as
// the workspace holds (none without one). mass_prepare checks the arguments
// and fills the launch's arguments; mass_group also launches.
fam_status mass_prepare(const void* q, const void* k, const float* lse, const ScoreShape& s, int W,
                        float scale, float* mass, void* workspace, size_t workspace_bytes,
                        fam::MassArgs& a) {
  if (!lse || !mass) return fail(FAM_ERR_INVALID_ARG, "lse and mass must be non-null");
  if (W < 0) return fail(FAM_ERR_INVALID_ARG, "window W must be >= 0 (got %d)", W);
  if (const fam_status sc = check_mass_scale(scale, s.d); sc != FAM_OK) return sc;
  if (workspace && !aligned16(workspace))
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t per_split = (size_t)s.B * s.Hkv * s.S * sizeof(float);
  const MassPlan plan = mass_plan(s);
  if (workspace && plan.range_tiles > 0 && mass_split_bytes(s, plan.nsplit) <= workspace_bytes) {
    a = mass_args(q, k, lse, s, W, scale, mass, nullptr, static_cast<float*>(workspace), plan.nsplit);
    a.range_tiles = plan.range_tiles;
    return ok();
  }
  // even shares, as many as wanted and as the workspace holds
  int nsplit = mass_splits(s.B, s.Hkv, s.S);
  if (!workspace) nsplit = 1;
  if ((size_t)nsplit * per_split > workspace_bytes) nsplit = (int)(workspace_bytes / per_split);
  if (nsplit < 2) nsplit = 1;
  a = mass_args(q, k, lse, s, W, scale, mass, nullptr,
                nsplit > 1 ? static_cast<float*>(workspace) : nullptr, nsplit);
  return ok();
}

fam_status mass_group(const void* q, const void* k, const float* lse, int dtype,
                      const ScoreShape& s, int W, float scale, float* mass, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, const char* what) {
  fam::MassArgs a{};
  if (const fam_status st = mass_prepare(q, k, lse, s, W, scale, mass, workspace, workspace_bytes, a);
      st != FAM_OK)
    return st;
  return launched(fam::launch_mass(a, elem_of(dtype), stream), stream, what);
}

// Key norms, the bounded first pass and the group-sum mass pass. The
// key-norm partial maxima ([B * Hkv][P] floats, P <= S) occupy the start of
// `mass` until the mass pass overwrites it.
fam_status compute_all(const void* q, const void* k, int dtype, const ScoreShape& s, int W,
                       float scale, float* lse, float* mass, void* workspace,
                       size_t workspace_bytes, hipStream_t hs, const char* who) {
  if (!lse || !mass) return fail(FAM_ERR_INVALID_ARG, "lse and mass must be non-null");
  if (W < 0) return fail(FAM_ERR_INVALID_ARG, "window W must be >= 0 (got %d)", W);
  if (const fam_status sc = check_mass_scale(scale, s.d); sc != FAM_OK) return sc;
  if (workspace && !aligned16(workspace))
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  fam::LseArgs a = lse_args(q, k, s, scale, lse, mass);
  // the first pass's partial sums are consumed before the mass pass reuses
  // the workspace (stream order)
  int nks = workspace ? lse_splits(s) : 1;
  while (nks > 1 && lse_split_bytes(s, nks) > workspace_bytes) --nks;
  if (nks > 1) {
    a.nks = nks;
    a.part = static_cast<float*>(workspace);
  }
  std::string what = std::string(who) + " key-norm launch";
  hipError_t e = fam::launch_knorm(a, elem_of(dtype), hs);
  if (e != hipSuccess) return hip_status(e, what.c_str());
  e = fam::launch_lse(a, elem_of(dtype), hs);
  what = std::string(who) + " lse launch";
  if (e != hipSuccess) return hip_status(e, what.c_str());
  what = std::string(who) + " mass launch";
  return mass_group(q, k, lse, dtype, s, W, scale, mass, workspace, workspace_bytes, hs, what.c_str());
}

// Forced set and candidate range for a head of length S.
struct Plan {
  int c0, c1, forced;
};
Plan plan_of(int S, int sinks, int recent) {
  Plan p;
  p.c0 = sinks < S ? sinks : S;
  const int64_t tail = (int64_t)S - (int64_t)recent;
  p.c1 = tail > p.c0 ? (int)tail : p.c0;
  p.forced = S - (p.c1 - p.c0);
  return p;
}

}  // namespace

extern "C" {

const char* fam_status_string(fam_status st) {
  switch (enum_bits(&st)) {
    case FAM_OK: return "FAM_OK";
    case FAM_ERR_INVALID_ARG: return "FAM_ERR_INVALID_ARG";
    case FAM_ERR_UNSUPPORTED: return "FAM_ERR_UNSUPPORTED";
    case FAM_ERR_WORKSPACE: return "FAM_ERR_WORKSPACE";
    case FAM_ERR_HIP: return "FAM_ERR_HIP";
    case FAM_ERR_TIMEOUT: return "FAM_ERR_TIMEOUT";
  }
  return "FAM_ERR_UNKNOWN";
}

const char* fam_last_error(void) { return g_error.c_str(); }

int fam_key_norm_parts(int S) { return S < 1 ? 0 : (S < fam::kNormParts ? S : fam::kNormParts); }

fam_status fam_key_norms(const void* k, fam_dtype dtype_arg, int B, int Hkv, int S, int d,
                         int64_t k_sb, int64_t k_sh, int64_t k_ss, float* knorm, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hkv, Hkv, S, d, k_sb, k_sh, k_ss, k_sb, k_sh, k_ss, 0};
  fam_status st = check_scores(k, k, dtype, s);
  if (st != FAM_OK) return st;
  if (!knorm) return fail(FAM_ERR_INVALID_ARG, "knorm must be non-null");
  const fam::LseArgs a = lse_args(k, k, s, 0.f, nullptr, knorm);
  return launched(fam::launch_knorm(a, elem_of(dtype), static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                    "fam_key_norms launch");
}

fam_status fam_lse(const void* q, const void* k, fam_dtype dtype_arg, int B, int Hq, int Hkv, int S,
                   int d, int64_t q_sb, int64_t q_sh, int64_t q_ss, int64_t k_sb, int64_t k_sh,
                   int64_t k_ss, float scale, const float* knorm, float* lse, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  fam_status st = check_scores(q, k, dtype, s);
  if (st != FAM_OK) return st;
  if (!lse) return fail(FAM_ERR_INVALID_ARG, "lse must be non-null");
  if (!std::isfinite(scale)) return fail(FAM_ERR_INVALID_ARG, "scale must be finite");
  const fam::LseArgs a = lse_args(q, k, s, scale, lse, const_cast<float*>(knorm));
  return launched(fam::launch_lse(a, elem_of(dtype), static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "fam_lse launch");
}

size_t fam_mass_workspace_size(int B, int Hq, int Hkv, int S) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Hq % Hkv != 0) return 0;
  const ScoreShape s{B, Hq, Hkv, S, 64, 0, 0, 0, 0, 0, 0, 0};   // Sq = 0: every row is a query
  return mass_split_bytes(s, mass_plan(s).nsplit);
}

size_t fam_compute_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sk < 1 || Sq < 1 || Sq > Sk || Hq % Hkv != 0) return 0;
  const ScoreShape s{B, Hq, Hkv, Sk, 64, 0, 0, 0, 0, 0, 0, Sq};
  const size_t lse_bytes = lse_split_bytes(s, lse_splits(s));
  const size_t mass_bytes = mass_split_bytes(s, mass_plan(s).nsplit);
  return lse_bytes > mass_bytes ? lse_bytes : mass_bytes;
}

fam_status fam_mass(const void* q, const void* k, const float* lse, fam_dtype dtype_arg, int B, int Hq,
                    int Hkv, int S, int d, int64_t q_sb, int64_t q_sh, int64_t q_ss, int64_t k_sb,
                    int64_t k_sh, int64_t k_ss, int W, float scale, float* mass, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  fam_status st = check_scores(q, k, dtype, s);
  if (st != FAM_OK) return st;
  return mass_group(q, k, lse, dtype, s, W, scale, mass, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), "fam_mass launch");
}

fam_status fam_mass_per_head(const void* q, const void* k, const float* lse, fam_dtype dtype_arg, int B,
                             int Hq, int Hkv, int S, int d, int64_t q_sb, int64_t q_sh,
                             int64_t q_ss, int64_t k_sb, int64_t k_sh, int64_t k_ss, int W,
                             float scale, float* mass_q, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  fam_status st = check_scores(q, k, dtype, s);
  if (st != FAM_OK) return st;
  if (!lse || !mass_q) return fail(FAM_ERR_INVALID_ARG, "lse and mass_q must be non-null");
  if (W < 0) return fail(FAM_ERR_INVALID_ARG, "window W must be >= 0 (got %d)", W);
  if (const fam_status sc = check_mass_scale(scale, s.d); sc != FAM_OK) return sc;
  if (workspace && !aligned16(workspace))
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  fam::MassArgs a = mass_args(q, k, lse, s, W, scale, nullptr, mass_q, nullptr, 1);
  // ranges of query rows as for the group sum, one [B, Hq, S] slice each
  const MassPlan plan = mass_plan(s);
  const size_t need = per_head_split_bytes(s, plan.nsplit);
  if (workspace && plan.range_tiles > 0 && need <= workspace_bytes) {
    a.part = static_cast<float*>(workspace);
    a.nsplit = plan.nsplit;
    a.range_tiles = plan.range_tiles;
  }
  return launched(fam::launch_mass(a, elem_of(dtype), static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                    "fam_mass_per_head launch");
}

size_t fam_mass_per_head_workspace_size(int B, int Hq, int Hkv, int S) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Hq % Hkv != 0) return 0;
  const ScoreShape s{B, Hq, Hkv, S, 64, 0, 0, 0, 0, 0, 0, 0};   // Sq = 0: every row is a query
  const MassPlan plan = mass_plan(s);
  return plan.range_tiles > 0 ? per_head_split_bytes(s, plan.nsplit) : 0;
}

fam_status fam_kvpop_target(const float* mass_q, int B, int Hq, int Hkv, int S, int W, float eps,
                            fam_aggregate aggregate_arg, float* target, void* stream) {
  const int aggregate = enum_bits(&aggregate_arg);
  if (!mass_q || !target) return fail(FAM_ERR_INVALID_ARG, "mass_q and target must be non-null");
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1)
    return fail(FAM_ERR_INVALID_ARG, "B, Hq, Hkv and S must be >= 1 (got %d, %d, %d, %d)", B, Hq, Hkv, S);
  if (Hq % Hkv != 0) return fail(FAM_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (W < 0) return fail(FAM_ERR_INVALID_ARG, "window W must be >= 0 (got %d)", W);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FAM_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (aggregate != FAM_AGG_MAX && aggregate != FAM_AGG_MEAN)
    return fail(FAM_ERR_INVALID_ARG, "aggregate %d is not FAM_AGG_MAX or FAM_AGG_MEAN", aggregate);
  if ((reinterpret_cast<uintptr_t>(mass_q) | reinterpret_cast<uintptr_t>(target)) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "mass_q and target must be 4-byte aligned");
  const fam::TargetArgs a{mass_q, target, B, Hq, Hkv, S, W, eps, aggregate == FAM_AGG_MEAN ? 1 : 0};
  return launched(fam::launch_target(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "fam_kvpop_target launch");
}

fam_status fam_compute(const void* q, const void* k, fam_dtype dtype_arg, int B, int Hq, int Hkv, int S,
                       int d, int64_t q_sb, int64_t q_sh, int64_t q_ss, int64_t k_sb, int64_t k_sh,
                       int64_t k_ss, int W, float scale, float* lse, float* mass,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  fam_status st = check_scores(q, k, dtype, s);
  if (st != FAM_OK) return st;
  return compute_all(q, k, dtype, s, W, scale, lse, mass, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream), "fam_compute");
}

fam_status fam_compute_chunk(const void* q, const void* k, fam_dtype dtype_arg, int B, int Hq, int Hkv,
                             int Sq, int Sk, int d, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                             int64_t k_sb, int64_t k_sh, int64_t k_ss, int W, float scale,
                             float* lse, float* mass, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  if (Sq < 1 || Sq > Sk)
    return fail(FAM_ERR_INVALID_ARG, "query rows Sq = %d must be in [1, Sk = %d]", Sq, Sk);
  const ScoreShape s{B, Hq, Hkv, Sk, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, Sq};
  fam_status st = check_scores(q, k, dtype, s);
  if (st != FAM_OK) return st;
  return compute_all(q, k, dtype, s, W, scale, lse, mass, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream), "fam_compute_chunk");
}

fam_status evict_plan(int H, int S, const int64_t* budgets, int sinks, int recent, int64_t* kept,
                      int64_t* offsets) {
  if (H < 0) return fail(FAM_ERR_INVALID_ARG, "H must be >= 0 (got %d)", H);
  if (S < 1) return fail(FAM_ERR_INVALID_ARG, "S must be >= 1 (got %d)", S);
  if (sinks < 0 || recent < 0) return fail(FAM_ERR_INVALID_ARG, "sinks and recent must be >= 0");
  if (H > 0 && !budgets) return fail(FAM_ERR_INVALID_ARG, "budgets must be non-null");
  for (int h = 0; h < H; ++h)
    if (budgets[h] < 0) return fail(FAM_ERR_INVALID_ARG, "budget of head %d is negative", h);
  const Plan p = plan_of(S, sinks, recent);
  int64_t off = 0;
  if (offsets) offsets[0] = 0;
  for (int h = 0; h < H; ++h) {
    int64_t kh = budgets[h] > p.forced ? budgets[h] : p.forced;
    if (kh > S) kh = S;
    if (kept) kept[h] = kh;
    off += kh;
    if (offsets) offsets[h + 1] = off;
  }
  return ok();
}

fam_status fam_budgets_from_ratios(int H, const double* ratios, int64_t t, int64_t* budgets) {
  if (H < 0 || t < 0) return fail(FAM_ERR_INVALID_ARG, "H and t must be >= 0");
  if (H > 0 && (!ratios || !budgets)) return fail(FAM_ERR_INVALID_ARG, "ratios and budgets must be non-null");
  for (int h = 0; h < H; ++h) {
    const double r = ratios[h];
    if (!std::isfinite(r) || r < 0.0) return fail(FAM_ERR_INVALID_ARG, "ratio of head %d is invalid", h);
    const double b = std::floor(r * (double)t);
    if (b > 9.0e18) return fail(FAM_ERR_INVALID_ARG, "budget of head %d overflows", h);
  }
  for (int h = 0; h < H; ++h) budgets[h] = (int64_t)std::floor(ratios[h] * (double)t);
  return ok();
}

namespace {
int select_chunks(const Plan& p) {
  const int a0 = p.c0 & ~3;
  const int n = (p.c1 - a0 + fam::kSelectChunk - 1) / fam::kSelectChunk;
  return n < 1 ? 1 : n;
}
int select_slots(int H) { return H < fam::kSelectBatch ? (H < 1 ? 1 : H) : fam::kSelectBatch; }
}  // namespace

size_t evict_select_workspace_size(int H, int S, int sinks, int recent) {
  if (H < 0 || S < 1 || sinks < 0 || recent < 0) return 0;
  const Plan p = plan_of(S, sinks, recent);
  if (p.c1 - p.c0 > fam::kSelectMaxCandidates) return fam::select_long_workspace_bytes(select_slots(H));
  return fam::select_workspace_bytes(select_slots(H), select_chunks(p));
}

}  // extern "C"

namespace {
// Checks of the sizes, the scores and the workspace (evict_select_prepare's
// arguments).
fam_status select_ws_check(const float* scores, int64_t score_row_stride, int H, int S, int sinks,
                           int recent, const void* workspace, size_t workspace_bytes) {
  if (H < 0) return fail(FAM_ERR_INVALID_ARG, "H must be >= 0 (got %d)", H);
  if (S < 1 || S > kMaxSeq) return fail(FAM_ERR_INVALID_ARG, "S = %d out of range", S);
  if (sinks < 0 || recent < 0) return fail(FAM_ERR_INVALID_ARG, "sinks and recent must be >= 0");
  if (H == 0) return ok();
  if (!scores) return fail(FAM_ERR_INVALID_ARG, "scores must be non-null");
  if (H > 1 && score_row_stride < S) return fail(FAM_ERR_INVALID_ARG, "score row stride must be >= S");
  const Plan p = plan_of(S, sinks, recent);
  if (p.c1 - p.c0 > fam::kSelectLongMaxCandidates)
    return fail(FAM_ERR_UNSUPPORTED, "%d candidates per head exceed %d", p.c1 - p.c0,
                fam::kSelectLongMaxCandidates);
  const size_t need_ws = evict_select_workspace_size(H, S, sinks, recent);
  if (!workspace || workspace_bytes < need_ws)
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need_ws,
                workspace ? workspace_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (p.c1 - p.c0 > fam::kSelectMaxCandidates && fam::select_long_batch_heads(select_chunks(p)) < 1)
    return fail(FAM_ERR_UNSUPPORTED, "evict_select: the device cannot hold the %d chunk workgroups of one head",
                select_chunks(p));
  return ok();
}

// Checks of evict_select's arguments (all but the scores' values).
fam_status select_check(const float* scores, int64_t score_row_stride, int H, int S,
                        const int64_t* budgets, int sinks, int recent, const int32_t* idx,
                        const int64_t* offsets_dev, const void* workspace, size_t workspace_bytes) {
  if (H < 0) return fail(FAM_ERR_INVALID_ARG, "H must be >= 0 (got %d)", H);
  if (S < 1 || S > kMaxSeq) return fail(FAM_ERR_INVALID_ARG, "S = %d out of range", S);
  if (sinks < 0 || recent < 0) return fail(FAM_ERR_INVALID_ARG, "sinks and recent must be >= 0");
  if (H == 0) return ok();
  if (!scores || !idx || !offsets_dev || !budgets)
    return fail(FAM_ERR_INVALID_ARG, "scores, budgets, idx and offsets_dev must be non-null");
  if (H > 1 && score_row_stride < S) return fail(FAM_ERR_INVALID_ARG, "score row stride must be >= S");
  for (int h = 0; h < H; ++h)
    if (budgets[h] < 0) return fail(FAM_ERR_INVALID_ARG, "budget of head %d is negative", h);
  return select_ws_check(scores, score_row_stride, H, S, sinks, recent, workspace, workspace_bytes);
}

// Whether the select of these sizes can take its scores straight from the
// mass pass's partial slices (one batch of heads in three launches, more
// than one chunk a head, some head neither empty nor whole).
bool select_from_parts_ok(int H, int S, const int64_t* budgets, int sinks, int recent) {
  const Plan p = plan_of(S, sinks, recent);
  if (H < 1 || H > fam::kSelectBatch || p.c1 - p.c0 > fam::kSelectMaxCandidates || select_chunks(p) < 2)
    return false;
  for (int h = 0; h < H; ++h) {
    int64_t kh = budgets[h] > p.forced ? budgets[h] : p.forced;
    if (kh > S) kh = S;
    if (kh - p.forced != 0 && kh - p.forced != p.c1 - p.c0) return true;
  }
  return false;
}

// Whether evict_select of these sizes can be split at its first launch (the
// budget-free histograms): one batch of heads in three launches.
bool select_prepared_ok(int H, int S, int sinks, int recent) {
  const Plan p = plan_of(S, sinks, recent);
  return H >= 1 && H <= fam::kSelectBatch && p.c1 - p.c0 <= fam::kSelectMaxCandidates && select_chunks(p) >= 2;
}

// The launch arguments of one batch holding all H heads (select_prepared_ok
// holds). Without budgets every head is given one choice, so that no head
// skips the histogram launch.
fam::SelectArgs prepared_args(const float* scores, int64_t score_row_stride, int H, int S, int sinks,
                              int recent, const int64_t* budgets, int32_t* idx, int64_t* offsets_dev,
                              void* workspace) {
  const Plan p = plan_of(S, sinks, recent);
  fam::SelectArgs a{};
  a.scores = scores;
  a.row_stride = score_row_stride;
  a.idx = idx;
  a.offsets_dev = offsets_dev;
  a.ws = workspace;
  a.S = S;
  a.H = H;
  a.c0 = p.c0;
  a.c1 = p.c1;
  a.slots = select_slots(H);
  a.nchunk = select_chunks(p);
  a.head0 = 0;
  a.nheads = H;
  int64_t off = 0;
  for (int h = 0; h < H; ++h) {
    int64_t kh = budgets ? (budgets[h] > p.forced ? budgets[h] : p.forced) : p.forced + 1;
    if (kh > S) kh = S;
    a.out_off[h] = off;
    a.n_choose[h] = (int32_t)(kh - p.forced);
    off += kh;
  }
  a.total = off;
  return a;
}

// The select launches for checked arguments (H >= 1). With `part` non-null
// (select_from_parts_ok holds), `scores` is the [H, S] mass, which the first
// launch forms from the nsplit slices at `part` before it is read.
fam_status select_run(const float* scores, int64_t score_row_stride, int H, int S,
                      const int64_t* budgets, int sinks, int recent, int32_t* idx,
                      int64_t* offsets_dev, void* workspace, const float* part, int nsplit,
                      hipStream_t stream) {
  const Plan p = plan_of(S, sinks, recent);
  const bool long_path = p.c1 - p.c0 > fam::kSelectMaxCandidates;
  int64_t total = 0;
  for (int h = 0; h < H; ++h) {
    int64_t kh = budgets[h] > p.forced ? budgets[h] : p.forced;
    total += kh > S ? S : kh;
  }
  const int batch = long_path ? fam::select_long_batch_heads(select_chunks(p)) : fam::kSelectBatch;
  fam::SelectArgs a{};
  a.scores = scores;
  a.row_stride = score_row_stride;
  a.idx = idx;
  a.offsets_dev = offsets_dev;
  a.ws = workspace;
  a.total = total;
  a.S = S;
  a.H = H;
  a.c0 = p.c0;
  a.c1 = p.c1;
  a.slots = select_slots(H);
  a.nchunk = select_chunks(p);
  int64_t off = 0;
  for (int h0 = 0; h0 < H; h0 += batch) {
    const int n = H - h0 < batch ? H - h0 : batch;
    a.head0 = h0;
    a.nheads = n;
    for (int i = 0; i < n; ++i) {
      int64_t kh = budgets[h0 + i] > p.forced ? budgets[h0 + i] : p.forced;
      if (kh > S) kh = S;
      a.out_off[i] = off;
      a.n_choose[i] = (int32_t)(kh - p.forced);
      off += kh;
    }
    const hipError_t e = part ? fam::launch_select_from_parts(a, part, nsplit, stream)
                         : long_path ? fam::launch_select_long(a, stream, h0 == 0)
                                     : fam::launch_select(a, stream);
    if (e != hipSuccess) return hip_status(e, "evict_select launch");
  }
  const fam_status rc = launched(hipSuccess, stream, "evict_select launch");
  if (rc != FAM_OK || !long_path || !sync_check()) return rc;
  // under the sync check: the long path's error word counts waits that ran
  // out of polls
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "evict_select (sync check)");
  if (word != 0u)
    return fail(FAM_ERR_TIMEOUT, "evict_select: %u wait(s) ran out of polls; the index lists are incomplete", word);
  return ok();
}
}  // namespace

extern "C" {

fam_status evict_select(const float* scores, int64_t score_row_stride, int H, int S,
                        const int64_t* budgets, int sinks, int recent, int32_t* idx,
                        int64_t* offsets_dev, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (const fam_status st = select_check(scores, score_row_stride, H, S, budgets, sinks, recent, idx,
                                         offsets_dev, workspace, workspace_bytes);
      st != FAM_OK || H == 0)
    return st;
  return select_run(scores, score_row_stride, H, S, budgets, sinks, recent, idx, offsets_dev, workspace,
                    nullptr, 0, static_cast<hipStream_t>(stream));
}

fam_status fam_mass_select(const void* q, const void* k, const float* lse, fam_dtype dtype_arg, int B,
                           int Hq, int Hkv, int S, int d, int64_t q_sb, int64_t q_sh, int64_t q_ss,
                           int64_t k_sb, int64_t k_sh, int64_t k_ss, int W, float scale, float* mass,
                           void* mass_workspace, size_t mass_workspace_bytes,
                           const int64_t* budgets, int sinks, int recent, int32_t* idx,
                           int64_t* offsets_dev, void* select_workspace,
                           size_t select_workspace_bytes, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  if (const fam_status st = check_scores(q, k, dtype, s); st != FAM_OK) return st;
  fam::MassArgs a{};
  if (const fam_status st = mass_prepare(q, k, lse, s, W, scale, mass, mass_workspace,
                                         mass_workspace_bytes, a);
      st != FAM_OK)
    return st;
  const int H = B * Hkv;
  if (const fam_status st = select_check(mass, S, H, S, budgets, sinks, recent, idx, offsets_dev,
                                         select_workspace, select_workspace_bytes);
      st != FAM_OK)
    return st;
  if (a.nsplit > 1) {
    // the mass pass's slices are read while the select workspace is written
    const uintptr_t m0 = reinterpret_cast<uintptr_t>(a.part);
    const uintptr_t m1 = m0 + mass_split_bytes(s, a.nsplit);
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(select_workspace);
    const uintptr_t s1 = s0 + select_workspace_bytes;
    if (m0 < s1 && s0 < m1)
      return fail(FAM_ERR_INVALID_ARG, "mass and select workspaces must not overlap");
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fused = a.nsplit > 1 && select_from_parts_ok(H, S, budgets, sinks, recent);
  hipError_t e = fam::launch_mass(a, elem_of(dtype), hs, !fused);
  if (const fam_status st = launched(e, hs, "fam_mass_select (mass pass)"); st != FAM_OK) return st;
  return select_run(mass, S, H, S, budgets, sinks, recent, idx, offsets_dev, select_workspace,
                    fused ? a.part : nullptr, a.nsplit, hs);
}

fam_status evict_select_prepare(const float* scores, int64_t score_row_stride, int H, int S, int sinks,
                                int recent, void* workspace, size_t workspace_bytes, void* stream) {
  if (const fam_status st = select_ws_check(scores, score_row_stride, H, S, sinks, recent, workspace,
                                            workspace_bytes);
      st != FAM_OK || !select_prepared_ok(H, S, sinks, recent))
    return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const fam::SelectArgs a = prepared_args(scores, score_row_stride, H, S, sinks, recent, nullptr, nullptr,
                                          nullptr, workspace);
  return launched(fam::launch_select_hist(a, hs), hs, "evict_select_prepare launch");
}

fam_status evict_select_prepared(const float* scores, int64_t score_row_stride, int H, int S,
                                 const int64_t* budgets, int sinks, int recent, int32_t* idx,
                                 int64_t* offsets_dev, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (const fam_status st = select_check(scores, score_row_stride, H, S, budgets, sinks, recent, idx,
                                         offsets_dev, workspace, workspace_bytes);
      st != FAM_OK || H == 0)
    return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!select_prepared_ok(H, S, sinks, recent))
    return select_run(scores, score_row_stride, H, S, budgets, sinks, recent, idx, offsets_dev, workspace,
                      nullptr, 0, hs);
  const fam::SelectArgs a = prepared_args(scores, score_row_stride, H, S, sinks, recent, budgets, idx,
                                          offsets_dev, workspace);
  return launched(fam::launch_select_prepared(a, hs), hs, "evict_select_prepared launch");
}

fam_status fam_mass_prepare_select(const void* q, const void* k, const float* lse, fam_dtype dtype_arg,
                                   int B, int Hq, int Hkv, int S, int d, int64_t q_sb, int64_t q_sh,
                                   int64_t q_ss, int64_t k_sb, int64_t k_sh, int64_t k_ss, int W,
                                   float scale, float* mass, void* mass_workspace,
                                   size_t mass_workspace_bytes, int sinks, int recent,
                                   void* select_workspace, size_t select_workspace_bytes, void* stream) {
  const int dtype = enum_bits(&dtype_arg);
  const ScoreShape s{B, Hq, Hkv, S, d, q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, 0};   // Sq = 0: every row is a query
  if (const fam_status st = check_scores(q, k, dtype, s); st != FAM_OK) return st;
  fam::MassArgs a{};
  if (const fam_status st = mass_prepare(q, k, lse, s, W, scale, mass, mass_workspace,
                                         mass_workspace_bytes, a);
      st != FAM_OK)
    return st;
  const int H = B * Hkv;
  if (const fam_status st = select_ws_check(mass, S, H, S, sinks, recent, select_workspace,
                                            select_workspace_bytes);
      st != FAM_OK)
    return st;
  const bool prepared = select_prepared_ok(H, S, sinks, recent);
  if (prepared && a.nsplit > 1) {
    // the mass pass's slices are read while the select workspace is written
    const uintptr_t m0 = reinterpret_cast<uintptr_t>(a.part);
    const uintptr_t m1 = m0 + mass_split_bytes(s, a.nsplit);
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(select_workspace);
    const uintptr_t s1 = s0 + select_workspace_bytes;
    if (m0 < s1 && s0 < m1)
      return fail(FAM_ERR_INVALID_ARG, "mass and select workspaces must not overlap");
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fused = prepared && a.nsplit > 1;
  hipError_t e = fam::launch_mass(a, elem_of(dtype), hs, !fused);
  if (const fam_status st = launched(e, hs, "fam_mass_prepare_select (mass pass)"); st != FAM_OK || !prepared)
    return st;
  const fam::SelectArgs sa = prepared_args(mass, S, H, S, sinks, recent, nullptr, nullptr, nullptr,
                                           select_workspace);
  e = fused ? fam::launch_select_hist_reduce(sa, a.part, a.nsplit, hs) : fam::launch_select_hist(sa, hs);
  return launched(e, hs, "fam_mass_prepare_select (histograms)");
}

// evict_select without a caller workspace: the workspace is a static device
// array (one copy per GPU, kept until the process ends). Host code never
// passes the array's name to a kernel or a copy: on each device, the first
// call looks up the array's device address with that device current and
// keeps it; every later call uses that address.
static __device__ __align__(256) unsigned char scratch[FAM_NOALLOC_SCRATCH_BYTES];
static_assert(FAM_NOALLOC_SCRATCH_BYTES >=
                  4 * ((size_t)fam::kSelectLongHeaderWords + (size_t)fam::kSelectBatch * fam::kSelectLongSlotWordsMax),
              "the static scratch holds the long path's largest workspace");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fam_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FAM_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(FAM_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FAM_OK;
}
}  // namespace

fam_status evict_select_noalloc(const float* scores, int64_t score_row_stride, int H, int S,
                                const int64_t* budgets, int sinks, int recent, int32_t* idx,
                                int64_t* offsets_dev, void* stream) {
  if (H < 0 || S < 1 || sinks < 0 || recent < 0)
    return fail(FAM_ERR_INVALID_ARG, "need H >= 0, S >= 1, sinks >= 0 and recent >= 0");
  if (H == 0) return ok();
  const size_t need = evict_select_workspace_size(H, S, sinks, recent);
  if (need > (size_t)FAM_NOALLOC_SCRATCH_BYTES)
    return fail(FAM_ERR_UNSUPPORTED,
                "evict_select_noalloc: %d heads of %d positions need %zu bytes of scratch, more than the "
                "%zu of its static array (use evict_select with a workspace)",
                H, S, need, (size_t)FAM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const fam_status st = scratch_of_current_device(&ws);
  if (st != FAM_OK) return st;
  return evict_select(scores, score_row_stride, H, S, budgets, sinks, recent, idx, offsets_dev, ws,
                      (size_t)FAM_NOALLOC_SCRATCH_BYTES, stream);
}

fam_status kv_compact(const void* k, const void* v, int elem_bytes, int H, int S, int d,
                      int64_t k_sh, int64_t k_ss, int64_t v_sh, int64_t v_ss, const int32_t* idx,
                      const int64_t* offsets_dev, int64_t total_rows, void* k_new, void* v_new,
                      void* stream) {
  if (elem_bytes != 2) return fail(FAM_ERR_UNSUPPORTED, "elem_bytes %d (need 2)", elem_bytes);
  if (H < 1 || S < 1 || total_rows < 0)
    return fail(FAM_ERR_INVALID_ARG, "need H >= 1, S >= 1, total_rows >= 0");
  if (d != 64 && d != 128 && d != 256) return fail(FAM_ERR_UNSUPPORTED, "head dim %d (need 64, 128 or 256)", d);
  if (total_rows == 0) return ok();
  if (!k || !v || !idx || !offsets_dev || !k_new || !v_new)
    return fail(FAM_ERR_INVALID_ARG, "pointers must be non-null");
  const int64_t st[4] = {k_sh, k_ss, v_sh, v_ss};
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0 || st[i] % 8 != 0)
      return fail(FAM_ERR_INVALID_ARG, "strides must be >= 0 and multiples of 8 elements");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_new) || !aligned16(v_new))
    return fail(FAM_ERR_INVALID_ARG, "k, v, k_new and v_new must be 16-byte aligned");
  fam::CompactArgs a{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), k_sh, k_ss,
                     v_sh, v_ss, idx, offsets_dev, total_rows, static_cast<uint16_t*>(k_new),
                     static_cast<uint16_t*>(v_new), H, S, d};
  return launched(fam::launch_compact(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "kv_compact launch");
}


fam_status kv_append(const void* k_src, const void* v_src, int elem_bytes, int H, int n, int d,
                     int64_t ks_sh, int64_t ks_ss, int64_t vs_sh, int64_t vs_ss, void* k_cache,
                     void* v_cache, int64_t kc_sh, int64_t kc_ss, int64_t vc_sh, int64_t vc_ss,
                     int capacity, int row0, int32_t* pos, int64_t pos_sh, int pos0, void* stream) {
  if (elem_bytes != 2) return fail(FAM_ERR_UNSUPPORTED, "elem_bytes %d (need 2)", elem_bytes);
  if (d != 64 && d != 128 && d != 256) return fail(FAM_ERR_UNSUPPORTED, "head dim %d (need 64, 128 or 256)", d);
  if (H < 0 || n < 0 || capacity < 0 || row0 < 0)
    return fail(FAM_ERR_INVALID_ARG, "H, n, capacity and row0 must be >= 0");
  if ((int64_t)row0 + n > capacity)
    return fail(FAM_ERR_INVALID_ARG, "rows %d .. %lld exceed the capacity %d", row0,
                (long long)row0 + n - 1, capacity);
  if (H > 65535) return fail(FAM_ERR_UNSUPPORTED, "H = %d exceeds 65535", H);
  if (H == 0 || n == 0) return ok();
  if (!k_src || !v_src || !k_cache || !v_cache)
    return fail(FAM_ERR_INVALID_ARG, "pointers must be non-null");
  const int64_t st[8] = {ks_sh, ks_ss, vs_sh, vs_ss, kc_sh, kc_ss, vc_sh, vc_ss};
  for (int i = 0; i < 8; ++i)
    if (st[i] < 0 || st[i] % 8 != 0)
      return fail(FAM_ERR_INVALID_ARG, "strides must be >= 0 and multiples of 8 elements");
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FAM_ERR_INVALID_ARG, "k_src, v_src, k_cache and v_cache must be 16-byte aligned");
  if (pos && (pos_sh < capacity || (reinterpret_cast<uintptr_t>(pos) & 3u)))
    return fail(FAM_ERR_INVALID_ARG, "pos needs a head stride >= capacity and 4-byte alignment");
  if (pos && (int64_t)pos0 + n - 1 > 0x7fffffffLL)
    return fail(FAM_ERR_INVALID_ARG, "positions overflow int32");
  fam::AppendArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.ks_sh = ks_sh, a.ks_ss = ks_ss, a.vs_sh = vs_sh, a.vs_ss = vs_ss;
  a.k = static_cast<uint16_t*>(k_cache);
  a.v = static_cast<uint16_t*>(v_cache);
  a.k_sh = kc_sh, a.k_ss = kc_ss, a.v_sh = vc_sh, a.v_ss = vc_ss;
  a.pos = pos;
  a.pos_sh = pos_sh;
  a.H = H, a.n = n, a.d = d, a.row0 = row0, a.pos0 = pos0;
  return launched(fam::launch_append(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "kv_append launch");
}

fam_status kv_compact_inplace(void* k, void* v, int elem_bytes, int H, int S, int d, int64_t k_sh,
                              int64_t k_ss, int64_t v_sh, int64_t v_ss, const int32_t* idx,
                              const int64_t* offsets_dev, int64_t total_rows, int32_t* pos,
                              int64_t pos_sh, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (elem_bytes != 2) return fail(FAM_ERR_UNSUPPORTED, "elem_bytes %d (need 2)", elem_bytes);
  if (d != 64 && d != 128 && d != 256) return fail(FAM_ERR_UNSUPPORTED, "head dim %d (need 64, 128 or 256)", d);
  if (H < 0 || S < 1 || total_rows < 0)
    return fail(FAM_ERR_INVALID_ARG, "need H >= 0, S >= 1 and total_rows >= 0");
  if (total_rows > (int64_t)H * S)
    return fail(FAM_ERR_INVALID_ARG, "total_rows %lld exceeds H * S", (long long)total_rows);
  if (H == 0 || total_rows == 0) return ok();
  if (!k || !v || !idx || !offsets_dev) return fail(FAM_ERR_INVALID_ARG, "pointers must be non-null");
  const int64_t st[4] = {k_sh, k_ss, v_sh, v_ss};
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0 || st[i] % 8 != 0)
      return fail(FAM_ERR_INVALID_ARG, "strides must be >= 0 and multiples of 8 elements");
  if (!aligned16(k) || !aligned16(v)) return fail(FAM_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (pos && (pos_sh < S || (reinterpret_cast<uintptr_t>(pos) & 3u)))
    return fail(FAM_ERR_INVALID_ARG, "pos needs a head stride >= S and 4-byte alignment");
  const size_t need = fam::inplace_workspace_bytes(total_rows);
  if (!workspace || workspace_bytes < need)
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  fam::InplaceArgs a{};
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.k_sh = k_sh, a.k_ss = k_ss, a.v_sh = v_sh, a.v_ss = v_ss;
  a.idx = idx;
  a.offsets = offsets_dev;
  a.pos = pos;
  a.pos_sh = pos_sh;
  a.total = total_rows;
  a.H = H, a.S = S, a.d = d;
  a.ws = static_cast<uint32_t*>(workspace);
  a.spin_limit = fam::kInplaceSpinLimit;
  if (const char* lim = std::getenv("FAM_INPLACE_SPIN_LIMIT")) {   // test and debug switch
    const long v = std::strtol(lim, nullptr, 10);
    if (v >= 0 && v < fam::kInplaceSpinLimit) a.spin_limit = (int)v;
  }
  const fam_status rc = launched(fam::launch_compact_inplace(a, static_cast<hipStream_t>(stream)),
                                 static_cast<hipStream_t>(stream), "kv_compact_inplace launch");
  if (rc != FAM_OK || !sync_check()) return rc;
  return kv_compact_inplace_status(workspace, stream);
}

fam_status kv_compact_inplace_status(const void* workspace, void* stream) {
  if (!workspace) return fail(FAM_ERR_INVALID_ARG, "workspace must be non-null");
  if (reinterpret_cast<uintptr_t>(workspace) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  uint32_t word = 0;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&word, static_cast<const uint32_t*>(workspace) + fam::kInplaceErrorWord,
                                sizeof word, hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_status(e, "kv_compact_inplace_status");
  if (word != 0u)
    return fail(FAM_ERR_TIMEOUT, "kv_compact_inplace: %u chunk(s) gave up waiting for earlier chunks "
                "and left their rows unwritten", word);
  return ok();
}


size_t kv_compact_inplace_workspace_size(int64_t total_rows) {
  return total_rows < 0 ? 0 : fam::inplace_workspace_bytes(total_rows);
}

size_t fam_rank_order_workspace_size(int H, int n) {
  if (H < 0 || n < 0) return 0;
  return fam::rank_workspace_bytes(H, n);
}

fam_status fam_rank_order(const float* scores, int64_t row_stride, int H, int n, int32_t* order,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (H < 0 || n < 0) return fail(FAM_ERR_INVALID_ARG, "H and n must be >= 0");
  if (n > kMaxSeq) return fail(FAM_ERR_UNSUPPORTED, "n = %d exceeds %d", n, kMaxSeq);
  if (H == 0 || n == 0) return ok();
  if (!scores || !order) return fail(FAM_ERR_INVALID_ARG, "scores and order must be non-null");
  if (H > 1 && row_stride < n) return fail(FAM_ERR_INVALID_ARG, "row stride must be >= n");
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(order)) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "scores and order must be 4-byte aligned");
  const size_t need = fam_rank_order_workspace_size(H, n);
  if (!workspace || workspace_bytes < need)
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 7u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  if (H > 65535) return fail(FAM_ERR_UNSUPPORTED, "H = %d exceeds 65535", H);
  fam::RankArgs a{scores, row_stride, order, workspace, H, n, fam::rank_tiles(n)};
  return launched(fam::launch_rank(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "fam_rank_order launch");
}

size_t fam_eviction_cost_workspace_size(int H, int n) {
  if (H < 0 || n < 0) return 0;
  return (size_t)H * fam::cost_blocks(n) * sizeof(double);
}

fam_status fam_eviction_cost(const float* importance, int64_t row_stride, const int32_t* order, int H,
                             int n, double* cost, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (H < 0 || n < 0) return fail(FAM_ERR_INVALID_ARG, "H and n must be >= 0");
  if (n > kMaxSeq) return fail(FAM_ERR_UNSUPPORTED, "n = %d exceeds %d", n, kMaxSeq);
  if (H == 0) return ok();
  if (!cost) return fail(FAM_ERR_INVALID_ARG, "cost must be non-null");
  if (n > 0 && (!importance || !order))
    return fail(FAM_ERR_INVALID_ARG, "importance and order must be non-null");
  if (H > 1 && row_stride < n) return fail(FAM_ERR_INVALID_ARG, "row stride must be >= n");
  if ((reinterpret_cast<uintptr_t>(importance) | reinterpret_cast<uintptr_t>(order)) & 3u ||
      (reinterpret_cast<uintptr_t>(cost) & 7u))
    return fail(FAM_ERR_INVALID_ARG, "importance and order must be 4-byte, cost 8-byte aligned");
  const size_t need = fam_eviction_cost_workspace_size(H, n);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 7u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  if (H > 65535) return fail(FAM_ERR_UNSUPPORTED, "H = %d exceeds 65535", H);
  fam::CostArgs a{importance, row_stride, order, cost, static_cast<double*>(workspace), H, n};
  return launched(fam::launch_cost(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "fam_eviction_cost launch");
}

static size_t align8(size_t x) { return (x + 7) & ~(size_t)7; }

size_t fam_eviction_cost_ratio_workspace_size(int H, int n) {
  if (H < 0 || n < 0) return 0;
  return align8(fam::rank_workspace_bytes(H, n)) + align8((size_t)H * n * sizeof(int32_t)) +
         2 * fam_eviction_cost_workspace_size(H, n);
}

fam_status fam_eviction_cost_ratio(const float* scores, int64_t scores_row_stride, const float* importance,
                                   int64_t importance_row_stride, int H, int n, double* ratio,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (H < 0 || n < 0) return fail(FAM_ERR_INVALID_ARG, "H and n must be >= 0");
  if (n > kMaxSeq) return fail(FAM_ERR_UNSUPPORTED, "n = %d exceeds %d", n, kMaxSeq);
  if (H == 0) return ok();
  if (!ratio) return fail(FAM_ERR_INVALID_ARG, "ratio must be non-null");
  if (n > 0 && (!scores || !importance))
    return fail(FAM_ERR_INVALID_ARG, "scores and importance must be non-null");
  if (H > 1 && (scores_row_stride < n || importance_row_stride < n))
    return fail(FAM_ERR_INVALID_ARG, "row strides must be >= n");
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(importance)) & 3u ||
      (reinterpret_cast<uintptr_t>(ratio) & 7u))
    return fail(FAM_ERR_INVALID_ARG, "scores and importance must be 4-byte, ratio 8-byte aligned");
  if (H > 65535) return fail(FAM_ERR_UNSUPPORTED, "H = %d exceeds 65535", H);
  const size_t need = fam_eviction_cost_ratio_workspace_size(H, n);
  if (!workspace || workspace_bytes < need)
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 7u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  char* ws = static_cast<char*>(workspace);
  void* rank_ws = ws;
  int32_t* order = reinterpret_cast<int32_t*>(ws + align8(fam::rank_workspace_bytes(H, n)));
  double* part = reinterpret_cast<double*>(reinterpret_cast<char*>(order) + align8((size_t)H * n * sizeof(int32_t)));
  double* part_opt = part + (size_t)H * fam::cost_blocks(n);
  const int nt = fam::rank_tiles(n);
  fam::RankArgs rs{scores, scores_row_stride, order, rank_ws, H, n, nt};
  fam::RankArgs ri{importance, importance_row_stride, order, rank_ws, H, n, nt};
  fam::CostArgs c{importance, importance_row_stride, order, nullptr, part, H, n};
  return launched(fam::launch_cost_ratio(rs, ri, c, part_opt, ratio, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                    "fam_eviction_cost_ratio launch");
}

fam_status fam_retention_overlap(const int32_t* idx_a, const int64_t* offsets_a, const int32_t* idx_b,
                                 const int64_t* offsets_b, int H, int S, int64_t* common,
                                 void* stream) {
  if (H < 0 || S < 1) return fail(FAM_ERR_INVALID_ARG, "need H >= 0 and S >= 1");
  if (S > fam::kOverlapMaxS)
    return fail(FAM_ERR_UNSUPPORTED, "S = %d exceeds %d positions", S, fam::kOverlapMaxS);
  if (H == 0) return ok();
  if (!idx_a || !offsets_a || !idx_b || !offsets_b || !common)
    return fail(FAM_ERR_INVALID_ARG, "pointers must be non-null");
  if ((reinterpret_cast<uintptr_t>(offsets_a) | reinterpret_cast<uintptr_t>(offsets_b) |
       reinterpret_cast<uintptr_t>(common)) & 7u)
    return fail(FAM_ERR_INVALID_ARG, "offsets and common must be 8-byte aligned");
  fam::OverlapArgs a{idx_a, offsets_a, idx_b, offsets_b, common, H, S};
  return launched(fam::launch_overlap(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                    "fam_retention_overlap launch");
}


size_t fam_topk_cutoff_workspace_size(int H, int S) {
  if (H < 0 || S < 1 || S > fam::kCutoffMaxS) return 0;
  return (size_t)H * S * sizeof(int32_t) + fam::cutoff_workspace_bytes(H, S);
}

fam_status fam_topk_cutoff(const int32_t* order, int H, int S, int sinks, int w, int k, int32_t* tau,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (H < 0 || S < 1 || sinks < 0 || w < 0 || k < 0)
    return fail(FAM_ERR_INVALID_ARG, "need H >= 0, S >= 1, sinks >= 0, w >= 0 and k >= 0");
  if (S > fam::kCutoffMaxS)
    return fail(FAM_ERR_UNSUPPORTED, "S = %d exceeds %d positions", S, fam::kCutoffMaxS);
  if (H > 65535) return fail(FAM_ERR_UNSUPPORTED, "H = %d exceeds 65535", H);
  if (H == 0) return ok();
  if (!order || !tau) return fail(FAM_ERR_INVALID_ARG, "order and tau must be non-null");
  if ((reinterpret_cast<uintptr_t>(order) | reinterpret_cast<uintptr_t>(tau)) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "order and tau must be 4-byte aligned");
  const size_t need = fam_topk_cutoff_workspace_size(H, S);
  if (!workspace || workspace_bytes < need)
    return fail(FAM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 3u)
    return fail(FAM_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
  fam::CutoffArgs a{};
  a.order = order;
  a.rank = static_cast<int32_t*>(workspace);
  a.tau = tau;
  a.ws = static_cast<int32_t*>(workspace) + (size_t)H * S;
  a.H = H, a.S = S, a.sinks = sinks, a.w = w, a.k = k;
  fam::cutoff_shape(S, a.L, a.nw, a.ntiles);
  return launched(fam::launch_cutoff(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream), "fam_topk_cutoff launch");
}


fam_status fam_soft_topk(const double* x, int n, double k, double tau, double* out) {
  if (n < 1 || !x || !out) return fail(FAM_ERR_INVALID_ARG, "need n >= 1 and non-null x and out");
  if (!(k > 0.0) || !(k < (double)n)) return fail(FAM_ERR_INVALID_ARG, "need 0 < k < n (got k = %g, n = %d)", k, n);
  if (!(tau > 0.0) || !std::isfinite(tau)) return fail(FAM_ERR_INVALID_ARG, "tau must be finite and > 0");
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(x[i])) return fail(FAM_ERR_INVALID_ARG, "x[%d] is not finite", i);
  // z = x / tau in decreasing order
  std::vector<double> z(n);
  for (int i = 0; i < n; ++i) z[i] = x[i] / tau;
  std::sort(z.begin(), z.end(), [](double a, double b) { return a > b; });
  // log S1(m) = log sum_{i<m} exp(-z_i) and log S2(m) = log sum_{i>=m} exp(z_i)
  auto lae = [](double a, double b) {   // log(exp(a) + exp(b))
    if (a == -HUGE_VAL) return b;
    if (b == -HUGE_VAL) return a;
    const double hi = a > b ? a : b, lo = a > b ? b : a;
    return hi + std::log1p(std::exp(lo - hi));
  };
  std::vector<double> ls1(n + 1), ls2(n + 1);
  ls1[0] = -HUGE_VAL;
  for (int m = 1; m <= n; ++m) ls1[m] = lae(ls1[m - 1], -z[m - 1]);
  ls2[n] = -HUGE_VAL;
  for (int m = n - 1; m >= 0; --m) ls2[m] = lae(ls2[m + 1], z[m]);
  // With m entries at or above lambda the masks sum to
  // m - e^lambda S1 / 2 + e^-lambda S2 / 2; setting that to k gives a
  // quadratic in e^lambda. Exactly one m is consistent with its own lambda.
  double lam = 0.0;
  bool found = false;
  for (int m = 0; m <= n && !found; ++m) {
    const double a = k - m;
    double l;
    if (m == 0) {
      l = ls2[0] - std::log(2.0 * k);
    } else if (m == n) {
      l = std::log(2.0 * (n - k)) - ls1[n];
    } else if (a > 0) {   // e^lambda = S2 / (sqrt(a^2 + S1 S2) + a)
      const double root = 0.5 * lae(2.0 * std::log(a), ls1[m] + ls2[m]);
      l = ls2[m] - lae(root, std::log(a));
    } else if (a < 0) {   // e^lambda = (sqrt(a^2 + S1 S2) - a) / S1
      const double root = 0.5 * lae(2.0 * std::log(-a), ls1[m] + ls2[m]);
      l = lae(root, std::log(-a)) - ls1[m];
    } else {
      l = 0.5 * (ls1[m] + ls2[m]) - ls1[m];
    }
    if ((m == 0 || z[m - 1] >= l) && (m == n || l > z[m])) {
      lam = l;
      found = true;
    }
  }
  if (!found) return fail(FAM_ERR_INVALID_ARG, "no consistent threshold (degenerate input)");
  for (int i = 0; i < n; ++i) {
    const double u = x[i] / tau - lam;
    out[i] = u >= 0.0 ? 1.0 - 0.5 * std::exp(-u) : 0.5 * std::exp(u);
  }
  return ok();
}

}  // extern "C"

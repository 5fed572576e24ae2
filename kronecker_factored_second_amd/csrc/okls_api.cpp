// Host side of the batched OKLS / Shampoo preconditioner step: argument
// validation, workspace layout, launch planning and the C ABI of okls.h.
//
// One okls_step enqueues, per chunk of matrices, this fixed sequence
// (all launches grouped over every matrix / factor of the chunk):
//   stats(G, N, P_old)  -> cast(G16, G16^T, N16 [+ M update], P16_old)
//   GEMM  X_a = G P_b, X_b^T = G^T P_a          (OKLS only)
//   stats -> cast(X16)                          (OKLS only)
//   GEMM  S <- c0 S + c1 X X^T + eps I          (upper tiles, mirrored)
//   stats(S) -> cast(Y_0 = S/c, Z_1 = a_0 I + b_0 S/c)
//   GEMM  Newton-Schulz: 1 + 3*(K-2) + 2 GEMMs per root in 2K-1 launches
//         (Shampoo: a second chain on the first chain's square root)
//   GEMM  V^T = P_b N^T -> stats -> cast
//   GEMM  U = P_a V with the fused update W <- decay W - lr c_shape U
// The order is the "Online KL Shampoo" README's "How it works": factors
// with the previous preconditioners, fresh roots, whitening, update.
// The Nystrom mode (plan_nys) keeps low-rank factors refreshed by the Clean
// paper's Algorithm 3 and preconditions the momentum with P^-1/2 (fp32).
// The SOAP mode (plan_soap) runs the Clean paper's Algorithm 4 instead:
// rotations into the eigenbasis, the Adam kernel, the rotation back with the
// fused update, the factor EMAs, and on refresh steps Q^T S Q followed by
// block Jacobi sweeps on it that rotate the bases in place.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <limits>
#include <map>
#include <new>
#include <string>
#include <vector>

#include "../../include/okls.h"
#include "okls_kernels.h"

using namespace okls;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDim = 32768;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
// Sides up to 512 pad to 128, larger ones to 256 (so the 256 tile applies).
int pad_tile(int x) {
  const int u = x > kBigPadFrom ? kBigTile : kTile;
  return (x + u - 1) / u * u;
}

// ---------------------------------------------------------------------------
// Newton-Schulz coefficients.  The README ("How it works" and the intro
// list) names Chebyshev-optimised coefficients with deterministic per-step
// scales for a 10-step coupled iteration but prints no values.  Reading
// taken here: each step k applies sigma -> sigma (a_k + b_k sigma^2) to every
// eigen-direction of Z_k Y_k = sigma^2; (a_k, b_k) is the odd cubic with the
// least maximum deviation from 1 on the current interval [lo, hi].  With
// equal deviation E at lo, at the interior maximum x* and at hi:
//   a = -b (hi^2 + hi lo + lo^2),  x*^2 = (hi^2 + hi lo + lo^2) / 3,
//   b = -2 / (2 x*^3 + lo hi (lo + hi)),  E = -2 b x*^3 - 1.
// Every step except the last is divided by (1 + E) so the next interval is
// [(1 - E)/(1 + E), 1] and no iterate's spectrum exceeds 1 (the fp16 range
// guard); the last is left unscaled so the result is centred on 1.
// ---------------------------------------------------------------------------
void ns_table(double floor, int steps, std::vector<double>& a, std::vector<double>& b, double* final_err) {
  a.assign(steps, 0.0);
  b.assign(steps, 0.0);
  double lo = floor, hi = 1.0, err = 0.0;
  for (int k = 0; k < steps; ++k) {
    const double q = hi * hi + hi * lo + lo * lo;
    const double xs = std::sqrt(q / 3.0);
    double bk = -2.0 / (2.0 * xs * xs * xs + lo * hi * (lo + hi));
    double ak = -bk * q;
    err = -2.0 * bk * xs * xs * xs - 1.0;
    if (k < steps - 1) {
      ak /= (1.0 + err);
      bk /= (1.0 + err);
      lo = (1.0 - err) / (1.0 + err);
      hi = 1.0;
    }
    a[k] = ak;
    b[k] = bk;
  }
  if (final_err) *final_err = err;
}

// The table a handle uses: the minimax table above, or (ns_classical) the
// classical Newton-Schulz step T = (3 I - Z Y) / 2 at every step.
void coeff_table(const okls_config& c, std::vector<double>& a, std::vector<double>& b) {
  if (c.ns_classical) {
    a.assign(c.ns_steps, 1.5);
    b.assign(c.ns_steps, -0.5);
    return;
  }
  ns_table(c.ns_floor, c.ns_steps, a, b, nullptr);
}

float pow2_for_bound(double bound) {   // largest 2^e with bound * 2^e <= 2^kScaleExp
  const int e = kScaleExp - static_cast<int>(std::ceil(std::log2(std::max(bound, 1e-30))));
  return std::ldexp(1.0f, e);
}

struct FacBufs {
  int d = 0, dp = 0, ld = 0, ldw = 0;
  size_t Y[2] = {0, 0}, Z[2] = {0, 0}, T = 0, R32 = 0;
  size_t P16w = 0;   // the root's fp16 copy (ld ldw) the cross-preconditioning and whitening read
  size_t YT[2] = {0, 0}, ZT[2] = {0, 0}, TT = 0;   // transposed copies
  int s_pold = 0, s_cinv = 0, s_rho = 0, s_sqrtc = 0, s_p16 = 0;
  int s_cinv2 = 0, s_rho2 = 0, s_sqrtc2 = 0;
  // SOAP: the basis' fp16 copies (ld), the factor's copy, (Q^T S)^T = Q^T S
  // as fp16, Q^T S Q in fp32 (d x d) and the Jacobi rotations of a round
  size_t Q16 = 0, Q16T = 0, L16 = 0, HT16 = 0, B32 = 0, jbuf = 0;
  int ldq = 0;   // row stride of those four: [hi | lo] always (the refresh's last products are split)
  int s_l = 0, s_lx = 0;
  int mat = -1, side = 0;   // the matrix (in group order) and side this factor belongs to
};

struct MatBufs {
  int group = 0, index = 0, m = 0, n = 0, mp = 0, np = 0, ldm = 0, ldn = 0;
  int ldmw = 0, ldnw = 0;   // strides of the whitening operands N16 (ldnw) and VT16 (ldmw)
  size_t G16 = 0, G16T = 0, N16 = 0, Xa32 = 0, XbT32 = 0, Xa16 = 0, XbT16 = 0, VT32 = 0, VT16 = 0;
  int s_g = 0, s_n = 0, s_xa = 0, s_xb = 0, s_vt = 0;
  FacBufs fa, fb;
  // Muon: N^T, the iterates X_k and X_k^T, the Gram of the smaller side (p x p)
  int pd = 0, pdp = 0, ldp = 0;
  size_t NT16 = 0, X[2] = {0, 0}, XT[2] = {0, 0}, A32 = 0, A16 = 0;
  int s_gcinv = 0, s_grho = 0;
  // SOAP: M' fp16, (G Q_b)^T and (M Q_b)^T fp16, G' and M' fp32, N' fp16, (N' Q_b^T)^T fp16
  size_t M16 = 0, XGT16 = 0, XMT16 = 0, Gr32 = 0, Mr32 = 0, NP16 = 0, ZT16 = 0;
  int s_m = 0, s_gx = 0, s_mx = 0;
  // Nystrom: the momentum N (fp32); XU = [X | U_a E_a] (m x (r_b + r_a)) with X = N U_b;
  // ZB = [(U_b E_b)^T ; Z] ((r_b + r_a) x n) with Z = U_a^T N + (U_a^T X) (U_b E_b)^T;
  // Ct = (U_a^T X)^T (r_b x r_a)
  size_t N32 = 0, XU = 0, ZB = 0, Ct = 0;
  struct NysSide {
    int d = 0, k = 0, r = 0;           // side, sketch columns, kept eigenpairs
    size_t Om = 0, Yb = 0, Fb = 0, T1 = 0, T2 = 0, gram = 0, cm = 0, zp = 0, kout = 0, scratch = 0;
    int s_nu = 0, s_nuu = 0;
  } ns[2];
};

enum LaunchType { L_STAT = 0, L_CAST = 1, L_GEMM = 2, L_FORK = 3, L_JOIN = 4, L_SYM = 5, L_ADAM = 6, L_JAC = 7,
                  L_NORTH = 9, L_NSMALL = 10, L_NELEM = 11, L_THIN = 12 };

struct LaunchRec {
  int type = L_STAT;
  int first = 0, count = 0;     // jobs (stat/cast) or tiles (gemm)
  int nblocks = 0;
  int blk_offset = 0;
  int prob_base = 0;
  int split_in = 0, write_lo = 0;
  float ka = 0.f, kb = 0.f;
  int cat = 0;                  // profiling category
  int tile = kTile;             // GEMM block tile
  int epi = EPI_STORE32;        // GEMM epilogue kind (one per launch)
  int stream = 0;               // 0: the caller's stream; 1: the library's side stream (between a fork and a join)
  int jac_kind = 0, round = 0;  // L_JAC: JacKind and tournament round
  size_t jac_part = 0, jac_flag = 0;   // L_JAC: workspace offsets of the chunk's partials and flags
  int thin_ta = 0, thin_mom = 0;       // L_THIN: the launch's operand form
  int thin_cbm = 1;                    // L_THIN: 32-column blocks of C the kernel holds (1, 2 or 4)
  int thin_wupd = 0;                   // L_THIN: the weight-update form (every job wupd)
};

enum { CAT_NS = 0, CAT_FACTOR = 1, CAT_WHITEN = 2, CAT_STAT = 3, CAT_CAST = 4, CAT_EIG = 5 };

// The factors' Newton-Schulz chains are independent: they run as two chains
// of launches, one on the caller's stream and one on a side stream, so one
// chain's launches fill the CUs the other's leave idle in their last round.
#ifndef OKLS_NS_STREAMS
#define OKLS_NS_STREAMS 2
#endif
constexpr int kNsStreams = OKLS_NS_STREAMS;

// Global scale slots.  SOAP adds SL_Q (the bases' static fp16 scale), SL_NP
// (the Adam direction's) and SL_ZT + e (the direction's scale / 2^e, e =
// ceil(log2 sqrt(n)): the rotated direction (N' Q_b^T)^T, whose rows have
// Euclidean norm at most sqrt(n) max|N'|); its chunk slots start after them.
enum { SL_ONE = 0, SL_Y = 1, SL_Z = 2, SL_T = 3, SL_FIRST_DYN = 4 };
enum { SL_Q = 4, SL_NP = 5, SL_ZT = 6, kZtSlots = 16, SL_FIRST_DYN_SOAP = SL_ZT + kZtSlots };

Ref ws_ref(size_t off) { return Ref{REF_WS, 0, static_cast<int64_t>(off)}; }
Ref user_ref(int kind, int group, size_t byte_off) { return Ref{kind, group, static_cast<int64_t>(byte_off)}; }
Ref no_ref() { return Ref{REF_NONE, 0, 0}; }

bool env_fault(const char* call) {
  const char* f = std::getenv("OKLS_FAULT");
  return f != nullptr && std::strcmp(f, call) == 0;
}

}  // namespace

struct okls_handle {
  okls_config cfg{};
  std::vector<okls_group_desc> groups;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  size_t off_probs = 0, off_tiles = 0, off_stat = 0, off_cast = 0, off_sym = 0, off_scal = 0, off_part = 0, off_flag = 0;
  size_t off_adam = 0, off_jac = 0, off_north = 0, off_nsmall = 0, off_nelem = 0, off_thin = 0;
  size_t off_resid = 0, resid_floats = 0;   // Newton-Schulz residual partials
  struct Resid { int mat, side, chain, first, count; };
  std::vector<Resid> resid;
  int n_mats = 0;
  float s_np = 1.0f;                        // SOAP: static scale of the Adam direction
  std::vector<std::vector<LaunchRec>> chunks;        // steps that recompute the roots
  std::vector<std::vector<LaunchRec>> chunks_stale;  // steps that keep them
  std::vector<double> na, nb;
  double step_flops[OKLS_PROFILE_CATEGORIES] = {};
  double step_bytes[OKLS_PROFILE_CATEGORIES] = {};
  double step_flops_stale[OKLS_PROFILE_CATEGORIES] = {};
  double step_bytes_stale[OKLS_PROFILE_CATEGORIES] = {};
  // profiling
  bool prof = false;
  std::vector<hipEvent_t> events;           // pool
  std::vector<std::pair<int, int>> pending; // (category, event pair index) of unread launches
  size_t next_event = 0;
  okls_profile_stats acc{};
  // side streams of the Newton-Schulz chains after the first, the fork event
  // and one join event per side stream (created by okls_init when the plan
  // forks; default priority)
  std::vector<hipStream_t> side;
  hipEvent_t ev_fork = nullptr;
  std::vector<hipEvent_t> ev_join;
  size_t part_stride = 0;                   // floats between the streams' partial regions
  ~okls_handle() {
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    if (ev_fork != nullptr) (void)hipEventDestroy(ev_fork);
    for (hipEvent_t e : ev_join) (void)hipEventDestroy(e);
    for (hipStream_t x : side) (void)hipStreamDestroy(x);
  }
};

namespace {

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------
okls_status check_config(const okls_config* c) {
  if (c == nullptr) return OKLS_ERR_INVALID_ARG;
  if (c->mode != OKLS_MODE_OKLS && c->mode != OKLS_MODE_SHAMPOO && c->mode != OKLS_MODE_MUON && c->mode != OKLS_MODE_SOAP &&
      c->mode != OKLS_MODE_NYSTROM)
    return OKLS_ERR_INVALID_ARG;
  if (c->ns_steps < 2 || c->ns_steps > 16) return OKLS_ERR_INVALID_ARG;
  if (c->ns_split_steps < 0 || c->ns_split_steps > c->ns_steps) return OKLS_ERR_INVALID_ARG;
  if (c->factor_split != 0 && c->factor_split != 1) return OKLS_ERR_INVALID_ARG;
  if (c->whiten_split != 0 && c->whiten_split != 1) return OKLS_ERR_INVALID_ARG;
  if (c->nesterov_var_corr != 0 && c->nesterov_var_corr != 1) return OKLS_ERR_INVALID_ARG;
  if (c->chunk_matrices < 0) return OKLS_ERR_INVALID_ARG;
  if (!(c->beta1 >= 0.f && c->beta1 < 1.f)) return OKLS_ERR_INVALID_ARG;
  if (c->mode == OKLS_MODE_OKLS && !(c->beta2 >= 0.f && c->beta2 < 1.f)) return OKLS_ERR_INVALID_ARG;
  if (!(c->eps >= 0.f && std::isfinite(c->eps))) return OKLS_ERR_INVALID_ARG;
  if (!(c->weight_decay >= 0.f && std::isfinite(c->weight_decay))) return OKLS_ERR_INVALID_ARG;
  if (!(c->lr_peak > 0.f && std::isfinite(c->lr_peak))) return OKLS_ERR_INVALID_ARG;
  if (!(c->ns_floor > 0.f && c->ns_floor < 1.f)) return OKLS_ERR_INVALID_ARG;
  if (!(c->ns_damping >= 0.f && c->ns_damping < 1.f)) return OKLS_ERR_INVALID_ARG;
  if (c->root_period < 1) return OKLS_ERR_INVALID_ARG;
  if ((c->eps_convex | c->decay_after | c->shape_scale | c->ns_classical) & ~1) return OKLS_ERR_INVALID_ARG;
  if (c->mode == OKLS_MODE_SOAP) {
    if (!(c->beta2 >= 0.f && c->beta2 < 1.f) || !(c->soap_beta >= 0.f && c->soap_beta < 1.f)) return OKLS_ERR_INVALID_ARG;
    if (!(c->eps > 0.f)) return OKLS_ERR_INVALID_ARG;      // the direction divides by sqrt(V) + eps
    if (c->precond_freq < 1 || ((c->soap_moments | c->bias_correction) & ~1)) return OKLS_ERR_INVALID_ARG;
    if (c->jacobi_sweeps < 1 || c->jacobi_sweeps > 64 || !(c->jacobi_tol > 0.f && c->jacobi_tol < 1.f))
      return OKLS_ERR_INVALID_ARG;
    if (c->jacobi_apply_tiles != 0 && c->jacobi_apply_tiles != 1 && c->jacobi_apply_tiles != kJacApplyItems)
      return OKLS_ERR_INVALID_ARG;
    // the direction is bounded (and its fp16 operand can take a static scale)
    // only when beta1^2 < beta2, or beta1 = 0
    if (!(c->beta1 == 0.f || static_cast<double>(c->beta1) * c->beta1 < c->beta2)) return OKLS_ERR_UNSUPPORTED;
  }
  if (c->mode == OKLS_MODE_NYSTROM) {
    if (!(c->beta2 >= 0.f && c->beta2 < 1.f)) return OKLS_ERR_INVALID_ARG;
    if (!(c->eps > 0.f)) return OKLS_ERR_INVALID_ARG;      // P^-1/2 divides by lambda + eps
    if (c->nys_rank < 1 || c->nys_oversample < 0 || c->nys_passes < 0 || c->nys_passes > 8) return OKLS_ERR_INVALID_ARG;
    if (c->nys_rank + c->nys_oversample > kNysMaxK) return OKLS_ERR_UNSUPPORTED;
  }
  return OKLS_OK;
}

// Largest |N'| the Adam direction can take.  By Cauchy-Schwarz on the two
// EMAs of step t, |sum_k a_k g_k| <= sqrt(sum_k a_k^2 / b_k) sqrt(sum_k b_k g_k^2)
// with a_k = (1-beta1) beta1^k and b_k = (1-beta2) beta2^k (k < t), so
// |M'| / sqrt(V) <= (1-beta1) / sqrt(1-beta2) sqrt(sum_{k<t} (beta1^2/beta2)^k),
// times sqrt(1-beta2^t) / (1-beta1^t) with bias correction; eps only lowers
// it.  The supremum over t (dense to 2000, then geometric, then the limit).
double adam_ratio_bound(const okls_config& c) {
  const double b1 = c.beta1, b2 = c.beta2;
  if (b2 == 0.0) return 1.0;                  // then beta1 = 0: |G'| / (|G'| + eps)
  const double r = b1 * b1 / b2;
  auto at = [&](double t) {
    const double sum = r == 0.0 ? 1.0 : (1.0 - std::pow(r, t)) / (1.0 - r);
    double v = (1.0 - b1) / std::sqrt(1.0 - b2) * std::sqrt(sum);
    if (c.bias_correction) v *= std::sqrt(1.0 - std::pow(b2, t)) / (1.0 - std::pow(b1, t));
    return v;
  };
  double best = at(1.0);
  for (double t = 2.0; t < 1e9; t = t < 2000.0 ? t + 1.0 : std::floor(t * 1.01)) best = std::max(best, at(t));
  best = std::max(best, (1.0 - b1) / std::sqrt((1.0 - b2) * (1.0 - r)));
  return best;
}

okls_status check_groups(int n_groups, const okls_group_desc* g) {
  if (g == nullptr) return OKLS_ERR_INVALID_ARG;
  if (n_groups < 1 || n_groups > kMaxGroups) return OKLS_ERR_SHAPE;
  for (int i = 0; i < n_groups; ++i) {
    if (g[i].batch < 1 || g[i].m < 1 || g[i].n < 1 || g[i].m > kMaxDim || g[i].n > kMaxDim) return OKLS_ERR_SHAPE;
    if (g[i].g_dtype != OKLS_F32 && g[i].g_dtype != OKLS_BF16 && g[i].g_dtype != OKLS_F16) return OKLS_ERR_DTYPE;
  }
  return OKLS_OK;
}

// ---------------------------------------------------------------------------
// Planner
// ---------------------------------------------------------------------------
// The planner's description of a product C = alpha op(A) B (+ beta C),
// op(A) M x K (A stored K x M when ta), rows of C scaled by an optional
// vector; every such product runs as a ThinJob (N <= kThinMaxR).
struct ProdDesc {
  Ref A, B, C;
  int32_t M, N, K;
  int32_t lda, ldb, ldc;   // row strides in elements
  int32_t ta;              // op(A) = A^T (A stored K x M)
  int32_t a_fmt;           // GradFmt of A (fp32 except a gradient)
  float alpha;
  int32_t alpha_slot;      // >= 0: alpha is multiplied by scal[alpha_slot]
  float beta;              // 0: C is written without being read
  Ref rowscale;            // REF_NONE, or M floats: row i of the product times rowscale[i]
};

struct Planner {
  const okls_config& cfg;
  const std::vector<okls_group_desc>& groups;
  bool okls_mode;
  bool muon_mode;
  bool soap_mode;
  bool nys_mode;
  bool lo_layout;
  bool single_chain = false;   // never plan a second Newton-Schulz chain (no side stream)
  std::vector<double> na, nb;
  float sY = 0, sZ = 0, sT = 0;

  // tables
  std::vector<GemmProb> probs;
  std::vector<TileRef> tiles;
  std::vector<StatJob> stat_jobs;
  std::vector<CastJob> cast_jobs;
  std::vector<SymJob> sym_jobs;
  std::vector<AdamJob> adam_jobs;
  std::vector<JacJob> jac_jobs;
  std::vector<NysOrthJob> north_jobs;
  std::vector<NysSmallJob> nsmall_jobs;
  std::vector<NysElemJob> nelem_jobs;
  std::vector<ThinJob> thin_jobs;
  float s_np = 1.0f;          // SOAP: static scale of the Adam direction's fp16 operand
  std::vector<std::vector<LaunchRec>> chunks;        // steps that recompute the roots
  std::vector<std::vector<LaunchRec>> chunks_stale;  // steps that keep them (root_period > 1)
  std::map<std::string, std::pair<int, int>> tile_cache;

  std::vector<std::map<size_t, size_t>> ws_bufs;   // per chunk: workspace buffer offset -> bytes
  size_t chunk_bytes = 0;     // per-chunk buffer region size (max over chunks)
  int n_slots = SL_FIRST_DYN; // max over chunks
  int first_dyn = SL_FIRST_DYN;
  int max_partials = 1;
  // Newton-Schulz residual partials: per (matrix, side, chain) a range of
  // floats in the residual region, of which the last T launch writes count
  struct ResidSlot { int mat, side, chain, first, count; };
  std::vector<ResidSlot> resid_slots;
  int resid_floats = 0;
  std::vector<int> mat_base;   // first matrix of each group (group order)

  Planner(const okls_config& c, const std::vector<okls_group_desc>& g)
      : cfg(c), groups(g), okls_mode(c.mode == OKLS_MODE_OKLS), muon_mode(c.mode == OKLS_MODE_MUON),
        soap_mode(c.mode == OKLS_MODE_SOAP), nys_mode(c.mode == OKLS_MODE_NYSTROM),
        lo_layout(c.factor_split != 0 || c.ns_split_steps > 0) {
    if (soap_mode) {
      first_dyn = n_slots = SL_FIRST_DYN_SOAP;
      s_np = pow2_for_bound(adam_ratio_bound(cfg));
    }
    coeff_table(cfg, na, nb);
    int nm = 0;
    for (const okls_group_desc& gd : groups) { mat_base.push_back(nm); nm += gd.batch; }
    double prod = 1.0, amax = 0.0;
    for (int k = 0; k < cfg.ns_steps; ++k) {
      prod *= std::max(std::fabs(na[k]), std::fabs(na[k] + nb[k]));
      amax = std::max(amax, std::max(std::fabs(na[k]), std::fabs(na[k] + nb[k])));
    }
    sY = pow2_for_bound(1.0);
    sZ = pow2_for_bound(prod);
    sT = pow2_for_bound(amax);
  }

  int ld_for(int dp) const { return lo_layout ? 2 * dp : dp; }
  // rows of a buffer hold [hi | lo] only where a split product reads it: the
  // factor operands, the Newton-Schulz iterates and the whitening operands
  int ld_fac(int dp) const { return cfg.factor_split ? 2 * dp : dp; }
  int ld_ns(int dp) const { return cfg.ns_split_steps > 0 ? 2 * dp : dp; }
  int ld_wh(int dp) const { return wsplit() ? 2 * dp : dp; }
  // relative shift of the rooted matrix: delta = nu / sqrt(d)
  float damping(int d) const { return static_cast<float>(cfg.ns_damping / std::sqrt(static_cast<double>(d))); }

  // lays out one chunk's buffers from offset 0 (relative); returns size
  std::vector<std::pair<size_t, size_t>> pending;   // chunk-relative buffers of the chunk being laid out
  size_t jac_part_rel = 0, jac_flag_rel = 0;   // SOAP: chunk-relative Jacobi partials and flags
  size_t layout_chunk(std::vector<MatBufs>& mats, int& slot) {
    size_t off = 0;
    pending.clear();
    auto take = [&](size_t bytes) {
      size_t o = off;
      off = align_up(off + bytes, kAlign);
      pending.push_back({o, bytes});
      return o;
    };
    if (nys_mode) {
      for (MatBufs& mb : mats) {
        const okls_group_desc& g = groups[mb.group];
        mb.m = g.m; mb.n = g.n;
        const size_t mn = static_cast<size_t>(g.m) * g.n * 4;
        mb.N32 = take(mn);
        const int ra = nys_r(g.m), rb = nys_r(g.n);
        mb.XU = take(static_cast<size_t>(g.m) * (rb + ra) * 4);
        mb.ZB = take(static_cast<size_t>(rb + ra) * g.n * 4);
        mb.Ct = take(static_cast<size_t>(rb) * ra * 4);
        for (int sd = 0; sd < 2; ++sd) {
          MatBufs::NysSide& S = mb.ns[sd];
          S.d = sd == 0 ? g.m : g.n;
          S.k = nys_k(S.d);
          S.r = nys_r(S.d);
          const int other = sd == 0 ? g.n : g.m;
          const size_t dk = static_cast<size_t>(S.d) * S.k * 4, kk = static_cast<size_t>(S.k) * S.k * 4,
                       kr = static_cast<size_t>(S.k) * S.r * 4;
          S.Om = take(dk); S.Yb = take(dk); S.Fb = take(dk);
          S.T1 = take(static_cast<size_t>(S.r) * S.k * 4); S.T2 = take(static_cast<size_t>(other) * S.k * 4);
          S.gram = take(kk); S.cm = take(kk); S.zp = take(kr); S.kout = take(kr);
          S.scratch = take(static_cast<size_t>(S.k) * S.k * 8 * 2);
          S.s_nu = slot++; S.s_nuu = slot++;
        }
      }
      return off;
    }
    if (soap_mode) {
      int parts = 0, flags = 0;
      auto sfac = [&](FacBufs& f, int d) {
        f.d = d; f.dp = pad_tile(d); f.ld = ld_fac(f.dp); f.ldq = 2 * f.dp;
        const size_t b16 = static_cast<size_t>(f.dp) * f.ldq * 2;
        f.Q16 = take(b16); f.Q16T = take(b16);
        f.L16 = take(b16); f.HT16 = take(b16);
        f.B32 = take(static_cast<size_t>(d) * d * 4);
        const int nb = jac_blocks(d), np = nb / 2;
        f.jbuf = take(static_cast<size_t>(np) * kJp * kJp * 4);
        parts += np * (np + 1) / 2;
        flags += 1;
        f.s_l = slot++; f.s_lx = slot++;
      };
      for (MatBufs& mb : mats) {
        const okls_group_desc& g = groups[mb.group];
        mb.m = g.m; mb.n = g.n; mb.mp = pad_tile(g.m); mb.np = pad_tile(g.n);
        mb.ldm = ld_fac(mb.mp); mb.ldn = ld_fac(mb.np);
        const size_t bmn = static_cast<size_t>(mb.mp) * mb.ldn * 2, bnm = static_cast<size_t>(mb.np) * mb.ldm * 2;
        const size_t f32 = static_cast<size_t>(mb.m) * mb.n * 4;
        mb.G16 = take(bmn); mb.G16T = take(bnm); mb.XGT16 = take(bnm); mb.Gr32 = take(f32);
        if (!cfg.soap_moments) { mb.M16 = take(bmn); mb.XMT16 = take(bnm); mb.Mr32 = take(f32); }
        mb.NP16 = take(bmn); mb.ZT16 = take(bnm);
        mb.s_g = slot++; mb.s_gx = slot++; mb.s_m = slot++; mb.s_mx = slot++; mb.s_n = slot++; mb.s_vt = slot++;
        sfac(mb.fa, g.m);
        sfac(mb.fb, g.n);
      }
      jac_part_rel = take(static_cast<size_t>(parts) * 2 * sizeof(float));
      jac_flag_rel = take(static_cast<size_t>(flags) * sizeof(int32_t));
      return off;
    }
    auto fac = [&](FacBufs& f, int d) {
      f.d = d; f.dp = pad_tile(d); f.ld = ld_ns(f.dp); f.ldw = ld_wh(f.dp);
      const size_t b16 = static_cast<size_t>(f.dp) * f.ld * 2;
      f.Y[0] = take(b16); f.Y[1] = take(b16); f.Z[0] = take(b16); f.Z[1] = take(b16); f.T = take(b16);
      f.YT[0] = take(b16); f.YT[1] = take(b16); f.ZT[0] = take(b16); f.ZT[1] = take(b16); f.TT = take(b16);
      f.P16w = take(static_cast<size_t>(f.dp) * f.ldw * 2);
      if (!okls_mode) f.R32 = take(static_cast<size_t>(d) * d * 4);
      f.s_pold = slot++; f.s_cinv = slot++; f.s_rho = slot++; f.s_sqrtc = slot++; f.s_p16 = slot++;
      f.s_cinv2 = slot++; f.s_rho2 = slot++; f.s_sqrtc2 = slot++;
    };
    for (MatBufs& mb : mats) {
      const okls_group_desc& g = groups[mb.group];
      mb.m = g.m; mb.n = g.n; mb.mp = pad_tile(g.m); mb.np = pad_tile(g.n);
      mb.ldm = ld_for(mb.mp); mb.ldn = ld_for(mb.np);
      if (muon_mode) {
        const size_t bx = static_cast<size_t>(mb.mp) * mb.ldn * 2, bxt = static_cast<size_t>(mb.np) * mb.ldm * 2;
        mb.pd = std::min(g.m, g.n); mb.pdp = pad_tile(mb.pd); mb.ldp = ld_for(mb.pdp);
        mb.N16 = take(bx); mb.NT16 = take(bxt);
        mb.X[0] = take(bx); mb.X[1] = take(bx); mb.XT[0] = take(bxt); mb.XT[1] = take(bxt);
        mb.A32 = take(static_cast<size_t>(mb.pd) * mb.pd * 4);
        mb.A16 = take(static_cast<size_t>(mb.pdp) * mb.ldp * 2);
        mb.s_n = slot++; mb.s_gcinv = slot++; mb.s_grho = slot++;
        continue;
      }
      mb.ldm = ld_fac(mb.mp); mb.ldn = ld_fac(mb.np);
      mb.ldmw = ld_wh(mb.mp); mb.ldnw = ld_wh(mb.np);
      mb.G16 = take(static_cast<size_t>(mb.mp) * mb.ldn * 2);
      mb.G16T = take(static_cast<size_t>(mb.np) * mb.ldm * 2);
      mb.N16 = take(static_cast<size_t>(mb.mp) * mb.ldnw * 2);
      if (okls_mode) {
        mb.Xa32 = take(static_cast<size_t>(mb.m) * mb.n * 4);
        mb.XbT32 = take(static_cast<size_t>(mb.n) * mb.m * 4);
        mb.Xa16 = take(static_cast<size_t>(mb.mp) * mb.ldn * 2);
        mb.XbT16 = take(static_cast<size_t>(mb.np) * mb.ldm * 2);
      }
      mb.VT32 = take(static_cast<size_t>(mb.n) * mb.m * 4);
      mb.VT16 = take(static_cast<size_t>(mb.np) * mb.ldmw * 2);
      mb.s_g = slot++; mb.s_n = slot++; mb.s_xa = slot++; mb.s_xb = slot++; mb.s_vt = slot++;
      fac(mb.fa, g.m);
      fac(mb.fb, g.n);
    }
    return off;
  }

  // Jacobi blocks of a side d: ceil(d / kJb), even (the round-robin pairs them all)
  static int jac_blocks(int d) {
    const int nb = (d + kJb - 1) / kJb;
    return nb + (nb & 1);
  }
  // e = ceil(log2 sqrt(k)): 2^-e bounds sqrt(k) from below by its reciprocal,
  // the scale factor of a product of an operand with k columns and an orthogonal matrix
  static int sqrt_exp(int k) { return static_cast<int>(std::ceil(0.5 * std::log2(static_cast<double>(k)) - 1e-12)); }

  // ---- tiles
  // Workgroup w of a launch runs on XCD w % 8.  Tiles are grouped into cost
  // classes (same K); each class's list (in locality order) is cut into 8
  // contiguous chunks, XCD x gets chunk x of every class (costliest class
  // first), and the per-XCD lists are dealt round-robin: every XCD gets the
  // same work and a contiguous band of each class for its L2.
  static std::vector<TileRef> xcd_order(const std::vector<TileRef>& t, const std::vector<GemmProb>& ps) {
    const size_t X = 8;
    std::map<int, std::vector<TileRef>, std::greater<int>> classes;   // by K, descending
    for (const TileRef& r : t) classes[ps[r.prob].Kp].push_back(r);
    std::vector<std::vector<TileRef>> per(X);
    for (auto& kv : classes) {
      const std::vector<TileRef>& c = kv.second;
      const size_t n = c.size();
      size_t s = 0;
      for (size_t x = 0; x < X; ++x) {
        const size_t len = n / X + (x < n % X ? 1 : 0);
        per[x].insert(per[x].end(), c.begin() + s, c.begin() + s + len);
        s += len;
      }
    }
    std::vector<TileRef> out;
    out.reserve(t.size());
    for (size_t y = 0; out.size() < t.size(); ++y)
      for (size_t x = 0; x < X; ++x)
        if (y < per[x].size()) out.push_back(per[x][y]);
    return out;
  }

  std::pair<int, int> tiles_for(const std::vector<GemmProb>& ps, bool upper, int bt) {
    std::string key = (upper ? "U" : "F") + std::to_string(bt);
    for (const GemmProb& p : ps) key += ":" + std::to_string(p.Mp) + "x" + std::to_string(p.Np);
    auto it = tile_cache.find(key);
    if (it != tile_cache.end()) return it->second;
    // per problem: bands of 8 tile rows, column-major inside a band, so the
    // 32 blocks an XCD runs at once share few operand row strips
    constexpr int kBand = 8;
    std::vector<TileRef> t;
    for (size_t q = 0; q < ps.size(); ++q) {
      const int tm = ps[q].Mp / bt, tn = ps[q].Np / bt;
      for (int i0 = 0; i0 < tm; i0 += kBand)
        for (int j = 0; j < tn; ++j)
          for (int i = i0; i < std::min(tm, i0 + kBand); ++i)
            if (!upper || j >= i) t.push_back(TileRef{static_cast<int32_t>(q), (i << 16) | j});
    }
    t = xcd_order(t, ps);
    const int first = static_cast<int>(tiles.size());
    tiles.insert(tiles.end(), t.begin(), t.end());
    const std::pair<int, int> r{first, static_cast<int>(t.size())};
    tile_cache[key] = r;
    return r;
  }

  int gemm_cat = CAT_NS;   // category of the GEMM launches being planned
  double step_flops[OKLS_PROFILE_CATEGORIES] = {0, 0, 0, 0, 0};
  double step_bytes[OKLS_PROFILE_CATEGORIES] = {0, 0, 0, 0, 0};
  double step_flops_stale[OKLS_PROFILE_CATEGORIES] = {0, 0, 0, 0, 0};
  double step_bytes_stale[OKLS_PROFILE_CATEGORIES] = {0, 0, 0, 0, 0};

  void add_gemm(std::vector<LaunchRec>& L, const std::vector<GemmProb>& ps, bool upper, int split_in,
                int write_lo, float ka = 0.f, float kb = 0.f) {
    if (ps.empty()) return;
    LaunchRec r;
    r.type = L_GEMM;
    r.cat = gemm_cat;
    r.prob_base = static_cast<int>(probs.size());
    for (GemmProb p : ps) {
      if (p.ld16T < 0) { p.ld16T = p.ld16; p.lo16T = p.lo16; }   // square problems: same layout
      probs.push_back(p);
    }
    // algorithmic bytes: both fp16 operands once (hi and lo halves when split),
    // every output and the fp32 matrix the epilogue reads, once
    for (const GemmProb& p : ps) {
      const double mn = static_cast<double>(p.M) * p.N;
      double b = 2.0 * (split_in ? 2.0 : 1.0) * (static_cast<double>(p.M) + p.N) * p.Kp;
      if (p.out32.kind != REF_NONE) b += 4.0 * mn;
      if (p.out16.kind != REF_NONE) b += (write_lo ? 4.0 : 2.0) * mn;
      if (p.out16T.kind != REF_NONE) b += (write_lo ? 4.0 : 2.0) * mn;
      const bool aux16 = p.epi == EPI_POLAR || p.epi == EPI_POLAR_UPDATE;
      if (p.aux.kind != REF_NONE) b += (aux16 ? (p.aux_lo >= 0 ? 4.0 : 2.0) : 4.0) * mn;
      step_bytes[gemm_cat] += b;
    }
    // one epilogue kind per launch (the kernel is specialised on it)
    r.epi = ps.front().epi;
    // the large tile when every problem's padded sides are multiples of it and
    // the launch has enough blocks of it: 64 for the fp16-output kinds
    // (measured faster than the 128 tile from a quarter of a block per CU on
    // up), 512 for the other fp32-output kinds (the factor update and the
    // whitening products, whose epilogues favour the 128 tile's second block
    // per CU below two blocks per CU); otherwise the 128 tile
    r.tile = kBigTile;
    long big_tiles = 0;
    for (const GemmProb& p : ps) {
      if (p.Mp % kBigTile || p.Np % kBigTile) r.tile = kTile;
      const long tm = p.Mp / kBigTile, tn = p.Np / kBigTile;
      big_tiles += upper ? tm * (tm + 1) / 2 : tm * tn;
    }
    const bool f16_out = r.epi == EPI_NS_T || r.epi == EPI_NS_T_RES || r.epi == EPI_NS_Y1 || r.epi == EPI_STORE16 || r.epi == EPI_NS_FINAL ||
                         r.epi == EPI_POLAR;
    // a Muon launch has no concurrent chain to fill a partly idle round: the
    // 256 tile only from one full round of it
    // the cross-preconditioning products X = G P (fp32 stores, no
    // read-modify-write) take it from 64 like the fp16 kinds
    const bool x_product = r.epi == EPI_STORE32 && gemm_cat == CAT_FACTOR;
    if (big_tiles < ((f16_out || x_product) ? (muon_mode ? 256 : 64) : 512)) r.tile = kTile;
    const std::pair<int, int> t = tiles_for(ps, upper, r.tile);
    r.first = t.first;
    r.count = t.second;
    r.split_in = split_in;
    r.write_lo = write_lo;
    r.ka = ka;
    r.kb = kb;
    L.push_back(r);
  }

  // ---- statistics: returns (part_begin, part_count) per job appended
  struct StatSpec { int kind; Ref src; int ld; Ref src2; int g_fmt; int rows, cols; };
  std::vector<std::pair<int, int>> add_stats(std::vector<LaunchRec>& L, const std::vector<StatSpec>& specs) {
    std::vector<std::pair<int, int>> parts;
    LaunchRec r;
    r.type = L_STAT;
    r.cat = CAT_STAT;
    r.first = static_cast<int>(stat_jobs.size());
    int blk = 0, part = 0;
    for (const StatSpec& s : specs) {
      StatJob j{};
      j.kind = s.kind; j.src = s.src; j.src_ld = s.ld; j.src2 = s.src2; j.g_fmt = s.g_fmt;
      j.rows = s.rows; j.cols = s.cols;
      // about 16K elements per block: twice the blocks the chip holds at once
      // on the larger launches, so the scheduler balances their tails
      j.rows_per_blk = std::max(1, std::min(s.rows, 16384 / std::max(1, s.cols)));
      // at most kMaxJobParts partials per job: every cast block of the job combines them all
      j.rows_per_blk = std::max(j.rows_per_blk, (s.rows + kMaxJobParts - 1) / kMaxJobParts);
      const double src_b = s.kind == ST_F32 ? 4.0 : s.kind == ST_H16 ? 2.0 : 4.0 + (s.g_fmt == GF_F32 ? 4.0 : 2.0);
      step_bytes[CAT_STAT] += src_b * s.rows * s.cols;
      const int nb = (s.rows + j.rows_per_blk - 1) / j.rows_per_blk;
      j.part_begin = part;
      j.blk_begin = blk;
      parts.push_back({part, nb});
      part += nb;
      blk += nb;
      stat_jobs.push_back(j);
    }
    r.count = static_cast<int>(specs.size());
    r.nblocks = blk;
    max_partials = std::max(max_partials, part);
    if (!specs.empty()) L.push_back(r);
    return parts;
  }

  struct CastSpec {
    int kind; Ref src; int src_ld; Ref src2; int g_fmt; int write_m; int transpose;
    int rows, cols, dst_rows_p, dst_cols_p; Ref dst; int dst_ld; int dst_lo;
    std::pair<int, int> parts; int scale_mode; int scale_slot;
    int cinv_slot, rho_slot, sqrtc_slot, p16_slot, p16_inv_sqrt; int write_lo; float damp; int sym_read;
    Ref dst2; int scale_slot2; int write_lo2;
    Ref dstT; int dstT_ld; int dstT_lo;
    int aux_slot; float aux_mul;
  };
  CastSpec cast_spec() {
    CastSpec c{};
    c.src2 = no_ref();
    c.dst = no_ref();
    c.dst2 = no_ref();
    c.dstT = no_ref();
    c.cinv_slot = c.rho_slot = c.sqrtc_slot = c.p16_slot = c.scale_slot2 = c.aux_slot = -1;
    c.aux_mul = 1.0f;
    return c;
  }
  void add_cast(std::vector<LaunchRec>& L, const std::vector<CastSpec>& specs, float ka = 0.f, float kb = 0.f) {
    if (specs.empty()) return;
    LaunchRec r;
    r.type = L_CAST;
    r.cat = CAT_CAST;
    r.first = static_cast<int>(cast_jobs.size());
    int blk = 0;
    for (const CastSpec& s : specs) {
      CastJob j{};
      j.kind = s.kind; j.src = s.src; j.src_ld = s.src_ld; j.src2 = s.src2; j.g_fmt = s.g_fmt;
      j.write_m = s.write_m; j.transpose = s.transpose; j.rows = s.rows; j.cols = s.cols;
      j.dst_rows_p = s.dst_rows_p; j.dst_cols_p = s.dst_cols_p; j.dst = s.dst; j.dst_ld = s.dst_ld;
      j.dst_lo = s.dst_lo; j.part_begin = s.parts.first; j.part_count = s.parts.second;
      j.scale_mode = s.scale_mode; j.scale_slot = s.scale_slot; j.cinv_slot = s.cinv_slot;
      j.rho_slot = s.rho_slot; j.sqrtc_slot = s.sqrtc_slot; j.p16_slot = s.p16_slot;
      j.p16_static = s.p16_inv_sqrt ? sY : sZ / 16.0f; j.p16_inv_sqrt = s.p16_inv_sqrt; j.write_lo = s.write_lo; j.damp = s.damp; j.sym_read = s.sym_read;
      j.dst2 = s.dst2; j.scale_slot2 = s.scale_slot2; j.write_lo2 = s.write_lo2;
      j.dstT = s.dstT; j.dstT_ld = s.dstT_ld; j.dstT_lo = s.dstT_lo;
      j.aux_slot = s.aux_slot; j.aux_mul = s.aux_mul;
      j.tiles_x = (s.dst_cols_p + kCastCols - 1) / kCastCols;
      const double src_b = s.kind == CA_H16 ? 2.0
                         : s.kind == CA_NESTEROV ? 4.0 + (s.g_fmt == GF_F32 ? 4.0 : 2.0) + (s.write_m ? 4.0 : 0.0)
                         : 4.0;
      const double dst2_b = s.dst2.kind == REF_NONE ? 0.0 : s.write_lo2 ? 4.0 : 2.0;
      const double dstT_b = s.dstT.kind == REF_NONE ? 0.0 : s.write_lo ? 4.0 : 2.0;
      step_bytes[CAT_CAST] += (src_b + (s.write_lo ? 4.0 : 2.0) + dst2_b + dstT_b) * s.rows * s.cols;
      j.blk_begin = blk;
      blk += j.tiles_x * (s.dst_rows_p / kCastRows);
      cast_jobs.push_back(j);
    }
    r.count = static_cast<int>(specs.size());
    r.nblocks = blk;
    r.ka = ka;
    r.kb = kb;
    L.push_back(r);
  }

  // ---- root symmetrisation: P <- (P + P^T) / 2 in place for each factor of
  // a chain, with the fp16 copy the whitening reads (scale slot s_p16)
  void add_sym(std::vector<LaunchRec>& L, const std::vector<FacBufs*>& facs, const std::vector<Ref>& pdst) {
    LaunchRec r;
    r.type = L_SYM;
    r.cat = CAT_CAST;
    r.first = static_cast<int>(sym_jobs.size());
    int blk = 0;
    for (size_t f = 0; f < facs.size(); ++f) {
      const FacBufs& F = *facs[f];
      SymJob j{};
      j.p = pdst[f]; j.d = F.d; j.dp = F.dp; j.nt = F.dp / kSymTile;   // the padded side: zeros beyond d
      j.dst16 = ws_ref(F.P16w); j.ld16 = F.ldw; j.lo16 = F.dp; j.write_lo = wsplit();
      j.scale_slot = F.s_p16; j.blk_begin = blk;
      blk += j.nt * (j.nt + 1) / 2;
      step_bytes[CAT_CAST] += (8.0 + (j.write_lo ? 4.0 : 2.0)) * static_cast<double>(F.d) * F.d;
      sym_jobs.push_back(j);
    }
    r.count = static_cast<int>(facs.size());
    r.nblocks = blk;
    if (!facs.empty()) L.push_back(r);
  }

  // split-fp16 whitening products (and the lo halves of the operands they read)
  int wsplit() const { return (cfg.factor_split || cfg.whiten_split) ? 1 : 0; }
  // SOAP: every product split-fp16 with factor_split
  bool wsplit_soap() const { return cfg.factor_split != 0; }

  // eps term of every factor update: + eps I (R1), or (1 - beta2) eps I in
  // the convex form of the OKLS update
  float factor_eps() const {
    return (okls_mode && cfg.eps_convex) ? static_cast<float>((1.0 - cfg.beta2) * cfg.eps) : cfg.eps;
  }
  // multiplier of lr U in the weight update: the muP c_shape = sqrt(m/n) /
  // (sqrt(m) + sqrt(n)), or 1 for the plain update (shape_scale = 0)
  float update_scale(const MatBufs& mb) const {
    if (!cfg.shape_scale) return 1.0f;
    const double m = mb.m, n = mb.n;
    return static_cast<float>(std::sqrt(m / n) / (std::sqrt(m) + std::sqrt(n)));
  }

  GemmProb prob() {
    GemmProb p{};
    p.A = p.B = p.out32 = p.out16 = p.out16T = p.aux = no_ref();
    p.s_out = -1;
    p.cslot = -1;
    p.ld16T = -1;
    p.aux_lo = -1;
    p.s_aux = -1;
    p.resid = -1;
    return p;
  }

  // Z_k^T: Z_1 = a_0 I + b_0 Y_0 is exactly symmetric (the cast writes one copy);
  // later Z_k come with a transposed copy from their GEMM.
  static size_t zt_of(const FacBufs& F, int k) { return k == 1 ? F.Z[1] : F.ZT[k & 1]; }

  // ---- Newton-Schulz chain for a list of factors.  Every product X W runs as
  // NT(X, W^T) on the transposed copy of W, so it is the plain product of the
  // iteration (no symmetry of the iterates is assumed: the coupled iteration
  // is only stable when Y and Z carry consistent rounding).  src(f) is the fp32
  // matrix being rooted (d x d, ld d); returns launches appended to L.
  // out OUT_INV: the inverse root Z_K / sqrt(c) into pdst (fp32);
  // out OUT_SQRT: the square root Y_K sqrt(c) into pdst.  With p16 the last
  // product also writes the output's fp16 copy into Z[K % 2] (Z_K s_Z or
  // Y_K s_Y), the operand the whitening reads, and the start cast records its
  // scale.  The Shampoo fourth root chains OUT_INV (into fac.R32, no copy)
  // and OUT_SQRT of that result.
  enum { OUT_INV = 0, OUT_SQRT = 1 };
  void ns_chain(std::vector<LaunchRec>& L, std::vector<FacBufs*>& facs, std::vector<Ref>& src,
                std::vector<Ref>& pdst, int out, bool p16, int chain) {
    const int K = cfg.ns_steps;
    const int ks = cfg.ns_split_steps;
    const size_t nf = facs.size();
    // statistics (sum of squares) of the rooted matrix
    std::vector<StatSpec> st;
    for (size_t f = 0; f < nf; ++f)
      st.push_back(StatSpec{ST_F32, src[f], facs[f]->d, no_ref(), 0, facs[f]->d, facs[f]->d});
    std::vector<std::pair<int, int>> parts = add_stats(L, st);
    // Y_0 = S/c and Z_1 = a_0 I + b_0 S/c
    std::vector<CastSpec> cs;
    for (size_t f = 0; f < nf; ++f) {
      FacBufs& F = *facs[f];
      CastSpec y = cast_spec();
      y.kind = CA_NS_Y0; y.src = src[f]; y.src_ld = F.d; y.rows = F.d; y.cols = F.d;
      y.dst_rows_p = F.dp; y.dst_cols_p = F.dp; y.dst = ws_ref(F.Y[0]); y.dst_ld = F.ld; y.dst_lo = F.dp;
      y.parts = parts[f]; y.scale_mode = SC_STATIC; y.scale_slot = SL_Y;
      y.cinv_slot = chain == 0 ? F.s_cinv : F.s_cinv2;
      y.rho_slot = chain == 0 ? F.s_rho : F.s_rho2;
      y.sqrtc_slot = chain == 0 ? F.s_sqrtc : F.s_sqrtc2;
      y.p16_slot = p16 ? F.s_p16 : -1;
      y.p16_inv_sqrt = out == OUT_SQRT;
      y.write_lo = ks > 0;
      y.damp = damping(F.d);
      y.sym_read = chain == 1;      // the second chain roots a computed square root
      y.dst2 = ws_ref(F.Z[1]); y.scale_slot2 = SL_Z; y.write_lo2 = ks > 1;   // Z_1 in the same pass
      cs.push_back(y);
    }
    add_cast(L, cs, static_cast<float>(na[0]), static_cast<float>(nb[0]));
    // step 0: Y_1 = a_0 Y_0 + b_0 Y_0 Y_0
    {
      std::vector<GemmProb> ps;
      for (size_t f = 0; f < nf; ++f) {
        FacBufs& F = *facs[f];
        GemmProb p = prob();
        p.A = p.B = ws_ref(F.Y[0]); p.lda = p.ldb = F.ld; p.M = p.N = F.d; p.Kp = F.dp; p.Mp = p.Np = F.dp;
        p.epi = EPI_NS_Y1; p.aux = src[f]; p.ldaux = F.d; p.cslot = chain == 0 ? F.s_cinv : F.s_cinv2;
        p.c2 = damping(F.d) / (1.0f + damping(F.d));
        p.aux_sym = chain == 1;
        p.out16 = ws_ref(F.Y[1]); p.out16T = ws_ref(F.YT[1]); p.ld16 = F.ld; p.lo16 = F.dp; p.s_out = SL_Y;
        p.sA = p.sB = SL_Y;
        // Y_0 Y_0 with plain fp16 operands is symmetric bit for bit (entry
        // (i, j) and (j, i) sum the same products in the same order): its
        // upper tiles, each written with its transpose.  The split product
        // sums the hi-lo and lo-hi parts in the other order for (j, i), so it
        // stays whole.
        p.sym_out = ks == 0 ? 1 : 0;
        ps.push_back(p);
      }
      add_gemm(L, ps, ks == 0, 0 < ks, 1 < ks, static_cast<float>(na[0]), static_cast<float>(nb[0]));
    }
    for (int k = 1; k < K; ++k) {
      const int cb = k & 1, nbuf = (k + 1) & 1;
      const float ka = static_cast<float>(na[k]), kb = static_cast<float>(nb[k]);
      // T_k = a_k I + b_k Z_k Y_k
      std::vector<GemmProb> pt;
      const size_t first_slot = resid_slots.size();
      for (size_t f = 0; f < nf; ++f) {
        FacBufs& F = *facs[f];
        GemmProb p = prob();
        // T_k = a_k I + b_k Z_k Y_k as NT(Z_k, Y_k^T); both copies of T are written
        p.A = ws_ref(F.Z[cb]); p.B = ws_ref(F.YT[cb]); p.lda = p.ldb = F.ld; p.M = p.N = F.d; p.Kp = F.dp;
        p.Mp = p.Np = F.dp; p.epi = EPI_NS_T; p.out16 = ws_ref(F.T); p.out16T = ws_ref(F.TT); p.ld16 = F.ld;
        p.lo16 = F.dp;
        p.s_out = SL_T; p.sA = SL_Z; p.sB = SL_Y;
        if (k == K - 1 && F.mat >= 0) {
          // the last T's epilogue leaves the partials of ||Z_{K-1} Y_{K-1} - I||_F:
          // room for the small tile's count (one per wave and tile), the larger
          p.epi = EPI_NS_T_RES;
          p.resid = resid_floats;
          const int tt = F.dp / kTile;
          resid_slots.push_back(ResidSlot{F.mat, F.side, chain, resid_floats, 0});
          resid_floats += tt * tt * 4;
        }
        pt.push_back(p);
      }
      add_gemm(L, pt, false, k < ks, k < ks, ka, kb);
      // partials written: one per wave of every tile of the class the launch took
      const int bt = L.back().tile;
      for (size_t q = first_slot, f = 0; f < nf; ++f) {
        if (k != K - 1 || facs[f]->mat < 0) continue;
        const int n = facs[f]->dp / bt;
        resid_slots[q++].count = n * n * (bt == kBigTile ? 8 : 4);
      }
      std::vector<GemmProb> pu;
      if (k < K - 1) {
        for (size_t f = 0; f < nf; ++f) {   // Y_{k+1} = Y_k T_k
          FacBufs& F = *facs[f];
          GemmProb p = prob();
          p.A = ws_ref(F.Y[cb]); p.B = ws_ref(F.TT); p.lda = p.ldb = F.ld; p.M = p.N = F.d; p.Kp = F.dp;
          p.Mp = p.Np = F.dp; p.epi = EPI_STORE16; p.out16 = ws_ref(F.Y[nbuf]); p.out16T = ws_ref(F.YT[nbuf]);
          p.ld16 = F.ld; p.lo16 = F.dp;
          p.s_out = SL_Y; p.sA = SL_Y; p.sB = SL_T;
          pu.push_back(p);
        }
        for (size_t f = 0; f < nf; ++f) {   // Z_{k+1} = T_k Z_k
          FacBufs& F = *facs[f];
          GemmProb p = prob();
          p.A = ws_ref(F.T); p.B = ws_ref(zt_of(F, k)); p.lda = p.ldb = F.ld; p.M = p.N = F.d; p.Kp = F.dp;
          p.Mp = p.Np = F.dp; p.epi = EPI_STORE16; p.out16 = ws_ref(F.Z[nbuf]); p.out16T = ws_ref(F.ZT[nbuf]);
          p.ld16 = F.ld; p.lo16 = F.dp;
          p.s_out = SL_Z; p.sA = SL_T; p.sB = SL_Z;
          pu.push_back(p);
        }
        add_gemm(L, pu, false, k < ks, k + 1 < ks);
      } else {
        for (size_t f = 0; f < nf; ++f) {
          FacBufs& F = *facs[f];
          GemmProb p = prob();
          p.lda = p.ldb = F.ld; p.M = p.N = F.d; p.Kp = F.dp; p.Mp = p.Np = F.dp; p.epi = EPI_NS_FINAL;
          p.out32 = pdst[f]; p.ld32 = F.d;
          if (out == OUT_INV) {       // P = Z_K / sqrt(c), fp16 copy Z_K * s_Z
            p.A = ws_ref(F.T); p.B = ws_ref(zt_of(F, k)); p.sA = SL_T; p.sB = SL_Z;
            p.cslot = chain == 0 ? F.s_rho : F.s_rho2; p.s_out = SL_Z;
          } else {                    // P = Y_K sqrt(c), fp16 copy Y_K * s_Y
            p.A = ws_ref(F.Y[cb]); p.B = ws_ref(F.TT); p.sA = SL_Y; p.sB = SL_T;
            p.cslot = chain == 0 ? F.s_sqrtc : F.s_sqrtc2; p.s_out = SL_Y;
          }
          pu.push_back(p);
        }
        add_gemm(L, pu, false, k < ks, 0);    // fp32 output only
        // the stored root is symmetrised (the iteration's output is symmetric
        // only up to rounding), and its fp16 copy written from the symmetric values
        if (p16) add_sym(L, facs, pdst);
      }
    }
  }

  // Muon: N's fp16 copies (both orientations, M' written), then the polar
  // iteration X <- a_k X + b_k (X X^T) X from X_0 = N / ||N N^T||_F^{1/2},
  // with the Gram of the smaller side; the last step's product goes straight
  // into the weight update.  Step k's GEMMs are split-fp16 when k <
  // ns_split_steps.
  void plan_muon(std::vector<LaunchRec>& L, std::vector<MatBufs>& mats) {
    const int K = cfg.ns_steps, ks = cfg.ns_split_steps;
    auto sp = [&](int k) { return k < ks ? 1 : 0; };
    auto gdt = [&](const MatBufs& mb) { return groups[mb.group].g_dtype; };
    auto gfmt = [&](const MatBufs& mb) {
      return gdt(mb) == OKLS_F32 ? GF_F32 : gdt(mb) == OKLS_BF16 ? GF_BF16 : GF_F16;
    };
    auto goff = [&](const MatBufs& mb) {
      return static_cast<size_t>(mb.index) * mb.m * mb.n * (gdt(mb) == OKLS_F32 ? 4 : 2);
    };
    auto moff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.n * 4; };
    auto wide = [](const MatBufs& mb) { return mb.m <= mb.n; };
    // 1. statistics of N
    std::vector<StatSpec> st;
    for (const MatBufs& mb : mats)
      st.push_back(StatSpec{ST_NESTEROV, user_ref(REF_G, mb.group, goff(mb)), mb.n,
                            user_ref(REF_M, mb.group, moff(mb)), gfmt(mb), mb.m, mb.n});
    std::vector<std::pair<int, int>> parts = add_stats(L, st);
    // 2. N and N^T in fp16 (absmax scale), M' written
    std::vector<CastSpec> cs;
    for (size_t q = 0; q < mats.size(); ++q) {
      const MatBufs& mb = mats[q];
      CastSpec nn = cast_spec();
      nn.kind = CA_NESTEROV; nn.src = user_ref(REF_M, mb.group, moff(mb)); nn.src_ld = mb.n;
      nn.src2 = user_ref(REF_G, mb.group, goff(mb)); nn.g_fmt = gfmt(mb); nn.write_m = 1;
      nn.rows = mb.m; nn.cols = mb.n; nn.dst_rows_p = mb.mp; nn.dst_cols_p = mb.np; nn.dst = ws_ref(mb.N16);
      nn.dst_ld = mb.ldn; nn.dst_lo = mb.np; nn.parts = parts[q]; nn.scale_mode = SC_ABSMAX;
      nn.scale_slot = mb.s_n; nn.write_lo = sp(0);
      nn.dstT = ws_ref(mb.NT16); nn.dstT_ld = mb.ldm; nn.dstT_lo = mb.mp;
      cs.push_back(nn);
    }
    add_cast(L, cs);
    gemm_cat = CAT_NS;
    for (const MatBufs& mb : mats) {
      const double p = mb.pd, q = std::max(mb.m, mb.n);
      // a Gram and an update product per step; the unsplit Grams after the
      // first run on their upper half
      step_flops[CAT_NS] += 4.0 * K * p * p * q;
      for (int k = 1; k < K; ++k)
        if (!sp(k)) step_flops[CAT_NS] -= p * p * q;
    }
    // 3. Gram of the smaller side in fp32: A_0 = N N^T (wide) or N^T N (tall)
    {
      std::vector<GemmProb> pg;
      for (const MatBufs& mb : mats) {
        GemmProb g = prob();
        const bool w = wide(mb);
        g.A = g.B = ws_ref(w ? mb.N16 : mb.NT16); g.lda = g.ldb = w ? mb.ldn : mb.ldm;
        g.M = g.N = mb.pd; g.Kp = w ? mb.np : mb.mp; g.Mp = g.Np = mb.pdp; g.epi = EPI_STORE32;
        g.out32 = ws_ref(mb.A32); g.ld32 = mb.pd; g.sA = g.sB = mb.s_n;
        pg.push_back(g);
      }
      add_gemm(L, pg, false, sp(0), 0);
    }
    // 4-5. ||A_0||_F, then A_0 / ||A_0||_F in fp16; the cast records
    // 1 / ||A_0||_F^{1/2}, the scaling of X_0 = N / ||A_0||_F^{1/2}
    {
      std::vector<StatSpec> sa;
      for (const MatBufs& mb : mats) sa.push_back(StatSpec{ST_F32, ws_ref(mb.A32), mb.pd, no_ref(), 0, mb.pd, mb.pd});
      std::vector<std::pair<int, int>> pa = add_stats(L, sa);
      std::vector<CastSpec> ca;
      for (size_t q = 0; q < mats.size(); ++q) {
        const MatBufs& mb = mats[q];
        CastSpec y = cast_spec();
        y.kind = CA_NS_Y0; y.src = ws_ref(mb.A32); y.src_ld = mb.pd; y.rows = y.cols = mb.pd;
        y.dst_rows_p = y.dst_cols_p = mb.pdp; y.dst = ws_ref(mb.A16); y.dst_ld = mb.ldp; y.dst_lo = mb.pdp;
        y.parts = pa[q]; y.scale_mode = SC_STATIC; y.scale_slot = SL_Y;
        y.cinv_slot = mb.s_gcinv; y.rho_slot = mb.s_grho; y.write_lo = sp(0); y.damp = 0.0f;
        ca.push_back(y);
      }
      add_cast(L, ca);
    }
    // 6. the steps
    for (int k = 0; k < K; ++k) {
      const int cur = k & 1, nxt = (k + 1) & 1;
      if (k > 0) {   // Gram A_k of the current iterate (fp16, |A_k| <= 1)
        std::vector<GemmProb> pg;
        for (const MatBufs& mb : mats) {
          GemmProb g = prob();
          const bool w = wide(mb);
          g.A = g.B = ws_ref(w ? mb.X[cur] : mb.XT[cur]); g.lda = g.ldb = w ? mb.ldn : mb.ldm;
          g.M = g.N = mb.pd; g.Kp = w ? mb.np : mb.mp; g.Mp = g.Np = mb.pdp; g.epi = EPI_STORE16;
          g.out16 = ws_ref(mb.A16); g.ld16 = mb.ldp; g.lo16 = mb.pdp; g.s_out = SL_Y; g.sA = g.sB = SL_Y;
          // X X^T with plain fp16 operands is symmetric bit for bit: its
          // upper tiles, each also written transposed
          g.sym_out = sp(k) ? 0 : 1;
          pg.push_back(g);
        }
        add_gemm(L, pg, !sp(k), sp(k), sp(k));
      }
      // update: X_{k+1} = c (a_k X_k + b_k A_k X_k), c = ||A_0||_F^{-1/2} at k = 0 (X_0 = N c), else 1
      std::vector<GemmProb> pu;
      const bool last = k == K - 1;
      for (const MatBufs& mb : mats) {
        GemmProb u = prob();
        const bool w = wide(mb);
        const size_t xk = k == 0 ? mb.N16 : mb.X[cur], xtk = k == 0 ? mb.NT16 : mb.XT[cur];
        const int sx = k == 0 ? mb.s_n : SL_Y;
        if (w) {   // A_k X_k = NT(A_k, X_k^T), K = m
          u.A = ws_ref(mb.A16); u.lda = mb.ldp; u.B = ws_ref(xtk); u.ldb = mb.ldm; u.Kp = mb.mp;
          u.sA = SL_Y; u.sB = sx;
        } else {   // X_k A_k = NT(X_k, A_k), K = n
          u.A = ws_ref(xk); u.lda = mb.ldn; u.B = ws_ref(mb.A16); u.ldb = mb.ldp; u.Kp = mb.np;
          u.sA = sx; u.sB = SL_Y;
        }
        u.M = mb.m; u.N = mb.n; u.Mp = mb.mp; u.Np = mb.np;
        u.aux = ws_ref(xk); u.ldaux = mb.ldn; u.aux_lo = sp(k) ? mb.np : -1; u.s_aux = sx;
        u.cslot = k == 0 ? mb.s_grho : SL_ONE;
        if (!last) {
          u.epi = EPI_POLAR;
          u.out16 = ws_ref(mb.X[nxt]); u.ld16 = mb.ldn; u.lo16 = mb.np; u.s_out = SL_Y;
          u.out16T = ws_ref(mb.XT[nxt]); u.ld16T = mb.ldm; u.lo16T = mb.mp;
        } else {
          u.epi = EPI_POLAR_UPDATE;
          u.out32 = user_ref(REF_W, mb.group, moff(mb)); u.ld32 = mb.n;
          u.c0 = update_scale(mb);
        }
        pu.push_back(u);
      }
      add_gemm(L, pu, false, sp(k), last ? 0 : sp(k + 1), static_cast<float>(na[k]), static_cast<float>(nb[k]));
    }
  }

  // ---- SOAP (the Clean paper's Algorithm 4).  Every product with a basis
  // runs on the basis' fp16 copies (scale 2^kScaleExp: |q| <= 1); an operand
  // X with k columns multiplied by an orthogonal matrix has rows of norm at
  // most sqrt(k) max|X|, so its product gets X's scale over 2^sqrt_exp(k).
  //   casts: G, G^T; M' = beta1 M + (1-beta1) G (written back); Q_a, Q_a^T, Q_b, Q_b^T
  //   GEMM   (G Q_b)^T = Q_b^T G^T, (M' Q_b)^T                 -> fp16
  //   GEMM   G' = Q_a^T (G Q_b), M' rotated                     -> fp32
  //   Adam   V <- beta2 V + (1-beta2) G'^2, N'                  -> fp16 (static scale)
  //   GEMM   (N' Q_b^T)^T = Q_b N'^T                             -> fp16
  //   GEMM   W <- decay W - lr Q_a (N' Q_b^T)
  //   GEMM   S_a <- sb S_a + (1-sb) G G^T, S_b likewise (upper tiles, mirrored)
  //   refresh: stats + cast of S, (Q^T S) as fp16, B = Q^T S Q in fp32 (these
  //   products split-fp16 in either precision), then block Jacobi sweeps on B
  //   that rotate the caller's Q in place, then one orthogonalisation step.
  void plan_soap(std::vector<LaunchRec>& L, std::vector<MatBufs>& mats, bool refresh) {
    const int fs = cfg.factor_split;
    const bool param_m = cfg.soap_moments == 0;
    auto gdt = [&](const MatBufs& mb) { return groups[mb.group].g_dtype; };
    auto gfmt = [&](const MatBufs& mb) {
      return gdt(mb) == OKLS_F32 ? GF_F32 : gdt(mb) == OKLS_BF16 ? GF_BF16 : GF_F16;
    };
    auto goff = [&](const MatBufs& mb) {
      return static_cast<size_t>(mb.index) * mb.m * mb.n * (gdt(mb) == OKLS_F32 ? 4 : 2);
    };
    auto moff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.n * 4; };
    auto aoff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.m * 4; };
    auto boff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.n * mb.n * 4; };
    auto xmul = [](int k) { return std::ldexp(1.0f, -sqrt_exp(k)); };

    // 1. statistics of G and of M' (the plain EMA: the step's momentum read with (1, 0))
    std::vector<StatSpec> st;
    for (const MatBufs& mb : mats) {
      const int gk = gdt(mb) == OKLS_F32 ? ST_F32 : ST_H16;
      st.push_back(StatSpec{gk, user_ref(REF_G, mb.group, goff(mb)), mb.n, no_ref(), gfmt(mb), mb.m, mb.n});
      if (param_m)
        st.push_back(StatSpec{ST_NESTEROV, user_ref(REF_G, mb.group, goff(mb)), mb.n,
                              user_ref(REF_M, mb.group, moff(mb)), gfmt(mb), mb.m, mb.n});
    }
    std::vector<std::pair<int, int>> parts = add_stats(L, st);
    const int per = param_m ? 2 : 1;
    // 2. casts
    std::vector<CastSpec> cs;
    for (size_t q = 0; q < mats.size(); ++q) {
      const MatBufs& mb = mats[q];
      CastSpec g = cast_spec();
      g.kind = gdt(mb) == OKLS_F32 ? CA_F32 : CA_H16; g.g_fmt = gfmt(mb);
      g.src = user_ref(REF_G, mb.group, goff(mb)); g.src_ld = mb.n;
      g.rows = mb.m; g.cols = mb.n; g.dst_rows_p = mb.mp; g.dst_cols_p = mb.np; g.dst = ws_ref(mb.G16);
      g.dst_ld = mb.ldn; g.dst_lo = mb.np; g.parts = parts[per * q]; g.scale_mode = SC_ABSMAX;
      g.scale_slot = mb.s_g; g.write_lo = fs;
      g.dstT = ws_ref(mb.G16T); g.dstT_ld = mb.ldm; g.dstT_lo = mb.mp;
      g.aux_slot = mb.s_gx; g.aux_mul = xmul(mb.n);
      cs.push_back(g);
      if (param_m) {
        CastSpec mm = cast_spec();
        mm.kind = CA_NESTEROV; mm.src = user_ref(REF_M, mb.group, moff(mb)); mm.src_ld = mb.n;
        mm.src2 = user_ref(REF_G, mb.group, goff(mb)); mm.g_fmt = gfmt(mb); mm.write_m = 1;
        mm.rows = mb.m; mm.cols = mb.n; mm.dst_rows_p = mb.mp; mm.dst_cols_p = mb.np; mm.dst = ws_ref(mb.M16);
        mm.dst_ld = mb.ldn; mm.dst_lo = mb.np; mm.parts = parts[per * q + 1]; mm.scale_mode = SC_ABSMAX;
        mm.scale_slot = mb.s_m; mm.write_lo = fs;
        mm.aux_slot = mb.s_mx; mm.aux_mul = xmul(mb.n);
        cs.push_back(mm);
      }
      const FacBufs* fl[2] = {&mb.fa, &mb.fb};
      const int kinds[2] = {REF_PA, REF_PB};
      const size_t offs[2] = {aoff(mb), boff(mb)};
      for (int sd = 0; sd < 2; ++sd) {   // the bases and their transposes, static scale
        const FacBufs& F = *fl[sd];
        CastSpec c = cast_spec();
        c.kind = CA_F32; c.src = user_ref(kinds[sd], mb.group, offs[sd]); c.src_ld = F.d;
        c.rows = c.cols = F.d; c.dst_rows_p = c.dst_cols_p = F.dp; c.dst = ws_ref(F.Q16);
        c.dst_ld = F.ldq; c.dst_lo = F.dp; c.parts = parts[per * q]; c.scale_mode = SC_STATIC;
        c.scale_slot = SL_Q; c.write_lo = refresh ? 1 : fs;   // a refresh reads Q^T split
        c.dstT = ws_ref(F.Q16T); c.dstT_ld = F.ldq; c.dstT_lo = F.dp;
        cs.push_back(c);
      }
    }
    add_cast(L, cs);

    for (const MatBufs& mb : mats) {
      const double m = mb.m, n = mb.n;
      step_flops[CAT_WHITEN] += (param_m ? 6.0 : 4.0) * m * n * (m + n);
      step_flops[CAT_FACTOR] += m * n * (m + n);
      if (refresh) step_flops[CAT_NS] += 4.0 * (m * m * m + n * n * n);
    }
    // 3. rotations into the basis: (X Q_b)^T = Q_b^T X^T (n x m), X = G, M'
    gemm_cat = CAT_WHITEN;
    {
      std::vector<GemmProb> px;
      for (const MatBufs& mb : mats) {
        for (int w = 0; w < (param_m ? 2 : 1); ++w) {
          GemmProb p = prob();
          p.A = ws_ref(mb.fb.Q16T); p.lda = mb.fb.ldq; p.B = ws_ref(w == 0 ? mb.G16 : mb.M16); p.ldb = mb.ldn;
          p.M = mb.n; p.N = mb.m; p.Kp = mb.np; p.Mp = mb.np; p.Np = mb.mp; p.epi = EPI_STORE16;
          p.out16 = ws_ref(w == 0 ? mb.XGT16 : mb.XMT16); p.ld16 = mb.ldm; p.lo16 = mb.mp;
          p.sA = SL_Q; p.sB = w == 0 ? mb.s_g : mb.s_m; p.s_out = w == 0 ? mb.s_gx : mb.s_mx;
          px.push_back(p);
        }
      }
      add_gemm(L, px, false, fs, fs);
      std::vector<GemmProb> pr;
      for (const MatBufs& mb : mats) {
        for (int w = 0; w < (param_m ? 2 : 1); ++w) {   // X' = Q_a^T (X Q_b), fp32
          GemmProb p = prob();
          p.A = ws_ref(mb.fa.Q16T); p.lda = mb.fa.ldq; p.B = ws_ref(w == 0 ? mb.XGT16 : mb.XMT16); p.ldb = mb.ldm;
          p.M = mb.m; p.N = mb.n; p.Kp = mb.mp; p.Mp = mb.mp; p.Np = mb.np; p.epi = EPI_STORE32;
          p.out32 = ws_ref(w == 0 ? mb.Gr32 : mb.Mr32); p.ld32 = mb.n;
          p.sA = SL_Q; p.sB = w == 0 ? mb.s_gx : mb.s_mx;
          pr.push_back(p);
        }
      }
      add_gemm(L, pr, false, fs, 0);
    }
    // 4. Adam in the basis.  With the moments kept in the basis, M' and V
    // are EMAs of the same sequence of rotated entries, so |N'| has the
    // static bound of adam_ratio_bound and N' goes straight to fp16.  With M
    // in the parameter space (Algorithm 4) M' is rotated by the current
    // bases while V accumulated the coordinates of earlier ones: after a
    // refresh |N'| can reach |M'| / eps, so N' is written in fp32 (over G',
    // which it no longer needs) and cast with its own absmax scale.
    {
      LaunchRec r;
      r.type = L_ADAM;
      r.cat = CAT_CAST;
      r.first = static_cast<int>(adam_jobs.size());
      int blk = 0;
      for (const MatBufs& mb : mats) {
        AdamJob j{};
        j.g = ws_ref(mb.Gr32);
        j.m = param_m ? ws_ref(mb.Mr32) : user_ref(REF_M, mb.group, moff(mb));
        j.v = user_ref(REF_V, mb.group, moff(mb));
        j.dst = param_m ? no_ref() : ws_ref(mb.NP16);
        j.dst32 = param_m ? ws_ref(mb.Gr32) : no_ref();
        j.rows = mb.m; j.cols = mb.n; j.rows_p = mb.mp; j.cols_p = mb.np; j.ld16 = mb.ldn; j.lo16 = mb.np;
        j.eigen_m = param_m ? 0 : 1;
        j.tiles_x = (mb.np + 255) / 256;
        j.blk_begin = blk;
        blk += j.tiles_x * (mb.mp / kAdamRows);
        // G', M' (or M, read and written), V read and written, N' written
        step_bytes[CAT_CAST] += (4.0 + 4.0 * (param_m ? 1 : 2) + 8.0 + (param_m ? 4.0 : fs ? 4.0 : 2.0)) * mb.m * mb.n;
        adam_jobs.push_back(j);
      }
      r.count = static_cast<int>(mats.size());
      r.nblocks = blk;
      L.push_back(r);
      if (param_m) {
        std::vector<StatSpec> sn;
        for (const MatBufs& mb : mats) sn.push_back(StatSpec{ST_F32, ws_ref(mb.Gr32), mb.n, no_ref(), 0, mb.m, mb.n});
        std::vector<std::pair<int, int>> pn = add_stats(L, sn);
        std::vector<CastSpec> cn;
        for (size_t q = 0; q < mats.size(); ++q) {
          const MatBufs& mb = mats[q];
          CastSpec c = cast_spec();
          c.kind = CA_F32; c.src = ws_ref(mb.Gr32); c.src_ld = mb.n; c.rows = mb.m; c.cols = mb.n;
          c.dst_rows_p = mb.mp; c.dst_cols_p = mb.np; c.dst = ws_ref(mb.NP16); c.dst_ld = mb.ldn; c.dst_lo = mb.np;
          c.parts = pn[q]; c.scale_mode = SC_ABSMAX; c.scale_slot = mb.s_n; c.write_lo = fs;
          c.aux_slot = mb.s_vt; c.aux_mul = xmul(mb.n);
          cn.push_back(c);
        }
        add_cast(L, cn);
      }
    }
    // 5. the rotation back with the update: (N' Q_b^T)^T = Q_b N'^T, then W
    {
      std::vector<GemmProb> pz;
      for (const MatBufs& mb : mats) {
        GemmProb p = prob();
        p.A = ws_ref(mb.fb.Q16); p.lda = mb.fb.ldq; p.B = ws_ref(mb.NP16); p.ldb = mb.ldn;
        p.M = mb.n; p.N = mb.m; p.Kp = mb.np; p.Mp = mb.np; p.Np = mb.mp; p.epi = EPI_STORE16;
        p.out16 = ws_ref(mb.ZT16); p.ld16 = mb.ldm; p.lo16 = mb.mp;
        p.sA = SL_Q; p.sB = param_m ? mb.s_n : SL_NP; p.s_out = param_m ? mb.s_vt : SL_ZT + sqrt_exp(mb.n);
        pz.push_back(p);
      }
      add_gemm(L, pz, false, fs, fs);
      std::vector<GemmProb> pu;
      for (const MatBufs& mb : mats) {
        GemmProb p = prob();
        p.A = ws_ref(mb.fa.Q16); p.lda = mb.fa.ldq; p.B = ws_ref(mb.ZT16); p.ldb = mb.ldm;
        p.M = mb.m; p.N = mb.n; p.Kp = mb.mp; p.Mp = mb.mp; p.Np = mb.np; p.epi = EPI_UPDATE;
        p.out32 = user_ref(REF_W, mb.group, moff(mb)); p.ld32 = mb.n;
        p.sA = SL_Q; p.sB = param_m ? mb.s_vt : SL_ZT + sqrt_exp(mb.n); p.c0 = 1.0f;
        pu.push_back(p);
      }
      add_gemm(L, pu, false, fs, 0);
    }
    // 6. factor EMAs (upper tiles, mirrored)
    gemm_cat = CAT_FACTOR;
    {
      std::vector<GemmProb> ps;
      for (const MatBufs& mb : mats) {
        GemmProb a = prob();
        a.A = a.B = ws_ref(mb.G16); a.lda = a.ldb = mb.ldn;
        a.M = a.N = mb.m; a.Kp = mb.np; a.Mp = a.Np = mb.mp; a.epi = EPI_SYRK;
        a.out32 = user_ref(REF_SA, mb.group, aoff(mb)); a.ld32 = mb.m;
        a.sA = a.sB = mb.s_g; a.c0 = cfg.soap_beta; a.c1 = 1.0f - cfg.soap_beta; a.c2 = 0.0f;
        ps.push_back(a);
        GemmProb b = prob();
        b.A = b.B = ws_ref(mb.G16T); b.lda = b.ldb = mb.ldm;
        b.M = b.N = mb.n; b.Kp = mb.mp; b.Mp = b.Np = mb.np; b.epi = EPI_SYRK;
        b.out32 = user_ref(REF_SB, mb.group, boff(mb)); b.ld32 = mb.n;
        b.sA = b.sB = mb.s_g; b.c0 = cfg.soap_beta; b.c1 = 1.0f - cfg.soap_beta; b.c2 = 0.0f;
        ps.push_back(b);
      }
      add_gemm(L, ps, true, fs, 0);
    }
    if (!refresh) return;
    // 7. basis refresh: B = Q^T S Q for every factor
    gemm_cat = CAT_NS;
    std::vector<FacBufs*> facs;
    std::vector<Ref> fsrc, fbasis;
    for (MatBufs& mb : mats) {
      facs.push_back(&mb.fa);
      fsrc.push_back(user_ref(REF_SA, mb.group, aoff(mb)));
      fbasis.push_back(user_ref(REF_PA, mb.group, aoff(mb)));
      facs.push_back(&mb.fb);
      fsrc.push_back(user_ref(REF_SB, mb.group, boff(mb)));
      fbasis.push_back(user_ref(REF_PB, mb.group, boff(mb)));
    }
    std::vector<StatSpec> sf;
    for (size_t f = 0; f < facs.size(); ++f)
      sf.push_back(StatSpec{ST_F32, fsrc[f], facs[f]->d, no_ref(), 0, facs[f]->d, facs[f]->d});
    std::vector<std::pair<int, int>> fparts = add_stats(L, sf);
    std::vector<CastSpec> cf;
    for (size_t f = 0; f < facs.size(); ++f) {
      const FacBufs& F = *facs[f];
      CastSpec c = cast_spec();
      c.kind = CA_F32; c.src = fsrc[f]; c.src_ld = F.d; c.rows = c.cols = F.d;
      c.dst_rows_p = c.dst_cols_p = F.dp; c.dst = ws_ref(F.L16); c.dst_ld = F.ldq; c.dst_lo = F.dp;
      c.parts = fparts[f]; c.scale_mode = SC_ABSMAX; c.scale_slot = F.s_l; c.write_lo = 1;
      c.aux_slot = F.s_lx; c.aux_mul = xmul(F.d);
      cf.push_back(c);
    }
    add_cast(L, cf);
    {
      std::vector<GemmProb> ph, pb;
      for (size_t f = 0; f < facs.size(); ++f) {
        const FacBufs& F = *facs[f];
        GemmProb h = prob();   // (S Q)^T = Q^T S (S symmetric: its rows are its columns)
        h.A = ws_ref(F.Q16T); h.lda = F.ldq; h.B = ws_ref(F.L16); h.ldb = F.ldq;
        h.M = h.N = F.d; h.Kp = F.dp; h.Mp = h.Np = F.dp; h.epi = EPI_STORE16;
        h.out16 = ws_ref(F.HT16); h.ld16 = F.ldq; h.lo16 = F.dp; h.sA = SL_Q; h.sB = F.s_l; h.s_out = F.s_lx;
        ph.push_back(h);
        GemmProb b = prob();   // B = Q^T (S Q)
        b.A = ws_ref(F.Q16T); b.lda = F.ldq; b.B = ws_ref(F.HT16); b.ldb = F.ldq;
        b.M = b.N = F.d; b.Kp = F.dp; b.Mp = b.Np = F.dp; b.epi = EPI_STORE32;
        b.out32 = ws_ref(F.B32); b.ld32 = F.d; b.sA = SL_Q; b.sB = F.s_lx;
        pb.push_back(b);
      }
      // split-fp16 whatever the precision: the sweeps converge on B as it is
      // computed, and fp16 operands would leave ~1e-3 of it off the diagonal
      // for them to chase
      add_gemm(L, ph, false, 1, 1);
      add_gemm(L, pb, false, 1, 0);
    }
    // 8. Jacobi sweeps: reset, then per sweep every round's solve and apply, and a check.
    // The factors are independent: with more than one, they form two sets of
    // near-equal cost (d^3, largest first) whose launches run on two streams,
    // so one set's solve (a few hundred latency-bound workgroups) overlaps the
    // other set's apply.
    const int nset = (!single_chain && facs.size() > 1) ? 2 : 1;
    std::vector<std::vector<size_t>> sets(nset);
    {
      std::vector<size_t> order(facs.size());
      for (size_t f = 0; f < order.size(); ++f) order[f] = f;
      std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return facs[x]->d > facs[y]->d; });
      std::vector<double> load(nset, 0.0);
      for (size_t f : order) {
        const int b = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
        sets[b].push_back(f);
        load[b] += std::pow(static_cast<double>(facs[f]->d), 3.0);
      }
    }
    double sweep_flops = 0.0, sweep_bytes = 0.0;
    std::vector<std::vector<LaunchRec>> jl(nset);
    int part_base = 0, flag_base = 0;
    for (int st = 0; st < nset; ++st) {
      std::sort(sets[st].begin(), sets[st].end());
      const int first = static_cast<int>(jac_jobs.size());
      int solve_blk = 0, apply_blk = 0, part = 0, max_rounds = 0;
      // tiles per apply block: several, with the next one's loads in flight,
      // where a round has many (measured on the 1.2B-class workload: warm
      // refresh 6.7 -> 4.0 s); one on small rounds, whose blocks would
      // otherwise leave CUs idle (d=1024 block: 141 against 147 ms)
      long set_items = 0;
      for (const size_t f : sets[st]) {
        const long np = jac_blocks(facs[f]->d) / 2;
        set_items += np * (np + 1) / 2 + static_cast<long>((facs[f]->d + kJp - 1) / kJp) * np;
      }
      const int items = cfg.jacobi_apply_tiles != 0 ? cfg.jacobi_apply_tiles
                        : set_items >= kJacManyItems ? kJacApplyItems : 1;
      for (size_t q = 0; q < sets[st].size(); ++q) {
        const size_t f = sets[st][q];
        const FacBufs& F = *facs[f];
        JacJob j{};
        j.B = ws_ref(F.B32); j.V = fbasis[f]; j.d = F.d; j.nb = jac_blocks(F.d); j.npairs = j.nb / 2;
        j.btiles = j.npairs * (j.npairs + 1) / 2; j.vrows = (F.d + kJp - 1) / kJp;
        j.jbuf = static_cast<int64_t>(F.jbuf); j.part = part; j.flag = static_cast<int32_t>(q);
        j.solve_begin = solve_blk; j.apply_begin = apply_blk;
        // the rotations and the basis are fp32: the basis' own residual stops
        // near u sqrt(d) (measured at d = 2816: 8e-6 of ||L|| from the eighth
        // sweep of a cold start on), so the stop is the larger of jacobi_tol
        // and 2^-23 sqrt(d) (6.3e-6 at d = 2816); sweeps below it only shrink
        // B's off-diagonal, not the basis' error
        j.tol = std::max(cfg.jacobi_tol, static_cast<float>(std::ldexp(std::sqrt(static_cast<double>(F.d)), -23)));
        j.apply_items = items;
        solve_blk += j.npairs;
        apply_blk += (j.btiles + j.vrows * j.npairs + items - 1) / items;
        part += j.btiles;
        max_rounds = std::max(max_rounds, j.nb - 1);
        const double tile = static_cast<double>(kJp) * kJp * kJp;   // one 64^3 product
        sweep_flops += (j.nb - 1) * (2.0 * tile * 2.0 * j.btiles + 2.0 * tile * j.vrows * j.npairs);
        // per round: B and V read and written once, the rotations written and read
        sweep_bytes += (j.nb - 1) * (16.0 * F.d * F.d + 8.0 * j.npairs * kJp * kJp);
        jac_jobs.push_back(j);
      }
      const int count = static_cast<int>(sets[st].size());
      const size_t part_off = jac_part_rel + static_cast<size_t>(part_base) * 2 * sizeof(float);
      const size_t flag_off = jac_flag_rel + static_cast<size_t>(flag_base) * sizeof(int32_t);
      auto jac = [&](int kind, int round, int nblocks) {
        LaunchRec r;
        r.type = L_JAC;
        r.cat = CAT_EIG;
        r.first = first;
        r.count = count;
        r.jac_kind = kind;
        r.round = round;
        r.nblocks = nblocks;
        r.jac_part = part_off;
        r.jac_flag = flag_off;
        r.stream = st;
        jl[st].push_back(r);
      };
      jac(JAC_RESET, 0, 1);
      for (int sw = 0; sw < cfg.jacobi_sweeps; ++sw) {
        for (int rd = 0; rd < max_rounds; ++rd) {
          jac(JAC_SOLVE, rd, solve_blk);
          jac(JAC_APPLY, rd, apply_blk);
        }
        jac(JAC_CHECK, 0, count);
      }
      part_base += part;
      flag_base += count;
    }
    step_flops[CAT_EIG] += cfg.jacobi_sweeps * sweep_flops;
    step_bytes[CAT_EIG] += cfg.jacobi_sweeps * sweep_bytes;
    if (nset > 1) {
      LaunchRec fork;
      fork.type = L_FORK;
      L.push_back(fork);
    }
    // issue the sets' launches interleaved, so both streams have work queued
    for (size_t i = 0;; ++i) {
      bool any = false;
      for (int st = 0; st < nset; ++st)
        if (i < jl[st].size()) { L.push_back(jl[st][i]); any = true; }
      if (!any) break;
    }
    if (nset > 1) {
      LaunchRec join;
      join.type = L_JOIN;
      L.push_back(join);
    }
    // 9. one Newton-Schulz step towards the nearest orthogonal matrix,
    // Q <- Q (3 I - Q^T Q) / 2, split-fp16 (fp32-accurate) whatever the
    // precision: each sweep's rotations leave Q orthogonal only to ~1e-6, and
    // a basis that is refreshed from itself would otherwise drift a little
    // further from orthogonal at every refresh; the step squares that error.
    // T and T^T go through the buffers of S's copy and of (Q^T S).
    std::vector<CastSpec> cq;
    for (size_t f = 0; f < facs.size(); ++f) {
      const FacBufs& F = *facs[f];
      CastSpec c = cast_spec();
      c.kind = CA_F32; c.src = fbasis[f]; c.src_ld = F.d; c.rows = c.cols = F.d;
      c.dst_rows_p = c.dst_cols_p = F.dp; c.dst = ws_ref(F.Q16); c.dst_ld = F.ldq; c.dst_lo = F.dp;
      c.parts = fparts[f]; c.scale_mode = SC_STATIC; c.scale_slot = SL_Q; c.write_lo = 1;
      c.dstT = ws_ref(F.Q16T); c.dstT_ld = F.ldq; c.dstT_lo = F.dp;
      cq.push_back(c);
    }
    add_cast(L, cq);
    std::vector<GemmProb> pt, pq;
    for (size_t f = 0; f < facs.size(); ++f) {
      const FacBufs& F = *facs[f];
      GemmProb t = prob();   // T = 3/2 I - 1/2 Q^T Q (and T^T)
      t.A = t.B = ws_ref(F.Q16T); t.lda = t.ldb = F.ldq;
      t.M = t.N = F.d; t.Kp = F.dp; t.Mp = t.Np = F.dp; t.epi = EPI_NS_T;
      t.out16 = ws_ref(F.L16); t.out16T = ws_ref(F.HT16); t.ld16 = F.ldq; t.lo16 = F.dp;
      t.sA = t.sB = SL_Q; t.s_out = SL_Q;
      pt.push_back(t);
      GemmProb q = prob();   // Q <- Q T
      q.A = ws_ref(F.Q16); q.lda = F.ldq; q.B = ws_ref(F.HT16); q.ldb = F.ldq;
      q.M = q.N = F.d; q.Kp = F.dp; q.Mp = q.Np = F.dp; q.epi = EPI_STORE32;
      q.out32 = fbasis[f]; q.ld32 = F.d; q.sA = q.sB = SL_Q;
      pq.push_back(q);
      step_flops[CAT_NS] += 4.0 * std::pow(static_cast<double>(F.d), 3.0);
    }
    add_gemm(L, pt, false, 1, 1, 1.5f, -0.5f);
    add_gemm(L, pq, false, 1, 0);
  }

  // ---- Nystrom mode (the Clean paper's low-rank factors, Algorithm 3, and
  // the preconditioner of its eq. 9-10), fp32 throughout.
  ProdDesc prod(Ref A, int lda, int ta, Ref B, int ldb, Ref C, int ldc, int M, int N, int K, float alpha,
                float beta) {
    ProdDesc p{};
    p.A = A; p.B = B; p.C = C; p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ta = ta;
    p.M = M; p.N = N; p.K = K; p.alpha = alpha; p.beta = beta; p.alpha_slot = -1; p.rowscale = no_ref();
    p.a_fmt = GF_F32;
    return p;
  }
  // C = alpha op(A) B + beta C with op(A) Mo x K (ta: A stored K x Mo), B K x R, C Mo x R (ot: R x Mo)
  ThinJob thin(Ref A, int lda, int ta, Ref B, int ldb, Ref C, int ldc, int ot, int Mo, int K, int R, float alpha,
               float beta) {
    ThinJob j{};
    j.A = A; j.B = B; j.C = C; j.M = j.Nout = no_ref(); j.wupd = 0; j.aux = no_ref(); j.c0 = 0.0f;
    j.lda = lda; j.ldb = ldb; j.ldc = ldc; j.ldn = 0; j.ta = ta; j.ot = ot; j.a_fmt = GF_F32; j.mom = 0;
    j.Mo = Mo; j.K = K; j.R = R; j.alpha = alpha; j.beta = beta; j.alpha_slot = -1; j.rowscale = no_ref();
    return j;
  }
  // a product description as a thin job (N <= kThinMaxR)
  ThinJob thin_of(const ProdDesc& p) {
    ThinJob j = thin(p.A, p.lda, p.ta, p.B, p.ldb, p.C, p.ldc, 0, p.M, p.K, p.N, p.alpha, p.beta);
    j.a_fmt = p.a_fmt; j.alpha_slot = p.alpha_slot; j.rowscale = p.rowscale;
    return j;
  }
  // products of both operand forms: one launch per form
  void add_thin_any(std::vector<LaunchRec>& L, const std::vector<ProdDesc>& ps, int cat) {
    std::vector<ThinJob> by_ta[2];
    for (const ProdDesc& p : ps) by_ta[p.ta ? 1 : 0].push_back(thin_of(p));
    add_thin(L, by_ta[0], cat);
    add_thin(L, by_ta[1], cat);
  }
  // one launch per (ta, mom) kind
  void add_thin(std::vector<LaunchRec>& L, const std::vector<ThinJob>& js, int cat) {
    if (js.empty()) return;
    LaunchRec r;
    r.type = L_THIN;
    r.cat = cat;
    r.first = static_cast<int>(thin_jobs.size());
    r.thin_ta = js.front().ta;
    r.thin_mom = js.front().mom;
    for (const ThinJob& j : js) r.thin_cbm = std::max(r.thin_cbm, j.R <= 32 ? 1 : j.R <= 64 ? 2 : 4);
    r.thin_wupd = js.front().wupd;
    int blk = 0;
    for (ThinJob j : js) {
      j.blk_begin = blk;
      blk += (j.Mo + kThinTile - 1) / kThinTile;
      step_flops[cat] += 2.0 * j.Mo * static_cast<double>(j.K) * j.R;
      // op(A) once (gradient bytes as stored), B once, C once (twice when read)
      const double ae = j.a_fmt == GF_F32 ? 4.0 : 2.0;
      double b = ae * j.Mo * static_cast<double>(j.K) + 4.0 * j.K * static_cast<double>(j.R) +
                 4.0 * (j.wupd ? 3.0 : j.beta != 0.0f ? 2.0 : 1.0) * j.Mo * static_cast<double>(j.R);
      if (j.mom) b += 12.0 * j.Mo * static_cast<double>(j.K);   // M read and written, N written
      step_bytes[cat] += b;
      thin_jobs.push_back(j);
    }
    r.count = static_cast<int>(js.size());
    r.nblocks = blk;
    L.push_back(r);
  }
  void add_north(std::vector<LaunchRec>& L, const std::vector<NysOrthJob>& js) {
    LaunchRec r;
    r.type = L_NORTH;
    r.cat = CAT_EIG;
    r.first = static_cast<int>(north_jobs.size());
    for (const NysOrthJob& j : js) {
      north_jobs.push_back(j);
      step_flops[CAT_EIG] += 4.0 * j.d * static_cast<double>(j.k) * j.k;   // two Gram-Schmidt passes
    }
    r.count = static_cast<int>(js.size());
    r.nblocks = r.count;
    L.push_back(r);
  }
  void add_nelem(std::vector<LaunchRec>& L, std::vector<NysElemJob> js) {
    LaunchRec r;
    r.type = L_NELEM;
    r.cat = CAT_CAST;
    r.first = static_cast<int>(nelem_jobs.size());
    int blk = 0;
    for (NysElemJob& j : js) {
      const size_t total = static_cast<size_t>(j.rows) * j.cols;
      j.blocks = static_cast<int>(std::max<size_t>(1, std::min<size_t>((total + 255) / 256, 4096)));
      j.blk_begin = blk;
      blk += j.blocks;
      step_bytes[CAT_CAST] += 8.0 * total;   // one fp32 read and one write per element
      nelem_jobs.push_back(j);
    }
    r.count = static_cast<int>(js.size());
    r.nblocks = blk;
    L.push_back(r);
  }
  NysElemJob nelem(int kind) {
    NysElemJob j{};
    j.kind = kind;
    j.dst = j.src = j.src2 = j.lam = no_ref();
    return j;
  }

  void plan_nys(std::vector<LaunchRec>& L, std::vector<MatBufs>& mats, bool refresh) {
    auto gdt = [&](const MatBufs& mb) { return groups[mb.group].g_dtype; };
    auto gfmt = [&](const MatBufs& mb) {
      return gdt(mb) == OKLS_F32 ? GF_F32 : gdt(mb) == OKLS_BF16 ? GF_BF16 : GF_F16;
    };
    auto goff = [&](const MatBufs& mb) {
      return static_cast<size_t>(mb.index) * mb.m * mb.n * (gdt(mb) == OKLS_F32 ? 4 : 2);
    };
    auto moff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.n * 4; };
    // the caller's U (N, d, r), Lambda (N, r) and Psi (N, d, k) of a side
    auto uref = [&](const MatBufs& mb, int sd) {
      const MatBufs::NysSide& S = mb.ns[sd];
      return user_ref(sd == 0 ? REF_PA : REF_PB, mb.group, static_cast<size_t>(mb.index) * S.d * S.r * 4);
    };
    auto lref = [&](const MatBufs& mb, int sd) {
      const MatBufs::NysSide& S = mb.ns[sd];
      return user_ref(sd == 0 ? REF_SA : REF_SB, mb.group, static_cast<size_t>(mb.index) * S.r * 4);
    };
    auto pref = [&](const MatBufs& mb, int sd) {
      const MatBufs::NysSide& S = mb.ns[sd];
      return user_ref(sd == 0 ? REF_PSA : REF_PSB, mb.group, static_cast<size_t>(mb.index) * S.d * S.k * 4);
    };
    const float b2 = cfg.beta2;
    if (refresh) {
      // Omega_0 = [U_prev | Psi's first k - r columns] (a first refresh has U = 0:
      // those columns are dependent and take Psi's remaining columns instead)
      std::vector<NysElemJob> ge;
      std::vector<NysOrthJob> go;
      for (const MatBufs& mb : mats)
        for (int sd = 0; sd < 2; ++sd) {
          const MatBufs::NysSide& S = mb.ns[sd];
          NysElemJob j = nelem(NE_GATHER);
          j.dst = ws_ref(S.Om); j.src = uref(mb, sd); j.src2 = pref(mb, sd);
          j.rows = S.d; j.cols = S.k; j.ld_dst = S.k; j.ld_src = S.r; j.ld_src2 = S.k; j.cols1 = S.r;
          ge.push_back(j);
          go.push_back(NysOrthJob{ws_ref(S.Om), pref(mb, sd), S.d, S.k, S.k, S.k, S.k - S.r});
        }
      add_nelem(L, ge);
      add_north(L, go);
      // q passes of Y = A Omega, Omega = Q(Y); then the final sketch Y = A Omega.
      // A Omega = beta2 U (Lambda U^T Omega) + (1 - beta2) G (G^T Omega) on the
      // left, with G^T and G exchanged on the right (eq. 8).
      for (int pass = 0; pass <= cfg.nys_passes; ++pass) {
        std::vector<ProdDesc> p1, p2, p3;
        std::vector<NysOrthJob> po;
        for (const MatBufs& mb : mats)
          for (int sd = 0; sd < 2; ++sd) {
            const MatBufs::NysSide& S = mb.ns[sd];
            const int other = sd == 0 ? mb.n : mb.m;
            ProdDesc t1 = prod(uref(mb, sd), S.r, 1, ws_ref(S.Om), S.k, ws_ref(S.T1), S.k, S.r, S.k, S.d, b2, 0.0f);
            t1.rowscale = lref(mb, sd);
            p1.push_back(t1);
            // left: T2 = G^T Omega (n x k); right: T2 = G Omega (m x k)
            ProdDesc t2 = prod(user_ref(REF_G, mb.group, goff(mb)), mb.n, sd == 0 ? 1 : 0, ws_ref(S.Om), S.k, ws_ref(S.T2), S.k, other, S.k, S.d, 1.0f, 0.0f);
            t2.a_fmt = gfmt(mb);
            p1.push_back(t2);
            // Y = (1 - beta2) G T2 (left) or G^T T2 (right)
            ProdDesc y = prod(user_ref(REF_G, mb.group, goff(mb)), mb.n, sd == 0 ? 0 : 1, ws_ref(S.T2), S.k, ws_ref(S.Yb), S.k, S.d, S.k, other, 1.0f - b2, 0.0f);
            y.a_fmt = gfmt(mb);
            p2.push_back(y);
            // Y += U T1
            p3.push_back(prod(uref(mb, sd), S.r, 0, ws_ref(S.T1), S.k, ws_ref(S.Yb), S.k, S.d, S.k, S.r, 1.0f, 1.0f));
            if (pass < cfg.nys_passes) po.push_back(NysOrthJob{ws_ref(S.Yb), pref(mb, sd), S.d, S.k, S.k, S.k, 0});
          }
        add_thin_any(L, p1, CAT_NS);
        add_thin_any(L, p2, CAT_NS);
        add_thin_any(L, p3, CAT_NS);
        if (pass < cfg.nys_passes) {
          add_north(L, po);
          // the orthonormalised Y is the next Omega
          for (MatBufs& mb : mats)
            for (MatBufs::NysSide& S : mb.ns) std::swap(S.Om, S.Yb);
        }
      }
      // G_Y = Y^T Y and C = Omega^T Y; phase 1 (shift, Cholesky, R^-1 over C);
      // F = Y R^-1 + nu_u Omega R^-1; F^T F and F^T U_prev; phase 2
      // (eigenpairs, signs, Lambda); U = F K into the caller's U (read above
      // for the last time)
      auto small = [&](int phase) {
        LaunchRec r;
        r.type = L_NSMALL;
        r.cat = CAT_EIG;
        r.round = phase;
        r.first = static_cast<int>(nsmall_jobs.size());
        for (const MatBufs& mb : mats)
          for (int sd = 0; sd < 2; ++sd) {
            const MatBufs::NysSide& S = mb.ns[sd];
            NysSmallJob j{};
            j.gram = ws_ref(S.gram); j.cmat = ws_ref(S.cm); j.ftu = ws_ref(S.zp); j.kout = ws_ref(S.kout);
            j.lam = lref(mb, sd); j.scratch = ws_ref(S.scratch);
            j.k = S.k; j.r = S.r; j.nu_slot = S.s_nu; j.nuu_slot = S.s_nuu;
            nsmall_jobs.push_back(j);
            step_flops[CAT_EIG] += 2.0 * std::pow(static_cast<double>(S.k), 3.0);
            ++r.count;
          }
        r.nblocks = r.count;
        L.push_back(r);
      };
      std::vector<ProdDesc> pg, pf1, pf2, pt, pu;
      for (const MatBufs& mb : mats)
        for (int sd = 0; sd < 2; ++sd) {
          const MatBufs::NysSide& S = mb.ns[sd];
          pg.push_back(prod(ws_ref(S.Yb), S.k, 1, ws_ref(S.Yb), S.k, ws_ref(S.gram), S.k, S.k, S.k, S.d, 1.0f, 0.0f));
          pg.push_back(prod(ws_ref(S.Om), S.k, 1, ws_ref(S.Yb), S.k, ws_ref(S.cm), S.k, S.k, S.k, S.d, 1.0f, 0.0f));
          pf1.push_back(prod(ws_ref(S.Yb), S.k, 0, ws_ref(S.cm), S.k, ws_ref(S.Fb), S.k, S.d, S.k, S.k, 1.0f, 0.0f));
          ProdDesc f2 = prod(ws_ref(S.Om), S.k, 0, ws_ref(S.cm), S.k, ws_ref(S.Fb), S.k, S.d, S.k, S.k, 1.0f, 1.0f);
          f2.alpha_slot = S.s_nuu;
          pf2.push_back(f2);
          pt.push_back(prod(ws_ref(S.Fb), S.k, 1, ws_ref(S.Fb), S.k, ws_ref(S.gram), S.k, S.k, S.k, S.d, 1.0f, 0.0f));
          pt.push_back(prod(ws_ref(S.Fb), S.k, 1, uref(mb, sd), S.r, ws_ref(S.zp), S.r, S.k, S.r, S.d, 1.0f, 0.0f));
          pu.push_back(prod(ws_ref(S.Fb), S.k, 0, ws_ref(S.kout), S.r, uref(mb, sd), S.r, S.d, S.r, S.k, 1.0f, 0.0f));
        }
      add_thin_any(L, pg, CAT_NS);
      small(1);
      add_thin_any(L, pf1, CAT_NS);
      add_thin_any(L, pf2, CAT_NS);
      add_thin_any(L, pt, CAT_NS);
      small(2);
      add_thin_any(L, pu, CAT_NS);
      // the buffer roles are back where the layout put them for the next plan
      if (cfg.nys_passes & 1)
        for (MatBufs& mb : mats)
          for (MatBufs::NysSide& S : mb.ns) std::swap(S.Om, S.Yb);
    }
    // every step: the preconditioned U = P_a^-1/2 N P_b^-1/2 with
    // P^-1/2 = I + U diag(e) U^T, e_j = sqrt((lambda_r + eps) / (lambda_j + eps)) - 1,
    // expanded so that the m x n data is read three times:
    //   X = N U_b (N computed from G and M on the fly, M and N written),
    //   Z = U_a^T N + (U_a^T X) (U_b E_b)^T,
    //   U = N + X (U_b E_b)^T + (U_a E_a) Z  (= P_a^-1/2 N' with N' = N + X (U_b E_b)^T),
    // the last product in the weight update's epilogue.
    {
      std::vector<NysElemJob> e1;
      for (const MatBufs& mb : mats) {
        const int ra = mb.ns[0].r, rb = mb.ns[1].r;
        NysElemJob sa = nelem(NE_SCALE);      // U_a E_a into XU's last r_a columns
        sa.dst = ws_ref(mb.XU + static_cast<size_t>(rb) * 4); sa.src = uref(mb, 0); sa.lam = lref(mb, 0);
        sa.rows = mb.m; sa.cols = ra; sa.ld_dst = rb + ra; sa.ld_src = ra;
        e1.push_back(sa);
        NysElemJob sb = nelem(NE_SCALE);      // (U_b E_b)^T into ZB's first r_b rows
        sb.dst = ws_ref(mb.ZB); sb.src = uref(mb, 1); sb.lam = lref(mb, 1);
        sb.rows = mb.n; sb.cols = rb; sb.ld_dst = mb.n; sb.ld_src = rb; sb.trans = 1;
        e1.push_back(sb);
      }
      add_nelem(L, e1);
    }
    std::vector<ThinJob> t1, t2, t3, t4, fin;
    double wupd_a_bytes = 0.0;
    // the weight update's column chunk: one 32-column block per thin block
    // (the one-block kernel's registers leave room for the block's W and X
    // quads, loaded before the product; the m x (r_a + r_b) operand is
    // re-read per chunk from L2)
    constexpr int kWupdCols = 32;
    for (const MatBufs& mb : mats) {
      const int ra = mb.ns[0].r, rb = mb.ns[1].r, ld = rb + ra;
      // X = N U_b with N = momentum(G, M)
      ThinJob x = thin(user_ref(REF_G, mb.group, goff(mb)), mb.n, 0, uref(mb, 1), rb, ws_ref(mb.XU), ld, 0,
                       mb.m, mb.n, rb, 1.0f, 0.0f);
      x.a_fmt = gfmt(mb); x.mom = 1; x.M = user_ref(REF_M, mb.group, moff(mb)); x.Nout = ws_ref(mb.N32); x.ldn = mb.n;
      t1.push_back(x);
      // Z = U_a^T N (written as r_a x n below ZB's first r_b rows): op(A) = N^T
      t2.push_back(thin(ws_ref(mb.N32), mb.n, 1, uref(mb, 0), ra, ws_ref(mb.ZB + static_cast<size_t>(rb) * mb.n * 4),
                        mb.n, 1, mb.n, mb.m, ra, 1.0f, 0.0f));
      // Ct = X^T U_a (r_b x r_a): op(A) = X^T, X the first r_b columns of XU
      t3.push_back(thin(ws_ref(mb.XU), ld, 1, uref(mb, 0), ra, ws_ref(mb.Ct), ra, 0, rb, mb.m, ra, 1.0f, 0.0f));
      // Z += (U_a^T X) (U_b E_b)^T, as Z^T += (U_b E_b) Ct: op(A) = ((U_b E_b)^T)^T from ZB's first rows
      t4.push_back(thin(ws_ref(mb.ZB), mb.n, 1, ws_ref(mb.Ct), ra, ws_ref(mb.ZB + static_cast<size_t>(rb) * mb.n * 4),
                        mb.n, 1, mb.n, rb, ra, 1.0f, 1.0f));
      // W <- decay W - lr c_shape (N + [X | U_a E_a] [(U_b E_b)^T ; Z]): a
      // thin product per kWupdCols columns of W (op(A) = [X | U_a E_a],
      // m x (r_a + r_b)), the update fused into its epilogue
      for (int j0 = 0; j0 < mb.n; j0 += kWupdCols) {
        const size_t cb = static_cast<size_t>(j0) * 4;
        ThinJob f = thin(ws_ref(mb.XU), ld, 0, ws_ref(mb.ZB + cb), mb.n, user_ref(REF_W, mb.group, moff(mb) + cb),
                         mb.n, 0, mb.m, ld, std::min(kWupdCols, mb.n - j0), 1.0f, 0.0f);
        f.wupd = 1; f.aux = ws_ref(mb.N32 + cb); f.c0 = update_scale(mb);
        fin.push_back(f);
      }
      wupd_a_bytes += 4.0 * mb.m * ld * (((mb.n + kWupdCols - 1) / kWupdCols) - 1);
    }
    add_thin(L, t1, CAT_WHITEN);
    add_thin(L, t2, CAT_WHITEN);
    add_thin(L, t3, CAT_WHITEN);
    add_thin(L, t4, CAT_WHITEN);
    add_thin(L, fin, CAT_WHITEN);
    // algorithmic bytes: [X | U_a E_a] once per matrix, not once per chunk
    step_bytes[CAT_WHITEN] -= wupd_a_bytes;
  }

  // Whether a second concurrent Newton-Schulz chain pays for this chunk.
  // It fills the CUs that the last, partly filled round of a launch leaves
  // idle; with a full last round, or many rounds, it only adds launches and
  // contention.  The measure is the single-chain T_k launch in rounds of
  // kCUs blocks, each tile weighted by its K against the largest K.  Measured
  // (A/B per workload): two chains +5.5 % on the d=1024 block (1.7 rounds);
  // one chain +6 % on the 1.2B-class workload and +11 % on the 13B-class
  // layer, and +1.6 to +5.7 % on batches of equal square factors whose
  // launches are whole rounds.
  static constexpr int kCUs = 256;
  bool two_chains_pay(const std::vector<FacBufs*>& facs) const {
    if (facs.size() < 2) return false;
    int kmax = 0;
    long big = 0;
    bool big_ok = true;
    for (const FacBufs* f : facs) {
      kmax = std::max(kmax, f->dp);
      if (f->dp % kBigTile) big_ok = false;
      big += static_cast<long>(f->dp / kBigTile) * (f->dp / kBigTile);
    }
    // the tile the launch takes (add_gemm's rule for the fp16-output kinds)
    const int bt = (big_ok && big >= 64) ? kBigTile : kTile;
    const double slots = bt == kBigTile ? kCUs : 2.0 * kCUs;   // the 128 tile runs two blocks per CU
    double w = 0.0;
    for (const FacBufs* f : facs) w += std::pow(static_cast<double>(f->dp / bt), 2.0) * f->dp / kmax;
    const double rounds = w / slots;
    const double last = rounds - std::floor(rounds);
    return rounds < 4.0 && last > 0.0 && last <= 0.75;
  }


  // refresh: the launches of a step that recomputes the roots; otherwise the
  // roots are kept and the whitening uses the fp16 copies of the previous P.
  // The first call for a chunk rebases its buffers and registers them.
  void plan_chunk(std::vector<MatBufs>& mats, size_t base, bool refresh, bool rebase) {
    if (rebase) {
      for (MatBufs& mb : mats) {
        size_t* offs[] = {&mb.G16, &mb.G16T, &mb.N16, &mb.Xa32, &mb.XbT32, &mb.Xa16, &mb.XbT16, &mb.VT32, &mb.VT16,
                          &mb.NT16, &mb.X[0], &mb.X[1], &mb.XT[0], &mb.XT[1], &mb.A32, &mb.A16,
                          &mb.M16, &mb.XGT16, &mb.XMT16, &mb.Gr32, &mb.Mr32, &mb.NP16, &mb.ZT16,
                          &mb.N32, &mb.XU, &mb.ZB, &mb.Ct};
        for (size_t* o : offs) *o += base;
        for (MatBufs::NysSide& S : mb.ns) {
          size_t* so[] = {&S.Om, &S.Yb, &S.Fb, &S.T1, &S.T2, &S.gram, &S.cm, &S.zp, &S.kout, &S.scratch};
          for (size_t* o : so) *o += base;
        }
        for (FacBufs* f : {&mb.fa, &mb.fb}) {
          f->Y[0] += base; f->Y[1] += base; f->Z[0] += base; f->Z[1] += base; f->T += base; f->R32 += base;
          f->YT[0] += base; f->YT[1] += base; f->ZT[0] += base; f->ZT[1] += base; f->TT += base;
          f->P16w += base;
          f->Q16 += base; f->Q16T += base; f->L16 += base; f->HT16 += base; f->B32 += base; f->jbuf += base;
        }
      }
      if (soap_mode) {
        jac_part_rel += base;
        jac_flag_rel += base;
      }
      ws_bufs.emplace_back();
      for (const std::pair<size_t, size_t>& b : pending) ws_bufs.back()[b.first + base] = b.second;
    }
    std::vector<LaunchRec> L;
    if (muon_mode) {
      plan_muon(L, mats);
      chunks.push_back(std::move(L));
      return;
    }
    if (soap_mode) {
      plan_soap(L, mats, refresh);
      (refresh ? chunks : chunks_stale).push_back(std::move(L));
      return;
    }
    if (nys_mode) {
      plan_nys(L, mats, refresh);
      (refresh ? chunks : chunks_stale).push_back(std::move(L));
      return;
    }
    // fp16 copies of the previous preconditioners: the OKLS factor products
    // read them, and a step that keeps the roots whitens with them
    const bool p_old = okls_mode || !refresh;
    const int fs = cfg.factor_split;
    auto gdt = [&](const MatBufs& mb) { return groups[mb.group].g_dtype; };
    auto gfmt = [&](const MatBufs& mb) {
      return gdt(mb) == OKLS_F32 ? GF_F32 : gdt(mb) == OKLS_BF16 ? GF_BF16 : GF_F16;
    };
    auto goff = [&](const MatBufs& mb) {
      return static_cast<size_t>(mb.index) * mb.m * mb.n * (gdt(mb) == OKLS_F32 ? 4 : 2);
    };
    auto moff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.n * 4; };
    auto aoff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.m * mb.m * 4; };
    auto boff = [&](const MatBufs& mb) { return static_cast<size_t>(mb.index) * mb.n * mb.n * 4; };

    // 1. statistics of G, N and the previous preconditioners
    std::vector<StatSpec> st;
    for (const MatBufs& mb : mats) {
      const int gk = gdt(mb) == OKLS_F32 ? ST_F32 : ST_H16;
      st.push_back(StatSpec{gk, user_ref(REF_G, mb.group, goff(mb)), mb.n, no_ref(), gfmt(mb), mb.m, mb.n});
      st.push_back(StatSpec{ST_NESTEROV, user_ref(REF_G, mb.group, goff(mb)), mb.n,
                            user_ref(REF_M, mb.group, moff(mb)), gfmt(mb), mb.m, mb.n});
      if (p_old) {
        st.push_back(StatSpec{ST_F32, user_ref(REF_PA, mb.group, aoff(mb)), mb.m, no_ref(), 0, mb.m, mb.m});
        st.push_back(StatSpec{ST_F32, user_ref(REF_PB, mb.group, boff(mb)), mb.n, no_ref(), 0, mb.n, mb.n});
      }
    }
    std::vector<std::pair<int, int>> parts = add_stats(L, st);
    // 2. casts
    std::vector<CastSpec> cs;
    const int per = p_old ? 4 : 2;
    for (size_t q = 0; q < mats.size(); ++q) {
      const MatBufs& mb = mats[q];
      CastSpec g = cast_spec();
      g.kind = gdt(mb) == OKLS_F32 ? CA_F32 : CA_H16; g.g_fmt = gfmt(mb); g.src = user_ref(REF_G, mb.group, goff(mb)); g.src_ld = mb.n;
      g.rows = mb.m; g.cols = mb.n; g.dst_rows_p = mb.mp; g.dst_cols_p = mb.np; g.dst = ws_ref(mb.G16);
      g.dst_ld = mb.ldn; g.dst_lo = mb.np; g.parts = parts[per * q]; g.scale_mode = SC_ABSMAX;
      g.scale_slot = mb.s_g; g.write_lo = fs;
      g.dstT = ws_ref(mb.G16T); g.dstT_ld = mb.ldm; g.dstT_lo = mb.mp;   // G^T from the same pass over G
      cs.push_back(g);
      CastSpec nn = cast_spec();
      nn.kind = CA_NESTEROV; nn.src = user_ref(REF_M, mb.group, moff(mb)); nn.src_ld = mb.n;
      nn.src2 = user_ref(REF_G, mb.group, goff(mb)); nn.g_fmt = gfmt(mb); nn.write_m = 1;
      nn.rows = mb.m; nn.cols = mb.n; nn.dst_rows_p = mb.mp; nn.dst_cols_p = mb.np; nn.dst = ws_ref(mb.N16);
      nn.dst_ld = mb.ldnw; nn.dst_lo = mb.np; nn.parts = parts[per * q + 1]; nn.scale_mode = SC_ABSMAX;
      nn.scale_slot = mb.s_n; nn.write_lo = wsplit();
      cs.push_back(nn);
      if (p_old) {
        const FacBufs* fl[2] = {&mb.fa, &mb.fb};
        const int kinds[2] = {REF_PA, REF_PB};
        const size_t offs[2] = {aoff(mb), boff(mb)};
        for (int s = 0; s < 2; ++s) {
          const FacBufs& F = *fl[s];
          CastSpec p = cast_spec();
          p.kind = CA_F32; p.src = user_ref(kinds[s], mb.group, offs[s]); p.src_ld = F.d;
          p.rows = p.cols = F.d; p.dst_rows_p = p.dst_cols_p = F.dp; p.dst = ws_ref(F.P16w);
          p.dst_ld = F.ldw; p.dst_lo = F.dp; p.parts = parts[per * q + 2 + s]; p.scale_mode = SC_ABSMAX;
          p.scale_slot = F.s_pold; p.write_lo = wsplit();
          cs.push_back(p);
        }
      }
    }
    add_cast(L, cs);

    // algorithmic work of this chunk (see okls_profile_stats)
    for (const MatBufs& mb : mats) {
      const double m = mb.m, n = mb.n;
      step_flops[CAT_FACTOR] += (okls_mode ? 3.0 : 1.0) * m * n * (m + n);
      step_flops[CAT_WHITEN] += 2.0 * m * n * (m + n);
      // 3K - 3 GEMMs per inverse square root (27 at K = 10), the first (Y_0
      // Y_0) on its upper half on the unsplit path; two chains for the fourth root
      if (refresh)
        step_flops[CAT_NS] += (okls_mode ? 1.0 : 2.0) * (3.0 * cfg.ns_steps - 3.0 - (cfg.ns_split_steps == 0 ? 0.5 : 0.0)) *
                              2.0 * (m * m * m + n * n * n);
    }
    gemm_cat = CAT_FACTOR;
    if (okls_mode) {
      // 3. X_a = G P_b (m x n), X_b^T = G^T P_a (n x m)
      std::vector<GemmProb> px;
      for (const MatBufs& mb : mats) {
        GemmProb p = prob();
        p.A = ws_ref(mb.G16); p.lda = mb.ldn; p.B = ws_ref(mb.fb.P16w); p.ldb = mb.fb.ldw;
        p.M = mb.m; p.N = mb.n; p.Kp = mb.np; p.Mp = mb.mp; p.Np = mb.np; p.epi = EPI_STORE32;
        p.out32 = ws_ref(mb.Xa32); p.ld32 = mb.n; p.sA = mb.s_g; p.sB = mb.fb.s_pold;
        px.push_back(p);
        GemmProb r = prob();
        r.A = ws_ref(mb.G16T); r.lda = mb.ldm; r.B = ws_ref(mb.fa.P16w); r.ldb = mb.fa.ldw;
        r.M = mb.n; r.N = mb.m; r.Kp = mb.mp; r.Mp = mb.np; r.Np = mb.mp; r.epi = EPI_STORE32;
        r.out32 = ws_ref(mb.XbT32); r.ld32 = mb.m; r.sA = mb.s_g; r.sB = mb.fa.s_pold;
        px.push_back(r);
      }
      add_gemm(L, px, false, fs, 0);
      std::vector<StatSpec> sx;
      for (const MatBufs& mb : mats) {
        sx.push_back(StatSpec{ST_F32, ws_ref(mb.Xa32), mb.n, no_ref(), 0, mb.m, mb.n});
        sx.push_back(StatSpec{ST_F32, ws_ref(mb.XbT32), mb.m, no_ref(), 0, mb.n, mb.m});
      }
      std::vector<std::pair<int, int>> px_parts = add_stats(L, sx);
      std::vector<CastSpec> cx;
      for (size_t q = 0; q < mats.size(); ++q) {
        const MatBufs& mb = mats[q];
        CastSpec a = cast_spec();
        a.kind = CA_F32; a.src = ws_ref(mb.Xa32); a.src_ld = mb.n; a.rows = mb.m; a.cols = mb.n;
        a.dst_rows_p = mb.mp; a.dst_cols_p = mb.np; a.dst = ws_ref(mb.Xa16); a.dst_ld = mb.ldn; a.dst_lo = mb.np;
        a.parts = px_parts[2 * q]; a.scale_mode = SC_ABSMAX; a.scale_slot = mb.s_xa; a.write_lo = fs;
        cx.push_back(a);
        CastSpec b = cast_spec();
        b.kind = CA_F32; b.src = ws_ref(mb.XbT32); b.src_ld = mb.m; b.rows = mb.n; b.cols = mb.m;
        b.dst_rows_p = mb.np; b.dst_cols_p = mb.mp; b.dst = ws_ref(mb.XbT16); b.dst_ld = mb.ldm; b.dst_lo = mb.mp;
        b.parts = px_parts[2 * q + 1]; b.scale_mode = SC_ABSMAX; b.scale_slot = mb.s_xb; b.write_lo = fs;
        cx.push_back(b);
      }
      add_cast(L, cx);
    }

    // 4. factor update (upper tiles, mirrored)
    {
      std::vector<GemmProb> ps;
      for (const MatBufs& mb : mats) {
        GemmProb a = prob();
        a.A = a.B = ws_ref(okls_mode ? mb.Xa16 : mb.G16); a.lda = a.ldb = mb.ldn;
        a.M = a.N = mb.m; a.Kp = mb.np; a.Mp = a.Np = mb.mp; a.epi = EPI_SYRK;
        a.out32 = user_ref(REF_SA, mb.group, aoff(mb)); a.ld32 = mb.m;
        a.sA = a.sB = okls_mode ? mb.s_xa : mb.s_g;
        a.c0 = okls_mode ? cfg.beta2 : 1.0f;
        a.c1 = okls_mode ? static_cast<float>((1.0 - cfg.beta2) / mb.n) : 1.0f;
        a.c2 = factor_eps();
        ps.push_back(a);
        GemmProb b = prob();
        b.A = b.B = ws_ref(okls_mode ? mb.XbT16 : mb.G16T); b.lda = b.ldb = mb.ldm;
        b.M = b.N = mb.n; b.Kp = mb.mp; b.Mp = b.Np = mb.np; b.epi = EPI_SYRK;
        b.out32 = user_ref(REF_SB, mb.group, boff(mb)); b.ld32 = mb.n;
        b.sA = b.sB = okls_mode ? mb.s_xb : mb.s_g;
        b.c0 = okls_mode ? cfg.beta2 : 1.0f;
        b.c1 = okls_mode ? static_cast<float>((1.0 - cfg.beta2) / mb.m) : 1.0f;
        b.c2 = factor_eps();
        ps.push_back(b);
      }
      add_gemm(L, ps, true, fs, 0);
    }

    // 5. inverse roots
    gemm_cat = CAT_NS;
    if (refresh) {
      std::vector<FacBufs*> facs;
      std::vector<Ref> src, pdst;
      for (MatBufs& mb : mats) {
        mb.fa.mat = mb.fb.mat = mat_base[mb.group] + mb.index;
        mb.fa.side = 0;
        mb.fb.side = 1;
        facs.push_back(&mb.fa);
        src.push_back(user_ref(REF_SA, mb.group, aoff(mb)));
        pdst.push_back(user_ref(REF_PA, mb.group, aoff(mb)));
        facs.push_back(&mb.fb);
        src.push_back(user_ref(REF_SB, mb.group, boff(mb)));
        pdst.push_back(user_ref(REF_PB, mb.group, boff(mb)));
      }
      // split the factors into kNsStreams sets of near-equal cost (d^3, largest first)
      std::vector<size_t> order(facs.size());
      for (size_t f = 0; f < order.size(); ++f) order[f] = f;
      std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return facs[x]->d > facs[y]->d; });
      const int nset = (!single_chain && two_chains_pay(facs)) ? std::min<int>(kNsStreams, static_cast<int>(facs.size())) : 1;
      std::vector<double> load(nset, 0.0);
      std::vector<std::vector<size_t>> sets(nset);
      for (size_t f : order) {
        const int b = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
        sets[b].push_back(f);
        load[b] += std::pow(static_cast<double>(facs[f]->d), 3.0);
      }
      std::vector<std::vector<LaunchRec>> chains(nset);
      for (int c = 0; c < nset; ++c) {
        std::sort(sets[c].begin(), sets[c].end());
        std::vector<FacBufs*> cf;
        std::vector<Ref> cs, cp;
        for (size_t f : sets[c]) { cf.push_back(facs[f]); cs.push_back(src[f]); cp.push_back(pdst[f]); }
        if (okls_mode) {
          ns_chain(chains[c], cf, cs, cp, OUT_INV, true, 0);
        } else {
          // S^{-1/4} = (S^{-1/2})^{1/2}: the first chain's inverse root into
          // R32, then the square root of sym(R32) into the caller's P
          std::vector<Ref> rsrc;
          for (FacBufs* f : cf) rsrc.push_back(ws_ref(f->R32));
          ns_chain(chains[c], cf, cs, rsrc, OUT_INV, false, 0);
          ns_chain(chains[c], cf, rsrc, cp, OUT_SQRT, true, 1);
        }
        for (LaunchRec& r : chains[c]) r.stream = c;
      }
      if (nset > 1) {
        LaunchRec fork;
        fork.type = L_FORK;
        L.push_back(fork);
      }
      // issue the chains' launches interleaved so both streams have work queued
      for (size_t i = 0;; ++i) {
        bool any = false;
        for (int c = 0; c < nset; ++c)
          if (i < chains[c].size()) { L.push_back(chains[c][i]); any = true; }
        if (!any) break;
      }
      if (nset > 1) {
        LaunchRec join;
        join.type = L_JOIN;
        L.push_back(join);
      }
    }
    // the fp16 preconditioner each whitening product reads: the symmetrised
    // chain output's copy when the roots were just recomputed, else the copy
    // cast above (both in P16w)
    auto pw = [&](const FacBufs& F) { return ws_ref(F.P16w); };
    auto pw_scale = [&](const FacBufs& F) { return refresh ? F.s_p16 : F.s_pold; };

    // 6. whitening: V^T = P_b N^T (n x m), then U = P_a V fused with the update
    gemm_cat = CAT_WHITEN;
    {
      std::vector<GemmProb> pv;
      for (const MatBufs& mb : mats) {
        GemmProb p = prob();
        p.A = pw(mb.fb); p.lda = mb.fb.ldw; p.B = ws_ref(mb.N16); p.ldb = mb.ldnw;
        p.M = mb.n; p.N = mb.m; p.Kp = mb.np; p.Mp = mb.np; p.Np = mb.mp; p.epi = EPI_STORE32;
        p.out32 = ws_ref(mb.VT32); p.ld32 = mb.m; p.sA = pw_scale(mb.fb); p.sB = mb.s_n;
        pv.push_back(p);
      }
      add_gemm(L, pv, false, wsplit(), 0);
      std::vector<StatSpec> sv;
      for (const MatBufs& mb : mats) sv.push_back(StatSpec{ST_F32, ws_ref(mb.VT32), mb.m, no_ref(), 0, mb.n, mb.m});
      std::vector<std::pair<int, int>> pvp = add_stats(L, sv);
      std::vector<CastSpec> cv;
      for (size_t q = 0; q < mats.size(); ++q) {
        const MatBufs& mb = mats[q];
        CastSpec c = cast_spec();
        c.kind = CA_F32; c.src = ws_ref(mb.VT32); c.src_ld = mb.m; c.rows = mb.n; c.cols = mb.m;
        c.dst_rows_p = mb.np; c.dst_cols_p = mb.mp; c.dst = ws_ref(mb.VT16); c.dst_ld = mb.ldmw; c.dst_lo = mb.mp;
        c.parts = pvp[q]; c.scale_mode = SC_ABSMAX; c.scale_slot = mb.s_vt; c.write_lo = wsplit();
        cv.push_back(c);
      }
      add_cast(L, cv);
      std::vector<GemmProb> pu;
      for (const MatBufs& mb : mats) {
        GemmProb p = prob();
        p.A = pw(mb.fa); p.lda = mb.fa.ldw; p.B = ws_ref(mb.VT16); p.ldb = mb.ldmw;
        p.M = mb.m; p.N = mb.n; p.Kp = mb.mp; p.Mp = mb.mp; p.Np = mb.np; p.epi = EPI_UPDATE;
        p.out32 = user_ref(REF_W, mb.group, moff(mb)); p.ld32 = mb.n; p.sA = pw_scale(mb.fa); p.sB = mb.s_vt;
        p.c0 = update_scale(mb);
        pu.push_back(p);
      }
      add_gemm(L, pu, false, wsplit(), 0);
    }
    (refresh ? chunks : chunks_stale).push_back(std::move(L));
  }

  // ---- host-side extent checks of every descriptor against the buffer it
  // points into; a failure is a planning error and nothing is launched.
  const std::map<size_t, size_t>* cur_bufs = nullptr;
  bool fits_ws(const Ref& r, size_t bytes) const {
    auto it = cur_bufs->upper_bound(static_cast<size_t>(r.off));
    if (it == cur_bufs->begin()) return false;
    --it;
    return static_cast<size_t>(r.off) >= it->first && static_cast<size_t>(r.off) + bytes <= it->first + it->second;
  }
  size_t user_bytes(int kind, int group) const {
    const okls_group_desc& g = groups[group];
    const size_t b = static_cast<size_t>(g.batch);
    if (nys_mode) {   // U (N, d, r'), Lambda (N, r'), Psi (N, d, k) per side
      switch (kind) {
        case REF_SA: return b * nys_r(g.m) * 4;
        case REF_SB: return b * nys_r(g.n) * 4;
        case REF_PA: return b * g.m * nys_r(g.m) * 4;
        case REF_PB: return b * g.n * nys_r(g.n) * 4;
        case REF_PSA: return b * g.m * nys_k(g.m) * 4;
        case REF_PSB: return b * g.n * nys_k(g.n) * 4;
        default: break;
      }
    }
    switch (kind) {
      case REF_W: case REF_M: case REF_V: return b * g.m * g.n * 4;
      case REF_G: return b * g.m * g.n * (g.g_dtype == OKLS_F32 ? 4 : 2);
      case REF_SA: case REF_PA: return b * g.m * g.m * 4;
      case REF_SB: case REF_PB: return b * g.n * g.n * 4;
    }
    return 0;
  }
  bool fits(const Ref& r, size_t bytes) const {
    if (r.kind == REF_WS) return fits_ws(r, bytes);
    if (r.kind < REF_W || r.kind > REF_PSB || r.group < 0 || r.group >= static_cast<int>(groups.size())) return false;
    if (r.kind == REF_V && !soap_mode) return false;
    if ((r.kind == REF_PSA || r.kind == REF_PSB) && !nys_mode) return false;
    return r.off >= 0 && static_cast<size_t>(r.off) + bytes <= user_bytes(r.kind, r.group);
  }
  bool slot_ok(int s) const { return s >= 0 && s < n_slots; }

  // whether some steps keep the roots (SOAP: the bases) and run their own plan
  bool has_stale() const { return soap_mode ? cfg.precond_freq > 1 : (cfg.root_period > 1 && !muon_mode); }
  // Nystrom: (sketch columns, kept eigenpairs) of a side d
  int nys_k(int d) const { return std::min(cfg.nys_rank + cfg.nys_oversample, d); }
  int nys_r(int d) const { return std::min(cfg.nys_rank, nys_k(d)); }
  bool validate() {
    if (!validate_plan(chunks)) return false;
    return has_stale() ? validate_plan(chunks_stale) : chunks_stale.empty();
  }
  bool validate_plan(const std::vector<std::vector<LaunchRec>>& plan_chunks) {
    if (ws_bufs.size() != plan_chunks.size()) return false;
    for (size_t ci = 0; ci < plan_chunks.size(); ++ci) {
      cur_bufs = &ws_bufs[ci];
      bool forked = false;
      for (const LaunchRec& r : plan_chunks[ci]) {
        if (r.type == L_FORK || r.type == L_JOIN) {
          if (forked == (r.type == L_FORK)) return false;
          forked = r.type == L_FORK;
          continue;
        }
        if (r.stream < 0 || r.stream >= kNsStreams || (r.stream != 0 && !forked)) return false;
        if (r.type == L_GEMM) {
          if (r.first < 0 || r.first + r.count > static_cast<int>(tiles.size())) return false;
          if (r.tile != kTile && r.tile != kBigTile) return false;
          if (r.epi < EPI_STORE32 || r.epi > EPI_NS_T_RES) return false;
          const int segs = r.split_in ? 2 : 1;
          for (int t = r.first; t < r.first + r.count; ++t) {
            const TileRef tr = tiles[t];
            const int q = r.prob_base + tr.prob;
            if (tr.prob < 0 || q >= static_cast<int>(probs.size())) return false;
            const GemmProb& p = probs[q];
            if (p.epi != r.epi) return false;
            const int ti = tr.ij >> 16, tj = tr.ij & 0xffff;
            if (p.Mp % r.tile || p.Np % r.tile || p.Kp % kTile || p.Kp <= 0) return false;
            if (ti < 0 || tj < 0 || ti >= p.Mp / r.tile || tj >= p.Np / r.tile) return false;
            if (p.M > p.Mp || p.N > p.Np || p.M < 1 || p.N < 1) return false;
            if (p.sym_out != 0 && p.sym_out != 1) return false;
            // a symmetric product on its upper tiles: one unsplit square operand
            // and two fp16 copies of one layout
            if (p.sym_out && ((p.epi != EPI_NS_Y1 && p.epi != EPI_STORE16) || r.split_in || r.write_lo || ti > tj ||
                              p.M != p.N || p.Mp != p.Np || p.A.kind != p.B.kind || p.A.group != p.B.group ||
                              p.A.off != p.B.off || p.lda != p.ldb || p.out16.kind == REF_NONE ||
                              (p.out16T.kind != REF_NONE && (p.ld16T != p.ld16 || p.lo16T != p.lo16))))
              return false;
            if (p.lda < segs * p.Kp || p.ldb < segs * p.Kp) return false;
            if (!fits(p.A, static_cast<size_t>(p.Mp) * p.lda * 2) || !fits(p.B, static_cast<size_t>(p.Np) * p.ldb * 2))
              return false;
            if (!slot_ok(p.sA) || !slot_ok(p.sB)) return false;
            if (p.s_out >= 0 && !slot_ok(p.s_out)) return false;
            if (p.cslot >= 0 && !slot_ok(p.cslot)) return false;
            const bool need32 = p.epi == EPI_STORE32 || p.epi == EPI_SYRK || p.epi == EPI_UPDATE ||
                                p.epi == EPI_POLAR_UPDATE || (p.epi == EPI_NS_FINAL && p.out32.kind != REF_NONE);
            if (need32) {
              if (p.out32.kind == REF_NONE || p.ld32 < p.N) return false;
              if (!fits(p.out32, (static_cast<size_t>(p.M - 1) * p.ld32 + p.N) * 4)) return false;
              if (p.epi == EPI_SYRK && p.M != p.N) return false;
            }
            const bool need16 = p.epi == EPI_NS_T || p.epi == EPI_NS_T_RES || p.epi == EPI_NS_Y1 || p.epi == EPI_STORE16 ||
                                p.epi == EPI_POLAR || (p.epi == EPI_NS_FINAL && p.out16.kind != REF_NONE);
            if (need16) {
              if (p.out16.kind == REF_NONE || !slot_ok(p.s_out)) return false;
              const int need_ld = r.write_lo ? p.lo16 + p.Np : p.Np;
              if (p.ld16 < need_ld || (r.write_lo && p.lo16 < p.Np)) return false;
              if (!fits(p.out16, static_cast<size_t>(p.Mp) * p.ld16 * 2)) return false;
              if (p.out16T.kind != REF_NONE) {   // Np x Mp with its own stride and lo offset
                const int need_ldT = r.write_lo ? p.lo16T + p.Mp : p.Mp;
                if (p.ld16T < need_ldT || (r.write_lo && p.lo16T < p.Mp)) return false;
                if (!fits(p.out16T, static_cast<size_t>(p.Np) * p.ld16T * 2)) return false;
              }
            }
            if (p.epi == EPI_POLAR || p.epi == EPI_POLAR_UPDATE) {   // fp16 aux over the padded output
              if (p.aux.kind == REF_NONE || !slot_ok(p.s_aux) || !slot_ok(p.cslot)) return false;
              const int need_lda = p.aux_lo >= 0 ? p.aux_lo + p.Np : p.Np;
              if (p.ldaux < need_lda || (p.aux_lo >= 0 && p.aux_lo < p.Np) || (p.ldaux & 3) || (p.aux_lo > 0 && (p.aux_lo & 3)))
                return false;
              if (!fits(p.aux, static_cast<size_t>(p.Mp) * p.ldaux * 2)) return false;
            }
            if (p.epi == EPI_NS_T_RES) {   // one partial per wave and tile: the small tile's count at most
              if (p.resid < 0 || p.Mp % kTile || p.Np % kTile) return false;
              const long need = static_cast<long>(p.Mp / kTile) * (p.Np / kTile) * 4;
              if (p.resid + need > resid_floats) return false;
            }
            if (p.epi == EPI_NS_Y1) {
              if (p.aux.kind == REF_NONE || p.ldaux < p.N || !slot_ok(p.cslot)) return false;
              if (!fits(p.aux, (static_cast<size_t>(p.M - 1) * p.ldaux + p.N) * 4)) return false;
            }
          }
        } else if (r.type == L_THIN) {
          if (r.first < 0 || r.first + r.count > static_cast<int>(thin_jobs.size())) return false;
          if (r.thin_ta < 0 || r.thin_ta > 1 || r.thin_mom < 0 || r.thin_mom > 1 || (r.thin_ta && r.thin_mom)) return false;
          if (r.thin_cbm != 1 && r.thin_cbm != 2 && r.thin_cbm != 4) return false;
          if (r.thin_wupd != 0 && (r.thin_wupd != 1 || r.thin_cbm != 1 || r.thin_ta || r.thin_mom)) return false;
          int blk = 0;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const ThinJob& q = thin_jobs[j];
            if (q.ta != r.thin_ta || q.mom != r.thin_mom || q.ot < 0 || q.ot > 1) return false;
            if (q.Mo < 1 || q.K < 1 || q.R < 1 || q.R > 32 * r.thin_cbm || q.blk_begin != blk) return false;
            blk += (q.Mo + kThinTile - 1) / kThinTile;
            const int ar = q.ta ? q.K : q.Mo, ac = q.ta ? q.Mo : q.K;
            const int cr = q.ot ? q.R : q.Mo, cc = q.ot ? q.Mo : q.R;
            if (q.lda < ac || q.ldb < q.R || q.ldc < cc) return false;
            if (!fits(q.A, (static_cast<size_t>(ar - 1) * q.lda + ac) * (q.a_fmt == GF_F32 ? 4 : 2))) return false;
            if (!fits(q.B, (static_cast<size_t>(q.K - 1) * q.ldb + q.R) * 4)) return false;
            if (!fits(q.C, (static_cast<size_t>(cr - 1) * q.ldc + cc) * 4)) return false;
            if (q.mom) {   // M: the gradient's shape and stride; N: Mo x K, stride ldn
              if (q.ldn < q.K || !fits(q.M, (static_cast<size_t>(ar - 1) * q.lda + ac) * 4) ||
                  !fits(q.Nout, (static_cast<size_t>(q.Mo - 1) * q.ldn + q.K) * 4))
                return false;
            }
            if (q.alpha_slot >= 0 && !slot_ok(q.alpha_slot)) return false;
            if (q.rowscale.kind != REF_NONE && (q.ot != 0 || !fits(q.rowscale, static_cast<size_t>(q.Mo) * 4))) return false;
            if (q.wupd != r.thin_wupd) return false;
            if (q.wupd && (q.ot != 0 || q.ta != 0 || q.mom != 0 || q.C.kind != REF_W || q.rowscale.kind != REF_NONE ||
                           !fits(q.aux, (static_cast<size_t>(q.Mo - 1) * q.ldc + q.R) * 4)))
              return false;
          }
          if (blk != r.nblocks) return false;
        } else if (r.type == L_NORTH) {
          if (r.first < 0 || r.first + r.count > static_cast<int>(north_jobs.size()) || r.nblocks != r.count) return false;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const NysOrthJob& q = north_jobs[j];
            if (q.d < 1 || q.k < 1 || q.k > q.d || q.k > kNysMaxK || q.ld < q.k || q.ldf < q.k || q.fb_shift < 0) return false;
            if (!fits(q.Y, (static_cast<size_t>(q.d - 1) * q.ld + q.k) * 4)) return false;
            if (!fits(q.fb, (static_cast<size_t>(q.d - 1) * q.ldf + q.k) * 4)) return false;
          }
        } else if (r.type == L_NSMALL) {
          if (r.first < 0 || r.first + r.count > static_cast<int>(nsmall_jobs.size()) || r.nblocks != r.count) return false;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const NysSmallJob& q = nsmall_jobs[j];
            if (q.k < 1 || q.k > kNysMaxK || q.r < 1 || q.r > q.k || (r.round != 1 && r.round != 2)) return false;
            const size_t kk = static_cast<size_t>(q.k) * q.k * 4, kr = static_cast<size_t>(q.k) * q.r * 4;
            if (!fits(q.gram, kk) || !fits(q.cmat, kk) || !fits(q.ftu, kr) || !fits(q.kout, kr)) return false;
            if (!fits(q.lam, static_cast<size_t>(q.r) * 4) || !fits(q.scratch, 2 * static_cast<size_t>(q.k) * q.k * 8)) return false;
            if (!slot_ok(q.nu_slot) || !slot_ok(q.nuu_slot)) return false;
          }
        } else if (r.type == L_NELEM) {
          if (r.first < 0 || r.first + r.count > static_cast<int>(nelem_jobs.size())) return false;
          int blk = 0;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const NysElemJob& q = nelem_jobs[j];
            if (q.kind < NE_GATHER || q.kind > NE_SCALE || q.rows < 1 || q.cols < 1 || q.blk_begin != blk || q.blocks < 1) return false;
            blk += q.blocks;
            if (q.trans && q.kind != NE_SCALE) return false;
            const int dr = q.trans ? q.cols : q.rows, dc = q.trans ? q.rows : q.cols;
            if (q.ld_dst < dc || !fits(q.dst, (static_cast<size_t>(dr - 1) * q.ld_dst + dc) * 4)) return false;
            const int scols = q.kind == NE_GATHER ? q.cols1 : q.cols;
            if (scols > 0 && (q.ld_src < scols || !fits(q.src, (static_cast<size_t>(q.rows - 1) * q.ld_src + scols) * 4)))
              return false;
            if (q.kind == NE_GATHER) {
              const int c2 = q.cols - q.cols1;
              if (q.cols1 < 0 || q.cols1 > q.cols) return false;
              if (c2 > 0 && (q.ld_src2 < c2 || !fits(q.src2, (static_cast<size_t>(q.rows - 1) * q.ld_src2 + c2) * 4))) return false;
            }
            if (q.kind == NE_SCALE && !fits(q.lam, static_cast<size_t>(q.cols) * 4)) return false;
          }
          if (blk != r.nblocks) return false;
        } else if (r.type == L_ADAM) {
          int blk = 0;
          if (r.first < 0 || r.first + r.count > static_cast<int>(adam_jobs.size())) return false;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const AdamJob& a = adam_jobs[j];
            if (a.blk_begin != blk || a.rows < 1 || a.cols < 1 || a.rows_p < a.rows || a.cols_p < a.cols) return false;
            if (a.rows_p % kAdamRows || a.cols_p % 4 || a.tiles_x != (a.cols_p + 255) / 256) return false;
            blk += a.tiles_x * (a.rows_p / kAdamRows);
            const size_t f32 = static_cast<size_t>(a.rows) * a.cols * 4;
            if (!fits(a.g, f32) || !fits(a.m, f32) || !fits(a.v, f32)) return false;
            if (a.dst.kind == REF_NONE) {
              if (!fits(a.dst32, f32)) return false;
            } else {
              const int need_ld = wsplit_soap() ? a.lo16 + a.cols_p : a.cols_p;
              if (a.ld16 < need_ld || (wsplit_soap() && a.lo16 < a.cols_p)) return false;
              if (!fits(a.dst, static_cast<size_t>(a.rows_p) * a.ld16 * 2)) return false;
            }
          }
          if (blk != r.nblocks) return false;
        } else if (r.type == L_JAC) {
          if (r.jac_kind < JAC_RESET || r.jac_kind > JAC_CHECK) return false;
          if (r.first < 0 || r.first + r.count > static_cast<int>(jac_jobs.size())) return false;
          int solve = 0, apply = 0, part = 0;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const JacJob& q = jac_jobs[j];
            if (q.d < 1 || q.nb < 2 || (q.nb & 1) || q.nb * kJb < q.d || q.npairs * 2 != q.nb) return false;
            if (q.btiles != q.npairs * (q.npairs + 1) / 2 || q.vrows != (q.d + kJp - 1) / kJp) return false;
            if (q.solve_begin != solve || q.apply_begin != apply || q.part != part || q.flag != j - r.first) return false;
            solve += q.npairs;
            if (q.apply_items != 1 && q.apply_items != kJacApplyItems) return false;
            apply += (q.btiles + q.vrows * q.npairs + q.apply_items - 1) / q.apply_items;
            part += q.btiles;
            const size_t dd = static_cast<size_t>(q.d) * q.d * 4;
            if (!fits(q.B, dd) || !fits(q.V, dd)) return false;
            if (q.V.kind != REF_PA && q.V.kind != REF_PB) return false;
            if (!fits(ws_ref(static_cast<size_t>(q.jbuf)), static_cast<size_t>(q.npairs) * kJp * kJp * 4)) return false;
          }
          if (!fits(ws_ref(r.jac_part), static_cast<size_t>(part) * 2 * sizeof(float))) return false;
          if (!fits(ws_ref(r.jac_flag), static_cast<size_t>(r.count) * sizeof(int32_t))) return false;
          const int want = r.jac_kind == JAC_SOLVE ? solve : r.jac_kind == JAC_APPLY ? apply
                         : r.jac_kind == JAC_CHECK ? r.count : 1;
          if (r.nblocks != want || r.round < 0) return false;
        } else if (r.type == L_SYM) {
          int blk = 0;
          if (r.first < 0 || r.first + r.count > static_cast<int>(sym_jobs.size())) return false;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const SymJob& y = sym_jobs[j];
            if (y.blk_begin != blk || y.d < 1 || y.dp < y.d || y.dp % kSymTile || y.nt != y.dp / kSymTile) return false;
            blk += y.nt * (y.nt + 1) / 2;
            if (!fits(y.p, static_cast<size_t>(y.d) * y.d * 4)) return false;
            if (y.dst16.kind != REF_NONE) {
              const int need_ld = y.write_lo ? y.lo16 + y.dp : y.dp;
              if (y.ld16 < need_ld || (y.write_lo && y.lo16 < y.dp) || !slot_ok(y.scale_slot)) return false;
              if (!fits(y.dst16, static_cast<size_t>(y.dp) * y.ld16 * 2)) return false;
            }
          }
          if (blk != r.nblocks) return false;
        } else if (r.type == L_STAT) {
          int blk = 0;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const StatJob& s = stat_jobs[j];
            if (s.blk_begin != blk || s.rows < 1 || s.cols < 1 || s.src_ld < s.cols || s.rows_per_blk < 1) return false;
            const int nb = (s.rows + s.rows_per_blk - 1) / s.rows_per_blk;
            blk += nb;
            if (s.part_begin < 0 || s.part_begin + nb > max_partials) return false;
            const size_t esz = (s.kind == ST_H16 || (s.kind == ST_NESTEROV && s.g_fmt != GF_F32)) ? 2 : 4;
            if (!fits(s.src, (static_cast<size_t>(s.rows - 1) * s.src_ld + s.cols) * esz)) return false;
            if (s.kind == ST_NESTEROV && !fits(s.src2, (static_cast<size_t>(s.rows - 1) * s.src_ld + s.cols) * 4))
              return false;
          }
          if (blk != r.nblocks) return false;
        } else {
          int blk = 0;
          for (int j = r.first; j < r.first + r.count; ++j) {
            const CastJob& c = cast_jobs[j];
            if (c.blk_begin != blk) return false;
            if (c.dst_rows_p % kCastRows || c.dst_cols_p % 4 ||
                c.tiles_x != (c.dst_cols_p + kCastCols - 1) / kCastCols) return false;
            blk += c.tiles_x * (c.dst_rows_p / kCastRows);
            const int drows = c.transpose ? c.cols : c.rows, dcols = c.transpose ? c.rows : c.cols;
            if (drows > c.dst_rows_p || dcols > c.dst_cols_p || c.src_ld < c.cols || c.rows < 1 || c.cols < 1) return false;
            const int need_ld = c.write_lo ? c.dst_lo + c.dst_cols_p : c.dst_cols_p;
            if (c.dst_ld < need_ld || (c.write_lo && c.dst_lo < c.dst_cols_p)) return false;
            if (!fits(c.dst, static_cast<size_t>(c.dst_rows_p) * c.dst_ld * 2)) return false;
            const size_t esz = (c.kind == CA_H16) ? 2 : 4;
            if (!fits(c.src, (static_cast<size_t>(c.rows - 1) * c.src_ld + c.cols) * esz)) return false;
            if (c.kind == CA_NESTEROV) {
              if (c.transpose) return false;
              if (!fits(c.src2, (static_cast<size_t>(c.rows - 1) * c.src_ld + c.cols) * (c.g_fmt == GF_F32 ? 4 : 2))) return false;
            }
            if (c.kind == CA_NS_Y0 && (c.rows != c.cols || c.transpose)) return false;
            if (c.dstT.kind != REF_NONE) {   // dst_cols_p x dst_rows_p, same lo flag
              if (c.transpose) return false;
              const int need_ldT = c.write_lo ? c.dstT_lo + c.dst_rows_p : c.dst_rows_p;
              if (c.dstT_ld < need_ldT || (c.write_lo && c.dstT_lo < c.dst_rows_p)) return false;
              if (!fits(c.dstT, static_cast<size_t>(c.dst_cols_p) * c.dstT_ld * 2)) return false;
            }
            if (c.dst2.kind != REF_NONE) {
              if (c.kind != CA_NS_Y0 || !slot_ok(c.scale_slot2)) return false;
              if (c.write_lo2 && !c.write_lo) return false;     // the lo offset is checked through dst's
              if (!fits(c.dst2, static_cast<size_t>(c.dst_rows_p) * c.dst_ld * 2)) return false;
            }
            if (c.part_begin < 0 || c.part_count < 1 || c.part_count > kMaxJobParts ||
                c.part_begin + c.part_count > max_partials) return false;
            if (!slot_ok(c.scale_slot)) return false;
            if (c.aux_slot >= 0 && !slot_ok(c.aux_slot)) return false;
            for (int s : {c.cinv_slot, c.rho_slot, c.sqrtc_slot, c.p16_slot})
              if (s >= 0 && !slot_ok(s)) return false;
          }
          if (blk != r.nblocks) return false;
        }
      }
      if (forked) return false;
    }
    return true;
  }

  // Plans every chunk; chunk buffers start at `base` (identical across chunks).
  void plan(size_t base) {
    resid_slots.clear();
    resid_floats = 0;
    std::vector<std::vector<MatBufs>> all;
    std::vector<MatBufs> cur;
    const int cap = cfg.chunk_matrices > 0 ? cfg.chunk_matrices : (1 << 30);
    for (size_t g = 0; g < groups.size(); ++g)
      for (int i = 0; i < groups[g].batch; ++i) {
        MatBufs mb;
        mb.group = static_cast<int>(g);
        mb.index = i;
        cur.push_back(mb);
        if (static_cast<int>(cur.size()) == cap) { all.push_back(cur); cur.clear(); }
      }
    if (!cur.empty()) all.push_back(cur);
    chunk_bytes = 0;
    for (std::vector<MatBufs>& c : all) {
      int slot = first_dyn;
      chunk_bytes = std::max(chunk_bytes, layout_chunk(c, slot));
      n_slots = std::max(n_slots, slot);
      plan_chunk(c, base, true, true);
    }
    if (has_stale()) {
      // the plan of the steps that keep the roots (SOAP: the bases), over
      // the same buffers, with its own algorithmic work
      double f[OKLS_PROFILE_CATEGORIES], b[OKLS_PROFILE_CATEGORIES];
      for (int i = 0; i < OKLS_PROFILE_CATEGORIES; ++i) {
        f[i] = step_flops[i]; b[i] = step_bytes[i];
        step_flops[i] = step_bytes[i] = 0.0;
      }
      for (std::vector<MatBufs>& c : all) plan_chunk(c, base, false, false);
      for (int i = 0; i < OKLS_PROFILE_CATEGORIES; ++i) {
        step_flops_stale[i] = step_flops[i]; step_bytes_stale[i] = step_bytes[i];
        step_flops[i] = f[i]; step_bytes[i] = b[i];
      }
    }
  }
};

struct WsLayout {
  size_t probs = 0, tiles = 0, stat = 0, cast = 0, sym = 0, adam = 0, jac = 0, north = 0, nsmall = 0,
         nelem = 0, thin = 0, scal = 0, part = 0, flag = 0, resid = 0, chunk = 0, total = 0;
};

WsLayout ws_layout(Planner& P) {
  // tables depend on the chunk base only through offsets; plan with base 0 to size them
  P.plan(0);
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max<size_t>(bytes, 1), kAlign); return o; };
  w.probs = take(P.probs.size() * sizeof(GemmProb));
  w.tiles = take(P.tiles.size() * sizeof(TileRef));
  w.stat = take(P.stat_jobs.size() * sizeof(StatJob));
  w.cast = take(P.cast_jobs.size() * sizeof(CastJob));
  w.sym = take(P.sym_jobs.size() * sizeof(SymJob));
  w.adam = take(P.adam_jobs.size() * sizeof(AdamJob));
  w.jac = take(P.jac_jobs.size() * sizeof(JacJob));
  w.north = take(P.north_jobs.size() * sizeof(NysOrthJob));
  w.nsmall = take(P.nsmall_jobs.size() * sizeof(NysSmallJob));
  w.nelem = take(P.nelem_jobs.size() * sizeof(NysElemJob));
  w.thin = take(P.thin_jobs.size() * sizeof(ThinJob));
  w.scal = take(static_cast<size_t>(P.n_slots) * sizeof(float));
  w.part = take(static_cast<size_t>(P.max_partials) * 2 * sizeof(float) * kNsStreams);   // one region per stream
  w.flag = take(sizeof(int));
  w.resid = take(static_cast<size_t>(P.resid_floats) * sizeof(float));
  w.chunk = off;
  w.total = off + P.chunk_bytes;
  return w;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

UserPtrs user_ptrs(const okls_handle* h, const okls_group_tensors* t) {
  UserPtrs u;
  std::memset(&u, 0, sizeof(u));
  for (size_t g = 0; g < h->groups.size(); ++g) {
    u.p[g][REF_W] = t[g].W;
    u.p[g][REF_G] = const_cast<void*>(t[g].G);
    u.p[g][REF_M] = t[g].M;
    u.p[g][REF_SA] = t[g].Sa;
    u.p[g][REF_SB] = t[g].Sb;
    u.p[g][REF_PA] = t[g].Pa;
    u.p[g][REF_PB] = t[g].Pb;
    u.p[g][REF_V] = t[g].V;
    u.p[g][REF_PSA] = const_cast<float*>(t[g].PsiA);
    u.p[g][REF_PSB] = const_cast<float*>(t[g].PsiB);
  }
  return u;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

void okls_default_config(okls_config* c) {
  if (c == nullptr) return;
  std::memset(c, 0, sizeof(*c));
  c->mode = OKLS_MODE_OKLS;
  c->ns_steps = 10;
  c->ns_split_steps = 0;
  c->factor_split = 0;
  c->nesterov_var_corr = 1;
  c->chunk_matrices = 0;
  c->beta1 = 0.9684f;
  c->beta2 = 0.9482f;
  c->eps = 1e-9f;
  c->weight_decay = 0.0303f;
  c->lr_peak = 0.09434f;
  c->ns_floor = 3e-2f;
  c->ns_damping = 0.0f;
  c->root_period = 1;
  c->eps_convex = 0;
  c->decay_after = 0;
  c->shape_scale = 1;
  c->ns_classical = 0;
  c->whiten_split = 1;
  c->soap_beta = 0.95f;
  c->precond_freq = 10;
  c->soap_moments = 0;
  c->bias_correction = 1;
  c->jacobi_sweeps = 20;
  c->jacobi_tol = 2e-6f;
  c->nys_rank = 32;
  c->nys_oversample = 8;
  c->nys_passes = 1;
  c->jacobi_apply_tiles = 0;
}

size_t okls_workspace_size(const okls_config* cfg, int n_groups, const okls_group_desc* groups) {
  if (check_config(cfg) != OKLS_OK || check_groups(n_groups, groups) != OKLS_OK) return 0;
  std::vector<okls_group_desc> g(groups, groups + n_groups);
  Planner P(*cfg, g);
  const WsLayout w = ws_layout(P);
  if (!P.validate()) return 0;
  return w.total;
}

okls_status okls_plan_query(const okls_config* cfg, int n_groups, const okls_group_desc* groups,
                            okls_plan_info* out) {
  if (out == nullptr) return OKLS_ERR_INVALID_ARG;
  okls_status st = check_config(cfg);
  if (st != OKLS_OK) return st;
  st = check_groups(n_groups, groups);
  if (st != OKLS_OK) return st;
  std::vector<okls_group_desc> g(groups, groups + n_groups);
  Planner P(*cfg, g);
  (void)ws_layout(P);
  if (!P.validate()) return OKLS_ERR_INVALID_ARG;
  static_assert(OKLS_PROFILE_CATEGORIES == 6, "okls_plan_info holds six categories");
  okls_plan_info info{};
  auto kernels = [](const std::vector<std::vector<LaunchRec>>& cs) {
    int n = 0;
    for (const std::vector<LaunchRec>& L : cs)
      for (const LaunchRec& r : L)
        n += (r.type == L_STAT || r.type == L_CAST || r.type == L_GEMM || r.type == L_SYM || r.type == L_ADAM ||
              r.type == L_JAC || r.type == L_NORTH || r.type == L_NSMALL || r.type == L_NELEM ||
              r.type == L_THIN);
    return n;
  };
  info.chunks = static_cast<int>(P.chunks.size());
  info.launches = kernels(P.chunks);
  info.launches_stale = P.chunks_stale.empty() ? info.launches : kernels(P.chunks_stale);
  info.ns_chains = 0;
  if (!P.muon_mode && !P.soap_mode && !P.nys_mode) {
    for (const std::vector<LaunchRec>& L : P.chunks) {
      int streams = 1;
      for (const LaunchRec& r : L) streams = std::max(streams, r.stream + 1);
      info.ns_chains = std::max(info.ns_chains, streams);
    }
  }
  for (int i = 0; i < OKLS_PROFILE_CATEGORIES; ++i) {
    info.flops[i] = P.step_flops[i];
    info.bytes[i] = P.step_bytes[i];
  }
  *out = info;
  return OKLS_OK;
}

int okls_ns_coefficients(const okls_config* cfg, double* a, double* b, int max_steps) {
  if (check_config(cfg) != OKLS_OK || a == nullptr || b == nullptr || max_steps < cfg->ns_steps) return -1;
  std::vector<double> na, nb;
  coeff_table(*cfg, na, nb);
  for (int k = 0; k < cfg->ns_steps; ++k) {
    a[k] = na[k];
    b[k] = nb[k];
  }
  return cfg->ns_steps;
}

namespace {
okls_status init_impl(okls_handle** out, const okls_config* cfg, int n_groups, const okls_group_desc* groups,
                      void* workspace, size_t ws_bytes, void* stream, bool single_chain) {
  if (out == nullptr) return OKLS_ERR_INVALID_ARG;
  *out = nullptr;
  okls_status st = check_config(cfg);
  if (st != OKLS_OK) return st;
  st = check_groups(n_groups, groups);
  if (st != OKLS_OK) return st;
  if (workspace == nullptr || !aligned(workspace, kAlign)) return OKLS_ERR_WORKSPACE;
  if (env_fault("okls_init")) return OKLS_ERR_HIP;

  std::vector<okls_group_desc> g(groups, groups + n_groups);
  Planner sizing(*cfg, g);
  sizing.single_chain = single_chain;
  const WsLayout w = ws_layout(sizing);
  if (ws_bytes < w.total) return OKLS_ERR_WORKSPACE;

  // plan again with the real chunk base
  Planner P(*cfg, g);
  P.single_chain = single_chain;
  P.plan(w.chunk);
  if (!P.validate() || P.probs.size() != sizing.probs.size() || P.chunk_bytes != sizing.chunk_bytes ||
      P.adam_jobs.size() != sizing.adam_jobs.size() || P.jac_jobs.size() != sizing.jac_jobs.size() ||
      P.nelem_jobs.size() != sizing.nelem_jobs.size() ||
      P.thin_jobs.size() != sizing.thin_jobs.size())
    return OKLS_ERR_UNSUPPORTED;
  // the regions the tables and slots occupy must end before the chunk buffers
  if (w.flag + sizeof(int) > w.chunk) return OKLS_ERR_UNSUPPORTED;

  okls_handle* h = new (std::nothrow) okls_handle();
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->groups = g;
  h->ws = static_cast<char*>(workspace);
  h->ws_bytes = ws_bytes;
  h->off_probs = w.probs;
  h->off_tiles = w.tiles;
  h->off_stat = w.stat;
  h->off_cast = w.cast;
  h->off_sym = w.sym;
  h->off_adam = w.adam;
  h->off_jac = w.jac;
  h->off_north = w.north;
  h->off_nsmall = w.nsmall;
  h->off_nelem = w.nelem;
  h->off_thin = w.thin;
  h->s_np = P.s_np;
  h->off_scal = w.scal;
  h->off_part = w.part;
  h->off_flag = w.flag;
  h->off_resid = w.resid;
  h->resid_floats = static_cast<size_t>(P.resid_floats);
  for (const Planner::ResidSlot& q : P.resid_slots) h->resid.push_back({q.mat, q.side, q.chain, q.first, q.count});
  for (const okls_group_desc& gd : g) h->n_mats += gd.batch;
  h->chunks = P.chunks;
  h->chunks_stale = P.chunks_stale;
  h->part_stride = static_cast<size_t>(P.max_partials) * 2;
  int nstreams = 1;
  for (const std::vector<LaunchRec>& L : P.chunks)
    for (const LaunchRec& r : L) nstreams = std::max(nstreams, r.stream + 1);
  if (nstreams > 1) {
    bool ok = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) == hipSuccess;
    for (int i = 1; i < nstreams && ok; ++i) {
      hipStream_t x = nullptr;
      hipEvent_t j = nullptr;
      ok = hipStreamCreateWithFlags(&x, hipStreamNonBlocking) == hipSuccess;
      if (ok) h->side.push_back(x);
      ok = ok && hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess;
      if (ok) h->ev_join.push_back(j);
    }
    if (!ok) {
      delete h;
      return OKLS_ERR_HIP;
    }
  }
  h->na = P.na;
  h->nb = P.nb;
  for (int i = 0; i < OKLS_PROFILE_CATEGORIES; ++i) {
    h->step_flops[i] = P.step_flops[i];
    h->step_bytes[i] = P.step_bytes[i];
    h->step_flops_stale[i] = P.step_flops_stale[i];
    h->step_bytes_stale[i] = P.step_bytes_stale[i];
  }

  std::vector<float> scal(static_cast<size_t>(P.n_slots), 1.0f);
  scal[SL_ONE] = 1.0f;
  scal[SL_Y] = P.sY;
  scal[SL_Z] = P.sZ;
  scal[SL_T] = P.sT;
  if (P.soap_mode) {
    scal[SL_Q] = std::ldexp(1.0f, kScaleExp);
    scal[SL_NP] = P.s_np;
    for (int e = 0; e < kZtSlots; ++e) scal[SL_ZT + e] = std::ldexp(P.s_np, -e);
  }

  hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  auto up = [&](size_t off, const void* src, size_t bytes) {
    if (e == hipSuccess && bytes > 0) e = hipMemcpyAsync(h->ws + off, src, bytes, hipMemcpyHostToDevice, s);
  };
  up(w.probs, P.probs.data(), P.probs.size() * sizeof(GemmProb));
  up(w.tiles, P.tiles.data(), P.tiles.size() * sizeof(TileRef));
  up(w.stat, P.stat_jobs.data(), P.stat_jobs.size() * sizeof(StatJob));
  up(w.cast, P.cast_jobs.data(), P.cast_jobs.size() * sizeof(CastJob));
  up(w.sym, P.sym_jobs.data(), P.sym_jobs.size() * sizeof(SymJob));
  up(w.adam, P.adam_jobs.data(), P.adam_jobs.size() * sizeof(AdamJob));
  up(w.jac, P.jac_jobs.data(), P.jac_jobs.size() * sizeof(JacJob));
  up(w.north, P.north_jobs.data(), P.north_jobs.size() * sizeof(NysOrthJob));
  up(w.nsmall, P.nsmall_jobs.data(), P.nsmall_jobs.size() * sizeof(NysSmallJob));
  up(w.nelem, P.nelem_jobs.data(), P.nelem_jobs.size() * sizeof(NysElemJob));
  up(w.thin, P.thin_jobs.data(), P.thin_jobs.size() * sizeof(ThinJob));
  up(w.scal, scal.data(), scal.size() * sizeof(float));
  // residual partials start as NaN: no root computed yet
  const std::vector<float> nan_fill(h->resid_floats, std::numeric_limits<float>::quiet_NaN());
  up(w.resid, nan_fill.data(), nan_fill.size() * sizeof(float));
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete h;
    return OKLS_ERR_HIP;
  }
  *out = h;
  return OKLS_OK;
}
}  // namespace

okls_status okls_init(okls_handle** out, const okls_config* cfg, int n_groups, const okls_group_desc* groups,
                      void* workspace, size_t ws_bytes, void* stream) {
  return init_impl(out, cfg, n_groups, groups, workspace, ws_bytes, stream, false);
}

// The workspace is the library's static device scratch; the plan runs one
// Newton-Schulz chain, so no side stream or event is created, and nothing
// is allocated on the device.
okls_status okls_init_static(okls_handle** out, const okls_config* cfg, int n_groups,
                             const okls_group_desc* groups, void* stream) {
  if (out == nullptr) return OKLS_ERR_INVALID_ARG;
  *out = nullptr;
  okls_status st = check_config(cfg);
  if (st != OKLS_OK) return st;
  st = check_groups(n_groups, groups);
  if (st != OKLS_OK) return st;
  if (okls_workspace_size(cfg, n_groups, groups) > kStaticScratchBytes) return OKLS_ERR_WORKSPACE;
  void* ptr = nullptr;
  if (static_scratch(&ptr) != hipSuccess) return OKLS_ERR_HIP;
  return init_impl(out, cfg, n_groups, groups, ptr, kStaticScratchBytes, stream, true);
}

static okls_status check_tensors(const okls_handle* h, const okls_group_tensors* t, bool need_wg) {
  if (t == nullptr) return OKLS_ERR_INVALID_ARG;
  for (size_t g = 0; g < h->groups.size(); ++g) {
    const okls_group_tensors& x = t[g];
    if (x.M == nullptr || !aligned(x.M, 4)) return OKLS_ERR_INVALID_ARG;
    // the Muon mode has no factors or roots: Sa, Sb, Pa and Pb are not read and may be null
    if (h->cfg.mode != OKLS_MODE_MUON) {
      if (x.Sa == nullptr || x.Sb == nullptr || x.Pa == nullptr || x.Pb == nullptr) return OKLS_ERR_INVALID_ARG;
      if (!aligned(x.Sa, 4) || !aligned(x.Sb, 4) || !aligned(x.Pa, 4) || !aligned(x.Pb, 4)) return OKLS_ERR_INVALID_ARG;
    }
    if (h->cfg.mode == OKLS_MODE_SOAP && (x.V == nullptr || !aligned(x.V, 4))) return OKLS_ERR_INVALID_ARG;
    if (h->cfg.mode == OKLS_MODE_NYSTROM && need_wg &&
        (x.PsiA == nullptr || x.PsiB == nullptr || !aligned(x.PsiA, 4) || !aligned(x.PsiB, 4)))
      return OKLS_ERR_INVALID_ARG;
    if (need_wg) {
      if (x.W == nullptr || x.G == nullptr) return OKLS_ERR_INVALID_ARG;
      if (!aligned(x.W, 4) || !aligned(x.G, h->groups[g].g_dtype == OKLS_F32 ? 4 : 2)) return OKLS_ERR_INVALID_ARG;
    }
  }
  return OKLS_OK;
}

okls_status okls_init_state(okls_handle* h, const okls_group_tensors* t, void* stream) {
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  okls_status st = check_tensors(h, t, false);
  if (st != OKLS_OK) return st;
  if (env_fault("okls_init_state")) return OKLS_ERR_HIP;
  InitArgs a;
  std::memset(&a, 0, sizeof(a));
  a.user = user_ptrs(h, t);
  int n = 0;
  for (size_t g = 0; g < h->groups.size(); ++g) {
    const okls_group_desc& d = h->groups[g];
    if (h->cfg.mode == OKLS_MODE_NYSTROM) {   // no factors yet: U = 0, Lambda = 0 (a first refresh is a cold start)
      const int ra = std::min(h->cfg.nys_rank, std::min(h->cfg.nys_rank + h->cfg.nys_oversample, d.m));
      const int rb = std::min(h->cfg.nys_rank, std::min(h->cfg.nys_rank + h->cfg.nys_oversample, d.n));
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SA, d.batch, 1, ra, 0.0f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SB, d.batch, 1, rb, 0.0f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PA, d.batch, d.m, ra, 0.0f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PB, d.batch, d.n, rb, 0.0f};
    } else if (h->cfg.mode != OKLS_MODE_MUON) {
      // SOAP: zero factors (the Clean paper's Algorithm 4 starts from none), identity bases
      const float s0 = h->cfg.mode == OKLS_MODE_SOAP ? 0.0f : h->cfg.eps;
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SA, d.batch, d.m, d.m, s0};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SB, d.batch, d.n, d.n, s0};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PA, d.batch, d.m, d.m, 1.0f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PB, d.batch, d.n, d.n, 1.0f};
    }
    a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_M, d.batch, d.m, d.n, 0.0f};
    if (h->cfg.mode == OKLS_MODE_SOAP) a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_V, d.batch, d.m, d.n, 0.0f};
  }
  hipStream_t s = as_stream(stream);
  if (launch_init_state(a, n, s) != hipSuccess) return OKLS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return OKLS_ERR_HIP;
  return OKLS_OK;
}

okls_status okls_step(okls_handle* h, const okls_group_tensors* t, int64_t step, float lr, void* stream) {
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  if (step < 1 || !(lr >= 0.f && std::isfinite(lr))) return OKLS_ERR_INVALID_ARG;
  okls_status st = check_tensors(h, t, true);
  if (st != OKLS_OK) return st;
  if (env_fault("okls_step")) return OKLS_ERR_HIP;

  // host scalars of this step
  const double b1 = h->cfg.beta1;
  double s_t = 1.0;
  if (h->cfg.nesterov_var_corr) {
    // variance of beta1 M_t + (1-beta1) G_t for independent unit-variance G and M_0 = 0
    const double w0 = (1.0 - b1) * (1.0 + b1);
    double v = w0 * w0;
    const double q = b1 * b1;
    const double tail = (1.0 - b1) * (1.0 - b1) * q * q;     // weight^2 of G_{t-1}
    if (step > 1) {
      // sum_{j=0}^{t-2} q^j = (1 - q^(t-1)) / (1 - q)
      v += tail * (1.0 - std::pow(q, static_cast<double>(step - 1))) / (1.0 - q);
    }
    s_t = 1.0 / std::sqrt(v);
  }
  const bool soap = h->cfg.mode == OKLS_MODE_SOAP;
  // SOAP: AdamW's decoupled decay 1 - lr wd (the Clean paper's Table 4); the
  // other modes: AdamC's 1 - lr wd lr / lr_peak
  const double decay = soap ? 1.0 - static_cast<double>(lr) * h->cfg.weight_decay
                            : 1.0 - static_cast<double>(lr) * h->cfg.weight_decay * (static_cast<double>(lr) / h->cfg.lr_peak);
  if (soap) s_t = 1.0;
  // the momentum read: the Nesterov look-ahead, or (SOAP) the first moment itself
  const float nest_a = soap ? 1.0f : static_cast<float>(b1), nest_b = soap ? 0.0f : 1.0f - static_cast<float>(b1);
  const double bc1 = (soap && h->cfg.bias_correction) ? 1.0 / (1.0 - std::pow(b1, static_cast<double>(step))) : 1.0;
  const double bc2 = (soap && h->cfg.bias_correction)
                         ? 1.0 / (1.0 - std::pow(static_cast<double>(h->cfg.beta2), static_cast<double>(step))) : 1.0;
  // the update epilogue computes decay W - lr_update c U: decay after the
  // update, decay (W - lr c U), is the same form with lr_update = decay lr
  const float lr_update = (h->cfg.decay_after && !soap) ? static_cast<float>(decay * lr) : lr;

  const UserPtrs user = user_ptrs(h, t);
  hipStream_t s = as_stream(stream);
  char* ws = h->ws;
  float* scal = reinterpret_cast<float*>(ws + h->off_scal);
  float* part = reinterpret_cast<float*>(ws + h->off_part);

  // the roots are recomputed on steps 1, 1 + p, 1 + 2p, ... (p = root_period)
  const bool nys = h->cfg.mode == OKLS_MODE_NYSTROM;
  (void)nys;
  // SOAP: the bases are recomputed after steps t with t % precond_freq == 0
  const bool refresh = soap ? (h->cfg.precond_freq <= 1 || step % h->cfg.precond_freq == 0)
                            : (h->cfg.mode == OKLS_MODE_MUON || h->cfg.root_period <= 1 || (step - 1) % h->cfg.root_period == 0);
  if (h->prof) {
    h->acc.steps += 1;
    for (int i = 0; i < OKLS_PROFILE_CATEGORIES; ++i) {
      h->acc.flops[i] += refresh ? h->step_flops[i] : h->step_flops_stale[i];
      h->acc.bytes[i] += refresh ? h->step_bytes[i] : h->step_bytes_stale[i];
    }
  }
  for (const std::vector<LaunchRec>& L : refresh ? h->chunks : h->chunks_stale) {
    for (const LaunchRec& r : L) {
      hipError_t e = hipSuccess;
      if (r.type == L_FORK) {          // the side streams start after everything queued so far
        if (hipEventRecord(h->ev_fork, s) != hipSuccess) return OKLS_ERR_HIP;
        for (hipStream_t x : h->side)
          if (hipStreamWaitEvent(x, h->ev_fork, 0) != hipSuccess) return OKLS_ERR_HIP;
        continue;
      }
      if (r.type == L_JOIN) {          // the caller's stream continues after the side streams' work
        for (size_t i = 0; i < h->side.size(); ++i)
          if (hipEventRecord(h->ev_join[i], h->side[i]) != hipSuccess || hipStreamWaitEvent(s, h->ev_join[i], 0) != hipSuccess)
            return OKLS_ERR_HIP;
        continue;
      }
      const hipStream_t rs = r.stream == 0 ? s : h->side[r.stream - 1];
      float* rpart = part + static_cast<size_t>(r.stream) * h->part_stride;
      size_t ev = 0;
      if (h->prof) {
        ev = h->next_event;
        while (h->events.size() < ev + 2) {
          hipEvent_t x;
          if (hipEventCreate(&x) != hipSuccess) return OKLS_ERR_HIP;
          h->events.push_back(x);
        }
        h->next_event += 2;
        if (hipEventRecord(h->events[ev], rs) != hipSuccess) return OKLS_ERR_HIP;
      }
      if (r.type == L_STAT) {
        StatArgs a;
        a.jobs = reinterpret_cast<const StatJob*>(ws + h->off_stat) + r.first;
        a.n_jobs = r.count;
        a.blk_offset = 0;
        a.partials = rpart;
        a.beta1 = static_cast<float>(b1);
        a.s_t = static_cast<float>(s_t);
        a.nest_a = nest_a;
        a.nest_b = nest_b;
        a.ws = ws;
        a.user = user;
        e = launch_stats(a, r.nblocks, rs);
      } else if (r.type == L_CAST) {
        CastArgs a;
        a.jobs = reinterpret_cast<const CastJob*>(ws + h->off_cast) + r.first;
        a.n_jobs = r.count;
        a.blk_offset = 0;
        a.partials = rpart;
        a.scal = scal;
        a.beta1 = static_cast<float>(b1);
        a.s_t = static_cast<float>(s_t);
        a.ka = r.ka;
        a.kb = r.kb;
        a.nest_a = nest_a;
        a.nest_b = nest_b;
        a.ws = ws;
        a.user = user;
        e = launch_cast(a, r.nblocks, rs);
      } else if (r.type == L_SYM) {
        SymArgs a;
        a.jobs = reinterpret_cast<const SymJob*>(ws + h->off_sym) + r.first;
        a.n_jobs = r.count;
        a.scal = scal;
        a.ws = ws;
        a.user = user;
        e = launch_sym(a, r.nblocks, rs);
      } else if (r.type == L_ADAM) {
        AdamArgs a;
        a.jobs = reinterpret_cast<const AdamJob*>(ws + h->off_adam) + r.first;
        a.n_jobs = r.count;
        a.beta1 = static_cast<float>(b1);
        a.beta2 = h->cfg.beta2;
        a.eps = h->cfg.eps;
        a.bc1 = static_cast<float>(bc1);
        a.bc2 = static_cast<float>(bc2);
        a.s_out = h->s_np;
        a.write_lo = h->cfg.factor_split;
        a.ws = ws;
        a.user = user;
        e = launch_adam(a, r.nblocks, rs);
      } else if (r.type == L_JAC) {
        JacArgs a;
        a.jobs = reinterpret_cast<const JacJob*>(ws + h->off_jac) + r.first;
        a.n_jobs = r.count;
        a.round = r.round;
        a.partials = reinterpret_cast<float*>(ws + r.jac_part);
        a.flags = reinterpret_cast<int32_t*>(ws + r.jac_flag);
        a.ws = ws;
        a.user = user;
        e = launch_jacobi(a, r.jac_kind, r.nblocks, rs);
      } else if (r.type == L_THIN) {
        ThinArgs a;
        a.jobs = reinterpret_cast<const ThinJob*>(ws + h->off_thin) + r.first;
        a.n_jobs = r.count;
        a.scal = scal;
        a.beta1 = static_cast<float>(b1);
        a.s_t = static_cast<float>(s_t);
        a.lr = lr_update;
        a.decay = static_cast<float>(decay);
        a.ws = ws;
        a.user = user;
        e = launch_thin(a, r.thin_ta, r.thin_mom, r.thin_cbm, r.thin_wupd, r.nblocks, rs);
      } else if (r.type == L_NORTH) {
        NysOrthArgs a;
        a.jobs = reinterpret_cast<const NysOrthJob*>(ws + h->off_north) + r.first;
        a.n_jobs = r.count;
        a.ws = ws;
        a.user = user;
        e = launch_nys_orth(a, rs);
      } else if (r.type == L_NSMALL) {
        NysSmallArgs a;
        a.jobs = reinterpret_cast<const NysSmallJob*>(ws + h->off_nsmall) + r.first;
        a.n_jobs = r.count;
        a.phase = r.round;
        a.scal = scal;
        a.ws = ws;
        a.user = user;
        e = launch_nys_small(a, rs);
      } else if (r.type == L_NELEM) {
        NysElemArgs a;
        a.jobs = reinterpret_cast<const NysElemJob*>(ws + h->off_nelem) + r.first;
        a.n_jobs = r.count;
        a.mu = h->cfg.eps;
        a.ws = ws;
        a.user = user;
        e = launch_nys_elem(a, r.nblocks, rs);
      } else {
        GemmArgs a;
        a.probs = reinterpret_cast<const GemmProb*>(ws + h->off_probs);
        a.tiles = reinterpret_cast<const TileRef*>(ws + h->off_tiles);
        a.tile_begin = r.first;
        a.prob_base = r.prob_base;
        a.split_in = r.split_in;
        a.write_lo = r.write_lo;
        a.ka = r.ka;
        a.kb = r.kb;
        a.lr = lr_update;
        a.decay = static_cast<float>(decay);
        a.ws = ws;
        a.scal = scal;
        a.resid = reinterpret_cast<float*>(ws + h->off_resid);
        a.user = user;
        e = launch_gemm(a, r.count, r.tile, r.epi, rs);
      }
      if (e != hipSuccess) return OKLS_ERR_HIP;
      if (h->prof) {
        if (hipEventRecord(h->events[ev + 1], rs) != hipSuccess) return OKLS_ERR_HIP;
        h->pending.push_back({r.cat, static_cast<int>(ev)});
      }
    }
  }
  return OKLS_OK;
}

okls_status okls_ns_residuals(okls_handle* h, double* out, int64_t count, void* stream) {
  if (h == nullptr || out == nullptr) return OKLS_ERR_INVALID_ARG;
  if (h->cfg.mode != OKLS_MODE_OKLS && h->cfg.mode != OKLS_MODE_SHAMPOO) return OKLS_ERR_UNSUPPORTED;
  if (count < 4 * static_cast<int64_t>(h->n_mats)) return OKLS_ERR_INVALID_ARG;
  std::vector<float> part(h->resid_floats);
  hipStream_t s = as_stream(stream);
  if (!part.empty() && hipMemcpyAsync(part.data(), h->ws + h->off_resid, part.size() * sizeof(float),
                                      hipMemcpyDeviceToHost, s) != hipSuccess)
    return OKLS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return OKLS_ERR_HIP;
  for (int64_t i = 0; i < 4 * static_cast<int64_t>(h->n_mats); ++i) out[i] = std::numeric_limits<double>::quiet_NaN();
  for (const okls_handle::Resid& q : h->resid) {
    double sum = 0.0;   // in the partials' order: a fixed order, so repeatable
    for (int k = 0; k < q.count; ++k) sum += static_cast<double>(part[static_cast<size_t>(q.first) + k]);
    out[(static_cast<int64_t>(q.mat) * 2 + q.side) * 2 + q.chain] = std::sqrt(sum);
  }
  return OKLS_OK;
}

okls_status okls_check_finite(okls_handle* h, const okls_group_tensors* t, void* stream) {
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  okls_status st = check_tensors(h, t, true);
  if (st != OKLS_OK) return st;
  InitArgs a;
  std::memset(&a, 0, sizeof(a));
  a.user = user_ptrs(h, t);
  int n = 0;
  for (size_t g = 0; g < h->groups.size(); ++g) {
    const okls_group_desc& d = h->groups[g];
    if (h->cfg.mode == OKLS_MODE_NYSTROM) {
      const int ra = std::min(h->cfg.nys_rank, std::min(h->cfg.nys_rank + h->cfg.nys_oversample, d.m));
      const int rb = std::min(h->cfg.nys_rank, std::min(h->cfg.nys_rank + h->cfg.nys_oversample, d.n));
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SA, d.batch, 1, ra, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SB, d.batch, 1, rb, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PA, d.batch, d.m, ra, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PB, d.batch, d.n, rb, 0.f};
    } else if (h->cfg.mode != OKLS_MODE_MUON) {
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SA, d.batch, d.m, d.m, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_SB, d.batch, d.n, d.n, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PA, d.batch, d.m, d.m, 0.f};
      a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_PB, d.batch, d.n, d.n, 0.f};
    }
    a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_M, d.batch, d.m, d.n, 0.f};
    if (h->cfg.mode == OKLS_MODE_SOAP) a.jobs[n++] = InitJob{static_cast<int32_t>(g), REF_V, d.batch, d.m, d.n, 0.f};
  }
  hipStream_t s = as_stream(stream);
  int* flag = reinterpret_cast<int*>(h->ws + h->off_flag);
  if (launch_check_finite(a, n, flag, s) != hipSuccess) return OKLS_ERR_HIP;
  // W too
  InitArgs w = a;
  int nw = 0;
  for (size_t g = 0; g < h->groups.size(); ++g) {
    const okls_group_desc& d = h->groups[g];
    w.jobs[nw++] = InitJob{static_cast<int32_t>(g), REF_W, d.batch, d.m, d.n, 0.f};
  }
  int host_flag = 0;
  if (hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return OKLS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return OKLS_ERR_HIP;
  if (host_flag) return OKLS_ERR_NONFINITE;
  if (launch_check_finite(w, nw, flag, s) != hipSuccess) return OKLS_ERR_HIP;
  if (hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return OKLS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return OKLS_ERR_HIP;
  return host_flag ? OKLS_ERR_NONFINITE : OKLS_OK;
}

okls_status okls_profile_enable(okls_handle* h, int enable) {
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  h->prof = enable != 0;
  return OKLS_OK;
}

okls_status okls_profile_read(okls_handle* h, okls_profile_stats* out) {
  if (h == nullptr || out == nullptr) return OKLS_ERR_INVALID_ARG;
  // summed into a copy: on an event error the handle's sums and pending
  // launches stay as they were
  okls_profile_stats acc = h->acc;
  if (!h->pending.empty()) {
    if (hipEventSynchronize(h->events[h->pending.back().second + 1]) != hipSuccess) return OKLS_ERR_HIP;
    // intervals relative to the first event; union per category
    const hipEvent_t ref = h->events[h->pending.front().second];
    std::vector<std::vector<std::pair<float, float>>> iv(OKLS_PROFILE_CATEGORIES);
    for (const std::pair<int, int>& p : h->pending) {
      float t0 = 0.f, t1 = 0.f;
      if (hipEventElapsedTime(&t0, ref, h->events[p.second]) != hipSuccess ||
          hipEventElapsedTime(&t1, ref, h->events[p.second + 1]) != hipSuccess)
        return OKLS_ERR_HIP;
      acc.ms[p.first] += t1 - t0;
      acc.launches[p.first] += 1;
      iv[p.first].push_back({t0, t1});
    }
    for (int c = 0; c < OKLS_PROFILE_CATEGORIES; ++c) {
      std::sort(iv[c].begin(), iv[c].end());
      double busy = 0.0, lo = 0.0, hi = -1.0;
      for (const std::pair<float, float>& x : iv[c]) {
        if (x.first > hi) {
          if (hi > lo) busy += hi - lo;
          lo = x.first;
          hi = x.second;
        } else if (x.second > hi) {
          hi = x.second;
        }
      }
      if (hi > lo) busy += hi - lo;
      acc.busy_ms[c] += busy;
    }
  }
  *out = acc;
  h->acc = okls_profile_stats{};
  h->pending.clear();
  h->next_event = 0;
  return OKLS_OK;
}

okls_status okls_destroy(okls_handle* h) {
  if (h == nullptr) return OKLS_ERR_INVALID_ARG;
  delete h;
  return OKLS_OK;
}

const char* okls_status_string(okls_status s) {
  switch (s) {
    case OKLS_OK: return "ok";
    case OKLS_ERR_INVALID_ARG: return "invalid argument";
    case OKLS_ERR_SHAPE: return "invalid shape";
    case OKLS_ERR_DTYPE: return "unsupported dtype";
    case OKLS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case OKLS_ERR_HIP: return "HIP runtime error";
    case OKLS_ERR_NONFINITE: return "non-finite values in the optimizer state";
    case OKLS_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

}  // extern "C"

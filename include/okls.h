/*
 * okls.h - C ABI of the MI355X (gfx950) batched Online KL Shampoo / Shampoo
 * preconditioner step.
 *
 * What one okls_step computes, for every matrix parameter G in R^{m x n}
 * of every group ("Online KL Shampoo" project README, section "How it works",
 * and its intro list):
 *   1. two-sided factor updates with the previous preconditioners
 *        S_a <- beta2 S_a + (1-beta2)/n (G P_b)(G P_b)^T + eps I
 *        S_b <- beta2 S_b + (1-beta2)/m (P_a G)^T (P_a G) + eps I
 *      or, in Shampoo mode, the sums S_a += G G^T, S_b += G^T G (+ eps I)
 *      ("Clean: Second-order LLM Training at Linear Memory Cost via Nystrom
 *      Sketching", section 2, eq. (2); the optim-book Shampoo chapter's
 *      worked example);
 *   2. fresh inverse roots P = S^{-1/2} (Shampoo: S^{-1/4}, the Clean paper's
 *      eq. (3)) from a coupled Newton-Schulz iteration made of GEMMs only
 *      (10 steps, 27 GEMMs per root, fp16 GEMM inputs with fp32 accumulation);
 *   3. Nesterov momentum with variance correction, M <- beta1 M + (1-beta1) G,
 *      N = s_t (beta1 M + (1-beta1) G), whitened U = P_a N P_b;
 *   4. W <- (1 - lr wd lr/lr_peak) W - lr c_shape U,
 *      c_shape = sqrt(m/n) / (sqrt(m) + sqrt(n))  (README "How it works";
 *      AdamC decay per "Learning-rate schedule" and "Hyperparameters").
 * With okls_config.root_period = p > 1 the roots of step 2 are recomputed
 * only on steps 1, 1 + p, ... and kept in between.  OKLS_MODE_MUON replaces
 * steps 1-3's whitening by the polar iteration of N (see okls_mode).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     row-major and contiguous, aligned to their element size (16-byte
 *     alignment lets the kernels use their 16-byte access paths).  A group of N
 *     same-shaped matrices is one (N, rows, cols) tensor ("Batched matrices"
 *     section: a 3-D parameter is N independent matrices that share the
 *     hyperparameters).
 *   - The caller owns every tensor and the workspace.  The library never
 *     allocates device memory; the handle owns host memory plus, when the
 *     plan runs two concurrent Newton-Schulz chains, one HIP stream and two
 *     events (created by okls_init, destroyed by okls_destroy).
 *   - All device work is ordered on the given stream (a hipStream_t passed
 *     as void*; NULL is the default stream).  The plan runs a second,
 *     concurrent Newton-Schulz chain where it fills otherwise idle compute
 *     units (launches of few, partly filled rounds of tiles).  That chain
 *     runs on the handle's stream, which waits for everything queued on the
 *     given stream before it and which the given stream waits for before the
 *     step's remaining work, so the step is ordered on the given stream as a
 *     whole.  okls_init and
 *     okls_init_state synchronise that stream once (init uploads descriptor
 *     tables); okls_step never synchronises.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Errors are returned as okls_status; no exception crosses the ABI.
 *     Argument errors are detected on the host before any launch.
 *   - A handle may be used by one host thread at a time.  Two steps that
 *     share a workspace must be ordered on one stream.
 */
#ifndef OKLS_H_
#define OKLS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OKLS_OK = 0,
    OKLS_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, bad hyperparameter */
    OKLS_ERR_SHAPE = -2,         /* non-positive or too large dimensions, too many groups */
    OKLS_ERR_DTYPE = -3,         /* unsupported gradient dtype */
    OKLS_ERR_WORKSPACE = -4,     /* workspace null, misaligned or smaller than okls_workspace_size */
    OKLS_ERR_HIP = -5,           /* a HIP runtime call or launch failed */
    OKLS_ERR_NONFINITE = -6,     /* okls_check_finite found Inf/NaN in the state */
    OKLS_ERR_UNSUPPORTED = -7    /* a combination the library does not implement */
} okls_status;

typedef enum { OKLS_F32 = 0, OKLS_BF16 = 1, OKLS_F16 = 2 } okls_dtype;

typedef enum {
    OKLS_MODE_OKLS = 0,      /* KL factor EMAs, P = S^{-1/2} */
    OKLS_MODE_SHAMPOO = 1,   /* plain sums, P = S^{-1/4} via two chained roots */
    OKLS_MODE_MUON = 2,      /* no factors: the momentum N is orthogonalised by the polar
                                Newton-Schulz iteration X <- a_k X + b_k (X X^T) X from
                                X_0 = N / ||N N^T||_F^{1/2} (the Shampoo chapter's
                                "ML에서: 대회 우승과 그다음": the un-accumulated Shampoo
                                step, every singular value set to 1, by products alone;
                                the Clean paper's Table 6: 5 iterations).  ns_steps and
                                ns_floor are the iteration's (Muon setting: 5 and 1e-2);
                                beta2, eps, ns_damping and root_period are not used */
    OKLS_MODE_SOAP = 3,      /* Adam in the factors' eigenbasis ("Clean: Second-order LLM
                                Training at Linear Memory Cost via Nystrom Sketching",
                                Appendix C, Algorithm 4 (SOAP); "KPOP Optimiser Explained",
                                "Transforming the Gradient"): per matrix
                                  G' = Q_a^T G Q_b, M <- beta1 M + (1-beta1) G, M' = Q_a^T M Q_b,
                                  V <- beta2 V + (1-beta2) G'^2,
                                  N' = (M'/(1-beta1^t)) / (sqrt(V/(1-beta2^t)) + eps),
                                  W <- (1 - lr wd) W - lr Q_a N' Q_b^T,
                                  S_a <- sb S_a + (1-sb) G G^T, S_b <- sb S_b + (1-sb) G^T G
                                  (sb = soap_beta), and after steps t with t % precond_freq
                                  == 0 the bases Q_a, Q_b become eigenbases of S_a, S_b,
                                  computed by block Jacobi sweeps warm-started from the
                                  current bases.  The tensors' Sa, Sb hold the factors, Pa,
                                  Pb the bases (columns = eigenvectors), V the second moment;
                                  ns_*, nesterov_var_corr, root_period, eps_convex,
                                  decay_after and shape_scale are not used; the GEMMs are
                                  split-fp16 (fp32-accurate) when factor_split is 1 */
    OKLS_MODE_NYSTROM = 4    /* low-rank Nystrom factors ("Clean: Second-order LLM Training at
                                Linear Memory Cost via Nystrom Sketching", section 2.2 eq. (4)-(5),
                                section 3 eq. (6)-(10), Appendix A Algorithms 2-3): per side
                                (S_a = L of G G^T, S_b = R of G^T G) only U (d x r', orthonormal
                                columns) and Lambda (r') are stored, r' = min(nys_rank, d).  On
                                steps t = 1, 1 + T, ... (T = root_period) both are refreshed by
                                the warm-started randomized Nystrom approximation of
                                beta2 U Lambda U^T + (1 - beta2) G G^T (the sketch formed through
                                the stored factors, eq. (8)), with nys_oversample extra columns
                                and nys_passes subspace-iteration passes; every step then
                                preconditions the Nesterov momentum N of the OKLS mode,
                                U = P_a^-1/2 N P_b^-1/2 with P^-1/2 = c U D U^T + (I - U U^T),
                                D = (Lambda + eps)^-1/2, c = (lambda_r' + eps)^1/2 (eq. (9)), and
                                updates W as the OKLS mode does.  Tensors: Pa / Pb hold U
                                ((N, m, r'a) / (N, n, r'b)), Sa / Sb hold Lambda ((N, r'a) /
                                (N, r'b)), PsiA / PsiB the refresh's Gaussian matrices.  All
                                arithmetic is fp32 (the products are thin); r + p <= 128. */
} okls_mode;

typedef struct {
    int32_t mode;              /* okls_mode */
    int32_t ns_steps;          /* Newton-Schulz steps, 2..16 (pages: 10) */
    int32_t ns_split_steps;    /* first k NS steps use split-fp16 (hi*hi + hi*lo + lo*hi)
                                  GEMMs; 0 = every NS GEMM plain fp16 (the pages' FP16
                                  path), ns_steps = every NS GEMM fp32-accurate */
    int32_t factor_split;      /* 1: factor, cross-preconditioning and whitening GEMMs
                                  also use split-fp16 (the fp32-accurate path) */
    int32_t nesterov_var_corr; /* 1: N scaled by s_t = 1/sqrt(var) (reading of "variance
                                  correction"); 0: s_t = 1 */
    int32_t chunk_matrices;    /* 0: all matrices in one pass; k > 0: at most k matrices
                                  per pass (bounds the workspace) */
    float beta1;               /* Nesterov momentum EMA coefficient (default 0.9684) */
    float beta2;               /* factor EMA coefficient (default 0.9482); ignored in Shampoo mode */
    float eps;                 /* added at factor init and after every update (default 1e-9) */
    float weight_decay;        /* AdamC decoupled decay coefficient (default 0.0303) */
    float lr_peak;             /* initial learning rate kept for the AdamC correction */
    float ns_floor;            /* lower end l_0 of the interval the NS coefficients are
                                  optimised on, for sqrt(lambda / ||S||_F); default 3e-2, matched
                                  to fp16 GEMM inputs: the table's gain on directions below
                                  the interval is about 1/l_0-fold larger than 1, and fp16
                                  rounding noise in them must stay bounded (1e-3 suits the
                                  fp32-accurate split path) */
    float ns_damping;          /* nu: the root is taken of S + (nu / sqrt(d)) ||S||_F I; default
                                  0 (the root of S itself, P = S^{-1/2}) */
    int32_t root_period;       /* p >= 1: the roots are recomputed on steps t = 1, 1 + p,
                                  1 + 2p, ... and kept in between (the factors, momentum,
                                  whitening and update run every step).  1 (default) is the
                                  README's every-step refresh; the Shampoo chapter and the
                                  Clean paper describe refreshing only every few steps. */
    /* Readings of the pages kept as switches (the defaults are the readings the
       library takes; see the README's "Hyperparameters" and "How it works"): */
    int32_t eps_convex;        /* 0 (default): + eps I after every factor update;
                                  1: the OKLS update stays a convex combination,
                                  beta2 S + (1 - beta2)(X X^T / n + eps I), so eps I is its
                                  fixed point.  Shampoo mode: no effect (+ eps I either way) */
    int32_t decay_after;       /* 0 (default): W <- decay W - lr c U (the decay multiplies the
                                  previous weights); 1: W <- decay (W - lr c U) */
    int32_t shape_scale;       /* 1 (default): c = c_shape(m, n), the README's muP multiplier;
                                  0: c = 1, the original Shampoo update W - lr P_a N P_b
                                  (with beta1 = 0, nesterov_var_corr = 0 and weight_decay = 0
                                  it is W - lr S_a^{-1/4} G S_b^{-1/4}, the Shampoo chapter's
                                  step) */
    int32_t ns_classical;      /* 0 (default): the per-step minimax table on [ns_floor, 1];
                                  1: the classical Newton-Schulz step a = 3/2, b = -1/2 at every
                                  step (ns_floor unused); 10 such steps converge only for
                                  condition numbers up to about 1e2 */
    int32_t whiten_split;      /* 1 (default): the whitening products P_b N^T and P_a V run
                                  split-fp16 (fp32-accurate) also when factor_split is 0:
                                  their fp16 rounding error grows with the preconditioners'
                                  eigenvalue spread, which rank-deficient factors make large;
                                  0: plain fp16 inputs (the fp16 path's other products) */
    /* OKLS_MODE_SOAP only (the Clean paper's Tables 4 and 6 give the values in
       brackets; beta1, beta2, eps and weight_decay are Adam's there): */
    float soap_beta;           /* EMA coefficient of the factors [0.95] */
    int32_t precond_freq;      /* f >= 1: bases recomputed after steps t with t % f == 0 [10] */
    int32_t soap_moments;      /* 0 (default): M in the parameter space, rotated every step
                                  (Algorithm 4); 1: M kept in the eigenbasis, M <- beta1 M +
                                  (1-beta1) G' (KPOP's Adam) */
    int32_t bias_correction;   /* 1 (default): Adam's 1/(1-beta^t) corrections; 0: none */
    int32_t jacobi_sweeps;     /* most sweeps of a basis refresh, 1..64 (default 20; a refresh
                                  stops once converged: measured cold starts from the identity
                                  need 12 sweeps at d = 1024 and 13 at d = 2816) */
    float jacobi_tol;          /* a refresh stops once ||off(Q^T S Q)||_F <= tol ||diag||_F
                                  (default 2e-6), tol raised per factor of side d to
                                  2^-23 sqrt(d), where the fp32 basis' own rounding sets
                                  its accuracy */
    /* OKLS_MODE_NYSTROM only: */
    int32_t nys_rank;          /* r >= 1: eigenpairs kept per factor (default 32) */
    int32_t nys_oversample;    /* p >= 0: extra sketch columns, r + p <= 128 (default 8) */
    int32_t nys_passes;        /* q, 0..8: subspace-iteration passes of a refresh (default 1) */
    /* OKLS_MODE_SOAP only: */
    int32_t jacobi_apply_tiles; /* tiles per workgroup of the eigensolver's rotation apply:
                                   0 (default) chooses by the size of a round (4 on rounds with
                                   at least 65536 tiles, else 1); 1 or 4 forces it.  The results
                                   are bitwise the same either way. */
} okls_config;

typedef struct {
    int32_t batch;     /* N >= 1 matrices of this shape */
    int32_t m, n;      /* rows (fan-out) and columns of each matrix, 1..32768 */
    int32_t g_dtype;   /* okls_dtype of the gradient (fp32, bf16 or fp16); W, M, S, P are fp32 */
} okls_group_desc;

typedef struct {
    float* W;          /* (N, m, n) weights, updated in place */
    const void* G;     /* (N, m, n) gradient, read only, fp32, bf16 or fp16 */
    float* M;          /* (N, m, n) momentum, updated in place */
    float* Sa;         /* (N, m, m) left factor, symmetric, updated in place */
    float* Sb;         /* (N, n, n) right factor */
    float* Pa;         /* (N, m, m) left preconditioner S_a^{-1/2} (Shampoo S_a^{-1/4}) */
    float* Pb;         /* (N, n, n) right preconditioner */
                       /* OKLS_MODE_MUON reads none of Sa, Sb, Pa, Pb: they may be NULL */
    float* V;          /* (N, m, n) second moment, OKLS_MODE_SOAP only (else NULL) */
    const float* PsiA; /* OKLS_MODE_NYSTROM: (N, m, k_a) standard Gaussian matrix of the refresh,
                          k_a = min(nys_rank + nys_oversample, m), read on refresh steps (the
                          caller draws it: the method's random numbers are inputs); else NULL */
    const float* PsiB; /* (N, n, k_b), likewise */
} okls_group_tensors;

typedef struct okls_handle okls_handle;

/* Fills cfg with the pages' defaults ("Hyperparameters" table of the README;
 * 10 NS steps) and the fp16 path. */
void okls_default_config(okls_config* cfg);

/* Bytes of device workspace that okls_init needs for these groups.  Pure
 * host function.  Returns 0 if the arguments are invalid. */
size_t okls_workspace_size(const okls_config* cfg, int n_groups, const okls_group_desc* groups);

/* What a step of these groups runs, from the same plan okls_init builds.
 * Pure host function (no device, no workspace).  chunks: matrix chunks per
 * step; launches / launches_stale: kernel launches of a step that recomputes
 * the roots / keeps them (equal when root_period is 1 and in Muon mode);
 * ns_chains: the most Newton-Schulz chains any chunk runs at once (2 when a
 * second chain on the library's side stream fills a partly idle last round
 * of tiles, else 1; 0 in Muon mode); flops / bytes: the algorithmic work of
 * a step that recomputes the roots, per profile category, as
 * okls_profile_read counts it (categories and units below).
 * OKLS_ERR_INVALID_ARG for a NULL out or invalid config or groups. */
typedef struct {
    int chunks;
    int launches;
    int launches_stale;
    int ns_chains;
    double flops[6];
    double bytes[6];
} okls_plan_info;
okls_status okls_plan_query(const okls_config* cfg, int n_groups, const okls_group_desc* groups,
                            okls_plan_info* out);

/* Validates the groups, plans the launches and uploads descriptor tables into
 * the caller's workspace (ws_bytes >= okls_workspace_size, 256-byte aligned).
 * The workspace must stay valid and unused by others until okls_destroy.
 * Synchronises `stream` once.  *out is NULL on error. */
okls_status okls_init(okls_handle** out, const okls_config* cfg, int n_groups,
                      const okls_group_desc* groups, void* workspace, size_t ws_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): okls_init
 * with the library's own static device scratch as the workspace, so the
 * caller passes only its tensors.  The scratch is OKLS_STATIC_SCRATCH_BYTES
 * per device, held by the library until the process ends; groups whose
 * okls_workspace_size exceeds it return OKLS_ERR_WORKSPACE (set
 * chunk_matrices to fit).  Nothing is allocated on the device: the plan runs
 * one Newton-Schulz chain (no side stream or event), and the handle holds
 * host memory only.  Every static handle on a device shares that device's
 * scratch, which keeps the last init's tables: a static handle is valid
 * until the next okls_init_static on the same device, and steps of static
 * handles that overlap on one device race.  Nothing in the scratch is
 * assumed zero: every step writes each buffer before reading it.  Results
 * are bit-identical to okls_init with a workspace.  Synchronises `stream`
 * once (table upload). */
#define OKLS_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
okls_status okls_init_static(okls_handle** out, const okls_config* cfg, int n_groups,
                             const okls_group_desc* groups, void* stream);

/* Fills the state for a fresh start (README "Hyperparameters": eps at factor
 * initialisation): S = eps I, P = I, M = 0 (Muon mode: M = 0 only; SOAP
 * mode: S = 0, bases P = I, M = V = 0).  W and G
 * are not touched (may be NULL).  `tensors` points to n_groups entries.
 * Synchronises `stream` once. */
okls_status okls_init_state(okls_handle* h, const okls_group_tensors* tensors, void* stream);

/* One optimizer step (1-based step counter t, current learning rate lr) for
 * every matrix of every group: steps 1-4 in the header comment.  G is read
 * only; W, M, S_a, S_b, P_a, P_b are updated in place (P only on steps that
 * recompute the roots; Muon mode: W and M only).  S must be symmetric on
 * entry (only its upper triangle is read).  Asynchronous on `stream`; it
 * issues no allocation, memset or synchronisation, so it can be captured
 * into a HIP graph.  t and lr, and what follows from them (the Nesterov
 * scale, the decay, whether the roots are recomputed), are launch arguments:
 * a captured step replays with the values it was captured with, so capture
 * one graph per distinct (t-dependent, lr) step rather than replaying one
 * graph across steps. */
okls_status okls_step(okls_handle* h, const okls_group_tensors* tensors, int64_t t, float lr,
                      void* stream);

/* Scans W, M, S and P of every group (Muon mode: W and M) for Inf/NaN;
 * synchronises `stream`.  Returns OKLS_OK or OKLS_ERR_NONFINITE. */
okls_status okls_check_finite(okls_handle* h, const okls_group_tensors* tensors, void* stream);

/* Convergence diagnostic of the coupled Newton-Schulz roots ("Online KL
 * Shampoo" README, "How it works": the roots come from the coupled
 * iteration).  The last step's T = a I + b Z Y is formed from the product
 * Z_{K-1} Y_{K-1}, which converges to I; that launch's epilogue also sums
 * (Z_{K-1} Y_{K-1} - I)^2 over the factor, in fp32 per wave and tile, and
 * this call reads the partials back (synchronising `stream`) and returns
 * ||Z_{K-1} Y_{K-1} - I||_F summed in double, in the same order every call.
 * Y and Z are the iteration's own scaled fp16 (split: hi + lo) iterates, so
 * the value includes their rounding.
 * out: host array of `count` >= 4 * (matrices over all groups) doubles,
 * out[(mat * 2 + side) * 2 + chain] with mat the matrix index in group order,
 * side 0 for S_a and 1 for S_b, chain 0 for the inverse root and, in the
 * Shampoo mode, chain 1 for the square root of that result (its fourth root).
 * Values are those of the most recent step that recomputed the roots; NaN
 * where none has yet, and for the OKLS mode's chain 1.  OKLS and Shampoo
 * modes only (else OKLS_ERR_UNSUPPORTED); needs ns_steps >= 2 (else NaN). */
okls_status okls_ns_residuals(okls_handle* h, double* out, int64_t count, void* stream);

/* The Newton-Schulz coefficient table the handle uses: a[k], b[k] for
 * k < ns_steps (T_k = a_k I + b_k Z_k Y_k; in Muon mode X <- a_k X +
 * b_k (X X^T) X), written to caller host arrays of length >= max_steps.
 * Returns the number of steps, or -1 on bad arguments. */
int okls_ns_coefficients(const okls_config* cfg, double* a, double* b, int max_steps);

/* Per-launch timing.  While enabled, okls_step records a HIP event before and
 * after every launch on the stream it runs on (events are created on first
 * use and owned by the handle).  okls_profile_read synchronises the last
 * profiled step, sums the elapsed times per category since the last read
 * (ms) and the length of the union of each category's launch intervals
 * (busy_ms: launches of two concurrent Newton-Schulz chains overlap, so
 * their durations add up to more than the time the category keeps the GPU
 * busy), then clears them.  Categories (index into the arrays):
 *   0 Newton-Schulz GEMMs, 1 factor GEMMs (cross-preconditioning and the
 *   factor update), 2 whitening GEMMs (with the fused weight update),
 *   3 statistics kernels, 4 cast / momentum kernels, 5 eigensolver (SOAP
 *   mode: the Jacobi kernels of a basis refresh; the refresh's products
 *   Q^T S Q count in category 0, the rotations into and out of the basis
 *   in category 2 and the Adam kernel in category 4).
 * flops[i] is the algorithmic floating-point work of category i summed over
 * the profiled steps: 27 GEMMs of 2 d^3 per inverse square root (54 for the
 * Shampoo fourth root), 3 m n (m + n) for the OKLS factors (m n (m + n) in
 * Shampoo mode), 2 m n (m + n) for the whitening; in Muon mode every GEMM
 * is in category 0, 4 K p^2 q per matrix (p, q = its smaller and larger
 * side, K = ns_steps: a Gram and an update product per step).  bytes[i] is the
 * algorithmic memory traffic of category i over the profiled steps: every
 * job reads its source once (4 bytes per fp32 element, 2 per bf16 or fp16,
 * twice that for split hi/lo operands; the momentum jobs read M and G and
 * write M'), reads the matrix its epilogue combines with once (4 bytes per
 * fp32 element, 2 per fp16, 4 with low halves), and
 * writes each output once (fp16 outputs 2 bytes per element, 4 with the low
 * halves; fp32 outputs 4). */
#define OKLS_PROFILE_CATEGORIES 6
typedef struct {
    double ms[OKLS_PROFILE_CATEGORIES];       /* sum of the launches' durations */
    double busy_ms[OKLS_PROFILE_CATEGORIES];  /* length of the union of the launches' intervals */
    double flops[OKLS_PROFILE_CATEGORIES];
    double bytes[OKLS_PROFILE_CATEGORIES];
    int64_t launches[OKLS_PROFILE_CATEGORIES];
    int64_t steps;
} okls_profile_stats;

/* okls_profile_enable returns OKLS_ERR_INVALID_ARG for a NULL handle;
 * okls_profile_read returns OKLS_ERR_INVALID_ARG for NULL arguments and
 * OKLS_ERR_HIP if an event query fails (the accumulated sums are then kept). */
okls_status okls_profile_enable(okls_handle* h, int enable);
okls_status okls_profile_read(okls_handle* h, okls_profile_stats* out);

/* Destroys the handle's stream and events and frees its host memory; the
 * caller's tensors and workspace are not touched.  Work already queued by
 * okls_step still completes: each step joins the handle's stream back into
 * the caller's stream, so once the caller's stream has passed the last step
 * the workspace may be freed.  OKLS_ERR_INVALID_ARG for a NULL handle. */
okls_status okls_destroy(okls_handle* h);

/* Static string describing a status code ("unknown status" for any other value). */
const char* okls_status_string(okls_status s);

#ifdef __cplusplus
}
#endif
#endif /* OKLS_H_ */

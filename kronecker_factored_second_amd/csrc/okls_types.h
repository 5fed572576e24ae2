// Internal descriptor types shared by the host scheduler and the gfx950
// kernels.  Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace okls {

constexpr int kMaxGroups = 16;
constexpr int kTile = 128;           // smallest GEMM output tile and padding unit
constexpr int kBigTile = 256;        // large GEMM output tile; sides above kBigPadFrom pad to it
constexpr int kBigPadFrom = 512;
constexpr int kBK = 64;              // GEMM K step
constexpr int kCastRows = 64;        // destination rows of one cast block
constexpr int kCastCols = 256;       // destination columns of one cast block
// bytes of the library's static device scratch (the workspace of handles
// made by okls_init_static, for callers that cannot allocate device memory)
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
constexpr int kMaxJobParts = 1024;   // statistics partials per job, at most
constexpr int kStatThreads = 256;
constexpr int kScaleExp = 14;        // dynamic casts put max |x| in (2^13, 2^14]

// Where a buffer lives: the workspace (byte offset from its base) or a
// caller tensor of one group (byte offset from that tensor's base).
enum RefKind : int32_t {
  REF_NONE = -1, REF_WS = 0, REF_W = 1, REF_G = 2, REF_M = 3,
  REF_SA = 4, REF_SB = 5, REF_PA = 6, REF_PB = 7, REF_V = 8, REF_PSA = 9, REF_PSB = 10
};
struct Ref {
  int32_t kind;
  int32_t group;
  int64_t off;
};

// One GEMM workgroup: problem index (relative to the launch's prob_base)
// and output tile coordinates packed as (ti << 16) | tj.
struct TileRef {
  int32_t prob;
  int32_t ij;
};

// Caller pointers of one okls_step, passed by value to every launch.
struct UserPtrs {
  void* p[kMaxGroups][11];
};

// ---------------------------------------------------------------------------
// GEMM: C (M x N) = alpha * A (M x K) * B (N x K)^T, fp16 operands stored
// row-major with zero padding to multiples of kTile; fp32 accumulation;
// epilogue selected per problem.
// ---------------------------------------------------------------------------
enum Epi : int32_t {
  EPI_STORE32 = 0,   // out32 = v                                  (logical region)
  EPI_SYRK = 1,      // S = c0*S + c1*v + c2*I, mirrored, upper tiles only
  EPI_NS_T = 2,      // T = ka*I + kb*v -> out16 (static scale)
  EPI_NS_Y1 = 3,     // Y1 = ka*(aux*scal[cslot] + c2*I) + kb*v -> out16
  EPI_STORE16 = 4,   // out16 = v * scal[s_out]
  EPI_NS_FINAL = 5,  // out32 = v * scal[cslot] (fp32 root), out16 = v * scal[s_out]
  EPI_UPDATE = 6,    // W = decay*W - lr*c0*v
  EPI_POLAR = 7,     // X' = scal[cslot] * (ka*X + kb*v) -> out16 (+ out16T), X = fp16 aux
  EPI_POLAR_UPDATE = 8,  // W = decay*W - lr*c0*scal[cslot]*(ka*X + kb*v), X = fp16 aux
  EPI_NS_T_RES = 9   // EPI_NS_T, and the partials of ||v - I||_F^2 (one per wave and tile) into resid
};

struct GemmProb {
  Ref A, B;
  int32_t lda, ldb;        // row strides in halves
  int32_t M, N;            // logical output dims
  int32_t Kp;              // padded K (multiple of kTile): length of the hi part of a row
  int32_t epi;
  Ref out32; int32_t ld32;
  Ref out16; int32_t ld16; int32_t lo16;   // lo part at +lo16 halves within a row
  Ref out16T;              // optional transposed copy (Np x Mp)
  int32_t ld16T, lo16T;    // its row stride and lo offset, in halves
  Ref aux; int32_t ldaux;  // EPI_NS_Y1: fp32; EPI_POLAR*: fp16 (padded, Mp x Np)
  int32_t aux_sym;         // EPI_NS_Y1: 1 = read (aux + aux^T) / 2
  int32_t aux_lo;          // EPI_POLAR*: lo part at +aux_lo halves within a row, or -1
  int32_t s_aux;           // EPI_POLAR*: scale slot of the fp16 aux
  int32_t sA, sB;          // scale slots of the operands (alpha = 1/(scal[sA]*scal[sB]))
  int32_t s_out;           // scale slot for fp16 output
  int32_t cslot;           // per-problem device scalar used by the epilogue
  float c0, c1, c2;        // per-problem constants
  int32_t Mp, Np;          // padded output dims
  int32_t resid;           // EPI_NS_T: first float of this problem's residual partials
                           // (one per wave and tile), or -1
  int32_t sym_out;         // EPI_NS_Y1: 1 = the product is symmetric bit for bit (A = B,
                           // unsplit): upper tiles only, each written with its transpose
                           // into both fp16 copies
};

struct GemmArgs {
  const GemmProb* probs;   // device
  const TileRef* tiles;    // device
  int32_t tile_begin;
  int32_t prob_base;
  int32_t split_in;        // 3-segment K loop over [hi | lo] rows
  int32_t write_lo;        // fp16 outputs also write their lo part
  float ka, kb;            // Newton-Schulz step coefficients
  float lr, decay;         // update epilogue
  char* ws;
  float* scal;             // device scalar slots
  float* resid;            // residual partials (problems with resid >= 0)
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Statistics (absmax, sum of squares) per job, as per-block partials.
// ---------------------------------------------------------------------------
// Element format of a gradient source (g_fmt below).
enum GradFmt : int32_t { GF_F32 = 0, GF_BF16 = 1, GF_F16 = 2 };

enum StatKind : int32_t {
  ST_F32 = 0,        // plain fp32 source
  ST_H16 = 1,        // 16-bit gradient source, bf16 or fp16 (g_fmt)
  ST_NESTEROV = 2    // N = s*(beta1*(beta1*M + (1-beta1)*G) + (1-beta1)*G)
};

struct StatJob {
  int32_t kind;
  Ref src; int32_t src_ld;
  Ref src2;                // M for ST_NESTEROV
  int32_t g_fmt;           // ST_H16 / ST_NESTEROV: the gradient's GradFmt
  int32_t rows, cols;
  int32_t rows_per_blk;
  int32_t part_begin;      // partial index of the job's first block
  int32_t blk_begin;       // first block of the job in its launch
};

struct StatArgs {
  const StatJob* jobs;
  int32_t n_jobs;
  int32_t blk_offset;      // block numbering offset (jobs' blk_begin is global)
  float* partials;         // float2 per block: (absmax, sumsq)
  float beta1, s_t;
  float nest_a, nest_b;    // ST_NESTEROV value s_t (nest_a M' + nest_b G)
  char* ws;
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Casts to padded fp16 (hi, optional lo), optional transpose, with a scale
// derived from statistics partials.
// ---------------------------------------------------------------------------
enum CastKind : int32_t {
  CA_F32 = 0,        // x from fp32 source
  CA_H16 = 1,        // x from a 16-bit gradient source, bf16 or fp16 (g_fmt)
  CA_NESTEROV = 2,   // x = N from (G, M); the non-transposed job also writes M'
  CA_NS_Y0 = 3       // x = (S + delta c I) / c', c = sqrt(sumsq); static output scale; the
                     // second destination, if any, gets ka*I + kb*x (Z_1) in the same pass
};
enum ScaleMode : int32_t {
  SC_ABSMAX = 0,     // scale = 2^(kScaleExp - ceil(log2(absmax)))
  SC_STATIC = 1      // scale = scal[scale_slot] (already set)
};

struct CastJob {
  int32_t kind;
  Ref src; int32_t src_ld;
  Ref src2;                // G for CA_NESTEROV (src is M)
  int32_t g_fmt;           // CA_H16 / CA_NESTEROV: the gradient's GradFmt
  int32_t write_m;         // CA_NESTEROV: write M' (non-transposed job only)
  int32_t transpose;
  int32_t rows, cols;      // logical source dims
  int32_t dst_rows_p, dst_cols_p;   // padded destination dims (after transpose)
  Ref dst; int32_t dst_ld; int32_t dst_lo;  // lo at +dst_lo halves within a row
  int32_t part_begin, part_count;
  int32_t scale_mode;
  int32_t scale_slot;      // SC_ABSMAX: written; SC_STATIC: read
  int32_t cinv_slot;       // CA_NS_*: writes 1/c here (if >= 0)
  int32_t rho_slot;        // CA_NS_*: writes 1/sqrt(c) here (if >= 0)
  int32_t sqrtc_slot;      // CA_NS_*: writes sqrt(c) here (if >= 0)
  int32_t p16_slot;        // CA_NS_*: writes the scale of the root's fp16 copy here (if >= 0):
                           // p16_static * sqrt(c) (inverse root, copy Z_K s_Z / 16), or
                           // p16_static / sqrt(c) with p16_inv_sqrt (square root, copy Y_K s_Y)
  float p16_static;        // s_Z / 16 (headroom for directions the iteration does not
                           // resolve, which can leave the last step above the iterates'
                           // bound), or s_Y with p16_inv_sqrt
  int32_t p16_inv_sqrt;
  float damp;              // CA_NS_*: delta; the chain roots (S + delta c I) / (c (1 + delta))
  int32_t sym_read;        // CA_NS_*: 1 = read (S + S^T) / 2 (source not exactly symmetric)
  int32_t tiles_x;         // blocks along destination columns (kCastCols each)
  int32_t blk_begin;
  int32_t write_lo;
  Ref dst2;                // CA_NS_Y0: second destination (same ld and lo offset), or REF_NONE
  int32_t scale_slot2;     // its static scale
  int32_t write_lo2;
  Ref dstT;                // non-transposed jobs: transposed copy of the destination, or REF_NONE
  int32_t dstT_ld, dstT_lo;   // (dst_cols_p x dst_rows_p; same scale and lo flag as dst)
  int32_t aux_slot;        // if >= 0: receives the job's scale times aux_mul (a derived static
  float aux_mul;           // scale for a product of this operand with an orthogonal matrix)
};

struct CastArgs {
  const CastJob* jobs;
  int32_t n_jobs;
  int32_t blk_offset;
  const float* partials;
  float* scal;
  float beta1, s_t, ka, kb;
  float nest_a, nest_b;    // CA_NESTEROV value s_t (nest_a M' + nest_b G)
  char* ws;
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Symmetrisation of a computed root in place, P <- (P + P^T) / 2, with its
// fp16 copy (static scale): one block per pair of kSymTile x kSymTile tiles
// (I, J), I <= J, so every element pair is read and written by one block.
// ---------------------------------------------------------------------------
constexpr int kSymTile = 64;
constexpr int kSymThreads = 256;

struct SymJob {
  Ref p;                   // fp32 d x d, row stride d
  int32_t d, dp;           // side and padded side of the fp16 copy (a multiple of kSymTile)
  int32_t nt;              // tiles per padded side, dp / kSymTile; the copy gets zeros beyond d
  Ref dst16;               // the fp16 copy (dp rows of ld16 halves, lo at +lo16), or REF_NONE
  int32_t ld16, lo16, write_lo;
  int32_t scale_slot;      // the copy's scale
  int32_t blk_begin;
};

struct SymArgs {
  const SymJob* jobs;
  int32_t n_jobs;
  const float* scal;
  char* ws;
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Eigenbasis Adam (SOAP): element-wise second moment and direction from the
// rotated gradient G' and first moment M' (fp32), written as the padded fp16
// operand of the rotation back (static scale).
// ---------------------------------------------------------------------------
constexpr int kAdamRows = 16;        // destination rows of one block (256 columns)
constexpr int kAdamThreads = 256;

struct AdamJob {
  Ref g;                   // G' (rows x cols fp32, row stride cols)
  Ref m;                   // M' (same layout); with eigen_m the caller's M, updated in place
  Ref v;                   // the caller's V (same layout), updated in place
  Ref dst;                 // N' fp16, rows_p rows of ld16 halves, lo at +lo16 (static scale s_out);
                           // REF_NONE: N' goes to dst32 instead
  Ref dst32;               // N' fp32 (rows x cols, row stride cols); may be g itself (read first)
  int32_t rows, cols, rows_p, cols_p, ld16, lo16;
  int32_t eigen_m;         // 1: M <- beta1 M + (1 - beta1) G' first (moments kept in the eigenbasis)
  int32_t tiles_x;         // blocks along the columns (256 each)
  int32_t blk_begin;
};

struct AdamArgs {
  const AdamJob* jobs;
  int32_t n_jobs;
  float beta1, beta2, eps;
  float bc1, bc2;          // 1 / (1 - beta^t), or 1 without bias correction
  float s_out;             // static scale of the fp16 direction
  int32_t write_lo;
  char* ws;
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Block Jacobi eigensolver (two-sided, cyclic over pairs of kJb-row blocks in
// round-robin order).  A round pairs every block with one other; the solve
// kernel diagonalises each pair's 2 kJb x 2 kJb principal submatrix with
// scalar Jacobi rotations and stores the accumulated rotation J; the apply
// kernel then updates B <- R^T B R (R the block-diagonal product of the
// round's J, in the pair ordering) and V <- V R.  A sweep is nb - 1 rounds;
// after each sweep the check kernel compares the off-diagonal Frobenius norm
// with the diagonal's and marks the matrix converged.
// ---------------------------------------------------------------------------
constexpr int kJb = 32;
constexpr int kJp = 2 * kJb;         // side of a pair block
constexpr int kJacThreads = 256;
constexpr int kJacApplyItems = 4;     // B and V tiles per apply block on large rounds
constexpr long kJacManyItems = 65536; // a set's tiles per round from which the rounds are large

struct JacJob {
  Ref B;                   // d x d fp32 (row stride d): Q^T A Q on entry, rotated in place
  Ref V;                   // d x d fp32 (row stride d): the basis Q on entry, rotated in place
  int32_t d, nb, npairs;   // nb: blocks (even, nb * kJb >= d), npairs = nb / 2
  int32_t btiles;          // pair-block tiles of B on and above the diagonal, npairs (npairs + 1) / 2
  int32_t vrows;           // kJp-row chunks of V, ceil(d / kJp)
  int64_t jbuf;            // workspace byte offset of npairs kJp x kJp rotations (fp32)
  int32_t part;            // first partial (float2 per B tile)
  int32_t flag;            // index of the converged flag
  int32_t solve_begin;     // first block of the job in a solve launch
  int32_t apply_begin;     // first block of the job in an apply launch
  int32_t apply_items;     // B and V tiles per apply block (1 or kJacApplyItems)
  float tol;               // converged when ||off(B)||_F <= tol ||diag(B)||_F
};

struct JacArgs {
  const JacJob* jobs;
  int32_t n_jobs;
  int32_t round;           // 0 .. nb - 2 (jobs with fewer rounds skip the rest)
  float* partials;         // float2 (off^2, diag^2) per B tile
  int32_t* flags;
  char* ws;
  UserPtrs user;
};

// ---------------------------------------------------------------------------
// Nystrom low-rank factors.  All arithmetic is fp32 (the sketches are thin:
// k = r + p <= kNysMaxK columns), in four kernels:
//  - thin: fp32 products with at most kThinMaxR columns on the matrix cores
//    (ThinJob below), also the momentum with X = N U_b and the weight update;
//  - nys_orth: thin QR's Q of a d x k matrix in place by classical
//    Gram-Schmidt with reorthogonalisation, a dependent column replaced by a
//    column of the refresh's Gaussian matrix;
//  - nys_small: the k x k end of a refresh (shift, Cholesky, triangular
//    inverse, the Gram of the triangular solve and its eigendecomposition,
//    ordering, sign alignment), one workgroup per factor;
//  - nys_elem: element-wise gather, momentum, column scaling and update.
// ---------------------------------------------------------------------------
constexpr int kNysMaxK = 128;

// Thin fp32 products C = alpha op(A) B (+ beta C) where op(A) is Mo x K (the
// large operand, streamed once) and B is K x R with R <= kThinMaxR: the sketch
// products and the per-step preconditioning.  TA: op(A) = A^T (A stored
// K x Mo).  OT: C stored transposed (R x Mo).  Momentum mode (TA = 0 only):
// op(A) is the Nesterov momentum N computed from the gradient (A, a_fmt) and
// M (same shape, row stride lda), which is updated in place; N is written to
// Nout (row stride ldn).
constexpr int kThinTile = 128;     // rows of op(A) per block
constexpr int kThinK = 32;         // K per LDS stage
constexpr int kThinMaxR = 128;     // columns of B and C
struct ThinJob {
  Ref A, B, C, M, Nout;
  int32_t Mo, K, R;
  int32_t lda, ldb, ldc, ldn;
  int32_t ta, ot, a_fmt, mom;
  float alpha, beta;
  int32_t alpha_slot;      // >= 0: alpha is multiplied by scal[alpha_slot]
  Ref rowscale;            // REF_NONE, or Mo floats: row i of op(A) B times rowscale[i] (ot = 0 only)
  int32_t wupd;            // 1: C is W (Mo x R, stride ldc): W <- decay W - lr c0 (alpha op(A) B + aux)
  Ref aux;                 // wupd: Mo x R fp32, stride ldc
  float c0;                // wupd: the update's shape scale
  int32_t blk_begin;
};

struct ThinArgs {
  const ThinJob* jobs;
  int32_t n_jobs;
  const float* scal;
  float beta1, s_t;        // momentum mode
  float lr, decay;         // weight-update mode
  char* ws;
  UserPtrs user;
};

struct NysOrthJob {
  Ref Y;                   // d x k fp32, row stride ld: replaced by Q
  Ref fb;                  // d x k fp32, row stride ldf: column (j + fb_shift) % k replaces a dependent column j
  int32_t d, k, ld, ldf, fb_shift;
};

struct NysOrthArgs {
  const NysOrthJob* jobs;
  int32_t n_jobs;
  char* ws;
  UserPtrs user;
};

struct NysSmallJob {
  Ref gram;                // k x k: phase 1 Y^T Y; phase 2 F^T F (fp32)
  Ref cmat;                // k x k: phase 1 Omega^T Y in, R^-1 out (fp32)
  Ref ftu;                 // k x r: phase 2 F^T U_prev (fp32)
  Ref kout;                // k x r: phase 2 U = F K (fp32)
  Ref lam;                 // r floats: phase 2 the eigenvalues (the caller's factor)
  Ref scratch;             // 2 k x k doubles (phase 1)
  int32_t k, r;
  int32_t nu_slot, nuu_slot;   // scal slots: the shift nu, and the multiplier nu_u of Omega in Y_nu
};

struct NysSmallArgs {
  const NysSmallJob* jobs;
  int32_t n_jobs;
  int32_t phase;           // 1: shift, Cholesky, R^-1; 2: eigenpairs of F^T F, K, Lambda
  float* scal;
  char* ws;
  UserPtrs user;
};

enum NysElemKind : int32_t {
  NE_GATHER = 0,           // dst (rows x cols) = [src (cols1 columns) | src2 (the rest)]
  NE_SCALE = 1             // dst = src * e_j by column, e_j = sqrt((lam_{r-1} + mu) / (lam_j + mu)) - 1
};

struct NysElemJob {
  int32_t kind;
  Ref dst, src, src2, lam;
  int32_t rows, cols, ld_dst, ld_src, ld_src2, cols1;
  int32_t trans;           // NE_SCALE: dst holds the transpose (cols x rows, row stride ld_dst)
  int32_t blk_begin, blocks;
};

struct NysElemArgs {
  const NysElemJob* jobs;
  int32_t n_jobs;
  float mu;                // NE_SCALE: the eps of eq. (5)
  char* ws;
  UserPtrs user;
};

}  // namespace okls

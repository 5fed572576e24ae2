// Host-side launchers of the gfx950 kernels (okls_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "okls_types.h"

namespace okls {

constexpr int kMaxInitJobs = 6 * kMaxGroups;   // SOAP: S_a, S_b, P_a, P_b, M and V per group

// One caller tensor of one group: batch x rows x cols fp32, filled with
// `diag` on each matrix's diagonal and zero elsewhere (init), or scanned
// for Inf/NaN (finiteness check).
struct InitJob {
  int32_t group;
  int32_t kind;     // RefKind of the tensor
  int32_t batch, rows, cols;
  float diag;
};

struct InitArgs {
  InitJob jobs[kMaxInitJobs];
  UserPtrs user;
};

hipError_t launch_gemm(const GemmArgs& a, int n_tiles, int tile, int epi, hipStream_t s);  // tile 128 or 256; epi: the launch's (single) Epi kind
hipError_t launch_stats(const StatArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_cast(const CastArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_sym(const SymArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_adam(const AdamArgs& a, int n_blocks, hipStream_t s);
enum JacKind { JAC_RESET = 0, JAC_SOLVE = 1, JAC_APPLY = 2, JAC_CHECK = 3 };
// JAC_RESET ignores n_blocks (one block clears every job's flag); JAC_CHECK
// takes one block per job
hipError_t launch_jacobi(const JacArgs& a, int kind, int n_blocks, hipStream_t s);
// Thin fp32 products; every job of one launch has the same ta and mom.
hipError_t launch_thin(const ThinArgs& a, int ta, int mom, int cbm, int wupd, int n_blocks, hipStream_t s);
hipError_t launch_nys_orth(const NysOrthArgs& a, hipStream_t s);     // one block per job
hipError_t launch_nys_small(const NysSmallArgs& a, hipStream_t s);   // one block per job
hipError_t launch_nys_elem(const NysElemArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_init_state(const InitArgs& a, int n_jobs, hipStream_t s);
hipError_t launch_check_finite(const InitArgs& a, int n_jobs, int* flag_dev, hipStream_t s);
// device address of the static scratch (kStaticScratchBytes) on the current
// device; looked up once per device and kept
hipError_t static_scratch(void** ptr);

}  // namespace okls

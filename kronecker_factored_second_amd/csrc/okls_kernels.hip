// gfx950 kernels of the batched OKLS / Shampoo preconditioner step.
//
//  gemm_nt_kernel   grouped fp16 MFMA GEMM, C = alpha A B^T, fp32 accumulation,
//                   256x256 output tiles on 8 waves (two per SIMD, each a
//                   128x64 region) or 128x128 tiles on 4 waves (two blocks per
//                   CU, fragments double-buffered), v_mfma_f32_32x32x16_f16,
//                   operands streamed global -> LDS by direct loads through a
//                   4-deep ring, optional split-fp16 (hi*hi + hi*lo + lo*hi) as
//                   a 3-segment K loop, fused epilogues (factor EMA with
//                   mirrored store, the Newton-Schulz step polynomial, the
//                   weight update).
//  stats_kernel     per-block absmax / sum of squares partials.
//  cast_kernel      fp32/bf16/fp16 -> padded fp16 (hi, lo) with a power-of-two
//                   scale derived from the partials, optional transpose; also
//                   the Nesterov momentum update and the Newton-Schulz start.
//  init_state_kernel, finite_kernel.
//
// The operation each epilogue performs is documented on okls::Epi; the
// mathematics follows the "Online KL Shampoo" README, section "How it works".
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "okls_kernels.h"

namespace okls {

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ char* resolve(const Ref& r, char* ws, const UserPtrs& u) {
  if (r.kind == REF_WS) return ws + r.off;
  return static_cast<char*>(u.p[r.group][r.kind]) + r.off;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// one gradient element of format fmt (GradFmt) at element offset o
__device__ __forceinline__ float grad_elem(const void* p, size_t o, int fmt) {
  if (fmt == GF_F32) return reinterpret_cast<const float*>(p)[o];
  if (fmt == GF_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[o]);
  return static_cast<float>(reinterpret_cast<const half_t*>(p)[o]);
}
// four consecutive gradient elements from one aligned 16-byte (fp32) or
// 8-byte (bf16, fp16) load
template <int FMT>
__device__ __forceinline__ float4 grad_quad(const void* p, size_t o) {
  if constexpr (FMT == GF_F32) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + o);
  } else if constexpr (FMT == GF_BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + o);
    return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  } else {
    const half4_t h = *reinterpret_cast<const half4_t*>(reinterpret_cast<const half_t*>(p) + o);
    return float4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]), static_cast<float>(h[3])};
  }
}
// kPass quads at element offsets o0 + p * op, all issued before any is used
template <int FMT, int N>
__device__ __forceinline__ void load_quads(float4 (&v)[N], const void* p, size_t o0, size_t op) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = grad_quad<FMT>(p, o0 + k * op);
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------

__device__ __forceinline__ void store16(half_t* p, int lo_off, bool write_lo, const float (&x)[4], float s) {
  half4_t hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float y = x[e] * s;
    half_t h = static_cast<half_t>(y);
    hi[e] = h;
    lo[e] = static_cast<half_t>(y - static_cast<float>(h));
  }
  *reinterpret_cast<half4_t*>(p) = hi;
  if (write_lo) *reinterpret_cast<half4_t*>(p + lo_off) = lo;
}

// Tile shape of one GEMM instantiation: BT x BT output tile, WM x WN waves,
// each wave a (BT/WM) x (BT/WN) region of GI x GJ blocks of 32 x 32.  DB
// double-buffers the fragments across stages (one wave per SIMD); without it
// the second wave on each SIMD hides the fragment reads.
template <int BT_, int WM_, int WN_, bool DB_>
struct TileCfg {
  static constexpr int BT = BT_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, THREADS = 64 * NW;
  static constexpr int RM = BT / WM, RN = BT / WN;
  static constexpr int GI = RM / 32, GJ = RN / 32;
  static constexpr int LPW = (BT / 16) / NW;        // wave-loads per operand per stage
  static constexpr bool DB = DB_;
  static constexpr int BLOCKS_PER_CU = BT == 128 ? 2 : 1;
  static_assert(LPW * NW * 16 == BT, "loads must cover the tile");
};
using TileSmall = TileCfg<128, 2, 2, true>;
using TileBig8 = TileCfg<256, 2, 4, false>;

struct EpiCtx {
  float alpha;
  int M, N, ti, tj, rbase, cbase;
  int tr0, tc0;             // origin of this wave's region in the output
  half_t* lds0;             // this wave's staging region (rows [0, RPA) and [RPA, RM))
  half_t* lds1;
  float* out32;
  half_t* out16;
  half_t* out16T;
  const float* aux;
  const half_t* aux16;      // EPI_POLAR*: previous iterate (fp16, scale 1 / aux_inv)
  float s_out, cval, aux_inv;
  int ld32, ld16, lo16, ld16T, lo16T, ldaux, aux_sym, aux_lo;
  bool aux_vec, out32_vec;  // fp32 aux rows / fp32 output rows are 16-byte aligned
  float c0, c1, c2, ka, kb, lr, decay;
  float* resid;             // EPI_NS_T_RES: this wave's residual partial
  int sym_out;              // EPI_NS_Y1, EPI_STORE16: also write the transposed tile into the copies
};

// K advances in stages of 32 through a 4-deep LDS ring filled by
// global_load_lds_dwordx4 (one wave-instruction = 16 rows of 64 B).  Chunk c
// (0..3) of row r is stored at position c ^ ((r >> 2) & 3) so 16-row fragment
// reads hit distinct banks.
constexpr int kSK = 32;                 // K per stage
__device__ __forceinline__ int swz4(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }
// s_waitcnt with vmcnt = v, other counters untouched (gfx9 encoding)
#define WAIT_VMCNT(v) __builtin_amdgcn_s_waitcnt(((v) & 15) | (7 << 4) | (15 << 8) | (((v) >> 4) << 14))
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))

// fp16 outputs go through LDS: each wave stages its RM x RN region (rows of
// RN halves, 16-byte chunks XOR-swizzled by the row so that the accumulator
// writes, the row reads and the column reads below avoid bank conflicts),
// then writes the row-major copy as 16-byte row segments and the transposed
// copy as 16-byte segments of eight rows of one column, so both copies leave
// as whole cache lines.  The stores are non-temporal: every block of a launch
// finishes its tile at about the same time and the burst of outputs (larger
// than L2) is the next launch's input, not this one's.  The region spans one or two ring slots of
// BT * kSK halves; RPA rows fit in one.
template <class C>
struct Stage {
  static constexpr int CH = C::RN / 8;
  static constexpr int RPA = C::BT * kSK / C::RN;
  __device__ static __forceinline__ int off(int r, int c) {
    const int sw = ((r & 7) ^ (r >> 3)) & (CH - 1);
    return (r % RPA) * C::RN + (((c >> 3) ^ sw) << 3) + (c & 7);
  }
  __device__ static __forceinline__ half_t* base(const EpiCtx& x, int r) {
    return (C::RM > RPA && r >= RPA) ? x.lds1 : x.lds0;
  }
  __device__ static __forceinline__ void put(const EpiCtx& x, int r, int c, half4_t h) {
    *reinterpret_cast<half4_t*>(base(x, r) + off(r, c)) = h;
  }
  __device__ static __forceinline__ void flush(const EpiCtx& x, int col_off, int col_off_t) {
    const int lane = threadIdx.x & 63;
    WAIT_LGKM0();                                  // this wave's LDS writes done
    asm volatile("" ::: "memory");
    if (x.out16 != nullptr) {
      constexpr int RPI = 64 / CH;                 // rows per instruction
#pragma unroll
      for (int it = 0; it < C::RM / RPI; ++it) {
        const int r = it * RPI + lane / CH, k = lane % CH;
        const half8_t v = *reinterpret_cast<const half8_t*>(base(x, r) + off(r, k * 8));
        __builtin_nontemporal_store(v, reinterpret_cast<half8_t*>(x.out16 + static_cast<size_t>(x.tr0 + r) * x.ld16 + col_off + x.tc0 + k * 8));
      }
    }
    if (x.out16T != nullptr) {
      constexpr int LPC = C::RM / 8;               // lanes per column (8 rows each)
      constexpr int CPI = 64 / LPC;                // columns per instruction
      const int r0 = 8 * (lane % LPC);
      const half_t* b = base(x, r0);
#pragma unroll
      for (int it = 0; it < C::RN / CPI; ++it) {
        const int c = it * CPI + lane / LPC;
        half8_t v;
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = b[off(r0 + q, c)];
        __builtin_nontemporal_store(v, reinterpret_cast<half8_t*>(x.out16T + static_cast<size_t>(x.tc0 + c) * x.ld16T + col_off_t + x.tr0 + r0));
      }
    }
    // the next staging pass overwrites this wave's region
    WAIT_LGKM0();
    asm volatile("" ::: "memory");
  }
};

// fp32 outputs (plain store, the weight update, the factor update with its
// mirrored lower triangle) also go through LDS, half of the wave's region at
// a time (RM/2 rows of RN floats fill one ring slot): 16-byte chunks of four
// floats, XOR-swizzled by (r ^ (r >> 2)) so that the accumulator writes, the
// row reads and the 4-row column reads of the mirror avoid bank conflicts.
// Rows leave as 16-byte segments (read-modify-write for the update and the
// factor); the factor's mirrored copy leaves as 16-byte segments of four
// rows of one column.
template <class C>
struct Stage32 {
  static constexpr int HR = C::RM / 2;          // rows per half
  static constexpr int CH = C::RN / 4;          // chunks per row
  static_assert(HR * C::RN * 4 <= C::BT * kSK * 2, "half region fits one ring slot");
  __device__ static __forceinline__ int off(int r, int c) {
    const int sw = (r ^ (r >> 2)) & (CH - 1);
    return r * C::RN + (((c >> 2) ^ sw) << 2) + (c & 3);
  }
};

// Four consecutive elements (r, c..c+3) of the fp16 aux (the polar
// iteration's previous iterate), hi + lo when it has lo halves, unscaled.
// The aux is padded to the tile grid, so the quad is always inside it.
__device__ __forceinline__ void aux16_quad(const EpiCtx& x, int r, int c, float (&v)[4]) {
  const half_t* p = x.aux16 + static_cast<size_t>(r) * x.ldaux + c;
  const half4_t h = *reinterpret_cast<const half4_t*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(h[e]);
  if (x.aux_lo >= 0) {
    const half4_t l = *reinterpret_cast<const half4_t*>(p + x.aux_lo);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += static_cast<float>(l[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] *= x.aux_inv;
}

template <class C, int EPI>
__device__ __forceinline__ void epilogue_f32(const floatx16 (&acc)[C::GI][C::GJ], const EpiCtx& x) {
  using S32 = Stage32<C>;
  float* lds = reinterpret_cast<float*>(x.lds0);
  const int lane = threadIdx.x & 63;
  const bool vec_ok = x.out32_vec;    // 16-byte rows: stride and base pointer both aligned
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // stage rows [h HR, (h + 1) HR) of the wave's region
#pragma unroll
    for (int i = h * C::GI / 2; i < (h + 1) * C::GI / 2; ++i) {
      const int rl = x.rbase - x.tr0 + i * 32 - h * S32::HR;
#pragma unroll
      for (int jg = 0; jg < 4 * C::GJ; ++jg) {
        const int j = jg >> 2, g = jg & 3;
        const int cl = x.cbase - x.tc0 + j * 32 + g * 8;
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * x.alpha;
        *reinterpret_cast<floatx4*>(lds + S32::off(rl, cl)) = v;
      }
    }
    WAIT_LGKM0();
    asm volatile("" ::: "memory");
    const int rb = x.tr0 + h * S32::HR;           // global row of local row 0
    constexpr int RPI = 64 / S32::CH;             // rows per instruction
    constexpr int NIT = S32::HR / RPI;
    // read-modify-write kinds: the half's old values (S or W) are all
    // loaded before its first store.  Every quad is read and written by one
    // lane only, and the mirror writes land below the diagonal, which the row
    // pass never reads, so this is the same data; the loads no longer wait
    // one by one behind stores the compiler cannot tell apart from them.
    // (Loading the polar aux ahead too measured slower: its registers spill.)
    constexpr bool kRmw = EPI == EPI_SYRK || EPI == EPI_UPDATE || EPI == EPI_POLAR_UPDATE;
    floatx4 old[kRmw ? NIT : 1];
    if constexpr (kRmw) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int r = rb + it * RPI + lane / S32::CH, c = x.tc0 + 4 * (lane % S32::CH);
        old[it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        if (r < x.M && vec_ok && c + 3 < x.N)
          old[it] = *reinterpret_cast<const floatx4*>(x.out32 + static_cast<size_t>(r) * x.ld32 + c);
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rl = it * RPI + lane / S32::CH, k = lane % S32::CH;
      const int r = rb + rl, c = x.tc0 + 4 * k;
      floatx4 v = *reinterpret_cast<const floatx4*>(lds + S32::off(rl, 4 * k));
      if (r < x.M) {
        float* row = x.out32 + static_cast<size_t>(r) * x.ld32;
        const bool full = vec_ok && c + 3 < x.N;
        if constexpr (EPI == EPI_STORE32) {
          if (full) {
            *reinterpret_cast<floatx4*>(row + c) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < x.N) row[c + e] = v[e];
          }
        } else if constexpr (EPI == EPI_UPDATE || EPI == EPI_POLAR_UPDATE) {
          if constexpr (EPI == EPI_POLAR_UPDATE) {
            float xa[4];
            aux16_quad(x, r, c, xa);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = x.cval * (x.ka * xa[e] + x.kb * v[e]);
          }
          // one fixed rounding, W' = fma(decay, W, -(lr c) v), in both branches
          const float step = x.lr * x.c0;
          if (full) {
            const floatx4 w = old[it];
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(x.decay, w[e], -step * v[e]);
            *reinterpret_cast<floatx4*>(row + c) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < x.N) row[c + e] = __builtin_fmaf(x.decay, row[c + e], -step * v[e]);
          }
        } else {  // EPI_SYRK: S <- c0*S + c1*v + c2*I on the upper triangle
          const bool diag_tile = x.ti == x.tj;
          // one fixed rounding, S' = fma(c0, S, c1 v) (+ eps on the diagonal), in both branches
          if (full && (!diag_tile || r <= c)) {
            const floatx4 o = old[it];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(x.c0, o[e], x.c1 * v[e]) + (r == c + e ? x.c2 : 0.0f);
            *reinterpret_cast<floatx4*>(row + c) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (c + e < x.N && (!diag_tile || r <= c + e)) {
                v[e] = __builtin_fmaf(x.c0, row[c + e], x.c1 * v[e]) + (r == c + e ? x.c2 : 0.0f);
                row[c + e] = v[e];
              }
            }
          }
          *reinterpret_cast<floatx4*>(lds + S32::off(rl, 4 * k)) = v;   // the value the mirror copies
        }
      }
    }
    if constexpr (EPI == EPI_SYRK) {
      // mirrored copy: S[c][r] = S[r][c] for the upper elements, r < c
      WAIT_LGKM0();
      asm volatile("" ::: "memory");
      constexpr int LPC = S32::HR / 4;            // lanes per column (4 rows each)
      constexpr int CPI = 64 / LPC;               // columns per instruction
      const int r0 = 4 * (lane % LPC);
      const bool diag_tile = x.ti == x.tj;
#pragma unroll
      for (int it = 0; it < C::RN / CPI; ++it) {
        const int cl = it * CPI + lane / LPC;
        const int c = x.tc0 + cl, r = rb + r0;
        if (c < x.N) {
          floatx4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = lds[S32::off(r0 + q, cl)];
          float* row = x.out32 + static_cast<size_t>(c) * x.ld32;
          if (vec_ok && r + 3 < x.M && (!diag_tile || r + 3 < c)) {
            *reinterpret_cast<floatx4*>(row + r) = v;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (r + q < x.M && (!diag_tile || r + q < c)) row[r + q] = v[q];
          }
        }
      }
    }
    // the next half overwrites this wave's staging slot
    WAIT_LGKM0();
    asm volatile("" ::: "memory");
  }
}

// One pass over the accumulators of an fp16-output kind: stages PART 0 (the
// fp16 values, or the hi halves of the split layout) or PART 1 (the lo
// halves, y s - fp16(y s)) through LDS.  Block (i, j) of a
// wave holds, in each lane, row rbase + 32 i and the four groups of four
// consecutive columns cbase + 32 j + 8 g + e.
template <class C, int EPI, int PART>
__device__ __forceinline__ void epilogue_pass(const floatx16 (&acc)[C::GI][C::GJ], const EpiCtx& x) {
  static_assert(EPI == EPI_NS_T || EPI == EPI_NS_Y1 || EPI == EPI_STORE16 || EPI == EPI_NS_FINAL || EPI == EPI_POLAR,
                "fp32-output kinds go through epilogue_f32");
#pragma unroll
  for (int i = 0; i < C::GI; ++i) {
    const int r = x.rbase + i * 32;
#pragma unroll
    for (int jg = 0; jg < 4 * C::GJ; ++jg) {
      const int j = jg >> 2, g = jg & 3;
      const int c0 = x.cbase + j * 32 + g * 8;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * x.alpha;
      {
        // fp16 outputs into padded buffers (zeros outside the logical region)
        float xa[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (EPI == EPI_POLAR) aux16_quad(x, r, c0, xa);
        if constexpr (EPI == EPI_NS_Y1) {
          // the rooted matrix at (r, c0..c0+3): one 16-byte load when the quad
          // is inside and its rows are 16-byte aligned (not for the
          // symmetrised read, whose second term is a column)
          if (x.aux_vec && r < x.M && c0 + 3 < x.N) {
            const float4 a4 = *reinterpret_cast<const float4*>(x.aux + static_cast<size_t>(r) * x.ldaux + c0);
            xa[0] = a4.x; xa[1] = a4.y; xa[2] = a4.z; xa[3] = a4.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = c0 + e;
              if (r < x.M && c < x.N) {
                const float a0 = x.aux[static_cast<size_t>(r) * x.ldaux + c];
                xa[e] = x.aux_sym ? 0.5f * (a0 + x.aux[static_cast<size_t>(c) * x.ldaux + r]) : a0;
              }
            }
          }
        }
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c0 + e;
          float t = 0.0f;
          if (r < x.M && c < x.N) {
            if constexpr (EPI == EPI_NS_T) {
              t = (r == c ? x.ka : 0.0f) + x.kb * v[e];
            } else if constexpr (EPI == EPI_POLAR) {
              t = x.cval * (x.ka * xa[e] + x.kb * v[e]);
            } else if constexpr (EPI == EPI_NS_Y1) {
              t = x.ka * (xa[e] * x.cval + (r == c ? x.c2 : 0.0f)) + x.kb * v[e];
            } else {  // EPI_STORE16, EPI_NS_FINAL
              t = v[e];
            }
          }
          y[e] = t;
        }
        if constexpr (EPI == EPI_NS_FINAL && PART == 0) {
          if (x.out32 != nullptr && r < x.M) {
            float* o = x.out32 + static_cast<size_t>(r) * x.ld32 + c0;
            if (x.out32_vec && c0 + 3 < x.N) {
              *reinterpret_cast<float4*>(o) = float4{y[0] * x.cval, y[1] * x.cval, y[2] * x.cval, y[3] * x.cval};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (c0 + e < x.N) o[e] = y[e] * x.cval;
            }
          }
        }
        half4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ys = y[e] * x.s_out;
          const half_t hi = static_cast<half_t>(ys);
          h[e] = PART == 0 ? hi : static_cast<half_t>(ys - static_cast<float>(hi));
        }
        Stage<C>::put(x, r - x.tr0, c0 - x.tc0, h);
      }
    }
  }
  Stage<C>::flush(x, PART == 0 ? 0 : x.lo16, PART == 0 ? 0 : x.lo16T);
  if constexpr (EPI == EPI_NS_Y1 || EPI == EPI_STORE16) {
    // a symmetric product computed on its upper tiles: the tile's transpose
    // is the lower tile, so the copies swap roles for a second write (with
    // no transposed copy, only the transpose into the one copy; on a
    // diagonal tile the two writes of an entry carry the same value)
    if (x.sym_out) {
      EpiCtx y = x;
      y.out16 = x.out16T; y.out16T = x.out16;
      y.ld16 = x.out16T != nullptr ? x.ld16T : x.ld16; y.ld16T = x.ld16;
      y.lo16 = x.out16T != nullptr ? x.lo16T : x.lo16; y.lo16T = x.lo16;
      Stage<C>::flush(y, PART == 0 ? 0 : y.lo16, PART == 0 ? 0 : y.lo16T);
    }
  }
}

// The Newton-Schulz residual's partial: the sum of (Z Y - I)^2 over this
// wave's entries of the logical region (v = Z Y is the accumulator times
// alpha), reduced over the wave in a fixed butterfly order; lane 0 writes it.
template <class C>
__device__ __forceinline__ void resid_partial(const floatx16 (&acc)[C::GI][C::GJ], const EpiCtx& x) {
  float rsum = 0.0f;
#pragma unroll
  for (int i = 0; i < C::GI; ++i) {
    const int r = x.rbase + i * 32;
#pragma unroll
    for (int jg = 0; jg < 4 * C::GJ; ++jg) {
      const int j = jg >> 2, g = jg & 3;
      const int c0 = x.cbase + j * 32 + g * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + e;
        if (r < x.M && c < x.N) {
          const float q = acc[i][j][4 * g + e] * x.alpha - (r == c ? 1.0f : 0.0f);
          rsum = fmaf(q, q, rsum);
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) rsum += __shfl_xor(rsum, off, 64);
  if ((threadIdx.x & 63) == 0) *x.resid = rsum;
}

template <class C, int EPI, bool WL>
__global__ __launch_bounds__(C::THREADS, C::BLOCKS_PER_CU) void gemm_nt_kernel(GemmArgs args) {
  constexpr int BT = C::BT, GI = C::GI, GJ = C::GJ, LPW = C::LPW, NW = C::NW;
  __shared__ half_t sA0[BT * kSK], sA1[BT * kSK], sA2[BT * kSK], sA3[BT * kSK];
  __shared__ half_t sB0[BT * kSK], sB1[BT * kSK], sB2[BT * kSK], sB3[BT * kSK];
  auto bufA = [&](auto bc) -> half_t* {
    constexpr int b = decltype(bc)::value;
    if constexpr (b == 0) return sA0; else if constexpr (b == 1) return sA1; else if constexpr (b == 2) return sA2; else return sA3;
  };
  auto bufB = [&](auto bc) -> half_t* {
    constexpr int b = decltype(bc)::value;
    if constexpr (b == 0) return sB0; else if constexpr (b == 1) return sB1; else if constexpr (b == 2) return sB2; else return sB3;
  };
  // slot k of the eight ring arrays in order sA0..sA3, sB0..sB3
  auto slot = [&](int k) -> half_t* {
    return k == 0 ? sA0 : k == 1 ? sA1 : k == 2 ? sA2 : k == 3 ? sA3 : k == 4 ? sB0 : k == 5 ? sB1 : k == 6 ? sB2 : sB3;
  };

  const TileRef tr = args.tiles[args.tile_begin + blockIdx.x];
  const GemmProb& P = args.probs[args.prob_base + tr.prob];
  const int ti = tr.ij >> 16;
  const int tj = tr.ij & 0xffff;
  const int lda = P.lda, ldb = P.ldb, Kp = P.Kp;

  const half_t* A = reinterpret_cast<const half_t*>(resolve(P.A, args.ws, args.user)) +
                    static_cast<size_t>(ti) * BT * lda;
  const half_t* B = reinterpret_cast<const half_t*>(resolve(P.B, args.ws, args.user)) +
                    static_cast<size_t>(tj) * BT * ldb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int st_per_seg = Kp / kSK;
  const int nst = (args.split_in ? 3 : 1) * st_per_seg;

  const int lr = lane >> 2, lp = lane & 3;   // lane -> row 16h + lr, position lp
  auto gload = [&](int st, auto bc) {
    half_t* dA = bufA(bc);
    half_t* dB = bufB(bc);
    const int seg = st / st_per_seg;
    const int k0 = (st - seg * st_per_seg) * kSK;
    const int offA = (seg == 2 ? Kp : 0) + k0;
    const int offB = (seg == 1 ? Kp : 0) + k0;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int h = wave + NW * q;
      const int row = 16 * h + lr;
      const int c = swz4(row, lp);
      const half_t* ga = A + static_cast<size_t>(row) * lda + offA + c * 8;
      const half_t* gb = B + static_cast<size_t>(row) * ldb + offB + c * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)ga,
                                       (__attribute__((address_space(3))) void*)&dA[h * 16 * kSK], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gb,
                                       (__attribute__((address_space(3))) void*)&dB[h * 16 * kSK], 16, 0, 0);
    }
  };

  floatx16 acc[GI][GJ];
#pragma unroll
  for (int i = 0; i < GI; ++i)
#pragma unroll
    for (int j = 0; j < GJ; ++j) acc[i][j] = floatx16{};

  const int frow = lane & 31;
  const int fch = lane >> 5;
  const int arow = wm * C::RM + frow;
  const int brow = wn * C::RN + frow;
  auto lfrag = [&](half8_t (&fa)[GI], half8_t (&fb)[GJ], auto bc, int s) {
    const half_t* lA = bufA(bc);
    const half_t* lB = bufB(bc);
#pragma unroll
    for (int j = 0; j < GJ; ++j) {
      const int r = brow + 32 * j;
      fb[j] = *reinterpret_cast<const half8_t*>(&lB[r * kSK + swz4(r, 2 * s + fch) * 8]);
    }
#pragma unroll
    for (int i = 0; i < GI; ++i) {
      const int r = arow + 32 * i;
      fa[i] = *reinterpret_cast<const half8_t*>(&lA[r * kSK + swz4(r, 2 * s + fch) * 8]);
    }
  };
  auto mma = [&](const half8_t (&fa)[GI], const half8_t (&fb)[GJ]) {
#pragma unroll
    for (int i = 0; i < GI; ++i)
#pragma unroll
      for (int j = 0; j < GJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  gload(0, I0{});
  gload(1 < nst ? 1 : nst - 1, I1{});
  gload(2 < nst ? 2 : nst - 1, I2{});
  gload(3 < nst ? 3 : nst - 1, I3{});
  if constexpr (C::DB) {
    // Stage st's fragments are in registers F[st & 1] when body st starts.
    // Body st: wait for this wave's copies of stage st+1, barrier (all waves'
    // copies of st+1 visible, all waves done reading slot st % 4), refill
    // slot st % 4 with stage st+4, then read stage st+1's fragments while the
    // MFMAs of stage st run.
    half8_t fa[2][2][GI], fb[2][2][GJ];   // [register set][k16 step][fragment]
    WAIT_VMCNT(3 * 2 * LPW);
    barrier();
    lfrag(fa[0][0], fb[0][0], I0{}, 0);
    lfrag(fa[0][1], fb[0][1], I0{}, 1);
    auto body = [&](int st, auto rc, auto sc, auto nc) {
      constexpr int R = decltype(rc)::value;      // register set of stage st
      WAIT_VMCNT(2 * 2 * LPW);
      barrier();
      const int ld = st + 4;
      gload(ld < nst ? ld : nst - 1, sc);           // slot st % 4
      lfrag(fa[R ^ 1][0], fb[R ^ 1][0], nc, 0);     // stage st+1 from slot (st+1) % 4
      lfrag(fa[R ^ 1][1], fb[R ^ 1][1], nc, 1);
      mma(fa[R][0], fb[R][0]);
      mma(fa[R][1], fb[R][1]);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * LPW, 0);
#pragma unroll
      for (int q = 0; q < 2 * (GI + GJ); ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * GI * GJ / (2 * (GI + GJ)), 0);
      }
      // stage st+1's fragments complete before the next body's MFMAs
      WAIT_LGKM0();
    };
    for (int st = 0; st < nst; st += 4) {
      body(st, I0{}, I0{}, I1{});
      body(st + 1, I1{}, I1{}, I2{});
      body(st + 2, I0{}, I2{}, I3{});
      body(st + 3, I1{}, I3{}, I0{});
    }
  } else {
    // Body st: wait for this wave's copies of stage st, barrier (all waves'
    // copies of st visible, all waves done reading slot (st-1) % 4), refill
    // that slot with stage st+3, read stage st's fragments and run its MFMAs;
    // the other wave on the SIMD covers the fragment latency.
    half8_t fa[2][GI], fb[2][GJ];         // [k16 step][fragment]
    auto body = [&](int st, auto sc, auto pc) {
      // issued so far: stages up to st + 2 (st + 3 before the first body)
      if (st == 0) WAIT_VMCNT(3 * 2 * LPW); else WAIT_VMCNT(2 * 2 * LPW);
      barrier();
      const int ld = st + 3;
      if (st > 0) gload(ld < nst ? ld : nst - 1, pc);  // slot (st - 1) % 4
      lfrag(fa[0], fb[0], sc, 0);
      lfrag(fa[1], fb[1], sc, 1);
      mma(fa[0], fb[0]);
      mma(fa[1], fb[1]);
    };
    for (int st = 0; st < nst; st += 4) {
      body(st, I0{}, I3{});
      body(st + 1, I1{}, I0{});
      body(st + 2, I2{}, I1{});
      body(st + 3, I3{}, I2{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  // every wave is done reading the ring: its slots become the staging area
  __syncthreads();

  // ---------------- epilogue ----------------
  EpiCtx ctx;
  ctx.tr0 = ti * BT + wm * C::RM;
  ctx.tc0 = tj * BT + wn * C::RN;
  constexpr int kSlots = (C::RM + Stage<C>::RPA - 1) / Stage<C>::RPA;   // ring slots per wave region
  ctx.lds0 = slot(kSlots * wave);
  ctx.lds1 = slot(kSlots * wave + kSlots - 1);
  ctx.alpha = 1.0f / (args.scal[P.sA] * args.scal[P.sB]);
  ctx.M = P.M;
  ctx.N = P.N;
  ctx.ti = ti;
  ctx.tj = tj;
  ctx.rbase = ctx.tr0 + frow;
  ctx.cbase = ctx.tc0 + fch * 4;
  ctx.out32 = P.out32.kind != REF_NONE ? reinterpret_cast<float*>(resolve(P.out32, args.ws, args.user)) : nullptr;
  ctx.out16 = P.out16.kind != REF_NONE ? reinterpret_cast<half_t*>(resolve(P.out16, args.ws, args.user)) : nullptr;
  ctx.out16T = P.out16T.kind != REF_NONE ? reinterpret_cast<half_t*>(resolve(P.out16T, args.ws, args.user)) : nullptr;
  ctx.aux = P.aux.kind != REF_NONE ? reinterpret_cast<const float*>(resolve(P.aux, args.ws, args.user)) : nullptr;
  ctx.aux16 = reinterpret_cast<const half_t*>(ctx.aux);
  ctx.aux_vec = ctx.aux != nullptr && !P.aux_sym && (P.ldaux & 3) == 0 && (reinterpret_cast<uintptr_t>(ctx.aux) & 15) == 0;
  ctx.out32_vec = ctx.out32 != nullptr && (P.ld32 & 3) == 0 && (reinterpret_cast<uintptr_t>(ctx.out32) & 15) == 0;
  ctx.aux_inv = P.s_aux >= 0 ? 1.0f / args.scal[P.s_aux] : 1.0f;
  ctx.aux_lo = P.aux_lo;
  ctx.ld16T = P.ld16T;
  ctx.lo16T = P.lo16T;
  ctx.s_out = P.s_out >= 0 ? args.scal[P.s_out] : 1.0f;
  ctx.cval = P.cslot >= 0 ? args.scal[P.cslot] : 1.0f;
  ctx.ld32 = P.ld32;
  ctx.ld16 = P.ld16;
  ctx.lo16 = P.lo16;
  ctx.ldaux = P.ldaux;
  ctx.aux_sym = P.aux_sym;
  ctx.c0 = P.c0;
  ctx.c1 = P.c1;
  ctx.c2 = P.c2;
  ctx.ka = args.ka;
  ctx.kb = args.kb;
  ctx.lr = args.lr;
  ctx.decay = args.decay;
  ctx.resid = nullptr;
  ctx.sym_out = WL ? 0 : P.sym_out;   // symmetric products are unsplit, with no lo halves
  if constexpr (EPI == EPI_NS_T_RES)
    ctx.resid = args.resid + P.resid + (static_cast<size_t>(ti) * (P.Np / BT) + tj) * NW + wave;
  if constexpr (EPI == EPI_STORE32 || EPI == EPI_UPDATE || EPI == EPI_SYRK || EPI == EPI_POLAR_UPDATE) {
    epilogue_f32<C, EPI>(acc, ctx);
  } else {
    // the residual variant of the T product has its own instantiation, so
    // the other T launches keep their register allocation
    constexpr int EPO = EPI == EPI_NS_T_RES ? EPI_NS_T : EPI;
    if constexpr (EPI == EPI_NS_T_RES) resid_partial<C>(acc, ctx);
    epilogue_pass<C, EPO, 0>(acc, ctx);
    if constexpr (WL) epilogue_pass<C, EPO, 1>(acc, ctx);
  }
}

// ---------------------------------------------------------------------------
// Deterministic block reductions
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void block_reduce2(float& amax, float& ss, float* sh) {
  // wave-level butterfly, then one value per wave through LDS; fixed order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    ss += __shfl_xor(ss, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[2 * w] = amax;
    sh[2 * w + 1] = ss;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = sh[0], s = sh[1];
    for (int i = 1; i < NT / 64; ++i) {
      a = fmaxf(a, sh[2 * i]);
      s += sh[2 * i + 1];
    }
    sh[0] = a;
    sh[1] = s;
  }
  __syncthreads();
  amax = sh[0];
  ss = sh[1];
  __syncthreads();
}

template <typename Job>
__device__ __forceinline__ int find_job(const Job* jobs, int n, int gb) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (jobs[mid].blk_begin <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The momentum read of a step: s_t (na M' + nb G) with M' = beta1 M + (1 - beta1) G;
// (na, nb) = (beta1, 1 - beta1) is the Nesterov look-ahead, (1, 0) with s_t = 1
// the first moment M' itself.
__device__ __forceinline__ float nesterov_value(float m, float g, float beta1, float s_t, float na, float nb) {
  const float mn = beta1 * m + (1.0f - beta1) * g;
  return s_t * (na * mn + nb * g);
}

// Flat statistics loop over n4 quads from element e0: four quads per thread
// and iteration, all their loads issued before any is used (one loop per
// source form, so no branch sits between the loads).
template <int FMT, bool NEST>
__device__ __forceinline__ void stats_flat(const char* src, const float* m, size_t e0, size_t n4, float beta1,
                                           float s_t, float na, float nb, float& amax, float& ss) {
  auto acc1 = [&](float x) {
    const float ax = fabsf(x);
    amax = (ax > amax || ax != ax) ? ax : amax;   // NaN propagates
    ss += x * x;
  };
  auto ld = [&](size_t o) -> float4 { return grad_quad<FMT>(src, o); };
  auto use = [&](const float4& g, const float4& mm) {
    if constexpr (NEST) {
      acc1(nesterov_value(mm.x, g.x, beta1, s_t, na, nb));
      acc1(nesterov_value(mm.y, g.y, beta1, s_t, na, nb));
      acc1(nesterov_value(mm.z, g.z, beta1, s_t, na, nb));
      acc1(nesterov_value(mm.w, g.w, beta1, s_t, na, nb));
    } else {
      acc1(g.x); acc1(g.y); acc1(g.z); acc1(g.w);
    }
  };
  size_t q = threadIdx.x;
  for (; q + 3 * kStatThreads < n4; q += 4 * kStatThreads) {
    float4 g[4], mm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t o = e0 + 4 * (q + u * kStatThreads);
      g[u] = ld(o);
      if constexpr (NEST) mm[u] = *reinterpret_cast<const float4*>(m + o);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) use(g[u], mm[u]);
  }
  for (; q < n4; q += kStatThreads) {
    const size_t o = e0 + 4 * q;
    float4 mm{};
    if constexpr (NEST) mm = *reinterpret_cast<const float4*>(m + o);
    use(ld(o), mm);
  }
}

__global__ __launch_bounds__(kStatThreads) void stats_kernel(StatArgs a) {
  __shared__ float sh[2 * (kStatThreads / 64)];
  const int gb = blockIdx.x + a.blk_offset;
  const StatJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  const int lb = gb - J.blk_begin;
  const int r0 = lb * J.rows_per_blk;
  const int r1 = min(J.rows, r0 + J.rows_per_blk);
  const char* src = resolve(J.src, a.ws, a.user);
  const float* m = J.kind == ST_NESTEROV ? reinterpret_cast<const float*>(resolve(J.src2, a.ws, a.user)) : nullptr;
  const int fmt = (J.kind == ST_H16 || J.kind == ST_NESTEROV) ? J.g_fmt : static_cast<int>(GF_F32);
  float amax = 0.0f, ss = 0.0f;
  auto acc1 = [&](float x) {
    const float ax = fabsf(x);
    amax = (ax > amax || ax != ax) ? ax : amax;   // NaN propagates
    ss += x * x;
  };
  auto value = [&](size_t o, float raw) {
    return J.kind == ST_NESTEROV ? nesterov_value(m[o], raw, a.beta1, a.s_t, a.nest_a, a.nest_b) : raw;
  };
  // rows are contiguous when src_ld == cols: one flat range, 16-byte fp32 /
  // 8-byte bf16 and fp16 loads when aligned
  const size_t e0 = static_cast<size_t>(r0) * J.src_ld, e1 = static_cast<size_t>(r1) * J.src_ld;
  const bool flat = J.src_ld == J.cols && (e0 & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(src) & (fmt == GF_F32 ? 15 : 7)) == 0 &&
                    (m == nullptr || (reinterpret_cast<uintptr_t>(m) & 15) == 0);
  if (flat) {
    const size_t n4 = (e1 - e0) / 4;
    if (m != nullptr) {
      if (fmt == GF_BF16) stats_flat<GF_BF16, true>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
      else if (fmt == GF_F16) stats_flat<GF_F16, true>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
      else stats_flat<GF_F32, true>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
    } else {
      if (fmt == GF_BF16) stats_flat<GF_BF16, false>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
      else if (fmt == GF_F16) stats_flat<GF_F16, false>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
      else stats_flat<GF_F32, false>(src, m, e0, n4, a.beta1, a.s_t, a.nest_a, a.nest_b, amax, ss);
    }
    for (size_t o = e0 + 4 * n4 + threadIdx.x; o < e1; o += kStatThreads) {
      acc1(value(o, grad_elem(src, o, fmt)));
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      for (int c = threadIdx.x; c < J.cols; c += kStatThreads) {
        const size_t o = static_cast<size_t>(r) * J.src_ld + c;
        acc1(value(o, grad_elem(src, o, fmt)));
      }
    }
  }
  block_reduce2<kStatThreads>(amax, ss, sh);
  if (threadIdx.x == 0) {
    a.partials[2 * (J.part_begin + lb)] = amax;
    a.partials[2 * (J.part_begin + lb) + 1] = ss;
  }
}

// ---------------------------------------------------------------------------
// Casts
// ---------------------------------------------------------------------------
constexpr int kCastThreads = 256;

__device__ __forceinline__ float pow2_scale(float amax) {
  if (!(amax > 0.0f) || !(amax < 3.0e38f)) return 1.0f;      // zero, NaN or Inf: leave unscaled
  int e;
  const float f = frexpf(amax, &e);                          // amax = f * 2^e, f in [0.5, 1)
  const int ceil_log2 = (f == 0.5f) ? e - 1 : e;
  return ldexpf(1.0f, kScaleExp - ceil_log2);
}

// One in-range source element of a cast job (the edge blocks' path).
__device__ __noinline__ float cast_element(int kind, int ld, int g_fmt, bool write_m, bool sym_read, const char* src,
                                           const char* g, float beta1, float s_t, float na, float nb, int r, int c) {
  const size_t o = static_cast<size_t>(r) * ld + c;
  switch (kind) {
    case CA_F32: return reinterpret_cast<const float*>(src)[o];
    case CA_H16: return grad_elem(src, o, g_fmt);
    case CA_NESTEROV: {
      const float gv = grad_elem(g, o, g_fmt);
      float* m = const_cast<float*>(reinterpret_cast<const float*>(src));
      const float mn = beta1 * m[o] + (1.0f - beta1) * gv;
      if (write_m) m[o] = mn;
      return s_t * (na * mn + nb * gv);
    }
    default: {
      // the rooted matrix is read symmetrised when it is not exactly
      // symmetric (the Shampoo second chain starts from a computed square root)
      const float* f = reinterpret_cast<const float*>(src);
      return sym_read ? 0.5f * (f[o] + f[static_cast<size_t>(c) * ld + r]) : f[o];
    }
  }
}

// One block casts a kCastRows x kCastCols region of the destination.  Its
// source values are loaded first (16 per thread, all in flight together);
// the scale, which needs the job's statistics partials, is combined while
// they arrive, behind a barrier that waits for LDS only.  Transposed jobs go
// through an XOR-swizzled LDS tile.
__global__ __launch_bounds__(kCastThreads) void cast_kernel(CastArgs a) {
  constexpr int kPass = kCastRows * kCastCols / (4 * kCastThreads);   // quads per thread
  static_assert(kPass == 16 && kCastCols == 4 * 64 && kCastThreads == 256, "cast block layout");
  static_assert(kMaxJobParts % kCastThreads == 0, "partials per thread");
  __shared__ float sh[2 * (kCastThreads / 64)];
  __shared__ float tile[kCastCols * kCastRows];     // transposed jobs: [source row][source column]
  const int gb = blockIdx.x + a.blk_offset;
  // a copy in registers: the stores below could alias the table for all the compiler knows
  const CastJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  const int lb = gb - J.blk_begin;
  const int ty = lb / J.tiles_x, tx = lb - ty * J.tiles_x;
  const int dr0 = ty * kCastRows, dc0 = tx * kCastCols;
  const char* src = resolve(J.src, a.ws, a.user);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- 1. source values.  Non-transposed: thread (wave, lane) holds the
  // quad at destination columns dc0 + 4 lane, rows dr0 + wave + 4 p.
  // Transposed: source rows dc0 + (tid >> 4) + 16 p, columns dr0 + 4 (tid & 15).
  // CA_NS_Y0 holds the raw (symmetrised) factor here; it is normalised once c is known.
  const bool tr = J.transpose != 0;
  const int q_col = tr ? 4 * (threadIdx.x & 15) : 4 * lane;
  const int q_row = tr ? (threadIdx.x >> 4) : wave;
  const int q_step = tr ? 16 : 4;
  const int sr0 = tr ? dc0 : dr0, sc0 = tr ? dr0 : dc0;
  // gradient format of the source (CA_H16) or of the second source (CA_NESTEROV)
  const int gfmt = J.g_fmt;
  const bool src_h = J.kind == CA_H16;
  const char* g = J.kind == CA_NESTEROV ? resolve(J.src2, a.ws, a.user) : nullptr;
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & (src_h ? 7 : 15)) == 0) && (J.src_ld & 3) == 0 &&
                   (g == nullptr || (reinterpret_cast<uintptr_t>(g) & (gfmt == GF_F32 ? 15 : 7)) == 0);
  // the job's statistics partials (at most kMaxJobParts / kCastThreads per
  // thread, strided), loaded ahead of the data
  constexpr int kPartsPerThread = kMaxJobParts / kCastThreads;
  float part_a[kPartsPerThread], part_s[kPartsPerThread];
#pragma unroll
  for (int k = 0; k < kPartsPerThread; ++k) {
    const int i = static_cast<int>(threadIdx.x) + k * kCastThreads;
    const bool has = i < J.part_count;
    part_a[k] = has ? a.partials[2 * (J.part_begin + i)] : 0.0f;
    part_s[k] = has ? a.partials[2 * (J.part_begin + i) + 1] : 0.0f;
  }

  float x[kPass][4];
  // a block whose source region lies wholly inside the matrix loads without
  // per-element checks, every load of the thread issued before any is used
  const bool fast = vec && (tr ? (sr0 + kCastCols <= J.rows && sc0 + kCastRows <= J.cols)
                               : (dr0 + kCastRows <= J.rows && dc0 + kCastCols <= J.cols));
  // a symmetrised read (square source, non-transposed job) also needs the
  // mirrored region, source rows dc0.. dc0 + 255 and columns dr0 .. dr0 + 63,
  // loaded as 16-byte quads (row dc0 + (tid >> 4) + 16 p, columns dr0 + 4 (tid & 15))
  // and transposed through LDS once the scale is known
  const bool sym_fast = fast && J.sym_read && !tr;
  float xm[kPass][4];
  if (sym_fast) {
    const float* f32 = reinterpret_cast<const float*>(src);
    const size_t om = static_cast<size_t>(dc0 + (threadIdx.x >> 4)) * J.src_ld + dr0 + 4 * (threadIdx.x & 15);
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(f32 + om + static_cast<size_t>(16 * p) * J.src_ld);
      xm[p][0] = v.x; xm[p][1] = v.y; xm[p][2] = v.z; xm[p][3] = v.w;
    }
  }
  if (fast) {
    const size_t o0 = static_cast<size_t>(sr0 + q_row) * J.src_ld + sc0 + q_col;
    const size_t op = static_cast<size_t>(q_step) * J.src_ld;
    const float* f32 = reinterpret_cast<const float*>(src);
    if (src_h) {
      float4 v[kPass];
      if (gfmt == GF_BF16) load_quads<GF_BF16>(v, src, o0, op);
      else load_quads<GF_F16>(v, src, o0, op);
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        x[p][0] = v[p].x; x[p][1] = v[p].y; x[p][2] = v[p].z; x[p][3] = v[p].w;
      }
    } else if (J.kind == CA_NESTEROV) {
      float4 mo[kPass], gv[kPass];
      load_quads<GF_F32>(mo, src, o0, op);
      if (gfmt == GF_BF16) load_quads<GF_BF16>(gv, g, o0, op);
      else if (gfmt == GF_F16) load_quads<GF_F16>(gv, g, o0, op);
      else load_quads<GF_F32>(gv, g, o0, op);
      const float b1 = a.beta1, b0 = 1.0f - a.beta1, na = a.nest_a, nb = a.nest_b;
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const float4 mn{b1 * mo[p].x + b0 * gv[p].x, b1 * mo[p].y + b0 * gv[p].y,
                        b1 * mo[p].z + b0 * gv[p].z, b1 * mo[p].w + b0 * gv[p].w};
        if (J.write_m) *reinterpret_cast<float4*>(const_cast<float*>(f32) + o0 + p * op) = mn;
        x[p][0] = a.s_t * (na * mn.x + nb * gv[p].x);
        x[p][1] = a.s_t * (na * mn.y + nb * gv[p].y);
        x[p][2] = a.s_t * (na * mn.z + nb * gv[p].z);
        x[p][3] = a.s_t * (na * mn.w + nb * gv[p].w);
      }
    } else {
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(f32 + o0 + p * op);
        x[p][0] = v.x; x[p][1] = v.y; x[p][2] = v.z; x[p][3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int r = sr0 + q_row + q_step * p, c = sc0 + q_col;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[p][e] = (r < J.rows && c + e < J.cols)
                      ? cast_element(J.kind, J.src_ld, gfmt, J.write_m != 0, J.sym_read != 0, src, g, a.beta1, a.s_t,
                                     a.nest_a, a.nest_b, r, c + e)
                      : 0.0f;
    }
  }

  // ---- 2. the scale from the statistics partials (same fixed order in every
  // block): wave butterflies, then every thread combines the waves' results
  // in wave order
  float amax = part_a[0], ss = part_s[0];
#pragma unroll
  for (int k = 1; k < kPartsPerThread; ++k) {
    amax = (part_a[k] > amax || part_a[k] != part_a[k]) ? part_a[k] : amax;
    ss += part_s[k];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(amax, o, 64);
    amax = (om > amax || om != om) ? om : amax;
    ss += __shfl_xor(ss, o, 64);
  }
  if (lane == 0) {
    sh[2 * wave] = amax;
    sh[2 * wave + 1] = ss;
  }
  // LDS visibility only: the source loads stay in flight across the barrier
  WAIT_LGKM0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  amax = sh[0];
  ss = sh[1];
#pragma unroll
  for (int w = 1; w < kCastThreads / 64; ++w) {
    amax = (sh[2 * w] > amax || sh[2 * w] != sh[2 * w]) ? sh[2 * w] : amax;
    ss += sh[2 * w + 1];
  }
  const float scale = J.scale_mode == SC_ABSMAX ? pow2_scale(amax) : a.scal[J.scale_slot];
  if (J.scale_mode == SC_ABSMAX && lb == 0 && threadIdx.x == 0) a.scal[J.scale_slot] = scale;
  if (J.aux_slot >= 0 && lb == 0 && threadIdx.x == 0) a.scal[J.aux_slot] = scale * J.aux_mul;

  half_t* dst = reinterpret_cast<half_t*>(resolve(J.dst, a.ws, a.user));
  const bool write_lo = J.write_lo != 0;
  if (J.kind == CA_NS_Y0) {
    // damped and normalised: Y_0 = (S + delta c I) / c' with c' = c (1 + delta);
    // the second destination gets Z_1 = ka I + kb Y_0
    const float c = sqrtf(ss) * (1.0f + J.damp);
    const float cinv = 1.0f / c;
    const float ddiag = J.damp / (1.0f + J.damp);
    if (lb == 0 && threadIdx.x == 0) {
      if (J.cinv_slot >= 0) a.scal[J.cinv_slot] = cinv;
      if (J.rho_slot >= 0) a.scal[J.rho_slot] = 1.0f / sqrtf(c);
      if (J.sqrtc_slot >= 0) a.scal[J.sqrtc_slot] = sqrtf(c);
      if (J.p16_slot >= 0) a.scal[J.p16_slot] = J.p16_inv_sqrt ? J.p16_static / sqrtf(c) : J.p16_static * sqrtf(c);
    }
    if (sym_fast) {
      // x <- (x + mirrored^T) / 2: mirrored row i (0..255), column j (0..63)
      // at i * 64 + (j ^ ((i >> 2) & 31)), the transposed path's layout
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const int i = (threadIdx.x >> 4) + 16 * p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * (threadIdx.x & 15) + e;
          tile[i * kCastRows + (j ^ ((i >> 2) & 31))] = xm[p][e];
        }
      }
      WAIT_LGKM0();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const int j = wave + 4 * p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * lane + e;
          x[p][e] = 0.5f * (x[p][e] + tile[i * kCastRows + (j ^ ((i >> 2) & 31))]);
        }
      }
    }
    half_t* dst2 = J.dst2.kind != REF_NONE ? reinterpret_cast<half_t*>(resolve(J.dst2, a.ws, a.user)) : nullptr;
    const float scale2 = dst2 != nullptr ? a.scal[J.scale_slot2] : 1.0f;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int r = dr0 + wave + 4 * p, c0 = dc0 + 4 * lane;
      if (c0 >= J.dst_cols_p) continue;
      float y[4], z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = r < J.rows && c0 + e < J.cols;
        y[e] = in ? x[p][e] * cinv + (r == c0 + e ? ddiag : 0.0f) : 0.0f;
        z[e] = in ? (r == c0 + e ? a.ka : 0.0f) + a.kb * y[e] : 0.0f;
      }
      const size_t o = static_cast<size_t>(r) * J.dst_ld + c0;
      store16(dst + o, J.dst_lo, write_lo, y, scale);
      if (dst2 != nullptr) store16(dst2 + o, J.dst_lo, J.write_lo2 != 0, z, scale2);
    }
    return;
  }
  if (!tr) {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int r = dr0 + wave + 4 * p, c0 = dc0 + 4 * lane;
      if (c0 < J.dst_cols_p) store16(dst + static_cast<size_t>(r) * J.dst_ld + c0, J.dst_lo, write_lo, x[p], scale);
    }
    if (J.dstT.kind == REF_NONE) return;
    // transposed copy (dst_cols_p x dst_rows_p): column j (0..255) of the
    // block's region and row i (0..63) live at j * 64 + (i ^ ((j >> 2) & 31)),
    // so both the writes below (one row, columns 4 lane + e) and the reads
    // (one column, rows 4 q + e) spread over the banks
    half_t* dstT = reinterpret_cast<half_t*>(resolve(J.dstT, a.ws, a.user));
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int i = wave + 4 * p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * lane + e;
        tile[j * kCastRows + (i ^ ((j >> 2) & 31))] = x[p][e];
      }
    }
    WAIT_LGKM0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int q = threadIdx.x & 15;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int j = (threadIdx.x >> 4) + 16 * p;     // row dc0 + j of the transposed copy
      if (dc0 + j >= J.dst_cols_p) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[j * kCastRows + ((4 * q + e) ^ ((j >> 2) & 31))];
      store16(dstT + static_cast<size_t>(dc0 + j) * J.dstT_ld + dr0 + 4 * q, J.dstT_lo, write_lo, v, scale);
    }
    return;
  }
  // ---- transposed: destination (r, c) = source (c, r).  Source row i of the
  // block (0..255) and column j (0..63) live at i * 64 + (j ^ ((i >> 2) & 31)),
  // so the column reads below (rows 4 lane + e, one column) hit distinct banks.
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int i = q_row + 16 * p;
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[i * kCastRows + ((q_col + e) ^ ((i >> 2) & 31))] = x[p][e];
  }
  WAIT_LGKM0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int j = wave + 4 * p;                   // destination row dr0 + j = source column
    const int c0 = dc0 + 4 * lane;
    if (c0 >= J.dst_cols_p) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      v[e] = tile[i * kCastRows + (j ^ ((i >> 2) & 31))];
    }
    store16(dst + static_cast<size_t>(dr0 + j) * J.dst_ld + c0, J.dst_lo, write_lo, v, scale);
  }
}

// ---------------------------------------------------------------------------
// Root symmetrisation (SymJob): the block of pair (I, J) loads tiles (I, J)
// and (J, I), then writes (A + B^T) / 2 to the first and its transpose to the
// second, row by row, with the fp16 copy at the same positions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSymThreads) void sym_kernel(SymArgs a) {
  __shared__ float tA[kSymTile][kSymTile + 1], tB[kSymTile][kSymTile + 1];
  const int gb = blockIdx.x;
  const SymJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  int lb = gb - J.blk_begin;
  int ti = 0;                                  // pairs (ti, tj), tj >= ti, row by row
  while (lb >= J.nt - ti) {
    lb -= J.nt - ti;
    ++ti;
  }
  const int tj = ti + lb;
  float* P = reinterpret_cast<float*>(resolve(J.p, a.ws, a.user));
  const size_t d = static_cast<size_t>(J.d);
  const int r0 = ti * kSymTile, c0 = tj * kSymTile;
  half_t* dst = J.dst16.kind != REF_NONE ? reinterpret_cast<half_t*>(resolve(J.dst16, a.ws, a.user)) : nullptr;
  // rows of four: 16-byte fp32 and 8-byte fp16 accesses when every row
  // start is aligned (d, the copy's stride and lo offset multiples of 4)
  const bool vec = (d & 3) == 0 && (reinterpret_cast<uintptr_t>(P) & 15) == 0 &&
                   (dst == nullptr || ((J.ld16 & 3) == 0 && (J.lo16 & 3) == 0 && (reinterpret_cast<uintptr_t>(dst) & 7) == 0));
  constexpr int Q = kSymTile / 4;              // quads per tile row
  if (vec) {
    for (int k = threadIdx.x; k < kSymTile * Q; k += kSymThreads) {
      const int r = k / Q, c = (k % Q) * 4;
      float4 x = float4{0.0f, 0.0f, 0.0f, 0.0f}, y = float4{0.0f, 0.0f, 0.0f, 0.0f};
      // d is a multiple of 4, so a quad is wholly inside or wholly outside
      if (r0 + r < J.d && c0 + c < J.d) x = *reinterpret_cast<const float4*>(P + (r0 + r) * d + c0 + c);
      if (c0 + r < J.d && r0 + c < J.d) y = *reinterpret_cast<const float4*>(P + (c0 + r) * d + r0 + c);
      tA[r][c] = x.x; tA[r][c + 1] = x.y; tA[r][c + 2] = x.z; tA[r][c + 3] = x.w;
      tB[r][c] = y.x; tB[r][c + 1] = y.y; tB[r][c + 2] = y.z; tB[r][c + 3] = y.w;
    }
  } else {
    for (int k = threadIdx.x; k < kSymTile * kSymTile; k += kSymThreads) {
      const int r = k / kSymTile, c = k % kSymTile;
      const bool in_a = r0 + r < J.d && c0 + c < J.d, in_b = c0 + r < J.d && r0 + c < J.d;
      tA[r][c] = in_a ? P[(r0 + r) * d + c0 + c] : 0.0f;
      tB[r][c] = in_b ? P[(c0 + r) * d + r0 + c] : 0.0f;
    }
  }
  __syncthreads();
  const float sc = dst != nullptr ? a.scal[J.scale_slot] : 1.0f;
  auto put = [&](size_t gr, size_t gc, float v) {
    if (gr < d && gc < d) P[gr * d + gc] = v;
    if (dst != nullptr) {
      const float y = v * sc;
      const half_t h = static_cast<half_t>(y);
      half_t* q = dst + gr * J.ld16 + gc;
      q[0] = h;
      if (J.write_lo) q[J.lo16] = static_cast<half_t>(y - static_cast<float>(h));
    }
  };
  // (gr, gc .. gc + 3) from the symmetrised values v; the copy's padding
  // (positions beyond d) gets the zeros the tiles hold there
  auto put4 = [&](size_t gr, size_t gc, const float (&v)[4]) {
    if (gr < d && gc < d) *reinterpret_cast<float4*>(P + gr * d + gc) = float4{v[0], v[1], v[2], v[3]};
    if (dst != nullptr) {
      half4_t h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = v[e] * sc;
        h[e] = static_cast<half_t>(y);
        l[e] = static_cast<half_t>(y - static_cast<float>(h[e]));
      }
      half_t* q = dst + gr * J.ld16 + gc;
      *reinterpret_cast<half4_t*>(q) = h;
      if (J.write_lo) *reinterpret_cast<half4_t*>(q + J.lo16) = l;
    }
  };
  for (int half_pass = 0; half_pass < (ti == tj ? 1 : 2); ++half_pass) {
    // pass 0: tile (ti, tj) = (A + B^T) / 2; pass 1: its mirror (tj, ti)
    const int gr0 = half_pass == 0 ? r0 : c0, gc0 = half_pass == 0 ? c0 : r0;
    if (vec) {
      for (int k = threadIdx.x; k < kSymTile * Q; k += kSymThreads) {
        const int r = k / Q, c = (k % Q) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = half_pass == 0 ? 0.5f * (tA[r][c + e] + tB[c + e][r]) : 0.5f * (tB[r][c + e] + tA[c + e][r]);
        put4(gr0 + r, gc0 + c, v);
      }
    } else {
      for (int k = threadIdx.x; k < kSymTile * kSymTile; k += kSymThreads) {
        const int r = k / kSymTile, c = k % kSymTile;
        put(gr0 + r, gc0 + c, half_pass == 0 ? 0.5f * (tA[r][c] + tB[c][r]) : 0.5f * (tB[r][c] + tA[c][r]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// State initialisation and finiteness scan
// ---------------------------------------------------------------------------
__global__ void init_state_kernel(InitArgs a) {
  const InitJob& J = a.jobs[blockIdx.y];
  float* p = static_cast<float*>(a.user.p[J.group][J.kind]);
  const size_t dd = static_cast<size_t>(J.rows) * J.cols;
  const size_t total = dd * J.batch;
  for (size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t w = e % dd;
    const size_t r = w / J.cols, c = w - r * J.cols;
    p[e] = (r == c) ? J.diag : 0.0f;
  }
}

__global__ void finite_kernel(InitArgs a, int* flag) {
  const InitJob& J = a.jobs[blockIdx.y];
  const float* p = static_cast<const float*>(a.user.p[J.group][J.kind]);
  const size_t total = static_cast<size_t>(J.rows) * J.cols * J.batch;
  int bad = 0;
  for (size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const float x = p[e];
    bad |= !(fabsf(x) <= 3.4028235e38f);
  }
  if (bad) atomicOr(flag, 1);
}

__global__ void zero_int_kernel(int* p) { *p = 0; }

// ---------------------------------------------------------------------------
// Eigenbasis Adam (AdamJob): V <- beta2 V + (1 - beta2) G'^2 and the direction
// N' = (M' bc1) / (sqrt(V bc2) + eps) element by element (with eigen_m the
// first moment M <- beta1 M + (1 - beta1) G' is updated first and is M'),
// written into the zero-padded fp16 operand of the rotation back, or as fp32
// (where no static bound on |N'| holds, for a cast with its own scale).  One block
// covers kAdamRows x 256 of the padded destination; thread (wave, lane) holds
// columns 4 lane .. 4 lane + 3 of rows wave + 4 p.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAdamThreads) void adam_kernel(AdamArgs a) {
  const int gb = blockIdx.x;
  const AdamJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  const int lb = gb - J.blk_begin;
  const int ty = lb / J.tiles_x, tx = lb - ty * J.tiles_x;
  const int c0 = tx * 256 + 4 * (threadIdx.x & 63);
  const float* g = reinterpret_cast<const float*>(resolve(J.g, a.ws, a.user));
  float* m = reinterpret_cast<float*>(resolve(J.m, a.ws, a.user));
  float* v = reinterpret_cast<float*>(resolve(J.v, a.ws, a.user));
  const bool to16 = J.dst.kind != REF_NONE;
  half_t* dst = to16 ? reinterpret_cast<half_t*>(resolve(J.dst, a.ws, a.user)) : nullptr;
  float* d32 = to16 ? nullptr : reinterpret_cast<float*>(resolve(J.dst32, a.ws, a.user));
  const float b1 = a.beta1, b1c = 1.0f - a.beta1, b2 = a.beta2, b2c = 1.0f - a.beta2;
  const bool vec = (J.cols & 3) == 0 && (reinterpret_cast<uintptr_t>(g) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(m) & 15) == 0 && (reinterpret_cast<uintptr_t>(v) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(d32) & 15) == 0;
  if (c0 >= J.cols_p) return;
#pragma unroll
  for (int p = 0; p < kAdamRows / 4; ++p) {
    const int r = ty * kAdamRows + (threadIdx.x >> 6) + 4 * p;
    if (r >= J.rows_p) continue;
    float gq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, mq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const size_t o = static_cast<size_t>(r) * J.cols + c0;
    const bool row_in = r < J.rows;
    const bool full = row_in && vec && c0 + 3 < J.cols;
    if (full) {
      const float4 g4 = *reinterpret_cast<const float4*>(g + o);
      const float4 m4 = *reinterpret_cast<const float4*>(m + o);
      const float4 v4 = *reinterpret_cast<const float4*>(v + o);
      gq[0] = g4.x; gq[1] = g4.y; gq[2] = g4.z; gq[3] = g4.w;
      mq[0] = m4.x; mq[1] = m4.y; mq[2] = m4.z; mq[3] = m4.w;
      vq[0] = v4.x; vq[1] = v4.y; vq[2] = v4.z; vq[3] = v4.w;
    } else if (row_in) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < J.cols) { gq[e] = g[o + e]; mq[e] = m[o + e]; vq[e] = v[o + e]; }
    }
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (J.eigen_m) mq[e] = b1 * mq[e] + b1c * gq[e];
      vq[e] = b2 * vq[e] + b2c * gq[e] * gq[e];
      y[e] = (mq[e] * a.bc1) / (sqrtf(vq[e] * a.bc2) + a.eps);
      if (!(row_in && c0 + e < J.cols)) y[e] = 0.0f;
    }
    if (full) {
      *reinterpret_cast<float4*>(v + o) = float4{vq[0], vq[1], vq[2], vq[3]};
      if (J.eigen_m) *reinterpret_cast<float4*>(m + o) = float4{mq[0], mq[1], mq[2], mq[3]};
      if (!to16) *reinterpret_cast<float4*>(d32 + o) = float4{y[0], y[1], y[2], y[3]};
    } else if (row_in) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < J.cols) {
          v[o + e] = vq[e];
          if (J.eigen_m) m[o + e] = mq[e];
          if (!to16) d32[o + e] = y[e];
        }
    }
    if (to16) store16(dst + static_cast<size_t>(r) * J.ld16 + c0, J.lo16, a.write_lo != 0, y, a.s_out);
  }
}

// ---------------------------------------------------------------------------
// Block Jacobi (JacJob).  Pairing: the round-robin ("circle") schedule of n
// players, player 0 fixed and the others rotated by one each round, pairs
// position k with position n - 1 - k; over n - 1 rounds every pair meets once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void circle_pair(int round, int k, int n, int& p, int& q) {
  const int a = k == 0 ? 0 : ((k - 1 + round) % (n - 1)) + 1;
  const int kb = n - 1 - k;
  const int b = kb == 0 ? 0 : ((kb - 1 + round) % (n - 1)) + 1;
  p = min(a, b);
  q = max(a, b);
}
// global row of local index i (0 .. kJp - 1) of the pair block (p, q)
__device__ __forceinline__ int pair_index(int p, int q, int i) { return i < kJb ? p * kJb + i : q * kJb + i - kJb; }

template <bool APPLY>
__device__ __forceinline__ int find_jac_job(const JacJob* jobs, int n, int gb) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((APPLY ? jobs[mid].apply_begin : jobs[mid].solve_begin) <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One sweep over the pair block per round: the outer sweeps finish the job.
// Measured on a CPU model of this solver (fp32, Wishart factors at d = 160
// and 320): full inner diagonalisation (up to 12 sweeps) needs 6 and 12
// outer sweeps, one inner sweep 7 and 13, with a third of the inner work.
constexpr int kJacInnerSweeps = 1;

// Diagonalises the pair block A = sym(B[I, I]), I the rows of blocks p and q,
// by cyclic Jacobi rotations in round-robin order (kJb disjoint rotations per
// round, applied to rows, then columns and the accumulated J), and stores J.
// Rotation of (u, w): with tau = (a_ww - a_uu) / (2 a_uw), t = sign(tau) /
// (|tau| + sqrt(1 + tau^2)), c = 1 / sqrt(1 + t^2), s = t c, the plane rotation
// [[c, s], [-s, c]] zeroes a_uw (the symmetric Schur decomposition of a 2 x 2
// block, Golub and Van Loan, "Matrix Computations", the classical Jacobi method).
__global__ __launch_bounds__(kJacThreads) void jacobi_solve_kernel(JacArgs a) {
  __shared__ float A[kJp][kJp + 1];
  __shared__ float Jm[kJp][kJp + 1];
  __shared__ float rc[kJb], rs[kJb], rdu[kJb], rdw[kJb];
  __shared__ int ru[kJb], rw[kJb], rrot[kJb];
  __shared__ int any_rot;
  __shared__ float red[kJacThreads / 64];
  const int gb = blockIdx.x;
  const JacJob J = a.jobs[find_jac_job<false>(a.jobs, a.n_jobs, gb)];
  const int k = gb - J.solve_begin;
  if (a.round >= J.nb - 1 || a.flags[J.flag] != 0) return;
  int p, q;
  circle_pair(a.round, k, J.nb, p, q);
  const float* B = reinterpret_cast<const float*>(resolve(J.B, a.ws, a.user));
  const size_t d = static_cast<size_t>(J.d);
  float ss = 0.0f;
  for (int e = threadIdx.x; e < kJp * kJp; e += kJacThreads) {
    const int i = e / kJp, j = e % kJp;
    const size_t gi = pair_index(p, q, i), gj = pair_index(p, q, j);
    float x = 0.0f;
    if (gi < d && gj < d) x = 0.5f * (B[gi * d + gj] + B[gj * d + gi]);
    A[i][j] = x;
    Jm[i][j] = i == j ? 1.0f : 0.0f;
    ss += x * x;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float fro2 = 0.0f;
#pragma unroll
  for (int w = 0; w < kJacThreads / 64; ++w) fro2 += red[w];
  // rotations below this size are rounding noise of the block (or exact zeros)
  const float floor_abs = 1e-10f * sqrtf(fro2);
  for (int sweep = 0; sweep < kJacInnerSweeps; ++sweep) {
    if (threadIdx.x == 0) any_rot = 0;
    __syncthreads();
    for (int r = 0; r < kJp - 1; ++r) {
      if (threadIdx.x < kJb) {
        int u, w;
        circle_pair(r, threadIdx.x, kJp, u, w);
        const float auu = A[u][u], aww = A[w][w], auw = A[u][w];
        float c = 1.0f, sn = 0.0f, du = auu, dw = aww;
        int rot = 0;
        if (fabsf(auw) > floor_abs && fabsf(auw) > 1e-7f * sqrtf(fabsf(auu * aww))) {
          // in fp64, so that c and s are the fp32 roundings of one exact
          // rotation: fp32 arithmetic here leaves c^2 + s^2 - 1 biased, and the
          // bias compounds over the thousands of rotations a basis goes through
          // (measured: orthogonality 1e-4 against 4e-6)
          const double tau = (static_cast<double>(aww) - auu) / (2.0 * auw);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          const double cd = 1.0 / sqrt(1.0 + t * t);
          c = static_cast<float>(cd);
          sn = static_cast<float>(t * cd);
          du = static_cast<float>(auu - t * auw);
          dw = static_cast<float>(aww + t * auw);
          rot = 1;
          any_rot = 1;
        }
        ru[threadIdx.x] = u; rw[threadIdx.x] = w; rc[threadIdx.x] = c; rs[threadIdx.x] = sn;
        rdu[threadIdx.x] = du; rdw[threadIdx.x] = dw; rrot[threadIdx.x] = rot;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < kJb * kJp; e += kJacThreads) {   // rows u, w of A
        const int kk = e / kJp, col = e % kJp;
        if (rrot[kk]) {
          const int u = ru[kk], w = rw[kk];
          const float c = rc[kk], sn = rs[kk];
          const float xu = A[u][col], xw = A[w][col];
          A[u][col] = c * xu - sn * xw;
          A[w][col] = sn * xu + c * xw;
        }
      }
      __syncthreads();
      for (int e = threadIdx.x; e < kJb * kJp; e += kJacThreads) {   // columns u, w of A and of J
        const int kk = e / kJp, row = e % kJp;
        if (rrot[kk]) {
          const int u = ru[kk], w = rw[kk];
          const float c = rc[kk], sn = rs[kk];
          const float xu = A[row][u], xw = A[row][w];
          A[row][u] = c * xu - sn * xw;
          A[row][w] = sn * xu + c * xw;
          const float ju = Jm[row][u], jw = Jm[row][w];
          Jm[row][u] = c * ju - sn * jw;
          Jm[row][w] = sn * ju + c * jw;
        }
      }
      __syncthreads();
      if (threadIdx.x < kJb && rrot[threadIdx.x]) {   // the rotated 2 x 2 block exactly diagonal
        const int u = ru[threadIdx.x], w = rw[threadIdx.x];
        A[u][w] = 0.0f;
        A[w][u] = 0.0f;
        A[u][u] = rdu[threadIdx.x];
        A[w][w] = rdw[threadIdx.x];
      }
      __syncthreads();
    }
    const bool more = any_rot != 0;
    __syncthreads();
    if (!more) break;
  }
  float* jb = reinterpret_cast<float*>(a.ws + J.jbuf) + static_cast<size_t>(k) * kJp * kJp;
  for (int e = threadIdx.x; e < kJp * kJp; e += kJacThreads) jb[e] = Jm[e / kJp][e % kJp];
}

// B <- R^T B R on the pair-block tiles (P, Q), P <= Q (the lower tile gets the
// transpose), and V <- V R on kJp-row chunks of V; every B tile records the
// squared Frobenius norms of its off-diagonal and diagonal entries (the
// mirrored tile counted twice).  A block takes apply_items consecutive
// tiles, the next one's loads in flight during the current one's products.
// The 64 x 64 products run on the matrix cores in fp32 (v_mfma_f32_32x32x2_f32): wave w computes the 32 x 32 block
// (w / 2, w % 2) of each product from LDS operands stored k-major (row k
// holds the 64 entries of index k), so every fragment read is 32 contiguous
// floats.  Lane (h, n) of a product holds column n of its block and rows
// 8 (r / 4) + 4 h + r % 4 for accumulator element r.
__device__ __forceinline__ floatx16 jac_mfma64(const float (*L)[kJp + 4], const float (*R)[kJp + 4], int m0, int n0,
                                               int h, int n) {
  // sum over k of L[k][m0 + m] R[k][n0 + n]: lanes of half h take k = 2 kk + h
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll 8
  for (int kk = 0; kk < kJp / 2; ++kk)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(L[2 * kk + h][m0 + n], R[2 * kk + h][n0 + n], acc, 0, 0, 0);
  return acc;
}

// Entries (r, c .. c + 3) of a d x d row-major matrix, zeros outside it; c
// is a multiple of 4 inside one kJb block, so with d a multiple of 4 the
// quad is wholly inside or wholly outside.
__device__ __forceinline__ float4 jac_quad(const float* M, size_t r, size_t c, size_t d, bool vec) {
  float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
  if (r >= d) return v;
  if (vec) {
    if (c < d) v = *reinterpret_cast<const float4*>(M + r * d + c);
  } else {
    if (c < d) v.x = M[r * d + c];
    if (c + 1 < d) v.y = M[r * d + c + 1];
    if (c + 2 < d) v.z = M[r * d + c + 2];
    if (c + 3 < d) v.w = M[r * d + c + 3];
  }
  return v;
}

__global__ __launch_bounds__(kJacThreads) void jacobi_apply_kernel(JacArgs a) {
  constexpr int LD = kJp + 4;                      // 16-byte aligned rows
  static_assert(kJacThreads == 256 && kJp == 64, "four waves, each a 32 x 32 block of a 64 x 64 product");
  __shared__ __attribute__((aligned(16))) float X[kJp][LD];
  __shared__ __attribute__((aligned(16))) float JP[kJp][LD];
  __shared__ __attribute__((aligned(16))) float JQ[kJp][LD];
  __shared__ float red[2 * (kJacThreads / 64)];
  const int gb = blockIdx.x;
  const JacJob J = a.jobs[find_jac_job<true>(a.jobs, a.n_jobs, gb)];
  if (a.round >= J.nb - 1 || a.flags[J.flag] != 0) return;
  // the block's work items: B tiles 0 .. btiles - 1, then V tiles (chunk, Q)
  const int n_items = J.btiles + J.vrows * J.npairs;
  const int it0 = (gb - J.apply_begin) * J.apply_items;
  const int it1 = min(it0 + J.apply_items, n_items);
  const float* jb = reinterpret_cast<const float*>(a.ws + J.jbuf);
  const size_t d = static_cast<size_t>(J.d);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
  const int m0 = 32 * (wave >> 1), n0 = 32 * (wave & 1);
  float* B = reinterpret_cast<float*>(resolve(J.B, a.ws, a.user));
  float* V = reinterpret_cast<float*>(resolve(J.V, a.ws, a.user));
  // 16-byte accesses along rows: d a multiple of 4 and the matrix 16-byte
  // aligned (a block's 32 entries then start aligned)
  const bool bvec = (d & 3) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  const bool vvec = (d & 3) == 0 && (reinterpret_cast<uintptr_t>(V) & 15) == 0;

  // item it: B tile (P, Q), P <= Q, row by row; or V chunk `chunk` of pair Q
  struct Item { int P, Q, chunk; };
  auto item = [&](int it) __attribute__((always_inline)) {
    Item r;
    if (it < J.btiles) {
      int P = 0, rem = it;
      while (rem >= J.npairs - P) {
        rem -= J.npairs - P;
        ++P;
      }
      r.P = P; r.Q = P + rem; r.chunk = -1;
    } else {
      const int v = it - J.btiles;
      r.chunk = v / J.npairs; r.Q = v - r.chunk * J.npairs; r.P = -1;
    }
    return r;
  };
  // the item's operands into registers: quad u = threadIdx.x + 256 v is
  // row u / 16, columns 4 (u % 16) .. + 3 (of the B tile, of V's chunk, of
  // J_P and of J_Q); four named quads each, so that they stay in registers
  float4 ox0, ox1, ox2, ox3, op0, op1, op2, op3, oq0, oq1, oq2, oq3;
  auto fetch_quad = [&](const Item& w, int v, float4& x, float4& pq, float4& qq) __attribute__((always_inline)) {
    const int u = threadIdx.x + kJacThreads * v, i = u >> 4, j = (u & 15) * 4;
    int c1, c2;
    circle_pair(a.round, w.Q, J.nb, c1, c2);
    qq = *reinterpret_cast<const float4*>(jb + static_cast<size_t>(w.Q) * kJp * kJp + 4 * u);
    if (w.chunk < 0) {
      int r1, r2;
      circle_pair(a.round, w.P, J.nb, r1, r2);
      x = jac_quad(B, pair_index(r1, r2, i), pair_index(c1, c2, j), d, bvec);
      pq = *reinterpret_cast<const float4*>(jb + static_cast<size_t>(w.P) * kJp * kJp + 4 * u);
    } else {
      x = jac_quad(V, static_cast<size_t>(w.chunk) * kJp + i, pair_index(c1, c2, j), d, vvec);
      pq = float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto fetch = [&](const Item& w) __attribute__((always_inline)) {
    fetch_quad(w, 0, ox0, op0, oq0);
    fetch_quad(w, 1, ox1, op1, oq1);
    fetch_quad(w, 2, ox2, op2, oq2);
    fetch_quad(w, 3, ox3, op3, oq3);
  };
  auto stage_quad = [&](bool bt, int v, const float4& x, const float4& pq, const float4& qq) __attribute__((always_inline)) {
    const int u = threadIdx.x + kJacThreads * v, i = u >> 4, j = (u & 15) * 4;
    if (bt) {
      *reinterpret_cast<float4*>(&X[i][j]) = x;
      *reinterpret_cast<float4*>(&JP[i][j]) = pq;
    } else {
      // X holds V's chunk transposed: X[j][i] = V[r0 + i][col j]
      X[j][i] = x.x; X[j + 1][i] = x.y; X[j + 2][i] = x.z; X[j + 3][i] = x.w;
    }
    *reinterpret_cast<float4*>(&JQ[i][j]) = qq;
  };

  if (it0 >= it1) return;
  Item cur = item(it0);
  fetch(cur);
  for (int it = it0; it < it1; ++it) {
    __syncthreads();                               // the previous item's LDS reads are done
    const bool bt = cur.chunk < 0;
    stage_quad(bt, 0, ox0, op0, oq0);
    stage_quad(bt, 1, ox1, op1, oq1);
    stage_quad(bt, 2, ox2, op2, oq2);
    stage_quad(bt, 3, ox3, op3, oq3);
    __syncthreads();
    const Item w = cur;
    if (it + 1 < it1) {                            // the next item's loads, in flight during these products
      cur = item(it + 1);
      fetch(cur);
    }
    int q1, q2;
    circle_pair(a.round, w.Q, J.nb, q1, q2);
    const size_t gj = pair_index(q1, q2, n0 + n);
    if (w.chunk >= 0) {
      const floatx16 acc = jac_mfma64(X, JQ, m0, n0, h, n);   // Y = V_chunk J_Q
      if (gj < d) {
        const size_t r0 = static_cast<size_t>(w.chunk) * kJp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const size_t row = r0 + m0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < d) V[row * d + gj] = acc[r];
        }
      }
      continue;
    }
    int p1, p2;
    circle_pair(a.round, w.P, J.nb, p1, p2);
    floatx16 acc = jac_mfma64(JP, X, m0, n0, h, n);   // T = J_P^T X
    __syncthreads();
    // X <- T^T: row k of X holds column k of T (the lane's four rows at once)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&X[n0 + n][m0 + 8 * g + 4 * h]) =
          float4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    __syncthreads();
    acc = jac_mfma64(X, JQ, m0, n0, h, n);            // Y = T J_Q
    float off = 0.0f, dg = 0.0f;
    const float wgt = w.P == w.Q ? 1.0f : 2.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // rows m0 + 8 g + 4 h + e lie in one kJb block: consecutive in B
      const size_t gi0 = pair_index(p1, p2, m0 + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t gi = gi0 + e;
        if (gi < d && gj < d) {
          const float y = acc[4 * g + e];
          B[gi * d + gj] = y;
          if (gi == gj) dg += y * y; else off += wgt * y * y;
        }
      }
      if (w.P != w.Q && gj < d) {                  // the mirrored tile: four consecutive entries of row gj
        float* row = B + gj * d + gi0;
        if (bvec && gi0 + 3 < d) {
          *reinterpret_cast<float4*>(row) = float4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gi0 + e < d) row[e] = acc[4 * g + e];
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o, 64);
      dg += __shfl_xor(dg, o, 64);
    }
    if ((threadIdx.x & 63) == 0) {
      red[2 * (threadIdx.x >> 6)] = off;
      red[2 * (threadIdx.x >> 6) + 1] = dg;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float so = 0.0f, sd = 0.0f;
#pragma unroll
      for (int q = 0; q < kJacThreads / 64; ++q) {
        so += red[2 * q];
        sd += red[2 * q + 1];
      }
      a.partials[2 * (J.part + it)] = so;
      a.partials[2 * (J.part + it) + 1] = sd;
    }
  }
}

// After a sweep: converged when ||off(B)||_F <= tol ||diag(B)||_F (or B = 0).
__global__ __launch_bounds__(kJacThreads) void jacobi_check_kernel(JacArgs a) {
  __shared__ float red[2 * (kJacThreads / 64)];
  const JacJob J = a.jobs[blockIdx.x];
  if (a.flags[J.flag] != 0) return;
  float off = 0.0f, dg = 0.0f;
  for (int t = threadIdx.x; t < J.btiles; t += kJacThreads) {
    off += a.partials[2 * (J.part + t)];
    dg += a.partials[2 * (J.part + t) + 1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    off += __shfl_xor(off, o, 64);
    dg += __shfl_xor(dg, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = off;
    red[2 * (threadIdx.x >> 6) + 1] = dg;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float so = 0.0f, sd = 0.0f;
#pragma unroll
    for (int w = 0; w < kJacThreads / 64; ++w) {
      so += red[2 * w];
      sd += red[2 * w + 1];
    }
    a.flags[J.flag] = (so <= J.tol * J.tol * sd) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Nystrom low-rank factors (ThinJob, NysOrthJob, NysSmallJob, NysElemJob)
// ---------------------------------------------------------------------------
// Thin fp32 products (ThinJob): kThinTile rows of op(A) per block, K in
// stages of kThinK through LDS, the next stage's global loads in registers
// during the current stage's matrix-core products.  Each of the four waves
// owns 32 rows of the block and runs v_mfma_f32_32x32x2_f32 per 32-column
// block of C (fp32 operands, fp32 accumulation: the plain fp32 products,
// at twice the rate of the unpacked fp32 FMA).  op(A) and B are held in LDS
// with k contiguous per row (rows of op(A), columns of B), LK floats per
// row, and the 4-wide k groups of row i XOR-swizzled by i / 8: the 16-byte
// fragment reads are then free of bank conflicts and the transposing
// stores two-way at most.  An MFMA's two k slots take, for the lanes of
// half h, k = 8 p + 4 h + e of group p and element e, the same map on both
// operands, so each 16-byte read feeds four MFMAs.
constexpr int kThinLK = 40;
__device__ __forceinline__ int thin_at(int i, int k) {
  return i * kThinLK + ((((k >> 2) ^ (i >> 3)) & 7) << 2) + (k & 3);
}

__device__ __forceinline__ float4 quad_any(const char* p, size_t o, int fmt) {
  return fmt == GF_F32 ? grad_quad<GF_F32>(p, o) : fmt == GF_BF16 ? grad_quad<GF_BF16>(p, o) : grad_quad<GF_F16>(p, o);
}
__device__ __forceinline__ float& f4_at(float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// CBM: the most 32-column blocks of C a job of the launch has (1, 2 or 4);
// the narrower forms hold fewer accumulators and less of B's stage, so more
// blocks fit on a CU.  WU: the weight-update form (every job wupd, R <= 32).
// The weight-update form is held to four waves per SIMD (128 registers, no
// spills): its blocks are short and mostly stream W and X, so a fourth block
// per CU keeps more of that stream in flight than the three that its
// unconstrained allocation (132 registers) allows.
template <int TA, bool MOM, int CBM, bool WU>
__global__ __launch_bounds__(256, WU ? 4 : 1) void thin_kernel(ThinArgs a) {
  constexpr int TM = kThinTile, KC = kThinK, LK = kThinLK;
  static_assert(TM == 128 && KC == 32 && kThinMaxR == 128, "the load and fragment maps below assume these sizes");
  static_assert(!MOM || TA == 0, "the momentum operand is row-major");
  static_assert(CBM == 1 || CBM == 2 || CBM == 4, "one, two or four column blocks");
  static_assert(!WU || (TA == 0 && !MOM && CBM == 1), "the weight update is a row-major product of 32 columns");
  __shared__ __attribute__((aligned(16))) float As[TM * LK];
  __shared__ __attribute__((aligned(16))) float Bs[32 * CBM * LK];
  const int gb = blockIdx.x;
  const ThinJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  const int i0 = (gb - J.blk_begin) * TM;
  const char* A = resolve(J.A, a.ws, a.user);
  const float* B = reinterpret_cast<const float*>(resolve(J.B, a.ws, a.user));
  float* C = reinterpret_cast<float*>(resolve(J.C, a.ws, a.user));
  float* Mp = nullptr;
  float* Np = nullptr;
  if constexpr (MOM) {
    Mp = reinterpret_cast<float*>(resolve(J.M, a.ws, a.user));
    Np = reinterpret_cast<float*>(resolve(J.Nout, a.ws, a.user));
  }
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hl = lane >> 5, ln = lane & 31;
  const int CB = min((J.R + 31) >> 5, CBM);
  const uintptr_t amask = J.a_fmt == GF_F32 ? 15 : 7;
  bool avec = (J.lda & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & amask) == 0;
  if constexpr (MOM)
    avec = avec && (J.ldn & 3) == 0 && ((reinterpret_cast<uintptr_t>(Mp) | reinterpret_cast<uintptr_t>(Np)) & 15) == 0;
  const bool bvec = (J.ldb & 3) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  const bool cvec = (J.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
  const float b1 = a.beta1, b1c = 1.0f - a.beta1, st = a.s_t;

  float4 ra[4], rb[CBM];
  float4 rm[MOM ? 4 : 1];
  floatx16 acc[CBM];
#pragma unroll
  for (int c = 0; c < CBM; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

  // the weight update: the block's W and X quads (128 rows x 32 columns,
  // thread quads u = t + 256 v: row u / 8, columns 4 (u % 8) .. + 3) are
  // loaded before the product, so their latency passes during it
  float4 uw[WU ? 4 : 1], ux[WU ? 4 : 1];
  const float* X = nullptr;
  bool wvec = false;
  if constexpr (WU) {
    X = reinterpret_cast<const float*>(resolve(J.aux, a.ws, a.user));
    wvec = (J.ldc & 3) == 0 && ((reinterpret_cast<uintptr_t>(C) | reinterpret_cast<uintptr_t>(X)) & 15) == 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int u = t + 256 * v, gi = i0 + (u >> 3), gj = (u & 7) * 4;
      uw[v] = ux[v] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      if (gi < J.Mo) {
        const size_t o = static_cast<size_t>(gi) * J.ldc + gj;
        if (wvec && gj + 3 < J.R) {
          uw[v] = *reinterpret_cast<const float4*>(C + o);
          ux[v] = *reinterpret_cast<const float4*>(X + o);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gj + e < J.R) {
              f4_at(uw[v], e) = C[o + e];
              f4_at(ux[v], e) = X[o + e];
            }
        }
      }
    }
  }

  // stage k0 into registers: op(A) as 1024 quads (TA 0: 128 rows x 8 quads
  // along k; TA 1: 32 k-rows x 32 quads along i), B as 32 k-rows x 32 quads.
  // In the momentum form ra takes G and rm takes M; the momentum update and
  // its stores wait for lstore, so that these loads stay in flight during
  // the current stage's products.
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = t + 256 * j;
      float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
      float4 m = float4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (TA == 0) {
        const int row = q >> 3, gk = k0 + (q & 7) * 4, gi = i0 + row;
        if (gi < J.Mo && gk < J.K) {
          const size_t o = static_cast<size_t>(gi) * J.lda + gk;
          if (avec && gk + 3 < J.K) {
            v = quad_any(A, o, J.a_fmt);
            if constexpr (MOM) m = *reinterpret_cast<const float4*>(Mp + o);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (gk + e >= J.K) break;
              f4_at(v, e) = grad_elem(A, o + e, J.a_fmt);
              if constexpr (MOM) f4_at(m, e) = Mp[o + e];
            }
          }
        }
      } else {
        const int gk = k0 + (q >> 5), gi = i0 + (q & 31) * 4;
        if (gk < J.K && gi < J.Mo) {
          const size_t o = static_cast<size_t>(gk) * J.lda + gi;
          if (avec && gi + 3 < J.Mo) {
            v = quad_any(A, o, J.a_fmt);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gi + e < J.Mo) f4_at(v, e) = grad_elem(A, o + e, J.a_fmt);
          }
        }
      }
      ra[j] = v;
      if constexpr (MOM) rm[j] = m;
    }
    // B: 32 k-rows x 8 CBM quads, CBM per thread
#pragma unroll
    for (int j = 0; j < CBM; ++j) {
      const int q = t + 256 * j;
      float4 w = float4{0.0f, 0.0f, 0.0f, 0.0f};
      const int bk = k0 + q / (8 * CBM), bc = (q % (8 * CBM)) * 4;
      if (bk < J.K && bc < J.R) {
        const float* bp = B + static_cast<size_t>(bk) * J.ldb + bc;
        if (bvec && bc + 3 < J.R) {
          w = *reinterpret_cast<const float4*>(bp);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (bc + e < J.R) f4_at(w, e) = bp[e];
        }
      }
      rb[j] = w;
    }
  };
  // the momentum form: M' = beta1 M + (1 - beta1) G and N = s_t (beta1 M' +
  // (1 - beta1) G) for the staged quads of stage k0, M' and N stored, N
  // left in ra (zeros outside the matrix stay zeros)
  auto momentum = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = t + 256 * j;
      const int row = q >> 3, gk = k0 + (q & 7) * 4, gi = i0 + row;
      float4 mn, nv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f4_at(mn, e) = b1 * f4_at(rm[j], e) + b1c * f4_at(ra[j], e);
        f4_at(nv, e) = st * (b1 * f4_at(mn, e) + b1c * f4_at(ra[j], e));
      }
      if (gi < J.Mo && gk < J.K) {
        const size_t o = static_cast<size_t>(gi) * J.lda + gk;
        const size_t on = static_cast<size_t>(gi) * J.ldn + gk;
        if (avec && gk + 3 < J.K) {
          *reinterpret_cast<float4*>(Mp + o) = mn;
          *reinterpret_cast<float4*>(Np + on) = nv;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (gk + e >= J.K) break;
            Mp[o + e] = f4_at(mn, e);
            Np[on + e] = f4_at(nv, e);
          }
        }
      }
      ra[j] = nv;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = t + 256 * j;
      if constexpr (TA == 0) {
        const int row = q >> 3, kq = (q & 7) * 4;
        *reinterpret_cast<float4*>(&As[thin_at(row, kq)]) = ra[j];
      } else {
        const int kr = q >> 5, c4 = (q & 31) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) As[thin_at(c4 + e, kr)] = f4_at(ra[j], e);
      }
    }
    // B's columns as rows
#pragma unroll
    for (int j = 0; j < CBM; ++j) {
      const int q = t + 256 * j;
      const int bk = q / (8 * CBM), bc = (q % (8 * CBM)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[thin_at(bc + e, bk)] = f4_at(rb[j], e);
    }
  };

  const int nk = (J.K + KC - 1) / KC;
  const int arow = 32 * wave + ln;
  gload(0);
  for (int sidx = 0; sidx < nk; ++sidx) {
    if constexpr (MOM) momentum(sidx * KC);
    __syncthreads();                  // the previous stage's reads are done
    lstore();
    __syncthreads();
    if (sidx + 1 < nk) gload((sidx + 1) * KC);
#pragma unroll
    for (int p = 0; p < KC / 8; ++p) {
      const int kg = 8 * p + 4 * hl;
      const float4 av = *reinterpret_cast<const float4*>(&As[thin_at(arow, kg)]);
#pragma unroll
      for (int c = 0; c < CBM; ++c) {
        if (c >= CB) break;
        const float4 bv = *reinterpret_cast<const float4*>(&Bs[thin_at(32 * c + ln, kg)]);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc[c], 0, 0, 0);
      }
    }
  }

  // lane (h, n) holds column 32 c + n of C and, for element r of the
  // accumulator, row 32 wave + 8 (r / 4) + 4 h + r % 4 of the block
  const float alpha0 = J.alpha * (J.alpha_slot >= 0 ? a.scal[J.alpha_slot] : 1.0f);
  const float* rsc = J.rowscale.kind != REF_NONE ? reinterpret_cast<const float*>(resolve(J.rowscale, a.ws, a.user)) : nullptr;
  const float beta = J.beta;
  if constexpr (WU) {
    // W <- decay W - lr c0 (alpha acc + X), X the unpreconditioned part of
    // the update (W's layout, stride ldc).  The accumulators pass through
    // LDS (As is free after the last stage), so that each thread updates its
    // four prefetched 16-byte row quads.
    constexpr int LS = 36;                 // staging row stride (floats)
    static_assert(TM * LS <= TM * LK, "the staging fits As");
    const float sc = -(a.lr * J.c0);
    __syncthreads();                       // the products no longer read As
#pragma unroll
    for (int r = 0; r < 16; ++r) As[(32 * wave + 8 * (r >> 2) + 4 * hl + (r & 3)) * LS + ln] = acc[0][r];
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int u = t + 256 * v, row = u >> 3, gj = (u & 7) * 4, gi = i0 + row;
      if (gi >= J.Mo) continue;
      float4 pv = *reinterpret_cast<const float4*>(&As[row * LS + gj]);
      float4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        f4_at(o4, e) = __builtin_fmaf(a.decay, f4_at(uw[v], e), sc * __builtin_fmaf(alpha0, f4_at(pv, e), f4_at(ux[v], e)));
      const size_t o = static_cast<size_t>(gi) * J.ldc + gj;
      if (wvec && gj + 3 < J.R) {
        *reinterpret_cast<float4*>(C + o) = o4;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gj + e < J.R) C[o + e] = f4_at(o4, e);
      }
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < CBM; ++c) {
    if (c >= CB) break;
    const int col = 32 * c + ln;
    if (col >= J.R) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = i0 + 32 * wave + 8 * g + 4 * hl;
      if (J.ot == 0) {
        // lanes n = 0..31 write 32 consecutive columns of one row
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = r0 + e;
          if (gi >= J.Mo) break;
          const float alpha = rsc != nullptr ? alpha0 * rsc[gi] : alpha0;
          float* cp = C + static_cast<size_t>(gi) * J.ldc + col;
          const float v = alpha * acc[c][4 * g + e];
          *cp = beta != 0.0f ? __builtin_fmaf(beta, *cp, v) : v;
        }
      } else {
        // the transposed output: the lane's four rows are consecutive
        float* cp = C + static_cast<size_t>(col) * J.ldc + r0;
        if (cvec && r0 + 3 < J.Mo) {
          float4 o = float4{alpha0 * acc[c][4 * g], alpha0 * acc[c][4 * g + 1], alpha0 * acc[c][4 * g + 2],
                            alpha0 * acc[c][4 * g + 3]};
          if (beta != 0.0f) {
            const float4 old = *reinterpret_cast<const float4*>(cp);
            o.x = __builtin_fmaf(beta, old.x, o.x); o.y = __builtin_fmaf(beta, old.y, o.y);
            o.z = __builtin_fmaf(beta, old.z, o.z); o.w = __builtin_fmaf(beta, old.w, o.w);
          }
          *reinterpret_cast<float4*>(cp) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (r0 + e < J.Mo) {
              const float v = alpha0 * acc[c][4 * g + e];
              cp[e] = beta != 0.0f ? __builtin_fmaf(beta, cp[e], v) : v;
            }
        }
      }
    }
  }
}

// threads of a Gram-Schmidt block (a sketch is one block).  1024 threads
// measured slower than 256 (17.8 against 13.7 ms per launch on the
// 1.2B-class workload): the wider block reductions and barriers of every
// column cost more than the shorter row walks save.  The row walks are
// unrolled by two, so a thread has two rows' loads in flight (by four
// measured the same).
constexpr int kOrthThreads = 256;

// Block sum of one float (all threads get the result).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Thin QR's Q of Y (d x k) in place: column by column, classical
// Gram-Schmidt against the finished columns, repeated while a pass removes
// more than half the remaining norm (at most three passes), then
// normalised.  A column that keeps less than 1e-6 of its norm (dependent,
// or zero) is replaced by a column of the Gaussian fallback and
// orthogonalised again.  One workgroup per job; the projections of a pass
// are one wave per finished column, lanes over the rows.
__global__ __launch_bounds__(kOrthThreads) void nys_orth_kernel(NysOrthArgs a) {
  constexpr int NWV = kOrthThreads / 64;
  __shared__ float coef[kNysMaxK];
  __shared__ float part[NWV][16];
  __shared__ float red[NWV];
  // the block's sum of one float, fixed order (all threads get it)
  auto bsum = [&](float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) t += red[w];
    return t;
  };
  const NysOrthJob J = a.jobs[blockIdx.x];
  float* Y = reinterpret_cast<float*>(resolve(J.Y, a.ws, a.user));
  const float* F = reinterpret_cast<const float*>(resolve(J.fb, a.ws, a.user));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto col_norm2 = [&](int j) {
    float s = 0.0f;
#pragma unroll 4
    for (int r = threadIdx.x; r < J.d; r += kOrthThreads) {
      const float v = Y[static_cast<size_t>(r) * J.ld + j];
      s += v * v;
    }
    return bsum(s);
  };
  auto project_out = [&](int j) {       // y_j <- y_j - Q_{<j} (Q_{<j}^T y_j)
    // the coefficients 16 at a time: every thread walks its rows, reading
    // each row's 16 entries as one contiguous run, then a fixed-order
    // reduction over the wave and the waves of the block
    for (int c0 = 0; c0 < j; c0 += 16) {
      float s[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) s[c] = 0.0f;
#pragma unroll 2
      for (int r = threadIdx.x; r < J.d; r += kOrthThreads) {
        const float* row = Y + static_cast<size_t>(r) * J.ld;
        const float yj = row[j];
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (c0 + c < j) s[c] = __builtin_fmaf(row[c0 + c], yj, s[c]);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s[c] += __shfl_xor(s[c], o, 64);
      }
      if (lane == 0) {
#pragma unroll
        for (int c = 0; c < 16; ++c) part[wave][c] = s[c];
      }
      __syncthreads();
      if (threadIdx.x < 16 && c0 + static_cast<int>(threadIdx.x) < j) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) t += part[w][threadIdx.x];
        coef[c0 + threadIdx.x] = t;
      }
      __syncthreads();
    }
#pragma unroll 2
    for (int r = threadIdx.x; r < J.d; r += kOrthThreads) {
      float* row = Y + static_cast<size_t>(r) * J.ld;
      float v = row[j];
#pragma unroll 8
      for (int c = 0; c < j; ++c) v -= row[c] * coef[c];
      row[j] = v;
    }
    __syncthreads();
  };
  for (int j = 0; j < J.k; ++j) {
    for (int attempt = 0; attempt < 2; ++attempt) {
      const float n0 = col_norm2(j);
      float prev = n0, now = n0;
      for (int pass = 0; pass < 3 && j > 0; ++pass) {
        project_out(j);
        now = col_norm2(j);
        if (!(now < 0.25f * prev)) break;
        prev = now;
      }
      if (now > 1e-12f * n0 && now > 0.0f) {
        const float inv = 1.0f / sqrtf(now);
        for (int r = threadIdx.x; r < J.d; r += kOrthThreads) Y[static_cast<size_t>(r) * J.ld + j] *= inv;
        __syncthreads();
        break;
      }
      // dependent: take the fallback column and try once more
      const int fc = (j + J.fb_shift) % J.k;
      for (int r = threadIdx.x; r < J.d; r += kOrthThreads)
        Y[static_cast<size_t>(r) * J.ld + j] = attempt == 0 ? F[static_cast<size_t>(r) * J.ldf + fc] : (r == j ? 1.0f : 0.0f);
      __syncthreads();
    }
  }
}

// Cyclic Jacobi eigendecomposition of the symmetric n x n matrix A (LDS,
// row stride n + 1) accumulating V; round-robin order, rotations in fp64.
__device__ void nys_jacobi(float* A, float* V, int n, int ld) {
  __shared__ float rc[kNysMaxK / 2], rs[kNysMaxK / 2];
  __shared__ int ru[kNysMaxK / 2], rw[kNysMaxK / 2], rot_any;
  __shared__ float fro_sh;
  const int np = n + (n & 1);                    // an odd size pairs one index with a dummy
  float s2 = 0.0f;
  for (int e = threadIdx.x; e < n * n; e += 256) {
    const float x = A[(e / n) * ld + e % n];
    s2 += x * x;
  }
  __shared__ float red[4];
  s2 = block_sum256(s2, red);
  const float floor_abs = 1e-9f * sqrtf(s2);
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (threadIdx.x == 0) rot_any = 0;
    __syncthreads();
    for (int rd = 0; rd < np - 1; ++rd) {
      if (threadIdx.x < np / 2) {
        const int t = threadIdx.x;
        const int pa = t == 0 ? 0 : ((t - 1 + rd) % (np - 1)) + 1;
        const int tb = np - 1 - t;
        const int pb = tb == 0 ? 0 : ((tb - 1 + rd) % (np - 1)) + 1;
        const int u = min(pa, pb), w = max(pa, pb);
        float c = 1.0f, sn = 0.0f;
        if (w < n) {
          const float auu = A[u * ld + u], aww = A[w * ld + w], auw = A[u * ld + w];
          if (fabsf(auw) > floor_abs && fabsf(auw) > 1e-7f * sqrtf(fabsf(auu * aww))) {
            const double tau = (static_cast<double>(aww) - auu) / (2.0 * auw);
            const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
            const double cd = 1.0 / sqrt(1.0 + tt * tt);
            c = static_cast<float>(cd);
            sn = static_cast<float>(tt * cd);
            rot_any = 1;
          }
        }
        ru[t] = u; rw[t] = w; rc[t] = c; rs[t] = sn;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < (np / 2) * n; e += 256) {   // rows
        const int t = e / n, col = e % n;
        if (rs[t] != 0.0f) {
          const int u = ru[t], w = rw[t];
          const float xu = A[u * ld + col], xw = A[w * ld + col];
          A[u * ld + col] = rc[t] * xu - rs[t] * xw;
          A[w * ld + col] = rs[t] * xu + rc[t] * xw;
        }
      }
      __syncthreads();
      for (int e = threadIdx.x; e < (np / 2) * n; e += 256) {   // columns of A and V
        const int t = e / n, row = e % n;
        if (rs[t] != 0.0f) {
          const int u = ru[t], w = rw[t];
          const float xu = A[row * ld + u], xw = A[row * ld + w];
          A[row * ld + u] = rc[t] * xu - rs[t] * xw;
          A[row * ld + w] = rs[t] * xu + rc[t] * xw;
          const float vu = V[row * ld + u], vw = V[row * ld + w];
          V[row * ld + u] = rc[t] * vu - rs[t] * vw;
          V[row * ld + w] = rs[t] * vu + rc[t] * vw;
        }
      }
      __syncthreads();
    }
    const bool more = rot_any != 0;
    __syncthreads();
    if (!more) break;
  }
  (void)fro_sh;
}

// The k x k ends of a refresh, in two phases around the products that form
// F = Y_nu R^-1 and its Gram:
//   phase 1, from G_Y = Y^T Y and C = Omega^T Y (Omega orthonormal, so
//   B = Omega^T Y_nu = C + nu I for Y_nu = Y + nu Omega): nu = the fp32
//   spacing at ||Y||_2 (power iteration on G_Y); B = sym(C) + nu I = R^T R
//   (Cholesky, fp64, a pivot that rounding took below nu held at nu); R^-1
//   (fp64), written over C as fp32.  The products then form F = Y R^-1 +
//   nu Omega R^-1 and F^T F, F^T U_prev.
//   phase 2: the eigenpairs (S, V) of F^T F by Jacobi (fp32), in decreasing
//   order; U = F V_r S_r^-1/2 = F K, each column's sign set so that
//   u_i^T u_prev,i >= 0 (= K_i^T (F^T u_prev,i)); Lambda = max(0, S_r - nu).
// A zero sketch (phase 1 finds G_Y = 0) records nu = 0, nu_u = 1 and R^-1 = I,
// so that F = Omega; phase 2 then keeps K = the first r columns of I and
// Lambda = 0 (U = Omega's first columns).
__global__ __launch_bounds__(256) void nys_small_kernel(NysSmallArgs a) {
  constexpr int LD = kNysMaxK + 1;
  __shared__ float A[kNysMaxK * LD];
  __shared__ float V[kNysMaxK * LD];
  __shared__ float S[kNysMaxK];
  __shared__ int order[kNysMaxK];
  __shared__ float red[4];
  __shared__ float vec[kNysMaxK], vec2[kNysMaxK];
  const NysSmallJob J = a.jobs[blockIdx.x];
  const int k = J.k, r = J.r;
  float* Gy = reinterpret_cast<float*>(resolve(J.gram, a.ws, a.user));
  float* Cm = reinterpret_cast<float*>(resolve(J.cmat, a.ws, a.user));
  if (a.phase == 1) {
    double* R = reinterpret_cast<double*>(resolve(J.scratch, a.ws, a.user));   // R (k x k)
    double* X = R + static_cast<size_t>(k) * k;                               // R^-1
    float tr = 0.0f;
    for (int i = threadIdx.x; i < k; i += 256) tr += Gy[i * k + i];
    tr = block_sum256(tr, red);
    if (!(tr > 0.0f)) {                            // a zero sketch: nothing to factor
      for (int e = threadIdx.x; e < k * k; e += 256) Cm[e] = (e / k == e % k) ? 1.0f : 0.0f;
      if (threadIdx.x == 0) {
        a.scal[J.nu_slot] = 0.0f;
        a.scal[J.nuu_slot] = 1.0f;
      }
      return;
    }
    for (int i = threadIdx.x; i < k; i += 256) vec[i] = 1.0f;
    __syncthreads();
    float lmax = 0.0f;
    for (int it = 0; it < 60; ++it) {
      for (int i = threadIdx.x; i < k; i += 256) {
        float s = 0.0f;
        for (int j = 0; j < k; ++j) s += Gy[i * k + j] * vec[j];
        vec2[i] = s;
      }
      __syncthreads();
      float n2 = 0.0f, dotv = 0.0f, vn = 0.0f;
      for (int i = threadIdx.x; i < k; i += 256) {
        n2 += vec2[i] * vec2[i];
        dotv += vec2[i] * vec[i];
        vn += vec[i] * vec[i];
      }
      n2 = block_sum256(n2, red);
      dotv = block_sum256(dotv, red);
      vn = block_sum256(vn, red);
      lmax = dotv / vn;                            // Rayleigh quotient
      const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
      for (int i = threadIdx.x; i < k; i += 256) vec[i] = vec2[i] * inv;
      __syncthreads();
    }
    int e2;
    (void)frexpf(sqrtf(fmaxf(lmax, 0.0f)), &e2);   // ||Y||_2 = f 2^e2, f in [0.5, 1)
    const float nu = ldexpf(1.0f, e2 - 1 - 23);
    for (int e = threadIdx.x; e < k * k; e += 256) {
      const int i = e / k, j = e % k;
      R[e] = 0.5 * (static_cast<double>(Cm[i * k + j]) + Cm[j * k + i]) + (i == j ? static_cast<double>(nu) : 0.0);
    }
    __syncthreads();
    for (int j = 0; j < k; ++j) {                  // upper R, R^T R = B, in place
      if (threadIdx.x == 0) R[j * k + j] = sqrt(fmax(R[j * k + j], static_cast<double>(nu)));
      __syncthreads();
      const double djj = R[j * k + j];
      for (int l = j + 1 + threadIdx.x; l < k; l += 256) R[j * k + l] /= djj;
      __syncthreads();
      for (int e = threadIdx.x; e < (k - j - 1) * (k - j - 1); e += 256) {
        const int i = j + 1 + e / (k - j - 1), l = j + 1 + e % (k - j - 1);
        if (l >= i) R[i * k + l] -= R[j * k + i] * R[j * k + l];
      }
      __syncthreads();
    }
    for (int j = threadIdx.x; j < k; j += 256) {   // R^-1 by back substitution, a column per thread
      for (int i = j; i >= 0; --i) {
        double s = (i == j) ? 1.0 : 0.0;
        for (int l = i + 1; l <= j; ++l) s -= R[i * k + l] * X[l * k + j];
        X[i * k + j] = s / R[i * k + i];
      }
      for (int i = j + 1; i < k; ++i) X[i * k + j] = 0.0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < k * k; e += 256) Cm[e] = static_cast<float>(X[e]);
    if (threadIdx.x == 0) {
      a.scal[J.nu_slot] = nu;
      a.scal[J.nuu_slot] = nu;
    }
    return;
  }
  // ---- phase 2
  const float* Fu = reinterpret_cast<const float*>(resolve(J.ftu, a.ws, a.user));
  float* K = reinterpret_cast<float*>(resolve(J.kout, a.ws, a.user));
  float* lam = reinterpret_cast<float*>(resolve(J.lam, a.ws, a.user));
  const float nu = a.scal[J.nu_slot];
  if (nu == 0.0f) {                                // the zero sketch of phase 1: F = Omega
    for (int e = threadIdx.x; e < k * r; e += 256) K[e] = (e / r == e % r) ? 1.0f : 0.0f;
    for (int i = threadIdx.x; i < r; i += 256) lam[i] = 0.0f;
    return;
  }
  for (int e = threadIdx.x; e < k * k; e += 256) {
    const int i = e / k, j = e % k;
    A[i * LD + j] = 0.5f * (Gy[i * k + j] + Gy[j * k + i]);
    V[i * LD + j] = i == j ? 1.0f : 0.0f;
  }
  __syncthreads();
  nys_jacobi(A, V, k, LD);
  for (int i = threadIdx.x; i < k; i += 256) S[i] = A[i * LD + i];
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 256) {     // decreasing order (ties by index)
    int rank = 0;
    for (int j = 0; j < k; ++j) rank += (S[j] > S[i]) || (S[j] == S[i] && j < i);
    order[rank] = i;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < k * r; e += 256) {
    const int row = e / r, i = e % r;
    const int c = order[i];
    const float sv = S[c];
    K[e] = sv > 0.0f ? V[row * LD + c] / sqrtf(sv) : 0.0f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < r; i += 256) {
    float d = 0.0f;
    for (int row = 0; row < k; ++row) d += K[row * r + i] * Fu[row * r + i];
    const float sgn = d < 0.0f ? -1.0f : 1.0f;
    for (int row = 0; row < k; ++row) K[row * r + i] *= sgn;
    lam[i] = fmaxf(0.0f, S[order[i]] - nu);
  }
}

// Element-wise jobs (NysElemJob): each job has its own run of blocks, and
// its threads stride over the job's rows x cols elements.
__global__ __launch_bounds__(256) void nys_elem_kernel(NysElemArgs a) {
  const int gb = blockIdx.x;
  const NysElemJob J = a.jobs[find_job(a.jobs, a.n_jobs, gb)];
  const size_t total = static_cast<size_t>(J.rows) * J.cols;
  const size_t stride = static_cast<size_t>(J.blocks) * 256;
  float* dst = reinterpret_cast<float*>(resolve(J.dst, a.ws, a.user));
  const char* src = resolve(J.src, a.ws, a.user);
  const char* src2 = J.src2.kind != REF_NONE ? resolve(J.src2, a.ws, a.user) : nullptr;
  const float* lam = J.lam.kind != REF_NONE ? reinterpret_cast<const float*>(resolve(J.lam, a.ws, a.user)) : nullptr;
  float lam_r = 0.0f;
  if (J.kind == NE_SCALE) lam_r = lam[J.cols - 1];
  for (size_t e = static_cast<size_t>(gb - J.blk_begin) * 256 + threadIdx.x; e < total; e += stride) {
    const int r = static_cast<int>(e / J.cols), c = static_cast<int>(e % J.cols);
    const size_t od = J.trans ? static_cast<size_t>(c) * J.ld_dst + r : static_cast<size_t>(r) * J.ld_dst + c;
    if (J.kind == NE_GATHER) {
      dst[od] = c < J.cols1 ? reinterpret_cast<const float*>(src)[static_cast<size_t>(r) * J.ld_src + c]
                            : reinterpret_cast<const float*>(src2)[static_cast<size_t>(r) * J.ld_src2 + (c - J.cols1)];
    } else {   // NE_SCALE
      const float e_c = sqrtf((lam_r + a.mu) / (lam[c] + a.mu)) - 1.0f;
      dst[od] = reinterpret_cast<const float*>(src)[static_cast<size_t>(r) * J.ld_src + c] * e_c;
    }
  }
}

// Clears the converged flags of every job (start of a refresh).
__global__ void jacobi_reset_kernel(JacArgs a) {
  for (int j = threadIdx.x; j < a.n_jobs; j += blockDim.x) a.flags[a.jobs[j].flag] = 0;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <class C>
hipError_t launch_gemm_cfg(const GemmArgs& a, int n_tiles, int epi, hipStream_t s) {
  const dim3 grid(n_tiles), block(C::THREADS);
  // fp16-output kinds come in two forms: fp16 values only, or the split
  // layout's hi and lo halves (write_lo); the fp32 kinds ignore write_lo
  const bool wl = a.write_lo != 0;
#define OKLS_GEMM(E, W) hipLaunchKernelGGL((gemm_nt_kernel<C, E, W>), grid, block, 0, s, a)
  switch (epi) {
    case EPI_STORE32: OKLS_GEMM(EPI_STORE32, false); break;
    case EPI_SYRK: OKLS_GEMM(EPI_SYRK, false); break;
    case EPI_UPDATE: OKLS_GEMM(EPI_UPDATE, false); break;
    case EPI_NS_T: if (wl) OKLS_GEMM(EPI_NS_T, true); else OKLS_GEMM(EPI_NS_T, false); break;
    case EPI_NS_T_RES: if (wl) OKLS_GEMM(EPI_NS_T_RES, true); else OKLS_GEMM(EPI_NS_T_RES, false); break;
    case EPI_NS_Y1: if (wl) OKLS_GEMM(EPI_NS_Y1, true); else OKLS_GEMM(EPI_NS_Y1, false); break;
    case EPI_STORE16: if (wl) OKLS_GEMM(EPI_STORE16, true); else OKLS_GEMM(EPI_STORE16, false); break;
    case EPI_NS_FINAL: if (wl) OKLS_GEMM(EPI_NS_FINAL, true); else OKLS_GEMM(EPI_NS_FINAL, false); break;
    case EPI_POLAR: if (wl) OKLS_GEMM(EPI_POLAR, true); else OKLS_GEMM(EPI_POLAR, false); break;
    case EPI_POLAR_UPDATE: OKLS_GEMM(EPI_POLAR_UPDATE, false); break;
    default: return hipErrorInvalidValue;
  }
#undef OKLS_GEMM
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int n_tiles, int tile, int epi, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (tile == 256) return launch_gemm_cfg<TileBig8>(a, n_tiles, epi, s);
  if (tile == 128) return launch_gemm_cfg<TileSmall>(a, n_tiles, epi, s);
  return hipErrorInvalidValue;
}

hipError_t launch_stats(const StatArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(stats_kernel, dim3(n_blocks), dim3(kStatThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cast(const CastArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel, dim3(n_blocks), dim3(kCastThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch: the workspace of handles made by okls_init_static.  Each
// device holds its own copy for the life of the process; the host code uses
// only the address hipGetSymbolAddress returns for the current device (the
// array's name on the host is a stand-in, not a device address).
// ---------------------------------------------------------------------------
__device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_sym(const SymArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sym_kernel, dim3(n_blocks), dim3(kSymThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adam(const AdamArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  adam_kernel<<<dim3(n_blocks), dim3(kAdamThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_jacobi(const JacArgs& a, int kind, int n_blocks, hipStream_t s) {
  if (kind == JAC_RESET) {
    jacobi_reset_kernel<<<dim3(1), dim3(256), 0, s>>>(a);
    return hipGetLastError();
  }
  if (n_blocks <= 0) return hipSuccess;
  if (kind == JAC_SOLVE) jacobi_solve_kernel<<<dim3(n_blocks), dim3(kJacThreads), 0, s>>>(a);
  else if (kind == JAC_APPLY) jacobi_apply_kernel<<<dim3(n_blocks), dim3(kJacThreads), 0, s>>>(a);
  else jacobi_check_kernel<<<dim3(n_blocks), dim3(kJacThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <int CBM>
void launch_thin_cbm(const ThinArgs& a, int ta, int mom, int n_blocks, hipStream_t s) {
  const dim3 g(n_blocks), b(256);
  if (mom) thin_kernel<0, true, CBM, false><<<g, b, 0, s>>>(a);
  else if (ta) thin_kernel<1, false, CBM, false><<<g, b, 0, s>>>(a);
  else thin_kernel<0, false, CBM, false><<<g, b, 0, s>>>(a);
}

hipError_t launch_thin(const ThinArgs& a, int ta, int mom, int cbm, int wupd, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  if (mom && ta) return hipErrorInvalidValue;
  if (wupd) {
    if (ta || mom || cbm != 1) return hipErrorInvalidValue;
    thin_kernel<0, false, 1, true><<<dim3(n_blocks), dim3(256), 0, s>>>(a);
  } else if (cbm == 1) launch_thin_cbm<1>(a, ta, mom, n_blocks, s);
  else if (cbm == 2) launch_thin_cbm<2>(a, ta, mom, n_blocks, s);
  else if (cbm == 4) launch_thin_cbm<4>(a, ta, mom, n_blocks, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_nys_orth(const NysOrthArgs& a, hipStream_t s) {
  if (a.n_jobs <= 0) return hipSuccess;
  nys_orth_kernel<<<dim3(a.n_jobs), dim3(kOrthThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_nys_small(const NysSmallArgs& a, hipStream_t s) {
  if (a.n_jobs <= 0) return hipSuccess;
  nys_small_kernel<<<dim3(a.n_jobs), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_nys_elem(const NysElemArgs& a, int n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  nys_elem_kernel<<<dim3(n_blocks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_init_state(const InitArgs& a, int n_jobs, hipStream_t s) {
  if (n_jobs <= 0) return hipSuccess;
  hipLaunchKernelGGL(init_state_kernel, dim3(1024, n_jobs), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_check_finite(const InitArgs& a, int n_jobs, int* flag_dev, hipStream_t s) {
  if (n_jobs <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, s, flag_dev);
  hipLaunchKernelGGL(finite_kernel, dim3(1024, n_jobs), dim3(256), 0, s, a, flag_dev);
  return hipGetLastError();
}

}  // namespace okls

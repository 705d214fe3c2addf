// Shared device/host definitions of the DEX lattice-step library (gfx950).
//
// Storage types: T is either float (fp32 models) or bf16_t (bfloat16 bits in
// an unsigned short). The residual stream is always fp32; GEMM activations,
// weights and KV use T; every accumulation is fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "types.h"

namespace dex {

// k-steps the 8-wave wide GEMM stages in LDS between two barriers (1 or 2).
// Two halve the barriers: 13B-shaped batch 8 layer GEMMs -1.5% time (382.8
// -> 386.6 tokens/s, two passes of 60 rounds each), the other workloads the
// same within noise.
#ifndef DEX_WIDE_KPB
#define DEX_WIDE_KPB 2
#endif
constexpr int kWideKPB = DEX_WIDE_KPB;

typedef unsigned short bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Residual-stream buffers, indexed by a row's hrow: the fp32 residual h, its
// per-16-column sums of squares, and h multiplied elementwise by the RMSNorm
// weight of its next consumer (xn: next QKV or gate/up GEMM; xh: the exit
// head). A normalising GEMM reads xn or xh and scales its outputs by
// rstd = 1/sqrt(mean(h^2) + eps), so RMSNorm costs no pass of its own.
struct GemmArgs {
  GemmGroup g[kMaxGroups];
  int ngroups;
  int K;            // reduction length (multiple of the k-step)
  int N;            // output columns (multiple of 16)
  const RowInfo* rows;
  const void* a;    // EPI_RESID: activations [rows][K] (fp32)
  const float* xin; // normalising epilogues: xn or xh, [*][K]
  float* hidden;    // EPI_RESID: residual [*][N]
  float* ssq;       // [*][d/16]: read by normalising epilogues, written by EPI_RESID
  float* xn;        // EPI_RESID: h * gamma of the next consumer
  float* xh;        // EPI_RESID: h * final-norm weight (groups with xh set); EPI_ADAPT2: h~ * weight
  float* xa;        // EPI_RESID: h * adapter norm weight (groups with anorm set)
  float* ssq_head;  // [*][d/16] sums of squares of the exit head's input (h, or h~ for adapted rows)
  const float* gfinal;
  float eps;
  // EPI_QKV
  ModelDims dims;
  const float* cosT;
  const float* sinT;
  float* qout;      // [rows][nq][hd], pre-scaled by qscale
  bf16_t* kvc;      // committed K/V (tiles of 16-bit planes)
  bf16_t* exb;      // explore-buffer K/V
  int lattice, lam;  // layer slot lam; layer = layer_of(dims, lattice, row's stage, lam)
  float qscale;
  // EPI_SWIGLU
  void* act;        // [rows][N/2] (fp32)
  // EPI_HEAD
  float* out;       // debug logits [seq][N] or null
  int mode;         // 0 greedy, 1 sample
  float tau;
  const float* gumbel;   // [batch][gumbel_rows][N]
  int gumbel_rows;
  float* part;      // [rows][N/16][3] top-2 summaries per 16-column tile
  // split-range wide GEMM: per k range r, scratch rows [r][kSplitRows][N] (fp32)
  float* split;
  int xcd_rows;     // wide GEMM block order: 1 row-shards the first ngroups - ngroups % 8 groups over
                    // the XCDs (see gemm_wide_kernel); 0 puts every group of a column block on one XCD
  // Unsplit wide GEMM, groups that are not row-sharded: runs of consecutive
  // groups that share a weight, run r = groups [run0[r], run0[r + 1]); the
  // blocks of a run are consecutive (column block slowest). nrun = 0: every
  // group of a column block, then the next column block.
  int nrun;
  int run0[kMaxGroups + 1];
};

// Logical block of hardware block b out of nb: the hardware hands blocks to
// the 8 XCDs round-robin, and XCD x gets a contiguous run of logical ids.
__device__ __forceinline__ int xcd_block(int b, int nb) {
  const int x = b & 7, k = b >> 3, q = nb >> 3, rem = nb & 7;
  return x * q + (x < rem ? x : rem) + k;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((unsigned)v) << 16); }
// Two floats to packed bfloat16 (a in the low half), round-to-nearest-even
// (v_cvt_pk_bf16_f32). Every float-to-bf16 rounding of the library goes
// through here, so all kernels round identically.
__device__ __forceinline__ unsigned f2bf2(float a, float b) {
  const f32x2_t f = {a, b};
  const bf16x2_t v = __builtin_convertvector(f, bf16x2_t);
  unsigned u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}
__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)(f2bf2(f, 0.f) & 0xFFFFu); }
template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }
// The (hi, lo) bfloat16 pairs of two values, packed (a in the low halves).
__device__ __forceinline__ void split_bf2(float a, float b, unsigned& hi, unsigned& lo) {
  hi = f2bf2(a, b);
  lo = f2bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Two floats to packed fp16 (a in the low half), round-to-nearest-even, with
// magnitudes above the largest finite fp16 (65504) saturated to it (NaN
// passes through). SAT = false leaves out the saturation where the values are
// known to lie in range (softmax weights in [0, 1]), with the same results.
// Every float-to-fp16 rounding of the library goes through here.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sat_f16(float x) { return x > 65504.f ? 65504.f : (x < -65504.f ? -65504.f : x); }
template <bool SAT = true>
__device__ __forceinline__ unsigned f2h2(float a, float b) {
  const f32x2_t f = SAT ? f32x2_t{sat_f16(a), sat_f16(b)} : f32x2_t{a, b};
  const f16x2_t v = __builtin_convertvector(f, f16x2_t);
  unsigned u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}
__device__ __forceinline__ float h2f(unsigned bits16) {
  _Float16 h;
  const unsigned short b = (unsigned short)bits16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
// The (hi, lo) fp16 pairs of two values, packed (a in the low halves).
template <bool SAT = true>
__device__ __forceinline__ void split_h2(float a, float b, unsigned& hi, unsigned& lo) {
  hi = f2h2<SAT>(a, b);
  lo = f2h2<SAT>(a - h2f(hi & 0xFFFFu), b - h2f(hi >> 16));
}
// The (hi, lo) pair of two values in the 16-bit format of kvp planes: fp16
// (kvp = 1) or bfloat16 (kvp = 2).
template <int KVP, bool SAT = true>
__device__ __forceinline__ void split16(float a, float b, unsigned& hi, unsigned& lo) {
  if constexpr (KVP == 1) split_h2<SAT>(a, b, hi, lo);
  else split_bf2(a, b, hi, lo);
}

// Host-visible kernel launchers (defined in the .hip files).
struct Launch {
  hipStream_t stream;
};

}  // namespace dex

// Device helpers shared by the matrix-core kernels (bf16 MFMA 16x16x32 on gfx950).
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, li = l & 15, g = l >> 4):
//   A (16 x 32): lane holds A[li][8g .. 8g+7]      B (32 x 16): lane holds B[8g .. 8g+7][li]
//   D (16 x 16): lane holds D[4g + r][li], r = 0..3
// The kernels contract over a permuted K order, {4g + r, 16 + 4g + r}: with it, the D-layout
// tiles of rows 0-15 and 16-31 packed side by side are directly the B operand of the next product.
#pragma once

#include "kda_internal.h"

namespace kda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float float8v __attribute__((ext_vector_type(8)));

// two floats to packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf16x2v));
}
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ bf16x8 pack2(floatx4 a, floatx4 b) {
  const float8v f = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, __builtin_convertvector(f, bf16x8v));
}

// v_mfma_f32_16x16x16_bf16 (K = 16): lane holds A[li][4g .. 4g+3], B[4g .. 4g+3][li], D[4g + r][li].
// A D-layout tile packed to bf16 is directly the B operand of the next product.
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 ld4(const void* p) { return *reinterpret_cast<const bf16x4*>(p); }
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
// two v_cvt_pk_bf16_f32 (a four-wide vector conversion compiles to four one-value conversions and
// two permutes)
__device__ __forceinline__ bf16x4 pack4(floatx4 a) {
  const u32x2v w = {pk_bf16(a[0], a[1]), pk_bf16(a[2], a[3])};
  return __builtin_bit_cast(bf16x4, w);
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Workgroup barrier that waits only for this wave's LDS operations (so its LDS writes are visible
// after it), not for global memory operations in flight.
__device__ __forceinline__ void block_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// 128 x 16 fp32 slice in D layout (lane (li, lg), tile t, register r <-> row 16t+4lg+r, column li),
// stored as [t][lane] float4 blocks
__device__ __forceinline__ void store_slice(float* dst, const floatx4 (&S)[8], int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<floatx4*>(dst + (t * 64 + lane) * 4) = S[t];
}
__device__ __forceinline__ void load_slice(floatx4 (&S)[8], const float* src, int lane) {
#pragma unroll
  for (int t = 0; t < 8; ++t) S[t] = *reinterpret_cast<const floatx4*>(src + (t * 64 + lane) * 4);
}

// Segment plan shared by the segment kernels: P segments of L steps (32 tokens) per (b, h); workspace
// byte offsets of the per-segment X, M and S_start blocks (128 x 128 fp32 each).
struct SegPlan {
  int64_t P, L;   // segments per (b, h); steps per segment, segment 0 aside
  int64_t L0;     // steps of segment 0 (segment j >= 1 starts at L0 + (j - 1) L; the last one takes the rest)
  int64_t off_x, off_m, off_s;
  int64_t off_q;  // corrected plan: the propagated queries of every step (8 KiB each), 0 otherwise
};
constexpr int kSegState = 128 * 128 * 4;    // bytes of one block (64 KiB)
constexpr int kMHalf = 8 * 4 * 64 * 16;     // bytes of one bf16 part (hi or lo) of a transition M
constexpr int kMaxSeg = 32;                 // segments per (b, h), unless a segment would reach kMaxSegSteps
// the fused path's per-head statistics record of segment 0, in the (otherwise unused) entering-state
// block of segment 0, as uint32: the non-finite counts of the 8 state wavefronts, then chunks, flagged
// chunks and the bits of the minimum span
constexpr int kRecNonfinite = 0, kRecChunks = 8, kRecFlagged = 9, kRecMinSpan = 10;

// the fused segment kernels take this configuration (bf16, dk = dv = 128, 32-bit buffer offsets)
// the fused segment kernels (one launch: every segment's map when !out, every segment's outputs when out)
hipError_t launch_fused_segments(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg, bool out);
// the corrected plan: one pass over every segment (segment 0 exact from S0; segments 1 .. P-1 with outputs
// from a zero entering state, their maps and their propagated queries), then, after the chaining, the
// correction of their outputs by the true entering states
hipError_t launch_fused_corr(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg);
hipError_t launch_correct(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg);
constexpr int kQtStep = 8 * 64 * 16;     // bytes of one step's propagated queries (8 wavefronts x 64 lanes x 16 B)

}  // namespace kda

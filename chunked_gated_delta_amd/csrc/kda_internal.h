// Internal declarations shared by the HIP sources of libkda.so (not installed, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kda.h"

namespace kda {

constexpr int kChunk = 16;          // tokens per chunk of the matrix-core path (the tile the bounded gate is sized for)
constexpr float kSpanLimit = -80.f; // 16 * g_min for g_min = -5: below it exp(-G) may overflow

struct Params {
  const void *q, *k, *v, *w, *beta;
  const float* S0;
  float g_min;      // used when !unbounded
  int unbounded;    // 1: g = -softplus(w)
  int64_t B, H, T, dk, dv;
  int dtype;        // kda_dtype_t
  void* o;
  float* S_final;
  void* workspace;
  size_t workspace_bytes;
  kda_stats_t* stats;
  int disable_fallback, force_fallback;
  int chunk;           // tokens per chunk: 16 (every path), 32 or 64 (the vector path)
  int64_t seg_steps;   // matrix-core path: steps of 32 tokens per segment, 0 = automatic
#if KDA_PHASE_STAMPS
  // the phase-stamp build (libkda_stamps.so) only: workgroup `stamp_block` of the segment pass writes
  // s_memtime stamps to the workspace at byte offset stamp_off (-1: none); in the backward,
  // stamp_kernel picks the kernel whose workgroup stamps (0: the chains, 1: the gradient kernel)
  int64_t stamp_off;
  int stamp_block;
  int stamp_kernel;
#endif
  __host__ __device__ int64_t n_chunks() const { return (T + kChunk - 1) / kChunk; }
};

#if KDA_PHASE_STAMPS
// stamps of the segment pass: per wavefront, per interval (the first kStampSteps), kStampK phase
// boundaries, 8 bytes each, at the end of the workspace
constexpr int kStampSteps = 48, kStampK = 6;
constexpr int64_t kStampBytes = 16 * kStampSteps * kStampK * 8;
#endif

// Recurrent decode step (state in place)
struct DecodeParams {
  const void *q, *k, *v, *w, *beta;
  float* S;
  void* o;
  float g_min;
  int unbounded;
  int64_t B, H, T, dk, dv;
  int dtype;
};

// Backward pass: gradients (fp32) of a loss given dO (input dtype) and dS_final (fp32, nullable)
struct BwdParams {
  Params p;          // forward arguments (workspace: the chunk entering states)
  const void* dO;
  const float* dSf;
  float *dq, *dk, *dv, *dw, *dbeta, *dS0;   // dS0 nullable
};

// Raises kernel fn's dynamic LDS limit to `bytes` on the current device, once per device (the attribute
// belongs to the device; `done` holds one bit per device id below 64, beyond which it is set every call).
// Host-only and not a stream operation, so calls under graph capture keep it.
inline hipError_t set_dyn_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Error text for kda_last_hip_error(): both store the text for the calling thread and return KDA_ERR_HIP.
int record_hip_error(hipError_t e);
int record_error_text(const char* text);

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_stats_init(kda_stats_t* stats, hipStream_t s);
hipError_t launch_state_copy(const Params& p, hipStream_t s);          // T == 0
hipError_t launch_gate_prefix(const void* w, float g_min, int unbounded, int64_t B, int64_t H,
                              int64_t T, int64_t dk, int dtype, int chunk, float* g, float* G, float* span,
                              uint8_t* flags, hipStream_t s);
hipError_t launch_vec(const Params& p, hipStream_t s);                 // plain fp32 vector path
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);        // per-token recurrence on a resident state
size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv);
hipError_t launch_bwd(const BwdParams& b, hipStream_t s);              // backward, fp32 vector ALUs
// the matrix-core paths (path ids 3 and 4 of kda_opts_t): 3 fused (map pass, chaining, output pass),
// 4 fused with corrected outputs (one pass over every segment, chaining, correction)
enum MfmaMode { kModeFused = 3, kModeCorr = 4 };
// workspace of a matrix-core path for the segment plan that seg_steps (0: automatic) selects: the
// segment blocks of path 3 (none for a one-segment plan); the segment blocks and the propagated
// queries of path 4
size_t mfma_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int mode,
                            int64_t seg_steps);
bool fused_supported(int dtype, int64_t dk, int64_t dv, int64_t T);
// every segment of a plan stays below kMaxSegSteps steps, the limit of the fused kernels' 32-bit buffer
// views (2^18 steps of 32 tokens: 2 GiB of one bf16 tensor): the automatic plan takes more segments
// where needed, and a forced segment length must be shorter
constexpr int64_t kMaxSegSteps = (int64_t)1 << 18;
bool mfma_seg_steps_ok(int64_t T, int64_t seg_steps);                    // forced segment length allowed?
hipError_t launch_mfma(const Params& p, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end, int mode);
// the forward path a valid call takes: 1 vector, or a matrix-core mode; -1 for an unsupported request
int forward_path(const kda_shape_t* sh, int chunk, const kda_opts_t* opts);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even, NaN kept quiet
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T> __device__ __forceinline__ void store_f32(T* p, int64_t i, float x);
template <> __device__ __forceinline__ void store_f32<float>(float* p, int64_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void store_f32<uint16_t>(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }

// log-decay of one gate pre-activation: g_min * sigmoid(w), or -softplus(w)
__device__ __forceinline__ float gate_f32(float w, float g_min, int unbounded) {
  if (unbounded) return -(fmaxf(w, 0.f) + log1pf(expf(-fabsf(w))));
  return g_min / (1.f + expf(-w));
}

__device__ __forceinline__ void atomic_min_float(float* addr, float v) {
  if (v != v) return;
  if (v >= 0.f) atomicMin(reinterpret_cast<int*>(addr), __float_as_int(v));
  else atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

__device__ __forceinline__ bool not_finite(float x) { return !(fabsf(x) <= 3.402823466e38f); }

}  // namespace kda

// Small kernels shared by both evaluation paths: statistics reset, the T = 0
// state copy, and the stand-alone gate / in-chunk prefix stage.
#include "kda_internal.h"

namespace kda {

__global__ void stats_init_kernel(kda_stats_t* st) {
  if (threadIdx.x == 0) {
    st->n_chunks = 0;
    st->n_flagged = 0;
    st->n_nonfinite = 0;
    st->min_span = __int_as_float(0x7f800000);  // +inf
  }
}

hipError_t launch_stats_init(kda_stats_t* stats, hipStream_t s) {
  hipLaunchKernelGGL(stats_init_kernel, dim3(1), dim3(64), 0, s, stats);
  return hipGetLastError();
}

// S_final = S0 (or zeros); used when there are no tokens.
__global__ void state_copy_kernel(const float* __restrict__ S0, float* __restrict__ S, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    S[i] = S0 ? S0[i] : 0.f;
}

hipError_t launch_state_copy(const Params& p, hipStream_t s) {
  if (p.S0 == p.S_final) return hipSuccess;
  const int64_t n = p.B * p.H * p.dk * p.dv;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.S0, p.S_final, n);
  return hipGetLastError();
}

// One workgroup per (b, h, chunk); one thread per key channel.
// g = gate(w); G = inclusive prefix of g within the chunk; span = min_c G[last row, c].
template <typename TIn>
__global__ __launch_bounds__(128) void gate_prefix_kernel(const TIn* __restrict__ w, float g_min, int unbounded,
                                                          int64_t T, int dk, int chunk, int64_t NC,
                                                          float* __restrict__ g_out, float* __restrict__ G_out,
                                                          float* __restrict__ span_out, uint8_t* __restrict__ flags) {
  __shared__ float red[128];
  const int64_t bh = blockIdx.x / NC;
  const int64_t n = blockIdx.x % NC;
  const int c = threadIdx.x;
  const int64_t t0 = n * chunk;
  const int len = (int)((T - t0) < chunk ? (T - t0) : chunk);
  float G = 0.f;
  if (c < dk) {
    for (int r = 0; r < len; ++r) {
      const int64_t idx = (bh * T + t0 + r) * dk + c;
      const float g = gate_f32(load_f32(w, idx), g_min, unbounded);
      G += g;
      if (g_out) g_out[idx] = g;
      if (G_out) G_out[idx] = G;
    }
  }
  red[c] = (c < dk) ? G : __int_as_float(0x7f800000);
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (c < off) red[c] = fminf(red[c], red[c + off]);
    __syncthreads();
  }
  if (c == 0) {
    if (span_out) span_out[bh * NC + n] = red[0];
    if (flags) flags[bh * NC + n] = red[0] < kSpanLimit ? 1 : 0;
  }
}

hipError_t launch_gate_prefix(const void* w, float g_min, int unbounded, int64_t B, int64_t H, int64_t T,
                              int64_t dk, int dtype, int chunk, float* g, float* G, float* span, uint8_t* flags,
                              hipStream_t s) {
  const int64_t NC = (T + chunk - 1) / chunk;
  const int64_t blocks = B * H * NC;
  if (blocks == 0) return hipSuccess;
  if (dtype == KDA_DTYPE_BF16)
    hipLaunchKernelGGL(gate_prefix_kernel<uint16_t>, dim3((unsigned)blocks), dim3(128), 0, s,
                       (const uint16_t*)w, g_min, unbounded, T, (int)dk, chunk, NC, g, G, span, flags);
  else
    hipLaunchKernelGGL(gate_prefix_kernel<float>, dim3((unsigned)blocks), dim3(128), 0, s,
                       (const float*)w, g_min, unbounded, T, (int)dk, chunk, NC, g, G, span, flags);
  return hipGetLastError();
}

}  // namespace kda

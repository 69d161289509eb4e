// Recurrent decode step of KDA: the per-token form of the gated delta rule applied to a resident
// state, for inference that advances each sequence by one (or a few) tokens per call.
//
// Per token t and (b, h), with the state S (dk x dv, fp32) held by the caller:
//   S <- Diag(e^{g_t}) S            g_t = g_min sigmoid(w_t), or -softplus(w_t) when unbounded
//   u  = beta_t (v_t - S^T k_t)
//   S <- S + k_t u^T
//   o_t = S^T q_t
// which is the recurrence the chunk form evaluates in blocks ("From Numerical Stability to Load
// Balancing ..." section 2.1: a fixed-size state, forgotten per channel and written with key/value
// outer products, read by the query; delta-rule models are named there and in "Architecting
// Long-Context LLMs ..." section 2.1, the bounded gate in both pages' section 2.2).  Token by token
// there is no reciprocal decay factor, so no span check is needed.
//
// Value columns of S are independent, so a workgroup owns one (b, h) and a block of CB columns:
// thread (c, rq) holds column c of rows rq * DK/4 .. rq * DK/4 + DK/4 - 1 in registers for all the
// call's tokens, reading and writing S once per call (the step is bound by those two passes over
// S in HBM).  The two row reductions (S^T k and S^T q) combine the four row quarters through LDS.
#include "kda_internal.h"

namespace kda {

namespace {

template <typename TIn, int DK, int CB>
__global__ __launch_bounds__(CB * 4) void decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v, const TIn* __restrict__ w,
                                                        const TIn* __restrict__ beta, float* __restrict__ S,
                                                        TIn* __restrict__ o, float g_min, int unbounded, int64_t T,
                                                        int dv) {
  constexpr int RQ = DK / 4;                 // rows per thread
  __shared__ float kk[DK], qq[DK], aa[DK];   // k, q and e^{g} of the token
  __shared__ float vv[CB], bb;               // v of the column block, beta
  __shared__ float part[2][4][CB];           // row-quarter partial sums of S^T k and S^T q
  const int tid = threadIdx.x, c = tid % CB, rq = tid / CB;
  const int nblk = dv / CB;
  const int64_t bh = blockIdx.x / nblk;
  const int col = (blockIdx.x % nblk) * CB + c;
  float* Sb = S + bh * DK * dv;

  float s[RQ];
#pragma unroll
  for (int i = 0; i < RQ; ++i) s[i] = Sb[(int64_t)(rq * RQ + i) * dv + col];

  for (int64_t t = 0; t < T; ++t) {
    const int64_t tok = bh * T + t;
    // stage the token's inputs (the barrier after the previous token's reads has passed)
    for (int r = tid; r < DK; r += CB * 4) {
      kk[r] = load_f32(k, tok * DK + r);
      qq[r] = load_f32(q, tok * DK + r);
      aa[r] = expf(gate_f32(load_f32(w, tok * DK + r), g_min, unbounded));
    }
    if (tid < CB) vv[tid] = load_f32(v, tok * dv + (blockIdx.x % nblk) * CB + tid);
    if (tid == 0) bb = load_f32(beta, tok);
    __syncthreads();
    // forget, then the erase term S^T k over this thread's rows
    float pk = 0.f;
#pragma unroll
    for (int i = 0; i < RQ; ++i) {
      s[i] *= aa[rq * RQ + i];
      pk += s[i] * kk[rq * RQ + i];
    }
    part[0][rq][c] = pk;
    __syncthreads();
    const float u = bb * (vv[c] - (part[0][0][c] + part[0][1][c] + part[0][2][c] + part[0][3][c]));
    // write, then the read S^T q over this thread's rows
    float pq = 0.f;
#pragma unroll
    for (int i = 0; i < RQ; ++i) {
      s[i] += kk[rq * RQ + i] * u;
      pq += s[i] * qq[rq * RQ + i];
    }
    part[1][rq][c] = pq;
    __syncthreads();
    if (rq == 0) store_f32(o, tok * dv + col, part[1][0][c] + part[1][1][c] + part[1][2][c] + part[1][3][c]);
  }

#pragma unroll
  for (int i = 0; i < RQ; ++i) Sb[(int64_t)(rq * RQ + i) * dv + col] = s[i];
}

template <typename TIn, int DK>
hipError_t launch_dk(const DecodeParams& p, hipStream_t s) {
  const unsigned grid_bh = (unsigned)(p.B * p.H);
  if (p.dv >= 64) {
    hipLaunchKernelGGL((decode_kernel<TIn, DK, 64>), dim3(grid_bh * (unsigned)(p.dv / 64)), dim3(256), 0, s,
                       (const TIn*)p.q, (const TIn*)p.k, (const TIn*)p.v, (const TIn*)p.w, (const TIn*)p.beta, p.S,
                       (TIn*)p.o, p.g_min, p.unbounded, p.T, (int)p.dv);
  } else {
    hipLaunchKernelGGL((decode_kernel<TIn, DK, 32>), dim3(grid_bh * (unsigned)(p.dv / 32)), dim3(128), 0, s,
                       (const TIn*)p.q, (const TIn*)p.k, (const TIn*)p.v, (const TIn*)p.w, (const TIn*)p.beta, p.S,
                       (TIn*)p.o, p.g_min, p.unbounded, p.T, (int)p.dv);
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  switch (p.dk) {
    case 32: return launch_dk<TIn, 32>(p, s);
    case 64: return launch_dk<TIn, 64>(p, s);
    default: return launch_dk<TIn, 128>(p, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  return p.dtype == KDA_DTYPE_BF16 ? launch_t<uint16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace kda

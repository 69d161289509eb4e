// Plain fp32 vector path of the chunked KDA forward.
//
// One workgroup (256 threads) per (b, h, 32-wide slice of dv).  Chunks of 16
// tokens are processed in order; everything lives in LDS in fp32 and every
// product runs on the vector ALUs.  This path serves the fp32 dtype, any
// shape the matrix-core path does not take, and is the reference the
// matrix-core path is compared with during development.
//
// Per chunk (entering state S, chunk-local inclusive prefix G of the
// log-decay, span Gam = G at the last row), following the chunked evaluation
// of "From Numerical Stability to Load Balancing ..." section 2.1 (serial
// recurrence across chunks, matrix products inside a chunk, in-chunk scaling
// exp(G_i - G_j) for i >= j):
//   A[r][j] = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}   (j <  r)
//   P[r][j] =        sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)
//   Tm      = (I + A)^{-1}                              (unit lower triangular)
//   W  = Tm diag(beta) (K o e^{G})        Ut = Tm diag(beta) V
//   U  = Ut - W S
//   O  = (Q o e^{G}) S + P U
//   S <- diag(e^{Gam}) S + (K o e^{Gam - G})^T U
// A and P are formed either as (X o e^{G})(K o e^{-G})^T, the reciprocal
// form the bounded gate keeps finite ("Demystifying ..." Breakthrough 1
// part 2: a 16-token chunk's reciprocal stays below e^80), or, for a chunk
// whose span is below -80, pair by pair with exp(G_r - G_j) <= 1.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kDvs = 32;  // dv columns per workgroup

template <typename TIn, int DK>
__global__ __launch_bounds__(kThreads) void vec_kernel(Params p) {
  constexpr int C = kChunk;
  __shared__ float sQ[C][DK], sK[C][DK], sG[C][DK];
  __shared__ float sQb[C][DK], sKb[C][DK], sKh[C][DK], sKt[C][DK], sW[C][DK];
  __shared__ float sS[DK][kDvs];
  __shared__ float sV[C][kDvs], sUt[C][kDvs], sU[C][kDvs];
  __shared__ float sA[C][C + 1], sP[C][C + 1], sT[C][C + 1];
  __shared__ float sBeta[C], sEgam[DK], sRed[kThreads];
  __shared__ int sFlag;

  const int tid = threadIdx.x;
  const int dv = (int)p.dv;
  const int nslices = (dv + kDvs - 1) / kDvs;
  const int64_t bh = blockIdx.x / nslices;
  const int slice = blockIdx.x % nslices;
  const int d0 = slice * kDvs;
  const int dvs = (dv - d0) < kDvs ? (dv - d0) : kDvs;
  const int64_t T = p.T;
  const TIn* q = (const TIn*)p.q + bh * T * DK;
  const TIn* k = (const TIn*)p.k + bh * T * DK;
  const TIn* w = (const TIn*)p.w + bh * T * DK;
  const TIn* v = (const TIn*)p.v + bh * T * dv;
  const TIn* beta = (const TIn*)p.beta + bh * T;
  TIn* o = (TIn*)p.o + bh * T * dv;
  const bool count_chunks = (slice == 0);
  uint32_t my_flagged = 0, my_nonfinite = 0;
  float my_min_span = __int_as_float(0x7f800000);

  // initial state slice
  for (int i = tid; i < DK * kDvs; i += kThreads) {
    const int c = i / kDvs, d = i % kDvs;
    float s0 = 0.f;
    if (p.S0 && d < dvs) s0 = p.S0[(bh * DK + c) * dv + d0 + d];
    sS[c][d] = s0;
  }

  const int64_t NC = p.n_chunks();
  for (int64_t n = 0; n < NC; ++n) {
    const int64_t t0 = n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();  // previous chunk fully consumed

    // ---- load the chunk (rows past the end of the sequence are zero)
    for (int i = tid; i < C * DK; i += kThreads) {
      const int r = i / DK, c = i % DK;
      const bool ok = r < len;
      const int64_t idx = (t0 + r) * DK + c;
      sQ[r][c] = ok ? load_f32(q, idx) : 0.f;
      sK[r][c] = ok ? load_f32(k, idx) : 0.f;
      sG[r][c] = ok ? gate_f32(load_f32(w, idx), p.g_min, p.unbounded) : 0.f;  // g for now
    }
    for (int i = tid; i < C * kDvs; i += kThreads) {
      const int r = i / kDvs, d = i % kDvs;
      sV[r][d] = (r < len && d < dvs) ? load_f32(v, (t0 + r) * dv + d0 + d) : 0.f;
    }
    if (tid < C) sBeta[tid] = tid < len ? load_f32(beta, t0 + tid) : 0.f;
    __syncthreads();

    // ---- in-chunk inclusive prefix per key channel, span
    if (tid < DK) {
      float G = 0.f;
      for (int r = 0; r < C; ++r) { G += sG[r][tid]; sG[r][tid] = G; }
      sEgam[tid] = expf(G);
      sRed[tid] = G;
    } else {
      sRed[tid] = __int_as_float(0x7f800000);
    }
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
      if (tid < off) sRed[tid] = fminf(sRed[tid], sRed[tid + off]);
      __syncthreads();
    }
    if (tid == 0) {
      const float span = sRed[0];
      const bool flagged = span < kSpanLimit;
      sFlag = (p.force_fallback || (flagged && !p.disable_fallback)) ? 1 : 0;
      if (count_chunks) {
        my_flagged += flagged ? 1u : 0u;
        my_min_span = fminf(my_min_span, span);
      }
    }
    // ---- scaled operands
    for (int i = tid; i < C * DK; i += kThreads) {
      const int r = i / DK, c = i % DK;
      const float G = sG[r][c];
      const float eg = expf(G);
      const float kk = sK[r][c];
      sQb[r][c] = sQ[r][c] * eg;
      sKb[r][c] = kk * eg;
      sKh[r][c] = kk * expf(-G);
      sKt[r][c] = kk * expf(sG[C - 1][c] - G);
    }
    __syncthreads();
    const bool pairwise = sFlag != 0;

    // ---- A (strictly lower, rows scaled by beta) and P (lower incl. diagonal)
    {
      const int r = tid / C, j = tid % C;
      float a = 0.f, pp = 0.f;
      if (j <= r) {
        if (pairwise) {
          for (int c = 0; c < DK; ++c) {
            const float e = expf(sG[r][c] - sG[j][c]);
            const float kj = sK[j][c] * e;
            a += sK[r][c] * kj;
            pp += sQ[r][c] * kj;
          }
        } else {
          for (int c = 0; c < DK; ++c) {
            a += sKb[r][c] * sKh[j][c];
            pp += sQb[r][c] * sKh[j][c];
          }
        }
      }
      sA[r][j] = (j < r) ? sBeta[r] * a : 0.f;
      sP[r][j] = (j <= r) ? pp : 0.f;
    }
    __syncthreads();

    // ---- Tm = (I + A)^{-1} by forward substitution, one column per thread
    if (tid < C) {
      const int j = tid;
      for (int r = 0; r < C; ++r) {
        float x = (r == j) ? 1.f : 0.f;
        for (int i = j; i < r; ++i) x -= sA[r][i] * sT[i][j];
        sT[r][j] = (r < j) ? 0.f : x;
      }
    }
    __syncthreads();

    // ---- W = Tm diag(beta) Kbar,  Ut = Tm diag(beta) V
    for (int i = tid; i < C * DK; i += kThreads) {
      const int r = i / DK, c = i % DK;
      float acc = 0.f;
      for (int j = 0; j <= r; ++j) acc += sT[r][j] * sBeta[j] * sKb[j][c];
      sW[r][c] = acc;
    }
    for (int i = tid; i < C * kDvs; i += kThreads) {
      const int r = i / kDvs, d = i % kDvs;
      float acc = 0.f;
      for (int j = 0; j <= r; ++j) acc += sT[r][j] * sBeta[j] * sV[j][d];
      sUt[r][d] = acc;
    }
    __syncthreads();

    // ---- U = Ut - W S
    for (int i = tid; i < C * kDvs; i += kThreads) {
      const int r = i / kDvs, d = i % kDvs;
      float acc = sUt[r][d];
      for (int c = 0; c < DK; ++c) acc -= sW[r][c] * sS[c][d];
      sU[r][d] = acc;
    }
    __syncthreads();

    // ---- O = Qbar S + P U
    for (int i = tid; i < C * kDvs; i += kThreads) {
      const int r = i / kDvs, d = i % kDvs;
      float acc = 0.f;
      for (int c = 0; c < DK; ++c) acc += sQb[r][c] * sS[c][d];
      for (int j = 0; j <= r; ++j) acc += sP[r][j] * sU[j][d];
      if (r < len && d < dvs) {
        store_f32(o, (t0 + r) * dv + d0 + d, acc);
        my_nonfinite += not_finite(acc) ? 1u : 0u;
      }
    }
    __syncthreads();

    // ---- S <- diag(e^Gam) S + Ktil^T U
    for (int i = tid; i < DK * kDvs; i += kThreads) {
      const int c = i / kDvs, d = i % kDvs;
      float acc = sEgam[c] * sS[c][d];
      for (int j = 0; j < C; ++j) acc += sKt[j][c] * sU[j][d];
      sS[c][d] = acc;
    }
  }
  __syncthreads();

  for (int i = tid; i < DK * kDvs; i += kThreads) {
    const int c = i / kDvs, d = i % kDvs;
    if (d < dvs) {
      const float s = sS[c][d];
      p.S_final[(bh * DK + c) * dv + d0 + d] = s;
      my_nonfinite += not_finite(s) ? 1u : 0u;
    }
  }

  if (p.stats) {
    // per-thread counts: only thread 0 holds chunk statistics; non-finite counts are summed over threads
    sRed[tid] = __uint_as_float(my_nonfinite);
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int i = 0; i < kThreads; ++i) tot += __float_as_uint(sRed[i]);
      if (tot) atomicAdd(&p.stats->n_nonfinite, tot);
      if (count_chunks) {
        atomicAdd(&p.stats->n_chunks, (uint32_t)NC);
        if (my_flagged) atomicAdd(&p.stats->n_flagged, my_flagged);
        if (NC > 0) atomic_min_float(&p.stats->min_span, my_min_span);
      }
    }
  }
}

template <typename TIn>
hipError_t launch_dk(const Params& p, hipStream_t s) {
  const int nslices = (int)((p.dv + kDvs - 1) / kDvs);
  const dim3 grid((unsigned)(p.B * p.H * nslices));
  switch (p.dk) {
    case 32: hipLaunchKernelGGL((vec_kernel<TIn, 32>), grid, dim3(kThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL((vec_kernel<TIn, 64>), grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL((vec_kernel<TIn, 128>), grid, dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vec(const Params& p, hipStream_t s) {
  if (p.dtype == KDA_DTYPE_BF16) return launch_dk<uint16_t>(p, s);
  return launch_dk<float>(p, s);
}

}  // namespace kda

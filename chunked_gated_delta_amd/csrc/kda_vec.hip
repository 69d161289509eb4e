// Plain fp32 vector path of the chunked KDA forward, for any chunk size C in {16, 32, 64}.
//
// One workgroup (256 threads) per (b, h, slice of dv).  Chunks of C tokens are processed in order;
// everything lives in LDS in fp32 and every product runs on the vector ALUs.  This path serves the
// fp32 dtype, the shapes the matrix-core path does not take, and the chunk sizes other than 16 (the
// chunk-size and lower-bound co-design that "From Numerical Stability to Load Balancing ..." section
// 2.3 recommends); the matrix-core path is compared with it during development.
//
// Per chunk (entering state S, chunk-local inclusive prefix G of the log-decay, span Gam = G at the
// last row), following the chunked evaluation of the same page's section 2.1 (serial recurrence
// across chunks, matrix products inside a chunk, in-chunk scaling exp(G_i - G_j) for i >= j):
//   A[r][j] = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}   (j <  r)
//   P[r][j] =        sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)
//   Tm      = (I + A)^{-1}                              (unit lower triangular)
//   R  = diag(beta) (V - (K o e^{G}) S)     U = Tm R
//   O  = (Q o e^{G}) S + P U
//   S <- diag(e^{Gam}) S + (K o e^{Gam - G})^T U
// A and P are formed either as (X o e^{G})(K o e^{-G})^T, the reciprocal form, when the chunk's span
// (the minimum over key channels of Gam) is at or above -80, so that every reciprocal factor stays
// below e^80 ("Demystifying ..." Breakthrough 1 part 2 fixes that bound for 16 tokens at g_min = -5;
// a longer chunk keeps it only with a tighter lower bound), or, for a chunk whose span is below -80,
// pair by pair with exp(G_r - G_j) <= 1.
//
// LDS holds three [C][dk] arrays that change meaning within the chunk (in place, so that a 64-token
// chunk fits): k, q and the prefix G as loaded; then Kbar = k e^{G}, Qbar = q e^{G} and, after A and P,
// Ktil = k e^{Gam - G} in the place of G (a dense chunk first keeps Khat = k e^{-G} there for its tiles).
// Tm = (I + A)^{-1} likewise replaces A, row by row.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;

template <int DK, int C>
struct VecCfg {
  static constexpr int Dvs = C <= 32 ? 32 : 16;    // dv columns per workgroup (a 64-token chunk takes 16)
  static constexpr int Pad = C + 1;                // row stride of the C x C blocks
  // float offsets into the dynamic shared memory
  static constexpr int oK = 0, oQ = oK + C * DK, oG = oQ + C * DK;
  static constexpr int oS = oG + C * DK;           // [DK][Dvs]
  static constexpr int oV = oS + DK * Dvs;         // [C][Dvs], then R
  static constexpr int oU = oV + C * Dvs;          // [C][Dvs]
  static constexpr int oA = oU + C * Dvs;          // [C][Pad]: A, then Tm (in place, row by row)
  static constexpr int oP = oA + C * Pad;          // [C][Pad]
  static constexpr int oBeta = oP + C * Pad;       // [C]
  static constexpr int oGam = oBeta + C;           // [DK] Gam, then e^{Gam}
  static constexpr int oRed = oGam + DK;           // [kThreads]
  static constexpr int kFloats = oRed + kThreads;
  static constexpr size_t kBytes = (size_t)kFloats * 4 + 16;
};

template <typename TIn, int DK, int C>
__global__ __launch_bounds__(kThreads) void vec_kernel(Params p) {
  using Cfg = VecCfg<DK, C>;
  constexpr int Dvs = Cfg::Dvs, Pad = Cfg::Pad;
  extern __shared__ __align__(16) float vsm[];
  float (*sK)[DK] = reinterpret_cast<float (*)[DK]>(vsm + Cfg::oK);   // k, then Kbar
  float (*sQ)[DK] = reinterpret_cast<float (*)[DK]>(vsm + Cfg::oQ);   // q, then Qbar
  float (*sG)[DK] = reinterpret_cast<float (*)[DK]>(vsm + Cfg::oG);   // G, then Khat / Ktil
  float (*sS)[Dvs] = reinterpret_cast<float (*)[Dvs]>(vsm + Cfg::oS);
  float (*sV)[Dvs] = reinterpret_cast<float (*)[Dvs]>(vsm + Cfg::oV);  // V, then R
  float (*sU)[Dvs] = reinterpret_cast<float (*)[Dvs]>(vsm + Cfg::oU);
  float (*sA)[Pad] = reinterpret_cast<float (*)[Pad]>(vsm + Cfg::oA);  // A, then Tm
  float (*sP)[Pad] = reinterpret_cast<float (*)[Pad]>(vsm + Cfg::oP);
  float* sBeta = vsm + Cfg::oBeta;
  float* sGam = vsm + Cfg::oGam;
  float* sRed = vsm + Cfg::oRed;
  __shared__ int sFlag;

  const int tid = threadIdx.x;
  const int dv = (int)p.dv;
  const int nslices = (dv + Dvs - 1) / Dvs;
  const int64_t bh = blockIdx.x / nslices;
  const int slice = blockIdx.x % nslices;
  const int d0 = slice * Dvs;
  const int dvs = (dv - d0) < Dvs ? (dv - d0) : Dvs;
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
  for (int i = tid; i < DK * Dvs; i += kThreads) {
    const int c = i / Dvs, d = i % Dvs;
    float s0 = 0.f;
    if (p.S0 && d < dvs) s0 = p.S0[(bh * DK + c) * dv + d0 + d];
    sS[c][d] = s0;
  }

  const int64_t NC = (T + C - 1) / C;
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
    for (int i = tid; i < C * Dvs; i += kThreads) {
      const int r = i / Dvs, d = i % Dvs;
      sV[r][d] = (r < len && d < dvs) ? load_f32(v, (t0 + r) * dv + d0 + d) : 0.f;
    }
    if (tid < C) sBeta[tid] = tid < len ? load_f32(beta, t0 + tid) : 0.f;
    __syncthreads();

    // ---- in-chunk inclusive prefix per key channel, span
    if (tid < DK) {
      float G = 0.f;
      for (int r = 0; r < C; ++r) { G += sG[r][tid]; sG[r][tid] = G; }
      sGam[tid] = G;
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
    __syncthreads();
    const bool pairwise = sFlag != 0;

    // ---- A (strictly lower, rows scaled by beta) and P (lower incl. diagonal)
    if (pairwise) {
      // per pair, every factor exp(G_r - G_j) <= 1, from k, q and G as loaded
      for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, j = e % C;
        float a = 0.f, pp = 0.f;
        if (j <= r) {
          for (int c = 0; c < DK; ++c) {
            const float kj = sK[j][c] * expf(sG[r][c] - sG[j][c]);
            a += sK[r][c] * kj;
            pp += sQ[r][c] * kj;
          }
        }
        sA[r][j] = (j < r) ? sBeta[r] * a : 0.f;
        sP[r][j] = (j <= r) ? pp : 0.f;
      }
      __syncthreads();
      // Ktil = k e^{Gam - G} into G's place (k is still raw), then Kbar, Qbar in place
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        const float G = sG[r][c], eg = expf(G), kk = sK[r][c];
        sG[r][c] = kk * expf(sGam[c] - G);
        sK[r][c] = kk * eg;
        sQ[r][c] *= eg;
      }
    } else {
      // the reciprocal form: Kbar, Qbar and Khat = k e^{-G} in place, then the dense products
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        const float G = sG[r][c], kk = sK[r][c];
        sG[r][c] = kk * expf(-G);
        const float eg = expf(G);
        sK[r][c] = kk * eg;
        sQ[r][c] *= eg;
      }
      __syncthreads();
      for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, j = e % C;
        float a = 0.f, pp = 0.f;
        if (j <= r) {
          for (int c = 0; c < DK; ++c) {
            a += sK[r][c] * sG[j][c];
            pp += sQ[r][c] * sG[j][c];
          }
        }
        sA[r][j] = (j < r) ? sBeta[r] * a : 0.f;
        sP[r][j] = (j <= r) ? pp : 0.f;
      }
      __syncthreads();
      // Ktil = Khat e^{Gam} in place (finite: e^{-G} <= e^{80} on a chunk within the span bound)
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        sG[r][c] *= expf(sGam[c]);
      }
    }
    __syncthreads();

    // ---- Tm = (I + A)^{-1}, row by row in A's place: row r of Tm is e_r - sum_{i<r} A[r][i] Tm[i][:], and
    // once it is formed row r of A is not read again.  Thread j < C forms column j of the row; every
    // thread of the workgroup takes the same barriers (the loop is uniform).
    for (int r = 0; r < C; ++r) {
      float x = 0.f;
      if (tid < C) {
        const int j = tid;
        if (j <= r) {
          x = (r == j) ? 1.f : 0.f;
          for (int i = j; i < r; ++i) x -= sA[r][i] * sA[i][j];
        }
      }
      __syncthreads();   // row r of A fully read
      if (tid < C) sA[r][tid] = x;
      __syncthreads();
    }
    // e^{Gam} for the state update
    if (tid < DK) sGam[tid] = expf(sGam[tid]);
    __syncthreads();

    // ---- R = diag(beta) (V - Kbar S), in V's place
    for (int i = tid; i < C * Dvs; i += kThreads) {
      const int r = i / Dvs, d = i % Dvs;
      float acc = sV[r][d];
      for (int c = 0; c < DK; ++c) acc -= sK[r][c] * sS[c][d];
      sV[r][d] = sBeta[r] * acc;
    }
    __syncthreads();

    // ---- U = Tm R
    for (int i = tid; i < C * Dvs; i += kThreads) {
      const int r = i / Dvs, d = i % Dvs;
      float acc = 0.f;
      for (int j = 0; j <= r; ++j) acc += sA[r][j] * sV[j][d];
      sU[r][d] = acc;
    }
    __syncthreads();

    // ---- O = Qbar S + P U
    for (int i = tid; i < C * Dvs; i += kThreads) {
      const int r = i / Dvs, d = i % Dvs;
      float acc = 0.f;
      for (int c = 0; c < DK; ++c) acc += sQ[r][c] * sS[c][d];
      for (int j = 0; j <= r; ++j) acc += sP[r][j] * sU[j][d];
      if (r < len && d < dvs) {
        store_f32(o, (t0 + r) * dv + d0 + d, acc);
        my_nonfinite += not_finite(acc) ? 1u : 0u;
      }
    }
    __syncthreads();

    // ---- S <- diag(e^Gam) S + Ktil^T U
    for (int i = tid; i < DK * Dvs; i += kThreads) {
      const int c = i / Dvs, d = i % Dvs;
      float acc = sGam[c] * sS[c][d];
      for (int j = 0; j < C; ++j) acc += sG[j][c] * sU[j][d];
      sS[c][d] = acc;
    }
  }
  __syncthreads();

  for (int i = tid; i < DK * Dvs; i += kThreads) {
    const int c = i / Dvs, d = i % Dvs;
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

template <typename TIn, int DK, int C>
hipError_t launch_one(const Params& p, hipStream_t s) {
  using Cfg = VecCfg<DK, C>;
  static_assert(Cfg::kBytes <= 163840, "LDS budget");
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)vec_kernel<TIn, DK, C>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::kBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nslices = (int)((p.dv + Cfg::Dvs - 1) / Cfg::Dvs);
  hipLaunchKernelGGL((vec_kernel<TIn, DK, C>), dim3((unsigned)(p.B * p.H * nslices)), dim3(kThreads), Cfg::kBytes, s,
                     p);
  return hipGetLastError();
}

template <typename TIn, int C>
hipError_t launch_dk(const Params& p, hipStream_t s) {
  switch (p.dk) {
    case 32: return launch_one<TIn, 32, C>(p, s);
    case 64: return launch_one<TIn, 64, C>(p, s);
    case 128: return launch_one<TIn, 128, C>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIn>
hipError_t launch_chunk(const Params& p, hipStream_t s) {
  switch (p.chunk) {
    case 16: return launch_dk<TIn, 16>(p, s);
    case 32: return launch_dk<TIn, 32>(p, s);
    case 64: return launch_dk<TIn, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_vec(const Params& p, hipStream_t s) {
  if (p.dtype == KDA_DTYPE_BF16) return launch_chunk<uint16_t>(p, s);
  return launch_chunk<float>(p, s);
}

}  // namespace kda

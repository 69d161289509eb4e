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
//   R  = diag(beta) (V - (K o e^{G}) S)
//   U  = (I + A)^{-1} R          (forward substitution: U_r = R_r - sum_{i<r} A[r][i] U_i)
//   O  = (Q o e^{G}) S + P U
//   S <- diag(e^{Gam}) S + (K o e^{Gam - G})^T U
// A and P are formed either as (X o e^{G})(K o e^{-G})^T, the reciprocal form, when the chunk's span
// (the minimum over key channels of Gam) is at or above -80, so that every reciprocal factor stays
// below e^80 ("Demystifying ..." Breakthrough 1 part 2 fixes that bound for 16 tokens at g_min = -5;
// a longer chunk keeps it only with a tighter lower bound), or, for a chunk whose span is below -80,
// pair by pair with exp(G_r - G_j) <= 1.  The exponentials are taken base 2 of the prefix scaled by
// log2(e) once per element.
//
// LDS holds three [C][dk] arrays (rows padded by one float, so that a wavefront reading one channel
// of 16 different rows spreads over the banks) that change meaning within the chunk (in place, so that
// a 64-token chunk fits): k, q and the prefix G as loaded; then Kbar = k e^{G}, Qbar = q e^{G} and,
// after A and P, Ktil = k e^{Gam - G} in the place of G (a dense chunk first keeps Khat = k e^{-G} there
// for its products).  Each thread forms a (C/16) x (C/16) block of A and P; the substitution runs over
// 16-row blocks, each diagonal block on one lane per value column with its column of U in registers.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kDvs = 16;                           // dv columns per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int DK, int C>
struct VecCfg {
  static constexpr int DKP = DK + 1;               // row stride of the [C][dk] arrays
  static constexpr int CP = C + 4;                 // row stride of the C x C blocks (16-byte rows)
  // float offsets into the dynamic shared memory
  static constexpr int oK = 0, oQ = oK + C * DKP, oG = oQ + C * DKP;
  static constexpr int oS = oG + C * DKP;          // [DK][kDvs]
  static constexpr int oV = oS + DK * kDvs;        // [C][kDvs]: V, then R
  static constexpr int oU = oV + C * kDvs;         // [C][kDvs]
  static constexpr int oA = oU + C * kDvs;         // [C][CP]
  static constexpr int oP = oA + C * CP;           // [C][CP]
  static constexpr int oBeta = oP + C * CP;        // [C]
  static constexpr int oGam = oBeta + C;           // [DK] Gam * log2(e)
  static constexpr int oRed = oGam + DK;           // [kThreads]
  static constexpr int kFloats = oRed + kThreads;
  static constexpr size_t kBytes = (size_t)kFloats * 4 + 16;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename TIn, int DK, int C>
__global__ __launch_bounds__(kThreads) void vec_kernel(Params p) {
  using Cfg = VecCfg<DK, C>;
  constexpr int DKP = Cfg::DKP, CP = Cfg::CP;
  constexpr int BR = C / 16;        // rows and columns of A, P per thread: (C / BR)^2 = kThreads blocks
  constexpr int RPT = C / 16;       // rows of R, O per thread (16 row groups x kDvs columns)
  constexpr int CPT = DK / 16;      // state rows per thread in the update
  static_assert((C / BR) * (C / BR) == kThreads && 16 * kDvs == kThreads, "thread layout");
  extern __shared__ __align__(16) float vsm[];
  float (*sK)[DKP] = reinterpret_cast<float (*)[DKP]>(vsm + Cfg::oK);   // k, then Kbar
  float (*sQ)[DKP] = reinterpret_cast<float (*)[DKP]>(vsm + Cfg::oQ);   // q, then Qbar
  float (*sG)[DKP] = reinterpret_cast<float (*)[DKP]>(vsm + Cfg::oG);   // G log2(e), then Khat / Ktil
  float (*sS)[kDvs] = reinterpret_cast<float (*)[kDvs]>(vsm + Cfg::oS);
  float (*sV)[kDvs] = reinterpret_cast<float (*)[kDvs]>(vsm + Cfg::oV);  // V, then R
  float (*sU)[kDvs] = reinterpret_cast<float (*)[kDvs]>(vsm + Cfg::oU);
  float (*sA)[CP] = reinterpret_cast<float (*)[CP]>(vsm + Cfg::oA);
  float (*sP)[CP] = reinterpret_cast<float (*)[CP]>(vsm + Cfg::oP);
  float* sBeta = vsm + Cfg::oBeta;
  float* sGam = vsm + Cfg::oGam;
  float* sRed = vsm + Cfg::oRed;
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

  // thread roles: (row group rq, column d) for R, O and the update; (rb, jb) block of A, P
  const int rq = tid / kDvs, d = tid % kDvs;
  const int rb = tid >> 4, jb = tid & 15;

  // initial state slice
  for (int i = tid; i < DK * kDvs; i += kThreads) {
    const int c = i / kDvs, dd = i % kDvs;
    float s0 = 0.f;
    if (p.S0 && dd < dvs) s0 = p.S0[(bh * DK + c) * dv + d0 + dd];
    sS[c][dd] = s0;
  }

  // The next chunk's inputs are loaded into registers while the current one is computed: every load
  // is issued unconditionally (row index clamped into the sequence, value zeroed past its end), so that
  // no wait for them falls inside the chunk's work.
  constexpr int ME = C * DK / kThreads;          // q, k, w elements per thread
  constexpr int MV = C * kDvs / kThreads;        // v elements per thread
  float xq[ME], xk[ME], xw[ME], xv[MV], xb = 0.f;
  const int64_t NC = (T + C - 1) / C;
  auto fetch = [&](int64_t n) {
    const int64_t t0 = n * C;
#pragma unroll
    for (int m = 0; m < ME; ++m) {
      const int i = tid + m * kThreads, r = i / DK, c = i % DK;
      const int64_t t = (t0 + r) < T ? (t0 + r) : (T - 1);
      const int64_t idx = t * DK + c;
      xq[m] = load_f32(q, idx);
      xk[m] = load_f32(k, idx);
      xw[m] = load_f32(w, idx);
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const int i = tid + m * kThreads, r = i / kDvs, dd = i % kDvs;
      const int64_t t = (t0 + r) < T ? (t0 + r) : (T - 1);
      xv[m] = load_f32(v, t * dv + d0 + (dd < dvs ? dd : 0));
    }
    const int64_t tb = (t0 + (tid % C)) < T ? (t0 + (tid % C)) : (T - 1);
    xb = load_f32(beta, tb);
  };
  if (NC > 0) fetch(0);

  for (int64_t n = 0; n < NC; ++n) {
    const int64_t t0 = n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();  // previous chunk fully consumed

    // ---- the chunk into LDS (rows past the end of the sequence are zero), then the next one's loads
#pragma unroll
    for (int m = 0; m < ME; ++m) {
      const int i = tid + m * kThreads, r = i / DK, c = i % DK;
      const bool ok = r < len;
      sQ[r][c] = ok ? xq[m] : 0.f;
      sK[r][c] = ok ? xk[m] : 0.f;
      sG[r][c] = ok ? gate_f32(xw[m], p.g_min, p.unbounded) : 0.f;  // g for now
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const int i = tid + m * kThreads, r = i / kDvs, dd = i % kDvs;
      sV[r][dd] = (r < len && dd < dvs) ? xv[m] : 0.f;
    }
    if (tid < C) sBeta[tid] = tid < len ? xb : 0.f;
    fetch(n + 1 < NC ? n + 1 : n);
    __syncthreads();

    // ---- in-chunk inclusive prefix per key channel (kept as G log2(e)), span in natural units
    float span_part = __int_as_float(0x7f800000);
    if (tid < DK) {
      float G = 0.f;
#pragma unroll 8
      for (int r = 0; r < C; ++r) { G += sG[r][tid]; sG[r][tid] = G * kLog2e; }
      sGam[tid] = G * kLog2e;
      span_part = G;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) span_part = fminf(span_part, __shfl_xor(span_part, off));
    if ((tid & 63) == 0) sRed[tid >> 6] = span_part;
    __syncthreads();
    if (tid == 0) {
      const float span = fminf(fminf(sRed[0], sRed[1]), fminf(sRed[2], sRed[3]));
      const bool flagged = span < kSpanLimit;
      sFlag = (p.force_fallback || (flagged && !p.disable_fallback)) ? 1 : 0;
      if (count_chunks) {
        my_flagged += flagged ? 1u : 0u;
        my_min_span = fminf(my_min_span, span);
      }
    }
    __syncthreads();
    const bool pairwise = sFlag != 0;

    if (!pairwise) {
      // the reciprocal form: Kbar, Qbar and Khat = k e^{-G} in place
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        const float G2 = sG[r][c], kk = sK[r][c], eg = ex2(G2);
        sG[r][c] = kk * ex2(-G2);
        sK[r][c] = kk * eg;
        sQ[r][c] *= eg;
      }
      __syncthreads();
    }

    // ---- A (strictly lower, rows scaled by beta) and P (lower incl. diagonal), one BR x BR block per
    // thread; blocks above the diagonal are zero
    {
      float a[BR][BR], pp[BR][BR];
#pragma unroll
      for (int x = 0; x < BR; ++x)
#pragma unroll
        for (int y = 0; y < BR; ++y) a[x][y] = pp[x][y] = 0.f;
      if (jb <= rb) {
        if (pairwise) {
          // per pair, every factor exp(G_r - G_j) <= 1 for j <= r (the prefix does not increase along
          // the chunk; the clamp only guards the pairs above the diagonal inside a diagonal block, which
          // are discarded)
#pragma unroll 1
          for (int c = 0; c < DK; ++c) {
            float gr[BR], kr[BR], qr[BR], gj[BR], kj[BR];
#pragma unroll
            for (int x = 0; x < BR; ++x) {
              gr[x] = sG[rb * BR + x][c]; kr[x] = sK[rb * BR + x][c]; qr[x] = sQ[rb * BR + x][c];
              gj[x] = sG[jb * BR + x][c]; kj[x] = sK[jb * BR + x][c];
            }
#pragma unroll
            for (int x = 0; x < BR; ++x)
#pragma unroll
              for (int y = 0; y < BR; ++y) {
                const float f = kj[y] * ex2(fminf(gr[x] - gj[y], 0.f));
                a[x][y] += kr[x] * f;
                pp[x][y] += qr[x] * f;
              }
          }
        } else {
#pragma unroll 4
          for (int c = 0; c < DK; ++c) {
            float kr[BR], qr[BR], hj[BR];
#pragma unroll
            for (int x = 0; x < BR; ++x) {
              kr[x] = sK[rb * BR + x][c]; qr[x] = sQ[rb * BR + x][c]; hj[x] = sG[jb * BR + x][c];
            }
#pragma unroll
            for (int x = 0; x < BR; ++x)
#pragma unroll
              for (int y = 0; y < BR; ++y) {
                a[x][y] += kr[x] * hj[y];
                pp[x][y] += qr[x] * hj[y];
              }
          }
        }
      }
#pragma unroll
      for (int x = 0; x < BR; ++x) {
        const int r = rb * BR + x;
        const float br = sBeta[r];
#pragma unroll
        for (int y = 0; y < BR; ++y) {
          const int j = jb * BR + y;
          sA[r][j] = (j < r) ? br * a[x][y] : 0.f;
          sP[r][j] = (j <= r) ? pp[x][y] : 0.f;
        }
      }
    }
    __syncthreads();

    if (pairwise) {
      // Ktil = k e^{Gam - G} into G's place (k is still raw), then Kbar, Qbar in place
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        const float G2 = sG[r][c], eg = ex2(G2), kk = sK[r][c];
        sG[r][c] = kk * ex2(sGam[c] - G2);
        sK[r][c] = kk * eg;
        sQ[r][c] *= eg;
      }
    } else {
      // Ktil = Khat e^{Gam} in place (finite: e^{-G} <= e^{80} on a chunk within the span bound)
      for (int i = tid; i < C * DK; i += kThreads) {
        const int r = i / DK, c = i % DK;
        sG[r][c] *= ex2(sGam[c]);
      }
    }
    // ---- R = diag(beta) (V - Kbar S), in V's place (Kbar is final in both forms by now)
    __syncthreads();
    {
      float acc[RPT];
#pragma unroll
      for (int x = 0; x < RPT; ++x) acc[x] = sV[rq + 16 * x][d];
      #pragma unroll 8
      for (int c = 0; c < DK; ++c) {
        const float s = sS[c][d];
#pragma unroll
        for (int x = 0; x < RPT; ++x) acc[x] -= sK[rq + 16 * x][c] * s;
      }
#pragma unroll
      for (int x = 0; x < RPT; ++x) sV[rq + 16 * x][d] = sBeta[rq + 16 * x] * acc[x];
    }
    __syncthreads();

    // ---- U = (I + A)^{-1} R by forward substitution over 16-row blocks b: first every thread takes
    // one element of R_b - sum_{a<b} A_ba U_a, then one lane per value column of the first wavefront
    // solves the unit lower triangular diagonal block with its column of U_b in registers
#pragma unroll
    for (int b = 0; b < C / 16; ++b) {
      if (b > 0) {
        const int r = 16 * b + rq;
        float acc0 = sV[r][d], acc1 = 0.f;
        #pragma unroll 4
        for (int i = 0; i < 16 * b; i += 2) {
          acc0 -= sA[r][i] * sU[i][d];
          acc1 -= sA[r][i + 1] * sU[i + 1][d];
        }
        sV[r][d] = acc0 + acc1;
        __syncthreads();
      }
      if (tid < kDvs) {
        float u[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* arow = &sA[16 * b + r][16 * b];
          float s0 = sV[16 * b + r][tid], s1 = 0.f;
#pragma unroll
          for (int i = 0; i + 2 <= r; i += 2) {
            s0 -= arow[i] * u[i];
            s1 -= arow[i + 1] * u[i + 1];
          }
          if (r & 1) s0 -= arow[r - 1] * u[r - 1];
          u[r] = s0 + s1;
          sU[16 * b + r][tid] = u[r];
        }
      }
      __syncthreads();
    }

    // ---- O = Qbar S + P U
    {
      float acc[RPT];
#pragma unroll
      for (int x = 0; x < RPT; ++x) acc[x] = 0.f;
      #pragma unroll 8
      for (int c = 0; c < DK; ++c) {
        const float s = sS[c][d];
#pragma unroll
        for (int x = 0; x < RPT; ++x) acc[x] += sQ[rq + 16 * x][c] * s;
      }
      #pragma unroll 8
      for (int j = 0; j < C; ++j) {
        const float uj = sU[j][d];
#pragma unroll
        for (int x = 0; x < RPT; ++x) acc[x] += sP[rq + 16 * x][j] * uj;
      }
#pragma unroll
      for (int x = 0; x < RPT; ++x) {
        const int r = rq + 16 * x;
        if (r < len && d < dvs) {
          store_f32(o, (t0 + r) * dv + d0 + d, acc[x]);
          my_nonfinite += not_finite(acc[x]) ? 1u : 0u;
        }
      }
    }

    // ---- S <- diag(e^Gam) S + Ktil^T U (every read of S above precedes this barrier)
    __syncthreads();
    {
      float acc[CPT];
#pragma unroll
      for (int x = 0; x < CPT; ++x) {
        const int c = rq + 16 * x;
        acc[x] = ex2(sGam[c]) * sS[c][d];
      }
      #pragma unroll 8
      for (int j = 0; j < C; ++j) {
        const float uj = sU[j][d];
#pragma unroll
        for (int x = 0; x < CPT; ++x) acc[x] += sG[j][rq + 16 * x] * uj;
      }
#pragma unroll
      for (int x = 0; x < CPT; ++x) sS[rq + 16 * x][d] = acc[x];
    }
  }
  __syncthreads();

  for (int i = tid; i < DK * kDvs; i += kThreads) {
    const int c = i / kDvs, dd = i % kDvs;
    if (dd < dvs) {
      const float s = sS[c][dd];
      p.S_final[(bh * DK + c) * dv + d0 + dd] = s;
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
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_dyn_lds((const void*)vec_kernel<TIn, DK, C>, (int)Cfg::kBytes, lds_set);
  if (e != hipSuccess) return e;
  const int nslices = (int)((p.dv + kDvs - 1) / kDvs);
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

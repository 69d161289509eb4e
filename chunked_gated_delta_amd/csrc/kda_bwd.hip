// Backward pass of the chunked KDA forward: gradients of a loss L with respect to q, k, v, w, beta
// and S0, given dL/do and dL/dS_final, in fp32 on the vector ALUs.
//
// The forward of one 16-token chunk (entering state S, chunk-local inclusive prefix G of the
// log-decay, span Gam = G at the last row; "From Numerical Stability to Load Balancing ..."
// section 2.1), in the form this file differentiates:
//   X[r][j] = sum_c k_rc k_jc e^{G_rc - G_jc}   (j < r)      A = diag(beta) X
//   P[r][j] = sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)     T = (I + A)^{-1}
//   E = V - Kbar S,  R = diag(beta) E,  U = T R,  O = Qbar S + P U,  S' = e^{Gam} S + Ktil^T U
// with Kbar = k e^{G}, Qbar = q e^{G}, Ktil = k e^{Gam - G}.  X and P are formed pair by pair, every
// factor exp(G_r - G_j) <= 1 (the per-position form the pages give for chunks whose reciprocal
// factors would overflow), so the backward needs no span check and no reciprocal at all.
//
// Reverse mode through that chunk, given dO and dS' (one block of value columns at a time: the map
// is linear in the adjoint, so blocks of columns contribute independently and their contributions
// to the key-side gradients add up):
//   dU = P^T dO + Ktil dS'        dR = T^T dU        dv = diag(beta) dR
//   dT = dU R^T  ->  dA = -T^T dT T^T (strictly lower)      dP = dO U^T (lower, diagonal included)
//   dbeta_r = sum_d dR[r][d] E[r][d] + sum_j dA[r][j] X[r][j]
//   X, P pair by pair -> dk, dq, dG;   dQbar = dO S^T,  dKbar = -diag(beta) dR S^T,  dKtil = U dS'^T
//   dGam += e^{Gam} . rowsum(dS' o S) + colsum(dKtil o Ktil)
//   dS = e^{Gam} dS' + Qbar^T dO - Kbar^T diag(beta) dR
//   dg = reverse prefix of dG (+ dGam on every row),  dw = dg gate'(w)
// The chunk's entering states come from a first pass of the same forward, kept in the workspace.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;      // 16
constexpr int NT = 256;        // threads per workgroup
constexpr int CS = 32;         // value columns per workgroup
constexpr int NPAIR = C * (C + 1) / 2;

template <int DK>
struct BwdShared {
  float S[DK][CS], dS[DK][CS];
  float q[C][DK], k[C][DK], G[C][DK];
  float dq[C][DK], dk[C][DK], dG[C][DK];
  float gam[DK], dgam[DK];
  float V[C][CS], dO[C][CS], E[C][CS], R[C][CS], U[C][CS], dU[C][CS], dR[C][CS];
  float X[C][C + 1], P[C][C + 1], T[C][C + 1], dA[C][C + 1], dP[C][C + 1], dT[C][C + 1], M[C][C + 1];
  float beta[C];
};

__device__ __forceinline__ void pair_of(int pr, int& r, int& j) {   // pr -> (r, j), j <= r < 16
  r = 0;
  while ((r + 1) * (r + 2) / 2 <= pr) ++r;
  j = pr - r * (r + 1) / 2;
}

// gate derivative d g / d w: g_min sigma (1 - sigma), or -sigma for -softplus
__device__ __forceinline__ float gate_deriv(float w, float g_min, int unbounded) {
  const float s = 1.f / (1.f + expf(-w));
  return unbounded ? -s : g_min * s * (1.f - s);
}

// Loads chunk n (rows past the end are zero: k = q = v = beta = 0 and g = 0, which reproduces the
// shorter last chunk exactly), forms the prefix G and Gam, then X, P (pair by pair), T, E, R, U.
template <typename TIn, int DK>
__device__ void chunk_forward(BwdShared<DK>& sm, const Params& p, int64_t bh, int64_t n, int d0, int dvs) {
  const int tid = threadIdx.x;
  const int64_t T = p.T, t0 = n * C;
  const int len = (int)((T - t0) < C ? (T - t0) : C);
  const int dv = (int)p.dv;
  const TIn* q = (const TIn*)p.q + bh * T * DK;
  const TIn* k = (const TIn*)p.k + bh * T * DK;
  const TIn* w = (const TIn*)p.w + bh * T * DK;
  const TIn* v = (const TIn*)p.v + bh * T * dv;
  const TIn* beta = (const TIn*)p.beta + bh * T;
  for (int i = tid; i < C * DK; i += NT) {
    const int r = i / DK, c = i % DK;
    const bool ok = r < len;
    const int64_t idx = (t0 + r) * DK + c;
    sm.q[r][c] = ok ? load_f32(q, idx) : 0.f;
    sm.k[r][c] = ok ? load_f32(k, idx) : 0.f;
    sm.G[r][c] = ok ? gate_f32(load_f32(w, idx), p.g_min, p.unbounded) : 0.f;
  }
  for (int i = tid; i < C * CS; i += NT) {
    const int r = i / CS, d = i % CS;
    sm.V[r][d] = (r < len && d < dvs) ? load_f32(v, (t0 + r) * dv + d0 + d) : 0.f;
  }
  if (tid < C) sm.beta[tid] = tid < len ? load_f32(beta, t0 + tid) : 0.f;
  __syncthreads();
  if (tid < DK) {
    float g = 0.f;
    for (int r = 0; r < C; ++r) { g += sm.G[r][tid]; sm.G[r][tid] = g; }
    sm.gam[tid] = g;
  }
  __syncthreads();
  // X and P, one (r, j) pair per thread over every key channel
  if (tid < NPAIR) {
    int r, j;
    pair_of(tid, r, j);
    float x = 0.f, pp = 0.f;
    for (int c = 0; c < DK; ++c) {
      const float kj = sm.k[j][c] * expf(sm.G[r][c] - sm.G[j][c]);
      x += sm.k[r][c] * kj;
      pp += sm.q[r][c] * kj;
    }
    sm.X[r][j] = j < r ? x : 0.f;
    sm.P[r][j] = pp;
    if (j < r) { sm.X[j][r] = 0.f; sm.P[j][r] = 0.f; }
  }
  __syncthreads();
  // T = (I + A)^{-1}, A = diag(beta) X: forward substitution, one column per thread
  if (tid < C) {
    const int j = tid;
    for (int r = 0; r < C; ++r) {
      float x = (r == j) ? 1.f : 0.f;
      for (int i = j; i < r; ++i) x -= sm.beta[r] * sm.X[r][i] * sm.T[i][j];
      sm.T[r][j] = (r < j) ? 0.f : x;
    }
  }
  // E = V - Kbar S,  R = diag(beta) E
  for (int i = tid; i < C * CS; i += NT) {
    const int r = i / CS, d = i % CS;
    float acc = sm.V[r][d];
    for (int c = 0; c < DK; ++c) acc -= sm.k[r][c] * expf(sm.G[r][c]) * sm.S[c][d];
    sm.E[r][d] = acc;
    sm.R[r][d] = sm.beta[r] * acc;
  }
  __syncthreads();
  for (int i = tid; i < C * CS; i += NT) {
    const int r = i / CS, d = i % CS;
    float acc = 0.f;
    for (int j = 0; j <= r; ++j) acc += sm.T[r][j] * sm.R[j][d];
    sm.U[r][d] = acc;
  }
  __syncthreads();
}

template <typename TIn, int DK>
__global__ __launch_bounds__(NT) void bwd_kernel(Params p, const void* dO_in, const float* dSf, float* dq, float* dk,
                                                  float* dvo, float* dw, float* dbeta, float* dS0) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  BwdShared<DK>& sm = *reinterpret_cast<BwdShared<DK>*>(smem_raw);
  const int tid = threadIdx.x;
  const int dv = (int)p.dv;
  const int nslices = dv / CS;
  const int64_t bh = blockIdx.x / nslices;
  const int slice = blockIdx.x % nslices;
  const int d0 = slice * CS, dvs = CS;
  const int64_t T = p.T, NC = p.n_chunks();
  float* states = (float*)p.workspace + ((bh * nslices + slice) * NC) * (int64_t)(DK * CS);
  const TIn* dO = (const TIn*)dO_in + bh * T * dv;
  const TIn* w = (const TIn*)p.w + bh * T * DK;

  // ---- pass 1: entering state of every chunk
  for (int i = tid; i < DK * CS; i += NT) {
    const int c = i / CS, d = i % CS;
    sm.S[c][d] = p.S0 ? p.S0[(bh * DK + c) * dv + d0 + d] : 0.f;
  }
  __syncthreads();
  for (int64_t n = 0; n < NC; ++n) {
    for (int i = tid; i < DK * CS; i += NT) states[n * DK * CS + i] = (&sm.S[0][0])[i];
    chunk_forward<TIn, DK>(sm, p, bh, n, d0, dvs);
    for (int i = tid; i < DK * CS; i += NT) {
      const int c = i / CS, d = i % CS;
      float acc = expf(sm.gam[c]) * sm.S[c][d];
      for (int r = 0; r < C; ++r) acc += sm.k[r][c] * expf(sm.gam[c] - sm.G[r][c]) * sm.U[r][d];
      sm.S[c][d] = acc;
    }
    __syncthreads();
  }

  // ---- pass 2: chunks in reverse
  for (int i = tid; i < DK * CS; i += NT) {
    const int c = i / CS, d = i % CS;
    sm.dS[c][d] = dSf ? dSf[(bh * DK + c) * dv + d0 + d] : 0.f;
  }
  for (int64_t n = NC - 1; n >= 0; --n) {
    const int64_t t0 = n * C;
    const int len = (int)((T - t0) < C ? (T - t0) : C);
    for (int i = tid; i < DK * CS; i += NT) (&sm.S[0][0])[i] = states[n * DK * CS + i];
    for (int i = tid; i < C * CS; i += NT) {
      const int r = i / CS, d = i % CS;
      sm.dO[r][d] = r < len ? load_f32(dO, (t0 + r) * dv + d0 + d) : 0.f;
    }
    for (int i = tid; i < C * DK; i += NT) {
      (&sm.dq[0][0])[i] = 0.f;
      (&sm.dk[0][0])[i] = 0.f;
      (&sm.dG[0][0])[i] = 0.f;
    }
    if (tid < DK) sm.dgam[tid] = 0.f;
    __syncthreads();
    chunk_forward<TIn, DK>(sm, p, bh, n, d0, dvs);

    // dU = P^T dO + Ktil dS'
    for (int i = tid; i < C * CS; i += NT) {
      const int j = i / CS, d = i % CS;
      float acc = 0.f;
      for (int r = j; r < C; ++r) acc += sm.P[r][j] * sm.dO[r][d];
      for (int c = 0; c < DK; ++c) acc += sm.k[j][c] * expf(sm.gam[c] - sm.G[j][c]) * sm.dS[c][d];
      sm.dU[j][d] = acc;
    }
    __syncthreads();
    // dR = T^T dU, dv = diag(beta) dR
    for (int i = tid; i < C * CS; i += NT) {
      const int j = i / CS, d = i % CS;
      float acc = 0.f;
      for (int r = j; r < C; ++r) acc += sm.T[r][j] * sm.dU[r][d];
      sm.dR[j][d] = acc;
      if (j < len) dvo[(bh * T + t0 + j) * dv + d0 + d] = sm.beta[j] * acc;
    }
    __syncthreads();
    // dT = dU R^T (lower part), dP = dO U^T (lower, diagonal included)
    {
      const int r = tid / C, j = tid % C;
      float a = 0.f, b = 0.f;
      if (j <= r) {
        for (int d = 0; d < CS; ++d) {
          a += sm.dU[r][d] * sm.R[j][d];
          b += sm.dO[r][d] * sm.U[j][d];
        }
      }
      sm.dT[r][j] = j <= r ? a : 0.f;
      sm.dP[r][j] = j <= r ? b : 0.f;
    }
    __syncthreads();
    // M = T^T dT, then dA = -(M T^T), strictly lower
    {
      const int a = tid / C, b = tid % C;
      float acc = 0.f;
      for (int r = 0; r < C; ++r) acc += sm.T[r][a] * sm.dT[r][b];
      sm.M[a][b] = acc;
    }
    __syncthreads();
    {
      const int a = tid / C, b = tid % C;
      float acc = 0.f;
      for (int j = 0; j < C; ++j) acc += sm.M[a][j] * sm.T[b][j];
      sm.dA[a][b] = b < a ? -acc : 0.f;
    }
    __syncthreads();
    // dbeta_r = sum_d dR E + sum_j dA X (this block of columns' share)
    if (tid < C) {
      const int r = tid;
      float acc = 0.f;
      for (int d = 0; d < CS; ++d) acc += sm.dR[r][d] * sm.E[r][d];
      for (int j = 0; j < r; ++j) acc += sm.dA[r][j] * sm.X[r][j];
      if (r < len) atomicAdd(&dbeta[bh * T + t0 + r], acc);
    }
    // pair-by-pair terms of X (weighted beta_r dA) and P (weighted dP): one key channel per thread,
    // which owns column c of the gradient blocks
    if (tid < DK) {
      const int c = tid;
      for (int r = 0; r < C; ++r) {
        const float kr = sm.k[r][c], qr = sm.q[r][c], Gr = sm.G[r][c];
        for (int j = 0; j <= r; ++j) {
          const float e = expf(Gr - sm.G[j][c]);
          const float kj = sm.k[j][c];
          const float wa = j < r ? sm.beta[r] * sm.dA[r][j] : 0.f;
          const float wp = sm.dP[r][j];
          // X: d/dk_r = k_j e, d/dk_j = k_r e, d/dG_r = k_r k_j e = -d/dG_j
          // P: d/dq_r = k_j e, d/dk_j = q_r e, d/dG_r = q_r k_j e = -d/dG_j
          sm.dk[r][c] += wa * kj * e;
          sm.dk[j][c] += (wa * kr + wp * qr) * e;
          sm.dq[r][c] += wp * kj * e;
          const float t = (wa * kr + wp * qr) * kj * e;
          sm.dG[r][c] += t;
          sm.dG[j][c] -= t;
        }
      }
    }
    __syncthreads();
    // dQbar = dO S^T, dKbar = -diag(beta) dR S^T, dKtil = U dS'^T, through the scalings
    for (int i = tid; i < C * DK; i += NT) {
      const int r = i / DK, c = i % DK;
      float a = 0.f, b = 0.f, t = 0.f;
      for (int d = 0; d < CS; ++d) {
        a += sm.dO[r][d] * sm.S[c][d];
        b += sm.dR[r][d] * sm.S[c][d];
        t += sm.U[r][d] * sm.dS[c][d];
      }
      const float eg = expf(sm.G[r][c]), et = expf(sm.gam[c] - sm.G[r][c]);
      const float dKbar = -sm.beta[r] * b;
      sm.dq[r][c] += a * eg;
      sm.dk[r][c] += dKbar * eg + t * et;
      sm.dG[r][c] += a * sm.q[r][c] * eg + dKbar * sm.k[r][c] * eg - t * sm.k[r][c] * et;
    }
    __syncthreads();
    // dGam = e^{Gam} rowsum(dS' o S) + sum_r dKtil o Ktil
    if (tid < DK) {
      const int c = tid;
      float acc = 0.f;
      for (int d = 0; d < CS; ++d) acc += sm.dS[c][d] * sm.S[c][d];
      acc *= expf(sm.gam[c]);
      for (int r = 0; r < C; ++r) {
        float t = 0.f;
        for (int d = 0; d < CS; ++d) t += sm.U[r][d] * sm.dS[c][d];
        acc += t * sm.k[r][c] * expf(sm.gam[c] - sm.G[r][c]);
      }
      sm.dgam[c] = acc;
    }
    __syncthreads();
    // dS <- e^{Gam} dS' + Qbar^T dO - Kbar^T diag(beta) dR
    for (int i = tid; i < DK * CS; i += NT) {
      const int c = i / CS, d = i % CS;
      float acc = expf(sm.gam[c]) * sm.dS[c][d];
      for (int r = 0; r < C; ++r) {
        const float eg = expf(sm.G[r][c]);
        acc += sm.q[r][c] * eg * sm.dO[r][d] - sm.k[r][c] * eg * sm.beta[r] * sm.dR[r][d];
      }
      sm.dS[c][d] = acc;
    }
    // dg = reverse prefix of dG plus dGam; dw = dg gate'(w); this block's shares of dq, dk, dw
    if (tid < DK) {
      const int c = tid;
      float acc = sm.dgam[c];
      for (int r = C - 1; r >= 0; --r) {
        acc += sm.dG[r][c];
        if (r < len) {
          const int64_t idx = (bh * T + t0 + r) * DK + c;
          atomicAdd(&dw[idx], acc * gate_deriv(load_f32(w, idx - bh * T * DK), p.g_min, p.unbounded));
          atomicAdd(&dq[idx], sm.dq[r][c]);
          atomicAdd(&dk[idx], sm.dk[r][c]);
        }
      }
    }
    __syncthreads();
  }
  if (dS0) {
    for (int i = tid; i < DK * CS; i += NT) {
      const int c = i / CS, d = i % CS;
      dS0[(bh * DK + c) * dv + d0 + d] = sm.dS[c][d];
    }
  }
}

__global__ void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) x[i] = 0.f;
}

hipError_t zero(float* x, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

template <typename TIn, int DK>
hipError_t launch_bwd_dk(const BwdParams& b, hipStream_t s) {
  const Params& p = b.p;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_kernel<TIn, DK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(BwdShared<DK>));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)(p.B * p.H * (p.dv / CS));
  hipLaunchKernelGGL((bwd_kernel<TIn, DK>), dim3(grid), dim3(NT), sizeof(BwdShared<DK>), s, p, b.dO, b.dSf, b.dq,
                     b.dk, b.dv, b.dw, b.dbeta, b.dS0);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_bwd_t(const BwdParams& b, hipStream_t s) {
  switch (b.p.dk) {
    case 32: return launch_bwd_dk<TIn, 32>(b, s);
    case 64: return launch_bwd_dk<TIn, 64>(b, s);
    default: return launch_bwd_dk<TIn, 128>(b, s);
  }
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv) {
  const int64_t NC = (T + C - 1) / C;
  return (size_t)(B * H * NC * dk * dv) * sizeof(float);
}

hipError_t launch_bwd(const BwdParams& b, hipStream_t s) {
  const Params& p = b.p;
  hipError_t e;
  const int64_t nk = p.B * p.H * p.T * p.dk;
  if ((e = zero(b.dq, nk, s)) != hipSuccess) return e;
  if ((e = zero(b.dk, nk, s)) != hipSuccess) return e;
  if ((e = zero(b.dw, nk, s)) != hipSuccess) return e;
  if ((e = zero(b.dbeta, p.B * p.H * p.T, s)) != hipSuccess) return e;
  return p.dtype == KDA_DTYPE_BF16 ? launch_bwd_t<uint16_t>(b, s) : launch_bwd_t<float>(b, s);
}

}  // namespace kda

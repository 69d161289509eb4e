// Backward pass of the chunked KDA forward: gradients of a loss L with respect to q, k, v, w, beta
// and S0, given dL/do and dL/dS_final, in fp32 (matrix cores and vector ALUs).
//
// The forward of one 16-token chunk (entering state S, chunk-local inclusive prefix G of the
// log-decay, span Gam = G at the last row; "From Numerical Stability to Load Balancing ..."
// section 2.1), in the form this file differentiates:
//   X[r][j] = sum_c k_rc k_jc e^{G_rc - G_jc}   (j < r)      A = diag(beta) X
//   P[r][j] = sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)     T = (I + A)^{-1}
//   E = V - Kbar S,  R = diag(beta) E,  U = T R,  O = Qbar S + P U,  S' = e^{Gam} S + Ktil^T U
// with Kbar = k e^{G}, Qbar = q e^{G}, Ktil = k e^{Gam - G}.  X, P and the pair terms of the
// gradients through them are products of e^{+-(G - Gam/2)} factors (each at most e^{40}) for chunks
// whose every channel spans at least -80, and are formed pair by pair with factors
// exp(G_r - G_j) <= 1 (the per-position form the pages give for chunks whose reciprocal factors
// would overflow) for the others.
//
// With W = T diag(beta) Kbar and U0 = T diag(beta) V (the WY form: U = U0 - W S) the two chains
// through the chunks are affine and cheap:
//   S'      = e^{Gam} S + Ktil^T (U0 - W S)                                   (forward)
//   dS      = e^{Gam} dS' + Qbar^T dO - W^T (P^T dO + Ktil dS')                (reverse)
// and, given S and dS' of a chunk, everything else is local to it:
//   dU = P^T dO + Ktil dS'        dR = T^T dU        dv = diag(beta) dR
//   dT = dU R^T  ->  dA = -T^T dT T^T (strictly lower)      dP = dO U^T (lower, diagonal included)
//   dbeta_r = sum_d dR[r][d] E[r][d] + sum_j dA[r][j] X[r][j]
//   X, P (pair terms) -> dk, dq, dG;   dQbar = dO S^T,  dKbar = -diag(beta) dR S^T,  dKtil = U dS'^T
//   dg_u = e^{Gam} . rowsum(dS' o S) + sum_{r >= u} dG_r + sum_{r < u} (dKtil o Ktil)_r,  dw = dg gate'(w)
// (the Ktil scaling's share of dG, -dKtil o Ktil per row, and of dGam, its column sum, are combined
// into the sum over the earlier rows: in strongly decaying chunks the two long sums nearly cancel)
//
// Three launches:
//   prep   (one workgroup per chunk)            G, X, P, T -> W, Ktil, Qbar, U0, P^T dO, e^{Gam} records
//   chain  (one per head, 16 value columns and  forward chain: stores every chunk's entering state;
//           chain; both chains in one launch)   reverse chain: stores every chunk's exit adjoint, dS0
//   grad   (one per chunk)                      all gradients of the chunk, written once (no atomics)
// Only the chains are sequential; they are independent of each other, and each does two small
// contractions per chunk (three in the reverse one).
#include <cstdlib>
#include <cstring>

#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;      // 16
constexpr int NPAIR = C * (C + 1) / 2;
constexpr int CH = 16;         // value columns per chain workgroup
constexpr int kDepth = 4;      // chunks of chain operands in flight (an LDS ring of kDepth slots)
constexpr int NTP = 512;       // prep threads
constexpr int NTG = 512;       // grad threads

// Record of one chunk (fp32): W [C][dk], Ktil [C][dk], Qbar [C][dk], U0 [C][dv], Z0 = P^T dO [C][dv],
// e^{Gam} [dk]
__host__ __device__ __forceinline__ int64_t rec_floats(int64_t dk, int64_t dv) {
  return 3 * C * dk + 2 * C * dv + dk;
}
__host__ __device__ __forceinline__ int64_t off_kt(int64_t dk) { return C * dk; }
__host__ __device__ __forceinline__ int64_t off_qb(int64_t dk) { return 2 * C * dk; }
__host__ __device__ __forceinline__ int64_t off_u0(int64_t dk) { return 3 * C * dk; }
__host__ __device__ __forceinline__ int64_t off_z0(int64_t dk, int64_t dv) { return 3 * C * dk + C * dv; }
__host__ __device__ __forceinline__ int64_t off_eg(int64_t dk, int64_t dv) { return 3 * C * dk + 2 * C * dv; }

struct WsLayout {
  float *recs, *states, *dstates;
};

__host__ __device__ __forceinline__ WsLayout ws_layout(void* ws, int64_t BH, int64_t NC, int64_t dk, int64_t dv) {
  WsLayout L;
  L.recs = (float*)ws;
  L.states = L.recs + BH * NC * rec_floats(dk, dv);
  L.dstates = L.states + BH * NC * dk * dv;
  return L;
}

constexpr float kLog2eB = 1.4426950408889634f;
constexpr float kLn2B = 0.6931471805599453f;

// 2^x on the transcendental unit (one instruction; exponents here are <= 0 or small)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// barrier that waits for this wave's LDS operations only (global loads and stores stay in flight)
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// four consecutive elements p[i .. i + 3] as fp32 (i a multiple of 4; rows start 16-byte aligned)
__device__ __forceinline__ float4 load4_f32(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 load4_f32(const uint16_t* p, int64_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}

// value of lane src (0..3) of this lane's group of four, through a DPP quad permute
__device__ __forceinline__ float quad_bcast(float v, int src) {   // src is a constant after unrolling
  const int b = __float_as_int(v);
  switch (src) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false));
  }
}

// one 16 x 16 x 4 fp32 matrix-core step: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; the
// accumulator holds D[4 (l / 16) + i][l % 16] in register i
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// gate derivative d g / d w: g_min sigma (1 - sigma), or -sigma for -softplus
__device__ __forceinline__ float gate_deriv(float w, float g_min, int unbounded) {
  const float s = __builtin_amdgcn_rcpf(1.f + ex2(-w * kLog2eB));
  return unbounded ? -s : g_min * s * (1.f - s);
}

__device__ __forceinline__ void pair_of(int pr, int& r, int& j) {   // pr -> (r, j), j <= r < 16
  r = 0;
  while ((r + 1) * (r + 2) / 2 <= pr) ++r;
  j = pr - r * (r + 1) / 2;
}

// Phase stamps of one chain workgroup (the phase-stamp build, libkda_stamps.so, only; the product
// build compiles the calls away): lane 0 of wavefront w records the shader clock at boundary k of step
// n into the end of the workspace.  Kernel 0 is the chain kernel (steps: chunks), 1 the gradient
// kernel (steps 0-7: value tiles, 8: the setup, 9: the epilogue, 10: inside the chunk setup, which
// the prep kernel's workgroup of the same index stamps too, before the gradient kernel overwrites it).
#if KDA_PHASE_STAMPS
__device__ __forceinline__ void bwd_stamp(const Params& p, int kernel, int w, int64_t n, int k) {
  if (p.stamp_kernel != kernel || (int)blockIdx.x != p.stamp_block || n < 0 || n >= kStampSteps ||
      (threadIdx.x & 63) != 0)
    return;
  unsigned long long* pr = (unsigned long long*)((unsigned char*)p.workspace + p.stamp_off);
  pr[(w * kStampSteps + n) * kStampK + k] = __builtin_amdgcn_s_memtime();
}
#define KDA_BWD_STAMP(p, w, n, k) bwd_stamp(p, 0, w, n, k)
#define KDA_GRAD_STAMP(p, w, n, k) bwd_stamp(p, 1, w, n, k)
#else
#define KDA_BWD_STAMP(p, w, n, k) ((void)0)
#define KDA_GRAD_STAMP(p, w, n, k) ((void)0)
#endif

// G and gam are kept in log2 units (G * log2 e), so that every factor e^{G...} is one exp2; the
// gradients stay with respect to the natural-unit G.  Rows are padded by one float so that reads of
// one channel across rows fall on distinct LDS banks.
template <int DK>
struct ChunkCore {
  float q[C][DK + 1], k[C][DK + 1], G[C][DK + 1];
  float gam[DK];
  float beta[C];
  float X[C][C + 1], P[C][C + 1], T[C][C + 1], Tb[C][C + 1];   // Tb = T diag(beta)
  float spanw[(DK + 63) / 64];   // per wavefront of the prefix: the smallest chunk total of its channels
  // every channel's span >= -80: pair terms as products of e^{+-(G - Gam/2)} factors (valid after the
  // barrier that follows the prefix)
  __device__ __forceinline__ bool dense() const {
    float m = spanw[0];
#pragma unroll
    for (int i = 1; i < (DK + 63) / 64; ++i) m = fminf(m, spanw[i]);
    return m * kLn2B >= kSpanLimit;
  }
};

// Loads chunk n (rows past the end are zero: k = q = beta = 0 and g = 0, which reproduces the
// shorter last chunk exactly), forms the prefix G and Gam, the chunk's span flag (dense: every
// channel's span >= -80), X and P (dense chunks: fp32 matrix-core products of e^{+-(G - Gam/2)}
// factors, four wavefronts with two key blocks each; other chunks: pair by pair, each pair's sums
// split over groups of key channels; partial sums through `scratch`, 2 * 4 * 256 floats), and T by
// back substitution, the four lanes of a quad owning one row.  Ends with a barrier.
template <typename TIn, int DK, int NT>
__device__ void chunk_setup(ChunkCore<DK>& cc, float* scratch, const Params& p, int64_t bh, int64_t n, int len) {
  constexpr int NQ = NT >= 4 * NPAIR ? 4 : (NT >= 3 * NPAIR ? 3 : (NT >= 2 * NPAIR ? 2 : 1));   // channel groups
  const int tid = threadIdx.x;
  const int64_t T = p.T, t0 = n * C;
  const TIn* q = (const TIn*)p.q + bh * T * DK;
  const TIn* k = (const TIn*)p.k + bh * T * DK;
  const TIn* w = (const TIn*)p.w + bh * T * DK;
  const TIn* beta = (const TIn*)p.beta + bh * T;
  {   // every load issued before the first use, four channels per thread, with no branch around a load
      // (addresses clamped into the chunk, rows past its end zeroed afterwards)
    constexpr int N4 = C * DK / 4, PER = (N4 + NT - 1) / NT;
    float4 lq[PER], lk[PER], lw[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = min(tid + m * NT, N4 - 1);
      const int r = min(4 * i / DK, len - 1), c = 4 * i % DK;
      const int64_t idx = (t0 + r) * DK + c;
      lq[m] = load4_f32(q, idx);
      lk[m] = load4_f32(k, idx);
      lw[m] = load4_f32(w, idx);
    }
    const float lb = load_f32(beta, t0 + min(tid % C, len - 1));
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = tid + m * NT;
      if (i < N4) {
        const int r = 4 * i / DK, c = 4 * i % DK;
        const bool ok = r < len;
        const float qv[4] = {lq[m].x, lq[m].y, lq[m].z, lq[m].w};
        const float kv[4] = {lk[m].x, lk[m].y, lk[m].z, lk[m].w};
        const float wv[4] = {lw[m].x, lw[m].y, lw[m].z, lw[m].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cc.q[r][c + j] = ok ? qv[j] : 0.f;
          cc.k[r][c + j] = ok ? kv[j] : 0.f;
          cc.G[r][c + j] = ok ? gate_f32(wv[j], p.g_min, p.unbounded) * kLog2eB : 0.f;
        }
      }
    }
    if (tid < C) cc.beta[tid] = tid < len ? lb : 0.f;
  }
  KDA_GRAD_STAMP(p, tid / 64, 10, 0);
  __syncthreads();
  KDA_GRAD_STAMP(p, tid / 64, 10, 1);
  if (tid < DK) {
    float gv[C];
#pragma unroll
    for (int r = 0; r < C; ++r) gv[r] = cc.G[r][tid];
    float g = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) { g += gv[r]; cc.G[r][tid] = g; }
    cc.gam[tid] = g;
    // the chunk flag: each wavefront's smallest total over its own channels (all of them active), the
    // minimum over the wavefronts taken after the barrier
    float m = fminf(g, 0.f);
#pragma unroll
    for (int off = (DK < 64 ? DK : 64) / 2; off > 0; off >>= 1) m = fminf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) cc.spanw[tid >> 6] = m;
  }
  __syncthreads();
  KDA_GRAD_STAMP(p, tid / 64, 10, 2);
  float (*xs)[C][C] = reinterpret_cast<float (*)[C][C]>(scratch);              // [4][C][C] partial sums
  float (*ps)[C][C] = reinterpret_cast<float (*)[C][C]>(scratch + 4 * C * C);
  const bool dense = cc.dense();
  if (dense) {
    // X = Kbar' Kinv'^T, P = Qbar' Kinv'^T with Kbar' = k e^{G - Gam/2}, Kinv' = k e^{Gam/2 - G} (every
    // factor at most e^{40}): wavefront wq < 4 takes key blocks wq and wq + 4, K order c = 16 cb + 4g + i
    const int wq = tid / 64, lane = tid % 64, li = lane % 16, g = lane / 16;
    if (wq < 4) {
      f32x4 xa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int cb = wq + 4 * bb;
        if (cb < DK / 16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = 16 * cb + 4 * g + i;
            const float Gs = cc.G[li][c] - 0.5f * cc.gam[c];
            const float e = ex2(Gs), ei = ex2(-Gs), kv = cc.k[li][c];
            xa = mfma4(kv * e, kv * ei, xa);
            pa = mfma4(cc.q[li][c] * e, kv * ei, pa);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // lane (li, g) holds row 4g + i, column li
        xs[wq][4 * g + i][li] = xa[i];
        ps[wq][4 * g + i][li] = pa[i];
      }
    }
  } else {
    for (int task = tid; task < NPAIR * NQ; task += NT) {
      const int pr = task % NPAIR, qq = task / NPAIR;
      int r, j;
      pair_of(pr, r, j);
      float x = 0.f, pp = 0.f;
#pragma unroll 8
      for (int c = qq; c < DK; c += NQ) {
        const float kj = cc.k[j][c] * ex2(cc.G[r][c] - cc.G[j][c]);
        x += cc.k[r][c] * kj;
        pp += cc.q[r][c] * kj;
      }
      xs[qq][r][j] = x;
      ps[qq][r][j] = pp;
    }
  }
  __syncthreads();
  KDA_GRAD_STAMP(p, tid / 64, 10, 3);
  {
    const int nq = dense ? 4 : NQ;
    for (int e = tid; e < 2 * C * C; e += NT) {   // X from threads 0..255, P from 256..511
      const int which = e / (C * C), r = (e % (C * C)) / C, j = e % C;
      float (*src)[C][C] = which ? ps : xs;
      float x = 0.f;
      if (j <= r)
        for (int qq = 0; qq < nq; ++qq) x += src[qq][r][j];
      if (which) cc.P[r][j] = x;
      else cc.X[r][j] = j < r ? x : 0.f;
    }
  }
  __syncthreads();
  KDA_GRAD_STAMP(p, tid / 64, 10, 4);
  if (tid < 64) {
    // T = (I + A)^{-1}, A = diag(beta) X: the four lanes of quad li own row li of T, lane q of the quad
    // columns 4q .. 4q+3.  Row t of T satisfies t (I + A) = e_li, so its entries follow from the last one
    // backwards: once t_m is final (lane m/4 of the quad, broadcast inside the quad), t_k -= t_m A[m][k].
    const int li = tid >> 2, q = tid & 3;
    // every row of X this lane needs (its four columns) and beta, read before the serial steps so
    // that no step waits on LDS
    float xm[C][4], bm[C];
#pragma unroll
    for (int m = 1; m < C; ++m) {
      bm[m] = cc.beta[m];
#pragma unroll
      for (int c = 0; c < 4; ++c) xm[m][c] = cc.X[m][4 * q + c];
    }
    float t[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = (li == 4 * q + c) ? 1.f : 0.f;
#pragma unroll
    for (int m = C - 1; m >= 1; --m) {
      const float x = quad_bcast(t[m & 3], m >> 2) * bm[m];
#pragma unroll
      for (int c = 0; c < 4; ++c) t[c] -= x * xm[m][c];   // X[m][j] = 0 for j >= m
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cc.T[li][4 * q + c] = t[c];
      cc.Tb[li][4 * q + c] = t[c] * cc.beta[4 * q + c];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- prep: one workgroup per chunk
template <int DK>
struct PrepShared {
  ChunkCore<DK> cc;
  float kb[C][DK];      // diag(beta) Kbar
  float bv[C][128];     // diag(beta) V
  float go[C][128];     // dO
};

template <typename TIn, int DK>
__global__ __launch_bounds__(NTP) void bwd_prep_kernel(Params p, const void* __restrict__ dO_in, float* __restrict__ recs) {
  __shared__ PrepShared<DK> sm;
  const int tid = threadIdx.x;
  const int64_t NC = p.n_chunks();
  const int64_t bh = blockIdx.x / NC, n = blockIdx.x % NC;
  const int64_t T = p.T, t0 = n * C;
  const int len = (int)((T - t0) < C ? (T - t0) : C);
  const int dv = (int)p.dv;
  const TIn* v = (const TIn*)p.v + bh * T * dv;
  const TIn* dO = (const TIn*)dO_in + bh * T * dv;
  constexpr int PER = C * 128 / NTP;          // dv <= 128
  float lv[PER], lo[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {             // issued with the setup's loads: one memory latency
    const int i = tid + m * NTP, r = i / dv, d = i % dv;
    const bool ok = i < C * dv && r < len;
    const int64_t o = (t0 + min(r, len - 1)) * dv + (i < C * dv ? d : 0);   // no branch around the load
    const float x = load_f32(v, o), y = load_f32(dO, o);
    lv[m] = ok ? x : 0.f;
    lo[m] = ok ? y : 0.f;
  }
  chunk_setup<TIn, DK, NTP>(sm.cc, &sm.bv[0][0], p, bh, n, len);   // bv, go: 2 * 4 * 256 floats of scratch
  float* rec = recs + (bh * NC + n) * rec_floats(DK, dv);
  for (int i = tid; i < C * DK; i += NTP) {
    const int r = i / DK, c = i % DK;
    const float G = sm.cc.G[r][c], eG = ex2(G);
    sm.kb[r][c] = sm.cc.beta[r] * sm.cc.k[r][c] * eG;
    rec[off_kt(DK) + i] = sm.cc.k[r][c] * ex2(sm.cc.gam[c] - G);
    rec[off_qb(DK) + i] = sm.cc.q[r][c] * eG;
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = tid + m * NTP, r = i / dv, d = i % dv;
    if (i < C * dv) {
      sm.bv[r][d] = sm.cc.beta[r] * lv[m];
      sm.go[r][d] = lo[m];
    }
  }
  if (tid < DK) rec[off_eg(DK, dv) + tid] = ex2(sm.cc.gam[tid]);
  lds_barrier();                              // orders LDS only: the record stores stay in flight
  // W = T diag(beta) Kbar, U0 = T diag(beta) V, Z0 = P^T dO on the fp32 matrix cores, one 16 x 16 output
  // tile per task (T and P are triangular with zeros stored outside), K index 4s + g at step s
  {
    const int lane = tid % 64, wv = tid / 64, col = lane % 16, g = lane / 16;
    const int nk = DK / 16, nvb = dv / 16;
    for (int task = wv; task < nk + 2 * nvb; task += NTP / 64) {
      const int kind = task < nk ? 0 : (task < nk + nvb ? 1 : 2);
      const int cb = kind == 0 ? task : (kind == 1 ? task - nk : task - nk - nvb);
      const int c = 16 * cb + col;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kk = 4 * s4 + g;
        const float a = kind == 2 ? sm.cc.P[kk][col] : sm.cc.T[col][kk];
        const float b = kind == 0 ? sm.kb[kk][c] : (kind == 1 ? sm.bv[kk][c] : sm.go[kk][c]);
        acc = mfma4(a, b, acc);
      }
      float* dst = rec + (kind == 0 ? 0 : (kind == 1 ? off_u0(DK) : off_z0(DK, dv)));
      const int N = kind == 0 ? DK : dv;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(4 * g + i) * N + c] = acc[i];
    }
  }
}

// ---------------------------------------------------------------- chains
// One workgroup per (head, 16 value columns); compute wavefront w holds rows 32w .. 32w + 31 of the
// block as two fp32 matrix-core accumulator tiles (tile b, lane l: rows 32w + 16b + 4(l/16) + i, i < 4,
// column l % 16).  Per chunk: a 16 x 16 x 32 product per wavefront (its 32-key share of a K = dk
// contraction), written to LDS; after one barrier every wavefront sums all shares itself, in the
// same lane layout, and the update is one more product on each tile.  The K index of each 16 x 16 x 4 step is taken in the
// order the accumulator already holds its rows (row 4(l/16) + i at step i), so neither the state
// nor the summed shares need a reshuffle to serve as the B operand.
//
// Roles: compute wavefronts do the products and store the chain's states (stores only, never
// waited on); loader wavefronts copy each chunk's operands from its record straight into a ring of
// LDS slots (16-byte global-to-LDS loads, kDepth chunks ahead).  All reads of a chunk's slot come
// before the step's barrier, so right after it the loaders refill that slot with the chunk kDepth
// steps ahead, having made sure (before the barrier) that the next step's chunk has landed.
//
// Operand matrices [16][dk] sit in a slot as float4 units, row r's unit c4 at r * dk/4 + (c4 ^ r % (dk/4)),
// so that the 16 rows a matrix-core operand read touches fall on distinct LDS banks.
//
// States are stored in the accumulator's own order: the [dk][16] block of (head, chunk, columns
// 16j .. 16j + 15) is contiguous, element (row 16w + 4g + i, column cl) at w*256 + i*64 + g*16 + cl.

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

// wait until at most N of this wave's vector-memory operations are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  compiler_fence();
}

// 16 bytes from global memory to LDS: lane j of the wave writes dst_base + 16 j
__device__ __forceinline__ void dma16(const void* src, void* dst_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)dst_base, 16, 0, 0);
}

// blocks of one head on one XCD (consecutive block ids go round-robin over the 8 XCDs)
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nblocks) {
  return (nblocks % 8) ? b : (b % 8) * (nblocks / 8) + b / 8;
}

template <int DK>
__device__ __forceinline__ int swz(int r, int c4) {   // float4 unit of (r, c4) in a [16][DK] matrix
  constexpr int Q = DK / 4;
  return r * Q + (c4 ^ (r % Q));
}

// Per-chunk slot contents (float4 units), for the two chains
template <int DK, int NMAT, bool WITH_DO, typename TIn>
struct ChainSlot {
  static constexpr int Q = DK / 4;
  static constexpr int MAT = C * Q;                               // units of one [16][DK] matrix
  static constexpr int VEC = C * CH / 4;                          // U0 or Z0 slice, [16][16] fp32
  static constexpr int DOU = WITH_DO ? C * CH * (int)sizeof(TIn) / 16 : 0;   // dO slice
  static constexpr int EG = Q;                                    // e^{Gam}
  static constexpr int UNITS = NMAT * MAT + VEC + DOU + EG;
  static constexpr int O_VEC = NMAT * MAT, O_DO = O_VEC + VEC, O_EG = O_DO + DOU;
  static constexpr int NI = (UNITS + 63) / 64;                    // wave instructions per chunk
};


template <int DK>
struct ChainDims {
  static constexpr int RT = 2;                // 16-row tiles per compute wavefront
  static constexpr int NW = DK / (16 * RT);   // compute wavefronts
  static constexpr int NL = 4;                // loader wavefronts
  static constexpr int NT = (NW + NL) * 64;
};

// One loader lane's share of a chunk's operand copies into an LDS slot (float4 units).  Unit u of
// the slot comes from: matrix rows of the record (un-swizzled), the 16 x 16 vector block (U0 or Z0),
// the dO rows of tokens t0 .. t0 + 15 (clamped to the last token; the compute side zeroes rows past
// the end), e^{Gam}.  Every loader wave issues exactly PER instructions per chunk.  Where each of
// this lane's units comes from is the same for every chunk up to the chunk's base (its record, or
// its first token's dO row), so the offsets are worked out once.
template <int DK, int NMAT, bool WITH_DO, typename TIn>
struct SlotPlan {
  using SL = ChainSlot<DK, NMAT, WITH_DO, TIn>;
  static constexpr int NL = ChainDims<DK>::NL;
  static constexpr int PER = (SL::NI + NL - 1) / NL;
  int off[PER];    // bytes from the record, or (row >= 0) from the start of dO row t0 + row
  int row[PER];
  bool on[PER];
  int lw;

  __device__ __forceinline__ SlotPlan(int64_t off_vec, int64_t off_eg, int dv, int d0, int lw_, int lane) : lw(lw_) {
    constexpr int Q = SL::Q;
    constexpr int UPR = CH * (int)sizeof(TIn) / 16;          // dO units per row
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int u = ins(k) * 64 + lane;
      on[k] = u < SL::UNITS;
      row[k] = -1;
      if (u < SL::O_VEC) {
        const int mat = u / SL::MAT, vm = u % SL::MAT, r = vm / Q, c4 = (vm % Q) ^ (r % Q);
        off[k] = 4 * (mat * C * DK + r * DK + 4 * c4);
      } else if (u < SL::O_DO) {
        const int vv = u - SL::O_VEC;
        off[k] = 4 * ((int)off_vec + (vv / 4) * dv + d0 + 4 * (vv % 4));
      } else if (u < SL::O_EG) {
        const int vd = u - SL::O_DO;
        row[k] = vd / UPR;
        off[k] = (int)sizeof(TIn) * d0 + 16 * (vd % UPR);
      } else {
        off[k] = 4 * ((int)off_eg + 4 * min(u - SL::O_EG, Q - 1));
      }
    }
  }
  // instruction k of this wave (the last one repeated where the waves' shares are uneven: same
  // bytes to the same place)
  __device__ __forceinline__ int ins(int k) const { return min(lw + k * NL, SL::NI - 1); }

  __device__ __forceinline__ void issue(float4* slot, const float* rec, const TIn* dO_head, int64_t t0, int64_t T,
                                        int dv) const {
    const char* rb = reinterpret_cast<const char*>(rec);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const char* src = rb + off[k];
      if (WITH_DO && row[k] >= 0) {
        const int64_t t = min(t0 + row[k], T - 1);
        src = reinterpret_cast<const char*>(dO_head + t * dv) + off[k];
      }
      if (on[k]) dma16(src, slot + ins(k) * 64);
    }
  }
};

template <typename TIn, int DK>
struct ChainLds {   // float4 units of LDS: the ring (sized for the reverse chain's larger slot), partial sums
  using Dm = ChainDims<DK>;
  static constexpr int R = kDepth;
  static constexpr int SLOT = ChainSlot<DK, 3, true, TIn>::UNITS;
  static constexpr int PART = 2 * Dm::NW * 64;   // [step parity][wavefront][lane]
  static constexpr int UNITS = R * SLOT + PART;
};

// forward chain: states[n] = S entering chunk n.  Per chunk, with S held as described above:
//   Y = U0 - W S (16 x 16 x dk, one 16-key share per wavefront, partials summed by every wavefront)
//   S <- e^{Gam} S + Ktil^T Y
// The operands of step n + 1 are read from LDS right after step n's barrier, while step n's update runs.
template <typename TIn, int DK>
__device__ __forceinline__ void state_chain(const Params& p, const float* __restrict__ recs,
                                            float* __restrict__ states, float4* smem, int64_t L) {
  using Dm = ChainDims<DK>;
  using SL = ChainSlot<DK, 2, false, float>;
  using LD = ChainLds<TIn, DK>;
  using Plan = SlotPlan<DK, 2, false, float>;
  constexpr int NW = Dm::NW, R = LD::R, PER = Plan::PER;
  float4 (*part)[NW][64] = reinterpret_cast<float4 (*)[NW][64]>(smem + R * LD::SLOT);
  const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
  const bool loader = w >= NW;
  const int dv = (int)p.dv, nsl = dv / CH;
  const int64_t bh = L / nsl;
  const int sl = (int)(L % nsl), d0 = sl * CH;
  const int64_t NC = p.n_chunks();
  const int64_t RF = rec_floats(DK, dv);
  const float* rec_bh = recs + bh * NC * RF;
  const int col = lane % 16, g = lane / 16;

  if (loader) {
    const Plan plan(off_u0(DK), off_eg(DK, dv), dv, d0, w - NW, lane);
    auto issue = [&](int64_t m) {           // chunk m (clamped) into its ring slot
      const int64_t mc = m < NC ? m : NC - 1;
      plan.issue(smem + (m % R) * LD::SLOT, rec_bh + mc * RF, (const float*)nullptr, 0, 1, dv);
    };
#pragma unroll
    for (int k = 0; k < kDepth; ++k) issue(k);
    vm_wait<PER * (kDepth - 2)>();            // chunks 0 and 1 have landed
    lds_barrier();
    for (int64_t n = 0; n < NC; ++n) {
      KDA_BWD_STAMP(p, w, n, 0);
      vm_wait<PER * (kDepth - 2)>();          // chunk n + 1 has landed (n + 2 .. n + kDepth - 1 may not)
      KDA_BWD_STAMP(p, w, n, 1);
      lds_barrier();
      KDA_BWD_STAMP(p, w, n, 2);
      issue(n + kDepth);                      // into the slot chunk n used (all its reads were before)
      KDA_BWD_STAMP(p, w, n, 3);
    }
    vm_wait<0>();
    return;
  }

  constexpr int RT = Dm::RT;
  f32x4 acc[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.S0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] = p.S0[(bh * DK + 16 * (RT * w + b) + 4 * g + i) * dv + d0 + col];
    }
  }
  float wv[RT][4], ka[RT][4];
  f32x4 e4[RT], u0;
  auto operands = [&](int64_t n) {          // step n's operands from its slot
    const float4* sv = smem + (n % R) * LD::SLOT;
    const float* sf = reinterpret_cast<const float*>(sv);
    const float* kt = sf + 4 * SL::MAT;
#pragma unroll
    for (int b = 0; b < RT; ++b) {
      const int tb = RT * w + b, c = 16 * tb + col;
      const float4 x = sv[swz<DK>(col, 4 * tb + g)];          // W[col][16 tb + 4g + s]
      wv[b][0] = x.x; wv[b][1] = x.y; wv[b][2] = x.z; wv[b][3] = x.w;
      const float4 e = sv[SL::O_EG + 4 * tb + g];
      e4[b] = f32x4{e.x, e.y, e.z, e.w};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) ka[b][s4] = kt[4 * swz<DK>(4 * g + s4, c / 4) + c % 4];   // Ktil[4g + s][c]
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) u0[s4] = sf[4 * SL::O_VEC + (4 * g + s4) * CH + col];
  };
  lds_barrier();
  operands(0);
  for (int64_t n = 0; n < NC; ++n) {
    KDA_BWD_STAMP(p, w, n, 0);
    const int pb = (int)(n & 1);
    float* st = states + ((bh * NC + n) * nsl + sl) * DK * CH + RT * w * 256 + lane;
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[b * 256 + i * 64] = acc[b][i];
    f32x4 yp[RT];
#pragma unroll
    for (int b = 0; b < RT; ++b) yp[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int b = 0; b < RT; ++b) yp[b] = mfma4(wv[b][s4], acc[b][s4], yp[b]);
#pragma unroll
    for (int b = 1; b < RT; ++b) yp[0] += yp[b];
    part[pb][w][lane] = make_float4(yp[0][0], yp[0][1], yp[0][2], yp[0][3]);
    KDA_BWD_STAMP(p, w, n, 1);
    lds_barrier();
    KDA_BWD_STAMP(p, w, n, 2);
    f32x4 y = u0, eg[RT];
    float kc[RT][4];
#pragma unroll
    for (int b = 0; b < RT; ++b) {
      eg[b] = e4[b];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) kc[b][s4] = ka[b][s4];
    }
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float4 pv = part[pb][v][lane];
      y[0] -= pv.x; y[1] -= pv.y; y[2] -= pv.z; y[3] -= pv.w;
    }
    operands(n + 1);                         // landed before this barrier (a clamped copy past the end)
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] *= eg[b][i];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int b = 0; b < RT; ++b) acc[b] = mfma4(kc[b][s4], y[s4], acc[b]);
    KDA_BWD_STAMP(p, w, n, 3);
  }
}

// reverse chain: dstates[n] = dL/dS leaving chunk n; dS0 = dL/dS entering chunk 0.  Per chunk:
//   Z = Z0 + Ktil dS'  (partials summed by every wavefront as above)
//   dS <- e^{Gam} dS' + Qbar^T dO - W^T Z
// Qbar^T dO does not depend on the chain: it is formed for step it + 1 while step it's update runs.
template <typename TIn, int DK>
__device__ __forceinline__ void dstate_chain(const Params& p, const void* __restrict__ dO_in,
                                             const float* __restrict__ dSf, const float* __restrict__ recs,
                                             float* __restrict__ dstates, float* __restrict__ dS0, float4* smem,
                                             int64_t L) {
  using Dm = ChainDims<DK>;
  using SL = ChainSlot<DK, 3, true, TIn>;
  using LD = ChainLds<TIn, DK>;
  using Plan = SlotPlan<DK, 3, true, TIn>;
  constexpr int NW = Dm::NW, R = LD::R, PER = Plan::PER;
  float4 (*part)[NW][64] = reinterpret_cast<float4 (*)[NW][64]>(smem + R * LD::SLOT);
  const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
  const bool loader = w >= NW;
  const int dv = (int)p.dv, nsl = dv / CH;
  const int64_t bh = L / nsl;
  const int sl = (int)(L % nsl), d0 = sl * CH;
  const int64_t T = p.T, NC = p.n_chunks();
  const int64_t RF = rec_floats(DK, dv);
  const float* rec_bh = recs + bh * NC * RF;
  const TIn* dO = (const TIn*)dO_in + bh * T * dv;
  const int col = lane % 16, g = lane / 16;

  if (loader) {
    const Plan plan(off_z0(DK, dv), off_eg(DK, dv), dv, d0, w - NW, lane);
    auto issue = [&](int64_t it) {          // step it (chunk NC - 1 - it, clamped)
      int64_t m = NC - 1 - it;
      if (m < 0) m = 0;
      plan.issue(smem + (it % R) * LD::SLOT, rec_bh + m * RF, dO, m * C, T, dv);
    };
#pragma unroll
    for (int k = 0; k < kDepth; ++k) issue(k);
    vm_wait<PER * (kDepth - 2)>();
    lds_barrier();
    for (int64_t it = 0; it < NC; ++it) {
      KDA_BWD_STAMP(p, w, it, 0);
      vm_wait<PER * (kDepth - 2)>();
      KDA_BWD_STAMP(p, w, it, 1);
      lds_barrier();
      KDA_BWD_STAMP(p, w, it, 2);
      issue(it + kDepth);
      KDA_BWD_STAMP(p, w, it, 3);
    }
    vm_wait<0>();
    return;
  }

  constexpr int RT = Dm::RT;
  f32x4 acc[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (dSf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] = dSf[(bh * DK + 16 * (RT * w + b) + 4 * g + i) * dv + d0 + col];
    }
  }
  float kv[RT][4], wa[RT][4];
  f32x4 e4[RT], qd[RT], z0;
  auto operands = [&](int64_t it) {         // step it's operands from its slot, and its Qbar^T dO
    const float4* sv = smem + (it % R) * LD::SLOT;
    const float* sf = reinterpret_cast<const float*>(sv);
    const float* qb = sf + 4 * 2 * SL::MAT;
    const TIn* dOl = reinterpret_cast<const TIn*>(sv + SL::O_DO);
    const int64_t t0 = (NC - 1 - it) * C;
    float ob[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int r = 4 * g + s4;
      const float o = load_f32(dOl, r * CH + col);
      ob[s4] = t0 + r < T ? o : 0.f;                          // rows past the end hold a clamped copy
      z0[s4] = sf[4 * SL::O_VEC + r * CH + col];
    }
#pragma unroll
    for (int b = 0; b < RT; ++b) {
      const int tb = RT * w + b, c = 16 * tb + col;
      const float4 x = sv[SL::MAT + swz<DK>(col, 4 * tb + g)];   // Ktil[col][16 tb + 4g + s]
      kv[b][0] = x.x; kv[b][1] = x.y; kv[b][2] = x.z; kv[b][3] = x.w;
      const float4 e = sv[SL::O_EG + 4 * tb + g];
      e4[b] = f32x4{e.x, e.y, e.z, e.w};
      qd[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int r = 4 * g + s4;
        wa[b][s4] = -sf[4 * swz<DK>(r, c / 4) + c % 4];
        qd[b] = mfma4(qb[4 * swz<DK>(r, c / 4) + c % 4], ob[s4], qd[b]);
      }
    }
  };
  lds_barrier();
  operands(0);
  for (int64_t it = 0; it < NC; ++it) {
    KDA_BWD_STAMP(p, w, it, 0);
    const int64_t n = NC - 1 - it;
    const int pb = (int)(it & 1);
    float* st = dstates + ((bh * NC + n) * nsl + sl) * DK * CH + RT * w * 256 + lane;
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[b * 256 + i * 64] = acc[b][i];
    f32x4 zp[RT];
#pragma unroll
    for (int b = 0; b < RT; ++b) zp[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int b = 0; b < RT; ++b) zp[b] = mfma4(kv[b][s4], acc[b][s4], zp[b]);
#pragma unroll
    for (int b = 1; b < RT; ++b) zp[0] += zp[b];
    part[pb][w][lane] = make_float4(zp[0][0], zp[0][1], zp[0][2], zp[0][3]);
    KDA_BWD_STAMP(p, w, it, 1);
    lds_barrier();
    KDA_BWD_STAMP(p, w, it, 2);
    f32x4 z = z0, eg[RT], qc[RT];
    float wc[RT][4];
#pragma unroll
    for (int b = 0; b < RT; ++b) {
      eg[b] = e4[b];
      qc[b] = qd[b];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) wc[b][s4] = wa[b][s4];
    }
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float4 pv = part[pb][v][lane];
      z[0] += pv.x; z[1] += pv.y; z[2] += pv.z; z[3] += pv.w;
    }
    operands(it + 1);
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][i] = acc[b][i] * eg[b][i] + qc[b][i];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int b = 0; b < RT; ++b) acc[b] = mfma4(wc[b][s4], z[s4], acc[b]);
    KDA_BWD_STAMP(p, w, it, 3);
  }
  if (dS0) {
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS0[(bh * DK + 16 * (RT * w + b) + 4 * g + i) * dv + d0 + col] = acc[b][i];
  }
}

// both chains in one launch (they are independent): blocks [0, nchain) run the forward chain,
// [nchain, 2 nchain) the reverse one
template <typename TIn, int DK>
__global__ __launch_bounds__(ChainDims<DK>::NT) void bwd_chain_kernel(Params p, const void* __restrict__ dO_in,
                                                                      const float* __restrict__ dSf,
                                                                      const float* __restrict__ recs,
                                                                      float* __restrict__ states,
                                                                      float* __restrict__ dstates,
                                                                      float* __restrict__ dS0) {
  __shared__ __align__(16) float4 smem[ChainLds<TIn, DK>::UNITS];
  const int64_t nchain = p.B * p.H * (p.dv / CH);
  const int64_t b = blockIdx.x;
  if (b < nchain) state_chain<TIn, DK>(p, recs, states, smem, xcd_block(b, nchain));
  else dstate_chain<TIn, DK>(p, dO_in, dSf, recs, dstates, dS0, smem, xcd_block(b - nchain, nchain));
}

// ---------------------------------------------------------------- grad: one workgroup per chunk
// The chunk's value columns are taken one 16-column tile at a time (the stored [dk][16] blocks of
// S and dS', copied into LDS one tile ahead).  Per tile, on the fp32 matrix cores:
//   E = V - Kbar S and Ktil dS' (K = dk, split over the wavefronts, partial sums through LDS)
//   dQbar += dO S^T, dKbar' += dR S^T, dKtil += U dS'^T (K = 16; one (product, 16-key block) task per
//   wavefront slot, accumulated over the tiles in registers)
// and on the vector ALUs the 16 x 16 blocks U = T diag(beta) E, dU = Ktil dS' + P^T dO, dR = T^T dU,
// dv, and the tile's shares of dT, dP, dbeta and rowsum(dS' o S).
template <int DK>
struct GradShared {
  ChunkCore<DK> cc;
  union alignas(16) {                     // 16-byte aligned: read as float4
    float tile[2][2][DK * CH];            // [buffer][S, dS'] tiles in stored order, during the tile loop
    float g3[3][C][DK];                   // dq, dk, dG after it
  } u;
  union alignas(16) {
    float part[8][C][CH];                 // partial E (0..3) and Ktil dS' (4..7) of the tile; the
                                          // setup's partial pair sums before the tile loop
    float kt[C][DK];                      // dKtil o Ktil per row, after the tile loop
  } v;
  static_assert(sizeof(float) * 8 * C * CH >= sizeof(float) * 2 * 4 * C * C, "setup scratch");
  alignas(16) float dO[C][CH + 4];        // rows of 80 bytes: float4 reads stay aligned
  float E[C][CH + 4], U[C][CH + 4], dU[C][CH + 4], dR[C][CH + 4];
  float dT[C][C + 1], dP[C][C + 1];
  union {
    float Vt[C][CH + 4];                  // the value tile, during the tile loop
  } vt;
  float rs[DK];                           // rowsum(dS' o S) per channel
};
static_assert(sizeof(GradShared<128>) <= 80 * 1024, "two gradient workgroups per compute unit (160 KiB of LDS)");

template <typename TIn, int DK>
__global__ __launch_bounds__(NTG) __attribute__((amdgpu_waves_per_eu(4, 4))) void bwd_grad_kernel(Params p, const void* __restrict__ dO_in,
                                                      const float* __restrict__ states,
                                                      const float* __restrict__ dstates, float* __restrict__ dq,
                                                      float* __restrict__ dk, float* __restrict__ dvo,
                                                      float* __restrict__ dw, float* __restrict__ dbeta) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GradShared<DK>& sm = *reinterpret_cast<GradShared<DK>*>(smem_raw);
  constexpr int NCB = DK / 16;                  // 16-key blocks
  constexpr int NTASK = 3 * NCB;                // (product, key block) tasks of the K = 16 products
  constexpr int NI = 8 * DK / 64;               // wave instructions to copy one S + dS' tile pair
  const int tid = threadIdx.x, lane = tid % 64, w = tid / 64, col = lane % 16, g = lane / 16;
  const int64_t NC = p.n_chunks();
  const int64_t bh = blockIdx.x / NC, n = blockIdx.x % NC;
  const int64_t T = p.T, t0 = n * C;
  const int len = (int)((T - t0) < C ? (T - t0) : C);
  const int dv = (int)p.dv, nsl = dv / CH;
  const TIn* v = (const TIn*)p.v + bh * T * dv;
  const TIn* dO = (const TIn*)dO_in + bh * T * dv;
  const float* Sg = states + (bh * NC + n) * DK * dv;      // nsl [dk][16] blocks in stored order
  const float* dSg = dstates + (bh * NC + n) * DK * dv;
  KDA_GRAD_STAMP(p, w, 8, 0);

  auto copy_tile = [&](int t, int b) {          // S and dS' tiles t into buffer b
    float4* dst = reinterpret_cast<float4*>(sm.u.tile[b][0]);
    for (int ins = w; ins < NI; ins += NTG / 64) {
      const int u = ins * 64 + lane;            // < 8 DK: first 4 DK units from S, the rest from dS'
      const float* src = (u < 4 * DK ? Sg : dSg) + (int64_t)t * DK * CH + 4 * (u % (4 * DK));
      dma16(src, dst + ins * 64);
    }
  };
  copy_tile(0, 0);
  // w of the rows this thread finishes in the last phase (channel tid / NPC, rows (tid % NPC) * RPT ..)
  constexpr int NPC = NTG / DK, RPT = C / NPC;
  float wr[RPT];
  {
    const TIn* w_in = (const TIn*)p.w + bh * T * DK;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = (tid % NPC) * RPT + i;
      const float x = load_f32(w_in, (t0 + min(r, len - 1)) * DK + tid / NPC);   // no branch around the load
      wr[i] = r < len ? x : 0.f;
    }
  }
  // V and dO of every tile, element (er, ed) of each (threads < 256), loaded before the setup
  const int er = (tid % 256) / CH, ed = tid % CH;   // element (row, column) of a 16 x 16 tile
  constexpr int MAXT = 128 / CH;
  float vr[MAXT], orr[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const bool ok = tid < 256 && t < nsl && er < len;   // loads in bounds for every thread, then selected
    const int64_t o = (t0 + min(er, len - 1)) * dv + CH * min(t, nsl - 1) + ed;
    const float x = load_f32(v, o), y = load_f32(dO, o);
    vr[t] = ok ? x : 0.f;
    orr[t] = ok ? y : 0.f;
  }
  KDA_GRAD_STAMP(p, w, 8, 1);
  chunk_setup<TIn, DK, NTG>(sm.cc, &sm.v.part[0][0][0], p, bh, n, len);   // part: 2 * 4 * 256 floats
  KDA_GRAD_STAMP(p, w, 8, 2);

  // A operands of the K = dk products: wavefronts 0..3 take Kbar, 4..7 Ktil, on key blocks wq, wq + 4
  const bool eW = w < 4;
  const int wq = w % 4;
  float a1[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int cb = wq + 4 * b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a1[b][i] = 0.f;
      if (cb < NCB) {
        const int c = 16 * cb + 4 * g + i;
        const float G = sm.cc.G[col][c];
        a1[b][i] = sm.cc.k[col][c] * ex2(eW ? G : sm.cc.gam[c] - G);
      }
    }
  }

  f32x4 tacc[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) tacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float accT = 0.f, accRS = 0.f;
  f32x4 tdp = {0.f, 0.f, 0.f, 0.f};   // wavefront 6: dT (before the diag(beta) scaling), 7: dP

  KDA_GRAD_STAMP(p, w, 8, 3);
  vm_wait<0>();
  lds_barrier();
  KDA_GRAD_STAMP(p, w, 8, 4);
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= nsl) break;
    KDA_GRAD_STAMP(p, w, t, 0);
    const int b = t & 1;
    const float* St = sm.u.tile[b][0];
    const float* dSt = sm.u.tile[b][1];
    if (t + 1 < nsl) copy_tile(t + 1, b ^ 1);
    if (tid < 256) {
      sm.dO[er][ed] = orr[t];
      sm.vt.Vt[er][ed] = vr[t];
    }
    {   // partial E (Kbar S) or Ktil dS' over this wavefront's key blocks
      const float* B = eW ? St : dSt;
      f32x4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int cb = wq + 4 * bb;
        if (cb < NCB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pp = mfma4(a1[bb][i], B[cb * 256 + i * 64 + lane], pp);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.v.part[w][4 * g + i][col] = pp[i];
    }
    KDA_GRAD_STAMP(p, w, t, 1);
    lds_barrier();
    KDA_GRAD_STAMP(p, w, t, 2);
    // One wavefront each, on 16 x 16 tiles in the accumulator layout (lane: rows 4g + i, column col), so
    // that the first product's result is the second one's B operand (K index 4g + s at step s):
    if (w == 0) {          // E = V - Kbar S;  U = T diag(beta) E
      f32x4 e, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float x = sm.vt.Vt[r][col];
#pragma unroll
        for (int q = 0; q < 4; ++q) x -= sm.v.part[q][r][col];
        e[i] = x;
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) u = mfma4(sm.cc.Tb[col][4 * g + s4], e[s4], u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm.E[4 * g + i][col] = e[i];
        sm.U[4 * g + i][col] = u[i];
      }
    } else if (w == 1) {   // dU = Ktil dS' + P^T dO;  dR = T^T dU;  dv = diag(beta) dR
      f32x4 du, dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float x = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) x += sm.v.part[4 + q][r][col];
        du[i] = x;
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) du = mfma4(sm.cc.P[4 * g + s4][col], sm.dO[4 * g + s4][col], du);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) dr = mfma4(sm.cc.T[4 * g + s4][col], du[s4], dr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        sm.dU[r][col] = du[i];
        sm.dR[r][col] = dr[i];
        if (r < len) dvo[(bh * T + t0 + r) * dv + CH * t + col] = sm.cc.beta[r] * dr[i];
      }
    } else if ((w == 2 || w == 3) && tid - 128 < DK) {   // rowsum(dS' o S) over the tile's columns
      const int c = tid - 128;
      const int o = (c / 16) * 256 + (c % 4) * 64 + ((c % 16) / 4) * 16;
      const float4* s4 = reinterpret_cast<const float4*>(St + o);
      const float4* d4 = reinterpret_cast<const float4*>(dSt + o);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 a = s4[q4], bq = d4[q4];
        accRS += a.x * bq.x + a.y * bq.y + a.z * bq.z + a.w * bq.w;
      }
    }
    KDA_GRAD_STAMP(p, w, t, 3);
    lds_barrier();
    KDA_GRAD_STAMP(p, w, t, 4);
    // K = 16 products: task id = w + 8 j -> (product id / NCB, key block id % NCB)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int id = w + 8 * j;
      if (id < NTASK) {
        const int pr = id / NCB, cb = id % NCB;
        const float(*A)[CH + 4] = pr == 0 ? sm.dO : (pr == 1 ? sm.dR : sm.U);
        const float4 av = *reinterpret_cast<const float4*>(&A[col][4 * g]);
        const float4 bv = *reinterpret_cast<const float4*>(&(pr == 2 ? dSt : St)[cb * 256 + (col % 4) * 64 + (col / 4) * 16 + 4 * g]);
        tacc[j] = mfma4(av.x, bv.x, tacc[j]);
        tacc[j] = mfma4(av.y, bv.y, tacc[j]);
        tacc[j] = mfma4(av.z, bv.z, tacc[j]);
        tacc[j] = mfma4(av.w, bv.w, tacc[j]);
      }
    }
    if (w >= 6) {      // dT += dU E^T (wavefront 6), dP += dO U^T (7): K = the tile's 16 columns, order 4g + s
      const float(*A)[CH + 4] = w == 6 ? sm.dU : sm.dO;
      const float(*B)[CH + 4] = w == 6 ? sm.E : sm.U;
      const float4 av = *reinterpret_cast<const float4*>(&A[col][4 * g]);
      const float4 bv = *reinterpret_cast<const float4*>(&B[col][4 * g]);
      tdp = mfma4(av.x, bv.x, tdp);
      tdp = mfma4(av.y, bv.y, tdp);
      tdp = mfma4(av.z, bv.z, tdp);
      tdp = mfma4(av.w, bv.w, tdp);
    }
    if (tid >= 256 && tid < 256 + C) {   // dbeta share: sum_d dR E, in accT of threads 256 .. 271
      const int r = tid - 256;
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < CH; d += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&sm.dR[r][d]);
        const float4 y = *reinterpret_cast<const float4*>(&sm.E[r][d]);
        a += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      }
      accT += a;
    }
    KDA_GRAD_STAMP(p, w, t, 5);
    vm_wait<0>();      // the next tile pair has landed
    lds_barrier();
  }
  KDA_GRAD_STAMP(p, w, 9, 0);

  if ((w == 2 || w == 3) && tid - 128 < DK) sm.rs[tid - 128] = accRS;
  // wavefronts 6 and 7 hold dT and dP (lane: rows 4g + i, column col), lower parts kept;
  // tid 256..271: accT = dbeta share
  if (w == 6) {   // dA = -(M T^T) with M = T^T dT, strictly lower, into dT: two fp32 products on this wavefront
    float at[4];  // dT[4g + s][col], the A operand of M^T = dT^T T at step s
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) at[s4] = col <= 4 * g + s4 ? sm.cc.beta[col] * tdp[s4] : 0.f;
    f32x4 mt = {0.f, 0.f, 0.f, 0.f};   // M^T (lane: rows 4g + i, column col), the B operand of T M^T
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) mt = mfma4(at[s4], sm.cc.T[4 * g + s4][col], mt);
    f32x4 d = {0.f, 0.f, 0.f, 0.f};    // T M^T = (M T^T)^T: d[i] = (M T^T)[col][4g + i]
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) d = mfma4(sm.cc.T[col][4 * g + s4], mt[s4], d);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.dT[col][4 * g + i] = 4 * g + i < col ? -d[i] : 0.f;
  } else if (w == 7) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      sm.dP[r][col] = col <= r ? tdp[i] : 0.f;
    }
  }
  lds_barrier();
  if (tid >= 256 && tid < 256 + C) {
    const int r = tid - 256;
    float acc = accT;
#pragma unroll
    for (int j = 0; j < C; ++j) acc += sm.dT[r][j] * sm.cc.X[r][j];   // dA is strictly lower
    if (r < len) dbeta[bh * T + t0 + r] = acc;
  }
  KDA_GRAD_STAMP(p, w, 9, 1);
  float (*gq)[DK] = sm.u.g3[0];
  float (*gk)[DK] = sm.u.g3[1];
  float (*gG)[DK] = sm.u.g3[2];
  if (sm.cc.dense()) {
    // the pair terms as products of e^{+-(G - Gam/2)} factors (wavefront w: key channels 16w .. 16w + 15):
    //   P1 = Wa Kinv', P2 = Wp Kinv', P3 = Wa^T Kbar', P4 = Wp^T Qbar'   (Wa = diag(beta) dA, Wp = dP)
    //   dk_x = e^{G'_x} P1 + e^{-G'_x} (P3 + P4),  dq_x = e^{G'_x} P2,
    //   dG_x = k_x e^{G'_x} P1 + q_x e^{G'_x} P2 - k_x e^{-G'_x} (P3 + P4)
    if (w < NCB) {
      const int c = 16 * w + col;
      float eg[4], egi[4], kk[4], qq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {     // rows 4g + i of channel c: B operands, and the output rows
        const int r = 4 * g + i;
        const float Gs = sm.cc.G[r][c] - 0.5f * sm.cc.gam[c];
        eg[i] = ex2(Gs);
        egi[i] = ex2(-Gs);
        kk[i] = sm.cc.k[r][c];
        qq[i] = sm.cc.q[r][c];
      }
      f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = p1, p3 = p1, p4 = p1;
      const float bc = sm.cc.beta[col];
#pragma unroll
      for (int s = 0; s < 4; ++s) {     // K order: j (or r) = 4g + s
        const int r = 4 * g + s;
        const float kinv = kk[s] * egi[s], kbar = kk[s] * eg[s], qbar = qq[s] * eg[s];
        p1 = mfma4(bc * sm.dT[col][r], kinv, p1);
        p2 = mfma4(sm.dP[col][r], kinv, p2);
        p3 = mfma4(sm.cc.beta[r] * sm.dT[r][col], kbar, p3);
        p4 = mfma4(sm.dP[r][col], qbar, p4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 4 * g + i;
        const float a = eg[i] * p1[i], bq = eg[i] * p2[i], e = egi[i] * (p3[i] + p4[i]);
        gk[x][c] = a + e;
        gq[x][c] = bq;
        gG[x][c] = kk[i] * a + qq[i] * bq - kk[i] * e;
      }
    }
  } else {   // pair-by-pair terms of X (weights beta_r dA) and P (weights dP); thread (c, part) owns the
             // rows x = part (mod NTG / DK) of channel c and sums every pair touching them
    constexpr int NPART = NTG / DK;
    const int c = tid % DK, part = tid / DK;
    float Gc[C], kc[C];
#pragma unroll
    for (int r = 0; r < C; ++r) { Gc[r] = sm.cc.G[r][c]; kc[r] = sm.cc.k[r][c]; }
    for (int x = part; x < C; x += NPART) {
      const float kx = kc[x], qx = sm.cc.q[x][c], Gx = Gc[x], bx = sm.cc.beta[x];
      float dkx = 0.f, dqx = 0.f, dGx = 0.f;
      for (int j = 0; j <= x; ++j) {     // pairs (x, j): x is the later row
        const float e = ex2(Gx - Gc[j]);
        const float wa = bx * sm.dT[x][j];  // dA is strictly lower: 0 at j = x
        const float wp = sm.dP[x][j];
        dkx += wa * kc[j] * e;
        dqx += wp * kc[j] * e;
        dGx += (wa * kx + wp * qx) * kc[j] * e;
      }
      for (int r = x; r < C; ++r) {      // pairs (r, x): x is the earlier row
        const float e = ex2(Gc[r] - Gx);
        const float wa = sm.cc.beta[r] * sm.dT[r][x];
        const float wp = sm.dP[r][x];
        const float f = (wa * kc[r] + wp * sm.cc.q[r][c]) * e;
        dkx += f;
        dGx -= f * kx;
      }
      gk[x][c] = dkx;
      gq[x][c] = dqx;
      gG[x][c] = dGx;
    }
  }
  lds_barrier();
  KDA_GRAD_STAMP(p, w, 9, 2);
  // the K = 16 products through the scalings of Qbar, Kbar, Ktil (lane: rows 4g + i, key 16 cb + col)
  if (NCB == 8) {   // wavefront w holds all three products of key block w: plain updates
    const int c = 16 * w + col;
    const float gm = sm.cc.gam[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const float G = sm.cc.G[r][c], kr = sm.cc.k[r][c];
      const float eg = ex2(G), et = ex2(gm - G);
      const float a = tacc[0][i], dKbar = -sm.cc.beta[r] * tacc[1][i], t = tacc[2][i];
      gq[r][c] += a * eg;
      gk[r][c] += dKbar * eg + t * et;
      gG[r][c] += a * sm.cc.q[r][c] * eg + dKbar * kr * eg;
      // the Ktil scaling enters dG_r with one sign and dGam with the other; kept apart, so that dg
      // takes it as a sum over the earlier rows instead of a difference of two long sums
      sm.v.kt[r][c] = t * kr * et;
    }
  } else {
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int id = w + 8 * j;
    if (id < NTASK) {
      const int pr = id / NCB, c = 16 * (id % NCB) + col;
      const float gm = sm.cc.gam[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const float G = sm.cc.G[r][c], kr = sm.cc.k[r][c], x = tacc[j][i];
        if (pr == 0) {
          const float eg = ex2(G);
          atomicAdd(&gq[r][c], x * eg);
          atomicAdd(&gG[r][c], x * sm.cc.q[r][c] * eg);
        } else if (pr == 1) {
          const float eg = ex2(G), dKbar = -sm.cc.beta[r] * x;
          atomicAdd(&gk[r][c], dKbar * eg);
          atomicAdd(&gG[r][c], dKbar * kr * eg);
        } else {
          // the Ktil scaling enters dG_r with one sign and dGam with the other; kept apart, so that dg
          // takes it as a sum over the earlier rows instead of a difference of two long sums
          const float et = ex2(gm - G);
          atomicAdd(&gk[r][c], x * et);
          sm.v.kt[r][c] = x * kr * et;
        }
      }
    }
  }
  }
  lds_barrier();
  KDA_GRAD_STAMP(p, w, 9, 3);
  {   // dg and the outputs; NPC threads per channel, thread p of channel c owning rows p*RPT .. p*RPT + RPT-1:
      // dg_u = e^{Gam} rowsum(dS' o S) + sum_{r >= u} dG_r + sum_{r < u} (dKtil o Ktil)_r
    const int c = tid / NPC, pp = tid % NPC, r0 = pp * RPT;
    float gv[RPT], kv[RPT];
    float sg = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = r0 + i;
      gv[i] = gG[r][c];
      kv[i] = sm.v.kt[r][c];
      sg += gv[i];
      sk += kv[i];
    }
    // over the channel's NPC threads (consecutive lanes): dG of the later rows, Ktil terms of the earlier
    float later = 0.f, earlier = 0.f;
#pragma unroll
    for (int o = 1; o < NPC; o <<= 1) {
      const float a = __shfl_down(sg, o, NPC), b = __shfl_up(sk, o, NPC);
      if (pp + o < NPC) later += a;
      if (pp >= o) earlier += b;
      sg += (pp + o < NPC) ? a : 0.f;
      sk += (pp >= o) ? b : 0.f;
    }
    float acc = ex2(sm.cc.gam[c]) * sm.rs[c] + later;     // suffix from the rows after this thread's
    float pre[RPT];
    float run = earlier;
#pragma unroll
    for (int i = 0; i < RPT; ++i) { pre[i] = run; run += kv[i]; }
#pragma unroll
    for (int i = RPT - 1; i >= 0; --i) {
      const int r = r0 + i;
      acc += gv[i];
      if (r < len) {
        const int64_t o = bh * T * DK + (t0 + r) * DK + c;
        dw[o] = (acc + pre[i]) * gate_deriv(wr[i], p.g_min, p.unbounded);
        dq[o] = gq[r][c];
        dk[o] = gk[r][c];
      }
    }
  }
  KDA_GRAD_STAMP(p, w, 9, 4);
}

template <typename TIn, int DK>
hipError_t launch_bwd_dk(const BwdParams& b, hipStream_t s) {
  const Params& p = b.p;
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = set_dyn_lds((const void*)bwd_grad_kernel<TIn, DK>, (int)sizeof(GradShared<DK>), lds_set);
    if (e != hipSuccess) return e;
  }
  const int64_t BH = p.B * p.H, NC = p.n_chunks();
  const WsLayout L = ws_layout(p.workspace, BH, NC, p.dk, p.dv);
  const unsigned nchunks = (unsigned)(BH * NC), nchain = (unsigned)(BH * (p.dv / CH));
  hipLaunchKernelGGL((bwd_prep_kernel<TIn, DK>), dim3(nchunks), dim3(NTP), 0, s, p, b.dO, L.recs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chain_kernel<TIn, DK>), dim3(2 * nchain), dim3(ChainDims<DK>::NT), 0, s, p, b.dO, b.dSf,
                     (const float*)L.recs, L.states, L.dstates, b.dS0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<TIn, DK>), dim3(nchunks), dim3(NTG), sizeof(GradShared<DK>), s, p, b.dO,
                     (const float*)L.states, (const float*)L.dstates, b.dq, b.dk, b.dv, b.dw, b.dbeta);
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
#if KDA_PHASE_STAMPS
  const int64_t extra = kStampBytes;   // the chain stamps follow the states and adjoints
#else
  const int64_t extra = 0;
#endif
  return (size_t)(B * H * NC * (rec_floats(dk, dv) + 2 * dk * dv)) * sizeof(float) + (size_t)extra;
}

hipError_t launch_bwd(const BwdParams& b_in, hipStream_t s) {
#if KDA_PHASE_STAMPS
  // phase-stamp build: the chain workgroup KDA_STAMP_BLOCK stamps into the workspace's last kStampBytes
  BwdParams b = b_in;
  const char* sb = std::getenv("KDA_STAMP_BLOCK");
  const bool room = b.p.workspace && b.p.workspace_bytes >= (size_t)kStampBytes;
  b.p.stamp_off = room ? (int64_t)b.p.workspace_bytes - kStampBytes : -1;
  b.p.stamp_block = (room && sb) ? std::atoi(sb) : -1;
  const char* sk = std::getenv("KDA_STAMP_KERNEL");   // "grad": the gradient kernel's workgroup stamps
  b.p.stamp_kernel = (sk && std::strcmp(sk, "grad") == 0) ? 1 : 0;
#else
  const BwdParams& b = b_in;
#endif
  return b.p.dtype == KDA_DTYPE_BF16 ? launch_bwd_t<uint16_t>(b, s) : launch_bwd_t<float>(b, s);
}

}  // namespace kda

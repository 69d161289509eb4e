// Matrix-core path (bf16 MFMA 16x16x32 on gfx950) of the chunked KDA forward,
// for bf16 inputs with dk = dv = 128.
//
// Work is split into two kernels that meet in a workspace of per-step records:
//
//  prep_kernel   one workgroup per (b, h, step of 32 tokens = two 16-token
//                chunks), all steps in parallel.  Gate, in-chunk prefix, span
//                and overflow flag per chunk; the 32x32 causal tiles
//                P = (Q o e^G)(K o e^-G)^T and A = diag(beta)(K o e^G)(K o e^-G)^T
//                on bf16 MFMA; T = (I + A)^{-1}; W = T diag(beta) Kbar,
//                Qhat = Qbar - P W, Phat = P T diag(beta).  The record is
//                written already arranged in the per-lane operand order the
//                scan loads (16 contiguous bytes per lane per operand).
//  scan_kernel   one wavefront per (b, h, 16-column slice of dv), serial over
//                steps, state slice (128 x 16 fp32) in registers:
//                  U = T diag(beta) V - W S          (10 MFMA)
//                  O = Qhat S + Phat V               (10 MFMA)
//                  S <- diag(e^{Gam}) S + Ktil^T U   ( 8 MFMA)
//
// The in-chunk algebra follows "From Numerical Stability to Load Balancing
// ..." section 2.1 (serial recurrence between chunks, matrix products inside,
// in-chunk scaling exp(G_i - G_j) for i >= j) and the bounded gate of
// section 2.2 there and of "Demystifying Trillion-Parameter MoE Models ..."
// Breakthrough 1 part 2 (a 16-token chunk's span stays at or above -80, so the
// reciprocal e^{-G} stays below e^80 and the diagonal tile is a dense matrix
// product).  Within a 32-token step only the two diagonal 16x16 blocks use the
// reciprocal e^{-G}; the block coupling chunk 1 to chunk 0 uses factors
// referenced to the chunk boundary, e^{L_r} e^{Gam_0 - L_j}, both <= 1.  A
// chunk whose span falls below -80 gets its diagonal blocks from per-pair
// factors exp(L_r - L_j) <= 1 on the vector ALUs instead.
#include "kda_internal.h"

namespace kda {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int D = 128;     // dk = dv
constexpr int STEP = 32;   // tokens per step (two chunks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// record layout (bytes) of one (b, h, step)
constexpr int kOffWn = 0;        // -W,  [mt 2][u 4] blocks of 64 lanes x 16 B
constexpr int kOffQh = 8192;     // Qhat, same arrangement
constexpr int kOffKt = 16384;    // Ktil^T, [t 8] blocks
constexpr int kOffTb = 24576;    // T diag(beta), [mt 2] blocks
constexpr int kOffPh = 26624;    // Phat, [mt 2] blocks
constexpr int kOffEg = 28672;    // e^{Gam} per key channel, grouped by lane group: [g 4][t 8][r 4] fp32
constexpr int kOffMeta = 29184;  // StepMeta (16 B), then padding
constexpr int kRecBytes = 29696; // 29 KiB: the scan copies a record with 29 wave-wide 16-byte-per-lane loads

struct StepMeta {           // per (b, h, step)
  float span[2];            // chunk spans (natural log units); +inf for a chunk with no tokens
  uint32_t n_valid;         // chunks with at least one token (1 or 2)
  uint32_t n_flagged;       // of those, spans below -80
};

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// gate in log2 units: g * log2(e)
__device__ __forceinline__ float gate_log2(float w, float g_min, int unbounded) {
  if (unbounded) return -(fmaxf(w, 0.f) + log1pf(expf(-fabsf(w)))) * kLog2e;
  const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-w * kLog2e));
  return (g_min * kLog2e) * s;
}

__device__ __forceinline__ float bf(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// ------------------------------------------------------------------ prep kernel

struct PrepShared {
  alignas(16) float L[STEP][D];                 // in-chunk inclusive prefix, log2 units (per-pair fallback)
  alignas(16) __bf16 Qraw[STEP][D + 8];         // raw q, k (bf16 exact) for the per-pair fallback
  alignas(16) __bf16 Kraw[STEP][D + 8];
  alignas(16) __bf16 Qb[STEP][D + 8];           // q e^{L}      (chunk-local)
  alignas(16) __bf16 Kb[STEP][D + 8];           // k e^{L}
  alignas(16) __bf16 Kh[STEP][D + 8];           // k e^{-L}     (diagonal blocks only)
  alignas(16) __bf16 Kt0[16][D + 8];            // k e^{Gam_0 - L}, chunk 0 (block coupling chunk 1 to chunk 0)
  alignas(16) float Qbar[STEP][D + 4];          // q e^{G}      (G referenced to the step start)
  alignas(16) __bf16 KbarT[D][STEP + 8];        // (k e^{G})^T
  alignas(16) __bf16 KtilT[D][STEP + 8];        // (k e^{Gam_step - G})^T
  alignas(16) __bf16 WnT[D][STEP + 8];          // (-W)^T
  alignas(16) float A[STEP][STEP + 1], P[STEP][STEP + 1], T[STEP][STEP + 1], X[16][17];
  alignas(16) __bf16 Tb[STEP][STEP + 8];        // T diag(beta)
  alignas(16) __bf16 TbT[STEP][STEP + 8];       // (T diag(beta))^T
  alignas(16) __bf16 Pb[STEP][STEP + 8];        // P
  alignas(16) __bf16 Ph[STEP][STEP + 8];        // P T diag(beta)
  alignas(16) float Gam[2][D];                  // chunk spans per channel, log2 units
  alignas(16) float beta[STEP];
  alignas(16) float red[4];
  alignas(16) int pairwise[2];
};

__global__ __launch_bounds__(256) void prep_kernel(Params p, int64_t n_steps) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepShared& sm = *reinterpret_cast<PrepShared*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t bh = blockIdx.x / n_steps;
  const int64_t s = blockIdx.x % n_steps;
  const int64_t T = p.T;
  const int64_t t0 = s * STEP;
  const uint16_t* q = (const uint16_t*)p.q + bh * T * D;
  const uint16_t* k = (const uint16_t*)p.k + bh * T * D;
  const uint16_t* w = (const uint16_t*)p.w + bh * T * D;
  const uint16_t* beta = (const uint16_t*)p.beta + bh * T;
  unsigned char* rec = (unsigned char*)p.workspace + (bh * n_steps + s) * (int64_t)kRecBytes;

  // ---- phase 1: gate, chunk-local prefix, scaled operands.  Thread = (channel, chunk).
  const int ch = tid & (D - 1);
  const int c = tid >> 7;
  float qv[16], kv[16], eL[16], wv[16];
  // all loads first (addresses clamped into the sequence), so they are in flight together
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    const int64_t t = t0 + 16 * c + l;
    const int64_t tc = t < T ? t : T - 1;
    wv[l] = bf(w, tc * D + ch);
    qv[l] = bf(q, tc * D + ch);
    kv[l] = bf(k, tc * D + ch);
  }
  float Lp = 0.f;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    const int pp = 16 * c + l;
    const bool ok = t0 + pp < T;
    qv[l] = ok ? qv[l] : 0.f;
    kv[l] = ok ? kv[l] : 0.f;
    Lp += ok ? gate_log2(wv[l], p.g_min, p.unbounded) : 0.f;
    sm.L[pp][ch] = Lp;
    eL[l] = __builtin_amdgcn_exp2f(Lp);
    const float emL = __builtin_amdgcn_exp2f(-Lp);
    sm.Qraw[pp][ch] = (__bf16)qv[l];
    sm.Kraw[pp][ch] = (__bf16)kv[l];
    sm.Qb[pp][ch] = (__bf16)(qv[l] * eL[l]);
    sm.Kb[pp][ch] = (__bf16)(kv[l] * eL[l]);
    sm.Kh[pp][ch] = (__bf16)(kv[l] * emL);
  }
  sm.Gam[c][ch] = Lp;
  if (tid < STEP) sm.beta[tid] = (t0 + tid < T) ? bf(beta, t0 + tid) : 0.f;
  // span of this chunk: min over channels (each half of the block owns one chunk)
  float m = Lp;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fminf(m, __shfl_xor(m, off));
  if (lane == 0) sm.red[wave] = m;
  __syncthreads();

  const bool valid0 = t0 < T;
  const bool valid1 = t0 + 16 < T;
  const float span0 = fminf(sm.red[0], sm.red[1]) * kLn2;
  const float span1 = fminf(sm.red[2], sm.red[3]) * kLn2;
  const bool flag0 = valid0 && span0 < kSpanLimit;
  const bool flag1 = valid1 && span1 < kSpanLimit;
  if (tid == 0) {
    sm.pairwise[0] = (p.force_fallback || (flag0 && !p.disable_fallback)) ? 1 : 0;
    sm.pairwise[1] = (p.force_fallback || (flag1 && !p.disable_fallback)) ? 1 : 0;
    StepMeta mt;
    mt.span[0] = valid0 ? span0 : __int_as_float(0x7f800000);
    mt.span[1] = valid1 ? span1 : __int_as_float(0x7f800000);
    mt.n_valid = (valid0 ? 1u : 0u) + (valid1 ? 1u : 0u);
    mt.n_flagged = (flag0 ? 1u : 0u) + (flag1 ? 1u : 0u);
    *reinterpret_cast<StepMeta*>(rec + kOffMeta) = mt;
  }
  // step-level quantities (G referenced to the start of the step)
  {
    const float Gam0 = sm.Gam[0][ch], Gam1 = sm.Gam[1][ch];
    const float base = (c == 0) ? 0.f : Gam0;               // G = base + L
    const float egBase = __builtin_amdgcn_exp2f(base);       // e^{Gam_0} for chunk 1
    const float eGam1 = __builtin_amdgcn_exp2f(Gam1);
#pragma unroll
    for (int l = 0; l < 16; ++l) {
      const int pp = 16 * c + l;
      const float Lq = sm.L[pp][ch];
      const float eG = eL[l] * egBase;                       // e^{G} (both factors <= 1)
      sm.Qbar[pp][ch] = qv[l] * eG;
      sm.KbarT[ch][pp] = (__bf16)(kv[l] * eG);
      const float eGamL = __builtin_amdgcn_exp2f(sm.Gam[c][ch] - Lq);   // e^{Gam_c - L} <= 1
      if (c == 0) {
        sm.Kt0[l][ch] = (__bf16)(kv[l] * eGamL);
        sm.KtilT[ch][pp] = (__bf16)(kv[l] * eGamL * eGam1);        // e^{Gam_0 + Gam_1 - G}
      } else {
        sm.KtilT[ch][pp] = (__bf16)(kv[l] * eGamL);
      }
    }
    if (c == 0) {   // e^{Gam_step}, grouped by the scan's lane groups: index g*32 + t*4 + r <-> channel 16t + 4g + r
      const int t = ch >> 4, g = (ch >> 2) & 3, r = ch & 3;
      reinterpret_cast<float*>(rec + kOffEg)[g * 32 + t * 4 + r] = __builtin_amdgcn_exp2f(Gam0 + Gam1);
    }
  }
  __syncthreads();

  // ---- phase 2: the 32x32 tiles.  wave 0: diagonal block of chunk 0 (A and P), wave 1: chunk 1,
  // wave 2: A coupling chunk 1 to chunk 0, wave 3: P coupling chunk 1 to chunk 0.
  {
    const int cc = (wave == 0) ? 0 : 1;
    if (wave <= 1 && sm.pairwise[cc]) {
      // per-pair decay factors exp(L_r - L_j) <= 1 (no reciprocal), vector ALUs
      for (int pr = lane; pr < 136; pr += 64) {
        int r = 0;
        while ((r + 1) * (r + 2) / 2 <= pr) ++r;
        const int j = pr - r * (r + 1) / 2;             // j <= r
        const int R = 16 * cc + r, J = 16 * cc + j;
        float a = 0.f, pq = 0.f;
        for (int x = 0; x < D; ++x) {
          const float e = __builtin_amdgcn_exp2f(sm.L[R][x] - sm.L[J][x]);
          const float kj = (float)sm.Kraw[J][x] * e;
          a += (float)sm.Kraw[R][x] * kj;
          pq += (float)sm.Qraw[R][x] * kj;
        }
        sm.A[R][J] = (j < r) ? sm.beta[R] * a : 0.f;
        sm.P[R][J] = pq;
      }
      for (int pr = lane; pr < 256; pr += 64) {         // upper triangle of the block
        const int r = pr >> 4, j = pr & 15;
        if (j > r) { sm.A[16 * cc + r][16 * cc + j] = 0.f; sm.P[16 * cc + r][16 * cc + j] = 0.f; }
      }
    } else if (wave <= 1) {
      floatx4 accA = {0, 0, 0, 0}, accP = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int col = 32 * kk + 8 * lg;
        const bf16x8 bk = ld8(&sm.Kh[16 * cc + li][col]);
        accA = mfma(ld8(&sm.Kb[16 * cc + li][col]), bk, accA);
        accP = mfma(ld8(&sm.Qb[16 * cc + li][col]), bk, accP);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * lg + r;                     // D[row][li]
        const int R = 16 * cc + row, J = 16 * cc + li;
        sm.A[R][J] = (li < row) ? sm.beta[R] * accA[r] : 0.f;
        sm.P[R][J] = (li <= row) ? accP[r] : 0.f;
      }
    } else {
      floatx4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int col = 32 * kk + 8 * lg;
        const bf16x8 a = (wave == 2) ? ld8(&sm.Kb[16 + li][col]) : ld8(&sm.Qb[16 + li][col]);
        acc = mfma(a, ld8(&sm.Kt0[li][col]), acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int R = 16 + 4 * lg + r;
        if (wave == 2) { sm.A[R][li] = sm.beta[R] * acc[r]; sm.A[4 * lg + r][16 + li] = 0.f; }
        else { sm.P[R][li] = acc[r]; sm.P[4 * lg + r][16 + li] = 0.f; }
      }
    }
  }
  __syncthreads();

  // ---- phase 3: T = (I + A)^{-1}.  Diagonal blocks by forward substitution, one column per lane,
  // the column kept in registers (fully unrolled, no dependent shared-memory round trips) ...
  if (tid < STEP) {
    const int j = tid, b0 = (j < 16) ? 0 : 16;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = (b0 + r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) x -= sm.A[b0 + r][b0 + i] * col[i];
      col[r] = (b0 + r < j) ? 0.f : x;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sm.T[b0 + r][j] = col[r];
      if (b0 == 16) sm.T[r][j] = 0.f;                 // upper-right block
    }
  }
  __syncthreads();
  // ... then the coupling block T_10 = -T_11 (A_10 T_00)   (entries outside the triangles are zero)
  {
    const int r = tid >> 4, j = tid & 15;
    float x = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) x += sm.A[16 + r][n] * sm.T[n][j];
    sm.X[r][j] = x;
  }
  __syncthreads();
  {
    const int r = tid >> 4, j = tid & 15;
    float x = 0.f;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) x += sm.T[16 + r][16 + mm] * sm.X[mm][j];
    sm.T[16 + r][j] = -x;
  }
  __syncthreads();
  // T diag(beta) (row-major and transposed) and P in bf16
  for (int e = tid; e < STEP * STEP; e += 256) {
    const int r = e >> 5, j = e & 31;
    const __bf16 tb = (__bf16)(sm.T[r][j] * sm.beta[j]);
    sm.Tb[r][j] = tb;
    sm.TbT[j][r] = tb;
    sm.Pb[r][j] = (__bf16)sm.P[r][j];
  }
  __syncthreads();
  // Phat = P T diag(beta) on MFMA: wave w computes the 16x16 tile (w >> 1, w & 1)
  {
    const int mt = wave >> 1, nt = wave & 1;
    const floatx4 d = mfma(ld8(&sm.Pb[16 * mt + li][8 * lg]), ld8(&sm.TbT[16 * nt + li][8 * lg]), floatx4{0, 0, 0, 0});
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.Ph[16 * mt + 4 * lg + r][16 * nt + li] = (__bf16)d[r];
  }
  __syncthreads();

  // ---- phase 4: W^T = Kbar^T (T diag(beta))^T on MFMA; wave owns channel tiles 2w, 2w+1
  {
    const int u = wave;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 d[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nt = 2 * u + h;
        d[h] = mfma(ld8(&sm.KbarT[16 * nt + li][8 * lg]), ld8(&sm.Tb[16 * mt + li][8 * lg]), floatx4{0, 0, 0, 0});
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.WnT[16 * nt + 4 * lg + r][16 * mt + li] = (__bf16)(-d[h][r]);
      }
      bf16x8 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) { o[r] = (__bf16)(-d[0][r]); o[4 + r] = (__bf16)(-d[1][r]); }
      *reinterpret_cast<bf16x8*>(rec + kOffWn + ((mt * 4 + u) * 64 + lane) * 16) = o;
    }
  }
  __syncthreads();

  // ---- phase 5: Qhat^T = Qbar^T - W^T P^T on MFMA
  {
    const int u = wave;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 d[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nt = 2 * u + h;
        const floatx4 cq = *reinterpret_cast<const floatx4*>(&sm.Qbar[16 * mt + li][16 * nt + 4 * lg]);
        d[h] = mfma(ld8(&sm.WnT[16 * nt + li][8 * lg]), ld8(&sm.Pb[16 * mt + li][8 * lg]), cq);
      }
      bf16x8 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) { o[r] = (__bf16)d[0][r]; o[4 + r] = (__bf16)d[1][r]; }
      *reinterpret_cast<bf16x8*>(rec + kOffQh + ((mt * 4 + u) * 64 + lane) * 16) = o;
    }
  }

  // ---- phase 6: the remaining operands, arranged per lane: 8 values = positions {4g..4g+3, 16+4g..16+4g+3}
  for (int e = tid; e < 8 * 64; e += 256) {           // Ktil^T, 8 channel tiles
    const int t = e >> 6, ln = e & 63, i = ln & 15, g = ln >> 4;
    bf16x8 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) { o[r] = sm.KtilT[16 * t + i][4 * g + r]; o[4 + r] = sm.KtilT[16 * t + i][16 + 4 * g + r]; }
    *reinterpret_cast<bf16x8*>(rec + kOffKt + e * 16) = o;
  }
  if (tid < 128) {                                    // T diag(beta) and Phat, 2 row tiles each
    const int mt = tid >> 6, ln = tid & 63, i = ln & 15, g = ln >> 4;
    bf16x8 o1, o2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o1[r] = sm.Tb[16 * mt + i][4 * g + r]; o1[4 + r] = sm.Tb[16 * mt + i][16 + 4 * g + r];
      o2[r] = sm.Ph[16 * mt + i][4 * g + r]; o2[4 + r] = sm.Ph[16 * mt + i][16 + 4 * g + r];
    }
    *reinterpret_cast<bf16x8*>(rec + kOffTb + tid * 16) = o1;
    *reinterpret_cast<bf16x8*>(rec + kOffPh + tid * 16) = o2;
  }
}

// ------------------------------------------------------------------ scan kernel

__device__ __forceinline__ bf16x8 pack2(floatx4 a, floatx4 b) {
  bf16x8 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) { o[r] = (__bf16)a[r]; o[4 + r] = (__bf16)b[r]; }
  return o;
}

// Ring of records in LDS: each slot holds one step's record followed by the
// 32 x 16 slice of V for that step.  Six loader wavefronts keep kRing-1 steps
// in flight with direct-to-LDS 16-byte loads (one wavefront sustains only
// ~17 GB/s of such loads, so the stream is spread over several), and
// guarantee that the two oldest slots are complete at every step barrier, so
// the compute wavefronts can read step s+1's operands while step s is still
// computing.  The step's work is split over two
// compute wavefronts on different SIMDs (one wavefront's vector ALU issues too
// slowly for both halves):
//   chain wave   U = T diag(beta) V - W S;  S <- diag(e^Gam) S + Ktil^T U;
//                publishes the bf16 copy of the state entering each step
//   output wave  O = Qhat S + Phat V from that copy; stores o
constexpr int kRing = 5;
constexpr int kSlotBytes = kRecBytes + 1024;
constexpr int kLoadsPerStep = kRecBytes / 1024 + 1;   // 29 record chunks + 1 V chunk
constexpr int kLoaders = 6;
constexpr int kLoadsPerLoader = kLoadsPerStep / kLoaders;
constexpr int kStateBufBytes = 4 * 64 * 16;          // bf16 state operands, [u 4][lane 64] x 16 B
static_assert(kLoadsPerStep % kLoaders == 0, "loads must split evenly over the loader waves");
static_assert(kLoadsPerLoader * (kRing - 1) <= 63, "outstanding loads must fit the vmcnt counter");
static_assert(kRing >= 4, "two complete slots plus two in flight");
constexpr size_t kScanSmem = (size_t)kRing * kSlotBytes + 2 * kStateBufBytes;
static_assert(kScanSmem <= 163840, "LDS budget");
constexpr int kScanThreads = 64 * (2 + kLoaders);

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Workgroup barrier without a memory fence on global memory: waits only for this wave's
// shared-memory operations (so its LDS writes are visible after the barrier), never for the
// loaders' in-flight global loads or the output stores.
__device__ __forceinline__ void block_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima)
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_vm_dyn(int n) {   // n in multiples of kLoadsPerLoader
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<kLoadsPerLoader>(); break;
    case 2: wait_vm<2 * kLoadsPerLoader>(); break;
    default: wait_vm<3 * kLoadsPerLoader>(); break;
  }
}

// V operand rows {4g+r, 16+4g+r}, column li, from the slot's 32 x 16 V tile; rows at or past nrows are zero
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* slot, int lg, int li, int nrows) {
  const __bf16* vr = (const __bf16*)(slot + kRecBytes);
  bf16x8 vb;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    vb[r] = vr[(4 * lg + r) * 16 + li];
    vb[4 + r] = vr[(16 + 4 * lg + r) * 16 + li];
  }
  if (nrows < STEP) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * lg + r >= nrows) vb[r] = (__bf16)0.f;
      if (16 + 4 * lg + r >= nrows) vb[4 + r] = (__bf16)0.f;
    }
  }
  return vb;
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

struct ChainOps {
  bf16x8 tb[2], wn[8], kt[8], vb;
  floatx4 eg[8];
};

__device__ __forceinline__ void load_chain_ops(ChainOps& c, const unsigned char* rec, int lane, int lg, int li, int nrows) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) c.tb[mt] = ld8((const __bf16*)(rec + kOffTb + (mt * 64 + lane) * 16));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c.wn[i] = ld8((const __bf16*)(rec + kOffWn + (i * 64 + lane) * 16));
    c.kt[i] = ld8((const __bf16*)(rec + kOffKt + (i * 64 + lane) * 16));
    c.eg[i] = *reinterpret_cast<const floatx4*>(rec + kOffEg + (lg * 32 + 4 * i) * 4);
  }
  c.vb = v_operand(rec, lg, li, nrows);
}

struct OutOps {
  bf16x8 ph[2], qh[8], vb;
  StepMeta meta;
};

__device__ __forceinline__ void load_out_ops(OutOps& c, const unsigned char* rec, int lane, int lg, int li, int nrows) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) c.ph[mt] = ld8((const __bf16*)(rec + kOffPh + (mt * 64 + lane) * 16));
#pragma unroll
  for (int i = 0; i < 8; ++i) c.qh[i] = ld8((const __bf16*)(rec + kOffQh + (i * 64 + lane) * 16));
  c.vb = v_operand(rec, lg, li, nrows);
  c.meta = *reinterpret_cast<const StepMeta*>(rec + kOffMeta);
}

__device__ __forceinline__ int rows_of(int64_t T, int64_t st) {
  const int64_t rem = T - st * STEP;
  return rem < STEP ? (int)rem : STEP;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(Params p, int64_t n_steps, int xcd_map) {
  extern __shared__ __align__(16) unsigned char ring[];
  unsigned char* sbuf = ring + (size_t)kRing * kSlotBytes;   // two state buffers
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t BH = p.B * p.H;
  int64_t bh;
  int slice;
  if (xcd_map) {   // keep the 8 slices of one (b,h) on the same XCD (workgroups are dealt round-robin over 8 XCDs)
    const int64_t id = blockIdx.x, x = id & 7, j = id >> 3;
    bh = (j >> 3) * 8 + x;
    slice = (int)(j & 7);
  } else {
    bh = blockIdx.x >> 3;
    slice = (int)(blockIdx.x & 7);
  }
  if (bh >= BH) return;   // uniform over the workgroup
  const int64_t T = p.T;
  const int d0 = slice * 16;
  const unsigned char* recs = (const unsigned char*)p.workspace + bh * n_steps * (int64_t)kRecBytes;
  const uint16_t* v = (const uint16_t*)p.v + bh * T * D;
  const floatx4 zero = {0, 0, 0, 0};

  if (wave >= 2) {
    // ---------------- loader wavefronts
    const int L = wave - 2;
    auto issue = [&](int64_t st) {
      unsigned char* slot = ring + (st % kRing) * kSlotBytes;
      const unsigned char* src = recs + st * (int64_t)kRecBytes;
#pragma unroll
      for (int x = 0; x < kLoadsPerLoader; ++x) {
        const int j = L + kLoaders * x;
        if (j < kLoadsPerStep - 1) {
          __builtin_amdgcn_global_load_lds((const void*)(src + j * 1024 + lane * 16), (lds_void*)(slot + j * 1024), 16, 0, 0);
        } else {   // V rows: lane -> (row, 16-byte half); rows past the end read the last row (masked later)
          int64_t t = st * STEP + (lane >> 1);
          t = t < T ? t : T - 1;
          __builtin_amdgcn_global_load_lds((const void*)(v + t * D + d0 + (lane & 1) * 8), (lds_void*)(slot + kRecBytes), 16, 0, 0);
        }
      }
    };
    for (int64_t st = 0; st < kRing - 1 && st < n_steps; ++st) issue(st);
    for (int64_t s = 0; s < n_steps; ++s) {
      // at barrier s, slots s and s+1 must be complete
      const int64_t issued_max = (s + kRing - 2 < n_steps - 1) ? s + kRing - 2 : n_steps - 1;
      const int64_t need = (s + 1 < n_steps - 1) ? s + 1 : n_steps - 1;
      wait_vm_dyn((int)(issued_max - need));
      block_barrier();
      if (s + kRing - 1 < n_steps) issue(s + kRing - 1);
    }
    return;
  }

  if (wave == 0) {
    // ---------------- chain wavefront: the state slice lives here, in fp32
    floatx4 S[8];
    if (p.S0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][r] = p.S0[(bh * D + 16 * t + 4 * lg + r) * D + d0 + li];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = zero;
    }
    bf16x8 sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sb[u] = pack2(S[2 * u], S[2 * u + 1]);
      *reinterpret_cast<bf16x8*>(sbuf + (u * 64 + lane) * 16) = sb[u];
    }
    ChainOps cur;
    for (int64_t s = 0; s < n_steps; ++s) {
      block_barrier();
      if (s == 0) load_chain_ops(cur, ring, lane, lg, li, rows_of(T, 0));
      floatx4 cdec[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) cdec[t][r] = S[t][r] * cur.eg[t][r];
      floatx4 U[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) U[mt] = mfma(cur.tb[mt], cur.vb, zero);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) U[mt] = mfma(cur.wn[mt * 4 + u], sb[u], U[mt]);
      const bf16x8 ub = pack2(U[0], U[1]);
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = mfma(cur.kt[t], ub, cdec[t]);
      // operands of the next step (its slot is complete since this step's barrier)
      if (s + 1 < n_steps) load_chain_ops(cur, ring + ((s + 1) % kRing) * kSlotBytes, lane, lg, li, rows_of(T, s + 1));
      unsigned char* nb = sbuf + ((s + 1) & 1) * kStateBufBytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sb[u] = pack2(S[2 * u], S[2 * u + 1]);
        *reinterpret_cast<bf16x8*>(nb + (u * 64 + lane) * 16) = sb[u];
      }
    }
    uint32_t nonfinite = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p.S_final[(bh * D + 16 * t + 4 * lg + r) * D + d0 + li] = S[t][r];
        nonfinite += not_finite(S[t][r]) ? 1u : 0u;
      }
    if (p.stats) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) nonfinite += __shfl_xor(nonfinite, off);
      if (lane == 0 && nonfinite) atomicAdd(&p.stats->n_nonfinite, nonfinite);
    }
    return;
  }

  // ---------------- output wavefront
  uint16_t* o = (uint16_t*)p.o + bh * T * D + (4 * lg) * D + d0 + li;
  uint32_t nonfinite = 0, n_valid = 0, n_flagged = 0;
  float min_span = __int_as_float(0x7f800000);
  OutOps cur;
  for (int64_t s = 0; s < n_steps; ++s) {
    block_barrier();
    if (s == 0) load_out_ops(cur, ring, lane, lg, li, rows_of(T, 0));
    const int nrows = rows_of(T, s);
    const unsigned char* cb = sbuf + (s & 1) * kStateBufBytes;
    bf16x8 sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sb[u] = ld8((const __bf16*)(cb + (u * 64 + lane) * 16));
    floatx4 O[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) O[mt] = mfma(cur.ph[mt], cur.vb, zero);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) O[mt] = mfma(cur.qh[mt * 4 + u], sb[u], O[mt]);
    if (slice == 0) {
      n_valid += cur.meta.n_valid;
      n_flagged += cur.meta.n_flagged;
      min_span = fminf(min_span, fminf(cur.meta.span[0], cur.meta.span[1]));
    }
    if (s + 1 < n_steps) load_out_ops(cur, ring + ((s + 1) % kRing) * kSlotBytes, lane, lg, li, rows_of(T, s + 1));
    uint16_t* os = o + s * STEP * D;
    uint32_t mx = 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * lg + r;
        if (nrows == STEP || row < nrows) {
          os[(16 * mt + r) * D] = __builtin_bit_cast(uint16_t, (__bf16)O[mt][r]);
          mx = max(mx, abs_bits(O[mt][r]));
        }
      }
    if (mx >= 0x7f800000u) {   // rare: count exactly
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          nonfinite += ((nrows == STEP || 16 * mt + 4 * lg + r < nrows) && abs_bits(O[mt][r]) >= 0x7f800000u) ? 1u : 0u;
    }
  }
  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nonfinite += __shfl_xor(nonfinite, off);
    if (lane == 0) {
      if (nonfinite) atomicAdd(&p.stats->n_nonfinite, nonfinite);
      if (slice == 0) {
        atomicAdd(&p.stats->n_chunks, n_valid);
        if (n_flagged) atomicAdd(&p.stats->n_flagged, n_flagged);
        if (n_valid) atomic_min_float(&p.stats->min_span, min_span);
      }
    }
  }
}

}  // namespace

bool mfma_supported(const Params& p) {
  return p.dtype == KDA_DTYPE_BF16 && p.dk == D && p.dv == D;
}

size_t mfma_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv) {
  if (dk != D || dv != D) return 0;
  const int64_t n_steps = (T + STEP - 1) / STEP;
  return (size_t)(B * H * n_steps) * kRecBytes;
}

hipError_t launch_mfma(const Params& p, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int64_t n_steps = (p.T + STEP - 1) / STEP;
  const int64_t BH = p.B * p.H;
  const size_t smem = sizeof(PrepShared);
  const size_t smem_scan = kScanSmem;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)scan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_scan);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(BH * n_steps)), dim3(256), smem, s, p, n_steps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int xcd_map = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)(BH * 8)), dim3(kScanThreads), smem_scan, s, p, n_steps, xcd_map);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace kda

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
#include "kda_mfma_util.h"

namespace kda {

namespace {

constexpr int D = 128;     // dk = dv
constexpr int STEP = 32;   // tokens per step (two chunks)

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

__device__ __forceinline__ float bf(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// ------------------------------------------------------------------ prep kernel
//
// Thread layout of the elementwise phase: tid = c*128 + pair*2 + half; the
// thread owns channels 2*pair, 2*pair+1 of chunk c at positions
// 16c + 8*half + j (j < 8).  The in-chunk prefix crosses the two halves with
// one lane shuffle.  Shared memory is ~70 KB so two workgroups share a CU;
// arrays of the later phases alias ones that are dead by then.

constexpr int kRow = D + 8;        // padded row of a [position][channel] bf16 array
constexpr int kRowT = STEP + 8;    // padded row of a [channel][position] bf16 array

struct PrepShared {
  // ---- live from the elementwise phase through the tile phase
  alignas(16) __bf16 Qb[STEP][kRow];     // q e^{L} (chunk-local), kept for Qbar = Qb e^{Gam_0 [chunk 1]}
  alignas(16) __bf16 Kb[STEP][kRow];     // k e^{L}      | per-pair fallback: raw k of a flagged chunk
  alignas(16) __bf16 Kh[STEP][kRow];     // k e^{-L}     | per-pair fallback: raw q of a flagged chunk
  alignas(16) __bf16 Kt0[16][kRow];      // k e^{Gam_0 - L}, chunk 0 (block coupling chunk 1 to chunk 0)
  alignas(16) __bf16 KbarT[D][kRowT];    // (k e^{G})^T, G referenced to the step start | later (-W)^T
  alignas(16) __bf16 KtilT[D][kRowT];    // (k e^{Gam_step - G})^T
  alignas(16) float L[16][D];            // in-chunk prefix (log2 units) of one flagged chunk
  alignas(16) float A[STEP][STEP + 1], P[STEP][STEP + 1];
  alignas(16) float Gam[2][D];           // chunk spans per channel, log2 units
  alignas(16) float eGam0[D];            // e^{Gam_0}
  alignas(16) float beta[STEP];
  alignas(16) float red[4];
  alignas(16) int pairwise[2];
};

// arrays of the solve phase, placed over Kb / Kh / Kt0 (dead after the tile phase)
struct SolveShared {
  alignas(16) float T[STEP][STEP + 1];
  alignas(16) float X[16][17];
  alignas(16) __bf16 Tb[STEP][kRowT];    // T diag(beta)
  alignas(16) __bf16 TbT[STEP][kRowT];   // (T diag(beta))^T
  alignas(16) __bf16 Pb[STEP][kRowT];    // P
  alignas(16) __bf16 Ph[STEP][kRowT];    // P T diag(beta)
};
static_assert(sizeof(SolveShared) <= sizeof(__bf16) * (2 * STEP + 16) * kRow, "solve arrays must fit over Kb, Kh, Kt0");

// diagonal block of chunk cc from per-pair factors exp(L_r - L_j) <= 1 (no reciprocal); raw q in Kh rows,
// raw k in Kb rows, L of the chunk in L[][]
__device__ void pairwise_block(PrepShared& sm, int cc, int lane) {
  for (int pr = lane; pr < 136; pr += 64) {
    int r = 0;
    while ((r + 1) * (r + 2) / 2 <= pr) ++r;
    const int j = pr - r * (r + 1) / 2;                 // j <= r
    const int R = 16 * cc + r, J = 16 * cc + j;
    float a = 0.f, pq = 0.f;
    for (int x = 0; x < D; ++x) {
      const float e = __builtin_amdgcn_exp2f(sm.L[r][x] - sm.L[j][x]);
      const float kj = (float)sm.Kb[J][x] * e;
      a += (float)sm.Kb[R][x] * kj;
      pq += (float)sm.Kh[R][x] * kj;
    }
    sm.A[R][J] = (j < r) ? sm.beta[R] * a : 0.f;
    sm.P[R][J] = pq;
  }
  for (int pr = lane; pr < 256; pr += 64) {            // upper triangle of the block
    const int r = pr >> 4, j = pr & 15;
    if (j > r) { sm.A[16 * cc + r][16 * cc + j] = 0.f; sm.P[16 * cc + r][16 * cc + j] = 0.f; }
  }
}

__global__ __launch_bounds__(256, 2) void prep_kernel(Params p, int64_t n_steps) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepShared& sm = *reinterpret_cast<PrepShared*>(smem_raw);
  SolveShared& so = *reinterpret_cast<SolveShared*>(&sm.Kb[0][0]);
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

  // ---- phase 1: gate, chunk-local prefix, scaled operands
  const int c = tid >> 7, pair = (tid >> 1) & 63, half = tid & 1;
  const int ch = 2 * pair;
  const int pos0 = 16 * c + 8 * half;
  uint32_t qq[8], kk[8], ww[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {     // all loads in flight together; addresses clamped into the sequence
    const int64_t t = t0 + pos0 + j;
    const int64_t tc = t < T ? t : T - 1;
    qq[j] = *reinterpret_cast<const uint32_t*>(q + tc * D + ch);
    kk[j] = *reinterpret_cast<const uint32_t*>(k + tc * D + ch);
    ww[j] = *reinterpret_cast<const uint32_t*>(w + tc * D + ch);
  }
  if (tid < STEP) sm.beta[tid] = (t0 + tid < T) ? bf(beta, t0 + tid) : 0.f;
  float L0[8], L1[8];               // prefix within this thread's 8 positions, channels ch and ch+1
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool ok = t0 + pos0 + j < T;
    if (!ok) { qq[j] = 0u; kk[j] = 0u; }
    a0 += ok ? gate_log2(lo_bf16(ww[j]), p.g_min, p.unbounded) : 0.f;
    a1 += ok ? gate_log2(hi_bf16(ww[j]), p.g_min, p.unbounded) : 0.f;
    L0[j] = a0;
    L1[j] = a1;
  }
  const float o0 = __shfl_xor(a0, 1), o1 = __shfl_xor(a1, 1);   // the other half's total
  const float base0 = half ? o0 : 0.f, base1 = half ? o1 : 0.f;
  const float gam0 = a0 + o0, gam1 = a1 + o1;                   // chunk span per channel (log2 units)
#pragma unroll
  for (int j = 0; j < 8; ++j) { L0[j] += base0; L1[j] += base1; }
  if (half == 0) { sm.Gam[c][ch] = gam0; sm.Gam[c][ch + 1] = gam1; }
  float m = fminf(gam0, gam1);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fminf(m, __shfl_xor(m, off));
  if (lane == 0) sm.red[wave] = m;
  float eL0[8], eL1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pp = pos0 + j;
    eL0[j] = __builtin_amdgcn_exp2f(L0[j]);
    eL1[j] = __builtin_amdgcn_exp2f(L1[j]);
    const float q0 = lo_bf16(qq[j]), q1 = hi_bf16(qq[j]), k0 = lo_bf16(kk[j]), k1 = hi_bf16(kk[j]);
    *reinterpret_cast<uint32_t*>(&sm.Qb[pp][ch]) = pk_bf16(q0 * eL0[j], q1 * eL1[j]);
    *reinterpret_cast<uint32_t*>(&sm.Kb[pp][ch]) = pk_bf16(k0 * eL0[j], k1 * eL1[j]);
    *reinterpret_cast<uint32_t*>(&sm.Kh[pp][ch]) =
        pk_bf16(k0 * __builtin_amdgcn_exp2f(-L0[j]), k1 * __builtin_amdgcn_exp2f(-L1[j]));
  }
  __syncthreads();

  const bool valid0 = t0 < T;
  const bool valid1 = t0 + 16 < T;
  const float span0 = fminf(sm.red[0], sm.red[1]) * kLn2;
  const float span1 = fminf(sm.red[2], sm.red[3]) * kLn2;
  const bool flag0 = valid0 && span0 < kSpanLimit;
  const bool flag1 = valid1 && span1 < kSpanLimit;
  const bool pw0 = p.force_fallback || (flag0 && !p.disable_fallback);
  const bool pw1 = p.force_fallback || (flag1 && !p.disable_fallback);
  if (tid == 0) {
    StepMeta mt;
    mt.span[0] = valid0 ? span0 : __int_as_float(0x7f800000);
    mt.span[1] = valid1 ? span1 : __int_as_float(0x7f800000);
    mt.n_valid = (valid0 ? 1u : 0u) + (valid1 ? 1u : 0u);
    mt.n_flagged = (flag0 ? 1u : 0u) + (flag1 ? 1u : 0u);
    *reinterpret_cast<StepMeta*>(rec + kOffMeta) = mt;
  }
  // step-level quantities (G referenced to the start of the step)
  {
    const float G00 = sm.Gam[0][ch], G01 = sm.Gam[0][ch + 1];      // Gam_0 of my two channels
    const float G10 = sm.Gam[1][ch], G11 = sm.Gam[1][ch + 1];      // Gam_1
    const float gc0 = c ? G10 : G00, gc1 = c ? G11 : G01;           // Gam of my chunk
    const float e00 = __builtin_amdgcn_exp2f(G00), e01 = __builtin_amdgcn_exp2f(G01);
    const float s0 = c ? e00 : 1.f, s1 = c ? e01 : 1.f;            // e^{G - L}: 1 in chunk 0, e^{Gam_0} in chunk 1
    const float u0 = c ? 1.f : __builtin_amdgcn_exp2f(G10), u1 = c ? 1.f : __builtin_amdgcn_exp2f(G11);  // e^{Gam_1} for chunk 0
    uint32_t kb0[4], kb1[4], kt0[4], kt1[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float k0 = lo_bf16(kk[j]), k1 = hi_bf16(kk[j]);
      const float eg0 = __builtin_amdgcn_exp2f(gc0 - L0[j]), eg1 = __builtin_amdgcn_exp2f(gc1 - L1[j]);   // e^{Gam_c - L} <= 1
      const float kbar0 = k0 * eL0[j] * s0, kbar1 = k1 * eL1[j] * s1;
      const float ktil0 = k0 * eg0 * u0, ktil1 = k1 * eg1 * u1;
      if (j & 1) {
        kb0[j >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)kbar0) << 16;
        kb1[j >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)kbar1) << 16;
        kt0[j >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ktil0) << 16;
        kt1[j >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ktil1) << 16;
      } else {
        kb0[j >> 1] = __builtin_bit_cast(uint16_t, (__bf16)kbar0);
        kb1[j >> 1] = __builtin_bit_cast(uint16_t, (__bf16)kbar1);
        kt0[j >> 1] = __builtin_bit_cast(uint16_t, (__bf16)ktil0);
        kt1[j >> 1] = __builtin_bit_cast(uint16_t, (__bf16)ktil1);
      }
      if (c == 0) *reinterpret_cast<uint32_t*>(&sm.Kt0[pos0 + j][ch]) = pk_bf16(k0 * eg0, k1 * eg1);
    }
    typedef __attribute__((__vector_size__(16))) uint32_t u32x4;
    *reinterpret_cast<u32x4*>(&sm.KbarT[ch][pos0]) = u32x4{kb0[0], kb0[1], kb0[2], kb0[3]};
    *reinterpret_cast<u32x4*>(&sm.KbarT[ch + 1][pos0]) = u32x4{kb1[0], kb1[1], kb1[2], kb1[3]};
    *reinterpret_cast<u32x4*>(&sm.KtilT[ch][pos0]) = u32x4{kt0[0], kt0[1], kt0[2], kt0[3]};
    *reinterpret_cast<u32x4*>(&sm.KtilT[ch + 1][pos0]) = u32x4{kt1[0], kt1[1], kt1[2], kt1[3]};
    if (c == 0 && half == 0) {
      sm.eGam0[ch] = e00;
      sm.eGam0[ch + 1] = e01;
      // e^{Gam_step}, grouped by the scan's lane groups: index g*32 + t*4 + r <-> channel 16t + 4g + r
      float* eg = reinterpret_cast<float*>(rec + kOffEg);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int cx = ch + x, t = cx >> 4, g = (cx >> 2) & 3, r = cx & 3;
        eg[g * 32 + t * 4 + r] = __builtin_amdgcn_exp2f(x ? G01 + G11 : G00 + G10);
      }
    }
    if (pw0 && c == 0) {   // per-pair fallback inputs for chunk 0: L, raw k (in Kb rows), raw q (in Kh rows)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int l = 8 * half + j;
        sm.L[l][ch] = L0[j]; sm.L[l][ch + 1] = L1[j];
        *reinterpret_cast<uint32_t*>(&sm.Kb[l][ch]) = kk[j];
        *reinterpret_cast<uint32_t*>(&sm.Kh[l][ch]) = qq[j];
      }
    }
  }
  __syncthreads();

  // ---- phase 2: the 32x32 tiles.  wave 0: diagonal block of chunk 0 (A and P), wave 1: chunk 1,
  // wave 2: A coupling chunk 1 to chunk 0, wave 3: P coupling chunk 1 to chunk 0.
  if (wave == 0 && pw0) {
    pairwise_block(sm, 0, lane);
  } else if (wave <= 1 && !(wave == 1 && pw1)) {
    const int cc = wave;
    floatx4 accA = {0, 0, 0, 0}, accP = {0, 0, 0, 0};
#pragma unroll
    for (int kk4 = 0; kk4 < 4; ++kk4) {
      const int col = 32 * kk4 + 8 * lg;
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
  } else if (wave >= 2) {
    floatx4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int kk4 = 0; kk4 < 4; ++kk4) {
      const int col = 32 * kk4 + 8 * lg;
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
  if (pw1) {   // chunk 1's diagonal block per pair, once its dense operands are no longer needed
    __syncthreads();
    if (c == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int l = 8 * half + j;
        sm.L[l][ch] = L0[j]; sm.L[l][ch + 1] = L1[j];
        *reinterpret_cast<uint32_t*>(&sm.Kb[16 + l][ch]) = kk[j];
        *reinterpret_cast<uint32_t*>(&sm.Kh[16 + l][ch]) = qq[j];
      }
    }
    __syncthreads();
    if (wave == 1) pairwise_block(sm, 1, lane);
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
      so.T[b0 + r][j] = col[r];
      if (b0 == 16) so.T[r][j] = 0.f;                 // upper-right block
    }
  }
  __syncthreads();
  // ... then the coupling block T_10 = -T_11 (A_10 T_00)   (entries outside the triangles are zero)
  {
    const int r = tid >> 4, j = tid & 15;
    float x = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) x += sm.A[16 + r][n] * so.T[n][j];
    so.X[r][j] = x;
  }
  __syncthreads();
  {
    const int r = tid >> 4, j = tid & 15;
    float x = 0.f;
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) x += so.T[16 + r][16 + mm] * so.X[mm][j];
    so.T[16 + r][j] = -x;
  }
  __syncthreads();
  // T diag(beta) (row-major and transposed) and P in bf16
  for (int e = tid; e < STEP * STEP; e += 256) {
    const int r = e >> 5, j = e & 31;
    const __bf16 tb = (__bf16)(so.T[r][j] * sm.beta[j]);
    so.Tb[r][j] = tb;
    so.TbT[j][r] = tb;
    so.Pb[r][j] = (__bf16)sm.P[r][j];
  }
  __syncthreads();
  // Phat = P T diag(beta) on MFMA: wave w computes the 16x16 tile (w >> 1, w & 1)
  {
    const int mt = wave >> 1, nt = wave & 1;
    const floatx4 d = mfma(ld8(&so.Pb[16 * mt + li][8 * lg]), ld8(&so.TbT[16 * nt + li][8 * lg]), floatx4{0, 0, 0, 0});
#pragma unroll
    for (int r = 0; r < 4; ++r) so.Ph[16 * mt + 4 * lg + r][16 * nt + li] = (__bf16)d[r];
  }

  // ---- phase 4: W^T = Kbar^T (T diag(beta))^T on MFMA; wave owns channel tiles 2w, 2w+1
  floatx4 wd[2][2];
  {
    const int u = wave;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nt = 2 * u + h;
        wd[mt][h] = mfma(ld8(&sm.KbarT[16 * nt + li][8 * lg]), ld8(&so.Tb[16 * mt + li][8 * lg]), floatx4{0, 0, 0, 0});
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) { o[r] = (__bf16)(-wd[mt][0][r]); o[4 + r] = (__bf16)(-wd[mt][1][r]); }
      *reinterpret_cast<bf16x8*>(rec + kOffWn + ((mt * 4 + u) * 64 + lane) * 16) = o;
    }
  }
  __syncthreads();   // every wave is done reading Kbar^T: (-W)^T goes over it
  __bf16 (*WnT)[kRowT] = sm.KbarT;
  {
    const int u = wave;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) WnT[16 * (2 * u + h) + 4 * lg + r][16 * mt + li] = (__bf16)(-wd[mt][h][r]);
  }
  __syncthreads();

  // ---- phase 5: Qhat^T = Qbar^T - W^T P^T on MFMA, Qbar = Qb (chunk 0) or Qb e^{Gam_0} (chunk 1)
  {
    const int u = wave;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 d[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nt = 2 * u + h;
        const int c0 = 16 * nt + 4 * lg;
        const uint2 qv = *reinterpret_cast<const uint2*>(&sm.Qb[16 * mt + li][c0]);
        floatx4 cq = {lo_bf16(qv.x), hi_bf16(qv.x), lo_bf16(qv.y), hi_bf16(qv.y)};
        if (mt == 1) {
          const floatx4 e = *reinterpret_cast<const floatx4*>(&sm.eGam0[c0]);
#pragma unroll
          for (int r = 0; r < 4; ++r) cq[r] *= e[r];
        }
        d[h] = mfma(ld8(&WnT[16 * nt + li][8 * lg]), ld8(&so.Pb[16 * mt + li][8 * lg]), cq);
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
    const uint2 x0 = *reinterpret_cast<const uint2*>(&sm.KtilT[16 * t + i][4 * g]);
    const uint2 x1 = *reinterpret_cast<const uint2*>(&sm.KtilT[16 * t + i][16 + 4 * g]);
    *reinterpret_cast<uint4*>(rec + kOffKt + e * 16) = uint4{x0.x, x0.y, x1.x, x1.y};
  }
  if (tid < 128) {                                    // T diag(beta) and Phat, 2 row tiles each
    const int mt = tid >> 6, ln = tid & 63, i = ln & 15, g = ln >> 4;
    const uint2 a0 = *reinterpret_cast<const uint2*>(&so.Tb[16 * mt + i][4 * g]);
    const uint2 a1 = *reinterpret_cast<const uint2*>(&so.Tb[16 * mt + i][16 + 4 * g]);
    const uint2 b0 = *reinterpret_cast<const uint2*>(&so.Ph[16 * mt + i][4 * g]);
    const uint2 b1 = *reinterpret_cast<const uint2*>(&so.Ph[16 * mt + i][16 + 4 * g]);
    *reinterpret_cast<uint4*>(rec + kOffTb + tid * 16) = uint4{a0.x, a0.y, a1.x, a1.y};
    *reinterpret_cast<uint4*>(rec + kOffPh + tid * 16) = uint4{b0.x, b0.y, b1.x, b1.y};
  }
}

// ------------------------------------------------------------------ segmented scan
//
// Given the records, the step map S -> diag(e^{Gam}) S + Ktil^T (T diag(beta) V - W S) is affine in S,
// so the map of a run of steps is S_end = M S_start + X, with M (dk x dk) the product of the step
// transitions diag(e^{Gam}) - Ktil^T W and X the run's result from a zero state.  The steps of every
// (b, h) are cut into P segments of L steps:
//   seg_state_kernel    (b, h, segment j < P-1): X_j and M_j, both carried as 128 state columns through
//                       the step recurrence (M from the identity, with no V term)
//   seg_combine_kernel  (b, h, 16-column slice): S_start(j+1) = M_j S_start(j) + X_j, serially over j
//   seg_out_kernel      (b, h, segment j): the recurrence from S_start(j) with the outputs
//                       O = Qhat S + Phat V; the last segment writes S_final
// Every workgroup keeps all 128 columns of its segment's state, so each record is read from memory
// once per segment.  Within a workgroup, wavefront w owns the 16-column slice w (seg_state: one slice
// of X and one of M); all wavefronts also stream the records into a ring of LDS slots with
// direct-to-LDS 16-byte loads, kRingSlots-1 steps ahead of the compute.

constexpr int kRingSlots = 4;
constexpr int kSegWaves = 8;
constexpr int kSegThreads = 64 * kSegWaves;
constexpr int kVTileBytes = STEP * D * 2;                    // one step of V, all 128 columns, row-major
static_assert(2 * kMHalf == kSegState, "hi + lo parts of M fill one block");

// seg_out slot: the whole record, then V
constexpr int kOutSlot = kRecBytes + kVTileBytes;
constexpr int kOutChunks = kOutSlot / 1024;                  // 37
// seg_state slot: -W, Ktil^T, T diag(beta), e^{Gam} (+ meta), then V
constexpr int kStWn = 0, kStKt = 8192, kStTb = 16384, kStEg = 18432, kStV = 19456;
constexpr int kStSlot = kStV + kVTileBytes;
constexpr int kStChunks = kStSlot / 1024;                    // 27
constexpr size_t kOutSmem = (size_t)kRingSlots * kOutSlot;
constexpr size_t kStSmem = (size_t)kRingSlots * kStSlot;
static_assert(kOutSmem <= 163840 && kStSmem <= 163840, "LDS budget");
static_assert(kOutSlot % 1024 == 0 && kStSlot % 1024 == 0, "slots are whole 1 KiB chunks");
static_assert((kOutChunks / kSegWaves + 1) * (kRingSlots - 1) + 4 <= 63, "outstanding loads fit the vmcnt counter");

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima)
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most k * PER of this wave's memory operations are outstanding (k = steps in flight
// beyond the one needed, each of at least PER loads; later stores only make the wait longer)
template <int PER> __device__ __forceinline__ void wait_steps(int64_t k) {
  if (k <= 0) wait_vm<0>();
  else if (k == 1) wait_vm<PER>();
  else wait_vm<2 * PER>();
}
static_assert(kRingSlots - 2 <= 2, "wait_steps covers at most two steps in flight");

__device__ __forceinline__ void lds_load16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// one 1 KiB chunk (rows 4c..4c+3) of a step's V tile; rows at or past T re-read row T-1 (masked later)
__device__ __forceinline__ void load_v_chunk(const uint16_t* v, int64_t T, int64_t step, int c, int lane,
                                             unsigned char* dst) {
  int64_t t = step * STEP + 4 * c + (lane >> 4);
  t = t < T ? t : T - 1;
  lds_load16(v + t * D + (lane & 15) * 8, dst);
}

// B operand of V for columns col (rows {4g+r, 16+4g+r}); rows at or past nrows are zero
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* vt, int lg, int col, int nrows) {
  const __bf16* vr = (const __bf16*)vt;
  bf16x8 vb;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    vb[r] = vr[(4 * lg + r) * D + col];
    vb[4 + r] = vr[(16 + 4 * lg + r) * D + col];
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

__device__ __forceinline__ int rows_of(int64_t T, int64_t st) {
  const int64_t rem = T - st * STEP;
  return rem < STEP ? (int)rem : STEP;
}

// ---- seg_state_kernel: X_j and M_j of segment j < P-1
__global__ __launch_bounds__(kSegThreads) void seg_state_kernel(Params p, int64_t n_steps, SegPlan sg) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t nseg = sg.P - 1;
  const int64_t bh = blockIdx.x / nseg, j = blockIdx.x % nseg;
  const int64_t s0 = j * sg.L;
  const int64_t ns = sg.L;                 // never the last segment, so always a full one
  const int64_t T = p.T;
  const unsigned char* recs = (const unsigned char*)p.workspace + (bh * n_steps + s0) * (int64_t)kRecBytes;
  const uint16_t* v = (const uint16_t*)p.v + bh * T * D;
  constexpr int kPer = kStChunks / kSegWaves;          // loads per step of the wave with the fewest
  auto issue = [&](int64_t i) {
    unsigned char* slot = ring + (i % kRingSlots) * kStSlot;
    const unsigned char* src = recs + i * (int64_t)kRecBytes;
#pragma unroll
    for (int x = 0; x < (kStChunks + kSegWaves - 1) / kSegWaves; ++x) {
      const int c = wave + kSegWaves * x;
      if (c < 18) {                         // -W (record chunks 0..7), Ktil^T and T diag(beta) (16..25)
        const int rc = c < 8 ? c : c + 8;
        lds_load16(src + rc * 1024 + lane * 16, slot + c * 1024);
      } else if (c == 18) {                 // e^{Gam} and meta (record chunk 28)
        lds_load16(src + 28 * 1024 + lane * 16, slot + kStEg);
      } else if (c < kStChunks) {
        load_v_chunk(v, T, s0 + i, c - 19, lane, slot + kStV + (c - 19) * 1024);
      }
    }
  };
  for (int64_t i = 0; i < kRingSlots - 1 && i < ns; ++i) issue(i);

  const floatx4 zero = {0, 0, 0, 0};
  floatx4 X[8], M[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    X[t] = zero;
#pragma unroll
    for (int r = 0; r < 4; ++r) M[t][r] = (16 * t + 4 * lg + r == 16 * wave + li) ? 1.f : 0.f;
  }
  bf16x8 xb[4], mb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) { xb[u] = pack2(X[2 * u], X[2 * u + 1]); mb[u] = pack2(M[2 * u], M[2 * u + 1]); }

  for (int64_t i = 0; i < ns; ++i) {
    const int64_t issued = (i + kRingSlots - 2 < ns - 1) ? i + kRingSlots - 2 : ns - 1;
    wait_steps<kPer>(issued - i);
    block_barrier();
    if (i + kRingSlots - 1 < ns) issue(i + kRingSlots - 1);
    const unsigned char* slot = ring + (i % kRingSlots) * kStSlot;
    const bf16x8 vb = v_operand(slot + kStV, lg, 16 * wave + li, rows_of(T, s0 + i));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const floatx4 eg = *reinterpret_cast<const floatx4*>(slot + kStEg + (lg * 32 + 4 * t) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) { X[t][r] *= eg[r]; M[t][r] *= eg[r]; }
    }
    floatx4 UX[2], UM[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      UX[mt] = mfma(ld8((const __bf16*)(slot + kStTb + (mt * 64 + lane) * 16)), vb, zero);
      UM[mt] = zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 wn = ld8((const __bf16*)(slot + kStWn + ((mt * 4 + u) * 64 + lane) * 16));
        UX[mt] = mfma(wn, xb[u], UX[mt]);
        UM[mt] = mfma(wn, mb[u], UM[mt]);
      }
    const bf16x8 ux = pack2(UX[0], UX[1]), um = pack2(UM[0], UM[1]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 kt = ld8((const __bf16*)(slot + kStKt + (t * 64 + lane) * 16));
      X[t] = mfma(kt, ux, X[t]);
      M[t] = mfma(kt, um, M[t]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) { xb[u] = pack2(X[2 * u], X[2 * u + 1]); mb[u] = pack2(M[2 * u], M[2 * u + 1]); }
  }
  // X_j in slice-major D layout; M_j split into bf16 hi + lo parts, each arranged as the combine's
  // A operands: [mo 8][u 4][lane 64][8] <-> M[16 mo + (lane & 15)][32 u + {0, 16} + 4 (lane >> 4) + r]
  const int64_t blk = bh * sg.P + j;
  float* xo = (float*)((unsigned char*)p.workspace + sg.off_x + blk * (int64_t)kSegState) + wave * 8 * 64 * 4;
  store_slice(xo, X, lane);
  __bf16* mh = (__bf16*)((unsigned char*)p.workspace + sg.off_m + blk * (int64_t)kSegState);
  __bf16* ml = mh + kMHalf / 2;
  const int u = wave >> 1, pos = (wave & 1) * 4 + (li & 3);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // element M[16t + 4lg + r][16 wave + li]
      const int lane_c = (4 * lg + r) + 16 * (li >> 2);
      const int e = ((t * 4 + u) * 64 + lane_c) * 8 + pos;
      const __bf16 hi = (__bf16)M[t][r];
      mh[e] = hi;
      ml[e] = (__bf16)(M[t][r] - (float)hi);
    }
}

// ---- seg_combine_kernel: S_start(j+1) = M_j S_start(j) + X_j for one 16-column slice.  The product
// runs on bf16 MFMA in three passes, Mhi Shi + Mhi Slo + Mlo Shi (hi/lo: bf16 value and bf16 residual),
// which leaves a relative error near 2^-16, with fp32 accumulation.  Wavefront w owns the output row
// tiles 2w, 2w+1; the D-layout tiles of S feed the B operands directly through the permuted
// contraction order.  M_j and X_j are fetched two segments ahead.
// first = 0: the chain starts from S0 at segment 0 (records path).  first = 1 (fused path): the map
// pass already ran segment 0 with its outputs and left its leaving state in the block of segment 1,
// where the chain starts, and a statistics record per head, which workgroup 0 turns into the call's
// counters before the output pass adds to them.
__device__ __forceinline__ void split_bf16(floatx4 a, floatx4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = (__bf16)a[r];
    hi[4 + r] = (__bf16)b[r];
    lo[r] = (__bf16)(a[r] - (float)hi[r]);
    lo[4 + r] = (__bf16)(b[r] - (float)hi[4 + r]);
  }
}

struct CombineOps {
  bf16x8 mh[2][4], ml[2][4];
  floatx4 x[2];
};

// Chains the maps of one (b, h): S_start(j + 1) = M_j S_start(j) + X_j, fp32 via bf16 hi/lo products.
// first = 0 (records path): from S0 over maps 0 .. P-2.  first = 1: from S_start(1), which segment 0
// wrote, over maps 1 .. P-2 (fused plan), or over maps 1 .. P-1 (corr = 1, the corrected plan, whose
// last map gives S_final, written in the user's layout with its non-finite values counted).
__global__ __launch_bounds__(256) void seg_combine_kernel(Params p, SegPlan sg, int first, int corr) {
  __shared__ floatx4 Sx[2][8][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  // the grid is 8 slices x B*H: consecutive block ids go round-robin over the 8 XCDs, so block b
  // takes logical id (b % 8) (grid / 8) + b / 8, and the 8 slices of a head, which all read the same
  // M_j, share one XCD's L2 (whole heads whenever B*H is a multiple of 8)
  const int64_t lb = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t bh = lb >> 3;
  const int slice = (int)(lb & 7);
  const int64_t nseg = corr ? sg.P : sg.P - 1;   // maps first .. nseg-1 are chained
  const unsigned char* ws = (const unsigned char*)p.workspace;
  if (first && !corr && p.stats && blockIdx.x == 0) {   // uniform over workgroup 0: one head per thread, then a reduction
    const int64_t BH = p.B * p.H;
    uint32_t n_chunks = 0, n_flagged = 0, n_nonfinite = 0;
    float min_span = __int_as_float(0x7f800000);
    for (int64_t b = tid; b < BH; b += 256) {
      const uint32_t* rec = (const uint32_t*)(ws + sg.off_s + b * sg.P * (int64_t)kSegState);
#pragma unroll
      for (int i = kRecNonfinite; i < kRecChunks; ++i) n_nonfinite += rec[i];
      n_chunks += rec[kRecChunks];
      n_flagged += rec[kRecFlagged];
      if (rec[kRecChunks]) min_span = fminf(min_span, __uint_as_float(rec[kRecMinSpan]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      n_chunks += __shfl_xor(n_chunks, off);
      n_flagged += __shfl_xor(n_flagged, off);
      n_nonfinite += __shfl_xor(n_nonfinite, off);
      min_span = fminf(min_span, __shfl_xor(min_span, off));
    }
    __shared__ uint32_t red[4][4];
    if (lane == 0) {
      red[wave][0] = n_chunks;
      red[wave][1] = n_flagged;
      red[wave][2] = n_nonfinite;
      red[wave][3] = __float_as_uint(min_span);
    }
    __syncthreads();
    if (tid == 0) {
      for (int v = 1; v < 4; ++v) {
        n_chunks += red[v][0];
        n_flagged += red[v][1];
        n_nonfinite += red[v][2];
        min_span = fminf(min_span, __uint_as_float(red[v][3]));
      }
      p.stats->n_chunks = n_chunks;
      p.stats->n_flagged = n_flagged;
      p.stats->n_nonfinite = n_nonfinite;
      p.stats->min_span = min_span;
    }
  }
  floatx4 cur[2];
  if (first) {
    const float* s1 = (const float*)(ws + sg.off_s + (bh * sg.P + 1) * (int64_t)kSegState) + slice * 8 * 64 * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) cur[h] = *reinterpret_cast<const floatx4*>(s1 + ((2 * wave + h) * 64 + lane) * 4);
  } else {
    // records path: the chain starts from S0, which is also copied into segment 0's entering-state
    // block, where the output pass reads it (S_final may be S0: the output pass's last segment
    // overwrites S0 while its first segment would still be reading it)
    float* s0b = (float*)((unsigned char*)p.workspace + sg.off_s + bh * sg.P * (int64_t)kSegState) + slice * 8 * 64 * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mo = 2 * wave + h;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cur[h][r] = p.S0 ? p.S0[(bh * D + 16 * mo + 4 * lg + r) * D + 16 * slice + li] : 0.f;
      *reinterpret_cast<floatx4*>(s0b + (mo * 64 + lane) * 4) = cur[h];
    }
  }
  auto fetch = [&](CombineOps& c, int64_t j) {
    const int64_t blk = bh * sg.P + j;
    const unsigned char* mb = ws + sg.off_m + blk * (int64_t)kSegState;
    const float* xj = (const float*)(ws + sg.off_x + blk * (int64_t)kSegState) + slice * 8 * 64 * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mo = 2 * wave + h;
      c.x[h] = *reinterpret_cast<const floatx4*>(xj + (mo * 64 + lane) * 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int off = ((mo * 4 + u) * 64 + lane) * 16;
        c.mh[h][u] = *reinterpret_cast<const bf16x8*>(mb + off);
        c.ml[h][u] = *reinterpret_cast<const bf16x8*>(mb + kMHalf + off);
      }
    }
  };
  auto step = [&](const CombineOps& c, int64_t j) {
    floatx4 (*sx)[64] = Sx[j & 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) sx[2 * wave + h][lane] = cur[h];
    __syncthreads();
    bf16x8 sh[4], sl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) split_bf16(sx[2 * u][lane], sx[2 * u + 1][lane], sh[u], sl[u]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      floatx4 acc = c.x[h];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc = mfma(c.ml[h][u], sh[u], acc);
        acc = mfma(c.mh[h][u], sl[u], acc);
        acc = mfma(c.mh[h][u], sh[u], acc);
      }
      cur[h] = acc;
    }
    if (j + 1 < sg.P) {
      float* sn = (float*)((unsigned char*)p.workspace + sg.off_s + (bh * sg.P + j + 1) * (int64_t)kSegState) +
                  slice * 8 * 64 * 4;
#pragma unroll
      for (int h = 0; h < 2; ++h) *reinterpret_cast<floatx4*>(sn + ((2 * wave + h) * 64 + lane) * 4) = cur[h];
    } else {   // the corrected plan's last map: the final state
      uint32_t bad = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (2 * wave + h) + 4 * lg + r;
          p.S_final[(bh * D + row) * D + 16 * slice + li] = cur[h][r];
          bad += not_finite(cur[h][r]) ? 1u : 0u;
        }
      if (p.stats) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
        if (lane == 0 && bad) atomicAdd(&p.stats->n_nonfinite, bad);
      }
    }
  };
  // Every fetch is issued, its segment clamped to the last map (a valid block whose values are then
  // unused): fetches under a branch would make the memory-counter wait before each use also wait for
  // the loads issued after it, the prefetch of the next segment included.
  const int64_t last = nseg - 1;   // nseg >= 1: the kernel runs for plans of two or more segments
  auto ahead = [&](int64_t j) { return j < last ? j : last; };
  CombineOps c0, c1;
  fetch(c0, ahead(first));
  fetch(c1, ahead(first + 1));
  for (int64_t j = first; j < nseg; j += 2) {
    step(c0, j);
    fetch(c0, ahead(j + 2));
    if (j + 1 < nseg) step(c1, j + 1);
    fetch(c1, ahead(j + 3));
  }
}

// ---- correct_kernel: the corrected plan's outputs of segments 1 .. P-1, o_t += Qtil_t S_start(j)
// (Qtil_t: the propagated queries the segment pass stored, 32 x 128 bf16 per step; S_start(j): the
// chained entering state, fp32, as bf16 hi + lo parts).  Each workgroup takes kCorSteps consecutive
// steps of one segment; wavefront w owns output columns 16 w .. 16 w + 15.  Per step the workgroup
// stages Qtil and the 32 output rows in LDS with 16-byte loads (whole 256-byte rows), each wavefront
// adds its 32 x 16 block of the product, and the rows go back with 16-byte stores.  The next step's
// loads are issued before the current step's products, so one step of loads is always in flight.
constexpr int kCorSteps = 16;
constexpr int kCorThreads = 512;
constexpr int kCorRow = 272;   // staged output row: 256 bytes of data, 16 of pad (column reads spread over the banks)

__device__ __forceinline__ int64_t xcd_logical(int64_t b, int64_t G) {
  // blocks go round-robin over the 8 XCDs: number XCD x's blocks x (G / 8) + min(x, G % 8) onward, so
  // that consecutive logical ids (steps of one segment, which read the same entering state) share an L2
  const int64_t x = b & 7, i = b >> 3;
  return x * (G >> 3) + (x < (G & 7) ? x : (G & 7)) + i;
}

__global__ __launch_bounds__(kCorThreads) void correct_kernel(Params p, int64_t n_steps, SegPlan sg, int64_t cps) {
  __shared__ __align__(16) unsigned char qs[8 * 1024];
  __shared__ __align__(16) unsigned char os[STEP * kCorRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t lb = xcd_logical(blockIdx.x, gridDim.x);
  const int64_t seg = lb / cps, c = lb % cps;
  const int64_t bh = seg / (sg.P - 1);
  const int64_t j = 1 + seg % (sg.P - 1);
  const int64_t s0 = sg.L0 + (j - 1) * sg.L;
  const int64_t len = (n_steps - s0 < sg.L) ? n_steps - s0 : sg.L;
  const int64_t a = c * kCorSteps;
  if (a >= len) return;   // uniform over the workgroup: past the end of a short last segment
  const int64_t cnt = (len - a < kCorSteps) ? len - a : kCorSteps;
  const int64_t T = p.T;

  // entering state, columns 16 w .. 16 w + 15 as the A operands (hi and lo)
  bf16x8 sh[4], sl[4];
  {
    floatx4 S[8];
    load_slice(S, (const float*)((const unsigned char*)p.workspace + sg.off_s) +
                      (bh * sg.P + j) * (int64_t)(kSegState / 4) + w * 8 * 64 * 4, lane);
#pragma unroll
    for (int u = 0; u < 4; ++u) split_bf16(S[2 * u], S[2 * u + 1], sh[u], sl[u]);
  }
  const unsigned char* qbase = (const unsigned char*)p.workspace + sg.off_q + (bh * n_steps + s0 + a) * (int64_t)kQtStep;
  uint16_t* obase = (uint16_t*)p.o + bh * T * D;
  const int orow = tid >> 4, ocol = (tid & 15) * 8;   // this thread's 16 bytes of the staged rows
  auto rows_of = [&](int64_t st) { const int64_t r = T - st * STEP; return r < STEP ? (int)r : STEP; };
  uint4 qreg, oreg;
  auto fetch = [&](int64_t i) {
    const int64_t st = s0 + a + i;
    qreg = *reinterpret_cast<const uint4*>(qbase + i * (int64_t)kQtStep + tid * 16);
    oreg = orow < rows_of(st) ? *reinterpret_cast<const uint4*>(obase + (st * STEP + orow) * D + ocol) : uint4{0, 0, 0, 0};
  };
  fetch(0);
  uint32_t bad = 0;
#pragma unroll 1
  for (int64_t i = 0; i < cnt; ++i) {
    const int64_t st = s0 + a + i;
    const int nrows = rows_of(st);
    *reinterpret_cast<uint4*>(qs + tid * 16) = qreg;
    *reinterpret_cast<uint4*>(os + orow * kCorRow + ocol * 2) = oreg;
    __syncthreads();
    if (i + 1 < cnt) fetch(i + 1);
    // B operand (mt, u), lane (li, g): Qtil[16 mt + li][32 u + {4 g + r, 16 + 4 g + r}] = the mt-th
    // 8 bytes of blocks [2 u][lane] and [2 u + 1][lane] as the segment pass stored them
    floatx4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 x = *reinterpret_cast<const uint4*>(qs + ((2 * u) * 64 + lane) * 16);
      const uint4 y = *reinterpret_cast<const uint4*>(qs + ((2 * u + 1) * 64 + lane) * 16);
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, uint4{x.x, x.y, y.x, y.y});
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, uint4{x.z, x.w, y.z, y.w});
      acc[0] = mfma(sl[u], b0, acc[0]);
      acc[0] = mfma(sh[u], b0, acc[0]);
      acc[1] = mfma(sl[u], b1, acc[1]);
      acc[1] = mfma(sh[u], b1, acc[1]);
    }
    // lane (li, lg) holds the correction of row 16 mt + li, columns 16 w + 4 lg + r
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint2* cell = reinterpret_cast<uint2*>(os + (16 * mt + li) * kCorRow + (16 * w + 4 * lg) * 2);
      const uint2 ov = *cell;
      const float r0 = lo_bf16(ov.x) + acc[mt][0], r1 = hi_bf16(ov.x) + acc[mt][1];
      const float r2 = lo_bf16(ov.y) + acc[mt][2], r3 = hi_bf16(ov.y) + acc[mt][3];
      *cell = uint2{pk_bf16(r0, r1), pk_bf16(r2, r3)};
      if (16 * mt + li < nrows)
        bad += (not_finite(r0) ? 1u : 0u) + (not_finite(r1) ? 1u : 0u) + (not_finite(r2) ? 1u : 0u) + (not_finite(r3) ? 1u : 0u);
    }
    __syncthreads();
    if (orow < nrows) *reinterpret_cast<uint4*>(obase + (st * STEP + orow) * D + ocol) =
                          *reinterpret_cast<const uint4*>(os + orow * kCorRow + ocol * 2);
  }
  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
    if (lane == 0 && bad) atomicAdd(&p.stats->n_nonfinite, bad);
  }
}

// ---- seg_out_kernel: segment j from S_start(j), with the outputs
__global__ __launch_bounds__(kSegThreads) void seg_out_kernel(Params p, int64_t n_steps, SegPlan sg) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t bh = blockIdx.x / sg.P, j = blockIdx.x % sg.P;
  const int64_t s0 = j * sg.L;
  const int64_t ns = (n_steps - s0 < sg.L) ? n_steps - s0 : sg.L;
  const int64_t T = p.T;
  const int d0 = 16 * wave;
  const unsigned char* recs = (const unsigned char*)p.workspace + (bh * n_steps + s0) * (int64_t)kRecBytes;
  const uint16_t* v = (const uint16_t*)p.v + bh * T * D;
  constexpr int kPer = kOutChunks / kSegWaves;
  auto issue = [&](int64_t i) {
    unsigned char* slot = ring + (i % kRingSlots) * kOutSlot;
    const unsigned char* src = recs + i * (int64_t)kRecBytes;
#pragma unroll
    for (int x = 0; x < (kOutChunks + kSegWaves - 1) / kSegWaves; ++x) {
      const int c = wave + kSegWaves * x;
      if (c < kRecBytes / 1024) lds_load16(src + c * 1024 + lane * 16, slot + c * 1024);
      else if (c < kOutChunks) load_v_chunk(v, T, s0 + i, c - kRecBytes / 1024, lane, slot + c * 1024);
    }
  };
  for (int64_t i = 0; i < kRingSlots - 1 && i < ns; ++i) issue(i);

  const floatx4 zero = {0, 0, 0, 0};
  floatx4 S[8];
  if (sg.P > 1) {   // every entering state, segment 0's (a copy of S0) included, from the chaining pass
    load_slice(S, (const float*)((const unsigned char*)p.workspace + sg.off_s) +
                      (bh * sg.P + j) * (int64_t)(kSegState / 4) + wave * 8 * 64 * 4, lane);
  } else if (p.S0) {
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
  for (int u = 0; u < 4; ++u) sb[u] = pack2(S[2 * u], S[2 * u + 1]);

  uint16_t* o = (uint16_t*)p.o + bh * T * D + li * D + d0 + 4 * lg;
  uint32_t nonfinite = 0, n_valid = 0, n_flagged = 0;
  float min_span = __int_as_float(0x7f800000);
  for (int64_t i = 0; i < ns; ++i) {
    const int64_t issued = (i + kRingSlots - 2 < ns - 1) ? i + kRingSlots - 2 : ns - 1;
    wait_steps<kPer>(issued - i);
    block_barrier();
    if (i + kRingSlots - 1 < ns) issue(i + kRingSlots - 1);
    const unsigned char* slot = ring + (i % kRingSlots) * kOutSlot;
    const int64_t st = s0 + i;
    const int nrows = rows_of(T, st);
    const bf16x8 vb = v_operand(slot + kRecBytes, lg, d0 + li, nrows);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const floatx4 eg = *reinterpret_cast<const floatx4*>(slot + kOffEg + (lg * 32 + 4 * t) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) S[t][r] *= eg[r];
    }
    floatx4 U[2], O[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      U[mt] = mfma(ld8((const __bf16*)(slot + kOffTb + (mt * 64 + lane) * 16)), vb, zero);
      // O^T = V^T Phat^T + S^T Qhat^T: operand roles swapped so each lane holds four consecutive
      // columns of one output row (one 8-byte store per row tile)
      O[mt] = mfma(vb, ld8((const __bf16*)(slot + kOffPh + (mt * 64 + lane) * 16)), zero);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        U[mt] = mfma(ld8((const __bf16*)(slot + kOffWn + ((mt * 4 + u) * 64 + lane) * 16)), sb[u], U[mt]);
        O[mt] = mfma(sb[u], ld8((const __bf16*)(slot + kOffQh + ((mt * 4 + u) * 64 + lane) * 16)), O[mt]);
      }
    const bf16x8 ub = pack2(U[0], U[1]);
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = mfma(ld8((const __bf16*)(slot + kOffKt + (t * 64 + lane) * 16)), ub, S[t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) sb[u] = pack2(S[2 * u], S[2 * u + 1]);
    if (wave == 0) {
      const StepMeta meta = *reinterpret_cast<const StepMeta*>(slot + kOffMeta);
      n_valid += meta.n_valid;
      n_flagged += meta.n_flagged;
      min_span = fminf(min_span, fminf(meta.span[0], meta.span[1]));
    }
    uint16_t* os = o + st * STEP * D;
    uint32_t mx = 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      if (nrows == STEP || 16 * mt + li < nrows) {
        *reinterpret_cast<uint2*>(os + (16 * mt) * D) = uint2{pk_bf16(O[mt][0], O[mt][1]), pk_bf16(O[mt][2], O[mt][3])};
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = max(mx, abs_bits(O[mt][r]));
      }
    }
    if (mx >= 0x7f800000u) {   // rare: count exactly
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          nonfinite += ((nrows == STEP || 16 * mt + li < nrows) && abs_bits(O[mt][r]) >= 0x7f800000u) ? 1u : 0u;
    }
  }
  if (j == sg.P - 1) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p.S_final[(bh * D + 16 * t + 4 * lg + r) * D + d0 + li] = S[t][r];
        nonfinite += not_finite(S[t][r]) ? 1u : 0u;
      }
  }
  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nonfinite += __shfl_xor(nonfinite, off);
    if (lane == 0) {
      if (nonfinite) atomicAdd(&p.stats->n_nonfinite, nonfinite);
      if (wave == 0) {
        atomicAdd(&p.stats->n_chunks, n_valid);
        if (n_flagged) atomicAdd(&p.stats->n_flagged, n_flagged);
        if (n_valid) atomic_min_float(&p.stats->min_span, min_span);
      }
    }
  }
}

int64_t n_steps_of(int64_t T) { return (T + STEP - 1) / STEP; }

// Segment plan.  Automatic: about 256 workgroups (one per compute unit) per pass over (b, h, segment),
// at least 8 steps per segment and at most kMaxSeg segments.  The fused path's passes hold P - 1
// workgroups per head (segment 0 runs with outputs beside the maps of segments 1 .. P-2, then
// segments 1 .. P-1 run with outputs), so it takes one segment more, when that leaves at least three;
// the records path's output pass holds all P.  seg_steps > 0 fixes the segment length.  With
// `records`, the per-step records precede the segment blocks in the workspace.
// Segment 0 runs beside the other segments in the same pass but takes a different body: its own outputs
// next to their maps (fused plan: a step with outputs takes about 100/93 of a map step, so segment 0 is
// shorter), or its exact outputs next to their outputs from a zero entering state and their maps
// (corrected plan: segment 0 does less per step, so it is longer).  Percent of the other segments' length.
constexpr int64_t kSeg0PctFused = 93, kSeg0PctCorr = 110;

SegPlan make_plan(int64_t BH, int64_t T, int64_t seg_steps, int mode) {
  const bool records = mode == kModeRecords, corr = mode == kModeCorr;
  const int64_t n = n_steps_of(T);
  SegPlan sg{};
  if (n <= 0) {   // an empty sequence: one empty segment, nothing kept
    sg.P = 1;
    return sg;
  }
  int64_t P;
  if (seg_steps > 0) {
    sg.L = seg_steps;
    P = (n + seg_steps - 1) / seg_steps;
  } else {
    P = 256 / BH;
    if (mode == kModeFused) P = P >= 2 ? P + 1 : 1;
    const int64_t by_len = n / 8;
    P = P < by_len ? P : by_len;
    P = P < kMaxSeg ? P : kMaxSeg;
    P = P < 1 ? 1 : P;
    sg.L = (n + P - 1) / P;
    P = (n + sg.L - 1) / sg.L;
  }
  sg.L0 = sg.L;
  if (!records && seg_steps == 0 && P >= 2) {
    // segment 0 of length r L (r = pct / 100) beside P - 1 segments of length L, covering the sequence
    const int64_t pct = corr ? kSeg0PctCorr : kSeg0PctFused;
    const int64_t L = (100 * n + 100 * (P - 1) + pct - 1) / (100 * (P - 1) + pct);
    int64_t L0 = pct * L / 100;
    if (L0 < 1) L0 = 1;
    if (L0 > n) L0 = n;
    if (L0 + (P - 1) * L < n) L0 = n - (P - 1) * L;
    sg.L = L;
    sg.L0 = L0;
    P = n > L0 ? 1 + (n - L0 + L - 1) / L : 1;
    if (P == 1) sg.L = sg.L0 = n;
  }
  sg.P = P;
  const int64_t recs = records ? BH * n * (int64_t)kRecBytes : 0;
  const int64_t blk = BH * P * (int64_t)kSegState;
  sg.off_x = recs;
  sg.off_m = recs + blk;
  sg.off_s = recs + 2 * blk;
  sg.off_q = corr ? recs + 3 * blk : 0;
  return sg;
}

}  // namespace

hipError_t launch_correct(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg) {
  if (sg.P < 2) return hipSuccess;   // one segment: its outputs are exact
  if (sg.off_q == 0) return hipErrorInvalidValue;
  const int64_t cps = (sg.L + kCorSteps - 1) / kCorSteps;   // workgroups per segment
  const int64_t grid = p.B * p.H * (sg.P - 1) * cps;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(correct_kernel, dim3((unsigned)grid), dim3(kCorThreads), 0, s, p, n_steps, sg, cps);
  return hipGetLastError();
}

size_t mfma_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int mode, int64_t seg_steps) {
  if (dk != D || dv != D || T <= 0) return 0;
  const SegPlan sg = make_plan(B * H, T, seg_steps, mode);
  if (mode != kModeRecords && sg.P == 1) return 0;   // a one-segment fused plan keeps nothing between kernels
  if (mode == kModeCorr) return (size_t)(sg.off_q + B * H * n_steps_of(T) * (int64_t)kQtStep);
  return (size_t)(sg.off_s + B * H * sg.P * (int64_t)kSegState);
}

bool plan_fits(int64_t BH, int64_t T, int64_t seg_steps, int mode) {
  const SegPlan sg = make_plan(BH, T, seg_steps, mode);
  return (sg.L > sg.L0 ? sg.L : sg.L0) < kMaxSegSteps;
}

bool mfma_seg_steps_ok(int64_t T, int64_t seg_steps) {
  if (seg_steps < 0) return false;
  if (seg_steps == 0) return true;
  const int64_t n = n_steps_of(T);
  return (n + seg_steps - 1) / seg_steps <= kMaxSeg;
}

hipError_t launch_mfma(const Params& p, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end, int mode) {
  const int64_t n_steps = n_steps_of(p.T);
  const int64_t BH = p.B * p.H;
  if (mode != kModeRecords && !(fused_supported(p.dtype, p.dk, p.dv, p.T) && plan_fits(BH, p.T, p.seg_steps, mode)))
    mode = kModeRecords;
  const bool fused = mode == kModeFused;
  const SegPlan sg = make_plan(BH, p.T, p.seg_steps, mode);
  if (mode == kModeCorr) {
    // statistics reset first: every pass adds its counts with atomics
    hipError_t e;
    if (p.stats && (e = launch_stats_init(p.stats, s)) != hipSuccess) return e;
    if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
    if ((e = launch_fused_corr(p, s, n_steps, sg)) != hipSuccess) return e;
    if (sg.P > 1) {
      hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(BH * 8)), dim3(256), 0, s, p, sg, 1, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = launch_correct(p, s, n_steps, sg)) != hipSuccess) return e;
    }
    if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  // statistics reset: by the chaining pass of the fused path when there is one, else its own launch
  if (p.stats && !(fused && sg.P > 1)) {
    const hipError_t e = launch_stats_init(p.stats, s);
    if (e != hipSuccess) return e;
  }
  if (fused) {
    hipError_t e;
    if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
    if (sg.P > 1) {
      if ((e = launch_fused_segments(p, s, n_steps, sg, false)) != hipSuccess) return e;
      hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(BH * 8)), dim3(256), 0, s, p, sg, 1, 0);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_fused_segments(p, s, n_steps, sg, true)) != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(PrepShared));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)seg_state_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStSmem);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)seg_out_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kOutSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(BH * n_steps)), dim3(256), sizeof(PrepShared), s, p, n_steps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sg.P > 1) {
    hipLaunchKernelGGL(seg_state_kernel, dim3((unsigned)(BH * (sg.P - 1))), dim3(kSegThreads), kStSmem, s, p,
                       n_steps, sg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(BH * 8)), dim3(256), 0, s, p, sg, 0, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(seg_out_kernel, dim3((unsigned)(BH * sg.P)), dim3(kSegThreads), kOutSmem, s, p, n_steps, sg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace kda

// Fused matrix-core path of the chunked KDA forward (bf16 inputs, dk = dv = 128, bf16 MFMA on gfx950).
//
// The steps (32 tokens = two 16-token chunks) of every (b, h) sequence are cut into segments; one
// workgroup of 16 wavefronts owns one segment and builds every step's operands on chip, so only the
// inputs q, k, v, w, beta and the outputs o cross HBM.  Wavefronts 0-7 (C) each carry a 16-column
// slice of the state; wavefronts 8-15 (E) build the operands, four per chunk.  Per segment the steps
// run through a software pipeline.  Interval s has two halves, each closed by a workgroup barrier:
//   first half    C(s)      R = diag(beta)(V - Kbar S), U = T R, the outputs and the state update of step s
//                 TL(s+1)   the causal tiles of step s+1 on MFMA (wavefronts 0-5): the diagonal blocks of
//                           A go to the solver, -A_10 and P straight into their operand places
//                 E1(s+2)   gates, chunk-local inclusive prefix L, chunk totals Gam_c, spans, beta, e^{L}
//   second half   E2(s+2)   every operand of step s+2 built from k, q and the gate factors, the flags,
//                           and the per-pair diagonal blocks of flagged chunks (whole workgroup)
//                 S(s+1)    the diagonal blocks of T = (I + A)^{-1} of step s+1 (wavefront 7)
//
// Per step, with G the in-step prefix referenced to the step start, Kbar = k e^{G}, Qbar = q e^{G},
// Ktil = k e^{Gam_step - G}, A = strictly-lower diag(beta) Kbar (k e^{-G})^T, P = lower-inclusive
// Qbar (k e^{-G})^T and T = (I + A)^{-1}, the state S (dk x dv, fp32) advances as
//   R = diag(beta) (V - Kbar S)        U = T R
//   O = Qbar S + P U                   S <- diag(e^{Gam_step}) S + Ktil^T U
// which is the chunk form of the delta rule written out from "From Numerical Stability to Load
// Balancing ..." section 2.1 (matrix products inside a chunk, a serial state between chunks, in-chunk
// scaling exp(G_i - G_j) for i >= j) with the UT/WY correction of the delta rule.  U is formed by
// 16-row blocks, U_0 = T_00 R_0 and U_1 = T_11 (R_1 - A_10 U_0), so only the diagonal blocks of T are
// inverted.  The bounded gate
// (same page section 2.2; "Demystifying Trillion-Parameter MoE Models ..." Breakthrough 1 part 2)
// keeps each 16-token chunk's span at or above -80, so the reciprocal factors e^{-L} stay below e^80.
// Only the two diagonal 16 x 16 blocks use e^{+-L} (chunk-local); the block coupling chunk 1 to
// chunk 0 uses factors referenced to the chunk boundary, e^{L_r} e^{Gam_0 - L_j}, both <= 1.  A
// chunk whose span falls below -80 gets its diagonal blocks from per-pair factors exp(L_r - L_j) <= 1.
//
// Two workgroup kinds share the pipeline:
//   output   a segment from its true entering state, with the outputs o (and S_final at the end)
//   map      a segment's affine map S_end = M S_start + X: wavefront w carries column slice w
//            of X (from zero, with V) and of M (from the identity, without V)
// The map pass (kernel argument OUT = false) runs segment 0 as an output segment, from S0, beside
// the maps of segments 1 .. P-2; after the chaining, the output pass (OUT = true) runs segments
// 1 .. P-1.  Both passes hold P - 1 workgroups per head.
//
// The corrected plan has one pass over the sequence instead of two.  The outputs of a segment are
// affine in its entering state: with S_t = X_t + M_t S_start the state entering step t,
//   O_t = [Qbar X_t + P T diag(beta)(V - Kbar X_t)] + [Qbar M_t - P T diag(beta) Kbar M_t] S_start
//       = O_t(from zero) + Qtil_t S_start.
// Its pass runs segment 0 exactly, from S0, beside segments 1 .. P-1, each of which writes its
// outputs from a zero entering state (the C wavefronts run the output body from S = 0) and carries
// the eight 16-column slices of M_t on the wavefronts with idle time in one of the halves (the
// chunk-0 E wavefronts and state wavefronts 6-7 in the first, state wavefronts 4-5 in the second):
// they write Qtil_t (32 x 128, bf16) and, at the end, M, next to the C wavefronts' X.  After the
// chaining of the maps, a memory-bound pass adds Qtil_t S_start to the outputs of segments 1 .. P-1.
#include "kda_mfma_util.h"

namespace kda {

namespace {

constexpr int D = 128;
constexpr int STEP = 32;
constexpr int kCWaves = 8;                    // wavefronts 0-7: state slices, tiles, solve
static_assert(kCWaves == kRecChunks - kRecNonfinite, "one non-finite count per state wavefront in the record");
constexpr int kEWaves = 8;                    // wavefronts 8-15: the E stage
constexpr int kThreads = 64 * (kCWaves + kEWaves);
// gate kinds (kernel template argument): bounded with 16 g_min >= -80 (no chunk can need the flagged
// forms), bounded past that or with the fallback forced, and the unbounded gate
constexpr int kGatePlain = 0, kGateFlagged = 1, kGateUnbounded = 2;

// ---- operand blocks: one MFMA operand (64 lanes x 16 B), with a 16-byte pad after every 16 lanes,
// so that the 4-byte writes of the E stage (16 lanes 256 B apart) land in distinct LDS banks, while a
// 16-byte-per-lane read stays contiguous within each group of 16 lanes
constexpr int kBlk = 68 * 16;                                           // bytes of one block
__device__ __forceinline__ int slot16(int lane) { return (lane + (lane >> 4)) * 16; }

// ---- per-step operand record (LDS), arranged so that every MFMA operand is one 16-byte read per lane
constexpr int rKb = 0;                // -beta Kbar, [mt 2][u 4] blocks: row 16mt + li, channels 32u + {4g+r, 16+4g+r}
constexpr int rQb = rKb + 8 * kBlk;   // Qbar, same arrangement                                    (OUT only)
constexpr int rKt = rQb + 8 * kBlk;   // Ktil^T, [t 8] blocks: channel 16t + li, tokens {4g+r, 16+4g+r}
constexpr int rT = rKt + 8 * kBlk;    // T_00, T_11, -A_10: three K = 16 A operands (64 lanes x 4 bf16):
                                      // lane (li, g) holds row li, columns 4g .. 4g+3 of the block
constexpr int rP = rT + 2 * kBlk;     // P, [mt 2] blocks: row 16mt + li, tokens {4g+r, 16+4g+r}  (OUT only)
constexpr int rEg = rP + 2 * kBlk;    // e^{Gam_step}: [g 4][t 8][r 4] fp32 <-> channel 16t + 4g + r
constexpr int rBeta = rEg + 512;      // beta per token, fp32 (zero past the end of the sequence)
constexpr int rMeta = rBeta + 128;    // StepInfo
constexpr int kRec = rMeta + 32;
constexpr int kRecSlots = 3;          // steps s (C), s+1 (S), s+2 (E, TL)
static_assert(kRec % 16 == 0, "record slots stay 16-byte aligned");

// ---- tile operands of one step, same per-lane arrangement as rKb ([rt][u] blocks)
constexpr int oKh = 0;                // k e^{-L}, chunks 0 and 1 [cc 2][u 4]
constexpr int oKb1 = oKh + 8 * kBlk;  // k e^{L}, chunk 1
constexpr int oQb1 = oKb1 + 4 * kBlk; // q e^{L}, chunk 1                                          (OUT only)
constexpr int oKt0 = oQb1 + 4 * kBlk; // k e^{Gam_0 - L}, chunk 0
constexpr int kOps = oKt0 + 4 * kBlk;
// the per-pair path of a flagged chunk borrows the tile-operand buffer of step s+1 (free during the
// second half of interval s): L (fp32 [16][128]), raw k and raw q (bf16 [16][128]), rows padded so
// that the rows one pass of 16 lanes reads start 16 banks apart
constexpr int kPL = 144;    // floats per L row (128 + 16)
constexpr int kPK = 160;    // bf16 per k or q row (128 + 32)
constexpr int pL = 0, pK = 16 * kPL * 4, pQ = pK + 16 * kPK * 2;
static_assert(pQ + 16 * kPK * 2 <= kOps, "per-pair inputs fit the borrowed buffer");
static_assert(pK % 16 == 0 && pQ % 16 == 0 && kOps % 16 == 0, "16-byte reads of the per-pair inputs");

// the midpoint-referenced rows of flagged chunks (k e^{L - L_7}, q e^{L - L_7}) also go to the other
// tile-operand buffer, same arrangement as rKb, written with the step's operands and read by its tiles
constexpr int mK0 = 0, mQ0 = 4 * kBlk, mK1 = 8 * kBlk, mQ1 = 12 * kBlk;
static_assert(mQ1 + 4 * kBlk <= kOps, "the midpoint rows fit the borrowed buffer");
constexpr int kOpT00 = 0, kOpT11 = 512, kOpA10 = 1024;   // byte offsets of the three blocks within rT
static_assert(kOpA10 + 512 <= 2 * kBlk, "the T operands fit their region");
constexpr int kORow = D * 2 + 16;   // bytes per staged output row (256 of data, 16 of pad)
constexpr int kRowA = 20;     // row stride (floats) of the fp32 diagonal blocks: 16-byte aligned rows

struct StepInfo {
  float span[2];          // chunk spans, natural-log units (+inf for a chunk with no tokens)
  uint32_t n_valid;       // chunks with at least one token
  uint32_t n_flagged;     // of those, spans below -80
  uint32_t pairwise;      // bit c: chunk c's diagonal blocks come from per-pair factors
  uint32_t midpoint;      // bit c: chunk c's diagonal blocks come from the midpoint-referenced tiles
};

struct FusedShared {
  unsigned char rec[kRecSlots][kRec];
  unsigned char ops[2][kOps];
  float A[2][STEP][kRowA];                // diagonal blocks of A (rows 0-15: A_00, 16-31: A_11), by step parity
  float pwA[2][16][16], pwP[2][16][16];   // per-pair diagonal blocks [chunk][r][j]
  float gam[2][D];                        // chunk totals (log2 units) of the step in E
  float spanw[kEWaves];                   // per-E-wave minimum of the chunk totals
  uint32_t halfw[kEWaves];                // per E wave: 1 if one of its channels has a half-chunk span below -80
  // bf16 rows of the step in C, padded to 272 bytes so that column-slice accesses spread over the
  // banks.  First half: each C wavefront reads V and then writes o, both in its own 16 columns.
  // Second half: wavefronts 0-3 store eight rows of o each as whole rows, then fill the same rows
  // with V of the next step (loaded as whole rows at the end of the first half).
  alignas(16) unsigned char ostage[STEP][kORow];
};
constexpr size_t kFusedSmem = sizeof(FusedShared);
static_assert(kFusedSmem <= 163840, "LDS budget");

// Phase stamps (the phase-stamp build only, libkda_stamps.so; a no-op otherwise): lane 0 of wavefront w
// of the chosen workgroup records the shader clock at phase boundary k of interval `it` (the interval
// whose E stage handles step it, counted from the segment's first).
// The product build compiles the calls away entirely (KDA_STAMP expands to nothing), so its code is
// the same as without them.
#if KDA_PHASE_STAMPS
__device__ __forceinline__ void stamp(const Params& p, int w, int it, int k) {
  if ((int)blockIdx.x != p.stamp_block || it < 0 || it >= kStampSteps || (threadIdx.x & 63) != 0) return;
  unsigned long long* pr = (unsigned long long*)((unsigned char*)p.workspace + p.stamp_off);
  pr[(w * kStampSteps + it) * kStampK + k] = __builtin_amdgcn_s_memtime();
}
#define KDA_STAMP(p, w, it, k) stamp(p, w, it, k)
#else
#define KDA_STAMP(p, w, it, k) ((void)0)
#endif

// x, hidden from the optimizer: values derived from it inside a loop are recomputed there instead of
// being hoisted out of the loop and held in registers for its whole length
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// DPP moves within a wave (no LDS round trip): quad_perm selects within groups of four lanes;
// row_shr shifts within rows of 16 lanes (lanes without a source keep `old`); row_bcast:15 / :31
// carry lane 15 of each row, lane 31, into the following rows
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROW_MASK, 0xF, false));
}

// Lane n of this lane's row of 16 (DPP row_newbcast:n), n a constant after unrolling.  Folded into the
// instruction that uses it, the broadcast costs no instruction of its own.
__device__ __forceinline__ float row_bcast(float v, int n) {
  switch (n) {
#define KDA_ROW_BCAST_CASE(N) \
  case N: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
    KDA_ROW_BCAST_CASE(0) KDA_ROW_BCAST_CASE(1) KDA_ROW_BCAST_CASE(2) KDA_ROW_BCAST_CASE(3)
    KDA_ROW_BCAST_CASE(4) KDA_ROW_BCAST_CASE(5) KDA_ROW_BCAST_CASE(6) KDA_ROW_BCAST_CASE(7)
    KDA_ROW_BCAST_CASE(8) KDA_ROW_BCAST_CASE(9) KDA_ROW_BCAST_CASE(10) KDA_ROW_BCAST_CASE(11)
    KDA_ROW_BCAST_CASE(12) KDA_ROW_BCAST_CASE(13) KDA_ROW_BCAST_CASE(14)
#undef KDA_ROW_BCAST_CASE
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + 15, 0xF, 0xF, false));
  }
}

// gate in log2 units (g * log2 e), with the kind of gate fixed at compile time
template <bool UNB> __device__ __forceinline__ float gate2(float w, float g_min_log2);
template <> __device__ __forceinline__ float gate2<false>(float w, float g_min_log2) {
  return g_min_log2 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-w * kLog2e));
}
// -softplus(w) in log2 units, -(max(w, 0) log2 e + log2(1 + 2^{-|w| log2 e})), on the hardware exp2 and
// log2: the absolute error (about 2e-7, where 1 + 2^{-|w| log2 e} rounds) is far below what the bf16
// operands built from the prefix carry
template <> __device__ __forceinline__ float gate2<true>(float w, float) {
  return -(fmaxf(w, 0.f) * kLog2e + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(w) * kLog2e)));
}

// Raw buffer views of one segment of one (b, h) slice of a tensor, from the segment's first token to
// its last (or to the end of the sequence): loads past the end of a view return zero, so tokens past
// the end of the sequence read as k = q = v = beta = 0 (their gates are masked in E).  A view's byte
// count and the offsets inside it are 32-bit: a segment holds fewer than 2^18 steps (2 GiB of one
// tensor), whatever the length of the sequence.
struct Views {
  __amdgpu_buffer_rsrc_t k, w, q, beta, v;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t view(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- stage E
// Thread layout: wave w, lane l -> chunk cc = w >> 2, channel pair pr = 16 (w & 3) + (l >> 2)
// (channels 2pr, 2pr+1), token quarter h = l & 3 (tokens 16cc + 4h + j, j < 4).  The in-chunk prefix
// runs over j in registers and over h across the four consecutive lanes of the quarter group.
struct EIn {
  uint32_t q[4], k[4], w[4];   // two bf16 channels per word, tokens j
  uint32_t b[4];               // beta of the 4 tokens (bf16 in the low half)
};

struct EKeep {                 // E's values carried from its first half to its second
  uint32_t k[4], q[4];         // two bf16 channels per word, tokens j
  float L0[4], L1[4];          // chunk-local inclusive prefix (log2 units)
  float beta[4];
  float G0, G1;                // chunk totals of the two channels (log2 units)
};

template <bool OUT>
__device__ __forceinline__ void e_load(EIn& in, const Views& vw, int step, int voff, int boff) {
  const int so = step * (STEP * D * 2), sb = step * (STEP * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    in.k[j] = __builtin_amdgcn_raw_buffer_load_b32(vw.k, voff + j * D * 2, so, 0);
    in.w[j] = __builtin_amdgcn_raw_buffer_load_b32(vw.w, voff + j * D * 2, so, 0);
    in.q[j] = OUT ? __builtin_amdgcn_raw_buffer_load_b32(vw.q, voff + j * D * 2, so, 0) : 0u;
    in.b[j] = __builtin_amdgcn_raw_buffer_load_b16(vw.beta, boff + j * 2, sb, 0);
  }
}

// offset of (row li of row tile rt, this thread's channel pair) in a [rt][u] block array
__device__ __forceinline__ int rowk_off(int rt, int u, int li, int g, int pos) {
  return (rt * 4 + u) * kBlk + (li + 17 * g) * 16 + pos * 2;
}
// offset of (channel c, token quarter h, chunk cc) in the Ktil^T blocks
__device__ __forceinline__ int kt_off(int c, int h, int cc) { return (c >> 4) * kBlk + ((c & 15) + 17 * h) * 16 + cc * 8; }

// Minimum of the chunk totals over the wave, valid in lane 63.  Gates are never positive, so on the
// float bits an unsigned maximum is the minimum; the four lanes of a quarter group hold the same
// totals, so the reduction runs over the quarter groups only.
__device__ __forceinline__ float wave_min_totals(float g0, float g1) {
  uint32_t m = max(__float_as_uint(g0), __float_as_uint(g1));
  // lanes without a source, and rows outside the row mask, read 0: the identity of an unsigned maximum
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, true));   // row_shr:4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, true));   // row_shr:8
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x142, 0xA, 0xF, true));   // row_bcast:15
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x143, 0xC, 0xF, true));   // row_bcast:31
  return __uint_as_float(m);
}

// First half of E for chunk CC of the step: gates, the in-chunk prefix L, the chunk totals, the span
// of the wave's channels, and beta.
template <bool UNB, int CC, bool FLG>
__device__ __forceinline__ void e_first(FusedShared& sm, const EIn& in, EKeep& kp, const Params& p, int step,
                                        unsigned char* rec, int w, int l) {
  const int pr = 16 * (w & 3) + (l >> 2), h = l & 3;
  const int c0 = 2 * pr, c1 = 2 * pr + 1;
  // a step that lies wholly inside the sequence (every step but a ragged last one) needs no mask:
  // the test is uniform, so the common case runs without per-token selects
  const bool full = (step + 1) * STEP <= (int)p.T;
  const int nv = full ? 4 : min(max((int)p.T - (step * STEP + 16 * CC + 4 * h), 0), 4);   // this lane's tokens in the sequence
  const float gml2 = p.g_min * kLog2e;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kp.k[j] = in.k[j];
    kp.q[j] = in.q[j];
    kp.beta[j] = __uint_as_float(in.b[j] << 16);
    const float g0 = gate2<UNB>(lo_bf16(in.w[j]), gml2), g1 = gate2<UNB>(hi_bf16(in.w[j]), gml2);
    if (full) {
      a0 += g0;
      a1 += g1;
    } else {
      a0 += j < nv ? g0 : 0.f;
      a1 += j < nv ? g1 : 0.f;
    }
    kp.L0[j] = a0;
    kp.L1[j] = a1;
  }
  // prefix across the quarter group (lanes 4m .. 4m+3) with quad permutes
  float s0 = a0, s1 = a1;
  {
    const float t0 = dpp<0x90>(0.f, s0), t1 = dpp<0x90>(0.f, s1);   // quad_perm [0,0,1,2]: lane h <- h-1
    if (h >= 1) { s0 += t0; s1 += t1; }
    const float u0 = dpp<0x40>(0.f, s0), u1 = dpp<0x40>(0.f, s1);   // quad_perm [0,0,0,1]: lane h <- h-2
    if (h >= 2) { s0 += u0; s1 += u1; }
  }
  const float x0 = s0 - a0, x1 = s1 - a1;              // exclusive prefix
  kp.G0 = dpp<0xFF>(0.f, s0);                          // quad_perm [3,3,3,3]: the chunk totals
  kp.G1 = dpp<0xFF>(0.f, s1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kp.L0[j] += x0;
    kp.L1[j] += x1;
  }
  if (h == 0) { sm.gam[CC][c0] = kp.G0; sm.gam[CC][c1] = kp.G1; }
  const float m = wave_min_totals(kp.G0, kp.G1);
  if (l == 63) sm.spanw[w] = m;
  // the prefix at token 7 (lane h = 1, j = 3 of the quarter group) and the spans of the two 8-token
  // halves, L_7 and Gam - L_7: whether any of the wave's channels has a half below -80 decides between
  // the midpoint-referenced tiles and the per-pair blocks for a flagged chunk
  if (FLG) {
    const float H0 = dpp<0x55>(0.f, kp.L0[3]), H1 = dpp<0x55>(0.f, kp.L1[3]);   // quad_perm [1,1,1,1]
    const float lim = kSpanLimit * kLog2e;
    const bool bad = fminf(fminf(H0, kp.G0 - H0), fminf(H1, kp.G1 - H1)) < lim;
    const uint32_t anybad = __builtin_amdgcn_readfirstlane(__ballot(bad) != 0ull ? 1u : 0u);
    if (l == 0) sm.halfw[w] = anybad;
  }
  if ((w & 3) == 0 && (l >> 2) == 0) {
    float* bt = reinterpret_cast<float*>(rec + rBeta);
#pragma unroll
    for (int j = 0; j < 4; ++j) bt[16 * CC + 4 * h + j] = kp.beta[j];
  }
}

__device__ __forceinline__ void pair_of(int pr, int& r, int& j) {   // pr -> (r, j), j <= r < 16
  r = 0;
  while ((r + 1) * (r + 2) / 2 <= pr) ++r;
  j = pr - r * (r + 1) / 2;
}

// How the diagonal blocks of the step in E are formed.  A chunk whose span falls below -80 (or every
// chunk, when the fallback is forced) cannot take the chunk-start-referenced tiles, whose factor
// e^{-L} would pass e^{80}.  When both of its 8-token halves span at least -80 it takes the same tiles
// referenced to its token 7 instead: rows k e^{L - L_7} and q e^{L - L_7}, columns k e^{L_7 - L}, every
// factor at most e^{80} (rows of the first half and columns of the second are the ones above 1), and
// every kept product e^{L_r - L_j} exact.  Otherwise it takes the per-pair blocks.  The midpoint rows
// live in the other tile-operand buffer, which the per-pair blocks also borrow, so a step with any
// per-pair chunk takes the per-pair blocks for every chunk that needs more than the plain tiles.
// force_fallback = 2 forces the per-pair blocks on every chunk.  Every thread of the workgroup reads
// the same shared values, so the answer (and every branch on it) is uniform.
struct Modes {
  uint32_t pw, mid;   // bit c: chunk c takes the per-pair blocks / the midpoint-referenced tiles
};
__device__ __forceinline__ Modes step_modes(const FusedShared& sm, const Params& p, int step) {
  const int t0 = step * STEP;
  const bool valid0 = t0 < (int)p.T, valid1 = t0 + 16 < (int)p.T;
  const float span0 = fminf(fminf(sm.spanw[0], sm.spanw[1]), fminf(sm.spanw[2], sm.spanw[3])) * kLn2;
  const float span1 = fminf(fminf(sm.spanw[4], sm.spanw[5]), fminf(sm.spanw[6], sm.spanw[7])) * kLn2;
  const bool x0 = p.force_fallback || (valid0 && span0 < kSpanLimit && !p.disable_fallback);
  const bool x1 = p.force_fallback || (valid1 && span1 < kSpanLimit && !p.disable_fallback);
  const uint32_t x = (x0 ? 1u : 0u) | (x1 ? 2u : 0u);
  if (__builtin_expect(x == 0u, 1)) return Modes{0u, 0u};
  const bool bad0 = (sm.halfw[0] | sm.halfw[1] | sm.halfw[2] | sm.halfw[3]) != 0u;
  const bool bad1 = (sm.halfw[4] | sm.halfw[5] | sm.halfw[6] | sm.halfw[7]) != 0u;
  const bool pair = p.force_fallback == 2 || (x0 && bad0) || (x1 && bad1);
  return Modes{pair ? x : 0u, pair ? 0u : x};
}

// Second half of E for chunk CC: e^{L}, and every operand of the step built from k, q and the gate
// factors (the exponentials sit here rather than in the first half, which the state wavefronts bound).
//   chunk 0: k e^{-L} (tiles), -beta k e^{L} and q e^{L} (step-referenced = chunk-local), k e^{Gam_0 - L}
//            (tiles), Ktil = k e^{Gam_0 - L} e^{Gam_1}, and e^{Gam_step}
//   chunk 1: k e^{-L} (tiles), k e^{L} and q e^{L} (tiles), their step-referenced forms times e^{Gam_0}
//            (with -beta for k), Ktil = k e^{Gam_1 - L}
// e^{-L} = e^{Gam - L} e^{-Gam}: finite wherever the dense tile is used (a chunk whose e^{-Gam}
// overflows has a span below -80 and takes the per-pair blocks instead).
template <bool OUT, int CC, bool MID>
__device__ __forceinline__ void e_second(FusedShared& sm, const EKeep& kp, const Params& p, int step,
                                         unsigned char* rec, unsigned char* ops, unsigned char* opsM, Modes md,
                                         int w, int l) {
  const int pr = 16 * (w & 3) + (l >> 2), h = l & 3;
  const int u = w & 3, g = ((l >> 2) & 7) >> 1, pos = (l >> 5) * 4 + 2 * ((l >> 2) & 1);
  const int c0 = 2 * pr, c1 = 2 * pr + 1;
  const float iG0 = __builtin_amdgcn_exp2f(-kp.G0), iG1 = __builtin_amdgcn_exp2f(-kp.G1);
  // midpoint reference: the prefix at token 7 (lane h = 1, j = 3 of the quarter group)
  const float H0 = MID ? dpp<0x55>(0.f, kp.L0[3]) : 0.f, H1 = MID ? dpp<0x55>(0.f, kp.L1[3]) : 0.f;
  // e^{Gam} of the other chunk, per channel
  const float y0 = __builtin_amdgcn_exp2f(sm.gam[1 - CC][c0]), y1 = __builtin_amdgcn_exp2f(sm.gam[1 - CC][c1]);
  float eL0[4], eL1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    eL0[j] = __builtin_amdgcn_exp2f(kp.L0[j]);
    eL1[j] = __builtin_amdgcn_exp2f(kp.L1[j]);
  }
  float ktv0[4], ktv1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int li = 4 * h + j;
    const float k0 = lo_bf16(kp.k[j]), k1 = hi_bf16(kp.k[j]);
    const float kg0 = k0 * __builtin_amdgcn_exp2f(kp.G0 - kp.L0[j]), kg1 = k1 * __builtin_amdgcn_exp2f(kp.G1 - kp.L1[j]);
    const float ke0 = k0 * eL0[j], ke1 = k1 * eL1[j];
    const float nb = -kp.beta[j];
    if (MID) {   // midpoint-referenced tile operands: columns k e^{L_7 - L}, rows k e^{L - L_7}, q e^{L - L_7}
      const float rf0 = __builtin_amdgcn_exp2f(kp.L0[j] - H0), rf1 = __builtin_amdgcn_exp2f(kp.L1[j] - H1);
      const float cf0 = __builtin_amdgcn_exp2f(H0 - kp.L0[j]), cf1 = __builtin_amdgcn_exp2f(H1 - kp.L1[j]);
      *reinterpret_cast<uint32_t*>(ops + oKh + rowk_off(CC, u, li, g, pos)) = pk_bf16(k0 * cf0, k1 * cf1);
      *reinterpret_cast<uint32_t*>(opsM + (CC ? mK1 : mK0) + rowk_off(0, u, li, g, pos)) = pk_bf16(k0 * rf0, k1 * rf1);
      if (OUT)
        *reinterpret_cast<uint32_t*>(opsM + (CC ? mQ1 : mQ0) + rowk_off(0, u, li, g, pos)) =
            pk_bf16(lo_bf16(kp.q[j]) * rf0, hi_bf16(kp.q[j]) * rf1);
    } else {
      *reinterpret_cast<uint32_t*>(ops + oKh + rowk_off(CC, u, li, g, pos)) = pk_bf16(kg0 * iG0, kg1 * iG1);
    }
    if (CC == 0) {
      *reinterpret_cast<uint32_t*>(rec + rKb + rowk_off(0, u, li, g, pos)) = pk_bf16(nb * ke0, nb * ke1);
      if (OUT)
        *reinterpret_cast<uint32_t*>(rec + rQb + rowk_off(0, u, li, g, pos)) =
            pk_bf16(lo_bf16(kp.q[j]) * eL0[j], hi_bf16(kp.q[j]) * eL1[j]);
      *reinterpret_cast<uint32_t*>(ops + oKt0 + rowk_off(0, u, li, g, pos)) = pk_bf16(kg0, kg1);
      ktv0[j] = kg0 * y0;
      ktv1[j] = kg1 * y1;
    } else {
      *reinterpret_cast<uint32_t*>(ops + oKb1 + rowk_off(0, u, li, g, pos)) = pk_bf16(ke0, ke1);
      *reinterpret_cast<uint32_t*>(rec + rKb + rowk_off(1, u, li, g, pos)) = pk_bf16(nb * ke0 * y0, nb * ke1 * y1);
      if (OUT) {
        const float qe0 = lo_bf16(kp.q[j]) * eL0[j], qe1 = hi_bf16(kp.q[j]) * eL1[j];
        *reinterpret_cast<uint32_t*>(ops + oQb1 + rowk_off(0, u, li, g, pos)) = pk_bf16(qe0, qe1);
        *reinterpret_cast<uint32_t*>(rec + rQb + rowk_off(1, u, li, g, pos)) = pk_bf16(qe0 * y0, qe1 * y1);
      }
      ktv0[j] = kg0;
      ktv1[j] = kg1;
    }
  }
  // Ktil^T: channel c -> block c >> 4, lane (c & 15) + 16 h, positions 4 CC .. 4 CC + 3
  *reinterpret_cast<uint2*>(rec + rKt + kt_off(c0, h, CC)) = uint2{pk_bf16(ktv0[0], ktv0[1]), pk_bf16(ktv0[2], ktv0[3])};
  *reinterpret_cast<uint2*>(rec + rKt + kt_off(c1, h, CC)) = uint2{pk_bf16(ktv1[0], ktv1[1]), pk_bf16(ktv1[2], ktv1[3])};
  if (CC == 0) {
    if (h == 0) {
      float* eg = reinterpret_cast<float*>(rec + rEg);
      eg[((c0 >> 2) & 3) * 32 + (c0 >> 4) * 4 + (c0 & 3)] = __builtin_amdgcn_exp2f(kp.G0 + sm.gam[1][c0]);
      eg[((c1 >> 2) & 3) * 32 + (c1 >> 4) * 4 + (c1 & 3)] = __builtin_amdgcn_exp2f(kp.G1 + sm.gam[1][c1]);
    }
    // spans and flags: the step's information record
    if (w == 0 && l == 0) {
      const int t0 = step * STEP;
      const bool valid0 = t0 < (int)p.T, valid1 = t0 + 16 < (int)p.T;
      const float span0 = fminf(fminf(sm.spanw[0], sm.spanw[1]), fminf(sm.spanw[2], sm.spanw[3])) * kLn2;
      const float span1 = fminf(fminf(sm.spanw[4], sm.spanw[5]), fminf(sm.spanw[6], sm.spanw[7])) * kLn2;
      const bool flag0 = valid0 && span0 < kSpanLimit, flag1 = valid1 && span1 < kSpanLimit;
      StepInfo si;
      si.span[0] = valid0 ? span0 : __int_as_float(0x7f800000);
      si.span[1] = valid1 ? span1 : __int_as_float(0x7f800000);
      si.n_valid = (valid0 ? 1u : 0u) + (valid1 ? 1u : 0u);
      si.n_flagged = (flag0 ? 1u : 0u) + (flag1 ? 1u : 0u);
      si.pairwise = md.pw;
      si.midpoint = md.mid;
      *reinterpret_cast<StepInfo*>(rec + rMeta) = si;
    }
  }
}

// Per-pair diagonal blocks of flagged chunks, by the whole workgroup: A_rj = beta_r sum_c k_rc k_jc
// exp(L_rc - L_jc) (j < r), P_rj = sum_c q_rc k_jc exp(L_rc - L_jc) (j <= r), every factor <= 1.  The
// E wavefronts of the chunk first park L, raw k and raw q in `scratch`.
template <bool OUT, bool IS_E>
__device__ __forceinline__ void pairwise_blocks(FusedShared& sm, const EKeep* kp, const unsigned char* rec,
                                                unsigned char* scratch, uint32_t mask, int we, int l, int tid) {
  const int cc = we >> 2, pr = 16 * (we & 3) + (l >> 2), h = l & 3;
  const int c0 = 2 * pr, c1 = 2 * pr + 1;
#pragma unroll 1
  for (int fc = 0; fc < 2; ++fc) {
    if (!(mask & (1u << fc))) continue;
    if (IS_E && cc == fc) {
      float* Ls = reinterpret_cast<float*>(scratch + pL);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * h + j;
        Ls[row * kPL + c0] = kp->L0[j];
        Ls[row * kPL + c1] = kp->L1[j];
        *reinterpret_cast<uint32_t*>(scratch + pK + (row * kPK + c0) * 2) = kp->k[j];
        if (OUT) *reinterpret_cast<uint32_t*>(scratch + pQ + (row * kPK + c0) * 2) = kp->q[j];
      }
    }
    block_barrier();
    const float* Ls = reinterpret_cast<const float*>(scratch + pL);
    const unsigned char* Ks = scratch + pK;
    const unsigned char* Qs = scratch + pQ;
    const float* bt = reinterpret_cast<const float*>(rec + rBeta);
    {   // 136 pairs x 4 channel quarters over the workgroup's threads; all lanes run the shuffles
      const int pi = tid >> 2, cq = tid & 3;
      float a = 0.f, pq = 0.f;
      int r = 0, j = 0;
      if (pi < 136) {
        pair_of(pi, r, j);
        // eight channels at a time, blocks cq, cq + 4, cq + 8, cq + 12 (the four quarter threads of a
        // pair read adjacent pieces): 16-byte reads of L, k and q
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 8 * (cq + 4 * i);
          const float4 lr0 = *reinterpret_cast<const float4*>(Ls + r * kPL + c);
          const float4 lr1 = *reinterpret_cast<const float4*>(Ls + r * kPL + c + 4);
          const float4 lj0 = *reinterpret_cast<const float4*>(Ls + j * kPL + c);
          const float4 lj1 = *reinterpret_cast<const float4*>(Ls + j * kPL + c + 4);
          const uint4 kr = *reinterpret_cast<const uint4*>(Ks + (r * kPK + c) * 2);
          const uint4 kj = *reinterpret_cast<const uint4*>(Ks + (j * kPK + c) * 2);
          const uint4 qr = OUT ? *reinterpret_cast<const uint4*>(Qs + (r * kPK + c) * 2) : uint4{0, 0, 0, 0};
          const float dl[8] = {lr0.x - lj0.x, lr0.y - lj0.y, lr0.z - lj0.z, lr0.w - lj0.w,
                               lr1.x - lj1.x, lr1.y - lj1.y, lr1.z - lj1.z, lr1.w - lj1.w};
          const uint32_t kru[4] = {kr.x, kr.y, kr.z, kr.w}, kju[4] = {kj.x, kj.y, kj.z, kj.w};
          const uint32_t qru[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const uint32_t sh = (m & 1) ? 0u : 16u;   // element 2n in the low half of dword n
            const float kjm = __uint_as_float((kju[m >> 1] << sh) & 0xFFFF0000u) * __builtin_amdgcn_exp2f(dl[m]);
            a += __uint_as_float((kru[m >> 1] << sh) & 0xFFFF0000u) * kjm;
            if (OUT) pq += __uint_as_float((qru[m >> 1] << sh) & 0xFFFF0000u) * kjm;
          }
        }
      }
      a += __shfl_xor(a, 1); a += __shfl_xor(a, 2);
      if (OUT) { pq += __shfl_xor(pq, 1); pq += __shfl_xor(pq, 2); }
      if (pi < 136 && cq == 0) {
        sm.pwA[fc][r][j] = bt[16 * fc + r] * a;
        if (OUT) sm.pwP[fc][r][j] = pq;
      }
    }
    block_barrier();
  }
}

static_assert(136 * 4 <= kThreads, "one per-pair item per thread");

// ---------------------------------------------------------------- stage TL: causal tiles on MFMA
// Each tile is formed transposed (operands swapped), so that lane (li, g) holds row li, columns
// 4g .. 4g+3: the diagonal blocks of A go to the solver as fp32 rows, the coupling block -A_10 and
// the blocks of P go straight into their bf16 operand places.
template <bool OUT, bool MID>
__device__ __forceinline__ void tiles(FusedShared& sm, unsigned char* rec, const unsigned char* ops,
                                      const unsigned char* opsM, uint32_t pwmask, uint32_t mid_in, int par, int w,
                                      int lane) {
  const uint32_t mid = MID ? mid_in : 0u;
  const int li = lane & 15, lg = lane >> 4;
  if (w >= (OUT ? 6 : 3)) return;
  const float* bt = reinterpret_cast<const float*>(rec + rBeta);
  const unsigned char *a, *b;
  // a chunk in midpoint mode (mid bit c) takes its diagonal blocks' rows from the midpoint buffer; its
  // columns in oKh are then midpoint-referenced as well
  switch (w) {
    case 0: a = (mid & 1u) ? opsM + mK0 : rec + rKb; b = ops + oKh; break;              // A_00 (rows of -beta Kbar)
    case 1: a = (mid & 2u) ? opsM + mK1 : ops + oKb1; b = ops + oKh + 4 * kBlk; break;  // A_11
    case 2: a = ops + oKb1; b = ops + oKt0; break;                                      // A_10
    case 3: a = (mid & 1u) ? opsM + mQ0 : rec + rQb; b = ops + oKh; break;              // P_00
    case 4: a = (mid & 2u) ? opsM + mQ1 : ops + oQb1; b = ops + oKh + 4 * kBlk; break;  // P_11
    default: a = ops + oQb1; b = ops + oKt0; break;                                     // P_10
  }
  floatx4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u) acc = mfma(ld8(b + u * kBlk + slot16(lane)), ld8(a + u * kBlk + slot16(lane)), acc);
  floatx4 x;
  const bool mid0 = w == 0 && (mid & 1u);   // A_00 from midpoint rows, which carry no -beta
  const float b1 = (w == 1 || w == 2) ? bt[16 + li] : mid0 ? bt[li] : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = 4 * lg + r;   // element (li, c) of the block
    switch (w) {
      case 0: x[r] = c < li ? (mid0 ? b1 * acc[r] : -acc[r]) : 0.f; break;
      case 1: x[r] = c < li ? b1 * acc[r] : 0.f; break;
      case 2: x[r] = -b1 * acc[r]; break;
      case 3: case 4: x[r] = c <= li ? acc[r] : 0.f; break;
      default: x[r] = acc[r]; break;
    }
  }
  // a flagged chunk's diagonal block comes from its per-pair values instead (the test is uniform, so
  // the common step reads nothing more and takes no lane-dependent branch)
  if (pwmask && ((w == 0 || w == 3) ? (pwmask & 1u) : (w == 1 || w == 4) ? (pwmask & 2u) : 0u)) {
    const float (*pw)[16] = w == 0 ? sm.pwA[0] : w == 1 ? sm.pwA[1] : w == 3 ? sm.pwP[0] : sm.pwP[1];
    const floatx4 v = *reinterpret_cast<const floatx4*>(&pw[li][4 * lg]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 4 * lg + r;
      x[r] = (w == 0 || w == 1) ? (c < li ? v[r] : 0.f) : (c <= li ? v[r] : 0.f);
    }
  }
  switch (w) {
    case 0: *reinterpret_cast<floatx4*>(&sm.A[par][li][4 * lg]) = x; break;
    case 1: *reinterpret_cast<floatx4*>(&sm.A[par][16 + li][4 * lg]) = x; break;
    case 2: *reinterpret_cast<bf16x4*>(rec + rT + kOpA10 + lane * 8) = pack4(x); break;
    case 3: *reinterpret_cast<bf16x8*>(rec + rP + slot16(lane)) = pack2(x, floatx4{0, 0, 0, 0}); break;   // P_01 = 0
    case 4: *reinterpret_cast<bf16x4*>(rec + rP + kBlk + slot16(lane) + 8) = pack4(x); break;
    default: *reinterpret_cast<bf16x4*>(rec + rP + kBlk + slot16(lane)) = pack4(x); break;
  }
}

// ---------------------------------------------------------------- stage S: T = (I + A)^{-1}
// One wavefront per diagonal block; the four lanes of quad li own row li of T_bb, lane q of the quad
// columns 4q .. 4q+3.  Row t of T satisfies t (I + A) = e_li, so its entries follow from the last one
// backwards: once t_m is final (in lane m/4 of the quad, broadcast within the quad), t_k -= t_m A[m][k]
// for every k < m.  The coupling block is not formed: the chain applies it as U_1 = T_11 (R_1 - A_10 U_0).
__device__ __forceinline__ float quad_bcast(float v, int src) {   // src is a constant after unrolling
  switch (src) {
    case 0: return dpp<0x00>(0.f, v);
    case 1: return dpp<0x55>(0.f, v);
    case 2: return dpp<0xAA>(0.f, v);
    default: return dpp<0xFF>(0.f, v);
  }
}

__device__ __forceinline__ void solve_block(FusedShared& sm, unsigned char* rec, int par, int b, int lane_in) {
  const int lane = opaque(lane_in);
  const int li = lane >> 2, q = lane & 3;
  const float* Ab = &sm.A[par][16 * b][4 * q];
  floatx4 t;
#pragma unroll
  for (int c = 0; c < 4; ++c) t[c] = (li == 4 * q + c) ? 1.f : 0.f;
  floatx4 a[15];
#pragma unroll
  for (int m = 15; m >= 8; --m) a[m - 1] = *reinterpret_cast<const floatx4*>(Ab + m * kRowA);
#pragma unroll
  for (int m = 15; m >= 1; --m) {
    if (m == 7) {
#pragma unroll
      for (int mm = 7; mm >= 1; --mm) a[mm - 1] = *reinterpret_cast<const floatx4*>(Ab + mm * kRowA);
    }
    const float x = quad_bcast(t[m & 3], m >> 2);   // quad_perm broadcast of lane m/4
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = (4 * q + c < m) ? t[c] - x * a[m - 1][c] : t[c];
  }
  // operand lane li + 16 q holds row li, columns 4q .. 4q+3
  *reinterpret_cast<bf16x4*>(rec + rT + (b ? kOpT11 : kOpT00) + (li + 16 * q) * 8) = pack4(t);
}

// ---------------------------------------------------------------- stage C helpers
// V of one step in D layout for column col: rows 16mt + 4lg + r.  Each value is widened to 32 bits as
// it is loaded: with 16-bit values the compiler packs two loads into one register at once, waiting
// for them (and for every load issued before them, among them the next step's prefetch).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of V: step `step`, row `row` of it, columns 8 c8 .. 8 c8 + 7 (zero past the end of the view)
__device__ __forceinline__ uint4 v_load16(const Views& vw, int step, int row, int c8) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vw.v, (row * D + 8 * c8) * 2, step * (STEP * D * 2), 0);
  return uint4{x[0], x[1], x[2], x[3]};
}

// diag(beta) V of this lane's accumulator places (rows 16 mt + 4 lg + r, column col), V read from the
// stage.  The 16 lanes of a row share lg, hence their eight betas: lane li of the row reads the beta of
// place (mt, r) = (li / 4, li % 4), and each place takes it by a row broadcast from that lane.
__device__ __forceinline__ void beta_v(floatx4 (&bv)[2], const FusedShared& sm, const unsigned char* rec, int lg,
                                       int li, int col) {
  const float* bt = reinterpret_cast<const float*>(rec + rBeta);
  const float bl = bt[16 * ((li >> 2) & 1) + 4 * lg + (li & 3)];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t x = *reinterpret_cast<const uint16_t*>(&sm.ostage[16 * mt + 4 * lg + r][2 * col]);
      bv[mt][r] = row_bcast(bl, 4 * mt + r) * __uint_as_float(x << 16);
    }
  }
}

__device__ __forceinline__ int rows_left(int T, int step) {
  const int rem = T - step * STEP;
  return rem < STEP ? rem : STEP;
}

// One step of a corrected segment's transition, column slice 16 w' .. 16 w' + 15 of M (the E wavefront
// w' = w - 8 carries it), from the step's record: R_M = -diag(beta) Kbar M, U_M = T R_M, then
// Qtil = Qbar M + P U_M (the outputs' coefficient of the entering state, to this slice's 16 columns)
// and M <- diag(e^{Gam}) M + Ktil^T U_M.  Same products, operand places and broadcasts as the state
// step of the C wavefronts, with M for S and no V.  Lane (li, lg) writes Qtil[16 mt + li][16 w' + 4 lg + r],
// mt = 0, 1, as 16 bytes to qo.
__device__ __forceinline__ void transition_step(const unsigned char* rec, floatx4 (&M)[8], unsigned char* qo,
                                                int lane) {
  const floatx4 zero = {0, 0, 0, 0};
  const int ln = opaque(lane);
  const int sl = slot16(ln), lg = ln >> 4, li = ln & 15;
  bf16x8 mb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) mb[u] = pack2(M[2 * u], M[2 * u + 1]);
  floatx4 RM[2] = {zero, zero};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) RM[mt] = mfma(ld8(rec + rKb + (mt * 4 + u) * kBlk + sl), mb[u], RM[mt]);
  const int l8 = ln * 8;
  const floatx4 UM0 = mfma16(ld4(rec + rT + kOpT00 + l8), pack4(RM[0]), zero);
  const floatx4 RM1 = mfma16(ld4(rec + rT + kOpA10 + l8), pack4(UM0), RM[1]);
  const floatx4 UM1 = mfma16(ld4(rec + rT + kOpT11 + l8), pack4(RM1), zero);
  const bf16x8 um = pack2(UM0, UM1);
  floatx4 Qt[2] = {zero, zero};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) Qt[mt] = mfma(mb[u], ld8(rec + rQb + (mt * 4 + u) * kBlk + sl), Qt[mt]);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) Qt[mt] = mfma(um, ld8(rec + rP + mt * kBlk + sl), Qt[mt]);
  *reinterpret_cast<uint4*>(qo) = uint4{pk_bf16(Qt[0][0], Qt[0][1]), pk_bf16(Qt[0][2], Qt[0][3]),
                                        pk_bf16(Qt[1][0], Qt[1][1]), pk_bf16(Qt[1][2], Qt[1][3])};
  const float2 egl = *reinterpret_cast<const float2*>(rec + rEg + (lg * 32 + 2 * li) * 4);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) M[t][r] *= row_bcast((r & 1) ? egl.y : egl.x, 2 * t + (r >> 1));
    M[t] = mfma(ld8(rec + rKt + t * kBlk + sl), um, M[t]);
  }
}

// E wavefronts of chunk CC.  Interval s: first half E1(s+2), second half E2(s+2) and, for a flagged
// chunk, the per-pair blocks of step s+2.  COR (a corrected segment): the first half also advances the
// wavefront's slice of the transition M over step s (its record is complete and stays in place until
// the next barrier), while the C wavefronts advance the state over the same step; qdst: the
// segment's first step of propagated queries.
template <bool OUT, int GK, int CC, bool COR>
__device__ __forceinline__ void e_loop(FusedShared& sm, const Params& p, const Views& vw, int s0, int ns, int we,
                                       int lane, int tid, floatx4 (&M)[8], unsigned char* qdst) {
  if (COR) {
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) M[t][r] = (16 * t + 4 * lg + r == 16 * we + li) ? 1.f : 0.f;
  }
  const int e_voff = ((16 * CC + 4 * (lane & 3)) * D + 2 * (16 * (we & 3) + (lane >> 2))) * 2;
  const int e_boff = (16 * CC + 4 * (lane & 3)) * 2;
  EIn ein;
  EKeep ekeep;
  e_load<OUT>(ein, vw, 0, e_voff, e_boff);   // steps relative to the segment's first
  int slotE = 2;   // record slot of step it + 2 (it + 2 mod 3), advanced at the top of each pass
#pragma unroll 1
  for (int it = -2; it < ns; ++it) {
    const bool doE = it + 2 < ns;
    slotE = slotE == kRecSlots - 1 ? 0 : slotE + 1;
    unsigned char* recE = sm.rec[slotE];                  // step it + 2
    unsigned char* opsE = sm.ops[(it + 2) & 1];           // step it + 2
    unsigned char* opsF = sm.ops[(it + 3) & 1];           // step it + 1 (free once its tiles are formed)
    block_barrier();
    KDA_STAMP(p, 8 + we, it + 2, 0);
    const int ln = opaque(lane);   // lane-derived offsets are recomputed in the loop rather than held
    if (doE) e_first<GK == kGateUnbounded, CC, GK != kGatePlain>(sm, ein, ekeep, p, s0 + it + 2, recE, we, ln);
    KDA_STAMP(p, 8 + we, it + 2, 1);
    // prefetches are issued on every path (clamped to the segment's last step) so that the memory
    // counter waits before their uses stay exact
    e_load<OUT>(ein, vw, it + 3 < ns ? it + 3 : ns - 1, e_voff, e_boff);
    KDA_STAMP(p, 8 + we, it + 2, 2);
    if (COR && it >= 0)   // step it's record: the slot after step it + 2's
      transition_step(sm.rec[slotE == kRecSlots - 1 ? 0 : slotE + 1], M, qdst + it * (int64_t)kQtStep + we * 1024 + lane * 16,
                      lane);
    KDA_STAMP(p, 8 + we, it + 2, 3);
    block_barrier();
    KDA_STAMP(p, 8 + we, it + 2, 4);
    if (doE) {
      const Modes md = GK != kGatePlain ? step_modes(sm, p, s0 + it + 2) : Modes{0u, 0u};
      // the midpoint operands in a copy of their own, so that the common step runs the plain one
      if (GK != kGatePlain && __builtin_expect((md.mid >> CC) & 1u, 0))
        e_second<OUT, CC, true>(sm, ekeep, p, s0 + it + 2, recE, opsE, opsF, md, we, ln);
      else
        e_second<OUT, CC, false>(sm, ekeep, p, s0 + it + 2, recE, opsE, opsF, md, we, ln);
      KDA_STAMP(p, 8 + we, it + 2, 5);
      if (GK != kGatePlain && __builtin_expect(md.pw != 0u, 0))
        pairwise_blocks<OUT, true>(sm, &ekeep, recE, opsF, md.pw, we, ln, tid);
    }
  }
}

// ---------------------------------------------------------------- one segment, and the kernel
// Wavefronts 0-7 (C) own the state slices (slice w: 16 columns) and run the tiles and the solve;
// wavefronts 8-15 (E) run the E stage.  Both kinds meet at the same two barriers per interval.
//
// How segment 0 ends when other segments follow it in the same pass (OUT only): its leaving state is
// the entering state of segment 1, where the chaining pass starts, and its statistics go either to a
// per-head record that the chaining pass folds into the call's counters (the map pass, which runs
// before the counters are reset) or straight into the counters (the corrected plan's pass).
constexpr int kAlone = 0, kEarlyRecord = 1, kEarlyAtomic = 2;

// Map of segment j, column slice w: X_j in slice-major D layout; M_j split into bf16 hi + lo parts,
// each arranged as the chaining kernel's A operands:
// [mo 8][u 4][lane 64][8] <-> M[16 mo + (lane & 15)][32 u + {0,16} + 4 (lane >> 4) + r]
__device__ __forceinline__ void store_x(const Params& p, const SegPlan& sg, int64_t bh, int j, int w, int lane,
                                        const floatx4 (&X)[8]) {
  float* xo = (float*)((unsigned char*)p.workspace + sg.off_x + (bh * sg.P + j) * (int64_t)kSegState) + w * 8 * 64 * 4;
  store_slice(xo, X, lane);
}
__device__ __forceinline__ void store_m(const Params& p, const SegPlan& sg, int64_t bh, int j, int w, int lane,
                                        const floatx4 (&M)[8]) {
  const int li = lane & 15, lg = lane >> 4;
  const int64_t blk = bh * sg.P + j;
  __bf16* mh = (__bf16*)((unsigned char*)p.workspace + sg.off_m + blk * (int64_t)kSegState);
  __bf16* ml = mh + kMHalf / 2;
  const int u = w >> 1, pos = (w & 1) * 4 + (li & 3);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lane_c = (4 * lg + r) + 16 * (li >> 2);   // element M[16t + 4lg + r][16 w + li]
      const int e = ((t * 4 + u) * 64 + lane_c) * 8 + pos;
      const __bf16 hi = (__bf16)M[t][r];
      mh[e] = hi;
      ml[e] = (__bf16)(M[t][r] - (float)hi);
    }
}

// Where a corrected segment carries the eight 16-column slices of its transition M: in the idle time
// of the wavefronts that have it (per 32-token step, the first half lasts as long as the state chain
// plus a causal tile, the second as long as the E stage's second half).
//   slices 0-3   E wavefronts of chunk 0 (8-11), first half, after their share of E1
//   slices 4-5   state wavefronts 6-7, first half, after the state chain (they form no tile)
//   slices 6-7   state wavefronts 4-5, second half (they store nothing and solve nothing there)
// The chunk-1 E wavefronts, the slowest of the first half, carry none.
constexpr int kMNone = 0, kMFirst = 1, kMSecond = 2;   // a state wavefront's share of M

// One workgroup's segment, for the wavefronts of M role MR (kMNone: every wavefront but state
// wavefronts 4-7 of a corrected segment).  OUT: segment j from its entering state, with the outputs;
// !OUT: the map of segment j.  COR (with OUT): segment j >= 1 of the corrected plan, with its outputs
// from a zero entering state, its propagated queries Qtil and its map.  `early`: kAlone, or how
// segment 0 ends.
template <bool OUT, int GK, bool COR, int MR>
__device__ __forceinline__ void fused_part(FusedShared& sm, const Params& p, int64_t n_steps, const SegPlan& sg,
                                           int64_t bh, int j, int early) {
  static_assert(OUT || !COR, "the corrected segments write outputs");
  static_assert(COR || MR == kMNone, "only corrected segments carry M on their state wavefronts");
  const int tid = threadIdx.x;
  // the wavefront index through a scalar register: branches on it (and on the chunk and role derived
  // from it) are then uniform, rather than masked paths that every wavefront would step through
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_e = w >= kCWaves;
  const int we = w - kCWaves;                 // E wavefront index (valid when is_e)
  const int li = lane & 15, lg = lane >> 4;
  // step and token indices fit 32 bits (T < 2^30), which keeps the scalar index arithmetic short
  const int s0 = j == 0 ? 0 : (int)sg.L0 + (j - 1) * (int)sg.L;
  const int len = j == 0 ? (int)sg.L0 : (int)sg.L;
  const int ns = ((int)n_steps - s0 < len) ? (int)n_steps - s0 : len;
  const int64_t T = p.T;
  const int col = 16 * (w & 7) + li;
  const floatx4 zero = {0, 0, 0, 0};

  Views vw;   // this segment's tokens; loads take steps relative to s0
  {
    const int64_t tok0 = (int64_t)s0 * STEP;
    const int64_t ntok = (T - tok0 < (int64_t)ns * STEP) ? T - tok0 : (int64_t)ns * STEP;
    const int64_t nb = ntok * D * 2;
    vw.k = view((const uint16_t*)p.k + (bh * T + tok0) * D, nb);
    vw.w = view((const uint16_t*)p.w + (bh * T + tok0) * D, nb);
    vw.q = view((const uint16_t*)p.q + (bh * T + tok0) * D, nb);
    vw.v = view((const uint16_t*)p.v + (bh * T + tok0) * D, nb);
    vw.beta = view((const uint16_t*)p.beta + bh * T + tok0, ntok * 2);
  }

  // The two kinds of wavefront run separate copies of the step loop (same trip count, same barriers in
  // the same order), so that each copy holds only its own kind's values in registers.
  unsigned char* qdst = COR ? (unsigned char*)p.workspace + sg.off_q + (bh * n_steps + s0) * (int64_t)kQtStep : nullptr;
  if (MR == kMNone && is_e) {
    floatx4 M[8];
    if (we < 4) e_loop<OUT, GK, 0, COR>(sm, p, vw, s0, ns, we, lane, tid, M, qdst);
    else e_loop<OUT, GK, 1, false>(sm, p, vw, s0, ns, we, lane, tid, M, qdst);
    if (COR && we < 4) store_m(p, sg, bh, j, we, lane, M);
    return;
  }
  // which wavefronts run this copy (lets the compiler drop the other wavefronts' tile and store forms)
  if (MR == kMFirst) __builtin_assume(w == 6 || w == 7);
  if (MR == kMSecond) __builtin_assume(w == 4 || w == 5);
  if (COR && MR == kMNone) __builtin_assume(w < 4);
  // this state wavefront's slice of M (state wavefronts 4-7 of a corrected segment; the map pass: its own)
  const int mslice = MR == kMFirst ? w - 2 : MR == kMSecond ? w + 2 : (w & 7);

  // C wavefronts: OUT -> S (the slice of the true state; COR: from zero); !OUT -> X (from zero) and M
  // (from the identity)
  floatx4 S[8], M[8];
  if (OUT && !COR) {
    if (j > 0) {
      load_slice(S, (const float*)((const unsigned char*)p.workspace + sg.off_s) + (bh * sg.P + j) * (int64_t)(kSegState / 4) +
                        w * 8 * 64 * 4, lane);
    } else if (p.S0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][r] = p.S0[(bh * D + 16 * t + 4 * lg + r) * D + col];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = zero;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      S[t] = zero;
#pragma unroll
      for (int r = 0; r < 4; ++r) M[t][r] = (16 * t + 4 * lg + r == 16 * mslice + li) ? 1.f : 0.f;
    }
  }
  uint4 vq[2];   // wavefronts 0-3: V rows of the next step, 16 bytes per lane
  uint32_t nonfinite = 0, n_valid = 0, n_flagged = 0;
  float min_span = __int_as_float(0x7f800000);

  int slotC = 0;   // record slot of step it (it mod 3), advanced at the top of each pass
#pragma unroll 1
  for (int it = -2; it < ns; ++it) {
    const bool doE = it + 2 < ns, doS = it + 1 >= 0 && it + 1 < ns, doC = it >= 0;
    slotC = slotC == kRecSlots - 1 ? 0 : slotC + 1;
    const int slotS = slotC == kRecSlots - 1 ? 0 : slotC + 1, slotE = slotS == kRecSlots - 1 ? 0 : slotS + 1;
    unsigned char* recC = sm.rec[slotC];   // step it
    unsigned char* recS = sm.rec[slotS];   // step it + 1
    unsigned char* recE = sm.rec[slotE];   // step it + 2
    unsigned char* opsF = sm.ops[(it + 3) & 1];           // step it + 1
    block_barrier();
    KDA_STAMP(p, w, it + 2, 0);
    const int ln = opaque(lane);
    const int sl = slot16(ln);
    const bool low4 = MR == kMNone && w < 4;   // wavefronts 0-3 (the copies with M are wavefronts 4-7)
    if (OUT && low4) {   // V of step it + 1, issued first so that the whole first half covers its latency
      const int sn = it + 1 < 0 ? 0 : (it + 1 < ns ? it + 1 : ns - 1);   // relative to s0
#pragma unroll
      for (int i = 0; i < 2; ++i) vq[i] = v_load16(vw, sn, 8 * w + 4 * i + (lane >> 4), lane & 15);
    }
    // ---- first half: the whole recurrence step of step it (map pass: of X and M together, each
    // operand read once for both)
    if (doC) {
      bf16x8 sb[4];   // bf16 copies of the entering state, the B operands of this step
#pragma unroll
      for (int u = 0; u < 4; ++u) sb[u] = pack2(S[2 * u], S[2 * u + 1]);
      floatx4 bv[2];
      beta_v(bv, sm, recC, lg, li, col);
      floatx4 R[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) R[mt] = bv[mt];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) R[mt] = mfma(ld8(recC + rKb + (mt * 4 + u) * kBlk + sl), sb[u], R[mt]);
      // U = T R blockwise: U_0 = T_00 R_0, U_1 = T_11 (R_1 - A_10 U_0)
      const floatx4 U0 = mfma16(ld4(recC + rT + kOpT00 + ln * 8), pack4(R[0]), zero);
      const floatx4 R1 = mfma16(ld4(recC + rT + kOpA10 + ln * 8), pack4(U0), R[1]);
      const floatx4 U1 = mfma16(ld4(recC + rT + kOpT11 + ln * 8), pack4(R1), zero);
      const bf16x8 ub = pack2(U0, U1);
      if (OUT) {
        const int st = s0 + it;
        const int nrows = rows_left((int)T, st);
        floatx4 O[2] = {zero, zero};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) O[mt] = mfma(sb[u], ld8(recC + rQb + (mt * 4 + u) * kBlk + sl), O[mt]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) O[mt] = mfma(ub, ld8(recC + rP + mt * kBlk + sl), O[mt]);
        // this wavefront's 16 columns of every row into the stage; whole rows go out in the second half
        uint32_t mx = 0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          *reinterpret_cast<uint2*>(&sm.ostage[16 * mt + li][(16 * w + 4 * lg) * 2]) =
              uint2{pk_bf16(O[mt][0], O[mt][1]), pk_bf16(O[mt][2], O[mt][3])};
          if (!COR && (nrows == STEP || 16 * mt + li < nrows)) {   // corrected outputs are counted when final
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
        if (w == 0) {
          const StepInfo si = *reinterpret_cast<const StepInfo*>(recC + rMeta);
          n_valid += si.n_valid;
          n_flagged += si.n_flagged;
          min_span = fminf(min_span, fminf(si.span[0], si.span[1]));
        }
      }
      // state update: S <- diag(e^{Gam}) S + Ktil^T U.  The 16 lanes of a row share lg, hence the 32 rows
      // 16 t + 4 lg + r they hold: lane li reads the factors of places 2 li and 2 li + 1 (place 4 t + r),
      // and each place takes its factor by a row broadcast.
      {
        const float2 egl = *reinterpret_cast<const float2*>(recC + rEg + (lg * 32 + 2 * li) * 4);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) S[t][r] *= row_bcast((r & 1) ? egl.y : egl.x, 2 * t + (r >> 1));
          S[t] = mfma(ld8(recC + rKt + t * kBlk + sl), ub, S[t]);
        }
      }
      if (!OUT) {   // the transition slice, after the state slice so that the two need not be live at once
        // fresh offsets: reusing the state slice's loads would keep them live across both slices
        const int sl = opaque(slot16(ln)), lgm = opaque(lg), lim = opaque(li);
        bf16x8 mb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) mb[u] = pack2(M[2 * u], M[2 * u + 1]);
        floatx4 RM[2] = {zero, zero};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) RM[mt] = mfma(ld8(recC + rKb + (mt * 4 + u) * kBlk + sl), mb[u], RM[mt]);
        const int l8 = opaque(ln * 8);
        const floatx4 UM0 = mfma16(ld4(recC + rT + kOpT00 + l8), pack4(RM[0]), zero);
        const floatx4 RM1 = mfma16(ld4(recC + rT + kOpA10 + l8), pack4(UM0), RM[1]);
        const floatx4 UM1 = mfma16(ld4(recC + rT + kOpT11 + l8), pack4(RM1), zero);
        const bf16x8 um = pack2(UM0, UM1);
        const float2 egl = *reinterpret_cast<const float2*>(recC + rEg + (lgm * 32 + 2 * lim) * 4);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) M[t][r] *= row_bcast((r & 1) ? egl.y : egl.x, 2 * t + (r >> 1));
          M[t] = mfma(ld8(recC + rKt + t * kBlk + sl), um, M[t]);
        }
      }
    }
    KDA_STAMP(p, w, it + 2, 1);
    if (MR == kMFirst && doC)
      transition_step(recC, M, qdst + it * (int64_t)kQtStep + mslice * 1024 + lane * 16, lane);
    // ---- the causal tiles of step it + 1 (their chunk flags are in its information record)
    if (doS && MR != kMFirst) {   // (wavefronts 6-7 form no tile)
      const StepInfo* si = reinterpret_cast<const StepInfo*>(recS + rMeta);
      const uint32_t mid = GK != kGatePlain ? si->midpoint : 0u;
      if (GK != kGatePlain && __builtin_expect(mid != 0u, 0)) tiles<OUT, true>(sm, recS, opsF, sm.ops[(it + 2) & 1], si->pairwise, mid, (int)((it + 1) & 1), w, ln);
      else tiles<OUT, false>(sm, recS, opsF, sm.ops[(it + 2) & 1], si->pairwise, 0u, (int)((it + 1) & 1), w, ln);
    }
    if (!OUT && low4) {   // V of step it + 1 (the map pass has no registers to carry it over the chain)
      const int sn = it + 1 < 0 ? 0 : (it + 1 < ns ? it + 1 : ns - 1);   // relative to s0
#pragma unroll
      for (int i = 0; i < 2; ++i) vq[i] = v_load16(vw, sn, 8 * w + 4 * i + (lane >> 4), lane & 15);
    }
    KDA_STAMP(p, w, it + 2, 2);
    block_barrier();
    KDA_STAMP(p, w, it + 2, 3);
    // ---- second half: o of step it out of the stage as whole rows (wavefronts 0-3, eight rows each,
    // 16 bytes per lane: 256 contiguous bytes per row), per-pair blocks of step it + 2 (if any), T of
    // step it + 1
    if (OUT && doC && low4) {
      const int st = s0 + it;
      const int nrows = rows_left((int)T, st);
      uint16_t* ob = (uint16_t*)p.o + bh * T * D + (int64_t)st * STEP * D;
      const int c16 = lane & 15;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 8 * w + 4 * i + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.ostage[row][c16 * 16]);
        if (row < nrows) *reinterpret_cast<uint4*>(ob + row * D + c16 * 8) = v;
      }
    }
    if (low4 && it + 1 >= 0 && it + 1 < ns) {   // V of step it + 1 over the rows just stored
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<uint4*>(&sm.ostage[8 * w + 4 * i + (lane >> 4)][(lane & 15) * 16]) = vq[i];
    }
    // T of step it + 1 first: it shares nothing with the per-pair blocks, so on a flagged step it
    // overlaps the E stage instead of following the per-pair barriers
    KDA_STAMP(p, w, it + 2, 4);
    if (doS && w >= 6 && MR != kMSecond) solve_block(sm, recS, (int)((it + 1) & 1), w - 6, ln);
    KDA_STAMP(p, w, it + 2, 5);
    if (GK != kGatePlain && doE) {
      const uint32_t pwmask = step_modes(sm, p, s0 + it + 2).pw;
      if (__builtin_expect(pwmask != 0u, 0)) pairwise_blocks<OUT, false>(sm, nullptr, recE, opsF, pwmask, 0, ln, tid);
    }
    if (MR == kMSecond && doC)
      transition_step(recC, M, qdst + it * (int64_t)kQtStep + mslice * 1024 + lane * 16, lane);
  }

  if (OUT) {
    if (COR) {
      store_x(p, sg, bh, j, w, lane, S);
      if (MR != kMNone) store_m(p, sg, bh, j, mslice, lane, M);
    } else if (early != kAlone) {
      // segment 0 ran beside other segments: its leaving state enters segment 1, in the layout of the
      // chaining pass's states
      float* so = (float*)((unsigned char*)p.workspace + sg.off_s + (bh * sg.P + 1) * (int64_t)kSegState) + w * 8 * 64 * 4;
      store_slice(so, S, lane);
    } else if (j == sg.P - 1) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p.S_final[(bh * D + 16 * t + 4 * lg + r) * D + col] = S[t][r];
          nonfinite += not_finite(S[t][r]) ? 1u : 0u;
        }
    }
    if (p.stats) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) nonfinite += __shfl_xor(nonfinite, off);
      if (early == kEarlyRecord) {
        // plain stores into the head's record (the unused entering-state block of segment 0): the
        // counters are reset only after this pass, by the chaining pass, which adds these in
        uint32_t* rec = (uint32_t*)((unsigned char*)p.workspace + sg.off_s + bh * sg.P * (int64_t)kSegState);
        if (lane == 0) {
          rec[kRecNonfinite + w] = nonfinite;
          if (w == 0) {
            rec[kRecChunks] = n_valid;
            rec[kRecFlagged] = n_flagged;
            rec[kRecMinSpan] = __float_as_uint(min_span);
          }
        }
      } else if (lane == 0) {
        if (nonfinite) atomicAdd(&p.stats->n_nonfinite, nonfinite);
        if (w == 0) {
          atomicAdd(&p.stats->n_chunks, n_valid);
          if (n_flagged) atomicAdd(&p.stats->n_flagged, n_flagged);
          if (n_valid) atomic_min_float(&p.stats->min_span, min_span);
        }
      }
    }
  } else {
    store_x(p, sg, bh, j, w, lane, S);
    store_m(p, sg, bh, j, w, lane, M);
  }
}

// One workgroup's segment: state wavefronts 4-7 of a corrected segment take the copies of the step loop
// that carry their slice of M, every other wavefront the copy without it.
template <bool OUT, int GK, bool COR = false>
__device__ __forceinline__ void fused_body(FusedShared& sm, const Params& p, int64_t n_steps, const SegPlan& sg,
                                           int64_t bh, int j, int early) {
  if constexpr (COR) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w == 6 || w == 7) return fused_part<OUT, GK, COR, kMFirst>(sm, p, n_steps, sg, bh, j, early);
    if (w == 4 || w == 5) return fused_part<OUT, GK, COR, kMSecond>(sm, p, n_steps, sg, bh, j, early);
  }
  fused_part<OUT, GK, COR, kMNone>(sm, p, n_steps, sg, bh, j, early);
}

// OUT: the output pass, segments 1 .. P-1 (segment 0 ran in the map pass), or the only segment of a
// one-segment plan.  !OUT (plans of two or more segments): the map pass, segment 0 with its outputs
// (it needs no map: its entering state is S0) beside the maps of segments 1 .. P-2.
template <bool OUT, int GK>
__global__ __launch_bounds__(kThreads) void fused_kernel(Params p, int64_t n_steps, SegPlan sg) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FusedShared& sm = *reinterpret_cast<FusedShared*>(smem_raw);
  const int nb = sg.P > 1 ? (int)sg.P - 1 : 1;   // workgroups per head
  const int64_t bh = blockIdx.x / nb;
  const int i = (int)(blockIdx.x % nb);
  if (OUT) {
    fused_body<true, GK>(sm, p, n_steps, sg, bh, sg.P > 1 ? i + 1 : 0, kAlone);
  } else if (i == 0) {
    fused_body<true, GK>(sm, p, n_steps, sg, bh, 0, kEarlyRecord);
  } else {
    fused_body<false, GK>(sm, p, n_steps, sg, bh, i, kAlone);
  }
}

// The corrected plan's pass: P workgroups per head, segment 0 exact from S0 (all of the sequence when
// P = 1), segments 1 .. P-1 from a zero entering state with their propagated queries and maps.
template <int GK>
__global__ __launch_bounds__(kThreads) void fused_corr_kernel(Params p, int64_t n_steps, SegPlan sg) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FusedShared& sm = *reinterpret_cast<FusedShared*>(smem_raw);
  const int64_t bh = blockIdx.x / sg.P;
  const int i = (int)(blockIdx.x % sg.P);
  if (i == 0) fused_body<true, GK>(sm, p, n_steps, sg, bh, 0, sg.P > 1 ? kEarlyAtomic : kAlone);
  else fused_body<true, GK, true>(sm, p, n_steps, sg, bh, i, kAlone);
}

template <int GK>
hipError_t launch_corr(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_dyn_lds((const void*)fused_corr_kernel<GK>, (int)kFusedSmem, lds_set);
  if (e != hipSuccess) return e;
  if (sg.P > 1 && sg.off_q == 0) return hipErrorInvalidValue;   // a plan without room for the queries
  hipLaunchKernelGGL((fused_corr_kernel<GK>), dim3((unsigned)(p.B * p.H * sg.P)), dim3(kThreads), kFusedSmem, s, p,
                     n_steps, sg);
  return hipGetLastError();
}

template <bool OUT, int GK>
hipError_t launch_one(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_dyn_lds((const void*)fused_kernel<OUT, GK>, (int)kFusedSmem, lds_set);
  if (e != hipSuccess) return e;
  if (!OUT && sg.P < 2) return hipErrorInvalidValue;   // a one-segment plan has no map pass
  const int64_t nb = sg.P > 1 ? sg.P - 1 : 1;
  hipLaunchKernelGGL((fused_kernel<OUT, GK>), dim3((unsigned)(p.B * p.H * nb)), dim3(kThreads), kFusedSmem, s, p,
                     n_steps, sg);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(int dtype, int64_t dk, int64_t dv, int64_t T) {
  // token and step indices are 32-bit in the kernels (the segment length is checked with the plan)
  return dtype == KDA_DTYPE_BF16 && dk == D && dv == D && T < ((int64_t)1 << 30);
}

// The gate kind of a call.  With a bounded gate and 16 g_min >= -80 every chunk's span is at least -80
// (up to the rounding of its sum of 16 gates, which moves e^{-L} by a factor 1 + 2^-20 at most, far from
// the fp32 limit e^{88.7}), so no chunk can need more than the plain tiles and the kernel is built
// without the flagged-chunk forms; flags are still counted.  A deeper bound, a forced fallback or the
// unbounded gate take the kernel with them.
static int gate_kind(const Params& p) {
  if (p.unbounded) return kGateUnbounded;
  const bool plain = !p.force_fallback && (p.disable_fallback || 16.f * p.g_min >= kSpanLimit);
  return plain ? kGatePlain : kGateFlagged;
}

hipError_t launch_fused_segments(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg, bool out) {
  switch (gate_kind(p)) {
    case kGateUnbounded: return out ? launch_one<true, kGateUnbounded>(p, s, n_steps, sg) : launch_one<false, kGateUnbounded>(p, s, n_steps, sg);
    case kGatePlain: return out ? launch_one<true, kGatePlain>(p, s, n_steps, sg) : launch_one<false, kGatePlain>(p, s, n_steps, sg);
    default: return out ? launch_one<true, kGateFlagged>(p, s, n_steps, sg) : launch_one<false, kGateFlagged>(p, s, n_steps, sg);
  }
}

hipError_t launch_fused_corr(const Params& p, hipStream_t s, int64_t n_steps, const SegPlan& sg) {
  switch (gate_kind(p)) {
    case kGateUnbounded: return launch_corr<kGateUnbounded>(p, s, n_steps, sg);
    case kGatePlain: return launch_corr<kGatePlain>(p, s, n_steps, sg);
    default: return launch_corr<kGateFlagged>(p, s, n_steps, sg);
  }
}

}  // namespace kda

// Segment plans of the matrix-core forward (bf16 MFMA 16x16x32 on gfx950, bf16 inputs with
// dk = dv = 128), and the kernels that join the segments.
//
// The step of the chunk form (32 tokens, two 16-token chunks; "From Numerical Stability to Load
// Balancing ..." section 2.1) is affine in the entering state S, so a run of steps maps its entering
// state to its leaving one as S_end = M S_start + X: M (dk x dk) is the product of the step
// transitions diag(e^{Gam}) - Ktil^T T diag(beta) Kbar and X is the run from a zero state.  Each
// (b, h) sequence is cut into P segments (segment 0 of L0 steps, the others of L, the last one the
// rest) so that about 256 workgroups, one per compute unit, run the segments at once
// (kda_fused.hip).  Two plans join them:
//   fused (mode 3)       a pass of maps (segment 0 with its outputs beside the maps of segments
//                        1 .. P-2), the chaining of the maps, a pass of outputs from the chained
//                        entering states (segments 1 .. P-1)
//   corrected (mode 4)   one pass (segment 0 exactly; segments 1 .. P-1 with their outputs from a zero
//                        entering state, their propagated queries Qtil and their maps), the chaining,
//                        and an HBM-bound pass adding Qtil_t S_start(j) to those outputs
// This file holds the plan, the chaining (seg_combine_kernel), the correction (correct_kernel) and
// the launch sequence of each plan.
#include "kda_mfma_util.h"

namespace kda {

namespace {

constexpr int D = 128;     // dk = dv
constexpr int STEP = 32;   // tokens per step (two chunks)

// ---- seg_combine_kernel: S_start(j+1) = M_j S_start(j) + X_j for one 16-column slice.  The product
// runs on bf16 MFMA in three passes, Mhi Shi + Mhi Slo + Mlo Shi (hi/lo: bf16 value and bf16 residual),
// which leaves a relative error near 2^-16, with fp32 accumulation.  Wavefront w owns the output row
// tiles 2w, 2w+1; the D-layout tiles of S feed the B operands directly through the permuted
// contraction order.  M_j and X_j are fetched two segments ahead.  Segment 0 ran with its outputs in
// the first pass of either plan and left its leaving state in the entering-state block of segment 1,
// where the chain starts; in the fused plan it also left a statistics record per head, which
// workgroup 0 turns into the call's counters before the output pass adds to them.
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

// Chains the maps of one (b, h): S_start(j + 1) = M_j S_start(j) + X_j, fp32 via bf16 hi/lo products,
// from S_start(1) over maps 1 .. P-2 (fused plan), or over maps 1 .. P-1 (corr = 1, the corrected
// plan, whose last map gives S_final, written in the user's layout with its non-finite values counted).
__global__ __launch_bounds__(256) void seg_combine_kernel(Params p, SegPlan sg, int corr) {
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
  const int64_t nseg = corr ? sg.P : sg.P - 1;   // maps 1 .. nseg-1 are chained
  const unsigned char* ws = (const unsigned char*)p.workspace;
  if (!corr && p.stats && blockIdx.x == 0) {   // uniform over workgroup 0: one head per thread, then a reduction
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
  {
    const float* s1 = (const float*)(ws + sg.off_s + (bh * sg.P + 1) * (int64_t)kSegState) + slice * 8 * 64 * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) cur[h] = *reinterpret_cast<const floatx4*>(s1 + ((2 * wave + h) * 64 + lane) * 4);
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
  fetch(c0, ahead(1));
  fetch(c1, ahead(2));
  for (int64_t j = 1; j < nseg; j += 2) {
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

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const void* p) {
  const u32x4v x = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return uint4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void nt_store16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(p));
}

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
    // Qtil and the outputs stream through once (766 MB at the headline against 32 MB of L2): the
    // non-temporal forms keep them from displacing lines that other work still reads
    qreg = nt_load16(qbase + i * (int64_t)kQtStep + tid * 16);
    oreg = orow < rows_of(st) ? nt_load16(obase + (st * STEP + orow) * D + ocol) : uint4{0, 0, 0, 0};
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
    if (orow < nrows) nt_store16(obase + (st * STEP + orow) * D + ocol, *reinterpret_cast<const uint4*>(os + orow * kCorRow + ocol * 2));
  }
  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
    if (lane == 0 && bad) atomicAdd(&p.stats->n_nonfinite, bad);
  }
}

int64_t n_steps_of(int64_t T) { return (T + STEP - 1) / STEP; }

// Segment plan.  Automatic: about 256 workgroups (one per compute unit) per pass over (b, h, segment),
// at least 8 steps per segment and at most kMaxSeg segments, unless more segments are needed to keep
// every segment below kMaxSegSteps steps (the fused kernels' 32-bit buffer views).  The fused plan's
// passes hold P - 1 workgroups per head (segment 0 runs with outputs beside the maps of segments
// 1 .. P-2, then segments 1 .. P-1 run with outputs), so it takes one segment more, when that leaves
// at least three.  seg_steps > 0 fixes the segment length.
// Segment 0 runs beside the other segments in the same pass but takes a different body: its own outputs
// next to their maps (fused plan: a step with outputs takes about 100/93 of a map step, so segment 0 is
// shorter), or its exact outputs next to their outputs from a zero entering state and their maps
// (corrected plan: segment 0 carries no transition, so it is longer; with every compute unit busy the
// pass time hardly depends on it, 0.96 to 1.10 measuring alike).  Percent of the other segments' length.
constexpr int64_t kSeg0PctFused = 93, kSeg0PctCorr = 110;

// The automatic plan with (about) P segments: segment 0 of pct/100 of the others' length.
SegPlan auto_plan(int64_t n, int64_t P, int mode) {
  SegPlan sg{};
  sg.L = (n + P - 1) / P;
  P = (n + sg.L - 1) / sg.L;
  sg.L0 = sg.L;
  if (P >= 2) {
    // segment 0 of length r L (r = pct / 100) beside P - 1 segments of length L, covering the sequence
    const int64_t pct = mode == kModeCorr ? kSeg0PctCorr : kSeg0PctFused;
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
  return sg;
}

SegPlan make_plan(int64_t BH, int64_t T, int64_t seg_steps, int mode) {
  const int64_t n = n_steps_of(T);
  SegPlan sg{};
  if (n <= 0) {   // an empty sequence: one empty segment, nothing kept
    sg.P = 1;
    return sg;
  }
  if (seg_steps > 0) {
    sg.L = sg.L0 = seg_steps;
    sg.P = (n + seg_steps - 1) / seg_steps;
  } else {
    int64_t P = 256 / BH;
    if (mode == kModeFused) P = P >= 2 ? P + 1 : 1;
    const int64_t by_len = n / 8;
    P = P < by_len ? P : by_len;
    P = P < kMaxSeg ? P : kMaxSeg;
    P = P < 1 ? 1 : P;
    sg = auto_plan(n, P, mode);
    // more segments where one would reach kMaxSegSteps (sequences of 2^23 tokens and more per segment)
    while ((sg.L > sg.L0 ? sg.L : sg.L0) >= kMaxSegSteps) sg = auto_plan(n, ++P, mode);
  }
  const int64_t blk = BH * sg.P * (int64_t)kSegState;
  sg.off_x = 0;
  sg.off_m = blk;
  sg.off_s = 2 * blk;
  sg.off_q = mode == kModeCorr ? 3 * blk : 0;
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
#if KDA_PHASE_STAMPS
  const int64_t extra = kStampBytes;   // the stamps follow the plan's blocks
#else
  const int64_t extra = 0;
#endif
  if (sg.P == 1) return (size_t)extra;   // a one-segment plan keeps nothing between kernels
  if (mode == kModeCorr) return (size_t)(sg.off_q + B * H * n_steps_of(T) * (int64_t)kQtStep + extra);
  return (size_t)(sg.off_s + B * H * sg.P * (int64_t)kSegState + extra);
}

bool mfma_seg_steps_ok(int64_t T, int64_t seg_steps) {
  if (seg_steps < 0 || seg_steps >= kMaxSegSteps) return false;
  if (seg_steps == 0) return true;
  const int64_t n = n_steps_of(T);
  return (n + seg_steps - 1) / seg_steps <= kMaxSeg;
}

hipError_t launch_mfma(const Params& p, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end, int mode) {
  const int64_t n_steps = n_steps_of(p.T);
  const int64_t BH = p.B * p.H;
  if ((mode != kModeFused && mode != kModeCorr) || !fused_supported(p.dtype, p.dk, p.dv, p.T) ||
      !mfma_seg_steps_ok(p.T, p.seg_steps))
    return hipErrorInvalidValue;   // the host validation takes every call to one of the two plans
  const SegPlan sg = make_plan(BH, p.T, p.seg_steps, mode);
  hipError_t e;
  if (mode == kModeCorr) {
    // statistics reset first: every pass adds its counts with atomics
    if (p.stats && (e = launch_stats_init(p.stats, s)) != hipSuccess) return e;
    if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
    if ((e = launch_fused_corr(p, s, n_steps, sg)) != hipSuccess) return e;
    if (sg.P > 1) {
      hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(BH * 8)), dim3(256), 0, s, p, sg, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = launch_correct(p, s, n_steps, sg)) != hipSuccess) return e;
    }
    if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  // fused plan: the statistics are reset by the chaining pass when there is one, else by their own launch
  if (p.stats && sg.P == 1 && (e = launch_stats_init(p.stats, s)) != hipSuccess) return e;
  if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
  if (sg.P > 1) {
    if ((e = launch_fused_segments(p, s, n_steps, sg, false)) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(BH * 8)), dim3(256), 0, s, p, sg, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_fused_segments(p, s, n_steps, sg, true)) != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace kda

// Host side of libkda.so: argument validation, path selection and launches.
// Validation runs entirely on the host before any HIP call, so an invalid call
// returns its error code without touching the device.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kda_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_fail(hipError_t e) { return kda::record_hip_error(e); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// B,H,T,dk,dv sanity and overflow guard (every tensor stays below 2^46 bytes)
int check_shape(const kda_shape_t* sh) {
  if (!sh) return KDA_ERR_NULL;
  if (sh->B < 1 || sh->H < 1 || sh->T < 0 || sh->dk < 1 || sh->dv < 1) return KDA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 44;
  if (sh->B > lim || sh->H > lim || sh->T > lim || sh->dk > 4096 || sh->dv > 4096) return KDA_ERR_SHAPE;
  const double elems = (double)sh->B * (double)sh->H * (double)sh->T * (double)(sh->dk > sh->dv ? sh->dk : sh->dv);
  if (elems * 4.0 > (double)((int64_t)1 << 46)) return KDA_ERR_SHAPE;
  if ((double)sh->B * sh->H * ((sh->T + 15) / 16) >= 4294967295.0) return KDA_ERR_SHAPE;  // 32-bit chunk counters
  if (sh->dtype != KDA_DTYPE_F32 && sh->dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
  if (sh->reserved != 0) return KDA_ERR_ARG;
  auto ok_dim = [](int64_t d) { return d == 32 || d == 64 || d == 128; };
  if (!ok_dim(sh->dk) || !ok_dim(sh->dv)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

int check_gmin(float g_min) {
  if (std::isnan(g_min)) return KDA_ERR_ARG;
  if (g_min > 0.f) return KDA_ERR_ARG;
  if (std::isinf(g_min) && g_min > 0.f) return KDA_ERR_ARG;
  return KDA_OK;
}

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64; }

int pick_path(const kda_shape_t* sh, int chunk, const kda_opts_t* opts) { return kda::forward_path(sh, chunk, opts); }

// the matrix-core paths' ids are their modes (kModeFused, kModeCorr)
static_assert(kda::kModeFused == 3 && kda::kModeCorr == 4, "path ids are the modes");

size_t workspace_for(const kda_shape_t* sh, int path, int64_t seg_steps) {
  if (path < kda::kModeFused) return 0;
  return kda::mfma_workspace_bytes(sh->B, sh->H, sh->T, sh->dk, sh->dv, path, seg_steps);
}

}  // namespace

namespace kda {

// path actually taken for a valid shape: 1 vector, 3 fused, 4 corrected (the automatic choice on the
// matrix cores); -1 for an unsupported request.  The matrix-core kernels index tokens in 32 bits, so
// sequences of 2^30 tokens and more take the vector path (their inputs would not fit in HBM anyway).
int forward_path(const kda_shape_t* sh, int chunk, const kda_opts_t* opts) {
  const int req = opts ? opts->path : 0;
  const bool mfma = sh->dtype == KDA_DTYPE_BF16 && sh->dk == 128 && sh->dv == 128 && chunk == kChunk &&
                    fused_supported(sh->dtype, sh->dk, sh->dv, sh->T);
  if (req == 1) return 1;
  if (req == kModeFused || req == kModeCorr) return mfma ? req : -1;
  if (req != 0) return -1;
  return mfma ? kModeCorr : 1;
}

int record_hip_error(hipError_t e) {
  std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d)", hipGetErrorString(e), (int)e);
  return KDA_ERR_HIP;
}

int record_error_text(const char* text) {
  std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", text);
  return KDA_ERR_HIP;
}

}  // namespace kda

extern "C" {

const char* kda_strerror(int code) {
  switch (code) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid shape (B, H >= 1, T >= 0, dk, dv >= 1, sizes must not overflow)";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (chunk 16, 32 or 64, and 16 on the matrix-core paths; dk, dv in {32, 64, 128}; dtype f32 or bf16; path)";
    case KDA_ERR_ARG: return "invalid argument (g_min NaN or > 0, misaligned pointer, overlapping buffers, workspace too small, reserved field set)";
    case KDA_ERR_HIP: return "HIP runtime error (see kda_last_hip_error)";
    case KDA_ERR_SCRATCH: return "the call needs more scratch than the static array of kda_chunk_fwd_noalloc holds (KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
    default: return "unknown error code";
  }
}

const char* kda_last_hip_error(void) { return g_last_hip_error; }

int kda_version(void) { return KDA_VERSION; }

size_t kda_workspace_bytes(const kda_shape_t* shape, int chunk) {
  return kda_workspace_bytes_ex(shape, chunk, nullptr);
}

size_t kda_workspace_bytes_ex(const kda_shape_t* shape, int chunk, const kda_opts_t* opts) {
  if (check_shape(shape) != KDA_OK || !chunk_ok(chunk)) return (size_t)-1;
  if (opts && (opts->path < 0 || opts->path > 4)) return (size_t)-1;
  const int path = pick_path(shape, chunk, opts);
  if (path < 0) return (size_t)-1;
  const int64_t seg_steps = opts ? opts->seg_steps : 0;
  if (path >= kda::kModeFused && !kda::mfma_seg_steps_ok(shape->T, seg_steps)) return (size_t)-1;
  return workspace_for(shape, path, seg_steps);
}

int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* w, const void* beta,
                     const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                     void* o, float* S_final, void* workspace, size_t workspace_bytes,
                     kda_stats_t* stats, void* stream, const kda_opts_t* opts) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
  if ((rc = check_gmin(g_min)) != KDA_OK) return rc;
  if (opts) {
    if (opts->seg_steps < 0) return KDA_ERR_ARG;
    if (opts->disable_fallback && opts->force_fallback) return KDA_ERR_ARG;
    if (opts->force_fallback < 0 || opts->force_fallback > 2) return KDA_ERR_ARG;
    if (opts->path < 0 || opts->path > 4) return KDA_ERR_UNSUPPORTED;
  }
  const int64_t B = shape->B, H = shape->H, T = shape->T, dk = shape->dk, dv = shape->dv;
  const int64_t esz = shape->dtype == KDA_DTYPE_BF16 ? 2 : 4;
  if (!S_final) return KDA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !w || !beta || !o)) return KDA_ERR_NULL;

  const void* ptrs[] = {q, k, v, w, beta, S0, o, S_final, workspace, stats};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ARG;

  // overlap rules: outputs (o, S_final, workspace, stats) must not touch inputs or each other,
  // except S_final == S0 exactly
  const int64_t BH = B * H;
  const Range r_q = range_of(q, T > 0 ? BH * T * dk * esz : 0);
  const Range r_k = range_of(k, T > 0 ? BH * T * dk * esz : 0);
  const Range r_v = range_of(v, T > 0 ? BH * T * dv * esz : 0);
  const Range r_w = range_of(w, T > 0 ? BH * T * dk * esz : 0);
  const Range r_b = range_of(beta, T > 0 ? BH * T * esz : 0);
  const Range r_s0 = range_of(S0, S0 ? BH * dk * dv * 4 : 0);
  const Range r_o = range_of(o, T > 0 ? BH * T * dv * esz : 0);
  const Range r_sf = range_of(S_final, BH * dk * dv * 4);
  const Range r_ws = range_of(workspace, workspace ? (int64_t)workspace_bytes : 0);
  const Range r_st = range_of(stats, stats ? (int64_t)sizeof(kda_stats_t) : 0);
  const Range ins[] = {r_q, r_k, r_v, r_w, r_b};
  const Range outs[] = {r_o, r_sf, r_ws, r_st};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return KDA_ERR_ARG;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_ARG;
  if (S0 && S0 != S_final && overlap(r_s0, r_sf)) return KDA_ERR_ARG;
  if (overlap(r_s0, r_o) || overlap(r_s0, r_ws) || overlap(r_s0, r_st)) return KDA_ERR_ARG;

  kda::Params p{};
  p.q = q; p.k = k; p.v = v; p.w = w; p.beta = beta; p.S0 = S0;
  p.unbounded = std::isinf(g_min) ? 1 : 0;
  p.g_min = p.unbounded ? 0.f : g_min;
  p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv; p.dtype = shape->dtype;
  p.o = o; p.S_final = S_final; p.workspace = workspace; p.workspace_bytes = workspace_bytes;
  p.stats = stats;
  p.disable_fallback = opts ? opts->disable_fallback : 0;
  p.force_fallback = opts ? opts->force_fallback : 0;
  p.seg_steps = opts ? opts->seg_steps : 0;
  p.chunk = chunk;

  const int path = T > 0 ? pick_path(shape, chunk, opts) : 1;
  if (path < 0) return KDA_ERR_UNSUPPORTED;
  if (path >= kda::kModeFused && !kda::mfma_seg_steps_ok(T, p.seg_steps)) return KDA_ERR_ARG;
  const size_t need_ws = workspace_for(shape, path, p.seg_steps);
  if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) return KDA_ERR_ARG;
#if KDA_PHASE_STAMPS
  // phase-stamp build: the segment pass's workgroup KDA_STAMP_BLOCK stamps into the workspace's last
  // kStampBytes, which the matrix-core paths' workspace size includes in this build
  {
    const char* sb = std::getenv("KDA_STAMP_BLOCK");
    const bool room = path >= kda::kModeFused && workspace && workspace_bytes >= (size_t)kda::kStampBytes;
    p.stamp_off = room ? (int64_t)workspace_bytes - kda::kStampBytes : -1;
    p.stamp_block = (room && sb) ? std::atoi(sb) : -1;
    p.stamp_kernel = 0;
  }
#endif

  // ---- launches (first HIP call of the entry point)
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t ev0 = opts ? reinterpret_cast<hipEvent_t>(opts->ev_begin) : nullptr;
  hipEvent_t ev1 = opts ? reinterpret_cast<hipEvent_t>(opts->ev_end) : nullptr;
  hipError_t e;
  // statistics reset here for the vector path and T = 0; the matrix-core paths do it themselves
  if (stats && (T == 0 || path < kda::kModeFused) && (e = kda::launch_stats_init(stats, s)) != hipSuccess) return hip_fail(e);
  if (T == 0) {
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return hip_fail(e);
    if ((e = kda::launch_state_copy(p, s)) != hipSuccess) return hip_fail(e);
    if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return hip_fail(e);
    return KDA_OK;
  }
  if (path >= kda::kModeFused) {
    if ((e = kda::launch_mfma(p, s, ev0, ev1, path)) != hipSuccess) return hip_fail(e);
  } else {
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return hip_fail(e);
    if ((e = kda::launch_vec(p, s)) != hipSuccess) return hip_fail(e);
    if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return hip_fail(e);
  }
  return KDA_OK;
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* w, const void* beta,
                  const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                  void* o, float* S_final, void* workspace, size_t workspace_bytes,
                  kda_stats_t* stats, void* stream) {
  return kda_chunk_fwd_ex(q, k, v, w, beta, S0, g_min, chunk, shape, o, S_final, workspace,
                          workspace_bytes, stats, stream, nullptr);
}

int kda_decode(const void* q, const void* k, const void* v, const void* w, const void* beta,
               float* S, float g_min, const kda_shape_t* shape, void* o, void* stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if ((rc = check_gmin(g_min)) != KDA_OK) return rc;
  const int64_t B = shape->B, H = shape->H, T = shape->T, dk = shape->dk, dv = shape->dv;
  const int64_t esz = shape->dtype == KDA_DTYPE_BF16 ? 2 : 4;
  if (!S) return KDA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !w || !beta || !o)) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, w, beta, S, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ARG;
  const int64_t BH = B * H;
  const Range r_s = range_of(S, BH * dk * dv * 4);
  const Range r_o = range_of(o, T > 0 ? BH * T * dv * esz : 0);
  const Range ins[] = {range_of(q, T > 0 ? BH * T * dk * esz : 0), range_of(k, T > 0 ? BH * T * dk * esz : 0),
                       range_of(v, T > 0 ? BH * T * dv * esz : 0), range_of(w, T > 0 ? BH * T * dk * esz : 0),
                       range_of(beta, T > 0 ? BH * T * esz : 0)};
  for (const Range& a : ins)
    if (overlap(a, r_s) || overlap(a, r_o)) return KDA_ERR_ARG;
  if (overlap(r_s, r_o)) return KDA_ERR_ARG;
  if (T == 0) return KDA_OK;
  kda::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.w = w; p.beta = beta; p.S = S; p.o = o;
  p.unbounded = std::isinf(g_min) ? 1 : 0;
  p.g_min = p.unbounded ? 0.f : g_min;
  p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv; p.dtype = shape->dtype;
  hipError_t e = kda::launch_decode(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e);
}

size_t kda_bwd_workspace_bytes(const kda_shape_t* shape, int chunk) {
  if (check_shape(shape) != KDA_OK || chunk != kda::kChunk) return (size_t)-1;
  return kda::bwd_workspace_bytes(shape->B, shape->H, shape->T, shape->dk, shape->dv);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* w, const void* beta,
                  const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                  const void* dO, const float* dS_final, float* dq, float* dk, float* dv, float* dw,
                  float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (chunk != kda::kChunk) return KDA_ERR_UNSUPPORTED;
  if ((rc = check_gmin(g_min)) != KDA_OK) return rc;
  const int64_t B = shape->B, H = shape->H, T = shape->T, dkk = shape->dk, dvv = shape->dv;
  const int64_t esz = shape->dtype == KDA_DTYPE_BF16 ? 2 : 4;
  if (T > 0 && (!q || !k || !v || !w || !beta || !dO || !dq || !dk || !dv || !dw || !dbeta)) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, w, beta, S0, dO, dS_final, dq, dk, dv, dw, dbeta, dS0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ARG;
  const int64_t BH = B * H;
  const size_t need_ws = kda::bwd_workspace_bytes(B, H, T, dkk, dvv);
  if (T > 0 && (!workspace || workspace_bytes < need_ws)) return KDA_ERR_ARG;
  const Range ins[] = {range_of(q, T > 0 ? BH * T * dkk * esz : 0), range_of(k, T > 0 ? BH * T * dkk * esz : 0),
                       range_of(v, T > 0 ? BH * T * dvv * esz : 0), range_of(w, T > 0 ? BH * T * dkk * esz : 0),
                       range_of(beta, T > 0 ? BH * T * esz : 0), range_of(S0, S0 ? BH * dkk * dvv * 4 : 0),
                       range_of(dO, T > 0 ? BH * T * dvv * esz : 0),
                       range_of(dS_final, dS_final ? BH * dkk * dvv * 4 : 0)};
  const Range outs[] = {range_of(dq, T > 0 ? BH * T * dkk * 4 : 0), range_of(dk, T > 0 ? BH * T * dkk * 4 : 0),
                        range_of(dv, T > 0 ? BH * T * dvv * 4 : 0), range_of(dw, T > 0 ? BH * T * dkk * 4 : 0),
                        range_of(dbeta, T > 0 ? BH * T * 4 : 0), range_of(dS0, dS0 ? BH * dkk * dvv * 4 : 0),
                        range_of(workspace, T > 0 ? (int64_t)need_ws : 0)};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return KDA_ERR_ARG;
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i)
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (T == 0) {   // no tokens: dS0 = dS_final
    if (dS0) {
      kda::Params cp{};
      cp.S0 = dS_final; cp.S_final = dS0; cp.B = B; cp.H = H; cp.dk = dkk; cp.dv = dvv;
      if ((e = kda::launch_state_copy(cp, s)) != hipSuccess) return hip_fail(e);
    }
    return KDA_OK;
  }
  kda::BwdParams b{};
  kda::Params& p = b.p;
  p.q = q; p.k = k; p.v = v; p.w = w; p.beta = beta; p.S0 = S0;
  p.unbounded = std::isinf(g_min) ? 1 : 0;
  p.g_min = p.unbounded ? 0.f : g_min;
  p.B = B; p.H = H; p.T = T; p.dk = dkk; p.dv = dvv; p.dtype = shape->dtype;
  p.workspace = workspace; p.workspace_bytes = workspace_bytes;
  b.dO = dO; b.dSf = dS_final; b.dq = dq; b.dk = dk; b.dv = dv; b.dw = dw; b.dbeta = dbeta; b.dS0 = dS0;
  if ((e = kda::launch_bwd(b, s)) != hipSuccess) return hip_fail(e);
  return KDA_OK;
}

int kda_gate_prefix(const void* w, float g_min, int chunk, const kda_shape_t* shape,
                    float* g, float* G, float* span, uint8_t* flags, void* stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  if ((rc = check_gmin(g_min)) != KDA_OK) return rc;
  const int64_t B = shape->B, H = shape->H, T = shape->T, dk = shape->dk;
  if (T > 0 && !w) return KDA_ERR_NULL;
  const void* ptrs[] = {w, g, G, span, flags};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ARG;
  const int64_t esz = shape->dtype == KDA_DTYPE_BF16 ? 2 : 4;
  const int64_t NC = (T + chunk - 1) / chunk;
  const Range r_w = range_of(w, B * H * T * dk * esz);
  const Range outs[] = {range_of(g, g ? B * H * T * dk * 4 : 0), range_of(G, G ? B * H * T * dk * 4 : 0),
                        range_of(span, span ? B * H * NC * 4 : 0), range_of(flags, flags ? B * H * NC : 0)};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], r_w)) return KDA_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_ARG;
  }
  const int unbounded = std::isinf(g_min) ? 1 : 0;
  hipError_t e = kda::launch_gate_prefix(w, unbounded ? 0.f : g_min, unbounded, B, H, T, dk, shape->dtype, chunk,
                                         g, G, span, flags, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : hip_fail(e);
}

}  // extern "C"

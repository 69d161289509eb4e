/*
 * kda.h -- C ABI of libkda.so: the chunk-parallel forward pass of Kimi Delta
 * Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * The operation (per batch b and head h, independently):
 *
 *   state S (dk x dv, fp32), starting at S0 (zeros when S0 is NULL);
 *   for every token t:
 *     g_t = g_min * sigmoid(w_t)          bounded log-decay, one value per key channel
 *           or -softplus(w_t)             the unbounded form, when g_min = -INFINITY
 *     S   = Diag(exp(g_t)) S              forget
 *     u_t = beta_t (v_t - S^T k_t)        delta-rule correction
 *     S   = S + k_t u_t^T                 write
 *     o_t = S^T q_t                       read (inclusive of token t)
 *   S_final = S.
 *
 * Sources.  "From Numerical Stability to Load Balancing: A Technical Breakdown
 * of LLM Architecture Innovations", section 2.1: a fixed-shape state, decayed
 * per step and written with key/value outer products; chunked evaluation with
 * a serial recurrence between chunks and matrix products inside a chunk; the
 * in-chunk scaling between positions i >= j is exp(G_i - G_j) with G the
 * cumulative log-decay.  Section 2.2 of the same page, section 2.2 of
 * "Architecting Long-Context LLMs ..." and of "Architecture Analysis of
 * Ultra-Long Context Sparse MoE Models", and Breakthrough 1 part 2 of
 * "Demystifying Trillion-Parameter MoE Models ...": the bounded gate
 * g = g_min * sigmoid(w) with g_min = -5 keeps a 16-token chunk's span at or
 * above -80, so its reciprocal scaling exp(80) stays finite and the diagonal
 * tile runs as a dense matrix product.  The delta rule itself is only named on
 * the pages (Delta networks / Delta Net-like / delta-rule-based models); the
 * form above is the plainest reading with per-key-channel decay.
 *
 * Evaluation.  Chunks of 16 tokens (32 or 64 on request).  Inside a chunk the library uses the
 * exp(+-G) reciprocal form (dense tiles) when the chunk's span, the minimum
 * over key channels of the chunk-local sum of g, is at or above -80; a chunk
 * whose span falls below -80 (possible only with the unbounded gate or
 * g_min < -5) is detected and evaluated with per-position-pair decay factors
 * exp(G_r - G_j) instead (the per-position path the pages describe as the
 * fallback implementations are forced into).
 *
 * Layouts.  All tensors are dense row-major with no padding:
 *   q, k, w : [B, H, T, dk]      dtype = shape->dtype
 *   v, o    : [B, H, T, dv]      dtype = shape->dtype
 *   beta    : [B, H, T]          dtype = shape->dtype
 *   S0, S_final : [B, H, dk, dv] always fp32
 * bf16 means IEEE-754 binary32 truncated to its upper 16 bits; o is rounded to
 * nearest-even.  The library applies no scaling or normalisation to q or k.
 *
 * Ownership and memory.  Every pointer argument (except `shape`, `opts` and
 * the returned strings) is a DEVICE pointer on the current HIP device, owned
 * by the caller and aligned to 16 bytes.  The library allocates nothing on
 * these entry points: any scratch memory comes in through `workspace`.
 * Outputs must not overlap inputs or each other, except that S_final may be
 * exactly S0 (in-place state update).
 *
 * Errors.  Arguments are validated on the host before any HIP call; an invalid
 * call returns a negative code and launches nothing.  Launches are
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream):
 * faults inside kernels surface at the caller's next synchronisation.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 110 /* 1.1.0: path 2 retired */

#if defined(__GNUC__) || defined(__clang__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

typedef enum {
  KDA_DTYPE_F32 = 0,  /* inputs and o in fp32; arithmetic in fp32 */
  KDA_DTYPE_BF16 = 1  /* inputs and o in bf16; bf16 matrix-core operands, fp32 accumulation and state */
} kda_dtype_t;

typedef struct {
  int64_t B, H, T, dk, dv; /* B, H >= 1; T >= 0; dk, dv in {32, 64, 128} */
  int32_t dtype;           /* a kda_dtype_t */
  int32_t reserved;        /* must be 0 */
} kda_shape_t;

/* Device-resident counters, written with atomics by the kernels of one call.
 * The library resets them at the start of the call (stream-ordered).           */
typedef struct {
  uint32_t n_chunks;     /* B * H * ceil(T / chunk) */
  uint32_t n_flagged;    /* chunks whose span fell below -80 (detected, whatever path ran) */
  uint32_t n_nonfinite;  /* non-finite values written to o or S_final */
  float min_span;        /* minimum chunk span seen; +INFINITY when T = 0 */
} kda_stats_t;

/* Measurement knobs for kda_chunk_fwd_ex. Zero-initialised means "default". */
typedef struct {
  int32_t disable_fallback; /* 1: flagged chunks still take the dense exp(+-G) path (shows the overflow) */
  int32_t force_fallback;   /* 1: every chunk takes the handling of a flagged chunk (measures its cost):
                               on the fused and corrected paths the tiles referenced to the chunk's token 7 where both
                               8-token halves span at least -80, per-position factors otherwise; on the
                               other paths per-position factors.  2: every chunk takes the per-position
                               factors.  Other values are KDA_ERR_ARG. */
  int32_t path;             /* 0 auto (bf16 with dk = dv = 128 and T < 2^30: the corrected matrix-core
                               path; anything else: the vector path),
                               1 the plain fp32 vector path, 3 the fused matrix-core path (a pass that
                               maps every segment, the chaining of the maps, a pass that writes the
                               outputs from the chained entering states), 4 the corrected
                               matrix-core path (one pass over every segment: segment 0 from S0,
                               the others from a zero entering state with the coefficient Qtil of
                               their outputs on the entering state and their maps; the chaining; an
                               HBM-bound pass adding Qtil S_start to the outputs of segments >= 1).
                               2 (a retired path) and values above 4 are KDA_ERR_UNSUPPORTED, and so
                               are 3 and 4 where the matrix-core paths do not apply.  The automatic
                               segment plan of paths 3 and 4 has at most 32 segments per sequence,
                               more only where a segment would otherwise reach 2^18 steps */
  int32_t seg_steps;        /* matrix-core path: steps of 32 tokens per sequence segment (0 = automatic;
                               < 0, 2^18 or more, or more than 32 segments per sequence, is
                               KDA_ERR_ARG) */
  void* ev_begin;           /* optional hipEvent_t recorded on `stream` before the call's first kernel */
  void* ev_end;             /* optional hipEvent_t recorded on `stream` after the call's last kernel */
} kda_opts_t;

enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = -2,       /* B, H < 1, T < 0, dk or dv < 1, or sizes overflow */
  KDA_ERR_UNSUPPORTED = -3, /* chunk not in {16, 32, 64} (16 on the matrix-core paths), dk or dv not in
                               {32, 64, 128}, unknown dtype or path */
  KDA_ERR_ARG = -4,         /* g_min NaN or > 0, misaligned pointer, forbidden overlap,
                               workspace too small, non-zero reserved field, both opts set,
                               bad seg_steps */
  KDA_ERR_HIP = -5,         /* a HIP call failed; kda_last_hip_error() has the text */
  KDA_ERR_SCRATCH = -6      /* kda_chunk_fwd_noalloc: the call needs more than KDA_NOALLOC_SCRATCH_BYTES */
};

/* Forward pass.  Computes o and S_final as defined above.
 *   g_min   finite and <= 0 selects g = g_min * sigmoid(w); -INFINITY selects
 *           g = -softplus(w).  NaN or > 0 is KDA_ERR_ARG.
 *   chunk   tokens per chunk: 16 (the tile the pages fix for g_min = -5), or 32 or 64 (the
 *           chunk-size and lower-bound co-design of "From Numerical Stability to Load Balancing ..."
 *           section 2.3; evaluated on the fp32 vector path, where each chunk takes the reciprocal
 *           exp(+-G) tiles when its span is at or above -80 and per-pair factors otherwise).  The
 *           matrix-core paths (opts->path 3, 4) take 16 only.
 *   S0      may be NULL (zero initial state).
 *   workspace / workspace_bytes: device scratch of at least
 *           kda_workspace_bytes(shape, chunk) bytes (kda_workspace_bytes_ex with the same
 *           opts for kda_chunk_fwd_ex); may be NULL when that is 0.
 *   stats   optional device pointer (NULL: no statistics).
 *   stream  hipStream_t to launch on.
 * When T = 0, o is not touched and S_final receives S0 (or zeros).         */
KDA_API int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* w, const void* beta,
                  const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                  void* o, float* S_final, void* workspace, size_t workspace_bytes,
                  kda_stats_t* stats, void* stream);

/* Same as kda_chunk_fwd, with measurement options (opts may be NULL). */
KDA_API int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* w, const void* beta,
                     const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                     void* o, float* S_final, void* workspace, size_t workspace_bytes,
                     kda_stats_t* stats, void* stream, const kda_opts_t* opts);

/* Size of the static device array kda_chunk_fwd_noalloc takes its scratch from: 64 MiB per GPU the
 * library runs on, held from the first call on that GPU until the process ends.  It holds the fused
 * path's segment plan (which the entry point takes where the automatic path is the corrected one) of
 * up to 341 (b, h, segment) triples of 192 KiB: the plan holds at most 256 + B*H of them below 129
 * heads (e.g. 16 heads: 17 segments each at any length), so every B*H up to 113 fits; it keeps none
 * (and any shape is accepted) where it has one segment per sequence (B*H >= 129, or short sequences)
 * or takes the vector path; 114 to 128 heads fit only where short sequences limit the segments. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* Forward pass that allocates nothing, for callers that cannot allocate device memory at call time
 * (code under stream capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, validation and asynchrony as kda_chunk_fwd without workspace and
 * workspace_bytes.  Where kda_chunk_fwd would take the corrected matrix-core path, this entry point
 * takes the fused one (opts->path = 3), whose scratch is 64 KiB blocks per segment, not 8 KiB per 32
 * tokens: its results agree with kda_chunk_fwd's to the rounding of the two plans and equal, bit for
 * bit, those of kda_chunk_fwd_ex with that path.  The scratch (kda_workspace_bytes_ex for that plan)
 * is taken from a static device array of the library (KDA_NOALLOC_SCRATCH_BYTES, one per GPU, looked
 * up on the first call on each GPU with that GPU current).  Returns KDA_ERR_SCRATCH, launching nothing, when the call needs
 * more than that; every other error as kda_chunk_fwd.  No hipMalloc or hipFree, no allocating
 * library routine.  All calls on one GPU share its array: calls that overlap in time on one GPU
 * (concurrent streams, or several host threads) race on it and must be serialised by the caller;
 * calls queued one after another on one stream are safe. */
KDA_API int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* w, const void* beta,
                                  const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                                  void* o, float* S_final, kda_stats_t* stats, void* stream);

/* Recurrent decode: advance a resident state by shape->T tokens (typically 1), token by
 * token, in place.  The per-token form of the same gated delta rule ("From Numerical
 * Stability to Load Balancing ..." section 2.1; the gates of section 2.2), the reuse of the
 * trained operator's state at inference:
 *   S <- Diag(e^{g_t}) S;  u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T;  o_t = S^T q_t
 * Arguments: q, k, w [B,H,T,dk]; v, o [B,H,T,dv]; beta [B,H,T] (all shape->dtype, device);
 *   S [B,H,dk,dv] fp32, device, read and overwritten (the caller owns it; it must not overlap
 *   any other argument); g_min as for kda_chunk_fwd; dk, dv in {32, 64, 128}.
 * No workspace, no statistics (no chunking, hence no reciprocal factors and nothing to flag).
 * Same validation and error codes as kda_chunk_fwd (T = 0 launches nothing); asynchronous on
 * stream. */
KDA_API int kda_decode(const void* q, const void* k, const void* v, const void* w, const void* beta,
                       float* S, float g_min, const kda_shape_t* shape, void* o, void* stream);

/* Backward pass of the chunked forward: gradients of a loss L given dL/do and dL/dS_final.
 * The reverse mode of the 16-token chunk form ("From Numerical Stability to Load Balancing ..."
 * section 2.1), all in fp32: a chunk-parallel pass writes each chunk's WY record, two sequential
 * passes walk the chunk-to-chunk state forwards (entering states) and backwards (leaving adjoints),
 * and a chunk-parallel pass forms every gradient.  In-chunk pair terms use factors exp(+-(G - Gam/2))
 * when every channel's span is >= -80 and pair-by-pair factors exp(G_r - G_j) <= 1 otherwise, so
 * no input overflows.
 * Arguments: the forward's q, k, v, w, beta, S0 (nullable), g_min, chunk (16) and shape (dk in
 *   {32, 64, 128}, dv in {32, 64, 128});
 *   dO [B,H,T,dv] in shape->dtype; dS_final [B,H,dk,dv] fp32 or NULL (zero);
 *   outputs, fp32, device: dq, dk, dw [B,H,T,dk]; dv [B,H,T,dv]; dbeta [B,H,T];
 *   dS0 [B,H,dk,dv] or NULL (not wanted);
 *   workspace of at least kda_bwd_workspace_bytes(shape, chunk) bytes.
 * Outputs must not overlap inputs or each other.  Same validation and error codes as
 * kda_chunk_fwd; asynchronous on stream. */
KDA_API int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* w, const void* beta,
                          const float* S0, float g_min, int chunk, const kda_shape_t* shape,
                          const void* dO, const float* dS_final, float* dq, float* dk, float* dv, float* dw,
                          float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, void* stream);

/* Scratch bytes kda_chunk_bwd needs: per 16-token chunk its record (3*16*dk + 2*16*dv + dk floats),
 * entering state and leaving adjoint (dk*dv floats each), all fp32:
 * B*H*ceil(T/16)*(3*16*dk + 2*16*dv + dk + 2*dk*dv)*4.  (size_t)-1 for an invalid shape or chunk.
 * Host-only. */
KDA_API size_t kda_bwd_workspace_bytes(const kda_shape_t* shape, int chunk);

/* Gate and in-chunk prefix stage on its own (for checking that stage, and for the chunk-size
 * co-design sweep: chunk may be 16, 32 or 64 here; kda_chunk_fwd evaluates 16-token chunks).
 * Outputs (device, fp32 unless noted):
 *   g     [B,H,T,dk]   the per-step log-decay
 *   G     [B,H,T,dk]   inclusive prefix of g, restarted at every chunk
 *   span  [B,H,NC]     min over key channels of the chunk's total (NC = ceil(T/chunk))
 *   flags [B,H,NC]     uint8: 1 when span < -80 (the chunk's reciprocal factor e^{-G} could pass
 *                      e^{80}: "Demystifying ..." Breakthrough 1 part 2, whatever the chunk size)
 * Any output pointer may be NULL to skip it.  Same validation and error codes. */
KDA_API int kda_gate_prefix(const void* w, float g_min, int chunk, const kda_shape_t* shape,
                    float* g, float* G, float* span, uint8_t* flags, void* stream);

/* Scratch bytes kda_chunk_fwd needs for this shape (0 means none): three 64 KiB
 * blocks (a segment's map X and M, and its entering state) per sequence segment
 * of the plan the call takes (the automatic plan here, up to 32 segments per
 * (b, h) unless a segment would reach 2^18 steps of 32 tokens; nothing when the
 * plan has one segment); on the corrected path (the automatic one at bf16,
 * dk = dv = 128), also the propagated queries, 8 KiB per 32 tokens per (b, h).
 * Returns (size_t)-1 for an invalid shape, chunk or path.
 * Host-only, no HIP call.                                                    */
KDA_API size_t kda_workspace_bytes(const kda_shape_t* shape, int chunk);

/* Same for kda_chunk_fwd_ex with these options (opts may be NULL: the automatic path and plan;
 * opts->seg_steps fixes the segment length, and a length giving more than 32 segments per (b, h)
 * returns (size_t)-1). */
KDA_API size_t kda_workspace_bytes_ex(const kda_shape_t* shape, int chunk, const kda_opts_t* opts);

/* Static description of an error code. Host-only. */
KDA_API const char* kda_strerror(int code);

/* Text of the last HIP error seen by this thread ("" if none). Host-only. */
KDA_API const char* kda_last_hip_error(void);

/* KDA_VERSION of the loaded library. Host-only. */
KDA_API int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */

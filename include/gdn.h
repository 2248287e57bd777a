/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet library, CPR schedule.
 *
 * The layer is Gated DeltaNet, named in the IsoExec write-up on agentlenshq.com
 * (section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet"), whose pages
 * do not write its equations.  The definition implemented is the gated delta
 * rule in the form in which the problem this library solves is stated, per
 * sequence and value head h, with S a d_v x d_k fp32 matrix:
 *
 *     alpha_t = exp(g_t)
 *     S_t     = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t     = S_t q_t
 *
 * where q_t, k_t are the query/key head h / (H_v / H_qk) vectors, normalised
 * to unit length (x / sqrt(sum x^2 + 1e-6)) when qk_l2norm is set, and q is
 * then multiplied by `scale`.
 *
 * CPR ("chunkwise-parallel recurrent": the same section of the write-up, and
 * the daily.dev digest's Q&A on CPR) keeps the token recurrence as the main
 * computation, evaluated in parallel across C-token chunks, and has decode
 * resynchronise its state every C tokens.  This library's reading:
 *   - every chunk-start state comes from the chunk (WY) form of the
 *     recurrence, scanned sequentially over the chunks of a sequence;
 *   - every output o_t, and the state inside a chunk, comes from the token
 *     recurrence started from that chunk's start state;
 *   - decode runs the same token step and, after the C-th token of a chunk,
 *     replaces its running state by the chunk form applied to the chunk-start
 *     state and the chunk's buffered tokens.
 * Chunks are counted from each sequence's first token.  Because all three
 * entry points run the same device code on the same values, prefill, decode
 * and the trainer forward give bit-identical o and final states, for any
 * batch composition, run after run.
 *
 * Conventions for every call
 *   - All tensors are dense, row-major, on the current HIP device, and start
 *     at 16-byte aligned addresses (else GDN_ERR_INVALID_ARG); the caller
 *     owns every buffer.  The library never allocates or frees device memory
 *     in these calls; scratch comes from `ws`, sized by gdn_workspace_bytes.
 *   - Packed layouts: q, k [T, H_qk, d_k]; v [T, H_v, d_v] in in_dtype;
 *     beta, g [T, H_v] fp32; o [T, H_v, d_v] fp32.  States are fp32
 *     [N, H_v, d_k, d_v] with d_v fastest, i.e. the transpose of S.
 *   - cu_seqlens [N+1] int32: sequence n is tokens [cu[n], cu[n+1]).  It must
 *     start at 0 and be non-decreasing.  Calls take a device copy (read by the
 *     kernels) and a host copy (validated and used to size the launches); both
 *     must hold the same values.  Kernels clamp every index to the buffers'
 *     extents, so a mismatch gives wrong values but no out-of-bounds access.
 *     The host copy may be NULL: the call then first copies the device copy
 *     to the host on `stream` and waits for it (the library's only host
 *     synchronisation; a call made so cannot be captured in a graph).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without waiting.
 *   - Every argument is validated on the host before any launch; on a
 *     validation error nothing is enqueued and nothing is written.  Shapes
 *     outside the compiled claims return GDN_ERR_UNSUPPORTED -- they are never
 *     run through a different arithmetic.
 *   - Supported: d_k == d_v == 128 with C == 64, or d_k == d_v == 16 with
 *     C == 16; H_v a multiple of H_qk with at most 8 value heads per q/k
 *     head; in_dtype fp32 or bf16.
 *   - Calls that overlap on the same workspace or cache race; calls on
 *     separate buffers may run concurrently.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = -1, /* NULL pointer, bad cu_seqlens, negative size, ... */
  GDN_ERR_UNSUPPORTED = -2, /* shape outside the compiled claims              */
  GDN_ERR_WORKSPACE = -3,   /* ws NULL or smaller than gdn_workspace_bytes     */
  GDN_ERR_HIP = -4          /* a HIP runtime call failed                       */
} gdn_status_t;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

typedef enum {
  GDN_OP_PREFILL = 0,
  GDN_OP_DECODE = 1,
  GDN_OP_FWD_BWD = 2,
  GDN_OP_PREFILL_CHUNKED = 3,
  GDN_OP_PREFILL_CONTINUE = 4
} gdn_op_t;

/* Problem shape.  beta, g, states, o and gradients are always fp32. */
typedef struct {
  int32_t H_qk;      /* query/key heads                                     */
  int32_t H_v;       /* value heads; value head h reads q/k head h/(H_v/H_qk) */
  int32_t d_k, d_v;  /* head dimensions                                     */
  int32_t C;         /* chunk length                                        */
  int32_t in_dtype;  /* gdn_dtype_t of q, k, v                              */
  int32_t qk_l2norm; /* 1: normalise q and k in-kernel; 0: use as given     */
  float scale;       /* multiplies the (normalised) query                   */
} gdn_shape_t;

/*
 * Decode cache of N sequences: the resumable state of token-by-token decode.
 * It is plain device memory owned by the caller: copying it out and back in
 * resumes decode bit-exactly.
 */
typedef struct {
  float* S_run;   /* [N, H_v, d_k, d_v] running state after the last token      */
  float* S_chunk; /* [N, H_v, d_k, d_v] state at the start of the current chunk */
  float* kbuf;    /* [N, C, H_qk, d_k] normalised keys of the current chunk     */
  void* vbuf;     /* [N, C, H_v, d_v] values of the current chunk, in_dtype     */
  float* bbuf;    /* [N, C, H_v] beta of the current chunk                      */
  float* gbuf;    /* [N, C, H_v] g of the current chunk                         */
  int32_t* pos;   /* [N, H_v] tokens of the current chunk absorbed, 0..C-1     */
} gdn_cache_t;

/* Bytes of workspace `op` needs for n_seqs sequences of total_tokens tokens
 * (decode: total_tokens is ignored).  0 for an invalid or unsupported shape. */
size_t gdn_workspace_bytes(const gdn_shape_t* shape, int32_t n_seqs,
                           int64_t total_tokens, int32_t op);

/* Decode cache for n_seqs sequences with nothing decoded yet: S_run = S_chunk
 * = h0 (or zero when h0 is NULL), pos = 0.  h0 is [N, H_v, d_k, d_v] fp32. */
int gdn_cache_init(const gdn_shape_t* shape, int32_t n_seqs, const float* h0,
                   gdn_cache_t* cache, void* stream);

/*
 * Rollout prefill (case "engine_prefill" in the write-up's contract section).
 * h0 [N, H_v, d_k, d_v] nullable (zero).  Writes o; hT [N, H_v, d_k, d_v]
 * (nullable) receives each sequence's final state.  If `cache` is non-NULL it
 * is filled so that gdn_decode_step continues every sequence exactly where
 * this prefill stopped (each sequence's current chunk is its last, possibly
 * partial, chunk).
 */
int gdn_prefill(const gdn_shape_t* shape, int32_t n_seqs,
                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                const void* q, const void* k, const void* v, const float* beta,
                const float* g, const float* h0, float* o, float* hT,
                gdn_cache_t* cache, void* ws, size_t ws_bytes, void* stream);

/*
 * Rollout decode: one token for each of n_seqs sequences (case "engine
 * decode").  q, k [N, H_qk, d_k], v [N, H_v, d_v] in in_dtype; beta, g
 * [N, H_v] fp32; o [N, H_v, d_v] fp32.  Runs the token step on cache->S_run,
 * appends the token to the chunk buffers and, for every sequence whose chunk
 * is now complete, resynchronises S_run = S_chunk = chunk-form state and sets
 * pos to 0.  pos_host ([N, H_v] mirror of cache->pos, nullable) only lets the
 * host skip the resync launch when no sequence completes a chunk; with NULL
 * the decision is taken on the device.  Out-of-range device pos values are
 * clamped into [0, C).
 */
int gdn_decode_step(const gdn_shape_t* shape, int32_t n_seqs, const void* q,
                    const void* k, const void* v, const float* beta,
                    const float* g, gdn_cache_t* cache, const int32_t* pos_host,
                    float* o, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the fixed device scratch of gdn_decode_step_noalloc, per GPU. */
#define GDN_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * gdn_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and the same bits as gdn_decode_step, without the workspace:
 * the resync's chunk factors go to a fixed device array of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The resync runs in groups of sequences whose
 * factors fit that array together (H_v * C * (2 d_k + 1) * 4 bytes per
 * sequence: 15 sequences at H_v = 32, d = 128, C = 64), so a batch larger
 * than one group costs two launches per extra group on the steps that
 * resync (every step when pos_host is NULL).  No hipMalloc, hipFree or other
 * allocating call is made.  GDN_ERR_WORKSPACE if a single sequence's factors
 * do not fit.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (e.g. on two streams) race and must not be issued; the
 * array keeps the last call's contents, which no call reads before writing.
 */
int gdn_decode_step_noalloc(const gdn_shape_t* shape, int32_t n_seqs, const void* q,
                            const void* k, const void* v, const float* beta,
                            const float* g, gdn_cache_t* cache,
                            const int32_t* pos_host, float* o, void* stream);

/*
 * Chunked-prefill continuation: n_seqs sequences whose decode cache stands
 * anywhere inside a chunk (cache->pos = p, the same for every head of a
 * sequence) take their next tokens q, k, v, beta, g (packed by cu_seqlens, as
 * in gdn_prefill) in one call.  The result is bit-identical to having run
 * the whole history and these tokens through one gdn_prefill, or token by
 * token through gdn_decode_step (chunk grid anchored at each sequence's
 * first token, as everywhere): the current chunk is prefilled again from
 * its start state cache->S_chunk, its p buffered tokens (cache->kbuf, vbuf,
 * bbuf, gbuf) followed by the new ones, and the outputs of the new tokens
 * only are written to o [T, H_v, d_v].  hT (nullable) receives each
 * sequence's final state; the cache is left where the sequence now stands.
 * pos_host [n_seqs] (host memory) must hold each sequence's cache->pos; it
 * sizes the launches (a value that disagrees with the device gives wrong
 * results for that sequence, never an access outside the buffers).
 * GDN_ERR_INVALID_ARG if some pos_host value is outside [0, C).  Workspace
 * from gdn_workspace_bytes(..., T, GDN_OP_PREFILL_CONTINUE); it covers the
 * up to n_seqs * (C - 1) buffered tokens.
 */
int gdn_prefill_continue(const gdn_shape_t* shape, int32_t n_seqs,
                         const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                         const int32_t* pos_host, const void* q, const void* k,
                         const void* v, const float* beta, const float* g,
                         gdn_cache_t* cache, float* o, float* hT, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Trainer forward + backward (case "trainer_fwd" and its gradient).  The
 * forward runs exactly the prefill launches, so o and hT are bit-identical to
 * gdn_prefill's.  dO [T, H_v, d_v] fp32; dhT [N, H_v, d_k, d_v] nullable
 * (zero).  Writes dq, dk [T, H_qk, d_k], dv [T, H_v, d_v], dbeta, dg [T, H_v],
 * dh0 [N, H_v, d_k, d_v], all fp32.  h0 nullable (zero).  The backward
 * recomputes nothing it can keep: chunk-start states and chunk factors of the
 * forward stay in `ws`.  No atomics: results are bitwise reproducible.
 */
int gdn_fwd_bwd(const gdn_shape_t* shape, int32_t n_seqs,
                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                const void* q, const void* k, const void* v, const float* beta,
                const float* g, const float* h0, const float* dO,
                const float* dhT, float* o, float* hT, float* dq, float* dk,
                float* dv, float* dbeta, float* dg, float* dh0, void* ws,
                size_t ws_bytes, void* stream);

/*
 * gdn_fwd_bwd with the input-shaped gradients dq, dk [T, H_qk, d_k] and dv
 * [T, H_v, d_v] written in grad_dtype: GDN_F32 (then identical to
 * gdn_fwd_bwd) or GDN_BF16, the fp32 result rounded to nearest even (the
 * trainer that keeps its parameters and activations in bf16).  dbeta, dg and
 * dh0 stay fp32.  GDN_ERR_INVALID_ARG for any other grad_dtype.
 */
int gdn_fwd_bwd_ex(const gdn_shape_t* shape, int32_t n_seqs,
                   const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                   const void* q, const void* k, const void* v, const float* beta,
                   const float* g, const float* h0, const float* dO,
                   const float* dhT, float* o, float* hT, int32_t grad_dtype,
                   void* dq, void* dk, void* dv, float* dbeta, float* dg,
                   float* dh0, void* ws, size_t ws_bytes, void* stream);

/*
 * Native-mixed baseline (not the CPR contract): prefill whose outputs come
 * from the chunk form instead of the token recurrence,
 *     o_p = exp(G_p) S_c q_p + sum_{r<=p} (q_p . k_r) exp(G_p - G_r) Delta_r
 * for each chunk with start state S_c (the same chunk-state scan as
 * gdn_prefill, run over every chunk including a partial last one).  This is
 * the "native mixed" prefill of the write-up's stage table (CPR section):
 * the same function as gdn_prefill within the parity tolerance, but its bits
 * are NOT those of gdn_prefill / gdn_decode_step.  It exists to measure what
 * the bitwise guarantee costs.  hT (nullable) gets each sequence's final
 * state from the chunk form.  Same argument conventions as gdn_prefill, no
 * cache; workspace from gdn_workspace_bytes(..., GDN_OP_PREFILL_CHUNKED).
 * Supported at d_k = d_v = 128 only (GDN_ERR_UNSUPPORTED otherwise).
 */
int gdn_prefill_chunked(const gdn_shape_t* shape, int32_t n_seqs,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                        const void* q, const void* k, const void* v, const float* beta,
                        const float* g, const float* h0, float* o, float* hT, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Native-mixed baseline trainer step (not the CPR contract): gdn_fwd_bwd whose
 * forward outputs o, and the final state of a sequence whose last chunk is
 * partial, come from the chunk form (as in gdn_prefill_chunked) instead of
 * the token recurrence; the backward is gdn_fwd_bwd's.  The same function
 * within the parity tolerance, other bits.  It exists to measure what the
 * bitwise guarantee costs the trainer (the write-up's stage table, CPR
 * section: native mixed against CPR trainer fwd+bwd).  Arguments as
 * gdn_fwd_bwd (fp32 gradients); workspace from gdn_workspace_bytes(...,
 * GDN_OP_FWD_BWD).  d_k = d_v = 128 only (GDN_ERR_UNSUPPORTED otherwise).
 */
int gdn_fwd_bwd_chunked(const gdn_shape_t* shape, int32_t n_seqs,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                        const void* q, const void* k, const void* v, const float* beta,
                        const float* g, const float* h0, const float* dO,
                        const float* dhT, float* o, float* hT, float* dq, float* dk,
                        float* dv, float* dbeta, float* dg, float* dh0, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Native-mixed baseline decode (not the CPR contract): the plain recurrent
 * token step on the running state S [N, H_v, d_k, d_v] (in-out), with no
 * chunk buffers, no position and no resync.  Its arithmetic per token is
 * gdn_decode_step's token step, but without the resync its state leaves the
 * prefill's bits after the first completed chunk.  It exists to measure what
 * the bitwise guarantee costs decode (the write-up's stage table, CPR
 * section: native mixed against CPR rollout decode).  q, k, v, beta, g, o as
 * in gdn_decode_step; no workspace.
 */
int gdn_decode_step_native(const gdn_shape_t* shape, int32_t n_seqs, const void* q,
                           const void* k, const void* v, const float* beta,
                           const float* g, float* S, float* o, void* stream);

/*
 * Kernel timing (instrumentation).  While enabled, every launch the entry
 * points make is bracketed by HIP events recorded on the call's stream.
 * gdn_profile_read waits for the recorded events, returns the summed
 * duration (ms) and launch count of the kernels whose name contains `kernel`
 * (e.g. "k_rec"; NULL or "" = all), and forgets them.  Kernel names:
 * k_plan, k_prep, k_wy, k_scan, k_rec, k_decode, k_wy_resync, k_scan_resync,
 * k_cache_init, k_chunk_o (gdn_prefill_chunked, gdn_fwd_bwd_chunked),
 * k_decode_native (gdn_decode_step_native), k_cont_plan, k_cont_gather,
 * k_cont_scatter (gdn_prefill_continue) and the k_bwd_* kernels of
 * gdn_fwd_bwd.  Events are created
 * by the library on first use and reused; no device memory is allocated.
 * Thread-safe; records from concurrent calls are merged.
 */
int gdn_profile_enable(int on);
/* While timing is enabled, bracket only the launches whose kernel name
 * contains `kernel` (NULL or "" = all, the default): fewer events in a timed
 * loop.  Host only; GDN_OK. */
int gdn_profile_filter(const char* kernel);
int gdn_profile_read(const char* kernel, double* total_ms, int64_t* launches);

/* Identifier of the compiled arithmetic contract (chunk lengths, epsilon,
 * reduction orders, tiling) ending in "src=" and the first 16 hex digits of a
 * SHA-256 over this header, the library sources and the compile flags.  Two
 * builds give bit-identical results only if these strings are equal (the
 * write-up's contract section, identities: the engines that must agree carry
 * and compare such an identity). */
const char* gdn_contract_id(void);

/* Compares another build's gdn_contract_id() with this one's: GDN_OK if equal,
 * GDN_ERR_UNSUPPORTED if not (the two builds are not guaranteed to produce
 * the same bits, e.g. a trainer and a rollout engine built from different
 * sources), GDN_ERR_INVALID_ARG for NULL.  Host only. */
int gdn_contract_check(const char* id);

/* Human-readable text for a gdn_status_t. */
const char* gdn_error_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

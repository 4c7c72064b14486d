/*
 * slim.h -- C ABI of libslim.so: Slim-Attention K-cache-only decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (Slim Attention article, localbendi.com, section "K-Cache is
 * All You Need"): in multi-head attention W_K and W_V are square; when W_K is
 * invertible, W_KV = W_K^-1 . W_V is a new parameter matrix and the value
 * rows follow from the key rows, V = X.W_V = X.W_K.W_K^-1.W_V = K.W_KV.  So
 * only K is cached.  The prompt phase computes K for all tokens and caches
 * it; each generation step computes the new query, its scores against the
 * cached K and their softmax, and recovers V on the fly, either by forming
 * V = K.W_KV and multiplying the softmax by it, or, better for long
 * sequences, by multiplying the softmax by K first and the result by W_KV.
 * This library implements the second form for the decode step.
 *
 * Conventions (all entry points):
 *  - Row-vector convention (x.W).  d = H*dh.  Head h owns columns
 *    [h*dh, (h+1)*dh) of q, K and the output.
 *  - Every matrix is dense row-major with no padding.
 *  - Device pointers are caller-owned device memory (e.g. torch tensors).
 *    The library never allocates, frees or synchronises device memory or
 *    streams; work is enqueued on `stream` (0 = the null stream) and the call
 *    returns once it is enqueued.  Calls are re-entrant; calls that share a
 *    workspace must not overlap.
 *  - Argument checks run on the host before anything is enqueued; on an error
 *    nothing is enqueued.  Device-resident values (lengths, t0) cannot be
 *    checked on the host: they are clamped on the device as documented.
 *  - No C++ exception crosses this interface.
 */
#ifndef SLIM_H
#define SLIM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLIM_OK = 0,
  SLIM_ERR_INVALID = 1,      /* bad pointer, size, alignment or shape      */
  SLIM_ERR_UNSUPPORTED = 2,  /* valid but not built (dtype pair, H, dh...) */
  SLIM_ERR_WORKSPACE = 3,    /* workspace_bytes below the required size    */
  SLIM_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  SLIM_ERR_SINGULAR = 5,     /* W_K is singular to working precision       */
  SLIM_ERR_TIMEOUT = 6       /* device side: an attend workgroup gave up
                                waiting for its partner (slim_decode_status) */
} slim_status_t;

typedef enum { SLIM_F32 = 0, SLIM_BF16 = 1 } slim_dtype_t;

/* Human-readable name of a status code (static storage). */
const char* slim_status_string(slim_status_t s);

/*
 * slim_wkv -- the new parameter matrix W_KV = W_K^-1 . W_V (article section
 * "K-Cache is All You Need", first equation), computed once per layer on the
 * host.
 *   W_K, W_V : host, [d, d] float64, row-major.  W_K must be invertible.
 *   W_KV_out : host, [d, d] in `out_dt` (float32 or bf16 bit patterns,
 *              round-to-nearest-even from the float64 result).
 * Method: LU factorisation of W_K with partial pivoting in float64, then
 * forward and back substitution for the d right-hand sides W_V.  Multi-
 * threaded on the host CPU (SLIM_HOST_THREADS overrides the thread count).
 * Errors: SLIM_ERR_INVALID (null pointer, d <= 0), SLIM_ERR_UNSUPPORTED
 * (out_dt), SLIM_ERR_SINGULAR (a zero pivot).  No HIP call is made.
 */
slim_status_t slim_wkv(const double* W_K, const double* W_V, int d,
                       void* W_KV_out, slim_dtype_t out_dt);

/*
 * slim_prefill -- prompt phase / append: writes K rows into the cache
 * (article section "K-Cache is All You Need": the prompt phase computes K for
 * all input tokens in parallel and caches it instead of V; at the end of each
 * generation step the new k is appended).
 *   K_cache[b, t0[b] + i, :] = round(X[b, i, :] . W)   for i < n
 *   X       : device, [B, n, d] in x_dt
 *   W       : device, [d, d] in w_dt (W_K; any d x d projection works)
 *   K_cache : device, [B, T_max, d] in k_dt
 *   t0      : device int32 [B] start rows, or NULL for all zero.  Rows that
 *             would land at or beyond T_max are not written.
 * Supported dtype triples: (bf16, bf16, bf16) on MFMA with fp32 accumulation
 * and round-to-nearest-even output, and (f32, f32, f32) in fp32.
 * Errors: SLIM_ERR_INVALID (null X/W/K_cache, B, n, d or T_max <= 0,
 * n > T_max, bf16 with d % 8 != 0 or pointers not 16-byte aligned),
 * SLIM_ERR_UNSUPPORTED (other dtype triples), SLIM_ERR_HIP.
 */
slim_status_t slim_prefill(const void* X, slim_dtype_t x_dt,
                           const void* W, slim_dtype_t w_dt,
                           void* K_cache, slim_dtype_t k_dt,
                           int B, int n, int d, int T_max,
                           const int32_t* t0, hipStream_t stream);

/*
 * slim_decode_workspace_bytes -- device workspace slim_decode needs for this
 * shape on the current device (it depends on the device's compute-unit
 * count).  Returns 0 for shapes slim_decode rejects.
 */
size_t slim_decode_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t k_dt);

/*
 * slim_decode -- one generation step of Slim Attention for B sequences, one
 * new query each (article section "K-Cache is All You Need", generation step,
 * second option: softmax times K, then times W_KV).
 *   q       : device float32 [B, d], the new queries (unscaled)
 *   K_cache : device [B, T_max, d] in k_dt; sequence b reads rows [0, len_b)
 *   lengths : device int32 [B]; len_b is clamped to [0, T_max]; len_b = 0
 *             gives a zero output row.  Rows at or beyond len_b are never
 *             read, whatever they hold.
 *   W_KV    : device [d, d] in w_dt (from slim_wkv)
 *   out     : device float32 [B, H, dh]:
 *               out[b,h,:] = (softmax_t(scale * q_h . K[b,t,h-cols]) . K[b,:len_b,:])
 *                            . W_KV[:, h*dh:(h+1)*dh]
 *             which equals standard MHA with V = K . W_KV.
 *   scale   : score scale, normally 1/sqrt(dh)
 *   workspace, workspace_bytes : device scratch of at least
 *             slim_decode_workspace_bytes(B, H, dh, T_max, k_dt) bytes,
 *             16-byte aligned; its contents on entry do not matter.
 * Arithmetic: scores, softmax and all accumulation in float32; for bf16 caches
 * the softmax weights are rounded to bf16 for the MFMA contraction with K,
 * and each token chunk's partial (softmax-times-K sums, accumulated in fp32)
 * is rounded to bf16 once when stored for the merge.
 * Supported: k_dt bf16 (MFMA path: H <= 32, dh in {32, 64, 128}, d % 8 == 0)
 * or f32 (H <= 64, any dh); w_dt f32 or bf16; B <= 4096.
 * Alignment: K_cache, W_KV and workspace 16 bytes; q, lengths, out 4 bytes.
 * Errors: SLIM_ERR_INVALID (null pointers, B/H/dh/T_max <= 0, scale not
 * finite, misaligned pointers), SLIM_ERR_UNSUPPORTED, SLIM_ERR_WORKSPACE,
 * SLIM_ERR_HIP.
 * Score exchange (d = 4096-class shapes: bf16, dh = 128, d > 2048, d a
 * multiple of 512): the two workgroups that share a token chunk swap their
 * heads' scores through the workspace and wait for each other.  They take
 * their roles in arrival order, so a partner is always a workgroup that has
 * already started or is the next to start; the wait assumes that next one
 * becomes resident while the first waits (true unless other work keeps
 * almost every compute unit busy for a long time).  Each wait is bounded
 * (about a second); a workgroup that runs out of it marks its pieces
 * failed, those sequences' outputs become NaN, and slim_decode_status
 * reports SLIM_ERR_TIMEOUT.  The call itself returns SLIM_OK (the failure
 * happens on the device, after the call has returned).
 * Graph capture: the call may be captured into a HIP graph; while the stream
 * is capturing, a reset of the exchange's mailboxes is recorded before the
 * attend so that every replay starts clean.
 * Environment (testing): SLIM_CHUNKS=n fixes the number of token chunks the
 * attend phase cuts the rows into (the workspace size follows it, so query
 * slim_decode_workspace_bytes with the same setting); SLIM_XCHG=0 turns off
 * the score-exchange kernel.  Results agree to rounding with the defaults.
 * SLIM_PARTIALS=f32 keeps the chunk partials of bf16 caches in fp32 (by
 * default they are rounded once to bf16 when stored; every accumulation is
 * fp32 either way; query slim_decode_workspace_bytes with the same setting).
 * SLIM_XCHG_SPIN=n bounds each exchange wait to n re-polls, and
 * SLIM_XCHG_SKEW=1 makes one column group's entries never match, so that
 * every wait runs out (failure-path tests).
 */
slim_status_t slim_decode(const float* q,
                          const void* K_cache, slim_dtype_t k_dt,
                          const int32_t* lengths,
                          const void* W_KV, slim_dtype_t w_dt,
                          float* out,
                          int B, int H, int dh, int T_max, float scale,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * slim_decode_noalloc -- slim_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments and results without a workspace.
 * Its workspace is a device array inside the library, SLIM_NOALLOC_SCRATCH_BYTES
 * bytes per device, reserved when the library's code is loaded on a device
 * and held until the process ends; the call itself allocates nothing.
 * Shapes whose slim_decode_workspace_bytes exceeds that size are rejected
 * with SLIM_ERR_WORKSPACE (nothing is enqueued).  Every call on one device
 * shares that device's array: calls that may overlap on one device (other
 * streams, other threads) race and must not be issued; consecutive calls on
 * one stream are fine.  slim_decode_status cannot be queried for these
 * calls (the array is not the caller's).
 */
#define SLIM_NOALLOC_SCRATCH_BYTES (80u << 20)
slim_status_t slim_decode_noalloc(const float* q,
                                  const void* K_cache, slim_dtype_t k_dt,
                                  const int32_t* lengths,
                                  const void* W_KV, slim_dtype_t w_dt,
                                  float* out,
                                  int B, int H, int dh, int T_max, float scale,
                                  hipStream_t stream);

/*
 * slim_decode_status -- the device-side outcome of the last slim_decode,
 * slim_step or attend + finish pair that used `workspace` (the first 256
 * bytes of a decode or step workspace hold a status word: the attend clears
 * it and the finish sets it when a piece was marked failed).  Waits for
 * `stream` (this call synchronises), then returns SLIM_OK or
 * SLIM_ERR_TIMEOUT (see "Score exchange" above).
 * Errors: SLIM_ERR_INVALID (null or misaligned workspace, workspace_bytes
 * < 256), SLIM_ERR_HIP.
 */
slim_status_t slim_decode_status(const void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * slim_decode_attend / slim_decode_finish -- the two halves of slim_decode,
 * for callers that schedule or time them separately.  Same arguments and
 * checks as slim_decode; slim_decode is exactly attend followed by finish on
 * the same stream with the same workspace.
 *   attend : streams the K cache once; per token chunk: scores, online
 *            softmax and the softmax-times-K contraction, leaving per-chunk
 *            partial results (running max, normaliser, unnormalised
 *            softmax.K row per head) in the workspace.
 *   finish : merges the chunk partials of each sequence (log-sum-exp) and
 *            applies W_KV per head, writing `out`.
 */
slim_status_t slim_decode_attend(const float* q,
                                 const void* K_cache, slim_dtype_t k_dt,
                                 const int32_t* lengths,
                                 const void* W_KV, slim_dtype_t w_dt,
                                 float* out,
                                 int B, int H, int dh, int T_max, float scale,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
slim_status_t slim_decode_finish(const float* q,
                                 const void* K_cache, slim_dtype_t k_dt,
                                 const int32_t* lengths,
                                 const void* W_KV, slim_dtype_t w_dt,
                                 float* out,
                                 int B, int H, int dh, int T_max, float scale,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * slim_step -- one whole generation step for B sequences, in the order of the
 * Slim Attention article (section "K-Cache is All You Need", generation
 * phase): the new token's query, its attention over the K rows cached at
 * earlier steps with V recovered through W_KV (as slim_decode), and at the
 * end the new token's key appended to the cache for the next step.
 *   x        : device float32 [B, d], the new tokens' inputs
 *   W_Q, W_K : device [d, d] in w_dt (f32 or bf16): q = x.W_Q, k = x.W_K,
 *              both accumulated in float32
 *   K_cache  : device [B, T_max, d] in k_dt, read AND written: sequence b
 *              attends over rows [0, len_b), then row len_b receives
 *              round(k_b) (round to nearest even for bf16) when len_b < T_max;
 *              a full cache (len_b = T_max) takes no new row.  No other row
 *              is written.
 *   lengths  : device int32 [B], len_b before the step, clamped to [0, T_max]
 *   lengths_next : device int32 [B], written: len_b + 1, or T_max for a full
 *              cache.  Must not overlap `lengths` (callers alternate two
 *              buffers from step to step).
 *   W_KV, wkv_dt, out, scale : as slim_decode (out[b] is the attention output
 *              of the new token of sequence b; q itself stays in the workspace)
 *   workspace : at least slim_step_workspace_bytes(B, H, dh, T_max, k_dt)
 *              bytes (enough for either w_dt), 16-byte aligned.
 * Kernels, in stream order: the q/k projection (reduction split over row
 * blocks of W), its sum (writes q to the workspace, k to the cache,
 * lengths_next), then the decode kernels.  Shape support as slim_decode, and
 * d % 8 == 0.  Alignment: W_Q, W_K 16 bytes; x, lengths_next 4 bytes.
 * Errors: as slim_decode; SLIM_ERR_INVALID also for null x/W_Q/W_K/
 * lengths_next or lengths_next == lengths.
 */
size_t slim_step_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t k_dt);
slim_status_t slim_step(const float* x,
                        const void* W_Q, const void* W_K, slim_dtype_t w_dt,
                        void* K_cache, slim_dtype_t k_dt,
                        const int32_t* lengths, int32_t* lengths_next,
                        const void* W_KV, slim_dtype_t wkv_dt,
                        float* out,
                        int B, int H, int dh, int T_max, float scale,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * slim_multi_query -- n queries over ONE context of T key rows (Slim
 * Attention article, section "K-Cache is All You Need": only K is kept and
 * V = K.W_KV; the first option forms V and multiplies the softmax by it,
 * the second multiplies the softmax by K first and the result by W_KV).
 * Two uses: cross-attention of n decoder queries over one shared encoder
 * context (limits NULL), and the prompt phase, where the prompt's n tokens
 * attend causally over its own rows (limits[i] = t0 + i + 1).
 *   Q       : device float32 [n, d], unscaled queries
 *   K       : device bf16 [T, d], the context's key rows
 *   limits  : device int32 [n] or NULL: query i attends rows
 *             [0, min(max(limits[i], 0), T)); NULL means all T rows.  A query
 *             with no rows gets a zero output row.
 *   W_KV    : device [d, d] in w_dt
 *   out     : device float32 [n, H, dh]:
 *               out[i,h,:] = softmax_t(scale * Q[i,h-cols] . K[t,h-cols]) . K[t,:] . W_KV[:, h-cols]
 *   option  : 1 (form V = K.W_KV in the workspace, rounded to bf16, then the
 *             softmax times V), 2 (softmax times K on all d columns, then
 *             W_KV), 0 = the cheaper by multiply-accumulate count, with
 *             option 1's dense V product weighted by 2/3 for its higher rate
 *             on this device: option 1 costs (2/3) T d^2 + n T d, option 2
 *             n H T d + n d^2 (slim_multi_query_option returns the choice).
 *   workspace : at least slim_multi_query_workspace_bytes(...) bytes for the
 *             same shape and option, 16-byte aligned.
 * Arithmetic: scores on bf16 MFMA with Q split into high and low bf16 parts
 * (fp32 accumulation); softmax in fp32; softmax weights rounded to bf16 for
 * the MFMA product with K (or V); merge and projection in fp32.
 * Supported: k_dt bf16; w_dt bf16 or f32 (option 1: bf16 only); dh in
 * {64, 128}; d a multiple of 128.  Alignment: Q, K, W_KV, workspace 16
 * bytes; out, limits 4 bytes.
 * Errors: SLIM_ERR_INVALID (null pointers, sizes <= 0, option outside 0..2,
 * scale not finite, misalignment), SLIM_ERR_UNSUPPORTED, SLIM_ERR_WORKSPACE,
 * SLIM_ERR_HIP.
 */
int slim_multi_query_option(int n, int H, int dh, int T);
size_t slim_multi_query_workspace_bytes(int n, int H, int dh, int T, slim_dtype_t k_dt,
                                        slim_dtype_t w_dt, int option);
slim_status_t slim_multi_query(const float* Q,
                               const void* K, slim_dtype_t k_dt,
                               const int32_t* limits,
                               const void* W_KV, slim_dtype_t w_dt,
                               float* out,
                               int n, int H, int dh, int T, float scale, int option,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * mha_decode_kv -- comparator: standard MHA decode over explicit K and V
 * caches (the baseline the Slim Attention article halves), same conventions
 * as slim_decode with V_cache [B, T_max, d] in kv_dt in place of W_KV:
 *   out[b,h,:] = softmax_t(scale * q_h . K[b,t,h-cols]) . V[b,:len_b,h-cols]
 * Supported: kv_dt bf16 (dh in {32, 64, 128}, d % 8 == 0).  Workspace from
 * mha_decode_kv_workspace_bytes.
 */
size_t mha_decode_kv_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t kv_dt);
slim_status_t mha_decode_kv(const float* q,
                            const void* K_cache, const void* V_cache, slim_dtype_t kv_dt,
                            const int32_t* lengths,
                            float* out,
                            int B, int H, int dh, int T_max, float scale,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * HBM probes (measurement only; not part of the method):
 *   slim_probe_read : reads `bytes` from `src` with 16-byte loads and writes
 *                     one float per workgroup to `sink` (device, at least
 *                     slim_probe_sink_floats() floats); the achievable
 *                     streaming-read rate of the device.
 *   slim_probe_copy : copies `bytes` from `src` to `dst` (a plain copy kernel
 *                     of known size, used to calibrate traffic counters).
 * `bytes` must be a multiple of 16 and both pointers 16-byte aligned.
 */
int slim_probe_sink_floats(void);
slim_status_t slim_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
slim_status_t slim_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SLIM_H */

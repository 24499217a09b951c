/*
 * kdn.h -- C ABI of the MI355X (gfx950) delta-rule / Kalman-delta library.
 *
 * Per head the library keeps an associative memory S (d_k x d_v, float32)
 * and, for diagonal KDN, a per-channel variance p (d_k, float32), for
 * isotropic KDN one variance p per head (float32).  For each token, in this
 * order:
 *   1. decay vector a: 1 (DeltaNet), alpha_t * 1 (Gated DeltaNet), or the
 *      per-key-channel vector alpha_t (KDA, diagonal and isotropic KDN);
 *   2. write vector w: beta_t k_t, or for diagonal KDN the Kalman gain
 *        p- = a*a*p + xi_t,  s = r_t + sum_i p-_i k_i^2,  w = p- (.) k / s
 *      (w = 0 if s == 0) followed by the mean-field variance update
 *        p_i = p-_i r_t / (r_t + mu p-_i k_i^2)   (p-_i if that is 0/0);
 *      for isotropic KDN, with means over the d_k channels,
 *        p- = mean(a*a) p + mean(xi_t),  w = p- k / (r_t + p- |k|^2)
 *      (w = 0 if that is 0), then p = p- r_t / (r_t + (mu/d_k) p- |k|^2)
 *      (p- if that is 0/0);
 *   3. S <- diag(a) S;   4. e = v_t - S^T k_t;   5. S <- S + w e^T;
 *   6. o_t = S^T q_t.
 * Sources (page title, section):
 *   - "Внимание в LLM · часть 11 -- Память с поправкой", sections "Сначала
 *     решить, сколько прошлого оставить" (gated state) and "Записать не новое
 *     значение, а ошибку памяти" (read / compare / correct);
 *   - "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند", sections
 *     "تکامل قانون دلتا", "از فراموشی کلی به فراموشی جزئی" (decay before the
 *     delta write; per-channel retention) and "پیاده‌سازی فنی و گذارهای DPLR"
 *     (fused-recurrent decode vs chunkwise prefill);
 *   - "给记忆装一个信任度探测器：Kalman Delta Networks 如何让AI知道自己"记得准不准"",
 *     sections "把记忆问题重新想成一个滤波问题" and "对角近似：把矩阵压扁成一个向量"
 *     (Kalman predict/update, diagonal covariance with exact mean, information
 *     scaling mu) and "各向同性近似：把整个头压缩成一个数" (one variance per head,
 *     the delta rule with a derived write strength).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major data
 *     owned by the caller.  The library never allocates, frees or keeps them.
 *   - Per-token inputs (q, k, v, alpha, beta, proc_noise, obs_noise) and the
 *     output o use the call's dtype; S and p are always float32.
 *   - Alignment (else KDN_ERR_ALIGN): tensors whose last axis is d_k or d_v
 *     (q, k, v, per-channel alpha, proc_noise, o, S*, diagonal-KDN p*) start
 *     on a 16-byte boundary; per-head scalars (beta, obs_noise, the Gated
 *     DeltaNet alpha, isotropic-KDN p*) on their element size.
 *   - A pointer the variant does not use must be NULL.  An empty tensor may
 *     be passed as NULL: the per-token tensors when there are no tokens, the
 *     state tensors when there are no heads.
 *   - All validation runs on the host before any HIP call; on an error nothing
 *     is launched and no output is touched.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.  Faults surface at the caller's
 *     next synchronisation.  Non-finite inputs are not checked; they propagate.
 *   - Argument contracts that are not checked on the device: alpha in [0, 1],
 *     proc_noise >= 0, obs_noise >= 0.
 *   - Thread-safe.  The only global state is a per-device cache of the
 *     device's compute-unit count, filled on first use.
 */
#ifndef KDN_H
#define KDN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kdn_variant {
    KDN_DELTANET = 0,        /* no decay, write strength beta            */
    KDN_GATED_DELTANET = 1,  /* scalar decay alpha_t per token/head      */
    KDN_KDA = 2,             /* per-key-channel decay alpha_t[d_k]       */
    KDN_DIAG_KDN = 3,        /* per-channel decay + diagonal Kalman gain */
    KDN_ISO_KDN = 4          /* per-channel decay + one variance per head */
} kdn_variant;

typedef enum kdn_dtype {
    KDN_F32 = 0,
    KDN_BF16 = 1
} kdn_dtype;

typedef enum kdn_status {
    KDN_OK = 0,
    KDN_ERR_NULL = 1,         /* a required pointer is NULL, or a pointer the
                                 variant does not use is non-NULL          */
    KDN_ERR_SHAPE = 2,        /* negative or overflowing sizes             */
    KDN_ERR_UNSUPPORTED = 3,  /* variant/dtype/d_k/d_v/chunk not built      */
    KDN_ERR_ALIGN = 4,        /* a pointer is not aligned as required      */
    KDN_ERR_ALIAS = 5,        /* an output overlaps an input it may not    */
    KDN_ERR_HIP = 6,          /* the HIP runtime refused the launch        */
    KDN_ERR_WORKSPACE = 7,    /* workspace smaller than the size query     */
    KDN_ERR_SCRATCH = 8       /* kdn_chunk_prefill_noalloc: one chunk of
                                 every head of a sequence exceeds the
                                 library's static scratch                  */
} kdn_status;

/*
 * Chunkwise prefill of T tokens for B sequences x H heads (the chunked form
 * equals the serial recurrence exactly in exact arithmetic: provisional errors
 * resolved by a causal triangular solve -- "معماری KDA ...", section "حل مشکل
 * وابستگی علی").
 *
 * Two schedules compute the same result (up to floating-point rounding):
 *   - workspace == NULL: a single kernel walks the chunks of each sequence in
 *     order (no scratch memory);
 *   - workspace != NULL: the two-pass schedule.  Chunk-parallel kernels write
 *     each chunk's S-independent products (decay-scaled operands, A_qk, the
 *     triangular inverse; for KDN also the variance at each chunk
 *     start, from a scan over per-chunk variance maps, and for diagonal KDN
 *     the maps from each chunk start to its token segments) to the
 *     workspace, then
 *     a sequential pass carries S through the chunks.  This is the fast path
 *     for long sequences.
 * bf16 calls with 1 <= T <= 16 take neither: one kernel holds each head's
 * state on chip and applies the chunk algebra to the T tokens at once (a
 * chunk of 16), leaving any workspace untouched.  This is the fast way to
 * check a run of draft tokens of speculative decoding against a resident
 * state ("معماری KDA ...", section "گام بعدی شما"): S_out / p_out elsewhere
 * keep S0 / p0 as they were (the rollback of a rejected draft), and
 * S_out == S0, p_out == p0 update them in place.
 *
 *   q, k        [B, T, H, d_k]  dtype
 *   v           [B, T, H, d_v]  dtype
 *   alpha       NULL (DeltaNet) | [B, T, H] (Gated DeltaNet) |
 *               [B, T, H, d_k] (KDA, diagonal and isotropic KDN)   dtype
 *   beta        [B, T, H] dtype for DeltaNet / GDN / KDA; NULL for KDN
 *   proc_noise  [B, T, H, d_k] dtype, KDN only (else NULL)
 *   obs_noise   [B, T, H]      dtype, KDN only (else NULL)
 *   S0          [B, H, d_k, d_v] float32, or NULL for a zero memory
 *   p0          [B, H, d_k] float32 (diagonal KDN), [B, H] float32
 *               (isotropic KDN), required for KDN (else NULL)
 *   o           [B, T, H, d_v] dtype (output, o_t = S_t^T q_t)
 *   S_out       [B, H, d_k, d_v] float32 (output); may be exactly S0, must not
 *               overlap it otherwise
 *   p_out       shaped as p0, float32 (output, KDN only, else NULL); may be
 *               exactly p0 when a workspace is passed (or T = 0), must not
 *               overlap it otherwise (the single-pass schedule reads p0 from
 *               several workgroups of a head while one of them writes p_out)
 *   mu          information scaling of the variance update (KDN only; 1 =
 *               unscaled)
 *   chunk       chunk length C; 0 picks the library default (64 for bf16,
 *               32 for float32 with d_k = 128, else 64)
 *   workspace   NULL, or device memory of at least workspace_bytes >=
 *               kdn_chunk_prefill_workspace_size(...) bytes (else
 *               KDN_ERR_WORKSPACE), 256-byte aligned (else KDN_ERR_ALIGN),
 *               overlapping no other argument (else KDN_ERR_ALIAS).  Owned by
 *               the caller; its contents are scratch (ignored on entry,
 *               undefined after).  Calls sharing a workspace must not overlap
 *               in time.
 * Supported: d_k, d_v in {64, 128}; dtype KDN_F32 or KDN_BF16; chunk in
 * {0, 32, 64} subject to the per-dtype limits above; T >= 0 (T = 0 copies
 * S0 / p0 to S_out / p_out); B * H * d_k * d_v < 2^31.
 * o must not overlap any input.
 */
kdn_status kdn_chunk_prefill(kdn_variant variant, kdn_dtype dtype,
                             int B, int T, int H, int d_k, int d_v, int chunk,
                             float mu,
                             const void *q, const void *k, const void *v,
                             const void *alpha, const void *beta,
                             const void *proc_noise, const void *obs_noise,
                             const float *S0, const float *p0,
                             void *o, float *S_out, float *p_out,
                             void *workspace, unsigned long long workspace_bytes,
                             void *stream);

/*
 * kdn_chunk_prefill without a caller-provided workspace and without any
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and checks as kdn_chunk_prefill with a workspace
 * (the two-pass schedule; p_out may be exactly p0), but the workspace is the
 * library's own static device array of KDN_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's first use on that GPU until the process ends.
 * When the call's workspace would not fit in it, the call runs each sequence
 * in segments of whole chunks, one after another on `stream`, each segment
 * continuing from the previous one's S_out / p_out (the recurrence over
 * T1 + T2 tokens is the recurrence over T2 tokens from the state after T1);
 * results then differ from one kdn_chunk_prefill call by floating-point
 * rounding only.  KDN_ERR_SCRATCH if the workspace of a single chunk of all
 * H heads of one sequence exceeds the scratch (bf16, d_k = d_v = 128, C = 64:
 * H > 1016 for the write-strength variants, H > 978 for diagonal KDN).
 * Every argument is checked before the first launch.  Calls on one GPU share
 * its scratch: calls that overlap in time on one GPU race (serialise them,
 * e.g. on one stream).  Nothing is allocated or freed, on the host or the
 * device, by this call.
 */
#define KDN_NOALLOC_SCRATCH_BYTES (64ull << 20)

kdn_status kdn_chunk_prefill_noalloc(kdn_variant variant, kdn_dtype dtype,
                                     int B, int T, int H, int d_k, int d_v, int chunk,
                                     float mu,
                                     const void *q, const void *k, const void *v,
                                     const void *alpha, const void *beta,
                                     const void *proc_noise, const void *obs_noise,
                                     const float *S0, const float *p0,
                                     void *o, float *S_out, float *p_out,
                                     void *stream);

/* Size in bytes of the static scratch kdn_chunk_prefill_noalloc uses. */
unsigned long long kdn_noalloc_scratch_bytes(void);

/*
 * Bytes of workspace kdn_chunk_prefill's two-pass schedule needs for these
 * sizes (0 when there are no tokens or heads), or 0 with *status set when the
 * combination is invalid or unsupported (status may be NULL).  For bf16,
 * d_k = d_v = 128, C = 64 this is 66,048 bytes per (sequence, head, chunk),
 * plus 8,704 for diagonal KDN or 1,044 for isotropic KDN.
 */
unsigned long long kdn_chunk_prefill_workspace_size(kdn_variant variant, kdn_dtype dtype,
                                                    int B, int T, int H, int d_k,
                                                    int d_v, int chunk,
                                                    kdn_status *status);

/*
 * One decode step: one token for each of N sequences x H heads, from the
 * resident state (the fused-recurrent regime: "معماری KDA ...", section
 * "پیاده‌سازی فنی و گذارهای DPLR").
 *
 *   q, k        [N, H, d_k] dtype;   v [N, H, d_v] dtype
 *   alpha       NULL | [N, H] | [N, H, d_k] dtype (as for prefill)
 *   beta        [N, H] dtype, NULL for KDN
 *   proc_noise  [N, H, d_k] dtype, obs_noise [N, H] dtype (KDN only)
 *   S           [N, H, d_k, d_v] float32, read and updated IN PLACE
 *   p           [N, H, d_k] (diagonal KDN) or [N, H] (isotropic KDN) float32,
 *               read and updated in place (KDN only, else NULL)
 *   o           [N, H, d_v] dtype (output)
 * Supported: d_k, d_v in {64, 128}; dtype KDN_F32 or KDN_BF16; N, H >= 0.
 * o must not overlap any input or S / p.
 */
kdn_status kdn_recurrent_decode(kdn_variant variant, kdn_dtype dtype,
                                int N, int H, int d_k, int d_v, float mu,
                                const void *q, const void *k, const void *v,
                                const void *alpha, const void *beta,
                                const void *proc_noise, const void *obs_noise,
                                float *S, float *p, void *o, void *stream);

/*
 * Several decode steps in one pass over the state: T consecutive tokens for
 * each of N sequences x H heads (multi-token decode, e.g. verifying T draft
 * tokens of speculative decoding).  S and p are read once, stepped through
 * the T tokens in registers with exactly the arithmetic of
 * kdn_recurrent_decode, and written once, so the call costs about one decode
 * step of state traffic instead of T.  The token-by-token regime of
 * "معماری KDA ...", section "پیاده‌سازی فنی و گذارهای DPLR", applied to a
 * short run of tokens from a resident state.
 *
 *   q, k        [N, T, H, d_k] dtype;   v [N, T, H, d_v] dtype
 *   alpha       NULL | [N, T, H] | [N, T, H, d_k] dtype (as for prefill)
 *   beta        [N, T, H] dtype, NULL for KDN
 *   proc_noise  [N, T, H, d_k] dtype, obs_noise [N, T, H] dtype (KDN only)
 *   S0          [N, H, d_k, d_v] float32 state before the tokens (NULL: zeros)
 *   p0          [N, H, d_k] (diagonal KDN) or [N, H] (isotropic KDN) float32
 *               (KDN only, else NULL)
 *   o           [N, T, H, d_v] dtype (output, one row per token)
 *   S_out       [N, H, d_k, d_v] float32, the state after the T tokens
 *   p_out       shaped as p0 (KDN only, else NULL)
 * S_out may be S0 exactly and p_out may be p0 exactly (update in place);
 * any other overlap between outputs and inputs is KDN_ERR_ALIAS.  With S_out
 * and p_out elsewhere the resident state is left as it was, which is the
 * rollback of a rejected draft.  T = 0 copies the state.  Token t of
 * sequence n gives the same bits as the t-th of T kdn_recurrent_decode calls
 * on row (n, t) of the same inputs.  The same T tokens through
 * kdn_chunk_prefill (bf16, T <= 16: the chunk form on MFMA) are faster and
 * equal these up to the chunk form's rounding.
 * Supported: d_k, d_v in {64, 128}; dtype KDN_F32 or KDN_BF16; N, T, H >= 0.
 * Errors and asynchrony as for kdn_chunk_prefill.
 */
kdn_status kdn_recurrent_decode_multi(kdn_variant variant, kdn_dtype dtype,
                                      int N, int T, int H, int d_k, int d_v, float mu,
                                      const void *q, const void *k, const void *v,
                                      const void *alpha, const void *beta,
                                      const void *proc_noise, const void *obs_noise,
                                      const float *S0, const float *p0, void *o,
                                      float *S_out, float *p_out, void *stream);

/*
 * Gradients of kdn_chunk_prefill for every variant.  The pages give no
 * gradient ("معماری KDA ...", section "پیاده‌سازی فنی و گذارهای DPLR", names
 * training as a use of the chunk form); what is computed is the exact
 * derivative of the recurrence above for a scalar loss L whose cotangents
 * are d_o = dL/do, dS_out = dL/dS_out and (KDN) dp_out = dL/dp_out,
 * by the reverse of the chunk algebra.  The call re-runs the forward chunk
 * pass internally (it needs the state at every chunk start), then a reverse
 * pass over the chunks for the state gradient, then the chunk-parallel local
 * gradients; for KDN (whose write vector is derived from the variance,
 * "给记忆装一个信任度探测器 ...", sections "对角近似：把矩阵压扁成一个向量" and
 * "各向同性近似：把整个头压缩成一个数") also the reverse of the variance
 * recursion.
 *
 *   q, k, v, alpha, beta, proc_noise, obs_noise, S0, p0, mu, chunk
 *               as for kdn_chunk_prefill (S0 may be NULL)
 *   d_o         [B, T, H, d_v] dtype, dL/do
 *   dS_out      [B, H, d_k, d_v] float32, dL/dS_out, or NULL for zero
 *   dp_out      KDN: shaped as p0, float32, dL/dp_out, or NULL for zero;
 *               else NULL
 * Outputs, all float32 whatever the dtype:
 *   dq, dk      [B, T, H, d_k]
 *   dv          [B, T, H, d_v]
 *   dlog_alpha  alpha * dL/dalpha (the gradient with respect to log alpha):
 *               [B, T, H] (Gated DeltaNet), [B, T, H, d_k] (KDA, KDN), NULL
 *               for DeltaNet
 *   dbeta       [B, T, H] (DeltaNet, Gated DeltaNet, KDA; NULL for KDN)
 *   dproc_noise [B, T, H, d_k], dobs_noise [B, T, H] (KDN; else NULL)
 *   dS0         [B, H, d_k, d_v], dL/dS0; may be NULL (not computed)
 *   dp0         KDN: shaped as p0, dL/dp0, may be NULL; else NULL
 *   workspace   device memory of at least
 *               kdn_chunk_prefill_backward_workspace_size(...) bytes,
 *               256-byte aligned, overlapping no argument; required unless
 *               B*H*T = 0.  Scratch, as for kdn_chunk_prefill.
 * Outputs overlap no input and no other output (else KDN_ERR_ALIAS).
 * Alignment: 16 bytes for tensors whose last axis is d_k or d_v, the element
 * size for per-head scalars.  Validation, asynchrony and errors as for
 * kdn_chunk_prefill.
 */
kdn_status kdn_chunk_prefill_backward(kdn_variant variant, kdn_dtype dtype,
                                      int B, int T, int H, int d_k, int d_v, int chunk,
                                      float mu,
                                      const void *q, const void *k, const void *v,
                                      const void *alpha, const void *beta,
                                      const void *proc_noise, const void *obs_noise,
                                      const float *S0, const float *p0,
                                      const void *d_o, const float *dS_out,
                                      const float *dp_out,
                                      float *dq, float *dk, float *dv, float *dlog_alpha,
                                      float *dbeta, float *dproc_noise, float *dobs_noise,
                                      float *dS0, float *dp0,
                                      void *workspace, unsigned long long workspace_bytes,
                                      void *stream);

/*
 * Bytes of workspace kdn_chunk_prefill_backward needs (0 when there are no
 * tokens), or 0 with *status set when the combination is invalid or
 * unsupported.  It is the forward pass's workspace plus two states (S at
 * each chunk start, dS at each chunk end) per (sequence, head, chunk), kept
 * in the call's dtype (the precision in which the gradient products read
 * them): 66,048 + 65,536 bytes per (sequence, head, chunk) for bf16, d = 128,
 * C = 64, each section rounded up to 256 bytes; isotropic KDN adds 8 bytes
 * per token and 12 per chunk, diagonal KDN 12 d_k + 8 bytes per token and
 * 12 d_k per chunk.
 */
unsigned long long kdn_chunk_prefill_backward_workspace_size(kdn_variant variant,
                                                             kdn_dtype dtype, int B, int T,
                                                             int H, int d_k, int d_v,
                                                             int chunk, kdn_status *status);

/* Static, NUL-terminated description of a status code. */
const char *kdn_status_string(kdn_status status);

/* The chunk length kdn_chunk_prefill uses for `chunk` = 0 (or the validated
 * explicit value), or -1 if the combination is not supported. */
int kdn_chunk_prefill_chunk_size(kdn_dtype dtype, int d_k, int d_v, int chunk);

/* ABI version of this header (incremented on any incompatible change). */
int kdn_abi_version(void);

#define KDN_ABI_VERSION 5

#ifdef __cplusplus
}
#endif

#endif /* KDN_H */

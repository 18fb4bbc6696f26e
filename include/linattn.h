/*
 * linattn.h - C ABI of the kernelized (linear) attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (pages on linear attention):
 *   "Linear Attention" (marovi.ai), "Reformulación con núcleos":
 *       y_i = phi(q_i)^T S / phi(q_i)^T z,
 *       S = sum_j phi(k_j) v_j^T  (d' x d),  z = sum_j phi(k_j)  (d')
 *   causal form ("Forma recurrente e inferencia autorregresiva"): the sums run
 *       over j <= i, the current token included;
 *   blockwise evaluation ("Entrenamiento: forma paralela");
 *   the denominator may be omitted (same section as the definition; the
 *       "Linear Attention" glossary of ultralytics.com, "Ejemplo de código");
 *   phi = elu(x) + 1 ("Linear Transformer (Transformers are RNNs)",
 *       "La función ELU + 1"), d' = d;
 *   phi = positive random features ("Linear Attention", "Mapas de
 *       características"): phi(x) = exp(W x~ - |x~|^2/2) / sqrt(m),
 *       x~ = d^(-1/4) x, W of shape m x d, d' = m;
 *   phi = identity (same section), d' = d.
 * With normalization on, y = num / max(den, 1e-6).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte
 *     aligned. q, k, v, out: [B][H][N][d]. State S: [B][H][d'][d] fp32 (row =
 *     feature index, column = value index). Normalizer z: [B][H][d'] fp32.
 *   - Element type of q, k, v and out: LA_BF16 or LA_F32 (same for all four).
 *     bf16 inputs are multiplied on bf16 matrix cores with fp32 accumulation;
 *     fp32 inputs use fp32 matrix cores. State is always fp32.
 *   - Supported: d in {32, 64, 128} with elu+1 or the identity; random features with
 *     (d, m) in {(32, 64), (32, 128), (64, 64), (64, 128), (64, 256),
 *     (128, 64), (128, 128)}. Other valid requests return LA_ERR_UNSUPPORTED.
 *   - Ownership: the caller allocates and frees every buffer. The library
 *     keeps no pointer after returning and allocates no device memory.
 *   - Errors: validation happens before anything is enqueued, so a failed
 *     call has no side effect. Return value LA_OK (0) or a negative LA_ERR_*.
 *     On LA_OK the work is enqueued on `stream` (asynchronous); faults of the
 *     device work surface at the caller's next synchronization.
 *   - Thread safety: calls on different streams may run concurrently.
 */
#ifndef LINATTN_H_
#define LINATTN_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes */
#define LA_OK 0
#define LA_ERR_INVALID_ARG (-1)  /* null/misaligned pointer, bad size, overlapping output, bad flag */
#define LA_ERR_UNSUPPORTED (-2)  /* valid request outside the supported shapes/maps */
#define LA_ERR_WORKSPACE (-3)    /* workspace null or smaller than la_forward_workspace_size() */
#define LA_ERR_HIP (-4)          /* the HIP runtime rejected a launch */

/* Element types */
#define LA_F32 0
#define LA_BF16 1

/* Feature maps */
#define LA_ELU1 0      /* elu(x) + 1, d' = d */
#define LA_PERFORMER 1 /* positive random features, d' = m */
#define LA_IDENTITY 2  /* phi(x) = x, d' = d; the denominator may be <= 0 (then clamped to 1e-6),
                          so normalize = 0 is its usual use */
#define LA_POLY2 3     /* degree-2 polynomial map ("Mapas de características", polynomial item):
                          phi(x) = (1, x, x (x) x), unit coefficients, x (x) x row-major
                          (feature 1 + d + a d + b = x_a x_b), so phi(q).phi(k) = 1 + q.k + (q.k)^2
                          (>= 3/4); d' = 1 + d + d^2. d in {32, 64}; la_forward, la_decode_step and
                          la_feature_map_apply only */

typedef struct la_feature_map {
  int kind;        /* LA_ELU1, LA_PERFORMER, LA_IDENTITY or LA_POLY2 */
  int m;           /* LA_PERFORMER: number of features (d'); ignored otherwise */
  const float* W;  /* LA_PERFORMER: device pointer, m x d fp32 row-major, shared by all
                      batches and heads; bf16 inputs use W rounded to bf16. Ignored otherwise */
} la_feature_map;

/* Library version, (major << 16) | minor. */
int la_version(void);

/* Static description of a status code (never NULL). */
const char* la_status_string(int status);

/*
 * Status of the device work of earlier calls on the current device.
 * The chunked decay and gated kernels (la_forward_decay, la_backward_decay,
 * la_forward_gated) support decay factors and gates in [1/4, 1] only ("Linear
 * Attention", "Variantes y extensiones": decay and gates enter as powers of
 * up to 32 within a 64-token chunk). A value outside that range, NaN
 * included, cannot be seen on the host (it lives in device memory); the
 * kernels turn it into NaN, so every output that depends on it is NaN, and
 * raise a device flag. This call synchronizes `stream`, then reads and
 * clears that flag: LA_ERR_INVALID_ARG if any such value was met since the
 * last call, LA_OK if none, LA_ERR_HIP if the runtime fails. Work still
 * running on other streams may raise the flag after the read.
 */
int la_device_status(hipStream_t stream);

/*
 * Bytes of device workspace that la_forward needs for these sizes (0 when
 * none is needed; enough for either element type). Returns 0 also for
 * invalid arguments. It holds the fp32 states of the sequence segments and,
 * for random features outside the fused shapes, phi(q) and phi(k)
 * ([B][H][N][m] each, sized for fp32). Random features with d = 64 and bf16
 * input (causal or not) project q and k inside the chunked passes and need
 * the segment states only; this size, which does not know the element type,
 * still covers phi(q) and phi(k) for them (la_forward_workspace_size_dt
 * gives the exact figure). With LA_POLY2 it holds fp32 partial numerators
 * (2 per token at d = 32, 4 at d = 64, [N][d] each per (batch, head)) and
 * partial denominators (2 or 4 per token).
 */
size_t la_forward_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map, int causal);

/*
 * The workspace la_forward needs for inputs of element type `dtype` (LA_F32
 * or LA_BF16): the same as la_forward_workspace_size, except that it leaves
 * out phi(q) and phi(k) where the random-feature map is fused into the
 * chunked passes (d = 64, bf16). Returns 0 for invalid arguments, an unknown
 * dtype included.
 */
size_t la_forward_workspace_size_dt(int B, int H, int N, int d, const la_feature_map* feature_map, int causal,
                                    int dtype);

/*
 * Linear attention over whole sequences ("Reformulación con núcleos"; causal:
 * "Forma recurrente ..." evaluated blockwise as in "Entrenamiento: forma
 * paralela").
 *   q, k, v   in:  [B][H][N][d], element type `dtype`.
 *   out       out: [B][H][N][d], element type `dtype`; must not overlap any input.
 *   causal    1: sums over j <= i;  0: sums over all j.
 *   normalize 1: divide by the denominator;  0: numerator only.
 *   S_in,z_in optional (both or neither): state of earlier tokens, added to
 *             the sums of every position (split/resume of a sequence).
 *   S_out,z_out optional (both or neither): state after the last token,
 *             S_in + sum_j phi(k_j) v_j^T and z_in + sum_j phi(k_j) (the
 *             hand-off to la_decode_step).
 *   workspace device scratch of at least la_forward_workspace_size_dt()
 *             bytes for `dtype` (la_forward_workspace_size() covers both
 *             element types), 256-byte aligned (may be NULL when the size
 *             needed is 0). Its contents are overwritten.
 * N = 0 writes only S_out/z_out (= S_in/z_in, or zeros).
 */
int la_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
               const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
               const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * la_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with no workspace argument. Its workspace is
 * a fixed device array of the library, LA_STATIC_SCRATCH_BYTES per GPU,
 * reserved on each GPU by the first call there and held until the process
 * ends. The call itself allocates nothing.
 *   Arguments and results as la_forward.
 *   Returns LA_ERR_WORKSPACE when la_forward_workspace_size_dt() for the
 *   request exceeds LA_STATIC_SCRATCH_BYTES, LA_ERR_HIP when the array's
 *   address cannot be looked up.
 *   Every call on one GPU uses the same array and leaves its contents behind:
 *   calls that overlap in time on one GPU (concurrent streams, threads) race
 *   on it and must be serialized by the caller. Nothing in the array needs to
 *   start at zero.
 */
#define LA_STATIC_SCRATCH_BYTES (32u << 20)
int la_forward_static(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                      const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
                      const float* z_in, float* S_out, float* z_out, hipStream_t stream);

/*
 * la_forward, plus timing markers: when `events` is not NULL it points to 4
 * caller-created HIP events that are recorded on `stream` before the first
 * kernel (the random-feature map, when used, else the state pass), before the
 * carry scan, before the output pass and after the output pass (a skipped
 * pass has zero length).
 */
int la_forward_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                  const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
                  const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, hipEvent_t* events);

/*
 * One recurrent decode step for every (batch, head) ("Forma recurrente e
 * inferencia autorregresiva"; "La formulación recurrente paso a paso"):
 *   S <- S + phi(k) v^T,  z <- z + phi(k),  out = phi(q)^T S / max(phi(q).z, 1e-6)
 * (state updated first; normalize = 0 drops the division).
 *   S, z      in/out: [B][H][d'][d], [B][H][d'] fp32, updated in place.
 *   q, k, v   in:  [B][H][d] (one token per head), element type `dtype`.
 *   out       out: [B][H][d]; must not overlap q, k, v, S or z.
 */
int la_decode_step(float* S, float* z, const void* q, const void* k, const void* v, void* out, int B, int H,
                   int d, const la_feature_map* feature_map, int normalize, int dtype, hipStream_t stream);

/*
 * Causal linear attention with decay ("Linear Attention", "Variantes y
 * extensiones", RetNet item): S_t = gamma S_{t-1} + phi(k_t) v_t^T, with the
 * normalizer decayed alike, z_t = gamma z_{t-1} + phi(k_t) (reading: the
 * pages give the recurrence for S only), y_t = phi(q_t)^T S_t / phi(q_t).z_t.
 * Unrolled, token j enters output i with weight gamma^(i-j); S_in/z_in enter
 * output i with weight gamma^(i+1); S_out/z_out are the decayed state after
 * the last token.
 *   gamma  in: DEVICE pointer to H fp32 values, one per head (head h of every
 *          batch uses gamma[h]); each must lie in [1/4, 1] (1 = no decay;
 *          the kernels scale rows of a 64-token chunk by up to gamma^(-32)).
 *          A head whose gamma is outside that range gets NaN outputs (and
 *          NaN S_out/z_out) and raises the flag that la_device_status reports.
 * Everything else as la_forward with causal = 1 (same workspace size).
 */
int la_forward_decay(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                     const la_feature_map* feature_map, const float* gamma, int normalize, int dtype,
                     const float* S_in, const float* z_in, float* S_out, float* z_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * la_decode_step with decay: S <- gamma S + phi(k) v^T, z <- gamma z + phi(k),
 * then the readout. gamma: DEVICE pointer to H fp32 values (any value in
 * [0, 1] is valid here).
 */
int la_decode_step_decay(float* S, float* z, const void* q, const void* k, const void* v, void* out, int B, int H,
                         int d, const la_feature_map* feature_map, const float* gamma, int normalize, int dtype,
                         hipStream_t stream);

/*
 * The feature map alone ("Mapas de características"): phi applied to each row.
 *   x    in:  [rows][d], element type in_dtype.
 *   phi  out: [rows][d'], element type out_dtype; must not overlap x or W.
 * Random features with bf16 input multiply in bf16 (W rounded to bf16) with
 * fp32 accumulation; the exponential and the output are computed in fp32.
 */
int la_feature_map_apply(const void* x, void* phi, long long rows, int d, const la_feature_map* feature_map,
                         int in_dtype, int out_dtype, hipStream_t stream);

/*
 * Bytes of device workspace that la_backward needs (0 for invalid
 * arguments): the forward states entering each sequence segment, the
 * gradient states leaving each segment and two fp32 values per token.
 */
size_t la_backward_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map);

/*
 * Gradients of causal la_forward ("Entrenamiento: forma paralela" trains
 * through the blockwise form; the pages give no gradient formulas, so these
 * are the exact derivatives of the causal definition, up to rounding).
 * With L = <dout, out> + <dS_out, S_out> + <dz_out, z_out> for the outputs
 * of la_forward(q, k, v, causal = 1, normalize, S_in, z_in):
 *   dq, dk, dv out: dL/dq, dL/dk, dL/dv, [B][H][N][d], element type `dtype`;
 *             each must overlap no other buffer of the call.
 *   dout      in:  [B][H][N][d], element type `dtype`.
 *   S_in,z_in optional in (both or neither): the forward's initial state.
 *   dS_out,dz_out optional in (both or neither): cotangents of the final
 *             state (zero when absent).
 *   dS_in,dz_in optional out (both or neither): dL/dS_in, dL/dz_in
 *             ([B][H][d][d], [B][H][d] fp32; defined also without S_in).
 *   workspace at least la_backward_workspace_size() bytes, 256-byte aligned.
 * The forward is recomputed (no saved activations). Where max(den, 1e-6)
 * clamps, its derivative is taken as 0 (den < 1e-6) or 1 (den >= 1e-6).
 * Supported: elu+1 and the identity map, d in {32, 64, 128}; random
 * features return LA_ERR_UNSUPPORTED (decay: la_backward_decay). N = 0
 * writes only dS_in/dz_in (= dS_out/dz_out, or zeros).
 */
int la_backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv, int B,
                int H, int N, int d, const la_feature_map* feature_map, int normalize, int dtype, const float* S_in,
                const float* z_in, const float* dS_out, const float* dz_out, float* dS_in, float* dz_in,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gradients of la_forward_decay (causal, per-head decay, "Linear Attention",
 * "Variantes y extensiones", RetNet item), as la_backward for
 * L = <dout, out> + <dS_out, S_out> + <dz_out, z_out>:
 * dS_in/dz_in then hold dL/dS_in, dL/dz_in, in which every token's term
 * carries its decay factor. gamma: DEVICE pointer to H fp32 values in
 * [1/4, 1], as for la_forward_decay (outside it: NaN gradients for that head
 * and the la_device_status flag).
 * Workspace: la_backward_workspace_size() bytes. Everything else as
 * la_backward.
 */
int la_backward_decay(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, const la_feature_map* feature_map, const float* gamma, int normalize,
                      int dtype, const float* S_in, const float* z_in, const float* dS_out, const float* dz_out,
                      float* dS_in, float* dz_in, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace that la_forward_gated needs (0 for invalid
 * arguments or when none is needed).
 */
size_t la_forward_gated_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map);

/*
 * Gated linear attention, causal ("Linear Attention", "Variantes y
 * extensiones", GLA item: the scalar decay replaced by a data-dependent
 * gate). Reading: a per-token, per-feature gate alpha_t on the feature
 * dimension,
 *   S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T,  z_t = alpha_t * z_{t-1} + phi(k_t),
 *   out_t = phi(q_t)^T S_t / max(phi(q_t).z_t, 1e-6)  (normalize = 0: numerator only),
 * evaluated blockwise ("Entrenamiento: forma paralela").
 *   log_gates in: DEVICE pointer, [B][H][N][d] fp32, log(alpha) in [-log 4, 0]
 *             (alpha in [1/4, 1]; the kernels scale rows of a 64-token chunk by
 *             up to alpha^-32 per feature). A log-gate outside that range
 *             (NaN included) becomes NaN, so the outputs that depend on it
 *             are NaN, and raises the flag that la_device_status reports.
 *   S_in, z_in enter output t through feature f with the product of the gates
 *             of tokens 0..t; S_out, z_out are the gated state after the last token.
 * elu+1 and the identity map; random features return LA_ERR_UNSUPPORTED.
 * Everything else as la_forward with causal = 1; the workspace is
 * la_forward_gated_workspace_size() bytes.
 */
int la_forward_gated(const void* q, const void* k, const void* v, const float* log_gates, void* out, int B, int H,
                     int N, int d, const la_feature_map* feature_map, int normalize, int dtype, const float* S_in,
                     const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * la_decode_step with a per-feature gate: S <- diag(exp(log_gate)) S + phi(k) v^T,
 * z <- exp(log_gate) * z + phi(k), then the readout. log_gate: DEVICE pointer,
 * [B][H][d'] fp32 (any value <= 0 is valid here). Every map but LA_POLY2.
 */
int la_decode_step_gated(float* S, float* z, const void* q, const void* k, const void* v, const float* log_gate,
                         void* out, int B, int H, int d, const la_feature_map* feature_map, int normalize, int dtype,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H_ */

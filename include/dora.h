/*
 * dora.h - C ABI of libdora.so, the MI355X (gfx950) DoRA module hot path.
 *
 * Sources (by page title and section):
 *   [SD]   "Scaling DoRA: High-Rank Adaptation via Factored Norms and Fused
 *          Kernels" (Zelenin, Zhuravlyova; arXiv 2603.22276), abstract:
 *          the row-wise norm of W + sBA, its factored form (base, cross and
 *          Gram terms through O(d_out r + r^2) intermediates, no dense BA),
 *          and the single-pass, cancellation-safe composition.
 *   [DoRA] "DoRA: Weight-Decomposed Low-Rank Adaptation" (Liu et al. 2024),
 *          summary pages: "Method" (magnitude m and a direction updated by
 *          LoRA) and "Statistical analysis" (a training-memory modification,
 *          read here as a norm held constant in the backward pass).
 *
 * Notation.  W [d_out, d_in] is the frozen weight, A [r, d_in] and
 * B [d_out, r] the LoRA factors, s the LoRA scale, m [d_out] the magnitude,
 * x [T, d_in] the tokens.  V = W + s*B*A is never formed.
 *   n_i  = ||W_i + s*B_i*A||_2                       (row norm, [SD])
 *   g_i  = m_i / n_i
 *   y    = g (.) (x W^T + s * (x A^T) B^T)           ([SD], [DoRA])
 *
 * Conventions shared by every call:
 *   - Every matrix is dense, row-major and contiguous.  Matrix data (x, W,
 *     A, B, dy, y, P, base, lora, dx, dA, dB) has one element type given by
 *     the dora_dtype argument.  m, n, dm and the optional norm terms are
 *     always fp32.  s is an fp32 scalar passed by value.
 *   - Every pointer is device memory owned by the caller (e.g. torch
 *     tensors).  The library never allocates device memory and keeps no
 *     state between calls; its only scratch is the caller's workspace
 *     `ws` of at least the size the matching *_workspace() query returns.
 *     No workspace size has a d_out*d_in term: no dense [d_out, d_in]
 *     buffer is ever formed.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Arguments are
 *     validated on the host before anything is enqueued; kernels then run
 *     asynchronously on `stream` and results are valid once it is
 *     synchronised.  Nothing inside synchronises the host.
 *   - Every pointer must be 16-byte aligned.  Sizes need not be multiples
 *     of anything: T >= 0, and d_in, d_out, r >= 1 (all < 2^31).  Tails are
 *     masked in the kernels; a bf16 width that leaves rows unaligned to 16
 *     bytes (not a multiple of 8) runs on element-masked loads, slower than
 *     the pipelined path but with the same arithmetic.
 *   - Results are bitwise deterministic for identical inputs: there are no
 *     floating-point atomics and every reduction runs in a fixed order.
 *   - Arithmetic: products accumulate in fp32; matrix outputs are rounded
 *     once, to nearest even, to the element type.
 *   - Preconditions not checked per element: n_i > 0 (rows of W + sBA are
 *     not zero) and, for dora_backward, m_i != 0.  Violations propagate
 *     IEEE inf/NaN; they never fault.
 *
 * Errors: every call returns a dora_status.  On failure nothing has been
 * enqueued unless the status is DORA_E_HIP (a launch failed part-way; the
 * outputs are then unspecified).  dora_last_error() returns a thread-local
 * message describing the last failure on the calling thread.
 */
#ifndef DORA_H
#define DORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DORA_OK = 0,
    DORA_E_NULL = 1,      /* a required pointer is NULL                      */
    DORA_E_SHAPE = 2,     /* a size is out of range                          */
    DORA_E_DTYPE = 3,     /* unknown dora_dtype                              */
    DORA_E_ALIGN = 4,     /* a pointer is not 16-byte aligned                */
    DORA_E_WORKSPACE = 5, /* ws is NULL or ws_bytes is below the query       */
    DORA_E_ALIAS = 6,     /* two buffers overlap where that is not allowed   */
    DORA_E_HIP = 7        /* a HIP launch or runtime call failed             */
} dora_status;

typedef enum {
    DORA_F32 = 0,  /* IEEE binary32 */
    DORA_BF16 = 1  /* bfloat16 (upper 16 bits of binary32) */
} dora_dtype;

/* Human-readable name of a status code (static string). */
const char *dora_strerror(int status);

/* Message for the last failure on the calling thread ("" if none). */
const char *dora_last_error(void);

/* Workspace sizes in bytes for the calls below (0 if the arguments are
 * invalid).  They are pure host functions.  The norm workspace is
 * O(d_out*r + r^2) for fixed splits, as [SD] states for the factored
 * intermediates; forward and backward add O(T*d_out + T*r) activations. */
size_t dora_norm_workspace(int64_t d_out, int64_t d_in, int64_t r, int dtype);
size_t dora_forward_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype);
size_t dora_backward_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype);

/*
 * dora_factored_norm - row norms of W + s*B*A without forming B*A ([SD]
 * abstract, "factored norm"):
 *     n_i^2 = base_i + 2*s*cross_i + s^2*gram_i
 *     base_i  = sum_j W_ij^2
 *     cross_i = sum_k B_ik * U_ik,        U = W A^T      [d_out, r]
 *     gram_i  = sum_k B_ik * (B G)_ik,    G = A A^T      [r, r]
 * n is written as sqrt(max(n^2, 0)) (the factored sum can round below
 * zero only when ||W_i + s B_i A|| << ||W_i||).
 *   W [d_out, d_in], A [r, d_in], B [d_out, r] in `dtype`.
 *   n [d_out] fp32 (required).  base, cross, gram [d_out] fp32, each
 *   optional (NULL to skip).  U_out [d_out, r] fp32, optional: receives
 *   V A^T = (W + s B A) A^T = U + s B G, the two products the norm forms
 *   anyway (U by the cross term's product, s B G added by the Gram term's);
 *   keeping it lets the backward through the norm skip W A^T, A A^T and
 *   B G (its dB term is a row scale of exactly this matrix).
 *   ws: device scratch of dora_norm_workspace(d_out, d_in, r, dtype) bytes.
 */
int dora_factored_norm(const void *W, const void *A, const void *B, float s,
                       int64_t d_out, int64_t d_in, int64_t r, int dtype,
                       float *n, float *base, float *cross, float *gram, float *U_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * dora_compose - the single-pass composition ([SD] abstract, fused
 * compose with a numerically stable form for the near-unity regime):
 *     y[t,i] = base[t,i] + ( (g_i - 1) * base[t,i] + g_i * s * lora[t,i] )
 * with g_i - 1 = (m_i - n_i) / n_i and g_i s = m_i s / n_i each rounded once
 * to fp32, the bracket summed in fp32 before base is added, and one rounding
 * to `dtype` at the end.  Mathematically y = (m/n) (.) (base + s*lora).
 *   base, lora, y [T, d_out] in `dtype`; m, n [d_out] fp32.
 *   y may be the same pointer as base (in place); any other overlap of y
 *   with base or lora is DORA_E_ALIAS.
 */
int dora_compose(const void *base, const void *lora, const float *m, const float *n,
                 float s, int64_t T, int64_t d_out, int dtype, void *y, void *stream);

/*
 * dora_forward - the DoRA module forward ([SD], [DoRA]):
 *     n   = factored row norm (as dora_factored_norm), unless n_in is given
 *     P   = x A^T                            [T, r]
 *     h   = x W^T + (s P) B^T                one K-concatenated product,
 *                                            accumulated in fp32
 *     y   = h + ((m - n) / n) h              = (m/n) h, applied by the
 *                                            product's epilogue, rounded once
 *   The base and adapter products share one accumulator, so the composition
 *   happens in the same pass that produces them ([SD]'s single-pass compose,
 *   taken one step further): no [T, d_out] intermediate exists.  P and s P
 *   are each rounded once to the element type from the same fp32 sums of
 *   x A^T (s P is P itself when s = 1).
 *   x [T, d_in], W [d_out, d_in], A [r, d_in], B [d_out, r] in `dtype`;
 *   m [d_out] fp32.  y [T, d_out] in `dtype` (output).
 *   n_out [d_out] fp32: receives n (required; with n_in it receives a copy).
 *   P_out [T, r] in `dtype`: receives x A^T for the backward (NULL: kept in
 *   the workspace only).
 *   n_in [d_out] fp32 or NULL: a norm computed earlier (cached inference);
 *   when given, the norm is not recomputed.
 *   U_out [d_out, r] fp32 or NULL: receives the norm's V A^T = U + s B G
 *   (as in dora_factored_norm) for dora_backward_through_norm; needs n_in
 *   NULL.
 *   y must not overlap any input, n_out, P_out or U_out.
 */
int dora_forward(const void *x, const void *W, const void *A, const void *B, const float *m,
                 float s, int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype,
                 void *y, float *n_out, void *P_out, const float *n_in, float *U_out,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * dora_backward - gradients of L = sum(dy (.) y) with the row norm n held
 * constant (stop-gradient; [DoRA] "Statistical analysis", training-memory
 * modification).  With g = m / n and dh = g (.) dy:
 *     dm_i = sum_t dy[t,i] * y[t,i] / m_i    (= sum_t dy h / n_i, h = x V^T)
 *     Q    = s * dh B                        [T, r], in the workspace
 *     dx   = dh W + Q A
 *     dB   = s * dh^T P
 *     dA   = Q^T x
 * W is frozen and gets no gradient.  dx and dm equal the gradients without
 * the stop-gradient (n does not depend on x or m); dA and dB omit the path
 * through n.
 *   dy, y [T, d_out], x [T, d_in], P [T, r] (from dora_forward), W, A, B in
 *   `dtype`; m, n [d_out] fp32 (n as returned by dora_forward).
 *   Outputs: dx [T, d_in], dA [r, d_in], dB [d_out, r] in `dtype`,
 *   dm [d_out] fp32.  Outputs must not overlap each other or any input.
 *   With T = 0, dA, dB and dm are zero.
 */
int dora_backward(const void *dy, const void *x, const void *W, const void *A, const void *B,
                  const float *m, const float *n, float s, const void *P, const void *y,
                  int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype,
                  void *dx, void *dA, void *dB, float *dm,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * dora_backward_through_norm - the same gradients without the stop-gradient:
 * the gradient also flows through the row norm n = ||W + s B A|| into A and
 * B.  The DoRA summary page ("Statistical analysis", analysis design) names
 * the gradient with respect to the direction V and the magnitude as derived
 * in the method's gradient analysis; the plain chain rule through n_i =
 * ||V_i|| (dn_i / dV_i = V_i / n_i) gives, with c_i = m_i dm_i / n_i^2,
 *     dV = dh^T x - diag(c) V
 *     dA = s B^T dV = Q^T x - s (c (.) B)^T W - s^2 ((c (.) B)^T B) A
 *     dB = s dV A^T = s dh^T P - s c (.) (W A^T + s B (A A^T))
 * using only [d_out, r] and [r, r] intermediates (no dense V or B A, as in
 * the factored norm of the "Scaling DoRA" abstract).  dx and dm are those of
 * dora_backward, bit for bit.  Arguments, layouts, aliasing rules and the
 * T = 0 case (dm zero, dA and dB then zero as well) are those of
 * dora_backward; n is the norm dora_forward returned and is taken as the
 * exact norm of W + s B A.  U [d_out, r] fp32 or NULL: the norm's
 * V A^T = W A^T + s B (A A^T) as dora_forward's (or dora_factored_norm's)
 * U_out kept it, for the same W, A, B and s (the factored norm's products
 * are reused, so W A^T, A A^T and B G are not formed again); NULL forms
 * them here.
 *   ws: dora_backward_through_norm_workspace(T, d_in, d_out, r, dtype) bytes.
 */
size_t dora_backward_through_norm_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                            int dtype);
int dora_backward_through_norm(const void *dy, const void *x, const void *W, const void *A,
                               const void *B, const float *m, const float *n, float s,
                               const void *P, const void *y, const float *U, int64_t T,
                               int64_t d_in, int64_t d_out, int64_t r, int dtype, void *dx,
                               void *dA, void *dB, float *dm, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Grouped calls - many adapted modules in few launches.  The "Scaling DoRA"
 * abstract motivates the factored norm with models that carry hundreds of
 * adapted modules; these calls give each kernel of the norm (and of the
 * forward of sibling modules that share one input, such as the query, key
 * and value projections) one launch per 16 modules instead of one per
 * module, with every module's products sharing the GPU at once.
 *
 * dora_module describes one module: W [d_out, d_in], A [r, d_in],
 * B [d_out, r] in `dtype`, m [d_out] fp32 (not read by the norm), scale s.
 * The array is read on the host during the call only.
 */
typedef struct dora_module {
    const void *W;
    const void *A;
    const void *B;
    const float *m;
    float s;
    int64_t d_out, d_in, r;
} dora_module;

/*
 * dora_factored_norm_grouped - n[i] = the row norms of W_i + s_i B_i A_i for
 * every module, as dora_factored_norm computes them (the same terms and
 * precision; the split-K plan may differ, so bits may too).  n is a host
 * array of `count` device pointers ([d_out_i] fp32 each), pairwise disjoint
 * and disjoint from every module's W, A, B and the workspace.  fp32 modules
 * (and bf16 ones whose operands reach 2 GiB) run module by module.
 *   ws: dora_factored_norm_grouped_workspace(mods, count, dtype) bytes.
 */
size_t dora_factored_norm_grouped_workspace(const dora_module *mods, int count, int dtype);
int dora_factored_norm_grouped(const dora_module *mods, int count, int dtype, float *const *n,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * dora_forward_grouped - dora_forward for `count` modules on the same input
 * x [T, d_in] (every module's d_in must equal d_in): y[i] [T, d_out_i],
 * n_out[i] [d_out_i] fp32, optional P_out[i] [T, r_i] (P_out itself may be
 * NULL), optional cached norms n_in[i] (n_in itself may be NULL; a given
 * n_in[i] skips that module's norm and may equal n_out[i]).  Host arrays of
 * device pointers; every output is disjoint from every input and from every
 * other output.  Per 16 modules: one launch of all x A_i^T, one of the s P
 * scalings, one of the fused products with the magnitude epilogue.
 *   ws: dora_forward_grouped_workspace(mods, count, T, dtype, n_in, P_out)
 *   bytes (it depends on which norms are cached and which P are kept).
 */
size_t dora_forward_grouped_workspace(const dora_module *mods, int count, int64_t T, int dtype,
                                      const float *const *n_in, void *const *P_out);
int dora_forward_grouped(const void *x, int64_t T, int64_t d_in, const dora_module *mods,
                         int count, int dtype, void *const *y, float *const *n_out,
                         void *const *P_out, const float *const *n_in, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * dora_merge - the merged weight W' = g (.) (W + s B A), g = m / n by rows,
 * for inference: the DoRA summary pages ("Method"; Key Points 3 and 5) note
 * that the adapted weight folds into the base weight, so inference is a
 * plain linear layer (dora_linear).  n is the factored row norm of the
 * "Scaling DoRA" abstract (computed here unless n_in is given), so no dense
 * B A product is kept: B A is formed tile by tile inside one product whose
 * epilogue writes W'[i, j] = W[i, j] + ((g_i - 1) W[i, j] + g_i s (BA)[i, j])
 * in fp32, rounded once (the near-unity form of dora_compose).
 *   W, W_out [d_out, d_in], A [r, d_in], B [d_out, r] in `dtype`; m and
 *   n_in (nullable) [d_out] fp32.  W_out may be W itself (in place) but must
 *   not overlap it otherwise, nor A, B, m, n_in or the workspace.
 *   ws: dora_merge_workspace(d_out, d_in, r, dtype) bytes.
 */
size_t dora_merge_workspace(int64_t d_out, int64_t d_in, int64_t r, int dtype);
int dora_merge(const void *W, const void *A, const void *B, const float *m, float s,
               int64_t d_out, int64_t d_in, int64_t r, int dtype, const float *n_in, void *W_out,
               void *ws, size_t ws_bytes, void *stream);

/*
 * dora_linear - y = x W^T on the same kernel and launch plan dora_forward
 * uses for its base term.  With W = W' = g (.) (W + sBA), the weight merged
 * after training, this is the whole DoRA inference path: the DoRA summary
 * pages ("Method"; Key Points 3 and 5) note that the adapted weight merges
 * into the base weight, adding no inference latency.
 *   x [T, d_in], W [d_out, d_in], y [T, d_out] in `dtype`; y must not
 *   overlap x or W.  ws: dora_linear_workspace(T, d_in, d_out, dtype) bytes
 *   (0 when the product needs no split-K partials; ws may then be NULL).
 */
size_t dora_linear_workspace(int64_t T, int64_t d_in, int64_t d_out, int dtype);
int dora_linear(const void *x, const void *W, int64_t T, int64_t d_in, int64_t d_out, int dtype,
                void *y, void *ws, size_t ws_bytes, void *stream);

/*
 * dora_forward_noalloc - dora_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The arguments and results are those
 * of dora_forward without ws / ws_bytes; the scratch comes from a fixed
 * library-owned device array of DORA_NOALLOC_SCRATCH_BYTES (96 MiB), which
 * every GPU the library runs on holds from the library's load until the
 * process ends (its address on a device is looked up on the first call
 * there).  The call allocates nothing.
 *   Modules whose dora_forward_workspace() exceeds the array are rejected
 *   with DORA_E_WORKSPACE before anything touches the device.  The forward
 *   of every module of up to 16384 tokens at widths of the order of 28672
 *   with r = 384 fits.
 *   The array is shared by every call on one GPU and keeps the last call's
 *   contents (nothing in it needs to start at zero): calls that overlap in
 *   time on one GPU (on different streams or threads) race on it and must
 *   be serialised by the caller.  The stream's device is the GPU used.
 */
#define DORA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int dora_forward_noalloc(const void *x, const void *W, const void *A, const void *B,
                         const float *m, float s, int64_t T, int64_t d_in, int64_t d_out,
                         int64_t r, int dtype, void *y, float *n_out, void *P_out,
                         const float *n_in, float *U_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DORA_H */

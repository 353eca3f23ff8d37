/*
 * mhc.h -- C ABI of libmhc, the mHC seam block (manifold-constrained
 * hyper-connections) for AMD Instinct MI355X (gfx950).
 *
 * The seam sits between sublayers of a DeepSeek-V4.1-style decoder.  The
 * residual carries n = 4 streams, x[T][4][C] in bf16.  The pre stage projects
 * the RMS-scaled, flattened 4C row onto 24 logits ("mixes"), turns them into a
 * sigmoid pre-mix, a post gate in (0,2) and a 4x4 comb matrix normalised by
 * Sinkhorn iterations, and collapses the streams into the sublayer input
 * (optionally through a folded RMSNorm).  The post stage writes the next
 * residual, post_i * y + sum_j comb[i][j] x_j.
 *
 * Sources, cited by page title and section:
 *   [p1] vLLM PR "[ROCm][DSV4.1][Perf] Use AITER mHC for the delayed pre block"
 *   [p3] vLLM PR "[ROCm][DSv4.1] Fix TileLang mHC pre on 64-wide wavefronts and
 *        use the fused kernels on the AMD path"
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is caller-owned DEVICE memory unless stated, and
 *     must be 16-byte aligned.  bf16 tensors are passed as uint16_t bit
 *     patterns; float tensors are IEEE single.  All arrays are dense row-major.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream).  No call allocates memory, synchronises the host, or
 *     compiles code, so calls may be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and the status says why.  T == 0 is a no-op.
 *   - Supported shapes: n == 4 (MHC_ERR_UNSUPPORTED otherwise); C a multiple
 *     of 256 with 256 <= C <= 16384 (MHC_ERR_UNSUPPORTED otherwise);
 *     0 <= T <= MHC_MAX_TOKENS (MHC_ERR_SHAPE otherwise).
 *   - Outputs never overlap inputs or each other (MHC_ERR_ALIAS), except the
 *     exact in-place form out == x of mhc_post.
 *   - The library keeps no state between calls (the one process-wide
 *     setting is the test hook mhc_debug_force_wait_timeouts).  The workspace
 *     (see mhc_workspace_bytes) is scratch for one call at a time: calls that
 *     may run concurrently need separate workspaces.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_HC_MULT 4          /* residual streams n */
#define MHC_NUM_LOGITS 24      /* 2n + n*n: pre-mix | post | comb (row-major) */
#define MHC_MAX_TOKENS (1 << 22)
#define MHC_MAX_SINKHORN_ITERS 1024  /* larger iteration counts are MHC_ERR_SHAPE */

typedef enum {
    MHC_OK = 0,
    MHC_ERR_NULL = 1,        /* a required pointer is NULL */
    MHC_ERR_SHAPE = 2,       /* T < 0 or too large, eps < 0 or not finite, sinkhorn_iters
                                outside [1, MHC_MAX_SINKHORN_ITERS] */
    MHC_ERR_UNSUPPORTED = 3, /* n != 4, or C outside the supported set */
    MHC_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    MHC_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
    MHC_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than mhc_workspace_bytes */
    MHC_ERR_HIP = 7          /* the HIP runtime refused the launch (e.g. no device) */
} mhc_status;

/* Weights of one seam.
 *   fn_packed: the projection weight fn[K][24] (K = n*C, or C for the entry
 *              seam) in the library's packed form, produced once per weight by
 *              mhc_pack_fn.  p1 Approach: "projection against fn".
 *   bias:      [24] float, added to the logits.
 *   alpha:     [3] float, scale of the pre-mix, post and comb logit groups.
 * Logit j of a token is alpha[g(j)] * (r * P_j) + bias[j], with P = x . fn,
 * r = 1/sqrt(mean(x^2) + eps) over the K row elements and g(j) = 0 for j < 4,
 * 1 for 4 <= j < 8, 2 otherwise. */
typedef struct {
    const void *fn_packed;
    const float *bias;
    const float *alpha;
} mhc_weights;

/* Bytes of the packed projection weight for K rows (K a multiple of 32):
 * 96*K, the same as the float32 weight. */
size_t mhc_fn_packed_bytes(int K);

/* Pack fn[K][24] (float32, device) into fn_packed (device, mhc_fn_packed_bytes(K)
 * bytes): each weight is split into a bf16 pair hi + lo (hi = bf16(f),
 * lo = bf16(f - hi); |f - hi - lo| <= 2^-16 |f|) and laid out in the operand
 * order of the gfx950 bf16 matrix instructions.  Run once per weight, not per
 * call.  K must be a multiple of 32 and at most 4*16384. */
mhc_status mhc_pack_fn(const float *fn, int K, void *fn_packed, void *stream);

/* Workspace bytes needed by mhc_pre, mhc_pre_delayed, mhc_post_pre_delayed and
 * mhc_broadcast_entry for any T <= T_max with this n and C (few tokens: the
 * projection is split over workgroups that combine partial sums in it; with
 * C = 4096, 5120 or 7168 the persistent kernels of mhc_post_pre_delayed
 * (T > 3072), mhc_pre_delayed and mhc_pre (T > 4096) exchange partial sums
 * through it: about 4.5 MB at C = 5120 and 7.8 MB at C = 7168).  One
 * workspace serves all of these calls.  The caller zero-fills it once after
 * allocating it; every call leaves its counters back
 * at zero, so it can be reused (and captured) without clearing. */
size_t mhc_workspace_bytes(int T_max, int n, int C);

/* Workspace words the calls read before they write (counters, flags and
 * records) lie in bytes [0, MHC_WS_FLAG_BYTES); a call whose waits all
 * completed leaves them zero.  Workgroups of one call that exchange partial
 * sums wait for one another only in bounded waits (forward progress does not
 * depend on the bound: a correct call on a device of its own waits a few
 * sleeps at most).  A wait that runs out stops waiting, sets the 32-bit word
 * at byte MHC_WS_WAIT_ERROR_PERSIST (persistent kernels) or
 * MHC_WS_WAIT_ERROR_SPLIT (split projection) to a non-zero value and lets its
 * kernel end.  That call's outputs are then unspecified and must be
 * discarded, and the workspace must be zero-filled again before its next use.
 * The call itself still returns MHC_OK (it cannot know without waiting for
 * the device): a caller that must not consume a wrong result reads the two
 * words after the call's stream has drained (the Python binding's
 * check_workspace does this and raises). */
#define MHC_WS_FLAG_BYTES (192 * 1024)
#define MHC_WS_WAIT_ERROR_PERSIST 8
#define MHC_WS_WAIT_ERROR_SPLIT (96 * 1024 + 1024)

/* Test hook for the run-out path above.  sleeps > 0: every wait of later calls
 * of mhc_pre, mhc_pre_delayed, mhc_post_pre_delayed and mhc_broadcast_entry
 * counts as unsatisfied and is bounded by `sleeps` sleeps of 128 clocks, so
 * each call that waits at all reports a run-out (a call whose form has no
 * waits is unaffected).  sleeps == 0 restores the normal bound of 2^20 sleeps
 * (about a second).  Process-wide and read when a call is enqueued; not
 * synchronised with calls on other host threads.  MHC_ERR_SHAPE unless
 * 0 <= sleeps <= 2^20. */
mhc_status mhc_debug_force_wait_timeouts(int sleeps);

/* Pre stage, seam collapsed with its own pre-mix (p1 Purpose: the V4 form).
 *   x           [T][n][C] bf16    residual streams.
 *   norm_weight [C] bf16 or NULL  NULL: layer_input = bf16(y).  Otherwise the
 *                                 folded RMSNorm of p3 Measurements:
 *                                 layer_input = bf16((y * ry) * w), ry =
 *                                 1/sqrt(mean(y^2) + eps), evaluated in float
 *                                 and rounded once.
 *   eps         >= 0, used in the RMS of the projection and of the norm.
 *   sinkhorn_iters in [1, MHC_MAX_SINKHORN_ITERS]: rounds of (row normalise,
 *               column normalise) on exp(comb logits) (p1 Summary: 20
 *               iterations).
 *   pre  [T][n]    float out  sigmoid(l[0:4])
 *   post [T][n]    float out  2*sigmoid(l[4:8]), in (0,2)
 *   comb [T][n][n] float out  Sinkhorn(exp(l[8:24])), column sums 1
 *   layer_input [T][C] bf16 out  y_c = sum_i pre_i x_{i,c}, each product
 *               rounded to float and summed over i = 0..3 left to right.
 * Launches: one; past the one-sweep threshold (T > 4096 at C = 4096 and 5120,
 * T > 2048 at C = 7168), two: the gates, then the collapse with them (the
 * collapse needs this seam's gates). */
mhc_status mhc_pre(const uint16_t *x, int T, int n, int C, mhc_weights w,
                   const uint16_t *norm_weight, float eps, int sinkhorn_iters,
                   float *pre, float *post, float *comb, uint16_t *layer_input,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Pre stage of the delayed (V4.1) seam, p1 Purpose: the streams are collapsed
 * with the PREVIOUS seam's pre-mix pre_in[T][n] (float, device), and this
 * seam's pre-mix is returned in pre_out for the next seam.  The projection,
 * RMS, gates and Sinkhorn are those of mhc_pre (p1 Purpose: only the collapse
 * differs); so is everything else above. */
mhc_status mhc_pre_delayed(const uint16_t *x, const float *pre_in, int T, int n,
                           int C, mhc_weights w, const uint16_t *norm_weight,
                           float eps, int sinkhorn_iters, float *pre_out,
                           float *post, float *comb, uint16_t *layer_input,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Post stage (p1 Result, the mhc_post call sites):
 *   out[t][i][c] = bf16(post[t][i] * y[t][c] + sum_j comb[t][i][j] * x[t][j][c])
 * evaluated in float as fl(post_i * y) followed by one fused multiply-add per
 * j = 0..3 in order, rounded once (the same bits as mhc_post_pre_delayed's
 * x_out).  y [T][C] bf16 is the sublayer output,
 * x [T][n][C] bf16 the residual, post [T][n] and comb [T][n][n] float from
 * the pre stage.  out [T][n][C] bf16 may be exactly x (in place); any other
 * overlap is MHC_ERR_ALIAS.  No workspace. */
mhc_status mhc_post(const uint16_t *y, const uint16_t *x, const float *post,
                    const float *comb, int T, int n, int C, uint16_t *out,
                    void *stream);

/* Cross-seam fused form: the post stage of seam k and the delayed pre stage
 * of seam k+1 in one pass over the residual (p1 Notes / follow-ups: fewer
 * launches per seam; the delayed form makes it possible because the pre-mix
 * that collapses seam k+1 is seam k's, known before the pass).  The results
 * are those of mhc_post(y, x, post_in, comb_in) -> x_out followed by
 * mhc_pre_delayed(x_out, pre_in, ...): x_out bit for bit, layer_input without
 * the norm bit for bit; the gates, and the norm factor, up to the order in
 * which partial sums are added:
 *   y        [T][C] bf16      sublayer output of seam k.
 *   x        [T][n][C] bf16   residual entering seam k.
 *   post_in  [T][n] float     seam k's post gates; comb_in [T][n][n] float its comb.
 *   pre_in   [T][n] float     seam k's pre-mix, which collapses seam k+1.
 *   w, norm_weight, eps, sinkhorn_iters: seam k+1's, as in mhc_pre_delayed.
 *   x_out    [T][n][C] bf16 out  the residual entering seam k+1,
 *            bf16(post_i y + sum_j comb_in[i][j] x_j) evaluated in float as
 *            fl(post_i y) followed by one fused multiply-add per j in order and
 *            rounded once (the same bits as mhc_post).
 *   pre_out, post, comb, layer_input: seam k+1's outputs, from x_out, as in
 *            mhc_pre_delayed.
 * Launches: one; at hidden sizes other than 4096, 5120 and 7168 and T > 3072,
 * the post kernel and then the delayed pre kernel.  The
 * workspace is that of mhc_pre_delayed (mhc_workspace_bytes).  x_out must not
 * overlap x or any other argument: this form is not in place (MHC_ERR_ALIAS). */
mhc_status mhc_post_pre_delayed(const uint16_t *y, const uint16_t *x,
                                const float *post_in, const float *comb_in,
                                const float *pre_in, int T, int n, int C,
                                mhc_weights w, const uint16_t *norm_weight,
                                float eps, int sinkhorn_iters, uint16_t *x_out,
                                float *pre_out, float *post, float *comb,
                                uint16_t *layer_input, void *workspace,
                                size_t workspace_bytes, void *stream);

/* mhc_post_pre_delayed for callers that cannot allocate device memory or
 * bring a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments and results are those of
 * mhc_post_pre_delayed (same kernels, same bits) without the workspace pair:
 * the exchange workspace is a buffer of MHC_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on each GPU it runs on until the process
 * ends.  The call allocates nothing; the first call on a device looks up that
 * device's buffer and enqueues a clear of its flag region on `stream`.
 * Every shape mhc_post_pre_delayed accepts fits the buffer (the largest need
 * is the persistent kernels' at C = 7168, about 7.8 MB); a call whose plan
 * would need more returns MHC_ERR_WORKSPACE.  All calls on one GPU share the
 * buffer: calls that overlap on a device (other streams, other host threads
 * without ordering between them) race and give unspecified results.  The
 * waits of this form are bounded as described above; a run-out here is not
 * reported (the wait-error words live in the shared buffer) and
 * mhc_debug_force_wait_timeouts does not apply to it. */
#define MHC_NOALLOC_SCRATCH_BYTES (8u << 20)
mhc_status mhc_post_pre_delayed_noalloc(const uint16_t *y, const uint16_t *x,
                                        const float *post_in, const float *comb_in,
                                        const float *pre_in, int T, int n, int C,
                                        mhc_weights w, const uint16_t *norm_weight,
                                        float eps, int sinkhorn_iters, uint16_t *x_out,
                                        float *pre_out, float *post, float *comb,
                                        uint16_t *layer_input, void *stream);

/* Model-entry seam (p1 Summary and Approach: the broadcast seam projects a
 * narrower operand).  The single stream h[T][C] bf16 is broadcast to all n
 * streams, x_out[t][i][:] = h[t][:]; the logits come from h . fn_e with the
 * entry weight fn_e[C][24] (packed with K = C) and r = 1/sqrt(mean(h^2) + eps)
 * over C, which equals the RMS of the broadcast row.  Gates, Sinkhorn and the
 * collapse (with this seam's own pre-mix) are those of mhc_pre applied to
 * x_out.  layer_input may be NULL (not written).  pre is carried into the
 * first delayed seam. */
mhc_status mhc_broadcast_entry(const uint16_t *h, int T, int n, int C,
                               mhc_weights w_entry, const uint16_t *norm_weight,
                               float eps, int sinkhorn_iters, uint16_t *x_out,
                               float *pre, float *post, float *comb,
                               uint16_t *layer_input, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Standalone collapse (p1 Result: the collapse also runs on its own at other
 * call sites of the model, where no projection is needed):
 *   x           [T][n][C] bf16    residual streams.
 *   p           [T][n] float      mixing weights (a pre-mix).
 *   norm_weight [C] bf16 or NULL  as in mhc_pre: NULL gives out = bf16(y);
 *                                 otherwise out = bf16((y * ry) * w) with
 *                                 ry = 1/sqrt(mean(y^2) + eps).
 *   eps         >= 0 (used only with norm_weight).
 *   out         [T][C] bf16 out   y_c = sum_i p_i x_{i,c}, each product rounded
 *               to float and summed over i = 0..3 left to right: without the
 *               norm, bit-identical to mhc_pre_delayed's layer_input for
 *               pre_in = p.
 * No workspace.  out must not overlap x, p or norm_weight (MHC_ERR_ALIAS). */
mhc_status mhc_collapse(const uint16_t *x, const float *p, int T, int n, int C,
                        const uint16_t *norm_weight, float eps, uint16_t *out,
                        void *stream);

/* Static, human-readable name of a status code. */
const char *mhc_status_str(mhc_status s);

#ifdef __cplusplus
}
#endif
#endif /* MHC_H */

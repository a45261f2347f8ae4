/*
 * saf_hybrid.h -- C ABI of the SAF hybrid attention library for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The layer is one causal multi-head attention pass with two kinds of head
 * ("When Can Attention Heads Be Statically Defined?", Section 3.3 "Fused
 * computation" and Appendix D.2):
 *
 *   ordinary head (Appendix A.1, Equations 5-7):
 *       S = s * Q K^T, A = causal row softmax of S, O = A V,
 *       s = softmax_scale (default 1/sqrt(D));
 *   frozen head (Section 3.2, Equation 3):
 *       W[i][j] = exp(a[j] + r[i-j]) / N(i) for j <= i, 0 for j > i,
 *       N(i) = sum_{k<=i} exp(a[k] + r[i-k]),  O = W V.
 *       Q and K of a frozen head are never read; the logits carry no scale.
 *
 * Indices are 0-based: a[j] is the pages' alpha(j+1) and r[d] is rho(d).
 * Backward (Section 3.3 and Appendix D.2): ordinary heads get dQ, dK, dV of
 * the softmax attention; frozen heads get dV = W^T dO and exact +0.0 in their
 * dQ and dK slices (a frozen head has no query/key slot).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates device memory; scratch space is passed in as a
 *    workspace sized by saf_hybrid_attn_workspace_bytes().
 *  - Q, K, V, O, dO, dQ, dK, dV have logical shape [B][H][T][D] (K and V:
 *    [B][Hkv][T][D] with grouped-query attention, see kv_heads).  Their
 *    element strides for (b, h, t) are given per tensor; the stride of the
 *    last (d) dimension must be 1.  Base pointers must be 16-byte aligned
 *    and each (b, h, t) stride a multiple of 16 bytes.  The t stride may
 *    not exceed SAF_MAX_T_STRIDE elements (SAF_EUNSUPPORTED otherwise).
 *  - a and r are fp32 [H][prior_len] (row stride prior_len, prior_len >= T);
 *    rows of ordinary heads are never read.  Only entries [0, T) of a row are
 *    used, which is exact: causal rows never reach further.
 *  - lse is fp32 [B][H][T] contiguous.  For an ordinary head it holds the
 *    natural-log log-sum-exp of row i of s*QK^T; for a frozen head it holds
 *    log N(i) (the same for every b).  The forward writes it, the backward
 *    reads it.
 *  - dtype SAF_BF16: Q, K, V, dO and all outputs are bfloat16; products run
 *    on bf16 MFMA with fp32 accumulation, softmax and pattern weights are
 *    computed in fp32 and rounded to nearest-even bf16 before the second
 *    product.  dtype SAF_F32: everything is fp32.
 *  - Every argument is validated before anything is enqueued; on error
 *    nothing is launched and outputs are untouched.  The return value is a
 *    status code (SAF_OK or a negative SAF_E* value).
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream) and
 *    the call never synchronises.  A failed launch returns SAF_EHIP; faults
 *    inside a kernel surface at the caller's next synchronisation.
 *  - Apart from the scratch array of saf_hybrid_attn_fwd_noalloc and a
 *    per-device record of which kernels' LDS attribute is set (atomic), the
 *    library has no mutable global state; concurrent calls on different
 *    streams are safe.  Results are bitwise deterministic (no atomics), except dQ of the
 *    fused-dQ backward schedule (saf_attn_params.fused_dq).
 *  - Calls may be recorded by stream capture into a HIP graph: they enqueue
 *    kernel launches only (plus event records when stage events are asked
 *    for), allocate nothing and issue no memset.  Make one call with the
 *    same head dimension and dtype outside capture first on each device: it
 *    sets each kernel's LDS size attribute once per device (a failed attempt
 *    is not remembered and is retried by the next call).
 */
#ifndef SAF_HYBRID_H
#define SAF_HYBRID_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SAF_OK 0
#define SAF_EINVAL (-1)       /* bad pointer, size, stride or alignment */
#define SAF_EUNSUPPORTED (-2) /* valid but not implemented: D, dtype, H */
#define SAF_EWORKSPACE (-3)   /* workspace missing or too small */
#define SAF_EHIP (-4)         /* a HIP launch or runtime call failed */
#define SAF_ESCRATCH (-5)     /* saf_hybrid_attn_fwd_noalloc: the shape needs more
                                 than SAF_NOALLOC_SCRATCH_BYTES of scratch */

/* Element types of Q, K, V, O, dO, dQ, dK, dV. */
#define SAF_F32 0
#define SAF_BF16 1

/* Limits. */
#define SAF_MAX_HEADS 256
#define SAF_MAX_T (1 << 20)
#define SAF_MAX_T_STRIDE (1 << 24) /* elements between consecutive rows */
/* Scratch each GPU holds for saf_hybrid_attn_fwd_noalloc (32 MiB). */
#define SAF_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
/* Also rejected with SAF_EUNSUPPORTED: B * H * T > 2^40; for bf16,
 * B * H * ceil(T / 128) > 2^31 - 1 (programs per launch); for fp32,
 * B * H > 65535. */

/*
 * Shape, layout and head-state description of one call.
 * Fill every field; set struct_bytes = sizeof(saf_attn_params) (checked, so
 * that a binding with a different layout is rejected instead of misread).
 */
typedef struct saf_attn_params {
  uint32_t struct_bytes;
  int32_t B, H, T, D;       /* D in {64, 96, 128} for bf16; {16, 32, 64, 96, 128} for fp32 */
  int32_t prior_len;        /* stored length of each a/r row, >= T */
  int32_t dtype;            /* SAF_F32 or SAF_BF16 */
  float softmax_scale;      /* ordinary heads; <= 0 selects 1/sqrt(D) */
  /* element strides of dimensions (b, h, t); the d stride is 1 */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  int64_t do_stride[3], dq_stride[3], dk_stride[3], dv_stride[3];
  /* HOST array [H]: 1 = frozen head, 0 = ordinary head (the per-head state
   * flag of Section 3.3).  Read during the call only. */
  const uint8_t* frozen;
  /* Optional instrumentation: a HOST array of n_stage_events events created
   * by the caller.  When non-NULL, event 0 is recorded on `stream` before the
   * first kernel and event k after the k-th kernel of the call (k <= n-1);
   * kernels beyond n-1 are not bracketed.  Nothing is skipped or changed. */
  hipEvent_t* stage_events;
  int32_t n_stage_events;
  /* Key/value heads Hkv (grouped-query attention, the pages' Qwen path in
   * Appendix D.2): query head h reads key/value head h / (H / Hkv).  0 means
   * H (multi-head attention).  Otherwise 1 <= Hkv <= H and Hkv divides H; K
   * and V are then [B][Hkv][T][D] (their h strides step over key/value
   * heads).  Grouped-query layouts are supported by saf_hybrid_attn_fwd only
   * (prefill); the backward and saf_pattern_grad return SAF_EUNSUPPORTED. */
  int32_t kv_heads;
  /* Optional precomputed row normalisers of the frozen heads (the log Z the
   * paper stores with alpha and rho, Section 3.3 and Appendix D.2): a DEVICE
   * fp32 array [H][T], row h = log N of head h over rows 0..T-1, as
   * saf_pattern_lognorm writes it for the rows of a and r (rows of ordinary
   * heads are not read).  When non-NULL, saf_hybrid_attn_fwd reads it instead
   * of computing the normalisers (no normaliser kernel, no workspace) and
   * copies it into the frozen rows of lse; it must be the normaliser of the
   * a and r passed, which the library does not check.  NULL: computed by the
   * call.  Read by saf_hybrid_attn_fwd only. */
  const float* logz;
  /* Q/K layout (the pages give replaced heads no query or key slot, Section
   * 3.3 and Appendix D.2).  0: q, k, dq and dk have all H heads; frozen
   * heads' q, k are not read and their dq, dk slices are written +0.0.
   * 1 (packed): q and dq hold only the ordinary heads, in increasing head
   * order (slot s = the s-th ordinary head); so do k and dk with multi-head
   * K/V, while with kv_heads < H, k keeps its kv_heads key/value heads.
   * Nothing is read or written for frozen heads there (with no ordinary
   * head, q, k, dq and dk may be NULL).  v, o, dO and dV always have all
   * heads.  Strides of the packed tensors step over their own heads. */
  int32_t qk_packed;
  /* Backward schedule (saf_hybrid_attn_bwd; ignored by the other calls).
   * 0: two passes -- a query-block pass writes dQ, a key-block pass writes dK
   *    and dV; results are bitwise reproducible.
   * 1: fused dQ (bf16 with D = 64 only; otherwise SAF_EUNSUPPORTED) -- the
   *    key-block pass also accumulates dQ into an fp32 workspace with atomic
   *    adds (no query-block pass, which recomputes the scores); dK and dV are
   *    bitwise reproducible, dQ is not (its summation order varies).  The
   *    workspace grows by B * n_ordinary * T * D * 4 bytes. */
  int32_t fused_dq;
} saf_attn_params;

/*
 * Forward pass of the hybrid layer (Section 3.3 "Fused computation";
 * Appendix D.2): O in the original head order and lse.
 *   q, k, v : device [B][H][T][D] (strided as in p); frozen heads' q, k are
 *             not read and may hold anything (also NaN).
 *   a, r    : device fp32 [H][prior_len].
 *   o       : device [B][H][T][D] output.
 *   lse     : device fp32 [B][H][T] output (see conventions above).
 *   ws      : workspace of at least saf_hybrid_attn_workspace_bytes(p, 0)
 *             bytes, 256-byte aligned (may be NULL when that is 0).  bf16
 *             with frozen heads needs n_frozen * G * T * 8 bytes (rounded
 *             up to 256) for partial sums of the row normalisers over G key
 *             groups, G = ceil(T / K) with K the smallest multiple of 256
 *             that is >= T / 32 (so G <= 32); fp32, or no frozen head,
 *             needs none.
 *             Contents on entry are ignored and left undefined on return.
 * Kernels: the frozen heads' row normalisers (bf16: chunk partials, merged
 * by the frozen programs of the next launch; skipped when p->logz is given),
 * then one mixed-head launch.
 */
int saf_hybrid_attn_fwd(const saf_attn_params* p, const void* q, const void* k,
                        const void* v, const float* a, const float* r, void* o,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * saf_hybrid_attn_fwd for callers that cannot allocate device memory or pass
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, layout, semantics and results as
 * saf_hybrid_attn_fwd (the same kernels; bitwise the same outputs), minus the
 * workspace: the normaliser partials live in a static scratch array of
 * SAF_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends.  The call allocates nothing and issues no memset.
 *   - A shape whose forward needs more scratch than that (bf16 with frozen
 *     heads: about n_frozen * 32 * T * 8 bytes at most, see ws above; e.g.
 *     3 frozen heads at T = 32768 need 25.2 MB) is rejected with
 *     SAF_ESCRATCH before anything is enqueued.  fp32, no frozen head or a
 *     given p->logz need no scratch.
 *   - The scratch of the CURRENT device is used; `stream` must belong to it.
 *     The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress); make it outside stream capture.
 *   - Every call on a GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that
 *     overlap in time on one GPU (other streams, other host threads) race
 *     and must be serialised by the caller.
 */
int saf_hybrid_attn_fwd_noalloc(const saf_attn_params* p, const void* q, const void* k,
                                const void* v, const float* a, const float* r, void* o,
                                float* lse, hipStream_t stream);

/*
 * Backward pass of the hybrid layer (Section 3.3; Appendix D.2 key-block and
 * query-block passes).  Given dO and the forward's o and lse, writes
 *   dq, dk : ordinary heads' gradients; frozen heads' slices := +0.0
 *            (packed layout, p->qk_packed: no slices for frozen heads);
 *   dv     : gradients of every head (frozen: W^T dO).
 * q, k of frozen heads are not read.  o is read for ordinary heads only.
 * ws: at least saf_hybrid_attn_workspace_bytes(p, 1) bytes, 256-byte aligned.
 * Kernels (bf16): with p->fused_dq = 0, the query-block pass (dQ and the
 * rows' delta = sum_d dO O) then one mixed-head key-block launch; with
 * p->fused_dq = 1, a delta pass (which also clears the dQ accumulator), one
 * mixed-head key-block launch that also accumulates dQ, and the dQ
 * conversion to bf16.
 */
int saf_hybrid_attn_bwd(const saf_attn_params* p, const void* q, const void* k,
                        const void* v, const void* o, const void* dout,
                        const float* lse, const float* a, const float* r,
                        void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Workspace bytes a call with these parameters needs (0 if none; the
 * forward needs none when p->logz is given);
 * for_bwd = 0 for the forward, 1 for the backward.  Returns 0 for invalid p. */
size_t saf_hybrid_attn_workspace_bytes(const saf_attn_params* p, int for_bwd);

/*
 * Gradients of the frozen heads' pattern parameters, for the variant that
 * keeps training a and r (Appendix C.3.2 "Pattern content and
 * trainability"; pattern of Section 3.2, Equation 3).  For every frozen head
 * h, with W the compact pattern (row softmax of G[i][j] = a[j] + r[i-j] over
 * j <= i), dW_b = dO_b V_b^T, D_b[i] = sum_d dO_b[i][d] O_b[i][d] and
 * dG_b[i][j] = W[i][j] (dW_b[i][j] - D_b[i]) (the chain rule through the row
 * softmax, normaliser included):
 *   da[h][j] = sum_b sum_{i >= j} dG_b[i][j]       (column sums, 0 <= j < T)
 *   dr[h][d] = sum_b sum_{i >= d} dG_b[i][i - d]   (diagonal sums, 0 <= d < T)
 * and entries [T, prior_len) of these rows are set to 0.  Rows of ordinary
 * heads are not written; with no frozen head nothing is launched.
 *   v, o, dout : device [B][H][T][D] (o: the forward's output for these
 *                inputs); strides from p (v_stride, o_stride, do_stride).
 *                Only frozen heads' slices are read.
 *   lse        : device fp32 [B][H][T] from the forward (log N on frozen rows).
 *   a, r       : device fp32 [H][prior_len] (the parameters the forward used).
 *   da, dr     : device fp32 [H][prior_len] outputs.
 *   ws         : at least saf_pattern_grad_workspace_bytes(p) bytes, 256-byte
 *                aligned: per-row D_b, and per key block and batch group
 *                partial sums, reduced in a fixed order (no atomics; results
 *                are bitwise deterministic).
 * After the parameters change, the next forward call recomputes the
 * normalisers (saf_pattern_lognorm gives them alone).
 */
int saf_pattern_grad(const saf_attn_params* p, const void* v, const void* o, const void* dout,
                     const float* lse, const float* a, const float* r, float* da, float* dr,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes saf_pattern_grad needs (0 for invalid p or no frozen head). */
size_t saf_pattern_grad_workspace_bytes(const saf_attn_params* p);

/*
 * Dense compact pattern of one frozen head (Section 3.2, Equation 3), as an
 * eager reference: w[i][j] = exp(a[j] + r[i-j] - log N(i)) for j <= i and 0
 * above the diagonal.
 *   a, r : device fp32, at least prior_len (>= T) entries each.
 *   w    : device fp32 [T][T] row-major output (T*T*4 bytes).
 * T must be in [1, 32768].
 */
int saf_pattern_dense(int32_t T, int32_t prior_len, const float* a,
                      const float* r, float* w, hipStream_t stream);

/*
 * Row normalisers of frozen patterns (Section 3.2, Equation 3), computed
 * with a max-shifted log-sum-exp:
 *   logz[h][i] = log sum_{k<=i} exp(a[h][k] + r[h][i-k]),  0 <= i < T,
 * for n_heads rows of a, r (device fp32 [n_heads][prior_len]) into logz
 * (device fp32 [n_heads][T]).
 */
int saf_pattern_lognorm(int32_t n_heads, int32_t T, int32_t prior_len,
                        const float* a, const float* r, float* logz,
                        hipStream_t stream);

/*
 * Compact-pattern fitting ("When Can Attention Heads Be Statically
 * Defined?": Algorithm 1, which prepares a target from a head's calibration
 * mean, fits a and r, and accepts the fit by its row-averaged KL divergence;
 * Section 3.2 "Fitting", Equation 4; Appendix A.2 "Selection, fitting, and
 * installation"; Appendix D.1, Equation 20).
 */
#define SAF_MAX_FIT_HEADS 16384

/*
 * Target statistics of n_heads calibration means A (fp32 [T][T] each, the
 * average causal attention of one head; entries above the diagonal are never
 * read).  With P[i][j] = max(A[i][j], floor) / sum_{k<=i} max(A[i][k], floor)
 * for j <= i (the floored, row-normalised target):
 *   eta_abs[h][j] = sum_{i>=j} P[i][j]        (column sums, 0 <= j < T)
 *   eta_rel[h][d] = sum_{i>=d} P[i][i-d]      (diagonal sums, 0 <= d < T)
 *   negent[h]     = sum_i sum_{j<=i} P[i][j] ln P[i][j]
 * the sufficient statistics of the fit and of its acceptance test.
 *   ahat        : device fp32; row i of head h starts at
 *                 ahat + h * head_stride + i * row_stride (elements);
 *                 4-byte aligned, row_stride >= T, head_stride >= 0.  Rows
 *                 that start 16-byte aligned are read 16 bytes at a time.
 *   floor       : > 0 and finite (the pages floor at 1e-9).
 *   eta_abs, eta_rel : device fp32 [n_heads][T] outputs.
 *   negent      : device fp32 [n_heads] output.
 *   ws          : saf_fit_targets_workspace_bytes(n_heads, T) bytes,
 *                 256-byte aligned: row sums and entropies, and partial
 *                 marginals over row segments, summed in a fixed order
 *                 (results are bitwise deterministic).
 * Each row is accumulated in fp32; negent sums the rows in fp64.
 * n_heads in [1, SAF_MAX_FIT_HEADS], T in [1, SAF_MAX_T].
 */
int saf_fit_targets(int32_t n_heads, int32_t T, const float* ahat, int64_t head_stride,
                    int64_t row_stride, float floor, float* eta_abs, float* eta_rel,
                    float* negent, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes saf_fit_targets needs (0 for invalid sizes). */
size_t saf_fit_targets_workspace_bytes(int32_t n_heads, int32_t T);

/*
 * Fit one compact pattern per head to target marginals.  Each head starts
 * from a = 0 and r[d] = ln max(eta_rel[d] / (T - d), 1e-9) and takes `steps`
 * Adam steps (Kingma & Ba: moment decays beta1 and beta2, bias-corrected
 * moments, eps added to the square root of the second moment; the pages use
 * 400 steps at lr 0.05 with no early stopping) on Equation 4,
 *   L(a, r) = (1/T) [ sum_i ln N(i) - sum_j eta_abs[j] a[j]
 *                     - sum_d eta_rel[d] r[d] ],
 *   N(i) = sum_{k<=i} exp(a[k] + r[i-k]),
 * whose gradient is (fitted marginal - target marginal) / T for both
 * vectors (Equation 20); a and r are updated from the gradient at the same
 * point.
 *   eta_abs, eta_rel : device fp32 [n_heads][T] (saf_fit_targets).
 *   negent      : device fp32 [n_heads] or NULL; needed for kappa.
 *   a, r        : device fp32 [n_heads][T] outputs: the fitted parameters.
 *   logz        : device fp32 [n_heads][T] output: ln N(i) of the fitted
 *                 pattern (saf_attn_params.logz takes it, in [H][T] rows).
 *   loss        : device fp32 [n_heads] output or NULL: L at the result.
 *   kappa       : device fp32 [n_heads] output or NULL: negent / T + L,
 *                 the row-averaged KL divergence of the fitted pattern from
 *                 the target (the pages accept a fit when kappa <= 0.2 nats;
 *                 the decision is the caller's).
 *   ws          : saf_fit_pattern_workspace_bytes(n_heads, T) bytes,
 *                 256-byte aligned: a second parameter buffer and the four
 *                 Adam moment vectors.
 * steps >= 0; lr > 0; beta1, beta2 in [0, 1); eps > 0; all finite.
 * Arithmetic is fp32 (loss and kappa are summed in fp64).  Two kernels are
 * launched per step; on SAF_EHIP the outputs are unspecified.
 */
int saf_fit_pattern(int32_t n_heads, int32_t T, const float* eta_abs, const float* eta_rel,
                    const float* negent, int32_t steps, float lr, float beta1, float beta2,
                    float eps, float* a, float* r, float* logz, float* loss, float* kappa,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes saf_fit_pattern needs (0 for invalid sizes). */
size_t saf_fit_pattern_workspace_bytes(int32_t n_heads, int32_t T);

/*
 * Calibration statistics of attention heads ("When Can Attention Heads Be
 * Statically Defined?", Section 3.1, Equations 1 and 2; Algorithm 1 measures
 * them before fitting).  For each of H heads, over N calibration sequences,
 * with A^(n) the causal row softmax of s * Q^(n) K^(n)T (Appendix A.1,
 * Equations 5-6; s = softmax_scale, or 1/sqrt(D) when softmax_scale <= 0):
 *   ahat[h][i][j] = N^-1 sum_n A^(n)[i][j]                      for j <= i
 *   s_var[h] = sum_n sum_{i,j} (A^(n)[i][j] - ahat[i][j])^2 / ((N - 1) T^2)
 *              (0 when N = 1)
 *   s_kl[h]  = (N T)^-1 sum_n sum_i KL(A^(n)[i][0..i] || ahat[i][0..i])
 * in one pass over the sequences without storing any A^(n): every entry's
 * sums of deviations from its first sequence's value are kept on chip
 * (mean and squared deviations follow from them), and the KL sum uses
 * sum_n KL = sum_n sum A ln A - N sum ahat ln ahat.  Entries above the diagonal of ahat are not written.
 *   q, k        : device bf16 [N][H][T][D] with element strides
 *                 (sequence, head, row) in q_stride / k_stride; last
 *                 dimension contiguous; 16-byte aligned, strides multiples
 *                 of 8 elements, row stride at most SAF_MAX_T_STRIDE.
 *   ahat        : device fp32 output; row i of head h at
 *                 ahat + h * ahat_head_stride + i * ahat_row_stride;
 *                 4-byte aligned, row stride >= T, head stride >= 0 (rows
 *                 that all start 16-byte aligned are written 16 bytes at a
 *                 time).
 *   s_var, s_kl : device fp64 [H] outputs.
 *   ws          : saf_calib_stats_workspace_bytes(N, H, T) bytes, 256-byte
 *                 aligned: row log-sum-exps and per-program partial sums
 *                 (reduced in a fixed order: bitwise deterministic).
 * Scores and probabilities are fp32 (bf16 products on MFMA); partial sums of
 * the scores are fp64.  D in {64, 96, 128}; N in [1, 65535]; H in
 * [1, 65535]; T in [1, SAF_MAX_T].
 */
int saf_calib_stats(int32_t N, int32_t H, int32_t T, int32_t D, float softmax_scale,
                    const void* q, const int64_t q_stride[3], const void* k,
                    const int64_t k_stride[3], float* ahat, int64_t ahat_head_stride,
                    int64_t ahat_row_stride, double* s_var, double* s_kl, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Workspace bytes saf_calib_stats needs (0 for invalid sizes). */
size_t saf_calib_stats_workspace_bytes(int32_t N, int32_t H, int32_t T);

/* Static description of a status code (never NULL). */
const char* saf_status_string(int status);

/* Library version as (major << 16) | minor. */
int32_t saf_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAF_HYBRID_H */

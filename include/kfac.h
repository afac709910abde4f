/*
 * kfac.h -- C ABI of the MI355X (gfx950) K-FAC optimizer-step library.
 *
 * One optimizer step for a stack of layers, run on one GPU by hand-written
 * HIP kernels.  Two methods are provided:
 *
 *   kfac_step_full  K-FAC (Osawa et al., "Large-Scale Distributed
 *                   Second-Order Optimization Using Kronecker-Factored
 *                   Approximate Curvature for Deep Convolutional Neural
 *                   Networks", section 3.2): per layer, Kronecker factors
 *                   A = a^T a / N from the layer's inputs and G = g^T g / N from
 *                   its output gradients, an exponential moving average of
 *                   each, damped inverses (A + lambda I)^-1 and
 *                   (G + lambda I)^-1 (section 4.2: damping) refreshed when the
 *                   caller asks (sections 1 and 5.4: refreshed less often than
 *                   every step), the direction P = G^-1 grad_W A^-1, then
 *                   momentum, weight decay and the in-place parameter write.
 *
 *   kfac_step_diag  the AdaFisher-style diagonal variant (CAFIN briefing,
 *                   "Introduction" and "Kernel Fusion Strategy"): per-parameter
 *                   EMA of dG[o] * dA[j] (the diagonal of G kron A), division of
 *                   the gradient by (F + lambda), momentum, weight decay and the
 *                   parameter write, fused into one elementwise pass.
 *
 * Per step and layer (both methods; W, V, grad are the bias-augmented
 * [d_out x d_a] matrices [W | b] etc., the bias as the last column):
 *     D = P + weight_decay * W;   V = momentum * V + D;   W = W - lr * V
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers inside kfac_layer_t are DEVICE pointers to
 *    contiguous, 16-byte aligned buffers owned by the caller.  The library
 *    keeps no pointer after a call returns and frees nothing of the caller's.
 *  - `workspace` is a device buffer of at least kfac_workspace_size() bytes,
 *    256-byte aligned, owned by the caller.  One workspace must not be used
 *    by two calls that can run at the same time; its first 256 bytes hold the
 *    sticky device flag word (see kfac_read_flags) and must be zeroed by the
 *    caller once before first use (the library never clears it on its own).
 *  - `stream` is a hipStream_t (NULL = the default stream).  The step entry
 *    points only enqueue work on it and return; they never synchronise.
 *  - Arguments are validated on the host before anything is enqueued: on a
 *    validation error (KFAC_ERR_ARG, _DTYPE, _ALIGN, _WORKSPACE,
 *    _UNSUPPORTED) no kernel runs and no buffer is touched.  KFAC_ERR_HIP
 *    means a HIP call failed while the step was being enqueued: part of the
 *    step may have been enqueued (the library's side streams are still joined
 *    back into `stream` before the call returns), so the buffers are then in
 *    an unspecified state.
 *  - Numerical trouble (a damped factor that is not positive definite, a
 *    non-finite parameter) is reported through device flags, never through a
 *    return code, because it is only known once the kernels have run.
 *  - Calls on different workspaces and streams may be made from different
 *    host threads.  A full-method step forks work onto two side streams of
 *    the library and joins it back into `stream`; those side streams belong
 *    to the pair (device, `stream`): they are created at the first full step
 *    on that stream and kept until the process ends, and calls on the same
 *    stream are enqueued one at a time (an internal lock).  Steps on other
 *    streams never use them, so a step captured into a graph on one stream
 *    and steps run on other streams meanwhile stay apart.  The first full
 *    step on a stream must not be made while that stream is capturing (the
 *    side streams and events cannot be created then): it returns
 *    KFAC_ERR_UNSUPPORTED.
 */
#ifndef KFAC_H
#define KFAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KFAC_ABI_VERSION 2

typedef int32_t kfac_status_t;
enum {
  KFAC_OK = 0,
  KFAC_ERR_ARG = 1,          /* null pointer, bad count, inconsistent shape */
  KFAC_ERR_DTYPE = 2,        /* dtype code not supported for that operand */
  KFAC_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned (workspace: 256) */
  KFAC_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
  KFAC_ERR_UNSUPPORTED = 5,  /* valid request this build does not implement */
  KFAC_ERR_HIP = 6           /* a HIP launch or runtime call failed */
};

/* layer kinds */
enum { KFAC_LINEAR = 0, KFAC_CONV2D = 1, KFAC_BATCHNORM = 2 };
/* kfac_layer_t.factor_layout: storage of A and G (full method) */
enum { KFAC_FACTORS_FULL = 0, KFAC_FACTORS_PACKED = 1 };
/* element types of a / g (every other tensor is float32) */
enum { KFAC_F32 = 0, KFAC_BF16 = 1 };
/* kfac_workspace_size modes */
enum { KFAC_MODE_FULL = 0, KFAC_MODE_DIAG = 1 };
/* kfac_hparams_t.phase_mask bits; 0 means all phases.  RESCALE = the weight
 * rescaling (runs only when options has KFAC_OPT_RESCALE; after UPDATE).
 *   full: FACTORS = factor construction + EMA, INVERT = damped inverses
 *         (only when refresh != 0), UPDATE = precondition + momentum/decay/write
 *   diag: FACTORS = dA, dG of this batch (a streaming reduction of a and g
 *         through the workspace), written to the descriptor's dA / dG for
 *         every layer kind; UPDATE = the fused elementwise step, which reads
 *         dA / dG from those buffers (so an UPDATE-only call uses whatever
 *         they hold, e.g. the last FACTORS call's result). */
enum { KFAC_PHASE_FACTORS = 1, KFAC_PHASE_INVERT = 2, KFAC_PHASE_UPDATE = 4, KFAC_PHASE_RESCALE = 8,
       KFAC_PHASE_ALL = 15 };
/* kfac_hparams_t.refresh bits (full method): which damped inverses this step
 * recomputes */
enum { KFAC_REFRESH_A = 1, KFAC_REFRESH_G = 2, KFAC_REFRESH_BOTH = 3 };
/* kfac_hparams_t.options bits */
enum { KFAC_OPT_RESCALE = 1 };
/* sticky device flags */
enum { KFAC_FLAG_NOT_PD = 1u, KFAC_FLAG_NONFINITE = 2u };

/*
 * One layer.  Shapes (row-major, contiguous):
 *   linear : a [rows, d_in]           g [rows, d_out]          rows = N
 *   conv2d : a [batch, c_in, height, width]   g [batch, d_out, h_out, w_out] (NCHW)
 *            d_in = c_in * kh * kw (weights [d_out, c_in, kh, kw] flattened in
 *            (c, kh, kw) order), h_out = (height + 2 pad - kh) / stride + 1 (same for
 *            width), rows = batch * h_out * w_out; dilation 1, groups 1.
 *   d_a = d_in + (has_bias ? 1 : 0)   (the bias acts as a constant-1 input,
 *                                      appended as the last column)
 *   batchnorm: the affine parameters gamma, beta of a batch-norm layer over
 *            C channels (Osawa et al. section 1, "Curvature approximation",
 *            and section 5.4: a diagonal Fisher for batch normalisation).
 *            a = the normalised input x_hat [batch, C, height, width], g = the
 *            per-sample output gradient [batch, C, height, width] (float32);
 *            d_out = c_in = C, d_in = 1, rows = batch, kh = kw = stride = 1,
 *            pad = 0; w = gamma, b = beta (has_bias), grad_w / grad_b their
 *            gradients, all [C].  Both methods treat it the diagonal way:
 *            dA[c] = mean_b (sum_hw g x_hat)^2 and dG[c] = mean_b (sum_hw g)^2
 *            (the Fisher diagonal of gamma and of beta from per-sample
 *            gradients), F_w / F_b their EMA, damping_bn in place of damping.
 *   Full method: a layer with float32 a or g, and every conv2d layer, has at
 *   most INT32_MAX rows (KFAC_ERR_UNSUPPORTED otherwise).
 *   grad_w, w, mom_w, F_w : [d_out, d_in] float32
 *   grad_b, b, mom_b, F_b : [d_out] float32, NULL iff has_bias == 0
 * Full method:  A, A_inv : [d_a, d_a]; G, G_inv : [d_out, d_out]  (float32,
 *               symmetric; the library reads the upper triangle of A and G).
 *               With factor_layout KFAC_FACTORS_FULL, A and G are stored
 *               whole and the library writes both triangles; with
 *               KFAC_FACTORS_PACKED only the upper triangle is stored, row
 *               after row: element (i, j), i <= j, at i d - i (i - 1) / 2 +
 *               (j - i), d (d + 1) / 2 floats (section 3.4: a symmetric factor
 *               is carried as its N (N + 1) / 2 upper entries).  A, G are
 *               updated in place every step; A_inv, G_inv (always whole) are
 *               written on refresh steps and read every step; the UPDATE phase
 *               reads them as symmetric matrices (either triangle, rows in
 *               place of columns), so inverses a caller supplies must be
 *               symmetric too.  Batch-norm layers use F_w, F_b, dA, dG [C]
 *               instead (no factors).
 * Diag method:  F_w, F_b updated in place; dA [d_a], dG [d_out] are written by
 *               the FACTORS phase and read by the UPDATE phase.
 * Pointers a method does not use may be NULL.  w, mom_w, b, mom_b are updated
 * in place; a, g, grad_w, grad_b are only read.
 */
typedef struct kfac_layer {
  int32_t kind;        /* KFAC_LINEAR | KFAC_CONV2D */
  int32_t has_bias;    /* 0 | 1 */
  int32_t act_dtype;   /* KFAC_F32 | KFAC_BF16 (element type of a) */
  int32_t grad_dtype;  /* KFAC_F32 | KFAC_BF16 (element type of g) */
  int64_t rows;        /* N */
  int32_t d_in;
  int32_t d_out;
  int32_t batch, c_in, height, width, kh, kw, stride, pad;   /* conv2d and batchnorm */
  int32_t factor_layout;   /* KFAC_FACTORS_FULL | KFAC_FACTORS_PACKED (full method) */
  int32_t reserved;        /* must be 0 */
  const void* a;
  const void* g;
  const float* grad_w;
  const float* grad_b;
  float* w;
  float* b;
  float* mom_w;
  float* mom_b;
  float* A;
  float* G;
  float* A_inv;
  float* G_inv;
  float* F_w;
  float* F_b;
  float* dA;
  float* dG;
} kfac_layer_t;

/* Per-call scalars.  Schedules (warm-up damping, learning-rate decay, the
 * inverse-refresh policy) live with the caller: it passes this step's values
 * (kfac_schedule_hparams below computes the damping and refresh ones). */
typedef struct kfac_hparams {
  float lr;
  float momentum;
  float weight_decay;
  float ema_decay;     /* full: factor EMA decay; diag and batch-norm layers: F EMA decay */
  float damping;       /* lambda of the conv / linear layers */
  float damping_bn;    /* lambda of the batch-norm layers */
  float rescale_eps;   /* epsilon of the weight rescaling (KFAC_OPT_RESCALE) */
  int32_t refresh;     /* full: KFAC_REFRESH_* bits, the damped inverses recomputed this step */
  int32_t phase_mask;  /* KFAC_PHASE_* bits, 0 = all */
  int32_t options;     /* KFAC_OPT_* bits */
  int32_t reserved;    /* must be 0 */
} kfac_hparams_t;
/* KFAC_OPT_RESCALE (Osawa et al. section 4.4, weights rescaling): after the
 * update, the weight W (bias excluded) of every conv2d and linear layer is
 * scaled in place to Frobenius norm sqrt(2 d_out):
 *     W <- W sqrt(2 d_out) / (||W||_F + rescale_eps)
 * d_out = the layer's output width (channels of a conv2d).  Batch-norm
 * parameters are not rescaled.  Runs as the RESCALE phase, after UPDATE. */

/* Bytes of workspace the given stack needs in `mode` (host only, no GPU
 * call).  Returns KFAC_ERR_ARG / _DTYPE / _UNSUPPORTED for descriptors the
 * step would reject; pointers are not inspected. */
kfac_status_t kfac_workspace_size(const kfac_layer_t* layers, int32_t n_layers, int32_t mode,
                                  size_t* bytes);

/* Enqueue one full K-FAC step for all layers on `stream`:
 *   [FACTORS] A <- ema_decay A + (1 - ema_decay) a_bar^T a_bar / N, same for G
 *             (batch-norm layers: their dA, dG)
 *   [INVERT]  A_inv = (A + damping I)^-1 when refresh has KFAC_REFRESH_A,
 *             G_inv = (G + damping I)^-1 when it has KFAC_REFRESH_G, by
 *             Cholesky; a factor that is not positive definite keeps its
 *             previous inverse and sets KFAC_FLAG_NOT_PD
 *   [UPDATE]  P = G_inv [grad_w | grad_b] A_inv; D = P + wd W; V = mu V + D;
 *             W = W - lr V  (w, b, mom_w, mom_b in place); batch-norm layers
 *             take the diagonal step of kfac_step_diag with damping_bn; then
 *             the weight rescaling when options has KFAC_OPT_RESCALE
 * Layers are processed in order; phases are ordered as listed. */
kfac_status_t kfac_step_full(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                             void* workspace, size_t ws_bytes, void* stream);

/* Enqueue one diagonal step for all layers on `stream`:
 *   [FACTORS] dA[j] = mean_n a_bar[n, j]^2 (conv: over the unfolded rows,
 *             which are never materialised), dG[o] = mean_n g[n, o]^2
 *             (batch-norm layers: the per-channel Fisher diagonals above)
 *   [UPDATE]  in one pass F = beta F + (1 - beta) dG[o] dA[j] (batch norm:
 *             dA[c] for gamma, dG[c] for beta);
 *             P = grad / (F + damping); D = P + wd W; V = mu V + D; W = W - lr V;
 *             then the weight rescaling when options has KFAC_OPT_RESCALE */
kfac_status_t kfac_step_diag(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                             void* workspace, size_t ws_bytes, void* stream);

/* kfac_step_diag for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step with the same kernels, but no workspace argument.  The
 * reduction's intermediate sums live in a device array of the library that
 * holds at most 32 MiB (KFAC_NOALLOC_SCRATCH_BYTES); each GPU the library
 * runs on holds one until the process ends.  A stack whose
 * kfac_workspace_size(..., KFAC_MODE_DIAG, ...) exceeds that gets
 * KFAC_ERR_WORKSPACE before anything is enqueued (ResNet-18 at 224x224 needs
 * 17.8 MiB, at any batch).  `flags` is a caller-owned device word, zeroed by
 * the caller once, that receives the sticky flags (kfac_read_flags accepts
 * its address in place of a workspace).  The call allocates no memory on the
 * device and calls no allocating routine.  Every call on one GPU shares that
 * GPU's array: calls that can overlap on one GPU (different streams, host
 * threads) race and must be ordered by the caller. */
#define KFAC_NOALLOC_SCRATCH_BYTES (32u << 20)
kfac_status_t kfac_step_diag_noalloc(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                                     uint32_t* flags, void* stream);

/* Host-side schedule of the per-step scalars (no GPU call).
 *   Warm-up damping (Osawa et al. section 4.2): the damping starts at
 *   damping_init and decreases to damping_target over warmup_steps steps,
 *   then stays there.  Step t (1-based) uses u = min(t - 1, warmup_steps) /
 *   warmup_steps (u = 1 when warmup_steps is 0) and
 *       LINEAR:    damping = init + (target - init) u
 *       GEOMETRIC: damping = init (target / init)^u
 *   Batch-norm layers use bn_damping_scale (rho_BN > 1 on the page) times it.
 *   Inverse refresh (sections 1 and 5.4: the Fisher changes fast early on, so
 *   refreshes are reduced only after the first few hundred steps, and A
 *   changes less than G): steps 1 .. max(dense_steps, 1) refresh both
 *   inverses; after that, with D = max(dense_steps, 1), A is refreshed at the
 *   steps t with (t - D) a multiple of refresh_every_a, G likewise with
 *   refresh_every_g.
 * kfac_schedule_hparams writes damping, damping_bn and refresh of *hp for
 * step `step` (>= 1) and leaves the other fields alone; KFAC_ERR_ARG for a
 * step below 1, a negative warmup, intervals below 1, a non-positive damping
 * (geometric shape) or an unknown shape. */
enum { KFAC_WARMUP_LINEAR = 0, KFAC_WARMUP_GEOMETRIC = 1 };
typedef struct kfac_schedule {
  float damping_init;       /* gamma(0) */
  float damping_target;     /* gamma_target */
  int32_t warmup_steps;     /* t_warmup */
  int32_t warmup_shape;     /* KFAC_WARMUP_LINEAR | KFAC_WARMUP_GEOMETRIC */
  float bn_damping_scale;   /* rho_BN */
  int32_t dense_steps;      /* steps that refresh both inverses every step */
  int32_t refresh_every_a;  /* then: A inverse every this many steps */
  int32_t refresh_every_g;  /* and G inverse every this many steps */
} kfac_schedule_t;
kfac_status_t kfac_schedule_hparams(const kfac_schedule_t* schedule, int64_t step, kfac_hparams_t* hp);

/* Copy the workspace's sticky flag word to *flags (waits for `stream`), and
 * clear it on the device afterwards when `clear` is nonzero.  `workspace` may
 * also be the flag word given to kfac_step_diag_noalloc. */
kfac_status_t kfac_read_flags(void* workspace, void* stream, uint32_t* flags, int32_t clear);

/* Static description of a status code. */
const char* kfac_status_string(kfac_status_t status);

/* KFAC_ABI_VERSION of the built library. */
int32_t kfac_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KFAC_H */

/*
 * dense_layers_amd -- fused dense layer training path for AMD Instinct MI355X
 * (gfx950 / CDNA4), as a C ABI.
 *
 * What it computes (the Linear / LinearAct contract of the noeira.nn docs,
 * "The design in one page": every module has a forward and a vjp, and
 * MatMul + Bias + Activation is one fused kernel; the optimizer and loss
 * surface of the MuNet page, "What runs today" and "Python training"; the
 * fused cross-entropy of the Orthon page, "Selected Orthon vs. PyTorch
 * results"):
 *
 *   forward  Z = X W^T + b,  Y = act(Z)
 *   vjp      G = dY * act'(Z),  dX = G W,  dW = G^T X,  db = sum_rows G
 *   loss     mean softmax cross-entropy over the batch, dlogits = (p - onehot)/B
 *   update   SGD  w <- w - lr g
 *            AdamW (decoupled decay, bias-corrected)
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major and contiguous.  X is [B, in], W is
 *     [out, in] (PyTorch Linear layout), b is [out], Y and Z are [B, out].
 *   - Pointers marked "device" are HIP device pointers; everything else is
 *     host memory.  `stream` is a hipStream_t passed as void* (NULL = the
 *     null stream).  Work is enqueued on that stream and the call returns
 *     without synchronising; outputs are valid once the stream reaches them.
 *   - The library allocates no device memory.  Scratch space is a caller-
 *     owned device workspace whose size comes from the matching
 *     *_workspace_size query (256-byte aligned pointer required).
 *   - Calls keep no state between them and may be made from many threads;
 *     calls on different streams are independent.
 *   - Results are bit-reproducible run to run: no floating-point atomics.
 *   - Return value: DL_OK (0) or an error code below.  For codes 1-4 every
 *     argument was checked before anything was launched and no output was
 *     touched.  DL_HIP_ERROR means a launch failed; outputs are undefined.
 *     dl_last_error() returns a message for the last failure on this thread.
 *   - Arguments X and the saved Y/Z must not change between a forward call
 *     and the vjp call that uses them.
 */
#ifndef DENSE_LAYERS_AMD_H
#define DENSE_LAYERS_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- enums and status codes --------------------------------------------- */

enum dl_dtype {
  DL_F32 = 0,  /* float32 operands, float32 accumulation */
  DL_BF16 = 1  /* bfloat16 operands (RNE copies), float32 accumulation */
};

enum dl_act {
  DL_ACT_IDENTITY = 0,
  DL_ACT_RELU = 1,      /* max(z, 0); derivative 1 where z > 0, else 0 */
  DL_ACT_GELU_TANH = 2  /* 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
};

enum dl_status {
  DL_OK = 0,
  DL_INVALID_ARGUMENT = 1,     /* null required pointer, size <= 0, bad enum */
  DL_UNSUPPORTED = 2,          /* a dtype / activation combination not built */
  DL_ALIASING = 3,             /* an output overlaps an input it must not */
  DL_WORKSPACE_TOO_SMALL = 4,  /* ws_bytes below the size query's answer */
  DL_HIP_ERROR = 5             /* a HIP launch failed */
};

enum dl_opt_kind { DL_OPT_SGD = 0, DL_OPT_ADAMW = 1 };

/* Message for the last non-zero status returned on the calling thread. */
const char* dl_last_error(void);

/* Offload target the library was built for ("gfx950"). */
const char* dl_build_target(void);

/*
 * Per-launch timing for measurement (the per-kernel GPU timestamps of the
 * MuNet page, "Configuration": profile=True).  Between dl_profile_begin and
 * dl_profile_end, every kernel launch this library makes from the calling
 * thread is bracketed by a pair of HIP events recorded on the launch's own
 * stream.  At most `capacity` launches are recorded (later ones are counted
 * but not timed).  dl_profile_end waits for the recorded events, writes up to
 * `max` durations in milliseconds to ms[] and the launch names (each
 * NUL-terminated, at most 47 characters) to names[i * 48], releases the
 * events, and returns the number of launches seen; a negative value is a
 * HIP error.  Timing adds event records between launches, so it is meant for
 * a short measured pass, not the throughput run.  ms and names are host
 * arrays and may be NULL when max is 0.
 */
int dl_profile_begin(int capacity);
int dl_profile_end(int max, float* ms, char* names);

/* ---- dense layer forward ------------------------------------------------- */

/*
 * dense_act_fwd -- Y = act(X W^T + b) in one GEMM with the bias and the
 * activation in its epilogue (noeira.nn docs, "The design in one page":
 * LinearAct; bias and activation folded into the GEMM epilogue).
 *
 *   dtype   DL_F32: X, W, Y, Z are float32.  DL_BF16: X, W, Y, Z are
 *           bfloat16 (W is the bf16 working copy, see dense_cast_bf16);
 *           accumulation is float32 in both cases.
 *   act     enum dl_act.
 *   B, in, out  > 0.
 *   X       device [B, in]
 *   W       device [out, in]
 *   b       device float32 [out], or NULL for no bias
 *   Y       device [B, out] output
 *   Z       device [B, out] output pre-activation, or NULL.  Needed by the
 *           GELU vjp; ReLU's vjp can use Y instead.
 * Y must not overlap X, W or b; Z must not overlap Y.
 */
int dense_act_fwd(void* stream, int dtype, int act, int64_t B, int64_t in,
                  int64_t out, const void* X, const void* W, const float* b,
                  void* Y, void* Z);

/* ---- dense layer vector-Jacobian product -------------------------------- */

/*
 * dense_act_vjp -- the vjp of LinearAct (noeira.nn docs, "The design in one
 * page": forward and vjp per module, backward = composition of vjps):
 *   G = dY * act'(saved),  dX = G W,  dW = G^T X,  db = sum over rows of G.
 * dW and db are float32 and overwritten (not accumulated); db is reduced in
 * the same kernel as dW.
 *
 *   dY      device [B, out] (dtype)
 *   saved   device [B, out] (dtype): Z for GELU, Y or Z for ReLU, ignored
 *           (may be NULL) for identity.
 *   X       device [B, in] (dtype), the forward input
 *   W       device [out, in] (dtype)
 *   Wt      device [in, out] (dtype), the transpose of W, or NULL.  Only
 *           read for dX; with it the dX product reads both operands along
 *           the contraction index (see dense_cast_bf16_t).
 *   dX      device [B, in] (dtype) output, or NULL to skip (first layer)
 *   dW      device float32 [out, in] output, or NULL to skip
 *   db      device float32 [out] output, or NULL to skip
 *   dx_act, dx_saved  fold the previous layer's activation into dX: when
 *           dx_act != DL_ACT_IDENTITY, the call writes
 *           dX * dx_act'(dx_saved) instead of dX, where dx_saved [B, in]
 *           (dtype) is that layer's Z (GELU) or Y/Z (ReLU).  The result is
 *           the G of the previous layer, whose own vjp is then called with
 *           act = DL_ACT_IDENTITY.  dx_saved may equal dX (in place).
 *   ws, ws_bytes  device workspace, at least dense_act_vjp_workspace_size().
 * dX must not overlap dY, X, W or saved (dx_saved excepted); dW/db must not
 * overlap any input.
 */
int dense_act_vjp(void* stream, int dtype, int act, int64_t B, int64_t in,
                  int64_t out, const void* dY, const void* saved,
                  const void* X, const void* W, const void* Wt, void* dX,
                  float* dW, float* db, int dx_act, const void* dx_saved,
                  void* ws, size_t ws_bytes);

size_t dense_act_vjp_workspace_size(int dtype, int act, int64_t B, int64_t in,
                                    int64_t out);

/* ---- softmax cross-entropy, forward and backward ------------------------ */

/*
 * softmax_xent_fwd_bwd -- one pass over the logits gives the mean loss and
 * dlogits (Orthon page, "Selected Orthon vs. PyTorch results": one fused
 * kernel reads the logits once).  Per row: lse = max + log(sum exp(z - max)),
 * loss_i = lse - z[label_i], dlogits = (softmax - onehot(label)) / B;
 * loss = (1/B) sum_i loss_i, reduced in a fixed order.
 *
 *   B, C     > 0 (C = number of classes)
 *   logits   device float32 [B, C]
 *   labels   device int32 [B], each in [0, C).  A label outside the range
 *            makes that row's loss NaN (so the mean is NaN) and its dlogits
 *            row the plain softmax / B; it never causes an out-of-bounds read.
 *   loss     device float32 [1] output (mean over the batch)
 *   row_loss device float32 [B] output per-row loss, or NULL
 *   dlogits  device float32 [B, C] output; may equal logits (in place)
 *   ws, ws_bytes  at least softmax_xent_workspace_size(B, C)
 */
int softmax_xent_fwd_bwd(void* stream, int64_t B, int64_t C,
                         const float* logits, const int32_t* labels,
                         float* loss, float* row_loss, float* dlogits,
                         void* ws, size_t ws_bytes);

size_t softmax_xent_workspace_size(int64_t B, int64_t C);

/* ---- optimizers ---------------------------------------------------------- */

/*
 * sgd_step -- w <- w - lr g, elementwise over n float32 values (MuNet page,
 * "What runs today" and "Python training": SGD).  Plain: no momentum, no
 * decay.  lr is rounded once to float32.  w and g are device pointers; g
 * must not overlap w.
 */
int sgd_step(void* stream, int64_t n, float* w, const float* g, double lr);

/*
 * adamw_step -- one AdamW step on n float32 values (MuNet page, "What runs
 * today": AdamW; noeira.nn docs, "The design in one page": the moments m, v
 * live with the parameter and start at zero on the first step):
 *   w <- w (1 - lr wd);  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   w <- w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * step is t >= 1.  The hyper-parameters are taken in double and the derived
 * constants (1 - lr wd, 1 - b1, 1 - b2, lr / (1 - b1^t), 1 / sqrt(1 - b2^t))
 * are formed on the host in double, each then rounded once to float32 for
 * the element-wise float32 update.  beta1, beta2 in [0, 1).
 * w, g, m, v are distinct device arrays of n floats; m and v are updated.
 */
int adamw_step(void* stream, int64_t n, float* w, const float* g, float* m,
               float* v, double lr, double beta1, double beta2, double eps,
               double weight_decay, int64_t step);

/* ---- bf16 working copies -------------------------------------------------- */

/*
 * dense_cast_bf16 -- dst = bf16(src) with round-to-nearest-even, NaN kept
 * (the low-precision convention of the MuNet page, "Configuration":
 * round to nearest, NaN preserved; and the FP32-master-weight scheme of the
 * Orthon page, "Mixed-precision training on CUDA").
 *   n > 0; src device float32 [n]; dst device bf16 [n]; no overlap.
 */
int dense_cast_bf16(void* stream, int64_t n, const float* src, void* dst);

/*
 * dense_cast_bf16_t -- the same rounding for a [rows, cols] float32 matrix
 * (a weight W [out, in]), writing the bf16 copy dst [rows, cols] and/or its
 * transpose dst_t [cols, rows] in one pass.  The transposed copy lets the bf16
 * vjp read W along its contraction index (the `Wt` argument of
 * dense_act_vjp).  rows, cols > 0; src device float32; dst, dst_t device bf16
 * or NULL (not both); no overlaps.
 */
int dense_cast_bf16_t(void* stream, int64_t rows, int64_t cols, const float* src,
                      void* dst, void* dst_t);

/* ---- one MLP training step ------------------------------------------------ */

typedef struct dl_layer {
  int64_t in, out;  /* layer shape; layer l's in equals layer l-1's out */
  int32_t act;      /* enum dl_act (DL_ACT_IDENTITY or DL_ACT_RELU) */
  float* W;         /* device [out, in] parameters, updated in place */
  float* b;         /* device [out] bias, updated in place */
  float* dW;        /* device [out, in] gradient output */
  float* db;        /* device [out] gradient output */
  float* mW;        /* device [out, in] AdamW first moment (NULL for SGD) */
  float* vW;        /* device [out, in] AdamW second moment (NULL for SGD) */
  float* mb;        /* device [out] */
  float* vb;        /* device [out] */
} dl_layer_t;

typedef struct dl_opt {
  int32_t kind;     /* enum dl_opt_kind */
  double lr, beta1, beta2, eps, weight_decay;  /* betas/eps/wd: AdamW only */
  int64_t step;     /* AdamW step t >= 1 (ignored when step_dev is set) */
  /* AdamW, optional: device int64 [1] holding the number of steps taken.
   * When set, each call first adds 1 to it on the device (in stream order)
   * and the update uses that value as t, its bias corrections formed on the
   * device in double exactly as the host forms them from `step`.  This makes
   * the whole step replayable from a captured stream graph, which cannot see
   * a host-side step count.  Caller-owned; NULL to use `step`. */
  int64_t* step_dev;
} dl_opt_t;

/*
 * mlp_train_step -- forward through every layer, softmax cross-entropy on the
 * last layer's output, the composed vjps from the last layer to the first
 * (no dX for the first layer), then the optimizer on every W and b (MuNet
 * page, "Python training": the compiled forward / loss / backward / optimizer
 * step; noeira.nn docs, "A complete example": the LinearReLU, LinearReLU,
 * Linear MLP).  Float32 throughout.  The loss written is the one computed
 * before the update.  Hidden-layer activations are fused into the GEMM
 * epilogues and their derivatives into the dX epilogues.
 *
 *   B > 0; n_layers in [1, 16]; layers is a host array of n_layers entries.
 *   X        device float32 [B, layers[0].in]
 *   labels   device int32 [B], values in [0, layers[n-1].out)
 *   opt      host pointer
 *   loss     device float32 [1] output
 *   ws, ws_bytes  at least mlp_train_step_workspace_size()
 */
int mlp_train_step(void* stream, int64_t B, int32_t n_layers,
                   const dl_layer_t* layers, const float* X,
                   const int32_t* labels, const dl_opt_t* opt, float* loss,
                   void* ws, size_t ws_bytes);

size_t mlp_train_step_workspace_size(int64_t B, int32_t n_layers,
                                     const dl_layer_t* layers);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_LAYERS_AMD_H */

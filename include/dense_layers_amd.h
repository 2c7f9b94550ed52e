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
 *            mean squared error, dpred = 2 (p - t) / (B C)
 *   update   SGD  w <- w - lr g
 *            AdamW (decoupled decay, bias-corrected), Adam (coupled decay)
 *            with global-norm clipping, dynamic loss scaling, LR schedules,
 *            parameter EMA and a bf16 working copy fused into the update
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
  DL_F32 = 0,   /* float32 operands, float32 accumulation */
  DL_BF16 = 1,  /* bfloat16 operands (RNE copies), float32 accumulation */
  DL_F16 = 2    /* IEEE half operands (nearest-even, clamped to +-65504, NaN kept;
                 * the mixed precision of the MuNet page, "Configuration"),
                 * float32 accumulation */
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
  DL_HIP_ERROR = 5,            /* a HIP launch failed */
  DL_LABEL_OUT_OF_RANGE = 6    /* validate mode only (dl_set_validate): a
                                * label outside [0, C); nothing but the
                                * label check was launched */
};

enum dl_opt_kind {
  DL_OPT_SGD = 0,    /* w <- w - lr g */
  DL_OPT_ADAMW = 1,  /* decoupled decay: w <- w (1 - lr wd), then Adam */
  DL_OPT_ADAM = 2    /* coupled decay: g <- g + wd w, then Adam */
};

enum dl_lr_kind {
  DL_LR_CONSTANT = 0,
  DL_LR_STEP = 1,            /* lr gamma^floor(k / step_size) */
  DL_LR_WARMUP_COSINE = 2,   /* linear warmup, then cosine down to min_lr */
  DL_LR_WARMUP_LINEAR = 3    /* linear warmup, then linear down to min_lr */
};

/* Message for the last non-zero status returned on the calling thread.
 * dense_last_error and dl_last_error are the same function. */
const char* dense_last_error(void);
const char* dl_last_error(void);

/*
 * dl_set_validate -- validate mode for the calling thread (off by default).
 * When on, softmax_xent_fwd_bwd and mlp_train_step first count the labels
 * outside [0, C) on the device (one small launch into their workspace) and
 * wait for the count: a call with any such label returns
 * DL_LABEL_OUT_OF_RANGE having touched no output.  This is the one place
 * the library synchronises the caller's stream; outside validate mode an
 * out-of-range label is never read out of bounds and gives a NaN row loss
 * instead (see softmax_xent_fwd_bwd).  Returns the previous setting; any
 * non-zero `on` turns it on.  No GPU work.
 */
int dl_set_validate(int on);

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

/*
 * dl_set_mlp_fusion -- how much of mlp_train_step the calling thread runs
 * fused, for comparing the fused step with the composition it replaces (the
 * composed vjps of the noeira.nn docs, "The design in one page").
 *   2 (default): when the network ends in a hidden layer of at most 256
 *     inputs and outputs (multiples of 8) and a head of at most 16 classes,
 *     one kernel runs that layer's forward, the head's forward, softmax-xent
 *     and vjp, and that layer's dX; the hidden layer's output never reaches
 *     HBM.
 *   1: the head alone is fused; the hidden layer runs as GEMMs.
 * Both levels run every product in the same order and give bit-identical
 * results.  Returns the previous level, or -DL_INVALID_ARGUMENT for any
 * other level (the setting is unchanged).  Thread-local; no GPU work.
 */
int dl_set_mlp_fusion(int level);

/*
 * dl_empty_launches -- n launches of an empty kernel (one workgroup of 64
 * threads) on `stream`, for measurement: the launch floor that a
 * latency-bound step of k launches cannot go below is k times the time of
 * one such launch.  Returns DL_OK, DL_INVALID_ARGUMENT for n < 0, or
 * DL_HIP_ERROR.
 */
int dl_empty_launches(void* stream, int n);

/* ---- dense layer forward ------------------------------------------------- */

/*
 * dense_act_fwd -- Y = act(X W^T + b) in one GEMM with the bias and the
 * activation in its epilogue (noeira.nn docs, "The design in one page":
 * LinearAct; bias and activation folded into the GEMM epilogue).
 *
 *   dtype   DL_F32: X, W, Y, Z are float32.  DL_BF16: X, W, Y, Z are
 *           bfloat16 (W is the bf16 working copy, see dense_cast_bf16).
 *           DL_F16: X, W, Y, Z are IEEE half (see dense_cast_f16); Y and Z
 *           round with saturation at +-65504.  Accumulation is float32 in
 *           every case.
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

/*
 * dense_act_vjp_scaled -- dense_act_vjp for a gradient operand handed over
 * times a scale s (the mixed_safe precision of the MuNet page,
 * "Configuration": each half gradient operand is multiplied by a power of
 * two before its matmul, so that very small cotangents stay representable in
 * half with their relative accuracy).  dY holds the cotangent times s
 * (dense_cast_f16_scaled writes both).  dW and db are divided by s in
 * float32 inside the GEMM epilogues, so they come out unscaled (exact when s
 * is a power of two).  dX keeps the scale: it is the previous layer's
 * gradient operand, whose own vjp takes it with the same dy_scale (divided
 * there, a half dX of the unscaled size would fall back below the half
 * normal range).
 *   dy_scale  device float32 [1] holding s; must not overlap an output or
 *             the workspace.  Every other argument as dense_act_vjp.
 */
int dense_act_vjp_scaled(void* stream, int dtype, int act, int64_t B, int64_t in,
                         int64_t out, const void* dY, const void* saved,
                         const void* X, const void* W, const void* Wt, void* dX,
                         float* dW, float* db, int dx_act, const void* dx_saved,
                         void* ws, size_t ws_bytes, const float* dy_scale);

size_t dense_act_vjp_workspace_size(int dtype, int act, int64_t B, int64_t in,
                                    int64_t out);

/* ---- softmax cross-entropy, forward and backward ------------------------ */

/*
 * softmax_xent_fwd_bwd -- one pass over the logits gives the mean loss and
 * dlogits (Orthon page, "Selected Orthon vs. PyTorch results": the
 * cross-entropy fused into a single pass over the logits).  Per row: lse = max + log(sum exp(z - max)),
 * loss_i = lse - z[label_i], dlogits = (softmax - onehot(label)) / B;
 * loss = (1/B) sum_i loss_i, reduced in a fixed order.
 *
 *   B, C     > 0 (C = number of classes)
 *   logits   device float32 [B, C]
 *   labels   device int32 [B], each in [0, C).  In validate mode a label
 *            outside the range is DL_LABEL_OUT_OF_RANGE; otherwise it makes
 *            that row's loss NaN (so the mean is NaN) and its dlogits row
 *            the plain softmax / B, and is never read out of bounds.
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

/*
 * softmax_xent_fwd_bwd_noalloc -- for callers that cannot allocate device
 * memory (code under stream-graph capture, tight serving loops, harnesses
 * that forbid allocation): softmax_xent_fwd_bwd with no workspace argument.
 * Same kernels, same results bit for bit.  When row_loss is NULL the
 * per-row losses go to a fixed scratch array the library holds on each GPU
 * it runs on (DL_XENT_NOALLOC_MAX_ROWS floats, 4 MiB, kept until the process
 * ends); B above that limit is DL_WORKSPACE_TOO_SMALL unless row_loss is
 * given.  The call allocates nothing, host or device.  Calls on one GPU
 * share its scratch, so calls that overlap in time on one GPU (other
 * streams or threads) race; calls ordered on one stream do not.  Validate
 * mode does not apply here (its label check reads a count back to the host):
 * an out-of-range label gives a NaN row loss, as outside validate mode.
 * Arguments and errors otherwise as softmax_xent_fwd_bwd; the stream must
 * belong to the current device.
 */
#define DL_XENT_NOALLOC_MAX_ROWS (1 << 20)
int softmax_xent_fwd_bwd_noalloc(void* stream, int64_t B, int64_t C,
                                 const float* logits, const int32_t* labels,
                                 float* loss, float* row_loss, float* dlogits);

/* ---- fused classifier head over many classes ----------------------------- */

/*
 * dense_xent_fwd / dense_xent_vjp -- a Linear head closed by softmax
 * cross-entropy, for large class counts, in two calls that never
 * materialise the loss gradient (the fused cross-entropy of the Orthon
 * page, "Selected Orthon vs. PyTorch results", whose advantage grows with
 * the class count, taken into the GEMMs; the LinearAct forward / vjp pair of
 * the noeira.nn docs, "The design in one page").  Float32 throughout.
 *
 * dense_xent_fwd: logits = X W^T + b from one GEMM whose epilogue also
 * leaves, per row and tile of columns, the tile's max and sum of exp; a row
 * pass then forms lse_i = log sum_j exp(z_ij) and the row loss
 * lse_i - z[i, y_i], and the loss is their fixed-order mean.
 *   B, in, C > 0; X device [B, in]; W device [C, in]; b device [C] or NULL;
 *   labels device int32 [B] in [0, C) (validate mode: DL_LABEL_OUT_OF_RANGE;
 *   otherwise an out-of-range label gives a NaN row loss and is never read
 *   out of bounds); logits device [B, C] output; lse device [B] output;
 *   loss device [1] output (mean over the batch); row_loss device [B]
 *   output or NULL.  ws: dense_xent_fwd_workspace_size(B, in, C) bytes
 *   (the per-tile pairs, 8 B per row and column tile of 128 classes, or of
 *   64 for small problems, and the row losses).
 *   No output may overlap an input or another output.
 *
 * dense_xent_vjp: with g = (exp(z - lse) - onehot(y)) / B formed from the
 * logits inside both GEMMs as they read them,
 *   dX = g W,  dW = g^T X,  db = sum_rows g   (dW / db overwritten).
 *   logits, lse, labels as left by dense_xent_fwd (unchanged since); X, W
 *   as passed to it.  dX [B, in], dW [C, in], db [C]: outputs, each may be
 *   NULL (db needs dW: it is summed inside the dW kernel).  ws:
 *   dense_xent_vjp_workspace_size(B, in, C) bytes, 256-byte aligned (one
 *   8-byte record per row: the row's exponent offset and label, formed by a
 *   small pass before the GEMMs; then split-K slices of dW for small
 *   batches).
 * The gradient matches softmax_xent_fwd_bwd's to float32 rounding (it is
 * formed as exp(z - lse) rather than exp(z - max) / sum).
 */
int dense_xent_fwd(void* stream, int64_t B, int64_t in, int64_t C,
                   const float* X, const float* W, const float* b,
                   const int32_t* labels, float* logits, float* lse, float* loss,
                   float* row_loss, void* ws, size_t ws_bytes);
size_t dense_xent_fwd_workspace_size(int64_t B, int64_t in, int64_t C);
int dense_xent_vjp(void* stream, int64_t B, int64_t in, int64_t C,
                   const float* logits, const float* lse, const int32_t* labels,
                   const float* X, const float* W, float* dX, float* dW, float* db,
                   void* ws, size_t ws_bytes);
size_t dense_xent_vjp_workspace_size(int64_t B, int64_t in, int64_t C);

/* ---- optimizers ---------------------------------------------------------- */

/*
 * Learning-rate schedule (noeira.nn docs, "Optimizers & losses": LR
 * schedules).  Step t >= 1 of the optimizer uses k = t - 1 scheduler steps:
 *   DL_LR_CONSTANT       lr
 *   DL_LR_STEP           lr * gamma^floor(k / step_size)          (step_size >= 1)
 *   DL_LR_WARMUP_COSINE  lr (k + 1) / warmup for k < warmup, then
 *                        min_lr + (lr - min_lr) (1 + cos(pi j / T)) / 2,
 *                        j = min(k - warmup, T), T = total - warmup
 *   DL_LR_WARMUP_LINEAR  the same warmup, then min_lr + (lr - min_lr) (T - j) / T
 * (T <= 0 gives min_lr after the warmup.)  Evaluated in double, on the host
 * from a host step count or on the device from a device step count.
 */
typedef struct dl_lr_schedule {
  int32_t kind;        /* enum dl_lr_kind */
  int64_t warmup;      /* >= 0 */
  int64_t total;       /* step count at which the decay reaches min_lr */
  int64_t step_size;   /* DL_LR_STEP */
  double min_lr;
  double gamma;        /* DL_LR_STEP */
} dl_lr_schedule_t;

/* The learning rate of step `step` (>= 1) for base rate `lr` under schedule
 * `s` (NULL: constant).  Host function; returns NaN for a bad argument. */
double dl_lr_at(const dl_lr_schedule_t* s, double lr, int64_t step);

/*
 * Dynamic loss scaling (Orthon page, "Core capabilities": a loss scaler that
 * checks the gradients for Inf / NaN, drops such steps, and moves the scale
 * down after one and up after a run of good steps).  The loss gradient is
 * multiplied by S = *scale, so every gradient the backward forms is S times
 * the true one.  The optimizer looks at all of a step's gradients: if one of
 * them holds a NaN or an Inf, the step is skipped (no parameter, moment,
 * average or step-count change), *found_inf = 1, S <- S backoff_factor and
 * the tracker resets; otherwise the gradients are used divided by S,
 * *found_inf = 0, the tracker counts the step and, on reaching
 * growth_interval, S <- S growth_factor and the tracker resets.  All three
 * values live in device memory and are updated on the device, so no host
 * synchronisation is needed.  The caller initialises *scale (e.g. 65536)
 * and *growth_tracker (0).
 */
typedef struct dl_loss_scaler {
  float* scale;             /* device float32 [1] */
  int32_t* growth_tracker;  /* device int32 [1] */
  int32_t* found_inf;       /* device int32 [1] output */
  double growth_factor;     /* > 1, e.g. 2 */
  double backoff_factor;    /* in (0, 1), e.g. 0.5 */
  int32_t growth_interval;  /* >= 1, e.g. 2000 */
} dl_loss_scaler_t;

/*
 * Optimizer configuration, shared by optimizer_step and mlp_train_step.
 */
typedef struct dl_opt {
  int32_t kind;     /* enum dl_opt_kind */
  double lr, beta1, beta2, eps, weight_decay;  /* betas/eps/wd: Adam, AdamW */
  int64_t step;     /* Adam / AdamW step t >= 1, and the step of the
                     * schedule (ignored when step_dev is set) */
  /* optional: device int64 [1] holding the number of steps taken.  When set,
   * each call adds 1 to it on the device (in stream order; not for a step a
   * loss scaler skips) and the update uses that value as t, its bias
   * corrections and scheduled learning rate formed on the device in double
   * exactly as the host forms them from `step`.  This makes the whole step
   * replayable from a captured stream graph, which cannot see a host-side
   * step count.  Caller-owned; NULL to use `step`.  Required with a loss
   * scaler unless the optimizer is SGD without a schedule. */
  int64_t* step_dev;
  /* > 0: clip the global 2-norm of all of the call's gradients (after
   * unscaling): every gradient is multiplied by
   * min(1, max_grad_norm / (norm + 1e-6)) (MuNet page, "What runs today":
   * gradient clipping).  <= 0: no clipping. */
  double max_grad_norm;
  /* decay d of the parameter averages: e <- d e + (1 - d) w after the update,
   * for every array that has an average (MuNet page, "What runs today": EMA) */
  double ema_decay;
  const dl_lr_schedule_t* schedule;  /* host pointer, or NULL: constant lr */
  const dl_loss_scaler_t* scaler;    /* host pointer, or NULL: no loss scaling */
  /* optional device float32 [1] output: the global norm of the unscaled
   * gradients (formed when clipping or loss scaling is on) */
  float* grad_norm;
} dl_opt_t;


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

/*
 * adam_step -- one Adam step with coupled (L2) weight decay on n float32
 * values (noeira.nn docs, "Optimizers & losses" and the Orthon page, "Core
 * capabilities": Adam):
 *   g' = g + wd w;  m <- b1 m + (1-b1) g';  v <- b2 v + (1-b2) g'^2;
 *   w <- w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * Arguments, constants and errors as adamw_step.
 */
int adam_step(void* stream, int64_t n, float* w, const float* g, float* m,
              float* v, double lr, double beta1, double beta2, double eps,
              double weight_decay, int64_t step);

/*
 * ema_update -- e <- d e + (1 - d) w over n float32 values (MuNet page,
 * "What runs today": EMA of the parameters).  d in [0, 1]; e and w distinct
 * device arrays.
 */
int ema_update(void* stream, int64_t n, float* ema, const float* w,
               double decay);

/*
 * clip_grad_norm -- scale a set of gradient arrays in place so that their
 * global 2-norm is at most max_norm (MuNet page, "What runs today": gradient
 * clipping): norm = sqrt(sum over all arrays of g^2) (float64 partial sums in
 * a fixed order), every g is multiplied by min(1, max_norm / (norm + 1e-6)).
 *   count in [1, 4096]; grads a host array of `count` device float32
 *   pointers; n a host array of their lengths (> 0); max_norm > 0;
 *   total_norm optional device float32 [1] output (the norm before
 *   clipping); ws, ws_bytes at least clip_grad_norm_workspace_size().
 * The arrays must not overlap one another or the workspace.
 */
int clip_grad_norm(void* stream, int32_t count, float* const* grads,
                   const int64_t* n, double max_norm, float* total_norm,
                   void* ws, size_t ws_bytes);

size_t clip_grad_norm_workspace_size(int32_t count, const int64_t* n);

/*
 * One array the multi-tensor optimizer updates (noeira.nn docs, "The design
 * in one page": a Param holds its value, gradient and Adam moments).
 */
typedef struct dl_param {
  int64_t n;         /* element count, > 0 */
  float* w;          /* device float32 [n], updated in place */
  const float* g;    /* device float32 [n] gradient (times the loss scale) */
  float* m;          /* device float32 [n] first moment (Adam, AdamW) */
  float* v;          /* device float32 [n] second moment (Adam, AdamW) */
  float* ema;        /* device float32 [n] parameter average, or NULL */
  void* w_bf16;      /* device bf16 [n]: RNE copy of the updated w, or NULL
                      * (the FP32-master scheme of the Orthon page,
                      * "Mixed-precision training on CUDA") */
} dl_param_t;

/*
 * optimizer_step -- one update of `count` arrays by opt->kind with every
 * option of dl_opt_t: loss-scale finite check and unscaling, global-norm
 * clipping, the schedule's learning rate, the parameter averages and the
 * bf16 copies, all fused into one pass over the arrays (plus one reading
 * pass over the gradients and one single-workgroup launch when clipping or
 * loss scaling is on).  Arrays are processed 32 to a launch.
 *   count in [1, 4096]; params a host array; opt a host pointer.
 *   ws, ws_bytes at least optimizer_step_workspace_size().
 * No two arrays of the call (w, g, m, v, ema, w_bf16 of any param) may
 * overlap.
 */
int optimizer_step(void* stream, const dl_opt_t* opt, int32_t count,
                   const dl_param_t* params, void* ws, size_t ws_bytes);

size_t optimizer_step_workspace_size(int32_t count, const dl_param_t* params);

/* ---- mean squared error -------------------------------------------------- */

/*
 * mse_loss_fwd_bwd -- loss = (1/(B C)) sum (pred - target)^2 and
 * dpred = 2 (pred - target) / (B C) in one pass (MuNet page, "Python
 * training": the step's mse_loss; noeira.nn docs, package layout: MSE).  The
 * squares are summed in float64, per workgroup and then in a fixed order.
 *   B, C > 0; pred, target device float32 [B, C]; loss device float32 [1]
 *   output; dpred device float32 [B, C] output, may equal pred (in place),
 *   or NULL (loss only); ws, ws_bytes at least mse_loss_workspace_size(B, C).
 */
int mse_loss_fwd_bwd(void* stream, int64_t B, int64_t C, const float* pred,
                     const float* target, float* loss, float* dpred, void* ws,
                     size_t ws_bytes);

size_t mse_loss_workspace_size(int64_t B, int64_t C);

/* ---- bf16 working copies -------------------------------------------------- */

/*
 * dense_cast_bf16 -- dst = bf16(src), rounded to the nearest value with ties
 * to even and NaN kept (the low-precision convention of the MuNet page,
 * "Configuration"; and the FP32-master-weight scheme of the Orthon page,
 * "Mixed-precision training on CUDA").
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

/*
 * dense_cast_f16, dense_cast_f16_t -- the same two copies in IEEE half:
 * nearest-even rounding, clamped to +-65504 (a value past the largest half,
 * or an infinity, becomes +-65504), NaN kept (the mixed-precision
 * convention of the MuNet page, "Configuration").  Arguments and errors as
 * dense_cast_bf16 / dense_cast_bf16_t, with half outputs.
 */
int dense_cast_f16(void* stream, int64_t n, const float* src, void* dst);

/*
 * dense_cast_f16_scaled -- the half copy of a gradient operand with a
 * power-of-two scale (mixed_safe): with m the largest finite |src|,
 * s = 2^(14 - floor(log2 m)) puts it in [2^14, 2^15) (s = 1 for m = 0; the
 * exponent is capped at 127); writes *scale = s and dst = half(src s)
 * (nearest even, saturating, NaN kept; src s is exact in float32).  Pass dst
 * and scale to dense_act_vjp_scaled.  Deterministic (the maximum does not
 * depend on the order of reduction).
 *   n > 0; src device float32 [n]; dst device half [n]; scale device
 *   float32 [1] output; ws, ws_bytes at least
 *   dense_cast_f16_scaled_workspace_size(n); no overlaps.
 */
int dense_cast_f16_scaled(void* stream, int64_t n, const float* src, void* dst,
                          float* scale, void* ws, size_t ws_bytes);
size_t dense_cast_f16_scaled_workspace_size(int64_t n);
int dense_cast_f16_t(void* stream, int64_t rows, int64_t cols, const float* src,
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
  float* eW;        /* device [out, in] parameter average, or NULL */
  float* eb;        /* device [out] parameter average, or NULL */
} dl_layer_t;


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
 * Every option of dl_opt_t applies: SGD, Adam or AdamW; a device step count
 * and a learning-rate schedule; global-norm clipping over all W and b; a
 * loss scaler (the loss gradient is multiplied by S, dW / db hold S times the
 * gradient, a step with non-finite gradients is skipped); and the parameter
 * averages of the layers that have eW / eb (all or none).  With clipping or
 * a loss scaler the split weight-gradient sums are finished by the gradient
 * pass rather than the optimizer.  With plain SGD and none of those options
 * (nor a device step count), a hidden layer whose weight gradient runs as
 * one K slice takes its SGD step inside that launch, after its dX, with the
 * optimizer's arithmetic; the workspace holds the gradient buffers this
 * order needs.
 *
 *   B > 0; n_layers in [1, 16]; layers is a host array of n_layers entries.
 *   X        device float32 [B, layers[0].in]
 *   labels   device int32 [B], values in [0, layers[n-1].out) (checked in
 *            validate mode, DL_LABEL_OUT_OF_RANGE; C, the class count, is
 *            layers[n-1].out and is not passed again)
 *   opt      host pointer
 *   loss     device float32 [1] output
 *   ws, ws_bytes  at least mlp_train_step_workspace_size()
 */
int mlp_train_step(void* stream, int64_t B, int32_t n_layers,
                   const dl_layer_t* layers, const float* X,
                   const int32_t* labels, const dl_opt_t* opt, float* loss,
                   void* ws, size_t ws_bytes);

/*
 * mlp_train_step_mse -- the same step with the mean squared error against
 * float32 targets as the loss (MuNet page, "Python training": the compiled
 * step trains an MLP with mse_loss): loss = (1/(B C)) sum (y - t)^2 over the
 * last layer's output y [B, C], dy = 2 (y - t) / (B C) (times the loss scale
 * when a scaler is set).  Every other argument, option and rule as
 * mlp_train_step; the last layer always runs as a GEMM (the fused narrow
 * head is a cross-entropy kernel).
 *   targets  device float32 [B, layers[n-1].out]; must not overlap X
 */
int mlp_train_step_mse(void* stream, int64_t B, int32_t n_layers,
                       const dl_layer_t* layers, const float* X,
                       const float* targets, const dl_opt_t* opt, float* loss,
                       void* ws, size_t ws_bytes);

/* Workspace for mlp_train_step and mlp_train_step_mse (the larger of the two
 * needs). */
size_t mlp_train_step_workspace_size(int64_t B, int32_t n_layers,
                                     const dl_layer_t* layers);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_LAYERS_AMD_H */

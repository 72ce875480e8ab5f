/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step.
 *
 * One call of muon_step() applies one Muon step to a list of hidden 2-D
 * weight matrices on one GPU:
 *
 *   momentum with Nesterov look-ahead   (Muon README, "Hyperparameter tuning":
 *                                        momentum 0.95, Nesterov on)
 *   Frobenius normalisation of the update (Muon blog by Venkatramana, sec. 3)
 *   ns_steps quintic Newton-Schulz iterations on the short side
 *       A = X X^T,  B = b A + c A A,  X <- a X + B X   (same blog, sec. 3;
 *       a, b, c = 3.4445, -4.7750, 2.0315)
 *   W <- W - lr*wd*W - lr*scale*O        (Muon README, "Usage": decoupled
 *                                        weight decay; blog sec. 2: shape scale)
 *
 * optionally after the Newton-Muon right-preconditioner G <- G S^-1 built
 * from a d x d activation second moment (Newton-Muon README, "What Is
 * Newton-Muon?").
 *
 * Memory and ownership
 *   All tensor pointers are DEVICE pointers owned by the caller (param,
 *   grad, momentum, update_out, activations) together with one caller-
 *   allocated device WORKSPACE whose size muon_workspace_size() reports.  The
 *   library never allocates device memory (muon_init_static uses instead a
 *   fixed array that is part of the loaded library).  Everything registered at
 *   muon_init() must stay allocated and unmoved until muon_destroy(); re-init
 *   after reallocating any of it.  The library owns only a small host-side
 *   handle.
 *   Layout: row-major, rows = out-features, element (i, j) at ptr[i*ld + j],
 *   ld >= cols.  param and grad share one dtype; momentum is always float32.
 *
 * Errors
 *   Argument errors are returned synchronously by muon_workspace_size() and
 *   muon_init() (and muon_precond_refresh()).  muon_step() only enqueues
 *   work on the given stream: it never synchronises, never allocates, and
 *   returns MUON_ERR_HIP only if a launch fails.  Nothing aborts or throws
 *   across the ABI.  A human-readable detail of the last error on the
 *   calling thread is available from muon_last_error().  Non-finite values
 *   propagate as in the plain arithmetic and set bit 0 of the flags word.
 *
 * Threading: one handle may be used by one stream at a time.
 * Streams: `stream` arguments are hipStream_t values passed as void*;
 *   NULL means the default stream.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct muon_handle_s* muon_handle_t;

typedef enum {
  MUON_OK = 0,
  MUON_ERR_NULL_ARG = 1,           /* a required pointer is NULL                 */
  MUON_ERR_BAD_SHAPE = 2,          /* rows/cols < 1, ld < cols, bad split        */
  MUON_ERR_BAD_DTYPE = 3,          /* unknown dtype                              */
  MUON_ERR_ALIGNMENT = 4,          /* pointer not aligned to its element size    */
  MUON_ERR_ALIASING = 5,           /* two registered buffers overlap             */
  MUON_ERR_WORKSPACE_TOO_SMALL = 6,
  MUON_ERR_UNSUPPORTED = 7,        /* valid request the library does not support */
  MUON_ERR_HIP = 8,                /* a HIP runtime call or launch failed        */
  MUON_ERR_BAD_ARG = 9             /* other invalid argument (hyper-parameters)  */
} muon_status_t;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype_t;

/* Shape-dependent lr factor.  The pages name three conventions (Muon blog,
 * the practical-guidance section: the original implementation's, an
 * RMS-matching variant and a theoretical rule) without printing a formula;
 * the library offers:
 *   NONE            1
 *   ORIGINAL        sqrt(max(1, rows/cols))          (default)
 *   MATCH_RMS_ADAMW 0.2*sqrt(max(rows, cols))
 *   SPECTRAL        sqrt(rows/cols): a semi-orthogonal update then has RMS->RMS
 *                   operator norm 1 (blog section 4 defines that norm as
 *                   sqrt(d_in/d_out) times the spectral norm; rows = d_out)
 * rows/cols are those of the orthogonalised block (split_rows if set). */
typedef enum {
  MUON_SCALE_NONE = 0,
  MUON_SCALE_ORIGINAL = 1,
  MUON_SCALE_MATCH_RMS_ADAMW = 2,
  MUON_SCALE_SPECTRAL = 3
} muon_scale_t;

/* Momentum form (the pages give "momentum 0.95, nesterov" only):
 *   EMA: M' = mu M + (1-mu) G;  U = (1-mu) G + mu M'   (default)
 *   SGD: M' = mu M + G;         U = G + mu M'
 * Without Nesterov U = M'. */
typedef enum { MUON_MOM_EMA = 0, MUON_MOM_SGD = 1 } muon_momentum_form_t;

/* What a registered tensor is stepped with.  Muon takes the hidden weight
 * matrices; the other parameters (embeddings, classifier heads, hidden gains
 * and biases) take AdamW (Muon README, "Usage"), in the same muon_step. */
typedef enum { MUON_KIND_MUON = 0, MUON_KIND_ADAMW = 1 } muon_kind_t;

/* One parameter tensor.  For kind MUON: a hidden weight matrix.  For kind
 * ADAMW: any parameter viewed as rows x cols (a vector as 1 x n); momentum
 * holds AdamW's first moment and exp_avg_sq its second (both float32, same
 * leading dimension ld_momentum); split_rows, precond and update_out must be
 * 0, -1 and NULL. */
typedef struct {
  void* param;          /* rows x cols, dtype; updated in place               */
  const void* grad;     /* rows x cols, dtype; read only                      */
  float* momentum;      /* rows x cols float32; updated in place              */
  int64_t rows, cols;
  int64_t ld_param, ld_grad, ld_momentum;  /* elements; >= cols               */
  int32_t dtype;        /* muon_dtype_t of param and grad                     */
  int32_t split_rows;   /* 0: whole matrix; h > 0: orthogonalise each block of
                           h consecutive rows separately (packed Q/K/V; Muon
                           blog sec. 1); h must divide rows                   */
  int32_t precond;      /* -1: none; else preconditioner slot index           */
  float lr_mult;        /* per-matrix lr multiplier (1.0 = none)              */
  float* update_out;    /* optional: rows x cols float32, contiguous (ld =
                           cols); receives the orthogonalised update O of this
                           step, before lr/scale.  NULL = not written.        */
  int32_t kind;         /* muon_kind_t; 0 (MUON) in a zero-filled struct      */
  int32_t reserved;     /* 0                                                  */
  float* exp_avg_sq;    /* kind ADAMW: rows x cols float32 second moment,
                           leading dimension ld_momentum; NULL for MUON       */
} muon_tensor_t;

/* A preconditioner slot: nblocks inverse second moments of size d x d.  A
 * matrix using the slot must have cols == d * nblocks; block k acts on
 * columns [k*d, (k+1)*d) (Newton-Muon README: the MLP contraction uses four
 * diagonal blocks; Q/K/V, attention output and MLP expansion share one). */
typedef struct {
  int64_t d;
  int32_t nblocks;
  int32_t reserved;
} muon_precond_t;

typedef struct {
  float lr;              /* default 0.02 (Muon README, "Usage")               */
  float momentum;        /* 0.95                                              */
  float weight_decay;    /* 0.01                                              */
  float eps;             /* 1e-7, added to ||U||_F before dividing            */
  int32_t nesterov;      /* 1                                                 */
  int32_t ns_steps;      /* 5; 0 <= ns_steps <= 64                            */
  float ns_a, ns_b, ns_c;/* 3.4445, -4.7750, 2.0315                           */
  int32_t scale_mode;    /* muon_scale_t, default ORIGINAL                    */
  int32_t momentum_form; /* muon_momentum_form_t, default EMA                 */
  /* AdamW for kind-ADAMW tensors (Muon README, "Usage": lr 3e-4, betas
   * (0.9, 0.95), weight_decay 0.01; eps is AdamW's usual 1e-8).  Step t of
   * the AdamW count: M = b1 M + (1-b1) G, V = b2 V + (1-b2) G^2,
   * W = W - lr*wd*W - lr * (M/(1-b1^t)) / (sqrt(V/(1-b2^t)) + eps). */
  float adam_lr;         /* 3e-4 (times the tensor's lr_mult)                 */
  float adam_beta1;      /* 0.9;  0 <= beta1 < 1                              */
  float adam_beta2;      /* 0.95; 0 <= beta2 < 1                              */
  float adam_eps;        /* 1e-8                                              */
  float adam_weight_decay; /* 0.01                                            */
} muon_hparams_t;

/* Fills the defaults listed above. */
void muon_default_hparams(muon_hparams_t* hp);

/* Pure host: validates the request and reports the workspace bytes that
 * muon_init() needs for it.  No GPU call. */
muon_status_t muon_workspace_size(const muon_tensor_t* tensors, int32_t n_tensors,
                                  const muon_precond_t* preconds, int32_t n_preconds,
                                  const muon_hparams_t* hp, size_t* bytes);

/* Validates, plans and binds a handle to the tensors and the workspace
 * (device memory, >= muon_workspace_size() bytes, 256-byte aligned).  Enqueues
 * the workspace initialisation (descriptor upload and zero fill) on
 * `stream`.  The tensors array is copied; the pointers it holds are kept. */
muon_status_t muon_init(muon_handle_t* out, const muon_tensor_t* tensors, int32_t n_tensors,
                        const muon_precond_t* preconds, int32_t n_preconds,
                        const muon_hparams_t* hp, void* workspace, size_t workspace_bytes,
                        void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same as
 * muon_init, but the workspace is the library's own static device array of
 * 64 MiB per GPU (held by each GPU the library runs on until the process
 * ends), so the call takes no workspace and allocates nothing on the device.
 * The handle creates no streams or events either: muon_step runs every launch
 * on the caller's stream.  Requests whose workspace (muon_workspace_size)
 * exceeds 64 MiB return MUON_ERR_WORKSPACE_TOO_SMALL before any GPU call.
 * The array belongs to the calling thread's current device.  All static
 * handles of one GPU share it: each muon_init_static zero-fills it for its
 * own plan, which supersedes every earlier static handle of that GPU (their
 * calls then return MUON_ERR_BAD_ARG; muon_destroy still releases them).
 * Work of a superseded handle still queued, or of two static handles used on
 * one GPU at once, races on the array. */
muon_status_t muon_init_static(muon_handle_t* out, const muon_tensor_t* tensors, int32_t n_tensors,
                               const muon_precond_t* preconds, int32_t n_preconds,
                               const muon_hparams_t* hp, void* stream);

/* Newton-Muon: rebuilds block `block` of preconditioner slot `slot` from
 * n_rows x d activations (row-major, leading dimension ld, dtype) of the
 * layer input: S = X^T X / n_rows + damping * I (float32), then S^-1 by a
 * Cholesky factorisation done in float64 (Newton-Muon README, "What Is
 * Newton-Muon?").  Asynchronous on `stream`.  If S is not numerically
 * positive definite, the non-finite pivot propagates through the factor, so
 * the block's S^-1 is not finite (NaN), and flag bit 1 is set. */
muon_status_t muon_precond_refresh(muon_handle_t h, int32_t slot, int32_t block,
                                   const void* acts, int64_t n_rows, int64_t ld,
                                   int32_t dtype, float damping, void* stream);

/* Newton-Muon, online form (the second moment gathered from micro-batches
 * as they pass, instead of one activation batch): adds the n_rows x d
 * activations of one micro-batch to the running sums of block `block` of
 * slot `slot`,
 *     Sigma <- beta * Sigma + X^T X,    N <- beta * N + n_rows
 * (beta = 1: plain sum over micro-batches; beta < 1: older micro-batches
 * weighted down exponentially; 0 <= beta <= 1).  X^T X is formed as in
 * muon_precond_refresh (bf16 or float32 MFMA, float32 sums).  Asynchronous
 * on `stream`.  The sums start at zero at muon_init(). */
muon_status_t muon_precond_accumulate(muon_handle_t h, int32_t slot, int32_t block, const void* acts,
                                      int64_t n_rows, int64_t ld, int32_t dtype, float beta, void* stream);

/* Rebuilds block `block` of slot `slot` from its running sums:
 * S = Sigma / N + damping * I, then S^-1 exactly as muon_precond_refresh
 * (a block with N = 0 gets S = damping * I).  reset != 0 clears Sigma and
 * N afterwards.  Asynchronous on `stream`; flag bit 1 as for
 * muon_precond_refresh. */
muon_status_t muon_precond_refresh_accumulated(muon_handle_t h, int32_t slot, int32_t block, float damping,
                                               int32_t reset, void* stream);

/* One optimizer step over every registered tensor: Muon on the kind-MUON
 * matrices (lr < 0 uses hp.lr), AdamW on the kind-ADAMW tensors (hp.adam_lr).
 * Asynchronous on `stream`; no allocation, no synchronisation.  Part of the
 * work may run on streams the handle created at muon_init (large groups of
 * matrices split in lanes; a float32 group beside a single-lane bf16 group;
 * AdamW beside the Muon phases): they wait for an
 * event recorded on `stream` at the start of the call and `stream` waits for
 * theirs at the end, so to the caller the step is ordered on `stream` alone
 * (also when `stream` is being captured into a graph). */
muon_status_t muon_step(muon_handle_t h, float lr, void* stream);

/* Like muon_step(), but records HIP events around each kernel phase and
 * synchronises `stream` at the end; phase_ms[i] receives the elapsed
 * milliseconds of phase i (see muon_phase_name) and *n_phases their count
 * (at most max_phases are written).  Every launch runs on `stream`, one
 * after the other (no lanes), so each phase's time is that launch's alone.
 * For profiling only. */
muon_status_t muon_step_timed(muon_handle_t h, float lr, void* stream,
                              float* phase_ms, int32_t max_phases, int32_t* n_phases);
const char* muon_phase_name(muon_handle_t h, int32_t phase);

/* AdamW step count.  The count lives in the workspace: muon_init() sets it
 * to 0 and every muon_step() that has kind-ADAMW tensors advances it by one
 * on the device before using it (so the first step is t = 1).  To resume,
 * set the number of steps already taken; both calls are asynchronous on
 * `stream` except that muon_get_adam_step() synchronises it to return the
 * value. */
muon_status_t muon_set_adam_step(muon_handle_t h, int64_t steps_taken, void* stream);
muon_status_t muon_get_adam_step(muon_handle_t h, void* stream, int64_t* steps_taken);

/* Synchronises `stream` and returns the sticky flag word:
 * bit 0 = a non-finite value was seen in an update, bit 1 = a
 * preconditioner factorisation failed, bit 2 = (only in a library built
 * with MUON_DEBUG_BOUNDS=1) a kernel task failed its bounds check and was
 * skipped.  reset != 0 clears it. */
muon_status_t muon_get_flags(muon_handle_t h, void* stream, int32_t reset, uint32_t* flags);

/* Synchronises the last stream used and frees the host handle. */
muon_status_t muon_destroy(muon_handle_t h);

/* Pure host: a JSON description of the plan muon_init() would build
 * (units, sides, padded sizes, per-phase tile counts, launch order).
 * Writes at most `len` bytes including the terminator; returns the full
 * length needed in *needed. */
muon_status_t muon_plan_describe(const muon_tensor_t* tensors, int32_t n_tensors,
                                 const muon_precond_t* preconds, int32_t n_preconds,
                                 const muon_hparams_t* hp, char* buf, size_t len,
                                 size_t* needed);

const char* muon_status_str(muon_status_t s);
const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */

/*
 * muon_mi355x.h: C ABI of the MI355X (gfx950) Muon / Dimuon optimizer step.
 *
 * One call updates a batch of independent 2-D weight matrices of mixed
 * shapes:
 *
 *   momentum      M_t = mu * M_{t-1} + G
 *                 ("Muon Optimizer 정리", section "업데이트 규칙", eq. (1))
 *   orthogonalise O_t = NS5(M_t).  Divide by the Frobenius norm, then apply
 *                 X <- aX + b(XX^T)X + c(XX^T)^2 X a set number of times,
 *                 with (a, b, c) = (3.4445, -4.7750, 2.0315).
 *                 (same page, eq. (2) and section "Newton-Schulz 직교화";
 *                 sitech.ge Muon blog, section "SVD-ի փոխարեն՝ Newton–Schulz")
 *   update        W_t = W_{t-1} - lr * O_t   (same page, eq. (3))
 *
 * Gram side: when m > n, the library iterates on X^T, so the Gram matrix is
 * min(m, n) square ("From PCG to Muon", section "Muon's Gram Matrix").
 *
 * dimuon_step adds the diagonal conditioning of "Dimuon: LoRA 에 맞춰 다시 짠
 * Muon" (optim-book, "Dimuon diagonal conditioning"):
 *   - row energies R_i and column energies C_j are sums of squares of the
 *     momentum as it was BEFORE this step's update (section
 *     "왜 「지난」 모멘텀인가");
 *   - each factor is d = (E / max(E) + eps)^(-1/4) (section "문제 4");
 *   - the factors scale the momentum before orthogonalisation and the result
 *     after it (section "양쪽에서 −1/4 제곱");
 *   - the step is then rescaled so that ||O||_F equals the Frobenius norm of
 *     the orthogonaliser's output (the norm is fixed afterwards);
 *   - if the previous momentum is all zero, the factors are 1 and the step
 *     equals muon_step bit for bit.
 *
 * R and C are float32 sums in a fixed pairwise order.  Each square is
 * fl(x*x) of the stored value x.  The sequence along the row (column) is
 * zero-padded to a power of two.  Adjacent pairs are then added level by
 * level, left + right, each addition rounded to float32.  The order depends
 * only on (m, n).
 *
 * Optional extensions, all off by default:
 *   - Nesterov input G + mu*M_t ("From PCG to Muon", "DL Optimizer w/ Line
 *     Search");
 *   - decoupled weight decay, and a per-matrix update scale ("Muon
 *     Optimizer 정리", section "참고: 대규모 학습으로의 확장");
 *   - a per-iteration (a, b, c) schedule, the mechanism of the Polar Express
 *     iteration the Dimuon page names.
 *
 * Conventions
 *   - Every matrix is row-major and contiguous.  Its element size follows
 *     the dtype in the config.  Device pointers must be 16-byte aligned.
 *   - The caller owns all memory, including the workspace.  The library
 *     allocates no device memory.  It does allocate pinned host staging
 *     buffers, from which the batch's descriptor table (a few KB per matrix
 *     batch) is copied into the workspace: muon_step and dimuon_step keep
 *     them per host thread, take one whose previous copy has completed or
 *     else allocate another (hipHostMalloc), up to 64 per thread, and free
 *     them when the thread exits; a plan holds one, freed by
 *     muon_plan_destroy.  The only host-side wait: a thread that already
 *     has 64 descriptor copies in flight waits for its oldest.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     default stream).  Host-side validation runs before anything is
 *     enqueued.  An invalid call returns an error code and leaves every
 *     buffer untouched.
 *   - muon_step and dimuon_step upload the descriptor table (a few KB) into
 *     the workspace on every call.  Calls that share a workspace must be
 *     ordered, for example on one stream.
 *   - A plan (muon_plan_create) validates and uploads once; muon_plan_step
 *     then only launches kernels.  While a plan exists, its workspace and
 *     every buffer it names must stay allocated, and the caller must not
 *     write to the workspace.
 *   - Numerical edge cases are not errors.  ||M||_F = 0 gives O = 0.
 *     NaN and Inf propagate as IEEE arithmetic does.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 1

typedef enum muon_dtype {
  MUON_F32 = 0,  /* IEEE binary32 */
  MUON_BF16 = 1  /* bfloat16: 8 significant bits, binary32 exponent range */
} muon_dtype_t;

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1,  /* null pointer, bad size, count < 1, bad ns_steps, ... */
  MUON_ERR_DTYPE = 2,        /* unsupported dtype combination */
  MUON_ERR_WORKSPACE = 3,    /* workspace null, misaligned or too small */
  MUON_ERR_ALIAS = 4,        /* two buffers of the batch overlap where they must not */
  MUON_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed */
  MUON_ERR_UNSUPPORTED = 6   /* shape outside the supported range */
} muon_status_t;

/* One matrix of the batch.  Sizes are in elements. */
typedef struct muon_matrix {
  void* w;              /* device, m*n of cfg.w_dtype; W_{t-1} in, W_t out */
  const void* g;        /* device, m*n of cfg.g_dtype; gradient, read only */
  void* mom;            /* device, m*n of cfg.mom_dtype; M_{t-1} in, M_t out */
  float* o_out;         /* device or NULL: m*n float32, receives O_t (before lr) */
  float* energy_out;    /* device or NULL: m+n float32, receives R then C
                           (dimuon_step only; ignored by muon_step) */
  int64_t m;            /* rows, 1 <= m <= 65536 */
  int64_t n;            /* columns, 1 <= n <= 65536 */
  float update_scale;   /* multiplies O in the update; 1 for plain Muon */
  float reserved0;
} muon_matrix_t;

typedef struct muon_config {
  float lr;                     /* learning rate eta */
  float momentum;               /* mu */
  int32_t ns_steps;             /* Newton-Schulz iterations, 0..32; 5 is NS5 */
  float a, b, c;                /* quintic coefficients */
  const float* coeff_schedule;  /* host or NULL: ns_steps triples (a_t, b_t, c_t)
                                   replacing (a, b, c) iteration by iteration */
  muon_dtype_t w_dtype;         /* F32 or BF16 */
  muon_dtype_t g_dtype;         /* F32 or BF16 */
  muon_dtype_t mom_dtype;       /* F32 or BF16 */
  muon_dtype_t ns_dtype;        /* BF16: bf16 MFMA products with fp32 accumulation;
                                   F32: fp32 products and accumulation */
  float dimuon_eps;             /* floor added to the relative energy (1e-4) */
  int32_t nesterov;             /* nonzero: orthogonalise G + mu*M_t instead of M_t */
  float weight_decay;           /* W_t = W_{t-1} - lr*(scale*O_t + weight_decay*W_{t-1}) */
  int32_t reserved[4];
} muon_config_t;

/* Fill `cfg` with the defaults: lr 0.02, mu 0.95, NS5 (3.4445, -4.7750,
 * 2.0315), bf16 everywhere, eps 1e-4, no Nesterov, no weight decay. */
void muon_config_default(muon_config_t* cfg);

/* Bytes of device workspace a call over this batch needs.  The value covers
 * both muon_step and dimuon_step.  It is written to *bytes.  Checks the
 * arguments as a step would, but does not check pointers to buffers.
 * Errors: INVALID_ARG, DTYPE, UNSUPPORTED. */
muon_status_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t count,
                                   const muon_config_t* cfg, size_t* bytes);

/* One Muon step over `count` matrices (host array `mats`).  `workspace` is
 * device memory of at least muon_workspace_bytes() bytes, 256-byte aligned.
 * Enqueues on `stream` and returns without synchronising (a thread with 64
 * descriptor copies still in flight first waits for its oldest; see the
 * staging buffers above).
 * Errors: INVALID_ARG, DTYPE, WORKSPACE, ALIAS, UNSUPPORTED, HIP. */
muon_status_t muon_step(const muon_matrix_t* mats, int64_t count,
                        const muon_config_t* cfg, void* workspace,
                        size_t workspace_bytes, void* stream);

/* One Dimuon step.  Same arguments and errors as muon_step. */
muon_status_t dimuon_step(const muon_matrix_t* mats, int64_t count,
                          const muon_config_t* cfg, void* workspace,
                          size_t workspace_bytes, void* stream);

/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  One Muon step
 * (dimuon = 0) or Dimuon step (dimuon != 0) with the semantics of
 * muon_step / dimuon_step, but with no workspace argument: the library's
 * own static device array of MUON_NOALLOC_MAX_BYTES (64 MiB, held by each
 * GPU the library runs on until the process ends) serves as the workspace,
 * and the descriptor table reaches it through kernel arguments.  The call
 * allocates nothing: no device memory, no pinned host memory.
 *   - The batch must fit: a batch whose muon_workspace_bytes() exceeds
 *     MUON_NOALLOC_MAX_BYTES is rejected with MUON_ERR_WORKSPACE before
 *     anything is enqueued.  (Thin batches fit easily: the 64 LoRA pairs
 *     of 8 x 4096 and 4096 x 8 need about 7 MB.)
 *   - `stream` must belong to the current device; the array of that device
 *     is used.  Every call on one GPU shares that GPU's array, which keeps
 *     the last call's contents (no call depends on them): calls that
 *     overlap on one GPU race and must be ordered, for example on one
 *     stream.
 *   - Results equal muon_step / dimuon_step bit for bit (the same kernels).
 * Errors: INVALID_ARG, DTYPE, WORKSPACE (batch too large), ALIAS,
 * UNSUPPORTED, HIP. */
#define MUON_NOALLOC_MAX_BYTES ((size_t)64 << 20)
muon_status_t muon_step_noalloc(const muon_matrix_t* mats, int64_t count,
                                const muon_config_t* cfg, int32_t dimuon,
                                void* stream);

/* Kernel kinds reported by the launch-event hook. */
typedef enum muon_launch_kind {
  MUON_LAUNCH_START = -1,     /* event recorded before the first launch */
  MUON_LAUNCH_THIN = 0,       /* thin path pass B: k x k iteration, next energies, apply, update */
  MUON_LAUNCH_MOMENTUM = 1,   /* (not emitted: the momentum runs in the prescale pass) */
  MUON_LAUNCH_CONDITION = 2,  /* energies -> Dimuon factors */
  MUON_LAUNCH_PRESCALE = 3,   /* (not emitted: see MOMENTUM_PRESCALE) */
  MUON_LAUNCH_NORM = 4,       /* Frobenius norm of the prescaled copy */
  MUON_LAUNCH_GRAM = 5,       /* A = X X^T */
  MUON_LAUNCH_POLY = 6,       /* B = b A + c A A */
  MUON_LAUNCH_COMBINE = 7,    /* X = a X + B X (Muon, bf16 weights with rows of whole 8-element
                                 runs: the last one also applies the weight update) */
  MUON_LAUNCH_POSTNORM = 8,   /* Dimuon norm fix */
  MUON_LAUNCH_UPDATE = 9,     /* O and the weight update (not emitted when the last combine
                                 updated every matrix) */
  MUON_LAUNCH_THIN_ENERGY = 10, /* thin path: energies of M_{t-1} (no cached energies) */
  MUON_LAUNCH_THIN_A = 11,    /* thin path pass A: momentum, Gram partials */
  MUON_LAUNCH_MOMENTUM_PRESCALE = 12, /* momentum, Dimuon energies of M_t, conditioned and
                                         normalised bf16/f32 copy (+ transpose), one pass */
  MUON_LAUNCH_ENERGY = 13     /* energies of M_{t-1} (general path, no cached energies) */
} muon_launch_kind_t;

/* Timing hook, per host thread; not part of the method.  When `events` is
 * non-NULL, each later step on this thread records events[0] on the step's
 * stream before its first launch and events[i] after its i-th launch.  The
 * kind of launch i is written to kinds[i] (kinds[0] = MUON_LAUNCH_START).
 * `events` are hipEvent_t the caller created on the stream's device.  At
 * most `n` events are recorded.  Pass NULL to switch the hook off.  The
 * return value is the number of events the last step recorded. */
int32_t muon_set_launch_events(void* const* events, int32_t* kinds, int32_t n);

/* Prepared batch for repeated steps (an optimizer's fixed parameter list).
 * Validation, planning and the descriptor upload happen once, in create.
 * Each muon_plan_step runs one Muon step (dimuon = 0) or one Dimuon step
 * (dimuon != 0) over the batch, with the same semantics as muon_step /
 * dimuon_step.  The config, including the coefficient schedule, is copied.
 * Errors of create: as muon_step; of step: INVALID_ARG (NULL plan), HIP. */
typedef struct muon_plan muon_plan_t;
muon_status_t muon_plan_create(const muon_matrix_t* mats, int64_t count,
                               const muon_config_t* cfg, int32_t dimuon,
                               void* workspace, size_t workspace_bytes,
                               void* stream, muon_plan_t** plan);
muon_status_t muon_plan_step(muon_plan_t* plan, void* stream);
/* A Dimuon plan keeps, in its workspace, the row/column energies of the
 * momentum its last step wrote (the next step's R and C), so the next step
 * need not read M_{t-1} an extra time to compute them.  Call
 * muon_plan_reset after writing to the momentum buffers outside the plan
 * (resume, reset); the next step then recomputes them.  Muon plans ignore it. */
muon_status_t muon_plan_reset(muon_plan_t* plan);
/* Learning rate used by later steps of the plan (must be finite). */
muon_status_t muon_plan_set_lr(muon_plan_t* plan, float lr);
/* Replay the plan's launch sequence as a HIP graph (enable != 0) or launch
 * its kernels one by one (enable = 0, the default).  With graphs on, the
 * first step in each state of the sequence captures it (on a private stream
 * the plan creates; a Dimuon plan alternates between two states) and every
 * step then launches the instantiated graph on `stream`.  Results are the
 * same bit for bit.  Steps that run eagerly even with graphs on: a Dimuon
 * plan's first step and the step after muon_plan_reset (they also compute
 * the energies of M_{t-1}), and steps timed through muon_set_launch_events.
 * muon_plan_set_lr with a new rate discards the captured graphs.
 * Errors: INVALID_ARG (NULL plan), HIP. */
muon_status_t muon_plan_set_graph(muon_plan_t* plan, int32_t enable);
/* Waits for the plan's upload to finish, then frees the plan (NULL is a no-op). */
void muon_plan_destroy(muon_plan_t* plan);

/* Static description of a status code. */
const char* muon_status_string(muon_status_t status);

/* Detail message of the last failed call on this host thread ("" if none). */
const char* muon_last_error(void);

/* MUON_ABI_VERSION of the loaded library. */
int32_t muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */

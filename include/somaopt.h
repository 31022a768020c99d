/*
 * somaopt.h - fused clip + AdamW optimizer step for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (SomaSpeed landing page, prose paragraphs 7 and 8,
 * numbered in page order after the title: the post-backward optimizer work and
 * its fused form): after backward, over a table of many trainable tensors,
 *   1. divide every gradient by the effective-batch divisor D,
 *   2. measure one global L2 norm in which every owned gradient element counts
 *      once,
 *   3. take one global clip decision  c = min(1, max_norm / (norm + 1e-6))
 *      (the clip_grad_norm_ rule the veRL page applies with max_norm = 1.0,
 *      "Phase 4: Actor Update", section 4.2 "PPO Update"),
 *   4. in one fused pass that reads the ORIGINAL gradient, apply
 *      normalization, clipping and decoupled-weight-decay AdamW to the fp32
 *      weight and both fp32 moments, per parameter group:
 *        g_hat = g * c / D
 *        m     = beta1 * m + (1 - beta1) * g_hat
 *        v     = beta2 * v + (1 - beta2) * g_hat^2
 *        p     = p - lr*wd*p - (lr / (1 - beta1^t)) * m / (sqrt(v / (1 - beta2^t)) + eps)
 *      with t the group's update count, 1 on the first update.
 * Gradient buffers are never written and frozen tensors are never read or
 * written (paragraph 8).  bf16 and fp16 gradients are widened to fp32 for
 * the update, the optimizer state stays fp32, and an optional bf16/fp16
 * working copy of the weights is rewritten from the fp32 master (RLinf page,
 * "Retaining Low-Precision Gradients").
 *
 * Conventions for every call:
 *   - Pointers in somaopt_tensor_desc are DEVICE pointers on the device that
 *     is current when somaopt_init_tensor_table is called; the caller owns the
 *     memory, must keep it alive and at the same address for the handle's
 *     lifetime (no reallocation of gradients between steps).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Step-path calls only enqueue work on it and never wait for the device.
 *   - Every call returns a somaopt_status; on failure somaopt_last_error()
 *     returns a message (thread-local, valid until the next call on the same
 *     thread).  Nothing throws across this interface.
 *   - A handle is used from one host thread at a time.  Calls that mutate the
 *     device-side state (set_groups, set_clip, set_step, the step itself) are
 *     ordered by the stream they are enqueued on; use one stream per handle or
 *     order streams yourself.
 */
#ifndef SOMAOPT_H
#define SOMAOPT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SOMAOPT_MAX_GROUPS 64

typedef enum {
    SOMAOPT_OK = 0,
    SOMAOPT_E_INVALID = -1, /* an argument or a tensor descriptor is invalid      */
    SOMAOPT_E_HIP = -2,     /* a HIP runtime call or kernel launch failed         */
    SOMAOPT_E_NOMEM = -3,   /* a device or host allocation failed                 */
    SOMAOPT_E_STATE = -4    /* call order violated (see each call)                */
} somaopt_status;

typedef enum {
    SOMAOPT_F32 = 0,  /* IEEE binary32                                            */
    SOMAOPT_BF16 = 1, /* bfloat16 (top 16 bits of a binary32)                     */
    SOMAOPT_F16 = 2   /* IEEE binary16                                            */
} somaopt_dtype;

/* One entry of the tensor table.  A tensor cut by a shard boundary, or a
 * replica, is simply another entry whose pointers address that piece. */
typedef struct {
    void* param;          /* fp32 weights (the master copy), numel elements,
                             updated in place                                   */
    const void* grad;     /* gradient, grad_dtype (any somaopt_dtype), numel
                             elements, read only                                */
    void* exp_avg;        /* fp32 first moment m, updated in place             */
    void* exp_avg_sq;     /* fp32 second moment v, updated in place            */
    int64_t numel;        /* >= 0; 0 is allowed and skipped                    */
    int32_t grad_dtype;   /* somaopt_dtype                                      */
    int32_t group;        /* parameter group, 0 <= group < n_groups             */
    int32_t trainable;    /* 0: frozen; never read or written, pointers may be NULL */
    int32_t owner;        /* 1: counts in the global norm; 0: updated only (a
                             replica or a piece another rank owns)              */
    void* param_lowp;     /* optional (NULL = none): bf16 or fp16 working copy
                             of the weights, numel elements, overwritten by each
                             update with the updated fp32 master rounded to
                             nearest, ties to even (RLinf page, "Retaining
                             Low-Precision Gradients": BF16/FP16 parameters keep
                             an FP32 master copy)                               */
    int32_t lowp_dtype;   /* SOMAOPT_BF16 or SOMAOPT_F16 when param_lowp is set */
    int32_t reserved;     /* must be 0                                          */
} somaopt_tensor_desc;

/* Per-group hyperparameters (the group's lr at this step, after the caller's
 * schedule).  Doubles on input; derived per-step constants are computed on the
 * device in fp64 and the elementwise update runs in fp32. */
typedef struct {
    double lr;
    double weight_decay;
    double beta1;
    double beta2;
    double eps;
} somaopt_group;

/* Step statistics, resident in device memory (see somaopt_device_stats). */
typedef struct {
    double sumsq;        /* sum over owned trainable elements of g^2 (raw g)  */
    double norm;         /* sqrt(sumsq) / grad_divisor                        */
    double clip_coef;    /* min(1, max_norm / (norm + 1e-6)); NaN if norm is NaN */
    double grad_scale;   /* clip_coef / grad_divisor: multiplies raw g        */
    int32_t nonfinite;   /* 1 if sumsq is NaN or infinite (step still runs)   */
    int32_t n_groups;
} somaopt_stats;

/* Counts describing the device tables built at init. */
typedef struct {
    int64_t n_tensors;          /* descriptors passed in                       */
    int64_t n_trainable;        /* descriptors with trainable != 0             */
    int64_t trainable_numel;    /* elements updated per step (N)               */
    int64_t owned_numel;        /* elements summed in the norm (N_o)           */
    int64_t pass1_segments;     /* gradient segments read by the norm pass     */
    int64_t pass1_blocks;       /* workgroups of the norm pass                 */
    int64_t pass2_segments;     /* segments of the update pass                 */
    int64_t pass2_blocks;       /* workgroups of the update pass               */
    int64_t scalar_segments;    /* update segments that cannot use 16-byte loads */
    int64_t pass1_chunk;        /* max elements per norm-pass workgroup        */
    int64_t pass2_chunk;        /* max elements per update-pass workgroup      */
    int64_t table_bytes;        /* device bytes of the descriptor tables       */
    int64_t pass1_wg_per_cu;    /* resident norm-pass workgroups per CU (0: no limit)   */
    int64_t pass2_wg_per_cu;    /* resident update-pass workgroups per CU (0: no limit) */
    int64_t pass2_launches;     /* launches the update pass is split into (consecutive
                                   ranges of its workgroups, same stream; 0 if empty) */
} somaopt_plan_info;

/* One row of the host-side plan, for inspection (somaopt_debug_plan). */
typedef struct {
    int64_t tensor;      /* descriptor index                                   */
    int64_t offset;      /* first element of the segment inside the tensor    */
    int64_t numel;       /* elements in the segment                           */
    int64_t nvec;        /* aligned vectors after the scalar head             */
    int32_t head;        /* scalar elements before the first vector           */
    int32_t tail;        /* scalar elements after the last vector             */
    int32_t vec_elems;   /* elements per vector (0: all scalar)               */
    int32_t block;       /* workgroup index that processes the segment        */
} somaopt_plan_segment;

typedef struct somaopt_handle somaopt_handle;

/*
 * Build the device-resident tensor and chunk tables (the landing page,
 * paragraph 8, batches the optimizer work across tensors) so that each pass is
 * one kernel launch over all tensors.
 *
 *   descs[n_tensors]   tensor table (host memory, copied; may be freed after)
 *   groups[n_groups]   initial per-group hyperparameters, 1..SOMAOPT_MAX_GROUPS
 *   max_norm           clip threshold M (> 0)
 *   grad_divisor       effective-batch divisor D (> 0), e.g. the number of
 *                      micro-batches accumulated (veRL page, section 4.2)
 *   initial_step       updates already applied (0 for a fresh optimizer;
 *                      resume passes the saved count)
 *   stream             stream for the one-time upload; this call waits for it
 *   out                receives the new handle
 *
 * Frozen descriptors are dropped here and never appear in any table.
 * Validation (SOMAOPT_E_INVALID): NULL pointer or misaligned (4-byte fp32,
 * 2-byte bf16/fp16) buffer on a trainable tensor, numel < 0, group out of
 * range, unknown dtype, owner/trainable not 0/1, a working copy whose dtype is
 * not bf16/fp16, any overlap between the written buffers (p, m, v, working
 * copy) of trainable tensors or between a gradient and any written buffer,
 * a buffer that is not device memory of the current device or that runs past
 * the end of its allocation (skipped if SOMAOPT_SKIP_POINTER_CHECK=1).
 * Tuning (optional environment): SOMAOPT_PASS1_CHUNK, SOMAOPT_PASS2_CHUNK =
 * maximum elements per workgroup of the norm / update pass (unset: 8192, and
 * for the update pass 4096, or 2048 when most elements lie in full-length
 * segments; each at most 2^26, larger values are lowered to it);
 * SOMAOPT_PASS1_WG_PER_CU, SOMAOPT_PASS2_WG_PER_CU = resident
 * workgroups per compute unit (0: no limit; unset: chosen from the table
 * shape, reported in somaopt_plan_info); SOMAOPT_SEGMENT_COST,
 * SOMAOPT_UPDATE_SEGMENT_COST = elements charged per segment when short
 * segments are packed into the norm / update pass's workgroups (1024, 4096);
 * SOMAOPT_PASS2_SLICE_BLOCKS = update-pass workgroups per launch above which
 * the pass is split into several launches (262144; 0: always one launch).
 */
int somaopt_init_tensor_table(const somaopt_tensor_desc* descs, int64_t n_tensors,
                              const somaopt_group* groups, int32_t n_groups,
                              double max_norm, double grad_divisor, int64_t initial_step,
                              void* stream, somaopt_handle** out);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * table build as somaopt_init_tensor_table, with the same arguments, errors
 * and resulting handle, except that every device buffer of the handle (the
 * norm- and update-pass tables, the per-workgroup partials and the optimizer
 * state block) is carved from a per-device scratch array inside the library
 * instead of being allocated.  The call makes no hipMalloc, hipFree or other
 * device allocation (it uploads the tables with hipMemcpyAsync on `stream`
 * and waits for that stream, like the allocating call).
 *   - Limit: the array holds 32 MiB (33,554,432 bytes) per device, held from
 *     the first use until the process ends.  That fits tables of about 8.9e8
 *     elements in large tensors (the 302M-element action head needs 11.4 MB);
 *     a table that needs more is refused with SOMAOPT_E_INVALID and a message
 *     giving both sizes, before anything touches the device.
 *   - Sharing: every no-allocation handle of a device uses the same array.
 *     Each successful call overwrites it and supersedes the no-allocation
 *     handles built before it on that device: from then on every call on an
 *     older one returns SOMAOPT_E_STATE ("superseded"); only
 *     somaopt_destroy is still allowed.  Work still in flight from an older
 *     handle races with the new build: let it complete first (calls that
 *     overlap on one device race).
 *   - The other calls that allocate (somaopt_capture_step, the arrival
 *     registration) keep allocating when used on such a handle;
 *     somaopt_destroy frees nothing in the array.
 */
int somaopt_init_tensor_table_noalloc(const somaopt_tensor_desc* descs, int64_t n_tensors,
                                      const somaopt_group* groups, int32_t n_groups,
                                      double max_norm, double grad_divisor, int64_t initial_step,
                                      void* stream, somaopt_handle** out);

/*
 * Norm pass: one launch over every owned gradient segment (fp64 sum of
 * squares per workgroup), then a one-workgroup finalize kernel on the same
 * stream (no host sync) that adds the partials in a fixed order and derives the
 * norm, the clip coefficient and each group's bias-corrected constants for the
 * next update.  Landing page, paragraph 8: the statistics for the single
 * global clip decision are gathered first, with every gradient shard counted
 * exactly once under distributed ownership.
 * Calling it again before somaopt_fused_adamw_step recomputes the same
 * statistics for the same pending update (the step count advances once).
 */
int somaopt_grad_sqnorm(somaopt_handle* h, void* stream);

/*
 * Update pass: one launch over every trainable segment (a pass of more than
 * 262144 workgroups, about 5.4e8 elements, goes out as consecutive launches
 * over ranges of its workgroups, each still spanning many tensors: see
 * somaopt_plan_info.pass2_launches); reads g, p, m, v and writes p, m, v using
 * the statistics the preceding somaopt_grad_sqnorm left on the device.  Landing page, paragraph 8: the last pass works from the
 * unmodified gradients and does normalization, clipping and AdamW at once.
 * SOMAOPT_E_STATE if no somaopt_grad_sqnorm preceded it since the last update.
 */
int somaopt_fused_adamw_step(somaopt_handle* h, void* stream);

/*
 * Gradient arrival with the norm pass fused in -- the step just before the
 * optimizer path.  With sharded state (landing page, paragraph 1) every GPU
 * receives its already-reduced gradient shard after backward and adds it into
 * the gradient shard it holds; the fused optimizer then first needs the owned
 * sum of squares of those gradients (paragraph 8).  Doing both in one pass
 * removes the norm pass's separate read of every gradient.
 *
 * somaopt_register_arrival, once per handle: incoming[i] is the device buffer
 * whose values arrive for descriptor i (same numel, gradient dtype and element
 * order as its grad; ignored and may be NULL for frozen descriptors).  The
 * buffers must stay at these addresses for the handle's lifetime.  The arrival
 * pass writes the gradients, so for registration gradients must not overlap
 * one another or any param/exp_avg/exp_avg_sq/working copy, and no incoming
 * buffer may overlap any of those or any gradient (incoming buffers may
 * overlap each other).  Builds a device table (synchronizes `stream` once).
 * SOMAOPT_E_INVALID on a bad pointer, overlap or count; SOMAOPT_E_STATE if
 * already registered.  Tuning (optional environment, read here):
 * SOMAOPT_PASS3_CHUNK = maximum elements per arrival-pass workgroup (unset:
 * the norm pass's, halved to 4096 for a table of large tensors, at most 2^26);
 * SOMAOPT_PASS3_SLICE_BLOCKS = arrival-pass workgroups per launch above which
 * the pass is split into several launches (131072; 0: always one launch); the
 * statistics do not depend on the split.  SOMAOPT_PASS3_WG_PER_CU = resident
 * arrival-pass workgroups per compute unit, both modes (0: no limit; unset:
 * for a streaming table none when copying and six when accumulating, none
 * for a packed one).
 *
 * somaopt_arrival_sqnorm: for every trainable descriptor
 *     accumulate = 0:  grad <- incoming                      (bitwise copy)
 *     accumulate = 1:  grad <- round(grad + incoming)        (fp32 sum of the
 *                      exactly widened values, rounded once to the gradient
 *                      dtype, nearest even; fp32 gradients: the fp32 sum)
 * then, on the new gradients, exactly the statistics somaopt_grad_sqnorm
 * would produce (owned fp64 sum of squares in a fixed order, norm, clip
 * coefficient, per-group constants; the step count advances once per pending
 * update).  It takes the place of somaopt_grad_sqnorm: the next
 * somaopt_fused_adamw_step applies the update.  SOMAOPT_E_STATE before
 * registration.
 */
int somaopt_register_arrival(somaopt_handle* h, const void* const* incoming, int64_t n_tensors, void* stream);
int somaopt_arrival_sqnorm(somaopt_handle* h, int32_t accumulate, void* stream);

/* Replace every group's hyperparameters (n_groups must equal the handle's).
 * SomaSpeed landing page, paragraph 8: the fused optimizer keeps each
 * parameter group's settings and learning-rate schedule as configured; here a
 * group is the unit that carries lr, weight decay, betas and eps, and a
 * schedule evaluated on the host calls this before each step with the
 * group's new lr.  Enqueued as a tiny kernel whose arguments carry the
 * values, so the host array may be reused at once.  SOMAOPT_E_INVALID if
 * n_groups differs or a value is out of range (lr, weight_decay not finite;
 * beta outside [0, 1); eps negative or not finite). */
int somaopt_set_groups(somaopt_handle* h, const somaopt_group* groups, int32_t n_groups,
                       void* stream);

/* Learning-rate schedules evaluated on the device (optional; landing page,
 * paragraph 8: every parameter group keeps its own schedule).  A group with
 * a schedule takes, for its update t (1 on the first update), the lr below in
 * place of somaopt_group.lr; its other hyperparameters still come from init
 * or somaopt_set_groups.  The finalize of the norm (or arrival) pass computes
 * the lr in fp64 together with the bias corrections, so a captured step
 * replays the whole schedule with no host call between steps.  With
 * W = warmup, T = total, peak = peak_lr, floor = floor_lr:
 *   SOMAOPT_SCHED_NONE           lr = somaopt_group.lr (the default)
 *   SOMAOPT_SCHED_LINEAR_WARMUP  lr = peak * min(t, W) / W
 *   SOMAOPT_SCHED_COSINE         lr = floor + (peak - floor) * (1 + cos(pi * k / T)) / 2,
 *                                k = min(t - 1, T): peak at t = 1, floor from t = T + 1
 *   SOMAOPT_SCHED_WARMUP_COSINE  t <= W: the linear warmup; t > W: the cosine over
 *                                the remaining T - W updates (k = min(t - W - 1, T - W))
 * The new schedules apply from the next norm or arrival pass.  Errors
 * (SOMAOPT_E_INVALID): n_groups differs from the handle's, an unknown kind,
 * W < 1 for a warmup kind, T < 1 for a cosine kind, T <= W for warmup-cosine,
 * or a peak or floor lr that is negative or not finite. */
typedef enum {
    SOMAOPT_SCHED_NONE = 0,
    SOMAOPT_SCHED_LINEAR_WARMUP = 1,
    SOMAOPT_SCHED_COSINE = 2,
    SOMAOPT_SCHED_WARMUP_COSINE = 3
} somaopt_schedule_kind;
typedef struct {
    int32_t kind;      /* somaopt_schedule_kind */
    int32_t warmup;    /* W */
    int64_t total;     /* T */
    double peak_lr;
    double floor_lr;
} somaopt_schedule;
int somaopt_set_schedules(somaopt_handle* h, const somaopt_schedule* schedules, int32_t n_groups,
                          void* stream);

/* Replace max_norm and grad_divisor (both finite and > 0), stream ordered:
 * the clip threshold of the single global clip decision (landing page,
 * paragraph 8; the veRL page's section 4.2 clips at max_norm = 1.0) and the
 * effective-batch divisor (paragraph 7; the veRL page divides the loss by the
 * number of micro-batches).  Applies from the next norm or arrival pass. */
int somaopt_set_clip(somaopt_handle* h, double max_norm, double grad_divisor, void* stream);

/* Set every group's completed-update count (resume), stream ordered.  Clears
 * a pending norm pass.  The count is the t of the bias corrections, so a
 * resumed optimizer continues exactly where a saved one stopped (the veRL
 * page saves optimizer checkpoints periodically).  SOMAOPT_E_INVALID if
 * step < 0. */
int somaopt_set_step(somaopt_handle* h, int64_t step, void* stream);

/* Capture {norm pass, update pass} into a HIP graph owned by the handle
 * (captured on a private stream; nothing runs).  Replaces an earlier graph.
 * SomaSpeed landing page, paragraph 12: learner work that repeats every step
 * is recorded once as a graph and replayed, so a step costs one launch
 * instead of one per kernel.  Hyperparameters, schedules and the clip settings
 * live in device state that the captured kernels read, so they change without
 * a new capture.  SOMAOPT_E_HIP if capture or instantiation fails. */
int somaopt_capture_step(somaopt_handle* h);

/* Capture {arrival pass with the fused norm, update pass} instead -- the step
 * of somaopt_arrival_sqnorm(accumulate) followed by somaopt_fused_adamw_step
 * (graph replay of repeated learner work, landing page, paragraph 12; the
 * arrival of the gradient shard, paragraph 1).  Replaces an earlier graph.
 * SOMAOPT_E_STATE before somaopt_register_arrival; SOMAOPT_E_INVALID if
 * accumulate is not 0 or 1. */
int somaopt_capture_arrival_step(somaopt_handle* h, int32_t accumulate);

/* Launch the captured step on `stream`: one full step (norm or arrival pass
 * with its step advance, then update pass) in one graph launch (landing page,
 * paragraph 12: repeated learner work replayed from a graph).  Only enqueues.
 * SOMAOPT_E_STATE if not captured or if an eager norm pass is pending;
 * SOMAOPT_E_HIP if the launch fails. */
int somaopt_replay_step(somaopt_handle* h, void* stream);

/* Device address of the somaopt_stats block (valid for the handle's life). */
int somaopt_device_stats(somaopt_handle* h, const void** stats_dev);

/* Copy the stats and the per-group update counts (steps_out may be NULL,
 * else n_groups entries) to the host.  Waits for `stream`: not for the step
 * path. */
int somaopt_read_stats(somaopt_handle* h, somaopt_stats* out, int64_t* steps_out, void* stream);

/* Counts of the tables built at init. */
int somaopt_get_plan_info(const somaopt_handle* h, somaopt_plan_info* out);

/*
 * Host-only: validate `descs` (the checks of init that need no device) and
 * build the plan of one pass (pass = 1: norm pass, 2: update pass) without
 * touching a GPU.  Writes up to `cap` rows to `segs` (may be NULL) and the
 * counts to `info` (may be NULL).  pass1_chunk / pass2_chunk <= 0 select the
 * defaults; values above 2^26 are lowered to 2^26, as at init.  Returns the number of segments of that pass, or a negative status.
 */
int64_t somaopt_debug_plan(const somaopt_tensor_desc* descs, int64_t n_tensors, int32_t n_groups,
                           int32_t pass, int64_t pass1_chunk, int64_t pass2_chunk,
                           somaopt_plan_segment* segs, int64_t cap, somaopt_plan_info* info);

/* ------------------------------------------------------------------------
 * Tiled attention over frozen and trainable keys (SomaSpeed landing page,
 * paragraph 5: the action queries read context keys and values in tiles, the
 * full score matrix is never stored, and inputs that are frozen get no
 * gradient work).
 *
 * Per (batch b, head h): S = scale * Q K^T, P = softmax over keys, O = P V,
 * LSE = log sum_j exp(S_ij).  Keys [0, lk_frozen) are frozen: the backward
 * returns dQ for every query and dK, dV only for keys [lk_frozen, lk).
 * Layout (all row-major, rows contiguous, base pointers 16-byte aligned):
 *   q, o, d_o   bf16 [batch][heads][lq][head_dim]
 *   k, v        bf16 [batch][heads][lk][head_dim]
 *   lse, delta  fp32 [batch][heads][lq]
 *   dq          fp32 [batch][heads][lq][head_dim]
 *   dk, dv      fp32 [batch][heads][lk - lk_frozen][head_dim] (NULL allowed
 *               when lk_frozen == lk)
 * head_dim is 64 or 128; batch, heads <= 65535; lq, lk in [1, 2^22].  Products use
 * bf16 matrix-core inputs (P and dS rounded once to bf16) with fp32
 * accumulation.  Device pointers are caller-owned; the calls only enqueue
 * work on `stream`.  SOMAOPT_E_INVALID on a bad shape, a NULL or misaligned
 * pointer, or a buffer that is not device memory large enough for its shape.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t batch;
    int32_t heads;
    int32_t lq;          /* queries per (batch, head)                           */
    int32_t lk;          /* keys per (batch, head)                              */
    int32_t lk_frozen;   /* leading frozen keys, 0 <= lk_frozen <= lk           */
    int32_t head_dim;    /* 64 or 128                                           */
    float scale;         /* score scale, usually 1 / sqrt(head_dim)             */
} somaopt_attn_shape;

/* Forward: writes O (bf16) and LSE (fp32, natural log). */
int somaopt_attn_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                         const somaopt_attn_shape* shape, void* stream);

/* Backward from the saved O and LSE: writes dQ, and dK, dV of the trainable
 * keys; `delta` is a caller-provided fp32 [batch][heads][lq] workspace. */
int somaopt_attn_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                          float* delta, const somaopt_attn_shape* shape, void* stream);

/* ------------------------------------------------------------------------
 * The same attention with the keys split into two separate buffers, covering
 * the context structures of the landing page's paragraph 6 without copying
 * any key or value:
 *   - a frozen context (backbone features or a frozen prefix) shared by
 *     ctx_share consecutive query batches -- e.g. the sampled flow timesteps
 *     of one observation -- with no dK/dV;
 *   - trainable action keys/values, one set per query batch, whose dK/dV are
 *     returned.
 * Either part may be empty: l_act = 0 is cross-attention to frozen features
 * only, l_ctx = 0 is self-attention over trainable keys only.  For query
 * batch b the keys are context batch b / ctx_share followed by action batch
 * b; softmax runs over all of them.
 * Layout (row-major, rows contiguous, base pointers 16-byte aligned):
 *   q, o, d_o      bf16 [batch][heads][lq][head_dim]
 *   k_ctx, v_ctx   bf16 [batch / ctx_share][heads][l_ctx][head_dim] (NULL allowed if l_ctx == 0)
 *   k_act, v_act   bf16 [batch][heads][l_act][head_dim]             (NULL allowed if l_act == 0)
 *   lse, delta     fp32 [batch][heads][lq]
 *   dq             fp32 [batch][heads][lq][head_dim]
 *   dk_act, dv_act fp32 [batch][heads][l_act][head_dim]             (NULL allowed if l_act == 0)
 * Limits: head_dim 64 or 128; batch, heads <= 65535; lq in [1, 2^22];
 * l_ctx, l_act in [0, 2^22] with l_ctx + l_act >= 1; ctx_share >= 1 divides
 * batch.  Numerics, ownership and errors as for somaopt_attn_forward.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t batch;       /* query batches                                            */
    int32_t heads;
    int32_t lq;          /* queries per (batch, head)                                */
    int32_t l_ctx;       /* frozen context keys per (context batch, head)            */
    int32_t l_act;       /* trainable action keys per (batch, head)                  */
    int32_t ctx_share;   /* consecutive query batches reading one context batch      */
    int32_t head_dim;    /* 64 or 128                                                */
    float scale;         /* score scale, usually 1 / sqrt(head_dim)                  */
} somaopt_attn_ctx_shape;

/* Forward: writes O (bf16) and LSE (fp32, natural log). */
int somaopt_attn_ctx_forward(const void* q, const void* k_ctx, const void* v_ctx, const void* k_act,
                             const void* v_act, void* o, float* lse, const somaopt_attn_ctx_shape* shape,
                             void* stream);

/* Backward from the saved O and LSE: writes dQ, and dK, dV of the action
 * keys; `delta` is a caller-provided fp32 [batch][heads][lq] workspace. */
int somaopt_attn_ctx_backward(const void* q, const void* k_ctx, const void* v_ctx, const void* k_act,
                              const void* v_act, const void* o, const float* lse, const void* d_o, float* dq,
                              float* dk_act, float* dv_act, float* delta, const somaopt_attn_ctx_shape* shape,
                              void* stream);

/* Release the handle's device tables, graph and private stream.  NULL is
 * ignored.  The caller must first let every call it made with the handle
 * complete (synchronize the streams it passed, or wait on an event recorded
 * after its last call): the handle does not track the caller's streams and
 * destroy issues no stream or device wait of its own.  It frees device
 * memory with hipFree, however, and the HIP runtime makes hipFree wait until
 * all work on the device has finished, so destroy returns only once the
 * device is idle, streams the handle never used included (on MI355X a 1 MiB
 * hipFree returned only after an 83 ms kernel on an unrelated stream). */
void somaopt_destroy(somaopt_handle* h);

/* Message for the last failed call on this thread ("" if none). */
const char* somaopt_last_error(void);

/* Library version string. */
const char* somaopt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SOMAOPT_H */

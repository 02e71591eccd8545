/*
 * pararnn.h — C ABI of libpararnn.so: the ParaRNN / DEER parallel-in-time
 * Newton solve of ParaGRU and ParaLSTM, and its adjoint, on MI355X (gfx950).
 *
 * The method ("Параллельность RNN?", forpes.ru, section 1; voguetech.ru
 * ParaRNN article, "Что именно сделали технически"):
 *   - the T hidden states s_1..s_T of a sequence are the unknowns of the
 *     residual r_t = s_t - f(s_{t-1}, x_t) = 0, whose unique zero is the
 *     ordinary sequential trajectory (§1.1);
 *   - Newton's method solves it: J(s) ds = -r(s), s <- s + ds (§1.2);
 *   - J is block-bidiagonal (identity blocks, -df/ds(s_{t-1}) below), so
 *     each Newton system is the linear recurrence
 *     ds_t = A_t ds_{t-1} - r_t, A_t = df/ds(s_{t-1}) (§1.3, level 1),
 *     which is associative and is solved by a parallel scan of affine maps
 *     (§1.3, level 2);
 *   - for ParaGRU the local Jacobian A_t is diagonal, for ParaLSTM 2x2
 *     block diagonal per channel (ParaRNN article, item 3), so every
 *     channel (b, d) is an independent 1- or 2-dimensional problem.
 * The per-step transition is compiled into the kernels (the fully fused
 * tier of the ParaRNN article, "Три уровня производительности", item 3):
 *   ParaGRU  z = sig(a_z h + u_z), r = sig(a_r h + u_r),
 *            c = tanh(a_c (r h) + u_c),  h' = (1 - z) h + z c
 *   ParaLSTM i, f, o = sig(a_* h + u_*), g = tanh(a_g h + u_g),
 *            c' = f c + i g,  h' = o tanh(c')
 * u_* are the precomputed input projections W x_t + b (one plane per gate),
 * a_* the diagonal recurrent weights.
 *
 * Conventions for every entry point
 *   - Memory: every array pointer is a DEVICE pointer (HBM), owned by the
 *     caller; the library never allocates, frees or synchronises.  All work
 *     is enqueued on `stream` (a hipStream_t, NULL = default stream) and the
 *     call returns before it completes.  Outputs must not alias inputs.
 *     A call enqueues kernel launches only (per-launch state is cleared by
 *     a kernel, not by a memset), so it can be captured into a HIP graph;
 *     a captured call keeps its workspace, and two replays that overlap in
 *     time must not share one.
 *   - Layout: per-time-step planes are indexed (b, d, t); element offset of
 *     (b, d, t) = b*stride_b + d*stride_d + t*stride_t.  Planes of `u` (and
 *     of `du`) use u_stride_*; state, gradient and lambda planes use
 *     s_stride_*.  The fast layout is channel-major [B][D][T] (stride_t = 1):
 *     a lane's steps are contiguous and load as 16-byte vectors.  Any other
 *     layout whose elements do not overlap is accepted, e.g. time-major
 *     [B][T][D] (stride_t = D, stride_d = 1, as a [B][T][G*D] projection
 *     gives per gate with stride_t = G*D).  The solves, the adjoint and the
 *     scan stage such planes channel-major in the workspace when it is at
 *     least pararnn_workspace_bytes(...) / pararnn_scan_workspace_bytes(...)
 *     (which count that room), run there and copy the results back; with a
 *     smaller workspace (the channel-major size), and always in the
 *     sequential call, each step is gathered with its own 4-byte load
 *     instead.  Results are bitwise the same either way.
 *     pararnn_project writes channel-major planes directly.  Initial states are dense [B][D]; diagonal
 *     weights are dense [G][D] float32 in gate order (GRU: z, r, c;
 *     LSTM: i, f, g, o).  LSTM state order is (c, h).
 *   - Errors: arguments are checked on the host before any HIP call; a bad
 *     argument returns PARARNN_ERR_INVALID / _UNSUPPORTED / _WORKSPACE and
 *     enqueues nothing.  A HIP launch error returns PARARNN_ERR_HIP.
 *     Non-convergence is not an error: it is reported in pararnn_info_t.
 *   - Determinism: results are bitwise reproducible run to run (no
 *     floating-point atomics; reductions run in a fixed order).
 */
#ifndef PARARNN_H
#define PARARNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PARARNN_OK = 0,
    PARARNN_ERR_INVALID = 1,     /* null pointer, size < 0, bad stride      */
    PARARNN_ERR_UNSUPPORTED = 2, /* valid request this build does not serve */
    PARARNN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than needed   */
    PARARNN_ERR_HIP = 4,         /* the HIP runtime reported a launch error */
    PARARNN_ERR_SCRATCH = 5      /* needs more than the static scratch      */
} pararnn_status_t;

typedef enum { PARARNN_F32 = 0, PARARNN_BF16 = 1 } pararnn_dtype_t;
typedef enum { PARARNN_GRU = 0, PARARNN_LSTM = 1 } pararnn_cell_t;

typedef struct {
    int64_t B, T, D;                 /* batch rows, time steps, channels     */
    int64_t u_stride_b, u_stride_d;  /* elements, every u / du plane         */
    int64_t s_stride_b, s_stride_d;  /* elements, every state/grad plane     */
    int64_t u_stride_t, s_stride_t;  /* elements between steps (1: [B][D][T]) */
} pararnn_shape_t;

typedef struct {
    /* A channel (or, for long sequences, a time block of it) stops once the
     * largest |r_t| over its steps and state components is < tol and every
     * earlier time block of the channel has stopped; NaN never counts as
     * converged.  At most max_iters Newton updates are applied; the final
     * residual is always evaluated. */
    float tol;
    int32_t max_iters;        /* >= 0                                          */
    int32_t steps_per_lane;   /* K: 0 = automatic, else 1, 2, 4, 8, 16, or 32
                                 (ParaGRU forward solve with W = 1 or 2 only)  */
    int32_t waves_per_block;  /* W: 0 = automatic, else 1, 2, 4 or 8; one
                                 workgroup covers 64 * K * W time steps       */
    int32_t init_from_output; /* 1: Newton starts from the values already in
                                 the output planes; 0: from s = 0             */
} pararnn_newton_t;

/* Written on the device by the solve (pass a device pointer, or NULL): each
 * work unit stores its own final max|r| and update count in the workspace,
 * and a one-workgroup pass after the solve folds them into this record. */
typedef struct {
    int32_t iters;        /* max Newton updates applied, over channels       */
    int32_t converged;    /* 1 iff every channel stopped with max|r| < tol    */
    float max_abs_res;    /* max over channels of the final max|r_t|          */
    int32_t nan_seen;     /* 1 if any final residual was NaN                  */
    int64_t iters_sum;    /* sum over work units of updates applied           */
    int64_t units;        /* work units = channels x time blocks              */
} pararnn_info_t;

/* Bytes of device workspace pararnn_solve_* / pararnn_adjoint need for this
 * problem and tiling (0 is possible).  Returns 0 on a bad argument too; the
 * solve itself reports the error.  For the adjoint pass adjoint = 1.
 * For a solve the figure counts the time-block hand-off (several blocks per
 * channel that run side by side, i.e. fewer than 1024 channels; with more, a
 * channel's blocks are solved one after the other inside one workgroup and
 * need none), 8 bytes per work unit for the convergence records an info
 * record is folded from, and the staging room of planes that are not
 * time-contiguous; a solve without an info record, on time-contiguous
 * planes with one block per channel, runs with no workspace at all. */
size_t pararnn_workspace_bytes(pararnn_cell_t cell, const pararnn_shape_t *shape,
                               const pararnn_newton_t *opt, int adjoint);

/*
 * ParaGRU forward solve.
 *   u[3]   : gate planes (z, r, c), [B][D][T], dtype u_dtype (F32 or BF16)
 *   a      : [3][D] float32 diagonal recurrent weights
 *   h0     : [B][D] float32 initial state s_0 (given, not solved for)
 *   h      : [B][D][T] float32 output, the converged states s_1..s_T
 *            (also the Newton start if opt->init_from_output)
 *   info   : device pararnn_info_t or NULL
 *   ws     : device workspace of ws_bytes >= pararnn_workspace_bytes(...)
 * Residual, Jacobian, scan and convergence test run in one kernel; the
 * states stay on chip across Newton iterations.
 */
pararnn_status_t pararnn_solve_gru(const pararnn_shape_t *shape, const void *const u[3],
                                   pararnn_dtype_t u_dtype, const float *a,
                                   const float *h0, float *h,
                                   const pararnn_newton_t *opt, pararnn_info_t *info,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * ParaLSTM forward solve.  u[4] gate planes (i, f, g, o); a [4][D];
 * c0, h0 [B][D]; outputs c, h [B][D][T].  Jacobians are 2x2 per channel.
 */
pararnn_status_t pararnn_solve_lstm(const pararnn_shape_t *shape, const void *const u[4],
                                    pararnn_dtype_t u_dtype, const float *a,
                                    const float *c0, const float *h0, float *c, float *h,
                                    const pararnn_newton_t *opt, pararnn_info_t *info,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * Adjoint (backward pass) of a converged solve, for the loss
 * L = sum_t <dL/ds_t, s_t>.  The adjoint lam_t = dL/ds_t (total) solves the
 * transposed block-bidiagonal system of §1.3, i.e. the reverse-time linear
 * recurrence lam_t = g_t + A_{t+1}^T lam_{t+1}, lam_{T+1} = 0, with
 * A_{t+1} = df/ds at (s_t, u_{t+1}); it is computed by a reverse parallel
 * scan, then the gate gradients follow elementwise.
 *   cell   : PARARNN_GRU (S = 1 state, G = 3 gates) or PARARNN_LSTM (2, 4)
 *   u      : G gate planes as for the solve (dtype u_dtype)
 *   a      : [G][D]
 *   s0     : S pointers to [B][D] initial states (LSTM order c, h)
 *   s      : S pointers to [B][D][T] converged states s_1..s_T
 *   gs     : S pointers to [B][D][T] upstream gradients dL/ds_t; an entry
 *            may be NULL, meaning zero (e.g. dL/dc_t for an LSTM)
 *   gs_end : NULL, or S pointers to [B][D] (an entry may be NULL = zero):
 *            a gradient added to dL/ds_T at the last step — what a
 *            continuation of the sequence sends back, i.e. the ds0 of the
 *            adjoint of the next time chunk (A_{T+1}^T lam_{T+1} of the
 *            uncut recurrence), so a sequence cut into chunks is
 *            differentiated chunk by chunk, last chunk first
 *   du     : G pointers to [B][D][T] float32 outputs dL/du (u_stride_*)
 *   da     : [G][D] float32 output dL/da (summed over batch and time)
 *   da_accumulate : 0: da = the sum; 1: da += the sum (chunk by chunk)
 *   ds0    : S pointers to [B][D] float32 outputs dL/ds_0
 *   lam    : NULL, or S pointers to [B][D][T] float32 outputs lam_t
 *   opt    : only steps_per_lane / waves_per_block are read (may be NULL)
 *   ws     : workspace (per-block da partials and carries)
 */
pararnn_status_t pararnn_adjoint(pararnn_cell_t cell, const pararnn_shape_t *shape,
                                 const void *const *u, pararnn_dtype_t u_dtype,
                                 const float *a, const float *const *s0,
                                 const float *const *s, const float *const *gs,
                                 const float *const *gs_end, float *const *du, float *da,
                                 int32_t da_accumulate, float *const *ds0,
                                 float *const *lam, const pararnn_newton_t *opt,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * The linear recurrence of a Newton iteration on its own, for callers that
 * assemble (A_t, b_t) themselves: "Параллельность RNN?" (forpes.ru), §1.3,
 * level 1 (forward substitution) solved as in level 2 (associative scan of
 * affine maps); the "parallel reduction" tier of the voguetech.ru ParaRNN
 * article ("Три уровня производительности", item 2).  Per channel (b, d):
 *   reverse = 0:  x_t = A_t x_{t-1} + b_t,  t = 1..T,  x_0 given
 *   reverse = 1:  x_t = A_t x_{t+1} + b_t,  t = T..1,  x_{T+1} given
 *   state_size : 1 (A_t scalar) or 2 (A_t a 2x2 block)
 *   A          : state_size^2 planes [B][D][T] float32 (u_stride_*), 2x2 blocks
 *                row-major (a00, a01, a10, a11)
 *   b          : state_size planes [B][D][T] float32 (u_stride_*)
 *   x0         : NULL (boundary value zero) or state_size pointers to [B][D]
 *   x          : state_size planes [B][D][T] float32 out (s_stride_*)
 *   opt        : only steps_per_lane / waves_per_block are read (may be NULL)
 *   ws         : pararnn_scan_workspace_bytes(...) bytes (0 is possible)
 * Same conventions as above: device pointers, caller's stream, no
 * allocation, argument checks before any HIP call.
 */
size_t pararnn_scan_workspace_bytes(int32_t state_size, const pararnn_shape_t *shape,
                                    const pararnn_newton_t *opt);
pararnn_status_t pararnn_scan(int32_t state_size, const pararnn_shape_t *shape,
                              const float *const *A, const float *const *b,
                              const float *const *x0, float *const *x, int32_t reverse,
                              const pararnn_newton_t *opt, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Step-by-step application of the recurrence, one lane per channel:
 * s_t = f(s_{t-1}, u_t) for t = 1..T from the given s_0 — the sequential
 * evaluation whose result the Newton solve reaches ("Параллельность RNN?",
 * forpes.ru, §1.1: the trajectory is the unique zero of the residual) and
 * the baseline of the pages' parallel-vs-sequential speed-up (voguetech.ru
 * ParaRNN article, "Что именно сделали технически").  Its time is T times
 * one step's dependency-chain latency, nearly independent of the number of
 * channels until they fill the device, so for many channels and moderate T
 * it can beat the Newton solve; for few channels and long T it cannot.
 *   cell, shape, u, u_dtype, a : as for pararnn_solve_gru / _lstm
 *   s0 : S pointers to [B][D] initial states (LSTM order c, h)
 *   s  : S pointers to [B][D][T] float32 outputs (s_stride_*)
 * Same conventions: device pointers, caller's stream, no allocation, no
 * workspace, arguments checked before any HIP call.
 */
pararnn_status_t pararnn_sequential(pararnn_cell_t cell, const pararnn_shape_t *shape,
                                    const void *const *u, pararnn_dtype_t u_dtype,
                                    const float *a, const float *const *s0, float *const *s,
                                    void *stream);

/*
 * Input projection: u = W x + b for every time step, the dense product that
 * precedes the recurrence (the cells take u_t = W x_t + b as precomputed
 * projections: voguetech.ru ParaRNN article, "Что именно сделали
 * технически", item 3).  Per batch row b:
 *     u[b][m][t] = sum_k W[m][k] x[b][t][k] + bias[m],  m < M, t < T, k < I
 * Written channel-major with time contiguous, so for M = G*D the rows of
 * gate g form that gate's [B][D][T] plane for the solves (plane g starts at
 * u + g*D*u_stride_m; u_stride_b, u_stride_m are its strides).
 *   x    : bfloat16, x[b][t][k] at b*x_stride_b + t*x_stride_t + k
 *   w    : bfloat16, W[m][k] at m*w_stride_m + k
 *   bias : float32 [M], or NULL (no bias)
 *   u    : u_dtype (PARARNN_F32, or PARARNN_BF16 rounded to nearest even),
 *          u[b][m][t] at b*u_stride_b + m*u_stride_m + t
 * Products of bf16 values are exact in fp32 and accumulate in fp32 on the
 * matrix cores.  Device pointers, caller's stream, no allocation; arguments
 * checked before any HIP call (sizes >= 0, strides large enough that rows
 * do not overlap).
 */
typedef struct {
    int64_t B, T, I, M;
    int64_t x_stride_b, x_stride_t;
    int64_t w_stride_m;
    int64_t u_stride_b, u_stride_m;
} pararnn_proj_shape_t;

pararnn_status_t pararnn_project(const pararnn_proj_shape_t *shape, const void *x,
                                 const void *w, const float *bias, void *u,
                                 pararnn_dtype_t u_dtype, void *stream);

/*
 * pararnn_solve_gru without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results and errors are those
 * of pararnn_solve_gru; the workspace (time-block hand-off, convergence
 * records of the info record, staging of planes that are not
 * time-contiguous when it fits) comes from an array inside the library of
 * PARARNN_STATIC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  A problem that needs more returns
 * PARARNN_ERR_SCRATCH before any HIP call (planes that are not
 * time-contiguous and do not fit are read step by step instead of staged).
 * The call allocates nothing and frees nothing; the first call on a device
 * looks up the array's device address (the caller's stream must belong to
 * the current device, else PARARNN_ERR_INVALID).  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (the solve clears
 * what must start at zero with a kernel): calls whose executions overlap on
 * one GPU (different streams, concurrent graph replays) race and must be
 * serialised by the caller.
 */
#define PARARNN_STATIC_SCRATCH_BYTES (32u << 20)
pararnn_status_t pararnn_solve_gru_noalloc(const pararnn_shape_t *shape, const void *const u[3],
                                           pararnn_dtype_t u_dtype, const float *a,
                                           const float *h0, float *h,
                                           const pararnn_newton_t *opt, pararnn_info_t *info,
                                           void *stream);

/* Static description of a status code. */
const char *pararnn_status_string(pararnn_status_t status);

/* Tiling the library would use for this problem: K steps per lane, W waves
 * per workgroup, and time blocks per channel (1 = whole channel in one
 * workgroup).  Returns PARARNN_OK or the same error a solve would return. */
pararnn_status_t pararnn_plan(pararnn_cell_t cell, const pararnn_shape_t *shape,
                              const pararnn_newton_t *opt, int adjoint,
                              int32_t *steps_per_lane, int32_t *waves_per_block,
                              int64_t *time_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PARARNN_H */

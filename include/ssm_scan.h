/*
 * ssm_scan.h -- C ABI of libssmscan.so, the MI355X (gfx950) selective state-space scan.
 *
 * The operation (per batch b, channel d, state n, step t) is the selective SSM
 * recurrence that the pages describe:
 *   dt      = softplus(delta[b,d,t] + delta_bias[d])   -- step size from the input,
 *             bias inside the softplus ("Mamba: 基于选择状态空间的线性时间序列模型",
 *             freeguideonline.com, section 4.2 step 2; fsdata.site
 *             "mamba-state-space-model" article, section 3.2)
 *   A_bar   = exp(dt * A[d,n])                          -- fsdata.site article, section 3.2
 *   B_bar   = dt * B[b,n,t]                             -- same section (default)
 *           = (exp(dt*A) - 1) / A * B[b,n,t]            -- exact zero-order hold, with
 *             SSM_FLAG_ZOH (freeguideonline tutorial, section 2.2)
 *   h[n]    = A_bar * h[n] + B_bar * u[b,d,t]
 *   y       = sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]   -- output read from the updated
 *             state plus the skip term ("Mamba: Linear-Time Sequence Modeling with
 *             Selective State Spaces", ai.xwebgame.com, section on what an SSM is)
 *   out     = y * silu(z[b,d,t])                        -- gate by the second branch
 *             (same page, the PyTorch block's gating step)
 * Each channel d is an independent SSM with its own diagonal A[d,:]
 * (freeguideonline tutorial, section 4.3); B and C are shared by all channels of
 * a batch row.  The scan computes the sequential recurrence exactly up to
 * floating-point rounding order (freeguideonline tutorial, section 5.1).  The
 * state is fp32; streams are fp32 or bf16 (rounded to nearest even on output).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller (the library
 *     allocates nothing and keeps no pointer after returning).  Tensors are
 *     dense, row-major, with the layouts given below, and every base pointer
 *     must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Outputs are valid once the stream has been synchronised.
 *   - Every argument is checked on the host before anything is enqueued; on any
 *     error nothing is launched and no output is touched.  The return code is
 *     the only error channel.
 *   - `out` and `final_state` must not overlap any input (checked: SSM_ERR_OVERLAP).
 *   - Calls are reentrant; concurrent calls on different streams are safe when
 *     their output buffers are distinct.
 *   - Indexing is 64-bit: a tensor may hold more than 2^31 elements.
 *   - Arithmetic is fp32: a result whose exact magnitude is below about 1e-36
 *     (near or under fp32's smallest normal number) may come back as 0.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*` */

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,       /* a size is out of range (batch/dim/seqlen < 1, dstate not in [1,64],
                              conv width not in [1,4]) */
  SSM_ERR_DTYPE = 3,       /* io_dtype is not SSM_F32 or SSM_BF16 */
  SSM_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned */
  SSM_ERR_UNSUPPORTED = 5, /* unknown flag bits */
  SSM_ERR_WORKSPACE = 6,   /* workspace non-NULL but smaller than ssm_scan_workspace_size() */
  SSM_ERR_LAUNCH = 7,      /* the HIP runtime rejected a launch (hipGetLastError) */
  SSM_ERR_OVERLAP = 8,     /* an output buffer overlaps an input buffer */
  SSM_ERR_TOO_LARGE = 9    /* ssm_scan_fwd_noalloc: the shape needs more than its 34 MiB of scratch */
} ssm_status;

typedef enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* flag bits for ssm_shape.flags / ssm_state_update(flags) */
#define SSM_FLAG_ZOH 1u     /* exact zero-order-hold B_bar instead of dt*B */
#define SSM_FLAG_REVERSE 2u /* scan from t = L-1 down to 0 (a backward-in-time SSM;
                               fsdata.site article, section 7 pitfalls table) */

typedef struct ssm_shape {
  int64_t batch;   /* B >= 1 */
  int64_t dim;     /* D (d_inner) >= 1 */
  int64_t dstate;  /* N in [1, 64] */
  int64_t seqlen;  /* L >= 1 */
  int32_t io_dtype;/* ssm_dtype of u, delta, B, C, z and out */
  uint32_t flags;  /* SSM_FLAG_* bits */
} ssm_shape;

/* Version of this header's ABI (bumped on any incompatible change). */
#define SSM_ABI_VERSION 2
int ssm_abi_version(void);

/* Static string for a status code (never NULL). */
const char* ssm_status_str(int status);

/* Bytes of device workspace that ssm_scan_fwd may use for this shape to split
 * long sequences across workgroups (0 when no split is used).  Depends on the
 * shape only.  Returns 0 for an invalid shape. */
size_t ssm_scan_workspace_size(const ssm_shape* shape);

/* Selective scan over a whole sequence (prefill / training forward).
 *   u, delta, z, out : [B, D, L]  io_dtype
 *   A                : [D, N]     fp32 (the pages use negative reals)
 *   B, C             : [B, N, L]  io_dtype, shared by all D channels of a batch row
 *   D, delta_bias    : [D]        fp32, NULL means zero
 *   z                : NULL means no gate (out = y)
 *   initial_state    : [B, D, N]  fp32 state before the first processed step,
 *                      NULL means zero (lets a long sequence be scanned in
 *                      several calls; mlqm.cn article, section 6.2)
 *   final_state      : [B, D, N]  fp32 state after the last processed step,
 *                      NULL means not written
 *   workspace        : device scratch of workspace_bytes; NULL with 0 bytes runs
 *                      without splitting the sequence (always correct, slower when
 *                      batch*dim is small).  Non-NULL but smaller than
 *                      ssm_scan_workspace_size() is SSM_ERR_WORKSPACE.  The
 *                      library does not keep it; its contents are not preserved.
 * With SSM_FLAG_REVERSE the steps run from L-1 to 0; final_state is then the
 * state after step 0. */
ssm_status ssm_scan_fwd(const ssm_shape* shape,
                        const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D,
                        const void* z, const float* delta_bias,
                        const float* initial_state,
                        void* out, float* final_state,
                        void* workspace, size_t workspace_bytes,
                        struct ihipStream_t* stream);

/* ssm_scan_fwd that also saves what ssm_scan_bwd_saved needs, so a training step does
 * not recompute it:
 *   checkpoints      : [B, ceil(L/64), D, N] fp32, written: the state entering every
 *                      64-step block (block k starts at step 64 k in scan order).
 *                      Required; must not overlap any other argument.
 * Every other argument, the outputs and the errors are those of ssm_scan_fwd. */
ssm_status ssm_scan_fwd_save(const ssm_shape* shape,
                             const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D,
                             const void* z, const float* delta_bias,
                             const float* initial_state,
                             void* out, float* final_state, float* checkpoints,
                             void* workspace, size_t workspace_bytes,
                             struct ihipStream_t* stream);

/* ssm_scan_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): it takes no workspace
 * and allocates nothing.  A sequence split uses a scratch array of 34 MiB that the
 * library holds in static device memory, one copy per GPU, kept until the process
 * ends (it holds the split of 1 x 1024 x 16 x 2^20, bf16, which needs 33.996 MiB);
 * its address is looked up once per device, on the first call there.
 *   - Arguments, outputs and errors are those of ssm_scan_fwd, with the split always
 *     enabled; a shape whose split needs more than 34 MiB (ssm_scan_workspace_size()
 *     > 34 MiB) is refused with SSM_ERR_TOO_LARGE before anything is enqueued.
 *   - `stream` must belong to the device whose scratch is used (its own device).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last call's
 *     contents: calls that overlap in time on one GPU (on different streams, or
 *     from different host threads without ordering) race on it and give undefined
 *     results.  Serialise them, e.g. on one stream.
 * Results are bitwise those of ssm_scan_fwd with a workspace. */
ssm_status ssm_scan_fwd_noalloc(const ssm_shape* shape,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D,
                                const void* z, const float* delta_bias,
                                const float* initial_state,
                                void* out, float* final_state,
                                struct ihipStream_t* stream);

/* One recurrent generation step (the scan body with L = 1), state updated in place:
 * the fixed-size state replaces a growing cache (fsdata.site article, section 3.2
 * and the comparison table in section 5).
 *   state            : [B, D, N]  fp32, read and written
 *   u, delta, z, out : [B, D]     io_dtype
 *   A                : [D, N]     fp32
 *   B, C             : [B, N]     io_dtype
 *   D, delta_bias    : [D]        fp32, NULL means zero; z NULL means no gate
 * flags: SSM_FLAG_ZOH only. */
ssm_status ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int32_t io_dtype,
                            uint32_t flags, float* state,
                            const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias,
                            void* out, struct ihipStream_t* stream);

/* Bytes of device workspace ssm_scan_bwd needs for this shape (0 for an invalid
 * shape): block checkpoints of the state, B*D*ceil(L/64)*N fp32; per-workgroup
 * partial sums of dB and dC, 2*ceil(D/16)*B*N*L fp32; and the per-(segment,
 * batch row) partial sums of dA, dD and ddelta_bias.  When the shape has few
 * channels and a long sequence (fewer than 384 blocks of 16 channels over the batch
 * and L >= 2048) the sequence is split into S segments, as in the forward: then
 * also the carried states of the checkpoints and, per segment, the summary and the
 * carried value of the adjoint (O(S*B*D*N) fp32).  The choice depends on the shape
 * only. */
size_t ssm_scan_bwd_workspace_size(const ssm_shape* shape);

/* Gradients of ssm_scan_fwd (training backward pass).  The pages describe only the
 * forward recurrence; these are its exact derivatives by the chain rule (the
 * reverse-time adjoint recurrence), computed from the forward inputs alone: the
 * forward states are recomputed from checkpoints, nothing from the forward call
 * is needed.
 *   Inputs: the forward's inputs (same layouts, same NULL rules) plus
 *   dout             : [B, D, L] io_dtype, gradient of out
 *   dfinal_state     : [B, D, N] fp32 gradient of final_state, NULL means zero
 *   Outputs (all fully written):
 *   du, ddelta       : [B, D, L] io_dtype
 *   dA               : [D, N]    fp32, summed over batch rows and steps
 *   dB, dC           : [B, N, L] fp32, summed over channels
 *   dD, ddelta_bias  : [D]       fp32, NULL means not computed (written even when
 *                      D / delta_bias is NULL: the gradient at zero)
 *   dz               : [B, D, L] io_dtype, required when z is given, else ignored
 *   dinitial_state   : [B, D, N] fp32 gradient of initial_state, NULL means not written
 *   workspace        : required, at least ssm_scan_bwd_workspace_size() bytes
 * shape->flags may hold SSM_FLAG_REVERSE and SSM_FLAG_ZOH, as in the forward call
 * (under ZOH the derivatives of B_bar = (exp(dt A) - 1) / A * B with respect to dt, A,
 * B and u are taken, with the A -> 0 limit where A is zero).  No output may overlap an
 * input, another output or the workspace.  Every sum is taken in a fixed order, so
 * results are bitwise reproducible. */
ssm_status ssm_scan_bwd(const ssm_shape* shape,
                        const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D,
                        const void* z, const float* delta_bias,
                        const float* initial_state,
                        const void* dout, const float* dfinal_state,
                        void* du, void* ddelta, float* dA, float* dB, float* dC,
                        float* dD, void* dz, float* ddelta_bias, float* dinitial_state,
                        void* workspace, size_t workspace_bytes,
                        struct ihipStream_t* stream);

/* Bytes of device workspace ssm_scan_bwd_saved needs for this shape (0 for an invalid
 * shape): that of ssm_scan_bwd without the checkpoints and their split. */
size_t ssm_scan_bwd_saved_workspace_size(const ssm_shape* shape);

/* ssm_scan_bwd from the checkpoints that ssm_scan_fwd_save wrote for the same inputs
 * (same shape, flags, initial_state, A, B, delta, delta_bias and u), instead of a
 * checkpoint pass of its own:
 *   checkpoints      : [B, ceil(L/64), D, N] fp32, read only.  Required; must not
 *                      overlap an output or the workspace.
 *   workspace        : required, at least ssm_scan_bwd_saved_workspace_size() bytes
 * Every other argument, the outputs and the errors are those of ssm_scan_bwd. */
ssm_status ssm_scan_bwd_saved(const ssm_shape* shape,
                              const void* u, const void* delta, const float* A,
                              const void* B, const void* C, const float* D,
                              const void* z, const float* delta_bias,
                              const float* initial_state,
                              const void* dout, const float* dfinal_state,
                              const float* checkpoints,
                              void* du, void* ddelta, float* dA, float* dB, float* dC,
                              float* dD, void* dz, float* ddelta_bias, float* dinitial_state,
                              void* workspace, size_t workspace_bytes,
                              struct ihipStream_t* stream);

/* The step that produces u: causal depthwise conv1d over time, plus a bias, then
 * SiLU (ai.xwebgame.com Mamba page, the PyTorch block's step 2: a Conv1d with one
 * group per channel and width-1 padding whose output is cut to the sequence
 * length, followed by SiLU):
 *   u[b,d,t] = silu(bias[d] + sum_{k<width} weight[d,k] * x[b,d,t-(width-1)+k])
 * Inputs before step 0 are taken from initial_conv_state, else zero.
 *   x, u               : [B, D, L]        io_dtype
 *   weight             : [D, width]       fp32 (the page's Conv1d weight [D,1,width])
 *   bias               : [D]              fp32, NULL means zero
 *   initial_conv_state : [B, D, width-1]  io_dtype, the width-1 inputs before x,
 *                        oldest first; NULL means zeros
 *   final_conv_state   : [B, D, width-1]  io_dtype, the last width-1 inputs of the
 *                        sequence initial_conv_state followed by x (what the next
 *                        call or ssm_conv1d_update continues from); NULL means not
 *                        written.  Must not overlap any input (use two buffers when
 *                        processing a sequence in pieces).
 * width must be in [1, 4] (the pages use 4); with width 1 the state pointers are
 * ignored.  Other conventions as above (device pointers, 16-byte aligned bases,
 * host-side checks, asynchronous on `stream`, u must not overlap any input). */
ssm_status ssm_conv1d_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width,
                          int32_t io_dtype, const void* x, const float* weight,
                          const float* bias, const void* initial_conv_state, void* u,
                          void* final_conv_state, struct ihipStream_t* stream);

/* One generation step of the same convolution: u = silu(bias + weight . (state, x)),
 * then the state drops its oldest input and appends x (updated in place).
 *   conv_state : [B, D, width-1] io_dtype, read and written (NULL allowed if width == 1)
 *   x, u       : [B, D]          io_dtype
 *   weight     : [D, width] fp32; bias : [D] fp32 or NULL */
ssm_status ssm_conv1d_update(int64_t batch, int64_t dim, int64_t width, int32_t io_dtype,
                             void* conv_state, const void* x, const float* weight,
                             const float* bias, void* u, struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */

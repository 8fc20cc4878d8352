/*
 * ss.h -- Mamba selective scan (S6) on AMD MI355X (gfx950): the C ABI.
 *
 * The library (libss.so) runs the selective scan of Mamba-1 as hand-written
 * HIP kernels.  All tensor arguments are DEVICE pointers allocated by the
 * caller; the library allocates nothing, and its only global state is a
 * per-device cache of the compute-unit count (read once from the runtime, to
 * size the backward's launch to the resident workgroup slots).  Every
 * call validates its arguments on the host first and returns an error code
 * without touching the GPU when they are invalid; otherwise it enqueues its
 * kernels on `stream` (a hipStream_t, NULL = the null stream) and returns
 * without synchronising.  A failed launch returns SS_ERR_HIP.  Beside the
 * scan (forward, decode step, backward) it exports the depthwise causal
 * conv1d + SiLU that feeds the scan, and the Mamba-2 SSD chunked scan on the
 * matrix cores, each declared below with its own layouts.
 *
 * Problem (page "Mamba", Part IV Stage 5, the selective_scan_fn interface):
 *   per batch row b, channel d (d < dim = d_inner) and state n (n < dstate):
 *     Delta_t  = softplus(delta[b,d,t] + bias[d])   (softplus only if flagged;
 *                                                     the bias is always added)
 *     Abar_t   = exp(Delta_t * A[d,n])               (Stage 4, zero-order hold)
 *     h_t[n]   = Abar_t h_{t-1}[n] + Delta_t B[b,n,t] u[b,d,t]   (Euler for B)
 *     y0_t     = sum_n C[b,n,t] h_t[n] + D[d] u[b,d,t]           (Stage 6 skip)
 *     y[b,d,t] = y0_t * z_t * sigmoid(z_t)   (gate, Stage 6; y0_t if z absent)
 *   with h_{-1} = 0 (or a given initial state h0).  "mamba-metal" README
 *   ("Long-context prompts") adds the final state h_{L-1}, from which decode
 *   continues one token at a time.  With packed documents ("niverel-mamba"
 *   README, "seq_idx strict reset") the state is zero before every step t >= 1
 *   whose document id seq_idx[b,t] differs from seq_idx[b,t-1].
 *
 * Layouts of the scan (the SSD below keeps Mamba-2's time-major ones): every
 * tensor is C-contiguous with the time axis innermost:
 *   u, delta, z, y, dy, du, ddelta, dz : (batch, dim, seqlen)   io dtype
 *   Bm, Cm, dB, dC                     : (batch, dstate, seqlen) io dtype (dB, dC: fp32)
 *   A, dA                              : (dim, dstate)  fp32
 *   D, bias, dD, dbias                 : (dim)          fp32
 *   last_state, state_in, state_out,
 *   h0, dh0, dlast                     : (batch, dim, dstate) fp32
 *   seq_idx                            : (batch, seqlen) int32
 *   ckpt                               : (batch, dim, ceil(seqlen/64), dstate) fp32
 * Data tensors may be fp32, fp16 or bf16 (`io_dtype`); the weights A, D,
 * bias and every state are fp32, and all arithmetic is fp32 ("mamba-metal"
 * README: data in half, weights in float, fp32 scan accumulation).  Outputs
 * in fp16/bf16 are rounded to nearest-even.
 *
 * Limits: 1 <= dstate <= 16; batch, dim >= 1; batch * dim <= 2^26 - 8 (one
 * workgroup per 16 channels, twice over, within 2^23 workgroups);
 * 1 <= seqlen <= 2^24; every pointer 16-byte aligned (SS_ERR_MISALIGNED
 * otherwise).  Any finite A is accepted; A > 0
 * makes the state grow and may overflow.
 */
#ifndef SS_H
#define SS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ss_status {
    SS_OK = 0,
    SS_ERR_NULL_ARG = 1,     /* a required pointer is NULL, or an optional pair is half given */
    SS_ERR_BAD_SHAPE = 2,    /* a size is < 1 or overflows (also: a launch grid beyond
                                2^23 workgroups, so that every dispatch stays within
                                2^32 work-items) */
    SS_ERR_BAD_DTYPE = 3,    /* io_dtype is not one of ss_dtype */
    SS_ERR_MISALIGNED = 4,   /* a pointer is not 16-byte aligned */
    SS_ERR_UNSUPPORTED = 5,  /* a size outside the supported set, a workspace missing or
                                smaller than required, or overlapping buffers */
    SS_ERR_HIP = 6           /* the HIP runtime reported an error at launch */
} ss_status;

typedef enum ss_dtype { SS_F32 = 0, SS_F16 = 1, SS_BF16 = 2 } ss_dtype;

typedef struct ss_problem {
    int64_t batch;           /* B */
    int64_t dim;             /* D = d_inner, channels */
    int64_t dstate;          /* N, 1..16 */
    int64_t seqlen;          /* L */
    int32_t io_dtype;        /* ss_dtype of the data tensors */
    int32_t delta_softplus;  /* nonzero: Delta = softplus(delta + bias) */
} ss_problem;

/*
 * Bytes of device workspace ss_fwd runs fastest with for this problem.  A
 * problem with too few channels to fill the GPU splits time, and its
 * workspace holds a control block and per-chunk partial states of the
 * time-parallel scan: for a time chunk c of a channel, the decay product over
 * the chunk and the state reached from zero (the associative pair of the page
 * "Mamba", Part V "S6 ... forbids the convolution"), and the same pair for
 * groups of consecutive chunks.  Any other problem (batch <= 256) can
 * use a work queue, which ss_fwd takes for ragged rows (`lengths` given) and
 * for more 16-channel row blocks than the GPU holds at once when they do not
 * fill it evenly: units of 2048 steps of a 16-channel block, handed out
 * longest row first, each continuing from the state its block reached at the
 * end of the previous unit; its workspace holds a control block, a flag per
 * unit and that state per (channel, unit).  Returns 0 for an invalid problem.
 */
size_t ss_fwd_workspace_size(const ss_problem *p);

/*
 * The least workspace ss_fwd accepts for this problem: the time-chunked
 * scan's (0 when time is not split).  Between this and
 * ss_fwd_workspace_size() bytes (or with no workspace at all when this is 0)
 * ss_fwd runs without the work queue: the same results, a slower schedule for
 * ragged or uneven problems.  Returns 0 for an invalid problem.
 */
size_t ss_fwd_workspace_min(const ss_problem *p);

/*
 * Forward scan (the op of page "Mamba", Part IV Stage 5, with the final
 * state of the "mamba-metal" README).  Writes y for every t < seqlen.
 *   D, z, delta_bias  : optional (NULL = no skip / no gate / zero bias).
 *   lengths           : optional device int32[batch]; row b runs
 *                       min(max(lengths[b], 0), seqlen) steps from its
 *                       initial state, y is exactly 0 past that length and
 *                       last_state is the state after that many steps.
 *                       Out-of-range values are clamped, not reported.
 *   seq_idx           : optional device int32 (batch, seqlen) document ids
 *                       ("niverel-mamba" README, "seq_idx strict reset"):
 *                       the state is reset to zero before every step whose
 *                       id differs from the previous step's, so a packed row
 *                       gives the same y as its documents run one by one.
 *                       Any int32 values; only changes matter.
 *   h0                : optional (batch, dim, dstate) fp32 initial state
 *                       (NULL = zero): prefill in pieces, each piece started
 *                       from the previous piece's last_state, equals one
 *                       prefill of the whole sequence.  It feeds only the
 *                       row's first document.
 *   last_state        : optional (batch, dim, dstate) fp32 output.
 *   ckpt              : optional (batch, dim, ceil(seqlen/64), dstate) fp32
 *                       output: entry k is the state after min(64k, len)
 *                       steps (entry 0 is h0, or zero), the checkpoints of page
 *                       "Mamba, on a laptop GPU", "The state lives in
 *                       registers", used by ss_bwd.
 *   workspace         : device buffer of ss_fwd_workspace_size() bytes (at
 *                       least ss_fwd_workspace_min(); NULL when that is 0;
 *                       SS_ERR_UNSUPPORTED when it is smaller).  Its contents
 *                       on entry do not matter.  Time-chunked problems, and
 *                       ragged problems that use the work queue, record in
 *                       its second 32-bit word a nonzero value if a wait
 *                       between workgroups ever gave up (it never should:
 *                       the wait is bounded only so that every kernel ends).
 * y may be u, delta or z itself (in place); any other overlap between an
 * output (y, last_state, ckpt, workspace) and another buffer returns
 * SS_ERR_UNSUPPORTED.
 */
ss_status ss_fwd(const ss_problem *p,
                 const void *u, const void *delta, const float *A,
                 const void *Bm, const void *Cm,
                 const float *D, const void *z, const float *delta_bias,
                 const int32_t *lengths, const int32_t *seq_idx, const float *h0,
                 void *y, float *last_state, float *ckpt,
                 void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * ss_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, results and errors as ss_fwd, without the workspace: the
 * time-chunked scan keeps its chunk pairs (and a ragged problem its work
 * queue, when that fits) in a fixed array of
 * ss_fwd_noalloc_max_workspace() bytes (2 MiB) of device memory that the
 * library holds on every GPU it runs on until the process ends.  No call
 * allocates or frees memory.  The array is shared by every call on one GPU
 * and keeps the last call's contents (nothing in it needs clearing): calls
 * that overlap in time on one GPU, e.g. on two streams, race on it and must
 * be ordered by the caller.  `stream` must belong to the current device.
 * Returns SS_ERR_UNSUPPORTED for a problem whose least workspace
 * (ss_fwd_workspace_min) would exceed the array (no valid problem's does: the
 * scan splits time only for problems with fewer than 1024 wavefronts, which
 * bounds that workspace at 1.05 MB), and
 * SS_ERR_HIP when the array's device address cannot be obtained.
 */
ss_status ss_fwd_noalloc(const ss_problem *p,
                         const void *u, const void *delta, const float *A,
                         const void *Bm, const void *Cm,
                         const float *D, const void *z, const float *delta_bias,
                         const int32_t *lengths, const int32_t *seq_idx, const float *h0,
                         void *y, float *last_state, float *ckpt,
                         void *stream);

/* Bytes of the fixed device array ss_fwd_noalloc uses as its workspace. */
size_t ss_fwd_noalloc_max_workspace(void);

/*
 * One decode step from a carried state ("mamba-metal" README, "O(1) per
 * token via state caching"; page "Mamba", Part IV Stage 7, single-step
 * decoding updates the cached state in place).  p->seqlen is ignored.
 *   u_t, delta_t, z_t, y_t : (batch, dim) io dtype;  B_t, C_t : (batch, dstate) io dtype
 *   state_in, state_out    : (batch, dim, dstate) fp32; they may be the same
 *                            buffer (in-place update); partial overlap is not allowed.
 * D, z_t and delta_bias are optional as in ss_fwd.
 */
ss_status ss_fwd_step(const ss_problem *p,
                      const void *u_t, const void *delta_t, const float *A,
                      const void *B_t, const void *C_t,
                      const float *D, const void *z_t, const float *delta_bias,
                      const float *state_in, float *state_out, void *y_t,
                      void *stream);

/*
 * Bytes of device workspace ss_bwd needs: per 64-step chunk of every channel
 * and state, the chunk's decay product, its state-gradient from a zero
 * carry and the carried gradient (3 * batch*dim*ceil(seqlen/64)*16 floats).
 * Returns 0 for an invalid problem.
 */
size_t ss_bwd_workspace_size(const ss_problem *p);

/*
 * Backward scan for the loss sum(dy * y) + sum(dlast * last_state) (page
 * "Mamba", Part IV Stage 7: the states are recomputed, here from the 64-step
 * checkpoints that ss_fwd wrote, walking the chunks in reverse as page
 * "Mamba, on a laptop GPU", "The state lives in registers", describes).
 *   ckpt         : the checkpoints ss_fwd wrote for the same inputs (the same
 *                  seq_idx and h0; no lengths).
 *   seq_idx      : optional document ids, as in ss_fwd.
 *   dlast        : optional (batch, dim, dstate) fp32 gradient of the loss
 *                  w.r.t. the final state (NULL = zero).
 *   dh0          : optional (batch, dim, dstate) fp32 output, the gradient
 *                  w.r.t. the initial state.
 *   du, ddelta   : (batch, dim, seqlen) io dtype outputs.
 *   dz           : output iff z is given.  dD iff D.  dbias iff delta_bias.
 *   dA (dim, dstate), dB, dC (batch, dstate, seqlen), dD, dbias (dim): fp32,
 *   summed over the dimensions their inputs are shared across (dB, dC over
 *   channels; dA, dD, dbias over batch rows and time).  Every output is
 *   overwritten; the library clears its accumulation targets itself.
 *   workspace    : device buffer of ss_bwd_workspace_size() bytes.
 * Returns SS_ERR_NULL_ARG when a gradient output and its input are not given
 * together, SS_ERR_UNSUPPORTED when the workspace is missing or too small or
 * when an output or the workspace overlaps any other buffer (no in-place).
 */
ss_status ss_bwd(const ss_problem *p,
                 const void *u, const void *delta, const float *A,
                 const void *Bm, const void *Cm,
                 const float *D, const void *z, const float *delta_bias,
                 const int32_t *seq_idx, const float *ckpt, const void *dy, const float *dlast,
                 void *du, void *ddelta, void *dz,
                 float *dA, float *dB, float *dC, float *dD, float *dbias, float *dh0,
                 void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * ---- the step before the scan: depthwise causal conv1d + SiLU -------------
 * Page "Mamba" (walkthrough), Part IV Stage 2: every channel d has its own
 * filter of width W (d_conv, 4 by default); the input is padded on the left
 * only, so output t sees inputs t-W+1 .. t; a SiLU follows:
 *   out[b,d,t] = silu(bias[d] + sum_{k<W} w[d,k] * x[b,d,t-W+1+k])
 * (w[d,W-1] multiplies the current input; the layout of a (dim, 1, W)
 * depthwise weight with the middle axis dropped).  All arithmetic is fp32.
 */
typedef struct ss_conv_problem {
    int64_t batch;      /* B */
    int64_t dim;        /* D = d_inner */
    int64_t seqlen;     /* L (ignored by ss_conv1d_step) */
    int32_t width;      /* W = d_conv, 1..4 */
    int32_t io_dtype;   /* ss_dtype of x and out */
    int32_t silu;       /* nonzero: out = SiLU(pre); zero: out = pre */
    int32_t reserved;   /* must be 0 */
} ss_conv_problem;

/*
 * Forward convolution over whole rows.
 *   x, out     : (batch, dim, seqlen) io dtype; out must not overlap x.
 *   w          : (dim, W) fp32.  bias: (dim) fp32 or NULL.
 *   seq_idx    : optional (batch, seqlen) int32 document ids ("niverel-mamba"
 *                README, "seq_idx strict reset": the convolution resets with
 *                the scan): an input of another document than step t's
 *                counts as 0.
 *   conv_init  : optional (batch, dim, W-1) fp32, the W-1 inputs before t = 0
 *                (oldest first; NULL = zeros), e.g. the conv_final of the
 *                previous piece of the row.  It reaches only the first document.
 *   conv_final : optional (batch, dim, W-1) fp32 output, the last W-1 inputs of
 *                each row (0 where they belong to an earlier document, or
 *                precede the row without conv_init): the window that
 *                ss_conv1d_step continues from ("mamba-metal" README: the
 *                conv1d sliding window is carried across calls).
 * Errors as ss_fwd; SS_ERR_UNSUPPORTED when W is outside 1..4 or when out or
 * conv_final overlaps another buffer.
 */
ss_status ss_conv1d_fwd(const ss_conv_problem *p, const void *x, const float *w, const float *bias,
                        const int32_t *seq_idx, const float *conv_init, void *out, float *conv_final,
                        void *stream);

/*
 * One decode step of the convolution: out_t = silu(bias + w . [window, x_t]),
 * then the window drops its oldest input and appends x_t.
 *   x_t, out_t             : (batch, dim) io dtype.
 *   window_in, window_out  : (batch, dim, W-1) fp32; they may be the same buffer
 *                            (in-place); partial overlap is not allowed.
 */
ss_status ss_conv1d_step(const ss_conv_problem *p, const void *x_t, const float *w, const float *bias,
                         const float *window_in, float *window_out, void *out_t, void *stream);

/*
 * ---- Mamba-2 SSD chunked scan ----------------------------------------------
 * Page "Mamba" (walkthrough), "Deep dive: Mamba-2 and state-space duality":
 * A is a scalar per head and a group of heads shares B and C.  Per batch row
 * b and head h (state H[p][n], headdim x dstate, g = h / (nheads/ngroups)):
 *   Delta_t  = softplus(dt[b,t,h] + dt_bias[h])     (softplus only if flagged)
 *   H_t      = exp(Delta_t A[h]) H_{t-1} + Delta_t x[b,t,h,:] B[b,t,g,:]^T
 *   y[b,t,h,p] = sum_n H_t[p][n] C[b,t,g,n] + D[h] x[b,t,h,p]   (* SiLU(z) if z)
 * from H_{-1} = h0 (or 0).  With packed documents ("niverel-mamba" README,
 * "seq_idx strict reset": for Mamba-2 the SSM state resets at a document
 * boundary) H is zero before every step t >= 1 whose id seq_idx[b,t] differs
 * from seq_idx[b,t-1], so h0 feeds only a row's first document.  Computed by
 * the chunked algorithm the page describes (quadratic, attention-like
 * matmuls inside 256-step chunks, one state passed between chunks) on the
 * matrix cores, fp32 accumulation.
 * Layouts (time-major, as Mamba-2 stores them):
 *   x, z, y : (batch, seqlen, nheads, headdim)  io dtype
 *   dt      : (batch, seqlen, nheads)           io dtype
 *   Bm, Cm  : (batch, seqlen, ngroups, dstate)  io dtype
 *   A, D, dt_bias : (nheads) fp32
 *   seq_idx : (batch, seqlen) int32 (any values; only changes matter)
 *   h0, final_state : (batch, nheads, headdim, dstate) fp32
 */
typedef struct ss_ssd_problem {
    int64_t batch;
    int64_t seqlen;
    int64_t nheads;
    int64_t ngroups;      /* divides nheads */
    int32_t headdim;      /* 64 */
    int32_t dstate;       /* 32, 64, 96 or 128 */
    int32_t io_dtype;     /* SS_F16 or SS_BF16 */
    int32_t dt_softplus;  /* nonzero: Delta = softplus(dt + dt_bias) */
} ss_ssd_problem;

/* Bytes of device workspace ss_ssd_fwd needs: per 256-step chunk of every
 * (batch row, head), the state entering the chunk (headdim x dstate, io
 * dtype); per chunk of every (batch row, group), C B^T (256 x 256, fp32 sums
 * stored as bf16).  The
 * caller owns it; its contents on entry do not matter.  Returns 0 for an
 * invalid problem. */
size_t ss_ssd_workspace_size(const ss_ssd_problem *p);

/*
 * SSD forward.  D, z, dt_bias, seq_idx, h0 and final_state are optional (NULL).
 * Every pointer must be 16-byte aligned.  y may be x or z itself (in place)
 * and final_state may be h0 itself; any other overlap between an output or
 * the workspace and another buffer is rejected.  Returns SS_ERR_BAD_DTYPE for
 * fp32 I/O (the matrix-core path takes 16-bit data), SS_ERR_UNSUPPORTED for a
 * headdim other than 64, a dstate outside {32, 64, 96, 128}, ngroups not
 * dividing nheads, more than 32768 heads, document ids on a row longer than
 * 2^29 steps, a workspace missing or too small, or overlapping buffers.
 */
ss_status ss_ssd_fwd(const ss_ssd_problem *p, const void *x, const void *dt, const float *A,
                     const void *Bm, const void *Cm, const float *D, const void *z, const float *dt_bias,
                     const int32_t *seq_idx, const float *h0, void *y, float *final_state,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Number of floats of the checkpoint buffer: batch*dim*ceil(seqlen/64)*dstate (0 if invalid). */
size_t ss_ckpt_count(const ss_problem *p);

/* Static, human-readable text for a status code. */
const char *ss_status_str(ss_status s);

/*
 * Measurement utility, not part of the scan: copies `bytes` (a nonzero
 * multiple of 16) from src to dst on the device with a plain streaming
 * kernel.  Used to measure achievable HBM bandwidth and to calibrate
 * hardware traffic counters against a kernel of known traffic.
 */
ss_status ss_copy_probe(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Measurement utility, not part of the scan: the issue rate of the vector
 * instructions the scan is made of, so that its ALU ceiling is measured on
 * the chip rather than taken from a datasheet.  Launches `workgroups`
 * workgroups of 256 threads (4 waves), each with `lds_bytes` of LDS it does
 * not use (0..65536: it limits how many workgroups share a CU, as a kernel's
 * own LDS does); every wave runs `iters` iterations of 16 instructions of
 * `kind` (SS_PROBE_SCAN_STEP: 16 steps of the scan's per-lane state update,
 * each two DPP-broadcast multiplies, one exp2 and one FMA) between two reads
 * of the shader clock (s_memtime) and of the constant 100 MHz clock
 * (s_memrealtime), and writes to `out`, a device int64 array of 6 entries per
 * wave: [clock0, clock1, real0, real1, place, 0], where place holds the
 * hardware wave-id register (bits 0..31: SIMD, CU, shader engine) and the XCD
 * (bits 32..63), so that the host can count the waves each SIMD held.
 * SS_ERR_BAD_SHAPE unless 1 <= workgroups <= 2^20, 1 <= iters <= 2^20 and
 * 0 <= lds_bytes <= 65536; SS_ERR_UNSUPPORTED for an unknown kind.
 */
typedef enum ss_probe_kind {
    SS_PROBE_FMA = 0,        /* v_fma_f32, 16 independent chains */
    SS_PROBE_EXP = 1,        /* v_exp_f32, 16 independent chains */
    SS_PROBE_DPP_MUL = 2,    /* v_mul_f32 with a DPP row broadcast, 16 chains */
    SS_PROBE_SCAN_STEP = 3   /* the scan's per-lane step (4 instructions) */
} ss_probe_kind;

ss_status ss_alu_probe(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes, int64_t *out,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_H */

/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * The operation is the selective state-space scan of Mamba as the page
 * "scan output is different between sequential and parallel versions"
 * (alxndrTL/mamba.py issue 26) states its API in the test script's API
 * comment: x and delta of shape (Bs, L, ED), A (ED, N), B and C (Bs, L, N),
 * D (ED) and the output y (Bs, L, ED), computed by selective_scan /
 * selective_scan_seq. For every batch row b, channel e and state n:
 *
 *   a_t[n]   = exp(delta[b,t,e] * A[e,n])
 *   h_t[n]   = a_t[n] * h_{t-1}[n] + (delta[b,t,e] * x[b,t,e]) * B[b,t,n],   h_{-1} = 0
 *   y[b,t,e] = sum_n C[b,t,n] * h_t[n] + D[e] * x[b,t,e]
 *
 * delta is used as given (no softplus, bias or clamp). The initial state is
 * zero unless an h0 is passed: then h_{-1} = h0, which resumes a sequence
 * from a carried state (pass the h_last of the previous piece).
 *
 * The bidirectional variant follows "Some questions of Bi-Mamba2 and Hydra"
 * (Hprairie/Bi-Mamba2 issue 1), the author's first reply: the sum of two SSMs
 * with shared weights (A, B, C, delta), one over increasing and one over
 * decreasing time, plus D x once, with the inputs read in place (no flipped
 * copy) and no shift:
 *
 *   g_t[n]   = a_t[n] * g_{t+1}[n] + (delta x)[b,t,e] * B[b,t,n],   g_L = 0 (or g0)
 *   y[b,t,e] = sum_n C[b,t,n] * (h_t[n] + g_t[n]) + D[e] * x[b,t,e]
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers (memory from hipMalloc or any allocator on
 *    the device the stream belongs to). The caller owns every buffer,
 *    including the workspace. The library allocates nothing, keeps no pointer
 *    after returning and holds no global state, so calls are reentrant; two
 *    calls that run at the same time need separate workspaces.
 *  - Layout: dense row-major in the shapes above (last index fastest), no
 *    strides. h_last and g_first are (Bs, ED, N) float32.
 *  - dtype (ssm_dtype) applies to x, delta, B, C and y. A, D, h_last and
 *    g_first are float32 always. Internal state and accumulation are float32;
 *    bfloat16 outputs are rounded to nearest even.
 *  - Alignment: every pointer must be aligned to 16 bytes.
 *  - Asynchrony: each call validates its arguments on the host before any
 *    HIP call, enqueues its kernels on `stream` (a hipStream_t; NULL means
 *    the null stream) and returns. Faults inside a kernel surface at the
 *    caller's next synchronisation on that stream.
 *  - Numerics: inputs whose state overflows float32 (a > 1, i.e. delta*A > 0
 *    over long spans) propagate inf/NaN; no error code is returned for them.
 *  - Empty inputs: the batch size, the sequence length and the channel count
 *    (Bs, L, ED; Bs and L of the multi-head scan) may be zero, and a buffer
 *    with no elements may then be NULL. Nothing is scanned; over zero time
 *    steps each state stays where it entered, so h_last = h0 and g_first =
 *    g0 (zero without them), and every gradient of the backward pass is zero
 *    (dA, dD; dB and dC when there are time steps but no channels) except
 *    dh0 = dh_last and dg0 = dg_first. No workspace is needed.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_F32 = 0,  /* float32 x, delta, B, C, y */
  SSM_BF16 = 1  /* bfloat16 x, delta, B, C, y (bit patterns, uint16) */
} ssm_dtype;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL */
  SSM_ERR_DIM = 2,         /* a dimension is negative (or zero where it must be positive: N, and H,
                              P, G of the multi-head scan) or the sizes overflow int64 */
  SSM_ERR_UNSUPPORTED = 3, /* N not supported, unknown dtype, or a pointer not 16-byte aligned */
  SSM_ERR_ALIAS = 4,       /* an output overlaps an input, another output or the workspace */
  SSM_ERR_WORKSPACE = 5,   /* workspace smaller than ssm_scan_workspace_bytes() */
  SSM_ERR_LAUNCH = 6,      /* the HIP runtime rejected a launch */
  SSM_ERR_ARG = 7,         /* an option is invalid (dt_min > dt_max, or a NaN bound) */
  SSM_ERR_HANDOFF = 8      /* ssm_scan_fwd_status only: a split-sequence hand-off wait gave up */
} ssm_status;

/*
 * Optional step-size pre-processing and output gate, the options of the
 * Bi-Mamba2 forward ("Some questions of Bi-Mamba2 and Hydra", the
 * MambaChunkScanCombinedFn.forward listing: dt_bias, dt_softplus, dt_limit,
 * z), with their usual meaning:
 *   delta' = clamp(softplus?(delta + dt_bias[e]), dt_min, dt_max)
 *            softplus(v) = v for v > 20, else log(1 + exp(v))
 *   y'     = y * z * sigmoid(z)      (after D x; both directions for bidir)
 * delta' replaces delta everywhere in the recurrence. A NULL options pointer
 * means none of them (raw delta, no clamp, no gate).
 */
typedef struct {
  const float* dt_bias; /* (ED) float32 added to delta, or NULL */
  int dt_softplus;      /* nonzero: apply softplus after the bias */
  float dt_min;         /* clamp bounds applied last; -INFINITY / +INFINITY: none */
  float dt_max;
  const void* z;        /* (Bs, L, ED) of dtype, or NULL: no gate */
} ssm_scan_options;

/* Supported state sizes N. */
#define SSM_MAX_N 16

/*
 * Bytes of device workspace that ssm_scan_fwd (bidir = 0) or
 * ssm_scan_bidir_fwd (bidir = 1) needs for these sizes on the current
 * device (the forward scan splits long sequences over more workgroups when
 * the device has many compute units per channel group, and then needs room
 * to pass states between them; the bidirectional bf16 scan keeps float32
 * partial sums). Zero means the call may pass workspace = NULL. The
 * workspace needs no initialisation and holds nothing of interest after the
 * call. Returns 0 for invalid sizes too (the call itself then reports the
 * error).
 */
size_t ssm_scan_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int bidir);

/*
 * Forward selective scan (the recurrence above).
 * Long sequences with little channel parallelism are split into chunks that
 * run concurrently and hand their end states on through the workspace; each
 * chunk takes its place in the sequence from an atomic ticket, so a chunk's
 * predecessor has always started (no assumption on which workgroups are
 * resident, and other work may share the device). A hand-off wait is
 * bounded (about seven seconds); if it ever gives up, the chunk's outputs,
 * every later chunk's and h_last become NaN, and ssm_scan_fwd_status()
 * reports SSM_ERR_HANDOFF. A later chunk adds the decayed entering state's
 * contribution to the start of its outputs until every decay product
 * prod a[n] is below 2^-30 (or the entering state is zero); the terms left
 * out are below 2^-30 sum_n |C_t[n] h_in[n]|, under one float32 rounding.
 *   x, delta : (Bs, L, ED) of dtype        -- input sequence and step sizes
 *   A        : (ED, N) float32             -- state matrix (diagonal per channel)
 *   B, C     : (Bs, L, N) of dtype         -- input and output projections
 *   D        : (ED) float32, or NULL (treated as zero)
 *   h0       : (Bs, ED, N) float32, or NULL -- initial state h_{-1} (zero if NULL)
 *   opts     : pre-processing and gate (see ssm_scan_options), or NULL
 *   y        : (Bs, L, ED) of dtype        -- output, written in full
 *   h_last   : (Bs, ED, N) float32, or NULL -- state after the last step
 * Returns SSM_OK once the kernels are enqueued, else the first error found.
 */
int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const float* h0, const ssm_scan_options* opts, void* y, float* h_last, int64_t Bs, int64_t L, int64_t ED,
                 int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Round checkpoints: the scan state entering every 32-step round, for a
 * backward pass that then skips its own forward sweep. Like the forward of
 * the Bi-Mamba2 autograd function in "Some questions of Bi-Mamba2 and Hydra"
 * (the MambaChunkScanCombinedFn listing), which returns the per-chunk states
 * and keeps the forward's products for the backward to read.
 * ssm_scan_ckpt_bytes: bytes of the checkpoint buffer for these sizes,
 * (Bs, ceil(L / 32), 16 ceil(ED / 16), 16) float32 (channels padded to a
 * multiple of 16; N must be 16, else 0), 0 for invalid sizes.
 * ssm_scan_fwd_ckpt: ssm_scan_fwd (same arguments, results and errors) that
 * also writes ckpt[b][r][e][n] = h_{32 r - 1}[b, e, n], the state after the
 * first 32 r steps, for rounds r >= 1 (entries of round 0 are not written;
 * padded channels get their zero state). A split sequence's checkpoints
 * take the entering state's carried contribution with the same 2^-30 cut
 * as its outputs. ckpt: device buffer of at least ckpt_bytes >=
 * ssm_scan_ckpt_bytes(...) bytes, aligned to 16 bytes, overlapping no other
 * argument (SSM_ERR_NULL if NULL with data to scan, SSM_ERR_WORKSPACE if
 * too small, SSM_ERR_ALIAS if it overlaps).
 */
size_t ssm_scan_ckpt_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N);
int ssm_scan_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const float* h0, const ssm_scan_options* opts, void* y, float* h_last,
                      float* ckpt, size_t ckpt_bytes, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward selective scan that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Arguments, results
 * and errors as ssm_scan_fwd. The split-sequence hand-off buffer is the
 * library's own device array of SSM_NOALLOC_SCRATCH_BYTES per device (held
 * until the process ends; its address is resolved on the first call on each
 * device, with that device current); sizes whose split plan would need more
 * (ssm_scan_workspace_bytes(..., bidir = 0) larger than that, which no
 * device of up to 340 compute units reaches) return SSM_ERR_WORKSPACE. The
 * function calls no allocator. Every call on one device shares that array:
 * calls that overlap in time on one device (two streams, two threads) race
 * and give wrong results; calls in order on one stream are safe.
 */
#define SSM_NOALLOC_SCRATCH_BYTES (1u << 20)
int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const float* h0, const ssm_scan_options* opts, void* y, float* h_last,
                         int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* stream);

/*
 * Outcome of the split-sequence hand-off of the last ssm_scan_fwd call made
 * with this workspace and these sizes (workspace NULL: the last
 * ssm_scan_fwd_noalloc call on the current device): synchronises `stream`,
 * then returns SSM_ERR_HANDOFF if a wait gave up (that call's affected
 * outputs are NaN), SSM_OK otherwise (also when these sizes do not split the
 * sequence, or the input is empty). Size errors as ssm_scan_fwd;
 * SSM_ERR_WORKSPACE if the workspace is too small for a split call.
 */
int ssm_scan_fwd_status(const void* workspace, size_t workspace_bytes, int64_t Bs, int64_t L, int64_t ED,
                        int64_t N, int dtype, void* stream);

/*
 * Bidirectional selective scan (forward plus reverse-time scan plus D x).
 * Arguments as ssm_scan_fwd (h0 initialises the forward direction), and
 *   g0      : (Bs, ED, N) float32 or NULL -- reverse state entering at
 *             t = L-1, i.e. g_L = g0 (zero if NULL). The Bi-Mamba2 forward
 *             returns a final state per direction ("Some questions of
 *             Bi-Mamba2 and Hydra", final_states_f and final_states_b in the
 *             MambaChunkScanCombinedFn.forward listing); a sequence cut in
 *             pieces resumes the forward direction of a piece from the
 *             previous piece's h_last and the reverse direction from the
 *             next piece's g_first.
 *   h_last  : (Bs, ED, N) float32 or NULL -- forward state after t = L-1
 *   g_first : (Bs, ED, N) float32 or NULL -- reverse state after t = 0
 * Long sequences with little channel parallelism are split into chunks here
 * too: every chunk runs both directions from its own entering states (zero
 * inside the sequence), and a second kernel folds the chunks' aggregates
 * into the states entering each chunk from either side, then corrects both
 * ends of its output the way ssm_scan_fwd corrects a chunk's start (terms
 * below 2^-30 of the carried state are left out). Nothing waits on another
 * workgroup; the workspace (ssm_scan_workspace_bytes(..., bidir = 1)) holds
 * the aggregates, after the bf16 scan's float32 partials.
 */
int ssm_scan_bidir_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
                       float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_bidir_fwd (same arguments, results and errors) that also writes
 * the forward direction's round checkpoints, exactly as ssm_scan_fwd_ckpt
 * does for the same inputs: ckpt[b][r][e][n] = h_{32 r - 1}[b, e, n] of the
 * forward scan from h0, for rounds r >= 1 (the reverse direction's states
 * are not kept). Same ckpt sizes, alignment and errors as ssm_scan_fwd_ckpt;
 * for ssm_scan_bidir_bwd_ckpt.
 */
int ssm_scan_bidir_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
                            float* h_last, float* g_first, float* ckpt, size_t ckpt_bytes, int64_t Bs, int64_t L,
                            int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the forward scan: the gradients of L = sum(dy * y) for
 * y = ssm_scan_fwd(x, delta, A, B, C, D, h0, opts = NULL). This is the step
 * that follows the forward in the autograd function of "Some questions of
 * Bi-Mamba2 and Hydra" (the backward listing, which returns dx, ddt, dA, dB,
 * dC and dD from dout); the pages give no formula, so the gradients are the
 * adjoint of the recurrence above. With g_t[n] = dL/dh_t[n] (reverse time,
 * g_{L-1} = dy_{L-1} C_{L-1}):
 *   g_t      = dy_t C_t + a_{t+1} g_{t+1}
 *   dx_t     = delta_t sum_n g_t B_t + D dy_t
 *   ddelta_t = x_t sum_n g_t B_t + sum_n A[e,n] g_t a_t h_{t-1}
 *   dB_t[n]  = sum_e g_t delta_t x_t,      dC_t[n] = sum_e dy_t h_t
 *   dA[e,n]  = sum_{b,t} delta_t g_t a_t h_{t-1},   dD[e] = sum_{b,t} dy_t x_t
 *   dh0      = a_0 g_0
 * dh_last (the gradient of the final state h_last, the dfinal_states
 * argument of that page's backward listing) enters the adjoint at the last
 * step, g_{L-1} = dy_{L-1} C_{L-1} + dh_last: the loss is then
 * sum(dy * y) + sum(dh_last * h_last), so that a sequence cut in pieces
 * (h0 / h_last) is trained piece by piece, the later piece's dh0 being the
 * earlier piece's dh_last.
 * The bidirectional scan has ssm_scan_bidir_bwd below.
 * Step-size options (opts: dt_bias, dt_softplus, dt_min, dt_max, as given
 * to the forward): the recurrence above runs with delta' = clamp(softplus?(
 * delta + dt_bias), dt_min, dt_max) in place of delta, ddelta is the
 * gradient of the raw delta, ddelta' d delta'/d delta, where the derivative
 * is sigmoid(delta + dt_bias) (1 without softplus) and 0 where the clamp
 * holds delta' at a bound (taken as 0 at the bound itself), and ddt_bias[e]
 * is the sum of ddelta over rows and time. With the output gate (opts->z
 * set), y = y' z sigmoid(z) for the ungated output y': dz = dy y' silu'(z)
 * is written to dz, and the other gradients are those of y' for the output
 * gradient dy z sigmoid(z). The call recomputes y' with the forward scan
 * (into dz), forms both with an elementwise kernel, then runs the backward.
 *   x, delta, A, B, C, D, h0 : as ssm_scan_fwd (D and h0 may be NULL)
 *   opts    : step-size options of the forward, or NULL
 *   dy      : (Bs, L, ED) of dtype         -- dL/dy
 *   dh_last : (Bs, ED, N) float32, or NULL -- dL/dh_last (zero if NULL)
 *   dx, ddelta : (Bs, L, ED) of dtype      -- written in full
 *   dA      : (ED, N) float32              -- written in full
 *   dB, dC  : (Bs, L, N) of dtype          -- written in full
 *   dD      : (ED) float32, or NULL (not computed)
 *   dh0     : (Bs, ED, N) float32, or NULL (not computed)
 *   ddt_bias : (ED) float32, or NULL (not computed; with no option it is
 *              the sum of ddelta over rows and time)
 *   dz      : (Bs, L, ED) of dtype -- the gate's gradient, required with
 *             opts->z, ignored (may be NULL) without it
 *   workspace : at least ssm_scan_bwd_workspace_bytes(..., gate) bytes,
 *     gate = 1 when opts->z is set (required; it holds the state at every
 *     32-step boundary and float32 partial sums of dB, dC, dA and dD; with
 *     the gate also dy z sigmoid(z), one float32 value per element of x),
 *     no initialisation needed.
 * Sums over channels (dB, dC) and over batch rows and time (dA, dD) are
 * taken in a fixed order, so repeated calls give identical bits.
 * Conventions, alignment and error codes as ssm_scan_fwd.
 */
size_t ssm_scan_bwd_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int gate);

int ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const float* h0, const ssm_scan_options* opts, const void* dy, const float* dh_last, void* dx,
                 void* ddelta, float* dA, void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, void* dz,
                 int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * ssm_scan_bwd given the round checkpoints that ssm_scan_fwd_ckpt wrote for
 * the same inputs (x, delta, A, B, C, h0 and the step-size options): the
 * backward then skips its own forward sweep over the sequence. ckpt (read
 * only; at least ckpt_bytes >= ssm_scan_ckpt_bytes(...) bytes, aligned to 16
 * bytes, overlapping no output or the workspace) is required: NULL with
 * data to scan is SSM_ERR_NULL. Other arguments, results, workspace and
 * errors as ssm_scan_bwd; checkpoints of other inputs give wrong gradients
 * (no error).
 */
int ssm_scan_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const float* h0, const ssm_scan_options* opts, const void* dy,
                      const float* dh_last, const float* ckpt, size_t ckpt_bytes, void* dx, void* ddelta, float* dA,
                      void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, void* dz, int64_t Bs, int64_t L,
                      int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the bidirectional scan: the gradients of L = sum(dy * y)
 * (plus sum(dh_last * h_last) + sum(dg_first * g_first)) for y =
 * ssm_scan_bidir_fwd(x, delta, A, B, C, D, h0, g0, opts), the sum of the
 * forward scan (with D x and h0) and the reverse-time scan (from g0, shared
 * weights) of "Some questions of Bi-Mamba2 and Hydra" (the
 * author's first reply). Its gradient is the sum of the two scans' gradients:
 * the reverse scan's adjoint runs in increasing time, g'_t = dy_t C_t +
 * a_{t-1} g'_{t-1}, with the terms of ssm_scan_bwd at the same (b, t, e); D
 * and h0 enter the forward scan only. The inputs are read in place (no
 * flipped copy): two passes of the backward kernels, the second mapping
 * every step t to time L-1-t and adding its dx and ddelta to the first's
 * (kept in float32 in the workspace for bfloat16 outputs, so that they are
 * rounded once); dB, dC and dA sum both passes' partials in a fixed order.
 * The reverse scan starts from g0 (the forward's reverse initial state; zero
 * if NULL), its adjoint enters from dg_first (the gradient of g_first; zero
 * if NULL), and the gradient of g0 is written to dg0 (if not NULL); h0,
 * dh_last and dh0 belong to the forward-time scan as in ssm_scan_bwd.
 * Arguments, outputs and conventions as ssm_scan_bwd; the workspace is
 * ssm_scan_bidir_bwd_workspace_bytes(..., gate) bytes (both passes' partial
 * sums and, for bfloat16, two float32 values per element of x; with the gate
 * also dy z sigmoid(z)).
 */
size_t ssm_scan_bidir_bwd_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int gate);

int ssm_scan_bidir_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, const void* dy,
                       const float* dh_last, const float* dg_first, void* dx, void* ddelta, float* dA, void* dB,
                       void* dC, float* dD, float* dh0, float* dg0, float* ddt_bias, void* dz, int64_t Bs, int64_t L,
                       int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_bidir_bwd given the forward direction's round checkpoints that
 * ssm_scan_bidir_fwd_ckpt (or ssm_scan_fwd_ckpt) wrote for the same x,
 * delta, A, B, C, h0 and options: the forward-time half of the backward then
 * skips its own forward sweep; the reverse-time half keeps it. ckpt (read
 * only) is required (NULL with data to scan: SSM_ERR_NULL); sizes,
 * alignment and overlap rules as ssm_scan_bwd_ckpt; other arguments,
 * results, workspace and errors as ssm_scan_bidir_bwd. Checkpoints of other
 * inputs give wrong gradients (no error).
 */
int ssm_scan_bidir_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const float* h0, const float* g0, const ssm_scan_options* opts,
                            const void* dy, const float* dh_last, const float* dg_first, const float* ckpt,
                            size_t ckpt_bytes, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                            float* dh0, float* dg0, float* ddt_bias, void* dz, int64_t Bs, int64_t L, int64_t ED,
                            int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-head (Mamba-2 / SSD) selective scan, in the layout of the chunked
 * scan of "Some questions of Bi-Mamba2 and Hydra" (the
 * MambaChunkScanCombinedFn listings: x (batch, seqlen, nheads, headdim), dt
 * (batch, seqlen, nheads), one A per head, B and C per group of heads). For
 * batch row b, head h (group g = h / (H / G)), head channel p and state n:
 *
 *   a_t       = exp(dt[b,t,h] A[h])
 *   S_t[p][n] = a_t S_{t-1}[p][n] + (dt[b,t,h] x[b,t,h,p]) B[b,t,g,n],   S_{-1} = h0 (or 0)
 *   y[b,t,h,p] = sum_n C[b,t,g,n] S_t[p][n] + D[h] x[b,t,h,p]
 *
 * (the recurrence of ssm_scan_fwd with one decay per head and a shared B, C
 * per group).
 *   x      : (Bs, L, H, P) of dtype      dt : (Bs, L, H) of dtype
 *   A      : (H) float32                 B, C : (Bs, L, G, N) of dtype
 *   D      : (H) float32, or NULL        h0 : (Bs, H, P, N) float32, or NULL
 *   opts   : the options of ssm_scan_options, per head: dt_bias is (H)
 *            float32 (dt' = clamp(softplus?(dt + dt_bias[h]), dt_min,
 *            dt_max) replaces dt) and the gate z is (Bs, L, H, P) of dtype
 *            (y' = y z sigmoid(z), after D x); NULL: dt as given, no gate
 *            (the chunked-scan forward listing of that page passes dt_bias,
 *            dt_softplus, dt_limit and z to this scan)
 *   y      : (Bs, L, H, P) of dtype, written in full
 *   h_last : (Bs, H, P, N) float32, or NULL -- S after the last step
 * Supported: P = 64, N = 64 or 128, H a multiple of G. The state and every
 * accumulation are float32. With float32 inputs the chunk products take
 * float32 operands; with bfloat16 inputs they run on the bf16 matrix
 * instructions, with x, B and C as given and each float32 operand (the
 * decayed C B^T, the state, the decay-weighted B) split into a high and a
 * low bf16 part, so every product is within 2^-17 of its float32 value; y is
 * rounded to nearest even.
 *   workspace : device memory of ssm_ssd_workspace_bytes(...) bytes, owned by
 *               the caller; NULL when that is zero. With fewer (batch row,
 *               head) pairs than compute units each sequence is cut into
 *               ranges of whole 32-step chunks: a first pass forms every
 *               range's end state from zero, the second runs every range
 *               from the state folded in from the ranges before it; the
 *               workspace holds those states (it needs no initialisation,
 *               may not overlap an argument, and holds nothing of interest
 *               after the call). SSM_ERR_WORKSPACE if it is needed and
 *               missing or too small.
 * Conventions, alignment and error codes as ssm_scan_fwd (SSM_ERR_DIM also
 * when H is not a multiple of G).
 */
size_t ssm_ssd_workspace_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype);
int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                const float* h0, const ssm_scan_options* opts, void* y, float* h_last, int64_t Bs, int64_t L,
                int64_t H, int64_t P, int64_t G, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * Bidirectional multi-head scan (Bi-Mamba2 on the multi-head form): the
 * forward scan of ssm_ssd_fwd (with D x and h0) plus the same scan run in
 * decreasing time from g0 (zero if NULL) over the same inputs, read in place (no
 * flipped copy), the two outputs added -- the bidirectional combination of
 * "Some questions of Bi-Mamba2 and Hydra" (the author's first reply: two SSMs
 * with shared weights, the reverse one on the flipped sequence, plus D x):
 *
 *   g_t[p][n] = a_t g_{t+1}[p][n] + (dt[b,t,h] x[b,t,h,p]) B[b,t,g,n],   g_L = g0 (or 0)
 *   y[b,t,h,p] = sum_n C[b,t,g,n] (S_t[p][n] + g_t[p][n]) + D[h] x[b,t,h,p]
 *
 * with dt' in place of dt in both directions and the gate applied to the
 * complete sum when opts sets them. Arguments as ssm_ssd_fwd, and
 *   g0        : (Bs, H, P, N) float32, or NULL -- the reverse state entering
 *               at t = L-1 (zero if NULL; resumes the reverse direction from
 *               the next piece's g_first, as h0 resumes the forward one)
 *   g_first   : (Bs, H, P, N) float32, or NULL -- g after t = 0
 *   workspace : device memory of ssm_ssd_bidir_workspace_bytes(...) bytes:
 *               for bfloat16 the reverse direction's float32 partial of y
 *               (float32 puts it through y), and for a split sequence (as in
 *               ssm_ssd_fwd) both directions' range states; the reverse
 *               sweep of a split sequence runs in a launch of its own before
 *               the forward one. It may not overlap an argument; owned by
 *               the caller; NULL when the size is zero.
 * SSM_ERR_WORKSPACE if a needed workspace is missing or too small.
 * Otherwise conventions, numerics and error codes as ssm_ssd_fwd.
 */
size_t ssm_ssd_bidir_workspace_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype);
int ssm_ssd_bidir_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                      const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
                      float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* ssm_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */

/*
 * gla.h - C ABI of the chunkwise gated-linear-attention forward pass with
 * key-only decay over an H x W patch grid, for AMD Instinct MI355X (gfx950),
 * of the Spatial SwiGLU step that follows it in each block, and of the
 * SAGA-style non-causal gated linear attention.
 *
 * Operation (GTR news write-up, tokendh.com, section "What linear attention
 * saves": a running d_k x d_v summary, a learnable forget gate, decay on the
 * key side only with the value-side decay fixed at 1):
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t ,   o_t = q_t S_t ,   S_{-1} = 0
 *
 * with alpha_t = exp(log_alpha_t) in (0,1]^{d_k}, per token, head and key dim.
 * t runs over the H*W cells of the grid in the call's scan direction (same
 * write-up, section "The flaw of one-way scanning and GTR's fix": left->right,
 * right->left, top->bottom, bottom->top, cycled over the blocks); the state is
 * carried across row / column ends, one sequence of H*W steps per
 * (batch, head).  The computation is chunkwise (section "Where the speed comes
 * from": fixed-size chunks computed in parallel inside, a boundary state handed
 * between chunks, chunk summaries computed for all chunks at once and only the
 * boundary hand-off done in order).  No 1/sqrt(d_k) scale and no normaliser are
 * applied.
 *
 * Layout (all tensors dense, row-major, contiguous, 16-byte aligned):
 *   q, k, log_alpha : [B][heads][H][W][d_k]
 *   v, out          : [B][heads][H][W][d_v]      (out in grid order)
 *   One sequence's rows of one tensor, H*W*max(d_k, d_v) elements, must span
 *   less than 2 GiB (they are addressed with 32-bit byte offsets).
 *   final_state     : [B][heads][d_k][d_v] float32, the state after the last
 *                     scan step; may be NULL.
 *
 * Ownership and execution: the caller owns every buffer (device memory).  The
 * call validates its arguments on the host, then enqueues its kernels on
 * `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 * returns without waiting; errors raised while the kernels run surface at the
 * caller's next synchronisation.
 *
 * Workspace: a call that needs scratch memory (span states when the sequence
 * is split into spans; every backward and SAGA call) uses a device buffer that
 * the library keeps per (device, stream): allocated on the first such call on
 * that stream, grown (a new buffer) when a call needs more, and kept until
 * gla_release_workspaces.  Calls on one stream reuse it in stream order; each
 * use records an event that the next use on the same stream handle waits on.
 * Concurrent calls on different streams use different buffers and are
 * independent.  Under stream capture a call takes a stream-ordered
 * allocation of its own instead, released in the captured stream order.

 * Besides this table the library holds, process-wide: the forward mode
 * (gla_set_forward_mode), per-device caches of the resident workgroup slots
 * and CU count (read once from the device), a one-time read of tuning
 * environment variables, the measurement hook's per-thread events, and the
 * no-allocation entry's per-device array address.  With the single-pass
 * mode each stream's workspace also holds hand-off words (ticket and
 * finish counters, an epoch and one flag per span) that the kernel leaves
 * consistent for the next call on that stream.  The library keeps no
 * pointer to caller memory after returning.
 *
 * Errors: every argument check runs before any HIP call; on failure nothing is
 * enqueued and a negative status is returned (see gla_status_str).  Nothing
 * throws across this boundary.
 */
#ifndef GLA_H
#define GLA_H

#ifdef __cplusplus
extern "C" {
#endif

/* scan_dir values: the four directions, plus a batch rotation (batch element b
 * uses direction b mod 4, so one call covers a batch whose elements take
 * different directions). */
enum {
  GLA_SCAN_L2R = 0,           /* rows top to bottom, each left to right        */
  GLA_SCAN_R2L = 1,           /* rows top to bottom, each right to left        */
  GLA_SCAN_T2B = 2,           /* columns left to right, each top to bottom     */
  GLA_SCAN_B2T = 3,           /* columns left to right, each bottom to top     */
  GLA_SCAN_ROTATE_BATCH = 4
};

/* gate_mode values of gla_chunk_fwd_ex */
enum {
  GLA_GATE_LOG_ALPHA = 0,     /* `gate` holds log_alpha, as in gla_chunk_fwd          */
  GLA_GATE_LOGITS = 1         /* `gate` holds logits z: log_alpha = logsigmoid(z)/tau */
};

/* status codes */
enum {
  GLA_OK = 0,
  GLA_ERR_NULL = -1,          /* a required pointer is NULL                     */
  GLA_ERR_SHAPE = -2,         /* B, heads, H or W < 1, a size overflows, one
                                 sequence's rows of a tensor reach 2 GiB, or tau
                                 is not positive and finite                      */
  GLA_ERR_UNSUPPORTED = -3,   /* d_k / d_v / chunk combination not built, or a
                                 channel count that is not a multiple of 8       */
  GLA_ERR_ALIGN = -4,         /* a tensor pointer is not 16-byte aligned        */
  GLA_ERR_SCAN_DIR = -5,      /* scan_dir outside 0..4                          */
  GLA_ERR_ALIAS = -6,         /* an output overlaps another tensor              */
  GLA_ERR_HIP = -7,           /* a HIP runtime call failed while enqueueing     */
  GLA_ERR_SCRATCH = -8        /* gla_chunk_fwd_noalloc: the work split needs more
                                 span states than its fixed scratch holds       */
};

/*
 * Float16 entry: q, k, v, log_alpha and out are IEEE binary16; final_state is
 * float32.  Arithmetic: per-chunk cumulative log-decay in float32, 16-bit MFMA
 * tiles with float32 accumulation, float32 state; out is rounded to nearest
 * even.  Supported: chunk = 64, d_k in {64, 128}, d_v in {64, 128}.
 * Numerical domain: log_alpha finite and <= 0, of any strength.  A 32-token
 * step in which a scaled float16 operand could leave its range (a decay
 * below -10 in log2, about -6.9 in natural log, over 16 steps of one key dim,
 * or keys -- on the single-pass path queries or keys -- of magnitude 32 and
 * above) is computed exactly, token by token in float32, on every path
 * (strong forgetting: log-alpha of -2 per step, alpha -> 0).  Otherwise the
 * within-step attention scores q_t . k_s e^{b_t - b_s}, the state entries
 * (also a span's summary: the state its tokens alone reach) and the outputs
 * must lie in the float16 range (they pass through float16 MFMA operands or
 * are stored as float16).
 */
int gla_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                  int scan_dir, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                  void* out, float* final_state, void* stream);

/*
 * Execution paths of the float16 forward entries (gla_chunk_fwd,
 * gla_chunk_fwd_ex), chosen per call; results agree within the float16
 * tolerance, not bit for bit, since the span split differs:
 *   three passes: span summaries, the in-order scan of the span boundary
 *     states, the output pass (three kernels; only the output kernel when the
 *     sequence is not split into spans);
 *   two passes (d_k = d_v = 64, short sequences): span summaries, then the
 *     output pass, whose workgroups fold the initial state and the summaries
 *     of all earlier spans of their sequence into their own entry state (no
 *     scan kernel; the work of a span grows with its index, so it is used
 *     for few spans).  Chosen when a split into 2..16 spans of at most 4
 *     chunks puts every output workgroup on the device at once, and the call
 *     does not update its state in place (final_state == initial_state
 *     takes three passes);
 *   single pass (d_k = d_v = 64, only when forced): one kernel; each
 *     workgroup summarises its span, publishes the summary and a flag, folds
 *     the earlier spans' published summaries into its entry state and
 *     writes its outputs.  A 32-token step whose decay would push the
 *     float16 scaled operands out of range is computed exactly token by
 *     token, so this path has no domain limit on log_alpha beyond being
 *     finite and <= 0.
 * mode: GLA_FWD_AUTO (default, the rule above), GLA_FWD_THREE_PASS (always
 * three passes), GLA_FWD_TWO_PASS (two passes whenever the sequence splits
 * into 2..16 spans, of any length), GLA_FWD_SINGLE_PASS (the single pass
 * for d_k = d_v = 64, else the automatic choice).  Process-wide, for calls
 * made after it; a tuning and testing switch, all paths meet the same
 * accuracy.  Returns GLA_OK, or GLA_ERR_SHAPE for an unknown mode.  The
 * environment variable GLA_SPAN_CHUNKS (a forced span length) selects three
 * passes.
 */
enum {
  GLA_FWD_AUTO = 0,
  GLA_FWD_THREE_PASS = 1,
  GLA_FWD_TWO_PASS = 2,
  GLA_FWD_SINGLE_PASS = 3
};
int gla_set_forward_mode(int mode);

/*
 * No-allocation variant of gla_chunk_fwd, for callers that cannot allocate
 * device memory while they call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, layout, semantics
 * and errors as gla_chunk_fwd, plus GLA_ERR_SCRATCH.
 *
 * The span states of a split sequence live in one fixed device array of
 * GLA_NOALLOC_SCRATCH_BYTES, part of the library's device code: each device
 * gets its own copy when the library's code is loaded there and holds it until
 * the process ends; the call looks up the current device's copy on its first
 * use there (hipGetSymbolAddress) and allocates and frees nothing.  The call
 * takes the work split gla_chunk_fwd would take (gla_plan_forward), except
 * that the single-pass mode is not used: its hand-off words would need an
 * allocation, so under that mode the call takes the automatic choice.  The
 * span states take B*heads*n_spans*d_k floats (gate products) and
 * B*heads*n_spans*d_k*d_v float16 states on the three-pass path, and
 * B*heads*n_spans*(d_k*d_v + d_k) floats on the two-pass path (the
 * workspace of gla_plan_forward's split); an automatic split
 * has at most one span per resident output workgroup, which on an MI355X
 * stays within the array for every supported d_k, d_v.  A split that does not
 * fit (a forced one: gla_set_forward_mode with two or three passes, or
 * GLA_SPAN_CHUNKS) returns GLA_ERR_SCRATCH before anything is enqueued.
 *
 * The array is shared by every call on its device and keeps whatever the last
 * call left; nothing in it needs to start at zero (every state is written
 * before it is read).  Calls on one stream run in order; calls that overlap in
 * time on one device (different streams) race on the array and their results
 * are undefined.
 */
#define GLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                          int scan_dir, int B, int heads, int H, int W, int d_k, int d_v,
                          int chunk, void* out, float* final_state, void* stream);

/*
 * Extended float16 entry: gla_chunk_fwd plus an initial state and a fused
 * forget-gate activation.
 *
 * The pages describe a learnable forget gate on the key side (GTR news
 * write-up, section "What linear attention saves"); with gate_mode =
 * GLA_GATE_LOGITS the kernels read the gate's pre-activation logits z (same
 * layout and type as log_alpha) and use log_alpha = logsigmoid(z) / tau, i.e.
 * alpha = sigmoid(z)^(1/tau), computed in float32 and rounded to float16
 * where the kernels use it.  This saves the separate pass that would write
 * log_alpha.  tau must be positive and finite (16 in the GTR-style
 * workloads).  With GLA_GATE_LOG_ALPHA, `gate` is log_alpha and tau is
 * ignored.
 *
 * initial_state: [B][heads][d_k][d_v] float32, the state before the first scan
 * step (NULL = zero), as when resuming a scan that was cut into pieces: the
 * final_state of one call fed to the next reproduces the uncut scan.
 * final_state may be the same pointer as initial_state (updated in place);
 * any other overlap between them, or between initial_state and out, is
 * GLA_ERR_ALIAS.  Alignment: 4 bytes.
 *
 * Errors as gla_chunk_fwd, plus GLA_ERR_UNSUPPORTED for an unknown gate_mode
 * (checked first) and GLA_ERR_SHAPE for a bad tau.
 */
int gla_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* gate, int gate_mode,
                     float tau, const float* initial_state, int scan_dir, int B, int heads, int H,
                     int W, int d_k, int d_v, int chunk, void* out, float* final_state,
                     void* stream);

/*
 * Float32 entry: every tensor float32, float32 MFMA tiles, float32 state.
 * Same arguments and semantics.  Supported: chunk = 64, d_k in {64, 128},
 * d_v in {64, 128}.  Domain: log_alpha finite and <= 0, 16-step decay >= -80.
 */
int gla_chunk_fwd_f32(const float* q, const float* k, const float* v, const float* log_alpha,
                      int scan_dir, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                      float* out, float* final_state, void* stream);

/*
 * Work split the forward call would use on the current device: each sequence
 * of ceil(H*W/64) chunks is cut into n_spans spans of span_chunks chunks (the
 * last may be shorter), one output workgroup per (batch, head, span).  When
 * n_spans > 1 the call also runs the span-summary kernel, and the span-scan
 * kernel on the three-pass path, and uses a workspace of B*heads*n_spans*d_k
 * floats (gate products) plus B*heads*n_spans*d_k*d_v float16 span states
 * (summaries, which the scan turns into entry states in place) on the float16
 * three-pass path, or B*heads*n_spans*(d_k*d_v + d_k) floats otherwise; a
 * forced float16 three-pass split whose span states of one sequence reach
 * 2 GiB returns GLA_ERR_SHAPE.  gla_plan_forward also gives the
 * number of kernels the call runs: 1 (no split), 2 (two-pass path) or 3
 * (three-pass path; see gla_set_forward_mode).  use_f32 selects the float32
 * entry.  Reads device attributes (a HIP call); returns the same argument
 * errors as the forward entry points, and GLA_ERR_NULL for a NULL output.
 */
int gla_plan_forward(int use_f32, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                     int* span_chunks, int* n_spans, int* kernels);
int gla_plan_spans(int use_f32, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                   int* span_chunks, int* n_spans);

/*
 * Backward pass (float16; d_k, d_v in {64, 128}, chunk = 64): the gradients of
 *
 *   L = sum(d_out * out) + sum(d_final_state * final_state)
 *
 * for the forward call on the same q, k, v, log_alpha, scan_dir and
 * initial_state.  The adjoint of the state, G_t = dL/dS_t, runs backwards
 * along the scan, G_t = q_t^T dO_t + diag(alpha_{t+1}) G_{t+1} from
 * G = d_final_state, and gives dq_t = S_t dO_t, dk_t = G_t v_t,
 * dv_t = k_t G_t, dlog_alpha_t = alpha_t * rowsum(G_t * S_{t-1}) and
 * d_initial_state = diag(alpha_0) G_0; the pass is chunkwise like the
 * forward one (GTR news write-up, sections "What linear attention saves" and
 * "Where the speed comes from"): the forward state entering each chunk and
 * the adjoint state entering it from its right come from a summary kernel and
 * a scan kernel over chunks (the adjoint recurrence is the forward one read
 * from the end; per-chunk summaries and states are kept as float16, the scans
 * accumulate in float32), then every chunk computes its gradients
 * independently.  When every persistent workgroup of the chunk kernel gets at
 * least 16 chunks, the forward states are kept per pair of chunks instead, and
 * the second chunk of a pair starts from the state the first one reaches;
 * the environment variable GLA_BWD_PAIRS (1 or 0, read on every call) forces
 * the paired or the per-chunk form.
 *
 * Layout as gla_chunk_fwd; d_out is [B][heads][H][W][d_v] float16;
 * d_final_state and initial_state are float32 [B][heads][d_k][d_v] or NULL
 * (zero).  Outputs: dq, dk, dlog_alpha [B][heads][H][W][d_k] and dv
 * [B][heads][H][W][d_v] float16 (rounded to nearest even), d_initial_state
 * float32 [B][heads][d_k][d_v] or NULL (not wanted).  Pointers 16-byte
 * aligned; no output may overlap an input or another output.  A head wider
 * than 64 runs as a grid of 64 x 64 blocks (key dims x value dims): the key
 * rows and value columns of the state evolve independently, so each block is
 * the 64-dim problem on its dims, dv adds up over the key blocks and dq, dk,
 * dlog_alpha over the value blocks (each addition of a float16 partial
 * rounds once more), and d_initial_state is the blocks side by side.  The
 * call uses a workspace of B*heads*2*n_chunks*64 floats plus
 * B*heads*2*n_chunks*64*64 float16 chunk states and 256 bytes (a
 * work counter), n_chunks = ceil(H*W/64), reused by the blocks in turn.  Domain: log_alpha finite and <= 0 with the
 * decay summed over any 16 consecutive scan steps of one key dim >= -10
 * (natural log: the backward's scaled float16 tiles use factors up to e^10;
 * unlike the forward it has no exact fallback), plus d_out . v, both states
 * and their per-chunk summaries within float16 range.  Errors as gla_chunk_fwd
 * (GLA_ERR_UNSUPPORTED for any other d_k, d_v or chunk).  With the
 * measurement hook armed, event pairs bracket the kernel that forms both
 * summaries of every chunk (events 0, 1), the kernel that scans both (2, 3)
 * and the chunk kernel (4, 5), of the last block when there are several.
 */
int gla_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                  const void* d_out, const float* d_final_state, const float* initial_state,
                  int scan_dir, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                  void* dq, void* dk, void* dv, void* dlog_alpha, float* d_initial_state,
                  void* stream);

/*
 * Spatial SwiGLU step (float16), the other token mixer of each GTR block:
 *
 *   out[b,y,x,c] = silu(gate[b,y,x,c]) *
 *                  (bias[c] + sum_{i,j=0..2} weight[c][i][j] * value[b, y+i-1, x+j-1, c])
 *
 * SwiGLU with a 3x3 depthwise convolution inserted in its value branch, each
 * channel filtered with its own kernel, so that a patch sees its eight grid
 * neighbours directly (GTR news write-up, tokendh.com, section "The flaw of
 * one-way scanning and GTR's fix", the Spatial SwiGLU and depthwise
 * convolution notes).  silu(g) = g / (1 + exp(-g)).  Readings where the pages
 * are silent: zero padding of one cell, stride 1 (output grid = input grid);
 * taps applied as a cross-correlation (tap (i, j) weighs the neighbour at
 * row offset i-1, column offset j-1, as deep-learning convolution layers do);
 * an optional per-channel bias before the gate multiplies.  The projections
 * that produce gate and value, and the one after, are dense matrix products
 * and not part of this call.
 *
 * Layout (float16, channels last):
 *   gate, value : B*H*W tokens in grid order [B][H][W], token n at element
 *                 n * ld_in; its C channels contiguous.  ld_in = C for two
 *                 separate tensors, ld_in = 2C for the halves of one fused
 *                 [B][H][W][2C] projection (value = gate + C).
 *   weight      : [C][3][3] (a [C][1][3][3] layer weight as is).
 *   bias        : [C], or NULL for none.
 *   out         : [B][H][W][C], contiguous.
 * Arithmetic: each tap is a float16 x float16 product summed in float32, the
 * gate activation in float32, out rounded to nearest even.
 * Supported: C and ld_in multiples of 8, ld_in >= C; one image's rows
 * (H*W*ld_in elements) below 2 GiB.  Pointers 16-byte aligned.  out may not
 * overlap any input (a tile still reads its neighbours' values).
 * Ownership and errors as gla_chunk_fwd: asynchronous on `stream`, the caller
 * owns every buffer, all checks before any HIP call, nothing enqueued on
 * failure.  GLA_ERR_NULL (gate, value, weight or out NULL), GLA_ERR_SHAPE
 * (a size < 1, ld_in < C, a size overflow), GLA_ERR_UNSUPPORTED (C or ld_in
 * not a multiple of 8), GLA_ERR_ALIGN, GLA_ERR_ALIAS.
 */
int gla_spatial_swiglu(const void* gate, const void* value, int ld_in, const void* weight,
                       const void* bias, int B, int H, int W, int C, void* out, void* stream);

/*
 * SAGA-style non-causal gated linear attention (float16):
 *
 *   KV = (K * A)^T (V * B),   O = Q KV      per (batch, head)
 *
 * Each token's key-value map k_i^T v_i is scaled element by element by a gate
 * alpha_i^T beta_i before the maps are summed; by the Hadamard-product
 * identity the gate is applied to K and V instead, so no per-token map is
 * formed (SAGA summary, gist.science, Methodology sections A and B).  Every
 * token attends to all N tokens of its sequence (no causal order).  The gates
 * are inputs (produced upstream); no normaliser or scale is applied.
 *
 * Layout (dense, contiguous, 16-byte aligned, float16):
 *   q, k, alpha : [B][heads][N][d_k]
 *   v, beta, out: [B][heads][N][d_v]
 *   kv          : [B][heads][d_k][d_v] float32, the gated maps; may be NULL.
 * Arithmetic: k*alpha and v*beta rounded to float16, maps accumulated on
 * 16-bit MFMA tiles in float32 (span partials summed in a fixed order, so
 * results are bitwise reproducible), then read as float16 scaled by a power
 * of two per 16 value columns; out rounded to nearest even.
 * Supported: d_k, d_v in {64, 128}; one sequence's rows of a tensor below
 * 2 GiB.  out and kv may not overlap any input or each other.
 * Ownership and errors as gla_chunk_fwd (with a workspace of about
 * B*heads*d_k*d_v*(s + 1/2) floats, s the accumulation spans per sequence, a
 * few workgroups per CU in all): GLA_ERR_NULL, GLA_ERR_SHAPE, GLA_ERR_UNSUPPORTED
 * (d_k / d_v), GLA_ERR_ALIGN, GLA_ERR_ALIAS.  With the measurement hook armed
 * the accumulation, reduction and output kernels record event pairs 0, 1, 2
 * (the reduction's pair back to back when one span covers a sequence).
 */
int gla_saga_fwd(const void* q, const void* k, const void* v, const void* alpha,
                 const void* beta, int B, int heads, int N, int d_k, int d_v, void* out, float* kv,
                 void* stream);

/*
 * Measurement hook (for benchmarks and profilers, not needed for computing).
 * events: n = 6 hipEvent_t handles (as void*), or n = 0 to clear.  The next
 * forward call made by the calling thread has each of its three kernels (span
 * summary, span scan, output) record a start / stop pair, events[2i] and
 * events[2i+1], from its own dispatch (hipExtLaunchKernelGGL), so the interval
 * is that kernel's execution; a kernel the call does not run (no span split)
 * records its pair back to back.  A gla_spatial_swiglu call instead records
 * events[0] / events[1] around its one kernel.  The hook then clears itself.  The caller
 * owns the events.  Returns GLA_ERR_NULL if n = 6 and a handle is NULL,
 * GLA_ERR_SHAPE if n is neither 0 nor 6.
 */
int gla_set_kernel_events(void* const* events, int n);

/*
 * Frees every workspace buffer the library holds (see "Workspace" above):
 * for each device that holds one it waits for that device's work
 * (hipDeviceSynchronize), then frees its buffers; the calling thread's current
 * device is restored.  Calls made afterwards allocate again.  Must not run
 * concurrently with calls that are being enqueued.  Returns GLA_OK (also when
 * nothing is held, without any HIP call) or GLA_ERR_HIP if a HIP call fails
 * (the table is emptied regardless).
 */
int gla_release_workspaces(void);

/* Static, human-readable text for a status code. */
const char* gla_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int gla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */

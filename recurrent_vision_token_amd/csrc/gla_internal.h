// Internal interface between the host API layer (gla_api.cpp) and the HIP
// kernels (gla_kernels.hip).  Not installed, not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace gla {

enum class Dtype { kF16, kF32 };

// One call of the forward pass, already validated on the host.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* la;
  void* out;
  float* final_state;   // may be null
  const float* initial_state;  // [B][heads][d_k][d_v], may be null (zero state)
  float inv_tau;        // 1 / tau when `la` holds gate logits (fused activation)
  float* span_state;    // [BH][n_spans][d_k][d_v] span summaries, then entry states (float32
                        // three passes), or summaries in the output kernel's layout (two
                        // passes); unused on the float16 three-pass path
  float* span_gate;     // [BH][n_spans][d_k] product of the span's gates
  void* span_entry16;   // [BH][n_spans][d_k][d_v] float16 span summaries, then (in place)
                        // the entry states (float16 three passes)
  int B, heads, H, W, T;
  // t / W and t / H as (umulhi(t, m) + t) >> s, exact for t < 2^31
  unsigned int div_w_m, div_h_m;
  int div_w_s, div_h_s;
  int scan_dir;
  int n_chunks;         // ceil(T / 64)
  int span_chunks;      // chunks handled by one workgroup of the output kernel
  int n_spans;          // ceil(n_chunks / span_chunks)
  // backward pass (spans of one chunk): span_entry16 holds the float16 forward
  // summaries, then the entry states; the adjoint recurrence likewise
  int adj_slots;        // summary slots per sequence of the adjoint scan (n_spans)
  const void* dout;     // the output gradient, in place of v
  float* adj_gate;      // [BH][adj_slots][d_k]
  void* adj_entry16;    // [BH][adj_slots][d_k][d_v] float16 adjoint summaries, then entry states
  const float* adj_initial;  // the final-state gradient (scan start), may be null
  float* adj_final;     // the adjoint state after its last slot (the gradient of the state
                        // before the first step), float32 in the initial state's layout, or null
  int spans_per_wg;     // spans streamed by one workgroup of the summaries kernel
  unsigned int* bwd_ticket;  // the backward chunk kernel's ticket counter, cleared by the scans
  // the backward pass runs on 64 x 64 blocks of a larger head: row strides of
  // the [T][d_k]-side tensors (q, k, log-alpha) and the [T][d_v]-side ones
  // (v, d_out), in elements, and the layout of the caller's [BH][d_k][d_v]
  // float32 states (adj_initial, initial_state, adj_final): element (i, j) of
  // sequence bh at bh * st_bh + i * st_row + j
  unsigned int ldk, ldv, st_row, st_bh;
  // single-pass forward: hand-off words and span aggregates
  unsigned int* sync;   // [0] ticket, [1] finished workgroups, [2] epoch, [3] error bits,
                        // then one ready flag per (batch*head, span) from word kSyncFlags on
  float* agg;           // [BH][n_spans][64 + d_k * d_v]: gate product, then state
};

// Single-pass forward (float16, d_k = d_v = 64): one kernel; each workgroup
// summarises its span, publishes the summary, folds the summaries of the
// earlier spans of its sequence into its entry state as soon as they are
// published, then computes the span's outputs.  Needs p.sync (kSyncFlags +
// B*heads*n_spans words, zero before first use and left consistent by every
// call) and p.agg (B*heads*n_spans*kAggFloats floats).  events: null or six
// hipEvent_t; pair 2 brackets the kernel, pairs 0 and 1 are recorded back to
// back.
constexpr int kSyncFlags = 64;
constexpr int kAggFloats = 64 + 64 * 64;
bool has_fused(Dtype dt, int d_k, int d_v);
int fused_blocks_per_cu(bool gate_logits);
hipError_t launch_forward_fused(bool gate_logits, const FwdParams& p, hipStream_t stream,
                                hipEvent_t const* events);
// Error bits a single-pass call left in its hand-off words (bit 0: a wait
// for an earlier span's summary timed out).
constexpr unsigned int kSyncErrTimeout = 1u;
// Zero `words` 32-bit words at p on `stream` with a kernel (usable under
// stream capture, where a memset node is avoided).
hipError_t launch_zero_words(unsigned int* p, size_t words, hipStream_t stream);

// Multiply-shift constants for dividing t < 2^31 by d >= 1:
// t / d == (umulhi(t, m) + t) >> s.
void fast_div_constants(unsigned int d, unsigned int* m, int* s);

// Float16 forward with its span states in a caller-fixed device buffer
// instead of the workspace cache: scratch_of(dev) gives the current device's
// buffer of scratch_bytes (null on failure); nothing is allocated.
int forward_no_alloc(const void* q, const void* k, const void* v, const void* log_alpha,
                     int scan_dir, int B, int heads, int H, int W, int d_k, int d_v, int chunk,
                     void* out, float* final_state, void* stream, void* (*scratch_of)(int dev),
                     size_t scratch_bytes);

// Output-kernel workgroups resident per CU for this variant (occupancy).
int output_blocks_per_cu(Dtype dt, int d_k, int d_v, bool gate_logits);

// True when a kernel family is compiled for this (dtype, d_k, d_v).
bool has_variant(Dtype dt, int d_k, int d_v);

// Enqueue the span-summary, span-scan and output kernels on `stream`.
// The caller has validated p and supplied a workspace when n_spans > 1.
// events: null, or six hipEvent_t recorded around the kernels (see gla.h).
// gate_logits: `la` holds gate logits z and the kernels use
// log alpha = logsigmoid(z) * inv_tau (float16 only).
hipError_t launch_forward(Dtype dt, int d_k, int d_v, bool gate_logits, const FwdParams& p,
                          hipStream_t stream, hipEvent_t const* events);

// Two-pass forward (float16, d_k = d_v = 64): the span-summary kernel, with
// each summary stored in the output kernel's register layout, then the
// output kernel, whose workgroups fold the initial state and the summaries of
// all earlier spans of their sequence into their entry state (no scan
// kernel).  Needs 2 <= n_spans <= kTwoPassMaxSpans and span_state /
// span_gate as for the three-pass path.  events: null, or six hipEvent_t
// (pair 0 around the summary kernel, pair 1 back to back, pair 2 around the
// output kernel).
constexpr int kTwoPassMaxSpans = 16;
bool has_two_pass(Dtype dt, int d_k, int d_v);
// Resident workgroups per CU of the two-pass output kernel.
int two_pass_blocks_per_cu(bool gate_logits);
hipError_t launch_forward_two_pass(bool gate_logits, const FwdParams& p, hipStream_t stream,
                                   hipEvent_t const* events);

// Backward pass, float16, d_k = d_v = 64.  `p` describes the forward
// tensors (q, k, v, la; spans of one chunk, n_spans = n_chunks of them) with
// the forward-state workspace (span_entry16, span_gate, initial_state) and
// the adjoint recurrence: dout, adj_entry16, adj_gate, adj_initial (the
// final-state gradient), adj_slots = n_spans and adj_final.  Runs the
// fused summaries kernel and the fused scans kernel; events: null, or at
// least four hipEvent_t, the start / stop of each.
hipError_t launch_bwd_states(int d_k, int d_v, const FwdParams& p, hipStream_t stream,
                             hipEvent_t const* events);

// The chunk kernel of the backward pass: n_wg persistent workgroups take the
// (batch*head, chunk) pairs (the first n_wg one each, the rest by ticket from
// p.ticket, which must be zero at launch) and turn each chunk's tiles, its forward
// entry state and the adjoint state entering it from the right into dq, dk,
// dv and dlog_alpha.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* la;
  const void* dout;         // [B][heads][H][W][d_v]
  void* dq;                 // [B][heads][H][W][d_k]
  void* dk;
  void* dv;                 // [B][heads][H][W][d_v]
  void* dla;                // [B][heads][H][W][d_k]
  const void* fwd_state;    // [BH][ceil(n_chunks / fwd_span)][d_k][d_v] float16: slot
                            // c / fwd_span is the state entering chunk c, the
                            // first of its unit
  const void* adj_state;    // [BH][n_chunks][d_k][d_v] float16: slot n_chunks - 1 - c is the
                            // state gradient entering chunk c from the right
  int B, heads, H, W, T;
  unsigned int div_w_m, div_h_m;
  int div_w_s, div_h_s;
  int scan_dir;
  int n_chunks;
  // one 64 x 64 block of a larger head: row strides of the [T][d_k]-side
  // tensors (q, k, log-alpha, dq, dk, dlog-alpha) and the [T][d_v]-side ones
  // (v, d_out, dv), in elements; and which gradients add to what the outputs
  // already hold (a block after the first along the key dims adds dv, along
  // the value dims dq, dk and dlog-alpha)
  unsigned int ldk, ldv;
  int acc_dv, acc_dqk;
  int n_wg;                 // persistent workgroups (at most two per CU)
  int fwd_span;             // chunks per work unit: 2 (pairs, the second entering with
                            // the first one's next state) or 1
  // the chunks after each workgroup's first are handed out in ticket
  // order; the counter is zero when the kernel starts (the state scans
  // before it clear it)
  unsigned int* ticket;
};

hipError_t launch_bwd_chunks(int d_k, int d_v, const BwdParams& p, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop);

// One call of the Spatial SwiGLU step (float16), already validated on the host.
struct SwigluParams {
  const void* gate;     // [B][H][W] tokens of ld_in elements, first C used
  const void* value;    // same layout as gate
  const void* weight;   // [C][3][3]
  const void* bias;     // [C] or null (no bias)
  void* out;            // [B][H][W] tokens of ld_out elements
  int B, H, W, C;
  int ld_in, ld_out;
  int rows_per_tile;    // 8, 16 or 32 grid rows per workgroup
  int row_tiles, col_tiles, ch_tiles;
  int n_tiles;          // B * row_tiles * col_tiles * ch_tiles workgroups
};

// Fill the work split of p (rows_per_tile, the tile counts and n_tiles) from
// B, H, W, C; false when the launch would be too large.
bool swiglu_plan(SwigluParams& p);

// Enqueue the Spatial SwiGLU kernel on `stream`; start / stop (may be null)
// are recorded around its dispatch.
hipError_t launch_spatial_swiglu(const SwigluParams& p, hipStream_t stream, hipEvent_t start,
                                 hipEvent_t stop);

// One call of the SAGA-style non-causal gated linear attention (float16),
// already validated on the host.
struct SagaParams {
  const void* q;        // [B][heads][N][d_k]
  const void* k;        // [B][heads][N][d_k]
  const void* v;        // [B][heads][N][d_v]
  const void* a;        // key-side gates [B][heads][N][d_k]
  const void* b;        // value-side gates [B][heads][N][d_v]
  void* out;            // [B][heads][N][d_v]
  float* kv;            // [B*heads][d_k][d_v] gated key-value maps, or null
  void* amap;           // [B*heads][d_v/16][d_k/32][64] x 8 float16: the output kernel's
                        // A operands, each scaled by a power of two (workspace)
  float* unscale;       // [B*heads][d_v/16][d_k/32] the inverse scales (workspace)
  float* partial;       // [B*heads][n_spans][d_k][d_v] span partials (workspace)
  int B, heads, N, d_k, d_v;
  int n_chunks;         // ceil(N / saga_chunk_tokens()) accumulation steps
  int span_chunks;      // steps per span of the accumulation kernel
  int n_spans;          // ceil(n_chunks / span_chunks)
  int n_tblocks;        // ceil(N / saga_out_tokens()) output workgroups per (b, h)
};

int saga_chunk_tokens();
int saga_out_tokens();
bool saga_has_variant(int d_k, int d_v);

// Enqueue the accumulation, reduction and output kernels;
// events: null, or six hipEvent_t recorded around the three kernels.
hipError_t launch_saga(const SagaParams& p, hipStream_t stream, hipEvent_t const* events);

}  // namespace gla

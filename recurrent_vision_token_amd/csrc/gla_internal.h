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
  float* span_state;    // [BH][n_spans][d_k][d_v] span summaries, then entry states (three
                        // passes), or summaries in the output kernel's layout (two passes)
  float* span_gate;     // [BH][n_spans][d_k] product of the span's gates
  int B, heads, H, W, T;
  // t / W and t / H as (umulhi(t, m) + t) >> s, exact for t < 2^31
  unsigned int div_w_m, div_h_m;
  int div_w_s, div_h_s;
  int scan_dir;
  int n_chunks;         // ceil(T / 64)
  int span_chunks;      // chunks handled by one workgroup of the output kernel
  int n_spans;          // ceil(n_chunks / span_chunks)
  // backward pass: the adjoint recurrence's inputs and summaries
  int adj_slots;        // summary slots per sequence of the adjoint scan (n_spans + 1)
  const void* dout;     // the output gradient, in place of v
  float* adj_state;     // [BH][adj_slots][d_k][d_v]
  float* adj_gate;      // [BH][adj_slots][d_k]
  const float* adj_initial;  // the final-state gradient (scan start), may be null
  int spans_per_wg;     // spans streamed by one workgroup of the summaries kernel
};

// Multiply-shift constants for dividing t < 2^31 by d >= 1:
// t / d == (umulhi(t, m) + t) >> s.
void fast_div_constants(unsigned int d, unsigned int* m, int* s);

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
hipError_t launch_forward_two_pass(bool gate_logits, const FwdParams& p, hipStream_t stream,
                                   hipEvent_t const* events);

// Backward pass, float16, d_k = d_v = 64.  `p` describes the forward
// tensors (q, k, v, la; spans of span_chunks chunks, n_spans of them) with
// the forward-state workspace (span_state, span_gate, initial_state) and the
// adjoint recurrence: dout, adj_state, adj_gate, adj_initial (the final-state
// gradient) and adj_slots = n_spans + 1.  Runs the fused summaries kernel
// and the fused scans kernel; events: null, or at least four hipEvent_t, the
// start / stop of each.
hipError_t launch_bwd_states(int d_k, int d_v, const FwdParams& p, hipStream_t stream,
                             hipEvent_t const* events);

// The chunk kernel of the backward pass: one workgroup per (batch*head,
// chunk) turns the chunk's tiles, its forward entry state and the adjoint
// state entering it from the right into dq, dk, dv and dlog_alpha.
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
  const float* fwd_state;   // [BH][n_spans][d_k][d_v] state entering each span of two chunks
  const float* adj_state;   // [BH][n_spans + 1][d_k][d_v]: slot n_spans - 1 - s enters span s's
                            // last chunk from the right; slot n_spans is dL/dS_{-1}
  float* d_initial_state;   // [BH][d_k][d_v], or null
  int B, heads, H, W, T;
  unsigned int div_w_m, div_h_m;
  int div_w_s, div_h_s;
  int scan_dir;
  int n_chunks;
  int n_spans;              // ceil(n_chunks / 2)
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

// Chunkwise forward pass of gated linear attention with key-only decay over an
// H x W patch grid, for gfx950 (CDNA4, MI355X).
//
// The recurrence S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t is
// evaluated chunkwise (GTR news write-up, tokendh.com, section "Where the speed
// comes from"): the scan is cut into 64-token chunks; everything inside a chunk
// is dense 16x16 MFMA tiles, and only a d_k x d_v boundary state is handed
// along the scan.  The "summarise every chunk in parallel, hand off only the
// boundary state in order" split of the same section becomes three kernels:
//
//   1. span_summary : one workgroup per (batch*head, span of chunks) runs the
//                     span from a zero state and writes its summary
//                     (prod alpha over the span, state reached) - fully parallel;
//   2. span_scan    : per (batch*head) the short sequential scan over spans,
//                     elementwise over the d_k*d_v state, turning summaries into
//                     each span's entry state;
//   3. chunk_output : one workgroup per (batch*head, span) replays its chunks
//                     from the entry state and writes outputs in grid order.
//
// When batch*heads alone fills the chip there is one span per sequence and only
// kernel 3 runs.
//
// Inside a chunk (scan steps cC .. cC+63, b_t = inclusive cumulative log decay):
//   o_t = sum_{s<=t} (q_t . (k_s * exp(b_t - b_s))) v_s  +  (q_t * exp(b_t)) S_entry
// The decay mask exp(b_t - b_s) is rank one per key dim, so it splits into a
// row scaling of Q and a column scaling of K (the Hadamard-product identity of
// the SAGA summary, gist.science, Methodology section B).  Scalings are anchored
// per 16-token sub-block so every 16-bit factor stays in range: q_t*exp(c_t) and
// k_s*exp(-c_s) with c the cumulative decay inside the sub-block, and between
// sub-blocks J < I an extra per-dim factor exp(Bst_I - Bst_J) <= 1.
//
// The scan direction is an index remap applied to every 16-byte row load and
// store (cell = pi(t)); no transposed copy of any tensor is made.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "gla_device.h"
#include "gla_internal.h"
#include "gla_tiles.h"

namespace gla {
namespace {

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kSub = 16;       // tokens per sub-block (one MFMA tile edge)
constexpr int kThreads = 256;  // four wave64s

// Element traits of the generic (float32) kernels.
template <class T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kPerPiece = 4;  // elements per 16-byte row piece
  static constexpr int kPad = 4;       // LDS row padding (elements)
  typedef f32x4 piece_t;               // one 16-byte piece as a vector
};

template <class T>
__device__ __forceinline__ float fexp(float x) {
  return expf(x);
}

// Pair index of sub-block pair (I, J), J < I, in the factor table.
__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// ---------------------------------------------------------------------------
// Shared-memory tiles of one chunk (float32 output kernel).  Two tiles are
// reused within a chunk so that d_k = 128 fits (160 KB at d_v = 128):
// log-alpha arrives transposed in the tile of the decayed keys (each
// (key dim, sub-block) item reads its own 16 entries before it overwrites
// them), and the output staging shares the key tile, which is dead once the
// score tiles are formed.
template <class T, int DK, int DV>
struct ChunkSmem {
  static constexpr int P = Elt<T>::kPad;
  static constexpr int QS = DK + P;      // row stride: [token][d_k] tiles
  static constexpr int AS = kChunk + P;  // row stride: [*][token] tiles
  static constexpr int OS = DV + P;      // row stride: [token][d_v] tile
  alignas(16) T q[kChunk * QS];    // raw q, then q_t*exp(c_t)
  union {
    alignas(16) T k[kChunk * QS];  // raw k, then k_s*exp(-c_s)
    alignas(16) T o[kChunk * OS];  // output staging [token][d_v]
  };
  alignas(16) T sa[kChunk * AS];   // A^T tiles: A[t][s] at [t][s]
  alignas(16) T vt[DV * AS];       // V^T [d_v][token]
  alignas(16) T klt[DK * AS];      // log-alpha^T, then (k_s*exp(b_last-b_s))^T [d_k][token]
  alignas(16) float e[4 * DK];     // exp(Bst_I): decay from chunk start to sub-block I
  alignas(16) float f[6 * DK];     // exp(Bst_I - Bst_J), J < I
  alignas(16) float g[DK];         // exp(b_last): decay over the whole chunk
};

template <class T, int DK, int DV>
struct SummarySmem {
  static constexpr int P = Elt<T>::kPad;
  static constexpr int QS = DK + P;
  static constexpr int AS = kChunk + P;
  alignas(16) T k[kChunk * QS];
  alignas(16) T la[kChunk * QS];
  alignas(16) T vt[DV * AS];
  alignas(16) T klt[DK * AS];
  alignas(16) float g[DK];
};

// ---------------------------------------------------------------------------
// Row-piece loader: q, k, log-alpha as [token][d_k], v as token pairs for the
// transposed V tile.  Pieces beyond the sequence end read as zero.
template <class T, int DK, int DV>
struct Loader {
  static constexpr int EPP = Elt<T>::kPerPiece;
  static constexpr int PPT_K = DK / EPP;                 // pieces per token row (d_k)
  static constexpr int PPT_V = DV / EPP;                 // pieces per token row (d_v)
  static constexpr int NK = kChunk * PPT_K / kThreads;   // d_k pieces per thread
  static constexpr int NVP = (kChunk / 2) * PPT_V / kThreads;  // v token pairs per thread
  static_assert(NK >= 1 && NVP >= 1, "tile too small for the thread count");

  uint4 rq[NK], rk[NK], rl[NK], rv[2 * NVP];

  __device__ __forceinline__ static uint4 ld(const T* base, size_t off) {
    return *reinterpret_cast<const uint4*>(base + off);
  }

  template <bool WITH_Q>
  __device__ __forceinline__ void load(const T* q, const T* k, const T* la, const T* v,
                                       size_t off_k, size_t off_v, int t0, int valid, const GridMap& gm) {
    const int tid = threadIdx.x;
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int id = tid + kThreads * j;
      const int tok = id / PPT_K;
      const int pc = id - tok * PPT_K;
      if (tok < valid) {
        const size_t o = off_k + (size_t)gm.cell(t0 + tok) * DK + pc * EPP;
        if (WITH_Q) rq[j] = ld(q, o);
        rk[j] = ld(k, o);
        rl[j] = ld(la, o);
      } else {
        if (WITH_Q) rq[j] = zero;
        rk[j] = zero;
        rl[j] = zero;
      }
    }
#pragma unroll
    for (int j = 0; j < NVP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PPT_V;
      const int pc = id - tp * PPT_V;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = 2 * tp + h;
        rv[2 * j + h] = (tok < valid)
                            ? ld(v, off_v + (size_t)gm.cell(t0 + tok) * DV + pc * EPP)
                            : zero;
      }
    }
  }

  // Registers -> shared tiles: q, k row-major; la row-major, or with LA_T
  // transposed to [d_k][token] (row stride AS); v transposed to [d_v][token].
  template <bool WITH_Q, bool LA_T = false>
  __device__ __forceinline__ void store(T* sq, T* sk, T* sla, T* svt, int QS, int AS) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int id = tid + kThreads * j;
      const int tok = id / PPT_K;
      const int pc = id - tok * PPT_K;
      const int o = tok * QS + pc * EPP;
      if (WITH_Q) *reinterpret_cast<uint4*>(sq + o) = rq[j];
      *reinterpret_cast<uint4*>(sk + o) = rk[j];
      if constexpr (LA_T) {
        typedef typename Elt<T>::piece_t piece_t;
        const piece_t l = __builtin_bit_cast(piece_t, rl[j]);
#pragma unroll
        for (int u = 0; u < EPP; ++u) sla[(pc * EPP + u) * AS + tok] = l[u];
      } else {
        *reinterpret_cast<uint4*>(sla + o) = rl[j];
      }
    }
#pragma unroll
    for (int j = 0; j < NVP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PPT_V;
      const int pc = id - tp * PPT_V;
      typedef typename Elt<T>::piece_t piece_t;
      const piece_t a = __builtin_bit_cast(piece_t, rv[2 * j]);
      const piece_t b = __builtin_bit_cast(piece_t, rv[2 * j + 1]);
#pragma unroll
      for (int u = 0; u < EPP; ++u) {
        typedef T pair_t __attribute__((ext_vector_type(2)));
        pair_t pr;
        pr[0] = a[u];
        pr[1] = b[u];
        *reinterpret_cast<pair_t*>(svt + (pc * EPP + u) * AS + 2 * tp) = pr;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// d_k x d_v state held in MFMA accumulators.  Wave w owns value-column blocks
// cb = w + 4*j; tile (r, j) holds S[16r + 4g + u][16cb + n] in lane (g, n).
template <int DK, int DV>
struct StateRegs {
  static constexpr int NR = DK / 16;
  static constexpr int NC = DV / 64;
  f32x4 s[NR][NC];
};

// S <- diag(exp(b_last)) S + KL^T V for this wave's column blocks.
template <class T, int DK, int DV>
__device__ __forceinline__ void state_update(StateRegs<DK, DV>& st, const T* klt, const T* vt,
                                             const float* gch, int AS) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) {
    const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
    for (int r = 0; r < StateRegs<DK, DV>::NR; ++r) {
      f32x4 acc = st.s[r][j];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] *= gch[16 * r + 4 * g + u];
      const int dim = 16 * r + n16;
#pragma unroll
      for (int s0 = 0; s0 < kChunk; s0 += 4)
        acc = mma4(klt[dim * AS + s0 + g], vt[col * AS + s0 + g], acc);
      st.s[r][j] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: span summaries.  Runs the span's chunks from a zero state and
// writes the state reached and the product of the span's gates.
template <class T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void span_summary_kernel(FwdParams p) {
  using SM = SummarySmem<T, DK, DV>;
  __shared__ SM sm;
  constexpr int QS = SM::QS, AS = SM::AS;
  const int tid = threadIdx.x, lane = tid & 63;

  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const size_t off_k = (size_t)bh * p.T * DK;
  const size_t off_v = (size_t)bh * p.T * DV;
  const int c_begin = span * p.span_chunks;
  const int c_end = min(c_begin + p.span_chunks, p.n_chunks);

  const T* k = static_cast<const T*>(p.k);
  const T* la = static_cast<const T*>(p.la);
  const T* v = static_cast<const T*>(p.v);

  StateRegs<DK, DV> st;
#pragma unroll
  for (int r = 0; r < StateRegs<DK, DV>::NR; ++r)
#pragma unroll
    for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) st.s[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NI = DK / 64;  // (key dim, sub-block) items per thread
  float log_gate[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) log_gate[it] = 0.f;

  Loader<T, DK, DV> ld;
  {
    const int t0 = c_begin * kChunk;
    ld.template load<false>(nullptr, k, la, v, off_k, off_v, t0, min(kChunk, p.T - t0), gm);
  }
  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();  // previous chunk's MFMA reads of vt / klt are done
    ld.template store<false>(nullptr, sm.k, sm.la, sm.vt, QS, AS);
    if (c + 1 < c_end) {
      const int t0 = (c + 1) * kChunk;
      ld.template load<false>(nullptr, k, la, v, off_k, off_v, t0, min(kChunk, p.T - t0), gm);
    }
    __syncthreads();
    // Cumulative decay per (key dim, sub-block) and the decayed keys k_s*exp(b_last-b_s).
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int item = tid + kThreads * it;
      const int i = item >> 2, J = item & 3;
      float cs[kSub];
      float c_run = 0.f;
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
        c_run += (float)sm.la[(kSub * J + r) * QS + i];
        cs[r] = c_run;
      }
      const int base = lane & ~3;
      const float D0 = __shfl(c_run, base + 0, 64);
      const float D1 = __shfl(c_run, base + 1, 64);
      const float D2 = __shfl(c_run, base + 2, 64);
      const float D3 = __shfl(c_run, base + 3, 64);
      const float bst = (J > 0 ? D0 : 0.f) + (J > 1 ? D1 : 0.f) + (J > 2 ? D2 : 0.f);
      const float blast = D0 + D1 + D2 + D3;
      constexpr int EPP = Elt<T>::kPerPiece;
      typedef typename Elt<T>::piece_t piece_t;
#pragma unroll
      for (int r0 = 0; r0 < kSub; r0 += EPP) {
        piece_t w;
#pragma unroll
        for (int u = 0; u < EPP; ++u) {
          const float kv = (float)sm.k[(kSub * J + r0 + u) * QS + i];
          w[u] = (T)(kv * fexp<T>(blast - bst - cs[r0 + u]));
        }
        *reinterpret_cast<piece_t*>(sm.klt + i * AS + kSub * J + r0) = w;
      }
      if (J == 0) {
        sm.g[i] = fexp<T>(blast);
        log_gate[it] += blast;
      }
    }
    __syncthreads();
    state_update<T, DK, DV>(st, sm.klt, sm.vt, sm.g, AS);
  }

  // Write the span summary.
  const int wave = tid >> 6, n16 = lane & 15, g = lane >> 4;
  float* dst = p.span_state + ((size_t)bh * p.n_spans + span) * DK * DV;
#pragma unroll
  for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) {
    const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
    for (int r = 0; r < StateRegs<DK, DV>::NR; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u) dst[(16 * r + 4 * g + u) * DV + col] = st.s[r][j][u];
  }
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + kThreads * it;
    const int i = item >> 2, J = item & 3;
    if (J == 0)
      p.span_gate[((size_t)bh * p.n_spans + span) * DK + i] = fexp<T>(log_gate[it]);
  }
}

// ---------------------------------------------------------------------------
// Kernel 2 (float32 path; the float16 path runs scan16_body below): scan over
// spans, elementwise over the d_k x d_v state, turning each span summary
// (G_s, L_s) into the state entering span s:
//   E_0 = 0,  E_{s+1} = diag(G_s) E_s + L_s.
// The combine (G, L) o (G', L') = (G G', diag(G') L + L') is associative, so
// spans are taken in rounds of kScanSeg segments of U spans, one wave per
// segment: each lane loads its segment's summaries at once (one memory round
// trip), folds them from zero, the folds are exchanged through LDS to give
// every segment its carry-in, and the same registers then yield the entry
// states.  U is 16 when one round of 16 covers the sequence's spans (no lane
// then loads past them), else 32.
constexpr int kScanSeg = 4;
constexpr int kScanElems = kThreads / kScanSeg;   // state elements per workgroup

// One workgroup scans the state elements yb * kScanElems .. of sequence bh
// over n_spans summaries (state [BH][n_spans][DK][DV], gate [BH][n_spans][DK],
// initial state [BH][DK][DV] or null), in place.
template <int DK, int DV, int U>
__device__ __forceinline__ void span_scan_body(float* span_state, const float* span_gate,
                                               const float* initial_state, int n_spans, int bh,
                                               int yb) {
  __shared__ float seg_l[kScanSeg][kScanElems];
  __shared__ float seg_g[kScanSeg][kScanElems];
  const int seg = threadIdx.x / kScanElems;
  const int le = threadIdx.x - seg * kScanElems;
  const int e = yb * kScanElems + le;
  const int dim = e / DV;
  float* const L = span_state + (size_t)bh * n_spans * DK * DV + e;
  const float* const G = span_gate + (size_t)bh * n_spans * DK + dim;

  // state entering the current round; the first round starts from the
  // initial state, which the scan also writes as span 0's entry state
  float carry = initial_state ? initial_state[(size_t)bh * DK * DV + e] : 0.f;
  for (int r0 = 0; r0 < n_spans; r0 += kScanSeg * U) {
    const int s0 = r0 + seg * U;
    float l[U], gg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // slots past the last span re-read span 0 and are neutralised (no
      // branches around the loads, so all of them are in flight together)
      const bool in = s0 + u < n_spans;
      const int sp = in ? s0 + u : 0;
      const float lv = L[(size_t)sp * DK * DV];
      const float gv = G[(size_t)sp * DK];
      l[u] = in ? lv : 0.f;
      gg[u] = in ? gv : 1.f;
    }
    float fl = 0.f, fg = 1.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fl = gg[u] * fl + l[u];
      fg *= gg[u];
    }
    seg_l[seg][le] = fl;
    seg_g[seg][le] = fg;
    __syncthreads();
    float run = carry, next = carry;
    for (int j = 0; j < kScanSeg; ++j) {
      if (j < seg) run = seg_g[j][le] * run + seg_l[j][le];
      next = seg_g[j][le] * next + seg_l[j][le];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < n_spans) L[(size_t)(s0 + u) * DK * DV] = run;
      run = gg[u] * run + l[u];
    }
    carry = next;
    __syncthreads();  // the LDS folds are reused by the next round
  }
}

template <int DK, int DV, int U>
__global__ __launch_bounds__(kThreads) void span_scan_kernel(FwdParams p) {
  span_scan_body<DK, DV, U>(p.span_state, p.span_gate, p.initial_state, p.n_spans, blockIdx.x,
                            blockIdx.y);
}

// Scan over float16 summaries, in place: each slot's summary (the state
// reached from zero over the slot, with its float32 gate product) is replaced
// by the float16 state entering that slot.  The float16 forward's span scan
// and both scans of the backward pass (one chunk per slot) run on it.  The
// slots of a round are cut into kBScanSeg segments of U, one row of 16 lanes
// per segment, each lane taking 4 adjacent elements (a row reads 128
// contiguous bytes per slot), so a round spans 16 U slots; the segments'
// folds meet through LDS as in span_scan_body.  The caller's float32 states
// sit at bh * st_bh + i * st_row + j: `init` the state before the first slot
// (or null: zero), `final_out` (or null) receives the state after the last
// slot.
constexpr int kBScanSeg = 16;
constexpr int kBScanElems = 4 * kThreads / kBScanSeg;  // state elements per workgroup
template <int DK, int DV, int U>
__device__ __forceinline__ void scan16_body(f16* sum16, const float* gate, const float* init,
                                            int n_slots, int bh, int yb, size_t st_bh,
                                            unsigned int st_row, float* final_out) {
  static_assert(DV % 4 == 0 && kBScanElems <= DV, "a workgroup's elements share one state row");
  __shared__ f32x4 seg_l[kBScanSeg][kBScanElems / 4];
  __shared__ float seg_g[kBScanSeg][kBScanElems / 4];
  const int lg = threadIdx.x & 15;   // the lane's elements: 4 lg .. of the workgroup's
  const int seg = threadIdx.x >> 4;
  const int e = yb * kBScanElems + 4 * lg;
  const int dim = e / DV, col = e - dim * DV;
  // one sequence's slots as buffers (the host keeps them under 2^31 bytes):
  // slots at or past n_slots read as zero and their stores are dropped, so
  // every load is issued unconditionally
  const rsrc_t rl = seq_rsrc(sum16 + (size_t)bh * n_slots * DK * DV, (uint32_t)n_slots * DK * DV * 2);
  const rsrc_t rg = seq_rsrc(gate + (size_t)bh * n_slots * DK, (uint32_t)n_slots * DK * 4);
  const size_t io = (size_t)bh * st_bh + (size_t)dim * st_row + col;

  // (element by element: the forward's initial state need only be 4-byte
  // aligned)
  f32x4 carry = init ? f32x4{init[io], init[io + 1], init[io + 2], init[io + 3]}
                     : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n_slots; r0 += kBScanSeg * U) {
    const int s0 = r0 + seg * U;
    f32x4 l[U];
    float gg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t sl = (uint32_t)(s0 + u);
      const f16x4 lv = __builtin_bit_cast(
          f16x4, __builtin_amdgcn_raw_buffer_load_b64(rl, (sl * DK * DV + e) * 2u, 0, 0));
      const float gv = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rg, (sl * DK + dim) * 4u, 0, 0));
      l[u] = f32x4{(float)lv[0], (float)lv[1], (float)lv[2], (float)lv[3]};
      gg[u] = gv + (sl < (uint32_t)n_slots ? 0.f : 1.f);  // a slot past the end: gate 1
    }
    f32x4 fl = f32x4{0.f, 0.f, 0.f, 0.f};
    float fg = 1.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fl = gg[u] * fl + l[u];
      fg *= gg[u];
    }
    seg_l[seg][lg] = fl;
    seg_g[seg][lg] = fg;
    __syncthreads();
    f32x4 run = carry, next = carry;
    for (int j = 0; j < kBScanSeg; ++j) {
      const f32x4 lj = seg_l[j][lg];
      const float gj = seg_g[j][lg];
      if (j < seg) run = gj * run + lj;
      next = gj * next + lj;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t sl = (uint32_t)(s0 + u);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_f16(run)), rl,
                                            (sl * DK * DV + e) * 2u, 0, 0);
      run = gg[u] * run + l[u];
    }
    carry = next;
    __syncthreads();  // the LDS folds are reused by the next round
  }
  if (final_out && seg == 0) *reinterpret_cast<f32x4*>(final_out + io) = carry;
}

// The backward pass's two scans in one launch: blockIdx.y below half the grid
// scans the forward summaries (from the initial state), the rest the adjoint
// summaries (from the final-state gradient; the state after its last slot is
// the gradient of the state before the first step).
template <int DK, int DV, int U>
__global__ __launch_bounds__(kThreads) void bwd_state_scans_kernel(FwdParams p) {
  constexpr int kBlocks = DK * DV / kBScanElems;
  const bool adj = (int)blockIdx.y >= kBlocks;
  // the chunk kernel that follows hands out its chunks from this counter
  if (p.bwd_ticket != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    __hip_atomic_store(p.bwd_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  scan16_body<DK, DV, U>(static_cast<f16*>(adj ? p.adj_entry16 : p.span_entry16),
                          adj ? p.adj_gate : p.span_gate, adj ? p.adj_initial : p.initial_state,
                          adj ? p.adj_slots : p.n_spans, blockIdx.x,
                          adj ? blockIdx.y - kBlocks : blockIdx.y, p.st_bh, p.st_row,
                          adj ? p.adj_final : nullptr);
}

// The float16 forward's span scan: the summaries in span_entry16 become the
// entry states, from the initial state ([B*heads][d_k][d_v] float32).
template <int DK, int DV, int U>
__global__ __launch_bounds__(kThreads) void span_scan16_kernel(FwdParams p) {
  scan16_body<DK, DV, U>(static_cast<f16*>(p.span_entry16), p.span_gate, p.initial_state,
                         p.n_spans, blockIdx.x, blockIdx.y, (size_t)DK * DV, DV, nullptr);
}

// ---------------------------------------------------------------------------
// Kernel 3: outputs.  Replays the span's chunks from the span's entry state.
template <class T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void chunk_output_kernel(FwdParams p) {
  using SM = ChunkSmem<T, DK, DV>;
  __shared__ SM sm;
  constexpr int QS = SM::QS, AS = SM::AS, OS = SM::OS;
  constexpr int EPP = Elt<T>::kPerPiece;
  static_assert(std::is_same<T, float>::value, "the float16 output kernel is chunk_output_f16_kernel");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;

  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const size_t off_k = (size_t)bh * p.T * DK;
  const size_t off_v = (size_t)bh * p.T * DV;
  const int c_begin = span * p.span_chunks;
  const int c_end = min(c_begin + p.span_chunks, p.n_chunks);

  const T* q = static_cast<const T*>(p.q);
  const T* k = static_cast<const T*>(p.k);
  const T* la = static_cast<const T*>(p.la);
  const T* v = static_cast<const T*>(p.v);
  T* out = static_cast<T*>(p.out);

  // Entry state of the span.
  StateRegs<DK, DV> st;
  {
    const float* src =
        (p.n_spans > 1) ? p.span_state + ((size_t)bh * p.n_spans + span) * DK * DV
        : p.initial_state ? p.initial_state + (size_t)bh * DK * DV : nullptr;
#pragma unroll
    for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) {
      const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
      for (int r = 0; r < StateRegs<DK, DV>::NR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          st.s[r][j][u] = src ? src[(16 * r + 4 * g + u) * DV + col] : 0.f;
    }
  }

  constexpr int NI = DK / 64;
  // Sub-block tiles (I, J), J <= I, of the causal score matrix, spread over the
  // four waves (3, 3, 2, 2 tiles); one byte (I << 4 | J) per tile.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t tile_codes = (wave_u == 0) ? 0x313000u
                            : (wave_u == 1) ? 0x321110u
                            : (wave_u == 2) ? 0x2120u
                                            : 0x3322u;
  const int n_tiles = (wave_u < 2) ? 3 : 2;

  Loader<T, DK, DV> ld;
  {
    const int t0 = c_begin * kChunk;
    ld.template load<true>(q, k, la, v, off_k, off_v, t0, min(kChunk, p.T - t0), gm);
  }
  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * kChunk;
    const int valid = min(kChunk, p.T - t0);
    if (c > c_begin) __syncthreads();  // the previous chunk's rows are out of sm.o (= sm.k)
    ld.template store<true, true>(sm.q, sm.k, sm.klt, sm.vt, QS, AS);
    if (c + 1 < c_end) {
      const int t1 = t0 + kChunk;
      ld.template load<true>(q, k, la, v, off_k, off_v, t1, min(kChunk, p.T - t1), gm);
    }
    __syncthreads();

    // Phase P: cumulative decay per (key dim i, sub-block J); anchored q, k,
    // decayed keys for the state update, and the per-dim factor tables.
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int item = tid + kThreads * it;
      const int i = item >> 2, J = item & 3;
      float cs[kSub];
      float c_run = 0.f;
#pragma unroll
      for (int r = 0; r < kSub; ++r) {
        c_run += (float)sm.klt[i * AS + kSub * J + r];   // log-alpha^T
        cs[r] = c_run;
      }
      const int base = lane & ~3;
      float D[4];
      D[0] = __shfl(c_run, base + 0, 64);
      D[1] = __shfl(c_run, base + 1, 64);
      D[2] = __shfl(c_run, base + 2, 64);
      D[3] = __shfl(c_run, base + 3, 64);
      float bst[4];
      bst[0] = 0.f;
      bst[1] = D[0];
      bst[2] = D[0] + D[1];
      bst[3] = D[0] + D[1] + D[2];
      const float blast = bst[3] + D[3];
      const float my_bst = bst[J];
      const float fl = fexp<T>(blast - my_bst);
      typedef typename Elt<T>::piece_t piece_t;
#pragma unroll
      for (int r0 = 0; r0 < kSub; r0 += EPP) {
        piece_t w;
#pragma unroll
        for (int u = 0; u < EPP; ++u) {
          const int row = (kSub * J + r0 + u) * QS + i;
          const float eq = fexp<T>(cs[r0 + u]);
          const float ek = fexp<T>(-cs[r0 + u]);
          const float qv = (float)sm.q[row];
          const float kv = (float)sm.k[row];
          sm.q[row] = (T)(qv * eq);
          sm.k[row] = (T)(kv * ek);
          w[u] = (T)(kv * (ek * fl));
        }
        *reinterpret_cast<piece_t*>(sm.klt + i * AS + kSub * J + r0) = w;
      }
      sm.e[J * DK + i] = fexp<T>(my_bst);
#pragma unroll
      for (int I = 1; I < 4; ++I)
        if (I > J) sm.f[pair_index(I, J) * DK + i] = fexp<T>(bst[I] - my_bst);
      if (J == 0) sm.g[i] = fexp<T>(blast);
    }
    __syncthreads();

    // Phase A: A[t][s] for s <= t as transposed 16x16 tiles (rows s, cols t).
    T* sa = sm.sa;
    for (int ti = 0; ti < n_tiles; ++ti) {
      const int code = (tile_codes >> (8 * ti)) & 0xff;
      const int I = code >> 4, J = code & 0xf;
      const int s_row = kSub * J + n16;  // key token supplying the A operand
      const int t_row = kSub * I + n16;  // query token supplying the B operand
      const float* F = (J < I) ? sm.f + pair_index(I, J) * DK : nullptr;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int d0 = 0; d0 < DK; d0 += 4) {
        float a = sm.k[s_row * QS + d0 + g];
        if (F) a *= F[d0 + g];
        acc = mma4(a, sm.q[t_row * QS + d0 + g], acc);
      }
      // lane holds A^T[s = 16J + 4g + u][t = 16I + n16]
      if (I == J) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (4 * g + u > n16) acc[u] = 0.f;
      }
      typedef T quad_t __attribute__((ext_vector_type(4)));
      quad_t w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = (T)acc[u];
      *reinterpret_cast<quad_t*>(sa + t_row * AS + kSub * J + 4 * g) = w;
    }
    __syncthreads();

    // Phase O: O^T tiles (rows = value columns, cols = tokens) = V^T A^T + S^T (Q*exp(b))^T,
    // then the state update.
#pragma unroll
    for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) {
      const int col0 = 16 * (wave + 4 * j);
      const int col = col0 + n16;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int t = kSub * I + n16;
        const int len = kSub * (I + 1);
        const float* E = sm.e + I * DK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s0 = 0; s0 < len; s0 += 4)
          acc = mma4(sm.vt[col * AS + s0 + g], sa[t * AS + s0 + g], acc);
#pragma unroll
        for (int r = 0; r < DK / 16; ++r)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int d = 16 * r + 4 * g + u;
            acc = mma4(st.s[r][j][u], sm.q[t * QS + d] * E[d], acc);
          }
        // lane holds O^T[col0 + 4g + u][t]
        typedef T quad_t __attribute__((ext_vector_type(4)));
        quad_t w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (T)acc[u];
        *reinterpret_cast<quad_t*>(sm.o + t * OS + col0 + 4 * g) = w;
      }
    }
    state_update<T, DK, DV>(st, sm.klt, sm.vt, sm.g, AS);
    __syncthreads();

    // Phase W: output rows to their grid cells.
    constexpr int PPT_O = DV / EPP;
    constexpr int NO = kChunk * PPT_O / kThreads;
#pragma unroll
    for (int jj = 0; jj < NO; ++jj) {
      const int id = tid + kThreads * jj;
      const int tok = id / PPT_O;
      const int pc = id - tok * PPT_O;
      if (tok < valid) {
        const size_t o = off_v + (size_t)gm.cell(t0 + tok) * DV + pc * EPP;
        *reinterpret_cast<uint4*>(out + o) =
            *reinterpret_cast<const uint4*>(sm.o + tok * OS + pc * EPP);
      }
    }
  }

  if (span == p.n_spans - 1 && p.final_state != nullptr) {
    float* dst = p.final_state + (size_t)bh * DK * DV;
#pragma unroll
    for (int j = 0; j < StateRegs<DK, DV>::NC; ++j) {
      const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
      for (int r = 0; r < StateRegs<DK, DV>::NR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[(16 * r + 4 * g + u) * DV + col] = st.s[r][j][u];
    }
  }
}

// ===========================================================================
// Float16 kernels.  Chunk data moves from memory into LDS with buffer loads
// that write LDS directly (no registers, no staging code), row-major with a
// bank-spreading swizzle, and the operands that reduce over tokens are read
// back transposed (ds_read_b64_tr_b16).  The per-chunk elementwise work
// (cumulative decay, anchored q / k scalings, decayed keys) runs in MFMA
// register layouts:
//  * cumulative sums over tokens are 16x16x16 MFMAs against constant
//    triangular matrices, landing as "4 key dims of one token per lane"
//    (output kernel, log2(e) folded in as an exact hi + lo pair) or "4 tokens
//    of one key dim per lane" (summary);
//  * the decay over each 16-token sub-block is broadcast along each 16-lane
//    row with DPP, so the per-(dim, sub-block) factors need no exp and no LDS;
//  * keys are pre-scaled into the variants the causal score tiles need, so the
//    score MFMAs read unscaled operands.

// ---------------------------------------------------------------------------
// Output kernel, float16.  The span is walked in 32-token steps (two 16-token
// sub-blocks).  q, k, log-alpha and v of a step land row-major in LDS straight
// from memory (LDS-writing loads, two step buffers, the next step loading
// while this one is computed).  Per step:
//   P : wave w owns key dims 16w.. : cumulative decay c inside each sub-block
//       by MFMA (log-alpha read transposed), exp(+-c), DPP broadcast of the
//       sub-block decays; writes, in place of q, k, log-alpha, the anchored
//       q*exp(c), k*exp(-c) and the keys decayed to the step end, plus q
//       decayed from the step start; packed float16 products
//   O : wave w owns value columns 16w.. : the three causal score tiles in
//       transposed orientation (A^T, computed by every wave: cheaper than a
//       barrier), O^T = V^T A^T + S^T Qt^T with the score tiles used straight
//       from the accumulators, the outputs written over the wave's own value
//       columns of the step's v tile (out to their grid cells as whole rows
//       after the step's closing barrier), then S <- diag(exp(b_end)) S +
//       KL^T V.
// The x32 MFMAs that reduce over tokens use one token-slot order for both
// operands: slots 8g..8g+3 hold tokens 4g..4g+3 of sub-block 0 and slots
// 8g+4..8g+7 the same tokens of sub-block 1, which is what two transposed
// 16x16 reads (or two 16x16 accumulator tiles) deliver.
constexpr int kStep = 32;
// Cache policies of the output kernel's tile loads and output stores: both
// non-temporal.  The loads are the inputs' last use in the call; the outputs
// leave in whole 128-byte rows during the kernel, instead of lingering as
// dirty lines that drain while the next kernel streams its own inputs.
constexpr int kOutLoadAux = kAuxNT;
constexpr int kOutStoreAux = kAuxNT;
// log2 of the largest key factor exp(-c) the fast step path forms
constexpr float kKeyFactorLog2 = 10.f;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

// Column of key dim d (d % 4 == 0, four dims kept together) in token-slot
// order: within each 32-dim group, dims 4g..4g+3 and 16+4g..16+4g+3 sit side
// by side at 8g.., so one 128-bit read yields an x32 MFMA operand.
__device__ __forceinline__ int qt_slot(int d) {
  const int r = d & 31;
  return (d & ~31) + (r < 16 ? 2 * r : 2 * (r - 16) + 4);
}

template <int DK, int DV>
struct StepTiles {
  f16* q;
  f16* k;
  f16* la;
  f16* v;
};


// Load one state in the output layout: wave w owns value columns
// 16(w + 4j) .. ; tile (r, j) holds S[16r + 4g + u][16(w + 4j) + n] in lane
// (n, g).  src: [DK][DV] float32 row-major, or null (zero state).
template <int DK, int DV>
__device__ __forceinline__ void load_state_tiles(const float* src, int wave, int n16, int g,
                                                 f32x4 (&st)[DK / 16][DV / 64]) {
#pragma unroll
  for (int j = 0; j < DV / 64; ++j) {
    const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u) st[r][j][u] = src ? src[(16 * r + 4 * g + u) * DV + col] : 0.f;
  }
}

// The same from a float16 state (the three-pass scan's entry states).
template <int DK, int DV>
__device__ __forceinline__ void load_state_tiles16(const f16* src, int wave, int n16, int g,
                                                   f32x4 (&st)[DK / 16][DV / 64]) {
#pragma unroll
  for (int j = 0; j < DV / 64; ++j) {
    const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u) st[r][j][u] = (float)src[(16 * r + 4 * g + u) * DV + col];
  }
}

// The outputs of one span from its entry state `st` (output layout, see
// load_state_tiles) through two step buffers; `st` ends as the state after
// the span, written to final_state for the sequence's last span.  Returns
// with every load landed.
template <int DK, int DV, bool GATE, class Entry>
__device__ __forceinline__ void output_span(const FwdParams& p, int bh, int span,
                                            const StepTiles<DK, DV>& slot0,
                                            const StepTiles<DK, DV>& slot1, f16* sqt, float* sgd,
                                            uint32_t* sxf,
                                            f32x4 (&st)[DK / 16][DV / 64], Entry&& entry) {
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  constexpr int NR = DK / 16, NC = DV / 64, NRHO = DK / 32;
  constexpr int NBK = RBK / 128, NBV = RBV / 128;  // 1 KB blocks per wave and tile of one step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const SeqBufs sb = seq_bufs<DK, DV>(p, bh);
  const int t_begin = span * p.span_chunks * kChunk;
  const int t_end = min(t_begin + p.span_chunks * kChunk, p.T);
  const int n_steps = (t_end - t_begin + kStep - 1) / kStep;

  auto issue = [&](const StepTiles<DK, DV>& s, int step) {
    const int t0 = t_begin + kStep * step;
    const int valid = max(0, min(kStep, t_end - t0));
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = wave * NBK + i;
      const uint32_t off = dma_offset<RBK>(blk, t0, valid, gm);
      dma16p<kOutLoadAux>(sb.q, s.q + blk * 512, off);
      dma16p<kOutLoadAux>(sb.k, s.k + blk * 512, off);
      dma16p<kOutLoadAux>(sb.la, s.la + blk * 512, off);
      if (RBV == RBK) dma16p<kOutLoadAux>(sb.v, s.v + blk * 512, off);
    }
    if (RBV != RBK) {
#pragma unroll
      for (int i = 0; i < NBV; ++i) {
        const int blk = wave * NBV + i;
        dma16p<kOutLoadAux>(sb.v, s.v + blk * 512, dma_offset<RBV>(blk, t0, valid, gm));
      }
    }
  };
  // The outputs of step `step`, staged in place of its v tile (same swizzle),
  // out to their grid cells: each lane writes the 16 bytes at its own
  // position of the tile, i.e. the piece the swizzle put there, so 8 lanes
  // write one whole output row.  Rows past the span are dropped by the
  // buffer range check.  Returns once the tile has been read, so that the
  // buffer can take the next loads.
  auto flush = [&](const StepTiles<DK, DV>& s, int step) {
    const int t0 = t_begin + kStep * step;
    const int valid = max(0, min(kStep, t_end - t0));
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int blk = wave * NBV + i;
      const f16x8 x = ld128(s.v + blk * 512 + 8 * lane);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), sb.out,
                                             dma_offset<RBV>(blk, t0, valid, gm), 0, kOutStoreAux);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    asm volatile("" ::: "memory");
  };

  const f16x4 u_hi = upper_incl(kLog2eHi), u_lo = upper_incl(kLog2eLo);

  // ---- P: per-dim decays and the scaled operands of the step.  A step in
  // which some key factor exp(-c) would exceed 2^10, or some key reaches 32
  // in magnitude (its scaled copy could leave the float16 range), is marked
  // in *xf with `tag`; the O phase then computes it exactly (phase_x).
  auto phase_p = [&](const StepTiles<DK, DV>& s, int valid, uint32_t* xf, uint32_t tag) {
    bool bad = false;
    u16x4 kmax = {0, 0, 0, 0};
#pragma unroll
    for (int dbi = 0; dbi < DK / 64; ++dbi) {
      const int db = wave + 4 * dbi;
      const int dim0 = 16 * db + 4 * g;
      f16x4 lat4[2], q4[2], k4[2];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        lat4[I] = log_alpha_of<GATE>(tr_read<RBK>(s.la, 16 * I, 16 * db), p.inv_tau, 16 * I, valid);
        q4[I] = ld64(s.q + swz<RBK>(16 * I + n16, dim0));
        k4[I] = ld64(s.k + swz<RBK>(16 * I + n16, dim0));
      }
      // c2[I]: lane (t, g) holds log2-scaled cumulative decay of token
      // 16I + t at key dims dim0 .. dim0 + 3
      f32x4 c2[2], eq[2], ek[2], ed[2];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        c2[I] = mma16(lat4[I], u_hi, f32x4{0.f, 0.f, 0.f, 0.f});
        c2[I] = mma16(lat4[I], u_lo, c2[I]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          eq[I][u] = exp2_fast(c2[I][u]);
          ek[I][u] = exp2_fast(-c2[I][u]);
          ed[I][u] = row_bcast15(eq[I][u]);  // exp(decay over sub-block I)
          bad |= !(c2[I][u] >= -kKeyFactorLog2);
        }
        kmax = __builtin_elementwise_max(kmax, __builtin_bit_cast(u16x4, k4[I]) & (unsigned short)0x7fff);
      }
      if (n16 == 0) *reinterpret_cast<f32x4*>(sgd + dim0) = ed[0] * ed[1];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int row = 16 * I + n16;
        const f16x4 ql = q4[I] * to_f16(eq[I]);
        const f16x4 qt = (I == 0) ? ql : q4[I] * to_f16(eq[I] * ed[0]);
        const f16x4 kd = k4[I] * to_f16(ek[I]);
        const f16x4 kend = kd * to_f16(ed[I]);  // decayed to the end of sub-block I
        st64(s.q + swz<RBK>(row, dim0), ql);
        st64(sqt + swz<RBK>(row, qt_slot(dim0)), qt);
        st64(s.k + swz<RBK>(row, dim0), kd);
        st64(s.la + swz<RBK>(row, dim0), (I == 0) ? kend * to_f16(ed[1]) : kend);
      }
    }
    // |k| >= 32 (binary16 0x5000 and above, NaN included)
    const u16x4 km = __builtin_elementwise_max(kmax, kmax.wzyx);
    bad |= km[0] >= 0x5000 || km[1] >= 0x5000;
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) *xf = tag;
  };

  // ---- exact step: the recurrence token by token in float32, on this
  // wave's state columns, from the raw q, k and log-alpha (loaded again: the
  // P phase overwrote them; v is untouched)
  auto phase_x = [&](const StepTiles<DK, DV>& s, int step) {
    const int t0 = t_begin + kStep * step;
    const int valid = max(0, min(kStep, t_end - t0));
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = wave * NBK + i;
      const uint32_t off = dma_offset<RBK>(blk, t0, valid, gm);
      dma16(sb.q, s.q + blk * 512, off);
      dma16(sb.k, s.k + blk * 512, off);
      dma16(sb.la, s.la + blk * 512, off);
    }
    wait_barrier<vmcnt_imm(0)>();
    for (int t = 0; t < valid; ++t) {
      float vf[NC], part[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        vf[j] = (float)s.v[swz<RBV>(t, 16 * (wave + 4 * j) + n16)];
        part[j] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const f16x4 la4 = ld64(s.la + swz<RBK>(t, 16 * r + 4 * g));
        const f16x4 k4 = ld64(s.k + swz<RBK>(t, 16 * r + 4 * g));
        const f16x4 q4 = ld64(s.q + swz<RBK>(t, 16 * r + 4 * g));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float la = GATE ? logsigmoid_scaled((float)la4[u], p.inv_tau) : (float)la4[u];
          const float al = exp2_fast(la * 1.4426950408889634f);
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            st[r][j][u] = al * st[r][j][u] + (float)k4[u] * vf[j];
            part[j] += (float)q4[u] * st[r][j][u];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        float o = part[j] + __shfl_xor(part[j], 16);
        o += __shfl_xor(o, 32);
        if (g == 0) s.v[swz<RBV>(t, 16 * (wave + 4 * j) + n16)] = (f16)o;
      }
    }
  };

  // ---- O: scores, outputs, state update
  auto phase_o = [&](const StepTiles<DK, DV>& s, const uint32_t* xf, uint32_t tag, int step) {
    if (__builtin_amdgcn_readfirstlane(*xf) == tag) {
      phase_x(s, step);
      return;
    }
    // A^T tiles: lane (t, g) holds A[t][s = 4g + u] of the tile
    f32x4 d00 = {0.f, 0.f, 0.f, 0.f}, d01 = d00, d11 = d00;
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho) {
      const int col = 32 * rho + 8 * g;
      // tile (s in 0, t in 1): exp(b_t - b_s) splits into q_t exp(b_t) (Qt)
      // and k_s exp(-c_s) (Kd), since b = c inside sub-block 0
      const f16x8 kd0 = ld128(s.k + swz<RBK>(n16, col));
      const f16x8 kd1 = ld128(s.k + swz<RBK>(16 + n16, col));
      const f16x8 qa = ld128(s.q + swz<RBK>(n16, col));
      const f16x8 qb = ld128(s.q + swz<RBK>(16 + n16, col));
      // Qt columns are in token-slot order: gather the natural dims col..col+7
      const f16x8 qt1 = cat8(ld64(sqt + swz<RBK>(16 + n16, qt_slot(col))),
                             ld64(sqt + swz<RBK>(16 + n16, qt_slot(col + 4))));
      d00 = mma32(kd0, qa, d00);
      d01 = mma32(kd0, qt1, d01);
      d11 = mma32(kd1, qb, d11);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (4 * g + u > n16) {
        d00[u] = 0.f;
        d11[u] = 0.f;
      }
    const f16x4 z4 = {(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
    f16x8 sbt[2];
    sbt[0] = cat8(to_f16(d00), z4);
    sbt[1] = cat8(to_f16(d01), to_f16(d11));
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col0 = 16 * (wave + 4 * j);
      const f16x8 va = cat8(tr_read<RBV>(s.v, 0, col0), tr_read<RBV>(s.v, 16, col0));
      f16x8 sh[NRHO];
#pragma unroll
      for (int rho = 0; rho < NRHO; ++rho) sh[rho] = cat8(to_f16(st[2 * rho][j]), to_f16(st[2 * rho + 1][j]));
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int row = 16 * T + n16;
        f32x4 acc = mma32(va, sbt[T], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int rho = 0; rho < NRHO; ++rho)
          acc = mma32(sh[rho], ld128(sqt + swz<RBK>(row, 32 * rho + 8 * g)), acc);
        st64(s.v + swz<RBV>(row, col0 + 4 * g), to_f16(acc));
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const f16x8 kar = cat8(tr_read<RBK>(s.la, 0, 16 * r), tr_read<RBK>(s.la, 16, 16 * r));
        const f32x4 gv = *reinterpret_cast<const f32x4*>(sgd + 16 * r + 4 * g);
        st[r][j] = mma32(kar, va, st[r][j] * gv);
      }
    }
  };

  // rows of step `step` inside the span
  auto valid_rows = [&](int step) { return max(0, min(kStep, t_end - t_begin - kStep * step)); };
  // steps alternate between the two buffers; a step's exactness mark is its
  // index + 1 in its buffer's word (0 when the kernel starts)
  // A step's outputs replace its v tile (each wave's value columns of v are
  // in its registers by then, and no other wave reads them); they go out
  // after the barrier that ends the step, before the buffer is refilled.
  auto run_step = [&](const StepTiles<DK, DV>& s, int step) {
    prio_by_progress(step, n_steps);
    uint32_t* xf = sxf + (step & 1);
    phase_p(s, valid_rows(step), xf, (uint32_t)step + 1u);
    wait_barrier<kLgkmZero>();
    phase_o(s, xf, (uint32_t)step + 1u, step);
  };
  // Before step s the vector-memory operations in flight are the output
  // stores of step s - 2 and then the loads of step s; after it, those of
  // step s + 1 are the youngest, so the wait for them takes all.
  issue(slot0, 0);
  entry(st);                     // completes the entry state while step 0 loads
  wait_barrier<vmcnt_imm(0)>();  // the entry state and step 0 have landed
  for (int step = 0; step < n_steps; step += 2) {
    issue(slot1, step + 1);
    run_step(slot0, step);
    if (step + 1 >= n_steps) break;
    wait_barrier<vmcnt_lgkm0_imm(0)>();  // step + 1 landed; step's outputs staged
    flush(slot0, step);
    issue(slot0, step + 2);
    run_step(slot1, step + 1);
    if (step + 2 >= n_steps) break;
    wait_barrier<vmcnt_lgkm0_imm(0)>();
    flush(slot1, step + 1);
  }
  // the last step's outputs, staged by every wave
  wait_barrier<kLgkmZero>();
  flush((n_steps - 1) & 1 ? slot1 : slot0, n_steps - 1);
  // loads past the span's end (zero fills) must land before the workgroup's
  // LDS can be handed on
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  if (span == p.n_spans - 1 && p.final_state != nullptr) {
    // the lane index is recomputed here (mbcnt) and passed through an empty
    // asm, so the compiler forms these addresses here rather than holding
    // them across the loop
    int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    float* dst = p.final_state + (size_t)bh * DK * DV;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col = 16 * (wave + 4 * j) + (l & 15);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[(16 * r + 4 * (l >> 4) + u) * DV + col] = st[r][j][u];
    }
  }
}

// LOOKBACK (d_k = d_v = 64): the entry state is not read from span_state but
// formed here from the initial state and the summaries of the earlier spans
// of the sequence, stored by span_summary_f16_kernel<..., true> in this
// kernel's register layout as float16: S_entry = g_{s-1} (... (g_0 S_init +
// A_0) ...) + A_{s-1}, the scan's recurrence in float32, with four summaries'
// loads in flight at a time, overlapping the first step's tile loads.
template <int DK, int DV, bool GATE, bool LOOKBACK = false>
__global__ __launch_bounds__(kThreads, LOOKBACK ? 2 : (DK == 64 && DV == 64) ? 4 : (DK == 128 && DV == 128) ? 1 : 2) void chunk_output_f16_kernel(
    FwdParams p) {
  static_assert(!LOOKBACK || (DK == 64 && DV == 64), "look-back: d_k = d_v = 64");
  // Two step buffers (the next step loads while this one is computed; a
  // third buffer measured slower).  Separate LDS objects per buffer, so the
  // compiler's own waits for the LDS-writing loads can tell them apart.
  __shared__ __attribute__((aligned(16))) f16 q0[kStep * DK], k0[kStep * DK], la0[kStep * DK], v0[kStep * DV];
  __shared__ __attribute__((aligned(16))) f16 q1[kStep * DK], k1[kStep * DK], la1[kStep * DK], v1[kStep * DV];
  // q decayed from the step start, columns in token-slot order (see qt_slot)
  __shared__ __attribute__((aligned(16))) f16 sqt[kStep * DK];
  __shared__ __attribute__((aligned(16))) float sgd[DK];  // exp(decay over the step)
  // exactness mark of the step in each buffer (see output_span)
  __shared__ uint32_t sxf[2];
  if (threadIdx.x < 2) sxf[threadIdx.x] = 0u;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  f32x4 st[DK / 16][DV / 64];
  const StepTiles<DK, DV> slot0{q0, k0, la0, v0}, slot1{q1, k1, la1, v1};
  if constexpr (!LOOKBACK) {
    // the scan's entry states come as float16 (they enter the products as
    // float16 operands anyway; the state update runs on from them in float32)
    if (p.n_spans > 1)
      load_state_tiles16<DK, DV>(
          static_cast<const f16*>(p.span_entry16) + ((size_t)bh * p.n_spans + span) * DK * DV,
          wave, lane & 15, lane >> 4, st);
    else
      load_state_tiles<DK, DV>(p.initial_state ? p.initial_state + (size_t)bh * DK * DV : nullptr,
                               wave, lane & 15, lane >> 4, st);
    output_span<DK, DV, GATE>(p, bh, span, slot0, slot1, sqt, sgd, sxf, st, [](auto&) {});
  } else {
    const int g = lane >> 4;
    load_state_tiles<DK, DV>(p.initial_state ? p.initial_state + (size_t)bh * DK * DV : nullptr,
                             wave, lane & 15, g, st);
    auto fold_earlier = [&](f32x4 (&s)[DK / 16][DV / 64]) {
      const f16* A = reinterpret_cast<const f16*>(p.span_state) + (size_t)bh * p.n_spans * DK * DV +
                     ((size_t)wave * 4 * 64 + lane) * 4;
      const float* G = p.span_gate + (size_t)bh * p.n_spans * DK + 4 * g;
      constexpr int NB = 4;  // summaries in flight
      for (int j0 = 0; j0 < span; j0 += NB) {
        f32x4 av[NB][DK / 16], gv[NB][DK / 16];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int j = min(j0 + i, span - 1);
#pragma unroll
          for (int r = 0; r < DK / 16; ++r) {
            av[i][r] = __builtin_convertvector(ld64(A + (size_t)j * DK * DV + r * 256), f32x4);
            gv[i][r] = *reinterpret_cast<const f32x4*>(G + (size_t)j * DK + 16 * r);
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (j0 + i < span)
#pragma unroll
            for (int r = 0; r < DK / 16; ++r) s[r][0] = gv[i][r] * s[r][0] + av[i][r];
      }
    };
    output_span<DK, DV, GATE>(p, bh, span, slot0, slot1, sqt, sgd, sxf, st, fold_earlier);
  }
}

// ---------------------------------------------------------------------------
// Span-summary kernel, float16.  One workgroup per (batch*head, span) folds
// the span's chunks into (prod alpha, state reached from zero).  Chunks are
// taken last to first, so each key is scaled by its whole decay to the span
// end up front (k_t * exp(sum of log-alpha after t)) and the state is never
// rescaled: S^T += V^T Kl over the span.
//
// Wave w owns key dims 16 db .. (db = w, w + 4): S^T tile cb sits in lane
// (n, g) as S^T[16 cb + 4g + u][16 db + n].  Per chunk and key block:
//   - log-alpha and k arrive transposed from the tiles (lane (n, g): tokens
//     4g..4g+3 of dim n in each 16-token sub-block J);
//   - G, the decay from the chunk end to the span end, runs through an MFMA
//     chain: rest_J = U . la_J + G_J (U strictly upper triangular: the decay
//     after token t inside sub-block J) and G_{J-1} = 1 . la_J + G_J;
//   - Kl_J = k_J * exp(rest_J) in packed float16;
//   - S^T += V^T Kl as 16x16x32 MFMAs over sub-block pairs: the 32 token slots
//     of lane group g hold tokens 4g.. of the first sub-block, then of the
//     second, for both operands.
template <int DK, int DV>
struct SumTile {
  f16* k;
  f16* la;
  f16* v;
};

// One chunk's part of a span summary, for the wave's key blocks (tiles in
// LDS; `valid` tokens of the chunk are real).  Chunks are folded last to
// first.
//   ADJ false: the forward summary.  gdec holds the decay from this chunk's
//     end to the span's end; keys are decayed to the span end and
//     S^T += V^T Kl.
//   ADJ true: the adjoint summary, with q in place of k and the output
//     gradient in place of v: dR = (Q * exp(B))^T dO, B the decay from the
//     span start through each token (inclusive).  Each chunk is taken from
//     its own start, and the summary of the later chunks, already folded, is
//     decayed by this chunk's total before this chunk adds in; gdec then
//     holds the decay of the chunks folded so far.
template <int DK, int DV, bool GATE, bool ADJ>
__device__ __forceinline__ void fold_chunk(const SumTile<DK, DV>& s, int valid, float inv_tau,
                                           f16x4 m_tri, f16x4 m_ones, int wave,
                                           f32x4 (&st)[DK / 64][DV / 16],
                                           f32x4 (&gdec)[DK / 64]) {
  constexpr int NDB = DK / 64, NCB = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int db = wave + 4 * d;
    f16x4 lat[4], kt[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      lat[J] = log_alpha_of<GATE>(tr_read<RBK>(s.la, 16 * J, 16 * db), inv_tau, 16 * J, valid);
      kt[J] = tr_read<RBK>(s.k, 16 * J, 16 * db);
    }
    f32x4 rest[4];
    f32x4 c = gdec[d];
    if constexpr (ADJ) {
      f32x4 cl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        rest[J] = mma16(m_tri, lat[J], cl);
        cl = mma16(m_ones, lat[J], cl);
      }
      const float whole = exp2_fast(cl[0] * 1.4426950408889634f);  // key dim 16 db + n
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) st[d][cb] *= whole;
      c = c + cl;
    } else {
#pragma unroll
      for (int J = 3; J >= 0; --J) {
        rest[J] = mma16(m_tri, lat[J], c);
        c = mma16(m_ones, lat[J], c);
      }
    }
    gdec[d] = c;
    f16x4 kl[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 e;
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = exp2_fast(rest[J][u] * 1.4426950408889634f);
      kl[J] = kt[J] * __builtin_convertvector(e, f16x4);
    }
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const f16x8 bk = cat8(kl[2 * P], kl[2 * P + 1]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f16x8 av = cat8(tr_read<RBV>(s.v, 32 * P, 16 * cb), tr_read<RBV>(s.v, 32 * P + 16, 16 * cb));
        st[d][cb] = mma32(av, bk, st[d][cb]);
      }
    }
  }
}

// A operands of the decay chains: strictly upper triangular (s > t) for the
// forward summary, lower triangular inclusive (s <= t) for the adjoint one,
// and all ones.
template <bool ADJ>
__device__ __forceinline__ f16x4 tri_operand(int n16, int g) {
  f16x4 m;
#pragma unroll
  for (int u = 0; u < 4; ++u) m[u] = (f16)((ADJ ? (4 * g + u <= n16) : (4 * g + u > n16)) ? 1.f : 0.f);
  return m;
}

// Writes one summary to `slot` of the sequence's `slots`: the state rows of
// the wave's key blocks rounded to float16, the gate product in float32.
template <int DK, int DV>
__device__ __forceinline__ void store_summary16(f16* state16, float* span_gate, int bh,
                                                size_t slots, size_t slot, int wave, int n16, int g,
                                                const f32x4 (&st)[DK / 64][DV / 16],
                                                const f32x4 (&gdec)[DK / 64]) {
  f16* dst = state16 + ((size_t)bh * slots + slot) * DK * DV;
#pragma unroll
  for (int d = 0; d < DK / 64; ++d) {
    const int dim = 16 * (wave + 4 * d) + n16;
#pragma unroll
    for (int cb = 0; cb < DV / 16; ++cb)
      *reinterpret_cast<f16x4*>(dst + dim * DV + 16 * cb + 4 * g) = to_f16(st[d][cb]);
    if (g == 0)
      span_gate[((size_t)bh * slots + slot) * DK + dim] = exp2_fast(gdec[d][0] * 1.4426950408889634f);
  }
}

// The span's summary (st, gdec as in fold_chunk, from zero) through the two
// tile buffers; returns with every load landed, the buffers still being read
// by other waves (a barrier must come before they are refilled).
template <int DK, int DV, bool GATE>
__device__ __forceinline__ void summarize_span(const FwdParams& p, int bh, int span,
                                               const SumTile<DK, DV>& slot0,
                                               const SumTile<DK, DV>& slot1,
                                               f32x4 (&st)[DK / 64][DV / 16],
                                               f32x4 (&gdec)[DK / 64]) {
  constexpr int NDB = DK / 64, NCB = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  constexpr int NBK = RBK / 64, NBV = RBV / 64;  // 1 KB blocks per wave and tile
  constexpr int NDMA = 2 * NBK + NBV;             // LDS-writing loads per wave and chunk
  static_assert(NDMA < 64, "vmcnt range");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const SeqBufs sb = seq_bufs<DK, DV>(p, bh);
  const int c_begin = span * p.span_chunks;
  const int c_end = min(c_begin + p.span_chunks, p.n_chunks);

  // Fill a tile buffer with chunk c; a chunk before the span loads nothing.
  auto issue = [&](const SumTile<DK, DV>& s, int c) {
    const int t0 = c * kChunk;
    const int valid = c >= c_begin ? min(kChunk, p.T - t0) : 0;
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = wave * NBK + i;
      const uint32_t off = dma_offset<RBK>(blk, t0, valid, gm);
      dma16(sb.k, s.k + blk * 512, off);
      dma16(sb.la, s.la + blk * 512, off);
      if (RBV == RBK) dma16(sb.v, s.v + blk * 512, off);
    }
    if (RBV != RBK) {
#pragma unroll
      for (int i = 0; i < NBV; ++i) {
        const int blk = wave * NBV + i;
        dma16(sb.v, s.v + blk * 512, dma_offset<RBV>(blk, t0, valid, gm));
      }
    }
  };

  const f16x4 m_upper = tri_operand<false>(n16, g);
  const f16x4 m_ones = f16x4{(f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f};

  // gdec: decay (log) from the current chunk's end to the span end, per key dim
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    gdec[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st[d][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto fold = [&](const SumTile<DK, DV>& s, int c) {
    fold_chunk<DK, DV, GATE, false>(s, min(kChunk, p.T - c * kChunk), p.inv_tau, m_upper, m_ones,
                                    wave, st, gdec);
  };

  issue(slot0, c_end - 1);
  issue(slot1, c_end - 2);
  for (int c = c_end - 1; c >= c_begin; c -= 2) {
    prio_by_progress(c_end - 1 - c, c_end - c_begin);
    wait_barrier<vmcnt_imm(NDMA)>();  // every wave's part of slot0 has landed
    fold(slot0, c);
    wait_barrier<kLgkmZero>();        // every wave's reads of slot0 are done
    issue(slot0, c - 2);
    wait_barrier<vmcnt_imm(NDMA)>();
    if (c - 1 >= c_begin) fold(slot1, c - 1);
    wait_barrier<kLgkmZero>();
    issue(slot1, c - 3);
  }
  // the trailing loads target chunks before the span (zero fills): let them
  // land before the workgroup's LDS can be handed on
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// One summary stored where chunk_output_f16_kernel<..., true> reads it
// (d_k = d_v = 64): lane (n, g) of wave w holds S[16 w + n][16 cb + 4g + u];
// in the output kernel's layout that element belongs to wave cb, row block
// r = w, lane (4g + u) + 16 (n / 4), component n % 4, and the summary is
// [wave][r][lane][4] float16 values, so each reader lane loads 8-byte pieces
// (float16 halves the look-back's reads; the fold itself runs in float32).
// Each wave's four 1 KB blocks of floats go through its own 4 KB of LDS
// (`stage`, free once the workgroup is past the barrier before this call)
// and out as 8-byte stores.
template <int DK, int DV>
__device__ __forceinline__ void store_summary_out_layout(const FwdParams& p, int bh, int span,
                                                         int wave, int lane, float* stage,
                                                         const f32x4 (&st)[DK / 64][DV / 16],
                                                         const f32x4 (&gdec)[DK / 64]) {
  static_assert(DK == 64 && DV == 64, "output layout: d_k = d_v = 64");
  const int n16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < DV / 16; ++cb)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      stage[cb * 256 + (4 * g + u + 16 * (n16 >> 2)) * 4 + (n16 & 3)] = st[0][cb][u];
  f16* dst = reinterpret_cast<f16*>(p.span_state) + ((size_t)bh * p.n_spans + span) * DK * DV;
#pragma unroll
  for (int cb = 0; cb < DV / 16; ++cb)
    st64(dst + (cb * 4 + wave) * 256 + 4 * lane,
         to_f16(*reinterpret_cast<const f32x4*>(stage + cb * 256 + 4 * lane)));
  if (g == 0)
    p.span_gate[((size_t)bh * p.n_spans + span) * DK + 16 * wave + n16] =
        exp2_fast(gdec[0][0] * 1.4426950408889634f);
}

// OUT_LAYOUT: store the summary for the two-pass path's output kernel
// (store_summary_out_layout) instead of row-major for the scan.
template <int DK, int DV, bool GATE, bool OUT_LAYOUT = false>
__global__ __launch_bounds__(kThreads) void span_summary_f16_kernel(FwdParams p) {
  // six separate LDS objects, so the compiler's own waits for the LDS-writing
  // loads can tell the tiles apart
  __shared__ __attribute__((aligned(16))) f16 k0[kChunk * DK], la0[kChunk * DK], v0[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 k1[kChunk * DK], la1[kChunk * DK], v1[kChunk * DV];
  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  f32x4 st[DK / 64][DV / 16];
  f32x4 gdec[DK / 64];
  summarize_span<DK, DV, GATE>(p, bh, span, SumTile<DK, DV>{k0, la0, v0},
                               SumTile<DK, DV>{k1, la1, v1}, st, gdec);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (OUT_LAYOUT) {
    __syncthreads();  // every wave is done reading the tiles
    store_summary_out_layout<DK, DV>(p, bh, span, wave, lane,
                                     reinterpret_cast<float*>(wave < 2 ? k0 : la0) + (wave & 1) * 1024,
                                     st, gdec);
  } else
    store_summary16<DK, DV>(static_cast<f16*>(p.span_entry16), p.span_gate, bh, p.n_spans, span,
                            wave, lane & 15, lane >> 4, st, gdec);
}

// The backward pass's two kinds of summary: the forward one (k, v; the state
// entering each span, a span being a pair of chunks) and the adjoint one (q
// and the output gradient d_out; the state gradient entering each chunk from
// its right), sharing the log-alpha tile, stored as float16 (span_entry16,
// adj_entry16) with float32 gate products.  Chunk c's adjoint summary goes to
// slot adj_slots - 1 - c, so that the adjoint scan runs from the end of the
// sequence to its start.  float16, no fused gate activation.
//
// A workgroup takes spans_per_wg consecutive spans (of the flattened
// (batch*head, span) order) and streams their chunks through two tile
// buffers, so that the loads of one chunk overlap the folds of the previous
// one; a span's chunks are taken last to first, its forward summary stored
// when its first chunk (folded last) is done, each chunk's adjoint summary
// when that chunk is.  Eight waves: four fold the forward summary and four the adjoint one
// from the same tiles, so a SIMD has two waves to switch between even at one
// workgroup per CU.
constexpr int kSumThreads = 512;  // 8 waves: 4 fold the forward summary, 4 the adjoint
template <int DK, int DV>
__global__ __launch_bounds__(kSumThreads) void bwd_state_summaries_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) f16 k0[kChunk * DK], la0[kChunk * DK], v0[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 q0[kChunk * DK], do0[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 k1[kChunk * DK], la1[kChunk * DK], v1[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 q1[kChunk * DK], do1[kChunk * DV];
  const SumTile<DK, DV> fw0{k0, la0, v0}, fw1{k1, la1, v1};
  const SumTile<DK, DV> ad0{q0, la0, do0}, ad1{q1, la1, do1};
  constexpr int NDB = DK / 64, NCB = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  static_assert(RBK == 128 && RBV == 128, "built for 64 key and value dims");
  constexpr int NDMA = 5;  // LDS-writing loads per wave and chunk: one 1 KB block of each tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  // waves 0..3 fold the forward summary, 4..7 the adjoint one, each over key
  // block wq; all eight load the tiles
  const int fam = wave >> 2, wq = wave & 3;

  const int sc = p.span_chunks;
  const long long total = (long long)p.B * p.heads * p.n_spans;
  const long long s_begin = (long long)blockIdx.x * p.spans_per_wg;
  const long long s_end = s_begin + p.spans_per_wg < total ? s_begin + p.spans_per_wg : total;
  const int n_items = (int)(s_end - s_begin) * sc;

  // item i: chunk sc - 1 - i % sc of span s_begin + i / sc (chunks of a span
  // last to first); an item past the end or past its sequence is empty
  struct Item {
    int bh, span, c;
    bool live;
  };
  auto item = [&](int i) {
    Item it;
    const long long gs = s_begin + i / sc;
    it.bh = (int)(gs / p.n_spans);
    it.span = (int)(gs - (long long)it.bh * p.n_spans);
    it.c = it.span * sc + (sc - 1 - i % sc);
    it.live = i < n_items && it.c < p.n_chunks;
    return it;
  };
  auto issue = [&](const SumTile<DK, DV>& f, const SumTile<DK, DV>& a, int i) {
    const Item it = item(i < n_items ? i : 0);
    const bool live = i < n_items && it.live;
    const GridMap gm = grid_map(p, it.bh / p.heads);
    // rows of ldk / ldv elements (a 64-dim block of a wider head)
    typedef _Float16 h;
    const size_t ok = (size_t)it.bh * p.T * p.ldk, ov = (size_t)it.bh * p.T * p.ldv;
    const uint32_t kbytes = (uint32_t)p.T * p.ldk * 2u, vbytes = (uint32_t)p.T * p.ldv * 2u;
    const rsrc_t rk = seq_rsrc(static_cast<const h*>(p.k) + ok, kbytes);
    const rsrc_t rla = seq_rsrc(static_cast<const h*>(p.la) + ok, kbytes);
    const rsrc_t rq = seq_rsrc(static_cast<const h*>(p.q) + ok, kbytes);
    const rsrc_t rv = seq_rsrc(static_cast<const h*>(p.v) + ov, vbytes);
    const rsrc_t rdo = seq_rsrc(static_cast<const h*>(p.dout) + ov, vbytes);
    const int t0 = it.c * kChunk;
    const int valid = live ? min(kChunk, p.T - t0) : 0;
    const int blk = wave;
    const uint32_t offk = dma_offset_s<RBK>(blk, t0, valid, gm, p.ldk * 2u);
    const uint32_t offv = dma_offset_s<RBV>(blk, t0, valid, gm, p.ldv * 2u);
    dma16(rk, f.k + blk * 512, offk);
    dma16(rla, f.la + blk * 512, offk);
    dma16(rv, f.v + blk * 512, offv);
    dma16(rq, a.k + blk * 512, offk);
    dma16(rdo, a.v + blk * 512, offv);
  };

  const f16x4 m_tri = fam == 0 ? tri_operand<false>(n16, g) : tri_operand<true>(n16, g);
  const f16x4 m_ones = f16x4{(f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f};
  f32x4 st[NDB][NCB], gdec[NDB];   // this wave's summary (forward or adjoint)
  auto reset = [&]() {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      gdec[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) st[d][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset();
  const size_t slots = p.adj_slots;
  // fold item i from the given buffers; after a span's first chunk, store
  // its summaries and start the next span from zero
  auto step = [&](const SumTile<DK, DV>& f, const SumTile<DK, DV>& a, int i) {
    const Item it = item(i);
    if (it.live) {
      const int valid = min(kChunk, p.T - it.c * kChunk);
      if (fam == 0)
        fold_chunk<DK, DV, false, false>(f, valid, 1.f, m_tri, m_ones, wq, st, gdec);
      else
        fold_chunk<DK, DV, false, true>(a, valid, 1.f, m_tri, m_ones, wq, st, gdec);
    }
    if (fam == 0) {
      if (i % sc == sc - 1) {
        store_summary16<DK, DV>(static_cast<f16*>(p.span_entry16), p.span_gate, it.bh, p.n_spans,
                                it.span, wq, n16, g, st, gdec);
        reset();
      }
    } else if (it.live) {
      store_summary16<DK, DV>(static_cast<f16*>(p.adj_entry16), p.adj_gate, it.bh, slots,
                              slots - 1 - it.c, wq, n16, g, st, gdec);
      reset();
    }
  };

  issue(fw0, ad0, 0);
  issue(fw1, ad1, 1);
  for (int i = 0; i < n_items; i += 2) {
    wait_barrier<vmcnt_imm(NDMA)>();  // every wave's part of buffer 0 has landed
    step(fw0, ad0, i);
    wait_barrier<kLgkmZero>();        // every wave's reads of buffer 0 are done
    issue(fw0, ad0, i + 2);
    wait_barrier<vmcnt_imm(NDMA)>();
    if (i + 1 < n_items) step(fw1, ad1, i + 1);
    wait_barrier<kLgkmZero>();
    issue(fw1, ad1, i + 3);
  }
  // the trailing loads are zero fills: let them land before the workgroup's
  // LDS can be handed on
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Kernel choice per element type: float16 runs the MFMA-layout kernels,
// float32 the generic ones.
template <class T, int DK, int DV, bool GATE>
struct Family {
  static_assert(!GATE, "the fused gate activation is built for float16 only");
  static constexpr auto summary = span_summary_kernel<T, DK, DV>;
  static constexpr auto output = chunk_output_kernel<T, DK, DV>;
};
template <int DK, int DV, bool GATE>
struct Family<f16, DK, DV, GATE> {
  static constexpr auto summary = span_summary_f16_kernel<DK, DV, GATE>;
  static constexpr auto output = chunk_output_f16_kernel<DK, DV, GATE>;
};

// Launch one kernel; with measurement events, the dispatch itself records
// start / stop (hipExtLaunchKernelGGL), so the interval is the kernel's own.
template <class K>
hipError_t launch_one(K kernel, dim3 grid, hipStream_t stream, const FwdParams& p,
                      hipEvent_t const* ev, int slot) {
  if (ev != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, ev[2 * slot], ev[2 * slot + 1], 0,
                          p);
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

// A kernel that is not launched still gets its event pair (zero length).
hipError_t skip_one(hipStream_t stream, hipEvent_t const* ev, int slot) {
  if (ev == nullptr) return hipSuccess;
  hipError_t e = hipEventRecord(ev[2 * slot], stream);
  if (e != hipSuccess) return e;
  return hipEventRecord(ev[2 * slot + 1], stream);
}

template <class T, int DK, int DV, bool GATE>
hipError_t launch_variant(const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  using F = Family<T, DK, DV, GATE>;
  constexpr bool kE16 = std::is_same<T, f16>::value;  // float16 entry states
  const int BH = p.B * p.heads;
  hipError_t e;
  if (p.n_spans > 1) {
    if (kE16 && p.span_entry16 == nullptr) return hipErrorInvalidValue;
    if ((e = launch_one(F::summary, dim3(BH * p.n_spans), stream, p, ev, 0)) != hipSuccess) return e;
    if constexpr (kE16) {
      // float16 summaries scanned in place; segments of 4, 8 or 16 spans so
      // that one round of 16 segments covers the sequence when it can
      const dim3 scan_grid(BH, DK * DV / kBScanElems);
      e = p.n_spans <= kBScanSeg * 4
              ? launch_one(span_scan16_kernel<DK, DV, 4>, scan_grid, stream, p, ev, 1)
          : p.n_spans <= kBScanSeg * 8
              ? launch_one(span_scan16_kernel<DK, DV, 8>, scan_grid, stream, p, ev, 1)
              : launch_one(span_scan16_kernel<DK, DV, 16>, scan_grid, stream, p, ev, 1);
    } else {
      const dim3 scan_grid(BH, DK * DV / kScanElems);
      e = p.n_spans <= kScanSeg * 16
              ? launch_one(span_scan_kernel<DK, DV, 16>, scan_grid, stream, p, ev, 1)
              : launch_one(span_scan_kernel<DK, DV, 32>, scan_grid, stream, p, ev, 1);
    }
    if (e != hipSuccess) return e;
  } else {
    if ((e = skip_one(stream, ev, 0)) != hipSuccess) return e;
    if ((e = skip_one(stream, ev, 1)) != hipSuccess) return e;
  }
  return launch_one(F::output, dim3(BH * p.n_spans), stream, p, ev, 2);
}

template <int DK, int DV>
hipError_t launch_f16(bool gate_logits, const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  return gate_logits ? launch_variant<f16, DK, DV, true>(p, stream, ev)
                     : launch_variant<f16, DK, DV, false>(p, stream, ev);
}

hipError_t launch_forward_impl(Dtype dt, int d_k, int d_v, bool gate_logits, const FwdParams& p,
                               hipStream_t stream, hipEvent_t const* ev) {
  if (dt == Dtype::kF16) {
    if (d_k == 64 && d_v == 64) return launch_f16<64, 64>(gate_logits, p, stream, ev);
    if (d_k == 64 && d_v == 128) return launch_f16<64, 128>(gate_logits, p, stream, ev);
    if (d_k == 128 && d_v == 64) return launch_f16<128, 64>(gate_logits, p, stream, ev);
    if (d_k == 128 && d_v == 128) return launch_f16<128, 128>(gate_logits, p, stream, ev);
  } else if (!gate_logits) {
    if (d_k == 64 && d_v == 64) return launch_variant<float, 64, 64, false>(p, stream, ev);
    if (d_k == 64 && d_v == 128) return launch_variant<float, 64, 128, false>(p, stream, ev);
    if (d_k == 128 && d_v == 64) return launch_variant<float, 128, 64, false>(p, stream, ev);
    if (d_k == 128 && d_v == 128) return launch_variant<float, 128, 128, false>(p, stream, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <class T, int DK, int DV, bool GATE>
int output_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Family<T, DK, DV, GATE>::output, kThreads,
                                                   0) != hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

template <int DK, int DV>
int f16_occupancy(bool gate_logits) {
  return gate_logits ? output_occupancy<f16, DK, DV, true>() : output_occupancy<f16, DK, DV, false>();
}

int output_blocks_per_cu(Dtype dt, int d_k, int d_v, bool gate_logits) {
  if (dt == Dtype::kF16) {
    if (d_k == 64 && d_v == 64) return f16_occupancy<64, 64>(gate_logits);
    if (d_k == 64 && d_v == 128) return f16_occupancy<64, 128>(gate_logits);
    if (d_k == 128 && d_v == 64) return f16_occupancy<128, 64>(gate_logits);
    if (d_k == 128 && d_v == 128) return f16_occupancy<128, 128>(gate_logits);
  } else {
    if (d_k == 64 && d_v == 64) return output_occupancy<float, 64, 64, false>();
    if (d_k == 64 && d_v == 128) return output_occupancy<float, 64, 128, false>();
    if (d_k == 128 && d_v == 64) return output_occupancy<float, 128, 64, false>();
    if (d_k == 128 && d_v == 128) return output_occupancy<float, 128, 128, false>();
  }
  return 1;
}

bool has_variant(Dtype dt, int d_k, int d_v) {
  (void)dt;
  return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
}

bool has_two_pass(Dtype dt, int d_k, int d_v) {
  return dt == Dtype::kF16 && d_k == 64 && d_v == 64;
}

int two_pass_blocks_per_cu(bool gate_logits) {
  int n = 0;
  const hipError_t e =
      gate_logits ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n, chunk_output_f16_kernel<64, 64, true, true>, kThreads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n, chunk_output_f16_kernel<64, 64, false, true>, kThreads, 0);
  return (e != hipSuccess || n < 1) ? 1 : n;
}

template <bool GATE>
hipError_t launch_two_pass_variant(const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  const dim3 grid((unsigned)(p.B * p.heads * p.n_spans));
  hipError_t e;
  if ((e = launch_one(span_summary_f16_kernel<64, 64, GATE, true>, grid, stream, p, ev, 0)) !=
      hipSuccess)
    return e;
  if ((e = skip_one(stream, ev, 1)) != hipSuccess) return e;
  return launch_one(chunk_output_f16_kernel<64, 64, GATE, true>, grid, stream, p, ev, 2);
}

hipError_t launch_forward_two_pass(bool gate_logits, const FwdParams& p, hipStream_t stream,
                                   hipEvent_t const* ev) {
  if (p.n_spans < 2 || p.n_spans > kTwoPassMaxSpans) return hipErrorInvalidValue;
  return gate_logits ? launch_two_pass_variant<true>(p, stream, ev)
                     : launch_two_pass_variant<false>(p, stream, ev);
}

hipError_t launch_forward(Dtype dt, int d_k, int d_v, bool gate_logits, const FwdParams& p,
                          hipStream_t stream, hipEvent_t const* ev) {
  return launch_forward_impl(dt, d_k, d_v, gate_logits, p, stream, ev);
}

namespace {

// A kernel launch whose dispatch records `start` and / or `stop` (either may
// be null), so one event pair can bracket several kernels.
template <class K>
hipError_t launch_marked(K kernel, dim3 grid, hipStream_t stream, const FwdParams& p,
                         hipEvent_t start, hipEvent_t stop, int threads = kThreads) {
  if (start != nullptr || stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, start, stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_states_variant(const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  const int BH = p.B * p.heads;
  hipError_t e;
  // both summaries of every span, then both scans: the forward entry state
  // of every span, the adjoint state entering every span from its right, and
  // the gradient of the state before the first step in the adjoint's last slot
  const long long total = (long long)BH * p.n_spans;
  const dim3 sum_grid((unsigned)((total + p.spans_per_wg - 1) / p.spans_per_wg));
  if ((e = launch_marked(bwd_state_summaries_kernel<DK, DV>, sum_grid, stream, p,
                         ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, kSumThreads)) != hipSuccess)
    return e;
  // segments of 4, 8 or 16 slots, so that one round of 16 segments covers
  // the sequence when it can (a 64-chunk sequence in segments of 16 would
  // leave three quarters of every workgroup idle)
  const dim3 scan_grid(BH, 2 * DK * DV / kBScanElems);
  const int slots = p.n_spans > p.adj_slots ? p.n_spans : p.adj_slots;
  auto* scans = slots <= kBScanSeg * 4   ? bwd_state_scans_kernel<DK, DV, 4>
                : slots <= kBScanSeg * 8 ? bwd_state_scans_kernel<DK, DV, 8>
                                         : bwd_state_scans_kernel<DK, DV, 16>;
  return launch_marked(scans, scan_grid, stream, p, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr);
}

}  // namespace

hipError_t launch_bwd_states(int d_k, int d_v, const FwdParams& p, hipStream_t stream,
                             hipEvent_t const* ev) {
  if (d_k == 64 && d_v == 64) return launch_bwd_states_variant<64, 64>(p, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace gla

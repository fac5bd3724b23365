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

#include "gla_internal.h"

namespace gla {
namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kSub = 16;       // tokens per sub-block (one MFMA tile edge)
constexpr int kThreads = 256;  // four wave64s

template <class T>
struct Elt;
template <>
struct Elt<f16> {
  static constexpr int kPerPiece = 8;  // elements per 16-byte row piece
  static constexpr int kPad = 8;       // LDS row padding (elements)
  typedef f16x8 piece_t;               // one 16-byte piece as a vector
};
template <>
struct Elt<float> {
  static constexpr int kPerPiece = 4;
  static constexpr int kPad = 4;
  typedef f32x4 piece_t;
};

template <class T>
__device__ __forceinline__ float fexp(float x) {
  if constexpr (std::is_same<T, float>::value) {
    return expf(x);
  } else {
    return __expf(x);
  }
}

// Scan step t -> row-major grid cell for one of the four directions, with the
// divisions by W or H done by precomputed multiply-shift constants.
struct GridMap {
  int H, W, dir;
  unsigned int mw, mh;
  int sw, sh;
  __device__ __forceinline__ static int div(int t, unsigned int m, int s) {
    return (int)((__umulhi((unsigned)t, m) + (unsigned)t) >> s);
  }
  __device__ __forceinline__ int cell(int t) const {
    if (dir == 0) return t;
    if (dir == 1) {
      const int r = div(t, mw, sw);
      return r * W + (W - 1 - (t - r * W));
    }
    const int c = div(t, mh, sh);
    const int r = t - c * H;
    return (dir == 2 ? r : (H - 1 - r)) * W + c;
  }
};

__device__ __forceinline__ GridMap grid_map(const FwdParams& p, int b) {
  GridMap g;
  g.H = p.H;
  g.W = p.W;
  g.dir = (p.scan_dir == 4) ? (b & 3) : p.scan_dir;
  g.mw = p.div_w_m;
  g.mh = p.div_h_m;
  g.sw = p.div_w_s;
  g.sh = p.div_h_s;
  return g;
}

// Row of key / value dim d in a transposed [dim][token] tile: one padding row
// after every 8 dims, so that the 8 lanes writing dims 8pc+u (pc = 0..7) of a
// token pair land in different LDS banks.
__device__ __forceinline__ constexpr int trow(int d) { return d + (d >> 3); }

// Branch-free select of a loaded 16-byte piece.
__device__ __forceinline__ uint4 sel(bool c, uint4 a, uint4 b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Pair index of sub-block pair (I, J), J < I, in the factor table.
__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// ---------------------------------------------------------------------------
// Shared-memory tiles of one chunk.
template <class T, int DK, int DV>
struct ChunkSmem {
  static constexpr int P = Elt<T>::kPad;
  static constexpr int QS = DK + P;      // row stride: [token][d_k] tiles
  static constexpr int AS = kChunk + P;  // row stride: [*][token] tiles
  static constexpr int OS = DV + P;      // row stride: [token][d_v] tile
  static constexpr int LA_ELEMS = kChunk * QS;
  static constexpr int A_ELEMS = kChunk * AS;
  alignas(16) T q[kChunk * QS];    // raw q, then q_t*exp(c_t)
  alignas(16) T k[kChunk * QS];    // raw k, then k_s*exp(-c_s)
  alignas(16) T la[(LA_ELEMS > A_ELEMS) ? LA_ELEMS : A_ELEMS];  // raw log-alpha, then A[t][s]
  alignas(16) T vt[DV * AS];       // V^T [d_v][token]
  alignas(16) T klt[DK * AS];      // (k_s*exp(b_last-b_s))^T [d_k][token]
  alignas(16) T o[kChunk * OS];    // output staging [token][d_v]
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

  // Registers -> shared tiles: q, k, la row-major; v transposed to [d_v][token].
  template <bool WITH_Q>
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
      *reinterpret_cast<uint4*>(sla + o) = rl[j];
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
      if constexpr (std::is_same<T, f16>::value) {
#pragma unroll
        for (int s0 = 0; s0 < kChunk; s0 += 32) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(klt + dim * AS + s0 + 8 * g);
          const f16x8 b = *reinterpret_cast<const f16x8*>(vt + col * AS + s0 + 8 * g);
          acc = mma32(a, b, acc);
        }
      } else {
#pragma unroll
        for (int s0 = 0; s0 < kChunk; s0 += 4)
          acc = mma4(klt[dim * AS + s0 + g], vt[col * AS + s0 + g], acc);
      }
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
// Kernel 2: scan over spans, elementwise over the d_k x d_v state, turning each
// span summary (G_s, L_s) into the state entering span s:
//   E_0 = 0,  E_{s+1} = diag(G_s) E_s + L_s.
// The combine (G, L) o (G', L') = (G G', diag(G') L + L') is associative, so
// spans are taken in rounds of kScanSeg segments of kScanU spans, one wave per
// segment: each lane loads its segment's summaries at once (one memory round
// trip), folds them from zero, the folds are exchanged through LDS to give
// every segment its carry-in, and the same registers then yield the entry
// states.
constexpr int kScanSeg = 4;
constexpr int kScanU = 32;
constexpr int kScanElems = kThreads / kScanSeg;   // state elements per workgroup

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void span_scan_kernel(FwdParams p) {
  __shared__ float seg_l[kScanSeg][kScanElems];
  __shared__ float seg_g[kScanSeg][kScanElems];
  const int bh = blockIdx.x;
  const int seg = threadIdx.x / kScanElems;
  const int le = threadIdx.x - seg * kScanElems;
  const int e = blockIdx.y * kScanElems + le;
  const int dim = e / DV;
  float* const L = p.span_state + (size_t)bh * p.n_spans * DK * DV + e;
  const float* const G = p.span_gate + (size_t)bh * p.n_spans * DK + dim;

  float carry = 0.f;  // state entering the current round
  for (int r0 = 0; r0 < p.n_spans; r0 += kScanSeg * kScanU) {
    const int s0 = r0 + seg * kScanU;
    float l[kScanU], gg[kScanU];
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      // slots past the last span re-read span 0 and are neutralised (no
      // branches around the loads, so all of them are in flight together)
      const bool in = s0 + u < p.n_spans;
      const int sp = in ? s0 + u : 0;
      const float lv = L[(size_t)sp * DK * DV];
      const float gv = G[(size_t)sp * DK];
      l[u] = in ? lv : 0.f;
      gg[u] = in ? gv : 1.f;
    }
    float fl = 0.f, fg = 1.f;
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
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
    for (int u = 0; u < kScanU; ++u) {
      if (s0 + u < p.n_spans) L[(size_t)(s0 + u) * DK * DV] = run;
      run = gg[u] * run + l[u];
    }
    carry = next;
    __syncthreads();  // the LDS folds are reused by the next round
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: outputs.  Replays the span's chunks from the span's entry state.
template <class T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void chunk_output_kernel(FwdParams p) {
  using SM = ChunkSmem<T, DK, DV>;
  __shared__ SM sm;
  constexpr int QS = SM::QS, AS = SM::AS, OS = SM::OS;
  constexpr int EPP = Elt<T>::kPerPiece;
  constexpr bool kF16 = std::is_same<T, f16>::value;
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
        (span > 0) ? p.span_state + ((size_t)bh * p.n_spans + span) * DK * DV : nullptr;
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
    ld.template store<true>(sm.q, sm.k, sm.la, sm.vt, QS, AS);
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
        c_run += (float)sm.la[(kSub * J + r) * QS + i];
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
    T* sa = sm.la;
    for (int ti = 0; ti < n_tiles; ++ti) {
      const int code = (tile_codes >> (8 * ti)) & 0xff;
      const int I = code >> 4, J = code & 0xf;
      const int s_row = kSub * J + n16;  // key token supplying the A operand
      const int t_row = kSub * I + n16;  // query token supplying the B operand
      const float* F = (J < I) ? sm.f + pair_index(I, J) * DK : nullptr;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kF16) {
#pragma unroll
        for (int d0 = 0; d0 < DK; d0 += 32) {
          f16x8 a = *reinterpret_cast<const f16x8*>(sm.k + s_row * QS + d0 + 8 * g);
          if (F) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] = (f16)((float)a[u] * F[d0 + 8 * g + u]);
          }
          const f16x8 bq = *reinterpret_cast<const f16x8*>(sm.q + t_row * QS + d0 + 8 * g);
          acc = mma32(a, bq, acc);
        }
      } else {
#pragma unroll 8
        for (int d0 = 0; d0 < DK; d0 += 4) {
          float a = sm.k[s_row * QS + d0 + g];
          if (F) a *= F[d0 + g];
          acc = mma4(a, sm.q[t_row * QS + d0 + g], acc);
        }
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
      f16x8 sh[DK / 32];
      if constexpr (kF16) {
#pragma unroll
        for (int rho = 0; rho < DK / 32; ++rho)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            sh[rho][u] = (f16)st.s[2 * rho][j][u];
            sh[rho][4 + u] = (f16)st.s[2 * rho + 1][j][u];
          }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int t = kSub * I + n16;
        const int len = kSub * (I + 1);
        const float* E = sm.e + I * DK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kF16) {
#pragma unroll
          for (int s0 = 0; s0 + 32 <= len; s0 += 32) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(sm.vt + col * AS + s0 + 8 * g);
            const f16x8 bb = *reinterpret_cast<const f16x8*>(sa + t * AS + s0 + 8 * g);
            acc = mma32(a, bb, acc);
          }
          if (len & 16) {
            const int s0 = len - 16;
            const f16x4 a = *reinterpret_cast<const f16x4*>(sm.vt + col * AS + s0 + 4 * g);
            const f16x4 bb = *reinterpret_cast<const f16x4*>(sa + t * AS + s0 + 4 * g);
            acc = mma16(a, bb, acc);
          }
#pragma unroll
          for (int rho = 0; rho < DK / 32; ++rho) {
            const int dlo = 32 * rho + 4 * g, dhi = dlo + 16;
            const f16x4 qlo = *reinterpret_cast<const f16x4*>(sm.q + t * QS + dlo);
            const f16x4 qhi = *reinterpret_cast<const f16x4*>(sm.q + t * QS + dhi);
            f16x8 bq;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              bq[u] = (f16)((float)qlo[u] * E[dlo + u]);
              bq[4 + u] = (f16)((float)qhi[u] * E[dhi + u]);
            }
            acc = mma32(sh[rho], bq, acc);
          }
        } else {
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
// Float16 kernels.  The per-chunk elementwise work (cumulative decay, anchored
// q / k scalings, decayed keys) runs in MFMA-friendly register layouts so that
// every LDS access is a 64- or 128-bit vector op:
//  * log-alpha is staged transposed ([d_k][token]); cumulative sums over tokens
//    are 16x16x16 MFMAs against constant triangular matrices (log2(e) folded
//    in as an exact hi + lo pair), landing either as "4 key dims of one token
//    per lane" (output kernel) or "4 tokens of one key dim per lane" (summary);
//  * the decay over each 16-token sub-block is broadcast along each 16-lane
//    row with DPP, so the per-(dim, sub-block) factors need no exp and no LDS;
//  * keys are pre-scaled into the variants the causal score tiles need, so the
//    score MFMAs read unscaled operands;
//  * the decayed keys for the state update are transposed with an identity
//    MFMA (exact: one non-zero product per output).

__device__ __forceinline__ float row_bcast15(float x) {
  // every lane of a 16-lane row receives the row's lane 15 value
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                0x15F, 0xF, 0xF, false));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(e) split into two binary16 values whose sum is log2(e) to ~1e-7.
constexpr float kLog2eHi = 1.4423828125f;          // fp16(log2 e)
constexpr float kLog2eLo = 1.4426950408889634f - 1.4423828125f;


// Row pieces of q and k, token-pair pieces of log-alpha and v (for the
// transposed tiles).  Pieces past the sequence end read as zero.
template <int DK, int DV, bool WITH_Q, bool K_ROWS>
struct LoaderH {
  static constexpr int PK = DK / 8, PV = DV / 8;   // 16-byte pieces per token row
  static constexpr int NK = kChunk * PK / kThreads;          // row pieces per thread
  static constexpr int NKP = (kChunk / 2) * PK / kThreads;   // d_k token pairs per thread
  static constexpr int NVP = (kChunk / 2) * PV / kThreads;   // d_v token pairs per thread
  static_assert(NK >= 1 && NKP >= 1 && NVP >= 1, "tile too small");
  uint4 rq[WITH_Q ? NK : 1];
  uint4 rk[K_ROWS ? NK : 2 * NKP];
  uint4 rl[2 * NKP];
  uint4 rv[2 * NVP];
  // validity of each piece (bit j: row piece j, bit 16+i: pair piece i, bit
  // 24+i: v pair piece i); invalid pieces are zeroed when staged
  uint32_t okm;

  __device__ __forceinline__ static uint4 ld(const f16* p) {
    return *reinterpret_cast<const uint4*>(p);
  }

  __device__ __forceinline__ void load(const f16* q, const f16* k, const f16* la, const f16* v,
                                       size_t off_k, size_t off_v, int t0, int valid, const GridMap& gm) {
    const int tid = threadIdx.x;
    okm = 0;
    if (WITH_Q || K_ROWS) {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int id = tid + kThreads * j;
        const int tok = id / PK, pc = id - tok * PK;
        const bool in = tok < valid;
        // out-of-range lanes read the sequence's first row and drop it when
        // staging: no branches around the loads, so waits can count them
        const size_t o = off_k + (size_t)gm.cell(in ? t0 + tok : 0) * DK + pc * 8;
        if (WITH_Q) rq[j] = ld(q + o);
        if (K_ROWS) rk[j] = ld(k + o);
        okm |= (in ? 1u : 0u) << j;
      }
    }
#pragma unroll
    for (int j = 0; j < NKP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PK, pc = id - tp * PK;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = 2 * tp + h;
        const bool in = tok < valid;
        const size_t o = off_k + (size_t)gm.cell(in ? t0 + tok : 0) * DK + pc * 8;
        rl[2 * j + h] = ld(la + o);
        if (!K_ROWS) rk[2 * j + h] = ld(k + o);
        okm |= (in ? 1u : 0u) << (16 + 2 * j + h);
      }
    }
#pragma unroll
    for (int j = 0; j < NVP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PV, pc = id - tp * PV;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = 2 * tp + h;
        const bool in = tok < valid;
        rv[2 * j + h] = ld(v + off_v + (size_t)gm.cell(in ? t0 + tok : 0) * DV + pc * 8);
        okm |= (in ? 1u : 0u) << (24 + 2 * j + h);
      }
    }
  }

  // Write a token pair (a, b) of 8-element pieces transposed: dst[(8pc+u)*AS + 2tp].
  __device__ __forceinline__ static void put_pair_t(f16* dst, int AS, int pc, int tp, uint4 a,
                                                    uint4 b) {
    const f16x8 x = __builtin_bit_cast(f16x8, a);
    const f16x8 y = __builtin_bit_cast(f16x8, b);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      f16x2 pr;
      pr[0] = x[u];
      pr[1] = y[u];
      *reinterpret_cast<f16x2*>(dst + (9 * pc + u) * AS + 2 * tp) = pr;  // row trow(8pc+u)
    }
  }

  __device__ __forceinline__ void store(f16* sq, f16* sk, int QS, f16* skt, f16* slat, f16* svt,
                                        int AS) const {
    const int tid = threadIdx.x;
    const uint4 z = make_uint4(0, 0, 0, 0);
    auto ok = [&](int bit) { return ((okm >> bit) & 1u) != 0; };
    if (WITH_Q || K_ROWS) {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int id = tid + kThreads * j;
        const int tok = id / PK, pc = id - tok * PK;
        if (WITH_Q) *reinterpret_cast<uint4*>(sq + tok * QS + pc * 8) = sel(ok(j), rq[j], z);
        if (K_ROWS) *reinterpret_cast<uint4*>(sk + tok * QS + pc * 8) = sel(ok(j), rk[j], z);
      }
    }
#pragma unroll
    for (int j = 0; j < NKP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PK, pc = id - tp * PK;
      const bool a = ok(16 + 2 * j), b = ok(17 + 2 * j);
      put_pair_t(slat, AS, pc, tp, sel(a, rl[2 * j], z), sel(b, rl[2 * j + 1], z));
      if (!K_ROWS) put_pair_t(skt, AS, pc, tp, sel(a, rk[2 * j], z), sel(b, rk[2 * j + 1], z));
    }
#pragma unroll
    for (int j = 0; j < NVP; ++j) {
      const int id = tid + kThreads * j;
      const int tp = id / PV, pc = id - tp * PV;
      put_pair_t(svt, AS, pc, tp, sel(ok(24 + 2 * j), rv[2 * j], z),
                 sel(ok(25 + 2 * j), rv[2 * j + 1], z));
    }
  }
};

// Constant 16x16x16 MFMA B operands, lane (n, g) holding rows 4g..4g+3 of column n:
// U[s][t] = (s <= t) * v, and the identity.
__device__ __forceinline__ f16x4 upper_incl(float v) {
  const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  f16x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = (f16)((4 * g + u <= n16) ? v : 0.f);
  return r;
}
__device__ __forceinline__ f16x4 identity16() {
  const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  f16x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = (f16)((4 * g + u == n16) ? 1.f : 0.f);
  return r;
}

// ---------------------------------------------------------------------------
// Output kernel, float16.  The span is walked in 32-token steps (two 16-token
// sub-blocks), which keeps the shared tiles near 37 KB so four workgroups (four
// waves per SIMD) share a CU.  Per step:
//   stage  : q, k row-major; log-alpha and v transposed (token pairs)
//   P      : wave w owns key dims 16w.. : in-sub-block cumulative decay c by
//            MFMA, exp(+-c), DPP broadcast of the sub-block decays, anchored
//            q / k, q decayed from the step start, keys decayed to the end of
//            sub-block 0 and to the step end (transposed by an identity MFMA)
//   A      : score tiles (0,0), (1,0), (1,1); tile (0,1) is zeroed
//   O      : wave w owns value columns 16w.. : O^T = V^T A^T + S^T Qt^T, then
//            S <- diag(exp(b_end)) S + KL^T V
//   W      : output rows to their grid cells
constexpr int kStep = 32;

__host__ __device__ constexpr int trow_h(int d) { return d + (d >> 3); }

template <int DK, int DV>
struct StepSmem {
  static constexpr int QS = DK + 8;      // [token][d_k] rows
  static constexpr int AS = kStep + 8;   // [*][token] rows
  static constexpr int OS = DV + 8;      // [token][d_v] rows
  static constexpr int LAT_ELEMS =
      (trow_h(DK) * AS > kStep * AS) ? trow_h(DK) * AS : kStep * AS;
  alignas(16) f16 q[kStep * QS];     // raw q, then q_t*exp(c_t)  (c: decay inside the sub-block)
  alignas(16) f16 qt[kStep * QS];    // q_t*exp(b_t)              (b: decay from the step start)
  alignas(16) f16 k[kStep * QS];     // raw k, then k_s*exp(-c_s)
  alignas(16) f16 kv[kSub * QS];     // sub-block 0 keys decayed to the end of sub-block 0
  alignas(16) f16 lat[LAT_ELEMS];    // log-alpha^T [trow(d_k)][token], then A[t][s]
  alignas(16) f16 vt[trow_h(DV) * AS];
  alignas(16) f16 klt[DK * AS];      // keys decayed to the step end, [d_k][token]
  alignas(16) f16 o[kStep * OS];     // output staging
  alignas(16) float g[DK];           // exp(decay over the step)
};

// One 32-token step of q, k (row pieces) and log-alpha, v (token-pair pieces).
template <int DK, int DV>
struct StepLoader {
  static constexpr int PK = DK / 8, PV = DV / 8;
  static constexpr int NQ = kStep * PK / kThreads;                 // q / k row pieces per thread
  static constexpr int NPAIR = (kStep / 2) * (PK + PV);            // la + v pair items
  static constexpr int NP = (NPAIR + kThreads - 1) / kThreads;     // pair items per thread
  static_assert(NQ >= 1 && (kStep / 2) * PK % 64 == 0 && NPAIR % 64 == 0, "tile shape");
  uint4 rq[NQ], rk[NQ], rp[2 * NP];
  uint32_t okm;  // bit j: row piece j valid; bit 8+i: pair piece i valid

  __device__ __forceinline__ static uint4 ld(const f16* p) {
    return *reinterpret_cast<const uint4*>(p);
  }

  __device__ __forceinline__ void load(const f16* q, const f16* k, const f16* la, const f16* v,
                                       size_t off_k, size_t off_v, int t0, int valid,
                                       const GridMap& gm) {
    const int tid = threadIdx.x;
    okm = 0;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int id = tid + kThreads * j;
      const int tok = id / PK, pc = id - tok * PK;
      const bool in = tok < valid;
      const size_t o = off_k + (size_t)gm.cell(in ? t0 + tok : 0) * DK + pc * 8;
      rq[j] = ld(q + o);
      rk[j] = ld(k + o);
      okm |= (in ? 1u : 0u) << j;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int id = tid + kThreads * j;
      if (id < NPAIR) {
        const bool is_la = id < (kStep / 2) * PK;
        const int rel = is_la ? id : id - (kStep / 2) * PK;
        const int pp = is_la ? PK : PV;
        const int tp = rel / pp, pc = rel - tp * pp;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tok = 2 * tp + h;
          const bool in = tok < valid;
          const size_t cell = (size_t)gm.cell(in ? t0 + tok : 0);
          const f16* src = is_la ? la + off_k + cell * DK + pc * 8 : v + off_v + cell * DV + pc * 8;
          rp[2 * j + h] = ld(src);
          okm |= (in ? 1u : 0u) << (8 + 2 * j + h);
        }
      }
    }
  }

  __device__ __forceinline__ void store(StepSmem<DK, DV>& sm) const {
    constexpr int QS = StepSmem<DK, DV>::QS, AS = StepSmem<DK, DV>::AS;
    const int tid = threadIdx.x;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int id = tid + kThreads * j;
      const int tok = id / PK, pc = id - tok * PK;
      const bool in = ((okm >> j) & 1u) != 0;
      *reinterpret_cast<uint4*>(sm.q + tok * QS + pc * 8) = sel(in, rq[j], z);
      *reinterpret_cast<uint4*>(sm.k + tok * QS + pc * 8) = sel(in, rk[j], z);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int id = tid + kThreads * j;
      if (id < NPAIR) {
        const bool is_la = id < (kStep / 2) * PK;
        const int rel = is_la ? id : id - (kStep / 2) * PK;
        const int pp = is_la ? PK : PV;
        const int tp = rel / pp, pc = rel - tp * pp;
        f16* dst = is_la ? sm.lat : sm.vt;
        const f16x8 x = __builtin_bit_cast(f16x8, sel(((okm >> (8 + 2 * j)) & 1u) != 0, rp[2 * j], z));
        const f16x8 y =
            __builtin_bit_cast(f16x8, sel(((okm >> (9 + 2 * j)) & 1u) != 0, rp[2 * j + 1], z));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          f16x2 pr;
          pr[0] = x[u];
          pr[1] = y[u];
          *reinterpret_cast<f16x2*>(dst + (9 * pc + u) * AS + 2 * tp) = pr;  // row trow(8pc+u)
        }
      }
    }
  }
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreads, (DK == 64 && DV == 64) ? 4 : (DK == 128 && DV == 128) ? 1 : 2) void chunk_output_f16_kernel(
    FwdParams p) {
  using SM = StepSmem<DK, DV>;
  __shared__ SM sm;
  constexpr int QS = SM::QS, AS = SM::AS, OS = SM::OS;
  constexpr int NR = DK / 16, NC = DV / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const size_t off_k = (size_t)bh * p.T * DK;
  const size_t off_v = (size_t)bh * p.T * DV;
  const int t_begin = span * p.span_chunks * kChunk;
  const int t_end = min(t_begin + p.span_chunks * kChunk, p.T);

  const f16* q = static_cast<const f16*>(p.q);
  const f16* k = static_cast<const f16*>(p.k);
  const f16* la = static_cast<const f16*>(p.la);
  const f16* v = static_cast<const f16*>(p.v);
  f16* out = static_cast<f16*>(p.out);

  // State tiles: wave w owns value columns 16(w + 4j) .. ; tile (r, j) holds
  // S[16r + 4g + u][16(w + 4j) + n] in lane (g, n).
  f32x4 st[NR][NC];
  {
    const float* src =
        (span > 0) ? p.span_state + ((size_t)bh * p.n_spans + span) * DK * DV : nullptr;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) st[r][j][u] = src ? src[(16 * r + 4 * g + u) * DV + col] : 0.f;
    }
  }

  const f16x4 u_hi = upper_incl(kLog2eHi), u_lo = upper_incl(kLog2eLo);
  const f16x4 ident = identity16();
  f16* const sa = sm.lat;  // score tile reuses the log-alpha^T region

  StepLoader<DK, DV> ld;
  ld.load(q, k, la, v, off_k, off_v, t_begin, min(kStep, t_end - t_begin), gm);
  for (int t0 = t_begin; t0 < t_end; t0 += kStep) {
    const int valid = min(kStep, t_end - t0);
    ld.store(sm);
    if (t0 + kStep < t_end) ld.load(q, k, la, v, off_k, off_v, t0 + kStep, min(kStep, t_end - t0 - kStep), gm);
    __syncthreads();

    // ---- Phase P
#pragma unroll
    for (int dbi = 0; dbi < DK / 64; ++dbi) {
      const int db = wave + 4 * dbi;
      const int dim0 = 16 * db + 4 * g;
      f16x4 lat4[2], q4[2], k4[2];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        lat4[I] = *reinterpret_cast<const f16x4*>(sm.lat + trow_h(16 * db + n16) * AS + 16 * I + 4 * g);
        q4[I] = *reinterpret_cast<const f16x4*>(sm.q + (16 * I + n16) * QS + dim0);
        k4[I] = *reinterpret_cast<const f16x4*>(sm.k + (16 * I + n16) * QS + dim0);
      }
      f32x4 c2[2];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        c2[I] = mma16(lat4[I], u_hi, f32x4{0.f, 0.f, 0.f, 0.f});
        c2[I] = mma16(lat4[I], u_lo, c2[I]);
      }
      f32x4 eq[2], ek[2], ed[2];
#pragma unroll
      for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          eq[I][u] = exp2_fast(c2[I][u]);
          ek[I][u] = exp2_fast(-c2[I][u]);
          ed[I][u] = row_bcast15(eq[I][u]);  // exp(decay over sub-block I)
        }
      if (n16 == 0) {
        f32x4 gl;
#pragma unroll
        for (int u = 0; u < 4; ++u) gl[u] = ed[0][u] * ed[1][u];
        *reinterpret_cast<f32x4*>(sm.g + dim0) = gl;
      }
      f16x4 klh[2];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int row = 16 * I + n16;
        f16x4 ql, qt, kd, kv0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float qf = (float)q4[I][u];
          const float eqs = (I == 0) ? eq[I][u] : eq[I][u] * ed[0][u];
          ql[u] = (f16)(qf * eq[I][u]);
          qt[u] = (f16)(qf * eqs);
          const float kf = (float)k4[I][u] * ek[I][u];
          kd[u] = (f16)kf;
          const float kend = kf * ed[I][u];  // decayed to the end of sub-block I
          if (I == 0) {
            kv0[u] = (f16)kend;
            klh[I][u] = (f16)(kend * ed[1][u]);
          } else {
            klh[I][u] = (f16)kend;
          }
        }
        *reinterpret_cast<f16x4*>(sm.q + row * QS + dim0) = ql;
        *reinterpret_cast<f16x4*>(sm.qt + row * QS + dim0) = qt;
        *reinterpret_cast<f16x4*>(sm.k + row * QS + dim0) = kd;
        if (I == 0) *reinterpret_cast<f16x4*>(sm.kv + n16 * QS + dim0) = kv0;
      }
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const f32x4 tr = mma16(klh[I], ident, f32x4{0.f, 0.f, 0.f, 0.f});
        f16x4 trh;
#pragma unroll
        for (int u = 0; u < 4; ++u) trh[u] = (f16)tr[u];
        *reinterpret_cast<f16x4*>(sm.klt + (16 * db + n16) * AS + 16 * I + 4 * g) = trh;
      }
    }
    __syncthreads();

    // ---- Phase A: wave 0 -> (0,0), wave 1 -> (1,0), wave 2 -> (1,1), wave 3 zeroes (0,1).
    if (wave < 3) {
      const int I = (wave == 0) ? 0 : 1, J = (wave == 2) ? 1 : 0;
      const f16* kb = (I != J) ? sm.kv : sm.k + 16 * J * QS;
      f16x8 ta[DK / 32], tb[DK / 32];
#pragma unroll
      for (int st2 = 0; st2 < DK / 32; ++st2) {
        ta[st2] = *reinterpret_cast<const f16x8*>(kb + n16 * QS + 32 * st2 + 8 * g);
        tb[st2] = *reinterpret_cast<const f16x8*>(sm.q + (16 * I + n16) * QS + 32 * st2 + 8 * g);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st2 = 0; st2 < DK / 32; ++st2) acc = mma32(ta[st2], tb[st2], acc);
      if (I == J) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (4 * g + u > n16) acc[u] = 0.f;
      }
      f16x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = (f16)acc[u];
      *reinterpret_cast<f16x4*>(sa + (16 * I + n16) * AS + 16 * J + 4 * g) = w;
    } else {
      *reinterpret_cast<f16x4*>(sa + n16 * AS + 16 + 4 * g) =
          f16x4{(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
    }
    __syncthreads();

    // ---- Phase O
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col0 = 16 * (wave + 4 * j);
      const int col = col0 + n16;
      const f16x8 va = *reinterpret_cast<const f16x8*>(sm.vt + trow_h(col) * AS + 8 * g);
      f16x8 sb[2], qb[2][DK / 32];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int t = 16 * I + n16;
        sb[I] = *reinterpret_cast<const f16x8*>(sa + t * AS + 8 * g);
#pragma unroll
        for (int rho = 0; rho < DK / 32; ++rho) {
          const int dlo = 32 * rho + 4 * g;
          const f16x4 qlo = *reinterpret_cast<const f16x4*>(sm.qt + t * QS + dlo);
          const f16x4 qhi = *reinterpret_cast<const f16x4*>(sm.qt + t * QS + dlo + 16);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            qb[I][rho][u] = qlo[u];
            qb[I][rho][4 + u] = qhi[u];
          }
        }
      }
      f32x4 gv[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) gv[r] = *reinterpret_cast<const f32x4*>(sm.g + 16 * r + 4 * g);
      f16x8 sh[DK / 32];
#pragma unroll
      for (int rho = 0; rho < DK / 32; ++rho)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sh[rho][u] = (f16)st[2 * rho][j][u];
          sh[rho][4 + u] = (f16)st[2 * rho + 1][j][u];
        }
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int t = 16 * I + n16;
        f32x4 acc = mma32(va, sb[I], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int rho = 0; rho < DK / 32; ++rho) acc = mma32(sh[rho], qb[I][rho], acc);
        f16x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (f16)acc[u];
        *reinterpret_cast<f16x4*>(sm.o + t * OS + col0 + 4 * g) = w;
      }
      // S <- diag(exp(b_end)) S + KL^T V
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const f16x8 kar = *reinterpret_cast<const f16x8*>(sm.klt + (16 * r + n16) * AS + 8 * g);
        f32x4 acc = st[r][j];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] *= gv[r][u];
        st[r][j] = mma32(kar, va, acc);
      }
    }
    __syncthreads();

    // ---- Phase W
    constexpr int PO = DV / 8;
    constexpr int NO = kStep * PO / kThreads;
#pragma unroll
    for (int jj = 0; jj < NO; ++jj) {
      const int id = tid + kThreads * jj;
      const int tok = id / PO, pc = id - tok * PO;
      if (tok < valid) {
        const size_t o = off_v + (size_t)gm.cell(t0 + tok) * DV + pc * 8;
        *reinterpret_cast<uint4*>(out + o) = *reinterpret_cast<const uint4*>(sm.o + tok * OS + pc * 8);
      }
    }
  }

  if (span == p.n_spans - 1 && p.final_state != nullptr) {
    float* dst = p.final_state + (size_t)bh * DK * DV;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int col = 16 * (wave + 4 * j) + n16;
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[(16 * r + 4 * g + u) * DV + col] = st[r][j][u];
    }
  }
}

// ---------------------------------------------------------------------------
// Span-summary kernel, float16.  Keeps S^T in the accumulators, wave w owning
// key dims 16*db.. (db = w, w+4) for all value columns: lane (n, g) of tile cb
// holds S^T[16cb + 4g + u][16db + n], so each lane scales by one decay factor.
template <int DK, int DV>
struct SumSmemH {
  static constexpr int AS = kChunk + 8;
  alignas(16) f16 kt[trow(DK) * AS];   // k^T [trow(d_k)][token]
  alignas(16) f16 lat[trow(DK) * AS];  // log-alpha^T
  alignas(16) f16 vt[trow(DV) * AS];   // V^T
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void span_summary_f16_kernel(FwdParams p) {
  using SM = SumSmemH<DK, DV>;
  __shared__ SM sm;
  constexpr int AS = SM::AS;
  constexpr int NDB = DK / 64, NCB = DV / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  const int b = bh / p.heads;
  const GridMap gm = grid_map(p, b);
  const size_t off_k = (size_t)bh * p.T * DK;
  const size_t off_v = (size_t)bh * p.T * DV;
  const int c_begin = span * p.span_chunks;
  const int c_end = min(c_begin + p.span_chunks, p.n_chunks);
  const f16* k = static_cast<const f16*>(p.k);
  const f16* la = static_cast<const f16*>(p.la);
  const f16* v = static_cast<const f16*>(p.v);

  // Constant A operands (rows t, cols s of a 16x16 block): strict upper part
  // (s > t) of the diagonal block and the all-ones block for later sub-blocks,
  // so that the MFMA yields the decay from token t to the chunk end.
  f16x4 m_diag, m_ones;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m_diag[u] = (f16)((4 * g + u > n16) ? 1.f : 0.f);
    m_ones[u] = (f16)1.f;
  }

  f32x4 st[NDB][NCB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st[d][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float log_gate[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) log_gate[d] = 0.f;

  // Two chunks of loads in flight.  The loop is unrolled by two with
  // unconditional loads, so the compiler can wait for just the older chunk: a
  // chunk index past the span reads nothing and stages zeros, and an all-zero
  // chunk (no keys, no values, log-alpha 0) leaves the state unchanged.
  const int t_stop = min(c_end * kChunk, p.T);
  auto valid_of = [&](int c) { return max(0, min(kChunk, t_stop - c * kChunk)); };
  LoaderH<DK, DV, false, false> ld0, ld1;
  ld0.load(nullptr, k, la, v, off_k, off_v, c_begin * kChunk, valid_of(c_begin), gm);
  ld1.load(nullptr, k, la, v, off_k, off_v, (c_begin + 1) * kChunk, valid_of(c_begin + 1), gm);
  auto compute_chunk = [&]() {
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const int db = wave + 4 * d;
        const int dim = 16 * db + n16;
        f16x4 lat4[4];
  #pragma unroll
        for (int J = 0; J < 4; ++J)
          lat4[J] = *reinterpret_cast<const f16x4*>(sm.lat + trow(dim) * AS + 16 * J + 4 * g);
        // decay from token 16I+4g+u to the chunk end, at key dim `dim`
        f32x4 rest[4];
  #pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 acc = mma16(m_diag, lat4[I], f32x4{0.f, 0.f, 0.f, 0.f});
  #pragma unroll
          for (int J = I + 1; J < 4; ++J) acc = mma16(m_ones, lat4[J], acc);
          rest[I] = acc;
        }
        // whole-chunk decay of this dim: token 0's remainder plus its own log-alpha
        const float first = __shfl(rest[0][0] + (float)lat4[0][0], n16, 64);
        log_gate[d] += first;
        const float gch = exp2_fast(first * 1.4426950408889634f);
  #pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
  #pragma unroll
          for (int u = 0; u < 4; ++u) st[d][cb][u] *= gch;
  #pragma unroll
        for (int I = 0; I < 4; ++I) {
          const f16x4 k4 = *reinterpret_cast<const f16x4*>(sm.kt + trow(dim) * AS + 16 * I + 4 * g);
          f16x4 kl;
  #pragma unroll
          for (int u = 0; u < 4; ++u)
            kl[u] = (f16)((float)k4[u] * exp2_fast(rest[I][u] * 1.4426950408889634f));
  #pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const f16x4 vv =
                *reinterpret_cast<const f16x4*>(sm.vt + trow(16 * cb + n16) * AS + 16 * I + 4 * g);
            st[d][cb] = mma16(vv, kl, st[d][cb]);
          }
        }
      }
  };
  for (int c = c_begin; c < c_end; c += 2) {
    __syncthreads();  // previous chunk's reads of the tiles are done
    ld0.store(nullptr, nullptr, 0, sm.kt, sm.lat, sm.vt, AS);
    ld0.load(nullptr, k, la, v, off_k, off_v, (c + 2) * kChunk, valid_of(c + 2), gm);
    __syncthreads();
    compute_chunk();
    __syncthreads();
    ld1.store(nullptr, nullptr, 0, sm.kt, sm.lat, sm.vt, AS);
    ld1.load(nullptr, k, la, v, off_k, off_v, (c + 3) * kChunk, valid_of(c + 3), gm);
    __syncthreads();
    compute_chunk();
  }

  float* dst = p.span_state + ((size_t)bh * p.n_spans + span) * DK * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int dim = 16 * (wave + 4 * d) + n16;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<f32x4*>(dst + dim * DV + 16 * cb + 4 * g) = st[d][cb];
    if (g == 0) p.span_gate[((size_t)bh * p.n_spans + span) * DK + dim] = exp2_fast(log_gate[d] * 1.4426950408889634f);
  }
}

// Kernel choice per element type: float16 runs the MFMA-layout kernels,
// float32 the generic ones.
template <class T, int DK, int DV>
struct Family {
  static constexpr auto summary = span_summary_kernel<T, DK, DV>;
  static constexpr auto output = chunk_output_kernel<T, DK, DV>;
};
template <int DK, int DV>
struct Family<f16, DK, DV> {
  static constexpr auto summary = span_summary_f16_kernel<DK, DV>;
  static constexpr auto output = chunk_output_f16_kernel<DK, DV>;
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

template <class T, int DK, int DV>
hipError_t launch_variant(const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  const int BH = p.B * p.heads;
  hipError_t e;
  if (p.n_spans > 1) {
    if ((e = launch_one(Family<T, DK, DV>::summary, dim3(BH * p.n_spans), stream, p, ev, 0)) !=
        hipSuccess)
      return e;
    if ((e = launch_one(span_scan_kernel<DK, DV>, dim3(BH, DK * DV / kScanElems), stream, p, ev,
                        1)) != hipSuccess)
      return e;
  } else {
    if ((e = skip_one(stream, ev, 0)) != hipSuccess) return e;
    if ((e = skip_one(stream, ev, 1)) != hipSuccess) return e;
  }
  return launch_one(Family<T, DK, DV>::output, dim3(BH * p.n_spans), stream, p, ev, 2);
}

hipError_t launch_forward_impl(Dtype dt, int d_k, int d_v, const FwdParams& p, hipStream_t stream,
                               hipEvent_t const* ev) {
  if (dt == Dtype::kF16) {
    if (d_k == 64 && d_v == 64) return launch_variant<f16, 64, 64>(p, stream, ev);
    if (d_k == 64 && d_v == 128) return launch_variant<f16, 64, 128>(p, stream, ev);
    if (d_k == 128 && d_v == 64) return launch_variant<f16, 128, 64>(p, stream, ev);
    if (d_k == 128 && d_v == 128) return launch_variant<f16, 128, 128>(p, stream, ev);
  } else {
    if (d_k == 64 && d_v == 64) return launch_variant<float, 64, 64>(p, stream, ev);
    if (d_k == 64 && d_v == 128) return launch_variant<float, 64, 128>(p, stream, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <class T, int DK, int DV>
int output_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Family<T, DK, DV>::output, kThreads, 0) !=
          hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

int output_blocks_per_cu(Dtype dt, int d_k, int d_v) {
  if (dt == Dtype::kF16) {
    if (d_k == 64 && d_v == 64) return output_occupancy<f16, 64, 64>();
    if (d_k == 64 && d_v == 128) return output_occupancy<f16, 64, 128>();
    if (d_k == 128 && d_v == 64) return output_occupancy<f16, 128, 64>();
    if (d_k == 128 && d_v == 128) return output_occupancy<f16, 128, 128>();
  } else {
    if (d_k == 64 && d_v == 64) return output_occupancy<float, 64, 64>();
    if (d_k == 64 && d_v == 128) return output_occupancy<float, 64, 128>();
  }
  return 1;
}

bool has_variant(Dtype dt, int d_k, int d_v) {
  if (dt == Dtype::kF16)
    return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
  return d_k == 64 && (d_v == 64 || d_v == 128);
}

hipError_t launch_forward(Dtype dt, int d_k, int d_v, const FwdParams& p, hipStream_t stream,
                          hipEvent_t const* ev) {
  return launch_forward_impl(dt, d_k, d_v, p, stream, ev);
}

}  // namespace gla

// Tile helpers of the attention kernels (forward and backward): the scan-order
// remap, per-sequence buffer resources and the source offsets of the
// LDS-writing tile loads.  Device code for gfx950.
#pragma once

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {

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

// Row access of the float16 kernels goes through buffer resources, one per
// tensor and sequence: offsets are 32-bit byte offsets inside the sequence's
// rows, and an offset at or past their end (kNoRow) reads zeros and drops
// stores.  Rows past the span or the sequence thus need no branch and no
// select, every load is issued unconditionally, and each wait for a staged
// tile counts exactly the loads issued after it.
constexpr uint32_t kNoRow = 0x80000000u;     // beyond every sequence (its rows span < 2 GiB)
// The rows of one (batch, head) sequence: q, k, log-alpha [T][d_k], v, out [T][d_v].
struct SeqBufs {
  rsrc_t q, k, la, v, out;
};
template <int DK, int DV>
__device__ __forceinline__ SeqBufs seq_bufs(const FwdParams& p, int bh) {
  typedef _Float16 h;
  const uint32_t kb = (uint32_t)p.T * DK * 2, vb = (uint32_t)p.T * DV * 2;
  const size_t ok = (size_t)bh * p.T * DK, ov = (size_t)bh * p.T * DV;
  SeqBufs s;
  s.q = seq_rsrc(static_cast<const h*>(p.q) + ok, kb);
  s.k = seq_rsrc(static_cast<const h*>(p.k) + ok, kb);
  s.la = seq_rsrc(static_cast<const h*>(p.la) + ok, kb);
  s.v = seq_rsrc(static_cast<const h*>(p.v) + ov, vb);
  s.out = seq_rsrc(static_cast<h*>(p.out) + ov, vb);
  return s;
}


// Chunk tiles in LDS are filled by the LDS-writing loads of gla_device.h.
// Source offset of this lane's 16 bytes in block `blk` (1 KB) of a tile with
// RB-byte rows; rows of chunk-local tokens at or past `valid` get an offset
// past the buffer, so they read as zero.  Branch-free on purpose: a lane-
// dependent branch here would split one LDS-writing load into two partial
// ones and upset the explicit wait counts.
template <int RB>
__device__ __forceinline__ uint32_t dma_offset(int blk, int t0, int valid, const GridMap& gm) {
  const int lane = threadIdx.x & 63;
  const int byte = blk * 1024 + 16 * lane;
  const int r = byte / RB, pp = (byte % RB) / 16;
  const uint32_t off = (uint32_t)gm.cell(t0 + r) * RB + (uint32_t)((pp ^ (r & 7)) * 16);
  return off | ((uint32_t)(r >= valid) << 31);
}
// The same, also handing back the row's grid cell with the out-of-range flag
// in bit 31 (for the lanes that load piece 0 of a row, first_piece is set).
template <int RB>
__device__ __forceinline__ uint32_t dma_offset_cell(int blk, int t0, int valid, const GridMap& gm,
                                                    uint32_t* cell_flag, bool* first_piece) {
  const int lane = threadIdx.x & 63;
  const int byte = blk * 1024 + 16 * lane;
  const int r = byte / RB, pp = (byte % RB) / 16;
  const uint32_t flag = (uint32_t)(r >= valid) << 31;
  const uint32_t cell = (uint32_t)gm.cell(t0 + r);
  *cell_flag = cell | flag;
  *first_piece = pp == 0;
  return (cell * RB + (uint32_t)((pp ^ (r & 7)) * 16)) | flag;
}


// The same pair for rows of `gs` bytes in memory (a block of a wider row):
// the tile still holds RB bytes per row, the source row r starts at cell * gs.
template <int RB>
__device__ __forceinline__ uint32_t dma_offset_s(int blk, int t0, int valid, const GridMap& gm,
                                                 uint32_t gs) {
  const int lane = threadIdx.x & 63;
  const int byte = blk * 1024 + 16 * lane;
  const int r = byte / RB, pp = (byte % RB) / 16;
  const uint32_t off = (uint32_t)gm.cell(t0 + r) * gs + (uint32_t)((pp ^ (r & 7)) * 16);
  return off | ((uint32_t)(r >= valid) << 31);
}
template <int RB>
__device__ __forceinline__ uint32_t dma_offset_cell_s(int blk, int t0, int valid, const GridMap& gm,
                                                      uint32_t gs, uint32_t* cell_flag,
                                                      bool* first_piece) {
  const int lane = threadIdx.x & 63;
  const int byte = blk * 1024 + 16 * lane;
  const int r = byte / RB, pp = (byte % RB) / 16;
  const uint32_t flag = (uint32_t)(r >= valid) << 31;
  const uint32_t cell = (uint32_t)gm.cell(t0 + r);
  *cell_flag = cell | flag;
  *first_piece = pp == 0;
  return (cell * gs + (uint32_t)((pp ^ (r & 7)) * 16)) | flag;
}


// ---------------------------------------------------------------------------
// Per-chunk decay helpers shared by the forward kernels.

__device__ __forceinline__ float row_bcast15(float x) {
  // every lane of a 16-lane row receives the row's lane 15 value
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x15F,
                                                             0xF, 0xF, false));
}


// log2(e) split into two binary16 values whose sum is log2(e) to ~1e-7.
constexpr float kLog2eHi = 1.4423828125f;          // fp16(log2 e)
constexpr float kLog2eLo = 1.4426950408889634f - 1.4423828125f;


// Constant 16x16x16 MFMA B operand, lane (n, g) holding rows 4g..4g+3 of
// column n: U[s][t] = (s <= t) * v.
__device__ __forceinline__ f16x4 upper_incl(float v) {
  const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  f16x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = (f16)((4 * g + u <= n16) ? v : 0.f);
  return r;
}

// Fused gate activation: log alpha = logsigmoid(z) / tau from gate logits z,
// as min(z, 0) - ln(1 + e^{-|z|}) (no overflow for any z), with ln(1 + t) by
// its series below t = 1/64, where 1 + t would drop t's low bits.
__device__ __forceinline__ float logsigmoid_scaled(float z, float inv_tau) {
  const float t = exp2_fast(-fabsf(z) * 1.4426950408889634f);
  const float series = t * (1.f - t * (0.5f - t * (1.f / 3.f)));
  const float l = t < 0.015625f ? series : __builtin_amdgcn_logf(1.f + t) * 0.6931471805599453f;
  return (fminf(z, 0.f) - l) * inv_tau;
}
// The same for a result that is rounded to float16 next: ln(1 + t) as
// log2(1 + t) ln 2 throughout.  Where 1 + t drops t's low bits (small t) the
// absolute error stays below 2^-24 / tau, under one spacing of float16 at any
// value (2^-24 is its smallest) when tau >= 1, so the rounded log-decay moves
// by at most one unit in its last place.
__device__ __forceinline__ float logsigmoid_scaled_f16(float z, float inv_tau) {
  const float t = exp2_fast(-fabsf(z) * 1.4426950408889634f);
  return fminf(z, 0.f) * inv_tau - __builtin_amdgcn_logf(1.f + t) * (0.6931471805599453f * inv_tau);
}
// Log-alpha of a transposed 16 x 16 read (lane (i, g): rows row0 + 4g + u):
// the tile value itself, or with GATE the activation of the logits there.
// Rows at or past `valid` (zero fills) must not decay, so they get 0 rather
// than logsigmoid(0).
template <bool GATE>
__device__ __forceinline__ f16x4 log_alpha_of(f16x4 x, float inv_tau, int row0, int valid) {
  if constexpr (!GATE) {
    return x;
  } else {
    f32x4 r;
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = logsigmoid_scaled_f16((float)x[u], inv_tau);
    if (row0 + 16 > valid) {  // a tile with zero-filled rows (workgroup-uniform)
      const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (row0 + 4 * g + u >= valid) r[u] = 0.f;
    }
    return to_f16(r);
  }
}

}  // namespace
}  // namespace gla

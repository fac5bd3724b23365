// Spatial SwiGLU step for gfx950 (CDNA4, MI355X):
//
//   h[b, y, x, c] = silu(G[b, y, x, c]) * (bias[c] + sum_{i,j} w[c, i, j] V[b, y+i-1, x+j-1, c])
//
// SwiGLU with a 3x3 depthwise convolution in its value branch, each channel
// filtered on its own, zero padding (GTR news write-up, tokendh.com, section
// "The flaw of one-way scanning and GTR's fix", the Spatial SwiGLU and
// depthwise-convolution notes).  G and V are the two branch projections,
// channels-last on the patch grid; the projections themselves are plain
// matrix products and stay outside this kernel.
//
// The step is a stencil that streams 6 bytes per channel per token through
// HBM (read G and V, write h) against 9 FMAs and one SiLU, so it is bound by
// HBM bandwidth and the design is about the memory side:
//
//   * a workgroup owns a tile of 64 channels x 32 columns x ROWS rows; a lane
//     owns 8 consecutive channels (16 bytes) of one column, so a wave's load
//     covers 8 whole 128-byte lines (one per token);
//   * each lane walks down its column keeping the 3x3 window of V in registers:
//     per output row it loads one new row of V (its own column and the two
//     neighbours - the neighbours are lines the same wave fetches, so they hit
//     in L1/L2) and one row of G, two rows ahead of the arithmetic;
//   * G is read and h written non-temporally (each touched once), which keeps
//     the cached V rows that neighbouring tiles read again as halo; this is
//     worth about a fifth of the kernel time on a 16K-token grid;
//   * outside the grid, past the channel count, or past the tile's rows, the
//     byte offset is set beyond the buffer, so the buffer load returns zeros
//     (which is exactly the zero padding) and the store is dropped - no branch;
//   * the 72 fp16 weights of a lane stay packed in registers; each tap is one
//     mixed-precision FMA (fp16 x fp16 products, fp32 sums);
//   * tiles are numbered so that each XCD gets a contiguous run (all spatial
//     tiles of a few channel slices), so the halo rows and columns a tile
//     shares with its neighbours are read through the same L2.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "gla_internal.h"

namespace gla {
namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kThreads = 256;
constexpr int kTileCh = 64;     // channels per workgroup tile (8 lanes x 8)
constexpr int kTileCols = 32;   // columns per workgroup tile (4 waves x 8)
constexpr int kXcds = 8;        // XCDs a launch is spread over, round robin
constexpr uint32_t kOut = 0x80000000u;      // an offset past every buffer (each < 2 GiB)
constexpr int kRawBufferWord3 = 0x00020000;  // untyped buffer, 32-bit elements

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferWord3);
}
// Cache policy of the loads and stores: kStream marks an access non-temporal,
// for data touched once (the gate rows and the outputs), so it does not push
// out the value rows that neighbouring tiles read again as their halo.
constexpr int kKeep = 0, kStream = 2;
template <int POLICY = kKeep>
__device__ __forceinline__ f16x8 load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

// silu(g) = g / (1 + e^-g), with e^-g as a hardware exp2; for g below about
// -88 the exponential is +inf and the result the correctly signed zero.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.f + e);
}

template <int ROWS>
__global__ __launch_bounds__(kThreads) void spatial_swiglu_f16_kernel(SwigluParams p) {
  // tile number, XCD-contiguous: launch slot i runs on XCD i % 8
  const int n = p.n_tiles;
  const int i = blockIdx.x;
  const int per = n / kXcds, rem = n % kXcds;
  const int x8 = i % kXcds;
  const int tile = x8 * per + (x8 < rem ? x8 : rem) + i / kXcds;
  int t = tile;
  const int ct = t % p.col_tiles;
  t /= p.col_tiles;
  const int rt = t % p.row_tiles;
  t /= p.row_tiles;
  const int cht = t % p.ch_tiles;
  const int b = t / p.ch_tiles;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = cht * kTileCh + (lane & 7) * 8;
  const int x = ct * kTileCols + wave * 8 + (lane >> 3);
  const int r0 = rt * ROWS;
  const int r1 = (r0 + ROWS < p.H) ? r0 + ROWS : p.H;   // rows [r0, r1) are written
  const bool ch_ok = c0 < p.C;
  const int W = p.W;

  const size_t img = (size_t)b * p.H * W;
  const f16* gate = static_cast<const f16*>(p.gate) + img * p.ld_in;
  const f16* value = static_cast<const f16*>(p.value) + img * p.ld_in;
  f16* out = static_cast<f16*>(p.out) + img * p.ld_out;

  // weights [C][3][3] and bias [C]: this lane's 8 channels, 72 + 8 halves
  const rsrc_t rw = make_rsrc(p.weight, (uint32_t)p.C * 18);
  const rsrc_t rb = make_rsrc(p.bias != nullptr ? p.bias : p.weight,
                              p.bias != nullptr ? (uint32_t)p.C * 2 : 0u);
  f16x8 wr[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) wr[k] = load8(rw, ch_ok ? (uint32_t)c0 * 18 + 16 * k : kOut);
  const f16x8 bias = load8(rb, ch_ok ? (uint32_t)c0 * 2 : kOut);

  // Addressing: one buffer resource per grid row (wave-uniform, built on the
  // scalar unit each step), whose range is that row's tokens - or nothing for
  // a row outside the grid, so the whole row reads zeros - and three lane
  // offsets fixed for the whole walk, set past the row for a neighbour
  // outside the grid or a lane without channels.
  const bool x_ok = ch_ok && x < W, xm_ok = x_ok && x >= 1, xp_ok = x_ok && x + 1 < W;
  const uint32_t ld2 = (uint32_t)p.ld_in * 2;
  const uint32_t oc = (uint32_t)x * ld2 + (uint32_t)c0 * 2;
  const uint32_t om = xm_ok ? oc - ld2 : kOut, o0 = x_ok ? oc : kOut, op = xp_ok ? oc + ld2 : kOut;
  const uint32_t os = x_ok ? ((uint32_t)x * p.ld_out + c0) * 2 : kOut;
  const size_t in_row = (size_t)W * p.ld_in, out_row = (size_t)W * p.ld_out;
  const uint32_t in_row_bytes = (uint32_t)(((W - 1) * (size_t)p.ld_in + p.C) * 2);
  const uint32_t out_row_bytes = (uint32_t)(((W - 1) * (size_t)p.ld_out + p.C) * 2);
  const int H = p.H;
  auto row_of = [&](const f16* base, int row) -> rsrc_t {
    const bool in = row >= 0 && row < H;
    return make_rsrc(base + (in ? row : 0) * in_row, in ? in_row_bytes : 0u);
  };

  // window rows: a = y-1, m = y, d = y+1; columns 0/1/2 = x-1, x, x+1
  rsrc_t rr = row_of(value, r0 - 1);
  f16x8 a0 = load8(rr, om), a1 = load8(rr, o0), a2 = load8(rr, op);
  rr = row_of(value, r0);
  f16x8 m0 = load8(rr, om), m1 = load8(rr, o0), m2 = load8(rr, op);
  rr = row_of(value, r0 + 1);
  f16x8 d0 = load8(rr, om), d1 = load8(rr, o0), d2 = load8(rr, op);
  f16x8 g = load8<kStream>(row_of(gate, r0), o0);
  rr = row_of(value, r0 + 2 <= r1 ? r0 + 2 : -1);
  f16x8 n0 = load8(rr, om), n1 = load8(rr, o0), n2 = load8(rr, op);
  f16x8 gn = load8<kStream>(row_of(gate, r0 + 1 < r1 ? r0 + 1 : -1), o0);

#pragma unroll
  for (int s = 0; s < ROWS; ++s) {
    const int y = r0 + s;
    if (y >= r1) break;
    // one row ahead: V row y+2 (needed up to row r1) and G row y+1 (up to r1-1)
    const rsrc_t rn = row_of(value, y + 3 <= r1 ? y + 3 : -1);
    const f16x8 nn0 = load8(rn, om), nn1 = load8(rn, o0), nn2 = load8(rn, op);
    const f16x8 gnn = load8<kStream>(row_of(gate, y + 2 < r1 ? y + 2 : -1), o0);

    // Fresh names for the window and the weights in every row step: each
    // half is then used by exactly one tap per step, so every tap becomes one
    // mixed-precision FMA on the packed halves instead of a float32 copy of
    // the window and weights being kept live across steps.
#pragma unroll
    for (int k = 0; k < 9; ++k) asm volatile("" : "+v"(wr[k]));
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(m0), "+v"(m1), "+v"(m2));
    asm volatile("" : "+v"(d0), "+v"(d1), "+v"(d2));

    f16x8 h;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // tap (i, j) of channel c is weight element c*9 + 3i + j of the lane's 72
#define TAP(i, j, vec) acc = __builtin_fmaf((float)wr[(c * 9 + 3 * (i) + (j)) >> 3][(c * 9 + 3 * (i) + (j)) & 7], (float)(vec)[c], acc)
      float acc = (float)bias[c];
      TAP(0, 0, a0); TAP(0, 1, a1); TAP(0, 2, a2);
      TAP(1, 0, m0); TAP(1, 1, m1); TAP(1, 2, m2);
      TAP(2, 0, d0); TAP(2, 1, d1); TAP(2, 2, d2);
#undef TAP
      h[c] = (f16)(silu((float)g[c]) * acc);
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h),
                                           make_rsrc(out + y * out_row, out_row_bytes), os, 0, kStream);

    a0 = m0; a1 = m1; a2 = m2;
    m0 = d0; m1 = d1; m2 = d2;
    d0 = n0; d1 = n1; d2 = n2;
    n0 = nn0; n1 = nn1; n2 = nn2;
    g = gn;
    gn = gnn;
  }
}

}  // namespace

bool swiglu_plan(SwigluParams& p) {
  int rows = p.H >= 64 ? 16 : 8;
  const char* e = std::getenv("GLA_SWIGLU_ROWS");  // tuning override: 8, 16 or 32
  if (e != nullptr) {
    const int r = std::atoi(e);
    if (r == 8 || r == 16 || r == 32) rows = r;
  }
  p.rows_per_tile = rows;
  p.row_tiles = (p.H + rows - 1) / rows;
  p.col_tiles = (p.W + kTileCols - 1) / kTileCols;
  p.ch_tiles = (p.C + kTileCh - 1) / kTileCh;
  const long long tiles = (long long)p.B * p.row_tiles * p.col_tiles * p.ch_tiles;
  if (tiles > (1LL << 31) - 1) return false;
  p.n_tiles = (int)tiles;
  return true;
}

hipError_t launch_spatial_swiglu(const SwigluParams& p, hipStream_t stream, hipEvent_t start,
                                 hipEvent_t stop) {
  const dim3 grid(p.n_tiles), block(kThreads);
  switch (p.rows_per_tile) {
    case 8:
      hipExtLaunchKernelGGL(spatial_swiglu_f16_kernel<8>, grid, block, 0, stream, start, stop, 0, p);
      break;
    case 16:
      hipExtLaunchKernelGGL(spatial_swiglu_f16_kernel<16>, grid, block, 0, stream, start, stop, 0,
                            p);
      break;
    case 32:
      hipExtLaunchKernelGGL(spatial_swiglu_f16_kernel<32>, grid, block, 0, stream, start, stop, 0,
                            p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gla

// SAGA-style non-causal gated linear attention for gfx950 (CDNA4, MI355X):
//
//   KV = (K * A)^T (V * B),      O = Q KV
//
// per (batch, head): every token's key-value map k_i^T v_i is scaled by the
// gate alpha_i^T beta_i before the maps are summed, and the Hadamard-product
// identity moves the gate onto K and V, so no per-token map is formed (SAGA
// summary, gist.science, Methodology sections A and B).
//
// Three kernels:
//   1. saga_kv_partial : one workgroup per (batch*head, span of 64-token
//      chunks) accumulates its span's (K*A)^T (V*B) on the matrix cores - the
//      key-value accumulation of the attention path's chunk summaries, with
//      the gates in place of the decay;
//   2. saga_kv_reduce  : sums the span partials in a fixed order (skipped when
//      one span covers the sequence);
//   3. saga_out        : O^T = KV^T Q^T, 16 tokens by 16 value dims per MFMA,
//      queries read straight from memory into the MFMA operand layout.
// Chunk tiles move into LDS with LDS-writing buffer loads and are read back
// transposed (gla_device.h), as in the attention kernels.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {

constexpr int kThreads = 256;   // four wave64s
constexpr int kChunk = 64;      // tokens per chunk (tile rows)
constexpr int kOutTokens = 128; // tokens per output workgroup

// Source offset of this lane's 16 bytes in block `blk` (1 KB) of a tile with
// RB-byte rows holding tokens t0.., swizzled like the attention tiles; rows
// at or past `valid` get an offset past the buffer and read as zero.
template <int RB>
__device__ __forceinline__ uint32_t tile_offset(int blk, int t0, int valid) {
  const int lane = threadIdx.x & 63;
  const int byte = blk * 1024 + 16 * lane;
  const int r = byte / RB, pp = (byte % RB) / 16;
  const uint32_t off = (uint32_t)(t0 + r) * RB + (uint32_t)((pp ^ (r & 7)) * 16);
  return off | ((uint32_t)(r >= valid) << 31);
}

template <int DK, int DV>
struct SagaTile {
  f16* k;
  f16* a;
  f16* v;
  f16* b;
};

// Kernel 1.  Wave w owns key dims 16 db.. (db = w, w + 4, ...); the map
// tile cb sits in lane (n, g) as KV^T[16 cb + 4g + u][16 db + n].  Per chunk,
// k * alpha and v * beta are formed in packed float16 from transposed tile
// reads (lane (n, g): tokens 4g..4g+3 of dim n in each 16-token sub-block)
// and KV^T += (V*B)^T (K*A) runs as 16x16x32 MFMAs over sub-block pairs.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void saga_kv_partial_kernel(SagaParams p) {
  // eight separate LDS objects, so the compiler's own waits for the
  // LDS-writing loads can tell the tiles apart
  __shared__ __attribute__((aligned(16))) f16 k0[kChunk * DK], a0[kChunk * DK], v0[kChunk * DV],
      b0[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 k1[kChunk * DK], a1[kChunk * DK], v1[kChunk * DV],
      b1[kChunk * DV];
  const SagaTile<DK, DV> slot0{k0, a0, v0, b0}, slot1{k1, a1, v1, b1};
  constexpr int NDB = DK / 64, NCB = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  constexpr int NBK = RBK / 64, NBV = RBV / 64;  // 1 KB blocks per wave and tile
  constexpr int NDMA = 2 * NBK + 2 * NBV;         // LDS-writing loads per wave and chunk
  static_assert(NDMA < 64, "vmcnt range");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int bh = blockIdx.x / p.n_spans;
  const int span = blockIdx.x - bh * p.n_spans;
  const size_t ok = (size_t)bh * p.N * DK, ov = (size_t)bh * p.N * DV;
  const rsrc_t rk = seq_rsrc(static_cast<const f16*>(p.k) + ok, (uint32_t)p.N * RBK);
  const rsrc_t ra = seq_rsrc(static_cast<const f16*>(p.a) + ok, (uint32_t)p.N * RBK);
  const rsrc_t rv = seq_rsrc(static_cast<const f16*>(p.v) + ov, (uint32_t)p.N * RBV);
  const rsrc_t rb = seq_rsrc(static_cast<const f16*>(p.b) + ov, (uint32_t)p.N * RBV);
  const int c_begin = span * p.span_chunks;
  const int c_end = min(c_begin + p.span_chunks, p.n_chunks);

  // Fill a tile buffer with chunk c; a chunk past the span loads nothing.
  auto issue = [&](const SagaTile<DK, DV>& s, int c) {
    const int t0 = c * kChunk;
    const int valid = c < c_end ? min(kChunk, p.N - t0) : 0;
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = wave * NBK + i;
      const uint32_t off = tile_offset<RBK>(blk, t0, valid);
      dma16(rk, s.k + blk * 512, off);
      dma16(ra, s.a + blk * 512, off);
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int blk = wave * NBV + i;
      const uint32_t off = tile_offset<RBV>(blk, t0, valid);
      dma16(rv, s.v + blk * 512, off);
      dma16(rb, s.b + blk * 512, off);
    }
  };

  f32x4 st[NDB][NCB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st[d][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fold = [&](const SagaTile<DK, DV>& s) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int db = wave + 4 * d;
      f16x4 ka[4];
#pragma unroll
      for (int J = 0; J < 4; ++J)
        ka[J] = tr_read<RBK>(s.k, 16 * J, 16 * db) * tr_read<RBK>(s.a, 16 * J, 16 * db);
#pragma unroll
      for (int P = 0; P < 2; ++P) {
        const f16x8 bk = cat8(ka[2 * P], ka[2 * P + 1]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const f16x4 lo = tr_read<RBV>(s.v, 32 * P, 16 * cb) * tr_read<RBV>(s.b, 32 * P, 16 * cb);
          const f16x4 hi =
              tr_read<RBV>(s.v, 32 * P + 16, 16 * cb) * tr_read<RBV>(s.b, 32 * P + 16, 16 * cb);
          st[d][cb] = mma32(cat8(lo, hi), bk, st[d][cb]);
        }
      }
    }
  };

  issue(slot0, c_begin);
  issue(slot1, c_begin + 1);
  for (int c = c_begin; c < c_end; c += 2) {
    wait_barrier<vmcnt_imm(NDMA)>();  // every wave's part of slot0 has landed
    fold(slot0);
    wait_barrier<kLgkmZero>();        // every wave's reads of slot0 are done
    issue(slot0, c + 2);
    wait_barrier<vmcnt_imm(NDMA)>();
    if (c + 1 < c_end) fold(slot1);
    wait_barrier<kLgkmZero>();
    issue(slot1, c + 3);
  }
  // the trailing loads target chunks past the span (zero fills): let them land
  // before the workgroup's LDS can be handed on
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  float* dst = p.n_spans == 1 ? p.kv + (size_t)bh * DK * DV
                              : p.partial + ((size_t)bh * p.n_spans + span) * DK * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int dim = 16 * (wave + 4 * d) + n16;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<f32x4*>(dst + dim * DV + 16 * cb + 4 * g) = st[d][cb];
  }
}

// Kernel 2: kv[bh] = sum over spans of the partials, in span order.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void saga_kv_reduce_kernel(SagaParams p) {
  const int bh = blockIdx.x;
  const int e = (blockIdx.y * kThreads + threadIdx.x) * 4;
  const float* src = p.partial + (size_t)bh * p.n_spans * DK * DV + e;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.n_spans; ++s) acc += *reinterpret_cast<const f32x4*>(src + (size_t)s * DK * DV);
  *reinterpret_cast<f32x4*>(p.kv + (size_t)bh * DK * DV + e) = acc;
}

// Kernel 3.  Wave w owns value dims 16 jb.. (jb = w, w + 4, ...).  Its MFMA A
// operands are KV^T rows 16 jb + n, key dims 32 rho + 8g .. + 7 (lane (n, g)),
// scaled by a power of two that brings the wave's largest |KV| entry to
// [2^14, 2^15) before the float16 conversion (exact to undo, and it keeps
// both large and tiny maps inside float16); the B operand of 16 tokens is
// lane (n, g) = the 16 bytes of token n at key dims 32 rho + 8g, loaded
// straight from memory.  Out lane (n, g) holds tokens n, value dims
// 16 jb + 4g .. + 3: one 8-byte store.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void saga_out_kernel(SagaParams p) {
  constexpr int NRHO = DK / 32, NJW = DV / 64;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / p.n_tblocks;
  const int t_begin = (blockIdx.x - bh * p.n_tblocks) * kOutTokens;

  const rsrc_t rq = seq_rsrc(static_cast<const f16*>(p.q) + (size_t)bh * p.N * DK, (uint32_t)p.N * RBK);
  const rsrc_t ro = seq_rsrc(static_cast<f16*>(p.out) + (size_t)bh * p.N * DV, (uint32_t)p.N * RBV);
  const float* kv = p.kv + (size_t)bh * DK * DV;

  f16x8 am[NJW][NRHO];
  float unscale[NJW];
#pragma unroll
  for (int jj = 0; jj < NJW; ++jj) {
    const int j = 16 * (wave + 4 * jj) + n16;
    float vals[NRHO][8];
    float mx = 0.f;
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vals[rho][e] = kv[(32 * rho + 8 * g + e) * DV + j];
        mx = fmaxf(mx, fabsf(vals[rho][e]));
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    int ex = 0;
    (void)frexpf(mx, &ex);                    // mx = f * 2^ex, f in [0.5, 1)
    const int sh = (mx > 0.f) ? 15 - ex : 0;  // scaled maximum in [2^14, 2^15)
    const float scale = ldexpf(1.f, sh);
    unscale[jj] = ldexpf(1.f, -sh);
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho)
#pragma unroll
      for (int e = 0; e < 8; ++e) am[jj][rho][e] = (f16)(vals[rho][e] * scale);
  }

#pragma unroll
  for (int T = 0; T < kOutTokens / 16; ++T) {
    const int t = t_begin + 16 * T + n16;
    const uint32_t row_ok = t < p.N ? 0u : 0x80000000u;
    f16x8 qb[NRHO];
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho)
      qb[rho] = __builtin_bit_cast(
          f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                     rq, ((uint32_t)t * RBK + (uint32_t)(32 * rho + 8 * g) * 2) | row_ok, 0, 0));
#pragma unroll
    for (int jj = 0; jj < NJW; ++jj) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rho = 0; rho < NRHO; ++rho) acc = mma32(am[jj][rho], qb[rho], acc);
      const f16x4 o = to_f16(acc * unscale[jj]);
      const int jb = wave + 4 * jj;
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(u32x2, o), ro,
          ((uint32_t)t * RBV + (uint32_t)(16 * jb + 4 * g) * 2) | row_ok, 0, 0);
    }
  }
}

template <class K>
hipError_t launch_k(K kernel, dim3 grid, hipStream_t stream, const SagaParams& p,
                    hipEvent_t const* ev, int slot) {
  if (ev != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, ev[2 * slot], ev[2 * slot + 1],
                          0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_saga_variant(const SagaParams& p, hipStream_t stream, hipEvent_t const* ev) {
  const int BH = p.B * p.heads;
  hipError_t e;
  if ((e = launch_k(saga_kv_partial_kernel<DK, DV>, dim3(BH * p.n_spans), stream, p, ev, 0)) !=
      hipSuccess)
    return e;
  if (p.n_spans > 1) {
    if ((e = launch_k(saga_kv_reduce_kernel<DK, DV>, dim3(BH, DK * DV / (4 * kThreads)), stream, p,
                      ev, 1)) != hipSuccess)
      return e;
  } else if (ev != nullptr) {
    if ((e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  }
  return launch_k(saga_out_kernel<DK, DV>, dim3(BH * p.n_tblocks), stream, p, ev, 2);
}

}  // namespace

int saga_chunk_tokens() { return kChunk; }
int saga_out_tokens() { return kOutTokens; }

bool saga_has_variant(int d_k, int d_v) {
  return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
}

hipError_t launch_saga(const SagaParams& p, hipStream_t stream, hipEvent_t const* ev) {
  if (p.d_k == 64 && p.d_v == 64) return launch_saga_variant<64, 64>(p, stream, ev);
  if (p.d_k == 64 && p.d_v == 128) return launch_saga_variant<64, 128>(p, stream, ev);
  if (p.d_k == 128 && p.d_v == 64) return launch_saga_variant<128, 64>(p, stream, ev);
  if (p.d_k == 128 && p.d_v == 128) return launch_saga_variant<128, 128>(p, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace gla

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
//   1. saga_kv_partial : one workgroup per (batch*head, span of 32-token
//      steps) accumulates its span's (K*A)^T (V*B) on the matrix cores - the
//      key-value accumulation of the attention path's chunk summaries, with
//      the gates in place of the decay;
//   2. saga_kv_reduce  : sums the span partials in a fixed order, writes the
//      map, and writes kernel 3's MFMA A operands (the map transposed, scaled
//      by a power of two per operand of 16 value dims x 32 key dims, float16)
//      once per (batch*head), so that the output workgroups only load them;
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
constexpr int kStepTokens = 32; // tokens per accumulation step (tile rows)
constexpr int kOutTokens = 256; // tokens per output workgroup

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

// LDS-writing load with the non-temporal policy: the accumulation reads its
// inputs exactly once, so they are kept from displacing cached data (about
// 10 % faster on the 16K-token workload).
__device__ __forceinline__ void dma16_stream(rsrc_t src, f16* block, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)block, 16, off, 0, 0, 2);
}

template <int DK, int DV>
struct SagaTile {
  f16* k;
  f16* a;
  f16* v;
  f16* b;
};

// Kernel 1.  One workgroup per (batch*head, span of 32-token steps).  Wave w
// owns key dims 16 db.. (db = w, w + 4, ...); the map tile cb sits in lane
// (n, g) as KV^T[16 cb + 4g + u][16 db + n].  Per step, k * alpha and v * beta
// are formed in packed float16 from transposed tile reads (lane (n, g):
// tokens 4g..4g+3 of dim n in each 16-token half) and KV^T += (V*B)^T (K*A)
// is one 16x16x32 MFMA per (db, cb) tile.  Two step buffers: the next step
// loads while this one is folded.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void saga_kv_partial_kernel(SagaParams p) {
  constexpr int T = kStepTokens;
  // eight separate LDS objects, so the compiler's own waits for the
  // LDS-writing loads can tell the tiles apart
  __shared__ __attribute__((aligned(16))) f16 k0[T * DK], a0[T * DK], v0[T * DV], b0[T * DV];
  __shared__ __attribute__((aligned(16))) f16 k1[T * DK], a1[T * DK], v1[T * DV], b1[T * DV];
  const SagaTile<DK, DV> slot0{k0, a0, v0, b0}, slot1{k1, a1, v1, b1};
  constexpr int NDB = DK / 64, NCB = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  constexpr int NBK = RBK * T / 4096, NBV = RBV * T / 4096;  // 1 KB blocks per wave and tile
  constexpr int NDMA = 2 * NBK + 2 * NBV;                     // LDS-writing loads per wave and step
  static_assert(NBK >= 1 && NBV >= 1 && NDMA < 64, "tile split");
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

  // Fill a tile buffer with step c; a step past the span loads nothing.
  auto issue = [&](const SagaTile<DK, DV>& s, int c) {
    const int t0 = c * T;
    const int valid = c < c_end ? min(T, p.N - t0) : 0;
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = wave * NBK + i;
      const uint32_t off = tile_offset<RBK>(blk, t0, valid);
      dma16_stream(rk, s.k + blk * 512, off);
      dma16_stream(ra, s.a + blk * 512, off);
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int blk = wave * NBV + i;
      const uint32_t off = tile_offset<RBV>(blk, t0, valid);
      dma16_stream(rv, s.v + blk * 512, off);
      dma16_stream(rb, s.b + blk * 512, off);
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
      const f16x8 bk = cat8(tr_read<RBK>(s.k, 0, 16 * db) * tr_read<RBK>(s.a, 0, 16 * db),
                            tr_read<RBK>(s.k, 16, 16 * db) * tr_read<RBK>(s.a, 16, 16 * db));
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f16x4 lo = tr_read<RBV>(s.v, 0, 16 * cb) * tr_read<RBV>(s.b, 0, 16 * cb);
        const f16x4 hi = tr_read<RBV>(s.v, 16, 16 * cb) * tr_read<RBV>(s.b, 16, 16 * cb);
        st[d][cb] = mma32(cat8(lo, hi), bk, st[d][cb]);
      }
    }
  };

  issue(slot0, c_begin);
  issue(slot1, c_begin + 1);
  for (int c = c_begin; c < c_end; c += 2) {
    prio_by_progress(c - c_begin, c_end - c_begin);
    wait_barrier<vmcnt_imm(NDMA)>();  // every wave's part of slot0 has landed
    fold(slot0);
    wait_barrier<kLgkmZero>();        // every wave's reads of slot0 are done
    issue(slot0, c + 2);
    wait_barrier<vmcnt_imm(NDMA)>();
    if (c + 1 < c_end) fold(slot1);
    wait_barrier<kLgkmZero>();
    issue(slot1, c + 3);
  }
  // the trailing loads target steps past the span (zero fills): let them land
  // before the workgroup's LDS can be handed on
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  float* dst = p.partial + ((size_t)bh * p.n_spans + span) * DK * DV;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int dim = 16 * (wave + 4 * d) + n16;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<f32x4*>(dst + dim * DV + 16 * cb + 4 * g) = st[d][cb];
  }
}

// Kernel 2.  One workgroup of G waves per (batch*head, pair of MFMAs 2s and
// 2s + 1 of the output kernel, key block rho of 32 dims): value dims
// 32 s .. 32 s + 31 (whole 128-byte lines of the partials) over the key dims
// of rho.  Wave w sums the span partials s' = w, w + G, .. of its elements in
// order, the sums are added in a fixed order (results are bitwise
// reproducible), then the map is written (when wanted) and, through LDS,
// transposed into the output kernel's A operands (m, rho): lane (n, g) holds
// KV^T[value dim of row n][key dims 32 rho + 8g .. + 7] times 2^sh, sh
// bringing the largest |KV| of the operand into [2^14, 2^15) (exact to undo;
// it keeps both large and tiny maps inside float16).
template <int DK, int DV, int G>
__global__ __launch_bounds__(64 * G) void saga_kv_reduce_kernel(SagaParams p) {
  constexpr int NQ = 4;                   // float4 pieces per lane: 32 key dims x 8 pieces / 64
  constexpr int NRHO = DK / 32;
  __shared__ f32x4 part[G - 1][64 * NQ];
  __shared__ float tile[32][2][17];       // [key dim in rho][m - 2s][row r of MFMA m], padded
  __shared__ float wmax[2];
  const int bh = blockIdx.x, s2 = blockIdx.y, rho = blockIdx.z;
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  // piece j of this lane: key dim 32 rho + (64 j + lane) / 8, value dims
  // 32 s2 + 4 q .. + 3 with q = lane % 8: rows 4 (q / 2) .. + 3 of MFMA
  // 2 s2 + (q % 2)
  f32x4 acc[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* src = p.partial + (size_t)bh * p.n_spans * DK * DV + 32 * rho * DV + 32 * s2;
  for (int s = grp; s < p.n_spans; s += G) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = (64 * j + lane) >> 3, q = lane & 7;
      acc[j] += *reinterpret_cast<const f32x4*>(src + (size_t)s * DK * DV + i * DV + 4 * q);
    }
  }
  if (grp > 0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) part[grp - 1][64 * j + lane] = acc[j];
  }
  __syncthreads();
  if (grp == 0) {
    float mx[2] = {0.f, 0.f};
    const int q = lane & 7, h = q & 1;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      f32x4 sum = acc[j];
#pragma unroll
      for (int w = 0; w < G - 1; ++w) sum = sum + part[w][64 * j + lane];
      const int i = (64 * j + lane) >> 3;
      if (p.kv != nullptr)
        *reinterpret_cast<f32x4*>(p.kv + (size_t)bh * DK * DV + (32 * rho + i) * DV + 32 * s2 +
                                  4 * q) = sum;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        tile[i][h][4 * (q >> 1) + u] = sum[u];
        mx[h] = fmaxf(mx[h], fabsf(sum[u]));
      }
    }
    // lanes of one parity hold MFMA 2 s2 + parity: reduce each over its lanes
#pragma unroll
    for (int k = 32; k >= 2; k >>= 1) {
      mx[0] = fmaxf(mx[0], __shfl_xor(mx[0], k));
      mx[1] = fmaxf(mx[1], __shfl_xor(mx[1], k));
    }
    if (lane < 2) wmax[lane] = mx[lane];
  }
  __syncthreads();
  if (grp < 2) {
    // wave h writes operand (2 s2 + h, rho)
    const int h = grp, m = 2 * s2 + h;
    const float mx = wmax[h];
    int ex = 0;
    (void)frexpf(mx, &ex);                    // mx = f * 2^ex, f in [0.5, 1)
    const int sh = (mx > 0.f) ? 15 - ex : 0;  // scaled maximum in [2^14, 2^15)
    const float scale = ldexpf(1.f, sh);
    const size_t op = ((size_t)bh * (DV / 16) + m) * NRHO + rho;
    if (lane == 0) p.unscale[op] = ldexpf(1.f, -sh);
    const int n = lane & 15, g = lane >> 4;
    f16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (f16)(tile[8 * g + e][h][n] * scale);
    static_cast<f16x8*>(p.amap)[op * 64 + lane] = x;
  }
}

// Kernel 3.  Each wave takes 16-token blocks of its workgroup's 256 tokens and
// computes all value dims, as O^T = KV^T Q^T in 16x16x32 MFMAs (rows: value
// dims, columns: tokens, reduction: key dims).
//  * B operand: lane (n, g) holds the 16 bytes of token n at key dims
//    32 rho + 8g .. + 7, loaded straight from memory (64 bytes per token per
//    instruction).
//  * A operands: MFMA m's row r is value dim 32 (m / 2) + 8 (r / 4) +
//    4 (m % 2) + r % 4, so lane (n, g) ends up with value dims
//    32 s + 8g .. + 7 of token n from MFMAs 2s and 2s + 1: one 16-byte store
//    per s, and the four lane groups of a store fill 64 contiguous bytes.
//    Kernel 2 has laid them out (scaled float16, one 16-byte load per lane
//    and operand); each MFMA's result is multiplied by its inverse scale.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void saga_out_kernel(SagaParams p) {
  constexpr int NRHO = DK / 32, NM = DV / 16;
  constexpr int RBK = 2 * DK, RBV = 2 * DV;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / p.n_tblocks;
  const int t_begin = (blockIdx.x - bh * p.n_tblocks) * kOutTokens;

  const rsrc_t rq = seq_rsrc(static_cast<const f16*>(p.q) + (size_t)bh * p.N * DK, (uint32_t)p.N * RBK);
  const rsrc_t ro = seq_rsrc(static_cast<f16*>(p.out) + (size_t)bh * p.N * DV, (uint32_t)p.N * RBV);
  const f16x8* amap = static_cast<const f16x8*>(p.amap) + (size_t)bh * (DV / 16) * NRHO * 64;

  // With 64 key dims every block's queries are requested first, so their
  // latency overlaps the map reads below; with 128 the registers this takes
  // cost more occupancy than the overlap gains, and each block loads its own.
  constexpr int NBLK = kOutTokens / 64;
  constexpr bool kAhead = DK == 64;
  auto load_q = [&](f16x8* qv, int blk) {
    const int t = t_begin + 16 * (4 * blk + wave) + n16;
    const uint32_t ok = t < p.N ? 0u : 0x80000000u;
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho)
      qv[rho] = __builtin_bit_cast(
          f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                     rq, ((uint32_t)t * RBK + (uint32_t)(32 * rho + 8 * g) * 2) | ok, 0, 0));
  };
  f16x8 qa[kAhead ? NBLK : 1][NRHO];
  if constexpr (kAhead) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) load_q(qa[blk], blk);
  }

  f16x8 am[NM][NRHO];
  float unscale[NM][NRHO];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int rho = 0; rho < NRHO; ++rho) {
      am[m][rho] = amap[(m * NRHO + rho) * 64 + lane];
      unscale[m][rho] = p.unscale[((size_t)bh * NM + m) * NRHO + rho];
    }
  }

#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    const int t = t_begin + 16 * (4 * blk + wave) + n16;
    const uint32_t row_ok = t < p.N ? 0u : 0x80000000u;
    f16x8 qn[NRHO];
    if constexpr (!kAhead) load_q(qn, blk);
    const f16x8* qb = kAhead ? qa[blk] : qn;
#pragma unroll
    for (int s2 = 0; s2 < NM / 2; ++s2) {
      f32x4 acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rho = 0; rho < NRHO; ++rho) {
          // each key block carries its own scale: undo it before adding
          const f32x4 part = mma32(am[2 * s2 + h][rho], qb[rho], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[h] += part * unscale[2 * s2 + h][rho];
        }
      }
      const f16x8 o = cat8(to_f16(acc[0]), to_f16(acc[1]));
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, o), ro,
          ((uint32_t)t * RBV + (uint32_t)(32 * s2 + 8 * g) * 2) | row_ok, 0, 0);
    }
  }
}

template <class K>
hipError_t launch_k(K kernel, dim3 grid, hipStream_t stream, const SagaParams& p,
                    hipEvent_t const* ev, int slot, int threads = kThreads) {
  if (ev != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, ev[2 * slot], ev[2 * slot + 1],
                          0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, p);
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
  // eight waves split long span lists, four short ones (measured: 64 spans
  // per sequence 5.4 against 7.3 us; 2 spans 8.4 against 14.1 us)
  const dim3 rgrid(BH, DV / 32, DK / 32);
  e = p.n_spans >= 16 ? launch_k(saga_kv_reduce_kernel<DK, DV, 8>, rgrid, stream, p, ev, 1, 512)
                      : launch_k(saga_kv_reduce_kernel<DK, DV, 4>, rgrid, stream, p, ev, 1, 256);
  if (e != hipSuccess) return e;
  return launch_k(saga_out_kernel<DK, DV>, dim3(BH * p.n_tblocks), stream, p, ev, 2);
}

}  // namespace

int saga_chunk_tokens() { return kStepTokens; }
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

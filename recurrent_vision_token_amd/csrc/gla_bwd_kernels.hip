// Backward pass of the chunkwise gated linear attention with key-only decay,
// for gfx950 (CDNA4, MI355X), float16 tensors, d_k = d_v = 64.
//
// Gradients of L = <dO, O> + <dS_final, S_final> for the recurrence
// S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t (GTR news write-up,
// tokendh.com, section "What linear attention saves"), computed chunkwise
// like the forward pass (section "Where the speed comes from"): the state's
// adjoint G_t = dL/dS_t runs backwards along the scan,
// G_t = q_t^T dO_t + diag(alpha_{t+1}) G_{t+1}, which is the forward
// recurrence read from the end, so the same summary / scan kernels give
//   E_c : the forward state entering chunk c (summaries of k, v), and
//   R_c : the adjoint entering chunk c from its right,
//         R_{c-1} = diag(g_c) R_c + (Q * exp(B))^T dO  over chunk c,
// after which every chunk is independent.  With B the inclusive cumulative
// log-decay inside the chunk, for t, s in the chunk:
//   dq_t = e^{B_t} E_c dO_t + sum_{s<=t} (dO_t . v_s) k_s e^{B_t - B_s}
//   dk_t = e^{B_end - B_t} R_c v_t + sum_{s>=t} (v_t . dO_s) q_s e^{B_s - B_t}
//   dv_t = (k_t e^{B_end - B_t}) R_c + sum_{s>=t} ((k_t e^{-B_t}) . (q_s e^{B_s})) dO_s
//   dlog_alpha_t = sum_{s>=t, s in chunk} (q_s dq_s - k_s dk_s) + rowsum(E_{c+1} * R_c)
// (the last term is the same sum over every later token, by the adjoint
// identity dlog_alpha_t = alpha_t * rowsum(G_t * S_{t-1}) at the chunk's end).
//
// The state kernels work on spans of one chunk, so every chunk finds both of
// its states (float16) in memory.  The chunk kernel (one workgroup per
// (batch*head, chunk), wave w owning key dims and value dims 16w..16w+15):
//   1. q, k, v, log-alpha and dO land in LDS (LDS-writing loads, swizzled
//      rows); B is summed per key dim in float32;
//   2. float16 operand tiles with every decay factor bounded: Qs = q e^{c}
//      (c = B - B at the 16-token sub-block start, in [-10, 0]), Kd = k decayed
//      to its sub-block's end, Ke = k decayed to the chunk's end; the diagonal
//      sub-blocks use Kd times the sub-block decay back (<= e^10), and the
//      factors between sub-blocks (<= 1) scale 16x16 accumulators in float32;
//   3. the score tiles dO V^T, V dO^T and (Q e^B)(K e^-B)^T are formed per
//      sub-block pair on the matrix cores (every wave forms the ones it needs;
//      the accumulator of one is the next MFMA's operand, no LDS round trip),
//      then dq, dk, dv as 16x16 MFMA tiles, outputs rounded to float16 and
//      stored to their grid cells (scan-order remap as in the forward pass);
//   4. E_{c+1} = diag(e^{B_end}) E_c + Ke^T V, its row sums against R_c give
//      the carry, and dlog_alpha is a suffix sum across the 16 lanes of each
//      tile row plus the later sub-blocks' totals.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"
#include "gla_tiles.h"

namespace gla {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

__device__ __forceinline__ float ex(float x) { return exp2_fast(x * 1.4426950408889634f); }

// DPP moves within the 16-lane rows of a wave: lane n of a row reads lane
// n + k of the same row (zero past the row's end), or every lane reads lane k.
constexpr int kRowShl = 0x100, kRowBcast = 0x150;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void chunk_bwd_f16_kernel(BwdParams p) {
  static_assert(DK == 64 && DV == 64, "built for 64 key and value dims");
  constexpr int RB = 128;  // bytes per tile row
  // row stride (floats) of sEc: 4 floats of padding move consecutive rows 4
  // banks apart, so 16 lanes reading 16 bytes each from 16 rows hit 64
  // different banks
  constexpr int ES = DK + 4;
  __shared__ __attribute__((aligned(16))) f16 tq[kChunk * DK], tk[kChunk * DK], tv[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 tla[kChunk * DK], tdo[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 tqs[kChunk * DK], tkd[kChunk * DK];
  __shared__ __attribute__((aligned(16))) float sEc[kChunk * ES];  // e^{c_t}, c = decay since the sub-block start
  __shared__ __attribute__((aligned(16))) f16 sF[5][5][DK];  // e^{Bst_a - Bst_b} per key dim
  __shared__ float sTot[4][DK];
  __shared__ float sBst[5][DK];   // B before sub-block I (I = 0..3), [4] = chunk total
  __shared__ float sCarry[4][DK];
  __shared__ uint32_t srow[kChunk];
  f16* const tke = tla;           // k decayed to the chunk end, in place of log-alpha

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  const int bh = blockIdx.x / p.n_chunks;
  const int c = blockIdx.x - bh * p.n_chunks;
  const int b = bh / p.heads;
  GridMap gm;
  gm.H = p.H;
  gm.W = p.W;
  gm.dir = (p.scan_dir == 4) ? (b & 3) : p.scan_dir;
  gm.mw = p.div_w_m;
  gm.mh = p.div_h_m;
  gm.sw = p.div_w_s;
  gm.sh = p.div_h_s;

  // rows of ldk (q, k, log-alpha and their gradients) or ldv (v, d_out, dv)
  // elements: this block's 64 dims of a wider head, or the whole row
  const uint32_t gsk = p.ldk * 2u, gsv = p.ldv * 2u;  // row strides in bytes
  const uint32_t kbytes = (uint32_t)p.T * gsk, vbytes = (uint32_t)p.T * gsv;
  const size_t sok = (size_t)bh * p.T * p.ldk, sov = (size_t)bh * p.T * p.ldv;
  const rsrc_t rq = seq_rsrc(static_cast<const f16*>(p.q) + sok, kbytes);
  const rsrc_t rk = seq_rsrc(static_cast<const f16*>(p.k) + sok, kbytes);
  const rsrc_t rla = seq_rsrc(static_cast<const f16*>(p.la) + sok, kbytes);
  const rsrc_t rv = seq_rsrc(static_cast<const f16*>(p.v) + sov, vbytes);
  const rsrc_t rdo = seq_rsrc(static_cast<const f16*>(p.dout) + sov, vbytes);
  const rsrc_t wdq = seq_rsrc(static_cast<f16*>(p.dq) + sok, kbytes);
  const rsrc_t wdk = seq_rsrc(static_cast<f16*>(p.dk) + sok, kbytes);
  const rsrc_t wdv = seq_rsrc(static_cast<f16*>(p.dv) + sov, vbytes);
  const rsrc_t wdla = seq_rsrc(static_cast<f16*>(p.dla) + sok, kbytes);
  // the states of this chunk, float16 from the scans: the forward state
  // entering it and the adjoint entering it from the right
  const f16* E_c = static_cast<const f16*>(p.fwd_state) + ((size_t)bh * p.n_chunks + c) * DK * DV;
  const f16* R_c = static_cast<const f16*>(p.adj_state) +
                   ((size_t)bh * p.n_chunks + (p.n_chunks - 1 - c)) * DK * DV;
  const int kb = wave;          // key dims 16 kb .. owned by this wave (dq, dk, dla)
  const int vb = wave;          // value dims 16 vb .. (dv, next state rows)
  const int ki = 16 * kb + 4 * g;  // first of the lane's 4 key dims in a dq / dk tile
  const int vj = 16 * vb + 4 * g;

  // ---- 0. the states, read from memory before the tiles so that their
  // latency hides behind the tiles': E and R in the accumulator layout of the
  // next-state update (rows 16 kc + n, columns 16 w + 4g ..) and in the MFMA
  // operand layouts below (raw float16 bits until the tiles landed; 32-bit
  // byte offsets from the state bases, so each load is one uniform base plus
  // one lane offset)
  u32x2 e4h[4], r4h[4], eah[4], rah[4];
  unsigned short rtah[16];
  auto ld4 = [](const f16* base, uint32_t byte_off) {
    return *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(base) + byte_off);
  };
  auto ld1 = [](const f16* base, uint32_t byte_off) {
    return *reinterpret_cast<const unsigned short*>(reinterpret_cast<const char*>(base) + byte_off);
  };
  const uint32_t o_acc = 2u * (uint32_t)(n16 * DV + vj);            // row n, columns vj ..
  const uint32_t o_op = 2u * (uint32_t)((16 * kb + n16) * DV + 8 * g);  // row 16 kb + n, cols 8g ..
  const uint32_t o_t = 2u * (uint32_t)(8 * g * DV + 16 * vb + n16);   // R[8g][16 vb + n]
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    e4h[kc] = ld4(E_c, o_acc + 2u * 16 * kc * DV);
    r4h[kc] = ld4(R_c, o_acc + 2u * 16 * kc * DV);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    eah[2 * h] = ld4(E_c, o_op + 2u * 32 * h);
    eah[2 * h + 1] = ld4(E_c, o_op + 2u * (32 * h + 4));
    rah[2 * h] = ld4(R_c, o_op + 2u * 32 * h);
    rah[2 * h + 1] = ld4(R_c, o_op + 2u * (32 * h + 4));
    // R^T rows 16 vb + n: R[32 h + 8g + e][16 vb + n]
#pragma unroll
    for (int e = 0; e < 8; ++e) rtah[8 * h + e] = ld1(R_c, o_t + 2u * (32 * h + e) * DV);
  }

  // ---- 1. tiles, cumulative decay
  const int t0 = c * kChunk;
  const int valid = min(kChunk, p.T - t0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = wave * 2 + i;
    uint32_t cf;
    bool first;
    const uint32_t off = dma_offset_cell_s<RB>(blk, t0, valid, gm, gsk, &cf, &first);
    const uint32_t offv = dma_offset_s<RB>(blk, t0, valid, gm, gsv);
    if (first) srow[(blk * 1024 + 16 * lane) / RB] = cf;
    dma16(rq, tq + blk * 512, off);
    dma16(rk, tk + blk * 512, off);
    dma16(rv, tv + blk * 512, offv);
    dma16(rla, tla + blk * 512, off);
    dma16(rdo, tdo + blk * 512, offv);
  }
  wait_barrier<vmcnt_lgkm0_imm(0)>();  // tiles landed, row table written
  // the raw state values are used from here on only: the empty asm keeps their
  // conversions (and so the compiler's waits for them) after the wait above
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    asm volatile("" : "+v"(eah[j]), "+v"(rah[j]));
    asm volatile("" : "+v"(e4h[j]), "+v"(r4h[j]));
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(rtah[j]));
  auto wide = [](u32x2 x) {
    const f16x4 h = __builtin_bit_cast(f16x4, x);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  };
  f32x4 e4s[4], r4s[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    e4s[kc] = wide(e4h[kc]);
    r4s[kc] = wide(r4h[kc]);
  }
  // this chunk's states as float16 MFMA A operands: E and R rows of the
  // wave's key dims (lane (n, g): row 16 kb + n, columns 32 h + 8g .. + 7) and
  // R^T rows of its value dims
  f16x8 ea[2], ra[2], rta[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ea[h] = cat8(__builtin_bit_cast(f16x4, eah[2 * h]), __builtin_bit_cast(f16x4, eah[2 * h + 1]));
    ra[h] = cat8(__builtin_bit_cast(f16x4, rah[2 * h]), __builtin_bit_cast(f16x4, rah[2 * h + 1]));
    f16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __builtin_bit_cast(f16, rtah[8 * h + e]);
    rta[h] = x;
  }

  // Thread (key dims 2 i2, 2 i2 + 1; tokens 8h .. 8h + 7 of sub-block J, its
  // wave) walks its tokens: alpha_t = e^{la_t}, e^{c_t} as a running product
  // from the sub-block start and the decay to the sub-block end as a running
  // product from its end, one exponential per token; the two halves of a
  // sub-block (lanes l and l ^ 32) hand each other their decay products.
  {
    const int i2 = tid & 31, h = (tid >> 5) & 1, J = tid >> 6;
    const int i = 2 * i2;
    float al0[8], al1[8];
    float tot0 = 0.f, tot1 = 0.f, p0 = 1.f, p1 = 1.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f16x2 la2 = *reinterpret_cast<const f16x2*>(&tla[swz<RB>(16 * J + 8 * h + u, i)]);
      const float l0 = (float)la2[0], l1 = (float)la2[1];
      al0[u] = ex(l0);
      al1[u] = ex(l1);
      tot0 += l0;
      tot1 += l1;
      p0 *= al0[u];
      p1 *= al1[u];
    }
    const float o0 = __shfl_xor(p0, 32), o1 = __shfl_xor(p1, 32);
    const float ot0 = __shfl_xor(tot0, 32), ot1 = __shfl_xor(tot1, 32);
    float ec0 = h ? o0 : 1.f, ec1 = h ? o1 : 1.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 16 * J + 8 * h + u;
      const int e = swz<RB>(t, i);
      ec0 *= al0[u];
      ec1 *= al1[u];
      *reinterpret_cast<f32x2*>(&sEc[t * ES + i]) = f32x2{ec0, ec1};
      const f16x2 q2 = *reinterpret_cast<const f16x2*>(&tq[e]);
      *reinterpret_cast<f16x2*>(&tqs[e]) = f16x2{(f16)((float)q2[0] * ec0), (f16)((float)q2[1] * ec1)};
    }
    float sfx0 = h ? 1.f : o0, sfx1 = h ? 1.f : o1, kf0[8], kf1[8];
#pragma unroll
    for (int u = 7; u >= 0; --u) {
      const int e = swz<RB>(16 * J + 8 * h + u, i);
      const f16x2 k2 = *reinterpret_cast<const f16x2*>(&tk[e]);
      kf0[u] = (float)k2[0] * sfx0;   // k decayed to the sub-block end
      kf1[u] = (float)k2[1] * sfx1;
      *reinterpret_cast<f16x2*>(&tkd[e]) = f16x2{(f16)kf0[u], (f16)kf1[u]};
      sfx0 *= al0[u];
      sfx1 *= al1[u];
    }
    if (h == 0) *reinterpret_cast<f32x2*>(&sTot[J][i]) = f32x2{tot0 + ot0, tot1 + ot1};
    __syncthreads();
    if (tid < DK) {
      float acc = 0.f;
      sBst[0][tid] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc += sTot[j][tid];
        sBst[j + 1][tid] = acc;
      }
    }
    __syncthreads();
    // k decayed to the chunk end = k decayed to its sub-block end times the
    // decay of the later sub-blocks (log-alpha's tile is free now)
    const float te0 = ex(sBst[4][i] - sBst[J + 1][i]), te1 = ex(sBst[4][i + 1] - sBst[J + 1][i + 1]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = swz<RB>(16 * J + 8 * h + u, i);
      *reinterpret_cast<f16x2*>(&tke[e]) = f16x2{(f16)(kf0[u] * te0), (f16)(kf1[u] * te1)};
    }
    // factors between sub-block boundaries, thread (key dim, quarter)
    const int d = tid & 63;
    for (int ab = tid >> 6; ab < 25; ab += 4) {
      const int a = ab / 5, bb = ab % 5;
      sF[a][bb][d] = (f16)ex(sBst[a][d] - sBst[bb][d]);
    }
  }
  __syncthreads();

  // a block after the first adds its part of a gradient to what the
  // earlier blocks stored (the calls of one backward pass run in order)
  auto store4 = [&](rsrc_t dst, uint32_t gs, bool acc, int t, int col, f32x4 x) {
    const uint32_t cf = srow[t];
    const uint32_t off = ((cf & 0x7fffffffu) * gs + (uint32_t)col * 2) | (cf & 0x80000000u);
    if (acc) {
      const f16x4 old =
          __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(dst, off, 0, 0));
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] += (float)old[u];
    }
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_f16(x)), dst, off, 0, 0);
  };
  const bool acc_k = p.acc_dqk != 0, acc_v = p.acc_dv != 0;

  // ---- 3a. dq (rows: key dims of this wave, columns: tokens of sub-block I)
  f32x4 dqv[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const f16x8 dob0 = ld128(tdo + swz<RB>(16 * I + n16, 8 * g));
    const f16x8 dob1 = ld128(tdo + swz<RB>(16 * I + n16, 32 + 8 * g));
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      // (V dO^T)[s in J][t in I]: lane (n, g) holds s = 16J + 4g + u, t = 16I + n
      f32x4 sc = mma32(ld128(tv + swz<RB>(16 * J + n16, 8 * g)), dob0, f32x4{0.f, 0.f, 0.f, 0.f});
      sc = mma32(ld128(tv + swz<RB>(16 * J + n16, 32 + 8 * g)), dob1, sc);
      if (J == I) {
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = (4 * g + u <= n16) ? sc[u] : 0.f;
      }
      // Kd^T: key dim 16 kb + n, tokens 16J + 4g..; the row's factor is the
      // decay back to the sub-block start, k e^{-c} = Kd e^{Bst_J - Bst_{J+1}}
      // (>= 1) for J = I, or between the boundaries, e^{Bst_I - Bst_{J+1}}
      // (<= 1) for J < I
      const f16 fk = sF[J == I ? J : I][J + 1][16 * kb + n16];
      acc = mma16(tr_read<RB>(tkd, 16 * J, 16 * kb) * fk, to_f16(sc), acc);
    }
    // inter-chunk: (E dO^T)[key dim][token]
    f32x4 ed = mma32(ea[0], dob0, f32x4{0.f, 0.f, 0.f, 0.f});
    ed = mma32(ea[1], dob1, ed);
    const int t = 16 * I + n16;
    const f32x4 ec = *reinterpret_cast<const f32x4*>(&sEc[t * ES + ki]);
    const f16x4 fb = ld64(&sF[I][0][ki]);
    f32x4 dq;
#pragma unroll
    for (int u = 0; u < 4; ++u) dq[u] = ec[u] * (acc[u] + (float)fb[u] * ed[u]);
    dqv[I] = dq;
    store4(wdq, gsk, acc_k, t, ki, dq);
  }

  // ---- 3b. dk (rows: key dims of this wave, columns: tokens of sub-block J)
  f32x4 dkv[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    const f16x8 vb0 = ld128(tv + swz<RB>(16 * J + n16, 8 * g));
    const f16x8 vb1 = ld128(tv + swz<RB>(16 * J + n16, 32 + 8 * g));
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int I = J; I < 4; ++I) {
      // (dO V^T)[s in I][t in J]: lane (n, g) holds s = 16I + 4g + u, t = 16J + n
      f32x4 sc = mma32(ld128(tdo + swz<RB>(16 * I + n16, 8 * g)), vb0, f32x4{0.f, 0.f, 0.f, 0.f});
      sc = mma32(ld128(tdo + swz<RB>(16 * I + n16, 32 + 8 * g)), vb1, sc);
      if (I == J) {
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = (4 * g + u >= n16) ? sc[u] : 0.f;
      }
      // Qs^T: key dim 16 kb + n, tokens 16I + 4g..; for I > J its row takes
      // the decay between the boundaries, e^{Bst_I - Bst_J} (<= 1)
      f16x4 aop = tr_read<RB>(tqs, 16 * I, 16 * kb);
      if (I > J) aop = aop * sF[I][J][16 * kb + n16];
      acc = mma16(aop, to_f16(sc), acc);
    }
    // inter-chunk: (R V^T)[key dim][token]
    f32x4 rv = mma32(ra[0], vb0, f32x4{0.f, 0.f, 0.f, 0.f});
    rv = mma32(ra[1], vb1, rv);
    const int t = 16 * J + n16;
    const f32x4 ec = *reinterpret_cast<const f32x4*>(&sEc[t * ES + ki]);
    const f16x4 fe = ld64(&sF[4][J][ki]);
    f32x4 dk;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dk[u] = __builtin_amdgcn_rcpf(ec[u]) * (acc[u] + (float)fe[u] * rv[u]);
    dkv[J] = dk;
    store4(wdk, gsk, acc_k, t, ki, dk);
  }

  // ---- 3c. dv (rows: value dims of this wave, columns: tokens of sub-block J)
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    f16x8 kx0 = ld128(tkd + swz<RB>(16 * J + n16, 8 * g));
    f16x8 kx1 = ld128(tkd + swz<RB>(16 * J + n16, 32 + 8 * g));
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int I = J; I < 4; ++I) {
      // ((Q e^B)(K e^-B)^T)[s in I][t in J], bounded operands: Qs rows of I,
      // and Kd rows of J scaled by e^{B(I) - B(J+1)} (<= 1) for I > J, or by
      // e^{B(J) - B(J+1)} (>= 1, back to the sub-block start) for I = J;
      // the factor sits on the contraction index and is applied to Qs here
      f16x8 qa0 = ld128(tqs + swz<RB>(16 * I + n16, 8 * g));
      f16x8 qa1 = ld128(tqs + swz<RB>(16 * I + n16, 32 + 8 * g));
      const int top = (I == J) ? J : I;
      const f16x8 f0 = ld128(&sF[top][J + 1][8 * g]);
      const f16x8 f1 = ld128(&sF[top][J + 1][32 + 8 * g]);
      if (I == J) {
        // the >= 1 factor goes on the keys (Qs stays <= |q|)
        kx0 = kx0 * f0;
        kx1 = kx1 * f1;
      } else {
        qa0 = qa0 * f0;
        qa1 = qa1 * f1;
      }
      f32x4 sc = mma32(qa0, kx0, f32x4{0.f, 0.f, 0.f, 0.f});
      sc = mma32(qa1, kx1, sc);
      if (I == J) {
        kx0 = ld128(tkd + swz<RB>(16 * J + n16, 8 * g));
        kx1 = ld128(tkd + swz<RB>(16 * J + n16, 32 + 8 * g));
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = (4 * g + u >= n16) ? sc[u] : 0.f;
      }
      acc = mma16(tr_read<RB>(tdo, 16 * I, 16 * vb), to_f16(sc), acc);
    }
    // inter-chunk: (R^T Ke^T)[value dim][token]
    f32x4 rk = mma32(rta[0], ld128(tke + swz<RB>(16 * J + n16, 8 * g)), f32x4{0.f, 0.f, 0.f, 0.f});
    rk = mma32(rta[1], ld128(tke + swz<RB>(16 * J + n16, 32 + 8 * g)), rk);
    store4(wdv, gsv, acc_v, 16 * J + n16, vj, acc + rk);
  }

  // ---- 4. next state, carry, dlog_alpha
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const f16x8 av = cat8(tr_read<RB>(tv, 32 * P, 16 * vb), tr_read<RB>(tv, 32 * P + 16, 16 * vb));
      const f16x8 bk = cat8(tr_read<RB>(tke, 32 * P, 16 * kc), tr_read<RB>(tke, 32 * P + 16, 16 * kc));
      acc = mma32(av, bk, acc);
    }
    // lane (n, g): E_next[i = 16 kc + n][j = 16 vb + 4g + u]
    const int i = 16 * kc + n16;
    const float ebe = ex(sBst[4][i]);
    const f32x4 e4 = e4s[kc];
    const f32x4 r4 = r4s[kc];
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) part += (ebe * e4[u] + acc[u]) * r4[u];
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0) sCarry[vb][i] = part;
  }
  __syncthreads();

  {
    f32x4 running;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      running[u] = ((sCarry[0][ki + u] + sCarry[1][ki + u]) + sCarry[2][ki + u]) + sCarry[3][ki + u];
#pragma unroll
    for (int I = 3; I >= 0; --I) {
      const int t = 16 * I + n16;
      const f16x4 q4 = ld64(tq + swz<RB>(t, ki));
      const f16x4 k4 = ld64(tk + swz<RB>(t, ki));
      f32x4 x;
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = (float)q4[u] * dqv[I][u] - (float)k4[u] * dkv[I][u];
      // suffix sums over the 16 tokens of the tile row (lanes n .. 15)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] += dpp_f<kRowShl + 1>(x[u]);
        x[u] += dpp_f<kRowShl + 2>(x[u]);
        x[u] += dpp_f<kRowShl + 4>(x[u]);
        x[u] += dpp_f<kRowShl + 8>(x[u]);
      }
      f32x4 dla;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dla[u] = x[u] + running[u];
        running[u] += dpp_f<kRowBcast + 0>(x[u]);   // the row's total (lane 0)
      }
      store4(wdla, gsk, acc_k, t, ki, dla);
    }
  }
}

}  // namespace

hipError_t launch_bwd_chunks(int d_k, int d_v, const BwdParams& p, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
  if (d_k != 64 || d_v != 64) return hipErrorInvalidValue;
  const dim3 grid(p.B * p.heads * p.n_chunks), block(kThreads);
  const auto kernel = chunk_bwd_f16_kernel<64, 64>;
  if (start != nullptr || stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gla

// Single-pass forward kernel of the chunkwise gated linear attention with
// key-only decay, float16, d_k = d_v = 64, for gfx950 (CDNA4).
//
// The chunkwise scheme of the pages (GTR news write-up, tokendh.com, section
// "Where the speed comes from": chunk summaries for all chunks at once, only
// the boundary hand-off in order, small operators fused so intermediates stop
// making round trips) as one launch.  Each workgroup takes one span of
// consecutive chunks of one (batch, head) sequence, by ticket, so a workgroup
// only ever waits for workgroups that started before it:
//
//   phase A    fold the span into its summary (product of the gates, state
//              reached from zero) and publish it;
//   look-back  fold the published summaries of the earlier spans of the
//              sequence into the entry state (span 0 publishes its summary with
//              the initial state folded in, so nothing else reads that state);
//   phase C    replay the span from its entry state and write the outputs.
//
// Phase C re-reads k, v and log-alpha of the span, which phase A brought into
// the caches shortly before; q is read once, out written once.
//
// Inside a workgroup (eight waves) the span is cut into two streams of
// 32-token steps, each stream four waves: two P-waves per stream form the
// decays of a step and its scaled operands in LDS, two O-waves hold the
// stream's 64 x 64 float32 state (32 value columns each) in 32x32 MFMA
// accumulators and consume the operands.  Per stream four step buffers
// rotate: in each interval the O-waves consume step k, the P-waves prepare
// step k+1 and issue the loads of step k+3, and one barrier ends the
// interval.  The streams of one span are joined through LDS: phase A gives
// each stream's summary, the span summary is their composition, and the
// second stream starts phase C from the first one's summary applied to the
// span's entry state.
//
// Step arithmetic (inclusive cumulative log-decay b_t from the step start,
// anchor a = b at the step's 16th token, so every scaled factor stays within
// the decay of half a step):
//   Qb = q e^{b - a}, Kb = k e^{a - b}, Khat = k e^{b_end - b} (<= 1),
//   O  = mask(Qb Kb^T) V + Qb diag(e^a) S,
//   S <- diag(e^{b_end}) S + Khat^T V.
// A step whose half-step decay leaves 2^10 in some key dim, or whose queries
// or keys reach 32 in magnitude, is computed exactly token by token from the
// raw tiles instead (the P-waves agree on that before they overwrite anything).

#include <hip/hip_ext.h>

#include "gla_device.h"
#include "gla_internal.h"
#include "gla_tiles.h"

#ifndef GLA_FOLD_NB
#define GLA_FOLD_NB 8
#endif

namespace gla {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kFS = 32;          // tokens per step
constexpr int kFT = kFS * 64;    // float16 elements of one tile of one stream
constexpr int kFThreads = 512;   // two streams of four waves
constexpr float kHalfStepLimit = 10.f;   // log2 of the largest factor of the fast path
constexpr int kAuxSC1 = 16;      // device-coherent access (cache policy bit sc1)

__device__ __forceinline__ f32x16 mma3232(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Pointers of one step buffer for one stream.
struct FB {
  f16* q;          // raw q, then Qb with permuted key dims (kperm)
  f16* k;          // raw k, then Kb (permuted)
  f16* l;          // raw log-alpha (or gate logits), then Khat (natural order)
  f16* v;
  float* g;        // e^{b_end} per key dim
  float* ea;       // e^{a} per key dim
  uint32_t* rows;  // grid cell of each row (bit 31: past the stream)
  uint32_t* mode;  // 1: the step is computed token by token
};

// Stored position of key dim d (d % 4 == 0) in the Qb / Kb tiles: inside each
// group of 16 dims the blocks of four go to 0, 8, 4, 12, so that lane half h
// of a 32x32 MFMA operand reads dims 4h..4h+3 and 8+4h..8+4h+3 as one 16-byte
// piece -- the key-dim order in which a state accumulator holds its rows.
__device__ __forceinline__ int kperm(int d) {
  const int g = (d >> 2) & 3;
  return (d & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2);
}

// Transposed read of a 32-column block for a 32x32x16 MFMA operand: lane l
// receives rows r0 + 4 (l / 32) .. + 3 of column c0 + l % 32 of a swizzled
// tile with 128-byte rows (each 16-lane group transposes the 4 x 16 block its
// lanes address).
__device__ __forceinline__ f16x4 tr32(const f16* tile, int r0, int c0) {
  const int l = threadIdx.x & 63, G = l >> 4, j = l & 15;
  const int row = r0 + 4 * (G >> 1) + (j >> 2);
  const int col = c0 + 16 * (G & 1) + 4 * (j & 3);
  const f16* a = tile + row * 64 + (((col >> 3) ^ (row & 7)) << 3) + (col & 4);
  const lds_h4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_h4_t*)(lds_void_t*)a);
  return __builtin_bit_cast(f16x4, x);
}

// Per-stream context of a workgroup.
struct Ctx {
  int bh, span;
  GridMap gm;
  SeqBufs sb;
  int tb, te;      // this stream's scan steps [tb, te)
  int ni;          // intervals of the phase loop (steps of the longer stream)
};

__device__ __forceinline__ int step_valid(const Ctx& c, int j) {
  return max(0, min(kFS, c.te - (c.tb + kFS * j)));
}

// LDS-writing loads of step j into buffer B: P-wave kh moves rows 16 kh ..
// 16 kh + 15 of each tile (two 1 KB blocks per tile) and records their grid
// cells.  Phase A loads k, log-alpha, v; phase C also q, all non-temporally
// (the last read of each).
template <bool OUT>
__device__ __forceinline__ void issue_step(const Ctx& c, const FB& B, int j, int kh) {
  const int lane = threadIdx.x & 63;
  const int t0 = c.tb + kFS * j;
  const int valid = step_valid(c, j);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * kh + i;
    uint32_t cf;
    bool first;
    const uint32_t off = dma_offset_cell<128>(blk, t0, valid, c.gm, &cf, &first);
    if (OUT && first) B.rows[8 * blk + (lane >> 3)] = cf;
    if (OUT) dma16_asm<OUT>(c.sb.q, B.q + blk * 512, off);
    dma16_asm<OUT>(c.sb.k, B.k + blk * 512, off);
    dma16_asm<OUT>(c.sb.la, B.l + blk * 512, off);
    dma16_asm<OUT>(c.sb.v, B.v + blk * 512, off);
  }
}

// The two P-waves of a stream agree whether a step takes the exact path:
// each posts (tag | its verdict) in LDS and waits for the other's post of the
// same tag.  Bounded: a wait that exceeds the limit gives up (and reports the
// step as exact, which is always correct).
__device__ __forceinline__ bool agree_exact(uint32_t* pf, int kh, uint32_t tag, bool mine) {
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_store(&pf[kh], tag | (mine ? 1u : 0u), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
  uint32_t o = 0;
  for (int spin = 0; spin < (1 << 20); ++spin) {
    o = __hip_atomic_load(&pf[kh ^ 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((o & ~1u) == tag) return mine || (o & 1u);
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// P-wave work of step j (buffer B): the cumulative log-decay of each 16-token
// sub-block by MFMA against a constant triangle (log2 e folded in as an fp16
// hi + lo pair), the anchor a (end of the first sub-block) and the step decay
// broadcast along each 16-lane row, then the scaled operands written in place
// of the raw tiles.  P-wave kh owns key dims 32 kh .. 32 kh + 31; lane (t, g)
// holds dims 16 db + 4g .. + 3 of token 16 I + t.
//   phase A (OUT false): Khat and e^{b_end}; lg accumulates the step decays.
//   phase C (OUT true): Qb, Kb, Khat, e^{b_end}, e^{a}, unless the step must
//     be computed exactly (then the raw tiles stay).
template <bool OUT, bool GATE>
__device__ __forceinline__ void p_step(const FwdParams& p, const Ctx& c, const FB& B, int j, int kh,
                                       f16x4 u_hi, f16x4 u_lo, float (&lg)[8], uint32_t* pf,
                                       uint32_t tag) {
  const int lane = threadIdx.x & 63, t = lane & 15, g = lane >> 4;
  const int valid = step_valid(c, j);
  f16x4 qo[2][2], ko[2][2], ho[2][2];
  f32x4 gv[2], eav[2];
  bool bad = false;
  u16x4 kmax = {0, 0, 0, 0};
#pragma unroll
  for (int dbi = 0; dbi < 2; ++dbi) {
    const int db = 2 * kh + dbi;
    f16x4 lat[2], k4[2], q4[2];
    f32x4 c2[2];
#pragma unroll
    for (int I = 0; I < 2; ++I) {
      lat[I] = log_alpha_of<GATE>(tr_read<128>(B.l, 16 * I, 16 * db), p.inv_tau, 16 * I, valid);
      k4[I] = ld64(B.k + swz<128>(16 * I + t, 16 * db + 4 * g));
      if (OUT) q4[I] = ld64(B.q + swz<128>(16 * I + t, 16 * db + 4 * g));
    }
#pragma unroll
    for (int I = 0; I < 2; ++I) {
      c2[I] = mma16(lat[I], u_hi, f32x4{0.f, 0.f, 0.f, 0.f});
      c2[I] = mma16(lat[I], u_lo, c2[I]);
    }
    f32x4 a2, e2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a2[u] = row_bcast15(c2[0][u]);   // log2 decay of the first sub-block
      e2[u] = row_bcast15(c2[1][u]);   // log2 decay of the second
    }
    f32x4 x[2];
    x[0] = c2[0] - a2;                 // b - a >= 0 in the first sub-block
    x[1] = c2[1];                      // b - a <= 0 in the second
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      gv[dbi][u] = exp2_fast(a2[u] + e2[u]);
      if (!OUT) lg[4 * dbi + u] += a2[u] + e2[u];
      if (OUT) eav[dbi][u] = exp2_fast(a2[u]);
    }
#pragma unroll
    for (int I = 0; I < 2; ++I) {
      f32x4 eh;
      if constexpr (OUT) {
        f32x4 eq, ek;
        f32x4 ge;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          eq[u] = exp2_fast(x[I][u]);
          ek[u] = exp2_fast(-x[I][u]);
          ge[u] = exp2_fast(e2[u]);
          eh[u] = ek[u] * ge[u];
          bad |= (I == 0) ? (x[I][u] > kHalfStepLimit) : (x[I][u] < -kHalfStepLimit);
        }
        qo[dbi][I] = q4[I] * to_f16(eq);
        ko[dbi][I] = k4[I] * to_f16(ek);
        kmax = __builtin_elementwise_max(kmax, __builtin_bit_cast(u16x4, k4[I]) & (unsigned short)0x7fff);
        kmax = __builtin_elementwise_max(kmax, __builtin_bit_cast(u16x4, q4[I]) & (unsigned short)0x7fff);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) eh[u] = exp2_fast(e2[u] - x[I][u]);
      }
      ho[dbi][I] = k4[I] * to_f16(eh);
    }
  }
  bool exact = false;
  if constexpr (OUT) {
    // |q| or |k| >= 32 (binary16 0x5000 and above, NaN included): times a
    // factor up to 2^10, Qb or Kb could leave the float16 range
    bad |= __builtin_elementwise_max(kmax.xy, kmax.zw)[0] >= 0x5000 ||
           __builtin_elementwise_max(kmax.xy, kmax.zw)[1] >= 0x5000;
    exact = agree_exact(pf, kh, tag, __builtin_amdgcn_ballot_w64(bad) != 0);
  }
  if (!exact) {
#pragma unroll
    for (int dbi = 0; dbi < 2; ++dbi) {
      const int d0 = 16 * (2 * kh + dbi) + 4 * g;
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int row = 16 * I + t;
        if constexpr (OUT) {
          st64(B.q + swz<128>(row, kperm(d0)), qo[dbi][I]);
          st64(B.k + swz<128>(row, kperm(d0)), ko[dbi][I]);
        }
        st64(B.l + swz<128>(row, d0), ho[dbi][I]);
      }
      if (t == 0) {
        *reinterpret_cast<f32x4*>(B.g + d0) = gv[dbi];
        if (OUT) *reinterpret_cast<f32x4*>(B.ea + d0) = eav[dbi];
      }
    }
  }
  if (OUT && kh == 0 && lane == 0) B.mode[0] = exact ? 1u : 0u;
}

// O-wave state: the stream's state S (64 key dims x 64 values) split by value
// halves; tile kb of O-wave vh holds S[32 kb + i][32 vh + n] in lane
// (n, h) = (l % 32, l / 32), register r: i = 8 (r / 4) + 4h + r % 4.

// S <- diag(e^{b_end}) S + Khat^T V for the O-wave's value half.
__device__ __forceinline__ void o_state_update(const FB& B, int vh, const f16x8 (&vv)[2],
                                               f32x16 (&S)[2]) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(B.g + 32 * kb + 8 * jj + 4 * hf);
#pragma unroll
      for (int u = 0; u < 4; ++u) S[kb][4 * jj + u] *= g4[u];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const f16x8 ka = cat8(tr32(B.l, 16 * kk, 32 * kb), tr32(B.l, 16 * kk + 8, 32 * kb));
      S[kb] = mma3232(ka, vv[kk], S[kb]);
    }
  }
}

// V of a step as the token-slot operand (value columns 32 vh ..): K-step kk
// holds tokens 16kk + 4h .. + 3 and 16kk + 8 + 4h .. + 3 in lane half h.
__device__ __forceinline__ void load_v(const FB& B, int vh, f16x8 (&vv)[2]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    vv[kk] = cat8(tr32(B.v, 16 * kk, 32 * vh), tr32(B.v, 16 * kk + 8, 32 * vh));
}

// Exact step, token by token from the raw tiles, in float32: the recurrence
// itself on the O-wave's rows and value column.
template <bool GATE>
__device__ __forceinline__ void o_step_exact(const FwdParams& p, const Ctx& c, const FB& B, int vh,
                                             int valid, f32x16 (&S)[2]) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const int cv = 32 * vh + n;
  for (int tt = 0; tt < valid; ++tt) {
    const float vf = (float)B.v[swz<128>(tt, cv & ~3) + (cv & 3)];
    float part = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * kb + 8 * jj + 4 * hf;
        const f16x4 la4 = ld64(B.l + swz<128>(tt, d0));
        const f16x4 k4 = ld64(B.k + swz<128>(tt, d0));
        const f16x4 q4 = ld64(B.q + swz<128>(tt, d0));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float la = GATE ? logsigmoid_scaled((float)la4[u], p.inv_tau) : (float)la4[u];
          const float al = exp2_fast(la * 1.4426950408889634f);
          const int r = 4 * jj + u;
          S[kb][r] = al * S[kb][r] + (float)k4[u] * vf;
          part += (float)q4[u] * S[kb][r];
        }
      }
    }
    part += __shfl_xor(part, 32);
    const uint32_t cf = B.rows[tt];
    const uint32_t off = ((cf & 0x7fffffffu) * 128u | (cf & 0x80000000u)) + (uint32_t)(cv * 2);
    if (hf == 0)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (f16)part), c.sb.out,
                                            off, 0, 0);
  }
}

// O-wave work of step j.  Phase A: the state update only.  Phase C: scores
// D[s][t] = Kb_s . Qb_t (one 32x32 tile), O^T = V^T mask(D) + (diag(e^a) S)^T
// Qb^T, outputs stored to their grid cells, then the state update.
template <bool OUT, bool GATE>
__device__ __forceinline__ void o_step(const FwdParams& p, const Ctx& c, const FB& B, int j, int vh,
                                       const f16x8 (&mask)[2], f32x16 (&S)[2]) {
  const int lane = threadIdx.x & 63, tq = lane & 31, hf = lane >> 5;
  if constexpr (!OUT) {
    f16x8 vv[2];
    load_v(B, vh, vv);
    o_state_update(B, vh, vv, S);
  } else {
    if (B.mode[0] != 0) {
      o_step_exact<GATE>(p, c, B, vh, step_valid(c, j), S);
      return;
    }
    f16x8 qb[4], kbv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qb[kk] = ld128(B.q + swz<128>(tq, 16 * kk + 8 * hf));
      kbv[kk] = ld128(B.k + swz<128>(tq, 16 * kk + 8 * hf));
    }
    f16x8 vv[2];
    load_v(B, vh, vv);
    f32x16 D = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) D = mma3232(kbv[kk], qb[kk], D);
    f32x16 acc = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 e4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        e4[jj] = *reinterpret_cast<const f32x4*>(B.ea + 32 * kb + 8 * jj + 4 * hf);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        f16x8 sa;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int r = 8 * kk + m;
          sa[m] = (f16)(S[kb][r] * e4[r >> 2][r & 3]);
        }
        acc = mma3232(sa, qb[2 * kb + kk], acc);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 dm;
#pragma unroll
      for (int m = 0; m < 8; ++m) dm[m] = (f16)D[8 * kk + m];
      acc = mma3232(vv[kk], dm * mask[kk], acc);
    }
    const uint32_t cf = B.rows[tq];
    const uint32_t base = (cf & 0x7fffffffu) * 128u | (cf & 0x80000000u);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f16x4 o = to_f16(f32x4{acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]});
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), c.sb.out,
                                            base + (uint32_t)((32 * vh + 8 * jj + 4 * hf) * 2), 0,
                                            0);
    }
    o_state_update(B, vh, vv, S);
  }
}

// Causal mask of the score tile as two f16x8 operands: register r of lane
// (t, h) holds key token s = 8 (r / 4) + 4h + r % 4, kept when s <= t.
__device__ __forceinline__ void make_mask(f16x8 (&mask)[2]) {
  const int lane = threadIdx.x & 63, tq = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int r = 8 * kk + m;
      const int s = 8 * (r >> 2) + 4 * hf + (r & 3);
      mask[kk][m] = (f16)(s <= tq ? 1.f : 0.f);
    }
}

// The four step buffers of one stream.
struct FB4 {
  FB b[4];
};

// One interval: O-waves consume step k (buffer bo), P-waves issue the loads
// of step k + 3 (buffer bd), prepare step k + 1 (buffer bp) and wait for step
// k + 2; one barrier.
template <bool OUT, bool GATE>
__device__ __forceinline__ void interval(const FwdParams& p, const Ctx& c, const FB& bo, const FB& bp,
                                         const FB& bd, int k, bool is_o, int hsel, f16x4 u_hi,
                                         f16x4 u_lo, const f16x8 (&mask)[2], f32x16 (&S)[2],
                                         float (&lg)[8], uint32_t* pf) {
  constexpr int ND = OUT ? 8 : 6;
  if (is_o) {
    o_step<OUT, GATE>(p, c, bo, k, hsel, mask, S);
  } else {
    issue_step<OUT>(c, bd, k + 3, hsel);
    if (k + 1 < c.ni) p_step<OUT, GATE>(p, c, bp, k + 1, hsel, u_hi, u_lo, lg, pf, (uint32_t)(k + 2) << 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(ND));   // step k + 2 has landed
  }
  wait_barrier<kLgkmZero>();
}

// One phase over this stream's steps.  `pre` steps (0 or 2) were issued
// before the call.
template <bool OUT, bool GATE>
__device__ __forceinline__ void run_phase(const FwdParams& p, const Ctx& c, const FB4& B, bool is_o,
                                          int hsel, int pre, const f16x8 (&mask)[2],
                                          f32x16 (&S)[2], float (&lg)[8], uint32_t* pf) {
  constexpr int ND = OUT ? 8 : 6;
  const f16x4 u_hi = upper_incl(kLog2eHi), u_lo = upper_incl(kLog2eLo);
  if (!is_o) {
    if (pre == 0) {
      issue_step<OUT>(c, B.b[0], 0, hsel);
      issue_step<OUT>(c, B.b[1], 1, hsel);
    }
    issue_step<OUT>(c, B.b[2], 2, hsel);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * ND));   // step 0 has landed
  }
  wait_barrier<kLgkmZero>();
  if (!is_o) {
    p_step<OUT, GATE>(p, c, B.b[0], 0, hsel, u_hi, u_lo, lg, pf, 1u << 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(ND));       // step 1 has landed
  }
  wait_barrier<kLgkmZero>();
  for (int k0 = 0; k0 < c.ni; k0 += 4) {
    interval<OUT, GATE>(p, c, B.b[0], B.b[1], B.b[3], k0, is_o, hsel, u_hi, u_lo, mask, S, lg, pf);
    if (k0 + 1 >= c.ni) break;
    interval<OUT, GATE>(p, c, B.b[1], B.b[2], B.b[0], k0 + 1, is_o, hsel, u_hi, u_lo, mask, S, lg, pf);
    if (k0 + 2 >= c.ni) break;
    interval<OUT, GATE>(p, c, B.b[2], B.b[3], B.b[1], k0 + 2, is_o, hsel, u_hi, u_lo, mask, S, lg, pf);
    if (k0 + 3 >= c.ni) break;
    interval<OUT, GATE>(p, c, B.b[3], B.b[0], B.b[2], k0 + 3, is_o, hsel, u_hi, u_lo, mask, S, lg, pf);
  }
  if (!is_o) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));    // trailing zero-fill loads
  }
}

// The O-wave's state to / from a float32 [64][64] matrix kept in four tiles of
// 16 rows each (the LDS scratch of the join).
struct Tiles4 {
  f16 *t0, *t1, *t2, *t3;
};
__device__ __forceinline__ float* scratch_row(const Tiles4& t, int i) {
  f16* b = i < 16 ? t.t0 : i < 32 ? t.t1 : i < 48 ? t.t2 : t.t3;
  return reinterpret_cast<float*>(b) + (i & 15) * 64;
}
__device__ __forceinline__ void state_to_scratch(const Tiles4& t, int vh, const f32x16 (&S)[2]) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      scratch_row(t, 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3))[32 * vh + n] = S[kb][r];
}
__device__ __forceinline__ void state_from_scratch(const Tiles4& t, int vh, f32x16 (&S)[2]) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      S[kb][r] = scratch_row(t, 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3))[32 * vh + n];
}

// LDS of step buffer b: the tiles of both streams in one array, [stream]
// [q, k, log-alpha, v][32 x 64], plus small per-stream arrays.  Each buffer's
// tiles are one LDS object and the LDS-writing loads only ever target other
// buffers than the ones being read, so the compiler's own waits for those
// loads can tell them apart (it follows a handful of target objects only).
#define FUSED_BUF(b)                                                                             \
  __shared__ __attribute__((aligned(16))) f16 ft##b[2 * 4 * kFT];                              \
  __shared__ __attribute__((aligned(16))) float fg##b[2 * 64], fea##b[2 * 64];                  \
  __shared__ uint32_t frow##b[2 * kFS], fmode##b[2];

#define FUSED_FB(b, s)                                                                           \
  FB{ft##b + (s)*4 * kFT, ft##b + (s)*4 * kFT + kFT, ft##b + (s)*4 * kFT + 2 * kFT,            \
     ft##b + (s)*4 * kFT + 3 * kFT, fg##b + (s)*64, fea##b + (s)*64, frow##b + (s)*kFS,         \
     fmode##b + (s)}

template <bool GATE>
__global__ __launch_bounds__(kFThreads, 1) void fused_fwd_kernel(FwdParams p) {
  FUSED_BUF(0)
  FUSED_BUF(1)
  FUSED_BUF(2)
  FUSED_BUF(3)
  __shared__ uint32_t s_hdr[2];
  __shared__ uint32_t s_pflag[4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sig = wave >> 2;                 // stream
  const bool is_o = (wave & 1) == sig;       // one O-wave and one P-wave per SIMD
  const int hsel = (wave & 3) >> 1;          // value half (O) / key half (P)

  if (threadIdx.x == 0) {
    s_hdr[0] = __hip_atomic_fetch_add(&p.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_hdr[1] = __hip_atomic_load(&p.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < 4) s_pflag[threadIdx.x] = 0u;
  __syncthreads();
  const int BH = p.B * p.heads;
  const int n_wg = BH * p.n_spans;
  // tickets run 0 .. n_wg-1 when every call leaves the words consistent; the
  // modulo only keeps indices in range if they were not
  const uint32_t ticket = s_hdr[0] % (uint32_t)n_wg, epoch = s_hdr[1];
  const int span = (int)(ticket / (uint32_t)BH);
  const int bh = (int)(ticket - (uint32_t)span * BH);

  Ctx c;
  c.bh = bh;
  c.span = span;
  c.gm = grid_map(p, bh / p.heads);
  c.sb = seq_bufs<64, 64>(p, bh);
  const int t_begin = span * p.span_chunks * 64;
  const int t_end = min(t_begin + p.span_chunks * 64, p.T);
  const int nst = (t_end - t_begin + kFS - 1) / kFS;
  const int n0 = (nst + 1) >> 1;
  c.tb = t_begin + (sig ? kFS * n0 : 0);
  c.te = sig ? t_end : min(t_begin + kFS * n0, t_end);
  c.ni = n0;

  FB4 B;
  B.b[0] = FUSED_FB(0, sig);
  B.b[1] = FUSED_FB(1, sig);
  B.b[2] = FUSED_FB(2, sig);
  B.b[3] = FUSED_FB(3, sig);
  uint32_t* pf = s_pflag + 2 * sig;
  // join scratch: stream sigma's summary / entry state in the stream-0 tiles of
  // buffer 2 + sigma, its gate product in that buffer's gate array
  const Tiles4 L0{ft2, ft2 + kFT, ft2 + 2 * kFT, ft2 + 3 * kFT};
  const Tiles4 L1{ft3, ft3 + kFT, ft3 + 2 * kFT, ft3 + 3 * kFT};

  f16x8 mask[2];
  make_mask(mask);
  f32x16 S[2] = {};
  float lg[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 8;   // join / look-back mapping
  const size_t st_off = (size_t)bh * 64 * 64;

  // ---- phase A: each stream's summary
  run_phase<false, GATE>(p, c, B, is_o, hsel, 0, mask, S, lg, pf);
  if (is_o) {
    if (sig == 0) state_to_scratch(L0, hsel, S);
    else state_to_scratch(L1, hsel, S);
  } else if ((lane & 15) == 0) {
    float* G = sig ? fg3 : fg2;
#pragma unroll
    for (int dbi = 0; dbi < 2; ++dbi)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        G[16 * (2 * hsel + dbi) + 4 * (lane >> 4) + u] = exp2_fast(lg[4 * dbi + u]);
  }
  __syncthreads();

  // ---- the span summary: (G0 G1, G1 L0 + L1), with the initial state folded
  // in for span 0; published with device-coherent stores, then its flag
  const f32x4 l0a = *reinterpret_cast<const f32x4*>(scratch_row(L0, r) + c0);
  const f32x4 l0b = *reinterpret_cast<const f32x4*>(scratch_row(L0, r) + c0 + 4);
  const f32x4 l1a = *reinterpret_cast<const f32x4*>(scratch_row(L1, r) + c0);
  const f32x4 l1b = *reinterpret_cast<const f32x4*>(scratch_row(L1, r) + c0 + 4);
  const float g0 = fg2[r], g1 = fg3[r];
  f32x4 init_a = {0.f, 0.f, 0.f, 0.f}, init_b = init_a;
  if (span == 0 && p.initial_state != nullptr) {
    init_a = *reinterpret_cast<const f32x4*>(p.initial_state + st_off + r * 64 + c0);
    init_b = *reinterpret_cast<const f32x4*>(p.initial_state + st_off + r * 64 + c0 + 4);
  }
  const rsrc_t agg = seq_rsrc(p.agg + (size_t)bh * p.n_spans * kAggFloats,
                              (uint32_t)((size_t)p.n_spans * kAggFloats * 4));
  if (p.n_spans > 1) {
    const float gs = g0 * g1;
    f32x4 sa = l0a * g1 + l1a, sb = l0b * g1 + l1b;
    if (span == 0) {
      sa += init_a * gs;
      sb += init_b * gs;
    }
    const uint32_t base = (uint32_t)(span * kAggFloats) * 4u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sa), agg,
                                           base + (uint32_t)(64 + r * 64 + c0) * 4u, 0, kAuxSC1);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sb), agg,
                                           base + (uint32_t)(64 + r * 64 + c0 + 4) * 4u, 0, kAuxSC1);
    if ((threadIdx.x & 7) == 0)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, gs), agg,
                                            base + (uint32_t)r * 4u, 0, kAuxSC1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the summary has reached the coherence point
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(&p.sync[kSyncFlags + bh * p.n_spans + span], epoch + 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  // the first two steps of phase C load during the look-back (buffers 0 and
  // 1 hold no join scratch)
  if (!is_o) {
    issue_step<true>(c, B.b[0], 0, hsel);
    issue_step<true>(c, B.b[1], 1, hsel);
  }

  // ---- look-back: wait for the summaries of spans 0 .. span-1, fold them
  f32x4 ea = init_a, eb = init_b;
  if (span > 0) {
    if (wave == 0) {
      const uint32_t want = epoch + 1u;
      const long long t_start = clock64();
      bool timed_out = false;
      for (int j0 = 0; j0 < span && !timed_out; j0 += 64) {
        const int jj = j0 + lane;
        const unsigned int* fl = p.sync + kSyncFlags + (size_t)bh * p.n_spans + jj;
        bool ready = jj >= span;
        while (true) {
          if (!ready) ready = __hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
          if (__builtin_amdgcn_ballot_w64(!ready) == 0) break;
          if (clock64() - t_start > (1LL << 32)) {
            timed_out = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      if (timed_out && lane == 0)
        __hip_atomic_fetch_or(&p.sync[3], kSyncErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    ea = f32x4{0.f, 0.f, 0.f, 0.f};
    eb = ea;
    constexpr int NB = GLA_FOLD_NB;   // summaries whose loads are in flight together
    for (int j0 = 0; j0 < span; j0 += NB) {
      f32x4 la[NB], lb[NB];
      float gj[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        // only existing summaries are read (span is workgroup-uniform): these
        // loads go past the caches, and every workgroup folds at once
        if (j0 + i < span) {
          const uint32_t base = (uint32_t)((j0 + i) * kAggFloats) * 4u;
          la[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                agg, base + (uint32_t)(64 + r * 64 + c0) * 4u, 0, kAuxSC1));
          lb[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                agg, base + (uint32_t)(64 + r * 64 + c0 + 4) * 4u, 0, kAuxSC1));
          gj[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                agg, base + (uint32_t)r * 4u, 0, kAuxSC1));
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (j0 + i < span) {
          ea = ea * gj[i] + la[i];
          eb = eb * gj[i] + lb[i];
        }
      }
    }
  }
  // entry states of the two streams: E, then stream 0's summary applied to E
  {
    const f32x4 e1a = ea * g0 + l0a, e1b = eb * g0 + l0b;
    *reinterpret_cast<f32x4*>(scratch_row(L0, r) + c0) = ea;
    *reinterpret_cast<f32x4*>(scratch_row(L0, r) + c0 + 4) = eb;
    *reinterpret_cast<f32x4*>(scratch_row(L1, r) + c0) = e1a;
    *reinterpret_cast<f32x4*>(scratch_row(L1, r) + c0 + 4) = e1b;
  }
  __syncthreads();
  if (is_o) {
    if (sig == 0) state_from_scratch(L0, hsel, S);
    else state_from_scratch(L1, hsel, S);
  }
  wait_barrier<kLgkmZero>();

  // ---- phase C: outputs
  run_phase<true, GATE>(p, c, B, is_o, hsel, 2, mask, S, lg, pf);

  if (is_o && sig == 1 && span == p.n_spans - 1 && p.final_state != nullptr) {
    const int n = lane & 31, hf = lane >> 5;
    float* dst = p.final_state + st_off;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        dst[(32 * kb + 8 * (q >> 2) + 4 * hf + (q & 3)) * 64 + 32 * hsel + n] = S[kb][q];
  }

  // ---- the last workgroup to finish resets the ticket and finish counters
  // and advances the epoch for the next call
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&p.sync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)(n_wg - 1)) {
      __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sync[2], epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void zero_words_kernel(unsigned int* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <bool GATE>
hipError_t launch_fused_variant(const FwdParams& p, hipStream_t stream, hipEvent_t const* ev) {
  const dim3 grid((unsigned)(p.B * p.heads * p.n_spans));
  if (ev != nullptr) {
    hipError_t e;
    for (int s = 0; s < 2; ++s) {
      if ((e = hipEventRecord(ev[2 * s], stream)) != hipSuccess) return e;
      if ((e = hipEventRecord(ev[2 * s + 1], stream)) != hipSuccess) return e;
    }
    hipExtLaunchKernelGGL(fused_fwd_kernel<GATE>, grid, dim3(kFThreads), 0, stream, ev[4], ev[5], 0,
                          p);
  } else {
    hipLaunchKernelGGL(fused_fwd_kernel<GATE>, grid, dim3(kFThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool GATE>
int fused_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_fwd_kernel<GATE>, kFThreads, 0) !=
          hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

}  // namespace

bool has_fused(Dtype dt, int d_k, int d_v) { return dt == Dtype::kF16 && d_k == 64 && d_v == 64; }

int fused_blocks_per_cu(bool gate_logits) {
  return gate_logits ? fused_occupancy<true>() : fused_occupancy<false>();
}

hipError_t launch_forward_fused(bool gate_logits, const FwdParams& p, hipStream_t stream,
                                hipEvent_t const* events) {
  if (p.sync == nullptr || p.agg == nullptr || p.n_spans < 1) return hipErrorInvalidValue;
  return gate_logits ? launch_fused_variant<true>(p, stream, events)
                     : launch_fused_variant<false>(p, stream, events);
}

hipError_t launch_zero_words(unsigned int* p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((words + 255) / 256);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, stream, p, words);
  return hipGetLastError();
}

}  // namespace gla

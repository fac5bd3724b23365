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
// The state kernels give every chunk its adjoint state and every pair of
// consecutive chunks its forward state (float16, in memory).  The chunk
// kernel is persistent: two 8-wave workgroups per CU take the pairs of
// chunks of each (batch*head) sequence in turn, the first chunk of a pair and
// then the second, which enters with the first one's next state (step 3
// below), written into LDS by the workgroup instead of loaded.  Per chunk
// (wave w owning key dims and value dims 16 (w % 4) .. + 15 and the 16-token
// sub-blocks {0, 3} or {1, 2}):
//   1. q, k, v, log-alpha, dO and both states are in LDS (LDS-writing loads,
//      swizzled rows, issued during the previous chunk); B is summed per key
//      dim in float32;
//   2. float16 operand tiles with every decay factor bounded: Qs = q e^{c}
//      (c = B - B at the 16-token sub-block start, in [-10, 0]), Kd = k decayed
//      to its sub-block's end, Ke = k decayed to the chunk's end; the diagonal
//      sub-blocks use Kd times the sub-block decay back (<= e^10), and the
//      factors between sub-blocks scale the operands of the other pairs;
//   3. E_{c+1} = diag(e^{B_end}) E_c + Ke^T V and its row sums against R_c
//      (the carry);
//   4. the 20 score tiles dO V^T and (Q e^B)(K e^-B)^T of the sub-block pairs
//      are formed once on the matrix cores and kept in LDS, from which dv, dq
//      and dk are 16x16 MFMA tiles, rounded to float16 and stored to their
//      grid cells (scan-order remap as in the forward pass); as soon as a tile
//      is done with, the next chunk's data is loaded into it;
//   5. dlog_alpha is a suffix sum across the 16 lanes of each tile row plus
//      the later sub-blocks' totals and the carry.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla_device.h"
#include "gla_internal.h"
#include "gla_tiles.h"

namespace gla {
namespace {

constexpr int kThreads = 512;  // 8 waves
constexpr int kChunk = 64;

__device__ __forceinline__ float ex(float x) { return exp2_fast(x * 1.4426950408889634f); }

// DPP move within the 16-lane rows of a wave: lane n of a row reads lane
// n + k of the same row (zero past the row's end).
constexpr int kRowShl = 0x100;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// 16 x 16 float16 score tiles in LDS: row-major, 32-byte rows, the four
// 8-byte column groups of rows 8..15 stored in the order 2 3 0 1, so that the
// 16 lanes writing (or reading) one column group of rows 0..15 hit distinct
// banks.  Offset (elements) of row r, columns 4 c .. 4 c + 3:
__device__ __forceinline__ int st_tile_off(int r, int c) { return r * 16 + 4 * (c ^ ((r >> 2) & 2)); }

// Transposed read of such a tile (ds_read_b64_tr_b16): lane (n, g) receives
// rows 4g .. 4g + 3 of column n, the MFMA operand that reduces over rows.
// Lane j of each 16-lane group addresses row 4g + j / 4, columns 4 (j % 4) ...
__device__ __forceinline__ f16x4 tr_tile(const f16* tile, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const f16* a = tile + st_tile_off(4 * g + (j >> 2), j & 3);
  const lds_h4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_h4_t*)(lds_void_t*)a);
  return __builtin_bit_cast(f16x4, x);
}

// tr_read of a swizzled tile with 128-byte rows (see gla_device.h), for the
// lane index given
__device__ __forceinline__ f16x4 tr_read_l(const f16* tile, int row0, int col0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const int row = row0 + 4 * g + (j >> 2);
  const int col = col0 + 4 * (j & 3);
  const f16* a = tile + row * 64 + (((col >> 3) ^ (row & 7)) << 3) + (col & 4);
  const lds_h4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_h4_t*)(lds_void_t*)a);
  return __builtin_bit_cast(f16x4, x);
}

// Row swaps in the VALU: with both operands x, v_permlane16_swap returns x
// of this lane's 16-lane row and of its partner row q ^ 1, in .a and .b: the
// partner's in .a for odd rows (own in .b), in .b for even rows (own in .a).
// v_permlane32_swap likewise with partner row q ^ 2: the partner's in .a for
// rows 2, 3, in .b for rows 0, 1.  Sums and products over a row pair use
// both halves as they come, with no select.
struct SwapPair {
  float a, b;
};
// (The halves are copied out as values before the bit casts: a bit cast of
// the vector element r[1] itself was compiled as a read of element 0.)
__device__ __forceinline__ SwapPair swap16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return {__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}
__device__ __forceinline__ SwapPair swap32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return {__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}

// Over the four 16-lane groups of a wave (group q = lane / 16): the
// product of x over the groups before this lane's (*before) and after it
// (*after).
__device__ __forceinline__ void group_products(float x, int lane, float* before, float* after) {
  const bool odd = lane & 16, upper = lane & 32;
  const SwapPair s = swap16(x);
  const float bip = odd ? s.a : 1.f;   // group q - 1 of the pair (odd q)
  const float aip = odd ? 1.f : s.b;   // group q + 1 of the pair (even q)
  // the other pair's product: in groups 2 and 3, .a is the product over
  // groups 0 and 1; in groups 0 and 1, .b is that over groups 2 and 3
  const SwapPair t = swap32(s.a * s.b);
  *before = upper ? bip * t.a : bip;
  *after = upper ? aip : aip * t.b;
}
// The sum of x over the four 16-lane groups, the same in every lane.
__device__ __forceinline__ float group_sum(float x) {
  const SwapPair s = swap16(x);
  const SwapPair t = swap32(s.a + s.b);
  return t.a + t.b;
}

// Four gradient values of one token to float16 at `off` of `dst`; with ACC
// (a block after the first of a wider head) added to what the earlier blocks
// stored there (the calls of one backward pass run in order).  A template
// flag, so that the plain store carries no load of the old value.
template <bool ACC>
__device__ __forceinline__ void store_grad4(rsrc_t dst, uint32_t off, f32x4 x) {
  if constexpr (ACC) {
    const f16x4 old = __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(dst, off, 0, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] += (float)old[u];
  }
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_f16(x)), dst, off, 0, 0);
}

// VMEM operations one wave issues per chunk after its last prefetch: the
// two dlog-alpha stores, and the loads of the stored values they add to.
template <bool ACC_K>
constexpr int kVmemAfterPrefetch = ACC_K ? 4 : 2;

// Persistent: workgroup w starts with chunk w of the flattened
// (batch*head, chunk) order and then takes chunk gridDim.x + t, t a ticket
// from a counter, until the tickets run past the last chunk.  Two workgroups
// share a CU, and the one dispatched first issues ahead of the other (older
// waves win the arbitration); handing chunks out in ticket order lets the
// faster one take more of them, so both end together instead of the second
// running alone at half occupancy for the last chunks.  Each input tile is
// refilled with the next chunk's data as soon as the current chunk is done
// with it (log-alpha, k, d_out and both states after dq's products; q and v
// after dk), so that the loads run under the rest of the chunk's work, and a
// chunk's stores drain under the next one's.  ACC_V: dv adds to the stored
// values; ACC_K: dq, dk and dlog-alpha do.  PAIRS: the work units are pairs
// of chunks, the second entering with the first one's next state (else
// single chunks, each with its forward state from memory).
template <int DK, int DV, bool ACC_V, bool ACC_K, bool PAIRS>
__global__ __launch_bounds__(kThreads, 4) void chunk_bwd_f16_kernel(BwdParams p) {
  static_assert(DK == 64 && DV == 64, "built for 64 key and value dims");
  constexpr int RB = 128;  // bytes per tile row
  // row stride (floats) of sEc: 4 floats of padding move consecutive rows 4
  // banks apart, so 16 lanes reading 16 bytes each from 16 rows hit 64
  // different banks
  constexpr int ES = DK + 4;
  // the chunk's q, k, v, log-alpha and d_out; after the decay pass q's tile
  // holds Qs, k's Kd and log-alpha's Ke (each wave keeps the exact q and k of
  // its dlog-alpha tiles in registers)
  __shared__ __attribute__((aligned(16))) f16 tq[kChunk * DK], tk[kChunk * DK], tv[kChunk * DV];
  __shared__ __attribute__((aligned(16))) f16 tla[kChunk * DK], tdo[kChunk * DV];
  // grid cell of each token row of the current and the next chunk (bit 31:
  // past the sequence)
  __shared__ uint32_t srow[2][kChunk];
  __shared__ __attribute__((aligned(16))) float sEc[kChunk * ES];  // e^{c_t}, c = decay since the sub-block start
  // score tiles of the sub-block pairs J <= I (pair index I (I + 1) / 2 + J),
  // 16 x 16 row-major (st_tile layout): sM row s of J, column t of I holds
  // v_s . dO_t; sP row s of I, column t of J holds
  // sum_i q_si k_ti e^{B_si - B_ti}; diagonal tiles keep only s <= t (sM) or
  // s >= t (sP)
  __shared__ __attribute__((aligned(16))) f16 sM[10][256], sP[10][256];
  __shared__ __attribute__((aligned(16))) f16 sF[5][5][DK];  // e^{Bst_a - Bst_b} per key dim
  // per sub-block and key dim: the log-decay total (decay pass), later the
  // total of q dq - k dk (dlog-alpha)
  __shared__ float sTot[4][DK];
  __shared__ float sBst[DK];      // B at the chunk end (the chunk's log-decay total)
  __shared__ float sCarry[4][DK];
  __shared__ int sNext;            // the workgroup's next chunk (ticket)
  f16* const tqs = tq;            // q e^{c}
  f16* const tkd = tk;            // k decayed to its sub-block's end
  f16* const tke = tla;           // k decayed to the chunk end

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave w: key dims and value dims 16 kb .. 16 kb + 15 and two of the four
  // 16-token sub-blocks, {0, 3} or {1, 2} (five sub-block pairs either way);
  // lane (n, g) = (lane % 16, lane / 16) of its 16 x 16 tiles holds key dims
  // ki = 16 kb + 4g .. of a dq / dk tile, value dims vj = 16 vb + 4g .. of a
  // dv tile
  const int kb = wave & 3, vb = kb;
  const int hf = wave >> 2;
  const int sub[2] = {hf, 3 - hf};
  const uint32_t gsk = p.ldk * 2u, gsv = p.ldv * 2u;  // row strides in bytes
  const uint32_t kbytes = (uint32_t)p.T * gsk, vbytes = (uint32_t)p.T * gsv;
  const int total = p.B * p.heads * p.n_chunks;
  // work units: pairs of consecutive chunks of one sequence (the last one of
  // an odd sequence alone), taken whole by one workgroup in order; or single
  // chunks.  The forward states in memory are one per unit.
  constexpr int kSpan = PAIRS ? 2 : 1;
  const int n_units = PAIRS ? (p.n_chunks + 1) >> 1 : p.n_chunks;
  const int total_units = p.B * p.heads * n_units;

  // Loads of chunk `item`: this wave fills block `wave` (tokens 8 wave .. + 7;
  // lane l: 16 bytes of row 8 wave + l / 8, swizzled pieces) of each tile.  A
  // token row's grid cell serves both row widths; rows past the sequence get
  // an offset past the buffer and read as zero.  plan() also records the
  // rows' cells in srow[sel].
  struct Plan {
    uint32_t off, offv;
    size_t sok, sov;
  };
  auto plan = [&](int item, int sel, int lane) {
    const int bh = item / p.n_chunks, c = item - bh * p.n_chunks;
    GridMap gm;
    gm.H = p.H;
    gm.W = p.W;
    gm.dir = (p.scan_dir == 4) ? ((bh / p.heads) & 3) : p.scan_dir;
    gm.mw = p.div_w_m;
    gm.mh = p.div_h_m;
    gm.sw = p.div_w_s;
    gm.sh = p.div_h_s;
    const int t0 = c * kChunk, valid = min(kChunk, p.T - t0);
    const int r = 8 * wave + (lane >> 3);
    const uint32_t sw = (uint32_t)(((lane & 7) ^ (r & 7)) * 16);
    const uint32_t flag = (uint32_t)(r >= valid) << 31;
    const uint32_t cell = (uint32_t)gm.cell(t0 + r);
    if ((lane & 7) == 0) srow[sel][r] = cell | flag;
    Plan pl;
    pl.off = (cell * gsk + sw) | flag;
    pl.offv = (cell * gsv + sw) | flag;
    pl.sok = (size_t)bh * p.T * p.ldk;
    pl.sov = (size_t)bh * p.T * p.ldv;
    return pl;
  };
  auto load_k_side = [&](const Plan& pl, const void* src, f16* tile) {
    dma16_asm<false>(seq_rsrc(static_cast<const f16*>(src) + pl.sok, kbytes), tile + wave * 512, pl.off);
  };
  auto load_v_side = [&](const Plan& pl, const void* src, f16* tile) {
    dma16_asm<false>(seq_rsrc(static_cast<const f16*>(src) + pl.sov, vbytes), tile + wave * 512, pl.offv);
  };
  // The states of chunk `item`, float16 from the scans: the forward state
  // entering it and the adjoint entering it from the right, each a 64 x 64
  // tile swizzled like the input tiles, loaded into the area of sEc (free
  // from the end of one chunk's dk to the next chunk's decay pass).
  f16* const sE = reinterpret_cast<f16*>(sEc);
  f16* const sR = sE + DK * DV;
  static_assert(2 * DK * DV * 2 <= kChunk * ES * 4, "both states fit in sEc");
  // The forward state comes from memory only for the first chunk of a unit
  // (slot c / kSpan); a pair's second chunk's is the first one's next state,
  // which the workgroup writes into sE itself (with_e false).
  auto load_states = [&](int item, int lane, bool with_e) {
    const int bh = item / p.n_chunks, c = item - bh * p.n_chunks;
    const f16* E = static_cast<const f16*>(p.fwd_state) + ((size_t)bh * n_units + c / kSpan) * DK * DV;
    const f16* R = static_cast<const f16*>(p.adj_state) +
                   ((size_t)bh * p.n_chunks + (p.n_chunks - 1 - c)) * DK * DV;
    const int r = 8 * wave + (lane >> 3);
    const uint32_t off = (uint32_t)r * RB + (uint32_t)(((lane & 7) ^ (r & 7)) * 16);
    if (with_e) dma16_asm<false>(seq_rsrc(E, DK * DV * 2), sE + wave * 512, off);
    dma16_asm<false>(seq_rsrc(R, DK * DV * 2), sR + wave * 512, off);
  };
  // first chunk of work unit u, or `total` past the last unit
  auto unit_chunk = [&](int u) {
    if (u >= total_units) return total;
    if constexpr (!PAIRS) return u;
    const int bh = u / n_units;
    return bh * p.n_chunks + kSpan * (u - bh * n_units);
  };

  if ((int)blockIdx.x >= total_units) return;
  int item = unit_chunk(blockIdx.x);
  {
    const Plan pl = plan(item, 0, lane);
    load_k_side(pl, p.q, tq);
    load_k_side(pl, p.k, tk);
    load_v_side(pl, p.v, tv);
    load_k_side(pl, p.la, tla);
    load_v_side(pl, p.dout, tdo);
    load_states(item, lane, true);
    wait_barrier<vmcnt_lgkm0_imm(0)>();
  }
  for (int sel = 0; item < total; sel ^= 1) {
    // this chunk's inputs landed (what this wave issued after the last of
    // them are the previous chunk's dlog-alpha stores)
    wait_barrier<vmcnt_lgkm0_imm(kVmemAfterPrefetch<ACC_K>)>();
    // the next chunk: a ticket taken now, read after the decay pass (the
    // atomic's latency hides under it).  The counter's address goes through
    // a vector register, so the compiler treats it as per-lane and leaves the
    // atomic alone instead of combining it over the wave, which would wait
    // for the result right here.
    // the next chunk is this pair's second (workgroup-uniform)
    bool to_second = false;
    if constexpr (PAIRS) {
      const int c_cur = item - (item / p.n_chunks) * p.n_chunks;
      to_second = (c_cur & 1) == 0 && c_cur + 1 < p.n_chunks;
    }
    unsigned int ticket = 0;
    if (threadIdx.x == 0 && !to_second) {
      // (a global, not a flat, atomic: a flat one would also count against
      // the LDS waits of the decay pass)
      auto* ctr = (__attribute__((address_space(1))) unsigned int*)p.ticket;
      asm volatile("" : "+v"(ctr));
      ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the lane's indices, re-derived each chunk from a value the compiler
    // cannot see through: the many LDS addresses built from them are then
    // formed where they are used instead of held across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n16 = ln & 15, g = ln >> 4;
    const int ki = 16 * kb + 4 * g, vj = 16 * vb + 4 * g;
    // the states in this wave's layouts, read before the decay pass reuses
    // their area: E and R rows 16 kc + n, columns vj .. (the accumulator
    // layout of the next-state update, kc = 2 hf, 2 hf + 1); E and R rows of
    // the wave's key dims as MFMA A operands (lane (n, g): row 16 kb + n,
    // columns 32 h + 8g .. + 7); R^T rows of its value dims (lane (n, g):
    // R[32 h + 4g + u][16 vb + n] and R[32 h + 16 + 4g + u][16 vb + n], the
    // order in which the matching Ke operand takes the key dims)
    f16x4 e4h[2], r4h[2];
    f16x8 ea[2], ra[2], rta[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      e4h[x] = ld64(sE + swz<RB>(16 * (2 * hf + x) + n16, vj));
      r4h[x] = ld64(sR + swz<RB>(16 * (2 * hf + x) + n16, vj));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ea[h] = ld128(sE + swz<RB>(16 * kb + n16, 32 * h + 8 * g));
      ra[h] = ld128(sR + swz<RB>(16 * kb + n16, 32 * h + 8 * g));
      rta[h] = cat8(tr_read_l(sR, 32 * h, 16 * vb, ln), tr_read_l(sR, 32 * h + 16, 16 * vb, ln));
    }

    const int bh = item / p.n_chunks;
    const size_t sok = (size_t)bh * p.T * p.ldk, sov = (size_t)bh * p.T * p.ldv;
    const rsrc_t wdq = seq_rsrc(static_cast<f16*>(p.dq) + sok, kbytes);
    const rsrc_t wdk = seq_rsrc(static_cast<f16*>(p.dk) + sok, kbytes);
    const rsrc_t wdv = seq_rsrc(static_cast<f16*>(p.dv) + sov, vbytes);
    const rsrc_t wdla = seq_rsrc(static_cast<f16*>(p.dla) + sok, kbytes);
    // byte offset of token t's columns col .. in a gradient row of gs bytes
    auto grad_off = [&](uint32_t gs, int t, int col) {
      const uint32_t cf = srow[sel][t];
      return ((cf & 0x7fffffffu) * gs + (uint32_t)col * 2) | (cf & 0x80000000u);
    };

    // the exact q and k of this wave's dlog-alpha tiles (token 16 I + n of
    // its two sub-blocks, key dims ki ..), read before the decay pass
    // overwrites their tiles
    f16x4 q4r[2], k4r[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      q4r[x] = ld64(tq + swz<RB>(16 * sub[x] + n16, ki));
      k4r[x] = ld64(tk + swz<RB>(16 * sub[x] + n16, ki));
    }

    // ---- decay pass.  Wave w takes sub-block J = w % 4 and key dims
    // 32 (w / 4) ..; lane (i2, q) = (lane % 16, lane / 16) walks key dims
    // i, i + 1 (i = 32 (w / 4) + 2 i2) over the sub-block's tokens 4q .. 4q + 3:
    // alpha_t = e^{la_t}, e^{c_t} as a running product from the sub-block
    // start, the decay to the sub-block end as a running product from its end
    // (one exponential per token); the four lane groups hand each other their
    // decay products.  Qs, Kd and e^c stay in registers until every wave has
    // its q, k and states.
    {
      const int J = wave & 3;
      const int q = g;
      const int i = 32 * (wave >> 2) + 2 * n16;
      const int tb = 16 * J + 4 * q;
      float al0[4], al1[4];
      float tot0 = 0.f, tot1 = 0.f, p0 = 1.f, p1 = 1.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f16x2 la2 = *reinterpret_cast<const f16x2*>(&tla[swz<RB>(tb + u, i)]);
        const float l0 = (float)la2[0], l1 = (float)la2[1];
        al0[u] = ex(l0);
        al1[u] = ex(l1);
        tot0 += l0;
        tot1 += l1;
        p0 *= al0[u];
        p1 *= al1[u];
      }
      float pre0, pre1, suf0, suf1;
      group_products(p0, ln, &pre0, &suf0);
      group_products(p1, ln, &pre1, &suf1);
      tot0 = group_sum(tot0);
      tot1 = group_sum(tot1);
      // (the scaled operands are packed float16 products: the factors, all
      // <= 1, rounded to float16 first)
      float ec0 = pre0, ec1 = pre1;
      f16x2 qs2[4], kd2[4];
      f32x2 ecs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tb + u;
        ec0 *= al0[u];
        ec1 *= al1[u];
        ecs[u] = f32x2{ec0, ec1};
        const f16x2 q2 = *reinterpret_cast<const f16x2*>(&tq[swz<RB>(t, i)]);
        qs2[u] = q2 * __builtin_convertvector(ecs[u], f16x2);
      }
      float sfx0 = suf0, sfx1 = suf1;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        const f16x2 k2 = *reinterpret_cast<const f16x2*>(&tk[swz<RB>(tb + u, i)]);
        // k decayed to the sub-block end
        kd2[u] = k2 * __builtin_convertvector(f32x2{sfx0, sfx1}, f16x2);
        sfx0 *= al0[u];
        sfx1 *= al1[u];
      }
      if (q == 0) *reinterpret_cast<f32x2*>(&sTot[J][i]) = f32x2{tot0, tot1};
      // every wave holds its q, k and states; the sub-block totals are in
      wait_barrier<kLgkmZero>();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = swz<RB>(tb + u, i);
        *reinterpret_cast<f16x2*>(&tqs[e]) = qs2[u];
        *reinterpret_cast<f16x2*>(&tkd[e]) = kd2[u];
        *reinterpret_cast<f32x2*>(&sEc[(tb + u) * ES + i]) = ecs[u];
      }
      // B before each sub-block boundary for key dim ln (the boundary
      // factors), summed from the sub-block totals; the chunk total goes to
      // sBst for the next-state update
      float bs[5];
      bs[0] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) bs[j + 1] = bs[j] + sTot[j][ln];
      if (wave == 0) sBst[ln] = bs[4];
      // k decayed to the chunk end = k decayed to its sub-block end times the
      // decay of the later sub-blocks (log-alpha's tile is free now)
      float lt0 = 0.f, lt1 = 0.f;
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        if (j > J) {
          const f32x2 t2 = *reinterpret_cast<const f32x2*>(&sTot[j][i]);
          lt0 += t2[0];
          lt1 += t2[1];
        }
      }
      const f16x2 te2 = __builtin_convertvector(f32x2{ex(lt0), ex(lt1)}, f16x2);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = swz<RB>(tb + u, i);
        *reinterpret_cast<f16x2*>(&tke[e]) = kd2[u] * te2;
      }
      // factors between sub-block boundaries, thread (key dim, eighth): wave
      // w forms the pairs w, w + 8, .. (pair ab: a = ab / 5, b = ab % 5), each
      // as code of its own
      auto factor = [&](auto ab_c) __attribute__((always_inline)) {
        constexpr int ab = decltype(ab_c)::value;
        if constexpr (ab < 25) sF[ab / 5][ab % 5][ln] = (f16)ex(bs[ab / 5] - bs[ab % 5]);
      };
      auto factors = [&](auto w_c) __attribute__((always_inline)) {
        constexpr int w = decltype(w_c)::value;
        factor(std::integral_constant<int, w>{});
        factor(std::integral_constant<int, w + 8>{});
        factor(std::integral_constant<int, w + 16>{});
        factor(std::integral_constant<int, w + 24>{});
      };
      switch (wave) {
        case 0: factors(std::integral_constant<int, 0>{}); break;
        case 1: factors(std::integral_constant<int, 1>{}); break;
        case 2: factors(std::integral_constant<int, 2>{}); break;
        case 3: factors(std::integral_constant<int, 3>{}); break;
        case 4: factors(std::integral_constant<int, 4>{}); break;
        case 5: factors(std::integral_constant<int, 5>{}); break;
        case 6: factors(std::integral_constant<int, 6>{}); break;
        default: factors(std::integral_constant<int, 7>{}); break;
      }
      if (threadIdx.x == 0) sNext = to_second ? item + 1 : unit_chunk((int)gridDim.x + (int)ticket);
    }
    wait_barrier<kLgkmZero>();
    const int next = __builtin_amdgcn_readfirstlane(sNext);
    const bool more = next < total;

    // The next state: instantiated for each half of the waves, so that their
    // sub-blocks are constants and the loops over sub-block pairs unroll.
    // With PAIRS the lane's entries are also kept (float16), for a pair's
    // second chunk.
    f16x4 enext[2];
    auto next_state = [&](auto half) __attribute__((always_inline)) {
      constexpr int HF = decltype(half)::value;
      // ---- next state rows 16 kc + n (kc = 2 hf, 2 hf + 1), columns vj ..:
      // E_{c+1} = diag(e^{B_end}) E_c + Ke^T V; its row sums against R_c over
      // the wave's 16 value columns are its part of the carry (read after the
      // barrier before dlog-alpha)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kc = 2 * HF + x;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int P = 0; P < 2; ++P) {
          const f16x8 av = cat8(tr_read_l(tv, 32 * P, 16 * vb, ln), tr_read_l(tv, 32 * P + 16, 16 * vb, ln));
          const f16x8 bk = cat8(tr_read_l(tke, 32 * P, 16 * kc, ln), tr_read_l(tke, 32 * P + 16, 16 * kc, ln));
          acc = mma32(av, bk, acc);
        }
        // lane (n, g): E_next[i = 16 kc + n][j = 16 vb + 4g + u]
        const int i = 16 * kc + n16;
        const float ebe = ex(sBst[i]);
        const f16x4 e4 = e4h[x], r4 = r4h[x];
        float part = 0.f;
        f32x4 en;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          en[u] = ebe * (float)e4[u] + acc[u];
          part += en[u] * (float)r4[u];
        }
        if constexpr (PAIRS) enext[x] = to_f16(en);
        part = group_sum(part);
        if (g == 0) sCarry[vb][i] = part;
      }
    };
    if (hf == 0)
      next_state(std::integral_constant<int, 0>{});
    else
      next_state(std::integral_constant<int, 1>{});

    // ---- the score tiles (the ten sM tiles, then the ten sP tiles; wave w
    // forms tiles w, w + 8, w + 16), each once for all waves, each as code of
    // its own (its sub-blocks constants).  Lane (n, g) of a 16 x 16
    // accumulator holds row n, columns 4g .. 4g + 3 when the first operand
    // supplies the columns and the second the rows.
    const int soff = st_tile_off(n16, g);
    auto score_tile = [&](auto tau_c) __attribute__((always_inline)) {
      constexpr int tau = decltype(tau_c)::value;
      constexpr int pr = tau < 10 ? tau : tau - 10;
      constexpr int I = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
      constexpr int J = pr - I * (I + 1) / 2;
      if constexpr (tau < 10) {
        // rows s of J (values), columns t of I (output gradients)
        f32x4 sc = mma32(ld128(tdo + swz<RB>(16 * I + n16, 8 * g)),
                         ld128(tv + swz<RB>(16 * J + n16, 8 * g)), f32x4{0.f, 0.f, 0.f, 0.f});
        sc = mma32(ld128(tdo + swz<RB>(16 * I + n16, 32 + 8 * g)),
                   ld128(tv + swz<RB>(16 * J + n16, 32 + 8 * g)), sc);
        if constexpr (I == J) {
#pragma unroll
          for (int u = 0; u < 4; ++u) sc[u] = (n16 <= 4 * g + u) ? sc[u] : 0.f;
        }
        st64(sM[pr] + soff, to_f16(sc));
      } else {
        // rows s of I (Qs), columns t of J (Kd); the decay between the rows'
        // sub-block start and the columns' sub-block end sits on the key
        // dims: e^{Bst_I - Bst_{J+1}} (<= 1) on Qs for I > J, or
        // e^{Bst_J - Bst_{J+1}} (>= 1, back to the sub-block start) on Kd for
        // I = J (Qs stays <= |q|)
        f16x8 qa0 = ld128(tqs + swz<RB>(16 * I + n16, 8 * g));
        f16x8 qa1 = ld128(tqs + swz<RB>(16 * I + n16, 32 + 8 * g));
        f16x8 kx0 = ld128(tkd + swz<RB>(16 * J + n16, 8 * g));
        f16x8 kx1 = ld128(tkd + swz<RB>(16 * J + n16, 32 + 8 * g));
        const f16x8 f0 = ld128(&sF[I][J + 1][8 * g]);
        const f16x8 f1 = ld128(&sF[I][J + 1][32 + 8 * g]);
        if constexpr (I == J) {
          kx0 = kx0 * f0;
          kx1 = kx1 * f1;
        } else {
          qa0 = qa0 * f0;
          qa1 = qa1 * f1;
        }
        f32x4 sc = mma32(kx0, qa0, f32x4{0.f, 0.f, 0.f, 0.f});
        sc = mma32(kx1, qa1, sc);
        if constexpr (I == J) {
#pragma unroll
          for (int u = 0; u < 4; ++u) sc[u] = (n16 >= 4 * g + u) ? sc[u] : 0.f;
        }
        st64(sP[pr] + soff, to_f16(sc));
      }
    };
    using std::integral_constant;
    switch (wave) {
      case 0: score_tile(integral_constant<int, 0>{}); score_tile(integral_constant<int, 8>{});
              score_tile(integral_constant<int, 16>{}); break;
      case 1: score_tile(integral_constant<int, 1>{}); score_tile(integral_constant<int, 9>{});
              score_tile(integral_constant<int, 17>{}); break;
      case 2: score_tile(integral_constant<int, 2>{}); score_tile(integral_constant<int, 10>{});
              score_tile(integral_constant<int, 18>{}); break;
      case 3: score_tile(integral_constant<int, 3>{}); score_tile(integral_constant<int, 11>{});
              score_tile(integral_constant<int, 19>{}); break;
      case 4: score_tile(integral_constant<int, 4>{}); score_tile(integral_constant<int, 12>{}); break;
      case 5: score_tile(integral_constant<int, 5>{}); score_tile(integral_constant<int, 13>{}); break;
      case 6: score_tile(integral_constant<int, 6>{}); score_tile(integral_constant<int, 14>{}); break;
      default: score_tile(integral_constant<int, 7>{}); score_tile(integral_constant<int, 15>{}); break;
    }
    wait_barrier<kLgkmZero>();

    // dv, dq, dk and dlog-alpha: instantiated for each half of the waves, so that their
    // sub-blocks are constants and the loops over sub-block pairs unroll
    auto gradients = [&](auto half) __attribute__((always_inline)) {
      constexpr int HF = decltype(half)::value;
      // ---- dv (rows: value dims of this wave, columns: tokens of sub-block J)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int J = (x == 0 ? HF : 3 - HF);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = J; I < 4; ++I)
          acc = mma16(tr_read_l(tdo, 16 * I, 16 * vb, ln), tr_tile(sP[I * (I + 1) / 2 + J], ln), acc);
        // inter-chunk: (R^T Ke^T)[value dim][token], key dims in rta's order
        const int row = 16 * J + n16;
        f32x4 rk = mma32(rta[0], cat8(ld64(tke + swz<RB>(row, 4 * g)), ld64(tke + swz<RB>(row, 16 + 4 * g))),
                         f32x4{0.f, 0.f, 0.f, 0.f});
        rk = mma32(rta[1], cat8(ld64(tke + swz<RB>(row, 32 + 4 * g)), ld64(tke + swz<RB>(row, 48 + 4 * g))),
                   rk);
        store_grad4<ACC_V>(wdv, grad_off(gsv, row, vj), acc + rk);
      }

      // ---- dq (rows: key dims of this wave, columns: tokens of sub-block I):
      // the products first, which are the last reads of Kd and d_out
      f32x4 qacc[2], qed[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int I = (x == 0 ? HF : 3 - HF);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J <= I; ++J) {
          // Kd^T: key dim 16 kb + n, tokens 16J + 4g..; the row's factor is the
          // decay back to the sub-block start, k e^{-c} = Kd e^{Bst_J - Bst_{J+1}}
          // (>= 1) for J = I, or between the boundaries, e^{Bst_I - Bst_{J+1}}
          // (<= 1) for J < I; times (V dO^T)[s in J][t in I]
          const f16 fk = sF[I][J + 1][16 * kb + n16];
          acc = mma16(tr_read_l(tkd, 16 * J, 16 * kb, ln) * fk, tr_tile(sM[I * (I + 1) / 2 + J], ln), acc);
        }
        qacc[x] = acc;
        // inter-chunk: (E dO^T)[key dim][token]
        f32x4 ed = mma32(ea[0], ld128(tdo + swz<RB>(16 * I + n16, 8 * g)), f32x4{0.f, 0.f, 0.f, 0.f});
        qed[x] = mma32(ea[1], ld128(tdo + swz<RB>(16 * I + n16, 32 + 8 * g)), ed);
      }

      // e^c of this wave's dq / dk tiles (the same tokens and key dims), taken
      // out of the area the next chunk's states go into
      f32x4 ecr[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        ecr[x] = *reinterpret_cast<const f32x4*>(&sEc[(16 * (x == 0 ? HF : 3 - HF) + n16) * ES + ki]);

      // log-alpha (Ke), k (Kd), d_out and the states are done with: the next
      // chunk's go in
      Plan pn;
      if (more) {
        wait_barrier<kLgkmZero>();
        pn = plan(next, sel ^ 1, ln);
        load_k_side(pn, p.la, tla);
        load_k_side(pn, p.k, tk);
        load_v_side(pn, p.dout, tdo);
        load_states(next, ln, !to_second);
        if (PAIRS && to_second) {
          // the next chunk enters with this one's next state
#pragma unroll
          for (int x = 0; x < 2; ++x) st64(sE + swz<RB>(16 * (2 * HF + x) + n16, vj), enext[x]);
        }
      }

      // dq's scaling and stores
      f32x4 dqv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int I = (x == 0 ? HF : 3 - HF);
        const int t = 16 * I + n16;
        const f32x4 ec = ecr[x];
        const f16x4 fb = ld64(&sF[I][0][ki]);
        f32x4 dq;
#pragma unroll
        for (int u = 0; u < 4; ++u) dq[u] = ec[u] * (qacc[x][u] + (float)fb[u] * qed[x][u]);
        dqv[x] = dq;
        store_grad4<ACC_K>(wdq, grad_off(gsk, t, ki), dq);
      }

      // ---- dk (rows: key dims of this wave, columns: tokens of sub-block J)
      f32x4 dkv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int J = (x == 0 ? HF : 3 - HF);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = J; I < 4; ++I) {
          // Qs^T: key dim 16 kb + n, tokens 16I + 4g..; for I > J its row takes
          // the decay between the boundaries, e^{Bst_I - Bst_J} (<= 1); times
          // (dO V^T)[s in I][t in J], the transpose of an sM tile
          f16x4 aop = tr_read_l(tqs, 16 * I, 16 * kb, ln);
          if (I > J) aop = aop * sF[I][J][16 * kb + n16];
          acc = mma16(aop, ld64(sM[I * (I + 1) / 2 + J] + soff), acc);
        }
        // inter-chunk: (R V^T)[key dim][token]
        f32x4 rv = mma32(ra[0], ld128(tv + swz<RB>(16 * J + n16, 8 * g)), f32x4{0.f, 0.f, 0.f, 0.f});
        rv = mma32(ra[1], ld128(tv + swz<RB>(16 * J + n16, 32 + 8 * g)), rv);
        const int t = 16 * J + n16;
        const f32x4 ec = ecr[x];
        const f16x4 fe = ld64(&sF[4][J][ki]);
        f32x4 dk;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          dk[u] = __builtin_amdgcn_rcpf(ec[u]) * (acc[u] + (float)fe[u] * rv[u]);
        dkv[x] = dk;
        store_grad4<ACC_K>(wdk, grad_off(gsk, t, ki), dk);
      }

      // dlog_alpha terms of the wave's two sub-blocks, q dq - k dk per token
      // and key dim, summed over the tokens from each to its sub-block's end
      // (the 16 lanes of a tile row, lanes n .. 15); the sub-block totals go to
      // sTot
      f32x4 xs[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        f32x4 y;
#pragma unroll
        for (int u = 0; u < 4; ++u) y[u] = (float)q4r[x][u] * dqv[x][u] - (float)k4r[x][u] * dkv[x][u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y[u] += dpp_f<kRowShl + 1>(y[u]);
          y[u] += dpp_f<kRowShl + 2>(y[u]);
          y[u] += dpp_f<kRowShl + 4>(y[u]);
          y[u] += dpp_f<kRowShl + 8>(y[u]);
        }
        xs[x] = y;
        if (n16 == 0) *reinterpret_cast<f32x4*>(&sTot[(x == 0 ? HF : 3 - HF)][ki]) = y;   // the row's total
      }
      // q (Qs) and v are done with as well: the next chunk's go in (the
      // barrier also makes the sub-block totals and the carry visible)
      wait_barrier<kLgkmZero>();
      if (more) {
        load_k_side(pn, p.q, tq);
        load_v_side(pn, p.v, tv);
      }

      // dlog_alpha = the in-sub-block suffix sum + the later sub-blocks' totals
      // + the carry (the four value blocks' row sums)
      const f32x4 carry = ((*reinterpret_cast<const f32x4*>(&sCarry[0][ki]) +
                            *reinterpret_cast<const f32x4*>(&sCarry[1][ki])) +
                           *reinterpret_cast<const f32x4*>(&sCarry[2][ki])) +
                          *reinterpret_cast<const f32x4*>(&sCarry[3][ki]);
      f32x4 tot[4];
#pragma unroll
      for (int I2 = 1; I2 < 4; ++I2) tot[I2] = *reinterpret_cast<const f32x4*>(&sTot[I2][ki]);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int I = (x == 0 ? HF : 3 - HF);
        f32x4 run = carry;
#pragma unroll
        for (int I2 = 3; I2 > 0; --I2)
          if (I2 > I) run += tot[I2];
        store_grad4<ACC_K>(wdla, grad_off(gsk, 16 * I + n16, ki), xs[x] + run);
      }
    };
    if (hf == 0)
      gradients(std::integral_constant<int, 0>{});
    else
      gradients(std::integral_constant<int, 1>{});
    item = next;
  }
}

}  // namespace

hipError_t launch_bwd_chunks(int d_k, int d_v, const BwdParams& p, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
  if (d_k != 64 || d_v != 64) return hipErrorInvalidValue;
  const dim3 grid(p.n_wg), block(kThreads);
  auto pick = [&](auto pairs) {
    constexpr bool PR = decltype(pairs)::value;
    return p.acc_dv ? (p.acc_dqk ? chunk_bwd_f16_kernel<64, 64, true, true, PR>
                                 : chunk_bwd_f16_kernel<64, 64, true, false, PR>)
                    : (p.acc_dqk ? chunk_bwd_f16_kernel<64, 64, false, true, PR>
                                 : chunk_bwd_f16_kernel<64, 64, false, false, PR>);
  };
  const auto kernel = p.fwd_span == 2 ? pick(std::true_type{}) : pick(std::false_type{});
  if (start != nullptr || stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gla

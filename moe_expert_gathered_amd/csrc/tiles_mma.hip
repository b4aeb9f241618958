// Row tiles of 16 * MI sorted rows x 256 MFMA columns (MI = 8: experts that
// receive many rows, and dense many-row products; MI = 2: one tile per expert
// with fewer than 32 rows), weights dequantized straight into matrix-core
// registers.
//
// MLX PR 4567 (Proposed changes): each tile carries a row start, one expert
// and a valid-row count, so it makes exactly one K pass over one expert.
// MTPLX PR 558 (Change): the rows are the expert-sorted (token, slot) pairs;
// the gate/up pass gathers activation rows through lhs, the down pass reads
// the sorted intermediate rows in order.
//
// gfx950 mapping (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//  * 4 waves; each wave owns all 16 * MI rows and 64 MFMA columns (MI x 4
//    blocks; 128 fp32 accumulators at MI = 8).  A column's codes are read by exactly one wave,
//    so each code is dequantized once per tile, in registers, in the layout
//    the MFMA operand wants: lane (g = lane / 16, c = lane % 16) holds for
//    column c the 32 consecutive k of lane group g (k0 + 32 g ..), which it
//    loads as one (4-bit) or two (8-bit) 128-bit buffer loads.  Inside a K
//    step of 128, MFMA sub-step s contracts k0 + 32 g + 8 s + (0..7) in lane
//    group g; both operands use that same assignment, so the sum is the full
//    dot product over K.  Weights are dequantized to bf16 in natural k order
//    (deq4_bf16 / deq8_bf16).
//  * The activation rows are the caller's bf16 rows (gate/up: x gathered
//    through lhs; down: the bf16 intermediate), used as stored: no
//    conversion pass, and bf16's whole range.  They travel from HBM to LDS
//    with buffer loads that write LDS directly (no register staging), into a
//    ring of stages (4 KiB per 16 rows each), each row's 16-byte chunks
//    permuted (lds_swz) so that operand reads are free of bank conflicts.
//  * GLU: a wave's 4 column blocks are (gate f, up f, gate f+16, up f+16), so
//    silu(g) * u is applied in registers in the epilogue.
//  * The weights are the MFMA's first operand: each lane ends with four
//    consecutive output features of one row and writes them as one 8-byte
//    store.
//  * One barrier per K step: the next step's activations and codes are all
//    issued at the step's start and are in flight during its MFMAs.
//  * Workgroups are dealt to the 8 XCDs round-robin by the hardware; the
//    block index is remapped so that each XCD works on a contiguous range of
//    (tile, column block) pairs: the column blocks of one row tile, and the
//    consecutive tiles of one expert, then share that XCD's L2.
//  * An optional extra expert (index E, its own weight pointers) carries the
//    shared expert through the same launch.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "sort_dev.h"

namespace moegq {

constexpr int TM_C = 256;   // MFMA columns per tile
constexpr int TM_K = 128;   // K per step

// LDS slot permutation of a 256-byte activation row: row r keeps its 16-byte
// chunk c in slot c ^ lds_swz(r).  The 16 rows that one ds_read_b128 of an
// MFMA operand touches then spread over all banks (measured conflict-free on
// gfx950; a plain c ^ r still collides across lane groups).
MOEGQ_DEV int lds_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// The fp16 gate/up operands of 4-bit codes use subnormal codes: a code byte
// under a zero byte is the fp16 subnormal q * 2^-24, exactly, so with
// S = s * 2^24 one fused multiply-add gives q * s + b rounded once: two
// instructions per pair of codes (v_perm, v_pk_fma_f16), where the 1024 + q
// encoding needs its offset subtracted first.  S stays finite because the
// column's scaling puts every |s| * qmax below 2^-5.  The products are the
// same bits as with the 1024 + q encoding (the two scalings differ by an
// exact power of two).  8-bit codes keep the 1024 + q encoding (deq8_f16,
// column maximum in [2^13, 2^14)): their subnormal variant spilled registers
// and ran slower.
constexpr bool subnormal_codes(int bits) { return bits == 4; }

// eight codes (one 4-bit word, or two 8-bit words) -> one fp16 MFMA operand
// (4-bit: in the order q0 q2 q4 q6 q1 q3 q5 q7; 8-bit: natural).  s2 and b2
// are the group's scale (4-bit: times 2^24) and bias after the column scaling.
template <int BITS>
MOEGQ_DEV f16x8_t deq_operand_f16(uint32_t w0, uint32_t w1, f16x2_t s2, f16x2_t b2) {
  uint32_t o[4];
  if constexpr (subnormal_codes(BITS)) {
    auto pair = [&](uint32_t codes, uint32_t sel) -> uint32_t {
      const f16x2_t q = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0u, codes, sel));
      return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
    };
    const uint32_t lo = w0 & 0x0F0F0F0Fu, hi = (w0 >> 4) & 0x0F0F0F0Fu;   // bytes q0 q2 q4 q6 / q1 q3 q5 q7
    o[0] = pair(lo, 0x04010400u);
    o[1] = pair(lo, 0x04030402u);
    o[2] = pair(hi, 0x04010400u);
    o[3] = pair(hi, 0x04030402u);
  } else {
    deq8_f16(w0, s2, b2, o);
    deq8_f16(w1, s2, b2, o + 2);
  }
  return __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}
// the same as one bf16 operand in natural k order; s the group's scale, c = b - 1024 s
template <int BITS>
MOEGQ_DEV bf16x8_t deq_operand_bf16(uint32_t w0, uint32_t w1, float s, float c) {
  uint32_t o[4];
  if (BITS == 4) {
    deq4_bf16(w0, s, c, o);
  } else {
    deq8_bf16(w0, s, c, o);
    deq8_bf16(w1, s, c, o + 2);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// One tile: rows r0 .. r1 - 1 of expert e, MFMA columns n0 .. n0 + 255.
// Four distinct __shared__ arrays L[0..3] of LQ halfs each hold the
// activation ring: RA stages of 16 * MI rows x TM_K 16-bit values.
template <int MI, int BITS = 4> struct MmaRing {
  // K steps of activation (LDS) and code (register) prefetch: one for 128-row
  // tiles and for bf16 weights (register-bound), three for the shorter tiles
  static constexpr int PDA = (MI >= 8 || BITS == 16) ? 1 : 3;
  static constexpr int PDB = PDA;
  static constexpr int RA = PDA + 1, RB = PDB + 1;              // LDS and register ring stages
  static constexpr int U = (RA % RB == 0) ? RA : (RB % RA == 0) ? RB : RA * RB;   // steps per unrolled loop
  static constexpr int LQ = (MI >= 8 ? 64 : 16 * MI) * TM_K;     // halfs per ring array
};

// Operand precision per pass:
//  * gate/up (GLU, quantized weights): fp16 operands.  The activation rows
//    arrive as fp16 copies scaled by 2^-xexp[row] (launch_front / launch_prep:
//    the row's largest magnitude lands in [2^13, 2^14)), and each weight
//    column is scaled by 2^-ec, ec taken at the tile's start from the
//    column's largest |s| * qmax + |b| over all its groups (it lands in
//    [2^-6, 2^-5) for 4-bit codes, [2^13, 2^14) for 8-bit ones); the
//    epilogue multiplies the fp32 result by 2^(xexp + ec).  The scalings are
//    exact, so the products keep fp16's 11-bit weights (the precision
//    silu(g) * u needs: it rounds g and u to bf16 first) over bf16's whole
//    range.  A 4-bit dequantized weight more than about 2^9 below its
//    column's largest one is an fp16 subnormal (the matrix cores take fp16
//    subnormals as they are): rounded to a multiple of 2^-24, under 2^-19 of
//    the column's largest weight.
//  * down (and any pass without GLU): bf16 operands, the intermediate as
//    stored, weights dequantized to bf16.
//  * BITS = 16: the expert matrices are plain bf16 (no scales or biases);
//    their words go to the MFMA as loaded.
// xe_s: LDS for 16 * MI row exponents (gate/up pass).
template <int BITS, int GS, bool GLU, int MI>
MOEGQ_DEV void tile_body(const TileArgs& A, uint16_t* L0, uint16_t* L1, uint16_t* L2, uint16_t* L3, int* xe_s,
                         int r0, int r1, int e, int n0) {
  constexpr bool W16 = BITS == 16;
  constexpr bool F16 = GLU && !W16;
  constexpr int CB = 4 * BITS;                    // code bytes per lane per K step (32 codes)
  using Ring = MmaRing<MI, BITS>;
  constexpr int PDA = Ring::PDA, PDB = Ring::PDB, RA = Ring::RA, RB = Ring::RB, U = Ring::U;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  // The ring in four quarters L[0..3] of LQ halfs, which the compiler keeps
  // apart when it places its own waits if they are distinct __shared__
  // arrays: with the ring in one array it made a step's LDS reads wait for
  // the activation loads just issued into another stage, so the step's MFMAs
  // waited for the next step's rows.  RA = 4 (32- and 64-row tiles): stage s
  // in L[s].  RA = 2, 128 rows: stage s in L[2 s] (rows 0-63) and L[2 s + 1]
  // (rows 64-127), and each wave fills 16 rows of each half (so that every
  // load's array is a compile-time constant).  The 8-bit kernels, at the
  // register limit, keep the ring in one array (L[k] its quarters), a wave
  // filling 32 consecutive rows, the barrier's release fence and the window
  // loads in the switching step: each of these changes moved their spills
  // into the loop (3.37 against 2.96 ms for the 4123-row 8-bit layer).
  static_assert(RA * 16 * MI <= 4 * (MI >= 8 ? 64 : 16 * MI) && (MI < 8 || RA == 2), "ring layout");
  constexpr bool HALVES = MI >= 8 && BITS == 4;
  auto ring = [&](int k) -> uint16_t* { return k == 0 ? L0 : k == 1 ? L1 : k == 2 ? L2 : L3; };
  // row of the tile (without the lane group's g) that load v of this wave fills
  auto row_of = [&](int v) -> int {
    if constexpr (HALVES) return v < 4 ? 16 * wave + 4 * v : 64 + 16 * wave + 4 * (v - 4);
    else return 4 * (MI * wave + v);
  };
  // destination of load v in stage st, and row block i (16 rows) of stage st
  auto dma_dst = [&](int st, int v) -> uint16_t* {
    if constexpr (HALVES) return ring(2 * st + v / 4) + (row_of(v) % 64) * TM_K;
    else return ring(MI >= 8 ? 2 * st : st) + row_of(v) * TM_K;
  };
  auto row_blk = [&](int st, int i) -> const uint16_t* {
    if constexpr (HALVES) return ring(2 * st + i / 4) + (i % 4) * 16 * TM_K;
    else return ring(MI >= 8 ? 2 * st : st) + i * 16 * TM_K;
  };
  const int N = A.N, K = A.K;
  const int Kw = K * BITS / 32, G = K / GS;
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  e = __builtin_amdgcn_readfirstlane(e);

  // ---- activation loads: load v of a wave covers rows row_of(v) .. + 3; lane
  //      (g, c16) fetches chunk c16 ^ lds_swz(row) of row row_of(v) + g
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A.x, 0xFFFFFFFFu);
  uint32_t a_off[8];                          // MI <= 8 entries used
  // virtual row rr = batch rr / rpb, row rr % rpb of it; the batch's x rows start at
  // (lhs ? lhs[batch] : batch / lhs_div) * rpb (rpb and lhs_div of 0 mean 1).  The
  // conditions are uniform and tested once, so the MI index loads are issued
  // together and waited for once.
  int rr[8], bt[8];
  const bool batched = A.rows_per_batch > 1;
  const int rpb = batched ? (int)A.rows_per_batch : 1;
#pragma unroll
  for (int v = 0; v < MI; ++v) {
    rr[v] = min(r0 + row_of(v) + g, r1 - 1);   // rows past the tile repeat a valid row (never stored)
    bt[v] = batched ? rr[v] / rpb : rr[v];
  }
  if (A.lhs) {
#pragma unroll
    for (int v = 0; v < MI; ++v) bt[v] = A.lhs[bt[v]];
  } else if (A.lhs_div > 1) {
#pragma unroll
    for (int v = 0; v < MI; ++v) bt[v] /= (int)A.lhs_div;
  }
#pragma unroll
  for (int v = 0; v < MI; ++v) {
    const int src = batched ? bt[v] * rpb + rr[v] % rpb : bt[v];
    const int chunk = c16 ^ lds_swz(row_of(v) + g);
    a_off[v] = (uint32_t)src * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
    // the row exponents of the fp16 activations, for the epilogue (row-major
    // position in the tile; one lane per row writes)
    if (F16 && c16 == 0) xe_s[row_of(v) + g] = A.xexp[src];
  }
  // ---- code / scale loads: column block j of this wave
  const size_t wstride = (size_t)N * Kw, sstride = (size_t)N * G;
  const bool ex = e >= A.E;          // the extra (shared) expert
  const size_t eo = ex ? 0 : (size_t)e;
  const __amdgpu_buffer_rsrc_t rw0 = make_rsrc((ex ? A.xw0 : A.w0) + eo * wstride, (uint32_t)(wstride * 4));
  const uint16_t* s0p = W16 ? A.s0 : (ex ? A.xs0 : A.s0) + eo * sstride;   // unused for bf16 weights
  const uint16_t* b0p = W16 ? A.b0 : (ex ? A.xb0 : A.b0) + eo * sstride;
  const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(s0p, W16 ? 0u : (uint32_t)(sstride * 2));
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(b0p, W16 ? 0u : (uint32_t)(sstride * 2));
  __amdgpu_buffer_rsrc_t rw1 = rw0, rs1 = rs0, rb1 = rb0;
  if (GLU) {
    rw1 = make_rsrc((ex ? A.xw1 : A.w1) + eo * wstride, (uint32_t)(wstride * 4));
    if (!W16) {
      rs1 = make_rsrc((ex ? A.xs1 : A.s1) + eo * sstride, (uint32_t)(sstride * 2));
      rb1 = make_rsrc((ex ? A.xb1 : A.b1) + eo * sstride, (uint32_t)(sstride * 2));
    }
  }
  // MFMA column n of block j is output feature block_base(j) + n.  The MFMA
  // runs with the weights as the first operand, so lane (g, c16) ends up with
  // outputs n = 4 g .. 4 g + 3 of activation row c16, next to each other in
  // memory (one 8-byte store).
  auto block_base = [&](int j) { return GLU ? n0 + 32 * wave + 16 * (j >> 1) : n0 + 64 * wave + 16 * j; };
  uint32_t w_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = block_base(j) + c16;
    const int fr = min(col, N - 1);               // columns past N repeat a valid one (never stored)
    w_off[j] = (uint32_t)fr * (uint32_t)Kw * 4u + (uint32_t)(g * CB);
  }
  // Scales and biases come in windows of 8 groups: lane l of the wave fetches
  // the window of the wave's column block l / 16, column l % 16, with one
  // 16-byte load per array (instead of one 2-byte load per column block, array
  // and K step); each step's lanes then pick their group with ds_bpermute.
  // Window w covers groups 8 w .. 8 w + 7, i.e. K steps GS / 16 * w ..
  constexpr int WSTEPS = GS / 16;
  const int lj = lane >> 4;
  const int lcol = block_base(lj) + c16;
  const uint32_t sw_off = (uint32_t)min(lcol, N - 1) * (uint32_t)G * 2u;
  const bool lup = GLU && (lj & 1);
  auto load_win = [&](int w, uint4& ws, uint4& wb) {
    const uint32_t soff = (uint32_t)w * 16u;
    ws = buf_load16(rs0, sw_off, soff);
    wb = buf_load16(rb0, sw_off, soff);
    if (GLU) {
      const uint4 us = buf_load16(rs1, sw_off, soff), ub = buf_load16(rb1, sw_off, soff);
      if (lup) { ws = us; wb = ub; }
    }
  };
  int ecol = 0, ecj[4] = {0, 0, 0, 0};
  // group of (lane group g, step ks) inside its window: e = (8 ks / WSTEPS + 32 g / GS) % 8;
  // the dword holding it is the same for every lane except at GS = 32
  auto sel4 = [](const uint4& v, int d) -> uint32_t {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
  };
  auto pick = [&](const uint4& win, int ks, int j) -> float {
    const int src = (16 * j + c16) << 2;
    if (GS == 32) {          // e = 4 (ks % 2) + g: dword 2 (ks % 2) + g / 2, half g % 2
      const int d0 = 2 * (ks & 1);
      const uint32_t lo = __builtin_amdgcn_ds_bpermute(src, (int)sel4(win, d0));
      const uint32_t hi = __builtin_amdgcn_ds_bpermute(src, (int)sel4(win, d0 + 1));
      const uint32_t d = (g & 2) ? hi : lo;
      return (g & 1) ? bf16_hi(d) : bf16_lo(d);
    } else if (GS == 64) {   // e = 2 (ks % 4) + g / 2: dword ks % 4, half g / 2
      const uint32_t d = __builtin_amdgcn_ds_bpermute(src, (int)sel4(win, ks & 3));
      return (g & 2) ? bf16_hi(d) : bf16_lo(d);
    } else {                 // e = ks % 8: dword (ks % 8) / 2, half ks % 2
      const uint32_t d = __builtin_amdgcn_ds_bpermute(src, (int)sel4(win, (ks >> 1) & 3));
      return (ks & 1) ? bf16_hi(d) : bf16_lo(d);
    }
  };
  auto ld_codes = [&](int j, uint32_t soff) -> uint4 {
    return buf_load16((GLU && (j & 1)) ? rw1 : rw0, w_off[j], soff);
  };

  f32x4_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nK = K / TM_K;
  // ring of code registers: stage t % RB holds step t's codes (fixed extents:
  // the unused stages and halves are never touched and cost no registers)
  uint4 cw[4][4][W16 ? 4 : 2];
  uint4 win_s, win_b, nwin_s, nwin_b;
  constexpr int LPS = MI + 4 * (BITS / 4);        // loads per step: activations + codes
  // part p (0..3) of step t's loads: activation rows into LDS stage sa, codes of block p into register stage sb
  auto issue_a = [&](int t, int sa, int part) {
    if (t >= nK) return;
    constexpr int AV = (MI + 3) / 4;
#pragma unroll
    for (int v = part * AV; v < (part + 1) * AV && v < MI; ++v) {
      uint16_t* dst = dma_dst(sa, v);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)dst, 16, a_off[v],
                                               (uint32_t)t * TM_K * 2u, 0, 0);
    }
  };
  auto issue_b = [&](int t, int sb, int part) {
    if (t >= nK) return;
    const uint32_t soff = (uint32_t)t * TM_K * BITS / 8;
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h) cw[sb][part][h] = ld_codes(part, soff + 16 * h);
  };
  auto step = [&](int ks, auto phase) {
    constexpr int sa = decltype(phase)::value % RA, sb = decltype(phase)::value % RB;
    constexpr int fa = (sa + PDA) % RA, fb = (sb + PDB) % RB;
    // step ks's loads were issued at the start of step ks - PD, and the PD - 1 later steps'
    // loads after them (the compiler may move a step's loads within the step's first
    // sub-step, never across the scheduling barrier that ends that sub-step; extra window
    // loads only lengthen the wait)
    // Other waves read the rows this wave loaded, so its own loads of step ks
    // must be complete before it reaches the barrier: nothing but this wait
    // ensures that.  Steps past the end issue no loads, so near the end fewer
    // loads follow step ks's and the count shrinks with them.  lgkmcnt(0)
    // completes this wave's LDS writes (the row exponents) before the barrier.
    constexpr int VM = (PDA - 1) * LPS;
    static_assert(VM < 64 && (PDA == 1 || PDA == 3), "vmcnt range");
    auto wait_vm = [](auto n) {
      constexpr int c = decltype(n)::value;
      __builtin_amdgcn_s_waitcnt(0x0070 | (c & 15) | ((c >> 4) << 14));
    };
    if constexpr (BITS == 8) {
      // the 8-bit kernels keep the barrier's release fence, which completes
      // every load into LDS before the barrier anyway
      __builtin_amdgcn_s_waitcnt(0x0F70 | (VM & 15) | ((VM >> 4) << 14));
    } else if (PDA == 1 || ks + PDA - 1 < nK) {
      wait_vm(std::integral_constant<int, VM>{});
    } else if (ks + 1 < nK) {
      wait_vm(std::integral_constant<int, LPS>{});
    } else {
      wait_vm(std::integral_constant<int, 0>{});
    }
    // every wave's rows landed (each wave's own wait above) and every wave
    // has consumed its reads of step ks - 1's stage (each LDS read feeds an
    // MFMA of its step), so that stage is free.  The barrier takes no
    // release fence (8-bit codes aside): one would make it wait for every
    // LDS-bound load in flight, including those of later steps; the acquire
    // keeps this step's LDS reads after the barrier.
    if constexpr (BITS == 8) {
      __syncthreads();
    } else {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    f16x2_t s2[4], b2[4];
    float sj[4], cj[4];
    if constexpr (!W16) {
      // the next window is requested a step after the switch (8-bit codes
      // aside): its loads then write nwin's registers directly (issued in the
      // switching step, they went through temporaries whose copy waited for
      // them)
      if (BITS == 8) {
        if (ks % WSTEPS == 0) {
          win_s = nwin_s; win_b = nwin_b;
          if ((ks + WSTEPS) < nK) load_win(ks / WSTEPS + 1, nwin_s, nwin_b);
        }
      } else if (ks % WSTEPS == 0) {
        win_s = nwin_s; win_b = nwin_b;
      } else if (ks % WSTEPS == 1 && (ks - 1 + WSTEPS) < nK) {
        load_win(ks / WSTEPS + 1, nwin_s, nwin_b);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (F16) {
          s2[j] = f16_splat(__builtin_ldexpf(pick(win_s, ks, j), (subnormal_codes(BITS) ? 24 : 0) - ecj[j]));
          b2[j] = f16_splat(__builtin_ldexpf(pick(win_b, ks, j), -ecj[j]));
        } else {
          sj[j] = pick(win_s, ks, j);
          cj[j] = bias1024(sj[j], pick(win_b, ks, j));
        }
      }
    }
    // every load of step ks + PD at the step's start, so that each has a
    // whole step to land (issued a quarter per sub-step, the last quarter
    // had a quarter of a step: 3% slower at the 2048-row layer)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      issue_a(ks + PDA, fa, s);
      issue_b(ks + PDB, fb, s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t* wv = &cw[sb][j][0].x;
        if constexpr (W16) bq[j] = cw[sb][j][s];   // k 32 g + 8 s .. + 7
        else if constexpr (F16 && BITS == 4) bq[j] = __builtin_bit_cast(uint4, deq_operand_f16<4>(wv[s], 0, s2[j], b2[j]));
        else if constexpr (F16) bq[j] = __builtin_bit_cast(uint4, deq_operand_f16<8>(wv[2 * s], wv[2 * s + 1], s2[j], b2[j]));
        else if constexpr (BITS == 4) bq[j] = __builtin_bit_cast(uint4, deq_operand_bf16<4>(wv[s], 0, sj[j], cj[j]));
        else bq[j] = __builtin_bit_cast(uint4, deq_operand_bf16<8>(wv[2 * s], wv[2 * s + 1], sj[j], cj[j]));
      }
      const int slot = (4 * g + s) ^ lds_swz(c16);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4 a = *reinterpret_cast<const uint4*>(row_blk(sa, i) + c16 * TM_K + slot * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, bq[j]),
                                                               __builtin_bit_cast(f16x8_t, a), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bq[j]),
                                                                __builtin_bit_cast(bf16x8_t, a), acc[i][j], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (!W16) {
    load_win(0, win_s, win_b);
    nwin_s = win_s; nwin_b = win_b;
  }
  // prologue: activations of steps 0 .. PDA - 1, codes of steps 0 .. PDB - 1, in step order
#pragma unroll
  for (int t = 0; t < (PDA > PDB ? PDA : PDB); ++t)
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      if (t < PDA) issue_a(t, t % RA, part);
      if (t < PDB) issue_b(t, t % RB, part);
    }
  // fp16 weight columns: the owner lane of column (block lj, c16) finds the
  // column's exponent from all its groups' scales and biases; ecj[j] is the
  // exponent of this lane's column in block j (the picks), taken from its
  // owner.  Done after the prologue's loads are issued, so they are in flight
  // meanwhile.
  if constexpr (F16) {
    constexpr float QMAX = (float)((1 << BITS) - 1);
    const int nwin = G / 8;
    float mx = 0.f;
    for (int w0 = 0; w0 < nwin; w0 += 4) {        // four windows' loads in flight at a time
      uint4 ws[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) load_win(min(w0 + i, nwin - 1), ws[i], wb[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ds[4] = {ws[i].x, ws[i].y, ws[i].z, ws[i].w}, db[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          mx = fmaxf(mx, __builtin_fmaf(fabsf(bf16_lo(ds[d])), QMAX, fabsf(bf16_lo(db[d]))));
          mx = fmaxf(mx, __builtin_fmaf(fabsf(bf16_hi(ds[d])), QMAX, fabsf(bf16_hi(db[d]))));
        }
      }
    }
    // subnormal codes: mx * 2^-ecol in [2^-6, 2^-5), so S = s' * 2^24 < 2^19 / qmax
    // is a finite fp16; else mx * 2^-ecol in [2^13, 2^14)
    if constexpr (subnormal_codes(BITS)) ecol = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) + 5 : 0;
    else ecol = f16_exponent(mx);
#pragma unroll
    for (int j = 0; j < 4; ++j) ecj[j] = __shfl(ecol, 16 * j + c16, 64);
  }
  using std::integral_constant;
  for (int ks = 0; ks < nK; ks += U) {
    step(ks, integral_constant<int, 0>{});
    if (U > 1 && ks + 1 < nK) step(ks + 1, integral_constant<int, 1 % U>{});
    if (U > 2 && ks + 2 < nK) step(ks + 2, integral_constant<int, 2 % U>{});
    if (U > 3 && ks + 3 < nK) step(ks + 3, integral_constant<int, 3 % U>{});
    if (U > 4 && ks + 4 < nK) step(ks + 4, integral_constant<int, 4 % U>{});
    if (U > 5 && ks + 5 < nK) step(ks + 5, integral_constant<int, 5 % U>{});
  }
  static_assert(U <= 6, "unroll");

  // epilogue: acc[i][j][q] = output (row 16 i + c16, memory column block_base(j) + 4 g + q);
  // the fp16 pass undoes its scalings: column (j, 4 g + q) is owned by lane 16 j + 4 g + q
  int eo_col[4][4];
  if constexpr (F16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) eo_col[j][q] = __shfl(ecol, 16 * j + 4 * g + q, 64);
  }
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = r0 + 16 * i + c16;
    if (r >= r1) continue;
    const int xe = F16 ? xe_s[16 * i + c16] : 0;
    uint16_t* orow = A.out + (size_t)r * N;
#pragma unroll
    for (int j = 0; j < (GLU ? 2 : 4); ++j) {
      const int f = (GLU ? block_base(2 * j) : block_base(j)) + 4 * g;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GLU) {
          float gv = acc[i][2 * j][q], uv = acc[i][2 * j + 1][q];
          if (F16) {
            gv = __builtin_ldexpf(gv, xe + eo_col[2 * j][q]);
            uv = __builtin_ldexpf(uv, xe + eo_col[2 * j + 1][q]);
          }
          v[q] = glu(gv, uv);
        } else {
          v[q] = acc[i][j][q];
        }
      }
      // round to nearest even, two outputs per conversion
      const uint32_t lo = pk_bf16(v[0], v[1]), hi = pk_bf16(v[2], v[3]);
      if (vec && f + 3 < N) {
        *reinterpret_cast<uint2*>(orow + f) = make_uint2(lo, hi);
      } else {
        const uint16_t o[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (f + q < N) orow[f + q] = o[q];
      }
    }
  }
}

// With 4-bit codes, a 128-row tile with at most 32 (64) rows, often an
// expert's last one, runs as a 32-row (64-row) tile: the MFMAs of the 16-row
// blocks past its rows would compute outputs that are never stored.  The
// smaller bodies need no more LDS than the 128-row one.  With 8-bit codes the
// extra bodies push the kernel's registers into spills, so it keeps one body.
template <int BITS, int GS, bool GLU, int MI>
MOEGQ_DEV void tile_rows(const TileArgs& A, uint16_t* L0, uint16_t* L1, uint16_t* L2, uint16_t* L3, int* xe_s,
                         int r0, int r1, int e, int n0) {
  const int nrow = __builtin_amdgcn_readfirstlane(r1 - r0);
  if constexpr (MI == 8 && BITS == 4) {
    static_assert(MmaRing<4, BITS>::LQ <= MmaRing<8, BITS>::LQ && MmaRing<2, BITS>::LQ <= MmaRing<8, BITS>::LQ,
                  "LDS ring");
    if (nrow <= 32) return tile_body<BITS, GS, GLU, 2>(A, L0, L1, L2, L3, xe_s, r0, r1, e, n0);
    if (nrow <= 64) return tile_body<BITS, GS, GLU, 4>(A, L0, L1, L2, L3, xe_s, r0, r1, e, n0);
  }
  tile_body<BITS, GS, GLU, MI>(A, L0, L1, L2, L3, xe_s, r0, r1, e, n0);
}

// XCD-contiguous ranges: the hardware deals workgroups to the 8 XCDs round
// robin; block b of a range of `total` goes to XCD b % 8, so logical id
// (b % 8) * q + b / 8 keeps neighbours (column blocks of one tile, tiles of
// one expert) on one XCD's L2.  The last total % 8 blocks keep their index.
MOEGQ_DEV int xcd_remap(int b, int total) {
  const int q = total / 8;
  return b < 8 * q ? (b % 8) * q + b / 8 : b;
}

// The activation ring's quarters L0..L3 (tile_body): four distinct arrays,
// or with 8-bit codes the quarters of one array.
#define RING_ARRAYS(LQ)                                                            \
  __shared__ __attribute__((aligned(16))) uint16_t RA0[BITS == 8 ? 4 * (LQ) : (LQ)]; \
  __shared__ __attribute__((aligned(16))) uint16_t RA1[BITS == 8 ? 1 : (LQ)];        \
  __shared__ __attribute__((aligned(16))) uint16_t RA2[BITS == 8 ? 1 : (LQ)];        \
  __shared__ __attribute__((aligned(16))) uint16_t RA3[BITS == 8 ? 1 : (LQ)];        \
  uint16_t* const L0 = RA0;                                                          \
  uint16_t* const L1 = BITS == 8 ? RA0 + (LQ) : RA1;                                 \
  uint16_t* const L2 = BITS == 8 ? RA0 + 2 * (LQ) : RA2;                             \
  uint16_t* const L3 = BITS == 8 ? RA0 + 3 * (LQ) : RA3

// register budget: 2 workgroups per CU (128 accumulators per lane at MI = 8;
// the 32-row variant needs far fewer registers)
template <int BITS, int GS, bool GLU, int MI>
__global__ __launch_bounds__(256, 2) void tile_mma_kernel(TileArgs A) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;      // output features per tile
  constexpr int LQ = MmaRing<MI, BITS>::LQ;
  RING_ARRAYS(LQ);
  __shared__ int xe_s[16 * MI];
  const int NB = (A.N + NF - 1) / NF;
  const int total = A.tile_mode == 2 ? (int)gridDim.x : *A.n_tiles * NB;
  if ((int)blockIdx.x >= total) return;
  const int bid = xcd_remap(blockIdx.x, total);
  const int tile = bid / NB, n0 = (bid % NB) * NF;
  int r0, r1, e;
  if (A.tile_mode == 2) {            // dense rows, one weight matrix
    r0 = tile * 16 * MI;
    if (r0 >= A.P) return;
    r1 = (int)min(A.P, (int64_t)r0 + 16 * MI);
    e = 0;
  } else {
    const int32_t* t = A.tiles + 3 * tile;
    r0 = t[0]; e = t[1]; r1 = r0 + t[2];
  }
  tile_rows<BITS, GS, GLU, MI>(A, L0, L1, L2, L3, xe_s, r0, r1, e, n0);
}

// Both tile tables in one launch: blocks [0, n_big * NB) take the 128-row
// (bf16 weights: 64-row) tiles of `tiles`, the next n_small * NB blocks the
// 32-row tiles of `tiles2`.
// The few-row tiles stream their experts' weights from HBM while the last
// round of 128-row tiles keeps only part of the machine busy.
template <int BITS, int GS, bool GLU>
__global__ __launch_bounds__(256, 2) void tile_mma_dual_kernel(TileArgs A) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  constexpr int MIB = BITS == 16 ? 4 : 8;   // bf16 weights: 64-row big tiles (register budget)
  constexpr int LQ = MmaRing<MIB, BITS>::LQ > MmaRing<2, BITS>::LQ ? MmaRing<MIB, BITS>::LQ : MmaRing<2, BITS>::LQ;
  RING_ARRAYS(LQ);
  __shared__ int xe_s[16 * MIB];
  const int NB = (A.N + NF - 1) / NF;
  const int nbig = *A.n_tiles * NB, nsmall = *A.n_tiles2 * NB;
  const int b = blockIdx.x;
  if (b < nbig) {
    const int bid = xcd_remap(b, nbig);
    const int32_t* t = A.tiles + 3 * (bid / NB);
    tile_rows<BITS, GS, GLU, MIB>(A, L0, L1, L2, L3, xe_s, t[0], t[0] + t[2], t[1], (bid % NB) * NF);
  } else if (b < nbig + nsmall) {
    const int bid = b - nbig;
    const int32_t* t = A.tiles2 + 3 * (bid / NB);
    tile_body<BITS, GS, GLU, 2>(A, L0, L1, L2, L3, xe_s, t[0], t[0] + t[2], t[1], (bid % NB) * NF);
  }
}

// One activation row before the gate/up pass (256 threads, tid 0..255, per
// row): its exponent xexp[t] (the row's largest |x| lands in [2^13, 2^14)
// when scaled by 2^-xexp), the fp16 copy x16[t] = x[t] * 2^-xexp[t] in the
// dequantizer's element order (4-bit: x0 x2 x4 x6 x1 x3 x5 x7 per 8), and,
// given the shared expert's one-row sigmoid gate gw, its logit
// z[t] = bf16(x[t] . dequant(w)^T) with fp32 dequant and accumulation (MTPLX
// PR 558 Summary: the gated shared expert).  red holds 8 floats; every thread
// of the block calls this (it synchronises the block once).
template <int BITS, int GS>
MOEGQ_DEV void prep_row(const uint16_t* __restrict__ x, int64_t T, int H, uint16_t* __restrict__ x16,
                        int32_t* __restrict__ xexp, const uint32_t* __restrict__ gw,
                        const uint16_t* __restrict__ gs_, const uint16_t* __restrict__ gb,
                        uint16_t* __restrict__ z, int64_t t, int tid, float* red) {
  float part = 0.f, mx = 0.f;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (t < T ? t : 0) * (int64_t)H);
  if (t < T) {
    for (int c = tid; c < H / 8; c += 256) {
      const uint4 v = xr[c];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(d[i])), fabsf(bf16_hi(d[i]))));
      if (gw) {
        const int k0 = 8 * c;
        const float s = bf16_to_f32(gs_[k0 / GS]), b = bf16_to_f32(gb[k0 / GS]);
        uint32_t w0 = gw[k0 * BITS / 32], w1 = BITS == 8 ? gw[k0 * BITS / 32 + 1] : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t q = BITS == 4 ? (w0 >> (4 * j)) & 0xFu : ((j < 4 ? w0 : w1) >> (8 * (j & 3))) & 0xFFu;
          const float xv = (j & 1) ? bf16_hi(d[j >> 1]) : bf16_lo(d[j >> 1]);
          part = fmaf(xv, fmaf((float)q, s, b), part);
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    part += __shfl_xor(part, m, 64);
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if ((tid & 63) == 0) {
    red[tid >> 6] = part;
    red[4 + (tid >> 6)] = mx;
  }
  __syncthreads();
  if (t >= T) return;
  const int ex = f16_exponent(fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
  if (tid == 0) {
    xexp[t] = ex;
    if (gw) z[t] = f32_to_bf16(red[0] + red[1] + red[2] + red[3]);
  }
  uint4* xo = reinterpret_cast<uint4*>(x16 + t * (int64_t)H);
  for (int c = tid; c < H / 8; c += 256) xo[c] = act_f16_ldexp<BITS>(xr[c], -ex);
}

template <int BITS, int GS>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ x, int64_t T, int H,
                                                   uint16_t* __restrict__ x16, int32_t* __restrict__ xexp,
                                                   const uint32_t* __restrict__ gw, const uint16_t* __restrict__ gs_,
                                                   const uint16_t* __restrict__ gb, uint16_t* __restrict__ z) {
  __shared__ float red[8];
  prep_row<BITS, GS>(x, T, H, x16, xexp, gw, gs_, gb, z, blockIdx.x, threadIdx.x, red);
}

// The front of a prefill layer in one launch (at most SORT_ONE_MAX_P pairs):
// block 0 sorts the pairs and writes the tile tables, blocks 1 .. prepare four
// activation rows each.  The two parts touch disjoint memory.
template <int BITS, int GS>
__global__ __launch_bounds__(SORT_THREADS) void front_kernel(SortArgs S, const uint16_t* __restrict__ x, int64_t T,
                                                             int H, uint16_t* __restrict__ x16,
                                                             int32_t* __restrict__ xexp,
                                                             const uint32_t* __restrict__ gw,
                                                             const uint16_t* __restrict__ gs_,
                                                             const uint16_t* __restrict__ gb, uint16_t* __restrict__ z) {
  __shared__ float red[32];
  if (blockIdx.x == 0) {
    sort_one_block(S);
    return;
  }
  const int sub = threadIdx.x >> 8;
  prep_row<BITS, GS>(x, T, H, x16, xexp, gw, gs_, gb, z, (int64_t)(blockIdx.x - 1) * 4 + sub, threadIdx.x & 255,
                     red + 8 * sub);
}

// Above SORT_ONE_MAX_P pairs: blocks 0 .. nb - 1 count the block sort's
// blocks of pairs, blocks nb .. prepare four activation rows each.
template <int BITS, int GS>
__global__ __launch_bounds__(SORT_THREADS) void count_prep_kernel(SortArgs S, int64_t nb, const uint16_t* __restrict__ x,
                                                                  int64_t T, int H, uint16_t* __restrict__ x16,
                                                                  int32_t* __restrict__ xexp,
                                                                  const uint32_t* __restrict__ gw,
                                                                  const uint16_t* __restrict__ gs_,
                                                                  const uint16_t* __restrict__ gb,
                                                                  uint16_t* __restrict__ z) {
  __shared__ float red[32];
  if ((int64_t)blockIdx.x < nb) {
    sort_count_block(S.idx, S.P, S.E, S.block_counts, blockIdx.x);
    return;
  }
  const int sub = threadIdx.x >> 8;
  prep_row<BITS, GS>(x, T, H, x16, xexp, gw, gs_, gb, z, ((int64_t)blockIdx.x - nb) * 4 + sub, threadIdx.x & 255,
                     red + 8 * sub);
}

template <int BITS, int GS, bool GLU, int MI>
static hipError_t launch_mma_t(const TileArgs& a, hipStream_t st) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  const int64_t NB = (a.N + NF - 1) / NF;
  const int64_t nblk = a.grid_tiles * NB;
  if (nblk <= 0) return hipSuccess;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tile_mma_kernel<BITS, GS, GLU, MI>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS, int GS, int MI>
static hipError_t launch_mma_m(const TileArgs& a, bool glu, hipStream_t st) {
  return glu ? launch_mma_t<BITS, GS, true, MI>(a, st) : launch_mma_t<BITS, GS, false, MI>(a, st);
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_dual_t(const TileArgs& a, hipStream_t st) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  const int64_t NB = (a.N + NF - 1) / NF;
  const int64_t nblk = (a.grid_tiles + a.grid_tiles2) * NB;
  if (nblk <= 0) return hipSuccess;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tile_mma_dual_kernel<BITS, GS, GLU>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tiles_mma_dual(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st) {
#define MOEGQ_TD(B, G) \
  if (bits == B && gs == G) return glu ? launch_dual_t<B, G, true>(a, st) : launch_dual_t<B, G, false>(a, st);
  MOEGQ_TD(4, 32) MOEGQ_TD(4, 64) MOEGQ_TD(4, 128) MOEGQ_TD(8, 32) MOEGQ_TD(8, 64) MOEGQ_TD(8, 128)
#undef MOEGQ_TD
  return hipErrorInvalidValue;
}

// bf16 expert matrices (gather_mm): 64-row tiles (rows 64), 32-row tiles, or both tables (rows 0)
hipError_t launch_tiles_mma_w16(const TileArgs& a, bool glu, int rows, hipStream_t st) {
  if (rows == 64) return glu ? launch_mma_t<16, 64, true, 4>(a, st) : launch_mma_t<16, 64, false, 4>(a, st);
  if (rows == 32) return glu ? launch_mma_t<16, 64, true, 2>(a, st) : launch_mma_t<16, 64, false, 2>(a, st);
  if (rows == 0) return glu ? launch_dual_t<16, 64, true>(a, st) : launch_dual_t<16, 64, false>(a, st);
  return hipErrorInvalidValue;
}

bool tiles_mma_supported(int64_t K, int64_t N, int64_t src_rows, int gs) {
  return K % TM_K == 0 && K % (8 * gs) == 0 && N > 0 && src_rows * K * 2 < ((int64_t)1 << 32) &&
         N * K < ((int64_t)1 << 31);
}

hipError_t launch_tiles_mma(const TileArgs& a, int bits, int gs, bool glu, int rows, hipStream_t st) {
#define MOEGQ_TM(B, G)                                              \
  if (bits == B && gs == G) {                                       \
    if (rows == 128) return launch_mma_m<B, G, 8>(a, glu, st);      \
    if (rows == 32) return launch_mma_m<B, G, 2>(a, glu, st);       \
    return hipErrorInvalidValue;                                    \
  }
  MOEGQ_TM(4, 32) MOEGQ_TM(4, 64) MOEGQ_TM(4, 128) MOEGQ_TM(8, 32) MOEGQ_TM(8, 64) MOEGQ_TM(8, 128)
#undef MOEGQ_TM
  return hipErrorInvalidValue;
}

hipError_t launch_prep(const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16, int32_t* xexp,
                       const uint32_t* gw, const uint16_t* gsc, const uint16_t* gbi, uint16_t* z, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T >= ((int64_t)1 << 31) || H % 8 != 0) return hipErrorInvalidValue;
#define MOEGQ_PREP(B, G)                                                                                           \
  if (bits == B && gs == G) {                                                                                      \
    hipLaunchKernelGGL((prep_kernel<B, G>), dim3((unsigned)T), dim3(256), 0, st, x, T, H, x16, xexp, gw, gsc, gbi, z); \
    return hipGetLastError();                                                                                      \
  }
  MOEGQ_PREP(4, 32) MOEGQ_PREP(4, 64) MOEGQ_PREP(4, 128) MOEGQ_PREP(8, 32) MOEGQ_PREP(8, 64) MOEGQ_PREP(8, 128)
#undef MOEGQ_PREP
  return hipErrorInvalidValue;
}

hipError_t launch_front(const SortArgs& sa, const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16,
                        int32_t* xexp, const uint32_t* gw, const uint16_t* gsc, const uint16_t* gbi, uint16_t* z,
                        hipStream_t st) {
  if (T >= ((int64_t)1 << 30) || H % 8 != 0) return hipErrorInvalidValue;
  const bool one = sa.P <= SORT_ONE_MAX_P;
  if (sa.E <= 0 || sa.E > SORT_MAXE || (!one && !sa.block_counts)) return hipErrorInvalidValue;
  const int64_t nb = one ? 1 : sort_blocks(sa.P);
  const unsigned grid = (unsigned)(nb + (T + 3) / 4);
#define MOEGQ_FRONT(B, G)                                                                                      \
  if (bits == B && gs == G) {                                                                                  \
    if (one)                                                                                                   \
      hipLaunchKernelGGL((front_kernel<B, G>), dim3(grid), dim3(SORT_THREADS), 0, st, sa, x, T, H, x16, xexp,   \
                         gw, gsc, gbi, z);                                                                     \
    else                                                                                                       \
      hipLaunchKernelGGL((count_prep_kernel<B, G>), dim3(grid), dim3(SORT_THREADS), 0, st, sa, nb, x, T, H, x16, \
                         xexp, gw, gsc, gbi, z);                                                               \
    const hipError_t e = hipGetLastError();                                                                    \
    if (e != hipSuccess || one) return e;                                                                      \
    return launch_sort_rest(sa, st);                                                                           \
  }
  MOEGQ_FRONT(4, 32) MOEGQ_FRONT(4, 64) MOEGQ_FRONT(4, 128) MOEGQ_FRONT(8, 32) MOEGQ_FRONT(8, 64) MOEGQ_FRONT(8, 128)
#undef MOEGQ_FRONT
  return hipErrorInvalidValue;
}

}  // namespace moegq

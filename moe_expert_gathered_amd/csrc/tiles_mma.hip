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
// gfx950 mapping (v_mfma_f32_16x16x32_f16, fp32 accumulation):
//  * 4 waves; each wave owns all 16 * MI rows and 64 MFMA columns (MI x 4
//    blocks; 128 fp32 accumulators at MI = 8).  A column's codes are read by exactly one wave,
//    so each code is dequantized once per tile, in registers, in the layout
//    the MFMA B operand wants: lane (g = lane / 16, c = lane % 16) holds for
//    column c the 32 consecutive k of lane group g (k0 + 32 g ..), which it
//    loads as one (4-bit) or two (8-bit) 128-bit buffer loads.  Inside a K
//    step of 128, MFMA sub-step s contracts k0 + 32 g + 8 s + (0..7) in lane
//    group g; both operands use that same assignment, so the sum is the full
//    dot product over K.
//  * The activation rows are fp16 (converted once, before the tile pass) in
//    the element order the dequantizer produces inside each 8-element chunk
//    (4-bit: q0 q2 q4 q6 q1 q3 q5 q7; 8-bit: natural).  They travel from HBM
//    to LDS with buffer loads that write LDS directly (no register staging),
//    into a double buffer (2 x 4 KiB per 16 rows), each row's 16-byte chunks
//    permuted (lds_swz) so that operand reads are free of bank conflicts.
//  * GLU: a wave's 4 column blocks are (gate f, up f, gate f+16, up f+16), so
//    silu(g) * u is applied in registers in the epilogue.
//  * The weights are the MFMA's first operand: each lane ends with four
//    consecutive output features of one row and writes them as one 8-byte
//    store.
//  * One barrier per K step: the next step's activations and codes are in
//    flight during the current step's MFMAs.
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

// eight codes (one 4-bit word, or two 8-bit words) -> one fp16 MFMA operand
template <int BITS>
MOEGQ_DEV f16x8_t deq_operand(uint32_t w0, uint32_t w1, f16x2_t s2, f16x2_t b2) {
  uint32_t o[4];
  if (BITS == 4) {
    deq4_f16(w0, s2, b2, o);
  } else {
    deq8_f16(w0, s2, b2, o);
    deq8_f16(w1, s2, b2, o + 2);
  }
  return __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// One tile: rows r0 .. r1 - 1 of expert e, MFMA columns n0 .. n0 + 255.  lds
// holds the activation ring: RA stages of 16 * MI rows x TM_K fp16.
template <int MI, int BITS = 4> struct MmaRing {
  // K steps of activation (LDS) and code (register) prefetch: one for 128-row
  // tiles and for bf16 weights (register-bound), three for the shorter tiles
  static constexpr int PDA = (MI >= 8 || BITS == 16) ? 1 : 3;
  static constexpr int PDB = PDA;
  static constexpr int RA = PDA + 1, RB = PDB + 1;              // LDS and register ring stages
  static constexpr int U = (RA % RB == 0) ? RA : (RB % RA == 0) ? RB : RA * RB;   // steps per unrolled loop
  static constexpr int HALFS = RA * 16 * MI * TM_K;
};

// BITS = 16: the expert matrices are plain bf16 (no scales or biases); their
// words go to v_mfma_f32_16x16x32_bf16 as loaded, with the bf16 activations
// in natural order.
template <int BITS, int GS, bool GLU, bool OUT16, int MI>
MOEGQ_DEV void tile_body(const TileArgs& A, uint16_t* lds, int r0, int r1, int e, int n0) {
  constexpr bool W16 = BITS == 16;
  constexpr int CB = 4 * BITS;                    // code bytes per lane per K step (32 codes)
  using Ring = MmaRing<MI, BITS>;
  constexpr int PDA = Ring::PDA, PDB = Ring::PDB, RA = Ring::RA, RB = Ring::RB, U = Ring::U;
  constexpr int STAGE = 16 * MI * TM_K;           // halfs per ring stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int N = A.N, K = A.K;
  const int Kw = K * BITS / 32, G = K / GS;
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  e = __builtin_amdgcn_readfirstlane(e);

  // ---- activation loads: wave w, load v covers rows 4 (MI w + v) .. + 3; lane
  //      (g, c16) fetches chunk c16 ^ (row % 16) of row 4 (MI w + v) + g
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
    rr[v] = min(r0 + 4 * (MI * wave + v) + g, r1 - 1);   // rows past the tile repeat a valid row (never stored)
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
    const int chunk = c16 ^ lds_swz(4 * (MI * wave + v) + g);
    a_off[v] = (uint32_t)src * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
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
  // MFMA column n of block j is output feature block_base(j) + col_perm(n).
  // The MFMA runs with the weights as the first operand, so lane (g, c16) ends
  // up with outputs n = 4 g .. 4 g + 3 of activation row c16; col_perm makes
  // those four land next to each other in memory (one 8-byte store): the
  // identity, except for the fp16 intermediate of 4-bit codes, whose chunk
  // order (q0 q2 q4 q6 q1 q3 q5 q7) is undone by taking features 0 2 4 6 1 3 5 7.
  auto block_base = [&](int j) { return GLU ? n0 + 32 * wave + 16 * (j >> 1) : n0 + 64 * wave + 16 * j; };
  auto col_perm = [](int n) { return (OUT16 && BITS == 4) ? 8 * (n >> 3) + 2 * (n & 3) + ((n >> 2) & 1) : n; };
  uint32_t w_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = block_base(j) + col_perm(c16);
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
  const int lcol = block_base(lj) + col_perm(c16);
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
      uint16_t* dst = lds + sa * STAGE + 4 * (MI * wave + v) * TM_K;
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
    // step ks's activation rows were issued PDA steps ago; at least the PDA - 1 later steps'
    // loads were issued after them (the compiler may reorder loads inside a sub-step, never
    // across the sub-step barriers; extra window loads only lengthen the wait)
    constexpr int VM = (PDA - 1) * LPS;
    static_assert(VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (VM & 15) | ((VM >> 4) << 14));
    __syncthreads();                      // every wave's rows landed; the stage of step ks - 1 is free
    f16x2_t s2[4], b2[4];
    if constexpr (!W16) {
      if (ks % WSTEPS == 0) {
        win_s = nwin_s; win_b = nwin_b;
        if ((ks + WSTEPS) < nK) load_win(ks / WSTEPS + 1, nwin_s, nwin_b);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s2[j] = f16_splat(pick(win_s, ks, j));
        b2[j] = f16_splat(pick(win_b, ks, j));
      }
    }
    const uint16_t* base = lds + sa * STAGE + c16 * TM_K;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      issue_a(ks + PDA, fa, s);           // a quarter of later steps' loads per sub-step
      issue_b(ks + PDB, fb, s);
      f16x8_t bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t* wv = &cw[sb][j][0].x;
        if constexpr (W16) bq[j] = __builtin_bit_cast(f16x8_t, cw[sb][j][s]);   // k 32 g + 8 s .. + 7
        else if constexpr (BITS == 4) bq[j] = deq_operand<4>(wv[s], 0, s2[j], b2[j]);
        else bq[j] = deq_operand<8>(wv[2 * s], wv[2 * s + 1], s2[j], b2[j]);
      }
      const int slot = (4 * g + s) ^ lds_swz(c16);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(base + i * 16 * TM_K + slot * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (W16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bq[j]),
                                                                __builtin_bit_cast(bf16x8_t, a), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bq[j], a, acc[i][j], 0, 0, 0);
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

  // epilogue: acc[i][j][q] = output (row 16 i + c16, memory column block_base(j) + 4 g + q)
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = r0 + 16 * i + c16;
    if (r >= r1) continue;
    uint16_t* orow = A.out + (size_t)r * N;
#pragma unroll
    for (int j = 0; j < (GLU ? 2 : 4); ++j) {
      const int f = (GLU ? block_base(2 * j) : block_base(j)) + 4 * g;
      uint16_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GLU) {
          const float hv = round_bf16(glu(acc[i][2 * j][q], acc[i][2 * j + 1][q]));
          o[q] = OUT16 ? __builtin_bit_cast(uint16_t, (_Float16)hv) : f32_to_bf16(hv);
        } else {
          o[q] = f32_to_bf16(acc[i][j][q]);
        }
      }
      if (vec && f + 3 < N) {
        *reinterpret_cast<uint2*>(orow + f) = make_uint2(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (f + q < N) orow[f + q] = o[q];
      }
    }
  }
}

// XCD-contiguous ranges: the hardware deals workgroups to the 8 XCDs round
// robin; block b of a range of `total` goes to XCD b % 8, so logical id
// (b % 8) * q + b / 8 keeps neighbours (column blocks of one tile, tiles of
// one expert) on one XCD's L2.  The last total % 8 blocks keep their index.
MOEGQ_DEV int xcd_remap(int b, int total) {
  const int q = total / 8;
  return b < 8 * q ? (b % 8) * q + b / 8 : b;
}

// register budget: 2 workgroups per CU (128 accumulators per lane at MI = 8;
// the 32-row variant needs far fewer registers)
template <int BITS, int GS, bool GLU, bool OUT16, int MI>
__global__ __launch_bounds__(256, 2) void tile_mma_kernel(TileArgs A) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;      // output features per tile
  __shared__ __attribute__((aligned(16))) uint16_t As[MmaRing<MI, BITS>::HALFS];
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
  tile_body<BITS, GS, GLU, OUT16, MI>(A, As, r0, r1, e, n0);
}

// Both tile tables in one launch: blocks [0, n_big * NB) take the 128-row
// (bf16 weights: 64-row) tiles of `tiles`, the next n_small * NB blocks the
// 32-row tiles of `tiles2`.
// The few-row tiles stream their experts' weights from HBM while the last
// round of 128-row tiles keeps only part of the machine busy.
template <int BITS, int GS, bool GLU, bool OUT16>
__global__ __launch_bounds__(256, 2) void tile_mma_dual_kernel(TileArgs A) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  constexpr int MIB = BITS == 16 ? 4 : 8;   // bf16 weights: 64-row big tiles (register budget)
  constexpr int HALFS = MmaRing<MIB, BITS>::HALFS > MmaRing<2, BITS>::HALFS ? MmaRing<MIB, BITS>::HALFS
                                                                           : MmaRing<2, BITS>::HALFS;
  __shared__ __attribute__((aligned(16))) uint16_t As[HALFS];
  const int NB = (A.N + NF - 1) / NF;
  const int nbig = *A.n_tiles * NB, nsmall = *A.n_tiles2 * NB;
  const int b = blockIdx.x;
  if (b < nbig) {
    const int bid = xcd_remap(b, nbig);
    const int32_t* t = A.tiles + 3 * (bid / NB);
    tile_body<BITS, GS, GLU, OUT16, MIB>(A, As, t[0], t[0] + t[2], t[1], (bid % NB) * NF);
  } else if (b < nbig + nsmall) {
    const int bid = b - nbig;
    const int32_t* t = A.tiles2 + 3 * (bid / NB);
    tile_body<BITS, GS, GLU, OUT16, 2>(A, As, t[0], t[0] + t[2], t[1], (bid % NB) * NF);
  }
}

// One pass over the activation rows before the tile passes: bf16 -> fp16 in
// the dequantizer's element order (8-element chunks), and, given the shared
// expert's one-row sigmoid gate, its logit z[t] = bf16(x[t] . dequant(w)^T)
// (fp32 dequant and accumulation; MTPLX PR 558 Summary: the gated shared
// expert).  256 threads per row (tid 0..255); red holds 4 floats; every
// thread of the block calls this.
template <int BITS, int GS>
MOEGQ_DEV void prep_row(const uint16_t* __restrict__ x, int64_t T, int H, uint16_t* __restrict__ x16,
                        const uint32_t* __restrict__ gw, const uint16_t* __restrict__ gs_,
                        const uint16_t* __restrict__ gb, uint16_t* __restrict__ z, int64_t t, int tid, float* red) {
  float part = 0.f;
  if (t < T) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * (int64_t)H);
    uint4* xo = reinterpret_cast<uint4*>(x16 + t * (int64_t)H);
    for (int c = tid; c < H / 8; c += 256) {
      const uint4 v = xr[c];
      xo[c] = act_f16<BITS>(v);
      if (gw) {
        const int k0 = 8 * c;
        const float s = bf16_to_f32(gs_[k0 / GS]), b = bf16_to_f32(gb[k0 / GS]);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
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
  if (!gw) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  if (tid == 0 && t < T) z[t] = f32_to_bf16(red[0] + red[1] + red[2] + red[3]);
}

template <int BITS, int GS>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ x, int64_t T, int H,
                                                   uint16_t* __restrict__ x16, const uint32_t* __restrict__ gw,
                                                   const uint16_t* __restrict__ gs_, const uint16_t* __restrict__ gb,
                                                   uint16_t* __restrict__ z) {
  __shared__ float red[4];
  prep_row<BITS, GS>(x, T, H, x16, gw, gs_, gb, z, blockIdx.x, threadIdx.x, red);
}

// The front of a prefill layer in one launch (at most SORT_ONE_MAX_P pairs):
// block 0 sorts the pairs and writes the tile tables, blocks 1 .. prepare four
// activation rows each.  The two parts touch disjoint memory.
template <int BITS, int GS>
__global__ __launch_bounds__(SORT_THREADS) void front_kernel(SortArgs S, const uint16_t* __restrict__ x, int64_t T,
                                                             int H, uint16_t* __restrict__ x16,
                                                             const uint32_t* __restrict__ gw,
                                                             const uint16_t* __restrict__ gs_,
                                                             const uint16_t* __restrict__ gb, uint16_t* __restrict__ z) {
  __shared__ float red[16];
  if (blockIdx.x == 0) {
    sort_one_block(S);
    return;
  }
  const int sub = threadIdx.x >> 8;
  prep_row<BITS, GS>(x, T, H, x16, gw, gs_, gb, z, (int64_t)(blockIdx.x - 1) * 4 + sub, threadIdx.x & 255,
                     red + 4 * sub);
}

// Above SORT_ONE_MAX_P pairs: blocks 0 .. nb - 1 count the block sort's
// blocks of pairs, blocks nb .. prepare four activation rows each.
template <int BITS, int GS>
__global__ __launch_bounds__(SORT_THREADS) void count_prep_kernel(SortArgs S, int64_t nb, const uint16_t* __restrict__ x,
                                                                  int64_t T, int H, uint16_t* __restrict__ x16,
                                                                  const uint32_t* __restrict__ gw,
                                                                  const uint16_t* __restrict__ gs_,
                                                                  const uint16_t* __restrict__ gb,
                                                                  uint16_t* __restrict__ z) {
  __shared__ float red[16];
  if ((int64_t)blockIdx.x < nb) {
    sort_count_block(S.idx, S.P, S.E, S.block_counts, blockIdx.x);
    return;
  }
  const int sub = threadIdx.x >> 8;
  prep_row<BITS, GS>(x, T, H, x16, gw, gs_, gb, z, ((int64_t)blockIdx.x - nb) * 4 + sub, threadIdx.x & 255,
                     red + 4 * sub);
}

template <int BITS, int GS, bool GLU, bool OUT16, int MI>
static hipError_t launch_mma_t(const TileArgs& a, hipStream_t st) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  const int64_t NB = (a.N + NF - 1) / NF;
  const int64_t nblk = a.grid_tiles * NB;
  if (nblk <= 0) return hipSuccess;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tile_mma_kernel<BITS, GS, GLU, OUT16, MI>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS, int GS, int MI>
static hipError_t launch_mma_m(const TileArgs& a, bool glu, bool out16, hipStream_t st) {
  if (glu) return out16 ? launch_mma_t<BITS, GS, true, true, MI>(a, st) : launch_mma_t<BITS, GS, true, false, MI>(a, st);
  return launch_mma_t<BITS, GS, false, false, MI>(a, st);
}

template <int BITS, int GS, bool GLU, bool OUT16>
static hipError_t launch_dual_t(const TileArgs& a, hipStream_t st) {
  constexpr int NF = GLU ? TM_C / 2 : TM_C;
  const int64_t NB = (a.N + NF - 1) / NF;
  const int64_t nblk = (a.grid_tiles + a.grid_tiles2) * NB;
  if (nblk <= 0) return hipSuccess;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tile_mma_dual_kernel<BITS, GS, GLU, OUT16>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tiles_mma_dual(const TileArgs& a, int bits, int gs, bool glu, bool out16, hipStream_t st) {
#define MOEGQ_TD(B, G)                                                                              \
  if (bits == B && gs == G) {                                                                       \
    if (glu) return out16 ? launch_dual_t<B, G, true, true>(a, st) : launch_dual_t<B, G, true, false>(a, st); \
    return launch_dual_t<B, G, false, false>(a, st);                                                \
  }
  MOEGQ_TD(4, 32) MOEGQ_TD(4, 64) MOEGQ_TD(4, 128) MOEGQ_TD(8, 32) MOEGQ_TD(8, 64) MOEGQ_TD(8, 128)
#undef MOEGQ_TD
  return hipErrorInvalidValue;
}

// bf16 expert matrices (gather_mm): 64-row tiles (rows 64), 32-row tiles, or both tables (rows 0)
hipError_t launch_tiles_mma_w16(const TileArgs& a, bool glu, int rows, hipStream_t st) {
  if (rows == 64) return glu ? launch_mma_t<16, 64, true, false, 4>(a, st) : launch_mma_t<16, 64, false, false, 4>(a, st);
  if (rows == 32) return glu ? launch_mma_t<16, 64, true, false, 2>(a, st) : launch_mma_t<16, 64, false, false, 2>(a, st);
  if (rows == 0) return glu ? launch_dual_t<16, 64, true, false>(a, st) : launch_dual_t<16, 64, false, false>(a, st);
  return hipErrorInvalidValue;
}

bool tiles_mma_supported(int64_t K, int64_t N, int64_t src_rows, int gs) {
  return K % TM_K == 0 && K % (8 * gs) == 0 && N > 0 && src_rows * K * 2 < ((int64_t)1 << 32) &&
         N * K < ((int64_t)1 << 31);
}

hipError_t launch_tiles_mma(const TileArgs& a, int bits, int gs, bool glu, bool out16, int rows,
                            hipStream_t st) {
#define MOEGQ_TM(B, G)                                                                              \
  if (bits == B && gs == G) {                                                                       \
    if (rows == 128) return launch_mma_m<B, G, 8>(a, glu, out16, st);                               \
    if (rows == 32) return launch_mma_m<B, G, 2>(a, glu, out16, st);                                \
    return hipErrorInvalidValue;                                                                    \
  }
  MOEGQ_TM(4, 32) MOEGQ_TM(4, 64) MOEGQ_TM(4, 128) MOEGQ_TM(8, 32) MOEGQ_TM(8, 64) MOEGQ_TM(8, 128)
#undef MOEGQ_TM
  return hipErrorInvalidValue;
}

hipError_t launch_prep(const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16, const uint32_t* gw,
                       const uint16_t* gsc, const uint16_t* gbi, uint16_t* z, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T >= ((int64_t)1 << 31) || H % 8 != 0) return hipErrorInvalidValue;
#define MOEGQ_PREP(B, G)                                                                                     \
  if (bits == B && gs == G) {                                                                                \
    hipLaunchKernelGGL((prep_kernel<B, G>), dim3((unsigned)T), dim3(256), 0, st, x, T, H, x16, gw, gsc, gbi, z); \
    return hipGetLastError();                                                                                \
  }
  MOEGQ_PREP(4, 32) MOEGQ_PREP(4, 64) MOEGQ_PREP(4, 128) MOEGQ_PREP(8, 32) MOEGQ_PREP(8, 64) MOEGQ_PREP(8, 128)
#undef MOEGQ_PREP
  return hipErrorInvalidValue;
}

hipError_t launch_front(const SortArgs& sa, const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16,
                        const uint32_t* gw, const uint16_t* gsc, const uint16_t* gbi, uint16_t* z, hipStream_t st) {
  if (T <= 0 || sa.E <= 0 || sa.E > SORT_MAXE || (!sa.block_counts && sa.P > SORT_ONE_MAX_P)) {
    const hipError_t e = launch_sort(sa, st);
    if (e != hipSuccess) return e;
    return launch_prep(x, T, H, bits, gs, x16, gw, gsc, gbi, z, st);
  }
  if (H % 8 != 0 || T >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
  const bool one = sa.P <= SORT_ONE_MAX_P;
  const int64_t nb = one ? 1 : sort_blocks(sa.P);
  const unsigned grid = (unsigned)(nb + (T + 3) / 4);
#define MOEGQ_FRONT(B, G)                                                                                      \
  if (bits == B && gs == G) {                                                                                  \
    if (one)                                                                                                   \
      hipLaunchKernelGGL((front_kernel<B, G>), dim3(grid), dim3(SORT_THREADS), 0, st, sa, x, T, H, x16, gw, gsc, \
                         gbi, z);                                                                              \
    else                                                                                                       \
      hipLaunchKernelGGL((count_prep_kernel<B, G>), dim3(grid), dim3(SORT_THREADS), 0, st, sa, nb, x, T, H, x16, \
                         gw, gsc, gbi, z);                                                                     \
    const hipError_t e = hipGetLastError();                                                                    \
    if (e != hipSuccess || one) return e;                                                                      \
    return launch_sort_rest(sa, st);                                                                           \
  }
  MOEGQ_FRONT(4, 32) MOEGQ_FRONT(4, 64) MOEGQ_FRONT(4, 128) MOEGQ_FRONT(8, 32) MOEGQ_FRONT(8, 64) MOEGQ_FRONT(8, 128)
#undef MOEGQ_FRONT
  return hipErrorInvalidValue;
}

}  // namespace moegq

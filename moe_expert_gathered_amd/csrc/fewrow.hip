// Few-row quantized products (5..16 activation rows per weight matrix, and
// 2..4 where the matrix-vector kernel does not take the shape) on the bf16
// matrix cores, with the codes entering the MFMA exactly.
//
// MLX PR 4787: at 3-16 rows the weights should feed the matrix units rather
// than a per-row vector loop.  This kernel keeps the weights as codes on the
// matrix cores and applies each group's scale and bias in fp32 afterwards:
//   sum_k x_k (q_k s + b) = s * sum_k x_k q'_k + (b - o s) * sum_k x_k
// over the k of one group, with q' = q + o the code as an exact bf16 value
// (4-bit: 128 + q, built by placing the code under the bf16 exponent of 128,
// o = 128; 8-bit: q itself, o = 0).  One v_mfma_f32_16x16x32_bf16 contracts
// 32 k, always inside one group (group sizes 32, 64, 128); a second MFMA
// against ones gives the rows' sums of x over the same k.  Products of bf16
// values are exact and the sums run in fp32, so the result carries no
// rounding of the weights and the activations enter as stored: no range
// limit beyond fp32's.
//
// Layout: lane (g = lane / 16, r = lane % 16) supplies activation row r and
// weight column r of each 16-column block, k = 32 s + 8 g + (0..7) in MFMA
// step s; it ends with outputs (rows 4 g .. 4 g + 3, column r).  A
// workgroup (W waves: 4 for GLU pairs, 8 for plain products) owns 16 * NB
// columns of one pair and a range of 128-wide K chunks, its waves taking
// interleaved chunks with the loads of the next DEPTH chunks in flight; the
// waves' partial sums meet in LDS.
// Loads are buffer loads (the pair's rows and expert matrices in the
// descriptors, the chunk as a wave-uniform offset), coalesced: neighbouring
// lanes read neighbouring bytes of one row, and each wave passes its chunk
// through a staging area in LDS into the layout above.  With KS > 1 splits
// along K, each workgroup stores its
// fp32 partial and the last one of a column group to finish (counted with one
// atomic per workgroup) adds the KS partials in split order and writes the
// output, so the result does not depend on timing; it leaves its counter at
// zero for the next call.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int FR_CK = 128;     // K per chunk (four MFMA steps)
constexpr int kFewMaxSplit = 8; // splits along K at most

// t[j] of lane group G (lanes 16 G .. 16 G + 15) becomes t[G] of lane group j:
// a 4 x 4 transpose between the lane groups, lane by lane within a group.
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; v_permlane16_swap the odd 16-lane rows of its
// first operand with the even rows of its second.
MOEGQ_DEV void transpose4(uint32_t t[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(t[0], t[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(t[1], t[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  t[0] = c[0];
  t[1] = c[1];
  t[2] = d[0];
  t[3] = d[1];
}

template <int BITS, int GS, bool GLU, int NB, int DEPTH, int W>
__global__ __launch_bounds__(64 * W) void fewrow_kernel(FewArgs A) {
  constexpr int NM = GLU ? 2 : 1;
  constexpr int NGC = FR_CK / GS;                      // groups per chunk
  constexpr int SW = (NGC + 1) / 2;                    // 32-bit words of one chunk's scales
  constexpr float OFS = BITS == 4 ? 128.f : 0.f;       // code offset of the bf16 operand
  constexpr int SPG = GS / 32;                         // MFMA steps per group
  __shared__ f32x4_t red[W - 1][NM][NB][64];
  constexpr int PPR = 4 * (BITS / 4);                  // 16-byte code pieces per row and chunk
  constexpr int XS = 16 * 16, CS = NM * NB * 16 * PPR; // a wave's staging area, in pieces
  __shared__ uint4 few_stage[W * (XS + CS)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int K = A.K, N = A.N, M = A.M;
  const int Kw = K * BITS / 32, G = K / GS;
  const int ncg = (N + 16 * NB - 1) / (16 * NB);
  const int64_t item = blockIdx.x;
  const int64_t p = item / ncg;
  const int n0 = (int)(item % ncg) * 16 * NB;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int nchunk = K / FR_CK;
  const int c_lo = ks * A.cps, c_hi = min(nchunk, c_lo + A.cps);

  const int64_t xb = A.lhs ? (int64_t)A.lhs[p] : p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[p] : 0;
  // Buffer descriptors over this pair's activation rows and expert matrices.
  // Loads are coalesced (neighbouring lanes read neighbouring bytes of one
  // row) and pass through LDS into the MFMA layout, where the 16 lanes of a
  // lane group hold 16 different rows: loaded in that layout directly, every
  // 16-lane pass of every load touched 16 rows, and the loads' address
  // processing, not HBM, set the kernel's time.  Activation rows past M read
  // row M - 1 and columns past N column N - 1: their outputs are never stored.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(A.x + xb * M * (int64_t)K, (uint32_t)(M * K * 2));
  // activations, load i: row 4 i + lane / 16, 16-byte piece lane % 16 of the chunk's 256 bytes
  uint32_t vx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vx[i] = (uint32_t)(min(4 * i + (lane >> 4), M - 1) * K * 2 + 16 * (lane & 15));
  __amdgpu_buffer_rsrc_t rw[NM], rs[NM], rb[NM];
  {
    const uint32_t wbytes = (uint32_t)((int64_t)N * Kw * 4), sbytes = (uint32_t)((int64_t)N * G * 2);
    rw[0] = make_rsrc(A.w0 + e * N * (int64_t)Kw, wbytes);
    rs[0] = make_rsrc(A.s0 + e * N * (int64_t)G, sbytes);
    rb[0] = make_rsrc(A.b0 + e * N * (int64_t)G, sbytes);
    if (GLU) {
      rw[NM - 1] = make_rsrc(A.w1 + e * N * (int64_t)Kw, wbytes);
      rs[NM - 1] = make_rsrc(A.s1 + e * N * (int64_t)G, sbytes);
      rb[NM - 1] = make_rsrc(A.b1 + e * N * (int64_t)G, sbytes);
    }
  }
  // codes of column block b: row lane / 4, 16-byte piece lane % 4 of the
  // row's chunk (and piece 4 + lane % 4 at 8 bits)
  uint32_t vw[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    vw[b] = (uint32_t)(min(n0 + 16 * b + (lane >> 2), N - 1) * Kw * 4 + 16 * (lane & 3));
  // scales and biases: in scale load i, lane group g takes combination
  // k = 4 i + g of (array, matrix, column block b = k % NB), column
  // n0 + 16 b + r; stage() hands each lane its column's values with
  // ds_bpermute.  Lane groups of one load that read different matrices
  // issue their own buffer loads (the other lanes at an offset past the
  // range: nothing fetched, zeros).
  constexpr int NCOMB = NM * NB * 2, NSI = (NCOMB + 3) / 4;
  static_assert(NB == 1 || NB == 2, "one or two column blocks per workgroup");
  const uint32_t vsb = (uint32_t)(min(n0 + 16 * (g % NB) + r, N - 1) * G * 2);
  // the residual values of the lane's outputs, requested before the K loop
  uint32_t res_in[NB][4] = {};
  if (!GLU && A.residual) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        res_in[b][q] = A.residual[(p * M + min(4 * g + q, M - 1)) * (int64_t)N + min(n0 + 16 * b + r, N - 1)];
  }

  f32x4_t acc[NM][NB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[m][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = 0x3F803F80u;                     // bf16 (1, 1)
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(one2, one2, one2, one2));

  // one chunk's loads, as loaded (coalesced); stage() turns them into the
  // MFMA layout: lane (g, r) then holds activation row r's k in [32 s + 8 g,
  // + 8) for step s, and its column's codes of k in [32 g, 32 g + 32) of the
  // chunk (one 128-bit word at 4 bits, two at 8 bits; a 4 x 4 transpose
  // across the lane groups then gives it the codes of k = 32 s + 8 g + (0..7)
  // for each MFMA step s).
  struct Chunk {
    uint4 xl[4];                          // activations: 4 rows per load
    uint4 cl[NM][NB][BITS / 4];           // codes: 16 rows per load
    uint32_t sl[NSI][SW];                 // scale / bias combinations, two bf16 per word
  };
  struct Operands {
    uint4 xv[4];
    uint4 cw[NM][NB][BITS / 4];
    uint32_t sv[NM][NB][SW], bv[NM][NB][SW];
  };
  // chunk c's loads.  A chunk past the split's end (never computed) loads at
  // a lane offset beyond every descriptor's range, which returns zeros
  // without fetching, rather than being skipped: with no load under a branch the compiler's wait counts
  // stay exact, so computing one chunk waits for that chunk's loads only.
  auto load = [&](int c, Chunk& d) {
    constexpr uint32_t kNoFetch = 0x7FFFFFF0u;
    const bool live = c < c_hi;
    const uint32_t ox = live ? (uint32_t)c * FR_CK * 2 : 0u, ow = live ? (uint32_t)c * FR_CK * BITS / 8 : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) d.xl[i] = buf_load16(rx, live ? vx[i] : kNoFetch, ox);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < BITS / 4; ++h) d.cl[m][b][h] = buf_load16(rw[m], live ? vw[b] + 64 * h : kNoFetch, ow);
    const uint32_t os = live ? (uint32_t)(c * NGC) * 2 : 0u;
#pragma unroll
    for (int i = 0; i < NSI; ++i) {
#pragma unroll
      for (int w = 0; w < SW; ++w) d.sl[i][w] = 0u;
#pragma unroll
      for (int dd = 0; dd < 2 * NM; ++dd) {             // descriptor: array dd / NM, matrix dd % NM
        if (dd * NB > 4 * i + 3 || (dd + 1) * NB <= 4 * i) continue;   // no lane of this load reads it
        const int k = 4 * i + g;
        const __amdgpu_buffer_rsrc_t rd = dd / NM ? rb[dd % NM] : rs[dd % NM];
        const uint32_t vo = (live && k < NCOMB && k / NB == dd) ? vsb : kNoFetch;
        if (NGC == 4) {
          const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rd, vo, os, 0);
          d.sl[i][0] |= v2[0];
          d.sl[i][SW - 1] |= v2[1];
        } else if (NGC == 2) {
          d.sl[i][0] |= __builtin_amdgcn_raw_buffer_load_b32(rd, vo, os, 0);
        } else {
          d.sl[i][0] |= __builtin_amdgcn_raw_buffer_load_b16(rd, vo, os, 0);
        }
      }
    }
  };
  // the wave's staging area: the chunk's activations (16 rows of 16 pieces)
  // then its codes (NM x NB blocks of 16 rows of PPR pieces), 16 bytes a
  // piece, each row's pieces permuted so that both the coalesced writes and
  // the MFMA-layout reads (16 rows at one piece) are free of bank conflicts
  uint4* stg = few_stage + wave * (XS + CS);
  auto csw = [](int row) { return BITS == 4 ? (row >> 2) & 3 : ((row >> 1) & 3) << 1; };
  auto stage = [&](const Chunk& d, Operands& o) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the previous chunk's reads came first
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + (lane >> 4), q = lane & 15;
      stg[row * 16 + (q ^ row)] = d.xl[i];
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < BITS / 4; ++h) {
          const int row = lane >> 2, pc = 4 * h + (lane & 3);
          stg[XS + ((m * NB + b) * 16 + row) * PPR + (pc ^ csw(row))] = d.cl[m][b][h];
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int s = 0; s < 4; ++s) o.xv[s] = stg[r * 16 + ((4 * s + g) ^ r)];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < BITS / 4; ++h) {
          const int pc = BITS == 4 ? g : 2 * g + h;
          o.cw[m][b][h] = stg[XS + ((m * NB + b) * 16 + r) * PPR + (pc ^ csw(r))];
        }
    // scale and bias of the lane's column: combination k sits in load k / 4
    // at lane 16 (k % 4) + r
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int ks = m * NB + b, kb = (NM + m) * NB + b;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
          o.sv[m][b][w] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * (ks % 4) + r) * 4, (int)d.sl[ks / 4][w]);
          o.bv[m][b][w] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * (kb % 4) + r) * 4, (int)d.sl[kb / 4][w]);
        }
      }
  };
  // codes of one step -> the bf16 operand q + OFS, in the order k = 8 g + (0..7)
  auto operand = [&](const uint32_t* w) -> bf16x8_t {
    if (BITS == 4) {
      // nibbles j and j + 4 of the word pair up under 0x43 (bf16 128 + q): the
      // element order is q0 q4 q1 q5 q2 q6 q3 q7, matched on the activation side
      uint32_t pr[4];
      nib_pairs(w[0], pr);
      return __builtin_bit_cast(bf16x8_t, make_uint4(pr[0], pr[1], pr[2], pr[3]));
    } else {
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t v = w[h];
        o[2 * h] = pk_bf16((float)(v & 0xFFu), (float)((v >> 8) & 0xFFu));
        o[2 * h + 1] = pk_bf16((float)((v >> 16) & 0xFFu), (float)(v >> 24));
      }
      return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
    }
  };
  auto compute = [&](const Operands& d) {
    // st[m][b][s]: the lane's codes for step s (one word at 4 bits, two at 8)
    uint32_t st[NM][NB][4][BITS / 4];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (BITS == 4) {
          uint32_t t[4] = {d.cw[m][b][0].x, d.cw[m][b][0].y, d.cw[m][b][0].z, d.cw[m][b][0].w};
          transpose4(t);
#pragma unroll
          for (int s = 0; s < 4; ++s) st[m][b][s][0] = t[s];
        } else {
          // two-word units (8 codes); the lane holds units 4 g .. 4 g + 3
          uint32_t lo[4] = {d.cw[m][b][0].x, d.cw[m][b][0].z, d.cw[m][b][1].x, d.cw[m][b][1].z};
          uint32_t hi[4] = {d.cw[m][b][0].y, d.cw[m][b][0].w, d.cw[m][b][1].y, d.cw[m][b][1].w};
          transpose4(lo);
          transpose4(hi);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            st[m][b][s][0] = lo[s];
            st[m][b][s][BITS / 4 - 1] = hi[s];
          }
        }
      }
    f32x4_t part[NM][NB], xs = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 xa = d.xv[s];
      if (BITS == 4) {                   // x0..x7 -> x0 x4 x1 x5 x2 x6 x3 x7 (the codes' order)
        const uint32_t dd[4] = {xa.x, xa.y, xa.z, xa.w};
        uint32_t o[4];
        perm_pairs(dd, o);
        xa = make_uint4(o[0], o[1], o[2], o[3]);
      }
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa);
      const bool first = s % SPG == 0;
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : xs, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          part[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, operand(st[m][b][s]),
                                                               first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : part[m][b], 0, 0, 0);
      if (s % SPG == SPG - 1) {          // the group ends: scale and bias in fp32
        const int gi = s / SPG;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const uint32_t sw = d.sv[m][b][gi / 2], bw = d.bv[m][b][gi / 2];
            const float sc = gi % 2 ? bf16_hi(sw) : bf16_lo(sw);
            const float cb = __builtin_fmaf(-OFS, sc, gi % 2 ? bf16_hi(bw) : bf16_lo(bw));
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[m][b][q] = __builtin_fmaf(cb, xs[q], __builtin_fmaf(sc, part[m][b][q], acc[m][b][q]));
          }
      }
    }
  };
  // chunk c of the split belongs to wave (c - c_lo) % W; the loads of the
  // wave's next DEPTH chunks are in flight while one is computed (a ring of
  // DEPTH + 1 buffers, unrolled so that every buffer index is static; the
  // scheduling barriers keep each chunk's loads in ring order)
  Chunk buf[DEPTH + 1];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    load(c_lo + wave + W * i, buf[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c = c_lo + wave; c < c_hi; c += W * (DEPTH + 1)) {
#pragma unroll
    for (int i = 0; i <= DEPTH; ++i) {
      load(c + W * (i + DEPTH), buf[(i + DEPTH) % (DEPTH + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      if (c + W * i < c_hi) {
        Operands o;
        stage(buf[i], o);
        compute(o);
      }
    }
  }
  // the waves' partial sums meet in LDS (wave 0 adds them in wave order)
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave - 1][m][b][lane] = acc[m][b];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int w = 0; w < W - 1; ++w) acc[m][b] += red[w][m][b][lane];
  if (KS > 1) {
    // store this split's partial; the last workgroup of the column group adds
    // all splits in order.  The partials travel as device-scope atomic stores
    // and loads (written through to, and read from, the level every XCD
    // shares) and the counter as a device-scope atomic, so no fence has to
    // write back or invalidate an L2: the stores are complete (vmcnt 0)
    // before the counter moves, and the loads issue only after it has.
    float* mine = A.part + ((item * KS + ks) * NM * NB) * 256 + 4 * lane;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __hip_atomic_store(mine + (m * NB + b) * 256 + q, acc[m][b][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int arrived = 0;
    if (lane == 0) arrived = __hip_atomic_fetch_add(A.counters + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readlane(arrived, 0) != KS - 1) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // every split's partial is requested before any is added (KS <= kFewMaxSplit)
    const float* all = A.part + (item * KS * NM * NB) * 256 + 4 * lane;
    float pv[kFewMaxSplit][NM][NB][4];
#pragma unroll
    for (int k2 = 0; k2 < kFewMaxSplit; ++k2)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pv[k2][m][b][q] = k2 < KS ? __hip_atomic_load(all + (k2 * NM * NB + m * NB + b) * 256 + q,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float t = pv[0][m][b][q];
#pragma unroll
          for (int k2 = 1; k2 < kFewMaxSplit; ++k2)
            if (k2 < KS) t += pv[k2][m][b][q];
          acc[m][b][q] = t;
        }
    if (lane == 0) __hip_atomic_store(A.counters + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // out[p, row 4 g + q, column n0 + 16 b + r]
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int col = n0 + 16 * b + r;
    if (col >= N) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 4 * g + q;
      if (row < M) {
        float v = GLU ? glu(acc[0][b][q], acc[NM - 1][b][q]) : acc[0][b][q];
        if (!GLU && A.residual) v = bf16_to_f32(f32_to_bf16(v)) + bf16_to_f32((uint16_t)res_in[b][q]);
        A.out[(p * M + row) * (int64_t)N + col] = f32_to_bf16(v);
      }
    }
  }
}

// Workgroup shape and splits along K.  GLU pairs: 4 waves on one 16-column
// block (twice the workgroups of two blocks: 13.4 against 15.4 us for the
// 16-row 2 x 9728 x 2560 gate/up).  Plain products: 8 waves (K split over
// more waves of one workgroup, summed in LDS; one such workgroup per CU is
// resident) on one block while the blocks fit one workgroup per CU and no
// wave would stream more than kFewMaxWaveChunks chunks, else on two blocks.
// K splits over workgroups only when the column groups leave CUs idle, up to
// about one workgroup per CU while every wave keeps at least kFewMinChunks
// chunks: each split adds the store / count / reload tail to the critical
// path.  Measured on the dense chain's 16-row products (us, against 4 waves
// on two blocks with the split): 2560 x 4096 7.45 (one block, no split)
// against 8.65, 2560 x 9728 10.66 (two blocks, 3 splits) against 11.31,
// 6144 x 2560 8.02 (two blocks, no split) against 8.51.
constexpr int64_t kFewCUs = 256;
constexpr int64_t kFewMinChunks = 2;
constexpr int64_t kFewMaxWaveChunks = 6;

constexpr int few_waves(bool glu) { return glu ? 4 : 8; }

FewPlan fewrow_plan(int64_t P, int64_t N, int64_t K, bool glu, bool split_allowed) {
  FewPlan pl{};
  const int64_t W = few_waves(glu);
  const int64_t nchunk = K / FR_CK;
  const int64_t items1 = P * ((N + 15) / 16);
  if (glu) pl.NB = 1;
  else pl.NB = items1 <= kFewCUs && (nchunk <= W * kFewMaxWaveChunks || !split_allowed) ? 1 : 2;
  const int64_t items = P * ((N + 16 * pl.NB - 1) / (16 * pl.NB));
  int64_t KS = 1;
  if (split_allowed && items < kFewCUs && (glu || pl.NB == 2)) {
    KS = std::max<int64_t>(1, kFewCUs / items);
    KS = std::min<int64_t>({KS, (int64_t)kFewMaxSplit, std::max<int64_t>(1, nchunk / (W * kFewMinChunks))});
  }
  pl.cps = (int)((nchunk + KS - 1) / KS);
  pl.KS = (int)((nchunk + pl.cps - 1) / pl.cps);
  pl.items = items;
  const int NM = glu ? 2 : 1;
  pl.part_bytes = pl.KS > 1 ? (size_t)pl.items * pl.KS * NM * pl.NB * 64 * 16 : 0;
  pl.counter_bytes = pl.KS > 1 ? (size_t)pl.items * 4 : 0;
  return pl;
}

// K a multiple of the chunk; one expert matrix (and the activation rows of a
// pair) addressable with the buffer loads' 32-bit offsets
bool fewrow_supported(int64_t M, int64_t N, int64_t K, int bits) {
  return M >= 1 && M <= 16 && K % FR_CK == 0 && N * K * bits / 8 < ((int64_t)1 << 31) && M * K * 2 < ((int64_t)1 << 31);
}

// prefetch depth: as many chunks ahead as keep two waves per SIMD
template <int BITS, bool GLU>
constexpr int few_depth() { return GLU ? (BITS == 8 ? 1 : 2) : (BITS == 8 ? 2 : 3); }

template <int BITS, int GS, bool GLU>
static hipError_t launch_few_t(const FewArgs& a, int64_t items, int KS, int NB, hipStream_t st) {
  constexpr int D = few_depth<BITS, GLU>(), W = few_waves(GLU);
  const dim3 grid((unsigned)items, (unsigned)KS), block(64 * W);
  if constexpr (GLU) {                       // GLU pairs always take one block
    if (NB != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fewrow_kernel<BITS, GS, GLU, 1, D, W>), grid, block, 0, st, a);
  } else if (NB == 1) {
    hipLaunchKernelGGL((fewrow_kernel<BITS, GS, GLU, 1, D, W>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((fewrow_kernel<BITS, GS, GLU, 2, D, W>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_fewrow(const FewArgs& a, const FewPlan& pl, int bits, int gs, bool glu, hipStream_t st) {
  if (pl.items <= 0) return hipSuccess;
  if (pl.items >= ((int64_t)1 << 31) || pl.KS > 65535 || (pl.NB != 1 && pl.NB != 2)) return hipErrorInvalidValue;
  FewArgs b = a;
  b.cps = pl.cps;
#define MOEGQ_FEW(B, G)                                                                                 \
  if (bits == B && gs == G)                                                                             \
    return glu ? launch_few_t<B, G, true>(b, pl.items, pl.KS, pl.NB, st) : launch_few_t<B, G, false>(b, pl.items, pl.KS, pl.NB, st);
  MOEGQ_FEW(4, 32) MOEGQ_FEW(4, 64) MOEGQ_FEW(4, 128) MOEGQ_FEW(8, 32) MOEGQ_FEW(8, 64) MOEGQ_FEW(8, 128)
#undef MOEGQ_FEW
  return hipErrorInvalidValue;
}

}  // namespace moegq

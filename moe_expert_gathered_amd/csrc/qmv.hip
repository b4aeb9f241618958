// Gathered matrix-vector kernels for decode (one activation row per pair).
//
// For pair p the kernel computes out[p, n] = x[row(p)] . dequant(W[e(p)][n])^T
// (MLX issue 4509, gq(): gather_qmm with rhs_indices over x[M,1,1,H]), and in
// the GLU variant h[p, n] = silu(x . Wg^T) * (x . Wu^T) for the gate and up
// projections of SwitchGLU (same page, moe(): up, gate, silu(gate)*up).
//
// Mapping on gfx950: a workgroup owns one pair and 4 waves x RPW output rows.
// Each wave streams RPW rows (two matrices in the GLU variant) with 128-bit
// coalesced loads: lane l reads words [4l, 4l+4) of every 256-word slice of a
// row, so one load instruction covers 1 KiB of one row.  The activations are
// read straight from global memory (L2-resident: every wave of a pair reads
// the same row) and reordered in registers.
//
// Arithmetic (4-bit): per lane and group g the partial sum of x_k (q_k s + b)
// is s * D + (b - 128 s) * Sx with D = sum x_k (128 + q_k) and Sx = sum x_k,
// the group identity of the affine code (nuvec "composed": codes * s + b).
// D is formed with v_dot2_f32_bf16 on bf16 pairs (128 + q) built by one
// and/or per pair (no per-element conversion).  8-bit codes use
// v_cvt_f32_ubyte{0..3} and fp32 FMAs.  Accumulation is fp32; the wave's
// partial sums are combined with a butterfly that halves the number of live
// values at each step.
#include "common.h"
#include "launch.h"

namespace moegq {

// Sum of one float over the 16 lanes of each row (DPP row rotations).
MOEGQ_DEV float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

// Reduce V per-lane partial sums over the wave.  Two swap steps halve the
// live values without any select: v_permlane32_swap exchanges the upper half
// of one register with the lower half of another, so X + Y afterwards is the
// pairwise total of value i in lanes 0-31 and of value i + V/2 in lanes 32-63
// (v_permlane16_swap does the same between odd and even 16-lane rows).  The
// V/4 values left are then summed inside each 16-lane row.  On return every
// lane of row r = 2*bit5 + bit4 holds a[j] = total of value
// bit5*(V/2) + bit4*(V/4) + j, j < V/4.
template <int V>
MOEGQ_DEV void reduce_wave(float (&a)[V]) {
  static_assert(V >= 4 && (V & (V - 1)) == 0, "V must be a power of two >= 4");
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i]), __float_as_uint(a[i + V / 2]), false, false);
    a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + V / 4]), false, false);
    a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) a[i] = row_sum16(a[i]);
}

// One wave owns RPW output rows (two matrices in the GLU variant) of one
// pair, over the 256-word slices it0, it0 + 1, .. (chunks of NS slices, one
// chunk every `step` slices from `first`).  Every operand is read through a
// raw buffer descriptor (one per matrix of the pair's expert, one for the
// activation row): a lane's offset inside a slice is a single 32-bit VGPR
// shared by all rows, the row offsets are scalars (the range check covers the
// scalar offset too, so rows past N read zero).  Lanes past the end of a row
// load with an offset beyond every descriptor's range, so the hardware
// returns zero without fetching.  Codes are loaded with the non-temporal
// hint: each is read once per launch.  All loads of a chunk (codes, scales,
// biases, activations) are issued before any arithmetic.  acc holds the
// wave's per-lane partial sums (reduce_wave completes them).
// SEL: lanes past the row end also take zero scale and bias through a select.
// Their loads already return zero, so no value changes; the select makes the
// compiler wait for the whole chunk before the first arithmetic, which keeps
// the gate/up and plain kernels at fewer registers and more waves per SIMD
// (measured faster there).  The down+combine kernel runs faster without it:
// its arithmetic then starts as each row's loads land.
// MR > 1: each pair has A.rows (<= MR) activation rows, x rows xrow * rows + r,
// and every code a lane loads is applied to the first MRC of them (rows past
// A.rows repeat the last one and are never stored).  acc then holds value
// (m * MR + r) * RPW + rr for matrix m, activation row r, output row rr; the
// values of rows MRC .. MR - 1 stay zero (MR keeps V a power of two).
template <int BITS, int GS, bool GLU, int RPW, int NS, bool SEL = true, int MR = 1, int MRC = MR,
          int V = RPW * (GLU ? 2 : 1) * MR>
MOEGQ_DEV void qmv_rows(const QmvArgs& A, int64_t p, int n0, int lane, int first, int step, float (&acc)[V]) {
  constexpr int NM = GLU ? 2 : 1;
  constexpr int VC = RPW * NM;            // code rows of the wave
  constexpr int XV = BITS == 4 ? 4 : 2;   // uint4 of activations per lane per slice
  const int K = A.K, N = A.N;
  const int64_t xrow = A.lhs ? (int64_t)A.lhs[p] : (A.lhs_shift >= 0 ? p >> A.lhs_shift : p / A.lhs_div);
  const int64_t e = A.rhs ? (int64_t)A.rhs[p] : 0;
  const int Kw = K * BITS / 32;      // words per row
  const int G = K / GS;              // groups per row

  __amdgpu_buffer_rsrc_t rw[NM], rs[NM], rb[NM];
  rw[0] = make_rsrc(A.w0 + e * N * (int64_t)Kw, (uint32_t)N * Kw * 4);
  rs[0] = make_rsrc(A.s0 + e * N * (int64_t)G, (uint32_t)N * G * 2);
  rb[0] = make_rsrc(A.b0 + e * N * (int64_t)G, (uint32_t)N * G * 2);
  if (GLU) {
    rw[NM - 1] = make_rsrc(A.w1 + e * N * (int64_t)Kw, (uint32_t)N * Kw * 4);
    rs[NM - 1] = make_rsrc(A.s1 + e * N * (int64_t)G, (uint32_t)N * G * 2);
    rb[NM - 1] = make_rsrc(A.b1 + e * N * (int64_t)G, (uint32_t)N * G * 2);
  }
  __amdgpu_buffer_rsrc_t rx[MRC];
  if constexpr (MR == 1) {
    rx[0] = make_rsrc(A.x + xrow * (int64_t)K, (uint32_t)K * 2);
  } else {
    const int64_t nr = A.rows;
#pragma unroll
    for (int r = 0; r < MRC; ++r)
      rx[r] = make_rsrc(A.x + (xrow * nr + min((int64_t)r, nr - 1)) * (int64_t)K, (uint32_t)K * 2);
  }

#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  // 4-bit pair building: bytes of (w & 0x0F0F0F0F) are the even codes, of
  // ((w >> 4) & 0x0F0F0F0F) the odd ones; v_perm places two of them under the
  // bf16 exponent byte 0x43, giving (128 + q_a, 128 + q_b) per dword.
  const uint32_t C43 = 0x43434343u;

  const int n_it = (Kw + 255) / 256;
  constexpr uint32_t kNoFetch = 0x7FFFFFF0u;   // past every descriptor's range
  for (int it0 = first; it0 < n_it; it0 += step) {
    uint4 c[NS][VC], xv[NS][MRC][XV];
    uint16_t sv[NS][VC], bv[NS][VC];
    bool ok[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int wb = (it0 + t) * 256 + lane * 4;     // first word of the lane's 16 bytes
      ok[t] = wb < Kw;                               // lanes past the row end add nothing
      const int k0 = wb * (32 / BITS);
      const uint32_t g2 = (uint32_t)(k0 / GS) * 2;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint32_t row = (uint32_t)(n0 + r);
          c[t][m * RPW + r] = buf_load16_nt(rw[m], ok[t] ? (uint32_t)wb * 4 : kNoFetch, row * Kw * 4);
          sv[t][m * RPW + r] = buf_load2(rs[m], ok[t] ? g2 : kNoFetch, row * G * 2);
          bv[t][m * RPW + r] = buf_load2(rb[m], ok[t] ? g2 : kNoFetch, row * G * 2);
        }
#pragma unroll
      for (int r = 0; r < MRC; ++r)
#pragma unroll
        for (int j = 0; j < XV; ++j) xv[t][r][j] = buf_load16(rx[r], (uint32_t)(k0 + 8 * j) * 2, 0);
    }
    // gate/up: a wave whose loads are all issued takes issue priority, so the
    // waves whose data has landed finish first and hand their slots to waves
    // that have not issued yet (measured faster; not for the down+combine)
    if (GLU) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (BITS == 4 && MR == 1) {
        // activations in the pair order (x0,x2) (x4,x6) (x1,x3) (x5,x7) per 8
        uint32_t xp[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = xv[t][0][j];
          xp[4 * j + 0] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
          xp[4 * j + 1] = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
          xp[4 * j + 2] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
          xp[4 * j + 3] = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
        }
        float sx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sx = fdot2_bf16(xp[i], 0x3F803F80u, sx);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const uint32_t cw[4] = {c[t][i].x, c[t][i].y, c[t][i].z, c[t][i].w};
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = cw[j] & 0x0F0F0F0Fu, hi = (cw[j] >> 4) & 0x0F0F0F0Fu;
            d = fdot2_bf16(__builtin_amdgcn_perm(C43, lo, 0x04010400u), xp[4 * j + 0], d);
            d = fdot2_bf16(__builtin_amdgcn_perm(C43, lo, 0x04030402u), xp[4 * j + 1], d);
            d = fdot2_bf16(__builtin_amdgcn_perm(C43, hi, 0x04010400u), xp[4 * j + 2], d);
            d = fdot2_bf16(__builtin_amdgcn_perm(C43, hi, 0x04030402u), xp[4 * j + 3], d);
          }
          const float s = (!SEL || ok[t]) ? bf16_to_f32(sv[t][i]) : 0.f;
          const float b = (!SEL || ok[t]) ? bf16_to_f32(bv[t][i]) : 0.f;
          acc[i] = fmaf(s, d, fmaf(fmaf(-128.f, s, b), sx, acc[i]));
        }
      } else if (BITS == 4) {
        // several activation rows: each code pair is built once and applied to every row
        uint32_t xp[MRC][16];
        float sx[MRC];
#pragma unroll
        for (int r = 0; r < MRC; ++r) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 v = xv[t][r][j];
            xp[r][4 * j + 0] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
            xp[r][4 * j + 1] = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
            xp[r][4 * j + 2] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
            xp[r][4 * j + 3] = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
          }
          sx[r] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sx[r] = fdot2_bf16(xp[r][i], 0x3F803F80u, sx[r]);
        }
#pragma unroll
        for (int i = 0; i < VC; ++i) {
          const uint32_t cw[4] = {c[t][i].x, c[t][i].y, c[t][i].z, c[t][i].w};
          float d[MRC];
#pragma unroll
          for (int r = 0; r < MRC; ++r) d[r] = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = cw[j] & 0x0F0F0F0Fu, hi = (cw[j] >> 4) & 0x0F0F0F0Fu;
            const uint32_t q0 = __builtin_amdgcn_perm(C43, lo, 0x04010400u), q1 = __builtin_amdgcn_perm(C43, lo, 0x04030402u);
            const uint32_t q2 = __builtin_amdgcn_perm(C43, hi, 0x04010400u), q3 = __builtin_amdgcn_perm(C43, hi, 0x04030402u);
#pragma unroll
            for (int r = 0; r < MRC; ++r) {
              d[r] = fdot2_bf16(q0, xp[r][4 * j + 0], d[r]);
              d[r] = fdot2_bf16(q1, xp[r][4 * j + 1], d[r]);
              d[r] = fdot2_bf16(q2, xp[r][4 * j + 2], d[r]);
              d[r] = fdot2_bf16(q3, xp[r][4 * j + 3], d[r]);
            }
          }
          const float s = (!SEL || ok[t]) ? bf16_to_f32(sv[t][i]) : 0.f;
          const float b = (!SEL || ok[t]) ? bf16_to_f32(bv[t][i]) : 0.f;
          const float cb = fmaf(-128.f, s, b);
          const int m = i / RPW, rr = i % RPW;
#pragma unroll
          for (int r = 0; r < MRC; ++r) {
            float& a = acc[(m * MR + r) * RPW + rr];
            a = fmaf(s, d[r], fmaf(cb, sx[r], a));
          }
        }
      } else if (MR == 1) {
        float xf[16];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t d4[4] = {xv[t][0][j].x, xv[t][0][j].y, xv[t][0][j].z, xv[t][0][j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) { xf[8 * j + 2 * q] = bf16_lo(d4[q]); xf[8 * j + 2 * q + 1] = bf16_hi(d4[q]); }
        }
        float sx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sx += xf[i];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const uint32_t cw[4] = {c[t][i].x, c[t][i].y, c[t][i].z, c[t][i].w};
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            d = fmaf((float)((cw[j] >> 0) & 0xFFu), xf[4 * j + 0], d);
            d = fmaf((float)((cw[j] >> 8) & 0xFFu), xf[4 * j + 1], d);
            d = fmaf((float)((cw[j] >> 16) & 0xFFu), xf[4 * j + 2], d);
            d = fmaf((float)((cw[j] >> 24) & 0xFFu), xf[4 * j + 3], d);
          }
          const float s = (!SEL || ok[t]) ? bf16_to_f32(sv[t][i]) : 0.f;
          const float b = (!SEL || ok[t]) ? bf16_to_f32(bv[t][i]) : 0.f;
          acc[i] = fmaf(s, d, fmaf(b, sx, acc[i]));
        }
      } else {
        float xf[MRC][16], sx[MRC];
#pragma unroll
        for (int r = 0; r < MRC; ++r) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t d4[4] = {xv[t][r][j].x, xv[t][r][j].y, xv[t][r][j].z, xv[t][r][j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) { xf[r][8 * j + 2 * q] = bf16_lo(d4[q]); xf[r][8 * j + 2 * q + 1] = bf16_hi(d4[q]); }
          }
          sx[r] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sx[r] += xf[r][i];
        }
#pragma unroll
        for (int i = 0; i < VC; ++i) {
          const uint32_t cw[4] = {c[t][i].x, c[t][i].y, c[t][i].z, c[t][i].w};
          float d[MRC];
#pragma unroll
          for (int r = 0; r < MRC; ++r) d[r] = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float q0 = (float)((cw[j] >> 0) & 0xFFu), q1 = (float)((cw[j] >> 8) & 0xFFu);
            const float q2 = (float)((cw[j] >> 16) & 0xFFu), q3 = (float)((cw[j] >> 24) & 0xFFu);
#pragma unroll
            for (int r = 0; r < MRC; ++r) {
              d[r] = fmaf(q0, xf[r][4 * j + 0], d[r]);
              d[r] = fmaf(q1, xf[r][4 * j + 1], d[r]);
              d[r] = fmaf(q2, xf[r][4 * j + 2], d[r]);
              d[r] = fmaf(q3, xf[r][4 * j + 3], d[r]);
            }
          }
          const float s = (!SEL || ok[t]) ? bf16_to_f32(sv[t][i]) : 0.f;
          const float b = (!SEL || ok[t]) ? bf16_to_f32(bv[t][i]) : 0.f;
          const int m = i / RPW, rr = i % RPW;
#pragma unroll
          for (int r = 0; r < MRC; ++r) {
            float& a = acc[(m * MR + r) * RPW + rr];
            a = fmaf(s, d[r], fmaf(b, sx[r], a));
          }
        }
      }
    }
  }
}

// Sum the partial sums of the S waves of the workgroup into wave 0 (S > 1;
// the other waves return false), then reduce across wave 0's lanes.
template <int S, int V>
MOEGQ_DEV bool reduce_waves(float (&acc)[V], int lane, int wave) {
  if (S > 1) {
    __shared__ float part[S > 1 ? S - 1 : 1][V][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) part[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return false;
#pragma unroll
    for (int w = 0; w < S - 1; ++w)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += part[w][i][lane];
  }
  reduce_wave<V>(acc);
  return true;
}

// A workgroup of S waves owns RPW output rows of one pair; wave w takes the
// chunks w, w + S, .. of K (S > 1 when the grid alone would not keep enough
// loads in flight: few pairs, few rows).  MR > 1: the pair's A.rows (<= MR)
// activation rows share every code the waves load (qmv_rows).
template <int BITS, int GS, bool GLU, int RPW, int NS, int S, int MR = 1, int MRC = MR>
__global__ __launch_bounds__(64 * S) void qmv_kernel(QmvArgs A, int64_t p_base) {
  constexpr int V = RPW * (GLU ? 2 : 1) * MR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * RPW;
  const int64_t p = p_base + blockIdx.y;
  const int N = A.N;
  const int rowg = lane >> 4;
  const int64_t nr = MR > 1 ? A.rows : 1;
  // value q = rowg * V / 4 + j of this lane's row group, once the wave's sums
  // are reduced, is output (activation row q / RPW, column n0 + q % RPW); in
  // the GLU variant the gate values fill rows 0-1 and the up values rows 2-3
  auto out_index = [&](int q, bool& ok) -> int64_t {
    const int r = q / RPW, n = n0 + q % RPW;
    ok = r < nr && n < N;
    return (p * nr + min((int64_t)r, nr - 1)) * (int64_t)N + min(n, N - 1);
  };
  // the residual of the values this lane writes is requested before the
  // weight stream (clamped addresses, 32-bit registers), so the epilogue
  // waits for no memory
  uint32_t res_in[V / 4];
#pragma unroll
  for (int j = 0; j < V / 4; ++j) res_in[j] = 0;
  if (!GLU && A.residual && wave == 0) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      if constexpr (MR == 1) {
        res_in[j] = A.residual[p * (int64_t)N + min(n0 + rowg * (V / 4) + j, N - 1)];
      } else {
        bool ok;
        res_in[j] = A.residual[out_index(rowg * (V / 4) + j, ok)];
      }
    }
  }
  float acc[V];
  qmv_rows<BITS, GS, GLU, RPW, NS, true, MR, MRC>(A, p, n0, lane, wave * NS, S * NS, acc);
  if (!reduce_waves<S>(acc, lane, wave)) return;
  // lane 16*r (r = 2*bit5 + bit4) holds values r*V/4 .. r*V/4 + V/4 - 1
  if (GLU) {
    // gate values sit in rows 0-1, up values in rows 2-3
    float u[V / 4];
#pragma unroll
    for (int j = 0; j < V / 4; ++j) u[j] = __shfl_xor(acc[j], 32, 64);
    if ((lane & 15) == 0 && rowg < 2) {
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        if constexpr (MR == 1) {
          const int n = n0 + rowg * (V / 4) + j;
          if (n < N) A.out[p * (int64_t)N + n] = f32_to_bf16(glu(acc[j], u[j]));
        } else {
          bool ok;
          const int64_t o = out_index(rowg * (V / 4) + j, ok);
          if (ok) A.out[o] = f32_to_bf16(glu(acc[j], u[j]));
        }
      }
    }
  } else {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        bool ok;
        int64_t o;
        if constexpr (MR == 1) {
          const int n = n0 + rowg * (V / 4) + j;
          ok = n < N;
          o = p * (int64_t)N + n;
        } else {
          o = out_index(rowg * (V / 4) + j, ok);
        }
        if (ok) {
          float y = acc[j];
          if (A.residual) y = bf16_to_f32(f32_to_bf16(y)) + bf16_to_f32((uint16_t)res_in[j]);
          A.out[o] = f32_to_bf16(y);
        }
      }
    }
  }
}

// Unquantized bf16 expert rows (gather_mm with one activation row per pair):
// a wave owns 4 output rows of one pair and walks K in chunks of 512 (a lane
// takes 8 consecutive elements: one 16-byte load per row and one of x),
// accumulating with v_dot2_f32_bf16; then reduce_wave.  Rows past N repeat
// the last row (never stored); lanes past K load nothing.
__global__ __launch_bounds__(64) void mv16_kernel(QmvArgs A, int64_t p_base) {
  constexpr int RPW = 4;
  const int lane = threadIdx.x;
  const int n0 = blockIdx.x * RPW;
  const int64_t p = p_base + blockIdx.y;
  const int K = A.K, N = A.N;
  const int64_t xrow = A.lhs ? (int64_t)A.lhs[p] : p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[p] : 0;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(A.w0) + e * (int64_t)N * K;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (uint32_t)N * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(A.x + xrow * (int64_t)K, (uint32_t)K * 2u);
  constexpr uint32_t kNoFetch = 0x7FFFFFF0u;
  uint32_t soff[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) soff[r] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K * 2u;
  float acc[RPW] = {0.f, 0.f, 0.f, 0.f};
  const int nchunk = (K + 511) / 512;
#pragma unroll 2
  for (int c = 0; c < nchunk; ++c) {
    const int k = c * 512 + lane * 8;
    const uint32_t vo = k < K ? (uint32_t)k * 2u : kNoFetch;
    const uint4 xv = buf_load16(rx, vo, 0);
    uint4 wv[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) wv[r] = buf_load16_nt(rw, vo, soff[r]);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      acc[r] = fdot2_bf16(wv[r].x, xv.x, acc[r]);
      acc[r] = fdot2_bf16(wv[r].y, xv.y, acc[r]);
      acc[r] = fdot2_bf16(wv[r].z, xv.z, acc[r]);
      acc[r] = fdot2_bf16(wv[r].w, xv.w, acc[r]);
    }
  }
  reduce_wave<RPW>(acc);
  // lane 16 r holds row r's total
  if ((lane & 15) == 0) {
    const int n = n0 + (lane >> 4);
    if (n < N) A.out[p * (int64_t)N + n] = f32_to_bf16(acc[0]);
  }
}

hipError_t launch_mv16(const QmvArgs& a, int64_t P, hipStream_t st) {
  if (P <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 8 != 0) return hipErrorInvalidValue;
  const unsigned nrb = (unsigned)((a.N + 3) / 4);
  for (int64_t p0 = 0; p0 < P; p0 += 65535) {
    dim3 grid(nrb, (unsigned)(P - p0 < 65535 ? P - p0 : 65535));
    hipLaunchKernelGGL(mv16_kernel, grid, dim3(64), 0, st, a, p0);
  }
  return hipGetLastError();
}

// Decode down projection fused with the combine tail (MTPLX PR 558: unsort,
// multiply by the routing scores, sum over top_k and add the shared expert in
// one pass).  A workgroup is one token: wave k computes y for pair
// t*top_k + k over RPW output rows (the same rows for every slot), rounds it
// to bf16 as the materialized tensor would be, and the first RPW threads then
// run the combine arithmetic of combine_kernel on those values in slot order:
// out = bf16( bf16( sum_k bf16(y_k * score_k) ) + shared ).
template <int BITS, int GS, int RPW, int NS>
__global__ __launch_bounds__(512) void qmv_combine_kernel(QmvArgs A, const uint16_t* __restrict__ scores,
                                                           const uint16_t* __restrict__ shared, int top_k,
                                                           uint16_t* __restrict__ out) {
  __shared__ float ys[8][RPW];
  const int lane = threadIdx.x & 63;
  const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = blockIdx.y;
  const int n0 = blockIdx.x * RPW;
  const int N = A.N;
  const int64_t p = t * top_k + k;
  float acc[RPW];
  qmv_rows<BITS, GS, false, RPW, NS, false>(A, p, n0, lane, 0, NS, acc);
  reduce_wave<RPW>(acc);
  if ((lane & 15) == 0) {
    const int rowg = lane >> 4;
#pragma unroll
    for (int j = 0; j < RPW / 4; ++j) {
      const int r = rowg * (RPW / 4) + j;
      const uint16_t yb = f32_to_bf16(acc[j]);
      ys[k][r] = bf16_to_f32(yb);
      if (A.out && n0 + r < N) A.out[p * (int64_t)N + n0 + r] = yb;
    }
  }
  __syncthreads();
  if (threadIdx.x < RPW && n0 + (int)threadIdx.x < N) {
    const int r = threadIdx.x;
    float s = 0.f;
    for (int kk = 0; kk < top_k; ++kk) {
      const float pk = bf16_to_f32(f32_to_bf16(ys[kk][r] * bf16_to_f32(scores[t * top_k + kk])));
      s = (kk == 0) ? pk : s + pk;
    }
    float o = s;
    if (shared) o = bf16_to_f32(f32_to_bf16(s)) + bf16_to_f32(shared[t * (int64_t)N + n0 + r]);
    out[t * (int64_t)N + n0 + r] = f32_to_bf16(o);
  }
}

template <int BITS, int GS>
static hipError_t launch_qmv_combine_t(const QmvArgs& a, const uint16_t* scores, const uint16_t* shared, int64_t T,
                                      int top_k, uint16_t* out, hipStream_t st) {
  constexpr int RPW = 8;
  const unsigned nrb = (unsigned)((a.N + RPW - 1) / RPW);
  const int Kw = a.K * BITS / 32;
  for (int64_t t0 = 0; t0 < T; t0 += 65535) {
    QmvArgs b = a;
    const int64_t nt = T - t0 < 65535 ? T - t0 : 65535;
    // shift the token base into the pointers so blockIdx.y is the local token
    b.rhs = a.rhs + t0 * top_k;
    b.lhs = a.lhs ? a.lhs + t0 * top_k : nullptr;
    b.x = a.lhs ? a.x : a.x + (t0 * top_k / a.lhs_div) * (int64_t)a.K;
    b.out = a.out ? a.out + t0 * top_k * (int64_t)a.N : nullptr;
    const uint16_t* sc = scores + t0 * top_k;
    const uint16_t* sh = shared ? shared + t0 * (int64_t)a.N : nullptr;
    uint16_t* o = out + t0 * (int64_t)a.N;
    dim3 grid(nrb, (unsigned)nt);
    if (Kw > 256 && Kw <= 512 && BITS == 4)
      hipLaunchKernelGGL((qmv_combine_kernel<BITS, GS, RPW, 2>), grid, dim3(64 * top_k), 0, st, b, sc, sh, top_k, o);
    else
      hipLaunchKernelGGL((qmv_combine_kernel<BITS, GS, RPW, 1>), grid, dim3(64 * top_k), 0, st, b, sc, sh, top_k, o);
  }
  return hipGetLastError();
}

hipError_t launch_qmv_combine(const QmvArgs& a_in, int bits, int gs, const uint16_t* scores, const uint16_t* shared,
                              int64_t T, int top_k, uint16_t* out, hipStream_t st) {
  if (T <= 0 || a_in.N <= 0) return hipSuccess;
  QmvArgs a = a_in;
  a.lhs_shift = -1;
  if (a.lhs_div > 0 && (a.lhs_div & (a.lhs_div - 1)) == 0) {
    a.lhs_shift = 0;
    while ((int64_t(1) << a.lhs_shift) < a.lhs_div) ++a.lhs_shift;
  }
#define MOEGQ_QC(B, G) if (bits == B && gs == G) return launch_qmv_combine_t<B, G>(a, scores, shared, T, top_k, out, st);
  MOEGQ_QC(4, 32) MOEGQ_QC(4, 64) MOEGQ_QC(4, 128) MOEGQ_QC(8, 32) MOEGQ_QC(8, 64) MOEGQ_QC(8, 128)
#undef MOEGQ_QC
  return hipErrorInvalidValue;
}

// Waves in flight wanted for the whole launch: with fewer, each wave's loads
// are too few to cover the memory latency.
constexpr int64_t kQmvWaves = 4096;

template <int BITS, int GS, bool GLU, int RPW, int NS, int S, int MR = 1, int MRC = MR>
static void launch_qmv_cfg(const QmvArgs& a, int64_t P, hipStream_t st) {
  const unsigned nrb = (unsigned)((a.N + RPW - 1) / RPW);
  for (int64_t p0 = 0; p0 < P; p0 += 65535) {
    dim3 grid(nrb, (unsigned)(P - p0 < 65535 ? P - p0 : 65535));
    hipLaunchKernelGGL((qmv_kernel<BITS, GS, GLU, RPW, NS, S, MR, MRC>), grid, dim3(64 * S), 0, st, a, p0);
  }
}

// 2..4 activation rows per pair: one chunk of codes at a time (the rows'
// activations take the registers a second chunk would), 2 (GLU; one row of
// each matrix per wave was slower) or 4 output rows per wave, K split over up
// to 4 waves when the grid is small.  3 rows compute 3 and keep the 4-row
// layout.
template <int BITS, int GS, bool GLU, int MR, int MRC>
static hipError_t launch_qmv_rows_t(const QmvArgs& a, int64_t P, hipStream_t st) {
  if (GLU) {
    launch_qmv_cfg<BITS, GS, true, 2, 1, 1, MR, MRC>(a, P, st);
    return hipGetLastError();
  }
  const int n_it = (a.K * BITS / 32 + 255) / 256;
  const int64_t w4 = (int64_t)((a.N + 3) / 4) * P;
  int S = 1;
  while (S < 4 && 2 * S <= n_it && w4 * S < kQmvWaves) S *= 2;
  if (S == 4) launch_qmv_cfg<BITS, GS, false, 4, 1, 4, MR, MRC>(a, P, st);
  else if (S == 2) launch_qmv_cfg<BITS, GS, false, 4, 1, 2, MR, MRC>(a, P, st);
  else launch_qmv_cfg<BITS, GS, false, 4, 1, 1, MR, MRC>(a, P, st);
  return hipGetLastError();
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_qmv_t(const QmvArgs& a, int64_t P, hipStream_t st) {
  if (a.rows > 1) return a.rows == 2   ? launch_qmv_rows_t<BITS, GS, GLU, 2, 2>(a, P, st)
                         : a.rows == 3 ? launch_qmv_rows_t<BITS, GS, GLU, 4, 3>(a, P, st)
                                       : launch_qmv_rows_t<BITS, GS, GLU, 4, 4>(a, P, st);
  const int Kw = a.K * BITS / 32;
  const int n_it = (Kw + 255) / 256;
  const bool two = Kw > 256 && Kw <= 512 && (GLU || BITS == 4);   // the whole row in one chunk of 2 slices
  if (GLU) {
    // 2 rows x 2 matrices per wave
    if (two) launch_qmv_cfg<BITS, GS, true, 2, 2, 1>(a, P, st);
    else launch_qmv_cfg<BITS, GS, true, 2, 1, 1>(a, P, st);
    return hipGetLastError();
  }
  if ((int64_t)((a.N + 7) / 8) * P >= kQmvWaves) {      // many pairs: 8 rows per wave
    if (two) launch_qmv_cfg<BITS, GS, false, 8, 2, 1>(a, P, st);
    else launch_qmv_cfg<BITS, GS, false, 8, 1, 1>(a, P, st);
    return hipGetLastError();
  }
  // few pairs (a dense product): 4 rows per wave, and K split over up to 4
  // waves of a workgroup
  const int64_t w4 = (int64_t)((a.N + 3) / 4) * P;
  int S = 1;
  while (S < 4 && 2 * S <= n_it && w4 * S < kQmvWaves) S *= 2;
  if (S == 4) launch_qmv_cfg<BITS, GS, false, 4, 1, 4>(a, P, st);
  else if (S == 2) launch_qmv_cfg<BITS, GS, false, 4, 1, 2>(a, P, st);
  else launch_qmv_cfg<BITS, GS, false, 4, 1, 1>(a, P, st);
  return hipGetLastError();
}

template <int BITS, bool GLU>
static hipError_t launch_qmv_gs(const QmvArgs& a, int gs, int64_t P, hipStream_t st) {
  switch (gs) {
    case 32: return launch_qmv_t<BITS, 32, GLU>(a, P, st);
    case 64: return launch_qmv_t<BITS, 64, GLU>(a, P, st);
    case 128: return launch_qmv_t<BITS, 128, GLU>(a, P, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qmv(const QmvArgs& a_in, int bits, int gs, bool glu, int64_t P, hipStream_t st) {
  if (P <= 0 || a_in.N <= 0) return hipSuccess;
  if (a_in.rows > 4) return hipErrorInvalidValue;
  QmvArgs a = a_in;
  a.lhs_shift = -1;
  if (a.lhs_div > 0 && (a.lhs_div & (a.lhs_div - 1)) == 0) {
    a.lhs_shift = 0;
    while ((int64_t(1) << a.lhs_shift) < a.lhs_div) ++a.lhs_shift;
  }
  if (bits == 4) return glu ? launch_qmv_gs<4, true>(a, gs, P, st) : launch_qmv_gs<4, false>(a, gs, P, st);
  if (bits == 8) return glu ? launch_qmv_gs<8, true>(a, gs, P, st) : launch_qmv_gs<8, false>(a, gs, P, st);
  return hipErrorInvalidValue;
}

}  // namespace moegq

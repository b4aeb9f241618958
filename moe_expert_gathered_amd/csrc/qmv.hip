// Gathered matrix-vector kernels for decode (one activation row per pair).
//
// For pair p the kernel computes out[p, n] = x[row(p)] . dequant(W[e(p)][n])^T
// (MLX issue 4509, gq(): gather_qmm with rhs_indices over x[M,1,1,H]), and in
// the GLU variant h[p, n] = silu(x . Wg^T) * (x . Wu^T) for the gate and up
// projections of SwitchGLU (same page, moe(): up, gate, silu(gate)*up).
//
// Mapping on gfx950: a workgroup owns one pair and 4 waves x RPW output rows.
// The pair's activation row is staged once in LDS (already in the lane order
// the dot products use).  Each wave streams RPW rows (two matrices in the GLU
// variant) with 128-bit coalesced loads: lane l reads words [4l, 4l+4) of every
// 256-word slice of a row, so one load instruction covers 1 KiB of one row.
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

template <int V>
MOEGQ_DEV void butterfly(float (&a)[V], int lane) {
  // After the halving steps lane l holds value v(l) = sum over steps of
  // (l & (32 >> s)) ? V >> (s+1) : 0, partially reduced; the remaining
  // offsets finish the sum.  Value v ends in lane v * (64 / V).
#pragma unroll
  for (int s = 0; (V >> s) > 1; ++s) {
    const int half = V >> (s + 1);
    const int off = 32 >> s;
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      float send = upper ? a[i] : a[i + half];
      float keep = upper ? a[i + half] : a[i];
      a[i] = keep + shfl_xor(send, off);
    }
  }
  constexpr int lg = (V >= 64) ? 6 : (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
#pragma unroll
  for (int off = 32 >> lg; off >= 1; off >>= 1) a[0] += shfl_xor(a[0], off);
}

template <int BITS, int GS, bool GLU, int RPW>
__global__ __launch_bounds__(256) void qmv_kernel(QmvArgs A) {
  extern __shared__ uint4 xs[];  // activation row, K bf16 (4-bit: pair-permuted)
  constexpr int NM = GLU ? 2 : 1;
  constexpr int V = RPW * NM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 1-D grid: consecutive blocks walk the row blocks of one pair, so one
  // expert matrix is streamed front to back by neighbouring workgroups
  const int nrb = (A.N + 4 * RPW - 1) / (4 * RPW);
  const int64_t p = blockIdx.x / nrb;
  const int rb = blockIdx.x % nrb;
  const int K = A.K, N = A.N;
  const int64_t xrow = A.lhs ? (int64_t)A.lhs[p] : p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[p] : 0;

  // stage the activation row
  const uint4* xg = reinterpret_cast<const uint4*>(A.x + xrow * (int64_t)K);
  for (int c = tid; c < K / 8; c += 256) {
    uint4 v = xg[c];
    if (BITS == 4) {
      uint32_t d[4] = {v.x, v.y, v.z, v.w}, o[4];
      perm_pairs(d, o);
      v = make_uint4(o[0], o[1], o[2], o[3]);
    }
    xs[c] = v;
  }
  __syncthreads();

  const int Kw = K * BITS / 32;      // words per row
  const int G = K / GS;              // groups per row
  const int n0 = rb * (4 * RPW) + wave * RPW;
  const uint32_t* wm[NM];
  const uint16_t* sm[NM];
  const uint16_t* bm[NM];
  wm[0] = A.w0 + e * (int64_t)N * Kw;
  sm[0] = A.s0 + e * (int64_t)N * G;
  bm[0] = A.b0 + e * (int64_t)N * G;
  if (GLU) {
    wm[NM - 1] = A.w1 + e * (int64_t)N * Kw;
    sm[NM - 1] = A.s1 + e * (int64_t)N * G;
    bm[NM - 1] = A.b1 + e * (int64_t)N * G;
  }
  int rown[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) rown[r] = min(n0 + r, N - 1);  // clamp: rows past N are computed and dropped

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;

  const int n_it = (Kw + 255) / 256;
  uint4 cur[V];
  auto load = [&](int it, uint4 (&dst)[V]) {
    const int wb = it * 256 + lane * 4;
    const bool ok = wb < Kw;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const uint4* src = reinterpret_cast<const uint4*>(wm[m] + (int64_t)rown[r] * Kw + wb);
        dst[m * RPW + r] = ok ? ld_nt(src) : make_uint4(0, 0, 0, 0);
      }
  };
  load(0, cur);
  for (int it = 0; it < n_it; ++it) {
    uint4 nxt[V];
    if (it + 1 < n_it) load(it + 1, nxt);
    const int wb = it * 256 + lane * 4;
    const bool ok = wb < Kw;
    const int k0 = wb * (32 / BITS);
    const int g = min(k0 / GS, G - 1);
    if (BITS == 4) {
      // 32 codes per lane: x chunks k0/8 .. k0/8+3, each 8 bf16 in pair order
      uint32_t xp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 v = ok ? xs[k0 / 8 + j] : make_uint4(0, 0, 0, 0);
        xp[4 * j + 0] = v.x; xp[4 * j + 1] = v.y; xp[4 * j + 2] = v.z; xp[4 * j + 3] = v.w;
      }
      float sx = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sx = fdot2_bf16(xp[i], 0x3F803F80u, sx);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint4 c = cur[m * RPW + r];
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t pr[4];
            nib_pairs(cw[j], pr);
#pragma unroll
            for (int q = 0; q < 4; ++q) d = fdot2_bf16(pr[q], xp[4 * j + q], d);
          }
          const int64_t gi = (int64_t)rown[r] * G + g;
          const float s = ok ? bf16_to_f32(sm[m][gi]) : 0.f;
          const float b = ok ? bf16_to_f32(bm[m][gi]) : 0.f;
          acc[m * RPW + r] += s * d + (b - 128.f * s) * sx;
        }
    } else {
      // 16 codes per lane: x chunks k0/8, k0/8+1 in natural order
      float xf[16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 v = ok ? xs[k0 / 8 + j] : make_uint4(0, 0, 0, 0);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { xf[8 * j + 2 * q] = bf16_lo(d[q]); xf[8 * j + 2 * q + 1] = bf16_hi(d[q]); }
      }
      float sx = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sx += xf[i];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint4 c = cur[m * RPW + r];
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            d = fmaf((float)((cw[j] >> 0) & 0xFFu), xf[4 * j + 0], d);
            d = fmaf((float)((cw[j] >> 8) & 0xFFu), xf[4 * j + 1], d);
            d = fmaf((float)((cw[j] >> 16) & 0xFFu), xf[4 * j + 2], d);
            d = fmaf((float)((cw[j] >> 24) & 0xFFu), xf[4 * j + 3], d);
          }
          const int64_t gi = (int64_t)rown[r] * G + g;
          const float s = ok ? bf16_to_f32(sm[m][gi]) : 0.f;
          const float b = ok ? bf16_to_f32(bm[m][gi]) : 0.f;
          acc[m * RPW + r] += s * d + b * sx;
        }
    }
    if (it + 1 < n_it) {
#pragma unroll
      for (int i = 0; i < V; ++i) cur[i] = nxt[i];
    }
  }

  butterfly<V>(acc, lane);
  constexpr int STRIDE = 64 / V;
  if (GLU) {
    const float u = __shfl_xor(acc[0], 32, 64);   // up of row r sits 32 lanes above its gate
    const int r = lane / STRIDE;
    if ((lane % STRIDE) == 0 && r < RPW) {
      const int n = n0 + r;
      if (n < N) {
        float h = glu(acc[0], u);
        A.out[p * (int64_t)N + n] = f32_to_bf16(h);
      }
    }
  } else {
    const int r = lane / STRIDE;
    if ((lane % STRIDE) == 0 && r < RPW) {
      const int n = n0 + r;
      if (n < N) {
        float y = acc[0];
        if (A.residual) {
          y = bf16_to_f32(f32_to_bf16(y)) + bf16_to_f32(A.residual[p * (int64_t)N + n]);
        }
        A.out[p * (int64_t)N + n] = f32_to_bf16(y);
      }
    }
  }
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_qmv_t(const QmvArgs& a, int64_t P, hipStream_t st) {
  constexpr int RPW = GLU ? 4 : 8;
  const int64_t nrb = (a.N + 4 * RPW - 1) / (4 * RPW);
  dim3 grid((unsigned)(nrb * P));
  size_t lds = (size_t)a.K * 2;
  hipLaunchKernelGGL((qmv_kernel<BITS, GS, GLU, RPW>), grid, dim3(256), lds, st, a);
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

hipError_t launch_qmv(const QmvArgs& a, int bits, int gs, bool glu, int64_t P, hipStream_t st) {
  if (P <= 0 || a.N <= 0) return hipSuccess;
  if (bits == 4) return glu ? launch_qmv_gs<4, true>(a, gs, P, st) : launch_qmv_gs<4, false>(a, gs, P, st);
  if (bits == 8) return glu ? launch_qmv_gs<8, true>(a, gs, P, st) : launch_qmv_gs<8, false>(a, gs, P, st);
  return hipErrorInvalidValue;
}

}  // namespace moegq

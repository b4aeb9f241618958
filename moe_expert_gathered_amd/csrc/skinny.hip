// Few-row quantized matmul (2..16 activation rows per weight matrix) on MFMA.
//
// MLX PR 4787: at 3-16 rows the weights should feed the matrix units rather
// than a per-row vector loop (the pages' qmv_mma).  On gfx950 a wave computes
// a 16 (rows, zero-padded) x 16 (outputs) block with v_mfma_f32_16x16x32_f16.
//
// The contraction order over K inside an MFMA is free as long as both
// operands use the same order, so each lane loads 128-bit runs of its output
// row (lane (n, j) takes words [4j, 4j+4) of every 16-word chunk) and the
// activation operand is read at the matching K offsets.  Codes are
// dequantized to fp16 (q * s + b with one rounding; nuvec "composed") and the
// activations converted to fp16 for v_mfma_f32_16x16x32_f16; all 32 codes of
// a lane share one group.
// The 4 to 16 waves of a workgroup take interleaved 128-code chunks of K for
// the same 16 outputs (each with the next chunk's loads in flight) and are
// summed through LDS at the end.
#include "common.h"
#include "launch.h"

namespace moegq {

template <int BITS, int GS, bool GLU, int SK, int CL>
__global__ __launch_bounds__(64 * SK) void skinny_kernel(SkinnyArgs A) {
  // CL codes per lane and chunk (32 or 64): a chunk is 4 * CL codes of K
  constexpr int NM = GLU ? 2 : 1;
  constexpr int BV = BITS * CL / 128;   // uint4 per lane per chunk
  constexpr int NG = CL / 32 > 1 && GS < CL ? CL / GS : 1;   // groups per lane and chunk
  constexpr int ST = CL / 8;            // MFMA steps per chunk
  constexpr int CK = 4 * CL;            // codes per chunk
  __shared__ f32x4_t red[SK - 1][NM][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrb = (A.N + 15) / 16;
  const int64_t p = blockIdx.x / nrb;
  const int n0 = (blockIdx.x % nrb) * 16;
  const int K = A.K, N = A.N, M = A.M;
  const int Kw = K * BITS / 32, G = K / GS;
  const int64_t xb = A.lhs ? (int64_t)A.lhs[p] : p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[p] : 0;
  const int li = lane % 16, lj = lane / 16;
  const int n = min(n0 + li, N - 1);
  const bool m_ok = li < M;
  const uint16_t* xrow = A.x + (xb * M + (m_ok ? li : 0)) * (int64_t)K;

  const uint32_t* wr[NM];
  const uint16_t* sr[NM];
  const uint16_t* br[NM];
  wr[0] = A.w0 + (e * N + n) * (int64_t)Kw;
  sr[0] = A.s0 + (e * N + n) * (int64_t)G;
  br[0] = A.b0 + (e * N + n) * (int64_t)G;
  if (GLU) {
    wr[NM - 1] = A.w1 + (e * N + n) * (int64_t)Kw;
    sr[NM - 1] = A.s1 + (e * N + n) * (int64_t)G;
    br[NM - 1] = A.b1 + (e * N + n) * (int64_t)G;
  }
  f32x4_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the residual of the lane's four outputs (wave 0 writes them) is requested
  // before the K loop, so the epilogue waits for no memory
  uint32_t res_in[4] = {0, 0, 0, 0};      // 32-bit: no packing step that would wait for the loads
  if (!GLU && A.residual && wave == 0) {
    // clamped to a valid element (the epilogue uses only valid ones): no
    // per-lane branch, so no wait before the values are used
#pragma unroll
    for (int q = 0; q < 4; ++q)
      res_in[q] = A.residual[(p * M + min(4 * lj + q, M - 1)) * (int64_t)N + min(n0 + li, N - 1)];
  }

  // one chunk's operands: CL codes per lane and matrix, their groups' scales
  // and biases, and the matching activations (8-element runs)
  struct Chunk {
    uint4 cw[NM][BV];
    uint16_t s[NM][NG], b[NM][NG];
    uint4 xv[ST];
  };
  const int nchunk = (K + CK - 1) / CK;
  auto load = [&](int c, Chunk& d) {
    const int kl = c * CK + CL * lj;           // first of this lane's CL codes
    const bool ok = c < nchunk && kl < K;
    // K is a multiple of 32: each run of 32 codes is all in or all out
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int v = 0; v < BV; ++v)
        d.cw[m][v] = (ok && kl + v * (128 / BITS) < K)
                         ? ldg(reinterpret_cast<const uint4*>(wr[m] + kl * BITS / 32 + 4 * v)) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        d.s[m][gi] = (ok && kl + gi * GS < K) ? sr[m][kl / GS + gi] : (uint16_t)0;
        d.b[m][gi] = (ok && kl + gi * GS < K) ? br[m][kl / GS + gi] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int st = 0; st < ST; ++st)
      d.xv[st] = (ok && m_ok && kl + 8 * st < K) ? *reinterpret_cast<const uint4*>(xrow + kl + 8 * st)
                                                 : make_uint4(0, 0, 0, 0);
  };
  auto compute = [&](const Chunk& d) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const f16x8_t xa = __builtin_bit_cast(f16x8_t, act_f16<BITS>(d.xv[st]));   // shared by both matrices
      const int gi = NG > 1 ? (8 * st) / GS : 0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f16x2_t s2 = f16_splat(bf16_to_f32(d.s[m][gi])), b2 = f16_splat(bf16_to_f32(d.b[m][gi]));
        uint32_t o[4];
        if (BITS == 4) {
          deq4_f16((&d.cw[m][0].x)[st], s2, b2, o);
        } else {
          deq8_f16((&d.cw[m][0].x)[2 * st], s2, b2, &o[0]);
          deq8_f16((&d.cw[m][0].x)[2 * st + 1], s2, b2, &o[2]);
        }
        const f16x8_t bw = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, bw, acc[m], 0, 0, 0);
      }
    }
  };
  // chunk c belongs to wave c % SK; the next chunk's loads are in flight
  // while the current one is computed
  Chunk cur, nxt;
  load(wave, cur);
  for (int c = wave; c < nchunk; c += SK) {
    load(c + SK, nxt);
    compute(cur);
    cur = nxt;
  }
  // sum the waves' partial blocks
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NM; ++m) red[wave - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int w = 0; w < SK - 1; ++w) acc[m] += red[w][m][lane];
  // C[row = 4*lj + q][col = li]
  const int col = n0 + li;
  if (col >= N) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * lj + q;
    if (row < M) {
      const int64_t o = (p * M + row) * (int64_t)N + col;
      float v = GLU ? glu(acc[0][q], acc[NM - 1][q]) : acc[0][q];
      if (!GLU && A.residual) v = bf16_to_f32(f32_to_bf16(v)) + bf16_to_f32((uint16_t)res_in[q]);
      A.out[o] = f32_to_bf16(v);
    }
  }
}

// Expert tiles with few rows (the long tail of a skewed routing): tile t of
// the small-tile list is (row_start, expert, valid <= 16 * MB); the rows are
// sorted rows whose activations are gathered through lhs.  Each workgroup
// streams 16 features of the expert once for all of the tile's rows (MB
// 16-row MFMA blocks share every dequantized weight operand).
template <int BITS, int GS, bool GLU, int MB>
__global__ __launch_bounds__(256) void skinny_tiles_kernel(TileArgs A) {
  constexpr int NM = GLU ? 2 : 1;
  constexpr int BV = BITS / 4;
  __shared__ f32x4_t red[3][NM][MB][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrb = (A.N + 15) / 16;
  const int64_t tile = blockIdx.x / nrb;
  if (tile >= *A.n_tiles) return;
  const int n0 = (blockIdx.x % nrb) * 16;
  const int K = A.K, N = A.N;
  const int Kw = K * BITS / 32, G = K / GS;
  const int32_t* tl = A.tiles + 3 * tile;
  const int64_t r0 = tl[0];
  const int e = tl[1];
  const int valid = tl[2];
  const int li = lane % 16, lj = lane / 16;
  const int n = min(n0 + li, N - 1);
  const uint16_t* xrow[MB];
  bool m_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + li;
    m_ok[mb] = m < valid;
    const int64_t r = r0 + (m_ok[mb] ? m : 0);
    const int64_t xr = A.lhs ? (int64_t)A.lhs[r] : r;
    xrow[mb] = A.x + xr * (int64_t)K;
  }
  const uint32_t* wr[NM];
  const uint16_t* sr[NM];
  const uint16_t* br[NM];
  wr[0] = A.w0 + ((int64_t)e * N + n) * Kw;
  sr[0] = A.s0 + ((int64_t)e * N + n) * G;
  br[0] = A.b0 + ((int64_t)e * N + n) * G;
  if (GLU) {
    wr[NM - 1] = A.w1 + ((int64_t)e * N + n) * Kw;
    sr[NM - 1] = A.s1 + ((int64_t)e * N + n) * G;
    br[NM - 1] = A.b1 + ((int64_t)e * N + n) * G;
  }
  f32x4_t acc[NM][MB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[m][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunk = (K + 127) / 128;
  for (int c = wave; c < nchunk; c += 4) {
    const int kl = c * 128 + 32 * lj;
    const bool ok = kl < K;
    uint4 cw[NM][BV];
    float s[NM], b[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int v = 0; v < BV; ++v)
        cw[m][v] = ok ? ld_nt(reinterpret_cast<const uint4*>(wr[m] + kl * BITS / 32 + 4 * v)) : make_uint4(0, 0, 0, 0);
      s[m] = ok ? bf16_to_f32(sr[m][kl / GS]) : 0.f;
      b[m] = ok ? bf16_to_f32(br[m][kl / GS]) : 0.f;
    }
    f16x8_t xa[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint4 v = (ok && m_ok[mb]) ? *reinterpret_cast<const uint4*>(xrow[mb] + kl + 8 * st) : make_uint4(0, 0, 0, 0);
        xa[mb][st] = __builtin_bit_cast(f16x8_t, act_f16<BITS>(v));
      }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t o[4];
        const f16x2_t s2 = f16_splat(s[m]), b2 = f16_splat(b[m]);
        if (BITS == 4) {
          deq4_f16((&cw[m][0].x)[st], s2, b2, o);
        } else {
          deq8_f16((&cw[m][0].x)[2 * st], s2, b2, &o[0]);
          deq8_f16((&cw[m][0].x)[2 * st + 1], s2, b2, &o[2]);
        }
        const f16x8_t bw = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[m][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[mb][st], bw, acc[m][mb], 0, 0, 0);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red[wave - 1][m][mb][lane] = acc[m][mb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int w = 0; w < 3; ++w) acc[m][mb] += red[w][m][mb][lane];
  const int col = n0 + li;
  if (col >= N) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = mb * 16 + 4 * lj + q;
      if (row < valid) {
        const float v = GLU ? glu(acc[0][mb][q], acc[NM - 1][mb][q]) : acc[0][mb][q];
        A.out[(r0 + row) * (int64_t)N + col] = f32_to_bf16(v);
      }
    }
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_skt(const TileArgs& a, hipStream_t st) {
  const int64_t nrb = (a.N + 15) / 16;
  const int64_t nblk = a.grid_tiles * nrb;
  if (nblk <= 0) return hipSuccess;
  if (a.bm <= 16)
    hipLaunchKernelGGL((skinny_tiles_kernel<BITS, GS, GLU, 1>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((skinny_tiles_kernel<BITS, GS, GLU, 2>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tiles_small(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st) {
#define MOEGQ_SKT(B, G)                                                                   \
  if (bits == B && gs == G) return glu ? launch_skt<B, G, true>(a, st) : launch_skt<B, G, false>(a, st);
  MOEGQ_SKT(4, 32) MOEGQ_SKT(4, 64) MOEGQ_SKT(4, 128) MOEGQ_SKT(8, 32) MOEGQ_SKT(8, 64) MOEGQ_SKT(8, 128)
#undef MOEGQ_SKT
  return hipErrorInvalidValue;
}

// Waves per workgroup: 4, or up to 16 when the grid alone would not keep
// enough loads in flight (a dense product: one pair, few column blocks).
constexpr int64_t kSkinnyWaves = 4096;

template <int BITS, int GS, bool GLU>
static hipError_t launch_sk(const SkinnyArgs& a, int64_t P, hipStream_t st) {
  constexpr int CL = 32;   // 64 codes per lane measured slower at 4 and 16 rows
  const int64_t nrb = (a.N + 15) / 16;
  const int64_t nblk = nrb * P;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int nchunk = (a.K + 4 * CL - 1) / (4 * CL);
  int SK = 4;
  while (SK < 16 && 2 * SK <= nchunk && nblk * SK < kSkinnyWaves) SK *= 2;
  if (SK == 16)
    hipLaunchKernelGGL((skinny_kernel<BITS, GS, GLU, 16, CL>), dim3((unsigned)nblk), dim3(1024), 0, st, a);
  else if (SK == 8)
    hipLaunchKernelGGL((skinny_kernel<BITS, GS, GLU, 8, CL>), dim3((unsigned)nblk), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((skinny_kernel<BITS, GS, GLU, 4, CL>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS, bool GLU>
static hipError_t launch_sk_gs(const SkinnyArgs& a, int gs, int64_t P, hipStream_t st) {
  switch (gs) {
    case 32: return launch_sk<BITS, 32, GLU>(a, P, st);
    case 64: return launch_sk<BITS, 64, GLU>(a, P, st);
    case 128: return launch_sk<BITS, 128, GLU>(a, P, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_skinny(const SkinnyArgs& a, int bits, int gs, bool glu, int64_t P, hipStream_t st) {
  if (P <= 0 || a.N <= 0) return hipSuccess;
  if (bits == 4) return glu ? launch_sk_gs<4, true>(a, gs, P, st) : launch_sk_gs<4, false>(a, gs, P, st);
  if (bits == 8) return glu ? launch_sk_gs<8, true>(a, gs, P, st) : launch_sk_gs<8, false>(a, gs, P, st);
  return hipErrorInvalidValue;
}

}  // namespace moegq

// Prefill gathered GEMM over expert-sorted rows (bf16 MFMA on gfx950).
//
// MLX PR 4567 (Description / Proposed changes): with tiles cut independently
// of the expert boundaries a tile runs one K pass per expert it touches ("as
// many matmuls as necessary"); the expert-aware schedule gives every tile a
// row start, one expert and a valid-row count, so each tile makes exactly one
// K pass.  Both modes are built here: SCHEDULED reads the tile table, NAIVE
// cuts fixed BM-row tiles and loops over the experts present.
// MTPLX PR 558 (Change): the rows are the expert-sorted (token, slot) pairs;
// the gate/up pass gathers x rows by lhs = token of the pair, the down pass
// reads the sorted intermediate rows in place.
//
// Per K step (BK = 128) a 256-thread workgroup
//   * gathers BM activation rows (bf16) into LDS,
//   * loads BN x BK packed codes per matrix, dequantizes them to fp16
//     (q * s + b with one rounding, nuvec "composed") into LDS next to the
//     activations converted to fp16,
//   * runs v_mfma_f32_16x16x32_f16 with fp32 accumulation; the 4 waves split
//     the BM x BN tile.
// The next step's global loads are issued before the current step's MFMAs.
// GLU: gate and up share the activation tile; the epilogue writes
// bf16(silu(g) * u) (MLX issue 4509, moe()).
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int TBN = 64;     // output columns per matrix per workgroup
constexpr int TBK = 128;    // K per step
constexpr int TPAD = 8;     // bf16 padding per LDS row (bank spread)
constexpr int TLD = TBK + TPAD;

template <int BITS, int GS, bool GLU, int BM>
__global__ __launch_bounds__(256) void tile_kernel(TileArgs A) {
  constexpr int NM = GLU ? 2 : 1;
  constexpr int WAVES_M = BM >= 32 ? 2 : 1;   // 4 waves split the tile WAVES_M x WAVES_N
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M;            // rows per wave
  constexpr int WN = TBN / WAVES_N;           // columns per wave
  constexpr int MI = WM / 16;                 // 16-row MFMA blocks per wave
  constexpr int NI = WN / 16;                 // 16-col MFMA blocks per wave
  constexpr int AV = (BM * TBK / 8 + 255) / 256; // uint4 of A per thread per step
  constexpr int BV = BITS / 4;          // uint4 of codes per thread per matrix per step
  extern __shared__ uint4 lds_raw[];
  uint16_t* As = reinterpret_cast<uint16_t*>(lds_raw);                 // [BM][TLD]
  uint16_t* Bs = As + BM * TLD;                                         // [NM][TBN][TLD]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int NB = (A.N + TBN - 1) / TBN;
  const int64_t tile = blockIdx.x / NB;
  const int nb = blockIdx.x % NB;
  const int n0 = nb * TBN;
  const int K = A.K, N = A.N;
  const int Kw = K * BITS / 32, G = K / GS;

  int64_t r0, r1;      // sorted rows [r0, r1) of this tile
  int e_lo, e_hi;      // experts to visit
  if (A.tile_mode == 0) {
    if (tile >= *A.n_tiles) return;
    const int32_t* t = A.tiles + 3 * tile;
    r0 = t[0]; e_lo = e_hi = t[1]; r1 = r0 + t[2];
  } else {
    r0 = tile * BM;
    if (r0 >= A.P) return;
    r1 = min(A.P, r0 + BM);
    if (A.tile_mode == 1) {
      e_lo = A.sorted_rhs[r0];
      e_hi = A.sorted_rhs[r1 - 1];
    } else {
      e_lo = e_hi = 0;       // dense: one weight matrix, tiles over the rows
    }
  }

  // per-thread roles in the global loads
  const int a_row0 = tid / 16, a_chunk = tid % 16;     // A: rows a_row0 + 16 i, 8 bf16 at chunk
  const int b_n = tid / 4, b_q = tid % 4;              // B: row b_n, codes [32 b_q, 32 b_q + 32)
  // rows past the tile look up row r0 (always valid) and are marked -1 after,
  // so the AV index loads are issued together and waited for once
  int64_t a_src[AV], a_r[AV], a_bx[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int64_t r = r0 + a_row0 + 16 * i;
    a_r[i] = (a_row0 + 16 * i < BM && r < r1) ? r : -1;
    a_bx[i] = (a_r[i] >= 0 ? a_r[i] : r0) / A.rows_per_batch;
  }
  if (A.lhs) {
#pragma unroll
    for (int i = 0; i < AV; ++i) a_bx[i] = A.lhs[a_bx[i]];
  } else {
#pragma unroll
    for (int i = 0; i < AV; ++i) a_bx[i] /= A.lhs_div;
  }
#pragma unroll
  for (int i = 0; i < AV; ++i)
    a_src[i] = a_r[i] >= 0 ? a_bx[i] * A.rows_per_batch + a_r[i] % A.rows_per_batch : -1;
  const int bn_g = min(n0 + b_n, N - 1);

  f32x4_t acc[NM][MI][NI];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nK = (K + TBK - 1) / TBK;
  for (int e = e_lo; e <= e_hi; ++e) {
    int64_t s0 = r0, s1 = r1;   // rows of this expert inside the tile
    if (A.tile_mode == 1) {
      s0 = max(r0, (int64_t)A.offsets[e]);
      s1 = min(r1, (int64_t)A.offsets[e + 1]);
      if (s0 >= s1) continue;
    }
    bool a_ok[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int64_t r = r0 + a_row0 + 16 * i;
      a_ok[i] = a_src[i] >= 0 && r >= s0 && r < s1;
    }
    const uint32_t* wsrc[NM];
    const uint16_t* ssrc[NM];
    const uint16_t* bsrc[NM];
    wsrc[0] = A.w0 + ((int64_t)e * N + bn_g) * Kw;
    ssrc[0] = A.s0 + ((int64_t)e * N + bn_g) * G;
    bsrc[0] = A.b0 + ((int64_t)e * N + bn_g) * G;
    if (GLU) {
      wsrc[NM - 1] = A.w1 + ((int64_t)e * N + bn_g) * Kw;
      ssrc[NM - 1] = A.s1 + ((int64_t)e * N + bn_g) * G;
      bsrc[NM - 1] = A.b1 + ((int64_t)e * N + bn_g) * G;
    }

    uint4 ra[AV], rb[NM][BV];
    float rs[NM], rbias[NM];
    auto gload = [&](int ks) {
      const int kk = ks * TBK;
#pragma unroll
      for (int i = 0; i < AV; ++i)
        ra[i] = (a_ok[i] && kk + a_chunk * 8 < K)
                    ? *reinterpret_cast<const uint4*>(A.x + a_src[i] * K + kk + a_chunk * 8)
                    : make_uint4(0, 0, 0, 0);
      const int kc = kk + 32 * b_q;            // first code of this thread's 32
      const bool kok = kc < K;                 // codes past K meet zero activations
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int v = 0; v < BV; ++v)
          rb[m][v] = kok ? *reinterpret_cast<const uint4*>(wsrc[m] + kc * BITS / 32 + 4 * v)
                         : make_uint4(0, 0, 0, 0);
        rs[m] = kok ? bf16_to_f32(ssrc[m][kc / GS]) : 0.f;
        rbias[m] = kok ? bf16_to_f32(bsrc[m][kc / GS]) : 0.f;
      }
    };
    gload(0);
    for (int ks = 0; ks < nK; ++ks) {
      __syncthreads();   // previous step's MFMAs are done with the LDS tiles
#pragma unroll
      for (int i = 0; i < AV; ++i)
        if (a_row0 + 16 * i < BM)
          *reinterpret_cast<uint4*>(As + (a_row0 + 16 * i) * TLD + a_chunk * 8) = act_f16<BITS>(ra[i]);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        uint32_t o[16];
        const f16x2_t s2 = f16_splat(rs[m]), b2 = f16_splat(rbias[m]);
        if (BITS == 4) {
#pragma unroll
          for (int v = 0; v < 4; ++v) deq4_f16((&rb[m][0].x)[v], s2, b2, &o[4 * v]);
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) deq8_f16((&rb[m][0].x)[v], s2, b2, &o[2 * v]);
        }
        uint4* dst = reinterpret_cast<uint4*>(Bs + (m * TBN + b_n) * TLD + 32 * b_q);
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[v] = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
      }
      __syncthreads();
      if (ks + 1 < nK) gload(ks + 1);
#pragma unroll
      for (int k32 = 0; k32 < TBK / 32; ++k32) {
        const int kof = k32 * 32 + 8 * (lane / 16);
        f16x8_t af[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
          af[i] = *reinterpret_cast<const f16x8_t*>(As + (wm * WM + i * 16 + (lane % 16)) * TLD + kof);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const f16x8_t bfr =
                *reinterpret_cast<const f16x8_t*>(Bs + (m * TBN + wn * WN + j * 16 + (lane % 16)) * TLD + kof);
#pragma unroll
            for (int i = 0; i < MI; ++i)
              acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr, acc[m][i][j], 0, 0, 0);
          }
      }
    }
  }

  // epilogue: C[row = 4*(lane/16) + q][col = lane % 16] of each 16x16 block
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = n0 + wn * WN + j * 16 + (lane % 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = r0 + wm * WM + i * 16 + 4 * (lane / 16) + q;
        if (r < r1 && col < N) {
          float v;
          if (GLU) v = glu(acc[0][i][j][q], acc[NM - 1][i][j][q]);
          else v = acc[0][i][j][q];
          A.out[r * N + col] = f32_to_bf16(v);
        }
      }
    }
}

template <int BITS, int GS, bool GLU, int BM>
static hipError_t launch_t(const TileArgs& a, hipStream_t st) {
  constexpr int NM = GLU ? 2 : 1;
  const int NB = (a.N + TBN - 1) / TBN;
  const size_t lds = (size_t)(BM + NM * TBN) * TLD * 2;
  const int64_t nblk = a.grid_tiles * NB;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((tile_kernel<BITS, GS, GLU, BM>), dim3((unsigned)nblk), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_bm(const TileArgs& a, hipStream_t st) {
  switch (a.bm) {
    case 16: return launch_t<BITS, GS, GLU, 16>(a, st);
    case 32: return launch_t<BITS, GS, GLU, 32>(a, st);
    case 64: return launch_t<BITS, GS, GLU, 64>(a, st);
    case 128: return launch_t<BITS, GS, GLU, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int BITS, bool GLU>
static hipError_t launch_gs(const TileArgs& a, int gs, hipStream_t st) {
  switch (gs) {
    case 32: return launch_bm<BITS, 32, GLU>(a, st);
    case 64: return launch_bm<BITS, 64, GLU>(a, st);
    case 128: return launch_bm<BITS, 128, GLU>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tiles(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st) {
  if (bits == 4) return glu ? launch_gs<4, true>(a, gs, st) : launch_gs<4, false>(a, gs, st);
  if (bits == 8) return glu ? launch_gs<8, true>(a, gs, st) : launch_gs<8, false>(a, gs, st);
  return hipErrorInvalidValue;
}

}  // namespace moegq

// Large row tiles for experts that receive many rows (and for dense
// many-row products): 128 rows x 256 MFMA columns per workgroup.
//
// MLX PR 4567 (Proposed changes): each tile has a row start, one expert and a
// valid-row count, so it runs exactly one K pass over that expert's weights.
// MTPLX PR 558 (Change): the rows are the expert-sorted (token, slot) pairs;
// the gate/up pass gathers x rows through lhs, the down pass reads the sorted
// intermediate rows in order.
//
// gfx950 mapping:
//  * 4 waves in a 2 x 2 grid; a wave owns 64 rows x 128 MFMA columns
//    (4 x 8 blocks of v_mfma_f32_16x16x32_f16, 128 fp32 accumulators), so it
//    reads 0.375 KiB of LDS per MFMA and LDS bandwidth stays below the matrix
//    cores' demand.
//  * GLU: MFMA column blocks alternate gate / up for the same 16 features, so
//    the gate and up results of one (row, feature) meet in one lane and the
//    epilogue applies silu(g) * u without any exchange.
//  * Per K step (64): the activation rows (gathered) and the packed codes are
//    fetched into registers one step ahead; codes are dequantized to fp16
//    (q * s + b with one rounding; nuvec "composed") and the activations
//    converted to fp16, both stored to LDS for v_mfma_f32_16x16x32_f16.
//  * 2 workgroups fit per CU (54 KiB LDS, ~200 registers per lane), so one
//    workgroup's dequant and barriers overlap the other's MFMAs.
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int BG_M = 128;        // rows per tile
constexpr int BG_C = 256;        // MFMA columns per tile
constexpr int BG_K = 64;         // K per step
constexpr int BG_LD = BG_K + 8;  // padded LDS row (fp16 elements)

template <int BITS, int GS, bool GLU>
__global__ __launch_bounds__(256, 2) void tile_big_kernel(TileArgs A) {
  constexpr int NF = GLU ? BG_C / 2 : BG_C;          // output features per tile
  constexpr int CV = BITS * BG_K / 8 / 16;            // uint4 of codes per column per step (2 or 4)
  constexpr int GPS = (BG_K + GS - 1) / GS;           // groups per column per step (1 or 2)
  __shared__ __attribute__((aligned(16))) uint16_t As[BG_M * BG_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BG_C * BG_LD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int N = A.N, K = A.K;
  const int NB = (N + NF - 1) / NF;
  const int64_t tile = blockIdx.x / NB;
  const int n0 = (blockIdx.x % NB) * NF;
  const int Kw = K * BITS / 32, G = K / GS;

  int64_t r0, r1;
  int e;
  if (A.tile_mode == 2) {           // dense rows, one weight matrix
    r0 = tile * BG_M;
    if (r0 >= A.P) return;
    r1 = min(A.P, r0 + BG_M);
    e = 0;
  } else {
    if (tile >= *A.n_tiles) return;
    const int32_t* t = A.tiles + 3 * tile;
    r0 = t[0]; e = t[1]; r1 = r0 + t[2];
  }

  // ---- this thread's roles in the global loads
  // A: row (tid >> 1), 32 bf16 at k offset 32 * (tid & 1)
  const int a_row = tid >> 1, a_half = tid & 1;
  int64_t a_src = -1;
  if (r0 + a_row < r1) {
    const int64_t r = r0 + a_row;
    const int64_t bq = r / A.rows_per_batch;
    const int64_t bx = A.lhs ? (int64_t)A.lhs[bq] : bq / A.lhs_div;
    a_src = bx * A.rows_per_batch + r % A.rows_per_batch;
  }
  // B: MFMA column tid -> (matrix, feature)
  const int bj = tid >> 4, bw = tid & 15;
  const int b_mat = GLU ? (bj & 1) : 0;
  const int b_feat = n0 + (GLU ? (bj >> 1) * 16 + bw : tid);
  const bool b_ok = b_feat < N;
  const int64_t b_row = (int64_t)e * N + (b_ok ? b_feat : 0);
  const uint32_t* wsrc = (b_mat ? A.w1 : A.w0) + b_row * Kw;
  const uint16_t* ssrc = (b_mat ? A.s1 : A.s0) + b_row * G;
  const uint16_t* bsrc = (b_mat ? A.b1 : A.b0) + b_row * G;

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[CV];
  uint16_t rsc[GPS], rbi[GPS];
  auto gload = [&](int ks) {
    const int k0 = ks * BG_K;
    const int ka = k0 + 32 * a_half;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      ra[v] = (a_src >= 0 && ka + 8 * v < K) ? *reinterpret_cast<const uint4*>(A.x + a_src * K + ka + 8 * v)
                                             : make_uint4(0, 0, 0, 0);
    const bool kok = b_ok && k0 < K;
#pragma unroll
    for (int v = 0; v < CV; ++v)
      rb[v] = (kok && k0 + v * (128 / BITS) < K)
                  ? *reinterpret_cast<const uint4*>(wsrc + k0 * BITS / 32 + 4 * v) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int gi = 0; gi < GPS; ++gi) {
      const int g = min((k0 + gi * GS) / GS, G - 1);
      rsc[gi] = kok ? ssrc[g] : (uint16_t)0;
      rbi[gi] = kok ? bsrc[g] : (uint16_t)0;
    }
  };

  const int nK = (K + BG_K - 1) / BG_K;
  gload(0);
  for (int ks = 0; ks < nK; ++ks) {
    __syncthreads();   // the previous step's MFMAs are done with the LDS tiles
    {
      uint4* dst = reinterpret_cast<uint4*>(As + a_row * BG_LD + 32 * a_half);
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v] = act_f16<BITS>(ra[v]);
    }
    {
      // dequantize 64 codes of column tid to fp16
      uint32_t o[32];
      if (BITS == 4) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int gi = min((v * 8) / GS, GPS - 1);   // codes 8v..8v+7
          deq4_f16((&rb[0].x)[v], f16_splat(bf16_to_f32(rsc[gi])), f16_splat(bf16_to_f32(rbi[gi])), &o[4 * v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gi = min((v * 4) / GS, GPS - 1);   // codes 4v..4v+3
          deq8_f16((&rb[0].x)[v], f16_splat(bf16_to_f32(rsc[gi])), f16_splat(bf16_to_f32(rbi[gi])), &o[2 * v]);
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(Bs + tid * BG_LD);
#pragma unroll
      for (int v = 0; v < 8; ++v) dst[v] = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
    }
    __syncthreads();
    if (ks + 1 < nK) gload(ks + 1);
#pragma unroll
    for (int k32 = 0; k32 < BG_K / 32; ++k32) {
      const int kof = k32 * 32 + 8 * (lane >> 4);
      f16x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const f16x8_t*>(As + (wm * 64 + i * 16 + (lane & 15)) * BG_LD + kof);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x8_t bfr = *reinterpret_cast<const f16x8_t*>(Bs + (wn * 128 + j * 16 + (lane & 15)) * BG_LD + kof);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr, acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: acc[i][j][q] = C[row 64 wm + 16 i + 4 (lane >> 4) + q][col 128 wn + 16 j + (lane & 15)]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = r0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
      if (r >= r1) continue;
      if (GLU) {
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const int f = n0 + (wn * 4 + jp) * 16 + (lane & 15);
          if (f < N) A.out[r * N + f] = f32_to_bf16(glu(acc[i][2 * jp][q], acc[i][2 * jp + 1][q]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int f = n0 + wn * 128 + j * 16 + (lane & 15);
          if (f < N) A.out[r * N + f] = f32_to_bf16(acc[i][j][q]);
        }
      }
    }
}

template <int BITS, int GS, bool GLU>
static hipError_t launch_big_t(const TileArgs& a, hipStream_t st) {
  constexpr int NF = GLU ? BG_C / 2 : BG_C;
  const int64_t NB = (a.N + NF - 1) / NF;
  const int64_t nblk = a.grid_tiles * NB;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((tile_big_kernel<BITS, GS, GLU>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tiles_big(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st) {
#define MOEGQ_BG(B, G)                                                                   \
  if (bits == B && gs == G) return glu ? launch_big_t<B, G, true>(a, st) : launch_big_t<B, G, false>(a, st);
  MOEGQ_BG(4, 32) MOEGQ_BG(4, 64) MOEGQ_BG(4, 128) MOEGQ_BG(8, 32) MOEGQ_BG(8, 64) MOEGQ_BG(8, 128)
#undef MOEGQ_BG
  return hipErrorInvalidValue;
}

}  // namespace moegq

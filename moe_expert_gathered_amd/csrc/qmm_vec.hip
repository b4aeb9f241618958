// Vector-unit quantized products for the rest of the operation's surface:
// weights without the transpose (W is [K, N] with its groups along N), and
// float16 / float32 activations in either layout.
//
// nuvec "reference": the product is x . dequant(W)^T, or x . dequant(W)
// without the transpose, in the type that the activation and scale types
// promote to; "quantized_matmul_equals_the_dequantized_product" runs both
// layouts (without the transpose, W's rows are the K axis) and lets half
// precision promote.  With bf16 scales the result is bf16 for bf16
// activations and float32 for float16 or float32 ones.  MLX issue 4509, gq():
// gather_qmm over (lhs, rhs) index pairs; nuvec "gather_qmm_selects_batches".
//
// Arithmetic: fp32 throughout.  For one group g of a weight row,
//   sum_k x_k (q_k s + b) = s * sum_k x_k q_k + b * sum_k x_k,
// the group identity of the affine code (nuvec "composed": codes * s + b).
// Codes become floats with v_cvt_f32_ubyte on masked bytes (exact).
//
// gfx950 mapping.  Every wave is one independent work item: a pair, a block
// of up to MB activation rows, a strip of output columns and a range of K.
// Four waves share a workgroup and nothing else (no LDS, no barriers).
//  * Without the transpose (qvm_kernel): lane l owns WPL consecutive packed
//    words of each weight row k, i.e. 8 * WPL (4-bit) or 4 * WPL (8-bit)
//    consecutive output columns, which lie in one quantization group (the
//    group size is at least 32 and a lane's columns are aligned to their
//    count).  A weight row is a contiguous run of words, so a wave's load of
//    one row is one coalesced 256 B (WPL = 1) or 1 KiB (WPL = 4) access.
//    The activations of 64 consecutive k are loaded one per lane and handed
//    to the whole wave with v_readlane, one value per row step.
//  * With the transpose (qmt_kernel): W is [N, K] with groups along K; lane
//    l owns 2 packed words (16 or 8 codes, one group) of RPW consecutive
//    weight rows and the matching activations; the wave walks K in slices
//    of 128 words and finishes with a butterfly over its 64 lanes.
//  * K is split over KS work items when the pairs, rows and columns alone
//    give too few waves; each split writes fp32 partial sums to the
//    workspace and vec_reduce_kernel adds the KS partials in split order and
//    rounds once (to bf16 or float32), so results do not depend on timing.
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr uint32_t kVecNoFetch = 0x7FFFFFF0u;   // beyond every descriptor's range: loads return 0

// activation element i of a row (type XT: 0 bf16, 1 float16, 2 float32)
template <int XT>
MOEGQ_DEV float act_at(const void* x, int64_t i) {
  if constexpr (XT == 0) return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
  else if constexpr (XT == 1) return (float)static_cast<const _Float16*>(x)[i];
  else return static_cast<const float*>(x)[i];
}

// code j (0..32/BITS-1) of a packed word as a float; lo = w & 0x0F0F0F0F and
// hi = (w >> 4) & 0x0F0F0F0F hold the even and odd 4-bit codes as bytes.  A
// byte extraction followed by the conversion is one v_cvt_f32_ubyteN.
template <int BITS>
MOEGQ_DEV float code_f(uint32_t w, uint32_t lo, uint32_t hi, int j) {
  if constexpr (BITS == 4) {
    const uint32_t src = (j & 1) ? hi : lo;
    return (float)((src >> (8 * (j >> 1))) & 0xFFu);
  } else {
    return (float)((w >> (8 * j)) & 0xFFu);
  }
}

// n (a multiple of 4) consecutive activations from element i (16-byte aligned
// for the wider types) as floats
template <int XT, int NV>
MOEGQ_DEV void load_acts(const void* x, int64_t i, float (&v)[NV]) {
  static_assert(NV % 4 == 0, "");
  if constexpr (XT == 2) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
      const float4 t = p[j];
      v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
  } else {
    const uint2* p = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + i);
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
      const uint2 t = p[j];
      const uint32_t d[2] = {t.x, t.y};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t half = (d[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
        if constexpr (XT == 0) v[4 * j + h] = __uint_as_float(half << 16);
        else v[4 * j + h] = (float)__builtin_bit_cast(_Float16, (uint16_t)half);
      }
    }
  }
}

MOEGQ_DEV void store_result(void* out, int out_f32, int64_t i, float v) {
  if (out_f32) static_cast<float*>(out)[i] = v;
  else static_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
}

// work item of wave `item`: split ks fastest, then column strip / row block,
// row block of the activations, pair
struct VecItem { int64_t p; int mb, cs, ks; };
MOEGQ_DEV VecItem vec_item(const VecArgs& A, int64_t item) {
  VecItem it;
  it.ks = (int)(item % A.KS); item /= A.KS;
  it.cs = (int)(item % A.NC); item /= A.NC;
  it.mb = (int)(item % A.MBLK);
  it.p = item / A.MBLK;
  return it;
}

// ---------------------------------------------------------------- without the transpose
template <int BITS, int XT, int MB, int WPL>
__global__ __launch_bounds__(256) void qvm_kernel(VecArgs A) {
  constexpr int CPW = 32 / BITS;        // codes per word
  constexpr int CPL = CPW * WPL;        // output columns per lane
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  if (item >= A.items) return;                       // whole waves leave together
  const VecItem it = vec_item(A, item);
  const int K = A.K, N = A.N, M = A.M;
  const int Nw = N / CPW, G = N / A.gs;
  const int64_t xb = A.lhs ? (int64_t)A.lhs[it.p] : it.p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[it.p] : 0;
  const int w0 = (it.cs * 64 + lane) * WPL;          // first word of the lane's columns
  const bool act = w0 < Nw;
  const int col0 = w0 * CPW;
  const uint32_t g2 = act ? (uint32_t)(col0 / A.gs) * 2 : kVecNoFetch;
  const uint32_t wo = act ? (uint32_t)w0 * 4 : kVecNoFetch;
  const int k0 = it.ks * A.kchunk;
  const int k1 = min(K, k0 + A.kchunk);
  const int m0 = it.mb * MB;
  const int nm = min(MB, M - m0);

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(A.w + e * (int64_t)K * Nw, (uint32_t)((int64_t)K * Nw * 4));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(A.s + e * (int64_t)K * G, (uint32_t)((int64_t)K * G * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(A.b + e * (int64_t)K * G, (uint32_t)((int64_t)K * G * 2));
  const int64_t xrow0 = (xb * M + m0) * (int64_t)K;

  float acc[MB][CPL], bacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    bacc[m] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[m][c] = 0.f;
  }
  constexpr int U = 4;   // weight rows in flight per step
  for (int kb = k0; kb < k1; kb += 64) {
    const int kn = min(64, k1 - kb);
    float xl[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
      xl[m] = (lane < kn && m < nm) ? act_at<XT>(A.x, xrow0 + (int64_t)m * K + kb + lane) : 0.f;
    for (int j = 0; j < kn; j += U) {
      uint32_t cw[U][WPL];
      uint16_t sv[U], bv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = j + u < kn;                   // uniform
        const uint32_t row = (uint32_t)(kb + j + u);
        const uint32_t off = ok ? wo : kVecNoFetch;
        if constexpr (WPL == 4) {
          const uint4 v = buf_load16(rw, off, ok ? row * Nw * 4 : 0);
          cw[u][0] = v.x; cw[u][1] = v.y; cw[u][2] = v.z; cw[u][3] = v.w;
        } else {
          cw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, off, ok ? row * Nw * 4 : 0, 0);
        }
        sv[u] = buf_load2(rs, ok ? g2 : kVecNoFetch, ok ? row * G * 2 : 0);
        bv[u] = buf_load2(rb, ok ? g2 : kVecNoFetch, ok ? row * G * 2 : 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u >= kn) break;                       // uniform
        const float s = bf16_to_f32(sv[u]), b = bf16_to_f32(bv[u]);
        float xs[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float xm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xl[m]), j + u));
          xs[m] = xm * s;
          bacc[m] = fmaf(xm, b, bacc[m]);
        }
#pragma unroll
        for (int wi = 0; wi < WPL; ++wi) {
          const uint32_t w = cw[u][wi];
          const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
          for (int jj = 0; jj < CPW; ++jj) {
            const float q = code_f<BITS>(w, lo, hi, jj);
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[m][wi * CPW + jj] = fmaf(xs[m], q, acc[m][wi * CPW + jj]);
          }
        }
      }
    }
  }
  if (!act) return;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= nm) break;
    const int64_t orow = (it.p * M + m0 + m) * (int64_t)N + col0;   // a multiple of 4
    float v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = acc[m][c] + bacc[m];
    if (A.KS > 1 || A.out_f32) {
      float* dst = A.KS > 1 ? A.part + (int64_t)it.ks * A.P * M * N + orow : static_cast<float*>(A.out) + orow;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) *reinterpret_cast<float4*>(dst + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
    } else {
      uint16_t* dst = static_cast<uint16_t*>(A.out) + orow;
#pragma unroll
      for (int c = 0; c < CPL; c += 4)
        *reinterpret_cast<uint2*>(dst + c) = make_uint2(pack_bf16x2(v[c], v[c + 1]), pack_bf16x2(v[c + 2], v[c + 3]));
    }
  }
}

// ---------------------------------------------------------------- with the transpose
template <int V>
MOEGQ_DEV void wave_sum(float (&a)[V]) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < V; ++i) a[i] += __shfl_xor(a[i], off, 64);
}

template <int BITS, int XT, int MB, int RPW>
__global__ __launch_bounds__(256) void qmt_kernel(VecArgs A) {
  constexpr int CPW = 32 / BITS;
  constexpr int CPL = 2 * CPW;          // codes per lane per slice (two words)
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  if (item >= A.items) return;
  const VecItem it = vec_item(A, item);
  const int K = A.K, N = A.N, M = A.M;
  const int Kw = K / CPW, G = K / A.gs;
  const int64_t xb = A.lhs ? (int64_t)A.lhs[it.p] : it.p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[it.p] : 0;
  const int n0 = it.cs * RPW;
  const int kw0 = it.ks * A.kchunk;                  // in words
  const int kw1 = min(Kw, kw0 + A.kchunk);
  const int m0 = it.mb * MB;
  const int nm = min(MB, M - m0);

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(A.w + e * (int64_t)N * Kw, (uint32_t)((int64_t)N * Kw * 4));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(A.s + e * (int64_t)N * G, (uint32_t)((int64_t)N * G * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(A.b + e * (int64_t)N * G, (uint32_t)((int64_t)N * G * 2));
  const int64_t xrow0 = (xb * M + m0) * (int64_t)K;

  float acc[MB * RPW];
#pragma unroll
  for (int i = 0; i < MB * RPW; ++i) acc[i] = 0.f;
  for (int sw = kw0; sw < kw1; sw += 128) {
    const int wi = sw + 2 * lane;
    const bool ok = wi < kw1;
    const int kc = wi * CPW;                          // first code of the lane
    const uint32_t g2 = ok ? (uint32_t)(kc / A.gs) * 2 : kVecNoFetch;
    uint2 cw[RPW];
    uint16_t sv[RPW], bv[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const bool rok = ok && n0 + r < N;
      const uint32_t row = (uint32_t)min(n0 + r, N - 1);
      const uint32_t off = rok ? (uint32_t)wi * 4 : kVecNoFetch;
      cw[r].x = __builtin_amdgcn_raw_buffer_load_b32(rw, off, row * Kw * 4, 0);
      cw[r].y = __builtin_amdgcn_raw_buffer_load_b32(rw, rok ? off + 4 : kVecNoFetch, row * Kw * 4, 0);
      sv[r] = buf_load2(rs, rok ? g2 : kVecNoFetch, row * G * 2);
      bv[r] = buf_load2(rb, rok ? g2 : kVecNoFetch, row * G * 2);
    }
    float xv[MB][CPL], sx[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (ok && m < nm) {
        load_acts<XT>(A.x, xrow0 + (int64_t)m * K + kc, xv[m]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) xv[m][c] = 0.f;
      }
      sx[m] = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) sx[m] += xv[m][c];
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float d[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) d[m] = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? cw[r].y : cw[r].x;
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj) {
          const float q = code_f<BITS>(w, lo, hi, jj);
#pragma unroll
          for (int m = 0; m < MB; ++m) d[m] = fmaf(xv[m][h * CPW + jj], q, d[m]);
        }
      }
      const float s = bf16_to_f32(sv[r]), b = bf16_to_f32(bv[r]);
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[m * RPW + r] = fmaf(s, d[m], fmaf(b, sx[m], acc[m * RPW + r]));
    }
  }
  wave_sum(acc);
  if (lane != 0) return;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= nm) break;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (n0 + r >= N) break;
      const int64_t o = (it.p * M + m0 + m) * (int64_t)N + n0 + r;
      if (A.KS > 1) A.part[(int64_t)it.ks * A.P * M * N + o] = acc[m * RPW + r];
      else store_result(A.out, A.out_f32, o, acc[m * RPW + r]);
    }
  }
}

// out[i] = round(sum_{ks < KS} part[ks][i]), the splits added in order
__global__ __launch_bounds__(256) void vec_reduce_kernel(const float* __restrict__ part, int KS, int64_t total,
                                                         void* out, int out_f32) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    float v = part[i];
    for (int k = 1; k < KS; ++k) v += part[(int64_t)k * total + i];
    store_result(out, out_f32, i, v);
  }
}

// ---------------------------------------------------------------- host side
constexpr int64_t kVecWaves = 4096;                 // waves the split aims for
constexpr int64_t kVecPartMax = (int64_t)1 << 26;   // bytes of partial sums at most

VecPlan vec_plan(int64_t P, int64_t M, int64_t N, int64_t K, int bits, int transpose) {
  VecPlan pl{};
  const int cpw = 32 / bits;
  pl.MB = M >= 3 ? 4 : (int)M;
  pl.MBLK = (M + pl.MB - 1) / pl.MB;
  int64_t steps;                 // units of K a split can take
  if (!transpose) {
    const int64_t Nw = N / cpw;
    pl.WPL = Nw >= 256 ? 4 : 1;
    pl.NC = (Nw + 64 * pl.WPL - 1) / (64 * pl.WPL);
    steps = (K + 15) / 16;                           // at least 16 weight rows per split
  } else {
    pl.WPL = 2;
    pl.NC = (N + kQmtRows - 1) / kQmtRows;
    steps = (K / cpw + 127) / 128;                   // 128-word slices
  }
  const int64_t items0 = P * pl.MBLK * pl.NC;
  int64_t ks = (kVecWaves + items0 - 1) / items0;
  if (ks > steps) ks = steps;
  const int64_t out_elems = P * M * N;
  const int64_t ks_cap = kVecPartMax / (out_elems * 4);
  if (ks > ks_cap) ks = ks_cap;
  if (ks < 1) ks = 1;
  const int64_t per = (steps + ks - 1) / ks;         // steps per split
  pl.kchunk = (int)(transpose ? per * 128 : per * 16);
  const int64_t kunits = transpose ? K / cpw : K;
  pl.KS = (int)((kunits + pl.kchunk - 1) / pl.kchunk);
  pl.items = items0 * pl.KS;
  pl.part_bytes = pl.KS > 1 ? (size_t)(pl.KS * out_elems * 4) : 0;
  return pl;
}

template <int BITS, int XT>
static hipError_t launch_vec_t(const VecArgs& a, int transpose, hipStream_t st) {
  const dim3 grid((unsigned)((a.items + 3) / 4)), block(256);
  if (!transpose) {
#define MOEGQ_QVM(RB, WL) \
  if (a.MB == RB && a.WPL == WL) { hipLaunchKernelGGL((qvm_kernel<BITS, XT, RB, WL>), grid, block, 0, st, a); return hipGetLastError(); }
    MOEGQ_QVM(1, 1) MOEGQ_QVM(2, 1) MOEGQ_QVM(4, 1) MOEGQ_QVM(1, 4) MOEGQ_QVM(2, 4) MOEGQ_QVM(4, 4)
#undef MOEGQ_QVM
  } else {
#define MOEGQ_QMT(RB) \
  if (a.MB == RB) { hipLaunchKernelGGL((qmt_kernel<BITS, XT, RB, kQmtRows>), grid, block, 0, st, a); return hipGetLastError(); }
    MOEGQ_QMT(1) MOEGQ_QMT(2) MOEGQ_QMT(4)
#undef MOEGQ_QMT
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qmm_vec(const VecArgs& a, int bits, int transpose, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  if ((a.items + 3) / 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  if (bits == 4) {
    if (a.x_type == 0) e = launch_vec_t<4, 0>(a, transpose, st);
    else if (a.x_type == 1) e = launch_vec_t<4, 1>(a, transpose, st);
    else if (a.x_type == 2) e = launch_vec_t<4, 2>(a, transpose, st);
  } else if (bits == 8) {
    if (a.x_type == 0) e = launch_vec_t<8, 0>(a, transpose, st);
    else if (a.x_type == 1) e = launch_vec_t<8, 1>(a, transpose, st);
    else if (a.x_type == 2) e = launch_vec_t<8, 2>(a, transpose, st);
  }
  if (e != hipSuccess || a.KS <= 1) return e;
  const int64_t total = a.P * a.M * (int64_t)a.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(vec_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.part, a.KS, total, a.out,
                     a.out_f32);
  return hipGetLastError();
}

}  // namespace moegq

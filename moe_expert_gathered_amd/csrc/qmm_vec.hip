// Vector-unit quantized products for the rest of the operation's surface:
// weights without the transpose (W is [K, N] with its groups along N),
// float16 / float32 activations in either layout, and the bit widths 1, 2, 3,
// 5 and 6 next to 4 and 8.
//
// nuvec "reference": the product is x . dequant(W)^T, or x . dequant(W)
// without the transpose, in the type that the activation and scale types
// promote to; "quantized_matmul_equals_the_dequantized_product" runs both
// layouts (without the transpose, W's rows are the K axis), the widths
// 1-6 and 8, and lets half precision promote.  With bf16 scales the result is
// bf16 for bf16 activations and float32 for float16 or float32 ones.  Code k
// of a packed row occupies bits [k b, k b + b) of the row's little-endian word
// stream, so 3-, 5- and 6-bit codes straddle words.  MLX issue 4509, gq():
// gather_qmm over (lhs, rhs) index pairs; nuvec "gather_qmm_selects_batches".
//
// The mx modes (MLX PR 4787 benchmark script: mode "mxfp4" / "mxfp8", no
// biases) read their elements as E2M1 / E4M3 floats, 32 per block along the
// packed axis, each block scaled by an E8M0 power of two (the OCP
// Microscaling encoding): the gfx950 conversions v_cvt_scalef32_pk_f32_fp4 /
// _fp8 turn two elements into fp32 per instruction, and the block scale
// multiplies the block's dot product.
//
// Arithmetic: fp32 throughout.  For one group g of a weight row,
//   sum_k x_k (q_k s + b) = s * sum_k x_k q_k + b * sum_k x_k,
// the group identity of the affine code (nuvec "composed": codes * s + b).
// Codes become floats exactly (byte or bit-field extraction, then a convert).
//
// gfx950 mapping.  A lane owns a chunk of CH consecutive codes of a weight
// row: CH * b / 32 whole words, all in one quantization group (CH divides 32
// and the group size is at least 32).  CH is 32 for every width (b words), or
// 8 (4-bit) / 4 (8-bit) for narrow rows.
//  * Without the transpose (qvm_kernel): the chunk is CH output columns of
//    weight row k.  One workgroup per work item (a pair, a block of up to MB
//    activation rows, a strip of 64 CH columns, a range of K); its 4 waves take
//    the rows k0 + w, k0 + w + 4, .. (the workgroup streams a contiguous run of
//    rows), U rows in flight per wave with the activations of those rows (one
//    per lane, handed to the wave with v_readlane), and add their sums through
//    LDS at the end.
//  * With the transpose (qmt_kernel): the chunk is 32 codes of K of RPW
//    consecutive weight rows; each wave is a work item and walks K in slices
//    of 64 chunks, loading the next slice before the current one's arithmetic,
//    and ends with a butterfly over its lanes.
//  * K is split over KS work items when the pairs, rows and columns alone
//    give too few; each split writes fp32 partial sums to the workspace and
//    vec_reduce_kernel adds the KS partials in split order and rounds once
//    (to bf16 or float32), so results do not depend on timing.
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr uint32_t kVecNoFetch = 0x7FFFFFF0u;   // beyond every descriptor's range: loads return 0

// NW consecutive 32-bit words at byte offset voff + soff (4-byte aligned)
template <int NW>
MOEGQ_DEV void load_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t (&w)[NW]) {
  int i = 0;
#pragma unroll
  for (; i + 4 <= NW; i += 4) {
    const uint4 v = buf_load16(r, voff == kVecNoFetch ? voff : voff + 4 * i, soff);
    w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
  }
  if constexpr (NW % 4 >= 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff == kVecNoFetch ? voff : voff + 4 * (NW / 4) * 4,
                                                        soff, 0);
    w[(NW / 4) * 4] = v[0]; w[(NW / 4) * 4 + 1] = v[1];
  }
  if constexpr (NW % 2 == 1)
    w[NW - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, voff == kVecNoFetch ? voff : voff + 4 * (NW - 1), soff, 0);
}

// The CH codes of a chunk as floats.  4-bit: w & 0x0F0F0F0F and
// (w >> 4) & 0x0F0F0F0F hold the even and odd codes as bytes; 8-bit: the bytes;
// other widths: a funnel shift across the word boundary, then a mask.  A byte
// extraction followed by the conversion is one v_cvt_f32_ubyteN.
template <int BITS, int CH>
MOEGQ_DEV void codes_f(const uint32_t (&w)[CH * BITS / 32], float (&q)[CH]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q[8 * i + 2 * j] = (float)((lo >> (8 * j)) & 0xFFu);
        q[8 * i + 2 * j + 1] = (float)((hi >> (8 * j)) & 0xFFu);
      }
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < CH / 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) q[4 * i + j] = (float)((w[i] >> (8 * j)) & 0xFFu);
  } else {
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int o = j * BITS, wi = o >> 5, sh = o & 31;
      uint32_t v;
      if (sh + BITS <= 32) v = w[wi] >> sh;
      else v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], (uint32_t)sh);
      q[j] = (float)(v & mask);
    }
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The CH elements of a chunk as floats, by mode: 0 the affine codes, 1 E2M1
// (code k in the nibble at bit 4k, two per byte), 2 E4M3 (one per byte).
template <int BITS, int CH, int MODE>
MOEGQ_DEV void elems_f(const uint32_t (&w)[CH * BITS / 32], float (&q)[CH]) {
  if constexpr (MODE == 0) {
    codes_f<BITS, CH>(w, q);
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
      const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
      const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
      q[8 * i] = a.x; q[8 * i + 1] = a.y; q[8 * i + 2] = b.x; q[8 * i + 3] = b.y;
      q[8 * i + 4] = c.x; q[8 * i + 5] = c.y; q[8 * i + 6] = d.x; q[8 * i + 7] = d.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, false);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, true);
      q[4 * i] = a.x; q[4 * i + 1] = a.y; q[4 * i + 2] = b.x; q[4 * i + 3] = b.y;
    }
  }
}

// E8M0 block scale: 2^(e - 127) as an fp32 (e = 0 gives the subnormal 2^-127,
// e = 255 NaN)
MOEGQ_DEV float e8m0_f32(uint32_t e) {
  if (e == 255u) return __uint_as_float(0x7FC00000u);
  return e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// scale (and bias) loads: bf16 per group, or one byte per mx block
template <int MODE>
MOEGQ_DEV uint16_t load_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (MODE == 0) return buf_load2(r, voff, soff);
  else return (uint16_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
template <int MODE>
MOEGQ_DEV float scale_f(uint16_t v) {
  if constexpr (MODE == 0) return bf16_to_f32(v);
  else return e8m0_f32(v);
}

// NV (a multiple of 8) consecutive activations at byte offset `off` of the
// row descriptor r, as floats; an offset past the range gives zeros
template <int XT, int NV>
MOEGQ_DEV void load_acts(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[NV]) {
  static_assert(NV % 8 == 0, "");
  if constexpr (XT == 2) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
      const uint4 t = buf_load16(r, off == kVecNoFetch ? off : off + 16 * j, 0);
      v[4 * j] = __uint_as_float(t.x); v[4 * j + 1] = __uint_as_float(t.y);
      v[4 * j + 2] = __uint_as_float(t.z); v[4 * j + 3] = __uint_as_float(t.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV / 8; ++j) {
      const uint4 t = buf_load16(r, off == kVecNoFetch ? off : off + 16 * j, 0);
      const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t half = (d[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
        if constexpr (XT == 0) v[8 * j + h] = __uint_as_float(half << 16);
        else v[8 * j + h] = (float)__builtin_bit_cast(_Float16, (uint16_t)half);
      }
    }
  }
}

MOEGQ_DEV void store_result(void* out, int out_f32, int64_t i, float v) {
  if (out_f32) static_cast<float*>(out)[i] = v;
  else static_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
}

// work item `item`: split ks, column strip (row block) cs, block mb of the
// activation rows, pair p; `cs_fast` puts the strip first (neighbouring
// waves then read the same activations), else the split
struct VecItem { int64_t p; int mb, cs, ks; };
MOEGQ_DEV VecItem vec_item(const VecArgs& A, int64_t item, bool cs_fast) {
  VecItem it;
  if (cs_fast) {
    it.cs = (int)(item % A.NC); item /= A.NC;
    it.ks = (int)(item % A.KS); item /= A.KS;
  } else {
    it.ks = (int)(item % A.KS); item /= A.KS;
    it.cs = (int)(item % A.NC); item /= A.NC;
  }
  it.mb = (int)(item % A.MBLK);
  it.p = item / A.MBLK;
  return it;
}

// ---------------------------------------------------------------- without the transpose
template <int BITS, int XT, int MB, int CH, int U, int MODE>
__global__ __launch_bounds__(256) void qvm_kernel(VecArgs A) {
  constexpr bool MX = MODE != 0;        // mx block scales: one byte per 32 columns, no biases
  constexpr int SSZ = MX ? 1 : 2;
  constexpr int NW = CH * BITS / 32;    // words per lane per row
  __shared__ float red[3][CH][64];      // waves 1..3, one activation row at a time
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t item = blockIdx.x;
  if (item >= A.items) return;                       // the whole workgroup leaves
  const VecItem it = vec_item(A, item, false);
  const int K = A.K, N = A.N, M = A.M;
  const int Nw = N / 32 * BITS, G = N / (MX ? 32 : A.gs);   // N is a multiple of 32
  const int64_t xb = A.lhs ? (int64_t)A.lhs[it.p] : it.p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[it.p] : 0;
  const int col0 = (it.cs * 64 + lane) * CH;         // first of the lane's columns
  const bool act = col0 < N;
  const uint32_t g2 = act ? (uint32_t)(col0 / (MX ? 32 : A.gs)) * SSZ : kVecNoFetch;
  const uint32_t wo = act ? (uint32_t)(col0 * BITS / 32) * 4 : kVecNoFetch;   // CH * BITS is a multiple of 32
  const int k0 = it.ks * A.kchunk;
  const int k1 = min(K, k0 + A.kchunk);
  const int m0 = it.mb * MB;
  const int nm = min(MB, M - m0);
  const int kw = k0 + wave;                          // the wave's first row; its rows step by 4
  const int nr = k1 > kw ? (k1 - kw + 3) / 4 : 0;    // rows of this wave

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(A.w + e * (int64_t)K * Nw, (uint32_t)((int64_t)K * Nw * 4));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char*>(A.s) + e * (int64_t)K * G * SSZ,
                                              (uint32_t)((int64_t)K * G * SSZ));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(MX ? A.s : A.b + e * (int64_t)K * G, MX ? 0u : (uint32_t)((int64_t)K * G * 2));
  const int64_t xrow0 = (xb * M + m0) * (int64_t)K;
  constexpr int XSZ = XT == 2 ? 4 : 2;
  __amdgpu_buffer_rsrc_t rx[MB];                      // one descriptor per activation row (empty past M)
#pragma unroll
  for (int m = 0; m < MB; ++m)
    rx[m] = make_rsrc(static_cast<const char*>(A.x) + (xrow0 + (int64_t)(m < nm ? m : 0) * K) * XSZ,
                      m < nm ? (uint32_t)K * XSZ : 0u);

  float acc[MB][CH], bacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    bacc[m] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[m][c] = 0.f;
  }
  for (int j = 0; j < nr; j += U) {
    uint32_t cw[U][NW];
    uint16_t sv[U], bv[U];
    // lane u < U: the activations of the batch's row u
    float xl[MB];
    {
      const bool xok = lane < U && j + lane < nr;
      const uint32_t xo = xok ? (uint32_t)(kw + 4 * (j + lane)) * XSZ : kVecNoFetch;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if constexpr (XT == 2) xl[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx[m], xo, 0, 0));
        else {
          const uint16_t h = buf_load2(rx[m], xo, 0);
          xl[m] = XT == 0 ? bf16_to_f32(h) : (float)__builtin_bit_cast(_Float16, h);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = j + u < nr;                     // uniform
      const uint32_t row = ok ? (uint32_t)(kw + 4 * (j + u)) : 0u;
      load_words<NW>(rw, ok ? wo : kVecNoFetch, row * Nw * 4, cw[u]);
      sv[u] = load_scale<MODE>(rs, ok ? g2 : kVecNoFetch, row * G * SSZ);
      bv[u] = MX ? (uint16_t)0 : buf_load2(rb, ok ? g2 : kVecNoFetch, row * G * 2);
    }
    // rows past nr loaded zeros (codes, scale, bias) and their activation
    // lanes hold zero: they add nothing, and no branch separates the loads
    // above from the arithmetic below
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // rows past nr: scale byte 0 (2^-127) times zero elements and zero activations
      const float s = scale_f<MODE>(sv[u]), b = bf16_to_f32(bv[u]);
      float xs[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float xm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xl[m]), u));
        xs[m] = xm * s;
        if constexpr (!MX) bacc[m] = fmaf(xm, b, bacc[m]);
      }
      float q[CH];
      elems_f<BITS, CH, MODE>(cw[u], q);
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m][c] = fmaf(xs[m], q[c], acc[m][c]);
    }
  }
  // wave 0 adds the sums of waves 1, 2, 3 (in that order) and writes
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= nm) break;                               // uniform over the workgroup
    float v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = acc[m][c] + bacc[m];
    if (wave > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) red[wave - 1][c][lane] = v[c];
    }
    __syncthreads();
    if (wave == 0 && act) {
#pragma unroll
      for (int c = 0; c < CH; ++c) v[c] = ((v[c] + red[0][c][lane]) + red[1][c][lane]) + red[2][c][lane];
      const int64_t orow = (it.p * M + m0 + m) * (int64_t)N + col0;   // a multiple of 4
      if (A.KS > 1 || A.out_f32) {
        float* dst = A.KS > 1 ? A.part + (int64_t)it.ks * A.P * M * N + orow : static_cast<float*>(A.out) + orow;
#pragma unroll
        for (int c = 0; c < CH; c += 4) *reinterpret_cast<float4*>(dst + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
      } else {
        uint16_t* dst = static_cast<uint16_t*>(A.out) + orow;
#pragma unroll
        for (int c = 0; c < CH; c += 4)
          *reinterpret_cast<uint2*>(dst + c) = make_uint2(pack_bf16x2(v[c], v[c + 1]), pack_bf16x2(v[c + 2], v[c + 3]));
      }
    }
    __syncthreads();
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

// one slice (64 chunks of 32 codes) of RPW weight rows and the activations
template <int BITS, int MB, int RPW>
struct QmtSlice {
  uint32_t c[RPW][BITS];
  uint16_t s[RPW], b[RPW];
  float x[MB][32];
};

template <int BITS, int XT, int MB, int RPW, int MODE>
__global__ __launch_bounds__(256) void qmt_kernel(VecArgs A) {
  using Slice = QmtSlice<BITS, MB, RPW>;
  constexpr bool MX = MODE != 0;        // mx block scales: one byte per 32 codes, no biases
  constexpr int SSZ = MX ? 1 : 2;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  if (item >= A.items) return;                       // whole waves leave together
  const VecItem it = vec_item(A, item, true);
  const int K = A.K, N = A.N, M = A.M;
  const int Kw = K / 32 * BITS, G = K / (MX ? 32 : A.gs);   // K is a multiple of 32
  const int64_t xb = A.lhs ? (int64_t)A.lhs[it.p] : it.p / A.lhs_div;
  const int64_t e = A.rhs ? (int64_t)A.rhs[it.p] : 0;
  const int n0 = it.cs * RPW;
  const int kc0 = it.ks * A.kchunk;                  // in codes (a multiple of 2048)
  const int kc1 = min(K, kc0 + A.kchunk);
  const int m0 = it.mb * MB;
  const int nm = min(MB, M - m0);

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(A.w + e * (int64_t)N * Kw, (uint32_t)((int64_t)N * Kw * 4));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char*>(A.s) + e * (int64_t)N * G * SSZ,
                                              (uint32_t)((int64_t)N * G * SSZ));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(MX ? A.s : A.b + e * (int64_t)N * G, MX ? 0u : (uint32_t)((int64_t)N * G * 2));
  constexpr int XSZ = XT == 2 ? 4 : 2;
  __amdgpu_buffer_rsrc_t rx[MB];                      // one descriptor per activation row (empty past M)
#pragma unroll
  for (int m = 0; m < MB; ++m)
    rx[m] = make_rsrc(static_cast<const char*>(A.x) + ((xb * M + m0 + (m < nm ? m : 0)) * (int64_t)K) * XSZ,
                      m < nm ? (uint32_t)K * XSZ : 0u);

  auto load = [&](int sc, Slice& S) {
    const int kc = sc + 32 * lane;                    // the lane's first code
    const bool ok = kc < kc1;                         // kc1 is a multiple of 32
    const uint32_t g2 = ok ? (uint32_t)(kc / (MX ? 32 : A.gs)) * SSZ : kVecNoFetch;
    const uint32_t wo = ok ? (uint32_t)(kc / 32 * BITS) * 4 : kVecNoFetch;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const bool rok = ok && n0 + r < N;
      const uint32_t row = (uint32_t)min(n0 + r, N - 1);
      load_words<BITS>(rw, rok ? wo : kVecNoFetch, row * Kw * 4, S.c[r]);
      S.s[r] = load_scale<MODE>(rs, rok ? g2 : kVecNoFetch, row * G * SSZ);
      S.b[r] = MX ? (uint16_t)0 : buf_load2(rb, rok ? g2 : kVecNoFetch, row * G * 2);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) load_acts<XT>(rx[m], ok ? (uint32_t)kc * XSZ : kVecNoFetch, S.x[m]);
  };

  float acc[MB * RPW];
#pragma unroll
  for (int i = 0; i < MB * RPW; ++i) acc[i] = 0.f;
  auto compute = [&](const Slice& S) {
    float sx[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      sx[m] = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) sx[m] += S.x[m][c];
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float q[32];
      elems_f<BITS, 32, MODE>(S.c[r], q);
      float d[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) d[m] = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c)
#pragma unroll
        for (int m = 0; m < MB; ++m) d[m] = fmaf(S.x[m][c], q[c], d[m]);
      const float s = scale_f<MODE>(S.s[r]), b = bf16_to_f32(S.b[r]);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if constexpr (MX) acc[m * RPW + r] = fmaf(s, d[m], acc[m * RPW + r]);
        else acc[m * RPW + r] = fmaf(s, d[m], fmaf(b, sx[m], acc[m * RPW + r]));
      }
    }
  };

  // the slice after the last one loads zeros (offsets past kc1) without a branch
  Slice cur, nxt;
  load(kc0, cur);
  for (int sc = kc0; sc < kc1; sc += 2048) {
    load(sc + 2048, nxt);
    compute(cur);
    cur = nxt;
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

// out[i] = round(sum_{ks < KS} part[ks][i]), the splits added in order.  KS is
// at most kVecMaxSplits: every partial of an output is requested before the
// first is added (one memory latency, not KS of them).  One wave per
// workgroup, so that the requests spread over every CU.
constexpr int kVecMaxSplits = 64;
__global__ __launch_bounds__(64) void vec_reduce_kernel(const float* __restrict__ part, int KS, int64_t total,
                                                        void* out, int out_f32) {
  const int64_t stride = (int64_t)gridDim.x * 64;
  for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < total; i += stride) {
    float t[kVecMaxSplits];
#pragma unroll
    for (int k = 0; k < kVecMaxSplits; ++k) t[k] = k < KS ? part[(int64_t)k * total + i] : -0.f;
    float v = t[0];
#pragma unroll
    for (int k = 1; k < kVecMaxSplits; ++k) v += t[k];   // -0 past KS: the additive identity
    store_result(out, out_f32, i, v);
  }
}

// ---------------------------------------------------------------- host side
constexpr int64_t kVecWaves = 4096;                 // waves the split aims for (half that with the transpose)
constexpr int64_t kVecPartMax = (int64_t)1 << 26;   // bytes of partial sums at most

static int qmt_rows(int bits) { return bits <= 4 ? 8 : 4; }

VecPlan vec_plan(int64_t P, int64_t M, int64_t N, int64_t K, int bits, int transpose, int mode) {
  VecPlan pl{};
  int64_t items0, steps, target;
  if (!transpose) {
    // workgroup items; a split takes at least 64 weight rows (16 per wave)
    pl.MB = M >= 3 ? 4 : (int)M;
    // codes per lane: 32, or one word (4-bit, 8-bit) when the row is narrow
    pl.WPL = (mode == 0 && (bits == 4 || bits == 8) && N < 2048) ? 32 / bits : 32;
    pl.NC = (N + 64 * pl.WPL - 1) / (64 * pl.WPL);
    steps = (K + 63) / 64;
    target = kVecWaves / 4;
  } else {
    // wave items; a split takes whole slices of 2048 codes
    pl.MB = M >= 2 ? 2 : 1;
    pl.WPL = 32;
    pl.NC = (N + qmt_rows(bits) - 1) / qmt_rows(bits);
    steps = (K + 2047) / 2048;
    target = kVecWaves / 2;
  }
  pl.MBLK = (M + pl.MB - 1) / pl.MB;
  items0 = P * pl.MBLK * pl.NC;
  int64_t ks = (target + items0 - 1) / items0;
  if (ks > steps) ks = steps;
  const int64_t out_elems = P * M * N;
  const int64_t ks_cap = kVecPartMax / (out_elems * 4);
  if (ks > ks_cap) ks = ks_cap;
  if (ks > kVecMaxSplits) ks = kVecMaxSplits;
  if (ks < 1) ks = 1;
  const int64_t per = (steps + ks - 1) / ks;         // steps per split
  pl.kchunk = (int)(transpose ? per * 2048 : per * 64);
  pl.KS = (int)((K + pl.kchunk - 1) / pl.kchunk);
  pl.items = items0 * pl.KS;
  pl.part_bytes = pl.KS > 1 ? (size_t)(pl.KS * out_elems * 4) : 0;
  return pl;
}

template <int BITS, int XT, int MODE>
static hipError_t launch_vec_t(const VecArgs& a, int transpose, hipStream_t st) {
  const dim3 block(256);
  if (!transpose) {
    const dim3 grid((unsigned)a.items);                       // one workgroup per item
#define MOEGQ_QVM(RB, CC, UU) \
  if (a.MB == RB && a.WPL == CC) { hipLaunchKernelGGL((qvm_kernel<BITS, XT, RB, CC, UU, MODE>), grid, block, 0, st, a); return hipGetLastError(); }
    MOEGQ_QVM(1, 32, 16) MOEGQ_QVM(2, 32, 8) MOEGQ_QVM(4, 32, 8)
    if constexpr (MODE == 0 && (BITS == 4 || BITS == 8)) {
      MOEGQ_QVM(1, 32 / BITS, 16) MOEGQ_QVM(2, 32 / BITS, 8) MOEGQ_QVM(4, 32 / BITS, 8)
    }
#undef MOEGQ_QVM
  } else {
    const dim3 grid((unsigned)((a.items + 3) / 4));           // one wave per item
    constexpr int R = BITS <= 4 ? 8 : 4;
#define MOEGQ_QMT(RB) \
  if (a.MB == RB) { hipLaunchKernelGGL((qmt_kernel<BITS, XT, RB, R, MODE>), grid, block, 0, st, a); return hipGetLastError(); }
    MOEGQ_QMT(1) MOEGQ_QMT(2)
#undef MOEGQ_QMT
  }
  return hipErrorInvalidValue;
}

template <int BITS, int MODE = 0>
static hipError_t launch_vec_bits(const VecArgs& a, int transpose, hipStream_t st) {
  if (a.x_type == 0) return launch_vec_t<BITS, 0, MODE>(a, transpose, st);
  if (a.x_type == 1) return launch_vec_t<BITS, 1, MODE>(a, transpose, st);
  if (a.x_type == 2) return launch_vec_t<BITS, 2, MODE>(a, transpose, st);
  return hipErrorInvalidValue;
}

hipError_t launch_qmm_vec(const VecArgs& a, int bits, int transpose, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  if (a.items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  if (a.mode == 1) e = bits == 4 ? launch_vec_bits<4, 1>(a, transpose, st) : hipErrorInvalidValue;
  else if (a.mode == 2) e = bits == 8 ? launch_vec_bits<8, 2>(a, transpose, st) : hipErrorInvalidValue;
  else switch (bits) {
    case 1: e = launch_vec_bits<1>(a, transpose, st); break;
    case 2: e = launch_vec_bits<2>(a, transpose, st); break;
    case 3: e = launch_vec_bits<3>(a, transpose, st); break;
    case 4: e = launch_vec_bits<4>(a, transpose, st); break;
    case 5: e = launch_vec_bits<5>(a, transpose, st); break;
    case 6: e = launch_vec_bits<6>(a, transpose, st); break;
    case 8: e = launch_vec_bits<8>(a, transpose, st); break;
    default: break;
  }
  if (e != hipSuccess || a.KS <= 1) return e;
  const int64_t total = a.P * a.M * (int64_t)a.N;
  int64_t blocks = (total + 63) / 64;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(vec_reduce_kernel, dim3((unsigned)blocks), dim3(64), 0, st, a.part, a.KS, total, a.out,
                     a.out_f32);
  return hipGetLastError();
}

}  // namespace moegq

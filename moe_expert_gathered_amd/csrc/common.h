// Device helpers shared by the gfx950 kernels: bf16 encode/decode, packed
// pair construction for 4-bit codes, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOEGQ_DEV __device__ __forceinline__

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace moegq {

// bf16 (as the upper half of an fp32) -> fp32
MOEGQ_DEV float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
MOEGQ_DEV float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
MOEGQ_DEV float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN 0x7FC0.
MOEGQ_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
MOEGQ_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

MOEGQ_DEV float fdot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Four bf16 pairs holding 128 + q for the eight 4-bit codes of a word w:
// pair j = (128 + q_j, 128 + q_{j+4}).  0x4300 is bf16 128.0 and codes < 16
// land in its low mantissa bits, so each lane is exactly 128 + q.
// The empty asm statements emit nothing: they hide the two constants' values
// from the compiler, which then keeps the mask in a VGPR and 0x4300 in an
// SGPR and selects one v_and_or_b32 per pair (with the constants visible it
// picks two VOP2 instructions with literal operands instead).
MOEGQ_DEV void nib_pairs(uint32_t w, uint32_t p[4]) {
  uint32_t m = 0x000F000Fu, magic = 0x43004300u;
  asm("" : "+v"(m));
  asm("" : "+s"(magic));
  p[0] = (w & m) | magic;
  p[1] = ((w >> 4) & m) | magic;
  p[2] = ((w >> 8) & m) | magic;
  p[3] = ((w >> 12) & m) | magic;
}

// Reorder eight consecutive bf16 values (four pairs d[0..3] = (x0,x1),
// (x2,x3), (x4,x5), (x6,x7)) into the nib_pairs order (x0,x4), (x1,x5),
// (x2,x6), (x3,x7).
MOEGQ_DEV void perm_pairs(const uint32_t d[4], uint32_t o[4]) {
  // __builtin_amdgcn_perm(hi_src, lo_src, sel): byte i of the result is
  // byte sel_i of the 8-byte value {hi_src:lo_src}.
  o[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);  // (lo of d0, lo of d2)
  o[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);  // (hi of d0, hi of d2)
  o[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
}

// ---- fp16 operands for the matrix cores ------------------------------------
// The MFMA paths dequantize to fp16 (11-bit significand): w = q * s + b is
// formed with one fused multiply-add and one rounding, and bf16 activations
// convert to fp16 exactly inside fp16's normal range.
//
// Codes enter fp16 through the exponent trick: 0x64XX is fp16 1024 + XX for
// XX < 1024, so v_perm placing a code byte under the byte 0x64 gives 1024 + q;
// subtracting 1024 is exact, then fma(q, s, b) rounds once.

MOEGQ_DEV f16x2_t f16_splat(float v) {
  const _Float16 h = (_Float16)v;
  return f16x2_t{h, h};
}
MOEGQ_DEV uint32_t deq_pair(uint32_t codes, uint32_t sel, f16x2_t s2, f16x2_t b2) {
  const f16x2_t q = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, codes, sel)) -
                    f16x2_t{(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
}
// eight 4-bit codes of one word -> four fp16 pairs in the order
// (q0,q2) (q4,q6) (q1,q3) (q5,q7)
MOEGQ_DEV void deq4_f16(uint32_t w, f16x2_t s2, f16x2_t b2, uint32_t o[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  o[0] = deq_pair(lo, 0x04010400u, s2, b2);
  o[1] = deq_pair(lo, 0x04030402u, s2, b2);
  o[2] = deq_pair(hi, 0x04010400u, s2, b2);
  o[3] = deq_pair(hi, 0x04030402u, s2, b2);
}
// four 8-bit codes of one word -> two fp16 pairs in natural order (q0,q1) (q2,q3)
MOEGQ_DEV void deq8_f16(uint32_t w, f16x2_t s2, f16x2_t b2, uint32_t o[2]) {
  o[0] = deq_pair(w, 0x04010400u, s2, b2);
  o[1] = deq_pair(w, 0x04030402u, s2, b2);
}
// fp32 pair -> fp16 pair, round to nearest even
MOEGQ_DEV uint32_t cvt_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)a, (_Float16)b});
}
// eight consecutive bf16 activations (four dwords) -> four fp16 pairs in the
// 4-bit code order (x0,x2) (x4,x6) (x1,x3) (x5,x7), or in natural order
template <int BITS>
MOEGQ_DEV uint4 act_f16(uint4 v) {
  if (BITS == 4)
    return make_uint4(cvt_f16x2(bf16_lo(v.x), bf16_lo(v.y)), cvt_f16x2(bf16_lo(v.z), bf16_lo(v.w)),
                      cvt_f16x2(bf16_hi(v.x), bf16_hi(v.y)), cvt_f16x2(bf16_hi(v.z), bf16_hi(v.w)));
  return make_uint4(cvt_f16x2(bf16_lo(v.x), bf16_hi(v.x)), cvt_f16x2(bf16_lo(v.y), bf16_hi(v.y)),
                    cvt_f16x2(bf16_lo(v.z), bf16_hi(v.z)), cvt_f16x2(bf16_lo(v.w), bf16_hi(v.w)));
}
// the same with every value multiplied by 2^e (exact: the bf16 values keep
// their 8 significant bits in fp16 down to 2^-14; smaller ones round to
// fp16's subnormal spacing, 2^-24)
template <int BITS>
MOEGQ_DEV uint4 act_f16_ldexp(uint4 v, int e) {
  auto lo = [&](uint32_t d) { return __builtin_ldexpf(bf16_lo(d), e); };
  auto hi = [&](uint32_t d) { return __builtin_ldexpf(bf16_hi(d), e); };
  if (BITS == 4)
    return make_uint4(cvt_f16x2(lo(v.x), lo(v.y)), cvt_f16x2(lo(v.z), lo(v.w)), cvt_f16x2(hi(v.x), hi(v.y)),
                      cvt_f16x2(hi(v.z), hi(v.w)));
  return make_uint4(cvt_f16x2(lo(v.x), hi(v.x)), cvt_f16x2(lo(v.y), hi(v.y)), cvt_f16x2(lo(v.z), hi(v.z)),
                    cvt_f16x2(lo(v.w), hi(v.w)));
}

// ---- bf16 operands for the matrix cores ------------------------------------
// The tile kernels dequantize to bf16 for v_mfma_f32_16x16x32_bf16, so the
// activations and intermediates enter the matrix cores as stored (bf16's
// whole range, no conversion).  A code enters fp16 exactly as 1024 + q (its
// byte under the exponent byte 0x64, one v_perm per two codes);
// v_fma_mix_f32 evaluates (1024 + q) * s + c in fp32, with c = b - 1024 s
// formed once per group, so w = q * s + b up to two fp32 roundings (far
// below bf16's); v_cvt_pk_bf16_f32 rounds two weights to bf16 (nearest
// even).  Limit: |s| < 2^117 (1024 s stays finite).
MOEGQ_DEV float bias1024(float s, float b) { return __builtin_fmaf(-1024.0f, s, b); }
MOEGQ_DEV uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}
MOEGQ_DEV f16x2_t magic_pair(uint32_t codes, uint32_t sel) {
  return __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, codes, sel));
}
// eight 4-bit codes of one word -> four bf16 pairs in natural order (q0,q1) .. (q6,q7)
MOEGQ_DEV void deq4_bf16(uint32_t w, float s, float c, uint32_t o[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;   // bytes: q0 q2 q4 q6 / q1 q3 q5 q7
  const f16x2_t a0 = magic_pair(lo, 0x04010400u), a1 = magic_pair(lo, 0x04030402u);
  const f16x2_t b0 = magic_pair(hi, 0x04010400u), b1 = magic_pair(hi, 0x04030402u);
  o[0] = pk_bf16(__builtin_fmaf((float)a0[0], s, c), __builtin_fmaf((float)b0[0], s, c));
  o[1] = pk_bf16(__builtin_fmaf((float)a0[1], s, c), __builtin_fmaf((float)b0[1], s, c));
  o[2] = pk_bf16(__builtin_fmaf((float)a1[0], s, c), __builtin_fmaf((float)b1[0], s, c));
  o[3] = pk_bf16(__builtin_fmaf((float)a1[1], s, c), __builtin_fmaf((float)b1[1], s, c));
}
// four 8-bit codes of one word -> two bf16 pairs in natural order (q0,q1) (q2,q3)
MOEGQ_DEV void deq8_bf16(uint32_t w, float s, float c, uint32_t o[2]) {
  const f16x2_t a = magic_pair(w, 0x04010400u), b = magic_pair(w, 0x04030402u);
  o[0] = pk_bf16(__builtin_fmaf((float)a[0], s, c), __builtin_fmaf((float)a[1], s, c));
  o[1] = pk_bf16(__builtin_fmaf((float)b[0], s, c), __builtin_fmaf((float)b[1], s, c));
}

// Exponent that brings a magnitude m > 0 into [2^13, 2^14) when divided out:
// m * 2^-e is in that range for e = frexp_exp(m) - 14 (exact for subnormal
// m too); 0 for m == 0.  Scaling fp16 operands this way keeps them normal
// and finite whatever the bf16 magnitudes, and undoing it on the fp32 result
// is exact.
MOEGQ_DEV int f16_exponent(float m) { return m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 14 : 0; }

// SwitchGLU's middle step on the two projections of one output: the gate and
// up results are bf16 tensors in the page's chain (MLX issue 4509, moe():
// g, u = gather_qmm(...), then g * sigmoid(g) * u), so both are rounded to
// bf16 before silu(g) * u, which is then rounded once by the caller.
// Both roundings are one hardware conversion of the pair (round to nearest
// even), and the sigmoid takes the hardware reciprocal (1 ulp) instead of a
// correctly rounded division: 2 instructions instead of about 10, well inside
// the bf16 rounding that follows.
MOEGQ_DEV float glu(float g, float u) {
  const uint32_t p = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)g, (__bf16)u});
  const float gr = __uint_as_float(p << 16), ur = __uint_as_float(p & 0xFFFF0000u);
  return gr * __builtin_amdgcn_rcpf(1.0f + __expf(-gr)) * ur;
}

MOEGQ_DEV float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <typename T>
MOEGQ_DEV T ldg(const T* p) { return *p; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes at `base`: loads outside the range
// return zero (the hardware bounds check), offsets are 32-bit.
MOEGQ_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
MOEGQ_DEV uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// the same with the non-temporal cache hint (policy bit 1 on gfx950): for
// weight streams read once per launch, which then do not push reused lines
// out of the caches
MOEGQ_DEV uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
MOEGQ_DEV uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
// 128-bit streaming load (non-temporal hint: weights are read once)
MOEGQ_DEV uint4 ld_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace moegq

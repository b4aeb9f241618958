// MoE router: from the router logits [T, E] (fp32) to the routing inputs of
// the expert path, idx [T, top_k] int32 and scores [T, top_k] bf16.
//
// MTPLX PR 558 (Change): the fused block computes the routing as the stock
// block does before the sorted experts and the combine.  The routing read
// here: the top_k experts by logit (ties to the lower id), stored in
// ascending expert id; a chosen expert's score is its softmax probability
// over all E logits in float64 (max-subtracted), not renormalised, rounded to
// fp32 and then to bf16.
//
// gfx950 mapping: one wave per token (4 tokens per workgroup).  Lane l holds
// the J = ceil(E / 64) consecutive ids l J .. l J + J - 1 in registers.  Top-k
// is k rounds of a wave argmax over (logit, -id) with a butterfly of shuffles;
// the winner's lane marks it.  A chosen id's slot is the number of chosen ids
// below it: the prefix of the per-lane counts plus the lane's own lower bits.
// The softmax sum runs in float64 (per-lane partial sums, then a butterfly).
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int ROUTE_MAXJ = 16;   // E <= 1024

// wave argmax of (v, id): larger v wins, equal v -> lower id (every lane gets the result)
MOEGQ_DEV void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oid = __shfl_xor(id, off, 64);
    if (ov > v || (ov == v && oid < id)) { v = ov; id = oid; }
  }
}

MOEGQ_DEV double shfl_xor_f64(double v, int m) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __shfl_xor((uint32_t)u, m, 64), hi = __shfl_xor((uint32_t)(u >> 32), m, 64);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int J>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int top_k,
                                                    int32_t* __restrict__ idx, uint16_t* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                  // whole waves leave together
  const float* row = logits + t * (int64_t)E;
  const int id0 = lane * J;
  float v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = id0 + j < E ? row[id0 + j] : -INFINITY;
  // the largest logit (exact in fp32)
  float m = v[0];
#pragma unroll
  for (int j = 1; j < J; ++j) m = fmaxf(m, v[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  // softmax terms and denominator in float64 (the terms stay in registers)
  double ex[J];
  double part = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    ex[j] = id0 + j < E ? exp((double)v[j] - (double)m) : 0.0;
    part += ex[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += shfl_xor_f64(part, off);
  // top_k by repeated argmax; chosen ids are marked in `sel`
  uint32_t sel = 0;
  for (int r = 0; r < top_k; ++r) {
    float bv = -INFINITY;
    int bid = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool free = id0 + j < E && !((sel >> j) & 1u);
      if (free && (v[j] > bv || bid == 0x7FFFFFFF)) { bv = v[j]; bid = id0 + j; }
    }
    wave_argmax(bv, bid);
    if (bid >= id0 && bid < id0 + J) sel |= 1u << (bid - id0);
  }
  // slot of each chosen id = chosen ids below it
  const int cnt = __popc(sel);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  int slot = incl - cnt;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if ((sel >> j) & 1u) {
      const double p = ex[j] / part;
      idx[t * top_k + slot] = id0 + j;
      scores[t * top_k + slot] = f32_to_bf16((float)p);
      ++slot;
    }
  }
}

hipError_t launch_route(const float* logits, int64_t T, int E, int top_k, int32_t* idx, uint16_t* scores,
                        hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (E < 1 || E > 64 * ROUTE_MAXJ || top_k < 1 || top_k > E || top_k > 64) return hipErrorInvalidValue;
  const int J = (E + 63) / 64;
  const int64_t nblk = (T + 3) / 4;
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
#define MOEGQ_RT(JJ) \
  if (J <= JJ) { hipLaunchKernelGGL((route_kernel<JJ>), dim3((unsigned)nblk), dim3(256), 0, st, logits, T, E, top_k, idx, scores); return hipGetLastError(); }
  MOEGQ_RT(1) MOEGQ_RT(2) MOEGQ_RT(4) MOEGQ_RT(8) MOEGQ_RT(16)
#undef MOEGQ_RT
  return hipErrorInvalidValue;
}

}  // namespace moegq

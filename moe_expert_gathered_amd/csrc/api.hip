// C ABI of the moegq library: argument validation (the format's error
// catalogue, nuvec-core tests/quantized.rs "invalid_arguments_are_rejected" and
// "gather_qmm_selects_batches"), workspace sizing and kernel dispatch.  No
// allocation, no synchronization (except the two documented checks).
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/moegq.h"
#include "launch.h"

using namespace moegq;

namespace {

constexpr int kMaxExperts = 1024;     // single-workgroup sort
constexpr int64_t kMaxQmvK = 32768;   // longest row of the one-row kernels (the size the tests cover)
constexpr int64_t kMaxDim = (int64_t)1 << 30;

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MOEGQ_OK : MOEGQ_ERR_LAUNCH; }

// The one-row kernels address one expert matrix through a 32-bit buffer
// range and park the lanes past a row's end at offset 0x7FFFFFF0, which must
// lie beyond that range: one matrix of codes stays at most 0x7FFFFFF0 bytes.
constexpr int64_t kNoFetchOffset = 0x7FFFFFF0;
bool one_row_fits(int64_t N, int64_t K, int bits) { return N * K * bits / 8 <= kNoFetchOffset; }
// most activation rows per pair on the vector kernel (more go to the matrix
// cores): 4, and 2 for 4-bit GLU pairs when the matrix-core kernel takes the
// shape (it runs a 4-bit GLU pair of 3-16 rows at about the cost of 2 rows on
// the vector kernel: 12.8-13.6 us for 2 x 9728 x 2560, against 16.6 at 3 rows
// and 18.5 at 4 on the vector kernel).  Plain products, and 8-bit GLU pairs
// (twice the code bytes per matrix-core step), stay on the vector kernel to
// 4 rows: 6.2 against 8.2 us for 2560 x 4096 at 4 rows.
constexpr int64_t kQmvRowsMax = 4, kQmvRowsMaxGlu4 = 2;

// bit width / group size / quantized length checks
int check_quant(int64_t K, int gs, int bits) {
  if (!(bits == 4 || bits == 8)) {
    if (bits == 1 || bits == 2 || bits == 3 || bits == 5 || bits == 6) return MOEGQ_ERR_UNSUPPORTED;
    return MOEGQ_ERR_BITS;
  }
  if (!(gs == 32 || gs == 64 || gs == 128)) return MOEGQ_ERR_GROUP_SIZE;
  if (K <= 0 || K > kMaxDim || K % gs != 0) return MOEGQ_ERR_SHAPE;
  return MOEGQ_OK;
}

int check_act_dtype(int d) {
  if (d == MOEGQ_BF16) return MOEGQ_OK;
  if (d == MOEGQ_F16 || d == MOEGQ_F32) return MOEGQ_ERR_UNSUPPORTED;
  return MOEGQ_ERR_DTYPE;   // f64 and integer activations are rejected by the format
}

// the format's checks for the vector-unit route, which takes every width of
// the format (1-6 and 8 bits)
int check_quant_any(int64_t L, int gs, int bits) {
  if (!(bits >= 1 && bits <= 6) && bits != 8) return MOEGQ_ERR_BITS;
  if (!(gs == 32 || gs == 64 || gs == 128)) return MOEGQ_ERR_GROUP_SIZE;
  if (L <= 0 || L > kMaxDim || L % gs != 0) return MOEGQ_ERR_SHAPE;
  return MOEGQ_OK;
}

// activations accepted by gather_qmm: bf16 on every route, float16 and
// float32 on the vector-unit route
int check_any_act_dtype(int d) {
  if (d == MOEGQ_BF16 || d == MOEGQ_F16 || d == MOEGQ_F32) return MOEGQ_OK;
  return MOEGQ_ERR_DTYPE;
}

int check_idx_dtype(int d) {
  if (d == MOEGQ_I32 || d == MOEGQ_U32) return MOEGQ_OK;
  if (d == MOEGQ_I64) return MOEGQ_ERR_UNSUPPORTED;
  return MOEGQ_ERR_DTYPE;   // float indices are rejected
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int auto_bm(int64_t P, int64_t E) {
  const int64_t active = P < E ? P : E;
  const int64_t mean = active > 0 ? P / active : 0;
  if (mean >= 96) return 64;
  if (mean >= 24) return 32;
  return 16;
}

int64_t tile_cap(int64_t P, int64_t E, int bm) { return (P + bm - 1) / bm + (P < E ? P : E); }

// hybrid schedule: experts with >= kSmallMax rows get kBigM-row tiles, the
// others one tile each for the few-row kernel
constexpr int kBigM = 128;
constexpr int kSmallMax = 32;
int64_t big_cap(int64_t P, int64_t E) {
  const int64_t nbig = P / kSmallMax < E ? P / kSmallMax : E;    // experts that can reach kSmallMax rows
  return (P + kBigM - 1) / kBigM + nbig;
}
// small tiles: at most ceil(c / kSmallMax) per expert, and as many for the extra rows
int64_t small_cap(int64_t P, int64_t E, int64_t extra = 0) {
  return P / kSmallMax + (P < E ? P : E) + (extra + kSmallMax - 1) / kSmallMax;
}

// Hybrid schedule parameters: two tile workgroups fit on each compute unit;
// the first pass (gate/up) has I / 128 column blocks per row tile.
// workgroup slots of the current device (2 per compute unit), cached per
// device; calls from several host threads may fill the cache concurrently
// (they store the same value)
int device_slots() {
  static std::atomic<int> slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int v = slots[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    v = 2 * cus;
    slots[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
// Result of the last moegq_selfcheck per device: 0 not run, 1 passed,
// 2 failed.  After a failure the entry points that would run the one-pass
// combine run the unfused tail instead (moe_prefill) or refuse
// (moe_combine, moe_combine_gated), for the rest of the process unless a
// later self-check passes (MTPLX PR 558 Change and Tests: a failed check turns
// the one-kernel route off).
std::atomic<int> g_selfcheck[64];
int selfcheck_state() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  return g_selfcheck[dev].load(std::memory_order_relaxed);
}
bool fused_tail_off() { return selfcheck_state() == 2; }
void set_selfcheck_state(int v) {
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) g_selfcheck[dev].store(v, std::memory_order_relaxed);
}

void set_hybrid_model(SortArgs& sa, int64_t I) {
  sa.small_max = kSmallMax;
  sa.cost_slots = device_slots();
  sa.cost_nb = (int)((I + 127) / 128);
}

// sorted-route workspace layout.  extra: rows of the extra (shared) expert
// appended after the P sorted rows; xexp: the exponents of the gate/up pass's
// fp16 activation rows (at most P rows); layer: also the fp16 activations
// [T, H], the expert outputs [P + extra, H], the shared gate logits [T] and
// the unfused tail's scratch.
struct SortedWs {
  int32_t* order; int32_t* lhs; int32_t* srhs; int32_t* counts; int32_t* offsets;
  int32_t* tiles; int32_t* small_tiles; int32_t* n_tiles; int32_t* bc; uint16_t* h; int32_t* xexp;
  uint16_t* x16; uint16_t* y; uint16_t* z;
  uint16_t* tail;     // layer: scratch of the unfused tail after a failed self-check, [(P + 2 T), H]
  size_t bytes;
};
SortedWs sorted_layout(char* base, int64_t P, int64_t E, int64_t I, int bm, int64_t extra = 0,
                       int64_t T = 0, int64_t H = 0, bool layer = false) {
  SortedWs w{};
  size_t off = 0;
  auto take = [&](size_t b) { char* p = base ? base + off : nullptr; off += align256(b); return p; };
  w.order = (int32_t*)take(4 * P);
  w.lhs = (int32_t*)take(4 * (P + extra));
  w.srhs = (int32_t*)take(4 * P);
  w.counts = (int32_t*)take(4 * E);
  w.offsets = (int32_t*)take(4 * (E + 1));
  const int64_t cap = (bm > 0 ? tile_cap(P, E, bm) : big_cap(P, E)) + (extra + kBigM - 1) / kBigM;
  w.tiles = (int32_t*)take(12 * cap);
  w.small_tiles = (int32_t*)take(12 * small_cap(P, E, extra));
  w.n_tiles = (int32_t*)take(8);
  w.bc = (int32_t*)take(4 * sort_blocks(P) * E);
  w.h = (uint16_t*)take(2 * (P + extra) * I);
  w.xexp = (int32_t*)take(4 * (layer ? T : P));
  if (layer) {
    w.x16 = (uint16_t*)take(2 * T * H);
    w.y = (uint16_t*)take(2 * (P + extra) * H);
    w.z = (uint16_t*)take(2 * T);
    w.tail = (uint16_t*)take(2 * (P + 2 * T) * H);
  }
  w.bytes = off;
  return w;
}

// generic gather (M > 16 rows per batch): pair-major virtual rows
__global__ void pair_tiles_kernel(const int32_t* rhs, int64_t P, int M, int bm, int32_t* tiles,
                                  int32_t* n_tiles) {
  const int ntm = (M + bm - 1) / bm;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t == 0) *n_tiles = (int32_t)(P * ntm);
  if (t >= P * ntm) return;
  const int64_t p = t / ntm, mt = t % ntm;
  tiles[3 * t] = (int32_t)(p * M + mt * bm);
  tiles[3 * t + 1] = rhs[p];
  tiles[3 * t + 2] = (int32_t)min((int64_t)bm, (int64_t)M - mt * bm);
}

// offsets of a non-decreasing expert list: offsets[e] = first p with rhs[p] >= e
__global__ void offsets_from_sorted_kernel(const int32_t* rhs, int64_t P, int E, int32_t* offsets) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e > E) return;
  int64_t lo = 0, hi = P;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (rhs[mid] < e) lo = mid + 1; else hi = mid;
  }
  offsets[e] = (int32_t)lo;
}

// few rows per pair (M <= 16): up to 4 rows (2 for 4-bit GLU pairs the
// matrix-core kernel takes) the matrix-vector kernel with every code applied to all the
// rows; else the exact-code matrix-core kernel when K is a multiple of 128 and
// the scales and biases start 8-byte aligned (K split over workgroups when ws
// holds its scratch: [counters | partials], counters zero before the first
// call), else the fp16-operand kernel
size_t few_ws_bytes(const FewPlan& pl) { return pl.KS > 1 ? align256(pl.counter_bytes) + pl.part_bytes : 0; }
int few_rows(const SkinnyArgs& sa, bool glu, int64_t P, int bits, int gs, void* ws, size_t wsb, hipStream_t s) {
  // the matrix-core kernel reads a chunk's scales and biases as one 32- or
  // 64-bit word: their arrays must start 8-byte aligned
  auto a8 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 7u) == 0; };
  const bool sb_ok = a8(sa.s0) && a8(sa.b0) && (!glu || (a8(sa.s1) && a8(sa.b1)));
  const bool few_ok = fewrow_supported(sa.M, sa.N, sa.K, bits) && sb_ok;
  const int64_t qmax = glu && bits == 4 && few_ok ? kQmvRowsMaxGlu4 : kQmvRowsMax;
  if (sa.M <= qmax && sa.K <= kMaxQmvK && one_row_fits(sa.N, sa.K, bits)) {
    // the vector kernel with every code applied to all the pair's rows (its
    // many one-wave workgroups keep more loads in flight than the
    // matrix-core kernel's few four-wave ones)
    QmvArgs a{};
    a.x = sa.x; a.lhs = sa.lhs; a.lhs_div = sa.lhs_div; a.rhs = sa.rhs;
    a.w0 = sa.w0; a.s0 = sa.s0; a.b0 = sa.b0; a.w1 = sa.w1; a.s1 = sa.s1; a.b1 = sa.b1;
    a.N = sa.N; a.K = sa.K; a.out = sa.out; a.residual = sa.residual; a.rows = sa.M;
    return status_of(launch_qmv(a, bits, gs, glu, P, s));
  }
  if (!few_ok) return status_of(launch_skinny(sa, bits, gs, glu, P, s));
  FewPlan pl = fewrow_plan(P, sa.N, sa.K, glu, ws != nullptr);
  if (few_ws_bytes(pl) > wsb || (pl.KS > 1 && !aligned16(ws))) pl = fewrow_plan(P, sa.N, sa.K, glu, false);
  FewArgs f{};
  f.x = sa.x; f.lhs = sa.lhs; f.lhs_div = sa.lhs_div; f.rhs = sa.rhs;
  f.w0 = sa.w0; f.s0 = sa.s0; f.b0 = sa.b0; f.w1 = sa.w1; f.s1 = sa.s1; f.b1 = sa.b1;
  f.M = sa.M; f.N = sa.N; f.K = sa.K; f.out = sa.out; f.residual = sa.residual;
  if (pl.KS > 1) {
    f.counters = (int32_t*)ws;
    f.part = (float*)((char*)ws + align256(pl.counter_bytes));
  }
  return status_of(launch_fewrow(f, pl, bits, gs, glu, s));
}

}  // namespace

extern "C" {

const char* moegq_status_string(int s) {
  switch (s) {
    case MOEGQ_OK: return "ok";
    case MOEGQ_ERR_NULL_ARG: return "null argument";
    case MOEGQ_ERR_BITS: return "unsupported bit width";
    case MOEGQ_ERR_GROUP_SIZE: return "group size must be 32, 64 or 128";
    case MOEGQ_ERR_SHAPE: return "shape mismatch";
    case MOEGQ_ERR_DTYPE: return "invalid dtype";
    case MOEGQ_ERR_UNSUPPORTED: return "valid but not supported by this library";
    case MOEGQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MOEGQ_ERR_LAUNCH: return "kernel launch failed";
    case MOEGQ_ERR_SELFCHECK: return "fused combine differs from the unfused tail";
    case MOEGQ_ERR_INDEX: return "index out of range or not sorted";
    case MOEGQ_ERR_ALIGN: return "pointer not 16-byte aligned";
  }
  return "unknown status";
}

const char* moegq_version(void) { return "moegq 0.1 gfx950"; }

size_t moegq_workspace_bytes(int op, int64_t P, int64_t E, int64_t N, int bm) {
  if (P < 0 || E < 0 || N < 0) return 0;
  switch (op) {
    case MOEGQ_OP_GATHER_QMM: {
      // M > 16 rows per batch (N carries M here): tile table; M == 1 sorted: offsets + tiles
      const int64_t M = N;
      const int b = 64;
      if (M > 16) return align256(12 * (P * ((M + b - 1) / b))) + 256;
      if (M == 1) return align256(4 * (E + 1)) + align256(12 * tile_cap(P, E, 16)) + 256;
      return 0;
    }
    case MOEGQ_OP_GATHER_MM: {
      // N carries M: M == 1 sorted: offsets + tiles; M > 1: the per-pair tile table
      const int64_t M = N;
      if (M > 1) return align256(12 * (P * ((M + 63) / 64))) + 256;
      return align256(4 * (E + 1)) + align256(12 * tile_cap(P, E, 16)) + 256;
    }
    case MOEGQ_OP_SWITCH_GLU_DECODE: return align256(2 * P * N);
    case MOEGQ_OP_SWITCH_GLU_SORTED: {
      const size_t a = sorted_layout(nullptr, P, E, N, bm).bytes;
      const size_t b = sorted_layout(nullptr, P, E, N, 16).bytes;   // covers every explicit bm
      return bm > 0 ? a : (a > b ? a : b);
    }
    case MOEGQ_OP_COMBINE_UNFUSED: {
      // N = H, P = T*top_k; T*H <= P*H
      return align256(2 * (2 * P * N + P * N));
    }
    case MOEGQ_OP_SELFCHECK: {
      const int64_t T = 128, K = 8, H = 2048;
      return align256(2 * T * K * H) + align256(4 * T * K) + align256(2 * T * K) + align256(2 * T * H) * 3 +
             align256(2 * 3 * T * K * H) + 256;
    }
    case MOEGQ_OP_SORT_PAIRS: return align256(4 * sort_blocks(P) * E);
    case MOEGQ_OP_MOE_DECODE: {
      // N = I; h [P, I], plus y [P, H] for top_k > 8 when the caller passes none (H unknown here:
      // callers with top_k > 8 pass y or size it with moegq_moe_decode_workspace)
      return align256(2 * P * N);
    }
  }
  return 0;
}

size_t moegq_gather_qmm_workspace_bytes(int64_t P, int64_t E, int64_t M, int64_t N, int64_t K, int x_dtype,
                                        int transpose, int bits, int sorted_indices) {
  if (P <= 0 || M <= 0 || N <= 0 || K <= 0 || E <= 0) return 0;
  if (!(bits >= 1 && bits <= 6) && bits != 8) return 0;
  if (!transpose || x_dtype != MOEGQ_BF16 || (bits != 4 && bits != 8))
    return vec_plan(P, M, N, K, bits, transpose).part_bytes;
  if ((M == 1 && !sorted_indices) || (M >= 2 && M <= 16)) return 0;
  return moegq_workspace_bytes(MOEGQ_OP_GATHER_QMM, P, E, M, 0);
}

// transpose = 0 (weights [E, K, N*bits/32], groups along N) or float16 /
// float32 activations: the vector-unit kernels, fp32 partial sums of the K
// split in the workspace
static int gather_vec(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* w,
                      const void* scales, const void* biases, int64_t E, int64_t N, const void* lhs_indices,
                      int64_t lhs_div, const void* rhs_indices, int64_t P, int transpose, int group_size,
                      int bits, void* out, void* workspace, size_t workspace_bytes, void* stream, int mode = 0) {
  int st;
  // the quantized axis: K with the transpose, N without it (mx: blocks of 32)
  if (mode) {
    const int64_t L = transpose ? K : N;
    if (L <= 0 || L > kMaxDim || L % 32 != 0) return MOEGQ_ERR_SHAPE;
  } else if ((st = check_quant_any(transpose ? K : N, group_size, bits))) {
    return st;
  }
  if (K <= 0 || K > kMaxDim || M > kMaxDim) return MOEGQ_ERR_SHAPE;
  // one expert matrix must fit a 2 GiB buffer range (32-bit offsets)
  if (K * N * bits / 8 >= ((int64_t)1 << 31)) return MOEGQ_ERR_UNSUPPORTED;
  if (!lhs_indices && lhs_div < 1) return MOEGQ_ERR_SHAPE;
  if (P == 0 || M == 0 || N == 0) return MOEGQ_OK;
  if (!x || !w || !scales || (!biases && !mode) || !rhs_indices || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return MOEGQ_ERR_ALIGN;
  if (!lhs_indices && (P - 1) / lhs_div >= X) return MOEGQ_ERR_SHAPE;
  const VecPlan pl = vec_plan(P, M, N, K, bits, transpose, mode);
  if (pl.part_bytes && (!workspace || workspace_bytes < pl.part_bytes)) return MOEGQ_ERR_WORKSPACE;
  if (pl.part_bytes && !aligned16(workspace)) return MOEGQ_ERR_ALIGN;
  VecArgs a{};
  a.x = x; a.x_type = x_dtype == MOEGQ_BF16 ? 0 : (x_dtype == MOEGQ_F16 ? 1 : 2);
  a.lhs = (const int32_t*)lhs_indices; a.lhs_div = lhs_div; a.rhs = (const int32_t*)rhs_indices;
  a.P = P; a.M = (int)M; a.N = (int)N; a.K = (int)K; a.gs = group_size;
  a.w = (const uint32_t*)w; a.s = (const uint16_t*)scales; a.b = (const uint16_t*)biases;
  a.mode = mode;
  a.out = out; a.out_f32 = x_dtype != MOEGQ_BF16;
  a.part = (float*)workspace;
  a.MB = pl.MB; a.MBLK = pl.MBLK; a.WPL = pl.WPL; a.NC = pl.NC; a.KS = pl.KS; a.kchunk = pl.kchunk;
  a.items = pl.items;
  return status_of(launch_qmm_vec(a, bits, transpose, S(stream)));
}

static int gather_impl(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* w,
                       int w_dtype, const void* scales, const void* biases, const void* w1, const void* s1,
                       const void* b1, bool glu, int64_t E, int64_t N, const void* lhs_indices,
                       int64_t lhs_div, const void* rhs_indices, int idx_dtype, int64_t P, int sorted_indices,
                       int transpose, int group_size, int bits, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_any_act_dtype(x_dtype))) return st;
  if (w_dtype != MOEGQ_U32) return MOEGQ_ERR_DTYPE;
  if ((st = check_idx_dtype(idx_dtype))) return st;
  if (X < 0 || M < 0 || E <= 0 || N < 0 || P < 0 || X > kMaxDim || N > kMaxDim || P > kMaxDim)
    return MOEGQ_ERR_SHAPE;
  if (!transpose || x_dtype != MOEGQ_BF16 || (bits != 4 && bits != 8)) {
    if (glu) return (bits >= 1 && bits <= 6) || bits == 8 ? MOEGQ_ERR_UNSUPPORTED : MOEGQ_ERR_BITS;
    return gather_vec(x, x_dtype, X, M, K, w, scales, biases, E, N, lhs_indices, lhs_div, rhs_indices, P,
                      transpose, group_size, bits, out, workspace, workspace_bytes, stream);
  }
  if ((st = check_quant(K, group_size, bits))) return st;
  if (!lhs_indices && lhs_div < 1) return MOEGQ_ERR_SHAPE;
  if (P == 0 || M == 0 || N == 0) return MOEGQ_OK;
  if (!x || !w || !scales || !biases || !rhs_indices || !out) return MOEGQ_ERR_NULL_ARG;
  if (glu && (!w1 || !s1 || !b1)) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (glu && !aligned16(w1))) return MOEGQ_ERR_ALIGN;
  if (!lhs_indices && (P - 1) / lhs_div >= X) return MOEGQ_ERR_SHAPE;
  const int32_t* lhs = (const int32_t*)lhs_indices;
  const int32_t* rhs = (const int32_t*)rhs_indices;
  hipStream_t s = S(stream);
  const size_t need = moegq_workspace_bytes(MOEGQ_OP_GATHER_QMM, P, E, M, 0);
  if (M == 1 && sorted_indices && P >= 64 && E <= kMaxExperts) {
    if (!workspace || workspace_bytes < need) return MOEGQ_ERR_WORKSPACE;
    char* base = (char*)workspace;
    int32_t* offsets = (int32_t*)base;
    int32_t* tiles = (int32_t*)(base + align256(4 * (E + 1)));
    int32_t* n_tiles = (int32_t*)(base + align256(4 * (E + 1)) + align256(12 * tile_cap(P, E, 16)));
    hipLaunchKernelGGL(offsets_from_sorted_kernel, dim3((unsigned)((E + 1 + 255) / 256)), dim3(256), 0, s,
                       rhs, P, (int)E, offsets);
    if (!glu && tiles_mma_supported(K, N, X, group_size)) {   // x rows (lhs indices address [0, X))
      // the matrix-core tiles with bf16 operands (the activations as stored,
      // weights dequantized in fp32 and rounded once to bf16): bf16's whole
      // range; 128-row tiles when the experts average 96 rows or more
      const int rows = auto_bm(P, E) >= 64 ? 128 : 32;
      if (launch_schedule(offsets, (int)E, rows, 0, tiles, n_tiles, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
      TileArgs a{};
      a.x = (const uint16_t*)x; a.lhs = lhs; a.lhs_div = lhs_div; a.rows_per_batch = 1;
      a.tiles = tiles; a.n_tiles = n_tiles; a.P = P; a.E = (int)E;
      a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
      a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = rows; a.tile_mode = 0;
      a.grid_tiles = tile_cap(P, E, rows);
      return status_of(launch_tiles_mma(a, bits, group_size, false, rows, s));
    }
    const int bm = auto_bm(P, E);
    hipError_t e = launch_schedule(offsets, (int)E, bm, 0, tiles, n_tiles, s);
    if (e != hipSuccess) return MOEGQ_ERR_LAUNCH;
    TileArgs a{};
    a.x = (const uint16_t*)x; a.lhs = lhs; a.lhs_div = lhs_div; a.rows_per_batch = 1;
    a.tiles = tiles; a.n_tiles = n_tiles; a.P = P; a.E = (int)E;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.w1 = (const uint32_t*)w1; a.s1 = (const uint16_t*)s1; a.b1 = (const uint16_t*)b1;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = bm; a.tile_mode = 0;
    a.grid_tiles = tile_cap(P, E, bm);
    return status_of(launch_tiles(a, bits, group_size, glu, s));
  }
  if (M == 1) {
    if (K > kMaxQmvK || !one_row_fits(N, K, bits)) return MOEGQ_ERR_UNSUPPORTED;
    QmvArgs a{};
    a.x = (const uint16_t*)x; a.lhs = lhs; a.lhs_div = lhs_div; a.rhs = rhs;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.w1 = (const uint32_t*)w1; a.s1 = (const uint16_t*)s1; a.b1 = (const uint16_t*)b1;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out;
    return status_of(launch_qmv(a, bits, group_size, glu, P, s));
  }
  if (M <= 16) {
    SkinnyArgs a{};
    a.x = (const uint16_t*)x; a.lhs = lhs; a.lhs_div = lhs_div; a.rhs = rhs;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.w1 = (const uint32_t*)w1; a.s1 = (const uint16_t*)s1; a.b1 = (const uint16_t*)b1;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out;
    return few_rows(a, glu, P, bits, group_size, nullptr, 0, s);
  }
  // M > 16: per-pair tiles over pair-major virtual rows
  if (!workspace || workspace_bytes < need) return MOEGQ_ERR_WORKSPACE;
  const int bm = 64;
  const int64_t nt = P * ((M + bm - 1) / bm);
  int32_t* tiles = (int32_t*)workspace;
  int32_t* n_tiles = (int32_t*)((char*)workspace + align256(12 * nt));
  hipLaunchKernelGGL(pair_tiles_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, rhs, P, (int)M,
                     bm, tiles, n_tiles);
  TileArgs a{};
  a.x = (const uint16_t*)x; a.lhs = lhs; a.lhs_div = lhs_div; a.rows_per_batch = M;
  a.tiles = tiles; a.n_tiles = n_tiles; a.P = P * M; a.E = (int)E;
  a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
  a.w1 = (const uint32_t*)w1; a.s1 = (const uint16_t*)s1; a.b1 = (const uint16_t*)b1;
  a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = bm; a.tile_mode = 0; a.grid_tiles = nt;
  return status_of(launch_tiles(a, bits, group_size, glu, s));
}

int moegq_gather_qmm(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* w,
                     int w_dtype, const void* scales, const void* biases, int64_t E, int64_t N,
                     const void* lhs_indices, int64_t lhs_div, const void* rhs_indices, int idx_dtype,
                     int64_t P, int sorted_indices, int transpose, int group_size, int bits, void* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return gather_impl(x, x_dtype, X, M, K, w, w_dtype, scales, biases, nullptr, nullptr, nullptr, false, E, N,
                     lhs_indices, lhs_div, rhs_indices, idx_dtype, P, sorted_indices, transpose, group_size,
                     bits, out, workspace, workspace_bytes, stream);
}

int moegq_gather_qmm_mx(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* w,
                        const void* scales, int64_t E, int64_t N, const void* lhs_indices, int64_t lhs_div,
                        const void* rhs_indices, int idx_dtype, int64_t P, int transpose, int mode, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_any_act_dtype(x_dtype))) return st;
  if ((st = check_idx_dtype(idx_dtype))) return st;
  if (mode != MOEGQ_MXFP4 && mode != MOEGQ_MXFP8) return MOEGQ_ERR_BITS;
  if (X < 0 || M < 0 || E <= 0 || N < 0 || P < 0 || X > kMaxDim || N > kMaxDim || P > kMaxDim)
    return MOEGQ_ERR_SHAPE;
  const int bits = mode == MOEGQ_MXFP4 ? 4 : 8;
  return gather_vec(x, x_dtype, X, M, K, w, scales, nullptr, E, N, lhs_indices, lhs_div, rhs_indices, P,
                    transpose, 32, bits, out, workspace, workspace_bytes, stream, mode);
}

size_t moegq_gather_qmm_mx_workspace_bytes(int64_t P, int64_t M, int64_t N, int64_t K, int transpose, int mode) {
  if (P <= 0 || M <= 0 || N <= 0 || K <= 0) return 0;
  if (mode != MOEGQ_MXFP4 && mode != MOEGQ_MXFP8) return 0;
  return vec_plan(P, M, N, K, mode == MOEGQ_MXFP4 ? 4 : 8, transpose, mode).part_bytes;
}

int moegq_gather_qmm_glu(const void* x, int x_dtype, int64_t X, int64_t M, int64_t K, const void* wg,
                         const void* sg, const void* bg, const void* wu, const void* su, const void* bu,
                         int64_t E, int64_t N, const void* lhs_indices, int64_t lhs_div,
                         const void* rhs_indices, int idx_dtype, int64_t P, int sorted_indices, int group_size,
                         int bits, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return gather_impl(x, x_dtype, X, M, K, wg, MOEGQ_U32, sg, bg, wu, su, bu, true, E, N, lhs_indices, lhs_div,
                     rhs_indices, idx_dtype, P, sorted_indices, 1, group_size, bits, out, workspace,
                     workspace_bytes, stream);
}

size_t moegq_affine_qmm_workspace_bytes(int64_t M, int64_t N, int64_t K, int glu) {
  // the bit width is not an argument: sized as if the narrowest codes (the
  // size only grows with the split, never with the bits)
  if (M < 2 || M > 16 || N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim || !fewrow_supported(M, N, K, 1)) return 0;
  return few_ws_bytes(fewrow_plan(1, N, K, glu != 0, true));
}

int moegq_affine_qmm(const void* x, int x_dtype, int64_t M, int64_t K, const void* w, int w_dtype,
                     const void* scales, const void* biases, int64_t N, int transpose, int group_size,
                     int bits, const void* residual, void* out, void* stream) {
  return moegq_affine_qmm_ws(x, x_dtype, M, K, w, w_dtype, scales, biases, N, transpose, group_size, bits,
                             residual, out, nullptr, 0, stream);
}

int moegq_affine_qmm_ws(const void* x, int x_dtype, int64_t M, int64_t K, const void* w, int w_dtype,
                        const void* scales, const void* biases, int64_t N, int transpose, int group_size,
                        int bits, const void* residual, void* out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st;
  if ((st = check_act_dtype(x_dtype))) return st;
  if (w_dtype != MOEGQ_U32) return MOEGQ_ERR_DTYPE;
  if ((st = check_quant(K, group_size, bits))) return st;
  if (!transpose) return MOEGQ_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return MOEGQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MOEGQ_OK;
  if (!x || !w || !scales || !biases || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return MOEGQ_ERR_ALIGN;
  hipStream_t s = S(stream);
  if (M == 1 && K <= kMaxQmvK && one_row_fits(N, K, bits)) {
    QmvArgs a{};
    a.x = (const uint16_t*)x; a.lhs_div = 1;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.residual = (const uint16_t*)residual;
    return status_of(launch_qmv(a, bits, group_size, false, 1, s));
  }
  if (M <= 16) {
    SkinnyArgs a{};
    a.x = (const uint16_t*)x; a.lhs_div = 1;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.residual = (const uint16_t*)residual;
    return few_rows(a, false, 1, bits, group_size, workspace, workspace ? workspace_bytes : 0, s);
  }
  if (residual) return MOEGQ_ERR_UNSUPPORTED;
  if (M >= kBigM && tiles_mma_supported(K, N, M, group_size)) {
    // 128 rows and more: the matrix-core tiles with bf16 operands (bf16's
    // whole range; 142 against 182 us at 4096 x 4096 x 4096).  Below, their
    // 32-row tiles give too few workgroups (47 against 31 us at 40 rows), so
    // the fp16 tiles keep 17..127 rows
    const int rows = 128;
    TileArgs a{};
    a.x = (const uint16_t*)x; a.lhs = nullptr; a.lhs_div = 1; a.rows_per_batch = 1;
    a.P = M; a.E = 1; a.tile_mode = 2;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = rows;
    a.grid_tiles = (M + rows - 1) / rows;
    return status_of(launch_tiles_mma(a, bits, group_size, false, rows, s));
  }
  if (M >= kBigM) {
    TileArgs a{};
    a.x = (const uint16_t*)x; a.lhs = nullptr; a.lhs_div = 1; a.rows_per_batch = 1;
    a.P = M; a.E = 1; a.tile_mode = 2;
    a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = kBigM;
    a.grid_tiles = (M + kBigM - 1) / kBigM;
    return status_of(launch_tiles_big(a, bits, group_size, false, s));
  }
  // many rows: one "expert", tiles over M on the device-free path
  const int bm = 32;
  static_assert(sizeof(int32_t) == 4, "");
  TileArgs a{};
  a.x = (const uint16_t*)x; a.lhs = nullptr; a.lhs_div = 1; a.rows_per_batch = 1;
  a.P = M; a.E = 1; a.tile_mode = 2;        // dense: tiles over the rows, one weight matrix
  a.w0 = (const uint32_t*)w; a.s0 = (const uint16_t*)scales; a.b0 = (const uint16_t*)biases;
  a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = bm;
  a.grid_tiles = (M + bm - 1) / bm;
  a.sorted_rhs = nullptr;
  return status_of(launch_tiles(a, bits, group_size, false, s));
}

int moegq_affine_qmm_glu(const void* x, int64_t M, int64_t K, const void* wg, const void* sg,
                         const void* bg, const void* wu, const void* su, const void* bu, int64_t N,
                         int group_size, int bits, void* out, void* stream) {
  return moegq_affine_qmm_glu_ws(x, M, K, wg, sg, bg, wu, su, bu, N, group_size, bits, out, nullptr, 0, stream);
}

int moegq_affine_qmm_glu_ws(const void* x, int64_t M, int64_t K, const void* wg, const void* sg,
                            const void* bg, const void* wu, const void* su, const void* bu, int64_t N,
                            int group_size, int bits, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int st;
  if ((st = check_quant(K, group_size, bits))) return st;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return MOEGQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MOEGQ_OK;
  if (!x || !wg || !sg || !bg || !wu || !su || !bu || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(out)) return MOEGQ_ERR_ALIGN;
  hipStream_t s = S(stream);
  if (M == 1 && K <= kMaxQmvK && one_row_fits(N, K, bits)) {
    QmvArgs a{};
    a.x = (const uint16_t*)x; a.lhs_div = 1;
    a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
    a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out;
    return status_of(launch_qmv(a, bits, group_size, true, 1, s));
  }
  if (M <= 16) {
    SkinnyArgs a{};
    a.x = (const uint16_t*)x; a.lhs_div = 1;
    a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
    a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out;
    return few_rows(a, true, 1, bits, group_size, workspace, workspace ? workspace_bytes : 0, s);
  }
  if (M >= kBigM) {
    TileArgs a{};
    a.x = (const uint16_t*)x; a.lhs_div = 1; a.rows_per_batch = 1;
    a.P = M; a.E = 1; a.tile_mode = 2;
    a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
    a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
    a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = kBigM;
    a.grid_tiles = (M + kBigM - 1) / kBigM;
    return status_of(launch_tiles_big(a, bits, group_size, true, s));
  }
  const int bm = 32;
  TileArgs a{};
  a.x = (const uint16_t*)x; a.lhs_div = 1; a.rows_per_batch = 1;
  a.P = M; a.E = 1; a.tile_mode = 2;
  a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
  a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
  a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out; a.bm = bm;
  a.grid_tiles = (M + bm - 1) / bm;
  return status_of(launch_tiles(a, bits, group_size, true, s));
}

int moegq_switch_glu_mode(int64_t T, int64_t top_k, int64_t E) {
  // the sorted route pays off once experts see several rows each; decode
  // (a handful of tokens) streams each pair's expert once
  const int64_t P = T * top_k;
  (void)E;
  return (T >= 32 && P >= 256) ? MOEGQ_MODE_SORTED : MOEGQ_MODE_DECODE;
}

int moegq_switch_glu(const void* x, int64_t T, int64_t H, int64_t I, int64_t E, const int32_t* idx,
                     int64_t top_k, const void* wg, const void* sg, const void* bg, const void* wu,
                     const void* su, const void* bu, const void* wd, const void* sd, const void* bd,
                     int group_size, int bits, int mode, int tile_mode, int bm, void* y, int32_t* inv,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_quant(H, group_size, bits))) return st;
  if ((st = check_quant(I, group_size, bits))) return st;
  if (T < 0 || top_k <= 0 || E <= 0 || T > kMaxDim || top_k > 64) return MOEGQ_ERR_SHAPE;
  if (!(mode == MOEGQ_MODE_AUTO || mode == MOEGQ_MODE_DECODE || mode == MOEGQ_MODE_SORTED))
    return MOEGQ_ERR_SHAPE;
  if (!(tile_mode == MOEGQ_TILES_SCHEDULED || tile_mode == MOEGQ_TILES_NAIVE)) return MOEGQ_ERR_SHAPE;
  if (!(bm == 0 || bm == 16 || bm == 32 || bm == 64 || bm == 128)) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!x || !idx || !wg || !sg || !bg || !wu || !su || !bu || !wd || !sd || !bd || !y)
    return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(y))
    return MOEGQ_ERR_ALIGN;
  const int64_t P = T * top_k;
  if (mode == MOEGQ_MODE_AUTO) {
    if (!inv) return MOEGQ_ERR_NULL_ARG;
    mode = moegq_switch_glu_mode(T, top_k, E);
  }
  hipStream_t s = S(stream);
  if (mode == MOEGQ_MODE_SORTED && (E > kMaxExperts)) return MOEGQ_ERR_UNSUPPORTED;
  if (mode == MOEGQ_MODE_SORTED && !inv) return MOEGQ_ERR_NULL_ARG;
  if (mode == MOEGQ_MODE_DECODE) {
    if (H > kMaxQmvK || I > kMaxQmvK || !one_row_fits(I, H, bits) || !one_row_fits(H, I, bits))
      return MOEGQ_ERR_UNSUPPORTED;
    const size_t need = moegq_workspace_bytes(MOEGQ_OP_SWITCH_GLU_DECODE, P, E, I, 0);
    if (!workspace || workspace_bytes < need) return MOEGQ_ERR_WORKSPACE;
    uint16_t* h = (uint16_t*)workspace;
    QmvArgs a{};
    a.x = (const uint16_t*)x; a.lhs = nullptr; a.lhs_div = top_k; a.rhs = idx;
    a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
    a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
    a.N = (int)I; a.K = (int)H; a.out = h;
    hipError_t e = launch_qmv(a, bits, group_size, true, P, s);
    if (e != hipSuccess) return MOEGQ_ERR_LAUNCH;
    QmvArgs d{};
    d.x = h; d.lhs = nullptr; d.lhs_div = 1; d.rhs = idx;
    d.w0 = (const uint32_t*)wd; d.s0 = (const uint16_t*)sd; d.b0 = (const uint16_t*)bd;
    d.N = (int)H; d.K = (int)I; d.out = (uint16_t*)y;
    e = launch_qmv(d, bits, group_size, false, P, s);
    if (e != hipSuccess) return MOEGQ_ERR_LAUNCH;
    if (inv) e = launch_iota(inv, P, s);
    return status_of(e);
  }
  // sorted route
  const bool hybrid = (bm == 0 && tile_mode == MOEGQ_TILES_SCHEDULED);
  const bool big = hybrid || (bm == kBigM && tile_mode == MOEGQ_TILES_SCHEDULED);
  if (bm == 0) bm = tile_mode == MOEGQ_TILES_NAIVE ? auto_bm(P, E) : 0;
  const SortedWs ws = sorted_layout((char*)workspace, P, E, I, bm);
  if (!workspace || workspace_bytes < ws.bytes) return MOEGQ_ERR_WORKSPACE;
  SortArgs sa{};
  sa.idx = idx; sa.P = P; sa.top_k = (int)top_k; sa.E = (int)E;
  sa.order = ws.order; sa.lhs = ws.lhs; sa.sorted_rhs = ws.srhs; sa.inv = inv;
  sa.counts = ws.counts; sa.offsets = ws.offsets;
  sa.tiles = ws.tiles; sa.n_tiles = ws.n_tiles;
  sa.bm = hybrid ? kBigM : bm; sa.tile_mode = hybrid ? 3 : tile_mode;
  sa.small_tiles = ws.small_tiles;
  if (hybrid) set_hybrid_model(sa, I);
  sa.block_counts = ws.bc;
  hipError_t e = launch_sort(sa, s);
  if (e != hipSuccess) return MOEGQ_ERR_LAUNCH;
  TileArgs g{};
  g.x = (const uint16_t*)x; g.lhs = ws.lhs; g.lhs_div = 1; g.rows_per_batch = 1;
  g.sorted_rhs = ws.srhs; g.offsets = ws.offsets; g.tiles = ws.tiles; g.n_tiles = ws.n_tiles;
  g.P = P; g.E = (int)E;
  g.w0 = (const uint32_t*)wg; g.s0 = (const uint16_t*)sg; g.b0 = (const uint16_t*)bg;
  g.w1 = (const uint32_t*)wu; g.s1 = (const uint16_t*)su; g.b1 = (const uint16_t*)bu;
  g.N = (int)I; g.K = (int)H; g.out = ws.h; g.bm = big ? kBigM : bm; g.tile_mode = tile_mode;
  g.grid_tiles = hybrid ? big_cap(P, E) : (tile_mode == MOEGQ_TILES_SCHEDULED ? tile_cap(P, E, bm) : (P + bm - 1) / bm);
  TileArgs d = g;
  d.x = ws.h; d.lhs = nullptr; d.lhs_div = 1;
  d.w0 = (const uint32_t*)wd; d.s0 = (const uint16_t*)sd; d.b0 = (const uint16_t*)bd;
  d.w1 = nullptr; d.s1 = nullptr; d.b1 = nullptr;
  d.N = (int)H; d.K = (int)I; d.out = (uint16_t*)y;
  if (!big) {
    if (launch_tiles(g, bits, group_size, true, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
    return status_of(launch_tiles(d, bits, group_size, false, s));
  }
  // 128-row tiles (all experts, or the experts with >= kSmallMax rows), then
  // the few-row tiles of the remaining experts
  TileArgs gs_ = g, ds_ = d;
  gs_.tiles = ws.small_tiles; gs_.n_tiles = ws.n_tiles + 1; gs_.bm = kSmallMax; gs_.tile_mode = 0;
  gs_.grid_tiles = small_cap(P, E);
  ds_.tiles = ws.small_tiles; ds_.n_tiles = ws.n_tiles + 1; ds_.bm = kSmallMax; ds_.tile_mode = 0;
  ds_.grid_tiles = small_cap(P, E);
  g.tile_mode = 0; d.tile_mode = 0;
  if (tiles_mma_supported(H, I, T, group_size) && tiles_mma_supported(I, H, P, group_size)) {
    // the gate/up pass reads x as scaled fp16 rows (their exponents in the
    // workspace), parked in y, which only the down pass writes, after every
    // reader of x; the down pass reads the bf16 intermediate as stored
    if (launch_prep((const uint16_t*)x, T, (int)H, bits, group_size, (uint16_t*)y, ws.xexp, nullptr, nullptr,
                    nullptr, nullptr, s) != hipSuccess)
      return MOEGQ_ERR_LAUNCH;
    g.x = (const uint16_t*)y;
    g.xexp = ws.xexp;
    if (hybrid) {
      g.tiles2 = d.tiles2 = ws.small_tiles; g.n_tiles2 = d.n_tiles2 = ws.n_tiles + 1;
      g.grid_tiles2 = d.grid_tiles2 = small_cap(P, E);
      if (launch_tiles_mma_dual(g, bits, group_size, true, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
      return status_of(launch_tiles_mma_dual(d, bits, group_size, false, s));
    }
    if (launch_tiles_mma(g, bits, group_size, true, 128, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
    return status_of(launch_tiles_mma(d, bits, group_size, false, 128, s));
  }
  if (launch_tiles_big(g, bits, group_size, true, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (hybrid && launch_tiles_small(gs_, bits, group_size, true, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (launch_tiles_big(d, bits, group_size, false, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (hybrid && launch_tiles_small(ds_, bits, group_size, false, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  return MOEGQ_OK;
}

size_t moegq_moe_prefill_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t I,
                                         int has_shared) {
  if (T < 0 || top_k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  const int64_t P = T * top_k;
  return sorted_layout(nullptr, P, E, I, 0, has_shared ? T : 0, T, H, true).bytes;
}

int moegq_moe_prefill_layout(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t I, int has_shared,
                             int64_t* offsets, int64_t* caps, int32_t* params) {
  if (T < 0 || top_k <= 0 || E <= 0 || H <= 0 || I <= 0 || T > kMaxDim || top_k > 64) return MOEGQ_ERR_SHAPE;
  if (E > kMaxExperts) return MOEGQ_ERR_UNSUPPORTED;
  if (!offsets || !caps || !params) return MOEGQ_ERR_NULL_ARG;
  const int64_t P = T * top_k, extra = has_shared ? T : 0;
  char* const base = (char*)(uintptr_t)4096;        // any aligned base: offsets are relative to it
  const SortedWs w = sorted_layout(base, P, E, I, 0, extra, T, H, true);
  const void* parts[9] = {w.order, w.lhs, w.srhs, w.counts, w.offsets, w.tiles, w.small_tiles, w.n_tiles, w.tail};
  for (int i = 0; i < 9; ++i) offsets[i] = (int64_t)((const char*)parts[i] - base);
  caps[0] = big_cap(P, E) + (extra + kBigM - 1) / kBigM;
  caps[1] = small_cap(P, E, extra);
  SortArgs sa{};
  set_hybrid_model(sa, I);
  params[0] = kBigM;
  params[1] = sa.small_max;
  params[2] = sa.cost_slots;
  params[3] = sa.cost_nb;
  return MOEGQ_OK;
}

int moegq_moe_prefill(const void* x, int64_t T, int64_t H, int64_t I, int64_t E, const int32_t* idx,
                      int64_t top_k, const void* scores, const void* wg, const void* sg, const void* bg,
                      const void* wu, const void* su, const void* bu, const void* wd, const void* sd,
                      const void* bd, const void* shg_w, const void* shg_s, const void* shg_b,
                      const void* shu_w, const void* shu_s, const void* shu_b, const void* shd_w,
                      const void* shd_s, const void* shd_b, const void* gate_w, const void* gate_s,
                      const void* gate_b, int group_size, int bits, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_quant(H, group_size, bits))) return st;
  if ((st = check_quant(I, group_size, bits))) return st;
  if (T < 0 || top_k <= 0 || E <= 0 || T > kMaxDim || top_k > 64 || H % 8 != 0) return MOEGQ_ERR_SHAPE;
  if (E > kMaxExperts) return MOEGQ_ERR_UNSUPPORTED;
  if (T == 0) return MOEGQ_OK;
  if (!x || !idx || !scores || !wg || !sg || !bg || !wu || !su || !bu || !wd || !sd || !bd || !out)
    return MOEGQ_ERR_NULL_ARG;
  const bool shared = shg_w != nullptr;
  if (shared && (!shg_s || !shg_b || !shu_w || !shu_s || !shu_b || !shd_w || !shd_s || !shd_b || !gate_w ||
                 !gate_s || !gate_b))
    return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(out) ||
      (shared && (!aligned16(shg_w) || !aligned16(shu_w) || !aligned16(shd_w) || !aligned16(gate_w))))
    return MOEGQ_ERR_ALIGN;
  const int64_t P = T * top_k;
  const int64_t extra = shared ? T : 0;
  if (!tiles_mma_supported(H, I, T, group_size) || !tiles_mma_supported(I, H, P + extra, group_size))
    return MOEGQ_ERR_UNSUPPORTED;
  const SortedWs ws = sorted_layout((char*)workspace, P, E, I, 0, extra, T, H, true);
  if (!workspace || workspace_bytes < ws.bytes) return MOEGQ_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  SortArgs sa{};
  sa.idx = idx; sa.P = P; sa.top_k = (int)top_k; sa.E = (int)E;
  int32_t* inv = ws.order;           // the layer keeps the inverse permutation, not the order
  sa.order = nullptr; sa.lhs = ws.lhs; sa.sorted_rhs = ws.srhs; sa.inv = inv;
  sa.counts = ws.counts; sa.offsets = ws.offsets;
  sa.tiles = ws.tiles; sa.n_tiles = ws.n_tiles; sa.bm = kBigM; sa.tile_mode = 3;
  sa.small_tiles = ws.small_tiles;
  set_hybrid_model(sa, I);
  sa.extra_rows = extra; sa.block_counts = ws.bc;
  // the sort, and the scaled fp16 activations with the shared expert's
  // sigmoid-gate logit (one pass over x), in one launch when the pairs allow
  if (launch_front(sa, (const uint16_t*)x, T, (int)H, bits, group_size, ws.x16, ws.xexp,
                   shared ? (const uint32_t*)gate_w : nullptr, (const uint16_t*)gate_s, (const uint16_t*)gate_b, ws.z,
                   s) != hipSuccess)
    return MOEGQ_ERR_LAUNCH;
  TileArgs g{};
  g.x = ws.x16; g.xexp = ws.xexp; g.lhs = ws.lhs; g.lhs_div = 1; g.rows_per_batch = 1;
  g.tiles = ws.tiles; g.n_tiles = ws.n_tiles; g.P = P; g.E = (int)E;
  g.w0 = (const uint32_t*)wg; g.s0 = (const uint16_t*)sg; g.b0 = (const uint16_t*)bg;
  g.w1 = (const uint32_t*)wu; g.s1 = (const uint16_t*)su; g.b1 = (const uint16_t*)bu;
  g.xw0 = (const uint32_t*)shg_w; g.xs0 = (const uint16_t*)shg_s; g.xb0 = (const uint16_t*)shg_b;
  g.xw1 = (const uint32_t*)shu_w; g.xs1 = (const uint16_t*)shu_s; g.xb1 = (const uint16_t*)shu_b;
  g.N = (int)I; g.K = (int)H; g.out = ws.h; g.bm = kBigM; g.tile_mode = 0;
  g.grid_tiles = big_cap(P, E) + (extra + kBigM - 1) / kBigM;
  TileArgs d = g;
  d.x = ws.h; d.lhs = nullptr;
  d.w0 = (const uint32_t*)wd; d.s0 = (const uint16_t*)sd; d.b0 = (const uint16_t*)bd;
  d.w1 = nullptr; d.s1 = nullptr; d.b1 = nullptr;
  d.xw0 = (const uint32_t*)shd_w; d.xs0 = (const uint16_t*)shd_s; d.xb0 = (const uint16_t*)shd_b;
  d.xw1 = nullptr; d.xs1 = nullptr; d.xb1 = nullptr;
  d.N = (int)H; d.K = (int)I; d.out = ws.y;
  // 128-row tiles (hot experts, shared expert) and 32-row tiles (tail experts) in one launch per pass
  g.tiles2 = d.tiles2 = ws.small_tiles; g.n_tiles2 = d.n_tiles2 = ws.n_tiles + 1;
  g.grid_tiles2 = d.grid_tiles2 = small_cap(P, E, extra);
  if (launch_tiles_mma_dual(g, bits, group_size, true, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (launch_tiles_mma_dual(d, bits, group_size, false, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  // out[t] = bf16(bf16(sum_k bf16(y[inv] * score)) + bf16(sigmoid(z[t]) * y[P + t]))
  if (fused_tail_off()) {
    // the self-check failed on this device: the unfused tail, the gate first
    // (its own kernel), then unsort, score, sum over top_k, add
    uint16_t* gated = nullptr;
    if (shared) {
      gated = ws.tail + (P + T) * H;
      if (launch_sigmoid_gate(ws.y + P * H, ws.z, 1, T, H, gated, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
    }
    return status_of(launch_combine_unfused(ws.y, inv, (const uint16_t*)scores, gated, T, (int)top_k, H,
                                            (uint16_t*)out, ws.tail, s, true));
  }
  return status_of(launch_combine(ws.y, inv, (const uint16_t*)scores, shared ? ws.y + P * H : nullptr,
                                  shared ? ws.z : nullptr, T, (int)top_k, H, (uint16_t*)out, s));
}

// The decode layer given the intermediate h [T * top_k, I] bf16 (workspace of
// the caller or the static scratch below): argument checks, then the two launches.
static int decode_layer(const void* x, int64_t T, int64_t H, int64_t I, int64_t E, const int32_t* idx,
                        int64_t top_k, const void* scores, const void* shared, const void* wg, const void* sg,
                        const void* bg, const void* wu, const void* su, const void* bu, const void* wd,
                        const void* sd, const void* bd, int group_size, int bits, void* out, void* y,
                        uint16_t* h, size_t h_bytes, hipStream_t s) {
  int st;
  if ((st = check_quant(H, group_size, bits))) return st;
  if ((st = check_quant(I, group_size, bits))) return st;
  if (T < 0 || top_k <= 0 || E <= 0 || T > kMaxDim || top_k > 64 || H % 8 != 0) return MOEGQ_ERR_SHAPE;
  if (H > kMaxQmvK || I > kMaxQmvK || !one_row_fits(I, H, bits) || !one_row_fits(H, I, bits))
    return MOEGQ_ERR_UNSUPPORTED;
  if (T == 0) return MOEGQ_OK;
  if (!x || !idx || !scores || !wg || !sg || !bg || !wu || !su || !bu || !wd || !sd || !bd || !out)
    return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || !aligned16(wd) || !aligned16(out) ||
      (y && !aligned16(y)) || (shared && !aligned16(shared)))
    return MOEGQ_ERR_ALIGN;
  const int64_t P = T * top_k;
  const size_t need = moegq_workspace_bytes(MOEGQ_OP_MOE_DECODE, P, E, I, 0);
  if (!h || h_bytes < need) return MOEGQ_ERR_WORKSPACE;
  if (top_k > 8 && !y) return MOEGQ_ERR_NULL_ARG;
  QmvArgs a{};
  a.x = (const uint16_t*)x; a.lhs = nullptr; a.lhs_div = top_k; a.rhs = idx;
  a.w0 = (const uint32_t*)wg; a.s0 = (const uint16_t*)sg; a.b0 = (const uint16_t*)bg;
  a.w1 = (const uint32_t*)wu; a.s1 = (const uint16_t*)su; a.b1 = (const uint16_t*)bu;
  a.N = (int)I; a.K = (int)H; a.out = h;
  if (launch_qmv(a, bits, group_size, true, P, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  QmvArgs d{};
  d.x = h; d.lhs = nullptr; d.lhs_div = 1; d.rhs = idx;
  d.w0 = (const uint32_t*)wd; d.s0 = (const uint16_t*)sd; d.b0 = (const uint16_t*)bd;
  d.N = (int)H; d.K = (int)I; d.out = (uint16_t*)y;
  if (top_k <= 8)
    return status_of(launch_qmv_combine(d, bits, group_size, (const uint16_t*)scores, (const uint16_t*)shared, T,
                                        (int)top_k, (uint16_t*)out, s));
  // wider top_k: separate down projection and combine, through the caller's y
  uint16_t* yw = (uint16_t*)y;
  d.out = yw;
  if (launch_qmv(d, bits, group_size, false, P, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  return status_of(launch_combine(yw, nullptr, (const uint16_t*)scores, (const uint16_t*)shared, nullptr, T,
                                  (int)top_k, H, (uint16_t*)out, s));
}

int moegq_moe_decode(const void* x, int64_t T, int64_t H, int64_t I, int64_t E, const int32_t* idx,
                     int64_t top_k, const void* scores, const void* shared, const void* wg, const void* sg,
                     const void* bg, const void* wu, const void* su, const void* bu, const void* wd,
                     const void* sd, const void* bd, int group_size, int bits, void* out, void* y,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_layer(x, T, H, I, E, idx, top_k, scores, shared, wg, sg, bg, wu, su, bu, wd, sd, bd, group_size,
                      bits, out, y, (uint16_t*)workspace, workspace ? workspace_bytes : 0, S(stream));
}

}  // extern "C"

namespace {
// Scratch of the allocation-free decode entry point: the gate/up intermediate
// h [T * top_k, I] bf16 lives in this file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::atomic<void*> g_scratch_ptr[64];

void* static_scratch(int* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *err = MOEGQ_ERR_LAUNCH;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  // several host threads may race here: each gets the same address
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    *err = MOEGQ_ERR_LAUNCH;
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

extern "C" {

size_t moegq_static_scratch_bytes(void) { return kStaticScratchBytes; }

int moegq_moe_decode_static(const void* x, int64_t T, int64_t H, int64_t I, int64_t E, const int32_t* idx,
                            int64_t top_k, const void* scores, const void* shared, const void* wg, const void* sg,
                            const void* bg, const void* wu, const void* su, const void* bu, const void* wd,
                            const void* sd, const void* bd, int group_size, int bits, void* out, void* y,
                            void* stream) {
  // sizes beyond the scratch are refused before the device is touched
  if (T > 0 && top_k > 0 && I > 0 && T <= kMaxDim && top_k <= 64 && I <= kMaxDim &&
      moegq_workspace_bytes(MOEGQ_OP_MOE_DECODE, T * top_k, E, I, 0) > kStaticScratchBytes)
    return MOEGQ_ERR_WORKSPACE;
  if (T == 0) return decode_layer(x, T, H, I, E, idx, top_k, scores, shared, wg, sg, bg, wu, su, bu, wd, sd, bd,
                                  group_size, bits, out, y, nullptr, 0, S(stream));
  int err = MOEGQ_OK;
  void* h = static_scratch(&err);
  if (!h) return err;
  return decode_layer(x, T, H, I, E, idx, top_k, scores, shared, wg, sg, bg, wu, su, bu, wd, sd, bd, group_size,
                      bits, out, y, (uint16_t*)h, kStaticScratchBytes, S(stream));
}

int moegq_moe_combine(const void* y, const int32_t* inv, const void* scores, const void* shared, int64_t T,
                      int64_t top_k, int64_t H, void* out, void* stream) {
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8 != 0 || T > kMaxDim || H > kMaxDim) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!y || !scores || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(y) || !aligned16(out) || (shared && !aligned16(shared))) return MOEGQ_ERR_ALIGN;
  if (fused_tail_off()) return MOEGQ_ERR_SELFCHECK;
  return status_of(launch_combine((const uint16_t*)y, inv, (const uint16_t*)scores, (const uint16_t*)shared,
                                  nullptr, T, (int)top_k, H, (uint16_t*)out, S(stream)));
}

int moegq_moe_combine_gated(const void* y, const int32_t* inv, const void* scores, const void* shared,
                            const void* z, int64_t T, int64_t top_k, int64_t H, void* out, void* stream) {
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8 != 0 || T > kMaxDim || H > kMaxDim) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!y || !scores || !shared || !z || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(y) || !aligned16(out) || !aligned16(shared)) return MOEGQ_ERR_ALIGN;
  if (fused_tail_off()) return MOEGQ_ERR_SELFCHECK;
  return status_of(launch_combine((const uint16_t*)y, inv, (const uint16_t*)scores, (const uint16_t*)shared,
                                  (const uint16_t*)z, T, (int)top_k, H, (uint16_t*)out, S(stream)));
}

int moegq_moe_combine_unfused(const void* y, const int32_t* inv, const void* scores, const void* shared,
                              int64_t T, int64_t top_k, int64_t H, void* out, void* scratch,
                              size_t scratch_bytes, void* stream) {
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8 != 0 || T > kMaxDim || H > kMaxDim) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!y || !scores || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(y) || !aligned16(out) || (shared && !aligned16(shared))) return MOEGQ_ERR_ALIGN;
  const size_t need = moegq_workspace_bytes(MOEGQ_OP_COMBINE_UNFUSED, T * top_k, 0, H, 0);
  if (!scratch || scratch_bytes < need || !aligned16(scratch)) return MOEGQ_ERR_WORKSPACE;
  return status_of(launch_combine_unfused((const uint16_t*)y, inv, (const uint16_t*)scores,
                                          (const uint16_t*)shared, T, (int)top_k, H, (uint16_t*)out,
                                          (uint16_t*)scratch, S(stream)));
}

int moegq_sort_pairs(const void* idx, int idx_dtype, int64_t T, int64_t top_k, int64_t E, int32_t* order,
                     int32_t* lhs, int32_t* sorted_rhs, int32_t* inv, int32_t* counts, int32_t* offsets,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_idx_dtype(idx_dtype))) return st;
  if (T < 0 || top_k <= 0 || E <= 0 || T > kMaxDim || top_k > 64) return MOEGQ_ERR_SHAPE;
  if (E > kMaxExperts) return MOEGQ_ERR_UNSUPPORTED;
  if (!idx || !inv || !counts || !offsets) return MOEGQ_ERR_NULL_ARG;
  const size_t need = moegq_workspace_bytes(MOEGQ_OP_SORT_PAIRS, T * top_k, E, 0, 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOEGQ_ERR_WORKSPACE;
  SortArgs sa{};
  sa.block_counts = (int32_t*)workspace;
  sa.idx = (const int32_t*)idx; sa.P = T * top_k; sa.top_k = (int)top_k; sa.E = (int)E;
  sa.order = order; sa.lhs = lhs; sa.sorted_rhs = sorted_rhs; sa.inv = inv;
  sa.counts = counts; sa.offsets = offsets; sa.tiles = nullptr; sa.n_tiles = nullptr; sa.bm = 0;
  return status_of(launch_sort(sa, S(stream)));
}

int moegq_schedule_tiles(const int32_t* offsets, int64_t E, int64_t P_max, int bm, int tile_mode,
                         int32_t* tiles, int64_t cap, int32_t* n_tiles, void* stream) {
  if (E <= 0 || P_max < 0 || !(bm == 16 || bm == 32 || bm == 64 || bm == 128)) return MOEGQ_ERR_SHAPE;
  if (!(tile_mode == MOEGQ_TILES_SCHEDULED || tile_mode == MOEGQ_TILES_NAIVE)) return MOEGQ_ERR_SHAPE;
  if (E > kMaxExperts) return MOEGQ_ERR_UNSUPPORTED;
  if (!offsets || !tiles || !n_tiles) return MOEGQ_ERR_NULL_ARG;
  if (cap < tile_cap(P_max, E, bm)) return MOEGQ_ERR_WORKSPACE;
  return status_of(launch_schedule(offsets, (int)E, bm, tile_mode, tiles, n_tiles, S(stream)));
}

int moegq_rms_norm(const void* x, const void* w, int64_t M, int64_t K, float eps, void* out, void* stream) {
  if (M < 0 || K <= 0) return MOEGQ_ERR_SHAPE;
  if (M == 0) return MOEGQ_OK;
  if (!x || !w || !out) return MOEGQ_ERR_NULL_ARG;
  return status_of(launch_rms_norm((const uint16_t*)x, (const uint16_t*)w, M, K, eps, (uint16_t*)out, S(stream)));
}

int moegq_gather_mm(const void* x, int64_t X, int64_t M, int64_t K, const void* w, int64_t E, int64_t N,
                    const int32_t* lhs_indices, int64_t lhs_div, const int32_t* rhs_indices, int64_t P,
                    int sorted_indices, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (X < 0 || M < 0 || K <= 0 || E <= 0 || N < 0 || P < 0 || X > kMaxDim || N > kMaxDim || P > kMaxDim ||
      K > kMaxDim || K % 8 != 0)
    return MOEGQ_ERR_SHAPE;
  if (!lhs_indices && lhs_div < 1) return MOEGQ_ERR_SHAPE;
  if (P == 0 || M == 0 || N == 0) return MOEGQ_OK;
  if (!x || !w || !rhs_indices || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return MOEGQ_ERR_ALIGN;
  if (!lhs_indices && (P - 1) / lhs_div >= X) return MOEGQ_ERR_SHAPE;
  if (N * K * 2 > kNoFetchOffset || X * M * K >= ((int64_t)1 << 31)) return MOEGQ_ERR_UNSUPPORTED;
  hipStream_t s = S(stream);
  const size_t need = moegq_workspace_bytes(MOEGQ_OP_GATHER_MM, P, E, M, 0);
  TileArgs a{};
  a.x = (const uint16_t*)x; a.lhs = lhs_indices; a.lhs_div = lhs_div; a.rows_per_batch = 1;
  a.E = (int)E; a.w0 = (const uint32_t*)w; a.N = (int)N; a.K = (int)K; a.out = (uint16_t*)out;
  a.tile_mode = 0;
  if (M == 1 && sorted_indices && P >= 64 && E <= kMaxExperts && K % 128 == 0) {
    // pairs already sorted by expert: per-expert offsets, the expert-aware schedule at
    // BM 64, one K pass per tile on the matrix cores
    if (!workspace || workspace_bytes < need) return MOEGQ_ERR_WORKSPACE;
    char* base = (char*)workspace;
    int32_t* offsets = (int32_t*)base;
    int32_t* tiles = (int32_t*)(base + align256(4 * (E + 1)));
    int32_t* n_tiles = (int32_t*)(base + align256(4 * (E + 1)) + align256(12 * tile_cap(P, E, 16)));
    hipLaunchKernelGGL(offsets_from_sorted_kernel, dim3((unsigned)((E + 1 + 255) / 256)), dim3(256), 0, s,
                       rhs_indices, P, (int)E, offsets);
    if (launch_schedule(offsets, (int)E, 64, 0, tiles, n_tiles, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
    a.tiles = tiles; a.n_tiles = n_tiles; a.P = P; a.bm = 64; a.grid_tiles = tile_cap(P, E, 64);
    return status_of(launch_tiles_mma_w16(a, false, 64, s));
  }
  if (M == 1) {
    QmvArgs q{};
    q.x = (const uint16_t*)x; q.lhs = lhs_indices; q.lhs_div = lhs_div; q.rhs = rhs_indices;
    q.w0 = (const uint32_t*)w; q.N = (int)N; q.K = (int)K; q.out = (uint16_t*)out;
    return status_of(launch_mv16(q, P, s));
  }
  // M > 1: per-pair tiles of up to 64 virtual rows (pair-major)
  if (K % 128 != 0) return MOEGQ_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < need) return MOEGQ_ERR_WORKSPACE;
  const int bm = 64;
  const int64_t nt = P * ((M + bm - 1) / bm);
  int32_t* tiles = (int32_t*)workspace;
  int32_t* n_tiles = (int32_t*)((char*)workspace + align256(12 * nt));
  hipLaunchKernelGGL(pair_tiles_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, rhs_indices, P, (int)M,
                     bm, tiles, n_tiles);
  a.rows_per_batch = M; a.tiles = tiles; a.n_tiles = n_tiles; a.P = P * M; a.bm = bm; a.grid_tiles = nt;
  return status_of(launch_tiles_mma_w16(a, false, 64, s));
}

int moegq_route(const void* logits, int64_t T, int64_t E, int64_t top_k, int32_t* idx, void* scores,
                void* stream) {
  if (T < 0 || T > kMaxDim || E < 1 || E > 1024 || top_k < 1 || top_k > E || top_k > 64) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!logits || !idx || !scores) return MOEGQ_ERR_NULL_ARG;
  return status_of(launch_route((const float*)logits, T, (int)E, (int)top_k, idx, (uint16_t*)scores, S(stream)));
}

int moegq_sigmoid_gate(const void* s, const void* z, int64_t z_stride, int64_t T, int64_t H, void* out,
                       void* stream) {
  if (T < 0 || H <= 0 || H % 8 != 0 || z_stride < 1) return MOEGQ_ERR_SHAPE;
  if (T == 0) return MOEGQ_OK;
  if (!s || !z || !out) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(s) || !aligned16(out)) return MOEGQ_ERR_ALIGN;
  return status_of(launch_sigmoid_gate((const uint16_t*)s, (const uint16_t*)z, z_stride, T, H, (uint16_t*)out,
                                       S(stream)));
}

int moegq_kv_feed(const void* q, const void* k, const void* v, int64_t M, int64_t Nq, int64_t Nk, int64_t Nv,
                  void* out, void* stream) {
  return moegq_kv_feed_ld(q, Nq, k, Nk, v, Nv, M, Nq, out, stream);
}

int moegq_kv_feed_ld(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv, int64_t M,
                     int64_t Nq, void* out, void* stream) {
  if (M < 0 || Nq <= 0 || ldq < Nq || ldk <= 0 || ldv <= 0) return MOEGQ_ERR_SHAPE;
  if (M == 0) return MOEGQ_OK;
  if (!q || !k || !v || !out) return MOEGQ_ERR_NULL_ARG;
  return status_of(launch_kv_feed((const uint16_t*)q, ldq, (const uint16_t*)k, ldk, (const uint16_t*)v, ldv, M, Nq,
                                  (uint16_t*)out, S(stream)));
}

int moegq_selfcheck(void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t T = 128, K = 8, H = 2048, P = T * K;
  if (!workspace || workspace_bytes < moegq_workspace_bytes(MOEGQ_OP_SELFCHECK, 0, 0, 0, 0) ||
      !aligned16(workspace))
    return MOEGQ_ERR_WORKSPACE;
  char* b = (char*)workspace;
  size_t off = 0;
  auto take = [&](size_t n) { char* p = b + off; off += align256(n); return p; };
  uint16_t* y = (uint16_t*)take(2 * P * H);
  int32_t* inv = (int32_t*)take(4 * P);
  uint16_t* scores = (uint16_t*)take(2 * P);
  uint16_t* shared = (uint16_t*)take(2 * T * H);
  uint16_t* o1 = (uint16_t*)take(2 * T * H);
  uint16_t* o2 = (uint16_t*)take(2 * T * H);
  uint16_t* scratch = (uint16_t*)take(2 * 3 * P * H);
  hipStream_t s = S(stream);
  if (launch_fill_selfcheck(y, inv, scores, shared, T, (int)K, H, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (launch_combine(y, inv, scores, shared, nullptr, T, (int)K, H, o1, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (launch_combine_unfused(y, inv, scores, shared, T, (int)K, H, o2, scratch, s) != hipSuccess)
    return MOEGQ_ERR_LAUNCH;
  std::vector<uint16_t> h1(T * H), h2(T * H);      // host copies (calls from several threads stay apart)
  const size_t nb = h1.size() * sizeof(uint16_t);
  if (hipMemcpyAsync(h1.data(), o1, nb, hipMemcpyDeviceToHost, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (hipMemcpyAsync(h2.data(), o2, nb, hipMemcpyDeviceToHost, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  const char* force = getenv("MOEGQ_FORCE_SELFCHECK_FAIL");
  const bool same = memcmp(h1.data(), h2.data(), nb) == 0 && !(force && force[0] == '1');
  set_selfcheck_state(same ? 1 : 2);
  return same ? MOEGQ_OK : MOEGQ_ERR_SELFCHECK;
}

int moegq_selfcheck_state(void) { return selfcheck_state(); }

int moegq_probe_stream_read(const void* buf, int64_t bytes, void* sink, int blocks, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || blocks <= 0) return MOEGQ_ERR_SHAPE;
  if (!buf || !sink) return MOEGQ_ERR_NULL_ARG;
  if (!aligned16(buf)) return MOEGQ_ERR_ALIGN;
  return status_of(launch_stream_read(buf, bytes, (uint32_t*)sink, blocks, S(stream)));
}

int moegq_probe_mfma_bf16(int iters, int blocks, void* out, void* stream) {
  if (iters <= 0 || blocks <= 0) return MOEGQ_ERR_SHAPE;
  if (!out) return MOEGQ_ERR_NULL_ARG;
  return status_of(launch_mfma_loop(iters, blocks, (float*)out, S(stream)));
}

int moegq_validate_indices(const int32_t* idx, int64_t n, int64_t E, int sorted, int32_t* workspace,
                           void* stream) {
  if (n < 0 || E <= 0) return MOEGQ_ERR_SHAPE;
  if (!workspace || (n > 0 && !idx)) return MOEGQ_ERR_NULL_ARG;
  hipStream_t s = S(stream);
  if (launch_validate(idx, n, E, sorted, workspace, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  int32_t flag = 0;
  if (hipMemcpyAsync(&flag, workspace, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return MOEGQ_ERR_LAUNCH;
  return flag ? MOEGQ_ERR_INDEX : MOEGQ_OK;
}

}  // extern "C"

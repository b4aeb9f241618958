// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moegq {

// gathered matrix-vector (decode): one activation row per pair
struct QmvArgs {
  const uint16_t* x;        // activation rows [*, K] bf16
  const int32_t* lhs;       // row of x per pair, or null -> p / lhs_div
  int64_t lhs_div;
  int lhs_shift;            // log2(lhs_div) when it is a power of two, else -1 (set by launch_qmv)
  const int32_t* rhs;       // expert per pair, or null -> 0
  const uint32_t* w0; const uint16_t* s0; const uint16_t* b0;   // [E, N, Kw], [E, N, G]
  const uint32_t* w1; const uint16_t* s1; const uint16_t* b1;   // GLU: up projection
  int N, K;
  uint16_t* out;            // [P, N] ([P, rows, N] with several rows)
  const uint16_t* residual; // null or shaped as out
  int64_t rows;             // activation rows per pair (x [X, rows, K]); 0 or 1: one row, at most 4
};
hipError_t launch_qmv(const QmvArgs& a, int bits, int gs, bool glu, int64_t P, hipStream_t st);
// unquantized bf16 expert rows [E, N, K] (a.w0), one activation row per pair; K % 8 == 0
hipError_t launch_mv16(const QmvArgs& a, int64_t P, hipStream_t st);
// decode down projection + combine: out[t] from pairs t*top_k .. t*top_k + top_k - 1
// (a.out, if not null, also receives y [T*top_k, N]); top_k <= 8
hipError_t launch_qmv_combine(const QmvArgs& a, int bits, int gs, const uint16_t* scores, const uint16_t* shared,
                              int64_t T, int top_k, uint16_t* out, hipStream_t st);

// few-row MFMA (2..16 rows per pair)
struct SkinnyArgs {
  const uint16_t* x;        // [X, M, K]
  const int32_t* lhs; int64_t lhs_div;
  const int32_t* rhs;
  const uint32_t* w0; const uint16_t* s0; const uint16_t* b0;
  const uint32_t* w1; const uint16_t* s1; const uint16_t* b1;
  int M, N, K;
  uint16_t* out;            // [P, M, N]
  const uint16_t* residual; // null or [P, M, N]
};
hipError_t launch_skinny(const SkinnyArgs& a, int bits, int gs, bool glu, int64_t P, hipStream_t st);

// few-row products on the bf16 matrix cores with exact codes (1..16 rows per
// pair, K a multiple of 128), K split over KS workgroups when a workspace
// holds the fp32 partials and the per-column-group counters (zero before the
// first call; every call leaves them zero)
struct FewArgs {
  const uint16_t* x;        // [X, M, K]
  const int32_t* lhs; int64_t lhs_div;
  const int32_t* rhs;
  const uint32_t* w0; const uint16_t* s0; const uint16_t* b0;
  const uint32_t* w1; const uint16_t* s1; const uint16_t* b1;
  int M, N, K;
  uint16_t* out;            // [P, M, N]
  const uint16_t* residual; // null or [P, M, N]
  float* part;              // [items, KS, ...] fp32 partials (KS > 1)
  int32_t* counters;        // [items] (KS > 1)
  int cps;                  // K chunks per split (set by launch_fewrow)
};
struct FewPlan {
  int NB, KS, cps;          // column blocks per workgroup, splits, chunks per split
  int64_t items;            // workgroups per split (pairs x column groups)
  size_t part_bytes, counter_bytes;
};
FewPlan fewrow_plan(int64_t P, int64_t N, int64_t K, bool glu, bool split_allowed);
bool fewrow_supported(int64_t M, int64_t N, int64_t K, int bits);
hipError_t launch_fewrow(const FewArgs& a, const FewPlan& pl, int bits, int gs, bool glu, hipStream_t st);

// expert sort + tile table (single workgroup)
struct SortArgs {
  const int32_t* idx; int64_t P; int top_k; int E;
  int32_t* order; int32_t* lhs; int32_t* sorted_rhs; int32_t* inv;
  int32_t* counts; int32_t* offsets;
  int32_t* tiles; int32_t* n_tiles; int bm; int tile_mode;   // tiles may be null
  // hybrid schedule (tile_mode 3): bm-row tiles in `tiles` for experts with
  // at least small_max rows, small_max-row tiles in `small_tiles` for the
  // others (counts in n_tiles[0..1]); when cost_slots > 0 and those bm-row
  // tiles times cost_nb column blocks come to at most cost_slots / 8 work
  // items, every expert gets small_max-row tiles instead.
  int32_t* small_tiles; int small_max;
  int cost_slots; int cost_nb;
  // extra expert E over rows [P, P + extra_rows) (the shared expert, row t = token t):
  // bm-row tiles appended to `tiles`, lhs[P + t] = t
  int64_t extra_rows;
  int32_t* block_counts;    // workspace: [sort_blocks(P), E] int32
};
int64_t sort_blocks(int64_t P);
hipError_t launch_sort(const SortArgs& a, hipStream_t st);
// the ranking launch of the block sort, once a.block_counts holds the block histograms
hipError_t launch_sort_rest(const SortArgs& a, hipStream_t st);
hipError_t launch_schedule(const int32_t* offsets, int E, int bm, int tile_mode, int32_t* tiles,
                           int32_t* n_tiles, hipStream_t st);

// prefill tile GEMM over expert-sorted rows
struct TileArgs {
  const uint16_t* x;        // activation rows [*, K]
  const int32_t* lhs;       // virtual row r -> x row (lhs ? lhs[r / rpb] : (r / rpb) / lhs_div) * rpb + r % rpb
  int64_t lhs_div;
  int64_t rows_per_batch;   // rpb
  const int32_t* sorted_rhs;// expert per sorted row (naive mode)
  const int32_t* offsets;   // [E+1] (naive mode)
  const int32_t* tiles;     // [cap, 3] scheduled tiles
  const int32_t* n_tiles;   // device count
  int64_t P;                // sorted rows
  int E;
  const uint32_t* w0; const uint16_t* s0; const uint16_t* b0;
  const uint32_t* w1; const uint16_t* s1; const uint16_t* b1;
  // extra expert (index E in the tile table; tiles_mma only): the shared expert's matrices
  const uint32_t* xw0; const uint16_t* xs0; const uint16_t* xb0;
  const uint32_t* xw1; const uint16_t* xs1; const uint16_t* xb1;
  int N, K;
  uint16_t* out;            // [P, N]
  int bm; int tile_mode;    // 0 scheduled table, 1 naive (loop over experts), 2 dense (expert 0)
  int64_t grid_tiles;       // upper bound of the tile count (grid size)
  // second tile table (tiles_mma dual launch: tiles of at most 32 rows)
  const int32_t* tiles2; const int32_t* n_tiles2; int64_t grid_tiles2;
  const int32_t* xexp;      // tiles_mma gate/up: exponent of each fp16 activation row (indexed like x)
};
hipError_t launch_tiles(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st);
// 128-row tiles (tile_mode 0: table, 2: dense rows); grid_tiles = table capacity or row tiles
hipError_t launch_tiles_big(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st);
// tiles of at most 16 (bm <= 16) or 32 rows from a table (tile_mode 0); rows gathered through lhs
hipError_t launch_tiles_small(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st);
// tiles with register-dequantized weights on the matrix cores (tile_mode 0: table, 2: dense rows).
// GLU (gate/up): a.x holds the fp16 rows of launch_prep and a.xexp their exponents, gathered
// through a.lhs (or row r); otherwise a.x holds bf16 rows
bool tiles_mma_supported(int64_t K, int64_t N, int64_t src_rows, int gs);
// rows: 128 (tile table of up to 128-row tiles, or dense rows) or 32 (tiles of at most 32 rows)
hipError_t launch_tiles_mma(const TileArgs& a, int bits, int gs, bool glu, int rows, hipStream_t st);
// both tables in one launch: `tiles` (up to 128 rows, n_tiles) and `tiles2` (up to 32 rows, n_tiles2)
// bf16 expert matrices as the first MFMA operand (no dequantization): rows 64 or 32 (one table), 0 (both)
hipError_t launch_tiles_mma_w16(const TileArgs& a, bool glu, int rows, hipStream_t st);
hipError_t launch_tiles_mma_dual(const TileArgs& a, int bits, int gs, bool glu, hipStream_t st);
// x [T, H] bf16 -> xexp[t] (row exponent) and x16 = fp16(x * 2^-xexp) in the dequantizer's chunk
// order, the input of the gate/up pass; with gw (a [1, H] quantized row) also z[t] = bf16(x[t] . w)
hipError_t launch_prep(const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16, int32_t* xexp,
                       const uint32_t* gw, const uint16_t* gsc, const uint16_t* gbi, uint16_t* z, hipStream_t st);
// sort (SortArgs) and prep: one launch when the pairs fit one workgroup's
// sort, else the block sort with prep riding in its count launch
hipError_t launch_front(const SortArgs& sa, const uint16_t* x, int64_t T, int H, int bits, int gs, uint16_t* x16,
                        int32_t* xexp, const uint32_t* gw, const uint16_t* gsc, const uint16_t* gbi, uint16_t* z,
                        hipStream_t st);

// combine tail
// shared (nullable) rows [T, H] are added as they are, or, with z (nullable, [T] bf16), gated first:
// bf16(sigmoid(z[t]) * shared[t]) with the arithmetic of launch_sigmoid_gate
hipError_t launch_combine(const uint16_t* y, const int32_t* inv, const uint16_t* scores,
                          const uint16_t* shared, const uint16_t* z, int64_t T, int top_k, int64_t H,
                          uint16_t* out, hipStream_t st);
// scratch: 2 P H + T H elements (unsorted, weighted, summed), or with compact
// (P + T) H (the weighting writes over the unsorted copy, element by element)
hipError_t launch_combine_unfused(const uint16_t* y, const int32_t* inv, const uint16_t* scores,
                                  const uint16_t* shared, int64_t T, int top_k, int64_t H,
                                  uint16_t* out, uint16_t* scratch, hipStream_t st, bool compact = false);

// glue
hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t K, float eps,
                           uint16_t* out, hipStream_t st);
// router: idx [T, top_k] and bf16 scores from fp32 logits [T, E] (E <= 1024, top_k <= min(E, 64))
hipError_t launch_route(const float* logits, int64_t T, int E, int top_k, int32_t* idx, uint16_t* scores,
                        hipStream_t st);
hipError_t launch_sigmoid_gate(const uint16_t* s, const uint16_t* z, int64_t zs, int64_t T, int64_t H,
                               uint16_t* out, hipStream_t st);
hipError_t launch_kv_feed(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                          int64_t ldv, int64_t M, int64_t Nq, uint16_t* out, hipStream_t st);
// vector-unit products: weights without the transpose, float16/float32 activations
struct VecPlan {
  int MB, MBLK, WPL, NC, KS, kchunk;   // rows per block, blocks, codes per lane, column strips (row blocks), splits, K per split
  int64_t items;                       // waves
  size_t part_bytes;                   // fp32 partial sums (workspace) when KS > 1
};
// mode 0: affine codes (bits 1-6, 8); 1: mxfp4; 2: mxfp8
VecPlan vec_plan(int64_t P, int64_t M, int64_t N, int64_t K, int bits, int transpose, int mode = 0);
struct VecArgs {
  const void* x; int x_type;           // [X, M, K]; 0 bf16, 1 float16, 2 float32
  const int32_t* lhs; int64_t lhs_div; // x batch per pair (or p / lhs_div)
  const int32_t* rhs;                  // weight batch per pair (or 0)
  int64_t P; int M, N, K, gs;
  const uint32_t* w; const uint16_t* s; const uint16_t* b;   // mx modes: s holds E8M0 bytes, b unused
  int mode;                            // 0 affine, 1 mxfp4, 2 mxfp8
  void* out; int out_f32;              // [P, M, N] bf16 or float32
  float* part;                         // [KS, P, M, N] when KS > 1
  int MB, MBLK, WPL, NC, KS, kchunk;   // from vec_plan
  int64_t items;
};
hipError_t launch_qmm_vec(const VecArgs& a, int bits, int transpose, hipStream_t st);
hipError_t launch_iota(int32_t* dst, int64_t n, hipStream_t st);
// measured ceilings (diagnostics): a streaming read of `bytes` and a bf16 MFMA loop
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, hipStream_t st);
hipError_t launch_mfma_loop(int iters, int blocks, float* out, hipStream_t st);
hipError_t launch_validate(const int32_t* idx, int64_t n, int64_t E, int sorted, int32_t* flag,
                           hipStream_t st);
hipError_t launch_fill_selfcheck(uint16_t* y, int32_t* inv, uint16_t* scores, uint16_t* shared,
                                 int64_t T, int top_k, int64_t H, hipStream_t st);

}  // namespace moegq

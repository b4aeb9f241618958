// Expert sort of the (token, slot) pairs and the row-tile table.
//
// MTPLX PR 558 (Change): the sorted chain sorts the flattened pairs by expert
// and later un-sorts with the inverse permutation.  MLX PR 4567 (Proposed
// changes): per-expert offsets precomputed from the expert ids feed a row-tile
// scheduler whose tiles carry (row to start from, expert, valid rows).
//
// One workgroup of 1024 threads (the pair lists here are <= a few 10^5):
//  1. histogram of expert ids with LDS atomics (counts are order-free);
//  2. exclusive scan -> offsets, and per-expert tile counts -> tile offsets;
//  3. stable scatter in chunks of 1024 pairs.  Inside a wave, the lanes with
//     the same expert id are found from one ballot per key bit (no loop over
//     distinct keys); a lane's rank among them is a popcount of the lower
//     lanes.  Per-wave counts go to a small LDS table so each wave adds the
//     counts of the waves before it; a running cursor per expert carries the
//     chunks.  Every position is a function of the input only: deterministic.
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_MAXE = 1024;

// exclusive scan of one int per thread over the workgroup; returns the total
MOEGQ_DEV int block_excl_scan(int v, int* wtot, int& excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < SORT_WAVES; ++w) {
    const int t = wtot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  excl = before + incl - v;
  return total;
}

MOEGQ_DEV void write_tiles(int e, int cnt, int off, int toff, int bm, int32_t* tiles) {
  for (int j = 0; j * bm < cnt; ++j) {
    int32_t* t = tiles + 3 * (int64_t)(toff + j);
    t[0] = off + j * bm;
    t[1] = e;
    t[2] = min(bm, cnt - j * bm);
  }
}

__global__ __launch_bounds__(SORT_THREADS) void sort_kernel(SortArgs A) {
  __shared__ int cnt[SORT_MAXE];
  __shared__ int cursor[SORT_MAXE];
  __shared__ uint8_t tab[SORT_WAVES][SORT_MAXE];
  __shared__ int wtot[SORT_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = A.E;
  const int64_t P = A.P;
  for (int e = tid; e < SORT_MAXE; e += SORT_THREADS) {
    cnt[e] = 0;
    for (int w = 0; w < SORT_WAVES; ++w) tab[w][e] = 0;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // 1. histogram (ids outside [0, E) break the precondition; clamp to stay in
  //    bounds).  Lanes with equal ids are matched with one ballot per id bit and
  //    only the first of them adds the group's count: no atomic contention on
  //    popular experts.
  for (int64_t base = 0; base < P; base += SORT_THREADS) {
    const int64_t p = base + tid;
    const bool valid = p < P;
    const int e = valid ? min(max(A.idx[p], 0), E - 1) : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    if (valid && __popcll(match & lt_mask) == 0) atomicAdd(&cnt[e], (int)__popcll(match));
  }
  __syncthreads();
  // 2. scans (E <= SORT_MAXE == SORT_THREADS: one expert per thread)
  const int c = tid < E ? cnt[tid] : 0;
  int off;
  block_excl_scan(c, wtot, off);
  const bool hybrid = A.tile_mode == 3;
  const bool is_big = !hybrid || c >= A.small_max;
  const int ntile = (A.bm > 0 && is_big) ? (c + A.bm - 1) / A.bm : 0;
  int toff;
  const int total_tiles = block_excl_scan(ntile, wtot, toff);
  const int nsmall = (hybrid && c > 0 && !is_big) ? 1 : 0;
  int soff;
  const int total_small = block_excl_scan(nsmall, wtot, soff);
  if (tid < E) {
    A.counts[tid] = c;
    A.offsets[tid] = off;
    cursor[tid] = off;
    if (A.tiles && (A.tile_mode == 0 || (hybrid && is_big))) write_tiles(tid, c, off, toff, A.bm, A.tiles);
    if (A.small_tiles && nsmall) {
      int32_t* t = A.small_tiles + 3 * soff;
      t[0] = off; t[1] = tid; t[2] = c;
    }
  }
  if (tid == 0) {
    A.offsets[E] = (int32_t)P;
    if (A.n_tiles) {
      A.n_tiles[0] = (A.tile_mode == 0 || hybrid) ? total_tiles : (int32_t)((P + A.bm - 1) / A.bm);
      if (hybrid) A.n_tiles[1] = total_small;
    }
  }
  if (A.tiles && A.tile_mode == 1) {
    const int64_t nt = (P + A.bm - 1) / A.bm;
    for (int64_t t = tid; t < nt; t += SORT_THREADS) {
      A.tiles[3 * t] = (int32_t)(t * A.bm);
      A.tiles[3 * t + 1] = -1;
      A.tiles[3 * t + 2] = (int32_t)min((int64_t)A.bm, P - t * A.bm);
    }
  }
  __syncthreads();
  // 3. stable scatter
  for (int64_t base = 0; base < P; base += SORT_THREADS) {
    const int64_t p = base + tid;
    const bool valid = p < P;
    const int e = valid ? min(max(A.idx[p], 0), E - 1) : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) tab[wave][e] = (uint8_t)__popcll(match);
    __syncthreads();
    if (valid) {
      int pos = cursor[e] + rank;
      for (int w = 0; w < wave; ++w) pos += tab[w][e];
      if (A.order) A.order[pos] = (int32_t)p;
      if (A.lhs) A.lhs[pos] = (int32_t)(p / A.top_k);
      if (A.sorted_rhs) A.sorted_rhs[pos] = e;
      A.inv[p] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += SORT_THREADS) {
      int s = 0;
      for (int w = 0; w < SORT_WAVES; ++w) { s += tab[w][ee]; tab[w][ee] = 0; }
      cursor[ee] += s;
    }
    __syncthreads();
  }
}

hipError_t launch_sort(const SortArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(SORT_THREADS), 0, st, a);
  return hipGetLastError();
}

// stand-alone schedule from offsets
__global__ __launch_bounds__(SORT_THREADS) void schedule_kernel(const int32_t* offsets, int E, int bm,
                                                                int tile_mode, int32_t* tiles,
                                                                int32_t* n_tiles) {
  __shared__ int wtot[SORT_WAVES];
  const int tid = threadIdx.x;
  const int P = offsets[E];
  if (tile_mode == 1) {
    const int nt = (P + bm - 1) / bm;
    for (int t = tid; t < nt; t += SORT_THREADS) {
      tiles[3 * t] = t * bm;
      tiles[3 * t + 1] = -1;
      tiles[3 * t + 2] = min(bm, P - t * bm);
    }
    if (tid == 0) *n_tiles = nt;
    return;
  }
  const int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int nt = (c + bm - 1) / bm;
  int toff;
  const int total = block_excl_scan(nt, wtot, toff);
  if (tid < E) write_tiles(tid, c, offsets[tid], toff, bm, tiles);
  if (tid == 0) *n_tiles = total;
}

hipError_t launch_schedule(const int32_t* offsets, int E, int bm, int tile_mode, int32_t* tiles,
                           int32_t* n_tiles, hipStream_t st) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SORT_THREADS), 0, st, offsets, E, bm, tile_mode,
                     tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace moegq

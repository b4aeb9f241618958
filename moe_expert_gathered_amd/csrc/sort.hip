// Expert sort of the (token, slot) pairs and the row-tile table.
//
// MTPLX PR 558 (Change): the sorted chain sorts the flattened pairs by expert
// and later un-sorts with the inverse permutation.  MLX PR 4567 (Proposed
// changes): per-expert offsets precomputed from the expert ids feed a row-tile
// scheduler whose tiles carry (row to start from, expert, valid rows).
//
// Three launches, each pair list split in blocks of 1024 pairs:
//  1. count: a per-block histogram of expert ids.  Lanes of a wave holding
//     the same id are matched with one ballot per id bit, and only the first
//     of them adds the group's count (one LDS atomic per distinct id per wave).
//  2. scan (one workgroup, one expert per thread): counts, exclusive offsets,
//     the base row of every (block, expert) for the stable scatter, and the
//     tile tables.
//  3. scatter: each pair's rank among the equal ids of its block is the
//     popcount of the matched lower lanes plus the counts of the lower waves
//     (per-wave LDS table); its row is the (block, expert) base plus that rank.
//     Rows depend on the input only: the sort is stable and deterministic.
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_MAXE = 1024;

int64_t sort_blocks(int64_t P) { return (P + SORT_THREADS - 1) / SORT_THREADS; }

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

// Lanes of this wave whose key equals this lane's key (keys < 2^nbits; invalid
// lanes are excluded).
MOEGQ_DEV uint64_t match_key(int key, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

MOEGQ_DEV int key_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

__global__ __launch_bounds__(SORT_THREADS) void sort_count_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                                  int32_t* __restrict__ bc) {
  __shared__ int cnt[SORT_MAXE];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < E; e += SORT_THREADS) cnt[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * SORT_THREADS + tid;
  const bool valid = p < P;
  // ids outside [0, E) break the precondition; clamp to stay in bounds
  const int e = valid ? min(max(idx[p], 0), E - 1) : 0;
  const uint64_t m = match_key(e, valid, key_bits(E));
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (valid && __popcll(m & lt) == 0) atomicAdd(&cnt[e], (int)__popcll(m));
  __syncthreads();
  for (int ee = tid; ee < E; ee += SORT_THREADS) bc[(int64_t)blockIdx.x * E + ee] = cnt[ee];
}

__global__ __launch_bounds__(SORT_THREADS) void sort_scan_kernel(SortArgs A, int nblk) {
  __shared__ int wtot[SORT_WAVES];
  const int tid = threadIdx.x;
  const int E = A.E;
  const int64_t P = A.P;
  // counts (16 independent loads in flight per batch)
  int c = 0;
  if (tid < E) {
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = b0 + j < nblk ? A.block_counts[(int64_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) c += v[j];
    }
  }
  int off;
  block_excl_scan(c, wtot, off);
  // per-block bases: the expert's first row plus the counts of the blocks before
  if (tid < E) {
    int run = off;
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = b0 + j < nblk ? A.block_counts[(int64_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nblk) A.block_counts[(int64_t)(b0 + j) * E + tid] = run;
        run += v[j];
      }
    }
  }
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
    if (A.tiles && (A.tile_mode == 0 || (hybrid && is_big))) write_tiles(tid, c, off, toff, A.bm, A.tiles);
    if (A.small_tiles && nsmall) {
      int32_t* t = A.small_tiles + 3 * soff;
      t[0] = off; t[1] = tid; t[2] = c;
    }
  }
  // the extra expert's tiles follow the routed ones
  const int extra_tiles = (A.extra_rows > 0 && A.tiles && A.bm > 0) ? (int)((A.extra_rows + A.bm - 1) / A.bm) : 0;
  for (int j = tid; j < extra_tiles; j += SORT_THREADS) {
    int32_t* t = A.tiles + 3 * (int64_t)(total_tiles + j);
    t[0] = (int32_t)(P + (int64_t)j * A.bm);
    t[1] = E;
    t[2] = (int32_t)min((int64_t)A.bm, A.extra_rows - (int64_t)j * A.bm);
  }
  if (A.lhs)
    for (int64_t t = tid; t < A.extra_rows; t += SORT_THREADS) A.lhs[P + t] = (int32_t)t;
  if (tid == 0) {
    A.offsets[E] = (int32_t)P;
    if (A.n_tiles) {
      A.n_tiles[0] = (A.tile_mode == 0 || hybrid) ? total_tiles + extra_tiles : (int32_t)((P + A.bm - 1) / A.bm);
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
}

__global__ __launch_bounds__(SORT_THREADS) void sort_scatter_kernel(SortArgs A) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[SORT_WAVES][SORT_MAXE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = A.E;
  reinterpret_cast<uint4*>(&tab[0][0])[tid] = make_uint4(0, 0, 0, 0);   // 16 KiB = 1024 x 16 B
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * SORT_THREADS + tid;
  const bool valid = p < A.P;
  const int e = valid ? min(max(A.idx[p], 0), E - 1) : 0;
  const uint64_t m = match_key(e, valid, key_bits(E));
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(m & lt);
  if (valid && rank == 0) tab[wave][e] = (uint8_t)__popcll(m);
  __syncthreads();
  if (!valid) return;
  int pos = A.block_counts[(int64_t)blockIdx.x * E + e] + rank;
  for (int w = 0; w < wave; ++w) pos += tab[w][e];
  if (A.order) A.order[pos] = (int32_t)p;
  if (A.lhs) A.lhs[pos] = (int32_t)(p / A.top_k);
  if (A.sorted_rhs) A.sorted_rhs[pos] = e;
  A.inv[p] = pos;
}

hipError_t launch_sort(const SortArgs& a, hipStream_t st) {
  if (a.E <= 0 || a.E > SORT_MAXE || (!a.block_counts && a.P > 0)) return hipErrorInvalidValue;
  const int64_t nb = sort_blocks(a.P);
  if (nb > 0) {
    hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)nb), dim3(SORT_THREADS), 0, st, a.idx, a.P, a.E,
                       a.block_counts);
  }
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(SORT_THREADS), 0, st, a, (int)nb);
  if (nb > 0) hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)nb), dim3(SORT_THREADS), 0, st, a);
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

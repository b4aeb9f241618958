// Expert sort of the (token, slot) pairs and the row-tile tables: the
// kernels and their launcher (the device code is in sort_dev.h).
//
// Up to SORT_ONE_MAX_P pairs: one workgroup does everything.  Beyond: two
// launches over blocks of 1024 pairs:
//  1. count: a per-block histogram of expert ids (one LDS atomic per distinct
//     id per wave, after ballot matching);
//  2. rank: every block reads all the histograms (one expert per thread), so
//     it has each expert's total, its exclusive offset (a workgroup scan) and
//     the block's base row per expert (the counts of the blocks before it);
//     a pair's row is that base plus its rank inside the block.  Block 0 also
//     writes counts, offsets and the tile tables.
#include "sort_dev.h"

namespace moegq {

int64_t sort_blocks(int64_t P) { return (P + SORT_THREADS - 1) / SORT_THREADS; }

__global__ __launch_bounds__(SORT_THREADS) void sort_count_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                                  int32_t* __restrict__ bc) {
  sort_count_block(idx, P, E, bc, blockIdx.x);
}

__global__ __launch_bounds__(SORT_THREADS) void sort_rank_kernel(SortArgs A, int nblk) {
  __shared__ int wtot[SORT_WAVES];
  __shared__ int base[SORT_MAXE];
  __shared__ __attribute__((aligned(16))) uint8_t tab[SORT_WAVES][SORT_MAXE];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int E = A.E;
  const int blk = blockIdx.x;
  reinterpret_cast<uint4*>(&tab[0][0])[tid] = make_uint4(0, 0, 0, 0);   // 16 KiB = 1024 x 16 B
  // expert tid: its total over all blocks and over the blocks before this one
  // (16 independent loads in flight per batch)
  int c = 0, before = 0;
  if (tid < E) {
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = b0 + j < nblk ? A.block_counts[(int64_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        c += v[j];
        before += b0 + j < blk ? v[j] : 0;
      }
    }
  }
  int off;
  block_excl_scan(c, wtot, off);   // synchronises: tab is clear after it
  if (tid < E) base[tid] = off + before;
  if (blk == 0) finish_tables(A, c, off, wtot);
  const int64_t p = (int64_t)blk * SORT_THREADS + tid;
  const bool valid = p < A.P;
  const int e = valid ? min(max(A.idx[p], 0), E - 1) : 0;
  const uint64_t m = match_key(e, valid, key_bits(E));
  const int rank = __popcll(m & lanes_below());
  if (valid && rank == 0) tab[wave][e] = (uint8_t)__popcll(m);
  __syncthreads();
  if (!valid) return;
  int pos = base[e] + rank;
  for (int w = 0; w < wave; ++w) pos += tab[w][e];
  write_pair(A, p, e, pos);
}

__global__ __launch_bounds__(SORT_THREADS) void sort_one_kernel(SortArgs A) { sort_one_block(A); }

hipError_t launch_sort_rest(const SortArgs& a, hipStream_t st) {
  const int64_t nb = sort_blocks(a.P);
  // block 0 writes the tables, so the launch has at least one block
  hipLaunchKernelGGL(sort_rank_kernel, dim3((unsigned)(nb > 0 ? nb : 1)), dim3(SORT_THREADS), 0, st, a, (int)nb);
  return hipGetLastError();
}

hipError_t launch_sort(const SortArgs& a, hipStream_t st) {
  if (a.E <= 0 || a.E > SORT_MAXE || (!a.block_counts && a.P > 0)) return hipErrorInvalidValue;
  if (a.P <= SORT_ONE_MAX_P) {
    hipLaunchKernelGGL(sort_one_kernel, dim3(1), dim3(SORT_THREADS), 0, st, a);
    return hipGetLastError();
  }
  const int64_t nb = sort_blocks(a.P);
  hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)nb), dim3(SORT_THREADS), 0, st, a.idx, a.P, a.E,
                     a.block_counts);
  return launch_sort_rest(a, st);
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

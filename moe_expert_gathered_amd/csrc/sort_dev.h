// Device side of the expert sort of the (token, slot) pairs and of the
// row-tile tables (1024-thread workgroups).
//
// MTPLX PR 558 (Change): the sorted chain sorts the flattened pairs by expert
// and later un-sorts with the inverse permutation.  MLX PR 4567 (Proposed
// changes): per-expert offsets precomputed from the expert ids feed a row-tile
// scheduler whose tiles carry (row to start from, expert, valid rows).
//
// Ranking: lanes of a wave holding the same id are matched with one ballot per
// id bit; a pair's rank among the equal ids before it is the popcount of the
// matched lower lanes plus the counts of the pairs of that id earlier in the
// input (earlier waves' chunks, or earlier blocks and lower waves).  Rows
// depend on the input only: the sort is stable and deterministic.
#pragma once
#include "common.h"
#include "launch.h"

namespace moegq {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_MAXE = 1024;
// pairs one workgroup sorts alone (each wave holds up to 4 ids per lane); more
// pairs go to the block sort, which spreads the ranking over many compute units
constexpr int SORT_ONE_ROUNDS = 4;
constexpr int64_t SORT_ONE_MAX_P = (int64_t)SORT_ONE_ROUNDS * SORT_THREADS;

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

MOEGQ_DEV uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---- hybrid schedule (tile_mode 3): an expert with fewer than theta rows
//      gets small_max-row tiles, a larger one bm-row tiles.
struct HybridSplit { int nbig, nsmall, big_rows; };
MOEGQ_DEV HybridSplit hybrid_split(int c, int theta, int bm, int sm) {
  if (c <= 0) return {0, 0, 0};
  if (c < theta) return {0, (c + sm - 1) / sm, 0};
  return {(c + bm - 1) / bm, 0, c};
}

// theta = small_max, except when the bm-row tiles of that choice would give
// the first pass (cost_nb column blocks per tile) at most cost_slots / 8 work
// items: those few long items would then set the pass time while most of the
// machine idles, so every expert gets small tiles (theta = infinity).  Every
// thread of the block calls this (it synchronises); c is the thread's count.
MOEGQ_DEV int choose_theta(const SortArgs& A, int c, bool valid) {
  __shared__ int part[SORT_WAVES];
  __shared__ int theta_s;
  if (A.cost_slots <= 0) return A.small_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int nb = valid ? hybrid_split(c, A.small_max, A.bm, A.small_max).nbig : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nb += __shfl_xor(nb, off, 64);
  if (lane == 0) part[wave] = nb;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t tiles = hybrid_split((int)A.extra_rows, A.small_max, A.bm, A.small_max).nbig;
    for (int w = 0; w < SORT_WAVES; ++w) tiles += part[w];
    theta_s = tiles * A.cost_nb > A.cost_slots / 8 ? A.small_max : 0x7FFFFFFF;
  }
  __syncthreads();
  return theta_s;
}

// Given every expert's count c and first row off (thread e < E holds expert
// e), write counts, offsets, the tile tables (with the extra expert's tiles
// after the routed ones), the identity lhs of the extra rows and n_tiles.
// Every thread of the block calls this.
MOEGQ_DEV void finish_tables(const SortArgs& A, int c, int off, int* wtot) {
  const int tid = threadIdx.x;
  const int E = A.E;
  const int64_t P = A.P;
  const bool hybrid = A.tile_mode == 3;
  HybridSplit hs{0, 0, 0};
  int theta = 0;
  if (hybrid) {
    theta = choose_theta(A, c, tid < E);
    hs = hybrid_split(c, theta, A.bm, A.small_max);
  }
  const int ntile = hybrid ? hs.nbig : (A.bm > 0 ? (c + A.bm - 1) / A.bm : 0);
  int toff;
  const int total_tiles = block_excl_scan(ntile, wtot, toff);
  int soff;
  const int total_small = block_excl_scan(hs.nsmall, wtot, soff);
  if (tid < E) {
    A.counts[tid] = c;
    A.offsets[tid] = off;
    if (A.tiles && A.tile_mode == 0) write_tiles(tid, c, off, toff, A.bm, A.tiles);
    if (hybrid) {
      if (A.tiles) write_tiles(tid, hs.big_rows, off, toff, A.bm, A.tiles);
      if (A.small_tiles) write_tiles(tid, c - hs.big_rows, off + hs.big_rows, soff, A.small_max, A.small_tiles);
    }
  }
  // the extra expert's rows are split by the same rule as a routed expert's
  int extra_big = 0, extra_small = 0, extra_big_rows = 0;
  if (A.extra_rows > 0 && A.bm > 0) {
    if (hybrid) {
      const HybridSplit xs = hybrid_split((int)A.extra_rows, theta, A.bm, A.small_max);
      extra_big = xs.nbig; extra_small = xs.nsmall; extra_big_rows = xs.big_rows;
    } else {
      extra_big = (int)((A.extra_rows + A.bm - 1) / A.bm);
      extra_big_rows = (int)A.extra_rows;
    }
  }
  if (A.tiles)
    for (int j = tid; j < extra_big; j += SORT_THREADS) {
      int32_t* t = A.tiles + 3 * (int64_t)(total_tiles + j);
      t[0] = (int32_t)(P + (int64_t)j * A.bm);
      t[1] = E;
      t[2] = min(A.bm, extra_big_rows - j * A.bm);
    }
  if (A.small_tiles)
    for (int j = tid; j < extra_small; j += SORT_THREADS) {
      int32_t* t = A.small_tiles + 3 * (int64_t)(total_small + j);
      t[0] = (int32_t)(P + extra_big_rows + (int64_t)j * A.small_max);
      t[1] = E;
      t[2] = (int32_t)min((int64_t)A.small_max, A.extra_rows - extra_big_rows - (int64_t)j * A.small_max);
    }
  if (A.lhs)
    for (int64_t t = tid; t < A.extra_rows; t += SORT_THREADS) A.lhs[P + t] = (int32_t)t;
  if (tid == 0) {
    A.offsets[E] = (int32_t)P;
    if (A.n_tiles) {
      A.n_tiles[0] = (A.tile_mode == 0 || hybrid) ? total_tiles + extra_big : (int32_t)((P + A.bm - 1) / A.bm);
      if (hybrid) A.n_tiles[1] = total_small + extra_small;
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

// Block blk of the block sort: the histogram of its 1024 pairs' expert ids
// into bc[blk][0 .. E).
MOEGQ_DEV void sort_count_block(const int32_t* __restrict__ idx, int64_t P, int E, int32_t* __restrict__ bc,
                                int64_t blk) {
  __shared__ int cnt[SORT_MAXE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += SORT_THREADS) cnt[e] = 0;
  __syncthreads();
  const int64_t p = blk * SORT_THREADS + tid;
  const bool valid = p < P;
  // ids outside [0, E) break the precondition; clamp to stay in bounds
  const int e = valid ? min(max(idx[p], 0), E - 1) : 0;
  const uint64_t m = match_key(e, valid, key_bits(E));
  if (valid && __popcll(m & lanes_below()) == 0) atomicAdd(&cnt[e], (int)__popcll(m));
  __syncthreads();
  for (int ee = tid; ee < E; ee += SORT_THREADS) bc[blk * E + ee] = cnt[ee];
}

MOEGQ_DEV void write_pair(const SortArgs& A, int64_t p, int e, int pos) {
  if (A.order) A.order[pos] = (int32_t)p;
  if (A.lhs) A.lhs[pos] = (int32_t)(p / A.top_k);
  if (A.sorted_rhs) A.sorted_rhs[pos] = e;
  A.inv[p] = pos;
}

// The whole sort in one workgroup for P <= SORT_ONE_MAX_P.  Wave w owns the
// contiguous chunk of pairs [w C, (w + 1) C) (C a multiple of 64), walked 64
// pairs at a time.  cnt[e][w] first counts expert e in chunk w; then it holds
// the row of chunk w's next pair of expert e (the expert's first row plus the
// chunk counts of the waves before), which only wave w reads and advances: no
// workgroup barrier inside the walks.  Rows are at most SORT_ONE_MAX_P < 2^16:
// 16 bits hold them.
static_assert(SORT_ONE_MAX_P < 65536, "16-bit rows");
MOEGQ_DEV void sort_one_block(const SortArgs& A) {
  __shared__ __attribute__((aligned(16))) uint16_t cnt[SORT_MAXE][SORT_WAVES];
  __shared__ int wtot[SORT_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = A.E;
  const int64_t P = A.P;
  const int nbits = key_bits(E);
  const int C = (int)(((P + SORT_WAVES - 1) / SORT_WAVES + 63) / 64 * 64);   // pairs per wave
  const int iters = C / 64;                                                  // <= SORT_ONE_ROUNDS
  const int64_t p0 = (int64_t)wave * C + lane;
  const uint64_t lt = lanes_below();
  reinterpret_cast<uint4*>(&cnt[0][0])[tid] = make_uint4(0, 0, 0, 0);         // 32 KiB = 2 x 1024 x 16 B
  reinterpret_cast<uint4*>(&cnt[0][0])[tid + SORT_THREADS] = make_uint4(0, 0, 0, 0);
  int ids[SORT_ONE_ROUNDS];
#pragma unroll
  for (int it = 0; it < SORT_ONE_ROUNDS; ++it) {
    const int64_t p = p0 + 64 * it;
    // ids outside [0, E) break the precondition; clamp to stay in bounds
    ids[it] = (it < iters && p < P) ? min(max(A.idx[p], 0), E - 1) : 0;
  }
  __syncthreads();
  // chunk counts: one LDS atomic per pair on the 32-bit word that holds the
  // 16-bit counters of waves 2 k and 2 k + 1 (a counter stays below 2^16, so
  // no carry crosses into the neighbour)
  uint32_t* cnt32 = reinterpret_cast<uint32_t*>(&cnt[0][0]);
  const uint32_t inc = 1u << (16 * (wave & 1));
#pragma unroll
  for (int it = 0; it < SORT_ONE_ROUNDS; ++it) {
    if (it >= iters) break;
    if (p0 + 64 * it < P) atomicAdd(cnt32 + ids[it] * (SORT_WAVES / 2) + (wave >> 1), inc);
  }
  __syncthreads();
  // expert totals, offsets, and each chunk's first row per expert
  uint4 cv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  int c = 0;
  if (tid < E) {
    cv[0] = reinterpret_cast<const uint4*>(&cnt[tid][0])[0];
    cv[1] = reinterpret_cast<const uint4*>(&cnt[tid][0])[1];
    const uint32_t* d = &cv[0].x;
#pragma unroll
    for (int i = 0; i < 8; ++i) c += (int)(d[i] & 0xFFFFu) + (int)(d[i] >> 16);
  }
  int off;
  block_excl_scan(c, wtot, off);
  if (tid < E) {
    uint32_t* d = &cv[0].x;
    int run = off;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lo = (int)(d[i] & 0xFFFFu), hi = (int)(d[i] >> 16);
      d[i] = (uint32_t)run | ((uint32_t)(run + lo) << 16);
      run += lo + hi;
    }
    reinterpret_cast<uint4*>(&cnt[tid][0])[0] = cv[0];
    reinterpret_cast<uint4*>(&cnt[tid][0])[1] = cv[1];
  }
  finish_tables(A, c, off, wtot);   // synchronises: the rows above are visible after it
  // rows
#pragma unroll
  for (int it = 0; it < SORT_ONE_ROUNDS; ++it) {
    if (it >= iters) break;
    const int64_t p = p0 + 64 * it;
    const bool valid = p < P;
    const int e = ids[it];
    const uint64_t m = match_key(e, valid, nbits);
    const int rank = __popcll(m & lt);
    const int pos = (int)cnt[e][wave] + rank;
    if (valid) write_pair(A, p, e, pos);
    if (valid && rank == 0) cnt[e][wave] = (uint16_t)(pos + __popcll(m));
  }
}

}  // namespace moegq

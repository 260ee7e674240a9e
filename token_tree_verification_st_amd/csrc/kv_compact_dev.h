// Device body of the accepted-path KV compaction (the depth-first KV-cache
// update of the SpecInfer news article, "Token 樹驗證器"): slot P + j of every
// kv head takes what slot P + path[j] held before, for j = 0..L.  Shared by
// st_kv_compact and by the last launch of st_verification_step, where each
// compaction workgroup can also run the walk (greedy or stochastic) that
// yields the path.
//
// The copy is in place.  A path strictly increases (path[j] >= j), so the
// source of a later move is never the destination of an earlier one.  One
// 256-thread workgroup moves the rows of one (request, cache, head): a batch
// of moves first reads all of its sources, then (after a barrier) writes all
// of its destinations, so within a batch no source is overwritten before it
// is read, and later batches read only slots no earlier move wrote.
#pragma once
#include "greedy_walk_dev.h"
#include "stoch_walk_dev.h"

namespace st {

struct CompactArgs {
  int B, Hkv, S_max, chunks;  // chunks: 16-byte pieces per cache row (<= 256)
  uint4* kc;
  uint4* vc;
  const int32_t* prefix_len;
  const int32_t* accept_len;
  const int32_t* accept_nodes;
  int max_path;
  int32_t* src_slot;
  int32_t* new_len;
  int32_t* status;
  KvPaging pg;          // block table of a paged pool (pg.bt null: contiguous caches)
  int walk;             // 0: the path is in accept_len / accept_nodes; 1: run the
  GreedyWalkArgs g;     // greedy walk with these inputs (the argmax partials);
  StochWalkArgs sw;     // 2: the stochastic walk over these node verdicts
};

enum { kWalkNone = 0, kWalkGreedy = 1, kWalkStochastic = 2 };

// Row `slot` of (request b, kv head) in 16-byte pieces: contiguous, or through
// the block table (an entry outside the pool is clamped and flagged).
__device__ inline uint4* kv_row_ptr(const CompactArgs& c, uint4* cache, int b, int head,
                                    int slot) {
  if (!c.pg.bt) return cache + (((size_t)b * c.Hkv + head) * c.S_max + slot) * c.chunks;
  const int e = c.pg.bt[(size_t)b * c.pg.bt_stride + (slot >> c.pg.lbs)];
  const int phys = min(max(e, 0), c.pg.n_blocks - 1);
  if (phys != e) st::set_status(c.status, ST_STATUS_BAD_BLOCK);
  return cache +
         ((((size_t)phys * c.Hkv + head) << c.pg.lbs) + (slot & ((1 << c.pg.lbs) - 1))) * c.chunks;
}

// Moves of one workgroup (blockDim.x == 256): request b, cache row set y
// (< Hkv: keys of head y, else values of head y - Hkv), path[0..L] of the
// accepted path (global or LDS).  Row set 0 also stores src_slot / new_len.
__device__ inline void kv_compact_rows(const CompactArgs& c, int b, int y, int L,
                                       const int* path) {
  const int P = c.prefix_len[b];
  int bad = 0;
  if (L < 0 || L + 1 > c.max_path || P < 0) {
    bad = ST_STATUS_PATH_OVERFLOW;
  } else {
    for (int j = 0; j <= L; ++j) {
      const int n = path[j];
      if (n < 0 || (long)P + n >= c.S_max || (j > 0 && n <= path[j - 1])) bad = ST_STATUS_BAD_PARENT;
    }
  }
  if (y == 0 && threadIdx.x == 0) {
    for (int j = 0; j < c.max_path; ++j)
      c.src_slot[(size_t)b * c.max_path + j] = (!bad && j <= L) ? P + path[j] : -1;
    c.new_len[b] = bad ? P : P + L + 1;
    st::set_status(c.status, bad);
  }
  if (bad) return;
  const int head = y % c.Hkv;
  uint4* cache = y < c.Hkv ? c.kc : c.vc;
  const int per_pass = 256 / c.chunks;
  const int col = threadIdx.x % c.chunks, jr = threadIdx.x / c.chunks;
  for (int j0 = 0; j0 <= L; j0 += per_pass) {
    const int j = j0 + jr;
    const bool move = jr < per_pass && j <= L && path[min(j, L)] != j;
    uint4 v;
    if (move) v = kv_row_ptr(c, cache, b, head, P + path[j])[col];
    __syncthreads();
    if (move) kv_row_ptr(c, cache, b, head, P + j)[col] = v;
    __syncthreads();
  }
}

// One compaction workgroup: the path comes from accept_len / accept_nodes,
// or from the walk that the first wavefront runs here; row set 0's
// workgroup also stores the walk's outputs.
__device__ inline void kv_compact_block(const CompactArgs& c, int b, int y) {
  if (c.walk == kWalkNone) {
    kv_compact_rows(c, b, y, c.accept_len[b], c.accept_nodes + (size_t)b * c.max_path);
    return;
  }
  __shared__ union {
    GreedyWalkLds gr;
    StochWalkLds sw;
  } s;
  __shared__ int sL;
  if (threadIdx.x < ST_WAVE) {
    const int L = c.walk == kWalkGreedy ? greedy_walk_wave(c.g, b, s.gr, y == 0)
                                        : stoch_walk_wave(c.sw, b, s.sw, y == 0);
    if (threadIdx.x == 0) sL = L;
  }
  __syncthreads();
  kv_compact_rows(c, b, y, sL, c.walk == kWalkGreedy ? s.gr.path : s.sw.path);
}

}  // namespace st

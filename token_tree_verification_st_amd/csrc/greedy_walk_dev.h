// Device pieces of greedy acceptance shared by st_verify_greedy and the
// one-call step (SpecInfer developer article §2.1: the longest path whose
// every token equals the target's choice after its parent).
#pragma once
#include "st_internal.h"

#include <limits.h>

namespace st {

// (value, index) argmax with the lowest index on equal values; NaN never wins.
struct ArgmaxPart {
  float v;
  int i;
};
__device__ inline void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

constexpr int kMaxPath = ST_MAX_NODES;

// accept_nodes / out_tokens / accept_len of request b, written by threads
// tid = 0..nthreads-1.
__device__ inline void write_path_outputs(int tid, int nthreads, int b, int L, int max_depth,
                                          const int* path, const int32_t* tokens, int lo,
                                          int last_token, int32_t* accept_len,
                                          int32_t* accept_nodes, int32_t* out_tokens) {
  const int mp = max_depth + 1;
  for (int j = tid; j <= mp; j += nthreads) {
    if (j < mp) accept_nodes[(size_t)b * mp + j] = j <= L ? path[j] : -1;
    int tok = -1;
    if (j < L) tok = tokens[lo + path[j + 1]];
    else if (j == L) tok = last_token;
    out_tokens[(size_t)b * (mp + 1) + j] = tok;
  }
  if (tid == 0) accept_len[b] = L;
}

struct GreedyWalkArgs {
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* tokens;
  const ArgmaxPart* part;  // [T][nslices] vocab-slice maxima of every node
  int nslices, T, V, max_nodes, max_depth;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  int32_t* status;
};

struct GreedyWalkLds {
  int path[kMaxPath + 1];
  int sp[ST_MAX_NODES], stok[ST_MAX_NODES], sa[ST_MAX_NODES];
};

// LDS ordering inside one wavefront (the other wavefronts of the workgroup
// may be doing something else).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Greedy walk of request b by one whole wavefront: merge each node's slice
// maxima into its argmax a[i], then from the root step to the lowest-index
// child c with tokens[c] == a[u] until none matches (at most max_depth steps).
// The path is left in s.path; returns L, or -1 for a request whose node range
// is invalid.  With `write` the wavefront also stores the path outputs and
// the status bits.
__device__ inline int greedy_walk_wave(const GreedyWalkArgs& g, int b, GreedyWalkLds& s,
                                       bool write) {
  const int lane = threadIdx.x % ST_WAVE;
  const int lo = g.node_off[b], hi = g.node_off[b + 1], n = hi - lo;
  if (lo < 0 || hi > g.T || n < 1 || n > g.max_nodes) {
    if (write && lane == 0) set_status(g.status, ST_STATUS_BAD_PARENT);
    return -1;
  }
  int bits = 0;
  for (int i = lane; i < n; i += ST_WAVE) {
    const int p = g.parent[lo + i], tok = g.tokens[lo + i];
    s.sp[i] = p;
    s.stok[i] = tok;
    if (i == 0 ? (p != -1) : (p < 0 || p >= i)) bits |= ST_STATUS_BAD_PARENT;
    if (i > 0 && (tok < 0 || tok >= g.V)) bits |= ST_STATUS_BAD_TOKEN;
    const ArgmaxPart* pp = g.part + (size_t)(lo + i) * g.nslices;
    float bv = pp[0].v;
    int bi = pp[0].i;
    for (int k = 1; k < g.nslices; ++k) argmax_merge(bv, bi, pp[k].v, pp[k].i);
    s.sa[i] = (bi == INT_MAX) ? 0 : bi;
  }
  for (int o = 32; o > 0; o >>= 1) bits |= __shfl_xor(bits, o, ST_WAVE);
  if (write && lane == 0) set_status(g.status, bits);
  wave_lds_sync();

  int u = 0, L = 0;
  bool overflow = false;
  if (lane == 0) s.path[0] = 0;
  while (true) {
    const int a = s.sa[u];
    int found = -1;
    // children of u have larger indices; the lowest matching index wins
    for (int c0 = u + 1; c0 < n && found < 0; c0 += ST_WAVE) {
      const int c = c0 + lane;
      const bool hit = c < n && s.sp[c] == u && s.stok[c] == a;
      const uint64_t m = __ballot(hit);
      if (m) found = c0 + __ffsll((unsigned long long)m) - 1;
    }
    if (found < 0) break;
    if (L == g.max_depth) {
      overflow = true;
      break;
    }
    ++L;
    if (lane == 0) s.path[L] = found;
    u = found;
  }
  wave_lds_sync();
  if (write) {
    if (overflow && lane == 0) set_status(g.status, ST_STATUS_PATH_OVERFLOW);
    write_path_outputs(lane, ST_WAVE, b, L, g.max_depth, s.path, g.tokens, lo,
                       overflow ? -1 : s.sa[u], g.accept_len, g.accept_nodes, g.out_tokens);
  }
  return L;
}

}  // namespace st

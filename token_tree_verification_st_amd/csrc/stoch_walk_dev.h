// Device body of the stochastic walk (speculative-decoding explainer §2.2:
// check candidates left to right, stop at the first rejection and emit a
// replacement token): every node's outcome was decided beforehand (the node
// kernel in verify.hip), so a walk only follows accepted children from the
// root.  Run by st_verify_stochastic's walk kernel and, in the one-call step,
// by the compaction workgroups, which need the path anyway.
#pragma once
#include "greedy_walk_dev.h"

namespace st {

// What the walk needs from a node: its first accepted child (local index, -1
// if none), the near ties among its tests and, when no child is accepted, the
// replacement token drawn there and whether that draw was a near tie.
struct NodeVerdict {
  int accepted, ties, token, token_tie;
};

struct StochWalkArgs {
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* tokens;
  const NodeVerdict* verdict;  // [T]
  int T, V, max_nodes, max_depth;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  int32_t* near_ties;  // may be null
  int32_t* status;
};

struct StochWalkLds {
  NodeVerdict v[ST_MAX_NODES];
  int path[kMaxPath + 1];
};

// Walk of request b by one whole wavefront: the request's verdicts are staged
// in LDS, checked with its parents and tokens, and followed from the root
// (at most max_depth steps).  The path is left in s.path; returns L, or -1
// for a request whose node range is invalid.  With `write` the wavefront also
// stores the path outputs, the near-tie count and the status bits.
__device__ inline int stoch_walk_wave(const StochWalkArgs& g, int b, StochWalkLds& s,
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
    if (i == 0 ? (p != -1) : (p < 0 || p >= i)) bits |= ST_STATUS_BAD_PARENT;
    if (i > 0 && (tok < 0 || tok >= g.V)) bits |= ST_STATUS_BAD_TOKEN;
    s.v[i] = g.verdict[lo + i];
  }
  for (int o = 32; o > 0; o >>= 1) bits |= __shfl_xor(bits, o, ST_WAVE);
  wave_lds_sync();
  int L = 0, ties = 0, last = -1;
  bool over = false;
  if (lane == 0) {
    int u = 0;
    s.path[0] = 0;
    while (true) {
      ties += s.v[u].ties;
      const int c = s.v[u].accepted;
      if (c <= u || c >= n) break;  // -1: stop here
      if (L == g.max_depth) {
        over = true;
        break;
      }
      s.path[++L] = c;
      u = c;
    }
    if (!over) {
      last = s.v[u].token;
      ties += s.v[u].token_tie;
    }
  }
  L = __shfl(L, 0, ST_WAVE);
  wave_lds_sync();
  if (write) {
    last = __shfl(last, 0, ST_WAVE);
    over = __shfl((int)over, 0, ST_WAVE);
    if (lane == 0) {
      set_status(g.status, bits | (over ? ST_STATUS_PATH_OVERFLOW : 0));
      if (g.near_ties) g.near_ties[b] = ties;
    }
    write_path_outputs(lane, ST_WAVE, b, L, g.max_depth, s.path, g.tokens, lo, last,
                       g.accept_len, g.accept_nodes, g.out_tokens);
  }
  return L;
}

}  // namespace st

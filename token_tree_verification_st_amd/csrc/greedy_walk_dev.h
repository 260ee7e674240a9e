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

// ---------------------------------------------------------------- vocab argmax

// A workgroup of kArgmaxBlock threads reduces one 8192-entry slice of one
// logits row to its maximum and lowest index.  Loading and reducing are split
// so that a caller can keep the loads in flight while it does other work.
constexpr int kArgmaxBlock = 256;
constexpr int kArgmaxPerThread = 32;                          // logits per thread
constexpr int kArgmaxSlice = kArgmaxBlock * kArgmaxPerThread;  // vocab entries per slice

typedef float am_f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int argmax_slices(int V) { return (V + kArgmaxSlice - 1) / kArgmaxSlice; }

struct ArgmaxRegs {
  am_f32x4 x[kArgmaxPerThread / 4];
};

// Every load of this thread's 32 entries of slice `slice` of row t, issued up
// front (16-byte non-temporal loads when VEC: V is a multiple of 4).
template <bool VEC>
__device__ inline void argmax_slice_load(const float* logits, int V, int t, int slice,
                                         ArgmaxRegs& r) {
  const float* row = logits + (size_t)t * V;
  const int base = slice * kArgmaxSlice;
  const int tid = threadIdx.x;
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < kArgmaxPerThread / 4; ++k) {
      const int v = base + 4 * (tid + k * kArgmaxBlock);
      r.x[k] = v < V ? __builtin_nontemporal_load((const am_f32x4*)(row + v))
                     : am_f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  } else {
#pragma unroll
    for (int k = 0; k < kArgmaxPerThread; ++k) {
      const int v = base + tid + k * kArgmaxBlock;
      r.x[k / 4][k % 4] = v < V ? row[v] : -INFINITY;
    }
  }
}

// Reduce the loaded entries over the workgroup (all kArgmaxBlock threads call
// it) and store the slice's (max, lowest index); a NaN or infinite logit sets
// ST_STATUS_NONFINITE.  `scratch` is 2 * (kArgmaxBlock / 64) + 1 words of LDS.
template <bool VEC>
__device__ inline void argmax_slice_finish(const ArgmaxRegs& r, int V, int t, int slice,
                                           int nslices, ArgmaxPart* part, int32_t* status,
                                           int* scratch) {
  const int base = slice * kArgmaxSlice;
  const int tid = threadIdx.x;
  float best = -INFINITY;
  int bidx = INT_MAX;
  bool finite = true;
#pragma unroll
  for (int k = 0; k < kArgmaxPerThread / 4; ++k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = VEC ? base + 4 * (tid + k * kArgmaxBlock) + j
                        : base + tid + (4 * k + j) * kArgmaxBlock;
      if (v < V) {
        const float x = r.x[k][j];
        // exponent bits all set: inf or NaN (a bit test, whatever the
        // compiler may assume about NaNs)
        finite = finite && (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u;
        argmax_merge(best, bidx, x, v);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o, ST_WAVE);
    const int i2 = __shfl_xor(bidx, o, ST_WAVE);
    argmax_merge(best, bidx, v2, i2);
  }
  constexpr int NW = kArgmaxBlock / ST_WAVE;
  float* sv = (float*)scratch;
  int* si = scratch + NW;
  int* sf = scratch + 2 * NW;
  if (tid == 0) *sf = 1;
  __syncthreads();
  const int w = tid / ST_WAVE;
  if (tid % ST_WAVE == 0) {
    sv[w] = best;
    si[w] = bidx;
  }
  if (!finite) *sf = 0;
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < NW; ++k) argmax_merge(best, bidx, sv[k], si[k]);
    part[(size_t)t * nslices + slice] = ArgmaxPart{best, bidx};
    if (!*sf) set_status(status, ST_STATUS_NONFINITE);
  }
  __syncthreads();  // the scratch words may be reused right after
}

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

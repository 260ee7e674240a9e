// Token-tree construction: several candidate continuations of one request
// merged into one speculated token tree (SpecInfer news article, "研究現狀":
// the outputs of several small speculative models are combined into a token
// tree that the target verifies; SpecInfer developer article §2.1-2.2: shared
// prefixes become shared nodes, and each node keeps a pointer to its parent).
//
// The tree's nodes are the root and every distinct non-empty prefix of a
// candidate.  They are numbered level by level (parents before children);
// within a level by the parent's number, then by the smallest candidate index
// that has the prefix.
//
// One workgroup per request (a single wavefront for up to 64 candidates, so
// the barriers cost nothing), one thread per candidate.  The candidates'
// tokens sit in LDS.  Level j is done in three barrier-separated phases, each
// a branch-free pass over the candidates' LDS words:
//   1. each candidate long enough finds its representative: the smallest
//      candidate whose prefix node at level j-1 is the same and whose token
//      at j is the same (equal parent node and equal token = equal prefix);
//   2. each representative counts the representatives ordered before it by
//      (parent number, candidate) -- that rank plus the nodes of the earlier
//      levels is its node number -- and writes its node;
//   3. every candidate takes its representative's number as its current node.
// Nodes numbered past the capacity are not written (their descendants have
// larger numbers still).  The work is O(K^2) compares per level for K <= 256
// candidates: latency-bound, a few microseconds.
//
// A second kernel packs the padded per-request trees into the concatenated
// node_off / parent / tokens layout of st_tree.
#include "st_internal.h"

#include <limits.h>

namespace {

constexpr int kMaxCand = 256;    // candidates per request (one thread each)
constexpr int kMaxCells = 8192;  // K * Lmax tokens staged in LDS (32 KB)

// Barrier-and-reduce helpers: a workgroup of one wavefront needs no LDS
// reduction, a ballot does.
template <int NT>
__device__ inline bool sync_or(bool p) {
  if constexpr (NT == ST_WAVE) {
    __syncthreads();
    return __ballot(p) != 0ull;
  } else {
    return __syncthreads_or(p);
  }
}
template <int NT>
__device__ inline int sync_count(bool p) {
  if constexpr (NT == ST_WAVE) {
    __syncthreads();
    return __popcll(__ballot(p));
  } else {
    return __syncthreads_count(p);
  }
}

// NT threads (one wavefront when K <= 64, else 256).
template <int NT>
__global__ void __launch_bounds__(NT)
tree_build_kernel(const int32_t* __restrict__ root_tokens, const int32_t* __restrict__ seqs,
                  const int32_t* __restrict__ lens, int K, int Lmax, int V, int cap,
                  int32_t* __restrict__ n_nodes, int32_t* __restrict__ parent,
                  int32_t* __restrict__ tokens, int32_t* __restrict__ depth, int32_t* status) {
  __shared__ int s_tok[kMaxCells];
  // per candidate: (node of its prefix at the last level, token at this
  // level) packed in one word, all ones once the candidate is too short
  __shared__ uint64_t s_kt[kMaxCand];
  __shared__ int s_rk[kMaxCand];   // representatives' order key (parent * 256 + k), else INT_MAX
  __shared__ int s_new[kMaxCand];  // node number of each representative at this level
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* sq = seqs + (size_t)b * K * Lmax;
  for (int c = tid; c < K * Lmax; c += blockDim.x) s_tok[c] = sq[c];
  const size_t ob = (size_t)b * cap;
  if (tid == 0) {
    parent[ob] = -1;
    tokens[ob] = root_tokens[b];
    depth[ob] = 0;
  }
  __syncthreads();

  // usable length: a length outside [0, Lmax] counts as 0; a token outside
  // [0, V) ends the candidate before it
  int bad = 0, use = 0;
  if (tid < K) {
    int n = lens[(size_t)b * K + tid];
    if (n < 0 || n > Lmax) {
      bad = ST_STATUS_BAD_TOKEN;
      n = 0;
    }
    for (int j = 0; j < n; ++j) {
      const int x = s_tok[tid * Lmax + j];
      if (x < 0 || x >= V) {
        bad = ST_STATUS_BAD_TOKEN;
        n = j;
        break;
      }
    }
    use = n;
  }
  // every candidate starts at the root (node 0)
  s_kt[tid] = use > 0 ? (uint64_t)(uint32_t)s_tok[tid * Lmax] : ~0ull;
  __syncthreads();
  int total = 1;  // nodes numbered so far (the root)
  for (int j = 0; j < Lmax; ++j) {
    // phase 1: representative of this candidate's prefix of length j + 1, the
    // smallest candidate with the same parent node and token (no early exit:
    // the LDS reads of the loop pipeline)
    const bool act = use > j;
    const uint64_t mine = s_kt[tid];
    int rep = tid;
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
      const bool eq = s_kt[k] == mine;
      rep = (eq && k < rep) ? k : rep;
    }
    const int cur = (int)(mine >> 32);
    const bool is_rep = act && rep == tid;
    s_rk[tid] = is_rep ? cur * kMaxCand + tid : INT_MAX;
    if (!sync_or<NT>(act)) break;  // no candidate reaches this level

    // phase 2: number the representatives by (parent number, candidate)
    if (is_rep) {
      const int key = cur * kMaxCand + tid;
      int rank = 0;
#pragma unroll 8
      for (int k = 0; k < K; ++k) rank += s_rk[k] < key;
      const int num = total + rank;
      s_new[tid] = num;
      if (num < cap) {
        parent[ob + num] = cur;
        tokens[ob + num] = s_tok[tid * Lmax + j];
        depth[ob + num] = j + 1;
      }
    }
    total += sync_count<NT>(is_rep);

    // phase 3: follow the representative to this level's node, with the
    // token of the next level
    const bool next = use > j + 1;
    s_kt[tid] = next ? ((uint64_t)(uint32_t)s_new[rep] << 32) |
                           (uint32_t)s_tok[tid * Lmax + j + 1]
                     : ~0ull;
    __syncthreads();
  }

  const int n = total < cap ? total : cap;
  for (int i = n + tid; i < cap; i += blockDim.x) {
    parent[ob + i] = -1;
    tokens[ob + i] = -1;
    depth[ob + i] = -1;
  }
  if (tid == 0) {
    n_nodes[b] = n;
    if (total > cap) bad |= ST_STATUS_PATH_OVERFLOW;
  }
  st::set_status(status, bad);
}

// Workgroup b: its offset is the sum of the node counts of the requests
// before it; it copies its nodes there.  The last one also writes node_off[B].
__global__ void __launch_bounds__(256)
tree_pack_kernel(const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ parent,
                 const int32_t* __restrict__ tokens, int B, int cap,
                 int32_t* __restrict__ node_off, int32_t* __restrict__ parent_out,
                 int32_t* __restrict__ tokens_out) {
  __shared__ int s_part[256 / ST_WAVE];
  const int b = blockIdx.x, tid = threadIdx.x;
  int s = 0;
  for (int i = tid; i < b; i += blockDim.x) s += n_nodes[i];
  s = st::wave_sum(s);
  if ((tid & (ST_WAVE - 1)) == 0) s_part[tid / ST_WAVE] = s;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < 256 / ST_WAVE; ++w) off += s_part[w];
  const int n = n_nodes[b];
  if (tid == 0) {
    node_off[b] = off;
    if (b == B - 1) node_off[B] = off + n;
  }
  const size_t ib = (size_t)b * cap;
  for (int i = tid; i < n; i += blockDim.x) {
    parent_out[off + i] = parent[ib + i];
    tokens_out[off + i] = tokens[ib + i];
  }
}

}  // namespace

extern "C" int st_tree_build(int B, int K, int Lmax, int V, int cap, const int32_t* root_tokens,
                             const int32_t* seqs, const int32_t* lens, int32_t* n_nodes,
                             int32_t* parent, int32_t* tokens, int32_t* depth, int32_t* node_off,
                             int32_t* parent_packed, int32_t* tokens_packed, int32_t* status,
                             void* stream) {
  if (B < 1 || K < 1 || Lmax < 1 || V < 1 || cap < 1) return ST_E_INVALID;
  if (K > kMaxCand || (long)K * Lmax > kMaxCells || cap > ST_MAX_NODES) return ST_E_UNSUPPORTED;
  if (!root_tokens || !seqs || !lens || !n_nodes || !parent || !tokens || !depth)
    return ST_E_INVALID;
  const int packed = (node_off != nullptr) + (parent_packed != nullptr) +
                     (tokens_packed != nullptr);
  if (packed != 0 && packed != 3) return ST_E_INVALID;
  hipStream_t s = (hipStream_t)stream;
  if (K <= ST_WAVE)
    hipLaunchKernelGGL(tree_build_kernel<ST_WAVE>, dim3(B), dim3(ST_WAVE), 0, s, root_tokens, seqs,
                       lens, K, Lmax, V, cap, n_nodes, parent, tokens, depth, status);
  else
    hipLaunchKernelGGL(tree_build_kernel<256>, dim3(B), dim3(256), 0, s, root_tokens, seqs, lens,
                       K, Lmax, V, cap, n_nodes, parent, tokens, depth, status);
  int rc = st::check_launch();
  if (rc || !packed) return rc;
  hipLaunchKernelGGL(tree_pack_kernel, dim3(B), dim3(256), 0, s, n_nodes, parent, tokens, B, cap,
                     node_off, parent_packed, tokens_packed);
  return st::check_launch();
}

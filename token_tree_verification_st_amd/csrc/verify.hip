// Acceptance of a verified token tree.
//
// Greedy (SpecInfer developer article §2.1, longest verified prefix): the
// vocab-wide argmax of every node's target logits is reduced by workgroups
// that each own an 8192-entry slice of one row (coalesced 16-byte loads, all
// issued up front, then wavefront and workgroup reductions); one wavefront
// per request then merges the slices and walks down the tree.
//
// Stochastic (speculative-decoding explainer §2.2: accept with probability
// min(1, p/q), check left to right, resample from the residual at the first
// rejection).  The residual after k rejected children of node u has a closed
// form: r_k = max(0, p_u - c_k q_u) / D_k with c_0 = 0, D_0 = 1,
// c_{k+1} = c_k + D_k and D_{k+1} = sum_v max(0, p_u - c_{k+1} q_u)
// (unchanged when that sum is 0).  It does not depend on which tokens were
// rejected, so every node can test its own children as soon as its logits are
// loaded: one workgroup per node keeps both logit rows in registers, computes
// max / sum-exp, then tests its children in order until the first acceptance,
// spending one vocab reduction per rejection.  A second kernel walks each
// request's tree through those per-node verdicts and draws the replacement
// token at the stop node by inverse CDF.
#include "step_internal.h"

#include <float.h>
#include <limits.h>

// Every comparison that decides a token must see the same value wherever it is
// recomputed, so products and sums are evaluated exactly as written.
#pragma clang fp contract(off)

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kTieEps = 1e-6;

// ---------------------------------------------------------------- reductions

template <int BLOCK, typename T, typename Op>
__device__ inline T block_reduce(T v, T* lds, Op op) {
  constexpr int NW = BLOCK / ST_WAVE;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, ST_WAVE));
  const int w = threadIdx.x / ST_WAVE, lane = threadIdx.x % ST_WAVE;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  T r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = op(r, lds[i]);
  return r;
}

struct MaxOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a > b ? a : b; }
};
struct SumOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};

using st::argmax_merge;
using st::ArgmaxPart;
using st::kMaxPath;

// ---------------------------------------------------------------- greedy

using st::kArgmaxBlock;
using st::kArgmaxSlice;

// Workgroup (t, slice) reduces logits[t][slice*8192 .. +8192) to its maximum
// and lowest index; all of a thread's loads are issued before any is used.
__global__ void __launch_bounds__(kArgmaxBlock)
row_argmax_kernel(const float* __restrict__ logits, int V, ArgmaxPart* __restrict__ part,
                  int32_t* status) {
  __shared__ int scratch[2 * (kArgmaxBlock / ST_WAVE) + 1];
  st::ArgmaxRegs r;
  if ((V & 3) == 0) {
    st::argmax_slice_load<true>(logits, V, blockIdx.x, blockIdx.y, r);
    st::argmax_slice_finish<true>(r, V, blockIdx.x, blockIdx.y, gridDim.y, part, status, scratch);
  } else {
    st::argmax_slice_load<false>(logits, V, blockIdx.x, blockIdx.y, r);
    st::argmax_slice_finish<false>(r, V, blockIdx.x, blockIdx.y, gridDim.y, part, status, scratch);
  }
}

// Checks the request's parents and draft tokens; returns the status bits.
__device__ inline int check_request(const int32_t* parent, const int32_t* tokens, int lo, int n,
                                    int V) {
  int bits = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int p = parent[lo + i];
    if (i == 0 ? (p != -1) : (p < 0 || p >= i)) bits |= ST_STATUS_BAD_PARENT;
    if (i > 0) {
      const int tok = tokens[lo + i];
      if (tok < 0 || tok >= V) bits |= ST_STATUS_BAD_TOKEN;
    }
  }
  return bits;
}

__device__ inline void write_path_outputs(int b, int L, int max_depth, const int* path,
                                          const int32_t* tokens, int lo, int last_token,
                                          int32_t* accept_len, int32_t* accept_nodes,
                                          int32_t* out_tokens) {
  st::write_path_outputs(threadIdx.x, blockDim.x, b, L, max_depth, path, tokens, lo, last_token,
                         accept_len, accept_nodes, out_tokens);
}


// One wavefront per request: the request's parents, tokens and merged argmax
// are staged in LDS, then the walk moves from node to node with the lowest
// matching child found by a ballot over the wavefront.
__global__ void __launch_bounds__(ST_WAVE)
greedy_walk_kernel(st::GreedyWalkArgs g) {
  __shared__ st::GreedyWalkLds s;
  st::greedy_walk_wave(g, blockIdx.x, s, true);
}

// ---------------------------------------------------------------- Philox4x64-10

// Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
__device__ inline void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// (u_acc, u_smp) of a node: top 24 bits of words 0 and 1, times 2^-24.
__device__ inline void node_uniforms(uint64_t seed, uint64_t offset, int req, int node,
                                     double& u_acc, double& u_smp) {
  uint64_t c[4] = {(uint64_t)node, (uint64_t)req, offset, 0};
  philox4x64_10(c, seed, 0);
  u_acc = (double)(c[0] >> 40) * 0x1p-24;
  u_smp = (double)(c[1] >> 40) * 0x1p-24;
}

// ---------------------------------------------------------------- stochastic

struct NodeVerdict {
  double c, D;      // residual after the tested children: max(0, p - c q) / D
  double Zt, Zd;    // sums of exp2((l - M) * log2e / T), target and draft
  float Mt, Md;     // row maxima
  int accepted;     // first accepted child (local index), -1 if none
  int ties;         // near ties among this node's tests
};

constexpr int kStochBlock = 512;
constexpr int kStochNpt = 64;  // logits per thread and row: V <= 32768

__global__ void __launch_bounds__(kStochBlock)
stoch_node_kernel(const int32_t* __restrict__ node_off, const int32_t* __restrict__ parent,
                  const int32_t* __restrict__ tokens, const float* __restrict__ tl,
                  const float* __restrict__ dl, int B, int T, int V, float temperature,
                  uint64_t seed, uint64_t offset, NodeVerdict* __restrict__ out,
                  int32_t* status) {
  __shared__ double red_d[kStochBlock / ST_WAVE];
  __shared__ float red_f[kStochBlock / ST_WAVE];
  __shared__ uint64_t kids[ST_MAX_NODES / 64];
  __shared__ int s_dec;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int b = st::request_of(node_off, B, t);
  const int lo = node_off[b], n = node_off[b + 1] - lo, i = t - lo;
  const float* rt = tl + (size_t)t * V;
  const float* rd = dl + (size_t)t * V;

  float xt[kStochNpt], xd[kStochNpt];
  bool finite = true;
  float mt = -INFINITY, md = -INFINITY;
#pragma unroll
  for (int k = 0; k < kStochNpt; ++k) {
    const int v = k * kStochBlock + tid;
    xt[k] = v < V ? __builtin_nontemporal_load(rt + v) : -INFINITY;
    xd[k] = v < V ? __builtin_nontemporal_load(rd + v) : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < kStochNpt; ++k) {
    if (k * kStochBlock + tid < V) finite = finite && isfinite(xt[k]) && isfinite(xd[k]);
    mt = fmaxf(mt, xt[k]);
    md = fmaxf(md, xd[k]);
  }
  if (!finite) st::set_status(status, ST_STATUS_NONFINITE);
  mt = block_reduce<kStochBlock>(mt, red_f, MaxOp());
  md = block_reduce<kStochBlock>(md, red_f, MaxOp());
  const float s = kLog2e / temperature;
  double zt = 0.0, zd = 0.0;
#pragma unroll
  for (int k = 0; k < kStochNpt; ++k) {
    xt[k] = exp2f((xt[k] - mt) * s);  // padding: exp2(-inf) = 0
    xd[k] = exp2f((xd[k] - md) * s);
    zt += xt[k];
    zd += xd[k];
  }
  zt = block_reduce<kStochBlock>(zt, red_d, SumOp());
  zd = block_reduce<kStochBlock>(zd, red_d, SumOp());
  const double a = 1.0 / zt, bq = 1.0 / zd;

  // children of local node i, as a bitmask over local indices
  if (tid < ST_MAX_NODES / 64) kids[tid] = 0;
  __syncthreads();
  const bool sane = n >= 1 && n <= ST_MAX_NODES && lo + n <= T;
  if (sane && tid < n && tid > i && parent[lo + tid] == i)
    atomicOr((unsigned long long*)&kids[tid >> 6], 1ull << (tid & 63));
  __syncthreads();

  double c = 0.0, D = 1.0;
  int ties = 0, accepted = -1;
  for (int w = 0; w < ST_MAX_NODES / 64 && accepted < 0; ++w) {
    uint64_t m = kids[w];
    while (m && accepted < 0) {
      const int child = w * 64 + __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      if (tid == 0) {
        const int x = tokens[lo + child];
        int dec = 0;
        if (x >= 0 && x < V) {
          double ua, us;
          node_uniforms(seed, offset, b, child, ua, us);
          const double px = (double)exp2f((rt[x] - mt) * s) * a;
          const double qx = (double)exp2f((rd[x] - md) * s) * bq;
          const double r = fmax(0.0, px - c * qx) / D;
          const double lhs = ua * qx;
          ties += fabs(r - lhs) < kTieEps;
          dec = lhs < r;
        }
        s_dec = dec;
      }
      __syncthreads();
      const int dec = s_dec;
      __syncthreads();
      if (dec) {
        accepted = child;
        break;
      }
      const double cn = c + D;
      const double cq = cn * bq;
      double part = 0.0;
#pragma unroll
      for (int k = 0; k < kStochNpt; ++k) {
        // keep the fp64 widening inside the loop (hoisting it would need 256
        // more registers)
        float et = xt[k], ed = xd[k];
        asm volatile("" : "+v"(et), "+v"(ed));
        part += fmax(0.0, (double)et * a - (double)ed * cq);
      }
      const double Dn = block_reduce<kStochBlock>(part, red_d, SumOp());
      if (Dn > 0.0) {
        c = cn;
        D = Dn;
      }
    }
  }
  if (tid == 0) {
    NodeVerdict nv;
    nv.c = c;
    nv.D = D;
    nv.Zt = zt;
    nv.Zd = zd;
    nv.Mt = mt;
    nv.Md = md;
    nv.accepted = accepted;
    nv.ties = ties;
    out[t] = nv;
  }
}

// Exclusive scan of one double per thread across the block.
template <int BLOCK>
__device__ inline double block_exclusive_scan(double v, double* lds, double& total) {
  constexpr int NW = BLOCK / ST_WAVE;
  const int lane = threadIdx.x % ST_WAVE, w = threadIdx.x / ST_WAVE;
  double incl = v;
#pragma unroll
  for (int o = 1; o < ST_WAVE; o <<= 1) {
    const double y = __shfl_up(incl, o, ST_WAVE);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == ST_WAVE - 1) lds[w] = incl;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
  for (int k = 0; k < NW; ++k) {
    if (k < w) before += lds[k];
    total += lds[k];
  }
  return before + incl - v;
}

__global__ void __launch_bounds__(kStochBlock)
stoch_walk_kernel(const int32_t* __restrict__ node_off, const int32_t* __restrict__ parent,
                  const int32_t* __restrict__ tokens, const float* __restrict__ tl,
                  const float* __restrict__ dl, const NodeVerdict* __restrict__ verdict, int T,
                  int V, int max_nodes, int max_depth, float temperature, uint64_t seed,
                  uint64_t offset, int32_t* accept_len, int32_t* accept_nodes,
                  int32_t* out_tokens, int32_t* near_ties, int32_t* status) {
  __shared__ int path[kMaxPath + 1];
  __shared__ int s_u, s_L, s_over, s_ties;
  __shared__ double red[kStochBlock / ST_WAVE];
  __shared__ int s_pick, s_last;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lo = node_off[b], hi = node_off[b + 1], n = hi - lo;
  if (lo < 0 || hi > T || n < 1 || n > max_nodes) {
    if (tid == 0) st::set_status(status, ST_STATUS_BAD_PARENT);
    return;
  }
  const int bits = check_request(parent, tokens, lo, n, V);
  if (bits) st::set_status(status, bits);

  if (tid == 0) {
    int u = 0, L = 0, ties = 0, over = 0;
    path[0] = 0;
    while (true) {
      const NodeVerdict nv = verdict[lo + u];
      ties += nv.ties;
      const int c = nv.accepted;
      if (c <= u || c >= n) break;  // -1: no child accepted
      if (L == max_depth) {
        over = 1;
        break;
      }
      path[++L] = c;
      u = c;
    }
    s_u = u;
    s_L = L;
    s_over = over;
    s_ties = ties;
    s_pick = INT_MAX;
    s_last = -1;
  }
  __syncthreads();
  const int u = s_u, L = s_L;
  int last_token = -1, ties = s_ties;
  if (!s_over) {
    // replacement token: inverse CDF of r = max(0, p_u - c q_u) / D at u
    const NodeVerdict nv = verdict[lo + u];
    const float s = kLog2e / temperature;
    const double a = 1.0 / nv.Zt, cq = nv.c / nv.Zd;
    const float* rt = tl + (size_t)(lo + u) * V;
    const float* rd = dl + (size_t)(lo + u) * V;
    const int chunk = (V + kStochBlock - 1) / kStochBlock;
    const int v0 = tid * chunk, v1 = min(V, v0 + chunk);
    double local = 0.0;
    int last_pos = -1;
    for (int v = v0; v < v1; ++v) {
      const double w = fmax(0.0, (double)exp2f((rt[v] - nv.Mt) * s) * a -
                                     (double)exp2f((rd[v] - nv.Md) * s) * cq);
      local += w;
      if (w > 0.0) last_pos = v;
    }
    double total;
    const double excl = block_exclusive_scan<kStochBlock>(local, red, total);
    double ua, us;
    node_uniforms(seed, offset, b, u, ua, us);
    const double thr = us * total;
    if (last_pos >= 0) atomicMax(&s_last, last_pos);
    int pick = -1;
    double c_hi = 0.0, c_lo = 0.0;
    if (excl <= thr && excl + local > thr) {
      // same summation order as `local`, so the last running sum equals it
      double run = 0.0;
      for (int v = v0; v < v1; ++v) {
        const double w = fmax(0.0, (double)exp2f((rt[v] - nv.Mt) * s) * a -
                                       (double)exp2f((rd[v] - nv.Md) * s) * cq);
        c_lo = excl + run;
        run += w;
        if (excl + run > thr) {
          pick = v;
          c_hi = excl + run;
          break;
        }
      }
      if (pick >= 0) atomicMin(&s_pick, pick);
    }
    __syncthreads();
    const int chosen = s_pick != INT_MAX ? s_pick : s_last;
    if (pick >= 0 && pick == chosen) {
      const bool tie = fabs(c_hi - thr) < kTieEps * total ||
                       (pick > 0 && fabs(c_lo - thr) < kTieEps * total);
      s_ties = s_ties + (int)tie;
    }
    __syncthreads();
    ties = s_ties;
    last_token = chosen < 0 ? 0 : chosen;
  } else if (tid == 0) {
    st::set_status(status, ST_STATUS_PATH_OVERFLOW);
  }
  write_path_outputs(b, L, max_depth, path, tokens, lo, last_token, accept_len, accept_nodes,
                     out_tokens);
  if (tid == 0 && near_ties) near_ties[b] = ties;
}

}  // namespace

// ---------------------------------------------------------------- entry points

using st::argmax_slices;

extern "C" size_t st_verify_greedy_workspace(const st_tree* tree, int V) {
  if (st::check_tree_host(tree) || V < 1) return 0;
  return st::align_up((size_t)tree->total_nodes * argmax_slices(V) * sizeof(ArgmaxPart), 256);
}

int st::greedy_prepare(const st_tree* tree, int V, const int32_t* tokens, const float* logits,
                       int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                       void* workspace, size_t ws_bytes, int32_t* status,
                       st::GreedyWalkArgs& g) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (V < 1 || !tokens || !logits || !accept_len || !accept_nodes || !out_tokens || !workspace)
    return ST_E_INVALID;
  if (tree->max_depth + 1 > kMaxPath) return ST_E_UNSUPPORTED;
  if (ws_bytes < st_verify_greedy_workspace(tree, V)) return ST_E_WORKSPACE;
  g = st::GreedyWalkArgs{tree->node_off, tree->parent, tokens, (ArgmaxPart*)workspace,
                         argmax_slices(V), tree->total_nodes, V, tree->max_nodes,
                         tree->max_depth, accept_len, accept_nodes, out_tokens, status};
  return ST_OK;
}

int st::greedy_argmax_launch(const st::GreedyWalkArgs& g, const float* logits, void* stream) {
  hipLaunchKernelGGL(row_argmax_kernel, dim3(g.T, g.nslices), dim3(kArgmaxBlock), 0,
                     (hipStream_t)stream, logits, g.V, (ArgmaxPart*)g.part, g.status);
  return st::check_launch();
}

extern "C" int st_verify_greedy(const st_tree* tree, int V, const int32_t* tokens,
                                const float* logits, int32_t* accept_len, int32_t* accept_nodes,
                                int32_t* out_tokens, void* workspace, size_t ws_bytes,
                                int32_t* status, void* stream) {
  st::GreedyWalkArgs g;
  int rc = st::greedy_prepare(tree, V, tokens, logits, accept_len, accept_nodes, out_tokens,
                              workspace, ws_bytes, status, g);
  if (rc || (rc = st::greedy_argmax_launch(g, logits, stream))) return rc;
  hipLaunchKernelGGL(greedy_walk_kernel, dim3(tree->B), dim3(ST_WAVE), 0, (hipStream_t)stream, g);
  return st::check_launch();
}

extern "C" size_t st_verify_stochastic_workspace(const st_tree* tree, int V) {
  (void)V;
  if (st::check_tree_host(tree)) return 0;
  return st::align_up((size_t)tree->total_nodes * sizeof(NodeVerdict), 256);
}

extern "C" int st_verify_stochastic(const st_tree* tree, int V, const int32_t* tokens,
                                    const float* target_logits, const float* draft_logits,
                                    float temperature, uint64_t seed, uint64_t offset,
                                    int32_t* accept_len, int32_t* accept_nodes,
                                    int32_t* out_tokens, int32_t* near_ties, void* workspace,
                                    size_t ws_bytes, int32_t* status, void* stream) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (V < 1 || !tokens || !target_logits || !draft_logits || !accept_len || !accept_nodes ||
      !out_tokens || !workspace || !(temperature > 0.0f))
    return ST_E_INVALID;
  if (V > kStochBlock * kStochNpt || tree->max_depth + 1 > kMaxPath) return ST_E_UNSUPPORTED;
  if (ws_bytes < st_verify_stochastic_workspace(tree, V)) return ST_E_WORKSPACE;
  NodeVerdict* nv = (NodeVerdict*)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(stoch_node_kernel, dim3(tree->total_nodes), dim3(kStochBlock), 0, s,
                     tree->node_off, tree->parent, tokens, target_logits, draft_logits, tree->B,
                     tree->total_nodes, V, temperature, seed, offset, nv, status);
  if ((rc = st::check_launch())) return rc;
  hipLaunchKernelGGL(stoch_walk_kernel, dim3(tree->B), dim3(kStochBlock), 0, s, tree->node_off,
                     tree->parent, tokens, target_logits, draft_logits, nv, tree->total_nodes, V,
                     tree->max_nodes, tree->max_depth, temperature, seed, offset, accept_len,
                     accept_nodes, out_tokens, near_ties, status);
  return st::check_launch();
}

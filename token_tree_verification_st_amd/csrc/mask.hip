// Ancestor bitmask of a token tree (SpecInfer news article, "Token 樹驗證器":
// each node attends along its own root path through a constructed mask; the
// parent pointer per node is from §2.1 of the SpecInfer developer article).
//
// One workgroup per request, one thread per node: the request's parent array
// is staged in LDS, then each thread follows parent pointers from its node to
// the root, setting one bit per node reached.  A request holds at most 256
// nodes, so a row is at most four 64-bit words and the walk at most 255 steps;
// this is latency-bound work of a few microseconds.
#include "st_internal.h"

namespace {

__device__ inline void set_bit4(uint64_t& w0, uint64_t& w1, uint64_t& w2, uint64_t& w3, int k) {
  const uint64_t bit = 1ull << (k & 63);
  switch (k >> 6) {
    case 0: w0 |= bit; break;
    case 1: w1 |= bit; break;
    case 2: w2 |= bit; break;
    default: w3 |= bit; break;
  }
}

__global__ void __launch_bounds__(256)
tree_mask_kernel(const int32_t* __restrict__ node_off, const int32_t* __restrict__ parent, int T,
                 int max_nodes, int W, uint64_t* __restrict__ mask, int32_t* __restrict__ depth,
                 int32_t* status) {
  __shared__ int sp[ST_MAX_NODES];
  const int b = blockIdx.x;
  const int lo = node_off[b], hi = node_off[b + 1];
  const int n = hi - lo;
  if (lo < 0 || hi > T || n < 1 || n > max_nodes) {
    if (threadIdx.x == 0) st::set_status(status, ST_STATUS_BAD_PARENT);
    return;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) sp[i] = parent[lo + i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    int j = i, d = 0, bad = 0;
    set_bit4(w0, w1, w2, w3, j);
    for (int steps = 0; steps < n; ++steps) {
      const int p = sp[j];
      if (j == 0) {
        bad = (p != -1);
        break;
      }
      if (p < 0 || p >= j) {
        bad = 1;
        break;
      }
      j = p;
      ++d;
      set_bit4(w0, w1, w2, w3, j);
    }
    uint64_t* row = mask + (size_t)(lo + i) * W;
    row[0] = w0;
    if (W > 1) row[1] = w1;
    if (W > 2) row[2] = w2;
    if (W > 3) row[3] = w3;
    depth[lo + i] = d;
    if (bad) st::set_status(status, ST_STATUS_BAD_PARENT);
  }
}

}  // namespace

extern "C" int st_mask_words(int max_nodes) { return st::mask_words(max_nodes); }

extern "C" int st_tree_mask(const st_tree* tree, uint64_t* mask, int32_t* depth, int32_t* status,
                            void* stream) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (!mask || !depth) return ST_E_INVALID;
  const int W = st::mask_words(tree->max_nodes);
  hipLaunchKernelGGL(tree_mask_kernel, dim3(tree->B), dim3(256), 0, (hipStream_t)stream,
                     tree->node_off, tree->parent, tree->total_nodes, tree->max_nodes, W, mask,
                     depth, status);
  return st::check_launch();
}

// Compaction of the accepted path's KV rows (the depth-first KV-cache update
// of the SpecInfer news article, "Token 樹驗證器"): slot P + j of every kv head
// takes what slot P + path[j] held before the call, for j = 0..L.
//
// The copy is in place.  Because a path strictly increases (path[j] >= j), the
// source of a later move is never the destination of an earlier one, so each
// thread owns one 16-byte column chunk of one (request, head, cache) row and
// moves it for j = 0, 1, ..., L in that order: every source is read before
// any move could overwrite it.
#include "st_internal.h"

namespace {

__global__ void __launch_bounds__(64)
kv_compact_kernel(int Hkv, int S_max, int chunks, uint4* __restrict__ kc, uint4* __restrict__ vc,
                  const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ accept_len,
                  const int32_t* __restrict__ accept_nodes, int max_path,
                  int32_t* __restrict__ src_slot, int32_t* __restrict__ new_len,
                  int32_t* status) {
  const int b = blockIdx.x, y = blockIdx.y;
  const int P = prefix_len[b], L = accept_len[b];
  const int32_t* path = accept_nodes + (size_t)b * max_path;
  int bad = 0;
  if (L < 0 || L + 1 > max_path || P < 0) {
    bad = ST_STATUS_PATH_OVERFLOW;
  } else {
    for (int j = 0; j <= L; ++j) {
      const int n = path[j];
      if (n < 0 || (long)P + n >= S_max || (j > 0 && n <= path[j - 1])) bad = ST_STATUS_BAD_PARENT;
    }
  }
  if (y == 0 && threadIdx.x == 0) {
    for (int j = 0; j < max_path; ++j)
      src_slot[(size_t)b * max_path + j] = (!bad && j <= L) ? P + path[j] : -1;
    new_len[b] = bad ? P : P + L + 1;
    st::set_status(status, bad);
  }
  if (bad) return;
  const int head = y % Hkv;
  uint4* cache = y < Hkv ? kc : vc;
  uint4* rows = cache + ((size_t)b * Hkv + head) * (size_t)S_max * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    for (int j = 0; j <= L; ++j) {
      const int src = P + path[j], dst = P + j;
      if (src != dst) rows[(size_t)dst * chunks + c] = rows[(size_t)src * chunks + c];
    }
  }
}

}  // namespace

extern "C" int st_kv_compact(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache,
                             int S_max, const int32_t* prefix_len, const int32_t* accept_len,
                             const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                             int32_t* new_len, int32_t* status, void* stream) {
  if (B < 1 || Hkv < 1 || S_max < 1 || max_path < 1 || !k_cache || !v_cache || !prefix_len ||
      !accept_len || !accept_nodes || !src_slot || !new_len)
    return ST_E_INVALID;
  if (dtype != ST_F32 && dtype != ST_BF16) return ST_E_INVALID;
  const int row_bytes = D * (dtype == ST_F32 ? 4 : 2);
  if (D < 8 || row_bytes % 16) return ST_E_UNSUPPORTED;
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) % 16) return ST_E_INVALID;
  hipLaunchKernelGGL(kv_compact_kernel, dim3(B, 2 * Hkv), dim3(64), 0, (hipStream_t)stream, Hkv,
                     S_max, row_bytes / 16, (uint4*)k_cache, (uint4*)v_cache, prefix_len,
                     accept_len, accept_nodes, max_path, src_slot, new_len, status);
  return st::check_launch();
}

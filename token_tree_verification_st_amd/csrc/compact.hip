// st_kv_compact: the accepted path's KV rows move into contiguous slots; the
// device body (and why the in-place order is safe) is in kv_compact_dev.h.
#include "kv_compact_dev.h"

namespace {

__global__ void __launch_bounds__(256) kv_compact_kernel(st::CompactArgs c) {
  st::kv_compact_block(c, blockIdx.x, blockIdx.y);
}

}  // namespace

namespace st {

int fill_compact_args(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache,
                      int S_max, const int32_t* prefix_len, const int32_t* accept_len,
                      const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                      int32_t* new_len, int32_t* status, CompactArgs& c) {
  if (B < 1 || Hkv < 1 || S_max < 1 || max_path < 1 || !k_cache || !v_cache || !prefix_len ||
      !accept_len || !accept_nodes || !src_slot || !new_len)
    return ST_E_INVALID;
  if (dtype != ST_F32 && dtype != ST_BF16) return ST_E_INVALID;
  const int row_bytes = D * (dtype == ST_F32 ? 4 : 2);
  if (D < 8 || row_bytes % 16 || row_bytes / 16 > 256) return ST_E_UNSUPPORTED;
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) % 16) return ST_E_INVALID;
  c.B = B;
  c.Hkv = Hkv;
  c.S_max = S_max;
  c.chunks = row_bytes / 16;
  c.kc = (uint4*)k_cache;
  c.vc = (uint4*)v_cache;
  c.prefix_len = prefix_len;
  c.accept_len = accept_len;
  c.accept_nodes = accept_nodes;
  c.max_path = max_path;
  c.src_slot = src_slot;
  c.new_len = new_len;
  c.status = status;
  c.pg = KvPaging{nullptr, 0, 0, 0};
  c.walk = kWalkNone;
  c.g = GreedyWalkArgs{};
  return ST_OK;
}

}  // namespace st

extern "C" int st_kv_compact(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache,
                             int S_max, const int32_t* prefix_len, const int32_t* accept_len,
                             const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                             int32_t* new_len, int32_t* status, void* stream) {
  st::CompactArgs c;
  const int rc = st::fill_compact_args(B, Hkv, D, dtype, k_cache, v_cache, S_max, prefix_len,
                                       accept_len, accept_nodes, max_path, src_slot, new_len,
                                       status, c);
  if (rc) return rc;
  hipLaunchKernelGGL(kv_compact_kernel, dim3(B, 2 * Hkv), dim3(256), 0, (hipStream_t)stream, c);
  return st::check_launch();
}

extern "C" int st_kv_compact_paged(int B, int Hkv, int D, st_dtype dtype, void* k_pool,
                                   void* v_pool, int n_blocks, int block_size,
                                   const int32_t* block_table, int max_blocks,
                                   const int32_t* prefix_len, const int32_t* accept_len,
                                   const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                                   int32_t* new_len, int32_t* status, void* stream) {
  if (!block_table || n_blocks < 1 || max_blocks < 1) return ST_E_INVALID;
  if (block_size < 1 || block_size > 4096 || (block_size & (block_size - 1)))
    return ST_E_UNSUPPORTED;
  const long cap = (long)max_blocks * block_size;
  if (cap > (1L << 30)) return ST_E_UNSUPPORTED;
  st::CompactArgs c;
  const int rc = st::fill_compact_args(B, Hkv, D, dtype, k_pool, v_pool, (int)cap, prefix_len,
                                       accept_len, accept_nodes, max_path, src_slot, new_len,
                                       status, c);
  if (rc) return rc;
  c.pg = st::KvPaging{block_table, max_blocks, __builtin_ctz(block_size), n_blocks};
  hipLaunchKernelGGL(kv_compact_kernel, dim3(B, 2 * Hkv), dim3(256), 0, (hipStream_t)stream, c);
  return st::check_launch();
}

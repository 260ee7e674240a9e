// Internal helpers shared by the HIP sources of libst.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "st.h"

#define ST_WAVE 64

namespace st {

// ---------------------------------------------------------------- host side

inline int check_launch() { return hipGetLastError() == hipSuccess ? ST_OK : ST_E_LAUNCH; }

inline int check_tree_host(const st_tree* t) {
  if (!t || !t->node_off || !t->parent) return ST_E_INVALID;
  if (t->B < 1 || t->total_nodes < t->B || t->max_nodes < 1 || t->max_depth < 0)
    return ST_E_INVALID;
  if (t->max_nodes > ST_MAX_NODES) return ST_E_UNSUPPORTED;
  return ST_OK;
}

// KV rows reached through a per-request block table instead of the
// contiguous [B][Hkv][S_max][D] layout: logical slot k of request b lives in
// physical block bt[b * bt_stride + (k >> lbs)] of a pool laid out
// [n_blocks][Hkv][1 << lbs][D].  bt == nullptr: contiguous.
struct KvPaging {
  const int32_t* bt;
  int bt_stride, lbs, n_blocks;
};

// Planner overrides installed by st_testing_set_plan (include/st_testing.h);
// the defaults leave every choice to the planners.
struct TestingPlan {
  int attn_shape = -1, attn_target_wg = 0, attn_split_keys = 0;
  int linear_ksplit = 0, linear_stages = 0;
  int attn_balance = 0;
  int step_serial = 0;
};
const TestingPlan& testing_plan();

inline int mask_words(int max_nodes) { return (max_nodes + 63) / 64; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device, queried once per device.
inline int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// ---------------------------------------------------------------- device side

__device__ inline void set_status(int32_t* status, int bits) {
  if (status && bits) atomicOr(status, bits);
}

// bf16 <-> fp32.  A bfloat16 is the upper half of a float32; the store rounds
// to nearest, ties to even (finite inputs).
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Request that owns global node t (node_off is [B+1], strictly increasing).
__device__ inline int request_of(const int32_t* node_off, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (node_off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T>
__device__ inline T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, ST_WAVE);
    v = v > w ? v : w;
  }
  return v;
}

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, ST_WAVE);
  return v;
}

}  // namespace st

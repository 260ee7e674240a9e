// A plain read-only pass over a buffer: the practical HBM read ceiling that
// the verification kernels' bandwidth is compared with (a measurement helper,
// not part of the method).  Grid-stride 16-byte non-temporal loads, eight per
// thread in flight, folded into a word that is stored only on a value the
// data never produces (so the loads cannot be dropped).
#include "st_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kReadBlock = 256;
constexpr int kReadUnroll = 8;

__global__ void __launch_bounds__(kReadBlock)
stream_read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t step = (size_t)gridDim.x * kReadBlock * kReadUnroll;
  for (size_t base = (size_t)blockIdx.x * kReadBlock * kReadUnroll + threadIdx.x; base < n16;
       base += step) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t i = base + (size_t)u * kReadBlock;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int st_stream_read(const void* src, size_t bytes, uint32_t* sink, int sink_len,
                              void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || ((uintptr_t)src % 16) || sink_len < 1)
    return ST_E_INVALID;
  const size_t n16 = bytes / 16;
  const size_t per_block = (size_t)kReadBlock * kReadUnroll;
  size_t blocks = (n16 + per_block - 1) / per_block;
  const size_t cap = (size_t)st::device_cus() * 8;
  if (blocks > cap) blocks = cap;
  if (blocks > (size_t)sink_len) blocks = (size_t)sink_len;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadBlock), 0,
                     (hipStream_t)stream, (const u32x4*)src, n16, sink);
  return st::check_launch();
}

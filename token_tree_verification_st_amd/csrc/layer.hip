// The target layer's own work around tree verification: token embedding,
// the projections (q/k/v, output with residual, vocabulary), and the rotary
// embedding of the tree nodes' queries and keys with the append of their keys
// and values to the cache.
//
// Incremental decoding keeps the keys and values of decoded tokens in a cache
// (SpecInfer news article, "研究現狀"); the target checks every tree path in a
// single pass (speculative-decoding explainer §3.2).  A node's position is its
// index in the sequence of its root path, P_b + depth, so after the accepted
// path is moved to slots P_b .. P_b + L its keys sit at their positions.
//
// st_linear, y = x w^T (+ residual), is a skinny product: x holds the tree's
// few dozen to few hundred rows, w is a weight matrix streamed once from HBM.
// A workgroup owns 64 output features (16 per wavefront) and 32 or 64 rows,
// and walks its range of the reduction in 64-wide stages.  Each stage of w
// (64 features x 64) and of x (rows x 64) is copied to LDS by direct
// global-to-LDS loads into a 4-deep ring shared by the 4 wavefronts; per
// 32-wide step a wavefront reads one w fragment and one x fragment per
// 16 rows and issues v_mfma_f32_16x16x32_bf16 (A = w, B = x^T).  When one
// pass over the features leaves CUs idle the reduction is split and a second
// launch adds the fp32 partials in a fixed order.
#include "st_internal.h"

#include <math.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LY_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
// vmcnt(n) with the other counters left alone (gfx9 encoding).
#define LY_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// ---------------------------------------------------------------- embedding

__global__ void __launch_bounds__(256) embed_kernel(int T, int d, int V, const int32_t* tokens,
                                                    const uint16_t* table, uint16_t* out,
                                                    int32_t* status) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int tok = tokens[t];
  const bool ok = tok >= 0 && tok < V;
  if (!ok && threadIdx.x == 0) st::set_status(status, ST_STATUS_BAD_TOKEN);
  const u32x4* src = (const u32x4*)(table + (size_t)(ok ? tok : 0) * d);
  u32x4* dst = (u32x4*)(out + (size_t)t * d);
  for (int i = threadIdx.x; i < d / 8; i += 256) dst[i] = ok ? src[i] : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------- rotary embedding + append

struct RopeArgs {
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* prefix_len;
  const uint16_t* qkv;  // [T][(Hq + 2 Hkv) D]
  uint16_t* q_out;      // [T][Hq][D]
  uint16_t* k_cache;    // [B][Hkv][S_max][D]
  uint16_t* v_cache;
  int32_t* status;
  int B, T, Hq, Hkv, D, S_max, max_prefix, max_nodes;
  double theta;
};

// One workgroup per tree node.  The request's parent array is staged in LDS
// and walked to the root for the depth; the angles pos * theta^(-2j/D) are
// formed in fp64 (positions reach tens of thousands, where an fp32 product
// would be off by more than a bf16 step) and their cosines and sines kept in
// LDS; then every (head, 4 pairs) unit rotates dims j..j+3 with j+D/2..j+D/2+3
// in fp32 and rounds once to bf16.  Values are copied as they are.
__global__ void __launch_bounds__(256) rope_append_kernel(RopeArgs a) {
  __shared__ int sPar[ST_MAX_NODES];
  __shared__ float2 sCS[64];
  __shared__ int sPos;
  const int t = blockIdx.x;
  if (t >= a.T) return;
  const int b = st::request_of(a.node_off, a.B, t);
  const int lo = a.node_off[b], hi = a.node_off[b + 1], n = hi - lo, P = a.prefix_len[b];
  if (lo < 0 || hi > a.T || n < 1 || n > a.max_nodes) {
    if (threadIdx.x == 0) st::set_status(a.status, ST_STATUS_BAD_PARENT);
    return;
  }
  if (P < 0 || P > a.max_prefix || P + n > a.S_max) {
    if (threadIdx.x == 0) st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    return;
  }
  const int i = t - lo;
  if ((int)threadIdx.x < n) sPar[threadIdx.x] = a.parent[lo + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    int j = i, d = 0;
    bool ok = true;
    while (j != 0) {
      const int p = sPar[j];
      if (p < 0 || p >= j) {
        ok = false;
        break;
      }
      j = p;
      ++d;
    }
    if (ok && sPar[0] != -1) ok = false;
    if (!ok) st::set_status(a.status, ST_STATUS_BAD_PARENT);
    sPos = ok ? P + d : -1;
  }
  __syncthreads();
  const int pos = sPos;
  if (pos < 0) return;
  const int half = a.D / 2;
  if ((int)threadIdx.x < half) {
    const double inv_freq = pow(a.theta, -2.0 * (double)threadIdx.x / (double)a.D);
    double s, c;
    sincos((double)pos * inv_freq, &s, &c);
    sCS[threadIdx.x] = make_float2((float)c, (float)s);
  }
  __syncthreads();
  const int H = a.Hq + 2 * a.Hkv;
  const uint16_t* row = a.qkv + (size_t)t * H * a.D;
  const int qpu = half / 4;                 // 4-pair units per head
  const int rot_units = (a.Hq + a.Hkv) * qpu;
  const int cp_units = a.Hkv * (a.D / 8);   // 16-byte value chunks
  const int slot = P + i;
  for (int u = threadIdx.x; u < rot_units + cp_units; u += 256) {
    if (u < rot_units) {
      const int h = u / qpu, j = 4 * (u % qpu);
      const uint16_t* src = row + (size_t)h * a.D;
      const uint2 x1 = *(const uint2*)(src + j), x2 = *(const uint2*)(src + half + j);
      const uint16_t* p1 = (const uint16_t*)&x1;
      const uint16_t* p2 = (const uint16_t*)&x2;
      uint16_t r1[4], r2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 cs = sCS[j + e];
        const float v1 = st::bf16_to_f32(p1[e]), v2 = st::bf16_to_f32(p2[e]);
        r1[e] = st::f32_to_bf16_rne(v1 * cs.x - v2 * cs.y);
        r2[e] = st::f32_to_bf16_rne(v2 * cs.x + v1 * cs.y);
      }
      uint16_t* dst;
      if (h < a.Hq) {
        dst = a.q_out + ((size_t)t * a.Hq + h) * a.D;
      } else {
        const int g = h - a.Hq;
        dst = a.k_cache + (((size_t)b * a.Hkv + g) * a.S_max + slot) * a.D;
      }
      *(uint2*)(dst + j) = *(const uint2*)r1;
      *(uint2*)(dst + half + j) = *(const uint2*)r2;
    } else {
      const int c = u - rot_units, g = c / (a.D / 8), off = 8 * (c % (a.D / 8));
      const u32x4 v = *(const u32x4*)(row + (size_t)(a.Hq + a.Hkv + g) * a.D + off);
      *(u32x4*)(a.v_cache + (((size_t)b * a.Hkv + g) * a.S_max + slot) * a.D + off) = v;
    }
  }
}

// ---------------------------------------------------------------- skinny bf16 product

constexpr int kNT = 64;      // output features per workgroup (16 per wavefront)
constexpr int kKC = 64;      // reduction width of one ring stage

struct LinArgs {
  const uint16_t* x;         // [M][K]
  const uint16_t* w;         // [N][K]
  const uint16_t* residual;  // [M][N] or null
  void* y;                   // [M][N], bf16 or fp32
  float* part;               // [KSPLIT][M][N] when KSPLIT > 1
  int M, N, K, y_f32;
  int KSPLIT, KSL;           // reduction splits, width of one (multiple of kKC)
  int n_ntile, n_mblk, items, per_xcd;
};

// Wait until at most n stages (DPW loads each) of this wavefront are in flight.
template <int N, int DPW>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      LY_WAIT_VMCNT(N * DPW);
      return;
    }
    wait_stages<N - 1, DPW>(n);
  } else {
    LY_WAIT_VMCNT(0);
  }
}

// Rows are 128 bytes (64 bf16) in LDS; 16-byte chunk c of row r sits at
// position c ^ (r & 7), so the 16 rows read by one fragment load hit distinct
// bank groups.  A direct load writes lane l's 16 bytes at position l of the
// instruction's 1 KB (8 rows), so the swizzle is applied to the global side.
__device__ __forceinline__ void stage_row_dma(uint16_t* lds_rows, const uint16_t* base,
                                              size_t row_stride, int row, int row_clamp,
                                              int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int r = row + lane / 8, pos = lane % 8;
  const uint16_t* src = base + (size_t)min(r, row_clamp) * row_stride + 8 * (pos ^ (r & 7));
  __builtin_amdgcn_global_load_lds(src, LY_LDS_PTR(lds_rows), 16, 0, 0);
#endif
}

template <int MBLK, int kStages>
__global__ void __launch_bounds__(256) linear_kernel(LinArgs a) {
  constexpr int XR = 16 * MBLK;                      // x rows per workgroup
  constexpr int WB = kNT * kKC * 2, XB = XR * kKC * 2;
  constexpr int STAGE = WB + XB;                     // bytes
  constexpr int XI = XR / 8 / 4;                     // x loads per wavefront and stage
  constexpr int DPW = 2 + XI;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * STAGE];

  const int bid = blockIdx.x;
  int item = (bid & 7) * a.per_xcd + (bid >> 3);     // workgroups go round-robin over 8 XCDs
  if (item >= a.items) return;
  const int mblk = item % a.n_mblk;
  item /= a.n_mblk;
  const int ks = item % a.KSPLIT;
  const int ntile = item / a.KSPLIT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, grp = lane >> 4;
  const int n0 = ntile * kNT, m0 = mblk * XR;
  const int kbeg = ks * a.KSL;
  const int nst = a.KSL / kKC;
  const uint16_t* wb = a.w + kbeg;
  const uint16_t* xb = a.x + kbeg;

  // this wavefront's loads of stage s: w rows n0 + 16 wave .. +15 (two
  // instructions), then XI instructions of the x rows
  auto issue = [&](int s) {
    uint8_t* st = lds + (s % kStages) * STAGE;
    const int kofs = s * kKC;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i;
      stage_row_dma((uint16_t*)(st + r * 128), wb + kofs, (size_t)a.K, n0 + r, a.N - 1,
                    lane);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = 8 * (wave * XI + i);
      stage_row_dma((uint16_t*)(st + WB + r * 128), xb + kofs, (size_t)a.K, m0 + r, a.M - 1,
                    lane);
    }
  };

  f32x4 acc[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nst) issue(s);

  for (int it = 0; it < nst; ++it) {
    wait_stages<kStages - 2, DPW>(min(kStages - 2, nst - 1 - it));
    // every wavefront's share of stage it has landed and its reads of stage
    // it - 1 are done: then that stage is refilled.  (A fence here would make
    // the compiler wait for every direct load in flight.)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (it + kStages - 1 < nst) issue(it + kStages - 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* st = lds + (it % kStages) * STAGE;
    const uint16_t* sw = (const uint16_t*)st;
    const uint16_t* sx = (const uint16_t*)(st + WB);
    // all fragments of the stage first, then its MFMAs
    constexpr int KK = kKC / 32;
    u32x4 af[KK], bf[KK][MBLK];
    const int wr = 16 * wave + r16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 4 * kk + grp;
      af[kk] = *(const u32x4*)(sw + wr * 64 + 8 * (c ^ (wr & 7)));
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) {
        const int xr = 16 * mb + r16;
        bf[kk][mb] = *(const u32x4*)(sx + xr * 64 + 8 * (c ^ (xr & 7)));
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[kk]),
                                                          __builtin_bit_cast(bf16x8, bf[kk][mb]),
                                                          acc[mb], 0, 0, 0);
  }

  // lane (r16, grp) holds outputs (row m0 + 16 mb + r16, features n..n+3)
  const int n = n0 + 16 * wave + 4 * grp;
  if (n >= a.N) return;
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) {
    const int m = m0 + 16 * mb + r16;
    if (m >= a.M) continue;
    const size_t o = (size_t)m * a.N + n;
    f32x4 v = acc[mb];
    if (a.KSPLIT > 1) {
      *(f32x4*)(a.part + (size_t)ks * a.M * a.N + o) = v;
      continue;
    }
    if (a.residual) {
      const uint2 r = *(const uint2*)(a.residual + o);
      v[0] += __uint_as_float(r.x << 16);
      v[1] += __uint_as_float(r.x & 0xFFFF0000u);
      v[2] += __uint_as_float(r.y << 16);
      v[3] += __uint_as_float(r.y & 0xFFFF0000u);
    }
    if (a.y_f32) {
      *(f32x4*)((float*)a.y + o) = v;
    } else {
      uint2 h;
      h.x = (uint32_t)st::f32_to_bf16_rne(v[0]) | ((uint32_t)st::f32_to_bf16_rne(v[1]) << 16);
      h.y = (uint32_t)st::f32_to_bf16_rne(v[2]) | ((uint32_t)st::f32_to_bf16_rne(v[3]) << 16);
      *(uint2*)((uint16_t*)a.y + o) = h;
    }
  }
}

// Sum of the reduction splits in split order, plus the residual; 4 outputs a
// thread.
__global__ void __launch_bounds__(256) linear_reduce_kernel(LinArgs a) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t MN = (size_t)a.M * a.N;
  if (4 * q >= MN) return;
  const size_t o = 4 * q;
  f32x4 v = *(const f32x4*)(a.part + o);
  for (int s = 1; s < a.KSPLIT; ++s) v += *(const f32x4*)(a.part + (size_t)s * MN + o);
  if (a.residual) {
    const uint2 r = *(const uint2*)(a.residual + o);
    v[0] += __uint_as_float(r.x << 16);
    v[1] += __uint_as_float(r.x & 0xFFFF0000u);
    v[2] += __uint_as_float(r.y << 16);
    v[3] += __uint_as_float(r.y & 0xFFFF0000u);
  }
  if (a.y_f32) {
    *(f32x4*)((float*)a.y + o) = v;
  } else {
    uint2 h;
    h.x = (uint32_t)st::f32_to_bf16_rne(v[0]) | ((uint32_t)st::f32_to_bf16_rne(v[1]) << 16);
    h.y = (uint32_t)st::f32_to_bf16_rne(v[2]) | ((uint32_t)st::f32_to_bf16_rne(v[3]) << 16);
    *(uint2*)((uint16_t*)a.y + o) = h;
  }
}

struct LinPlan {
  int mblk_rows, n_mblk, n_ntile, KSPLIT, KSL, items;
};

// Rows per workgroup 32 (M <= 32) or 64.  The reduction is split only when
// one pass over the features and row blocks would leave more than a quarter of
// the CUs idle: the smallest divisor of the stage count that fills 3/4 of
// them, keeping at least 4 stages a split.
int linear_plan(int M, int N, int K, LinPlan& p) {
  if (M < 1 || N < 1 || K < 1) return ST_E_INVALID;
  if (K % kKC || N % 4) return ST_E_UNSUPPORTED;
  p.mblk_rows = M <= 32 ? 32 : 64;
  p.n_mblk = (M + p.mblk_rows - 1) / p.mblk_rows;
  p.n_ntile = (N + kNT - 1) / kNT;
  const long base = (long)p.n_mblk * p.n_ntile;
  const int nk = K / kKC;
  const int cus = st::device_cus();
  int ks = 1;
  const int forced = st::testing_plan().linear_ksplit;
  if (forced > 0 && nk % forced == 0) {
    ks = forced;
  } else {
    while (base * ks < (long)cus * 3 / 4) {
      int next = ks + 1;
      while (next <= nk && nk % next) ++next;
      if (next > nk || nk / next < 4) break;
      ks = next;
    }
  }
  p.KSPLIT = ks;
  p.KSL = K / ks;
  p.items = (int)(base * ks);
  return ST_OK;
}

}  // namespace

extern "C" int st_embed(int T, int d, int V, const int32_t* tokens, const void* table, void* out,
                        int32_t* status, void* stream) {
  if (T < 0 || d < 8 || d % 8 || V < 1 || !tokens || !table || !out) return ST_E_INVALID;
  if (((uintptr_t)table | (uintptr_t)out) % 16) return ST_E_INVALID;
  if (T == 0) return ST_OK;
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, T, d, V, tokens,
                     (const uint16_t*)table, (uint16_t*)out, status);
  return st::check_launch();
}

extern "C" int st_tree_rope_append(const st_tree* tree, int Hq, int Hkv, int D, float theta,
                                   const void* qkv, const int32_t* prefix_len, int max_prefix,
                                   int S_max, void* q_out, void* k_cache, void* v_cache,
                                   int32_t* status, void* stream) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (!qkv || !prefix_len || !q_out || !k_cache || !v_cache) return ST_E_INVALID;
  if (Hq < 1 || Hkv < 1 || S_max < 1 || max_prefix < 0 || !(theta > 1.f) || !isfinite(theta))
    return ST_E_INVALID;
  if (D != 64 && D != 128) return ST_E_UNSUPPORTED;
  if (((uintptr_t)qkv | (uintptr_t)q_out | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16)
    return ST_E_INVALID;
  RopeArgs a;
  a.node_off = tree->node_off;
  a.parent = tree->parent;
  a.prefix_len = prefix_len;
  a.qkv = (const uint16_t*)qkv;
  a.q_out = (uint16_t*)q_out;
  a.k_cache = (uint16_t*)k_cache;
  a.v_cache = (uint16_t*)v_cache;
  a.status = status;
  a.B = tree->B;
  a.T = tree->total_nodes;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.S_max = S_max;
  a.max_prefix = max_prefix;
  a.max_nodes = tree->max_nodes;
  a.theta = (double)theta;
  hipLaunchKernelGGL(rope_append_kernel, dim3(a.T), dim3(256), 0, (hipStream_t)stream, a);
  return st::check_launch();
}

extern "C" size_t st_linear_workspace(int M, int N, int K) {
  LinPlan p;
  if (linear_plan(M, N, K, p)) return 0;
  return p.KSPLIT > 1 ? st::align_up((size_t)p.KSPLIT * M * N * 4, 256) : 0;
}

extern "C" int st_linear(int M, int N, int K, const void* x, const void* w, const void* residual,
                         void* y, st_dtype y_dtype, void* workspace, size_t ws_bytes,
                         void* stream) {
  if (!x || !w || !y) return ST_E_INVALID;
  if (y_dtype != ST_F32 && y_dtype != ST_BF16) return ST_E_INVALID;
  LinPlan p;
  int rc = linear_plan(M, N, K, p);
  if (rc) return rc;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)residual | (uintptr_t)y) % 16)
    return ST_E_INVALID;
  LinArgs a;
  a.x = (const uint16_t*)x;
  a.w = (const uint16_t*)w;
  a.residual = (const uint16_t*)residual;
  a.y = y;
  a.part = nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.y_f32 = y_dtype == ST_F32;
  a.KSPLIT = p.KSPLIT;
  a.KSL = p.KSL;
  a.n_ntile = p.n_ntile;
  a.n_mblk = p.n_mblk;
  a.items = p.items;
  a.per_xcd = (p.items + 7) / 8;
  if (p.KSPLIT > 1) {
    const size_t need = (size_t)p.KSPLIT * M * N * 4;
    if (!workspace || ws_bytes < need || (uintptr_t)workspace % 16) return ST_E_WORKSPACE;
    a.part = (float*)workspace;
  }
  const dim3 grid(8 * a.per_xcd);
  // 4 stages (64 KB of LDS at 64 rows: two workgroups per CU) measured
  // faster than 8 (one per CU) on the 7B-shaped projections
  const bool deep = st::testing_plan().linear_stages == 8;
  if (p.mblk_rows == 32) {
    if (deep)
      hipLaunchKernelGGL((linear_kernel<2, 8>), grid, dim3(256), 0, (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL((linear_kernel<2, 4>), grid, dim3(256), 0, (hipStream_t)stream, a);
  } else {
    if (deep)
      hipLaunchKernelGGL((linear_kernel<4, 8>), grid, dim3(256), 0, (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL((linear_kernel<4, 4>), grid, dim3(256), 0, (hipStream_t)stream, a);
  }
  if ((rc = st::check_launch())) return rc;
  if (p.KSPLIT > 1) {
    const size_t quads = (size_t)M * N / 4;
    hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, a);
    rc = st::check_launch();
  }
  return rc;
}

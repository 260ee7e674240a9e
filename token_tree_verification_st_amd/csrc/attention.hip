// Tree-masked attention of every tree node over its request's cached prefix
// and its own root path ("SpecInfer：基于树结构的LLM推测性推理加速技术" §2.1:
// scores = Q K^T, masked entries excluded, softmax, times V; the SpecInfer news
// article, "Token 樹驗證器": all tree paths are decoded in one pass).
//
// Work decomposition (split-KV).  For request b and kv head g the query rows
// are the N_b tree nodes times the G = Hq/Hkv query heads sharing g; every one
// of them reads the same keys, so a workgroup takes a block of rows and a
// contiguous range of keys ("split") and streams that range once.  Splits
// produce fp32 partials (running max m, sum l, unnormalised output) that a
// combine kernel merges with a log-sum-exp rescale; a request whose keys fit in
// one split writes its output directly.
//
// bf16 path (MFMA, gfx950).  One workgroup = 4 wavefronts = 64 query rows, 16
// per wavefront.  Each 64-key tile of K is copied to LDS with padded rows; the
// V tile is transposed on its way into LDS.  Per wavefront and tile:
//   S^T (keys x rows) = K . Q^T    with v_mfma_f32_16x16x32_bf16, A = K from
//                                  LDS, B = Q^T held in registers
//   online softmax on S^T          each lane holds 4 keys of one row, so the
//                                  row statistics live in that lane and need
//                                  only two cross-lane steps per tile
//   O^T (dims x rows) += V^T . P^T A = V^T from LDS, B = P^T straight from
//                                  the S^T accumulators converted to bf16
// Keys beyond the prefix are tree keys: key P_b + j is visible to a row iff
// bit j of its node's ancestor mask is set.
//
// fp32 path (VALU).  The same decomposition with 16 rows per workgroup and
// plain fp32 dot products; it serves fp32 inputs, which need 1e-5 accuracy.
#include "st_internal.h"

#include <math.h>
#include <stdlib.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKT = 64;  // keys per tile

struct AttnArgs {
  const int32_t* node_off;
  const int32_t* prefix_len;
  const uint64_t* mask;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  float2* ws_ml;   // [NS][T*Hq] (m in log2 units, l)
  float* ws_acc;   // [NS][T*Hq][D]
  int32_t* status;
  int B, T, Hq, Hkv, G, S_max, W, max_nodes, max_prefix;
  int KS;          // keys per split (multiple of kKT)
  int NS;          // splits of the longest request
  int RB;          // rows per workgroup
  int n_rblk;      // row blocks of the widest request
  int items;       // B * Hkv * NS * n_rblk
  int per_xcd;     // ceil(items / 8)
  float scale_log2;
};

struct Item {
  int b, g, split, rblk;
};

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).  Item w
// goes to XCD w / per_xcd, so consecutive items -- the row blocks of one
// (request, head, split), which read the same keys -- share an XCD's L2.
__device__ inline bool decode_item(const AttnArgs& a, Item& it) {
  const int bid = blockIdx.x;
  int w = (bid & 7) * a.per_xcd + (bid >> 3);
  if (w >= a.items) return false;
  it.rblk = w % a.n_rblk;
  w /= a.n_rblk;
  it.split = w % a.NS;
  w /= a.NS;
  it.g = w % a.Hkv;
  it.b = w / a.Hkv;
  return true;
}

struct ReqInfo {
  int lo, n, P, key_end, nsplit;
  bool ok;
};

__device__ inline ReqInfo request_info(const AttnArgs& a, int b) {
  ReqInfo r;
  r.lo = a.node_off[b];
  const int hi = a.node_off[b + 1];
  r.n = hi - r.lo;
  r.P = a.prefix_len[b];
  r.ok = r.lo >= 0 && hi <= a.T && r.n >= 1 && r.n <= a.max_nodes && r.P >= 0 &&
         r.P <= a.max_prefix && r.P + r.n <= a.S_max;
  r.key_end = r.P + r.n;
  r.nsplit = (r.key_end + a.KS - 1) / a.KS;
  return r;
}

__device__ inline bool tree_bit(uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3, int j) {
  const int wi = j >> 6;
  const uint64_t w = wi == 0 ? w0 : wi == 1 ? w1 : wi == 2 ? w2 : w3;
  return (w >> (j & 63)) & 1ull;
}

// ---------------------------------------------------------------- bf16 MFMA

template <int D>
__global__ void __launch_bounds__(256)
attn_mfma_kernel(AttnArgs a) {
  constexpr int DP = D + 8;       // K row pitch (bf16): 16-byte pad
  constexpr int KP = kKT + 4;     // V^T row pitch (bf16): 8-byte pad
  constexpr int NKS = D / 32;     // k-steps of S^T
  constexpr int NDB = D / 16;     // d-blocks of O^T
  constexpr int CH = D / 8;       // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * DP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * KP];

  Item it;
  if (!decode_item(a, it)) return;
  const ReqInfo rq = request_info(a, it.b);
  if (!rq.ok) {
    if (threadIdx.x == 0 && it.g == 0 && it.split == 0 && it.rblk == 0)
      st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    return;
  }
  const int rows_b = rq.n * a.G;
  if (it.rblk * 64 >= rows_b) return;
  const int k0 = it.split * a.KS;
  if (k0 >= rq.key_end) return;
  const int k1 = min(k0 + a.KS, rq.key_end);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int row = it.rblk * 64 + wave * 16 + r16;
  const bool row_ok = row < rows_b;
  const int node = row_ok ? row / a.G : 0;
  const int hq = it.g * a.G + (row_ok ? row % a.G : 0);
  const int grow = (rq.lo + node) * a.Hq + hq;

  const uint16_t* qp = (const uint16_t*)a.q + (size_t)grow * D;
  bf16x8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    uint4 u = row_ok ? *(const uint4*)(qp + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0);
    qf[s] = __builtin_bit_cast(bf16x8, u);
  }
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  if (row_ok) {
    const uint64_t* mr = a.mask + (size_t)(rq.lo + node) * a.W;
    mw0 = mr[0];
    if (a.W > 1) mw1 = mr[1];
    if (a.W > 2) mw2 = mr[2];
    if (a.W > 3) mw3 = mr[3];
  }

  const size_t head_off = ((size_t)it.b * a.Hkv + it.g) * (size_t)a.S_max * D;
  const uint16_t* kg = (const uint16_t*)a.k + head_off;
  const uint16_t* vg = (const uint16_t*)a.v + head_off;

  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // cooperative tile loads: K rows straight, V rows as 4-key x 8-dim blocks
  for (int kt = k0; kt < k1; kt += kKT) {
    const int nk = min(kKT, k1 - kt);
    __syncthreads();
#pragma unroll
    for (int e = tid; e < kKT * CH; e += 256) {
      const int r = e / CH, c = e % CH;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < nk) u = *(const uint4*)(kg + (size_t)(kt + r) * D + 8 * c);
      *(uint4*)(&sK[r * DP + 8 * c]) = u;
    }
#pragma unroll
    for (int e = tid; e < (kKT / 4) * CH; e += 256) {
      const int quad = e / CH, c = e % CH;
      uint4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * quad + i;
        x[i] = r < nk ? *(const uint4*)(vg + (size_t)(kt + r) * D + 8 * c) : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* x0 = (const uint32_t*)&x[0];
      const uint32_t* x1 = (const uint32_t*)&x[1];
      const uint32_t* x2 = (const uint32_t*)&x[2];
      const uint32_t* x3 = (const uint32_t*)&x[3];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint2 lo2, hi2;  // dims 8c+2e2 and 8c+2e2+1, keys 4quad..4quad+3
        lo2.x = (x0[e2] & 0xFFFFu) | (x1[e2] << 16);
        lo2.y = (x2[e2] & 0xFFFFu) | (x3[e2] << 16);
        hi2.x = (x0[e2] >> 16) | (x1[e2] & 0xFFFF0000u);
        hi2.y = (x2[e2] >> 16) | (x3[e2] & 0xFFFF0000u);
        *(uint2*)(&sVt[(8 * c + 2 * e2) * KP + 4 * quad]) = lo2;
        *(uint2*)(&sVt[(8 * c + 2 * e2 + 1) * KP + 4 * quad]) = hi2;
      }
    }
    __syncthreads();

    // S^T = K Q^T over four 16-key blocks
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 u = *(const uint4*)(&sK[(16 * kb + r16) * DP + 32 * ks + 8 * grp]);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), qf[ks],
                                                        s[kb], 0, 0, 0);
      }
    }
    // scale, mask, tile max (lane holds keys kt + 16kb + 4grp + j of its row)
    const bool tree_tile = kt + kKT > rq.P;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kt + 16 * kb + 4 * grp + j;
        bool vis = key < k1;
        if (tree_tile && key >= rq.P) vis = vis && tree_bit(mw0, mw1, mw2, mw3, key - rq.P);
        const float x = vis ? s[kb][j] * a.scale_log2 : -INFINITY;
        s[kb][j] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, ST_WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, ST_WAVE));
    const float m_new = fmaxf(m, tmax);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - mref);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(s[kb][j] - mref);
        s[kb][j] = p;
        psum += p;
      }
    }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] *= alpha;

    bf16x8 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pb[t][j] = (__bf16)s[2 * t][j];
        pb[t][4 + j] = (__bf16)s[2 * t + 1][j];
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* vr = &sVt[(16 * db + r16) * KP + 32 * t + 4 * grp];
        const uint2 lo2 = *(const uint2*)vr;
        const uint2 hi2 = *(const uint2*)(vr + 16);
        const uint4 u = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), pb[t],
                                                         acc[db], 0, 0, 0);
      }
    }
  }

  lsum += __shfl_xor(lsum, 16, ST_WAVE);
  lsum += __shfl_xor(lsum, 32, ST_WAVE);
  if (!row_ok) return;
  if (rq.nsplit == 1) {
    const float inv = 1.f / lsum;
    uint16_t* op = (uint16_t*)a.out + (size_t)grow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      uint2 o;
      o.x = (uint32_t)st::f32_to_bf16_rne(acc[db][0] * inv) |
            ((uint32_t)st::f32_to_bf16_rne(acc[db][1] * inv) << 16);
      o.y = (uint32_t)st::f32_to_bf16_rne(acc[db][2] * inv) |
            ((uint32_t)st::f32_to_bf16_rne(acc[db][3] * inv) << 16);
      *(uint2*)(op + 16 * db + 4 * grp) = o;
    }
    if (a.lse && grp == 0) a.lse[grow] = (m + log2f(lsum)) * kLn2;
  } else {
    const size_t TH = (size_t)a.T * a.Hq;
    const size_t pr = (size_t)it.split * TH + grow;
    float* wp = a.ws_acc + pr * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) *(f32x4*)(wp + 16 * db + 4 * grp) = acc[db];
    if (grp == 0) a.ws_ml[pr] = make_float2(m, lsum);
  }
}

// ---------------------------------------------------------------- VALU path

template <typename Tin>
__device__ inline float load_val(const Tin* p);
template <>
__device__ inline float load_val<float>(const float* p) { return *p; }
template <>
__device__ inline float load_val<uint16_t>(const uint16_t* p) { return st::bf16_to_f32(*p); }

template <typename Tin>
__device__ inline void store_val(Tin* p, float x);
template <>
__device__ inline void store_val<float>(float* p, float x) { *p = x; }
template <>
__device__ inline void store_val<uint16_t>(uint16_t* p, float x) { *p = st::f32_to_bf16_rne(x); }

template <typename Tin, int D>
__global__ void __launch_bounds__(256)
attn_valu_kernel(AttnArgs a) {
  constexpr int R = 16;                // rows per workgroup
  constexpr int DJ = D / 16;           // output dims per thread
  constexpr int KT = D > 64 ? 32 : 64; // keys per tile (LDS stays under 64 KB)
  constexpr int KJ = KT / 16;          // keys per thread and tile
  __shared__ float sQ[R][D];
  __shared__ float sK[KT][D + 1];
  __shared__ float sV[KT][D];
  __shared__ float sP[R][KT];

  Item it;
  if (!decode_item(a, it)) return;
  const ReqInfo rq = request_info(a, it.b);
  if (!rq.ok) {
    if (threadIdx.x == 0 && it.g == 0 && it.split == 0 && it.rblk == 0)
      st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    return;
  }
  const int rows_b = rq.n * a.G;
  if (it.rblk * R >= rows_b) return;
  const int k0 = it.split * a.KS;
  if (k0 >= rq.key_end) return;
  const int k1 = min(k0 + a.KS, rq.key_end);

  const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
  const int row = it.rblk * R + r;
  const bool row_ok = row < rows_b;
  const int node = row_ok ? row / a.G : 0;
  const int hq = it.g * a.G + (row_ok ? row % a.G : 0);
  const int grow = (rq.lo + node) * a.Hq + hq;

  const Tin* qp = (const Tin*)a.q + (size_t)grow * D;
  for (int d = c; d < D; d += 16) sQ[r][d] = row_ok ? load_val(qp + d) : 0.f;
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  if (row_ok) {
    const uint64_t* mr = a.mask + (size_t)(rq.lo + node) * a.W;
    mw0 = mr[0];
    if (a.W > 1) mw1 = mr[1];
    if (a.W > 2) mw2 = mr[2];
    if (a.W > 3) mw3 = mr[3];
  }
  const size_t head_off = ((size_t)it.b * a.Hkv + it.g) * (size_t)a.S_max * D;
  const Tin* kg = (const Tin*)a.k + head_off;
  const Tin* vg = (const Tin*)a.v + head_off;

  float acc[DJ];
#pragma unroll
  for (int j = 0; j < DJ; ++j) acc[j] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  for (int kt = k0; kt < k1; kt += KT) {
    const int nk = min(KT, k1 - kt);
    __syncthreads();
#pragma unroll 4
    for (int e = tid; e < KT * D; e += 256) {
      const int kr = e / D, d = e % D;
      const bool ok = kr < nk;
      sK[kr][d] = ok ? load_val(kg + (size_t)(kt + kr) * D + d) : 0.f;
      sV[kr][d] = ok ? load_val(vg + (size_t)(kt + kr) * D + d) : 0.f;
    }
    __syncthreads();
    float dot[KJ];
#pragma unroll
    for (int j = 0; j < KJ; ++j) dot[j] = 0.f;
#pragma unroll 4
    for (int d = 0; d < D; ++d) {
      const float qd = sQ[r][d];
#pragma unroll
      for (int j = 0; j < KJ; ++j) dot[j] += qd * sK[c + 16 * j][d];
    }
    float x[KJ];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int key = kt + c + 16 * j;
      bool vis = key < k1;
      if (key >= rq.P) vis = vis && tree_bit(mw0, mw1, mw2, mw3, key - rq.P);
      x[j] = vis ? dot[j] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[j]);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 16));
    const float m_new = fmaxf(m, tmax);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - mref);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const float p = exp2f(x[j] - mref);
      sP[r][c + 16 * j] = p;
      psum += p;
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 16);
    lsum = lsum * alpha + psum;
    m = m_new;
    __syncthreads();
    float pv[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) pv[j] = 0.f;
#pragma unroll 4
    for (int kk = 0; kk < KT; ++kk) {
      const float p = sP[r][kk];
#pragma unroll
      for (int j = 0; j < DJ; ++j) pv[j] += p * sV[kk][c + 16 * j];
    }
#pragma unroll
    for (int j = 0; j < DJ; ++j) acc[j] = acc[j] * alpha + pv[j];
  }
  if (!row_ok) return;
  if (rq.nsplit == 1) {
    const float inv = 1.f / lsum;
    Tin* op = (Tin*)a.out + (size_t)grow * D;
#pragma unroll
    for (int j = 0; j < DJ; ++j) store_val(op + c + 16 * j, acc[j] * inv);
    if (a.lse && c == 0) a.lse[grow] = (m + log2f(lsum)) * kLn2;
  } else {
    const size_t pr = (size_t)it.split * a.T * a.Hq + grow;
    float* wp = a.ws_acc + pr * D;
#pragma unroll
    for (int j = 0; j < DJ; ++j) wp[c + 16 * j] = acc[j];
    if (c == 0) a.ws_ml[pr] = make_float2(m, lsum);
  }
}

// ---------------------------------------------------------------- combine

template <typename Tout, int D>
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 4;        // lanes per row, 4 dims each
  constexpr int RPB = 256 / LPR;    // rows per block
  const int grow = blockIdx.x * RPB + threadIdx.x / LPR;
  const int d = 4 * (threadIdx.x % LPR);
  const int TH = a.T * a.Hq;
  if (grow >= TH) return;
  const int t = grow / a.Hq;
  const int b = st::request_of(a.node_off, a.B, t);
  const ReqInfo rq = request_info(a, b);
  if (!rq.ok || rq.nsplit <= 1) return;
  float M = -INFINITY;
  for (int s = 0; s < rq.nsplit; ++s) M = fmaxf(M, a.ws_ml[(size_t)s * TH + grow].x);
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < rq.nsplit; ++s) {
    const size_t pr = (size_t)s * TH + grow;
    const float2 ml = a.ws_ml[pr];
    const float w = exp2f(ml.x - M);  // empty split: exp2(-inf) = 0
    L += w * ml.y;
    const f32x4 x = *(const f32x4*)(a.ws_acc + pr * D + d);
    o += w * x;
  }
  const float inv = 1.f / L;
  Tout* op = (Tout*)a.out + (size_t)grow * D + d;
#pragma unroll
  for (int j = 0; j < 4; ++j) store_val(op + j, o[j] * inv);
  if (a.lse && d == 0) a.lse[grow] = (M + log2f(L)) * kLn2;
}

// ---------------------------------------------------------------- planning

struct Plan {
  bool mfma;
  int RB, n_rblk, KS, NS, items, per_xcd;
  size_t ml_bytes, ws_bytes;
};

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

int make_plan(const st_tree* t, int Hq, int Hkv, int D, st_dtype dtype, int max_prefix, Plan& p) {
  int rc = st::check_tree_host(t);
  if (rc) return rc;
  if (Hq < 1 || Hkv < 1 || max_prefix < 0) return ST_E_INVALID;
  if (dtype != ST_F32 && dtype != ST_BF16) return ST_E_INVALID;
  if (Hq % Hkv || (D != 64 && D != 128)) return ST_E_UNSUPPORTED;
  const int G = Hq / Hkv;
  p.mfma = dtype == ST_BF16;
  p.RB = p.mfma ? 64 : 16;
  p.n_rblk = (t->max_nodes * G + p.RB - 1) / p.RB;
  const long keys_max = (long)max_prefix + t->max_nodes;
  const long base = (long)t->B * Hkv * p.n_rblk;
  // aim for about `target` workgroups over the whole batch; the key range of
  // one split is a whole number of tiles
  const long target = env_int("ST_ATTN_TARGET_WG", 512);
  long ks = (keys_max * base + target - 1) / target;
  ks = (ks + kKT - 1) / kKT * kKT;
  const int forced = env_int("ST_ATTN_SPLIT_KEYS", 0);
  if (forced > 0) ks = (forced + kKT - 1) / kKT * kKT;
  const long kmax = (keys_max + kKT - 1) / kKT * kKT;
  if (ks < kKT) ks = kKT;
  if (ks > kmax) ks = kmax;
  p.KS = (int)ks;
  p.NS = (int)((keys_max + ks - 1) / ks);
  const long items = base * p.NS;
  if (items > (1L << 30)) return ST_E_UNSUPPORTED;
  p.items = (int)items;
  p.per_xcd = (p.items + 7) / 8;
  const size_t TH = (size_t)t->total_nodes * Hq;
  p.ml_bytes = p.NS > 1 ? st::align_up((size_t)p.NS * TH * sizeof(float2), 256) : 0;
  p.ws_bytes = p.NS > 1 ? p.ml_bytes + (size_t)p.NS * TH * D * sizeof(float) : 0;
  return ST_OK;
}

}  // namespace

extern "C" size_t st_tree_attention_workspace(const st_tree* tree, int Hq, int Hkv, int D,
                                              st_dtype dtype, int max_prefix) {
  Plan p;
  if (make_plan(tree, Hq, Hkv, D, dtype, max_prefix, p)) return 0;
  return p.ws_bytes;
}

extern "C" int st_tree_attention(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                                 float scale, const void* q, const void* k_cache,
                                 const void* v_cache, int S_max, const int32_t* prefix_len,
                                 int max_prefix, const uint64_t* mask, void* out, float* lse,
                                 void* workspace, size_t ws_bytes, int32_t* status,
                                 void* stream) {
  Plan p;
  int rc = make_plan(tree, Hq, Hkv, D, dtype, max_prefix, p);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !prefix_len || !mask || !out || S_max < 1 ||
      !(scale > 0.f) || !isfinite(scale))
    return ST_E_INVALID;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) % 16)
    return ST_E_INVALID;
  if (p.ws_bytes && (!workspace || ws_bytes < p.ws_bytes)) return ST_E_WORKSPACE;
  AttnArgs a;
  a.node_off = tree->node_off;
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.lse = lse;
  a.ws_ml = p.ws_bytes ? (float2*)workspace : nullptr;
  a.ws_acc = p.ws_bytes ? (float*)((char*)workspace + p.ml_bytes) : nullptr;
  a.status = status;
  a.B = tree->B;
  a.T = tree->total_nodes;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.S_max = S_max;
  a.W = st::mask_words(tree->max_nodes);
  a.max_nodes = tree->max_nodes;
  a.max_prefix = max_prefix;
  a.KS = p.KS;
  a.NS = p.NS;
  a.RB = p.RB;
  a.n_rblk = p.n_rblk;
  a.items = p.items;
  a.per_xcd = p.per_xcd;
  a.scale_log2 = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(8 * p.per_xcd), block(256);
  if (p.mfma) {
    if (D == 128) hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, block, 0, s, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((attn_valu_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_valu_kernel<float, 64>), grid, block, 0, s, a);
  }
  if ((rc = st::check_launch())) return rc;
  if (p.NS > 1) {
    const int TH = tree->total_nodes * Hq;
    const int rpb = 256 / (D / 4);
    const dim3 cg((TH + rpb - 1) / rpb);
    if (p.mfma) {
      if (D == 128) hipLaunchKernelGGL((attn_combine_kernel<uint16_t, 128>), cg, block, 0, s, a);
      else hipLaunchKernelGGL((attn_combine_kernel<uint16_t, 64>), cg, block, 0, s, a);
    } else {
      if (D == 128) hipLaunchKernelGGL((attn_combine_kernel<float, 128>), cg, block, 0, s, a);
      else hipLaunchKernelGGL((attn_combine_kernel<float, 64>), cg, block, 0, s, a);
    }
    rc = st::check_launch();
  }
  return rc;
}

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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKT = 64;  // keys per tile
// MFMA workgroup shapes (row-waves of 16 rows x key groups); the plan picks one
struct Shape {
  int rw, kw;
};
constexpr Shape kShapes[] = {{4, 1}, {4, 2}, {2, 2}, {2, 4}, {1, 4}};

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
  int KS;          // keys per split (multiple of 16)
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

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for all of its outstanding global loads
// -- including the prefetch of later tiles that should stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// V tiles sit in LDS in their natural [key][dim] layout (256-byte rows, no
// padding).  The MFMA operand V^T is read with ds_read_b64_tr_b16, which
// hands each lane one dim of four keys.  Each 16-byte chunk c of key row r is
// stored at chunk position c ^ vswz(r): the 16 lanes of one transposed read
// touch four key rows x two chunks, which land on eight distinct positions.
// (masked to the row's chunk count, so a position never leaves its row)
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return (((key & 3) << 1) | (((key >> 2) & 1) << 3)) & (D / 8 - 1);
}

// What one thread of a key group (GS threads) moves from global memory to LDS
// for one 64-key tile: N 16-byte chunks of K rows and N of V rows.
template <int D, int GS>
struct TileRegs {
  static constexpr int CH = D / 8;
  static constexpr int TOT = kKT * CH;
  static constexpr int N = (TOT + GS - 1) / GS;
  u32x4 k[N];
  u32x4 v[N];
};

// Every load is issued unconditionally (the compiler can then count them and
// keep the next round in flight): key indices are clamped into [k0, k1 - 1],
// so rows past the end of the range hold copies of valid rows, which the
// score mask excludes and which meet a zero probability in P V.
template <int D, int GS>
__device__ __forceinline__ void tile_load(TileRegs<D, GS>& r, const uint16_t* kg, const uint16_t* vg,
                                          int kt, int klast, int gt) {
  using TR = TileRegs<D, GS>;
#pragma unroll
  for (int i = 0; i < TR::N; ++i) {
    const int e = min(gt + i * GS, TR::TOT - 1), row = e / TR::CH, c = e % TR::CH;
    const size_t off = (size_t)min(kt + row, klast) * D + 8 * c;
    r.k[i] = *(const u32x4*)(kg + off);
    r.v[i] = *(const u32x4*)(vg + off);
  }
}

template <int D, int GS>
__device__ __forceinline__ void tile_store(const TileRegs<D, GS>& r, uint16_t* sK, uint16_t* sV,
                                           int gt) {
  using TR = TileRegs<D, GS>;
  constexpr int DP = D + 8;
#pragma unroll
  for (int i = 0; i < TR::N; ++i) {
    const int e = gt + i * GS, row = e / TR::CH, c = e % TR::CH;
    if (TR::N * GS == TR::TOT || e < TR::TOT) {
      *(u32x4*)(&sK[row * DP + 8 * c]) = r.k[i];
      *(u32x4*)(&sV[row * D + 8 * (c ^ vswz<D>(row))]) = r.v[i];
    }
  }
}

struct TileCtx {
  int P, k1, r16, grp;
  float scale_log2;
  uint64_t mw0, mw1, mw2, mw3;
};

// One wavefront's work on one 64-key tile in LDS: S^T = K Q^T, mask, online
// softmax update of (m, lsum, acc), O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void tile_compute(const TileCtx& cx, const uint16_t* sK,
                                             const uint16_t* sV, int kt,
                                             const bf16x8 (&qf)[D / 32], f32x4 (&acc)[D / 16],
                                             float& m, float& lsum) {
  constexpr int DP = D + 8, NKS = D / 32, NDB = D / 16;
  const int r16 = cx.r16, grp = cx.grp;

    // S^T = K Q^T over four 16-key blocks; lane holds keys kt+16kb+4grp+j
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
    const bool edge = kt + kKT > cx.P || kt + kKT > cx.k1;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[kb][j] * cx.scale_log2;
        if (edge) {
          const int key = kt + 16 * kb + 4 * grp + j;
          bool vis = key < cx.k1;
          if (key >= cx.P) vis = vis && tree_bit(cx.mw0, cx.mw1, cx.mw2, cx.mw3, key - cx.P);
          x = vis ? x : -INFINITY;
        }
        s[kb][j] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, ST_WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, ST_WAVE));
    const float m_new = fmaxf(m, tmax);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - mref);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(s[kb][j] - mref);
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
    // O^T += V^T P^T.  Transposed reads: lane k = 4j + q of each 16-lane
    // group points at V[key_j][16db + 4q .. +3]; lane i then receives dim
    // 16db + i of key_0..key_3 (keys 32t + 4grp + j, and + 16 for slots 4-7).
    const int jq = r16 >> 2, qq = r16 & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key1 = 32 * t + 4 * grp + jq, key2 = key1 + 16;
        const int c = 2 * db + (qq >> 1), sub = 4 * (qq & 1);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(sV + key1 * D + 8 * (c ^ vswz<D>(key1)) + sub));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(sV + key2 * D + 8 * (c ^ vswz<D>(key2)) + sub));
        const v8i16 u = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u), pb[t],
                                                         acc[db], 0, 0, 0);
      }
    }
}

// One workgroup = RW row-waves x KW key groups.  Row-wave rw owns 16 query
// rows; key group kg takes every KW-th 64-key tile of the workgroup's key
// range, with its own LDS buffers and its own running softmax state.  The
// tiles of the next round are loaded into registers while the current round
// is computed.  At the end the key groups' states are merged through LDS.
template <int D, int RW, int KW>
__global__ void __launch_bounds__(64 * RW * KW)
attn_mfma_kernel(AttnArgs a) {
  constexpr int GS = 64 * RW;      // threads per key group
  constexpr int ROWS = 16 * RW;    // query rows per workgroup
  constexpr int DP = D + 8;        // K row pitch (bf16): 16-byte pad
  constexpr int NKS = D / 32;      // k-steps of S^T
  constexpr int NDB = D / 16;      // d-blocks of O^T
  constexpr int KEL = kKT * DP, VEL = kKT * D;
  constexpr int MERGE_FLOATS = (KW - 1) * RW * 64 * (4 * NDB + 2);
  constexpr int TILE_BYTES = KW * (KEL + VEL) * 2;
  constexpr int LDS_BYTES = TILE_BYTES > MERGE_FLOATS * 4 ? TILE_BYTES : MERGE_FLOATS * 4;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_BYTES / 2];

  Item it;
  if (!decode_item(a, it)) return;
  const ReqInfo rq = request_info(a, it.b);
  if (!rq.ok) {
    if (threadIdx.x == 0 && it.g == 0 && it.split == 0 && it.rblk == 0)
      st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    return;
  }
  const int rows_b = rq.n * a.G;
  if (it.rblk * ROWS >= rows_b) return;
  const int k0 = it.split * a.KS;
  if (k0 >= rq.key_end) return;
  const int k1 = min(k0 + a.KS, rq.key_end);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rw = wave % RW, kg = wave / RW, gt = tid % GS;
  const int r16 = lane & 15, grp = lane >> 4;
  const int row = it.rblk * ROWS + rw * 16 + r16;
  const bool row_ok = row < rows_b;
  const int node = row_ok ? row / a.G : 0;
  const int hq = it.g * a.G + (row_ok ? row % a.G : 0);
  const int grow = (rq.lo + node) * a.Hq + hq;
  uint16_t* sK = lds + kg * (KEL + VEL);
  uint16_t* sV = sK + KEL;

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
  const uint16_t* kgp = (const uint16_t*)a.k + head_off;
  const uint16_t* vgp = (const uint16_t*)a.v + head_off;

  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const int niters = (k1 - k0 + KW * kKT - 1) / (KW * kKT);
  // Software pipeline two rounds deep: the tiles of round r+2 load into the
  // register set that round r has just stored to LDS, so two rounds of loads
  // are in flight while round r is computed.
  auto tile_at = [&](int r) { return k0 + (r * KW + kg) * kKT; };
  const TileCtx cx{rq.P, k1, r16, grp, a.scale_log2, mw0, mw1, mw2, mw3};
  TileRegs<D, GS> ra, rb;
  const int klast = k1 - 1;
  // keep the two rounds' loads in program order (the wait before each store
  // counts on it)
  tile_load<D, GS>(ra, kgp, vgp, tile_at(0), klast, gt);
  __builtin_amdgcn_sched_barrier(0);
  tile_load<D, GS>(rb, kgp, vgp, tile_at(1), klast, gt);
  __builtin_amdgcn_sched_barrier(0);
  for (int iter = 0; iter < niters; iter += 2) {
    {
      const int kt = tile_at(iter), nk = min(kKT, k1 - kt);
      lds_barrier();
      tile_store<D, GS>(ra, sK, sV, gt);
      lds_barrier();
      // unconditional (past the end it re-reads the clamped last row), so the
      // compiler can wait for exactly the older round at the next store
      __builtin_amdgcn_sched_barrier(0);
      tile_load<D, GS>(ra, kgp, vgp, tile_at(iter + 2), klast, gt);
      __builtin_amdgcn_sched_barrier(0);
      if (nk > 0) tile_compute<D>(cx, sK, sV, kt, qf, acc, m, lsum);
    }
    {  // runs even past the last round (its compute is then skipped): no early
       // exit, so the wait counts stay exact
      const int kt = tile_at(iter + 1), nk = min(kKT, k1 - kt);
      lds_barrier();
      tile_store<D, GS>(rb, sK, sV, gt);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      tile_load<D, GS>(rb, kgp, vgp, tile_at(iter + 3), klast, gt);
      __builtin_amdgcn_sched_barrier(0);
      if (nk > 0) tile_compute<D>(cx, sK, sV, kt, qf, acc, m, lsum);
    }
  }

  lsum += __shfl_xor(lsum, 16, ST_WAVE);
  lsum += __shfl_xor(lsum, 32, ST_WAVE);
  if constexpr (KW > 1) {
    // merge the key groups' states into group 0 (struct of arrays, lane-major)
    float* mb = (float*)lds;
    constexpr int SLOTS = (KW - 1) * RW * 64;
    __syncthreads();
    if (kg > 0) {
      const int sl = ((kg - 1) * RW + rw) * 64 + lane;
      mb[sl] = m;
      mb[SLOTS + sl] = lsum;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) mb[(2 + 4 * db + j) * SLOTS + sl] = acc[db][j];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int k = 1; k < KW; ++k) {
      const int sl = ((k - 1) * RW + rw) * 64 + lane;
      const float mk = mb[sl], lk = mb[SLOTS + sl];
      const float M = fmaxf(m, mk);
      const float ref = M == -INFINITY ? 0.f : M;
      const float e0 = fast_exp2(m - ref), e1 = fast_exp2(mk - ref);
      lsum = lsum * e0 + lk * e1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[db][j] = acc[db][j] * e0 + mb[(2 + 4 * db + j) * SLOTS + sl] * e1;
      m = M;
    }
  }
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

// Merge the splits of every row: the partial (m, l) pairs and 4 dims of the
// partial outputs of up to 8 splits are all loaded before any is used.
template <typename Tout, int D>
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 4;        // lanes per row, 4 dims each
  constexpr int RPB = 256 / LPR;    // rows per block
  constexpr int CHUNK = 8;
  const int grow = blockIdx.x * RPB + threadIdx.x / LPR;
  const int d = 4 * (threadIdx.x % LPR);
  const int TH = a.T * a.Hq;
  if (grow >= TH) return;
  const int t = grow / a.Hq;
  const int b = st::request_of(a.node_off, a.B, t);
  const ReqInfo rq = request_info(a, b);
  if (!rq.ok || rq.nsplit <= 1) return;
  const int ns = rq.nsplit;
  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += CHUNK) {
    float2 ml[CHUNK];
    f32x4 x[CHUNK];
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      const int s = min(s0 + j, ns - 1);
      const size_t pr = (size_t)s * TH + grow;
      ml[j] = a.ws_ml[pr];
      x[j] = *(const f32x4*)(a.ws_acc + pr * D + d);
    }
    float Mc = M;
#pragma unroll
    for (int j = 0; j < CHUNK; ++j)
      if (s0 + j < ns) Mc = fmaxf(Mc, ml[j].x);
    const float ref = Mc == -INFINITY ? 0.f : Mc;
    const float sc = exp2f(M - ref);  // rescale what is merged so far
    L *= sc;
    o *= sc;
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      if (s0 + j < ns) {
        const float w = exp2f(ml[j].x - ref);  // empty split: exp2(-inf) = 0
        L += w * ml[j].y;
        o += w * x[j];
      }
    }
    M = Mc;
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
  int shape;
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
  p.shape = env_int("ST_ATTN_SHAPE", 0);
  if (p.shape < 0 || p.shape >= (int)(sizeof(kShapes) / sizeof(kShapes[0]))) p.shape = 0;
  p.RB = p.mfma ? 16 * kShapes[p.shape].rw : 16;
  p.n_rblk = (t->max_nodes * G + p.RB - 1) / p.RB;
  const long keys_max = (long)max_prefix + t->max_nodes;
  const long base = (long)t->B * Hkv * p.n_rblk;
  // aim for about `target` workgroups over the whole batch (one per CU for
  // the MFMA kernel); splits are even, in multiples of 16 keys
  const long target = env_int("ST_ATTN_TARGET_WG", p.mfma ? 256 : 512);
  long ns = (target + base - 1) / base;
  if (ns < 1) ns = 1;
  long ks = (keys_max + ns - 1) / ns;
  ks = (ks + 15) / 16 * 16;
  const int forced = env_int("ST_ATTN_SPLIT_KEYS", 0);
  if (forced > 0) ks = (forced + 15) / 16 * 16;
  const long kmax = (keys_max + 15) / 16 * 16;
  if (ks < 64) ks = 64;
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
    const Shape sh = kShapes[p.shape];
    const dim3 mblock(64 * sh.rw * sh.kw);
#define ST_LAUNCH_MFMA(RW_, KW_)                                                             \
  if (sh.rw == RW_ && sh.kw == KW_) {                                                       \
    if (D == 128) hipLaunchKernelGGL((attn_mfma_kernel<128, RW_, KW_>), grid, mblock, 0, s, a); \
    else hipLaunchKernelGGL((attn_mfma_kernel<64, RW_, KW_>), grid, mblock, 0, s, a);          \
  }
    ST_LAUNCH_MFMA(4, 2)
    ST_LAUNCH_MFMA(4, 1)
    ST_LAUNCH_MFMA(2, 2)
    ST_LAUNCH_MFMA(2, 4)
    ST_LAUNCH_MFMA(1, 4)
#undef ST_LAUNCH_MFMA
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

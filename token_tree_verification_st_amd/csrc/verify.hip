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
// (unchanged when that sum is 0).  A first kernel reduces every logit row to
// its softmax statistics (max, sum of exponentials), one workgroup per row;
// with those, testing the first child of any node needs two logits only.  A
// second kernel walks each request's tree with one workgroup: the children's
// tests read precomputed values, and only the nodes where the walk rejects a
// child or stops have their two rows read again, for the residual masses and
// the inverse-CDF draw of the replacement token.
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
//
// Wavefront reductions and scans in VALU: DPP moves within 16-lane rows, and
// gfx950's permlane swaps between rows.  Every exchange is an involution and
// both partners add in the same operand order, so all lanes of a reduction
// end with the same bits.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {  // 0 where the source lane is absent
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// (own, partner) for the partners l ^ 16 and l ^ 32, in either order
template <bool X32>
__device__ __forceinline__ void swap_rows(double v, double& x0, double& x1) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto l = X32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                     : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = X32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                     : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  x0 = __longlong_as_double((long long)(((uint64_t)h[0] << 32) | l[0]));
  x1 = __longlong_as_double((long long)(((uint64_t)h[1] << 32) | l[1]));
}
template <bool X32>
__device__ __forceinline__ void swap_rows(float v, float& x0, float& x1) {
  const uint32_t u = __float_as_uint(v);
  const auto r = X32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x0 = __uint_as_float(r[0]);
  x1 = __uint_as_float(r[1]);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  double x0, x1;
  swap_rows<false>(v, x0, x1);
  v = x0 + x1;
  swap_rows<true>(v, x0, x1);
  return x0 + x1;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  float x0, x1;
  swap_rows<false>(v, x0, x1);
  v = fmaxf(x0, x1);
  swap_rows<true>(v, x0, x1);
  return fmaxf(x0, x1);
}

// Inclusive scan over the lanes of a wavefront.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<0x111>(v);       // row_shr:1
  v += dpp_f64<0x112>(v);       // row_shr:2
  v += dpp_f64<0x114>(v);       // row_shr:4
  v += dpp_f64<0x118>(v);       // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// The value of lane l - 1 (0 in lane 0).
__device__ __forceinline__ double wave_shr1(double v) { return dpp_f64<0x138>(v); }

// Workgroup-wide reductions: wavefront results through LDS, combined in
// wavefront order by every thread.
template <int BLOCK>
__device__ inline double block_sum(double v, double* lds) {
  constexpr int NW = BLOCK / ST_WAVE;
  v = wave_sum(v);
  const int w = threadIdx.x / ST_WAVE, lane = threadIdx.x % ST_WAVE;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  double r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += lds[i];
  return r;
}
template <int BLOCK>
__device__ inline float block_max(float v, float* lds) {
  constexpr int NW = BLOCK / ST_WAVE;
  v = wave_max(v);
  const int w = threadIdx.x / ST_WAVE, lane = threadIdx.x % ST_WAVE;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, lds[i]);
  return r;
}

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

// Softmax statistics of one logit row at temperature T: M = max logit and
// Z = sum over v of exp2((l_v - M) * log2e / T), each term rounded to fp32,
// groups of four consecutive terms summed in fp32 and the groups in fp64.
// Rows 2t and 2t+1 are node t's target and draft rows.
struct RowStat {
  float M;
  int pad;
  double Z;
};

// What the walk needs from a node: its first accepted child (local index, -1
// if none), the near ties among its tests and, when no child is accepted, the
// replacement token drawn there and whether that draw was a near tie.
struct NodeVerdict {
  int accepted, ties, token, token_tie;
};

struct StochArgs {
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* tokens;
  const float* tl;
  const float* dl;
  RowStat* stat;
  NodeVerdict* verdict;
  int B, T, V, max_nodes, max_depth;
  float temperature;
  uint64_t seed, offset;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  int32_t* near_ties;
  int32_t* status;
};

constexpr int kStochBlock = 1024;
constexpr int kStochWaves = kStochBlock / ST_WAVE;
constexpr int kStochMaxV = 32768;
constexpr int kStochNpt = kStochMaxV / kStochBlock;  // row entries per thread

// A row is spread over the workgroup wavefront by wavefront: wavefront w holds
// the kStochNpt*64 consecutive logits from w*kStochNpt*64, as tiles of
// 64*EPT.  With VEC (V % 4 == 0, 16-byte aligned rows) entries 4k..4k+3 of a
// lane are four consecutive logits of tile k (one coalesced 16-byte load per
// lane), else entry k is one logit of tile k.
template <bool VEC>
__device__ inline int row_index(int e, int tid) {
  const int w = tid / ST_WAVE, lane = tid % ST_WAVE;
  return w * (kStochNpt * ST_WAVE) +
         (VEC ? (e >> 2) * (4 * ST_WAVE) + lane * 4 + (e & 3) : e * ST_WAVE + lane);
}

// Loads a thread's row entries.  Every load is issued, unconditionally, before
// any is used, so the wait for one buffer does not also wait for loads issued
// after it: entries past the row end (all entries when `on` is false) read the
// row's first logit instead, which leaves the row maximum unchanged; sums mask
// them out with row_index(e) < V, applied to computed terms only.
template <bool VEC>
__device__ inline void load_row(const float* __restrict__ src, int V, bool on,
                                float (&x)[kStochNpt]) {
  const int tid = threadIdx.x;
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < kStochNpt / 4; ++k) {
      const int v = row_index<true>(4 * k, tid);
      const f32x4 q =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (on && v < V ? v : 0)));
      x[4 * k] = q.x;
      x[4 * k + 1] = q.y;
      x[4 * k + 2] = q.z;
      x[4 * k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kStochNpt; ++e) {
      const int v = row_index<false>(e, tid);
      x[e] = __builtin_nontemporal_load(src + (on && v < V ? v : 0));
    }
  }
}

// 2^x by the hardware instruction: results below 2^-126 flush to 0, which no
// sum here can see (every sum has a term equal to 1) and which only reaches
// the acceptance tests at sizes far inside their near-tie band.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2((l - M) * s), times `scale`, for the entries inside the row, else 0.
template <bool VEC>
__device__ inline void row_probs(float (&x)[kStochNpt], int V, float M, float s, float scale) {
#pragma unroll
  for (int e = 0; e < kStochNpt; ++e) {
    const float p = exp2_fast((x[e] - M) * s) * scale;
    x[e] = row_index<VEC>(e, threadIdx.x) < V ? p : 0.f;
  }
}

// The residual weight max(0, p_v - c q_v) of one row entry from its
// probabilities P = p_v and Q = q_v, both rounded to fp32: a fused
// multiply-add and a max in fp32.
__device__ __forceinline__ float resid(float P, float Q, float c) {
  return fmaxf(0.f, fmaf(-c, Q, P));
}
// Sum of the residual weights of entries [k*EPT, k*EPT+EPT) of a thread: fp32
// within the (at most 4) entries, fp64 from there on.
template <int EPT>
__device__ __forceinline__ double resid_group(const float (&P)[kStochNpt],
                                              const float (&Q)[kStochNpt], float c, int k) {
  float s = resid(P[k * EPT], Q[k * EPT], c);
#pragma unroll
  for (int j = 1; j < EPT; ++j) s += resid(P[k * EPT + j], Q[k * EPT + j], c);
  return (double)s;
}
// A thread's share of sum_v max(0, p_v - c q_v).
template <bool VEC>
__device__ __forceinline__ double resid_sum(const float (&P)[kStochNpt],
                                            const float (&Q)[kStochNpt], float c) {
  constexpr int EPT = VEC ? 4 : 1;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kStochNpt / EPT; ++k) s += resid_group<EPT>(P, Q, c, k);
  return s;
}

struct DrawLds {
  double wsum[kStochWaves];
  int pick, tie;
};

// Inverse-CDF draw from the residual w_v = max(0, p_v - c q_v) in ascending
// vocab order: the smallest v whose running sum exceeds u * sum(w).  Every
// wavefront reduces its slice of the row; the prefix over the slices (summed
// in wavefront order by every thread) names the slice that crosses the
// threshold, and that wavefront alone locates the tile, then the entry.  The
// threshold test at every level compares running sums that begin where the
// previous level's left off.  Returns sum(w); pick and tie are set when it is
// positive.
template <bool VEC>
__device__ inline double draw_residual(const float (&P)[kStochNpt], const float (&Q)[kStochNpt],
                                       float c, double u, DrawLds& s, int& pick, int& tie) {
  constexpr int EPT = VEC ? 4 : 1, NT = kStochNpt / EPT;
  const int tid = threadIdx.x, lane = tid % ST_WAVE;
  const int w = __builtin_amdgcn_readfirstlane(tid / ST_WAVE);
  const double mine = wave_sum(resid_sum<VEC>(P, Q, c));
  if (lane == 0) s.wsum[w] = mine;
  if (tid == 0) {
    s.pick = 0;
    s.tie = 0;
  }
  __syncthreads();
  double total = 0.0;
  for (int i = 0; i < kStochWaves; ++i) total += s.wsum[i];
  const double thr = u * total;
  // the slice: running sums over the wavefronts' slices, in the same order
  double base = 0.0, run0 = 0.0;
  int ws = -1;
  for (int i = 0; i < kStochWaves; ++i) {
    const double next = run0 + s.wsum[i];
    if (ws < 0 && next > thr) {
      ws = i;
      base = run0;
    }
    run0 = next;
  }
  if (ws < 0) {  // total == 0
    pick = 0;
    tie = 0;
    return total;
  }
  if (w == ws) {
    // recomputed from P and Q rather than kept from above (registers)
    float cw = c;
    asm volatile("" : "+v"(cw));
    // the tile: running sums over the wavefront's tiles from `base`
    double run = base, tbase = base;
    int kt = -1, klast = -1;
    double lbase = base;
    for (int k = 0; k < NT; ++k) {
      double part = 0.0;
#pragma unroll
      for (int kk = 0; kk < NT; ++kk)
        if (kk == k) part = resid_group<EPT>(P, Q, cw, kk);
      const double tsum = wave_sum(part);
      const double next = run + tsum;
      if (kt < 0 && next > thr) {
        kt = k;
        tbase = run;
      }
      if (tsum > 0.0) {
        klast = k;
        lbase = run;
      }
      run = next;
    }
    if (kt < 0) {  // rounding: no tile crosses; take the last positive one
      kt = klast;
      tbase = lbase;
    }
    // the entry: a scan over the lanes of tile kt
    float wt[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) wt[j] = 0.f;
#pragma unroll
    for (int k = 0; k < NT; ++k)
      if (k == kt) {
#pragma unroll
        for (int j = 0; j < EPT; ++j) wt[j] = resid(P[k * EPT + j], Q[k * EPT + j], cw);
      }
    double sub = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) sub += (double)wt[j];
    double run2 = tbase + wave_shr1(wave_incl_scan(sub));
    double lo_edge = 0.0, hi_edge = 0.0, last_lo = 0.0, last_hi = 0.0;
    int found = -1, last = -1;
    // within a lane the weights are added one by one in fp64
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const double x = (double)wt[j];
      const double before = run2;
      run2 += x;
      if (x > 0.0) {
        last = j;
        last_lo = before;
        last_hi = run2;
        if (found < 0 && run2 > thr) {
          found = j;
          lo_edge = before;
          hi_edge = run2;
        }
      }
    }
    const uint64_t fm = __ballot(found >= 0);
    // no entry-level crossing (rounding): the last positive entry of the tile
    const uint64_t lm = __ballot(last >= 0);
    const int who = fm ? __ffsll((unsigned long long)fm) - 1
                       : lm ? 63 - __clzll((long long)lm) : -1;
    if (lane == who) {
      const int j = fm ? found : last;
      const double ce_lo = fm ? lo_edge : last_lo, ce_hi = fm ? hi_edge : last_hi;
      const int v = row_index<VEC>(kt * EPT + j, tid);
      s.pick = v;
      s.tie = fabs(ce_hi - thr) < kTieEps * total || (v > 0 && fabs(ce_lo - thr) < kTieEps * total);
    }
  }
  __syncthreads();
  pick = s.pick;
  tie = s.tie;
  return total;
}

// Row statistics, persistent: workgroup g reduces rows g, g + G, g + 2G, ...
// (G = gridDim.x), with the next row's loads in flight while the current row
// is reduced (two register buffers, used alternately).
template <bool VEC>
__device__ inline void finish_row(const StochArgs& g, const float (&x)[kStochNpt], int r,
                                  float* red_f, double* red_d) {
  float m = -INFINITY;
  bool finite = true;
#pragma unroll
  for (int e = 0; e < kStochNpt; ++e) {
    finite &= (bool)isfinite(x[e]);
    m = fmaxf(m, x[e]);
  }
  if (!finite) st::set_status(g.status, ST_STATUS_NONFINITE);
  m = block_max<kStochBlock>(m, red_f);
  const float sc = kLog2e / g.temperature;
  // fp32 within a group of (at most 4) consecutive entries, fp64 from there on
  constexpr int EPT = VEC ? 4 : 1;
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < kStochNpt / EPT; ++k) {
    float zk = exp2_fast((x[k * EPT] - m) * sc);
#pragma unroll
    for (int j = 1; j < EPT; ++j) zk += exp2_fast((x[k * EPT + j] - m) * sc);
    z += (double)(row_index<VEC>(k * EPT, threadIdx.x) < g.V ? zk : 0.f);
  }
  z = block_sum<kStochBlock>(z, red_d);
  if (threadIdx.x == 0) {
    RowStat rs;
    rs.M = m;
    rs.pad = 0;
    rs.Z = z;
    g.stat[r] = rs;
  }
}

template <bool VEC>
__global__ void __launch_bounds__(kStochBlock)
row_stat_kernel(StochArgs g) {
  __shared__ float red_f[kStochWaves];
  __shared__ double red_d[kStochWaves];
  const int R = 2 * g.T, G = gridDim.x;
  // Past the last row a buffer is refilled from row 0 (read by every
  // workgroup, so from cache) and never used: the loads stay unconditional.
  auto row = [&](int r) { return r < R ? ((r & 1) ? g.dl : g.tl) + (size_t)(r >> 1) * g.V : g.tl; };
  float xa[kStochNpt], xb[kStochNpt];
  int r = blockIdx.x;
  load_row<VEC>(row(r), g.V, true, xa);
  while (true) {
    load_row<VEC>(row(r + G), g.V, true, xb);
    finish_row<VEC>(g, xa, r, red_f, red_d);
    r += G;
    if (r >= R) break;
    load_row<VEC>(row(r + G), g.V, true, xa);
    finish_row<VEC>(g, xb, r, red_f, red_d);
    r += G;
    if (r >= R) break;
  }
}

struct NodeLds {
  int place[4];  // b, lo, n, ok
  uint64_t kid_mask[ST_MAX_NODES / 64];
  int kids[ST_MAX_NODES];  // children, ascending
  double px[ST_MAX_NODES], qx[ST_MAX_NODES], ua[ST_MAX_NODES];  // per child
  int ok[ST_MAX_NODES];                                           // token in range
  double red[kStochWaves];
  double u_draw;
  DrawLds draw;
};

// One workgroup per node u decides what the walk would do on reaching u: test
// u's children in ascending order, child c with token x accepted iff
// u_acc(c) q_u[x] < r[x] with r starting at p_u, and draw the replacement
// token from r when no child is accepted.  The first test needs only the row
// statistics; u's rows are read (into registers, as fp32 probabilities) once
// a child is rejected, for the residual masses of the later tests and the
// draw.  A leaf reads its target row only, to draw from p_u.
template <bool VEC>
__global__ void __launch_bounds__(kStochBlock)
stoch_node_kernel(StochArgs g) {
  __shared__ NodeLds s;
  const int tid = threadIdx.x, t = blockIdx.x;
  if (tid < ST_WAVE) {  // node t's request: the number of request starts at or before t, less one
    int cnt = 0;
    for (int b0 = 0; b0 < g.B; b0 += ST_WAVE) {
      const int b = b0 + tid;
      cnt += __popcll(__ballot(b < g.B && g.node_off[b] <= t));
    }
    const int b = cnt > 0 ? cnt - 1 : 0;
    const int lo = g.node_off[b], hi = g.node_off[b + 1];
    if (tid == 0) {
      s.place[0] = b;
      s.place[1] = lo;
      s.place[2] = hi - lo;
      s.place[3] = (lo >= 0) & (hi <= g.T) & (hi - lo >= 1) & (hi - lo <= g.max_nodes) &
                   (t >= lo) & (t < hi);
    }
  }
  if (tid < ST_MAX_NODES / 64) s.kid_mask[tid] = 0;
  __syncthreads();
  if (!s.place[3]) return;  // the walk flags the request
  const int b = s.place[0], lo = s.place[1], n = s.place[2], i = t - lo;
  if (tid < n && tid > i && g.parent[lo + tid] == i)
    atomicOr((unsigned long long*)&s.kid_mask[tid >> 6], 1ull << (tid & 63));
  if (tid == kStochBlock - 1) {
    double ua, us;
    node_uniforms(g.seed, g.offset, b, i, ua, us);
    s.u_draw = us;
  }
  const RowStat rt = g.stat[2 * t];
  const double a = 1.0 / rt.Z;
  const float sc = kLog2e / g.temperature, af = (float)a;
  __syncthreads();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < ST_MAX_NODES / 64; ++w) nk += __popcll(s.kid_mask[w]);

  if (nk == 0) {  // a leaf: the walk stops here with r = p_u
    float P[kStochNpt];
    load_row<VEC>(g.tl + (size_t)t * g.V, g.V, true, P);
    row_probs<VEC>(P, g.V, rt.M, sc, af);
    int token, tie;
    draw_residual<VEC>(P, P, 0.f, s.u_draw, s.draw, token, tie);
    if (tid == 0) g.verdict[t] = NodeVerdict{-1, 0, token, tie};
    return;
  }

  const RowStat rd = g.stat[2 * t + 1];
  const double bq = 1.0 / rd.Z;
  if (tid < n && ((s.kid_mask[tid >> 6] >> (tid & 63)) & 1)) {
    int rank = __popcll(s.kid_mask[tid >> 6] & ((1ull << (tid & 63)) - 1));
    for (int w = 0; w < (tid >> 6); ++w) rank += __popcll(s.kid_mask[w]);
    s.kids[rank] = tid;
    const int x = g.tokens[lo + tid];
    const bool ok = x >= 0 && x < g.V;
    s.ok[rank] = ok;
    if (ok) {
      const size_t at = (size_t)t * g.V + x;
      s.px[rank] = (double)exp2_fast((g.tl[at] - rt.M) * sc) * a;
      s.qx[rank] = (double)exp2_fast((g.dl[at] - rd.M) * sc) * bq;
      double ua, us;
      node_uniforms(g.seed, g.offset, b, tid, ua, us);
      s.ua[rank] = ua;
    }
  }
  __syncthreads();

  int ties = 0, accepted = -1;
  double c = 0.0, D = 1.0;
  // child k's test against r = max(0, p - c q) / D
  auto test = [&](int k) {
    if (!s.ok[k]) return false;
    const double qv = s.qx[k];
    const double r = fmax(0.0, s.px[k] - c * qv) / D;
    const double lhs = s.ua[k] * qv;
    ties += fabs(r - lhs) < kTieEps;
    return lhs < r;
  };
  int token = -1, tie = 0;
  if (test(0)) {
    accepted = s.kids[0];
  } else {
    float P[kStochNpt], Q[kStochNpt];
    load_row<VEC>(g.tl + (size_t)t * g.V, g.V, true, P);
    load_row<VEC>(g.dl + (size_t)t * g.V, g.V, true, Q);
    row_probs<VEC>(P, g.V, rt.M, sc, af);
    row_probs<VEC>(Q, g.V, rd.M, sc, (float)bq);
    // after each rejection r <- max(0, r - q) renormalised, i.e. c <- c + D
    for (int k = 1; k < nk && accepted < 0; ++k) {
      const double cn = c + D;
      const double Dn = block_sum<kStochBlock>(resid_sum<VEC>(P, Q, (float)cn), s.red);
      if (Dn > 0.0) {
        c = cn;
        D = Dn;
      }
      if (test(k)) accepted = s.kids[k];
    }
    if (accepted < 0) {  // every child rejected: draw from the final residual
      const double total = draw_residual<VEC>(P, Q, (float)(c + D), s.u_draw, s.draw, token, tie);
      if (!(total > 0.0)) {  // the last rejection left no mass: r unchanged
        __syncthreads();
        draw_residual<VEC>(P, Q, (float)c, s.u_draw, s.draw, token, tie);
      }
    }
  }
  if (tid == 0) g.verdict[t] = NodeVerdict{accepted, ties, token, tie};
}

// One wavefront per request follows the verdicts from the root: step to the
// accepted child while there is one (at most max_depth steps), then emit the
// token drawn at the stop node.
__global__ void __launch_bounds__(ST_WAVE)
stoch_walk_kernel(StochArgs g) {
  __shared__ int path[kMaxPath + 1];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int lo = g.node_off[b], hi = g.node_off[b + 1], n = hi - lo;
  if (lo < 0 || hi > g.T || n < 1 || n > g.max_nodes) {
    if (lane == 0) st::set_status(g.status, ST_STATUS_BAD_PARENT);
    return;
  }
  const int bits = check_request(g.parent, g.tokens, lo, n, g.V);
  if (bits) st::set_status(g.status, bits);
  int L = 0, ties = 0, last = -1;
  bool over = false;
  if (lane == 0) {
    int u = 0;
    path[0] = 0;
    while (true) {
      const NodeVerdict v = g.verdict[lo + u];
      ties += v.ties;
      if (v.accepted <= u || v.accepted >= n) {  // -1: stop here
        last = v.token;
        ties += v.token_tie;
        break;
      }
      if (L == g.max_depth) {
        over = true;
        break;
      }
      path[++L] = v.accepted;
      u = v.accepted;
    }
    if (over) st::set_status(g.status, ST_STATUS_PATH_OVERFLOW);
    if (g.near_ties) g.near_ties[b] = ties;
  }
  L = __shfl(L, 0, ST_WAVE);
  last = __shfl(last, 0, ST_WAVE);
  st::wave_lds_sync();
  write_path_outputs(b, L, g.max_depth, path, g.tokens, lo, last, g.accept_len, g.accept_nodes,
                     g.out_tokens);
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
  return st::align_up((size_t)tree->total_nodes * (2 * sizeof(RowStat) + sizeof(NodeVerdict)),
                      256);
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
  if (V > kStochMaxV || tree->max_depth + 1 > kMaxPath) return ST_E_UNSUPPORTED;
  if (ws_bytes < st_verify_stochastic_workspace(tree, V)) return ST_E_WORKSPACE;
  const int T = tree->total_nodes;
  RowStat* stat = (RowStat*)workspace;
  const StochArgs g{tree->node_off, tree->parent, tokens, target_logits, draft_logits, stat,
                    (NodeVerdict*)(stat + 2 * T), tree->B, T, V, tree->max_nodes,
                    tree->max_depth, temperature, seed, offset, accept_len, accept_nodes,
                    out_tokens, near_ties, status};
  hipStream_t s = (hipStream_t)stream;
  // one persistent statistics workgroup per compute unit
  const int stat_wg = 2 * T < st::device_cus() ? 2 * T : st::device_cus();
  if ((V & 3) == 0) {
    hipLaunchKernelGGL(row_stat_kernel<true>, dim3(stat_wg), dim3(kStochBlock), 0, s, g);
    hipLaunchKernelGGL(stoch_node_kernel<true>, dim3(T), dim3(kStochBlock), 0, s, g);
  } else {
    hipLaunchKernelGGL(row_stat_kernel<false>, dim3(stat_wg), dim3(kStochBlock), 0, s, g);
    hipLaunchKernelGGL(stoch_node_kernel<false>, dim3(T), dim3(kStochBlock), 0, s, g);
  }
  if ((rc = st::check_launch())) return rc;
  hipLaunchKernelGGL(stoch_walk_kernel, dim3(tree->B), dim3(ST_WAVE), 0, s, g);
  return st::check_launch();
}

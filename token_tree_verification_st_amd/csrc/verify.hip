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
// c_{k+1} = c_k + D_k and D_{k+1} = sum_v max(0, p_u - c_{k+1} q_u).  One
// workgroup per node reads the node's target and draft rows once into
// registers, reduces them to their softmax statistics and decides the node
// as the walk would on reaching it: its children are tested in order (after
// each rejection one residual-mass reduction), and where none is accepted
// the replacement token is drawn from the final residual by inverse CDF.  A
// rejection that leaves a residual mass of at most 1e-6 of the current one
// (D_{k+1} <= 1e-6 D_k: the fp32 rounding residue of r <= q) keeps r as it
// was.  The node's verdict (first accepted child, near ties, drawn token) is
// 16 bytes; one wavefront per request then follows the verdicts from the
// root.
#include "step_internal.h"

#include <float.h>
#include <type_traits>
#include <limits.h>

// Every comparison that decides a token must see the same value wherever it is
// recomputed, so products and sums are evaluated exactly as written.
#pragma clang fp contract(off)

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kTieEps = 1e-6;
// A rejection whose residual mass, as a fraction of the current residual's
// (D_{k+1} / D_k, the mass of max(0, r - q) for the normalised r), is at most
// this leaves r as it was: where r <= q everywhere the exact mass is 0, and
// the fp32 terms max(0, P - c Q) leave up to about 1e-7 of rounding residue,
// which must not be renormalised into a distribution (a nucleus cut makes
// such agreement common: two one-token nuclei on the same token).
constexpr double kMassEps = 1e-6;

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

// Workgroup-wide reductions: wavefront results through LDS (2 * NW slots), then
// combined pairwise in a fixed order by every thread.  Consecutive calls on
// one slot array must alternate `set` (0, 1): a wavefront may then write its
// next result while others still read the previous set, and one barrier per
// call suffices.
template <int NW, typename T, typename Op>
__device__ __forceinline__ T tree_fold(const T* x, Op op) {
  T v[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) v[i] = x[i];
#pragma unroll
  for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
    for (int i = 0; i < h; ++i) v[i] = op(v[2 * i], v[2 * i + 1]);
  return v[0];
}
template <int BLOCK>
__device__ inline double block_sum(double v, double* lds, int set) {
  constexpr int NW = BLOCK / ST_WAVE;
  v = wave_sum(v);
  if (threadIdx.x % ST_WAVE == 0) lds[set * NW + threadIdx.x / ST_WAVE] = v;
  __syncthreads();
  return tree_fold<NW>(lds + set * NW, [](double a, double b) { return a + b; });
}
// A double moved to scalar registers (its value must be wave-uniform).
__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float uniform_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

// Two reductions sharing one barrier: (x, y) -> (max x, max y) and sums.
// They fill both slot sets of `lds`, so a barrier must separate them from
// the previous reduction on that array and from the next one.
template <int BLOCK>
__device__ inline void block_max2(float& x, float& y, float* lds) {
  constexpr int NW = BLOCK / ST_WAVE;
  x = wave_max(x);
  y = wave_max(y);
  if (threadIdx.x % ST_WAVE == 0) {
    lds[threadIdx.x / ST_WAVE] = x;
    lds[NW + threadIdx.x / ST_WAVE] = y;
  }
  __syncthreads();
  // block-uniform results, kept in scalar registers
  x = uniform_f32(tree_fold<NW>(lds, [](float a, float b) { return fmaxf(a, b); }));
  y = uniform_f32(tree_fold<NW>(lds + NW, [](float a, float b) { return fmaxf(a, b); }));
}
template <int BLOCK>
__device__ inline void block_sum2(double& x, double& y, double* lds) {
  constexpr int NW = BLOCK / ST_WAVE;
  x = wave_sum(x);
  y = wave_sum(y);
  if (threadIdx.x % ST_WAVE == 0) {
    lds[threadIdx.x / ST_WAVE] = x;
    lds[NW + threadIdx.x / ST_WAVE] = y;
  }
  __syncthreads();
  x = uniform_f64(tree_fold<NW>(lds, [](double a, double b) { return a + b; }));
  y = uniform_f64(tree_fold<NW>(lds + NW, [](double a, double b) { return a + b; }));
}

// Three sums over one of two slot sets of `lds` (6 * BLOCK / 64 doubles):
// consecutive calls that alternate `set` need no barrier between them.  Each
// lane of a 16-lane row reads one wavefront's partial and a butterfly adds
// them (a + b and b + a round alike, so every lane gets the same bits); the
// totals end in scalar registers.
template <int BLOCK>
__device__ inline void block_sum3_set(double& x, double& y, double& z, double* lds, int set) {
  constexpr int NW = BLOCK / ST_WAVE;
  static_assert(NW == 16, "one partial per lane of a 16-lane row");
  double* l = lds + set * 3 * NW;
  x = wave_sum(x);
  y = wave_sum(y);
  z = wave_sum(z);
  if (threadIdx.x % ST_WAVE == 0) {
    l[threadIdx.x / ST_WAVE] = x;
    l[NW + threadIdx.x / ST_WAVE] = y;
    l[2 * NW + threadIdx.x / ST_WAVE] = z;
  }
  __syncthreads();
  const int r = threadIdx.x & 15;
  double a = l[r], b = l[NW + r], c = l[2 * NW + r];
#pragma unroll
  for (int k = 1; k < 16; k <<= 1) {
    a += __shfl_xor(a, k, 16);
    b += __shfl_xor(b, k, 16);
    c += __shfl_xor(c, k, 16);
  }
  x = uniform_f64(a);
  y = uniform_f64(b);
  z = uniform_f64(c);
}

using st::argmax_merge;
using st::ArgmaxPart;
using st::kMaxPath;

// ---------------------------------------------------------------- greedy

using st::kArgmaxBlock;
using st::kArgmaxSlice;

// Workgroup u reduces unit u (row u / nslices, slice u % nslices: 8192
// logits) to its maximum and lowest index.  Every load is issued
// unconditionally, before any is used (an entry past the row end reads the
// row's first logit; the reduction skips it): with no branch around a load the
// wait for each one is exact.  (Workgroups that reduce several units in turn,
// the next unit's loads in flight during each reduction, measured slower on a
// 61 MB batch than one unit each: the dispatcher's fresh workgroups overlap
// better than one workgroup's prefetch.)
template <bool VEC>
__device__ inline void argmax_unit_load(const float* logits, int V, int nslices, int u,
                                        st::ArgmaxRegs& r) {
  const float* row = logits + (size_t)(u / nslices) * V;
  const int base = (u % nslices) * kArgmaxSlice, tid = threadIdx.x;
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < st::kArgmaxPerThread / 4; ++k) {
      const int v = base + 4 * (tid + k * kArgmaxBlock);
      r.x[k] = __builtin_nontemporal_load((const st::am_f32x4*)(row + (v < V ? v : 0)));
    }
  } else {
#pragma unroll
    for (int k = 0; k < st::kArgmaxPerThread; ++k) {
      const int v = base + tid + k * kArgmaxBlock;
      r.x[k / 4][k % 4] = row[v < V ? v : 0];
    }
  }
}
__global__ void __launch_bounds__(kArgmaxBlock)
row_argmax_kernel(const float* __restrict__ logits, int V, int nslices,
                  ArgmaxPart* __restrict__ part, int32_t* status) {
  __shared__ int scratch[2 * (kArgmaxBlock / ST_WAVE) + 1];
  const int u = blockIdx.x;
  st::ArgmaxRegs r;
  if ((V & 3) == 0) {
    argmax_unit_load<true>(logits, V, nslices, u, r);
    st::argmax_slice_finish<true>(r, V, u / nslices, u % nslices, nslices, part, status, scratch);
  } else {
    argmax_unit_load<false>(logits, V, nslices, u, r);
    st::argmax_slice_finish<false>(r, V, u / nslices, u % nslices, nslices, part, status,
                                   scratch);
  }
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

using st::NodeVerdict;

// Inputs of the node kernel.
struct StochArgs {
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* tokens;
  const float* tl;
  const float* dl;
  NodeVerdict* verdict;
  int B, T, V, max_nodes;
  float temperature;
  uint64_t seed, offset;
  int32_t* status;
  int draft_probs;  // dl holds probabilities (used as given) rather than logits
  float top_p;      // < 1: both rows restricted to their nucleus
  int uniform;      // T == B * max_nodes: every request has max_nodes nodes
};

constexpr int kStochMaxV = 32768;
constexpr int kNodeBlock = 1024;  // 32 entries of each row per thread
constexpr int kMaxWaves = kNodeBlock / ST_WAVE;

// A row is spread over a workgroup of kStochMaxV / NPT threads, NPT entries
// per thread, wavefront by wavefront: wavefront w holds the NPT*64
// consecutive logits from w*NPT*64, as tiles of 64*EPT.  With VEC (V % 4 == 0,
// 16-byte aligned rows) entries 4k..4k+3 of a lane are four consecutive
// logits of tile k (one coalesced 16-byte load per lane), else entry k is one
// logit of tile k.
template <bool VEC, int NPT>
__device__ inline int row_index(int e, int tid) {
  const int w = tid / ST_WAVE, lane = tid % ST_WAVE;
  return w * (NPT * ST_WAVE) +
         (VEC ? (e >> 2) * (4 * ST_WAVE) + lane * 4 + (e & 3) : e * ST_WAVE + lane);
}

// How many of this thread's entry groups (EPT entries each) lie inside a row
// of V logits: in the layout above they are a prefix of the thread's groups.
template <bool VEC, int NPT>
__device__ inline int groups_inside(int V, int tid) {
  constexpr int EPT = VEC ? 4 : 1, STRIDE = EPT * ST_WAVE;
  const int first = row_index<VEC, NPT>(0, tid);
  return V > first ? min(NPT / EPT, (V - first + STRIDE - 1) / STRIDE) : 0;
}

// Loads a thread's row entries.  Every load is issued, unconditionally, before
// any is used, so the wait for one buffer does not also wait for loads issued
// after it: entries past the row end (all entries when `on` is false) read the
// row's first logit instead, which leaves the row maximum unchanged; sums mask
// them out with row_index(e) < V, applied to computed terms only.
template <bool VEC, int NPT>
__device__ inline void load_row(const float* __restrict__ src, int V, bool on, float (&x)[NPT]) {
  const int tid = threadIdx.x;
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < NPT / 4; ++k) {
      const int v = row_index<true, NPT>(4 * k, tid);
      const f32x4 q =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (on && v < V ? v : 0)));
      x[4 * k] = q.x;
      x[4 * k + 1] = q.y;
      x[4 * k + 2] = q.z;
      x[4 * k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int v = row_index<false, NPT>(e, tid);
      x[e] = __builtin_nontemporal_load(src + (on && v < V ? v : 0));
    }
  }
}

// 2^x by the hardware instruction: results below 2^-126 flush to 0, which no
// sum here can see (every sum has a term equal to 1) and which only reaches
// the acceptance tests at sizes far inside their near-tie band.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The residual weight of one row entry, up to a common factor, from the
// rounded exponentials P = Z_t p_v and Q = Z_d q_v:
//   max(0, p_v - c q_v) = max(0, P - c' Q) / Z_t  with  c' = c Z_t / Z_d,
// a fused multiply-add and a max in fp32.
__device__ __forceinline__ float resid(float P, float Q, float c) {
  return fmaxf(0.f, fmaf(-c, Q, P));
}
// Sum of the residual weights of entries [k*EPT, k*EPT+EPT) of a thread: fp32
// within the (at most 4) entries, fp64 from there on.
template <int EPT, int NPT>
__device__ __forceinline__ double resid_group(const float (&P)[NPT], const float (&Q)[NPT],
                                              float c, int k) {
  float s = resid(P[k * EPT], Q[k * EPT], c);
#pragma unroll
  for (int j = 1; j < EPT; ++j) s += resid(P[k * EPT + j], Q[k * EPT + j], c);
  return (double)s;
}
// A thread's share of sum_v max(0, p_v - c q_v).
template <bool VEC, int NPT>
__device__ __forceinline__ double resid_sum(const float (&P)[NPT], const float (&Q)[NPT],
                                            float c) {
  constexpr int EPT = VEC ? 4 : 1;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < NPT / EPT; ++k) s += resid_group<EPT>(P, Q, c, k);
  return s;
}

// A thread's share of the mass at or above `cut` (fp32 within a group, fp64
// from there on, as the row totals), and how many entries that is.
template <bool VEC, int NPT>
__device__ __forceinline__ double kept_sum(const float (&X)[NPT], float cut, int& n) {
  constexpr int EPT = VEC ? 4 : 1;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < NPT / EPT; ++k) {
    float g = 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool in = X[k * EPT + j] >= cut;
      g += in ? X[k * EPT + j] : 0.f;
      n += in;
    }
    s += (double)g;
  }
  return s;
}

// The search's last phase: one wavefront, at most kCutLane candidates a lane.
constexpr int kCutLane = 8;
constexpr int kCutCand = kCutLane * ST_WAVE;  // per row
// The search's first phase: a histogram of each row's weights over the top
// 11 bits of their bit patterns (1/8 of a binade a bin), bin masses in
// integer units of 2^-36 of the row's total (order-independent exact sums:
// the weights scaled by the total's reciprocal in fp32 sum to at most
// 1 + 2^-23, each truncated by less than 2^-36, so a row's sums are within
// 6e-7 of the total's fractions, inside the 1e-6 tie band).  A bin's count
// rides in the same 64-bit word above bit 40 (one atomic an entry): masses
// stay below 2^37, counts below 2^24.
constexpr int kBinShift = 21;
constexpr int kBins = 1 << (32 - kBinShift);
constexpr double kFix = 68719476736.0;  // 2^36
constexpr int kCountShift = 40;
constexpr unsigned long long kCountOne = 1ull << kCountShift;
constexpr unsigned long long kMassMask = kCountOne - 1ull;
// floor(x * 2^36) for 0 <= x < 2 in fp32 arithmetic: x * 16 splits exactly
// into its integer part and its fraction (both exact in fp32), the fraction
// times 2^32 is exact too, and both convert without rounding.
__device__ __forceinline__ unsigned long long fix36(float x) {
  const float x16 = x * 16.f;
  const uint32_t hi = (uint32_t)x16;
  const uint32_t lo = (uint32_t)((x16 - (float)hi) * 4294967296.f);
  return ((unsigned long long)hi << 32) | lo;
}
struct BinCut {
  uint32_t lo, hi;
  double m_lo, m_hi;
  int n_lo, n_hi, found;
};
struct CutLds {
  double red[6 * kMaxWaves];  // two slot sets of three sums
  float cand[2][kCutCand];    // the entries still between the bounds
  int wtot[kMaxWaves];
  uint32_t cut[2];
  double kept[2];
  unsigned long long hm[2][kBins];  // bin masses and counts (kCountShift)
  double wm[2][kMaxWaves], wn[2][kMaxWaves];
  BinCut hb[2];
};

// One row's bisection state over fp32 bit patterns: `want` is top_p of the
// row's total; the mass at or above lo reaches it, the mass at or above hi
// does not.  Masses and entry counts at both bounds are kept (the count at
// lo is unknown, so large, until lo first moves).
struct CutRow {
  uint32_t lo, hi;
  double want, m_lo, m_hi;
  int n_lo, n_hi;
  __device__ bool open() const { return hi - lo > 1u; }
  __device__ uint32_t mid() const { return lo + (hi - lo) / 2u; }
  __device__ int between() const { return n_lo - n_hi; }  // entries in [lo, hi)
  __device__ void take(uint32_t m, double mass, int n) {
    if (!open()) return;
    if (mass >= want) {
      lo = m;
      m_lo = mass;
      n_lo = n;
    } else {
      hi = m;
      m_hi = mass;
      n_hi = n;
    }
  }
};

// The smaller and the larger of v and its partner lane's v (lane ^ JJ): DPP
// within 16-lane rows, permlane swaps across them, a shuffle for JJ = 4.
template <int JJ>
__device__ __forceinline__ void minmax_partner(float v, float& mn, float& mx) {
  if constexpr (JJ == 16 || JJ == 32) {
    float x0, x1;
    swap_rows<JJ == 32>(v, x0, x1);
    mn = fminf(x0, x1);
    mx = fmaxf(x0, x1);
  } else {
    const float p = JJ == 1   ? dpp_f32<0xB1>(v)   // quad_perm [1,0,3,2]
                    : JJ == 2 ? dpp_f32<0x4E>(v)   // quad_perm [2,3,0,1]
                    : JJ == 8 ? dpp_f32<0x128>(v)  // row_ror:8
                              : __shfl_xor(v, JJ);
    mn = fminf(v, p);
    mx = fmaxf(v, p);
  }
}

// Bitonic sort, largest first, of two sets of L * 64 values held as x[j] of
// lane l = element j * 64 + l.  Stage K merges runs of K elements; substage
// JJ compares elements i and i ^ JJ, the lower one keeping the larger value
// where bit K of i is clear (the run is ordered largest first) and the
// smaller where it is set.  JJ >= 64 pairs registers of one lane.  With
// TWO false only `a` is sorted (`b` is not touched).
template <int L, int K, int JJ, bool TWO>
__device__ __forceinline__ void bitonic_sub(float (&a)[L], float (&b)[L], int lane) {
  if constexpr (JJ >= ST_WAVE) {
    constexpr int R = JJ / ST_WAVE;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      if (j & R) continue;
      const bool desc = ((j * ST_WAVE) & K) == 0;
      const float a0 = a[j], a1 = a[j ^ R];
      a[j] = desc ? fmaxf(a0, a1) : fminf(a0, a1);
      a[j ^ R] = desc ? fminf(a0, a1) : fmaxf(a0, a1);
      if constexpr (TWO) {
        const float b0 = b[j], b1 = b[j ^ R];
        b[j] = desc ? fmaxf(b0, b1) : fminf(b0, b1);
        b[j ^ R] = desc ? fminf(b0, b1) : fmaxf(b0, b1);
      }
    }
  } else {
    const bool lower = (lane & JJ) == 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const bool desc = K < ST_WAVE ? (lane & K) == 0 : ((j * ST_WAVE) & K) == 0;
      float mn, mx;
      minmax_partner<JJ>(a[j], mn, mx);
      a[j] = lower == desc ? mx : mn;
      if constexpr (TWO) {
        minmax_partner<JJ>(b[j], mn, mx);
        b[j] = lower == desc ? mx : mn;
      }
    }
  }
  if constexpr (JJ > 1) bitonic_sub<L, K, JJ / 2, TWO>(a, b, lane);
}
template <int L, int K = 2, bool TWO = true>
__device__ __forceinline__ void bitonic_desc(float (&a)[L], float (&b)[L], int lane) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8, "a power-of-two count a lane");
  bitonic_sub<L, K, K / 2, TWO>(a, b, lane);
  if constexpr (K < L * ST_WAVE) bitonic_desc<L, K * 2, TWO>(a, b, lane);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// A row's cut from its candidates sorted largest first (negative: none):
// running sums from the mass at or above the row's upper bound (fp64, in
// sorted order), the first candidate whose sum reaches `want` becomes the
// lower bound with the sum at its value's last copy as its mass, and the row
// is decided.  An open row with no such candidate keeps its lower bound.
template <int L>
__device__ inline void sorted_cut(const float (&x)[L], int lane, CutRow& r) {
  if (!r.open()) return;  // wave-uniform
  double run[L];
  double carry = r.m_hi;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    run[j] = carry + wave_incl_scan((double)fmaxf(x[j], 0.f));
    carry = uniform_f64(readlane_f64(run[j], ST_WAVE - 1));
  }
  int fj = -1, fl = 0;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint64_t m = __ballot(x[j] >= 0.f && run[j] >= r.want);
    if (fj < 0 && m) {
      fj = j;
      fl = __ffsll((unsigned long long)m) - 1;
    }
  }
  if (fj >= 0) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j)
      if (j == fj) v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(x[j]), fl));
    // the value's last copy (copies are adjacent in the sorted order)
    int lj = 0, ll = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const uint64_t m = __ballot(x[j] == v);
      if (m) {
        lj = j;
        ll = 63 - __clzll((long long)m);
      }
    }
    double kept = 0.0;
#pragma unroll
    for (int j = 0; j < L; ++j)
      if (j == lj) kept = readlane_f64(run[j], ll);
    r.lo = __float_as_uint(v);
    r.m_lo = uniform_f64(kept);
  }
  r.hi = r.lo + 1u;
}

// Nucleus (top-p) cuts of the target and draft weights P and Q (totals zt,
// zd; largest entries at most pmax, qmax): the largest value `cut` whose mass
// at or above it still reaches top_p of the total, searched for over the bit
// patterns of non-negative floats (which order like the values).  The
// kept set {X >= cut} is the smallest set of most likely tokens holding top_p
// of the mass, with every token tied at the cut.  Entries below the cut are
// zeroed and zt, zd become the kept mass.  Only P is cut when `both` is false.
//
// While many entries lie between a row's bounds, each step is a pass over
// every entry of both rows with one block reduction (masses and counts).
// Once at most kCutCand entries of each open row remain between its bounds
// they are gathered into LDS and wavefront 0 finishes both searches alone: it
// sorts each row's candidates (largest first) and keeps running sums over
// them from the mass at or above the upper bound; the cut is the first
// candidate whose running sum reaches top_p of the total (every larger value
// keeps less), and the kept mass is the running sum at that value's last
// copy.  No candidate reaching it leaves the cut at the lower bound.
//
// Before the passes, one histogram pass brackets each row's cut: bin masses
// and counts of the weights at or above the row's starting bound, suffix sums
// over the bins (largest first) give the mass and count at or above every
// bin, and the bin whose suffix first reaches top_p of the total holds the
// cut.  Its bounds, with the masses and counts at them, start the search, so
// that the candidates are usually few enough to gather at once (the passes
// remain for a bin that holds more).
//
// The search starts from a lower bound that is always inside the nucleus:
// entries below (1 - top_p) Z / (2 V) hold at most half of the mass the
// nucleus may leave out, so the mass at or above it exceeds top_p Z.  (Its
// own mass is then unknown until the lower bound first moves.)
__device__ inline uint32_t nucleus_floor(double z, float top_p, int V, float xmax) {
  const float f = __double2float_rd((1.0 - (double)top_p) * z / (2.0 * V));
  return (f > 0.f && f < xmax) ? __float_as_uint(f) : 0u;
}

template <bool VEC, int NPT>
__device__ inline void nucleus_cut(float (&P)[NPT], float (&Q)[NPT], bool both, float pmax,
                                   float qmax, float top_p, int V, double& zt, double& zd,
                                   CutLds& c, float& cut_t, float& cut_d) {
  constexpr int kUnknown = 1 << 30;
  const int tid = threadIdx.x, lane = tid % ST_WAVE;
  // one register per entry from here on (otherwise the compiler may keep a
  // row value and its masked copy both live through the search and spill)
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    asm volatile("" : "+v"(P[e]));
    asm volatile("" : "+v"(Q[e]));
  }
  // every bound and total below is block-uniform: kept in scalar registers
  zt = uniform_f64(zt);
  zd = uniform_f64(zd);
  const uint32_t ft = nucleus_floor(zt, top_p, V, pmax);
  const uint32_t fd = both ? nucleus_floor(zd, top_p, V, qmax) : 0u;
  CutRow rt{ft, (uint32_t)__builtin_amdgcn_readfirstlane(__float_as_uint(pmax) + 1u),
            (double)top_p * zt, ft ? -1.0 : zt, 0.0, kUnknown, 0};
  CutRow rd{fd, (uint32_t)__builtin_amdgcn_readfirstlane(both ? __float_as_uint(qmax) + 1u : 1u),
            (double)top_p * zd, fd ? -1.0 : zd, 0.0, kUnknown, 0};
  {
    // histogram of the weights at or above the starting bounds
    for (int i = tid; i < 2 * kBins; i += kNodeBlock) (&c.hm[0][0])[i] = 0ull;
    if (tid < 2) c.hb[tid].found = 0;
    __syncthreads();
    // (a row without mass, as an all-zero probability row, bins nothing;
    // both factors are block-uniform, kept in scalar registers)
    const float it = __uint_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_uint(zt > 0.0 ? (float)(1.0 / zt) : 0.f)));
    const float id = __uint_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_uint(both && zd > 0.0 ? (float)(1.0 / zd) : 0.f)));
    // an entry is binned iff it is positive and at or above its row's floor:
    // max(floor, 1) <= bits <= bits(+inf) as one unsigned compare, the set
    // the value compares x > 0 and x >= floor select
    auto bin_row = [&](const float (&X)[NPT], uint32_t fl, float inv, unsigned long long* h) {
      const uint32_t l1 = fl > 1u ? fl : 1u, span = 0x7F800000u - l1;
#pragma unroll
      for (int e = 0; e < NPT; ++e) {
        const uint32_t u = __float_as_uint(X[e]);
        if (u - l1 <= span) atomicAdd(&h[u >> kBinShift], fix36(X[e] * inv) + kCountOne);
      }
    };
    bin_row(P, ft, it, c.hm[0]);
    if (both) bin_row(Q, fd, id, c.hm[1]);
    __syncthreads();
    // suffix sums, largest bin first: thread t holds bins kBins-1-2t and
    // kBins-2-2t; integers below 2^53, so every double sum is exact
    const int w = tid / ST_WAVE, b0 = kBins - 1 - 2 * tid, b1 = b0 - 1;
    double m0[2], m1[2], n0[2], n1[2], im[2], in_[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const unsigned long long h0 = c.hm[r][b0], h1 = c.hm[r][b1];
      m0[r] = (double)(h0 & kMassMask);
      m1[r] = (double)(h1 & kMassMask);
      n0[r] = (double)(h0 >> kCountShift);
      n1[r] = (double)(h1 >> kCountShift);
      im[r] = wave_incl_scan(m0[r] + m1[r]);
      in_[r] = wave_incl_scan(n0[r] + n1[r]);
      if (lane == ST_WAVE - 1) {
        c.wm[r][w] = im[r];
        c.wn[r][w] = in_[r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r == 1 && !both) break;
      // the waves before this one: lane k < w holds wave k's totals (integers
      // below 2^53, so the sums are exact in any order)
      const int wk = lane & (kMaxWaves - 1);
      const double pm = wave_sum(lane < w ? c.wm[r][wk] : 0.0);
      const double pn = wave_sum(lane < w ? c.wn[r][wk] : 0.0);
      const double am = pm + im[r] - (m0[r] + m1[r]);  // mass of the bins above b0
      const double an = pn + in_[r] - (n0[r] + n1[r]);
      const double z = r ? zd : zt;
      const double wf = z > 0.0 ? (double)top_p * kFix : 0.0;  // top_p of the total, bin units
      const uint32_t floor_bits = r ? fd : ft;
      // the crossing bin: its suffix reaches top_p of the total, the bins
      // above it do not (exactly one bin of one thread)
      int hit = -1;
      double sa = 0.0, sn = 0.0, bm = 0.0, bn = 0.0;
      if (am < wf && am + m0[r] >= wf) {
        hit = b0;
        sa = am;
        sn = an;
        bm = m0[r];
        bn = n0[r];
      } else if (am + m0[r] < wf && am + m0[r] + m1[r] >= wf) {
        hit = b1;
        sa = am + m0[r];
        sn = an + n0[r];
        bm = m1[r];
        bn = n1[r];
      }
      if (hit >= 0) {
        const uint32_t blo = (uint32_t)hit << kBinShift;
        const unsigned long long bhi = (unsigned long long)(hit + 1) << kBinShift;
        c.hb[r] = BinCut{blo > floor_bits ? blo : floor_bits,
                         (uint32_t)(bhi > 0xFFFFFFFFull ? 0xFFFFFFFFull : bhi),
                         (sa + bm) * (z / kFix), sa * (z / kFix), (int)(sn + bn), (int)sn, 1};
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r == 1 && !both) break;
      if (__builtin_amdgcn_readfirstlane(c.hb[r].found)) {
        CutRow& row = r ? rd : rt;
        row.lo = (uint32_t)__builtin_amdgcn_readfirstlane(c.hb[r].lo);
        row.hi = (uint32_t)__builtin_amdgcn_readfirstlane(c.hb[r].hi);
        row.m_lo = uniform_f64(c.hb[r].m_lo);
        row.m_hi = uniform_f64(c.hb[r].m_hi);
        row.n_lo = __builtin_amdgcn_readfirstlane(c.hb[r].n_lo);
        row.n_hi = __builtin_amdgcn_readfirstlane(c.hb[r].n_hi);
      }
    }
  }
  int set = 0;
  bool few = (!rt.open() || rt.between() <= kCutCand) && (!rd.open() || rd.between() <= kCutCand);
  while (!few && (rt.open() || rd.open())) {  // block-uniform
    const uint32_t mt = rt.mid(), md = rd.mid();
    int nt = 0, nd = 0;
    double st = kept_sum<VEC, NPT>(P, __uint_as_float(mt), nt);
    double sd = both ? kept_sum<VEC, NPT>(Q, __uint_as_float(md), nd) : 0.0;
    // both counts (each at most 32768) in one exactly summed double
    double sn = (double)(nt * 65536 + nd);
    block_sum3_set<kNodeBlock>(st, sd, sn, c.red, set);
    set ^= 1;
    const long long n = (long long)sn;
    rt.take(mt, st, (int)(n >> 16));
    rd.take(md, sd, (int)(n & 0xFFFF));
    few = (!rt.open() || rt.between() <= kCutCand) && (!rd.open() || rd.between() <= kCutCand);
    if (few) break;
  }
  if (few && (rt.open() || rd.open())) {
    // gather the candidates, each row's entries in [lo, hi), into LDS slots
    // taken from a counter (their order does not matter: they are sorted)
    const bool ot = rt.open(), od = rd.open();
    if (tid < 2) c.wtot[tid] = 0;
    __syncthreads();
    // x is a candidate iff x > 0 and lo <= bits(x) < hi (zeros are never
    // needed): (bits(x) - max(lo, 1)) < hi - max(lo, 1) as unsigned, which
    // -0, negative values and NaN patterns fail as the value compares would.
    // One branch per four entries: most wavefronts hold no candidate.
    static_assert(NPT % 4 == 0, "entries in fours");
    auto gather = [&](const float (&X)[NPT], uint32_t lo, uint32_t hi, int* cnt, float* dst) {
      const uint32_t l1 = lo > 1u ? lo : 1u, span = hi > l1 ? hi - l1 : 0u;
#pragma unroll
      for (int k = 0; k < NPT / 4; ++k) {
        bool m[4], any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m[j] = __float_as_uint(X[4 * k + j]) - l1 < span;
          any |= m[j];
        }
        if (any) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (m[j]) {
              const int p = atomicAdd(cnt, 1);
              if (p < kCutCand) dst[p] = X[4 * k + j];
            }
          }
        }
      }
    };
    if (ot) gather(P, rt.lo, rt.hi, &c.wtot[0], c.cand[0]);
    if (od) gather(Q, rd.lo, rd.hi, &c.wtot[1], c.cand[1]);
    __syncthreads();
    if (tid < 2 * ST_WAVE) {
      // wavefront 0 finishes the target row's search and wavefront 1 the
      // draft row's, at once: the row's candidates sorted, largest first
      // (missing entries are -1 and sort last), by the smallest network that
      // holds them, then the cut from running sums
      auto finish = [&](CutRow& row, int cnt, const float* cand, auto per_lane) {
        constexpr int L = decltype(per_lane)::value;
        float x[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
          const int q = j * ST_WAVE + lane;
          x[j] = q < cnt ? cand[q] : -1.f;
        }
        bitonic_desc<L, 2, false>(x, x, lane);
        sorted_cut<L>(x, lane, row);
      };
      auto one = [&](CutRow& row, bool open, int slot) {
        if (open) {  // wave-uniform
          const int cnt = row.between();
          if (cnt <= 2 * ST_WAVE) finish(row, cnt, c.cand[slot], std::integral_constant<int, 2>{});
          else finish(row, cnt, c.cand[slot], std::integral_constant<int, kCutLane>{});
        }
        if (lane == 0) {
          c.cut[slot] = row.lo;
          c.kept[slot] = row.m_lo;
        }
      };
      if (__builtin_amdgcn_readfirstlane(tid / ST_WAVE) == 0) one(rt, ot, 0);
      else one(rd, od, 1);
    }
    __syncthreads();
    rt.lo = (uint32_t)__builtin_amdgcn_readfirstlane(c.cut[0]);
    rd.lo = (uint32_t)__builtin_amdgcn_readfirstlane(c.cut[1]);
    rt.m_lo = uniform_f64(c.kept[0]);
    rd.m_lo = uniform_f64(c.kept[1]);
  }
  if ((rt.m_lo < 0.0) | (rd.m_lo < 0.0)) {  // a cut at the starting bound
    int nt = 0, nd = 0;
    double st = kept_sum<VEC, NPT>(P, __uint_as_float(rt.lo), nt);
    double sd = both ? kept_sum<VEC, NPT>(Q, __uint_as_float(rd.lo), nd) : 0.0;
    double sn = 0.0;
    block_sum3_set<kNodeBlock>(st, sd, sn, c.red, set);
    if (rt.m_lo < 0.0) rt.m_lo = st;
    if (rd.m_lo < 0.0) rd.m_lo = sd;
  }
  cut_t = __uint_as_float(rt.lo);
  cut_d = __uint_as_float(rd.lo);
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    P[e] = P[e] >= cut_t ? P[e] : 0.f;
    if (both) Q[e] = Q[e] >= cut_d ? Q[e] : 0.f;
  }
  zt = rt.m_lo;
  if (both) zd = rd.m_lo;
}

// v plus the partner lane's v at exchange stage S: the lanes l ^ 32, l ^ 16,
// l ^ 8 (a row rotation by 8), l ^ 7 (mirror inside 8 lanes), l ^ 2, l ^ 1.
// Both partners add the same two operands, so they end with the same bits.
template <int S>
__device__ __forceinline__ double xsum(double v) {
  if constexpr (S <= 1) {
    double x0, x1;
    swap_rows<S == 0>(v, x0, x1);
    return x0 + x1;
  } else if constexpr (S == 2) {
    return v + dpp_f64<0x128>(v);  // row_ror:8
  } else if constexpr (S == 3) {
    return v + dpp_f64<0x141>(v);  // row_half_mirror
  } else if constexpr (S == 4) {
    return v + dpp_f64<0x4E>(v);  // quad_perm [2,3,0,1]
  } else {
    return v + dpp_f64<0xB1>(v);  // quad_perm [1,0,3,2]
  }
}
// One halving exchange: every one of the M values is summed with the
// partner's, and a lane keeps the half selected by the stage's lane bit
// (bit 5 - S, which the two partners hold with opposite values).
template <int S, int M>
__device__ __forceinline__ void halve(double (&cur)[16], int lane) {
  const bool upper = lane & (32 >> S);
#pragma unroll
  for (int j = 0; j < M / 2; ++j) {
    const double lo = xsum<S>(cur[j]), hi = xsum<S>(cur[j + M / 2]);
    cur[j] = upper ? hi : lo;
  }
}
// The wavefront sums of N (8 or 16) per-lane values, all at once: log2(N)
// halving exchanges leave each lane with the partial sum of one value (value
// k in lanes k * 64 / N ...), and the remaining exchanges complete it.
template <int N>
__device__ inline void wave_sum_n(const double (&t)[N], double (&S)[N]) {
  static_assert(N == 8 || N == 16, "8 or 16 values");
  const int lane = threadIdx.x % ST_WAVE;
  double cur[16];
#pragma unroll
  for (int j = 0; j < N; ++j) cur[j] = t[j];
  halve<0, N>(cur, lane);
  halve<1, N / 2>(cur, lane);
  halve<2, N / 4>(cur, lane);
  if constexpr (N == 16)
    halve<3, 2>(cur, lane);
  else
    cur[0] = xsum<3>(cur[0]);
  cur[0] = xsum<4>(cur[0]);
  cur[0] = xsum<5>(cur[0]);
  const uint64_t bits = (uint64_t)__double_as_longlong(cur[0]);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int src = k * (ST_WAVE / N);
    const uint32_t lo32 = __builtin_amdgcn_readlane((int)(uint32_t)bits, src);
    const uint32_t hi32 = __builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), src);
    S[k] = __longlong_as_double((long long)(((uint64_t)hi32 << 32) | lo32));
  }
}

struct DrawLds {
  double wsum[kMaxWaves];
  int pick, tie;
};

// Inverse-CDF draw from the residual w_v = max(0, P_v - c Q_v) in ascending
// vocab order (any positive multiple of it draws the same token): the
// smallest v whose running sum exceeds u * sum(w).  Every
// wavefront reduces its slice of the row; the prefix over the slices (summed
// in wavefront order by every thread) names the slice that crosses the
// threshold, and that wavefront alone locates the tile, then the entry.  The
// threshold test at every level compares running sums that begin where the
// previous level's left off.  Returns sum(w); pick and tie are set when it is
// positive.
template <bool VEC, int NPT>
__device__ inline double draw_residual(const float (&P)[NPT], const float (&Q)[NPT], float c,
                                       double u, DrawLds& s, int& pick, int& tie) {
  constexpr int EPT = VEC ? 4 : 1, NT = NPT / EPT, NW = kStochMaxV / NPT / ST_WAVE;
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
  for (int i = 0; i < NW; ++i) total += s.wsum[i];
  const double thr = u * total;
  // the slice: running sums over the wavefronts' slices, in the same order
  double base = 0.0, run0 = 0.0;
  int ws = -1;
  for (int i = 0; i < NW; ++i) {
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
    auto visit = [&](int k, double tsum) {
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
    };
    if constexpr (NT == 8 || NT == 16) {
      double t[NT], S[NT];
#pragma unroll
      for (int k = 0; k < NT; ++k) t[k] = resid_group<EPT>(P, Q, cw, k);
      wave_sum_n<NT>(t, S);
#pragma unroll
      for (int k = 0; k < NT; ++k) visit(k, S[k]);
    } else {
      for (int k = 0; k < NT; ++k) {
        double part = 0.0;
#pragma unroll
        for (int kk = 0; kk < NT; ++kk)
          if (kk == k) part = resid_group<EPT>(P, Q, cw, kk);
        visit(k, wave_sum(part));
      }
    }
    if (kt < 0) {  // rounding: no tile crosses; take the last positive one
      kt = klast;
      tbase = lbase;
    }
    // the entry: a scan over the lanes of tile kt
    float sp[EPT], sq[EPT], wt[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      sp[j] = P[j];
      sq[j] = Q[j];
    }
#pragma unroll
    for (int k = 1; k < NT; ++k) {
      const bool sel = k == kt;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        sp[j] = sel ? P[k * EPT + j] : sp[j];
        sq[j] = sel ? Q[k * EPT + j] : sq[j];
      }
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) wt[j] = resid(sp[j], sq[j], cw);
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
      const int v = row_index<VEC, NPT>(kt * EPT + j, tid);
      s.pick = v;
      s.tie = fabs(ce_hi - thr) < kTieEps * total || (v > 0 && fabs(ce_lo - thr) < kTieEps * total);
    }
  }
  __syncthreads();
  pick = s.pick;
  tie = s.tie;
  return total;
}

struct NodeLds {
  uint64_t kid_mask[ST_MAX_NODES / 64];
  int kids[ST_MAX_NODES];  // children, ascending
  double px[ST_MAX_NODES], qx[ST_MAX_NODES], ua[ST_MAX_NODES];  // per child
  int ok[ST_MAX_NODES];                                           // token in range
  float redf[2 * kMaxWaves];
  double red[2 * kMaxWaves];
  CutLds cut;
  double u_draw;
  DrawLds draw;
};

// One workgroup per node u, which holds u's two logit rows in registers from
// start to end: it reduces them to their softmax statistics (max M and
// Z = sum of exp2((l - M) * log2e / T), terms rounded to fp32, groups of four
// summed in fp32 and the groups in fp64), then decides what the walk would do
// on reaching u: test u's children in ascending order, child c with token x
// accepted iff u_acc(c) q_u[x] < r[x] with r starting at p_u, and draw the
// replacement token from r when no child is accepted (a leaf draws from p_u).
// The tree is read before the rows' loads are issued, so that waiting for it
// never waits for them.
// EXT: the draft may be probabilities and the rows may be cut to their
// nucleus (a separate instance, so the plain path keeps its registers).
template <bool VEC, bool EXT>
__global__ void __launch_bounds__(kNodeBlock)
stoch_node_kernel(StochArgs g) {
  constexpr int NPT = kStochMaxV / kNodeBlock, EPT = VEC ? 4 : 1;
  __shared__ NodeLds s;
  const int tid = threadIdx.x;
  // Workgroup i * B + b takes local node i of request b: the requests'
  // first nodes go first.  Parents precede their children, so those are
  // mostly nodes with children, which also read the draft row; the leaves,
  // half the work, come in the later workgroups.
  const int b = blockIdx.x % g.B, i = blockIdx.x / g.B;
  // When every request has max_nodes nodes, node i of request b is row
  // b * max_nodes + i, and its tree entries and target row are requested
  // before node_off arrives.  Those rows lie inside the T rows whatever
  // node_off holds; they are kept only if node_off confirms them.  A thread's
  // node of the request is clamped, so the loads are unconditional.
  const int lo_u = b * g.max_nodes;
  int par = 0, tok = 0;
  float P[NPT], Q[NPT];
  if (g.uniform) {
    const int c = tid < g.max_nodes ? tid : 0;
    par = g.parent[lo_u + c];
    tok = g.tokens[lo_u + c];
    load_row<VEC>(g.tl + (size_t)(lo_u + i) * g.V, g.V, true, P);
  }
  const int lo = g.node_off[b], hi = g.node_off[b + 1], n = hi - lo, t = lo + i;
  if (!((lo >= 0) & (hi <= g.T) & (n >= 1) & (n <= g.max_nodes) & (i < n))) {
    __builtin_amdgcn_s_waitcnt(0);  // no load left in flight
    return;  // past the request's nodes (or a request the walk flags)
  }
  if (!g.uniform || lo != lo_u || n != g.max_nodes) {
    const int c = tid < n ? tid : 0;
    par = g.parent[lo + c];
    tok = g.tokens[lo + c];
    load_row<VEC>(g.tl + (size_t)t * g.V, g.V, true, P);
  }
  if (tid < ST_MAX_NODES / 64) s.kid_mask[tid] = 0;
  if (tid == kNodeBlock - 1) {
    double ua, us;
    node_uniforms(g.seed, g.offset, b, i, ua, us);
    s.u_draw = us;
  }
  __syncthreads();
  const bool kid = tid < n && tid > i && par == i;
  if (kid) atomicOr((unsigned long long*)&s.kid_mask[tid >> 6], 1ull << (tid & 63));
  __syncthreads();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < ST_MAX_NODES / 64; ++w) nk += __popcll(s.kid_mask[w]);
  nk = __builtin_amdgcn_readfirstlane(nk);  // block-uniform
  // The draft row only for a node with children: a leaf's draw uses p alone,
  // so its draft row is never read (nor checked for non-finite entries), and
  // nothing below reads Q unless nk > 0.  The target row's loads, issued
  // first, stay in flight meanwhile (the barriers above wait for LDS only).
  if (nk) {
    load_row<VEC>(g.dl + (size_t)t * g.V, g.V, true, Q);
  } else {
#pragma unroll
    for (int e = 0; e < NPT; ++e) asm("" : "=v"(Q[e]));  // defined, never read
  }
  // each child's token logits (issued now, used after the statistics)
  int rank = 0;
  float lt = 0.f, ld = 0.f;
  const bool ok = kid && tok >= 0 && tok < g.V;
  if (kid) {
    rank = __popcll(s.kid_mask[tid >> 6] & ((1ull << (tid & 63)) - 1));
    for (int w = 0; w < (tid >> 6); ++w) rank += __popcll(s.kid_mask[w]);
    const size_t at = (size_t)t * g.V + (ok ? tok : 0);
    lt = g.tl[at];
    ld = g.dl[at];
  }

  // statistics of both rows (the target row's first, while the draft row's
  // loads may still be in flight): maxima, and minima for the finite check
  const bool probs = EXT && g.draft_probs;  // a draft given as probabilities
  float mt = -INFINITY, md = -INFINITY, nt = INFINITY, nd = INFINITY;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    mt = fmaxf(mt, P[e]);
    nt = fminf(nt, P[e]);
  }
  if (nk) {
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      md = fmaxf(md, Q[e]);
      nd = fminf(nd, Q[e]);
    }
  }
  // Non-finite entries: -inf (or a negative probability) shows in the minima;
  // NaN and +inf make the sums below NaN (an exponential of NaN, or of
  // inf - inf), except +inf in a probability row, which shows in its maximum.
  bool bad = nt == -INFINITY || (nk && (probs ? !(nd >= 0.f) : nd == -INFINITY));
  block_max2<kNodeBlock>(mt, md, s.redf);
  if (nk && probs && md == INFINITY) bad = true;
  // Entries past the row end (only the wavefront holding the row end has
  // any; they hold copies of the row's first logit) become -inf, or 0 in a
  // probability row, so that their terms below are exactly 0.
  constexpr bool kWaveMask = VEC && !EXT;
  if (kWaveMask && __builtin_amdgcn_readfirstlane(tid / ST_WAVE + 1) * (NPT * ST_WAVE) > g.V) {
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const bool past = row_index<VEC, NPT>(e, tid) >= g.V;
      P[e] = past ? -INFINITY : P[e];
      Q[e] = past ? (probs ? 0.f : -INFINITY) : Q[e];
    }
  }
  const float sc = kLog2e / g.temperature;
  // the rows become their exponentials exp2((l - M) * s) in place (the draft
  // row only where it is used: a node with children; a probability row as it
  // is); a group's terms are summed in fp32, the groups in fp64
  const int kin = kWaveMask ? NPT / EPT : groups_inside<VEC, NPT>(g.V, tid);
  double zt = 0.0, zd = 0.0;
#pragma unroll
  for (int k = 0; k < NPT / EPT; ++k) {
    const bool in = kWaveMask || k < kin;
    float st_ = 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const float e = exp2_fast((P[k * EPT + j] - mt) * sc);
      P[k * EPT + j] = in ? e : 0.f;
      st_ = j ? st_ + P[k * EPT + j] : P[k * EPT + j];
    }
    zt += (double)st_;
  }
  if (nk) {
#pragma unroll
    for (int k = 0; k < NPT / EPT; ++k) {
      const bool in = kWaveMask || k < kin;
      float sd_ = 0.f;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const float e = probs ? Q[k * EPT + j] : exp2_fast((Q[k * EPT + j] - md) * sc);
        Q[k * EPT + j] = in ? e : 0.f;
        sd_ = j ? sd_ + Q[k * EPT + j] : Q[k * EPT + j];
      }
      zd += (double)sd_;
    }
  }
  block_sum2<kNodeBlock>(zt, zd, s.red);
  if (tid == 0 && (zt != zt || (nk && zd != zd))) bad = true;
  if (bad) st::set_status(g.status, ST_STATUS_NONFINITE);
  // nucleus sampling: both rows restricted to their top-p nucleus (the draft
  // row only where it is used)
  float cut_t = 0.f, cut_d = 0.f;
  if (EXT && g.top_p < 1.f)
    nucleus_cut<VEC, NPT>(P, Q, nk > 0, 1.f, g.draft_probs ? md : 1.f, g.top_p, g.V, zt, zd,
                          s.cut, cut_t, cut_d);
  const double a = 1.0 / zt;

  if (nk == 0) {  // a leaf: the walk stops here with r = p_u
    int token, tie;
    draw_residual<VEC>(P, P, 0.f, s.u_draw, s.draw, token, tie);
    if (tid == 0) g.verdict[t] = NodeVerdict{-1, 0, token, tie};
    return;
  }

  const double bq = 1.0 / zd, ratio = zt / zd;  // c' = c Z_t / Z_d
  if (kid) {
    s.kids[rank] = tid;
    s.ok[rank] = ok;
    if (ok) {
      // the same fp32 weights as the registers hold, cut the same way
      const float et = exp2_fast((lt - mt) * sc);
      const float ed = EXT && g.draft_probs ? ld : exp2_fast((ld - md) * sc);
      s.px[rank] = et >= cut_t ? (double)et * a : 0.0;
      s.qx[rank] = ed >= cut_d ? (double)ed * bq : 0.0;
      double ua, us;
      node_uniforms(g.seed, g.offset, b, tid, ua, us);
      s.ua[rank] = ua;
    }
  }
  __syncthreads();

  int ties = 0, accepted = -1;
  double cc = 0.0, D = 1.0;
  // child k's test against r = max(0, p - c q) / D
  auto test = [&](int k) {
    if (!s.ok[k]) return false;
    const double qv = s.qx[k];
    const double r = fmax(0.0, s.px[k] - cc * qv) / D;
    const double lhs = s.ua[k] * qv;
    ties += fabs(r - lhs) < kTieEps;
    return lhs < r;
  };
  int token = -1, tie = 0;
  if (test(0)) {
    accepted = s.kids[0];
  } else {
    // after each rejection r <- max(0, r - q) renormalised, i.e. c <- c + D
    for (int k = 1; k < nk && accepted < 0; ++k) {
      const double cn = cc + D;
      const double Dn =
          a * block_sum<kNodeBlock>(resid_sum<VEC>(P, Q, (float)(cn * ratio)), s.red, k & 1);
      if (Dn > kMassEps * D) {
        cc = cn;
        D = Dn;
      }
      if (test(k)) accepted = s.kids[k];
    }
    if (accepted < 0) {  // every child rejected: draw from the final residual
      const double total =
          draw_residual<VEC>(P, Q, (float)((cc + D) * ratio), s.u_draw, s.draw, token, tie);
      if (!(total * a > kMassEps * D)) {  // the last rejection left no mass: r unchanged
        __syncthreads();
        draw_residual<VEC>(P, Q, (float)(cc * ratio), s.u_draw, s.draw, token, tie);
      }
    }
  }
  if (tid == 0) g.verdict[t] = NodeVerdict{accepted, ties, token, tie};
}

// One wavefront per request follows the verdicts from the root.
__global__ void __launch_bounds__(ST_WAVE)
stoch_walk_kernel(st::StochWalkArgs g) {
  __shared__ st::StochWalkLds s;
  st::stoch_walk_wave(g, blockIdx.x, s, true);
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
  hipLaunchKernelGGL(row_argmax_kernel, dim3(g.T * g.nslices), dim3(kArgmaxBlock), 0,
                     (hipStream_t)stream, logits, g.V, g.nslices, (ArgmaxPart*)g.part, g.status);
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

int st::stochastic_prepare(const st_tree* tree, int V, const int32_t* tokens,
                           const float* target_logits, const float* draft_logits,
                           float temperature, int32_t* accept_len, int32_t* accept_nodes,
                           int32_t* out_tokens, int32_t* near_ties, void* workspace,
                           size_t ws_bytes, int32_t* status, st::StochWalkArgs& walk) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (V < 1 || !tokens || !target_logits || !draft_logits || !accept_len || !accept_nodes ||
      !out_tokens || !workspace || !(temperature > 0.0f))
    return ST_E_INVALID;
  if (V > kStochMaxV || tree->max_depth + 1 > kMaxPath) return ST_E_UNSUPPORTED;
  if (ws_bytes < st_verify_stochastic_workspace(tree, V)) return ST_E_WORKSPACE;
  walk = st::StochWalkArgs{tree->node_off, tree->parent, tokens, (const NodeVerdict*)workspace,
                           tree->total_nodes, V, tree->max_nodes, tree->max_depth, accept_len,
                           accept_nodes, out_tokens, near_ties, status};
  return ST_OK;
}

namespace {
int node_launch(const st::StochWalkArgs& w, const float* target_logits, const float* draft,
                int draft_probs, float temperature, float top_p, uint64_t seed, uint64_t offset,
                int B, void* stream) {
  const StochArgs g{w.node_off,   w.parent, w.tokens, target_logits, draft,
                    const_cast<NodeVerdict*>(w.verdict), B, w.T, w.V, w.max_nodes, temperature,
                    seed,         offset,   w.status, draft_probs, top_p,
                    w.T == B * w.max_nodes};
  // one workgroup per (local node, request) pair; a launch holds fewer
  // than 2^32 work-items
  if ((uint64_t)B * (uint64_t)w.max_nodes * kNodeBlock > 0xffffffffull) return ST_E_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const bool vec = (w.V & 3) == 0, ext = draft_probs || top_p < 1.f;
  const dim3 grid((unsigned)B * (unsigned)w.max_nodes);
  if (vec && !ext)
    hipLaunchKernelGGL((stoch_node_kernel<true, false>), grid, dim3(kNodeBlock), 0, s, g);
  else if (!ext)
    hipLaunchKernelGGL((stoch_node_kernel<false, false>), grid, dim3(kNodeBlock), 0, s, g);
  else if (vec)
    hipLaunchKernelGGL((stoch_node_kernel<true, true>), grid, dim3(kNodeBlock), 0, s, g);
  else
    hipLaunchKernelGGL((stoch_node_kernel<false, true>), grid, dim3(kNodeBlock), 0, s, g);
  return st::check_launch();
}
}  // namespace

int st::stochastic_node_launch(const st::StochWalkArgs& w, const float* target_logits,
                               const float* draft_logits, float temperature, uint64_t seed,
                               uint64_t offset, int B, void* stream, int draft_probs,
                               float top_p) {
  return node_launch(w, target_logits, draft_logits, draft_probs, temperature, top_p, seed,
                     offset, B, stream);
}

extern "C" int st_verify_stochastic(const st_tree* tree, int V, const int32_t* tokens,
                                    const float* target_logits, const float* draft_logits,
                                    float temperature, uint64_t seed, uint64_t offset,
                                    int32_t* accept_len, int32_t* accept_nodes,
                                    int32_t* out_tokens, int32_t* near_ties, void* workspace,
                                    size_t ws_bytes, int32_t* status, void* stream) {
  st::StochWalkArgs w;
  int rc = st::stochastic_prepare(tree, V, tokens, target_logits, draft_logits, temperature,
                                  accept_len, accept_nodes, out_tokens, near_ties, workspace,
                                  ws_bytes, status, w);
  if (rc || (rc = st::stochastic_node_launch(w, target_logits, draft_logits, temperature, seed,
                                             offset, tree->B, stream)))
    return rc;
  hipLaunchKernelGGL(stoch_walk_kernel, dim3(tree->B), dim3(ST_WAVE), 0, (hipStream_t)stream, w);
  return st::check_launch();
}

extern "C" int st_verify_stochastic_ex(const st_tree* tree, int V, const int32_t* tokens,
                                       const float* target_logits, const float* draft,
                                       int draft_is_probs, float temperature, float top_p,
                                       uint64_t seed, uint64_t offset, int32_t* accept_len,
                                       int32_t* accept_nodes, int32_t* out_tokens,
                                       int32_t* near_ties, void* workspace, size_t ws_bytes,
                                       int32_t* status, void* stream) {
  if (!(top_p > 0.f && top_p <= 1.f) || (draft_is_probs != 0 && draft_is_probs != 1))
    return ST_E_INVALID;
  st::StochWalkArgs w;
  int rc = st::stochastic_prepare(tree, V, tokens, target_logits, draft, temperature, accept_len,
                                  accept_nodes, out_tokens, near_ties, workspace, ws_bytes,
                                  status, w);
  if (rc || (rc = node_launch(w, target_logits, draft, draft_is_probs, temperature, top_p, seed,
                              offset, tree->B, stream)))
    return rc;
  hipLaunchKernelGGL(stoch_walk_kernel, dim3(tree->B), dim3(ST_WAVE), 0, (hipStream_t)stream, w);
  return st::check_launch();
}

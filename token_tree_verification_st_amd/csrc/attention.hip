// Tree-masked attention of every tree node over its request's cached prefix
// and its own root path ("SpecInfer：基于树结构的LLM推测性推理加速技术" §2.1:
// scores = Q K^T, masked entries excluded, softmax, times V; the SpecInfer news
// article, "Token 樹驗證器": all tree paths are decoded in one pass).
//
// Work decomposition (split-KV).  For request b and kv head g the query rows
// are the N_b tree nodes times the G = Hq/Hkv query heads sharing g; every one
// of them reads the same keys, so a workgroup takes a block of rows and a
// contiguous range of keys ("split") and streams that range once.  Splits
// produce fp32 partials (running max m, sum l, unnormalised output); a request
// whose keys fit in one split writes its output directly.
//
// bf16 path (MFMA, gfx950), the streaming kernel.  A wavefront owns up to 64
// query rows with Q^T held in registers and walks 32-key chunks of K and V,
// copied to LDS by direct global-to-LDS loads.  Per chunk:
//   S^T (keys x rows) = K . Q^T    v_mfma_f32_16x16x32_bf16, A = K from LDS
//   online softmax on S^T          each lane holds 4 keys of one row, so the
//                                  row statistics stay in that lane and need
//                                  two permlane swaps per chunk
//   O^T (dims x rows) += V^T . P^T A = V^T from LDS by transposing reads,
//                                  B = P^T straight from the S^T accumulators
// Keys beyond the prefix are tree keys: key P_b + j is visible to a row iff
// bit j of its node's ancestor mask is set.  A combine kernel merges the
// splits of every row (spread over the whole chip: one workgroup merging all
// splits of a row block would pull them through a single CU).
//
// fp32 path (VALU).  The same decomposition with 16 rows per workgroup and
// plain fp32 dot products; it serves fp32 inputs, which need 1e-5 accuracy.
#include "step_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
struct AttnArgs {
  const int32_t* node_off;
  const int32_t* parent;     // used when mask is null: masks are derived in the kernel
  const int32_t* prefix_len;
  const uint64_t* mask;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  float2* ws_ml;   // [NS][T*Hq] (m in log2 units, l)
  float* ws_acc;   // [NS][T*Hq][D]
  int32_t* ws_ns;  // balanced plans: [T] the split count of each node's request
  int32_t* status;
  st::ArgmaxJob am;  // vocab argmax slices reduced in the prologue (am.logits null: none)
  int B, T, Hq, Hkv, G, S_max, W, max_nodes, max_prefix;
  int KS;          // keys per split (multiple of 16); balanced plans: unused
  int NS;          // splits of the longest request; balanced plans: the most any request has
  int RB;          // rows per workgroup
  int n_rblk;      // row blocks of the widest request
  int items;       // B * Hkv * NS * n_rblk; balanced plans: an upper bound
  int per_xcd;     // ceil(items / 8)
  int balanced;    // splits sized per request on the device (B <= 64)
  int target;      // balanced plans: the workgroups the chunk budget aims for
  int cmax;        // balanced plans: 32-key chunks of the longest possible request
  float scale_log2;
  st::KvPaging pg; // pg.bt null: contiguous caches
};

// The physical block of key `key` of request b in a paged pool: its block-
// table entry, clamped into [0, n_blocks) and flagged when it was outside, so
// every address stays inside the pool.
__device__ inline int table_phys(const AttnArgs& a, int e) {
  const int phys = min(max(e, 0), a.pg.n_blocks - 1);
  if (phys != e) st::set_status(a.status, ST_STATUS_BAD_BLOCK);
  return phys;
}
__device__ inline int table_entry(const AttnArgs& a, int b, int key) {
  return table_phys(a, a.pg.bt[(size_t)b * a.pg.bt_stride + (key >> a.pg.lbs)]);
}

template <typename T>
__device__ inline const T* kv_block_row(const AttnArgs& a, const void* cache, int phys, int g,
                                        int key, int D) {
  return (const T*)cache +
         ((((size_t)phys * a.Hkv + g) << a.pg.lbs) + (key & ((1 << a.pg.lbs) - 1))) * D;
}

// First element of key row `key` of (request b, kv head g): contiguous
// [B][Hkv][S_max][D], or through the block table into a paged pool
// [n_blocks][Hkv][block][D].  Chunks start at multiples of 32 keys and blocks
// hold a multiple of 32, so the rows of one chunk never leave its block.
template <typename T>
__device__ inline const T* kv_row(const AttnArgs& a, const void* cache, int b, int g, int key,
                                  int D) {
  if (!a.pg.bt) return (const T*)cache + (((size_t)b * a.Hkv + g) * a.S_max + key) * D;
  return kv_block_row<T>(a, cache, table_entry(a, b, key), g, key, D);
}

struct Item {
  int w, b, g, split, rblk;
  int ks;  // keys per split of the item's request
};

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).  Item w
// goes to XCD w / per_xcd, so consecutive items -- the row blocks of one
// (request, head, split), which read the same keys -- share an XCD's L2.
__device__ inline bool decode_item(const AttnArgs& a, Item& it) {
  const int bid = blockIdx.x;
  int w = (bid & 7) * a.per_xcd + (bid >> 3);
  if (w >= a.items) return false;
  it.w = w;
  it.rblk = w % a.n_rblk;
  w /= a.n_rblk;
  it.split = w % a.NS;
  w /= a.NS;
  it.g = w % a.Hkv;
  it.b = w / a.Hkv;
  return true;
}

// The argmax slice of workgroup w (units never exceed the workgroups; V is a
// multiple of 4): loads issued at the start of the kernel, reduced once the
// prologue's own loads have been waited for.
__device__ inline void argmax_unit_finish(const AttnArgs& a, int w, const st::ArgmaxRegs& r,
                                          int* scratch) {
  const st::ArgmaxJob& j = a.am;
  st::argmax_slice_finish<true>(r, j.V, w / j.nslices, w % j.nslices, j.nslices, j.part,
                                j.status, scratch);
}

struct ReqInfo {
  int lo, n, P, key_end, nsplit;
  bool ok;
};

// The request's sizes.  The three loads are independent of each other and
// the checks use no branches, so all three are in flight together.
struct ReqWords {
  int lo, hi, P;
};
__device__ inline ReqWords request_load(const AttnArgs& a, int b) {
  return ReqWords{a.node_off[b], a.node_off[b + 1], a.prefix_len[b]};
}

__device__ inline ReqInfo request_finish(const AttnArgs& a, ReqWords w) {
  ReqInfo r;
  r.lo = w.lo;
  r.n = w.hi - w.lo;
  r.P = w.P;
  r.ok = (w.lo >= 0) & (w.hi <= a.T) & (r.n >= 1) & (r.n <= a.max_nodes) & (w.P >= 0) &
         (w.P <= a.max_prefix) & (w.P + r.n <= a.S_max);
  r.key_end = w.P + r.n;
  r.nsplit = (r.key_end + a.KS - 1) / a.KS;
  return r;
}

__device__ inline ReqInfo request_info(const AttnArgs& a, int b) {
  return request_finish(a, request_load(a, b));
}

__device__ inline bool tree_bit(uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3, int j) {
  const int wi = j >> 6;
  const uint64_t w = wi == 0 ? w0 : wi == 1 ? w1 : wi == 2 ? w2 : w3;
  return (w >> (j & 63)) & 1ull;
}

// Ancestor bitmask of request-local node `node` (the node itself and every
// node on its root path) from the request's parent array in LDS.  Each step
// moves to a smaller index, so the walk ends; it returns false when it meets a
// parent outside [0, j) or a root whose parent is not -1.
__device__ inline bool ancestor_words(const int* sPar, int node, uint64_t& w0, uint64_t& w1,
                                      uint64_t& w2, uint64_t& w3) {
  w0 = w1 = w2 = w3 = 0ull;
  int j = node;
  while (true) {
    const uint64_t bit = 1ull << (j & 63);
    const int wi = j >> 6;
    w0 |= wi == 0 ? bit : 0ull;
    w1 |= wi == 1 ? bit : 0ull;
    w2 |= wi == 2 ? bit : 0ull;
    w3 |= wi == 3 ? bit : 0ull;
    const int p = sPar[j];
    if (j == 0) return p == -1;
    if (p < 0 || p >= j) return false;
    j = p;
  }
}

// ---------------------------------------------------------------- bf16 MFMA, shared pieces

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for all of its outstanding global loads
// -- including the prefetch of later tiles that should stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier with the ring's prefetch left in flight.  A release fence
// on LDS makes the compiler wait for every outstanding direct load (they
// write LDS), including chunks still streaming into other ring stages; here
// each wavefront has already waited, with counted waits, for its own direct
// loads that other wavefronts read after the barrier, so only its LDS
// operations need to complete.  The asm's memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier_inflight() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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


#define ST_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// K rows are stored unpadded (D*2 bytes) with 16-byte chunk c at position
// c ^ kswz(row): the 16 lanes that read one chunk of 16 consecutive keys hit
// 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  return D >= 128 ? (key & (D / 8 - 1)) : ((key >> 1) & (D / 8 - 1));
}

// The 32-bit LDS address of a pointer into the workgroup's LDS block.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Eight ds_read_b64_tr_b16 (each lane gets one dim of four keys) issued
// together, with the wait for their results inside the same block.  Written
// out rather than through the builtin because the compiler, unable to tell
// these reads from the in-flight direct loads that refill other ring stages,
// would otherwise wait for every outstanding direct load before the first of
// them; the kernel's own waits already cover the stage read here.  The read
// at address a[j] goes to o[2j], the read OFF bytes further on (the key 16
// rows on: the V swizzle repeats every 8 rows) to o[2j + 1], an immediate
// offset rather than an address of its own.
template <int OFF>
__device__ __forceinline__ void ds_read_tr16_x8(const uint32_t (&a)[4], u32x2 (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
      : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 encoding).
#define ST_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// ---------------------------------------------------------------- bf16 MFMA, 64 rows per wavefront

// Each wavefront owns 64 query rows (four 16-row blocks, Q held in registers)
// and walks its keys in 32-key chunks, one k-step of the P V product.  A chunk
// of K and V is copied to LDS with direct global-to-LDS loads and read from
// there once per wavefront: K as the MFMA A operand, V through the transposing
// read.  Every K and V fragment read from LDS serves all four row blocks.
//
// A workgroup is RWV row groups (64 rows each) x KWV = 4 / RWV key groups.  Key
// group kg takes chunks kg, kg + KWV, ... of the workgroup's key range through
// its own NSTAGE-deep ring.  With RWV = 1 every wavefront has a ring of its
// own and never waits for another one; with RWV > 1 the row groups share the
// ring of their key group, split its loads and meet at one barrier per chunk.
// Key groups merge their softmax states through LDS at the end.
//
// The running max is moved only when a row's new scores exceed it by more
// than kLazy (log2 units), so most chunks skip the rescale of the 128
// accumulators; probabilities are then at most 2^kLazy before normalisation,
// and the final division uses the same reference, so the result is unchanged.
constexpr int kCK = 32;
constexpr float kLazy = 8.f;

// ---------------------------------------------------------------- balanced splits
//
// In a batch whose requests differ in length, one split size for all leaves
// the longest request's workgroups running alone at the end, each with one or
// two chunks in flight.  A balanced plan (batches of at most 64 requests)
// sizes each request's splits instead, from the sizes in device memory, which
// every workgroup of the attention kernel reads and turns into the same plan:
//   - request b of c_b 32-key chunks, for a budget of q chunks, gets
//     min(NS, ceil(c_b / q)) splits of kc_b = ceil(c_b / splits) chunks each
//     (then as many splits as that size needs, so none is empty), and kv
//     heads x row blocks x splits workgroups (items);
//   - q is the smallest budget (at least two chunks) whose items fit in
//     `target` workgroups, the ones the chip holds at once: the longest item
//     is as short as it can be without a second round of workgroups; when no
//     budget fits, no request is split;
//   - the workgroups of a request's first split and first kv head record the
//     split count of each of its nodes (ws_ns), which the merge reads;
//   - a unit is one (kv head, split) of a request; its row blocks read the
//     same keys.
// Lane i of a wavefront holds request i.  A request that fails the size
// checks gets one chunk and one row block per head (its workgroups report it).
struct BalLane {
  int lo, n, P, ok;  // the request's node offset, nodes, prefix and size check
  int rb, ns, kc;    // row blocks, splits, chunks per split
};

__device__ inline BalLane balanced_lane(const AttnArgs& a, int lane) {
  const int i = min(lane, a.B - 1);
  const int lo = a.node_off[i], hi = a.node_off[i + 1], P = a.prefix_len[i];
  BalLane r;
  r.lo = lo;
  r.n = hi - lo;
  r.P = P;
  r.ok = (lo >= 0) & (hi <= a.T) & (r.n >= 1) & (r.n <= a.max_nodes) & (P >= 0) &
         (P <= a.max_prefix) & (P + r.n <= a.S_max);
  const int c = r.ok ? (P + r.n + kCK - 1) / kCK : 1;
  r.rb = r.ok ? (r.n * a.G + a.RB - 1) / a.RB : 1;
  const int hr = lane < a.B ? a.Hkv * r.rb : 0;  // workgroups of one split of the request
  // The smallest budget q in [2, cmax] whose items fit in `target`
  // workgroups (cmax: the chunks of the longest possible request, so every
  // request is one split at q = cmax).  With W = sum of hr * c and H = sum of
  // hr, the items at q are at most W / q + H, so q = W / (target - H) fits
  // when H < target; they are at least W / q unless the cap NS binds, so the
  // search starts at W / target (where the cap binds, a larger q than the
  // smallest that fits may result; every q it picks fits).  The items only fall as
  // q grows: the 64 lanes test 64 budgets spread over the range at once and
  // the first that fits narrows it, until the budgets are consecutive (one
  // round when the range holds at most 64).  The search counts min(NS,
  // ceil(c / q)) splits a request, at least the final count below.  Nothing
  // fits at cmax: no request is split.
  // Request j's sizes are read from lane j four requests at a time, without
  // branches (lanes past B have hr = 0 and B <= 64, so j + 3 <= 63).
  long W = 0;
  int H = 0;
  for (int j = 0; j < a.B; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int hj = __builtin_amdgcn_readlane(hr, j + u);
      W += (long)hj * __builtin_amdgcn_readlane(c, j + u);
      H += hj;
    }
  }
  // (bounds in double precision: W and the quotients are exact there to well
  // past any size here; the upper bound gets one chunk of margin)
  const int cm = max(2, a.cmax);
  const double Wd = (double)W;
  int qlo = (int)fmin((double)cm, fmax(2.0, ceil(Wd / a.target)));
  int qhi = H < a.target ? (int)fmin((double)cm, fmax((double)qlo, ceil(Wd / (a.target - H)) + 1.0))
                         : cm;
  int q = cm;
  while (true) {
    const int step = (qhi - qlo + 62) / 63;  // lanes 0..63 reach qhi
    const int qj = lane == 63 ? qhi : min(qlo + lane * max(step, 1), qhi);
    const unsigned uq = (unsigned)qj;
    int items = 0;
    for (int j = 0; j < a.B; j += 4) {
      int part[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // c >= 1: a request within q chunks counts one
        const unsigned cj = (unsigned)__builtin_amdgcn_readlane(c, j + u);
        part[u] = __builtin_amdgcn_readlane(hr, j + u) * min(a.NS, (int)((cj + uq - 1u) / uq));
      }
      items += (part[0] + part[1]) + (part[2] + part[3]);
    }
    const uint64_t fit = __ballot(items <= a.target);
    if (!fit) break;  // only when the range ends at cmax
    const int jf = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)fit) - 1);
    q = __builtin_amdgcn_readlane(qj, jf);
    if (step <= 1 || jf == 0) break;
    qlo = __builtin_amdgcn_readlane(qj, jf - 1) + 1;
    qhi = q;
  }
  const int ns0 = q >= c ? 1 : min(a.NS, (c + q - 1) / q);
  r.kc = (c + ns0 - 1) / ns0;
  r.ns = (c + r.kc - 1) / r.kc;
  return r;
}

// The grid of a balanced plan: request b takes a run of workgroups [base,
// base + size), with its units padded to a multiple of 8: unit j = 8 * grp + x
// of the request sits at base + grp * 8 * rb + r * 8 + x for row block r.
// Workgroups go round-robin over the 8 XCDs (blockIdx % 8), so a request's
// units are dealt over the XCDs and the row blocks of one unit, which read
// the same keys, follow each other on one XCD (its L2 serves the second).
// Workgroups of a padding unit have no item.  The runs go longest item first
// (most chunks per split, then request order): workgroups are dispatched in
// index order and the later ones share a CU with an earlier one, whose
// first chunks their own queue behind, so the longest items start first.
__device__ inline void balanced_order(const AttnArgs& a, const BalLane& L, int lane, int& base,
                                      int& size, int& total) {
  const int units = lane < a.B ? a.Hkv * L.ns : 0;
  size = ((units + 7) & ~7) * L.rb;
  const int key = lane < a.B ? L.kc : -1;
  base = 0;
  total = 0;
  for (int j = 0; j < a.B; j += 4) {  // lanes past B have size 0 (B <= 64)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sj = __builtin_amdgcn_readlane(size, j + u);
      const int kj = __builtin_amdgcn_readlane(key, j + u);
      base += (kj > key || (kj == key && j + u < lane)) ? sj : 0;
      total += sj;
    }
  }
}

// The workgroup's item and its request's sizes; false for a workgroup with
// no item.  Uniform across the workgroup (every wavefront derives the same
// values).
__device__ inline bool locate_item(const AttnArgs& a, Item& it, ReqInfo& rq) {
  if (!a.balanced) {
    if (!decode_item(a, it)) return false;
    it.ks = a.KS;
    rq = request_info(a, it.b);
    return true;
  }
  const int lane = threadIdx.x & 63;
  const BalLane L = balanced_lane(a, lane);
  int base, size, total;
  balanced_order(a, L, lane, base, size, total);
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  const uint64_t hit = __ballot(lane < a.B && base <= bid && bid < base + size);
  const int b = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  const int rb = __builtin_amdgcn_readlane(L.rb, b);
  const int ns = __builtin_amdgcn_readlane(L.ns, b);
  const int local = bid - __builtin_amdgcn_readlane(base, b);
  const int grp = local / (8 * rb), rem = local - grp * 8 * rb;
  const int j = grp * 8 + (rem & 7);
  if (j >= a.Hkv * ns) return false;  // padding
  it.w = bid;
  it.b = b;
  it.rblk = rem >> 3;
  it.g = j / ns;
  it.split = j - it.g * ns;
  it.ks = __builtin_amdgcn_readlane(L.kc, b) * kCK;
  rq.lo = __builtin_amdgcn_readlane(L.lo, b);
  rq.n = __builtin_amdgcn_readlane(L.n, b);
  rq.P = __builtin_amdgcn_readlane(L.P, b);
  rq.ok = __builtin_amdgcn_readlane(L.ok, b) != 0;
  rq.key_end = rq.P + rq.n;
  rq.nsplit = ns;
  return true;
}

// Cross-lane reductions over the lane groups l, l^16, l^32, l^48, which hold
// the same query row: gfx950 permlane swaps exchange 16-lane rows in VALU.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_add(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// xor16_max and xor32_max of two values at once, in three swaps instead of
// four.  permlane16_swap(a, b) exchanges a's odd 16-lane rows with b's even
// ones, permlane32_swap(a, b) a's upper 32 lanes with b's lower ones.  With
// rows x0 = [a0 a1 a2 a3], x1 = [b0 b1 b2 b3]: the first swap and max give
// [a0|a1, b0|b1, a2|a3, b2|b3]; the 32-lane swap and max give [A, B, A, B]
// (A, B the maxima over all four rows); a last 16-lane swap spreads A over
// one register and B over the other.
__device__ __forceinline__ void xor_max_pair(float& x0, float& x1) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1),
                                                  false, false);
  const float v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  const float w = fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
  const auto r3 = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false,
                                                   false);
  x0 = __uint_as_float(r3[0]);
  x1 = __uint_as_float(r3[1]);
}

// Wait until at most n chunks (DPC loads each) of this wavefront are in flight.
template <int N, int DPC>
__device__ __forceinline__ void wait_chunks(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      ST_WAIT_VMCNT(N * DPC);
      return;
    }
    wait_chunks<N - 1, DPC>(n);
  } else {
    ST_WAIT_VMCNT(0);
  }
}

// This wavefront's share (row group rw of RWV) of the direct loads of one
// 32-key chunk starting at key kt; key rows past klast are clamped to it.  The
// chunk base is wave-uniform, each lane adds a 32-bit offset.
// Byte offsets of this lane's direct loads within a whole chunk (swizzled
// 16-byte pieces of its key rows), the same for every chunk: computed once,
// so a whole chunk's loads take a uniform base plus a fixed 32-bit offset and
// need no vector arithmetic.
template <int D, int RWV>
struct ChunkOff {
  static constexpr int CH = D / 8, RPI = 64 / CH, INST = kCK / RPI, PER = INST / RWV;
  uint32_t k[PER], v[PER];
  __device__ ChunkOff(int rw, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int inst = rw * PER + i;
      const int row = inst * RPI + lane / CH, pos = lane % CH;
      k[i] = 2u * (uint32_t)(row * D + 8 * (pos ^ kswz<D>(row)));
      v[i] = 2u * (uint32_t)(row * D + 8 * (pos ^ vswz<D>(row)));
    }
  }
};

// Byte offsets of this lane's LDS fragment reads within a stage's K and V
// tiles, the same for every chunk: K as the QK^T operand (key row r16, the
// lane group's 16-byte piece of each 32-dim k-step), V^T through the
// transposing read (key 4 grp + r16 / 4, one dims block per entry).  The
// reads of keys 16..31 are these plus 16 rows (both swizzles repeat within
// 16 rows), an immediate offset.
template <int D>
struct FragOff {
  static constexpr int NKS = D / 32, NDB = D / 16;
  static constexpr int ROW16 = 16 * D * 2;  // bytes of 16 key rows
  uint32_t k[NKS], v[NDB];
  __device__ FragOff(int r16, int grp) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      k[ks] = 2u * (uint32_t)(r16 * D + 8 * ((4 * ks + grp) ^ kswz<D>(r16)));
    const int jq = r16 >> 2, qq = r16 & 3, key1 = 4 * grp + jq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int ch = 2 * db + (qq >> 1), sub = 4 * (qq & 1);
      v[db] = 2u * (uint32_t)(key1 * D + 8 * (ch ^ vswz<D>(key1)) + sub);
    }
  }
};

// (PAGED: `phys` is the block that holds the chunk, looked up beforehand.)
template <int D, int RWV, bool PAGED>
__device__ __forceinline__ void chunk_dma(uint16_t* sK, uint16_t* sV, const AttnArgs& a,
                                          const Item& it, const uint16_t* kgp,
                                          const uint16_t* vgp, int kt, int klast, int rw,
                                          int lane, const ChunkOff<D, RWV>& off, int phys = 0) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass never runs this body
  constexpr int CH = D / 8, RPI = 64 / CH, INST = kCK / RPI, PER = INST / RWV;
  const uint16_t* kb =
      PAGED ? kv_block_row<uint16_t>(a, a.k, phys, it.g, kt, D) : kgp + (size_t)kt * D;
  const uint16_t* vb =
      PAGED ? kv_block_row<uint16_t>(a, a.v, phys, it.g, kt, D) : vgp + (size_t)kt * D;
  const int lim = klast - kt;
  if (lim >= kCK - 1) {  // a whole chunk: no row is clamped
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int inst = rw * PER + i;
      __builtin_amdgcn_global_load_lds((const char*)kb + off.k[i], ST_LDS_PTR(sK + inst * 512),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const char*)vb + off.v[i], ST_LDS_PTR(sV + inst * 512),
                                       16, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int inst = rw * PER + i;
    const int row = inst * RPI + lane / CH, pos = lane % CH;
    const uint32_t ro = (uint32_t)min(row, lim) * D;
    __builtin_amdgcn_global_load_lds(kb + (ro + 8 * (pos ^ kswz<D>(row))),
                                     ST_LDS_PTR(sK + inst * 512), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + (ro + 8 * (pos ^ vswz<D>(row))),
                                     ST_LDS_PTR(sV + inst * 512), 16, 0, 0);
  }
#endif
}

// One wavefront's work on one 32-key chunk for its RBW row blocks.
// NA <= RBW: the row blocks computed (the first NA; a wavefront whose later
// row blocks lie wholly past the request's rows leaves them untouched).
template <int D, int RBW, int NA = RBW>
__device__ __forceinline__ void chunk_compute(const uint16_t* sK, const uint16_t* sV,
                                              const FragOff<D>& fo,
                                              const uint64_t* sM, int kt, int P, int k1,
                                              float c, int r16, int grp,
                                              const bf16x8 (&qf)[RBW][D / 32],
                                              f32x4 (&acc)[RBW][D / 16], float (&m)[RBW],
                                              float (&l)[RBW]) {
  constexpr int NKS = D / 32, NDB = D / 16;
  u32x4 kf[2][NKS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[kb][ks] =
          *(const u32x4*)((const uint8_t*)sK + fo.k[ks] + kb * FragOff<D>::ROW16);
  f32x4 s[RBW][2];
#pragma unroll
  for (int rb = 0; rb < NA; ++rb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kf[kb][ks]), qf[rb][ks], s[rb][kb], 0, 0, 0);
    }
  if (kt + kCK > P || kt + kCK > k1) {  // the chunk reaches tree keys or the range end
    // bit o of win: key kt + o is visible to this lane's row; the shift
    // amounts are the same for the whole wavefront
    const int t0 = kt - P, nv = k1 - kt;
    const uint32_t in_range = nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
#pragma unroll
    for (int rb = 0; rb < NA; ++rb) {
      const uint64_t* mr = sM + (rb * 16 + r16) * 4;
      uint32_t win;
      if (t0 >= 0) {
        const int wi = t0 >> 6, sh = t0 & 63;
        const uint64_t lo = mr[wi], hi = wi < 3 ? mr[wi + 1] : 0ull;
        win = (uint32_t)((lo >> sh) | (sh ? hi << (64 - sh) : 0ull));
      } else {
        const int np = -t0;  // prefix keys at the start of the chunk
        win = np >= 32 ? 0xFFFFFFFFu : (uint32_t)(mr[0] << np) | ((1u << np) - 1u);
      }
      win &= in_range;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[rb][kb][j] = (win >> (16 * kb + 4 * grp + j)) & 1u ? s[rb][kb][j] : -INFINITY;
    }
  }
  // every row block's chunk maximum first, then one (rarely taken) branch
  // for the rescales, so that the row blocks' exponentials below form one
  // straight run of code that the scheduler can interleave with the MFMAs
  float mc[RBW];
  bool any = false;
#pragma unroll
  for (int rb = 0; rb < NA; ++rb) {  // the lane's eight scores, in max3 steps
    const float t1 = fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), s[rb][0][2]);
    const float t2 = fmaxf(fmaxf(s[rb][0][3], s[rb][1][0]), s[rb][1][1]);
    const float t3 = fmaxf(fmaxf(s[rb][1][2], s[rb][1][3]), t1);
    mc[rb] = fmaxf(t2, t3);
  }
#pragma unroll
  for (int rb = 0; rb < NA; rb += 2) {  // over the four lane groups of each row
    if (rb + 1 < NA) {
      xor_max_pair(mc[rb], mc[rb + 1]);
    } else {
      mc[rb] = xor16_max(mc[rb]);
      mc[rb] = xor32_max(mc[rb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NA; ++rb) {
    mc[rb] *= c;  // c > 0: the max of the scaled scores
    any |= mc[rb] > m[rb] + kLazy;
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int rb = 0; rb < NA; ++rb) {
      const bool need = mc[rb] > m[rb] + kLazy;
      const float alpha = need ? fast_exp2(m[rb] - mc[rb]) : 1.f;
      m[rb] = need ? mc[rb] : m[rb];
      l[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[rb][db] *= alpha;
    }
  }
  bf16x8 pb[RBW];
#pragma unroll
  for (int rb = 0; rb < NA; ++rb) {
    const float nm = m[rb] == -INFINITY ? 0.f : -m[rb];
    float ps;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(fmaf(s[rb][kb][j], c, nm));
        pb[rb][4 * kb + j] = (__bf16)p;
        ps = kb == 0 && j == 0 ? p : ps + p;
      }
    l[rb] += ps;
  }
  // V^T fragments, four dims blocks (eight transposed reads) at a time
  const uint32_t vb = lds_addr(sV);
#pragma unroll
  for (int d0 = 0; d0 < NDB; d0 += 4) {
    uint32_t ad[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = vb + fo.v[d0 + i];
    u32x2 t[8];
    ds_read_tr16_x8<FragOff<D>::ROW16>(ad, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(t[2 * i], t[2 * i + 1], 0, 1, 2, 3));
#pragma unroll
      for (int rb = 0; rb < NA; ++rb)
        acc[rb][d0 + i] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[rb], acc[rb][d0 + i], 0, 0, 0);
    }
  }
}

// Normalise and store one row's output (16 dims per MFMA block, 4 per lane
// group) and its log-sum-exp.
template <int D>
__device__ __forceinline__ void write_row_out(const AttnArgs& a, int grow, int grp, float m,
                                              float l, const f32x4 (&acc)[D / 16]) {
  const float inv = 1.f / l;
  uint16_t* op = (uint16_t*)a.out + (size_t)grow * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    uint2 o;
    o.x = (uint32_t)st::f32_to_bf16_rne(acc[db][0] * inv) |
          ((uint32_t)st::f32_to_bf16_rne(acc[db][1] * inv) << 16);
    o.y = (uint32_t)st::f32_to_bf16_rne(acc[db][2] * inv) |
          ((uint32_t)st::f32_to_bf16_rne(acc[db][3] * inv) << 16);
    *(uint2*)(op + 16 * db + 4 * grp) = o;
  }
  if (a.lse && grp == 0) a.lse[grow] = (m + log2f(l)) * kLn2;
}

// RWV row groups of RBW 16-row blocks; KWV = 4 / RWV key groups; MINB
// workgroups per CU (two let one workgroup's softmax run while the other's
// MFMAs do).
template <int D, int NSTAGE, int RWV, int RBW, int MINB = 1, bool PAGED = false>
__global__ void __launch_bounds__(256, MINB)
attn_stream_kernel(AttnArgs a) {
  constexpr int KWV = 4 / RWV;
  constexpr bool PRIVATE = RWV == 1;                  // every wavefront owns its ring
  constexpr bool QLDS = RWV == 1;                     // Q staged in LDS once for all key groups
  constexpr int NKS = D / 32, NDB = D / 16, CH = D / 8;
  constexpr int WROWS = 16 * RBW, ROWS = WROWS * RWV;
  constexpr int STAGE = 2 * kCK * D;                  // bf16 elements: K then V
  constexpr int DPC = 2 * (kCK * CH / 64) / RWV;      // direct loads per chunk and wavefront
  constexpr int PRIME = PRIVATE ? NSTAGE : NSTAGE - 1; // chunks in flight when the loop starts
  constexpr int RING_BYTES = KWV * NSTAGE * STAGE * 2;
  constexpr int SLOT = (NDB * 4 + 2) * 64;            // floats: one row block of one wave
  constexpr int MERGE_BYTES = KWV > 1 ? RWV * RBW * KWV * SLOT * 4 : 0;
  constexpr int BODY = RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES;
  constexpr int QBYTES = QLDS ? ROWS * D * 2 : 0;
  constexpr int MWORDS = ROWS * 4;
  constexpr int MPT = (MWORDS + 255) / 256;           // mask words per thread
  static_assert(DPC * PRIME <= 63, "in-flight loads exceed the vmcnt range");
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[BODY + QBYTES + MWORDS * 8 + ST_MAX_NODES * 4 + 64];
  uint16_t* sQ = (uint16_t*)(lds + BODY);
  uint64_t* sMask = (uint64_t*)(lds + BODY + QBYTES);
  int* sPar = (int*)(sMask + MWORDS);

  // the wavefront index is uniform: keep it (and all that derives from it) scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave % RWV, kg = wave / RWV;
  const int r16 = lane & 15, grp = lane >> 4;
  // (the argmax reduction's words follow the parent array, in the same LDS
  // object: a second LDS object would cost the ring's prefetch, as the
  // compiler then waits for every direct load before each LDS read)
  int* am_scratch = sPar + ST_MAX_NODES;
  // A vocab argmax slice (the one-call step), one for each workgroup of the
  // grid below the slice count, with an item or without: loaded after the
  // ring's first chunks and reduced after the loop, so that neither its loads
  // nor its reduction delay the first chunk's compute.
  const int au = blockIdx.x;
  const bool am = a.am.logits != nullptr && au < a.am.units;
  st::ArgmaxRegs amr;
  uint16_t* ring = (uint16_t*)lds + kg * NSTAGE * STAGE;
  const ChunkOff<D, RWV> coff(rw, lane);
  // The item and its request's sizes, waited for alone: every later address
  // depends on them.  (Loads issued behind the first chunks' direct loads,
  // 16 KB a wavefront all over the chip, wait for all of them.)  Contiguous
  // caches under one split size: the key group's first chunk depends on the
  // workgroup index alone, so its direct loads go out while the sizes are on
  // their way (issued after the sizes' scalar loads; rows below the cache
  // capacity, so in bounds whatever the sizes).  It is kept if all 32 of its
  // keys belong to the split, else waited for and loaded again clamped.
  Item it;
  ReqInfo rq;
  bool located, spec = false;
  // paged pool: the raw table entries of the first chunks (a chunk's key
  // depends on the split alone; the index is clamped into the table row, and
  // an entry is checked where it is used, for a chunk inside the request's
  // keys), loaded beside the sizes when the item is known without them
  int e_first[PRIME];
  auto first_entries = [&]() {
#pragma unroll
    for (int s = 0; s < PRIME; ++s)
      e_first[s] = PAGED ? a.pg.bt[(size_t)it.b * a.pg.bt_stride +
                                   min((it.split * it.ks + (s * KWV + kg) * kCK) >> a.pg.lbs,
                                       a.pg.bt_stride - 1)]
                         : 0;
  };
  if (!a.balanced) {
    located = decode_item(a, it);
    ReqWords w{0, 0, 0};
    if (located) {
      it.ks = a.KS;
      w = request_load(a, it.b);
      first_entries();
      __builtin_amdgcn_sched_barrier(0);  // both sets of loads issued before either wait
      const int kt0 = it.split * a.KS + kg * kCK;
      if (!PAGED && kg * kCK < a.KS && kt0 + kCK <= a.S_max) {
        const size_t ho = ((size_t)it.b * a.Hkv + it.g) * (size_t)a.S_max * D;
        chunk_dma<D, RWV, false>(ring, ring + kCK * D, a, it, (const uint16_t*)a.k + ho,
                                 (const uint16_t*)a.v + ho, kt0, kt0 + kCK - 1, rw, lane, coff);
        spec = true;
      }
      rq = request_finish(a, w);
    }
  } else {
    located = locate_item(a, it, rq);
    if (located) first_entries();
  }
  if (!located) {
    if (am) {
      st::argmax_slice_load<true>(a.am.logits, a.am.V, au / a.am.nslices, au % a.am.nslices, amr);
      argmax_unit_finish(a, au, amr, am_scratch);
    }
    return;
  }
  const int k0 = it.split * it.ks;
  // contiguous caches: the (request, head) base, fixed for the workgroup
  const size_t head_off = ((size_t)it.b * a.Hkv + it.g) * (size_t)a.S_max * D;
  const uint16_t* kgp = (const uint16_t*)a.k + head_off;
  const uint16_t* vgp = (const uint16_t*)a.v + head_off;

  const int rows_b = rq.n * a.G;
  const int row0 = it.rblk * ROWS;
  if (!rq.ok || row0 >= rows_b || k0 >= rq.key_end) {
    if (spec) ST_WAIT_VMCNT(0);
    if (!rq.ok && threadIdx.x == 0 && it.g == 0 && it.split == 0 && it.rblk == 0)
      st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    if (am) {
      st::argmax_slice_load<true>(a.am.logits, a.am.V, au / a.am.nslices, au % a.am.nslices, amr);
      argmax_unit_finish(a, au, amr, am_scratch);
    }
    return;
  }
  const int k1 = min(k0 + it.ks, rq.key_end);
  const int klast = k1 - 1;
  const int wrow0 = row0 + rw * WROWS;
  const int nch = (k1 - k0 + kCK - 1) / kCK;
  const int nmine = (nch - kg + KWV - 1) / KWV;  // chunks kg, kg + KWV, ...
  const int niter = (nch + KWV - 1) / KWV;       // the same for every wavefront
  const int want = min(PRIME, nmine);
  const FragOff<D> fo(r16, grp);
  // paged pool: the block of each chunk is looked up one refill ahead
  auto entry = [&](int c) { return PAGED ? table_entry(a, it.b, k0 + c * kCK) : 0; };

  // Q of the workgroup's rows (rows past the end repeat the last): staged in
  // LDS once when several key groups share the rows, else loaded directly.
  bf16x8 qf[RBW][NKS];
  if constexpr (QLDS) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int RPI = 64 / CH, QI = ROWS * CH / 64;
    for (int i = wave; i < QI; i += 4) {
      const int row = i * RPI + lane / CH, pos = lane % CH;
      const int rr = min(row0 + row, rows_b - 1);
      const uint16_t* src = (const uint16_t*)a.q +
                            ((size_t)(rq.lo + rr / a.G) * a.Hq + it.g * a.G + rr % a.G) * D +
                            8 * (pos ^ kswz<D>(row));
      __builtin_amdgcn_global_load_lds(src, ST_LDS_PTR(sQ + i * 512), 16, 0, 0);
    }
#endif
  } else {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const int row = min(wrow0 + rb * 16 + r16, rows_b - 1);
      const int node = row / a.G, hq = it.g * a.G + row % a.G;
      const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(rq.lo + node) * a.Hq + hq) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[rb][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 32 * ks + 8 * grp));
    }
  }

  // Ancestor masks are needed only when the key range reaches tree keys: the
  // workgroup's rows of `mask`, or (mask == null) the request's parent array,
  // from which they are derived below, copied straight to LDS (clamped
  // addresses; words past the tree's W are cleared after the copy).  Direct
  // loads like the ring's, so that the waits for the ring cover them too.
  const bool need_mask = k1 > rq.P;
  const bool derive = a.mask == nullptr;
  if (need_mask) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (derive) {
      if (wave * 64 < rq.n) {
        const int32_t* src = a.parent + rq.lo + min(tid, rq.n - 1);
        __builtin_amdgcn_global_load_lds(src, ST_LDS_PTR(sPar + wave * 64), 4, 0, 0);
      }
    } else {
      for (int i = wave; i < 2 * MWORDS / 64; i += 4) {  // 32-bit halves of mask words
        const int j = i * 64 + lane, idx = j >> 1;
        const int row = min(row0 + idx / 4, rows_b - 1), w = min(idx % 4, a.W - 1);
        const uint32_t* src =
            (const uint32_t*)(a.mask + (size_t)(rq.lo + row / a.G) * a.W + w) + (j & 1);
        __builtin_amdgcn_global_load_lds(src, ST_LDS_PTR((uint32_t*)sMask + i * 64), 4, 0, 0);
      }
    }
#endif
  }
  // the speculative first chunk stands if it holds 32 keys of the split
  const bool spec_ok = spec && nmine > 0 && klast - (k0 + kg * kCK) >= kCK - 1;
  if (spec && !spec_ok) ST_WAIT_VMCNT(0);  // landed before its stage is loaded again
  if (nmine > 0 && !spec_ok)
    chunk_dma<D, RWV, PAGED>(ring, ring + kCK * D, a, it, kgp, vgp, k0 + kg * kCK, klast, rw,
                             lane, coff, PAGED ? table_phys(a, e_first[0]) : 0);
#pragma unroll
  for (int s = 1; s < PRIME; ++s)
    if (s < nmine)
      chunk_dma<D, RWV, PAGED>(ring + s * STAGE, ring + s * STAGE + kCK * D, a, it, kgp, vgp,
                               k0 + (s * KWV + kg) * kCK, klast, rw, lane, coff,
                               PAGED ? table_phys(a, e_first[s]) : 0);
  wait_chunks<PRIME - 1, DPC>(want - 1);  // the first chunk, Q and the masks are older
  if (am)
    st::argmax_slice_load<true>(a.am.logits, a.am.V, au / a.am.nslices, au % a.am.nslices, amr);
  if (need_mask) {
    if (derive) {
      lds_barrier_inflight();  // every wavefront's share of the parent array has landed
      if (tid < ROWS) {
        const int row = row0 + tid;
        uint64_t w0 = 0ull, w1 = 0ull, w2 = 0ull, w3 = 0ull;
        if (row < rows_b && !ancestor_words(sPar, row / a.G, w0, w1, w2, w3))
          st::set_status(a.status, ST_STATUS_BAD_PARENT);
        sMask[tid * 4 + 0] = w0;
        sMask[tid * 4 + 1] = w1;
        sMask[tid * 4 + 2] = w2;
        sMask[tid * 4 + 3] = w3;
      }
    } else {
      // words past the tree's W and rows past the request are cleared, each
      // by the wavefront that copied it (its own copies have landed)
      for (int i = wave; i < 2 * MWORDS / 64; i += 4) {
        const int j = i * 64 + lane, idx = j >> 1;
        if (row0 + idx / 4 >= rows_b || idx % 4 >= a.W) ((uint32_t*)sMask)[j] = 0u;
      }
    }
  }
  lds_barrier_inflight();  // Q (when staged) and the masks are in LDS
  if constexpr (QLDS) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const int r = rb * 16 + r16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[rb][ks] = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(sQ + r * D + 8 * ((4 * ks + grp) ^ kswz<D>(r))));
    }
  }

  f32x4 acc[RBW][NDB];
  float m[RBW], l[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint64_t* sMw = sMask + rw * WROWS * 4;
  if constexpr (PRIVATE) {
    // A ring of one's own: compute chunk r, then refill its stage with chunk
    // r + NSTAGE; no other wavefront reads it, so no barrier is needed.
    int stage = 0;
    int next = NSTAGE < nmine ? entry(NSTAGE * KWV + kg) : 0;  // block of the next refill
    for (int r = 0; r < nmine; ++r) {
      wait_chunks<NSTAGE - 1, DPC>(min(NSTAGE - 1, nmine - r - 1));
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* sK = ring + stage * STAGE;
      chunk_compute<D, RBW>(sK, sK + kCK * D, fo, sMw, k0 + (r * KWV + kg) * kCK, rq.P, k1,
                            a.scale_log2, r16, grp, qf, acc, m, l);
      __builtin_amdgcn_sched_barrier(0);
      if (r + NSTAGE < nmine) {
        uint16_t* sb = ring + stage * STAGE;
        chunk_dma<D, RWV, PAGED>(sb, sb + kCK * D, a, it, kgp, vgp,
                                 k0 + ((r + NSTAGE) * KWV + kg) * kCK, klast, rw, lane, coff,
                                 next);
        if (PAGED && r + NSTAGE + 1 < nmine) next = entry((r + NSTAGE + 1) * KWV + kg);
      }
      __builtin_amdgcn_sched_barrier(0);
      stage = stage + 1 == NSTAGE ? 0 : stage + 1;
    }
  } else {
    // A ring shared by the row groups of a key group: at the top of round r
    // (after the barrier, so every row group is done with chunk r - 1) refill
    // the stage chunk r - 1 used with chunk r + NSTAGE - 1.  A row group
    // computes only its row blocks that hold rows of the request (all, half
    // or none of them); it still loads its share of every chunk.
    // (one instance of the loop for each count, chosen outside it)
    auto shared_loop = [&](auto na) {
      constexpr int NA = decltype(na)::value;
      int stage = 0, refill = NSTAGE - 1;
      int next = NSTAGE - 1 < nmine ? entry((NSTAGE - 1) * KWV + kg) : 0;  // next refill's block
      for (int r = 0; r < niter; ++r) {
        wait_chunks<NSTAGE - 2, DPC>(min(NSTAGE - 2, nmine - r - 1));
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (r + NSTAGE - 1 < nmine) {
          uint16_t* sb = ring + refill * STAGE;
          chunk_dma<D, RWV, PAGED>(sb, sb + kCK * D, a, it, kgp, vgp,
                                   k0 + ((r + NSTAGE - 1) * KWV + kg) * kCK, klast, rw, lane,
                                   coff, next);
          if (PAGED && r + NSTAGE < nmine) next = entry((r + NSTAGE) * KWV + kg);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (NA > 0 && r < nmine) {
          const uint16_t* sK = ring + stage * STAGE;
          chunk_compute<D, RBW, (NA > 0 ? NA : 1)>(sK, sK + kCK * D, fo, sMw,
                                                   k0 + (r * KWV + kg) * kCK, rq.P, k1,
                                                   a.scale_log2, r16, grp, qf, acc, m, l);
        }
        __builtin_amdgcn_sched_barrier(0);
        stage = stage + 1 == NSTAGE ? 0 : stage + 1;
        refill = refill + 1 == NSTAGE ? 0 : refill + 1;
      }
    };
    const int nact = min(max((rows_b - wrow0 + 15) / 16, 0), RBW);
    if (nact > RBW / 2) shared_loop(std::integral_constant<int, RBW>{});
    else if (nact > 0) shared_loop(std::integral_constant<int, (RBW > 1 ? RBW / 2 : RBW)>{});
    else shared_loop(std::integral_constant<int, 0>{});
  }
  if (am) argmax_unit_finish(a, au, amr, am_scratch);
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    l[rb] = xor16_add(l[rb]);
    l[rb] = xor32_add(l[rb]);
  }

  // row block rb of a row group is finalised by key group owner(rb)
  auto owner = [](int rb) { return RBW >= KWV ? rb * KWV / RBW : rb; };
  if constexpr (KWV > 1) {
    float* mb = (float*)lds;
    lds_barrier();  // every ring is idle
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      if (owner(rb) != kg) {
        float* sl = mb + ((rw * RBW + rb) * KWV + kg) * SLOT;
#pragma unroll
        for (int db = 0; db < NDB; ++db) *(f32x4*)(sl + (db * 64 + lane) * 4) = acc[rb][db];
        sl[NDB * 256 + lane] = m[rb];
        sl[NDB * 256 + 64 + lane] = l[rb];
      }
    }
    lds_barrier();
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      if (owner(rb) == kg) {
        float M = m[rb];
#pragma unroll
        for (int k = 0; k < KWV; ++k)
          if (k != kg) M = fmaxf(M, mb[((rw * RBW + rb) * KWV + k) * SLOT + NDB * 256 + lane]);
        const float ref = M == -INFINITY ? 0.f : M;
        const float w0 = fast_exp2(m[rb] - ref);
        l[rb] *= w0;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[rb][db] *= w0;
#pragma unroll
        for (int k = 0; k < KWV; ++k) {
          if (k != kg) {
            const float* sl = mb + ((rw * RBW + rb) * KWV + k) * SLOT;
            const float wk = fast_exp2(sl[NDB * 256 + lane] - ref);
            l[rb] += wk * sl[NDB * 256 + 64 + lane];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              acc[rb][db] += wk * *(const f32x4*)(sl + (db * 64 + lane) * 4);
          }
        }
        m[rb] = M;
      }
    }
  }

  const size_t TH = (size_t)a.T * a.Hq;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    if (owner(rb) != kg) continue;
    const int row = wrow0 + rb * 16 + r16;
    if (row >= rows_b) continue;
    const int grow = (rq.lo + row / a.G) * a.Hq + it.g * a.G + row % a.G;
    if (rq.nsplit == 1) {
      write_row_out<D>(a, grow, grp, m[rb], l[rb], acc[rb]);
    } else {
      const size_t pr = (size_t)it.split * TH + grow;
      float* wp = a.ws_acc + pr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *(f32x4*)(wp + 16 * db + 4 * grp) = acc[rb][db];
      if (grp == 0) a.ws_ml[pr] = make_float2(m[rb], l[rb]);
    }
  }
  // balanced plans: the split count of each node of the row block, for the
  // merge (once per node: first split, first kv head, the node's first row)
  if (a.balanced && it.split == 0 && it.g == 0 && tid < ROWS) {
    const int row = row0 + tid;
    if (row < rows_b && row % a.G == 0) a.ws_ns[rq.lo + row / a.G] = rq.nsplit;
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
  ReqInfo rq;
  if (!locate_item(a, it, rq)) return;
  if (!rq.ok) {
    if (threadIdx.x == 0 && it.g == 0 && it.split == 0 && it.rblk == 0)
      st::set_status(a.status, ST_STATUS_BAD_PREFIX);
    return;
  }
  const int rows_b = rq.n * a.G;
  if (it.rblk * R >= rows_b) return;
  const int k0 = it.split * it.ks;
  if (k0 >= rq.key_end) return;
  const int k1 = min(k0 + it.ks, rq.key_end);

  const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
  const int row = it.rblk * R + r;
  const bool row_ok = row < rows_b;
  const int node = row_ok ? row / a.G : 0;
  const int hq = it.g * a.G + (row_ok ? row % a.G : 0);
  const int grow = (rq.lo + node) * a.Hq + hq;

  // the first K/V tile's loads go out before Q and the masks are read
  static_assert(sizeof(Tin) == 4, "the VALU kernel serves fp32 inputs");
  constexpr int V4 = D / 4, LPT = KT * V4 / 256;  // 16-byte loads per thread and tile
  f32x4 rk[LPT], rv[LPT];
  auto load_tile = [&](int kt) {
    const int nk = min(KT, k1 - kt);
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int e = tid + 256 * j, kr = e / V4, d4 = 4 * (e % V4);
      const bool ok = kr < nk;
      rk[j] = ok ? *(const f32x4*)(kv_row<Tin>(a, a.k, it.b, it.g, kt + kr, D) + d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
      rv[j] = ok ? *(const f32x4*)(kv_row<Tin>(a, a.v, it.b, it.g, kt + kr, D) + d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_tile(k0);

  const Tin* qp = (const Tin*)a.q + (size_t)grow * D;
  for (int d = c; d < D; d += 16) sQ[r][d] = row_ok ? load_val(qp + d) : 0.f;
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  if (a.mask) {
    if (row_ok) {
      const uint64_t* mr = a.mask + (size_t)(rq.lo + node) * a.W;
      mw0 = mr[0];
      if (a.W > 1) mw1 = mr[1];
      if (a.W > 2) mw2 = mr[2];
      if (a.W > 3) mw3 = mr[3];
    }
  } else {  // derive the row's ancestor mask from the request's parent array
    __shared__ int sPar[ST_MAX_NODES];
    __shared__ uint64_t sRow[R][4];
    for (int i = tid; i < rq.n; i += 256) sPar[i] = a.parent[rq.lo + i];
    __syncthreads();
    if (c == 0) {
      uint64_t w0 = 0ull, w1 = 0ull, w2 = 0ull, w3 = 0ull;
      if (row_ok && !ancestor_words(sPar, node, w0, w1, w2, w3))
        st::set_status(a.status, ST_STATUS_BAD_PARENT);
      sRow[r][0] = w0;
      sRow[r][1] = w1;
      sRow[r][2] = w2;
      sRow[r][3] = w3;
    }
    __syncthreads();
    mw0 = sRow[r][0];
    mw1 = sRow[r][1];
    mw2 = sRow[r][2];
    mw3 = sRow[r][3];
  }

  float acc[DJ];
#pragma unroll
  for (int j = 0; j < DJ; ++j) acc[j] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  for (int kt = k0; kt < k1; kt += KT) {
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int e = tid + 256 * j, kr = e / V4, d4 = 4 * (e % V4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sK[kr][d4 + q] = rk[j][q];
        sV[kr][d4 + q] = rv[j][q];
      }
    }
    __syncthreads();
    if (kt + KT < k1) load_tile(kt + KT);  // in flight while this tile is computed
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
// partial outputs of up to 8 splits are all loaded before any is used.  Block
// `blk` covers 256 / (D/4) consecutive rows.
template <typename Tout, int D, int CHUNK>
__device__ inline void combine_block_n(const AttnArgs& a, int blk) {
  constexpr int LPR = D / 4;        // lanes per row, 4 dims each
  constexpr int RPB = 256 / LPR;    // rows per block
  const int grow = blk * RPB + threadIdx.x / LPR;
  const int d = 4 * (threadIdx.x % LPR);
  const int TH = a.T * a.Hq;
  if (grow >= TH) return;
  // Every row has a.NS partial slots.  With one request the first CHUNK
  // splits' loads go out before its split count is known; in a batch, where
  // short requests have fewer splits (or one, and no partials at all), the
  // row's request is looked up first and only its splits are read.
  float2 ml[CHUNK];
  f32x4 x[CHUNK];
  const bool single = a.B == 1;
  if (single) {
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      const size_t pr = (size_t)min(j, a.NS - 1) * TH + grow;
      ml[j] = a.ws_ml[pr];
      x[j] = *(const f32x4*)(a.ws_acc + pr * D + d);
    }
  }
  const int t = grow / a.Hq;
  int ns;
  if (a.balanced) {
    // recorded by the attention kernel for every node of a request that
    // passed its checks (a failed one's is stale; clamped, its reads stay in
    // the workspace)
    ns = min(max(a.ws_ns[t], 0), a.NS);
  } else {
    const int b = st::request_of(a.node_off, a.B, t);
    const ReqInfo rq = request_info(a, b);
    ns = rq.ok ? rq.nsplit : 0;
  }
  if (ns <= 1) return;
  if (!single) {
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      const size_t pr = (size_t)min(j, ns - 1) * TH + grow;
      ml[j] = a.ws_ml[pr];
      x[j] = *(const f32x4*)(a.ws_acc + pr * D + d);
    }
  }
  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += CHUNK) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < CHUNK; ++j) {
        const int s = min(s0 + j, ns - 1);
        const size_t pr = (size_t)s * TH + grow;
        ml[j] = a.ws_ml[pr];
        x[j] = *(const f32x4*)(a.ws_acc + pr * D + d);
      }
    }
    float Mc = M;
#pragma unroll
    for (int j = 0; j < CHUNK; ++j)
      if (s0 + j < ns) Mc = fmaxf(Mc, ml[j].x);
    const float ref = Mc == -INFINITY ? 0.f : Mc;
    const float sc = fast_exp2(M - ref);  // rescale what is merged so far
    L *= sc;
    o *= sc;
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      if (s0 + j < ns) {
        const float w = fast_exp2(ml[j].x - ref);  // empty split: exp2(-inf) = 0
        L += w * ml[j].y;
        o += w * x[j];
      }
    }
    M = Mc;
  }
  const float inv = 1.f / L;
  Tout* op = (Tout*)a.out + (size_t)grow * D + d;
  if constexpr (sizeof(Tout) == 2) {  // bf16: the lane's four dims in one 8-byte store
    uint2 w;
    w.x = (uint32_t)st::f32_to_bf16_rne(o[0] * inv) |
          ((uint32_t)st::f32_to_bf16_rne(o[1] * inv) << 16);
    w.y = (uint32_t)st::f32_to_bf16_rne(o[2] * inv) |
          ((uint32_t)st::f32_to_bf16_rne(o[3] * inv) << 16);
    *(uint2*)op = w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) store_val(op + j, o[j] * inv);
  }
  if (a.lse && d == 0) a.lse[grow] = (M + log2f(L)) * kLn2;
}

// Splits loaded before the first use: as many as a request can have, up to 8.
template <typename Tout, int D>
__device__ inline void combine_block(const AttnArgs& a, int blk) {
  if (a.NS <= 4) combine_block_n<Tout, D, 4>(a, blk);
  else combine_block_n<Tout, D, 8>(a, blk);
}

template <typename Tout, int D>
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnArgs a) {
  combine_block<Tout, D>(a, blockIdx.x);
}

// The compaction of the accepted paths (the first B * 2 * Hkv blocks: one per
// request and cache head, each walking its request's tree first) and, in the
// same launch, the merge of the splits (the blocks after them).  The walks
// are latency-bound chains, so they are dispatched first and run beside the
// merge.  The attention kernel has finished reading the tree slots when this
// starts, and the two parts touch disjoint memory.
template <typename Tout, int D>
__global__ void __launch_bounds__(256)
attn_combine_compact_kernel(AttnArgs a, st::CompactArgs c, int n_combine) {
  const int blk = blockIdx.x;
  const int n_compact = c.B * 2 * c.Hkv;
  if (blk < n_compact) {
    st::kv_compact_block(c, blk / (2 * c.Hkv), blk % (2 * c.Hkv));
  } else {
    combine_block<Tout, D>(a, blk - n_compact);
  }
  (void)n_combine;
}

// ---------------------------------------------------------------- planning

struct Plan {
  bool stream;  // bf16 streaming MFMA kernel (else fp32 VALU kernel + combine)
  int rwv, rbw; // streaming kernel: 64-row groups per workgroup, 16-row blocks per wave
  int RB, n_rblk, KS, NS, items, per_xcd;
  bool balanced;  // splits sized per request on the device
  int target;     // workgroups a split plan aims for
  size_t ml_bytes, ns_off, ws_bytes;
};

int make_plan(const st_tree* t, int Hq, int Hkv, int D, st_dtype dtype, int max_prefix, Plan& p) {
  const st::TestingPlan& ovr = st::testing_plan();
  int rc = st::check_tree_host(t);
  if (rc) return rc;
  if (Hq < 1 || Hkv < 1 || max_prefix < 0) return ST_E_INVALID;
  if (dtype != ST_F32 && dtype != ST_BF16) return ST_E_INVALID;
  if (Hq % Hkv || (D != 64 && D != 128)) return ST_E_UNSUPPORTED;
  const int G = Hq / Hkv;
  const long rows_max = (long)t->max_nodes * G;
  long gran = 16;  // split granularity in keys
  p.stream = dtype == ST_BF16;
  // Batches of 2..64 requests (bf16): splits sized per request on the device
  // (balanced_lane), from the sizes in device memory, so that the workgroups
  // of short and long requests stream about as many keys each.
  const int forced_ks = ovr.attn_split_keys;
  const int force_bal = ovr.attn_balance;
  // The planner's choice takes it only where a split can happen at all: one
  // workgroup per request and kv head must leave room under the workgroup
  // target of the shape it would run (below: (4,2), two per CU, above 64 rows
  // a kv head; one per CU up to 64).
  const long bal_target =
      ovr.attn_target_wg > 0 ? ovr.attn_target_wg : rows_max > 64 ? 512 : 256;
  const bool balanced =
      p.stream && t->B <= 64 && forced_ks == 0 &&
      (force_bal == 2 || (force_bal == 0 && t->B >= 2 && (long)t->B * Hkv < bal_target));
  if (!p.stream) {
    p.rwv = p.rbw = 0;
    p.RB = 16;
  } else {
    // Row groups: enough to hold every row of a kv head, so K and V are read
    // once per key range (at most 4); row blocks per wave: as many as the
    // rows need (a tree of 6 nodes uses one 16-row block, not four).  Up to
    // 64 rows, when the batch must be split over keys anyway to fill the
    // chip, two 32-row workgroups per kv head (the second reads K and V from
    // the L2 the first filled) halve the splits to merge and give each
    // wavefront twice the chunks, which evens out its chunk count.
    p.rwv = rows_max <= 64 ? 1 : rows_max <= 128 ? 2 : 4;
    p.rbw = rows_max <= 16 ? 1 : rows_max <= 32 ? 2 : 4;
    if (rows_max <= 64 && (long)t->B * Hkv * 2 <= 256) p.rbw = 2;
    // More than 64 rows a kv head: the MFMAs and the softmax of a chunk take
    // longer than its loads, so run two workgroups per CU (32 rows a
    // wavefront, half the registers), whose softmax and MFMA phases overlap.
    if (rows_max > 64) p.rbw = 2;
    // With splits sized per request (below), up to 128 rows a kv head go to
    // one workgroup of four row groups: (4,2) reads each key once, where (2,2)
    // needs two workgroups whose splits must run side by side, and its
    // one-key-group ring keeps three chunks in flight.
    if (balanced && rows_max > 64) p.rwv = 4;
    // 0..6: (1,1) (1,2) (1,4) (2,4) (4,4), then two workgroups per CU: (2,2) (4,2)
    const int forced = ovr.attn_shape;
    if (forced >= 0 && forced <= 6) {
      static const int kRwv[7] = {1, 1, 1, 2, 4, 2, 4}, kRbw[7] = {1, 2, 4, 4, 4, 2, 2};
      p.rwv = kRwv[forced];
      p.rbw = kRbw[forced];
    }
    p.RB = 16 * p.rbw * p.rwv;
    gran = 32;
  }
  p.n_rblk = (int)((rows_max + p.RB - 1) / p.RB);
  const long keys_max = (long)max_prefix + t->max_nodes;
  const long base = (long)t->B * Hkv * p.n_rblk;
  // aim for about `target` workgroups over the whole batch (one per CU for
  // the streaming kernel, two for its two-per-CU shapes); splits are even, in
  // multiples of `gran` keys
  const bool two_per_cu = p.stream && p.rbw == 2 && p.rwv > 1;
  const long target =
      ovr.attn_target_wg > 0 ? ovr.attn_target_wg : !p.stream ? 512 : two_per_cu ? 512 : 256;
  long ns = (target + base - 1) / base;
  if (ns < 1) ns = 1;
  long ks = (keys_max + ns - 1) / ns;
  ks = (ks + gran - 1) / gran * gran;
  if (forced_ks > 0) ks = (forced_ks + gran - 1) / gran * gran;
  const long kmax = (keys_max + gran - 1) / gran * gran;
  // the streaming kernel wants at least two chunks per wavefront; the fp32
  // kernel, whose tiles are not prefetched, is fastest with one tile a split
  if (ks < (p.stream ? 64 : gran)) ks = p.stream ? 64 : gran;
  if (ks > kmax) ks = kmax;
  p.KS = (int)ks;
  p.NS = (int)((keys_max + ks - 1) / ks);
  long items = base * p.NS;
  p.target = (int)target;
  // Balanced plans: NS becomes the most splits a request may take (the
  // uniform plan's count, at least 4, at most one per two chunks of the
  // longest request).  The grid bounds the device's layout: at most `target`
  // items when any request is split, else one per (request, head, row block),
  // plus each request's padding to a multiple of 8 units (none when the kv
  // heads are a multiple of 8).  Workgroups past the items run the plan and
  // exit, late in the launch: the bound is kept tight.
  p.balanced = balanced;
  if (p.balanced) {
    const long cap = (kmax / 32 + 1) / 2;
    p.NS = (int)std::max(1L, std::min(std::max((long)p.NS, 4L), cap));
    items = std::min(base * p.NS, std::max(target, base)) + (Hkv % 8 ? 7L * t->B * p.n_rblk : 0L);
    p.KS = 0;
  }
  if (items > (1L << 30)) return ST_E_UNSUPPORTED;
  p.items = (int)items;
  p.per_xcd = (p.items + 7) / 8;
  const size_t TH = (size_t)t->total_nodes * Hq;
  p.ml_bytes = p.NS > 1 ? st::align_up((size_t)p.NS * TH * sizeof(float2), 256) : 0;
  p.ws_bytes = p.NS > 1 ? p.ml_bytes + (size_t)p.NS * TH * D * sizeof(float) : 0;
  // balanced plans: the nodes' split counts after the partials
  p.ns_off = st::align_up(p.ws_bytes, 256);
  if (p.balanced) p.ws_bytes = p.ns_off + (size_t)t->total_nodes * sizeof(int32_t);
  return ST_OK;
}

}  // namespace

int st::attention_workgroups(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                             int max_prefix) {
  Plan p;
  if (make_plan(tree, Hq, Hkv, D, dtype, max_prefix, p)) return 0;
  return 8 * p.per_xcd;  // the grid: every workgroup can take an argmax slice
}

extern "C" size_t st_tree_attention_workspace(const st_tree* tree, int Hq, int Hkv, int D,
                                              st_dtype dtype, int max_prefix) {
  Plan p;
  if (make_plan(tree, Hq, Hkv, D, dtype, max_prefix, p)) return 0;
  return p.ws_bytes;
}

int st::tree_attention_impl(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                            float scale, const void* q, const void* k_cache, const void* v_cache,
                            int S_max, const int32_t* prefix_len, int max_prefix,
                            const uint64_t* mask, void* out, float* lse, void* workspace,
                            size_t ws_bytes, int32_t* status, void* stream,
                            const st::CompactArgs* compact, const st::ArgmaxJob* argmax,
                            const st::KvPaging* paging, const st::SideLaunch* side) {
  Plan p;
  int rc = make_plan(tree, Hq, Hkv, D, dtype, max_prefix, p);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !prefix_len || !out || S_max < 1 ||
      !(scale > 0.f) || !isfinite(scale))
    return ST_E_INVALID;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) % 16)
    return ST_E_INVALID;
  if (p.ws_bytes && (!workspace || ws_bytes < p.ws_bytes)) return ST_E_WORKSPACE;
  AttnArgs a;
  a.node_off = tree->node_off;
  a.parent = tree->parent;
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.lse = lse;
  a.ws_ml = p.ws_bytes ? (float2*)workspace : nullptr;
  a.ws_acc = p.ws_bytes ? (float*)((char*)workspace + p.ml_bytes) : nullptr;
  a.ws_ns = p.balanced ? (int32_t*)((char*)workspace + p.ns_off) : nullptr;
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
  a.balanced = p.balanced ? 1 : 0;
  a.target = p.target;
  a.cmax = (int)std::min<long>(((long)max_prefix + tree->max_nodes + kCK - 1) / kCK, 1L << 30);
  a.scale_log2 = scale * kLog2e;
  a.pg = paging ? *paging : st::KvPaging{nullptr, 0, 0, 0};
  a.am = st::ArgmaxJob{nullptr, nullptr, 0, 0, 0, nullptr};
  if (argmax && p.stream) a.am = *argmax;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(8 * p.per_xcd), block(256);
  if (p.stream) {
    const dim3 sblock(256);
    const int shape = p.rwv * 8 + p.rbw;
#define ST_LAUNCH_STREAM_P(RWV_, RBW_, NS128_, NS64_, MINB_, PG_)                              \
  if (shape == RWV_ * 8 + RBW_) {                                                              \
    if (D == 128)                                                                              \
      hipLaunchKernelGGL((attn_stream_kernel<128, NS128_, RWV_, RBW_, MINB_, PG_>), grid,      \
                         sblock, 0, s, a);                                                     \
    else                                                                                       \
      hipLaunchKernelGGL((attn_stream_kernel<64, NS64_, RWV_, RBW_, MINB_, PG_>), grid, sblock, \
                         0, s, a);                                                             \
  }
#define ST_LAUNCH_STREAM(RWV_, RBW_, NS128_, NS64_, MINB_)                                    \
  if (a.pg.bt) {                                                                               \
    ST_LAUNCH_STREAM_P(RWV_, RBW_, NS128_, NS64_, MINB_, true)                                 \
  } else {                                                                                     \
    ST_LAUNCH_STREAM_P(RWV_, RBW_, NS128_, NS64_, MINB_, false)                                \
  }
    ST_LAUNCH_STREAM(1, 1, 2, 4, 1)
    ST_LAUNCH_STREAM(1, 2, 2, 4, 1)
    ST_LAUNCH_STREAM(1, 4, 2, 4, 1)
    ST_LAUNCH_STREAM(2, 4, 4, 8, 1)
    ST_LAUNCH_STREAM(4, 4, 8, 16, 1)
    ST_LAUNCH_STREAM(2, 2, 2, 4, 2)
    ST_LAUNCH_STREAM(4, 2, 4, 8, 2)
#undef ST_LAUNCH_STREAM_P
#undef ST_LAUNCH_STREAM
  } else {
    if (D == 128) hipLaunchKernelGGL((attn_valu_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_valu_kernel<float, 64>), grid, block, 0, s, a);
  }
  if ((rc = st::check_launch())) return rc;
  if (side) {
    if ((rc = side->launch(side->ctx))) return rc;
    if (hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return ST_E_LAUNCH;
  }
  const int TH = tree->total_nodes * Hq;
  const int rpb = 256 / (D / 4);
  const int n_combine = p.NS > 1 ? (TH + rpb - 1) / rpb : 0;
  if (!compact) {
    if (n_combine == 0) return ST_OK;
    const dim3 cg(n_combine);
    if (p.stream) {
      if (D == 128) hipLaunchKernelGGL((attn_combine_kernel<uint16_t, 128>), cg, block, 0, s, a);
      else hipLaunchKernelGGL((attn_combine_kernel<uint16_t, 64>), cg, block, 0, s, a);
    } else {
      if (D == 128) hipLaunchKernelGGL((attn_combine_kernel<float, 128>), cg, block, 0, s, a);
      else hipLaunchKernelGGL((attn_combine_kernel<float, 64>), cg, block, 0, s, a);
    }
    return st::check_launch();
  }
  const dim3 cg(n_combine + compact->B * 2 * compact->Hkv);
  const st::CompactArgs& c = *compact;
  if (p.stream) {
    if (D == 128)
      hipLaunchKernelGGL((attn_combine_compact_kernel<uint16_t, 128>), cg, block, 0, s, a, c, n_combine);
    else
      hipLaunchKernelGGL((attn_combine_compact_kernel<uint16_t, 64>), cg, block, 0, s, a, c, n_combine);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((attn_combine_compact_kernel<float, 128>), cg, block, 0, s, a, c, n_combine);
    else
      hipLaunchKernelGGL((attn_combine_compact_kernel<float, 64>), cg, block, 0, s, a, c, n_combine);
  }
  return st::check_launch();
}

extern "C" int st_tree_attention_paged(const st_tree* tree, int Hq, int Hkv, int D,
                                       st_dtype dtype, float scale, const void* q,
                                       const void* k_pool, const void* v_pool, int n_blocks,
                                       int block_size, const int32_t* block_table,
                                       int max_blocks, const int32_t* prefix_len,
                                       int max_prefix, const uint64_t* mask, void* out,
                                       float* lse, void* workspace, size_t ws_bytes,
                                       int32_t* status, void* stream) {
  if (!block_table || n_blocks < 1 || max_blocks < 1) return ST_E_INVALID;
  if (block_size < 32 || block_size > 4096 || (block_size & (block_size - 1)))
    return ST_E_UNSUPPORTED;
  const long cap = (long)max_blocks * block_size;
  if (cap > (1L << 30)) return ST_E_UNSUPPORTED;
  const st::KvPaging pg{block_table, max_blocks, __builtin_ctz(block_size), n_blocks};
  return st::tree_attention_impl(tree, Hq, Hkv, D, dtype, scale, q, k_pool, v_pool, (int)cap,
                                 prefix_len, max_prefix, mask, out, lse, workspace, ws_bytes,
                                 status, stream, nullptr, nullptr, &pg);
}

extern "C" int st_tree_attention(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                                 float scale, const void* q, const void* k_cache,
                                 const void* v_cache, int S_max, const int32_t* prefix_len,
                                 int max_prefix, const uint64_t* mask, void* out, float* lse,
                                 void* workspace, size_t ws_bytes, int32_t* status,
                                 void* stream) {
  return st::tree_attention_impl(tree, Hq, Hkv, D, dtype, scale, q, k_cache, v_cache, S_max,
                                 prefix_len, max_prefix, mask, out, lse, workspace, ws_bytes,
                                 status, stream, nullptr, nullptr);
}

// st_verification_step: acceptance, attention with in-kernel ancestor masks,
// then the split merge and the KV compaction in one launch, whose workgroups
// also walk the trees.  For greedy acceptance the vocab argmax runs inside
// the attention launch when it fits (one 8192-entry slice per workgroup), so
// the step is two launches; the stochastic node kernel, or a greedy argmax
// too large for that, runs on a side stream beside the attention kernel.
#include "step_internal.h"

#include <math.h>

#include <mutex>

namespace {

size_t verify_ws(const st_tree* t, const st_step* s) {
  return s->draft_logits ? st_verify_stochastic_workspace(t, s->V)
                         : st_verify_greedy_workspace(t, s->V);
}

// A second stream per device, for the acceptance kernel of a step (the
// stochastic node kernel, or a large greedy argmax): it reads only logits and
// writes only the verification workspace, so it runs beside the attention
// kernel, and the merge + compaction launch that walks the trees waits for
// it.  The stream and its two events are created on a device's first such
// step and kept until the process ends (default priority, non-blocking,
// events without timing).  Every step re-records the events, so `side_mu` is
// held from the fork's record to the join's wait.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

std::mutex side_mu;

// The current device's side stream, or null when one cannot be made (the step
// then stays on the caller's stream).  Call with side_mu held.
const SideStream* side_stream_locked() {
  static SideStream dev_side[64];
  static bool tried[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& d = dev_side[dev];
  if (!tried[dev]) {
    tried[dev] = true;
    if (hipStreamCreateWithFlags(&d.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&d.join, hipEventDisableTiming) != hipSuccess) {
      d = SideStream{};
      (void)hipGetLastError();
    }
  }
  return d.s ? &d : nullptr;
}

bool step_fields_ok(const st_step* s) {
  return s && s->q && s->k_cache && s->v_cache && s->prefix_len && s->out && s->tokens &&
         s->logits && s->accept_len && s->accept_nodes && s->out_tokens && s->src_slot &&
         s->new_len && s->V >= 1 && s->S_max >= 1 && s->max_prefix >= 0 &&
         s->scale > 0.f && isfinite(s->scale) &&
         (!s->draft_logits || (s->temperature > 0.f && isfinite(s->temperature)));
}

}  // namespace

extern "C" size_t st_verification_step_workspace(const st_tree* tree, const st_step* s) {
  if (st::check_tree_host(tree) || !step_fields_ok(s)) return 0;
  const size_t a = st_tree_attention_workspace(tree, s->Hq, s->Hkv, s->D, s->dtype, s->max_prefix);
  return st::align_up(verify_ws(tree, s), 256) + a;
}

namespace {

// The step over contiguous caches (pg null) or a paged pool (pg: the block
// table; s->S_max is then the logical capacity).
int step_impl(const st_tree* tree, const st_step* s, void* workspace, size_t ws_bytes,
              int32_t* status, void* stream, const st::KvPaging* pg, int draft_probs = 0,
              float top_p = 1.f, bool serial = st::testing_plan().step_serial != 0) {
  int rc = st::check_tree_host(tree);
  if (rc) return rc;
  if (!step_fields_ok(s)) return ST_E_INVALID;
  // every check that the three launches would make, before enqueueing any
  if (s->Hq < 1 || s->Hkv < 1 || s->Hq % s->Hkv || (s->D != 64 && s->D != 128))
    return ST_E_UNSUPPORTED;
  if (s->dtype != ST_F32 && s->dtype != ST_BF16) return ST_E_INVALID;
  if (((uintptr_t)s->q | (uintptr_t)s->k_cache | (uintptr_t)s->v_cache | (uintptr_t)s->out) % 16)
    return ST_E_INVALID;
  const size_t vws = verify_ws(tree, s);
  const size_t off = st::align_up(vws, 256);
  const size_t aws = st_tree_attention_workspace(tree, s->Hq, s->Hkv, s->D, s->dtype, s->max_prefix);
  if ((vws || aws) && (!workspace || ws_bytes < off + aws)) return ST_E_WORKSPACE;
  st::CompactArgs c;
  const int max_path = tree->max_depth + 1;
  rc = st::fill_compact_args(tree->B, s->Hkv, s->D, s->dtype, s->k_cache, s->v_cache, s->S_max,
                             s->prefix_len, s->accept_len, s->accept_nodes, max_path,
                             s->src_slot, s->new_len, status, c);
  if (rc) return rc;
  if (pg) c.pg = *pg;

  // Each compaction workgroup of the last launch walks its request's tree
  // itself (a few microseconds of latency-bound work that then needs no
  // launch of its own).  The walk's inputs (node verdicts or argmax partials)
  // come from the acceptance kernel, launched below.
  if (s->draft_logits) {
    rc = st::stochastic_prepare(tree, s->V, s->tokens, s->logits, s->draft_logits,
                                s->temperature, s->accept_len, s->accept_nodes, s->out_tokens,
                                s->near_ties, workspace, vws, status, c.sw);
    c.walk = st::kWalkStochastic;
  } else {
    rc = st::greedy_prepare(tree, s->V, s->tokens, s->logits, s->accept_len, s->accept_nodes,
                            s->out_tokens, workspace, vws, status, c.g);
    c.walk = st::kWalkGreedy;
  }
  if (rc) return rc;
  // Greedy with bf16 attention: when there is at most one argmax slice per
  // attention workgroup (and V is a multiple of 4), the workgroups reduce them
  // in their prologue (the slice's loads overlap the first K/V chunk's);
  // otherwise the argmax gets a launch of its own.
  const st::ArgmaxJob job =
      s->draft_logits ? st::ArgmaxJob{}
                      : st::ArgmaxJob{s->logits, (st::ArgmaxPart*)c.g.part, s->V, c.g.nslices,
                                      tree->total_nodes * c.g.nslices, status};
  const bool fuse_argmax =
      !s->draft_logits && s->dtype == ST_BF16 && (s->V & 3) == 0 &&
      job.units <= st::attention_workgroups(tree, s->Hq, s->Hkv, s->D, s->dtype, s->max_prefix);
  const bool own_launch = s->draft_logits || !fuse_argmax;
  auto acceptance = [&](void* strm) {
    return s->draft_logits
               ? st::stochastic_node_launch(c.sw, s->logits, s->draft_logits, s->temperature,
                                            s->seed, s->offset, tree->B, strm, draft_probs, top_p)
               : st::greedy_argmax_launch(c.g, s->logits, strm);
  };
  auto attention = [&](const st::SideLaunch* side) {
    return st::tree_attention_impl(tree, s->Hq, s->Hkv, s->D, s->dtype, s->scale, s->q,
                                   s->k_cache, s->v_cache, s->S_max, s->prefix_len,
                                   s->max_prefix, nullptr, s->out, s->lse,
                                   (char*)workspace + off, aws, status, stream, &c,
                                   fuse_argmax ? &job : nullptr, pg, side);
  };
  // The stochastic node kernel goes beside attention, and so does a greedy
  // argmax launch over at least 16 MB of logits; a smaller one stays in
  // order (the fork and join cost more than the overlap gives).
  const bool big_argmax = !s->draft_logits && !fuse_argmax &&
                          (size_t)tree->total_nodes * (size_t)s->V * 4 >= ((size_t)16 << 20);
  if ((s->draft_logits || big_argmax) && !serial) {
    std::lock_guard<std::mutex> lock(side_mu);
    if (const SideStream* ss = side_stream_locked()) {
      // fork: the side stream starts after the caller's earlier work; the
      // attention launcher enqueues the acceptance kernel there after its own
      // kernel and makes the caller's stream wait for `join` before the
      // merge + compaction launch.
      if (hipEventRecord(ss->fork, (hipStream_t)stream) != hipSuccess ||
          hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
        return ST_E_LAUNCH;
      struct Ctx {
        decltype(acceptance)* run;
        const SideStream* ss;
      } ctx{&acceptance, ss};
      const st::SideLaunch side{[](void* p) {
                                  const Ctx& x = *(const Ctx*)p;
                                  const int r = (*x.run)(x.ss->s);
                                  if (r) return r;
                                  return hipEventRecord(x.ss->join, x.ss->s) == hipSuccess
                                             ? (int)ST_OK
                                             : (int)ST_E_LAUNCH;
                                },
                                &ctx, ss->join};
      return attention(&side);
    }
  }
  if (own_launch && (rc = acceptance(stream))) return rc;
  return attention(nullptr);
}

}  // namespace

extern "C" int st_verification_step(const st_tree* tree, const st_step* s, void* workspace,
                                    size_t ws_bytes, int32_t* status, void* stream) {
  return step_impl(tree, s, workspace, ws_bytes, status, stream, nullptr);
}

extern "C" int st_verification_step_paged(const st_tree* tree, const st_step* s, int n_blocks,
                                          int block_size, const int32_t* block_table,
                                          int max_blocks, void* workspace, size_t ws_bytes,
                                          int32_t* status, void* stream) {
  if (!s || !block_table || n_blocks < 1 || max_blocks < 1) return ST_E_INVALID;
  if (block_size < 32 || block_size > 4096 || (block_size & (block_size - 1)))
    return ST_E_UNSUPPORTED;
  const long cap = (long)max_blocks * block_size;
  if (cap > (1L << 30)) return ST_E_UNSUPPORTED;
  st_step sp = *s;
  sp.S_max = (int32_t)cap;
  const st::KvPaging pg{block_table, max_blocks, __builtin_ctz(block_size), n_blocks};
  return step_impl(tree, &sp, workspace, ws_bytes, status, stream, &pg);
}

extern "C" int st_verification_step_ex(const st_tree* tree, const st_step* s, int draft_is_probs,
                                       float top_p, void* workspace, size_t ws_bytes,
                                       int32_t* status, void* stream) {
  if (!s || !(top_p > 0.f && top_p <= 1.f) || (draft_is_probs != 0 && draft_is_probs != 1))
    return ST_E_INVALID;
  if ((draft_is_probs || top_p < 1.f) && !s->draft_logits) return ST_E_INVALID;
  return step_impl(tree, s, workspace, ws_bytes, status, stream, nullptr, draft_is_probs, top_p);
}

// ---------------------------------------------------------------- no allocation
//
// The one-call step for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid hipMalloc): its workspace is a
// file-scope device array of kScratchBytes, which every GPU the library runs
// on holds (at its own address) until the process ends.  Nothing in the
// step's workspace needs to start at zero: every partial, verdict and argmax
// slice that a later launch reads is written first by an earlier one.

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up on the
// first call on that device (null if the lookup fails).
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" int st_verification_step_noalloc(const st_tree* tree, const st_step* s,
                                            int32_t* status, void* stream) {
  const size_t need = st_verification_step_workspace(tree, s);
  if (need == 0) return ST_E_INVALID;
  if (need > kScratchBytes) return ST_E_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return ST_E_LAUNCH;
  // every launch on the caller's stream: no side stream to create on a first call
  return step_impl(tree, s, ws, kScratchBytes, status, stream, nullptr, 0, 1.f, true);
}


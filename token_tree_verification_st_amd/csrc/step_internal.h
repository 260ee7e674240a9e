// Host-side pieces shared by the separate entry points and the one-call
// verification step (not exported).
#pragma once
#include "kv_compact_dev.h"

namespace st {

// st_verify_greedy in parts (verify.hip): check the arguments and fill the
// walk's inputs (the argmax partials go to the start of `workspace`), launch
// the vocab argmax.  The one-call step runs the argmax inside the attention
// launch instead when it can, and the walk in its compaction workgroups.
int greedy_prepare(const st_tree* tree, int V, const int32_t* tokens, const float* logits,
                   int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                   void* workspace, size_t ws_bytes, int32_t* status, GreedyWalkArgs& walk);
int greedy_argmax_launch(const GreedyWalkArgs& walk, const float* logits, void* stream);

// st_verify_stochastic in parts (verify.hip): check the arguments and fill the
// walk's inputs (the node verdicts go to the start of `workspace`), launch the
// node kernel.  The one-call step runs the walk in its compaction workgroups.
int stochastic_prepare(const st_tree* tree, int V, const int32_t* tokens,
                       const float* target_logits, const float* draft_logits, float temperature,
                       int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                       int32_t* near_ties, void* workspace, size_t ws_bytes, int32_t* status,
                       StochWalkArgs& walk);
int stochastic_node_launch(const StochWalkArgs& walk, const float* target_logits,
                           const float* draft_logits, float temperature, uint64_t seed,
                           uint64_t offset, int B, void* stream,
                           int draft_probs = 0, float top_p = 1.f);

// Vocab argmax slices handed to the attention launch: its workgroups load them
// while their first K/V chunk is in flight and reduce them before their loop.
struct ArgmaxJob {
  const float* logits;
  ArgmaxPart* part;
  int V, nslices, units;  // units = rows * nslices
  int32_t* status;
};

// Work on another stream that the attention launcher enqueues after its
// attention kernel: `launch(ctx)` enqueues it and records `join` there.
struct SideLaunch {
  int (*launch)(void* ctx);
  void* ctx;
  hipEvent_t join;
};

// Checks the arguments of st_kv_compact and fills CompactArgs (compact.hip).
int fill_compact_args(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache,
                      int S_max, const int32_t* prefix_len, const int32_t* accept_len,
                      const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                      int32_t* new_len, int32_t* status, CompactArgs& c);

// st_tree_attention; with `compact` set, the launch that merges the splits
// also moves the accepted paths' KV rows (after the attention kernel has read
// them), or a compaction launch follows when there is nothing to merge; with
// `argmax` set, the streaming kernel's workgroups also reduce those argmax
// slices (the fp32 kernel does not: the slices are then launched first);
// with `side` set, its launch is enqueued right after the attention kernel
// (on another stream) and the stream waits for its `join` event before the
// merge (attention.hip).
int tree_attention_impl(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype, float scale,
                        const void* q, const void* k_cache, const void* v_cache, int S_max,
                        const int32_t* prefix_len, int max_prefix, const uint64_t* mask,
                        void* out, float* lse, void* workspace, size_t ws_bytes, int32_t* status,
                        void* stream, const CompactArgs* compact,
                        const ArgmaxJob* argmax = nullptr, const KvPaging* paging = nullptr,
                        const SideLaunch* side = nullptr);

// Workgroups of the attention launch for these sizes: each one, with an item
// or without, can take one vocab argmax slice.
int attention_workgroups(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                         int max_prefix);

}  // namespace st

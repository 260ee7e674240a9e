// Host-side pieces shared by the separate entry points and the one-call
// verification step (not exported).
#pragma once
#include "kv_compact_dev.h"

namespace st {

// st_verify_greedy without its walk: checks the arguments, launches the
// vocab argmax and fills the walk's inputs, for the walk to run in the
// compaction workgroups of the last launch (verify.hip).
int greedy_argmax_only(const st_tree* tree, int V, const int32_t* tokens, const float* logits,
                       int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                       void* workspace, size_t ws_bytes, int32_t* status, void* stream,
                       GreedyWalkArgs& walk);

// Checks the arguments of st_kv_compact and fills CompactArgs (compact.hip).
int fill_compact_args(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache,
                      int S_max, const int32_t* prefix_len, const int32_t* accept_len,
                      const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                      int32_t* new_len, int32_t* status, CompactArgs& c);

// st_tree_attention; with `compact` set, the launch that merges the splits
// also moves the accepted paths' KV rows (after the attention kernel has read
// them), or a compaction launch follows when there is nothing to merge
// (attention.hip).
int tree_attention_impl(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype, float scale,
                        const void* q, const void* k_cache, const void* v_cache, int S_max,
                        const int32_t* prefix_len, int max_prefix, const uint64_t* mask,
                        void* out, float* lse, void* workspace, size_t ws_bytes, int32_t* status,
                        void* stream, const CompactArgs* compact);

}  // namespace st

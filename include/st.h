/*
 * st.h -- C ABI of the token-tree verification library (libst.so, gfx950).
 *
 * The library runs the target model's side of tree-based speculative decoding
 * for one attention layer: the ancestor mask of a speculated token tree,
 * tree-masked attention of every tree node over the request's cached prefix
 * plus its own root path, greedy or rejection-sampling acceptance down the
 * tree, and compaction of the accepted path's KV rows.
 *
 * Sources (web pages, cited by title and section):
 *   SpecInfer news article (sunluscious.com.cn), "Token 樹驗證器": the draft
 *     outputs form one token tree; the verifier runs tree attention through a
 *     constructed mask matrix with a depth-first KV-cache update.
 *   "SpecInfer：基于树结构的LLM推测性推理加速技术" §2.1: tree nodes carry a
 *     parent pointer; tree_attention(query, key, value, tree_mask); the longest
 *     verified prefix is accepted.
 *   Speculative-decoding explainer (intelliparadigm.com) §2.2: accept with
 *     probability min(1, p_main/p_draft), left to right, replace at the first
 *     rejection; §3.2: all candidates are verified in one forward pass.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *     memory; the library never allocates device memory, frees or
 *     synchronises.  Every call enqueues its kernels on `stream` (a
 *     hipStream_t passed as void*; NULL is the default stream) and returns at
 *     once.  (The one-call step also uses a stream of its own on each device,
 *     ordered after and before `stream` by events: see st_verification_step.)
 *   - Request b owns tree nodes node_off[b] .. node_off[b+1]-1 (N_b >= 1
 *     nodes).  Local node 0 is the root, the last token the target already
 *     emitted; parent[] holds request-local indices with parent[root] = -1
 *     and 0 <= parent[i] < i for the others.
 *   - During verification node i of request b has its key/value at cache slot
 *     prefix_len[b] + i.  Caches are head-major: [B][Hkv][S_max][D].
 *   - Return value: ST_OK (0) or a negative ST_E_* code for a problem found on
 *     the host before launching (nothing is enqueued then).
 *   - Data-dependent problems found by the kernels are OR-ed into *status (a
 *     device int32 that the caller zeroes; may be NULL) as ST_STATUS_* bits.
 *     Outputs of a request with such a problem are unspecified but every
 *     write stays inside the documented output ranges.
 *   - Calls are stateless and thread-safe; concurrent calls on different
 *     streams may not share output or workspace buffers.
 */
#ifndef ST_H
#define ST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ST_OK 0
#define ST_E_INVALID (-1)     /* null pointer or out-of-range scalar             */
#define ST_E_UNSUPPORTED (-2) /* D not 64/128, Hq % Hkv != 0, max_nodes > 256... */
#define ST_E_WORKSPACE (-3)   /* workspace smaller than the *_workspace() size   */
#define ST_E_LAUNCH (-4)      /* the HIP runtime refused a launch                */

#define ST_STATUS_BAD_PARENT 1    /* parent[] breaks the rules above            */
#define ST_STATUS_BAD_TOKEN 2     /* a draft token outside [0, V)               */
#define ST_STATUS_NONFINITE 4     /* a logit that is NaN or infinite            */
#define ST_STATUS_PATH_OVERFLOW 8 /* accepted path longer than max_depth        */
#define ST_STATUS_BAD_PREFIX 16   /* prefix_len outside [0, max_prefix], or the
                                     request's slots run past S_max             */
#define ST_STATUS_BAD_BLOCK 32    /* a block-table entry outside [0, n_blocks)  */

#define ST_MAX_NODES 256          /* per request                                */

typedef enum { ST_F32 = 0, ST_BF16 = 1 } st_dtype;

/* A batch of B token trees, nodes concatenated request after request. */
typedef struct {
  int32_t B;                /* [host] number of requests, >= 1                     */
  int32_t total_nodes;      /* [host] T = node_off[B]                              */
  int32_t max_nodes;        /* [host] >= every N_b, <= ST_MAX_NODES                */
  int32_t max_depth;        /* [host] >= every node depth (root depth 0)           */
  const int32_t* node_off;  /* [B+1], node_off[0] = 0, strictly increasing         */
  const int32_t* parent;    /* [T] request-local parent index, root = -1           */
} st_tree;

/* Words per mask row: ceil(max_nodes / 64). */
int st_mask_words(int max_nodes);

/*
 * st_tree_mask -- ancestor bitmask and depth of every tree node.
 * Defines which tree keys each node may attend to (SpecInfer news article,
 * "Token 樹驗證器"; the parent pointer of §2.1 of the SpecInfer developer
 * article).  Bit (k % 64) of word (k / 64) of mask row i is set iff request-
 * local node k lies on node i's root path (i itself included).
 *   mask  [T][W] uint64, W = st_mask_words(max_nodes); unused bits are 0
 *   depth [T] int32, edges between the node and its root
 * A request with a bad parent array sets ST_STATUS_BAD_PARENT; its rows then
 * hold the node's own bit plus whatever valid ancestors were reached.
 */
int st_tree_mask(const st_tree* tree, uint64_t* mask, int32_t* depth, int32_t* status,
                 void* stream);

/* Bytes of workspace st_tree_attention needs for these sizes (0 is possible). */
size_t st_tree_attention_workspace(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                                   int max_prefix);

/*
 * st_tree_attention -- tree-masked attention of every tree node.
 * For node i of request b and query head h (kv head g = h / (Hq/Hkv)):
 *   out[i][h] = softmax_k(scale * q[i][h] . K[b][g][k]) . V[b][g][k]
 * over the keys k < prefix_len[b] (the cached prefix, always visible) and the
 * tree keys prefix_len[b] + j with bit j of mask row i set (SpecInfer
 * developer article §2.1, tree_attention; masked entries excluded).
 *   q        [T][Hq][D] of `dtype` (ST_F32 or ST_BF16)
 *   k_cache, v_cache  [B][Hkv][S_max][D] of `dtype`; S_max >= every
 *            prefix_len[b] + N_b; only slots below that are read
 *   prefix_len [B] int32 in [0, max_prefix]
 *   mask     [T][W] from st_tree_mask, or NULL: the kernel then derives each
 *            row's ancestor mask from tree->parent itself (the same relation
 *            st_tree_mask writes out), setting ST_STATUS_BAD_PARENT on a bad
 *            parent array
 *   out      [T][Hq][D] of `dtype` (bf16 stored round-to-nearest-even)
 *   lse      [T][Hq] fp32 natural-log sum of exp of the scaled scores, or NULL
 *   scale    the score scale; 1/sqrt(D) reproduces standard attention
 * Accumulation and softmax are fp32.  D must be 64 or 128; Hq % Hkv == 0.
 */
int st_tree_attention(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype, float scale,
                      const void* q, const void* k_cache, const void* v_cache, int S_max,
                      const int32_t* prefix_len, int max_prefix, const uint64_t* mask,
                      void* out, float* lse, void* workspace, size_t ws_bytes, int32_t* status,
                      void* stream);

/*
 * st_tree_attention_paged -- st_tree_attention over a paged KV pool: the
 * keys and values of request b are not one contiguous [S_max][D] run per kv
 * head but fixed-size blocks picked by a per-request block table (the paged
 * KV memory that the SpecInfer news article and the vAttention notes contrast
 * with contiguous per-request KV).  Logical slot k of request b (prefix keys
 * k < prefix_len[b], node i at prefix_len[b] + i, as before) lives in row
 * k % block_size of physical block block_table[b][k / block_size].
 *   k_pool, v_pool  [n_blocks][Hkv][block_size][D] of `dtype`
 *   block_table     [B][max_blocks] int32; the logical capacity is
 *                   S_max = max_blocks * block_size; only the entries that
 *                   cover slots below prefix_len[b] + N_b are read.  An entry
 *                   outside [0, n_blocks) sets ST_STATUS_BAD_BLOCK and reads
 *                   block 0 or n_blocks-1 instead (never outside the pool).
 *   block_size      a power of two from 32 to 4096
 * Everything else, including the workspace size (st_tree_attention_workspace
 * with the same arguments), as for st_tree_attention; the arithmetic is the
 * same, so the outputs equal those of st_tree_attention on the gathered
 * contiguous caches bit for bit.
 */
int st_tree_attention_paged(const st_tree* tree, int Hq, int Hkv, int D, st_dtype dtype,
                            float scale, const void* q, const void* k_pool, const void* v_pool,
                            int n_blocks, int block_size, const int32_t* block_table,
                            int max_blocks, const int32_t* prefix_len, int max_prefix,
                            const uint64_t* mask, void* out, float* lse, void* workspace,
                            size_t ws_bytes, int32_t* status, void* stream);

/* Bytes of workspace st_verify_greedy needs. */
size_t st_verify_greedy_workspace(const st_tree* tree, int V);

/*
 * st_verify_greedy -- accept the longest verified path (SpecInfer developer
 * article §2.1).  Row i of `logits` [T][V] fp32 is the target's next-token
 * distribution after node i; a[i] is its argmax (lowest index on ties).  From
 * the root, the walk moves to the lowest-index child c with tokens[c] == a[u]
 * and stops when there is none.
 *   tokens       [T] int32 draft token of each node (the root's is unused)
 *   accept_len   [B]   number L of accepted non-root nodes
 *   accept_nodes [B][max_depth+1] local node ids of the path, root first, -1 padded
 *   out_tokens   [B][max_depth+2] the L accepted tokens then the target's token
 *                a[last] (so L+1 tokens are emitted), -1 padded
 * If the path would pass max_depth nodes below the root it stops there, the
 * last emitted token is -1 and ST_STATUS_PATH_OVERFLOW is set.
 */
int st_verify_greedy(const st_tree* tree, int V, const int32_t* tokens, const float* logits,
                     int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                     void* workspace, size_t ws_bytes, int32_t* status, void* stream);

/* Bytes of workspace st_verify_stochastic needs. */
size_t st_verify_stochastic_workspace(const st_tree* tree, int V);

/*
 * st_verify_stochastic -- rejection sampling down the tree (speculative-
 * decoding explainer §2.2: accept with probability min(1, p/q), check left to
 * right, replace at the first rejection so the output keeps the target's
 * distribution).  p_i = softmax(target_logits[i] / temperature) and q_i =
 * softmax(draft_logits[i] / temperature) are the target's and the draft's
 * distributions for the children of node i.  At node u with residual r
 * (initially p_u) the children are tested in ascending index: child c with
 * token x is accepted iff u_acc(c) * q_u[x] < r[x]; after a rejection
 * r <- normalise(max(0, r - q_u)), left unchanged if that has a mass of at
 * most 1e-6 of the row (the rounding residue of r and q that agree).  On an
 * acceptance the walk moves to c with r = p_c.  When no child is accepted the
 * replacement token is the smallest v whose running sum of r (ascending v)
 * exceeds u_smp(u) * sum(r).  Uniforms come from Philox4x64-10 with key
 * (seed, 0) and counter (local node, request, offset, 0): u_acc = top 24 bits
 * of word 0, u_smp = top 24 bits of word 1, times 2^-24.
 *   target_logits, draft_logits [T][V] fp32; temperature > 0
 *   V <= 32768 (ST_E_UNSUPPORTED above: one workgroup holds a node's two
 *   rows in registers while it tests the node's children), and
 *   B * max_nodes < 2^22 (ST_E_UNSUPPORTED beyond: one 1024-thread workgroup
 *   per request and local node index); the draft row of
 *   a node without children takes no part in the result and is not read, so
 *   a non-finite entry there is not flagged;
 *   outputs as for st_verify_greedy;
 *   near_ties [B] int32 or NULL: comparisons on the taken path with
 *   |r[x] - u*q[x]| < 1e-6, plus 1 if the replacement draw's threshold lies
 *   within 1e-6 * sum(r) of its bin's edges.
 * Decisions use fp32 exponentials with fp64 sums.
 */
int st_verify_stochastic(const st_tree* tree, int V, const int32_t* tokens,
                         const float* target_logits, const float* draft_logits, float temperature,
                         uint64_t seed, uint64_t offset, int32_t* accept_len,
                         int32_t* accept_nodes, int32_t* out_tokens, int32_t* near_ties,
                         void* workspace, size_t ws_bytes, int32_t* status, void* stream);

/*
 * st_verify_stochastic_ex -- st_verify_stochastic with the two sampling
 * options the pages pair with it: nucleus (top-p) sampling (the SpecInfer
 * developer article's configuration example and the explainer's tuning
 * table recommend top-p 0.9 with temperature 0.7), and a draft given as
 * probabilities (the explainer's acceptance call takes the draft's
 * probabilities).
 *   draft_is_probs 0: `draft` holds logits, q_i = softmax(draft[i] / T);
 *                  1: `draft` holds probabilities (>= 0, any positive scale),
 *                     q_i = draft[i] / sum(draft[i]), no temperature; a
 *                     negative or non-finite entry sets ST_STATUS_NONFINITE.
 *   top_p in (0, 1]: below 1 both p_i and q_i are restricted to their nucleus
 *     before any test -- the smallest set of most likely tokens whose mass
 *     reaches top_p of the row, together with every token as likely as the
 *     least likely one kept -- and renormalised (the draft tokens are taken
 *     to come from the filtered draft, the output follows the filtered
 *     target).  The cut is found by bisection over fp32 values with fp64
 *     sums.  top_p = 1 and draft_is_probs = 0 give st_verify_stochastic.
 * Other arguments as for st_verify_stochastic; ST_E_INVALID for top_p
 * outside (0, 1] or draft_is_probs not 0/1.
 */
int st_verify_stochastic_ex(const st_tree* tree, int V, const int32_t* tokens,
                            const float* target_logits, const float* draft, int draft_is_probs,
                            float temperature, float top_p, uint64_t seed, uint64_t offset,
                            int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                            int32_t* near_ties, void* workspace, size_t ws_bytes,
                            int32_t* status, void* stream);

/*
 * st_kv_compact -- move the accepted path's keys and values into contiguous
 * slots (the depth-first KV-cache update of the SpecInfer news article,
 * "Token 樹驗證器").  For request b with P = prefix_len[b], L = accept_len[b]
 * and path = accept_nodes[b][0..L], slot P + j of every kv head takes what
 * slot P + path[j] held before the call, for j = 0..L, in k_cache and
 * v_cache ([B][Hkv][S_max][D] of `dtype`, updated in place).  Other slots are
 * not touched.
 *   accept_nodes [B][max_path] as written by the verify calls (max_path =
 *                max_depth + 1)
 *   src_slot [B][max_path] int32: P + path[j] for j <= L, -1 after
 *   new_len  [B] int32: P + L + 1
 * A request whose L + 1 exceeds max_path, or whose path leaves [0, S_max - P),
 * sets ST_STATUS_PATH_OVERFLOW or ST_STATUS_BAD_PARENT and is left unmoved
 * (new_len = P).  Call once per layer.
 */
int st_kv_compact(int B, int Hkv, int D, st_dtype dtype, void* k_cache, void* v_cache, int S_max,
                  const int32_t* prefix_len, const int32_t* accept_len,
                  const int32_t* accept_nodes, int max_path, int32_t* src_slot, int32_t* new_len,
                  int32_t* status, void* stream);

/*
 * st_kv_compact_paged -- st_kv_compact on a paged pool (layout and block
 * table as for st_tree_attention_paged; block_size any power of two up to
 * 4096): logical slot P + j takes what logical slot P + path[j] held, each
 * translated through the request's block table.  The table entries of one
 * request must name distinct blocks (the moves are in place).  src_slot and
 * new_len hold logical slots.  An out-of-range entry sets
 * ST_STATUS_BAD_BLOCK and is clamped into the pool.
 */
int st_kv_compact_paged(int B, int Hkv, int D, st_dtype dtype, void* k_pool, void* v_pool,
                        int n_blocks, int block_size, const int32_t* block_table, int max_blocks,
                        const int32_t* prefix_len, const int32_t* accept_len,
                        const int32_t* accept_nodes, int max_path, int32_t* src_slot,
                        int32_t* new_len, int32_t* status, void* stream);

/*
 * st_verification_step -- one verification step of one layer in one call:
 * acceptance of the tree (greedy, or stochastic when draft_logits is set),
 * tree attention of every node with the ancestor masks derived from
 * tree->parent inside the attention kernel, then compaction of the accepted
 * paths' KV rows (SpecInfer developer article §2.1: one pass decodes all tree
 * paths; the news article's depth-first KV-cache update).  Every field means
 * what the argument of the same name means for st_verify_greedy /
 * st_verify_stochastic, st_tree_attention and st_kv_compact; the results are
 * those of calling them in that order.  Acceptance reads neither the caches
 * nor the attention output; compaction runs after attention has read the
 * tree slots (it shares the launch that merges the attention splits), so the
 * three kernels need no other ordering.  All fields are checked before
 * anything is enqueued.
 *
 * The acceptance kernel when it is a launch of its own (stochastic
 * acceptance, or a greedy vocab argmax over 16 MB or more of logits) runs
 * beside the attention kernel on a second stream of the library's: it starts
 * after the work enqueued on `stream` before the call (an event recorded on
 * `stream`), and the launch that follows on `stream` waits for it (an event
 * recorded on the second stream), so to the caller the step is ordered on
 * `stream` as if it had one stream.  That stream (default priority,
 * non-blocking) and its two events are created on the first such step on
 * each device and kept until the process ends; a mutex orders concurrent
 * callers' use of the events.  Under HIP graph capture of `stream` the two
 * streams become parallel branches of the captured graph.
 */
typedef struct {
  int32_t Hq, Hkv, D;
  st_dtype dtype;
  float scale;                      /* 1/sqrt(D) reproduces standard attention */
  const void* q;                    /* [T][Hq][D]                              */
  void* k_cache;                    /* [B][Hkv][S_max][D], compacted in place  */
  void* v_cache;
  int32_t S_max;
  const int32_t* prefix_len;        /* [B]                                     */
  int32_t max_prefix;               /* [host]                                  */
  void* out;                        /* [T][Hq][D] of dtype                     */
  float* lse;                       /* [T][Hq] or NULL                         */
  int32_t V;
  const int32_t* tokens;            /* [T]                                     */
  const float* logits;              /* [T][V] target                           */
  const float* draft_logits;        /* [T][V], or NULL for greedy acceptance   */
  float temperature;                /* stochastic only                         */
  uint64_t seed, offset;            /* stochastic only                         */
  int32_t* accept_len;              /* [B]                                     */
  int32_t* accept_nodes;            /* [B][max_depth+1]                        */
  int32_t* out_tokens;              /* [B][max_depth+2]                        */
  int32_t* near_ties;               /* [B] or NULL (stochastic only)           */
  int32_t* src_slot;                /* [B][max_depth+1]                        */
  int32_t* new_len;                 /* [B]                                     */
} st_step;

/* Bytes of workspace st_verification_step needs (0 on invalid arguments). */
size_t st_verification_step_workspace(const st_tree* tree, const st_step* step);

int st_verification_step(const st_tree* tree, const st_step* step, void* workspace,
                         size_t ws_bytes, int32_t* status, void* stream);

/*
 * st_tree_build -- merge candidate continuations into one token tree per
 * request, the step before verification (SpecInfer news article, "研究現狀":
 * the outputs of several small speculative models are merged into one
 * speculated token tree; SpecInfer developer article §2.1-2.2: candidates that
 * share a prefix share its nodes, and every node points to its parent).
 * Request b's root is root_tokens[b] (the last token the target emitted);
 * candidate k continues it with seqs[b][k][0 .. lens[b][k]-1].  The tree's
 * nodes are the root and every distinct non-empty prefix of a candidate, the
 * node of a prefix being the child of the node of that prefix minus its last
 * token.  Nodes are numbered level by level (so parent < child); within a
 * level by their parent's number, then by the smallest k whose candidate has
 * the prefix.
 *   root_tokens [B], seqs [B][K][Lmax], lens [B][K]   int32 inputs
 *   n_nodes [B]          nodes of each tree, root included, at most cap
 *   parent  [B][cap]     request-local parent index (root -1)   } -1 past
 *   tokens  [B][cap]     token of each node (root: root_tokens)  } n_nodes[b]
 *   depth   [B][cap]     edges to the root                       }
 *   node_off [B+1], parent_packed [B*cap], tokens_packed [B*cap]: the same
 *     trees concatenated in the st_tree layout (entries past node_off[B]
 *     untouched); all three NULL to skip, written by a second kernel.
 * A length outside [0, Lmax] counts as 0 and a token outside [0, V) ends its
 * candidate before it, both setting ST_STATUS_BAD_TOKEN (the root token is
 * not checked); a tree of more than cap nodes keeps its first cap and sets
 * ST_STATUS_PATH_OVERFLOW.  Limits: 1 <= K <= 256, K * Lmax <= 8192,
 * 1 <= cap <= ST_MAX_NODES (ST_E_UNSUPPORTED beyond them).
 */
int st_tree_build(int B, int K, int Lmax, int V, int cap, const int32_t* root_tokens,
                  const int32_t* seqs, const int32_t* lens, int32_t* n_nodes, int32_t* parent,
                  int32_t* tokens, int32_t* depth, int32_t* node_off, int32_t* parent_packed,
                  int32_t* tokens_packed, int32_t* status, void* stream);

/*
 * st_verification_step_ex -- st_verification_step with the sampling options of
 * st_verify_stochastic_ex: nucleus filtering (top_p in (0, 1]) and the draft
 * given as probabilities (draft_is_probs 1: step->draft_logits holds
 * probabilities).  Both need stochastic acceptance (step->draft_logits set);
 * ST_E_INVALID otherwise or for values out of range.  top_p = 1 and
 * draft_is_probs = 0 give st_verification_step.  Same workspace size.
 */
int st_verification_step_ex(const st_tree* tree, const st_step* step, int draft_is_probs,
                            float top_p, void* workspace, size_t ws_bytes, int32_t* status,
                            void* stream);

/*
 * st_verification_step_noalloc -- st_verification_step for callers that
 * cannot allocate memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc).  It takes no workspace: the library's own
 * static device buffer of 64 MiB per GPU (ST_NOALLOC_SCRATCH_BYTES), reserved
 * when the library is loaded and held until the process ends, serves as the
 * step's workspace.  The call allocates and frees nothing.  Outputs equal
 * st_verification_step's for the same arguments.  Returns ST_E_WORKSPACE when
 * st_verification_step_workspace(tree, step) exceeds the buffer (nothing is
 * enqueued), ST_E_LAUNCH if the buffer's device address cannot be obtained,
 * otherwise as st_verification_step.  Every call on one GPU uses that GPU's
 * one buffer: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller; calls on one stream are ordered.
 */
#define ST_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int st_verification_step_noalloc(const st_tree* tree, const st_step* step, int32_t* status,
                                 void* stream);

/*
 * st_verification_step_paged -- st_verification_step over a paged KV pool:
 * step->k_cache / step->v_cache are pools [n_blocks][Hkv][block_size][D]
 * addressed through block_table [B][max_blocks] as for
 * st_tree_attention_paged (block_size a power of two from 32 to 4096);
 * step->S_max is ignored (the logical capacity is max_blocks * block_size).
 * Attention reads and compaction moves logical slots through the table; the
 * workspace size is st_verification_step_workspace's.  Outputs equal those of
 * st_verification_step on the contiguous caches the table describes.
 */
int st_verification_step_paged(const st_tree* tree, const st_step* step, int n_blocks,
                               int block_size, const int32_t* block_table, int max_blocks,
                               void* workspace, size_t ws_bytes, int32_t* status, void* stream);

/* ---------------------------------------------------------------------------
 * The target layer around verification.  The pages fix no architecture; the
 * calls below are the pieces one attention layer needs to run over a token
 * tree (news article, "研究現狀": decoded tokens' keys and values are cached;
 * explainer §3.2: all candidates are scored in one forward pass).  Every
 * matrix is bf16, row-major.
 * ------------------------------------------------------------------------- */

/* out[t][:] = table[tokens[t]][:] for t < T: a gather of d-wide bf16 rows
 * (d a multiple of 8, table [V][d]).  A token outside [0, V) sets
 * ST_STATUS_BAD_TOKEN and gives a row of zeros.  table and out 16-byte
 * aligned. */
int st_embed(int T, int d, int V, const int32_t* tokens, const void* table, void* out,
             int32_t* status, void* stream);

/* Rotary position embedding of the tree nodes' queries and keys, and the
 * append of their keys and values to the cache.  qkv [T][(Hq + 2 Hkv) D]
 * holds each node's Hq query heads, then Hkv key heads, then Hkv value heads
 * (the output of the fused projection).  Node i of request b sits at position
 * pos = prefix_len[b] + depth(i), the index its token has in the sequence of
 * its root path; dims j and j + D/2 (j < D/2) of a query or key head are
 * turned by the angle pos * theta^(-2j/D) ("rotate half" form; theta = 10000
 * is the usual value).  Writes q_out[T][Hq][D] (the rotated queries, as
 * st_tree_attention takes them), and for every kv head g the rotated key and
 * the value at slot prefix_len[b] + i of k_cache / v_cache [B][Hkv][S_max][D].
 * D is 64 or 128.  A bad parent array sets ST_STATUS_BAD_PARENT, a prefix
 * length outside [0, max_prefix] or slots past S_max ST_STATUS_BAD_PREFIX;
 * such a request's nodes write nothing.  Angles are formed in fp64, the
 * rotation in fp32, rounded once to bf16. */
int st_tree_rope_append(const st_tree* tree, int Hq, int Hkv, int D, float theta,
                        const void* qkv, const int32_t* prefix_len, int max_prefix, int S_max,
                        void* q_out, void* k_cache, void* v_cache, int32_t* status,
                        void* stream);

/* Bytes of workspace st_linear needs for these sizes (0 if none, or on
 * invalid sizes). */
size_t st_linear_workspace(int M, int N, int K);

/* y[M][N] = x[M][K] . w[N][K]^T (+ residual[M][N] if not NULL): bf16 inputs,
 * fp32 accumulation, y in y_dtype (ST_BF16 rounds to nearest even, ST_F32 as
 * accumulated).  w is a weight matrix in the usual [out][in] layout, read once
 * from HBM; x is the few dozen to few hundred rows of a token tree.  K must be
 * a multiple of 64 and N of 4 (ST_E_UNSUPPORTED otherwise); all pointers
 * 16-byte aligned.  The reduction may be split over workgroups (then the
 * workspace holds fp32 partials that a second kernel adds in a fixed order:
 * results do not depend on timing). */
int st_linear(int M, int N, int K, const void* x, const void* w, const void* residual, void* y,
              st_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream);

/* Measurement helper (not part of the method): one plain read-only pass over
 * `bytes` of device memory at `src` (16-byte aligned, a multiple of 16), the
 * practical HBM read ceiling the kernels above are compared with.  `sink`
 * [sink_len] uint32 is written only on a data pattern that practically never
 * occurs; at most sink_len workgroups are launched. */
int st_stream_read(const void* src, size_t bytes, uint32_t* sink, int sink_len, void* stream);

/* Text for a return code or for a status bit (host memory, static). */
const char* st_status_str(int code);

#ifdef __cplusplus
}
#endif

#endif /* ST_H */

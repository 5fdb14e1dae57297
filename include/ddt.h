/*
 * ddt.h -- C ABI of libddt.so, the MI355X (gfx950) DDTree tree-verify step.
 *
 * One verify step of DDTree speculative decoding runs as three device stages on
 * one HIP stream with no host round-trip between them, and a fourth commits
 * the accepted path to the KV cache:
 *
 *   ddt_draft_topk   drafter logits -> per-depth top-K log-probs (the builder's input)
 *   ddt_tree_build   drafter per-depth top-K log-probs -> draft tree
 *   ddt_verify_attn  every tree node of every request attends, in absorbed MLA
 *                    form, over its committed latent prefix and its ancestors
 *   ddt_tree_accept  greedy walk of the verified tree -> accepted tokens
 *   ddt_tree_accept_sampling  the same walk under temperature sampling, from the
 *                    target's logits at every tree node
 *   ddt_kv_commit    accepted path -> committed prefix slots (slot table rewrite)
 *
 * The operations are the ones described on the pages
 *   [P1] "The Architecture of a Thousand-Parameter Decision: Designing a Native
 *        DDTree Inference Engine for Kimi K2.6", section "What to Build New"
 *        (item 2, tree-verify MLA attention and its greedy and sampling-
 *        probability paths; item 3, GPU tree builder; item 4, per-depth top-k
 *        logit extraction; item 5, the paged latent KV cache, the append step
 *        and the greedy and temperature commit paths) and section "What to
 *        Reuse" (item 3, target-only tree speculative sampling);
 *   [P2] "The Architecture of Closure: How a Summary Message Encodes an Entire
 *        Engineering Session", section "The Table as a Decision Artifact"
 *        (tree_build, verify_attn, tree_accept and their chaining on device);
 *   [P3] "The Milestone Message: When an AI Summarizes Its Own Engineering
 *        Triumph", sections "MLA (Multi-Head Latent Attention)" and
 *        "Architectural Abstraction" (absorbed form; positions L+depth; the
 *        prefix fully visible, tree entries under the visibility mask).
 *
 * Conventions for every entry point:
 *  - Array arguments are DEVICE pointers to row-major, densely packed arrays
 *    owned by the caller; the library keeps no reference after the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A call
 *    only validates its scalar arguments on the host and enqueues kernels on
 *    `stream`: it never synchronizes, never reads device memory on the host and
 *    never allocates, so it may be recorded into a HIP graph.  The one
 *    exception is the measurement aid ddt_verify_attn_kernel_times, which
 *    waits for its own timing events.
 *  - Return value: DDT_OK, or a negative DDT_E* code with nothing enqueued (a
 *    launch failure, DDT_ELAUNCH, may leave earlier kernels of the same call
 *    enqueued).  ddt_last_error() then describes the failure.
 *  - Device-resident data is not validated on the host; out-of-range values are
 *    handled as documented per entry point and never cause out-of-bounds
 *    accesses.
 *  - Q = budget + 1 tree slots per request (the root plus `budget` draft
 *    nodes); W = ceil(Q / 64) 64-bit words per visibility row.
 */
#ifndef DDT_H
#define DDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DDT_OK 0
#define DDT_EINVAL (-1)       /* a scalar argument is out of range / NULL pointer */
#define DDT_EUNSUPPORTED (-2) /* valid but not compiled in (dtype / head dims)    */
#define DDT_ELAUNCH (-3)      /* the HIP runtime rejected a launch                 */

/* Element types of ddt_verify_attn's q_lat / q_pe / c_kv / k_pe. */
#define DDT_F32 0
#define DDT_BF16 1

/* Limits. */
#define DDT_MAX_Q 128        /* tree slots per request (budget <= 127)            */
#define DDT_MAX_DEPTH 64     /* drafter depth D                                   */
#define DDT_MAX_TOPK 64      /* drafter top-K                                     */
#define DDT_MAX_DK 4096      /* D * K                                             */
#define DDT_MAX_BATCH_ATTN 512 /* requests per ddt_verify_attn call               */
#define DDT_MAX_VOCAB 1048576  /* vocabulary of ddt_draft_topk                     */

/* Library version string, e.g. "ddt 0.1.0 gfx950". */
const char* ddt_version(void);

/* Message of the last failed call on the calling host thread ("" if none). */
const char* ddt_last_error(void);

/* ---------------------------------------------------------------------------
 * ddt_draft_topk -- per-depth top-K extraction from drafter logits ([P1] "What
 * to Build New", item 4: the fused draft helpers' per-depth top-k logit
 * extraction; its output is ddt_tree_build's topk_logp / topk_ids).
 *
 * Input (device): logits [B][D][V], element type `dtype` (DDT_F32 or DDT_BF16):
 *   the drafter's logits at depth d+1 of request b.
 * Scalars: B >= 1, D >= 1, B*D <= 65535, 1 <= K <= DDT_MAX_TOPK,
 *   K <= V <= DDT_MAX_VOCAB.
 * Outputs (device): topk_logp [B][D][K] f32, topk_ids [B][D][K] i32.
 * Workspace: device scratch of at least ddt_draft_topk_workspace_size(B, D, V, K)
 *   bytes, owned by the caller, clobbered (0 for invalid scalars).
 *
 * Semantics, per row: the K entries with the largest logits, largest first,
 * the lower index first among equal logits; topk_logp = logit - log sum_v
 * exp(logit_v) (natural log, fp32 accumulation; -inf for a -inf logit or an
 * all -inf row).  NaN logits count as -inf, -0 as +0.  The ids are exact; the
 * log-probs are within about 1e-6 of the exact value for V up to 2^20.
 * ------------------------------------------------------------------------- */
size_t ddt_draft_topk_workspace_size(int B, int D, int V, int K);

int ddt_draft_topk(const void* logits, int dtype, int B, int D, int V, int K, float* topk_logp,
                   int32_t* topk_ids, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ddt_tree_build -- best-first draft-tree construction ([P1] item 3; [P2]
 * tree_build row: replaces the per-request CPU heap queue and its host syncs).
 *
 * Inputs (device):
 *   topk_logp  [B][D][K] f32  drafter log-probs at depth d+1, rank order.
 *   topk_ids   [B][D][K] i32  the matching token ids.
 *   root_token [B]       i32  the verified token that roots each tree.
 *   prefix_len [B]       i32  committed prefix length L_b (positions only).
 * Scalars: 1 <= B, 0 <= D <= DDT_MAX_DEPTH, 0 <= K <= DDT_MAX_TOPK,
 *   D*K <= DDT_MAX_DK, 0 <= budget < DDT_MAX_Q.
 * Outputs (device), Q = budget+1 slots per request, node 0 = root:
 *   node_token, parent, depth, position, first_child, next_sibling [B][Q] i32,
 *   score [B][Q] f32, vis [B][Q][W] u64, n_nodes [B] i32 (root included).
 *
 * Semantics: a candidate is the rank-r token at depth d below a node p; its
 * score is score[p] + topk_logp[d-1][r] as one fp32 addition (root score 0).
 * Starting from the root's rank-0 child, repeatedly take the best candidate --
 * highest score, then lowest parent index, then lowest rank -- as the next node,
 * and offer its rank-0 child (if d < D) and its next-ranked sibling (if r+1 < K).
 * A candidate whose score is -inf or NaN is never offered.  Stop at Q nodes or
 * when nothing is on offer (underfull tree).  position = prefix_len + depth;
 * first_child = lowest-index child; next_sibling = next higher-index node with
 * the same parent; vis row i has bit k set iff node k is i or an ancestor of i.
 * Slots i >= n_nodes: all i32 fields -1, score -inf, vis 0.  Bit-exact
 * deterministic.  One 64-lane wavefront per request.
 * ------------------------------------------------------------------------- */
int ddt_tree_build(const float* topk_logp, const int32_t* topk_ids,
                   const int32_t* root_token, const int32_t* prefix_len,
                   int B, int D, int K, int budget,
                   int32_t* node_token, int32_t* parent, int32_t* depth,
                   int32_t* position, int32_t* first_child,
                   int32_t* next_sibling, float* score, uint64_t* vis,
                   int32_t* n_nodes, void* stream);

/* ---------------------------------------------------------------------------
 * ddt_verify_attn -- tree-verify attention in absorbed MLA form ([P1] item 2;
 * [P3] "MLA" and "Architectural Abstraction").
 *
 * Inputs (device; element type `dtype` for the four float tensors):
 *   q_lat [B][Q][H][d_lat]   absorbed query (q_nope times W_UK per head).
 *   q_pe  [B][Q][H][d_rope]  rotary part of the query.
 *   c_kv  [num_slots][d_lat] latent KV pool (paged, one token per page).
 *   k_pe  [num_slots][d_rope] rotary key pool.
 *   req_to_slot [B][max_kv] i32  pool slot of each KV entry of a request:
 *                    entries [0, L_b) are the prefix, entries [L_b, L_b+n_b)
 *                    are the tree nodes in node-index order.
 *   prefix_len [B] i32 (L_b), n_nodes [B] i32 (n_b), vis [B][Q][W] u64 (from
 *                    ddt_tree_build).
 * Scalars: 1 <= B <= DDT_MAX_BATCH_ATTN, 1 <= Q <= DDT_MAX_Q, H >= 1,
 *   max_kv >= 1, num_slots >= 1, (dtype, d_lat, d_rope) one of
 *   (DDT_BF16, 512, 64), (DDT_BF16, 64, 16), (DDT_F32, 64, 16);
 *   sm_scale finite and > 0.
 * Outputs (device): out [B][Q][H][d_lat] f32 (latent-space attention output),
 *   lse [B][Q][H] f32 natural-log sum-exp of the scaled scores (may be NULL).
 * Workspace: device scratch of at least
 *   ddt_verify_attn_workspace_size(B, Q, H, max_kv, d_lat) bytes, owned by the
 *   caller; its contents need no initialisation and are clobbered.
 *
 * Semantics, per request b, node i < n_b and head h:
 *   visible entries = prefix [0, L_b) and tree entries k < n_b with bit k of
 *   vis[b][i]; s_j = sm_scale * (q_lat . c_kv[slot_j] + q_pe . k_pe[slot_j]);
 *   out = sum_j softmax(s)_j * c_kv[slot_j]; lse = log sum_j exp(s_j).
 *   Rows with i >= n_b, or with no visible entry, get out = 0, lse = -inf.
 * Range handling: L_b is clamped to [0, max_kv] and n_b to
 *   [0, min(Q, max_kv - L_b)]; an entry whose slot id is outside
 *   [0, num_slots) is not visible.
 * Accuracy: fp32 accumulation; bf16 probabilities feed the value product.
 * Failure signal: the (DDT_BF16, 64, 16) and (DDT_F32, 64, 16) kernels pair
 *   two wavefronts of a workgroup through a bounded wait; if a wait ever gave
 *   up, the live rows of the wavefront that waited get out = NaN and
 *   lse = NaN (also after the split merge), so a give-up can never pass as a
 *   result.
 * ------------------------------------------------------------------------- */
size_t ddt_verify_attn_workspace_size(int B, int Q, int H, int max_kv, int d_lat);

int ddt_verify_attn(const void* q_lat, const void* q_pe, const void* c_kv,
                    const void* k_pe, int64_t num_slots,
                    const int32_t* req_to_slot, int max_kv,
                    const int32_t* prefix_len, const int32_t* n_nodes,
                    const uint64_t* vis, int B, int Q, int H, int d_lat,
                    int d_rope, int dtype, float sm_scale, float* out,
                    float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------
 * ddt_verify_attn_kernel_times -- measurement aid for ddt_verify_attn.
 *
 * Takes ddt_verify_attn's arguments, with the same checks and error codes,
 * plus reps (1 <= reps <= 100000) and kernel_ms, a HOST array of 2 floats.
 * Enqueues the call's attention kernel reps times back to back, then its
 * merge kernel reps times, with HIP events on `stream` around each run of
 * launches; waits for the last event and stores the mean time per launch in
 * milliseconds: kernel_ms[0] attention kernel, kernel_ms[1] merge kernel
 * (each includes the short gap between back-to-back launches).  out and lse
 * then hold the result of ddt_verify_attn.  Unlike every other entry point it
 * synchronizes (on its own events only) and so cannot be graph-captured.
 * ------------------------------------------------------------------------- */
int ddt_verify_attn_kernel_times(const void* q_lat, const void* q_pe, const void* c_kv,
                                 const void* k_pe, int64_t num_slots,
                                 const int32_t* req_to_slot, int max_kv,
                                 const int32_t* prefix_len, const int32_t* n_nodes,
                                 const uint64_t* vis, int B, int Q, int H, int d_lat,
                                 int d_rope, int dtype, float sm_scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int reps, float* kernel_ms);

/* ---------------------------------------------------------------------------
 * ddt_verify_attn_noalloc -- ddt_verify_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc): the same kernels and results, with the workspace
 * taken from a static device array that each GPU holds from the library's
 * first use until the process ends.
 *
 * Arguments, checks and outputs as for ddt_verify_attn, without the workspace.
 * The array holds ddt_verify_attn_noalloc_max_bytes() bytes (about 128.3 MiB),
 * the largest workspace ddt_verify_attn_workspace_size gives on a device of up
 * to 256 compute units; a call whose plan needs more returns DDT_EUNSUPPORTED
 * with nothing enqueued.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the first call on a device looks up that
 * device's copy of the array once.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined results; calls
 * ordered on one stream do not.  Nothing in the array needs clearing: each
 * call writes every entry it reads.
 * ------------------------------------------------------------------------- */
size_t ddt_verify_attn_noalloc_max_bytes(void);

int ddt_verify_attn_noalloc(const void* q_lat, const void* q_pe, const void* c_kv,
                            const void* k_pe, int64_t num_slots, const int32_t* req_to_slot,
                            int max_kv, const int32_t* prefix_len, const int32_t* n_nodes,
                            const uint64_t* vis, int B, int Q, int H, int d_lat, int d_rope,
                            int dtype, float sm_scale, float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * ddt_tree_accept -- greedy follow-the-verified-tree acceptance ([P2]
 * tree_accept row; composition with ddt_tree_build on device).
 *
 * Inputs (device): node_token, parent [B][Q] i32 and n_nodes [B] from
 *   ddt_tree_build; target_argmax [B][Q] i32, the target model's greedy next
 *   token at each tree node.
 * Scalars: 1 <= B, 1 <= Q <= DDT_MAX_Q.
 * Outputs (device):
 *   accept_len   [B]    number of accepted tree nodes including the root
 *                       (= accepted draft tokens + 1).
 *   accept_nodes [B][Q] the accepted root path, root first, -1 padded.
 *   out_tokens   [B][Q] accepted draft tokens followed by the bonus token
 *                       (target_argmax at the last accepted node), -1 padded.
 *   next_root    [B]    the bonus token (root of the next tree).
 * Semantics: from the root, move to the lowest-index child c (parent[c] == cur,
 * c > cur, c < n_b) whose node_token equals target_argmax[cur]; stop when there
 * is none.  n_b is clamped to [1, Q].  Bit-exact deterministic.
 * Precondition of a consistent step: L_b + n_b <= max_kv for the slot table
 *   that ddt_verify_attn and ddt_kv_commit use.  Those two clamp n_b to
 *   max_kv - L_b; this call does not see max_kv, so a tree that overran the
 *   table could accept a node that the commit then cuts off.
 * ------------------------------------------------------------------------- */
int ddt_tree_accept(const int32_t* node_token, const int32_t* parent,
                    const int32_t* n_nodes, const int32_t* target_argmax,
                    int B, int Q, int32_t* accept_len, int32_t* accept_nodes,
                    int32_t* out_tokens, int32_t* next_root, void* stream);

/* ---------------------------------------------------------------------------
 * ddt_tree_accept_sampling -- acceptance under temperature sampling ([P1]
 * "What to Build New", item 2: the sampling-probability path of tree
 * verification, normalized target probabilities at the tree nodes; "What to
 * Reuse", item 3: target-only tree speculative sampling from the verified
 * distribution; item 5: the temperature commit path).
 *
 * Inputs (device):
 *   target_logits [B][Q][V], element type `dtype` (DDT_F32 or DDT_BF16): the
 *                  target model's logits at every tree node (row i predicts the
 *                  token after node i); rows of nodes >= n_b are not read.
 *   temperature   [B] f32; a value that is not finite and > 0 (0, negative,
 *                  inf, NaN) makes the request greedy.
 *   node_token, parent [B][Q] i32 and n_nodes [B] from ddt_tree_build (n_b
 *                  clamped to [1, Q]).
 *   coins         [B][Q] f32 in [0, 1): the uniform draw used when node c is
 *                  tried as a child (each node is tried at most once).
 *   coin_final    [B] f32 in [0, 1): the draw for the bonus token.
 *   The caller draws the coins, so a seeded generator makes a call
 *   reproducible.
 * Scalars: 1 <= B, 1 <= Q <= DDT_MAX_Q, B*Q <= 2^24, 1 <= V <= DDT_MAX_VOCAB.
 * Outputs (device): accept_len, accept_nodes, out_tokens, next_root exactly as
 *   for ddt_tree_accept.
 * Workspace: device scratch of at least
 *   ddt_tree_accept_sampling_workspace_size(B, Q, V) bytes (0 for invalid
 *   scalars), owned by the caller, clobbered.
 * Semantics, per request, with p = softmax(logits[node] / T) (NaN logits count
 * as -inf): from the root, the children c of the current node (parent[c] ==
 * cur, c > cur, c < n_b) are tried in index order; a child whose token t lies
 * in [0, V) and was not tried before at this node is accepted when
 * coins[c] < p(t) / (1 - R), R the mass of the tokens rejected so far at this
 * node, and the walk moves to it.  When no child is accepted, the bonus token
 * is the first index v, in index order, of the residual r = p without the
 * rejected tokens whose running sum r(0) + ... + r(v) exceeds coin_final *
 * sum(r); the last v with r(v) > 0 if none does; the argmax if r is empty.  A
 * greedy request, and a node whose largest logit is not finite, use a point
 * mass on the argmax (the lowest index among the largest logits) and ignore
 * the coins: then the result equals ddt_tree_accept against the argmax tokens,
 * bit for bit.  Probabilities are computed in fp32 (about 1e-6 relative), so a
 * decision whose coin lies within that distance of its threshold may go the
 * other way than in exact arithmetic, and the bonus token may be a neighbour
 * of the exact one when the draw lies that close to an entry's boundary.
 * ------------------------------------------------------------------------- */
size_t ddt_tree_accept_sampling_workspace_size(int B, int Q, int V);

int ddt_tree_accept_sampling(const void* target_logits, int dtype, int V,
                             const float* temperature, const int32_t* node_token,
                             const int32_t* parent, const int32_t* n_nodes, const float* coins,
                             const float* coin_final, int B, int Q, int32_t* accept_len,
                             int32_t* accept_nodes, int32_t* out_tokens, int32_t* next_root,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ddt_kv_commit -- append the accepted path to the committed prefix ([P1]
 * "What to Build New", item 5: the paged MLA-latent KV cache and the "append"
 * step closing draft -> build -> verify -> accept; [P3] "Architectural
 * Abstraction": tree entries sit at positions L + depth).  With one token per
 * page this is a rewrite of the request's slot table.
 *
 * In/out (device): req_to_slot [B][max_kv] i32 (as for ddt_verify_attn: entries
 *   [L_b, L_b + n_b) are the tree nodes in node-index order), prefix_len [B] i32.
 * Inputs (device): n_nodes [B] i32 (ddt_tree_build), accept_len [B] and
 *   accept_nodes [B][Q] i32 (ddt_tree_accept: the root-first accepted path).
 * Scalars: 1 <= B, 1 <= Q <= DDT_MAX_Q, max_kv >= 1.
 * Outputs (device): freed_slots [B][Q] i32 -- the slot-table values of the tree
 *   entries not committed, in increasing node index, -1 padded; n_freed [B] i32.
 *
 * Semantics, per request b, with L = prefix_len[b] clamped to [0, max_kv],
 * n = n_nodes[b] clamped to [0, min(Q, max_kv - L)]: the path is
 * accept_nodes[b][0 .. a) for a = accept_len[b] clamped to [0, n], cut before
 * the first entry that is outside [0, n) or not larger than the one before it
 * (node indices increase along any root path).  Entry L + j (j < a) becomes
 * the slot of tree node path[j] (its value in req_to_slot before the call);
 * entries L + a .. L + n - 1 become -1; prefix_len[b] = L + a; the other
 * tree nodes' slots go to freed_slots.  Entries outside [L, L + n) are not
 * touched.  Node path[j] has depth j, so its KV, written at position L + j
 * during the verify step, is already where the committed prefix expects it.
 * Bit-exact deterministic.  One 64-lane wavefront per request.
 * ------------------------------------------------------------------------- */
int ddt_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                  const int32_t* n_nodes, const int32_t* accept_len,
                  const int32_t* accept_nodes, int B, int Q, int32_t* freed_slots,
                  int32_t* n_freed, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DDT_H */

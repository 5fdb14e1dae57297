/*
 * ddt_oracle.h -- plain CPU oracle for the DDTree tree-verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and ddt_oracle.c are the slow,
 * obviously-correct reference that the GPU library is checked against.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or constant with the HIP library.
 *
 * Sources ("the pages"):
 *   [P1] "The Architecture of a Thousand-Parameter Decision: Designing a Native
 *        DDTree Inference Engine for Kimi K2.6", section "What to Build New"
 *        (items 2 and 3: tree-verify MLA attention, GPU tree builder).
 *   [P2] "The Architecture of Closure: How a Summary Message Encodes an Entire
 *        Engineering Session", section "The Table as a Decision Artifact"
 *        (tree_build / verify_attn / tree_accept / composition test).
 *   [P3] "The Milestone Message: When an AI Summarizes Its Own Engineering
 *        Triumph", sections "MLA (Multi-Head Latent Attention)" and
 *        "Architectural Abstraction" (absorbed form; positions L+depth and the
 *        ones|visibility mask).
 *
 * Every function returns 0 on success, -1 on an invalid argument.
 * All arrays are host memory, row-major, owned by the caller.
 */
#ifndef DDT_ORACLE_H
#define DDT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Best-first draft-tree construction ([P1] item 3, [P2] tree_build row).
 *
 * in : topk_logp [B][D][K] f32 drafter log-probs per depth (rank 0 = best),
 *      topk_ids  [B][D][K] i32, root_token [B], prefix_len [B].
 * out: per request Q = budget+1 node slots:
 *      node_token, parent, depth, position, first_child, next_sibling [B][Q] i32,
 *      score [B][Q] f32, vis [B][Q][W] u64 (W = ceil(Q/64)), n_nodes [B]. */
int ddt_oracle_tree_build(const float* topk_logp, const int32_t* topk_ids,
                          const int32_t* root_token, const int32_t* prefix_len,
                          int B, int D, int K, int budget,
                          int32_t* node_token, int32_t* parent, int32_t* depth,
                          int32_t* position, int32_t* first_child,
                          int32_t* next_sibling, float* score, uint64_t* vis,
                          int32_t* n_nodes);

/* Tree-verify attention in MLA-absorbed form, evaluated in double precision
 * for a list of rows ([P1] item 2, [P3] "MLA").
 *
 * in : q_lat [B][Q][H][d_lat], q_pe [B][Q][H][d_rope] (f32; bf16 inputs are
 *      upcast exactly by the caller), c_kv [num_slots][d_lat],
 *      k_pe [num_slots][d_rope], req_to_slot [B][max_kv], prefix_len [B],
 *      n_nodes [B], vis [B][Q][W], sm_scale.
 *      rows [n_rows][3] = (b, i, h) triples to evaluate.
 * out: out [n_rows][d_lat] f64, lse [n_rows] f64 (natural log). */
int ddt_oracle_verify_attn_rows(const float* q_lat, const float* q_pe,
                                const float* c_kv, const float* k_pe,
                                int64_t num_slots, const int32_t* req_to_slot,
                                int max_kv, const int32_t* prefix_len,
                                const int32_t* n_nodes, const uint64_t* vis,
                                int B, int Q, int H, int d_lat, int d_rope,
                                float sm_scale, int64_t n_rows,
                                const int32_t* rows, double* out, double* lse);

/* All B*Q*H rows: out [B][Q][H][d_lat] f64, lse [B][Q][H] f64. */
int ddt_oracle_verify_attn(const float* q_lat, const float* q_pe,
                           const float* c_kv, const float* k_pe,
                           int64_t num_slots, const int32_t* req_to_slot,
                           int max_kv, const int32_t* prefix_len,
                           const int32_t* n_nodes, const uint64_t* vis,
                           int B, int Q, int H, int d_lat, int d_rope,
                           float sm_scale, double* out, double* lse);

/* Greedy follow-the-verified-tree acceptance ([P2] tree_accept row).
 *
 * in : node_token, parent [B][Q] (from the builder), n_nodes [B],
 *      target_argmax [B][Q] (the target model's greedy next token at each node).
 * out: accept_len [B], accept_nodes [B][Q], out_tokens [B][Q], next_root [B]. */
int ddt_oracle_tree_accept(const int32_t* node_token, const int32_t* parent,
                           const int32_t* n_nodes, const int32_t* target_argmax,
                           int B, int Q, int32_t* accept_len,
                           int32_t* accept_nodes, int32_t* out_tokens,
                           int32_t* next_root);

/* KV commit after acceptance ([P1] "What to Build New", item 5: append step;
 * [P3] "Architectural Abstraction": tree entries at positions L + depth).
 *
 * in/out: req_to_slot [B][max_kv] (entries [L, L+n) are the tree nodes in node
 *         order), prefix_len [B].
 * in    : n_nodes [B], accept_len [B], accept_nodes [B][Q] (root-first path).
 * out   : freed_slots [B][Q] (released slots in node order, -1 padded),
 *         n_freed [B].
 * With L and n clamped as for verification and the path cut before its first
 * entry outside [0, n) or not above its predecessor: entry L + j (j < a) takes
 * the slot of path node j, entries L + a .. L + n - 1 become -1, prefix_len =
 * L + a, and the slots of the other tree nodes are released. */
/* Per-depth top-K extraction ([P1] "What to Build New", item 4: per-depth
 * top-k logit extraction, the builder's input).
 *
 * in : logits [B][D][V] f32 (bf16 inputs upcast exactly by the caller).
 * out: topk_logp [B][D][K] f64 = logit - logsumexp(row) (natural log; -inf for
 *      a -inf logit or an all -inf row), topk_ids [B][D][K]: the K largest
 *      logits of the row, largest first, lower index first among equal logits.
 * NaN logits count as -inf.  Requires 1 <= K <= V. */
int ddt_oracle_draft_topk(const float* logits, int B, int D, int V, int K,
                          double* topk_logp, int32_t* topk_ids);

int ddt_oracle_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                         const int32_t* n_nodes, const int32_t* accept_len,
                         const int32_t* accept_nodes, int B, int Q,
                         int32_t* freed_slots, int32_t* n_freed);

/* Sampling acceptance ([P1] "What to Build New", item 2: the sampling-
 * probability path; "What to Reuse", item 3: target-only tree speculative
 * sampling from the verified distribution; item 5: the temperature commit).
 *
 * in : logits [B][Q][V] f32 (the target's logits at every tree node; bf16
 *      upcast exactly by the caller), temperature [B], node_token, parent
 *      [B][Q], n_nodes [B] (clamped to [1, Q]), coins [B][Q] (the uniform draw
 *      used when node c is tried as a child), coin_final [B] (the draw for the
 *      bonus token).
 * out: accept_len [B], accept_nodes [B][Q], out_tokens [B][Q], next_root [B]
 *      as for greedy acceptance.
 * Diagnostics (each may be NULL): margin [B] = the smallest |coin - p_res| of
 *      the request's sampled acceptance tests (+inf if none); bonus_lo/hi [B] =
 *      the index range of residual entries whose CDF interval comes within
 *      band_eps * (residual mass) of the bonus draw's target.
 * Readings R16 (target-only rejection sampling, children in index order,
 * inverse-CDF bonus) and R17 (greedy requests and nodes) are spelt out above
 * the definition. */
int ddt_oracle_tree_accept_sampling(const float* logits, int V, const float* temperature,
                                    const int32_t* node_token, const int32_t* parent,
                                    const int32_t* n_nodes, const float* coins,
                                    const float* coin_final, int B, int Q, double band_eps,
                                    int32_t* accept_len, int32_t* accept_nodes,
                                    int32_t* out_tokens, int32_t* next_root, double* margin,
                                    int32_t* bonus_lo, int32_t* bonus_hi);

/* Number of OpenMP threads the oracle runs with (1 if built without OpenMP). */
int ddt_oracle_num_threads(void);
/* Threads of the later parallel regions (n >= 1); returns the new count. */
int ddt_oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif /* DDT_ORACLE_H */

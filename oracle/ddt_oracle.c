/*
 * ddt_oracle.c -- plain CPU oracle for the DDTree tree-verify step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the library's product path.  It is
 * written for a reader who checks it against the pages by eye: no blocking, no
 * fusion, no reordering beyond what each definition states.  Attention runs in
 * double precision; the tree builder runs the pages' best-first expansion with
 * an ordinary binary heap in fp32 scores (the score type the builder's inputs
 * carry).
 *
 * Sources are listed in ddt_oracle.h ([P1], [P2], [P3]).
 *
 * Readings taken where the pages leave a step open (all listed in the design
 * notes as well):
 *   R1  The best-first key is the cumulative drafter log-prob of the path
 *       (score of the parent plus the log-prob of the rank at that depth, one
 *       fp32 addition).  Ties go to the lower parent node index, then to the
 *       lower rank.
 *   R2  A candidate whose score is not greater than -inf (-inf or NaN) is never
 *       put on the frontier, so trees may be underfull (n_nodes < Q).
 *   R3  Node i sees itself and all its ancestors (root included); the tree
 *       entries of the KV cache follow the prefix in node-index order.
 *   R4  The value vector is the latent c_kv row; the output stays latent.
 *   R9  Acceptance moves to the lowest-index child whose token equals the
 *       target's greedy token at the current node.
 *   R10 accept_len counts the root, i.e. accepted drafts + 1 (the bonus token).
 *
 * Range handling of device-side data (shared contract with the GPU library):
 *   prefix length L_b is clamped to [0, max_kv]; the number of tree entries n_b
 *   to [0, min(Q, max_kv - L_b)] in attention and to [1, Q] in acceptance; a
 *   slot id outside [0, num_slots) contributes no key; an acceptance child link
 *   must point forward (child index > current node).
 */
#include "ddt_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ddt_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int ddt_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Tree build: best-first expansion ([P1] "What to Build New" item 3; [P2]    */
/* tree_build row, which replaces the per-request CPU heap queue).            */
/* ------------------------------------------------------------------------ */

/* A frontier entry: the rank-th candidate token at depth `depth` below node
 * `parent`, with its cumulative score. */
typedef struct {
  float score;
  int parent;
  int depth;
  int rank;
} cand_t;

/* R1: a comes out of the frontier before b. */
static int cand_before(const cand_t* a, const cand_t* b) {
  if (a->score != b->score) return a->score > b->score;
  if (a->parent != b->parent) return a->parent < b->parent;
  return a->rank < b->rank;
}

typedef struct {
  cand_t* v;
  int n;
} heap_t;

static void heap_push(heap_t* h, cand_t c) {
  int i = h->n++;
  h->v[i] = c;
  while (i > 0) {
    int up = (i - 1) / 2;
    if (!cand_before(&h->v[i], &h->v[up])) break;
    cand_t t = h->v[i];
    h->v[i] = h->v[up];
    h->v[up] = t;
    i = up;
  }
}

static cand_t heap_pop(heap_t* h) {
  cand_t top = h->v[0];
  h->v[0] = h->v[--h->n];
  int i = 0;
  for (;;) {
    int l = 2 * i + 1, r = l + 1, m = i;
    if (l < h->n && cand_before(&h->v[l], &h->v[m])) m = l;
    if (r < h->n && cand_before(&h->v[r], &h->v[m])) m = r;
    if (m == i) break;
    cand_t t = h->v[i];
    h->v[i] = h->v[m];
    h->v[m] = t;
    i = m;
  }
  return top;
}

/* R2: only finite-or-+inf scores enter the frontier. */
static void push_if_live(heap_t* h, cand_t c) {
  if (c.score > -INFINITY) heap_push(h, c);
}

static void build_one(const float* logp, const int32_t* ids, int32_t root_tok,
                      int32_t L, int D, int K, int Q, int W, int32_t* tok,
                      int32_t* par, int32_t* dep, int32_t* pos, int32_t* fc,
                      int32_t* ns, float* sc, uint64_t* vis, int32_t* n_out) {
  /* The frontier never holds more than one entry per popped node plus one. */
  cand_t* store = (cand_t*)malloc(sizeof(cand_t) * (size_t)(Q + 2));
  heap_t h = {store, 0};

  for (int i = 0; i < Q; ++i) {
    tok[i] = par[i] = dep[i] = pos[i] = fc[i] = ns[i] = -1;
    sc[i] = -INFINITY;
    for (int w = 0; w < W; ++w) vis[(size_t)i * W + w] = 0;
  }

  /* Node 0 is the root: the verified token, depth 0, score 0. */
  int n = 1;
  tok[0] = root_tok;
  par[0] = -1;
  dep[0] = 0;
  sc[0] = 0.0f;

  if (D >= 1 && K >= 1) {
    cand_t c = {sc[0] + logp[0], 0, 1, 0};
    push_if_live(&h, c);
  }
  while (n < Q && h.n > 0) {
    cand_t c = heap_pop(&h);
    int i = n++;
    tok[i] = ids[(size_t)(c.depth - 1) * K + c.rank];
    par[i] = c.parent;
    dep[i] = c.depth;
    sc[i] = c.score;
    /* Its best child (rank 0 one level deeper) ... */
    if (c.depth < D) {
      cand_t child = {sc[i] + logp[(size_t)c.depth * K], i, c.depth + 1, 0};
      push_if_live(&h, child);
    }
    /* ... and its next-ranked sibling under the same parent. */
    if (c.rank + 1 < K) {
      float s = sc[c.parent] + logp[(size_t)(c.depth - 1) * K + c.rank + 1];
      cand_t sib = {s, c.parent, c.depth, c.rank + 1};
      push_if_live(&h, sib);
    }
  }
  *n_out = n;
  free(store);

  /* Derived arrays ([P1] item 3: parents, visibility mask, first-child and
   * next-sibling links; [P3] "Architectural Abstraction": position L+depth). */
  for (int i = 0; i < n; ++i) {
    pos[i] = (int32_t)((uint32_t)L + (uint32_t)dep[i]);
    for (int c = i + 1; c < n; ++c)
      if (par[c] == i) { fc[i] = c; break; }
    if (i > 0)
      for (int c = i + 1; c < n; ++c)
        if (par[c] == par[i]) { ns[i] = c; break; }
    /* R3: ancestors and self. */
    for (int a = i; a >= 0; a = par[a])
      vis[(size_t)i * W + a / 64] |= (uint64_t)1 << (a % 64);
  }
}

int ddt_oracle_tree_build(const float* topk_logp, const int32_t* topk_ids,
                          const int32_t* root_token, const int32_t* prefix_len,
                          int B, int D, int K, int budget,
                          int32_t* node_token, int32_t* parent, int32_t* depth,
                          int32_t* position, int32_t* first_child,
                          int32_t* next_sibling, float* score, uint64_t* vis,
                          int32_t* n_nodes) {
  if (B < 0 || D < 0 || K < 0 || budget < 0) return -1;
  const int Q = budget + 1;
  const int W = (Q + 63) / 64;
#pragma omp parallel for schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    size_t q0 = (size_t)b * Q;
    build_one(topk_logp + (size_t)b * D * K, topk_ids + (size_t)b * D * K,
              root_token[b], prefix_len[b], D, K, Q, W, node_token + q0,
              parent + q0, depth + q0, position + q0, first_child + q0,
              next_sibling + q0, score + q0, vis + q0 * W, n_nodes + b);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Verify attention ([P1] item 2: absorbed MLA over a shared paged latent     */
/* prefix plus the tree-node entries under a visibility mask; [P3] "MLA").    */
/* ------------------------------------------------------------------------ */

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

static void attn_row(const float* q_lat, const float* q_pe, const float* c_kv,
                     const float* k_pe, int64_t num_slots,
                     const int32_t* req_to_slot, int max_kv,
                     const int32_t* prefix_len, const int32_t* n_nodes,
                     const uint64_t* vis, int Q, int H, int d_lat, int d_rope,
                     double scale, int b, int i, int h, double* out,
                     double* lse, int32_t* keys, double* s) {
  const int W = (Q + 63) / 64;
  const int L = clampi(prefix_len[b], 0, max_kv);
  const int nb = clampi(n_nodes[b], 0, (Q < max_kv - L) ? Q : max_kv - L);
  for (int c = 0; c < d_lat; ++c) out[c] = 0.0;
  *lse = -INFINITY;
  if (i >= nb) return; /* padding row */

  /* The set of visible KV slots: the whole prefix, then (R3) the tree entries
   * whose bit is set in this node's visibility row. */
  const int32_t* slots = req_to_slot + (size_t)b * max_kv;
  const uint64_t* vrow = vis + ((size_t)b * Q + i) * W;
  int n = 0;
  for (int j = 0; j < L; ++j) keys[n++] = slots[j];
  for (int k = 0; k < nb; ++k)
    if ((vrow[k / 64] >> (k % 64)) & 1u) keys[n++] = slots[L + k];

  const size_t row = ((size_t)b * Q + i) * H + h;
  const float* ql = q_lat + row * d_lat;
  const float* qp = q_pe + row * d_rope;

  /* Scores: scale * (q_lat . c_kv + q_pe . k_pe). */
  double m = -INFINITY;
  int live = 0;
  for (int t = 0; t < n; ++t) {
    int64_t sl = keys[t];
    if (sl < 0 || sl >= num_slots) { s[t] = -INFINITY; continue; }
    double acc = 0.0;
    for (int c = 0; c < d_lat; ++c) acc += (double)ql[c] * (double)c_kv[sl * d_lat + c];
    for (int c = 0; c < d_rope; ++c) acc += (double)qp[c] * (double)k_pe[sl * d_rope + c];
    s[t] = scale * acc;
    if (s[t] > m) m = s[t];
    ++live;
  }
  if (live == 0) return;

  /* Softmax over the visible set, value = latent row (R4). */
  double z = 0.0;
  for (int t = 0; t < n; ++t) {
    if (s[t] == -INFINITY) continue;
    double p = exp(s[t] - m);
    z += p;
    const float* v = c_kv + (int64_t)keys[t] * d_lat;
    for (int c = 0; c < d_lat; ++c) out[c] += p * (double)v[c];
  }
  for (int c = 0; c < d_lat; ++c) out[c] /= z;
  *lse = m + log(z);
}

int ddt_oracle_verify_attn_rows(const float* q_lat, const float* q_pe,
                                const float* c_kv, const float* k_pe,
                                int64_t num_slots, const int32_t* req_to_slot,
                                int max_kv, const int32_t* prefix_len,
                                const int32_t* n_nodes, const uint64_t* vis,
                                int B, int Q, int H, int d_lat, int d_rope,
                                float sm_scale, int64_t n_rows,
                                const int32_t* rows, double* out, double* lse) {
  if (B < 0 || Q < 1 || H < 1 || d_lat < 1 || d_rope < 0 || max_kv < 0 || n_rows < 0)
    return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
    if (b < 0 || b >= B || i < 0 || i >= Q || h < 0 || h >= H) return -1;
  }
  int bad = 0;
#pragma omp parallel
  {
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(max_kv + 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv + 1));
    if (!keys || !s) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n_rows; ++r)
        attn_row(q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv,
                 prefix_len, n_nodes, vis, Q, H, d_lat, d_rope, (double)sm_scale,
                 rows[3 * r], rows[3 * r + 1], rows[3 * r + 2],
                 out + r * d_lat, lse + r, keys, s);
    }
    free(keys);
    free(s);
  }
  return bad ? -1 : 0;
}

int ddt_oracle_verify_attn(const float* q_lat, const float* q_pe,
                           const float* c_kv, const float* k_pe,
                           int64_t num_slots, const int32_t* req_to_slot,
                           int max_kv, const int32_t* prefix_len,
                           const int32_t* n_nodes, const uint64_t* vis,
                           int B, int Q, int H, int d_lat, int d_rope,
                           float sm_scale, double* out, double* lse) {
  if (B < 0 || Q < 1 || H < 1) return -1;
  int64_t n_rows = (int64_t)B * Q * H;
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)(n_rows + 1));
  if (!rows) return -1;
  int64_t r = 0;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < Q; ++i)
      for (int h = 0; h < H; ++h, ++r) {
        rows[3 * r] = b;
        rows[3 * r + 1] = i;
        rows[3 * r + 2] = h;
      }
  int rc = ddt_oracle_verify_attn_rows(q_lat, q_pe, c_kv, k_pe, num_slots,
                                       req_to_slot, max_kv, prefix_len, n_nodes,
                                       vis, B, Q, H, d_lat, d_rope, sm_scale,
                                       n_rows, rows, out, lse);
  free(rows);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Greedy acceptance ([P2] tree_accept row: follow the verified tree; the     */
/* composition test feeds it a synthesized target prediction).               */
/* ------------------------------------------------------------------------ */

int ddt_oracle_tree_accept(const int32_t* node_token, const int32_t* parent,
                           const int32_t* n_nodes, const int32_t* target_argmax,
                           int B, int Q, int32_t* accept_len,
                           int32_t* accept_nodes, int32_t* out_tokens,
                           int32_t* next_root) {
  if (B < 0 || Q < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int b = 0; b < B; ++b) {
    const int32_t* tok = node_token + (size_t)b * Q;
    const int32_t* par = parent + (size_t)b * Q;
    const int32_t* tgt = target_argmax + (size_t)b * Q;
    int32_t* path = accept_nodes + (size_t)b * Q;
    int32_t* outt = out_tokens + (size_t)b * Q;
    const int nb = clampi(n_nodes[b], 1, Q);
    for (int i = 0; i < Q; ++i) path[i] = outt[i] = -1;

    int len = 1, cur = 0;
    path[0] = 0;
    for (;;) {
      int32_t want = tgt[cur];
      int next = -1;
      for (int c = cur + 1; c < nb; ++c) /* R9: lowest index wins */
        if (par[c] == cur && tok[c] == want) { next = c; break; }
      if (next < 0) break;
      path[len++] = next;
      cur = next;
    }
    /* Accepted draft tokens, then the target's own token after the last one. */
    for (int k = 1; k < len; ++k) outt[k - 1] = tok[path[k]];
    outt[len - 1] = tgt[cur];
    accept_len[b] = len; /* R10 */
    next_root[b] = tgt[cur];
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* KV commit after acceptance ([P1] "What to Build New", item 5: the paged   */
/* latent KV cache and the append step that ends each DDTree step; [P3]      */
/* "Architectural Abstraction": tree entries at positions L + depth).        */
/* One token per page, so committing the accepted root path is a rewrite of  */
/* the request's slot table.                                                 */
/* ------------------------------------------------------------------------ */

int ddt_oracle_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                         const int32_t* n_nodes, const int32_t* accept_len,
                         const int32_t* accept_nodes, int B, int Q,
                         int32_t* freed_slots, int32_t* n_freed) {
  if (B < 0 || Q < 1 || Q > 128 || max_kv < 1) return -1;
  for (int b = 0; b < B; ++b) {
    int32_t* row = req_to_slot + (size_t)b * max_kv;
    const int32_t* path = accept_nodes + (size_t)b * Q;
    int32_t* freed = freed_slots + (size_t)b * Q;
    const int L = clampi(prefix_len[b], 0, max_kv);
    const int n = clampi(n_nodes[b], 0, Q < max_kv - L ? Q : max_kv - L);
    int a = clampi(accept_len[b], 0, n);
    /* The committed path stops before the first entry that is not a tree node
       or does not come after the previous one (indices grow along a path). */
    for (int j = 0; j < a; ++j) {
      const int node = path[j];
      if (node < 0 || node >= n || (j > 0 && node <= path[j - 1])) { a = j; break; }
    }
    /* Copy the tree entries' slots before rewriting them. */
    int32_t old[128];
    int on_path[128];
    for (int k = 0; k < n; ++k) { old[k] = row[L + k]; on_path[k] = 0; }
    for (int j = 0; j < a; ++j) on_path[path[j]] = 1;
    /* Path node j (at depth j) becomes prefix entry L + j. */
    for (int j = 0; j < n; ++j) row[L + j] = j < a ? old[path[j]] : -1;
    /* The other tree nodes' slots are released, in node order. */
    int m = 0;
    for (int k = 0; k < n; ++k)
      if (!on_path[k]) freed[m++] = old[k];
    for (int k = m; k < Q; ++k) freed[k] = -1;
    n_freed[b] = m;
    prefix_len[b] = L + a;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-depth top-K extraction ([P1] "What to Build New", item 4: the fused   */
/* draft helpers' per-depth top-k logit extraction that feeds the builder).  */
/* Each (request, depth) row: log-softmax over the vocabulary, then the K    */
/* entries with the largest logits (lower index first among equal logits).   */
/* NaN logits count as -inf.                                                 */
/* ------------------------------------------------------------------------ */

int ddt_oracle_draft_topk(const float* logits, int B, int D, int V, int K,
                          double* topk_logp, int32_t* topk_ids) {
  if (B < 0 || D < 0 || V < 1 || K < 1 || K > V) return -1;
  const long long rows = (long long)B * D;
#pragma omp parallel for schedule(dynamic)
  for (long long r = 0; r < rows; ++r) {
    const float* x = logits + r * (long long)V;
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
      const double xv = isnan(x[v]) ? -INFINITY : (double)x[v];
      if (xv > m) m = xv;
    }
    double lse = -INFINITY;
    if (m > -INFINITY) {
      double sum = 0.0;
      for (int v = 0; v < V; ++v) {
        const double xv = isnan(x[v]) ? -INFINITY : (double)x[v];
        sum += exp(xv - m);
      }
      lse = m + log(sum);
    }
    /* K rounds of "largest remaining logit, lowest index on a tie". */
    unsigned char* taken = (unsigned char*)calloc((size_t)V, 1);
    for (int k = 0; k < K; ++k) {
      int best = -1;
      double bv = 0.0;
      for (int v = 0; v < V; ++v) {
        if (taken[v]) continue;
        const double xv = isnan(x[v]) ? -INFINITY : (double)x[v];
        if (best < 0 || xv > bv) { best = v; bv = xv; }
      }
      taken[best] = 1;
      topk_ids[r * K + k] = best;
      topk_logp[r * K + k] = (bv == -INFINITY || lse == -INFINITY) ? -INFINITY : bv - lse;
    }
    free(taken);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampling acceptance ([P1] "What to Build New", item 2: the sampling-      */
/* probability path of tree verification, normalized target probabilities   */
/* at every tree node; [P1] "What to Reuse": the target-only tree            */
/* speculative-sampling step that samples from the verified distribution;   */
/* item 5: the temperature commit path).                                     */
/*                                                                           */
/* Readings (the pages name the step but do not spell it out):               */
/*   R16 The drafted tokens are fixed choices, so the draft distribution is   */
/*       a point mass on each drafted token and only the target's            */
/*       probabilities enter ("target only").  At node `cur` the target       */
/*       distribution is p = softmax(logits[cur] / T).  Its children are     */
/*       tried in index order; a child with token t is accepted when          */
/*       coin[child] < p(t) / (1 - R), R the mass of the tokens already      */
/*       rejected at this node; otherwise t joins the rejected set.  A token  */
/*       outside [0, V), or one already rejected, has probability 0 and is   */
/*       never accepted.  The walk moves to the accepted child.  When no      */
/*       child is accepted, the bonus token is drawn from the residual        */
/*       r(v) = p(v) for v not rejected (0 otherwise) by inverse CDF: the     */
/*       first v in index order with r(v) > 0 and r(0) + ... + r(v) >         */
/*       coin_final * (r(0) + ... + r(V-1)); if none qualifies (rounding, or  */
/*       coin_final >= 1) the last v with r(v) > 0; if the residual is       */
/*       empty, the argmax.                                                   */
/*   R17 A request whose temperature is not a finite value > 0, and a node    */
/*       whose largest logit is not finite (all -inf, or a +inf entry), is    */
/*       taken greedily: p is a point mass on the argmax (lowest index among  */
/*       equal logits; NaN counts as -inf).  Coins are then not consulted,    */
/*       and the result equals greedy acceptance against the argmax tokens.  */
/* ------------------------------------------------------------------------ */

int ddt_oracle_tree_accept_sampling(const float* logits, int V, const float* temperature,
                                    const int32_t* node_token, const int32_t* parent,
                                    const int32_t* n_nodes, const float* coins,
                                    const float* coin_final, int B, int Q, double band_eps,
                                    int32_t* accept_len, int32_t* accept_nodes,
                                    int32_t* out_tokens, int32_t* next_root, double* margin,
                                    int32_t* bonus_lo, int32_t* bonus_hi) {
  if (B < 0 || Q < 1 || V < 1) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    const int32_t* tok = node_token + (size_t)b * Q;
    const int32_t* par = parent + (size_t)b * Q;
    const float* coin = coins + (size_t)b * Q;
    int32_t* path = accept_nodes + (size_t)b * Q;
    int32_t* outt = out_tokens + (size_t)b * Q;
    const int nb = clampi(n_nodes[b], 1, Q);
    const double T = (double)temperature[b];
    const int greedy_req = !(T > 0.0 && isfinite(T));
    double* p = (double*)malloc((size_t)V * sizeof(double));
    unsigned char* rejected = (unsigned char*)calloc((size_t)V, 1);
    double min_margin = INFINITY;
    for (int i = 0; i < Q; ++i) path[i] = outt[i] = -1;

    int len = 1, cur = 0, bonus = -1, blo = -1, bhi = -1;
    path[0] = 0;
    for (;;) {
      /* The target distribution at node cur. */
      const float* x = logits + ((size_t)b * Q + cur) * (size_t)V;
      double M = -INFINITY;
      int amax = 0;
      for (int v = 0; v < V; ++v) {
        const double xv = isnan(x[v]) ? -INFINITY : (double)x[v];
        if (xv > M) { M = xv; amax = v; }
      }
      const int greedy = greedy_req || !isfinite(M);
      if (greedy) {
        for (int v = 0; v < V; ++v) p[v] = v == amax ? 1.0 : 0.0;
      } else {
        double Z = 0.0;
        for (int v = 0; v < V; ++v) {
          const double xv = isnan(x[v]) ? -INFINITY : (double)x[v];
          p[v] = exp((xv - M) / T);
          Z += p[v];
        }
        for (int v = 0; v < V; ++v) p[v] /= Z;
      }
      /* Try the children in index order. */
      memset(rejected, 0, (size_t)V);
      double R = 0.0;
      int next = -1;
      for (int c = cur + 1; c < nb; ++c) {
        if (par[c] != cur) continue;
        const int t = tok[c];
        if (t < 0 || t >= V || rejected[t] || !(p[t] > 0.0)) continue;
        if (greedy) { next = c; break; }  /* t is the argmax */
        const double pres = p[t] / (1.0 - R);
        const double d = fabs((double)coin[c] - pres);
        if (d < min_margin) min_margin = d;
        if ((double)coin[c] < pres) { next = c; break; }
        rejected[t] = 1;
        R += p[t];
      }
      if (next >= 0) {
        path[len++] = next;
        cur = next;
        continue;
      }
      /* No child accepted: the bonus token from the residual distribution. */
      if (greedy) {
        bonus = blo = bhi = amax;
        break;
      }
      double Zr = 0.0;
      int last = -1;
      for (int v = 0; v < V; ++v)
        if (!rejected[v] && p[v] > 0.0) { Zr += p[v]; last = v; }
      if (last < 0) {
        bonus = blo = bhi = amax;
        break;
      }
      const double target = (double)coin_final[b] * Zr;
      double cum = 0.0;
      for (int v = 0; v < V; ++v) {
        if (rejected[v] || !(p[v] > 0.0)) continue;
        cum += p[v];
        if (cum > target) { bonus = v; break; }
      }
      if (bonus < 0) bonus = last;
      /* Entries whose residual CDF interval comes within band_eps * Zr of the
         target: every one of them is a correct draw for a coin that far off. */
      cum = 0.0;
      for (int v = 0; v < V; ++v) {
        if (rejected[v] || !(p[v] > 0.0)) continue;
        const double lo = cum;
        cum += p[v];
        if (cum >= target - band_eps * Zr && lo <= target + band_eps * Zr) {
          if (blo < 0) blo = v;
          bhi = v;
        }
      }
      if (blo < 0 || bonus < blo) blo = bonus;
      if (bonus > bhi) bhi = bonus;
      break;
    }
    for (int k = 1; k < len; ++k) outt[k - 1] = tok[path[k]];
    outt[len - 1] = bonus;
    accept_len[b] = len;
    next_root[b] = bonus;
    if (margin) margin[b] = min_margin;
    if (bonus_lo) bonus_lo[b] = blo;
    if (bonus_hi) bonus_hi[b] = bhi;
    free(p);
    free(rejected);
  }
  return 0;
}

// api.hip -- the exported C entry points of libddt.so (declared in ddt.h).
//
// Each entry point validates its scalar arguments and pointers on the host,
// then enqueues its kernels on the caller's stream.  No entry point reads
// device memory on the host or allocates, and all but one never synchronize,
// so they may be captured into a HIP graph.  The exception is the measurement
// aid ddt_verify_attn_kernel_times, which waits for its own timing events.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/ddt.h"
#include "ddt_internal.h"

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace ddt {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DDT_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DDT_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int device_cu_count() {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cu;
}

bool attn_variant_supported(int dtype, int d_lat, int d_rope) {
  return (dtype == DDT_BF16 && d_lat == 512 && d_rope == 64) ||
         (dtype == DDT_BF16 && d_lat == 64 && d_rope == 16) ||
         (dtype == DDT_F32 && d_lat == 64 && d_rope == 16);
}

}  // namespace ddt

using ddt::attn_variant_supported;
using ddt::device_cu_count;
using ddt::fail;
using ddt::launch_status;
using ddt::ok;

namespace ddt {

int check_verify_attn(const char* who, const void* q_lat, const void* q_pe, const void* c_kv,
                      const void* k_pe, int64_t num_slots, const int32_t* req_to_slot,
                      int max_kv, const int32_t* prefix_len, const int32_t* n_nodes,
                      const uint64_t* vis, int B, int Q, int H, int d_lat, int d_rope,
                      int dtype, float sm_scale, const float* out, const void* workspace,
                      size_t workspace_bytes, bool check_ws, AttnPlan& plan) {
  if (B < 1 || B > DDT_MAX_BATCH_ATTN)
    return fail(DDT_EINVAL, "%s: B=%d outside [1, %d]", who, B, DDT_MAX_BATCH_ATTN);
  if (Q < 1 || Q > DDT_MAX_Q)
    return fail(DDT_EINVAL, "%s: Q=%d outside [1, %d]", who, Q, DDT_MAX_Q);
  if (H < 1) return fail(DDT_EINVAL, "%s: H=%d must be >= 1", who, H);
  if (max_kv < 1) return fail(DDT_EINVAL, "%s: max_kv=%d must be >= 1", who, max_kv);
  if (num_slots < 1)
    return fail(DDT_EINVAL, "%s: num_slots=%lld must be >= 1", who, (long long)num_slots);
  if (dtype != DDT_F32 && dtype != DDT_BF16)
    return fail(DDT_EINVAL, "%s: dtype=%d is not DDT_F32 or DDT_BF16", who, dtype);
  if (!(sm_scale > 0.0f) || sm_scale == INFINITY)
    return fail(DDT_EINVAL, "%s: sm_scale must be finite and > 0", who);
  if (!attn_variant_supported(dtype, d_lat, d_rope))
    return fail(DDT_EUNSUPPORTED,
                "%s: (dtype=%d, d_lat=%d, d_rope=%d) not compiled in; supported: "
                "(bf16,512,64) (bf16,64,16) (f32,64,16)", who, dtype, d_lat, d_rope);
  if (!q_lat || !q_pe || !c_kv || !k_pe || !req_to_slot || !prefix_len || !n_nodes || !vis ||
      !out)
    return fail(DDT_EINVAL, "%s: NULL array argument", who);
  plan = ddt::plan_verify_attn(B, Q, H, max_kv, d_lat, device_cu_count());
  if (check_ws && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(DDT_EINVAL, "%s: workspace of %zu bytes given, %zu needed", who,
                workspace ? workspace_bytes : (size_t)0, plan.ws_bytes);
  return DDT_OK;
}

}  // namespace ddt

using ddt::check_verify_attn;

extern "C" {

const char* ddt_version(void) { return "ddt 0.1.0 gfx950"; }

const char* ddt_last_error(void) { return g_err; }

int ddt_tree_build(const float* topk_logp, const int32_t* topk_ids, const int32_t* root_token,
                   const int32_t* prefix_len, int B, int D, int K, int budget,
                   int32_t* node_token, int32_t* parent, int32_t* depth, int32_t* position,
                   int32_t* first_child, int32_t* next_sibling, float* score, uint64_t* vis,
                   int32_t* n_nodes, void* stream) {
  if (B < 1) return fail(DDT_EINVAL, "ddt_tree_build: B=%d must be >= 1", B);
  if (D < 0 || D > DDT_MAX_DEPTH)
    return fail(DDT_EINVAL, "ddt_tree_build: D=%d outside [0, %d]", D, DDT_MAX_DEPTH);
  if (K < 0 || K > DDT_MAX_TOPK)
    return fail(DDT_EINVAL, "ddt_tree_build: K=%d outside [0, %d]", K, DDT_MAX_TOPK);
  if (D * K > DDT_MAX_DK)
    return fail(DDT_EINVAL, "ddt_tree_build: D*K=%d exceeds %d", D * K, DDT_MAX_DK);
  if (budget < 0 || budget + 1 > DDT_MAX_Q)
    return fail(DDT_EINVAL, "ddt_tree_build: budget=%d outside [0, %d]", budget, DDT_MAX_Q - 1);
  if ((D * K > 0 && (!topk_logp || !topk_ids)) || !root_token || !prefix_len || !node_token ||
      !parent || !depth || !position || !first_child || !next_sibling || !score || !vis ||
      !n_nodes)
    return fail(DDT_EINVAL, "ddt_tree_build: NULL array argument");
  const hipError_t e = ddt::launch_tree_build(
      topk_logp, topk_ids, root_token, prefix_len, B, D, K, budget + 1, node_token, parent,
      depth, position, first_child, next_sibling, score, vis, n_nodes,
      static_cast<hipStream_t>(stream));
  return launch_status(e, "ddt_tree_build");
}

size_t ddt_verify_attn_workspace_size(int B, int Q, int H, int max_kv, int d_lat) {
  if (B < 1 || Q < 1 || H < 1 || max_kv < 1 || d_lat < 1) return 0;
  return ddt::plan_verify_attn(B, Q, H, max_kv, d_lat, device_cu_count()).ws_bytes;
}


int ddt_verify_attn(const void* q_lat, const void* q_pe, const void* c_kv, const void* k_pe,
                    int64_t num_slots, const int32_t* req_to_slot, int max_kv,
                    const int32_t* prefix_len, const int32_t* n_nodes, const uint64_t* vis,
                    int B, int Q, int H, int d_lat, int d_rope, int dtype, float sm_scale,
                    float* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  ddt::AttnPlan plan;
  const int rc = check_verify_attn("ddt_verify_attn", q_lat, q_pe, c_kv, k_pe, num_slots,
                                   req_to_slot, max_kv, prefix_len, n_nodes, vis, B, Q, H,
                                   d_lat, d_rope, dtype, sm_scale, out, workspace,
                                   workspace_bytes, true, plan);
  if (rc != DDT_OK) return rc;
  const hipError_t e = ddt::launch_verify_attn(
      dtype, d_lat, d_rope, q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv, prefix_len,
      n_nodes, vis, B, Q, H, sm_scale, out, lse, workspace, plan,
      static_cast<hipStream_t>(stream));
  return launch_status(e, "ddt_verify_attn");
}

int ddt_verify_attn_kernel_times(const void* q_lat, const void* q_pe, const void* c_kv,
                                 const void* k_pe, int64_t num_slots,
                                 const int32_t* req_to_slot, int max_kv,
                                 const int32_t* prefix_len, const int32_t* n_nodes,
                                 const uint64_t* vis, int B, int Q, int H, int d_lat,
                                 int d_rope, int dtype, float sm_scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int reps, float* kernel_ms) {
  static const char* who = "ddt_verify_attn_kernel_times";
  if (reps < 1 || reps > 100000)
    return fail(DDT_EINVAL, "%s: reps=%d outside [1, 100000]", who, reps);
  if (!kernel_ms) return fail(DDT_EINVAL, "%s: NULL kernel_ms", who);
  ddt::AttnPlan plan;
  const int rc = check_verify_attn(who, q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot,
                                   max_kv, prefix_len, n_nodes, vis, B, Q, H, d_lat, d_rope,
                                   dtype, sm_scale, out, workspace, workspace_bytes, true,
                                   plan);
  if (rc != DDT_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 3 && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  const int phase[2] = {ddt::kPhaseAttention, ddt::kPhaseMerge};
  if (e == hipSuccess) e = hipEventRecord(ev[0], st);
  for (int p = 0; p < 2 && e == hipSuccess; ++p) {
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      e = ddt::launch_verify_attn(dtype, d_lat, d_rope, q_lat, q_pe, c_kv, k_pe, num_slots,
                                  req_to_slot, max_kv, prefix_len, n_nodes, vis, B, Q, H,
                                  sm_scale, out, lse, workspace, plan, st, phase[p]);
    if (e == hipSuccess) e = hipEventRecord(ev[p + 1], st);
  }
  if (e == hipSuccess) e = hipEventSynchronize(ev[2]);
  float ms[2] = {0.0f, 0.0f};
  for (int p = 0; p < 2 && e == hipSuccess; ++p) e = hipEventElapsedTime(&ms[p], ev[p], ev[p + 1]);
  for (int i = 0; i < 3; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  if (e != hipSuccess) return launch_status(e, who);
  kernel_ms[0] = ms[0] / (float)reps;
  kernel_ms[1] = ms[1] / (float)reps;
  return DDT_OK;
}

int ddt_tree_accept(const int32_t* node_token, const int32_t* parent, const int32_t* n_nodes,
                    const int32_t* target_argmax, int B, int Q, int32_t* accept_len,
                    int32_t* accept_nodes, int32_t* out_tokens, int32_t* next_root,
                    void* stream) {
  if (B < 1) return fail(DDT_EINVAL, "ddt_tree_accept: B=%d must be >= 1", B);
  if (Q < 1 || Q > DDT_MAX_Q)
    return fail(DDT_EINVAL, "ddt_tree_accept: Q=%d outside [1, %d]", Q, DDT_MAX_Q);
  if (!node_token || !parent || !n_nodes || !target_argmax || !accept_len || !accept_nodes ||
      !out_tokens || !next_root)
    return fail(DDT_EINVAL, "ddt_tree_accept: NULL array argument");
  const hipError_t e = ddt::launch_tree_accept(node_token, parent, n_nodes, target_argmax, B, Q,
                                               accept_len, accept_nodes, out_tokens, next_root,
                                               static_cast<hipStream_t>(stream));
  return launch_status(e, "ddt_tree_accept");
}

int ddt_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                  const int32_t* n_nodes, const int32_t* accept_len,
                  const int32_t* accept_nodes, int B, int Q, int32_t* freed_slots,
                  int32_t* n_freed, void* stream) {
  if (B < 1) return fail(DDT_EINVAL, "ddt_kv_commit: B=%d must be >= 1", B);
  if (Q < 1 || Q > DDT_MAX_Q)
    return fail(DDT_EINVAL, "ddt_kv_commit: Q=%d outside [1, %d]", Q, DDT_MAX_Q);
  if (max_kv < 1) return fail(DDT_EINVAL, "ddt_kv_commit: max_kv=%d must be >= 1", max_kv);
  if (!req_to_slot || !prefix_len || !n_nodes || !accept_len || !accept_nodes || !freed_slots ||
      !n_freed)
    return fail(DDT_EINVAL, "ddt_kv_commit: NULL array argument");
  const hipError_t e =
      ddt::launch_kv_commit(req_to_slot, max_kv, prefix_len, n_nodes, accept_len, accept_nodes,
                            B, Q, freed_slots, n_freed, static_cast<hipStream_t>(stream));
  return launch_status(e, "ddt_kv_commit");
}

size_t ddt_draft_topk_workspace_size(int B, int D, int V, int K) {
  if (B < 1 || D < 1 || K < 1 || K > DDT_MAX_TOPK || V < K || V > DDT_MAX_VOCAB) return 0;
  return ddt::draft_topk_ws_bound(B, D, K);
}

int ddt_draft_topk(const void* logits, int dtype, int B, int D, int V, int K, float* topk_logp,
                   int32_t* topk_ids, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1) return fail(DDT_EINVAL, "ddt_draft_topk: B=%d must be >= 1", B);
  if (D < 1) return fail(DDT_EINVAL, "ddt_draft_topk: D=%d must be >= 1", D);
  if ((long long)B * D > 65535)
    return fail(DDT_EINVAL, "ddt_draft_topk: B*D=%lld exceeds 65535 rows", (long long)B * D);
  if (K < 1 || K > DDT_MAX_TOPK)
    return fail(DDT_EINVAL, "ddt_draft_topk: K=%d outside [1, %d]", K, DDT_MAX_TOPK);
  if (V < K || V > DDT_MAX_VOCAB)
    return fail(DDT_EINVAL, "ddt_draft_topk: V=%d outside [K=%d, %d]", V, K, DDT_MAX_VOCAB);
  if (dtype != DDT_F32 && dtype != DDT_BF16)
    return fail(DDT_EINVAL, "ddt_draft_topk: dtype=%d is neither DDT_F32 nor DDT_BF16", dtype);
  if (!logits || !topk_logp || !topk_ids || !workspace)
    return fail(DDT_EINVAL, "ddt_draft_topk: NULL array argument");
  const ddt::TopkPlan plan = ddt::plan_draft_topk(B, D, V, K, device_cu_count());
  if (workspace_bytes < plan.ws_bytes)
    return fail(DDT_EINVAL, "ddt_draft_topk: workspace of %zu bytes, %zu needed", workspace_bytes,
                plan.ws_bytes);
  const hipError_t e = ddt::launch_draft_topk(dtype, logits, B, D, V, K, topk_logp, topk_ids,
                                              workspace, plan, static_cast<hipStream_t>(stream));
  return launch_status(e, "ddt_draft_topk");
}

size_t ddt_tree_accept_sampling_workspace_size(int B, int Q, int V) {
  if (B < 1 || Q < 1 || Q > DDT_MAX_Q || V < 1 || V > DDT_MAX_VOCAB ||
      (long long)B * Q > (1 << 24))
    return 0;
  return ddt::tree_accept_sampling_ws_bound(B, Q);
}

int ddt_tree_accept_sampling(const void* target_logits, int dtype, int V,
                             const float* temperature, const int32_t* node_token,
                             const int32_t* parent, const int32_t* n_nodes, const float* coins,
                             const float* coin_final, int B, int Q, int32_t* accept_len,
                             int32_t* accept_nodes, int32_t* out_tokens, int32_t* next_root,
                             void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "ddt_tree_accept_sampling";
  if (B < 1) return fail(DDT_EINVAL, "%s: B=%d must be >= 1", fn, B);
  if (Q < 1 || Q > DDT_MAX_Q) return fail(DDT_EINVAL, "%s: Q=%d outside [1, %d]", fn, Q, DDT_MAX_Q);
  if ((long long)B * Q > (1 << 24))
    return fail(DDT_EINVAL, "%s: B*Q=%lld exceeds 2^24 rows", fn, (long long)B * Q);
  if (V < 1 || V > DDT_MAX_VOCAB)
    return fail(DDT_EINVAL, "%s: V=%d outside [1, %d]", fn, V, DDT_MAX_VOCAB);
  if (dtype != DDT_F32 && dtype != DDT_BF16)
    return fail(DDT_EINVAL, "%s: dtype=%d is neither DDT_F32 nor DDT_BF16", fn, dtype);
  if (!target_logits || !temperature || !node_token || !parent || !n_nodes || !coins ||
      !coin_final || !accept_len || !accept_nodes || !out_tokens || !next_root || !workspace)
    return fail(DDT_EINVAL, "%s: NULL array argument", fn);
  const ddt::SamplingPlan plan = ddt::plan_tree_accept_sampling(B, Q, V, device_cu_count());
  if (workspace_bytes < plan.ws_bytes)
    return fail(DDT_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                plan.ws_bytes);
  const hipError_t e = ddt::launch_tree_accept_sampling(
      dtype, target_logits, V, temperature, node_token, parent, n_nodes, coins, coin_final, B, Q,
      accept_len, accept_nodes, out_tokens, next_root, workspace, plan,
      static_cast<hipStream_t>(stream));
  return launch_status(e, fn);
}

}  // extern "C"

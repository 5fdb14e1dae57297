// ddt_internal.h -- declarations shared by the HIP sources of libddt.so.
//
// Kernels are written for gfx950 (CDNA4): 64-lane wavefronts, MFMA matrix
// cores, 160 KiB of LDS per compute unit.  The library's interface is the C
// entry points that ddt.h declares (api.hip, noalloc.hip); the C++ functions
// declared here are internal to it and not part of that interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_split.h"

namespace ddt {

constexpr int kWave = 64;

// Launchers: enqueue on `stream`, return the launch status.  Arguments were
// validated by the C entry points.
hipError_t launch_tree_build(const float* topk_logp, const int32_t* topk_ids,
                             const int32_t* root_token, const int32_t* prefix_len,
                             int B, int D, int K, int Q, int32_t* node_token,
                             int32_t* parent, int32_t* depth, int32_t* position,
                             int32_t* first_child, int32_t* next_sibling,
                             float* score, uint64_t* vis, int32_t* n_nodes,
                             hipStream_t stream);

hipError_t launch_tree_accept(const int32_t* node_token, const int32_t* parent,
                              const int32_t* n_nodes, const int32_t* target_argmax,
                              int B, int Q, int32_t* accept_len,
                              int32_t* accept_nodes, int32_t* out_tokens,
                              int32_t* next_root, hipStream_t stream);

hipError_t launch_kv_commit(int32_t* req_to_slot, int max_kv, int32_t* prefix_len,
                            const int32_t* n_nodes, const int32_t* accept_len,
                            const int32_t* accept_nodes, int B, int Q, int32_t* freed_slots,
                            int32_t* n_freed, hipStream_t stream);

// Per-depth top-K: each (request, depth) row of logits is cut into `chunks`
// chunks of `chunk` entries (see draft_topk.hip).
struct TopkPlan {
  int chunks;        // chunks per row (1..128)
  int chunk;         // entries per chunk (multiple of 8, <= 12288)
  size_t ws_bytes;   // workspace bytes this plan uses
};
TopkPlan plan_draft_topk(int B, int D, int V, int K, int num_cu);
size_t draft_topk_ws_bound(int B, int D, int K);  // enough for any plan
hipError_t launch_draft_topk(int dtype, const void* logits, int B, int D, int V, int K,
                             float* topk_logp, int32_t* topk_ids, void* workspace,
                             const TopkPlan& plan, hipStream_t stream);

// Sampling acceptance: every (request, node) row of target logits is cut into
// `chunks` chunks of `chunk` entries (see tree_accept_sampling.hip).
struct SamplingPlan {
  int chunks;        // chunks per row (1..128)
  int chunk;         // entries per chunk (multiple of 8, <= 12288)
  size_t ws_bytes;   // workspace bytes this plan uses
};
SamplingPlan plan_tree_accept_sampling(int B, int Q, int V, int num_cu);
size_t tree_accept_sampling_ws_bound(int B, int Q);  // enough for any plan
hipError_t launch_tree_accept_sampling(int dtype, const void* logits, int V,
                                       const float* temperature, const int32_t* node_token,
                                       const int32_t* parent, const int32_t* n_nodes,
                                       const float* coins, const float* coin_final, int B, int Q,
                                       int32_t* accept_len, int32_t* accept_nodes,
                                       int32_t* out_tokens, int32_t* next_root, void* workspace,
                                       const SamplingPlan& plan, hipStream_t stream);

// Verify attention: rows of a request are (node, head) pairs, row = i*H + h.
// The key range of every 128-row tile is split across a fixed grid of
// workgroups (see attn_split.h, which holds the plan); partial results go to
// the workspace and a merge kernel combines them.
// Kernels of one verify-attention call: the attention kernel (prefix stream,
// tree window, unsplit rows finished in place) and the merge of split rows.
// A call runs both, in this order; the kernel-time measurement runs each
// phase on its own.
constexpr int kPhaseAttention = 1, kPhaseMerge = 2, kPhaseAll = 3;

hipError_t launch_verify_attn(int dtype, int d_lat, int d_rope, const void* q_lat,
                              const void* q_pe, const void* c_kv, const void* k_pe,
                              int64_t num_slots, const int32_t* req_to_slot,
                              int max_kv, const int32_t* prefix_len,
                              const int32_t* n_nodes, const uint64_t* vis, int B,
                              int Q, int H, float sm_scale, float* out, float* lse,
                              void* workspace, const AttnPlan& plan,
                              hipStream_t stream, int phases = kPhaseAll);

// Helpers of the C entry points (api.hip).  fail() records the message that
// ddt_last_error() returns and passes `code` through; ok() clears it;
// launch_status() maps a HIP launch status to DDT_OK / DDT_ELAUNCH.
int fail(int code, const char* fmt, ...);
int ok();
int launch_status(hipError_t e, const char* what);
int device_cu_count();  // compute units of the current device, 0 if unknown
bool attn_variant_supported(int dtype, int d_lat, int d_rope);

// Checks of ddt_verify_attn's arguments; `who` names the entry point in the
// error text.  On success fills `plan` from the current device.  With
// check_ws false the workspace arguments are ignored (the caller supplies the
// workspace itself and checks its size against plan.ws_bytes).
int check_verify_attn(const char* who, const void* q_lat, const void* q_pe, const void* c_kv,
                      const void* k_pe, int64_t num_slots, const int32_t* req_to_slot,
                      int max_kv, const int32_t* prefix_len, const int32_t* n_nodes,
                      const uint64_t* vis, int B, int Q, int H, int d_lat, int d_rope,
                      int dtype, float sm_scale, const float* out, const void* workspace,
                      size_t workspace_bytes, bool check_ws, AttnPlan& plan);

}  // namespace ddt

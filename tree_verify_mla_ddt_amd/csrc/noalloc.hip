// noalloc.hip -- ddt_verify_attn_noalloc: tree-verify attention for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops that forbid allocation).  It runs exactly the kernels of
// ddt_verify_attn; their workspace (partial rows, partial log-sum-exps and the
// work prefix of split row tiles) lives in one static device array per GPU
// instead of a caller-supplied buffer.
#include <mutex>

#include "../../include/ddt.h"
#include "ddt_internal.h"

namespace {

// The largest workspace any verify-attention plan takes on a device of up to
// kScratchCUs compute units (MI355X has 256): two partial 128-row tiles of
// d_lat + 1 floats for each of kScratchCUs workgroups at d_lat = 512, then the
// stream prefix of DDT_MAX_BATCH_ATTN requests, split mode and start cost
// (rounded up to 16 bytes).  About 128.3 MiB.
constexpr int kScratchCUs = 256;
constexpr size_t kScratchBytes =
    (size_t)2 * kScratchCUs * ddt::kRowsPerWG * (512 + 1) * sizeof(float) +
    ((size_t)DDT_MAX_BATCH_ATTN + 4) * sizeof(long long);
static_assert(kScratchBytes % 16 == 0, "scratch rows stay 16-byte aligned");

// The array itself.  In host code `scratch` names a host-side stand-in, never
// the device memory: host code uses the per-device address from
// hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current.  Returns DDT_OK or a DDT_E* code (message set).
int scratch_address(const char* who, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return ddt::fail(DDT_ELAUNCH, "%s: no current device: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return ddt::fail(DDT_EUNSUPPORTED, "%s: device %d beyond the %d this entry point serves",
                     who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p)
      return ddt::fail(DDT_ELAUNCH, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                       who, dev, hipGetErrorString(g));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DDT_OK;
}

}  // namespace

extern "C" {

size_t ddt_verify_attn_noalloc_max_bytes(void) { return kScratchBytes; }

int ddt_verify_attn_noalloc(const void* q_lat, const void* q_pe, const void* c_kv,
                            const void* k_pe, int64_t num_slots, const int32_t* req_to_slot,
                            int max_kv, const int32_t* prefix_len, const int32_t* n_nodes,
                            const uint64_t* vis, int B, int Q, int H, int d_lat, int d_rope,
                            int dtype, float sm_scale, float* out, float* lse, void* stream) {
  static const char* who = "ddt_verify_attn_noalloc";
  ddt::AttnPlan plan;
  int rc = ddt::check_verify_attn(who, q_lat, q_pe, c_kv, k_pe, num_slots, req_to_slot, max_kv,
                                  prefix_len, n_nodes, vis, B, Q, H, d_lat, d_rope, dtype,
                                  sm_scale, out, nullptr, 0, false, plan);
  if (rc != DDT_OK) return rc;
  if (plan.ws_bytes > kScratchBytes)
    return ddt::fail(DDT_EUNSUPPORTED,
                     "%s: this call needs %zu bytes of workspace, more than the %zu of the "
                     "static scratch array (a device with more than %d compute units?); use "
                     "ddt_verify_attn with a caller-supplied workspace",
                     who, plan.ws_bytes, kScratchBytes, kScratchCUs);
  void* ws = nullptr;
  rc = scratch_address(who, &ws);
  if (rc != DDT_OK) return rc;
  // The kernels write every workspace entry they read within the call, so
  // nothing needs clearing between calls.
  const hipError_t e = ddt::launch_verify_attn(dtype, d_lat, d_rope, q_lat, q_pe, c_kv, k_pe,
                                               num_slots, req_to_slot, max_kv, prefix_len,
                                               n_nodes, vis, B, Q, H, sm_scale, out, lse, ws,
                                               plan, static_cast<hipStream_t>(stream));
  return ddt::launch_status(e, who);
}

}  // extern "C"

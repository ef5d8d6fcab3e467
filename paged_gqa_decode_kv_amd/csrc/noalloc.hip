// The decode step for callers that cannot allocate device memory: paged_decode_step and
// paged_attn_balanced_merge with their workspace in a static device array of the library.
//
// `scratch` below is a device variable: in host code its name is only a host-side stand-in,
// so the kernels are never given it directly.  Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and that address is what the
// kernels receive, through the same workspace fields as a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "../../include/paged_attn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
int g_status[kMaxDevices];

// Device address of the current device's copy of `scratch`.
int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_addr[dev] = rc == hipSuccess ? p : nullptr;
    g_status[dev] = rc == hipSuccess && p != nullptr ? PA_OK : PA_ERR_LAUNCH;
  });
  *addr = g_addr[dev];
  return g_status[dev];
}

}  // namespace

extern "C" int paged_decode_step_noalloc(const pa_dims* dims, const void* q, const void* k_new,
                                         const void* v_new, void* k_cache, void* v_cache,
                                         const int32_t* block_tables, const int32_t* seq_lens,
                                         float sm_scale, int32_t num_workgroups, float* out,
                                         float* out_lse, void* stream) {
  pa::AttnArgs a{};
  int st = pa::decode_step_args(dims, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                                sm_scale, num_workgroups, out, out_lse, &a);
  if (st != PA_OK) return st;
  if (paged_attn_balanced_workspace_bytes(dims, 1, num_workgroups) > PA_NOALLOC_SCRATCH_BYTES)
    return PA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PA_OK) return st;
  st = pa::bind_balanced_workspace(dims, 1, num_workgroups, ws, PA_NOALLOC_SCRATCH_BYTES, out,
                                   out_lse, &a);
  if (st != PA_OK) return st;
  st = pa::launch_balanced_append(a, dims->q_dtype, dims->kv_dtype, stream);
  if (st != PA_OK) return st;
  return pa::launch_balanced_merge(a, out, out_lse, stream);
}

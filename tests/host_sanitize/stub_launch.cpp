// Host-only stand-ins for the HIP launchers, so that the C ABI's argument checks
// (paged_gqa_decode_kv_amd/csrc/api.cpp) can be built with the host compiler's address and
// undefined-behaviour sanitizers and driven without a GPU.  Every launcher records that it
// was reached and launches nothing.
#include "../../paged_gqa_decode_kv_amd/csrc/launch.hpp"
#include "../../include/paged_attn.h"

int g_launches = 0;

namespace pa {
int launch_attention(const AttnArgs&, int, int, void*) { return ++g_launches, PA_OK; }
int launch_multi_query(const AttnArgs&, int, int, void*) { return ++g_launches, PA_OK; }
int balanced_row_tile(int32_t rows) { return rows <= 16 ? 16 : 32; }
int balanced_waves() { return 4; }
int balanced_workgroups(int, int, int, int32_t) { return 256; }
int launch_balanced(const AttnArgs&, int, int, void*) { return ++g_launches, PA_OK; }
int launch_balanced_append(const AttnArgs&, int, int, void*) { return ++g_launches, PA_OK; }
int launch_balanced_merge(const AttnArgs&, float*, float*, void*) { return ++g_launches, PA_OK; }
int launch_merge(const float*, const float*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                 int32_t, int32_t, float*, float*, void*) {
  return ++g_launches, PA_OK;
}
int launch_append(const void*, const void*, const int64_t*, int32_t, int32_t, int32_t, int64_t,
                  int64_t, int, void*, void*, void*) {
  return ++g_launches, PA_OK;
}
int launch_append_quant(const void*, const void*, const int64_t*, const int32_t*, int32_t,
                        int32_t, int32_t, int32_t, int64_t, int64_t, bool, void*, void*, void*,
                        void*, float*, float*, void*) {
  return ++g_launches, PA_OK;
}
int launch_copy_blocks(const int32_t*, int32_t, int32_t, int32_t, int64_t, int64_t, int, void*,
                       void*, float*, float*, void*) {
  return ++g_launches, PA_OK;
}
int launch_gather(const void*, const void*, const int32_t*, const int32_t*, int32_t, int32_t,
                  int32_t, int32_t, int64_t, int64_t, int32_t, int, void*, void*, void*) {
  return ++g_launches, PA_OK;
}
}  // namespace pa

// Drives every C ABI entry point through its host-side checks with seeded random and
// extreme arguments (sizes near the int32 / int64 limits, negative values, null and
// misaligned pointers).  Built with -fsanitize=address,undefined against stub launchers:
// any overflow or out-of-bounds access in the checks aborts the run.  Pointers are never
// dereferenced by the host code; they only need to be non-null / aligned or not.
#include <stdint.h>
#include <stdio.h>
#include <limits.h>

#include "../../include/paged_attn.h"

extern int g_launches;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int32_t pick_i32() {
  static const int32_t edge[] = {0, 1, 2, 3, 4, 8, 15, 16, 17, 31, 32, 64, 100, 128, 129, 2047,
                                 2048, 2049, 65535, 1 << 20, 1 << 30, INT_MAX, INT_MAX - 1, -1,
                                 -16, INT_MIN};
  const uint64_t r = next_u64();
  if (r % 3 == 0) return edge[(r >> 8) % (sizeof edge / sizeof edge[0])];
  return (int32_t)(r >> 16) % 5000;
}
static int64_t pick_i64() {
  static const int64_t edge[] = {0, 1, 16, 1 << 20, (int64_t)1 << 31, (int64_t)1 << 40,
                                 INT64_MAX, INT64_MAX / 2, -1, INT64_MIN};
  const uint64_t r = next_u64();
  if (r % 3 == 0) return edge[(r >> 8) % (sizeof edge / sizeof edge[0])];
  return (int64_t)((r >> 16) % 100000);
}
static void* pick_ptr() {
  const uint64_t r = next_u64() % 20;
  if (r == 0) return NULL;
  if (r == 1) return (void*)(uintptr_t)0x100008;  // 8-byte aligned only
  return (void*)(uintptr_t)0x100000;              // 16-byte aligned
}
static int32_t small(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

// a valid shape, then (half the time) one field replaced by an edge value
static pa_dims pick_dims() {
  pa_dims d;
  d.num_kv_heads = small(1, 8);
  d.num_q_heads = d.num_kv_heads * small(1, 8);
  d.num_seqs = small(1, 64);
  d.head_dim = (next_u64() % 2) ? 64 : 128;
  d.block_size = 16;
  d.max_blocks_per_seq = small(1, 512);
  d.num_blocks = small(1, 100000);
  const int combo = (int)(next_u64() % 4);
  d.q_dtype = combo == 0 ? PA_F32 : PA_BF16;
  d.kv_dtype = combo == 0 ? PA_F32 : (combo == 1 ? PA_BF16 : (combo == 2 ? PA_I8 : PA_FP8));
  d.kv_tile_stride = (next_u64() % 2) ? 0 : 32 * (int64_t)d.head_dim;
  d.sliding_window = (next_u64() % 3) ? 0 : small(1, 5000);
  switch (next_u64() % 24) {
    case 0: d.num_seqs = pick_i32(); break;
    case 1: d.num_q_heads = pick_i32(); break;
    case 2: d.num_kv_heads = pick_i32(); break;
    case 3: d.head_dim = pick_i32(); break;
    case 4: d.block_size = pick_i32(); break;
    case 5: d.max_blocks_per_seq = pick_i32(); break;
    case 6: d.num_blocks = pick_i64(); break;
    case 7: d.q_dtype = (int32_t)(next_u64() % 6) - 1; break;
    case 8: d.kv_dtype = (int32_t)(next_u64() % 6) - 1; break;
    case 9: d.kv_tile_stride = pick_i64(); break;
    case 10: d.sliding_window = pick_i32(); break;
    case 11: d.num_seqs = 2048 + small(0, 1); d.max_blocks_per_seq = pick_i32(); break;
    default: break;
  }
  return d;
}
static int32_t arg(int32_t lo, int32_t hi) { return (next_u64() % 6) ? small(lo, hi) : pick_i32(); }

int main(void) {
  int ok = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    pa_dims d = pick_dims();
    const int32_t nq = arg(1, 300), n = arg(0, 200), G = arg(1, 1024),
                  pt = (next_u64() % 6) ? 16 * small(1, 64) : pick_i32(), mp = arg(1, 128);
    // a workspace of the right size (when the shape is valid), too small, or arbitrary
    size_t wsb = paged_attn_balanced_workspace_bytes(&d, nq, G);
    const uint64_t wr = next_u64() % 8;
    if (wr == 0) wsb = wsb > 0 ? wsb - 1 : 0;
    if (wr == 1) wsb = (size_t)pick_i64();
    void *p0 = pick_ptr(), *p1 = pick_ptr(), *p2 = pick_ptr(), *p3 = pick_ptr(),
         *p4 = pick_ptr(), *p5 = pick_ptr(), *p6 = pick_ptr(), *p7 = pick_ptr();
    const pa_dims* dp = (next_u64() % 50) ? &d : NULL;
    int st[20];
    int k = 0;
    st[k++] = kv_append(dp, p0, p1, (const int64_t*)p2, n, p3, p4, NULL);
    st[k++] = paged_decode_attn(dp, p0, p1, p2, (const float*)p3, (const float*)p4,
                                (const int32_t*)p5, (const int32_t*)p6, 0.1f, (float*)p7, NULL);
    st[k++] = paged_verify_attn(dp, nq, p0, p1, p2, (const float*)p3, (const float*)p4,
                                (const int32_t*)p5, (const int32_t*)p6, 0.1f, (float*)p7, NULL);
    st[k++] = paged_decode_attn_split(dp, p0, p1, p2, (const float*)p3, (const float*)p4,
                                      (const int32_t*)p5, (const int32_t*)p6, 0.1f, pt, mp,
                                      (float*)p7, (float*)p0, NULL);
    st[k++] = lse_merge(dp, (const float*)p0, (const float*)p1, (const int32_t*)p2, pt, mp,
                        (float*)p3, (float*)p4, NULL);
    st[k++] = kv_gather(dp, p0, p1, (const int32_t*)p2, (const int32_t*)p3, n, p4, p5, NULL);
    st[k++] = paged_attn_balanced(dp, nq, p0, p1, p2, (const float*)p3, (const float*)p4,
                                  (const int32_t*)p5, (const int32_t*)p6, 0.1f, G, p7, wsb,
                                  (float*)p0, (float*)p1, NULL);
    st[k++] = paged_decode_step(dp, p0, p1, p2, p3, p4, (const int32_t*)p5, (const int32_t*)p6,
                                0.1f, G, p7, wsb, (float*)p0, (float*)p1, NULL);
    st[k++] = paged_attn_balanced_merge(dp, nq, G, p7, wsb, (float*)p0, (float*)p1, NULL);
    st[k++] = kv_copy_blocks(dp, (const int32_t*)p0, n, p1, p2, (float*)p3, (float*)p4, NULL);
    st[k++] = kv_append_quant(dp, p0, p1, (const int64_t*)p2, (const int32_t*)p3, n, nq, p4,
                              p5, p6, p7, (float*)p0, (float*)p1, NULL);
    st[k++] = paged_multi_query_attn(dp, nq, p0, p1, p2, (const float*)p3, (const float*)p4,
                                     (const int32_t*)p5, (const int32_t*)p6,
                                     (next_u64() % 2) ? (const int32_t*)p7 : NULL, 0.1f,
                                     (float*)p0, (float*)p1, NULL);
    (void)paged_split_workspace_bytes(dp, mp);
    (void)paged_attn_balanced_workspace_bytes(dp, nq, G);
    st[k++] = paged_attn_balanced_workgroups(dp, nq);
    for (int i = 0; i < k; ++i) {
      if (st[i] == PA_OK || (i == k - 1 && st[i] > 0)) ++ok; else ++rejected;
      if (paged_status_string(st[i] > 0 ? 0 : st[i]) == NULL) return 2;
    }
  }
  printf("calls accepted %d, rejected %d, launches %d\n", ok, rejected, g_launches);
  return ok > 0 && rejected > 0 ? 0 : 3;
}

// C ABI of libpaged_attn.so: argument checks on the host, then one launch per call.
// Every check here runs before any HIP call, so a rejected call leaves the GPU untouched
// (and can be exercised on a host without a GPU).
#include <limits.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.hpp"
#include "../../include/paged_attn.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_BF16 ? 2 : 1); }

int check_dims(const pa_dims* d) {
  if (d == nullptr) return PA_ERR_NULL;
  if (d->block_size != 16) return PA_ERR_BLOCK_SIZE;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_HEAD_DIM;
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->max_blocks_per_seq < 1 || d->num_blocks < 1)
    return PA_ERR_DIMS;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_DIMS;
  // token positions are int32 inside the kernels
  if ((int64_t)d->max_blocks_per_seq * 16 > INT_MAX) return PA_ERR_DIMS;
  if (d->sliding_window < 0) return PA_ERR_DIMS;
  if (d->kv_tile_stride != 0) {
    const int eb = d->kv_dtype == PA_F32 ? 4 : (d->kv_dtype == PA_BF16 ? 2 : 1);
    if (d->kv_tile_stride < 16 * (int64_t)d->head_dim || d->kv_tile_stride > (INT64_MAX >> 40) ||
        (d->kv_tile_stride * eb) % 16 != 0)
      return PA_ERR_DIMS;
  }
  return PA_OK;
}

// elements from one (block, KV head) tile to the next
int64_t tile_stride(const pa_dims* d) {
  return d->kv_tile_stride != 0 ? d->kv_tile_stride : 16 * (int64_t)d->head_dim;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// 8-bit codes with per-(block, KV head) scales
bool scaled8(int dtype) { return dtype == PA_I8 || dtype == PA_FP8; }
bool known_kv(int dtype) { return dtype == PA_F32 || dtype == PA_BF16 || scaled8(dtype); }

int check_attn_types(const pa_dims* d) {
  if (d->q_dtype == PA_F32 && d->kv_dtype == PA_F32) return PA_OK;
  if (d->q_dtype == PA_BF16 && (d->kv_dtype == PA_BF16 || scaled8(d->kv_dtype))) return PA_OK;
  return PA_ERR_DTYPE;
}

int check_attn_inputs(const pa_dims* d, const void* q, const void* k, const void* v,
                      const float* ks, const float* vs, const int32_t* tables,
                      const int32_t* lens) {
  int st = check_dims(d);
  if (st != PA_OK) return st;
  st = check_attn_types(d);
  if (st != PA_OK) return st;
  if (!q || !k || !v || !tables || !lens) return PA_ERR_NULL;
  if (scaled8(d->kv_dtype) && (!ks || !vs)) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return PA_ERR_ALIGN;
  return PA_OK;
}

pa::AttnArgs make_args(const pa_dims* d, int32_t nq, const void* q, const void* k,
                       const void* v, const float* ks, const float* vs,
                       const int32_t* tables, const int32_t* lens, float sm_scale) {
  pa::AttnArgs a{};
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.k_scale = ks;
  a.v_scale = vs;
  a.block_tables = tables;
  a.seq_lens = lens;
  a.num_seqs = d->num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.head_dim = d->head_dim;
  a.max_blocks = d->max_blocks_per_seq;
  a.num_blocks = d->num_blocks;
  a.tile_stride = tile_stride(d) * elem_bytes(d->kv_dtype);
  a.num_q_pos = nq;
  a.rows = nq * a.group;
  a.scale_log2 = sm_scale * kLog2e;
  a.part_tokens = 0;
  a.max_parts = 1;
  a.split = 0;
  a.window = d->sliding_window;
  return a;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the balanced mode: block-count prefix, then partial lse, then partial rows.
struct BalancedLayout {
  size_t prefix, lse, out, total;
};
BalancedLayout balanced_layout(const pa_dims* d, int32_t nq, int32_t num_workgroups) {
  const int64_t rows = (int64_t)nq * (d->num_q_heads / d->num_kv_heads);
  const int rt = pa::balanced_row_tile((int32_t)rows);
  const int64_t nrg = (rows + rt - 1) / rt;
  const int64_t npid = (int64_t)num_workgroups * pa::balanced_waves() +
                       (int64_t)d->num_kv_heads * nrg * d->num_seqs;
  BalancedLayout l;
  l.prefix = 0;
  l.lse = align256(((size_t)d->num_seqs + 1) * sizeof(int32_t));
  l.out = l.lse + align256((size_t)npid * rt * sizeof(float));
  l.total = l.out + (size_t)npid * rt * d->head_dim * sizeof(float);
  return l;
}

int check_balanced(const pa_dims* d, int32_t nq, int32_t num_workgroups) {
  int st = check_dims(d);
  if (st != PA_OK) return st;
  if (nq < 1 || num_workgroups < 1 || d->num_seqs > pa::kMaxBalancedSeqs) return PA_ERR_DIMS;
  const int64_t rows = (int64_t)nq * (d->num_q_heads / d->num_kv_heads);
  if (rows > INT_MAX) return PA_ERR_DIMS;
  if ((int64_t)num_workgroups * pa::balanced_waves() > INT_MAX) return PA_ERR_DIMS;
  // inside the kernel block positions of the flat list, block counts of a slice and tile
  // indices (physical block * KV heads + head) are int32
  const int rt = pa::balanced_row_tile((int32_t)rows);
  const int64_t nrg = (rows + rt - 1) / rt;
  if ((int64_t)d->num_seqs * d->max_blocks_per_seq > INT_MAX / (d->num_kv_heads * nrg))
    return PA_ERR_DIMS;
  if (d->num_blocks > INT_MAX / d->num_kv_heads) return PA_ERR_DIMS;
  return PA_OK;
}

}  // namespace

extern "C" {

int kv_append(const pa_dims* dims, const void* k_new, const void* v_new,
              const int64_t* slot_mapping, int32_t num_tokens, void* k_cache, void* v_cache,
              void* stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->kv_dtype != PA_F32 && dims->kv_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0) return PA_ERR_DIMS;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  return pa::launch_append(k_new, v_new, slot_mapping, num_tokens, dims->num_kv_heads,
                           dims->head_dim, dims->num_blocks, tile_stride(dims),
                           elem_bytes(dims->kv_dtype), k_cache, v_cache, stream);
}

int paged_verify_attn(const pa_dims* dims, int32_t num_q_pos, const void* q,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables, const int32_t* seq_lens,
                      float sm_scale, float* out, void* stream) {
  int st = check_attn_inputs(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens);
  if (st != PA_OK) return st;
  if (!out) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  if (num_q_pos < 1 || (int64_t)num_q_pos * (dims->num_q_heads / dims->num_kv_heads) > INT_MAX)
    return PA_ERR_DIMS;
  pa::AttnArgs a = make_args(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale,
                             block_tables, seq_lens, sm_scale);
  a.out = out;
  return pa::launch_attention(a, dims->q_dtype, dims->kv_dtype, stream);
}

int paged_decode_attn(const pa_dims* dims, const void* q, const void* k_cache,
                      const void* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* seq_lens, float sm_scale,
                      float* out, void* stream) {
  return paged_verify_attn(dims, 1, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                           seq_lens, sm_scale, out, stream);
}

int paged_decode_attn_split(const pa_dims* dims, const void* q, const void* k_cache,
                            const void* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            float sm_scale, int32_t partition_tokens, int32_t max_partitions,
                            float* part_out, float* part_lse, void* stream) {
  int st = check_attn_inputs(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens);
  if (st != PA_OK) return st;
  if (partition_tokens <= 0 || partition_tokens % 16 != 0 || max_partitions < 1)
    return PA_ERR_PARTITION;
  if (!part_out || !part_lse) return PA_ERR_NULL;
  if (!aligned16(part_out)) return PA_ERR_ALIGN;
  pa::AttnArgs a = make_args(dims, 1, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                             seq_lens, sm_scale);
  a.out = part_out;
  a.part_lse = part_lse;
  a.part_tokens = partition_tokens;
  a.max_parts = max_partitions;
  a.split = 1;
  return pa::launch_attention(a, dims->q_dtype, dims->kv_dtype, stream);
}

int lse_merge(const pa_dims* dims, const float* part_out, const float* part_lse,
              const int32_t* seq_lens, int32_t partition_tokens, int32_t max_partitions,
              float* out, float* out_lse, void* stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (partition_tokens <= 0 || partition_tokens % 16 != 0 || max_partitions < 1)
    return PA_ERR_PARTITION;
  if (!part_out || !part_lse || !seq_lens || !out) return PA_ERR_NULL;
  return pa::launch_merge(part_out, part_lse, seq_lens, dims->num_seqs, dims->num_q_heads,
                          dims->head_dim, dims->max_blocks_per_seq, partition_tokens,
                          max_partitions, out, out_lse, stream);
}

size_t paged_split_workspace_bytes(const pa_dims* dims, int32_t max_partitions) {
  if (check_dims(dims) != PA_OK || max_partitions < 1) return 0;
  const size_t rows = (size_t)dims->num_seqs * (size_t)dims->num_q_heads * (size_t)max_partitions;
  return rows * ((size_t)dims->head_dim + 1) * sizeof(float);
}

int kv_gather(const pa_dims* dims, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, int32_t max_len,
              void* k_out, void* v_out, void* stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (!known_kv(dims->kv_dtype)) return PA_ERR_DTYPE;
  if (max_len < 0) return PA_ERR_DIMS;
  if (max_len == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !k_out || !v_out) return PA_ERR_NULL;
  return pa::launch_gather(k_cache, v_cache, block_tables, seq_lens, dims->num_seqs,
                           dims->num_kv_heads, dims->head_dim, dims->max_blocks_per_seq,
                           dims->num_blocks, tile_stride(dims), max_len,
                           elem_bytes(dims->kv_dtype), k_out, v_out, stream);
}

int kv_append_quant(const pa_dims* dims, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, const int32_t* stage_rows, int32_t num_tokens,
                    int32_t num_stage_rows, void* k_stage, void* v_stage, void* k_cache,
                    void* v_cache, float* k_scale, float* v_scale, void* stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (!scaled8(dims->kv_dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_stage_rows < 0) return PA_ERR_DIMS;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !stage_rows || !k_stage || !v_stage || !k_cache ||
      !v_cache || !k_scale || !v_scale)
    return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_stage) || !aligned16(v_stage) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_ALIGN;
  return pa::launch_append_quant(k_new, v_new, slot_mapping, stage_rows, num_tokens,
                                 num_stage_rows, dims->num_kv_heads, dims->head_dim,
                                 dims->num_blocks, tile_stride(dims), dims->kv_dtype == PA_FP8,
                                 k_stage, v_stage, k_cache, v_cache, k_scale, v_scale, stream);
}

int kv_copy_blocks(const pa_dims* dims, const int32_t* block_pairs, int32_t num_pairs,
                   void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   void* stream) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (!known_kv(dims->kv_dtype)) return PA_ERR_DTYPE;
  if (num_pairs < 0) return PA_ERR_DIMS;
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs || !k_cache || !v_cache) return PA_ERR_NULL;
  if (scaled8(dims->kv_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  return pa::launch_copy_blocks(block_pairs, num_pairs, dims->num_kv_heads, dims->head_dim,
                                dims->num_blocks, tile_stride(dims), elem_bytes(dims->kv_dtype),
                                k_cache, v_cache, scaled8(dims->kv_dtype) ? k_scale : nullptr,
                                scaled8(dims->kv_dtype) ? v_scale : nullptr, stream);
}

int paged_multi_query_attn(const pa_dims* dims, int32_t num_q_pos, const void* q,
                           const void* k_cache, const void* v_cache, const float* k_scale,
                           const float* v_scale, const int32_t* block_tables,
                           const int32_t* seq_lens, const int32_t* tree_mask, float sm_scale,
                           float* out, float* out_lse, void* stream) {
  int st = check_attn_inputs(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens);
  if (st != PA_OK) return st;
  if (num_q_pos < 1) return PA_ERR_DIMS;
  if (!out) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  if (tree_mask != nullptr && (num_q_pos > pa::kMaxTreeNodes || dims->sliding_window > 0))
    return PA_ERR_DIMS;
  if ((int64_t)num_q_pos * (dims->num_q_heads / dims->num_kv_heads) > INT_MAX / 2)
    return PA_ERR_DIMS;
  pa::AttnArgs a = make_args(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale,
                             block_tables, seq_lens, sm_scale);
  a.out = out;
  a.ws_out_lse = out_lse;
  a.tree_mask = tree_mask;
  a.mask_words = (num_q_pos + 31) / 32;
  return pa::launch_multi_query(a, dims->q_dtype, dims->kv_dtype, stream);
}

int paged_attn_balanced_workgroups(const pa_dims* dims, int32_t num_q_pos) {
  int st = check_balanced(dims, num_q_pos, 1);
  if (st != PA_OK) return st;
  st = check_attn_types(dims);
  if (st != PA_OK) return st;
  return pa::balanced_workgroups(dims->q_dtype, dims->kv_dtype, dims->head_dim,
                                 num_q_pos * (dims->num_q_heads / dims->num_kv_heads));
}

size_t paged_attn_balanced_workspace_bytes(const pa_dims* dims, int32_t num_q_pos,
                                           int32_t num_workgroups) {
  if (check_balanced(dims, num_q_pos, num_workgroups) != PA_OK) return 0;
  return balanced_layout(dims, num_q_pos, num_workgroups).total;
}

namespace {
int balanced_args(const pa_dims* dims, int32_t num_q_pos, int32_t num_workgroups, void* workspace,
                  size_t workspace_bytes, float* out, float* out_lse, pa::AttnArgs* a) {
  const BalancedLayout l = balanced_layout(dims, num_q_pos, num_workgroups);
  if (workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return PA_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a->num_workgroups = num_workgroups;
  a->num_workers = num_workgroups * pa::balanced_waves();
  a->ws_prefix = reinterpret_cast<int32_t*>(ws + l.prefix);
  a->ws_lse = reinterpret_cast<float*>(ws + l.lse);
  a->ws_out = reinterpret_cast<float*>(ws + l.out);
  a->out = out;
  a->ws_out_lse = out_lse;
  return PA_OK;
}
}  // namespace

int paged_attn_balanced(const pa_dims* dims, int32_t num_q_pos, const void* q,
                        const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        const int32_t* seq_lens, float sm_scale, int32_t num_workgroups,
                        void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                        void* stream) {
  int st = check_attn_inputs(dims, q, k_cache, v_cache, k_scale, v_scale, block_tables, seq_lens);
  if (st != PA_OK) return st;
  st = check_balanced(dims, num_q_pos, num_workgroups);
  if (st != PA_OK) return st;
  if (!out || !workspace) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  pa::AttnArgs a = make_args(dims, num_q_pos, q, k_cache, v_cache, k_scale, v_scale,
                             block_tables, seq_lens, sm_scale);
  st = balanced_args(dims, num_q_pos, num_workgroups, workspace, workspace_bytes, out, out_lse, &a);
  if (st != PA_OK) return st;
  return pa::launch_balanced(a, dims->q_dtype, dims->kv_dtype, stream);
}

int paged_decode_step(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                      void* k_cache, void* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, float sm_scale, int32_t num_workgroups,
                      void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                      void* stream) {
  pa::AttnArgs a{};
  int st = pa::decode_step_args(dims, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                                sm_scale, num_workgroups, out, out_lse, &a);
  if (st != PA_OK) return st;
  if (!workspace) return PA_ERR_NULL;
  st = pa::bind_balanced_workspace(dims, 1, num_workgroups, workspace, workspace_bytes, out,
                                   out_lse, &a);
  if (st != PA_OK) return st;
  return pa::launch_balanced_append(a, dims->q_dtype, dims->kv_dtype, stream);
}

int paged_attn_balanced_merge(const pa_dims* dims, int32_t num_q_pos, int32_t num_workgroups,
                              void* workspace, size_t workspace_bytes, float* out,
                              float* out_lse, void* stream) {
  int st = check_balanced(dims, num_q_pos, num_workgroups);
  if (st != PA_OK) return st;
  if (!out || !workspace) return PA_ERR_NULL;
  pa::AttnArgs a{};
  a.num_seqs = dims->num_seqs;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.group = dims->num_q_heads / dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.num_q_pos = num_q_pos;
  a.rows = num_q_pos * a.group;
  st = balanced_args(dims, num_q_pos, num_workgroups, workspace, workspace_bytes, out, out_lse, &a);
  if (st != PA_OK) return st;
  return pa::launch_balanced_merge(a, out, out_lse, stream);
}

const char* paged_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_DIMS: return "a size is out of range or num_q_heads % num_kv_heads != 0";
    case PA_ERR_DTYPE: return "unsupported element-type combination";
    case PA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PA_ERR_BLOCK_SIZE: return "block_size must be 16";
    case PA_ERR_PARTITION: return "partition_tokens must be a positive multiple of 16 and max_partitions >= 1";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
    case PA_ERR_ALIGN: return "q, k_cache, v_cache or out not 16-byte aligned";
    case PA_ERR_SCRATCH:
      return "the decode step needs more workspace than the library's static scratch "
             "(PA_NOALLOC_SCRATCH_BYTES): use paged_decode_step with a caller workspace";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace pa {

int decode_step_args(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, float sm_scale, int32_t num_workgroups, float* out,
                     float* out_lse, AttnArgs* a) {
  int st = check_dims(dims);
  if (st != PA_OK) return st;
  if (dims->kv_dtype != PA_F32 && dims->kv_dtype != PA_BF16) return PA_ERR_DTYPE;
  st = check_attn_inputs(dims, q, k_cache, v_cache, nullptr, nullptr, block_tables, seq_lens);
  if (st != PA_OK) return st;
  st = check_balanced(dims, 1, num_workgroups);
  if (st != PA_OK) return st;
  if (!k_new || !v_new || !out) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(k_new)) return PA_ERR_ALIGN;
  *a = make_args(dims, 1, q, k_cache, v_cache, nullptr, nullptr, block_tables, seq_lens,
                 sm_scale);
  a->k_new = k_new;
  a->v_new = v_new;
  a->out = out;
  a->ws_out_lse = out_lse;
  return PA_OK;
}

int bind_balanced_workspace(const pa_dims* dims, int32_t num_q_pos, int32_t num_workgroups,
                            void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                            AttnArgs* a) {
  return balanced_args(dims, num_q_pos, num_workgroups, workspace, workspace_bytes, out, out_lse,
                       a);
}

}  // namespace pa

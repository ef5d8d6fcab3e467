// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Arguments arrive here already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/paged_attn.h"

namespace pa {

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;        // normalised output (direct) or per-partition output (split)
  float* part_lse;   // split only: per-partition log-sum-exp
  int32_t num_seqs, num_q_heads, num_kv_heads, group, head_dim, max_blocks;
  int64_t num_blocks;
  int64_t tile_stride;      // bytes from one (block, KV head) tile to the next in each cache
  int32_t num_q_pos;        // query positions per sequence
  int32_t rows;             // query rows per (sequence, KV head) = num_q_pos * group
  int32_t part_tokens;      // split: tokens per partition
  int32_t max_parts;        // split: partitions per row in the workspace; direct: 1
  int32_t split;            // 0: direct, 1: write partials
  float scale_log2;         // sm_scale * log2(e)
  int32_t window;           // sliding window in tokens (0 = none)
  // balanced mode
  int32_t num_workgroups;   // workgroups launched
  int32_t num_workers;      // waves the flat block list is dealt to (workgroups * waves)
  float* ws_out;            // partial rows  [num_workers + segments][row tile][head_dim]
  float* ws_lse;            // partial lse   [num_workers + segments][row tile]
  int32_t* ws_prefix;       // block-count prefix over sequences [num_seqs + 1]
  float* ws_out_lse;        // final lse [B][nq][Hq] for whole segments, or null
  // decode step (balanced mode with the append folded in): the new token of every
  // sequence, [B][Hkv][head_dim] in the cache's element type
  const void* k_new;
  const void* v_new;
  // multi-query rows: candidate visibility bit rows [B][num_q_pos][mask_words] (null =
  // causal rows)
  const int32_t* tree_mask;
  int32_t mask_words;
};

// most candidates a visibility mask may cover (bit rows of up to 4 words per query row)
constexpr int kMaxTreeNodes = 128;

// most sequences the balanced mode accepts in one call (its prefix lives in LDS)
constexpr int kMaxBalancedSeqs = 2048;

int launch_attention(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream);
// multi-query rows (causal, or with a candidate mask in a.tree_mask): direct mode
int launch_multi_query(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream);

// rows of one partial (16 or 32): the row tile the kernel uses for `rows` query rows
int balanced_row_tile(int32_t rows);
// waves per workgroup of the balanced kernel
int balanced_waves();
// workgroups that fit on the current device at once for the balanced kernel (< 0: error)
int balanced_workgroups(int q_dtype, int kv_dtype, int head_dim, int32_t rows);
// balanced attention on `stream`; the AttnArgs workspace pointers must be set
int launch_balanced(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream);
// the same with the decode step's append folded in (a.k_new / a.v_new set, nq = 1,
// fp32 or bf16 caches); k_cache / v_cache are written
int launch_balanced_append(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream);

// merge of the balanced mode's partials into out [B][nq][Hq][d] (and out_lse, if given)
int launch_balanced_merge(const AttnArgs& a, float* out, float* out_lse, void* stream);

// The host checks of the decode step (paged_decode_step's arguments, the workspace aside)
// and its launch arguments in *a; PA_OK or the status the entry point returns.  No HIP call.
int decode_step_args(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, float sm_scale, int32_t num_workgroups, float* out,
                     float* out_lse, AttnArgs* a);
// Points the balanced mode's workspace fields of *a into `workspace` (PA_ERR_WORKSPACE if
// it is smaller than paged_attn_balanced_workspace_bytes or not 16-byte aligned).
int bind_balanced_workspace(const pa_dims* dims, int32_t num_q_pos, int32_t num_workgroups,
                            void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                            AttnArgs* a);

int launch_merge(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                 int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_blocks,
                 int32_t part_tokens, int32_t max_parts, float* out, float* out_lse,
                 void* stream);

// tile_stride in elements
int launch_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int64_t num_blocks, int64_t tile_stride, int elem_bytes, void* k_cache,
                  void* v_cache, void* stream);

// int8 cache, bf16 new tokens and staging rows; tile_stride in elements
int launch_append_quant(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                        const int32_t* stage_rows, int32_t num_tokens, int32_t num_stage_rows,
                        int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                        int64_t tile_stride, bool fp8, void* k_stage, void* v_stage,
                        void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                        void* stream);

// tile_stride in elements; scales may be null (non-int8 caches)
int launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_dim, int64_t num_blocks, int64_t tile_stride,
                       int elem_bytes, void* k_cache, void* v_cache, float* k_scale,
                       float* v_scale, void* stream);

int launch_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                  int32_t head_dim, int32_t max_blocks, int64_t num_blocks, int64_t tile_stride,
                  int32_t max_len, int elem_bytes, void* k_out, void* v_out, void* stream);

}  // namespace pa

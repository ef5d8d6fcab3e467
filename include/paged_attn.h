/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged GQA decode-attention library
 * (libpaged_attn.so).
 *
 * The operation (devpress.csdn.net KV Cache / GQA / PagedAttention tutorial, section 2
 * "KV Cache 到底缓存了什么？": Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V; CS336
 * lecture 10, "KV Cache 原理": at each decode step the new token's K and V are appended
 * to the cache and its query attends to every cached K and V):
 *
 *   for every sequence b, query position i and query head h, with g = h / (Hq / Hkv)
 *   (GQA: a group of query heads shares one KV head -- lecture 10, "Grouped Query
 *   Attention"), and lam = seq_lens[b] - nq + 1 + i visible tokens:
 *     s_t  = sm_scale * dot(q[b,i,h,:], K[b,g,t,:])          t < lam
 *     out  = sum_t exp(s_t) V[b,g,t,:] / sum_t exp(s_t)
 *     lse  = log sum_t exp(s_t)                               (natural log)
 *
 * Paged storage (tutorial section 7 "PagedAttention 如何解决显存碎片？"; lecture 10
 * "PagedAttention 与 vLLM"): the cache is cut into blocks of 16 tokens; block_tables[b][j]
 * names the physical block holding tokens 16j .. 16j+15 of sequence b.  Inside a block
 * this library uses
 *
 *   k_cache[num_blocks][num_kv_heads][head_dim / x][16][x]   x = 16 / element bytes
 *                                                (x = 4 fp32, 8 bf16, 16 int8 / fp8)
 *   v_cache[num_blocks][num_kv_heads][head_dim][16]
 *
 * so one (block, KV head) tile of K or V is one contiguous 16 x head_dim piece of memory.
 * Tile (block n, head g) starts kv_tile_stride * (n * num_kv_heads + g) elements into its
 * cache; kv_tile_stride = 16 * head_dim packs the tiles densely (the shapes above), and
 * kv_tile_stride = 32 * head_dim with v_cache = k_cache + 16 * head_dim lays K and V of one
 * (block, head) side by side in a single allocation [num_blocks][num_kv_heads][2][tile],
 * which HBM streams faster than two separate pools (each tile read becomes one 2-tile run).
 * Inside a K tile, element k of the token at offset o sits at [k / x][o][k % x]: each
 * 16-byte column of the 16 tokens' K rows is contiguous.  Inside a V tile, element k of
 * that token sits at [k][o].
 * int8 and fp8 caches carry one fp32 scale per (physical block, KV head) for each of K and V:
 * k_scale[num_blocks][num_kv_heads], v_scale[num_blocks][num_kv_heads]; the stored code x_q
 * stands for x_q * scale (lecture 10 "Quantization 量化 / 基本概念", zero point 0).
 *
 * Conventions for every call:
 *  - Pointers named as device memory must be device (HBM) pointers on the current HIP
 *    device; the caller owns all of them, including workspaces.  The library never
 *    allocates, frees or synchronises and keeps no mutable global state.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).  Every call
 *    only enqueues work on it and returns.
 *  - Return value: PA_OK (0) or a negative PA_ERR_* code.  Every argument check runs on
 *    the host before any HIP call, so a rejected call touches no GPU state.
 *    PA_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 *  - q, k_cache, v_cache and out must be 16-byte aligned (PA_ERR_ALIGN otherwise).
 *  - Device-side contract: table entries for logical blocks < ceil(seq_len/16) name
 *    physical blocks in [0, num_blocks).  An entry outside that range is not read: its
 *    tokens are skipped.  seq_lens[b] larger than 16 * max_blocks_per_seq is cut to that
 *    capacity; negative lengths count as 0.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types.  PA_I8 and PA_FP8 caches hold 8-bit codes with one fp32 scale per
   (physical block, KV head) for K and one for V (k_scale, v_scale [num_blocks][Hkv]):
   x = code * scale.  PA_I8 codes are signed integers; PA_FP8 codes are OCP e4m3 floats
   (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN).
   A per-head calibrated fp8 scale is every block of the head holding the same value. */
enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_FP8 = 3 };

/* status codes */
enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,       /* a required pointer is NULL                                   */
  PA_ERR_DIMS = -2,       /* a size is < 1 (or < 0 where 0 is allowed), or Hq % Hkv != 0  */
  PA_ERR_DTYPE = -3,      /* element-type combination not supported by the call           */
  PA_ERR_HEAD_DIM = -4,   /* head_dim is not 64 or 128                                     */
  PA_ERR_BLOCK_SIZE = -5, /* block_size is not 16                                          */
  PA_ERR_WORKSPACE = -6,  /* workspace smaller than the size query returns, or misaligned  */
  PA_ERR_LAUNCH = -7,     /* a kernel launch failed (or a device query failed)             */
  PA_ERR_PARTITION = -8,  /* partition_tokens not a positive multiple of 16, or
                             max_partitions < 1                                            */
  PA_ERR_ALIGN = -9,      /* q, k_cache, v_cache or out not 16-byte aligned                */
  PA_ERR_SCRATCH = -10    /* paged_decode_step_noalloc: the call needs more workspace than
                             the library's static scratch (PA_NOALLOC_SCRATCH_BYTES)       */
};

/* Shapes and element types shared by every call. */
typedef struct pa_dims {
  int32_t num_seqs;           /* B: sequences in the batch (>= 1)                          */
  int32_t num_q_heads;        /* Hq (>= 1)                                                 */
  int32_t num_kv_heads;       /* Hkv (>= 1, divides Hq; Hkv == 1 is MQA, Hkv == Hq is MHA)  */
  int32_t head_dim;           /* d: 64 or 128                                              */
  int32_t block_size;         /* tokens per block: must be 16                              */
  int32_t max_blocks_per_seq; /* row length of block_tables (>= 1)                         */
  int64_t num_blocks;         /* physical blocks in each of k_cache / v_cache (>= 1)       */
  int32_t q_dtype;            /* PA_F32 or PA_BF16                                         */
  int32_t kv_dtype;           /* PA_F32, PA_BF16, PA_I8 or PA_FP8                          */
  int64_t kv_tile_stride;     /* elements from one (block, KV head) tile to the next in
                                 k_cache and in v_cache; 0 means 16 * head_dim (dense).
                                 Otherwise >= 16 * head_dim and a multiple of 16 bytes
                                 (PA_ERR_DIMS)                                             */
  int32_t sliding_window;     /* W: 0 = every cached token; W > 0 = the row at position p
                                 attends tokens max(0, p - W + 1) .. p only (sliding-window
                                 attention, in-depth guide section 2.3).  Every attention
                                 call honours it; kv_append, kv_gather and kv_copy_blocks
                                 ignore it.  < 0 is PA_ERR_DIMS                             */
} pa_dims;
/* Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, I8), (BF16, FP8).
 * q may hold any finite value of its type on every cache type (8-bit K codes meet q as
 * exact bf16 operands); only the scores sm_scale * q . K must stay finite in fp32. */

/*
 * kv_append -- write each new token's K and V into its cache slot.
 * Tutorial section 2 / lecture 10 "KV Cache 原理": a decode step appends the new token's
 * K and V to the cache; tutorial section 7: the token lands in a block of the sequence's
 * table.  The slot (physical_block * 16 + offset) of each token is given by the caller.
 *   k_new, v_new   device, [num_tokens][num_kv_heads][head_dim], kv_dtype (F32 or BF16)
 *   slot_mapping   device, [num_tokens] int64; slot < 0 means "skip this token";
 *                  a slot >= num_blocks * 16 is also skipped
 *   k_cache, v_cache device, the cache layout above; written in place (a bit copy)
 * num_tokens may be 0 (nothing is launched).  int8 caches: PA_ERR_DTYPE.
 */
int kv_append(const pa_dims* dims, const void* k_new, const void* v_new,
              const int64_t* slot_mapping, int32_t num_tokens, void* k_cache, void* v_cache,
              void* stream);

/*
 * paged_decode_attn -- single-token decode attention over the paged cache (nq = 1).
 *   q            device, [B][Hq][head_dim], q_dtype
 *   k_cache, v_cache device, layout above, kv_dtype
 *   k_scale, v_scale device, [num_blocks][Hkv] fp32; required for PA_I8 and PA_FP8, ignored
 *                otherwise
 *   block_tables device, [B][max_blocks_per_seq] int32
 *   seq_lens     device, [B] int32: tokens attended, including the new one
 *   sm_scale     the softmax scale (1/sqrt(head_dim) for the pages' formula)
 *   out          device, [B][Hq][head_dim] fp32; a sequence with no token gets zeros
 */
int paged_decode_attn(const pa_dims* dims, const void* q, const void* k_cache,
                      const void* v_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* seq_lens, float sm_scale,
                      float* out, void* stream);

/*
 * paged_verify_attn -- the causal verify forward of speculative decoding: nq query
 * positions per sequence (the last accepted token plus nq - 1 draft tokens) scored in one
 * pass (guide section 4.2 "数学原理": the target model scores all draft positions in a
 * single forward; lecture 10 "Speculative Decoding").  seq_lens counts the nq positions,
 * whose K/V are already in the cache; position i is token seq_len - nq + i and sees tokens
 * 0 .. seq_len - nq + i.
 *   num_q_pos    nq >= 1 (nq == 1 is paged_decode_attn)
 *   q            device, [B][nq][Hq][head_dim], q_dtype
 *   out          device, [B][nq][Hq][head_dim] fp32; a row that sees no token gets zeros
 *   other arguments as paged_decode_attn.
 */
int paged_verify_attn(const pa_dims* dims, int32_t num_q_pos, const void* q,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables, const int32_t* seq_lens,
                      float sm_scale, float* out, void* stream);

/*
 * paged_decode_attn_split -- decode attention with each sequence's context cut into
 * partitions of partition_tokens tokens, each partition handled by its own workgroups.
 * A sequence of L tokens occupies n = min(ceil(L / partition_tokens), max_partitions)
 * partitions; the last one also takes any tokens beyond n * partition_tokens.  For each
 * occupied partition p it writes the partition's normalised result and log-sum-exp:
 *   part_out     device, [B][Hq][max_partitions][head_dim] fp32
 *   part_lse     device, [B][Hq][max_partitions] fp32 (natural log; -inf if p saw no token)
 * Entries of partitions a sequence does not occupy are not written.  lse_merge combines
 * them.  Other arguments as paged_decode_attn.
 */
int paged_decode_attn_split(const pa_dims* dims, const void* q, const void* k_cache,
                            const void* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            float sm_scale, int32_t partition_tokens, int32_t max_partitions,
                            float* part_out, float* part_lse, void* stream);

/*
 * lse_merge -- recombine partition results exactly: with M = max_p lse_p and
 * w_p = exp(lse_p - M), out = sum_p w_p o_p / sum_p w_p and lse = M + log sum_p w_p over the
 * n occupied partitions of each sequence (n as in paged_decode_attn_split, from seq_lens).
 * Partitions with lse_p = -inf carry no weight; if all do, out = 0 and lse = -inf.
 *   part_out, part_lse device, as written by paged_decode_attn_split
 *   out          device, [B][Hq][head_dim] fp32
 *   out_lse      device, [B][Hq] fp32, or NULL
 */
int lse_merge(const pa_dims* dims, const float* part_out, const float* part_lse,
              const int32_t* seq_lens, int32_t partition_tokens, int32_t max_partitions,
              float* out, float* out_lse, void* stream);

/* Bytes of part_out plus part_lse for paged_decode_attn_split (0 if dims are invalid). */
size_t paged_split_workspace_bytes(const pa_dims* dims, int32_t max_partitions);

/*
 * kv_gather -- copy each sequence's tokens out of the pool into contiguous order, using
 * the same block-table translation as the attention kernels (a check of that indexing).
 *   k_out, v_out device, [B][Hkv][max_len][head_dim], kv_dtype (int8 stays int8)
 * Tokens t >= min(seq_lens[b], max_len) are not written.
 */
int kv_gather(const pa_dims* dims, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, int32_t max_len,
              void* k_out, void* v_out, void* stream);

/*
 * paged_multi_query_attn -- num_q_pos query positions per sequence against its paged
 * cache: chunked prefill (guide section 4.1: a long prompt's prefill cut into chunks that
 * run beside decode steps) and speculative candidate trees (guide section 3.3).  The last
 * num_q_pos = nq tokens of each sequence (seq_lens counts them; their K and V are already
 * in the cache) are the query positions.
 *   tree_mask == NULL: causal rows, query i sees tokens t <= L - nq + i (as
 *                paged_verify_attn), within the sliding window if dims sets one.
 *   tree_mask != NULL: query i sees every token t < L - nq and candidate j (token
 *                L - nq + j) iff bit j % 32 of word j / 32 of its mask row is set (for a
 *                tree: i itself and its ancestors).  nq <= 128 and no sliding window,
 *                else PA_ERR_DIMS.
 *   q          device [B][nq][Hq][d] in q_dtype
 *   tree_mask  device int32 [B][nq][ceil(nq / 32)] bit rows, or NULL
 *   out        device fp32 [B][nq][Hq][d]; out_lse device fp32 [B][nq][Hq] (natural log)
 *              or NULL.  A row that sees nothing gets 0 and lse -inf.
 *   other arguments as paged_verify_attn.
 * A workgroup owns up to 32 query rows of a (sequence, KV head) (rows = nq * Hq / Hkv), its
 * four waves taking interleaved blocks of every token those rows may see and merging
 * through LDS.  Decode and short verify are faster through paged_attn_balanced.
 */
int paged_multi_query_attn(const pa_dims* dims, int32_t num_q_pos, const void* q,
                           const void* k_cache, const void* v_cache, const float* k_scale,
                           const float* v_scale, const int32_t* block_tables,
                           const int32_t* seq_lens, const int32_t* tree_mask, float sm_scale,
                           float* out, float* out_lse, void* stream);

/*
 * kv_append_quant -- append new tokens to an int8 or fp8 cache (lecture 10's symmetric int8
 * rule, zero point 0; in-depth guide section 5.2: per-head scales for KV caches, FP8 KV
 * caches).  A (block, KV head) keeps one fp32 scale over its live tokens: int8 scale =
 * max|x| / 127 and codes round-half-even(x / scale) clamped to +-127; fp8 scale =
 * max|x| / 448 and codes e4m3(x / scale), round to nearest even, saturating at +-448;
 * all codes 0 when the scale is 0.  That is the same encoding as a cache quantised whole.  Because the scale depends on every token of the
 * block, the open block of each sequence is kept in bf16 in a staging row; token i is
 * written to staging offset slot % 16 and the block's live tokens 0 .. slot % 16 are
 * re-encoded from the staging row into the cache together with the new scale.  Once the
 * block's 16th token is in, the block is final.
 *   k_new, v_new   device bf16 [num_tokens][Hkv][head_dim]
 *   slot_mapping   device int64 [num_tokens]; < 0 or outside the pool: token skipped
 *   stage_rows     device int32 [num_tokens]: the staging row of the token's sequence;
 *                  outside [0, num_stage_rows): token skipped
 *   k_stage, v_stage device bf16 [num_stage_rows][Hkv][16][head_dim] (token-major), read
 *                  and written: offsets 0 .. slot % 16 - 1 of the row must hold the
 *                  block's earlier tokens (written by earlier calls, or by the caller
 *                  after filling a block some other way)
 *   k_cache, v_cache device 8-bit, written (offsets after slot % 16 are left as they are)
 *   k_scale, v_scale device fp32 [num_blocks][Hkv], written
 * dims->kv_dtype must be PA_I8 or PA_FP8 (else PA_ERR_DTYPE).  No two tokens of one call
 * may share a block or a staging row (they would race); a decode step appends one token per
 * sequence.  New tokens, staging rows and caches must be 16-byte aligned (PA_ERR_ALIGN).
 */
int kv_append_quant(const pa_dims* dims, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, const int32_t* stage_rows, int32_t num_tokens,
                    int32_t num_stage_rows, void* k_stage, void* v_stage, void* k_cache,
                    void* v_cache, float* k_scale, float* v_scale, void* stream);

/*
 * kv_copy_blocks -- copy whole physical blocks: for each pair (src, dst), every KV head's K
 * and V of block src (and, for int8 / fp8, its k_scale / v_scale) is copied to block dst, bit
 * for bit.  This is the copy-on-write step of block sharing (tutorial section 7: shared
 * blocks carry reference counts; a sequence about to write into a shared, partly filled
 * block first gets a private copy of it).
 *   block_pairs  device, [num_pairs][2] int32 (src, dst); a pair with a block outside
 *                [0, num_blocks) or src == dst is skipped
 *   k_cache, v_cache device, written in place (either layout, kv_tile_stride honoured)
 *   k_scale, v_scale device, [num_blocks][Hkv] fp32, written; required for PA_I8 and
 *                PA_FP8, ignored otherwise
 * Copies run concurrently: no destination may also be a source or appear twice (a
 * destination is a freshly allocated block).  num_pairs may be 0 (nothing is launched).
 */
int kv_copy_blocks(const pa_dims* dims, const int32_t* block_pairs, int32_t num_pairs,
                   void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   void* stream);

/*
 * paged_attn_balanced -- decode (nq = 1) or causal verify (nq > 1) attention with the work
 * dealt evenly over the waves of num_workgroups workgroups (four waves each), whatever the
 * spread of sequence lengths.  Every (KV head, query-row tile, sequence) segment of the
 * batch is laid out, block after block, in one flat list (KV head outermost, sequence
 * innermost) and wave v takes the contiguous slice [v * per, (v + 1) * per),
 * per = ceil(total blocks / waves).  A
 * segment that lies inside one slice is written to out (and out_lse) by this call; a
 * segment cut by slice boundaries leaves partial results in the workspace -- one per
 * piece, or, when a row tile holds more than 16 rows (G * nq > 16), one per workgroup,
 * the pieces of a workgroup's waves being combined on chip first (a segment inside one
 * workgroup is then written to out by this call too) -- and paged_attn_balanced_merge,
 * enqueued next on the same stream with the same arguments, recombines them with the
 * log-sum-exp identity (see lse_merge).  The pair is the complete operation.
 *   num_q_pos    nq >= 1; q [B][nq][Hq][head_dim]; out [B][nq][Hq][head_dim] fp32
 *   out_lse      device, [B][nq][Hq] fp32 (natural log; -inf for a row that sees no token),
 *                or NULL
 *   num_workgroups >= 1; paged_attn_balanced_workgroups gives a good value for the current
 *                device (one or two per compute unit)
 *   workspace    device, >= paged_attn_balanced_workspace_bytes(dims, nq, num_workgroups)
 *                bytes, 16-byte aligned; contents need no initialisation and are scratch
 *                from this call to the end of the merge (calls sharing one workspace must be
 *                ordered)
 * B may be at most 2048, and B * max_blocks_per_seq * num_kv_heads * (row tiles) and
 * num_blocks * num_kv_heads must stay below 2^31 (PA_ERR_DIMS otherwise).
 * Other arguments as paged_verify_attn.
 */
int paged_attn_balanced(const pa_dims* dims, int32_t num_q_pos, const void* q,
                        const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        const int32_t* seq_lens, float sm_scale, int32_t num_workgroups,
                        void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                        void* stream);

/*
 * paged_decode_step -- one decode step in one launch: kv_append of every sequence's new
 * token followed by paged_attn_balanced with nq = 1 (tutorial section 2 / lecture 10 "KV
 * Cache 原理": a step writes the new token's K and V into the cache, then its query attends
 * to all cached tokens including itself).  Sequence b's new token is its token
 * L - 1, L = seq_lens[b] (which counts it); its slot comes from the block table,
 * block_tables[b][(L - 1) / 16] * 16 + (L - 1) % 16 (tutorial section 7), so no slot
 * mapping is passed.
 *   k_new, v_new   device, [B][Hkv][head_dim] in kv_dtype (PA_F32 or PA_BF16; PA_I8 and
 *                  PA_FP8 give PA_ERR_DTYPE: use kv_append_quant, then
 *                  paged_attn_balanced); k_new 16-byte aligned
 *   k_cache, v_cache device, read and written: the new token lands in its slot bit for bit
 *   other arguments as paged_attn_balanced with num_q_pos = 1; complete the step with
 *   paged_attn_balanced_merge (num_q_pos = 1) on the same stream.
 * The result equals kv_append (a sequence with seq_lens[b] <= 0 appends nothing; a table
 * entry outside the pool is skipped) followed by paged_attn_balanced, provided no other
 * sequence of the batch reads a block that receives a new token -- a block being written
 * belongs to one sequence, as under copy-on-write block sharing.
 */
int paged_decode_step(const pa_dims* dims, const void* q, const void* k_new, const void* v_new,
                      void* k_cache, void* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, float sm_scale, int32_t num_workgroups,
                      void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                      void* stream);

/* Second half of paged_attn_balanced: writes the rows of cut segments (and of empty
 * sequences: zeros, lse -inf) from the partials the attention call left in the workspace.
 * dims, num_q_pos, num_workgroups, workspace, out and out_lse as in that call. */
int paged_attn_balanced_merge(const pa_dims* dims, int32_t num_q_pos, int32_t num_workgroups,
                              void* workspace, size_t workspace_bytes, float* out,
                              float* out_lse, void* stream);

/*
 * paged_decode_step_noalloc -- for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it): paged_decode_step followed by paged_attn_balanced_merge, with the workspace taken
 * from a static device array of the library instead of a caller buffer.  Arguments and
 * results as paged_decode_step (num_q_pos = 1); out_lse may be NULL.
 *   The array holds PA_NOALLOC_SCRATCH_BYTES (16 MiB) on each device the library runs on,
 *   for the life of the process; its address is looked up (hipGetSymbolAddress, no
 *   allocation) on the first call on each device, which is the only HIP call besides the
 *   two launches.  A call whose paged_attn_balanced_workspace_bytes(dims, 1,
 *   num_workgroups) exceeds it returns PA_ERR_SCRATCH before any HIP call (Llama-3-8B
 *   shapes at the default workgroup count fit up to ~2,000 (sequence, KV head) pairs).
 *   Every call on one device shares that device's array, and no part of it needs to start
 *   at zero (each call writes what it reads); calls that overlap on one device -- on
 *   different streams, or from different threads without ordering -- race on it and must
 *   be serialised by the caller.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int paged_decode_step_noalloc(const pa_dims* dims, const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              float sm_scale, int32_t num_workgroups, float* out, float* out_lse,
                              void* stream);

/* Workspace bytes paged_attn_balanced needs (0 if the arguments are invalid). */
size_t paged_attn_balanced_workspace_bytes(const pa_dims* dims, int32_t num_q_pos,
                                           int32_t num_workgroups);

/* A good num_workgroups for paged_attn_balanced on the current HIP device: one per compute
 * unit for up to 16 query rows per KV head (nq * Hq / Hkv) over an fp32 or bf16 cache, two
 * per unit for more rows or an 8-bit cache (fewer if
 * the kernel cannot keep two resident); a negative PA_ERR_* code on failure.  This call
 * queries the device (HIP calls), unlike the argument checks. */
int paged_attn_balanced_workgroups(const pa_dims* dims, int32_t num_q_pos);

/* Text for a status code (static storage). */
const char* paged_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */

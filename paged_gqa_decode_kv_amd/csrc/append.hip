// Slot-mapped KV append and the block-table gather (gfx950).
//
// Append (devpress tutorial section 2; lecture 10 "KV Cache 原理"): each decode step
// writes the new token's K and V into the cache.  The caller gives the slot
// (physical_block * 16 + offset) of every new token, as a block manager hands them out
// (tutorial section 7); the kernel is a plain bit copy into that slot.  K lands in row
// `offset` of each 16-byte column of the K tile, V in column `offset` of the dim-major V
// tile.  One thread per (token, KV head, dim); negative or out-of-pool slots are skipped.
//
// Gather copies every sequence's tokens out of the pool in logical order through the same
// tile addressing the attention kernels use, so its output checks that translation
// bit for bit.
//
// Quantising append into an int8 or fp8 cache (lecture 10 symmetric int8 rule; in-depth
// guide section 5.2 per-head scales, FP8 KV caches): a block's scale is max|x| / 127
// (int8) or max|x| / 448 (fp8 e4m3) over its live tokens, so the sequence's open block is
// kept in bf16 in a staging row and re-encoded from it whenever a token arrives.  One workgroup per (token, KV head), 2 * head_dim threads:
// thread j owns token j / (d / 8) of the block and 8 dims of it.
//
// Block copy (copy-on-write of shared blocks, tutorial section 7): for each (src, dst)
// pair every KV head's K and V tile of block src is copied to block dst (and the int8
// scales).  Each thread moves one 16-byte piece of one pair.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "pa_common.hpp"
#include "../../include/paged_attn.h"

namespace pa {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int64_t total, int32_t num_kv_heads,
    int32_t head_dim, int64_t num_blocks, int64_t tile_stride, T* __restrict__ k_cache,
    T* __restrict__ v_cache) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int k = (int)(idx % head_dim);
  const int g = (int)((idx / head_dim) % num_kv_heads);
  const int64_t t = idx / ((int64_t)head_dim * num_kv_heads);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_blocks * kBlockTokens) return;
  const int64_t blk = slot / kBlockTokens;
  const int off = (int)(slot % kBlockTokens);
  const int64_t tile = kv_tile(blk, g, num_kv_heads) * tile_stride;
  k_cache[tile + k_elem<sizeof(T)>(off, k)] = k_new[idx];
  v_cache[tile + v_elem(off, k)] = v_new[idx];
}

template <typename T>
__global__ __launch_bounds__(256) void kv_gather_kernel(
    const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    int64_t total, int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks,
    int64_t num_blocks, int64_t tile_stride, int32_t max_len, T* __restrict__ k_out,
    T* __restrict__ v_out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  // idx enumerates [B][Hkv][max_len][head_dim]
  const int k = (int)(idx % head_dim);
  const int tpos = (int)((idx / head_dim) % max_len);
  const int64_t bg = idx / ((int64_t)head_dim * max_len);
  const int g = (int)(bg % num_kv_heads);
  const int b = (int)(bg / num_kv_heads);
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : L);
  if (tpos >= L) return;
  const int32_t phys = block_tables[(int64_t)b * max_blocks + tpos / kBlockTokens];
  if (phys < 0 || phys >= num_blocks) return;
  const int off = tpos % kBlockTokens;
  const int64_t tile = kv_tile(phys, g, num_kv_heads) * tile_stride;
  k_out[idx] = k_cache[tile + k_elem<sizeof(T)>(off, k)];
  v_out[idx] = v_cache[tile + v_elem(off, k)];
}

template <typename T>
int append_t(const void* k_new, const void* v_new, const int64_t* slot_mapping,
             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
             int64_t tile_stride, void* k_cache, void* v_cache, hipStream_t s) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * head_dim;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  hipLaunchKernelGGL(kv_append_kernel<T>, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), slot_mapping,
                     total, num_kv_heads, head_dim, num_blocks, tile_stride,
                     static_cast<T*>(k_cache), static_cast<T*>(v_cache));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <typename T>
int gather_t(const void* k_cache, const void* v_cache, const int32_t* block_tables,
             const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
             int32_t max_blocks, int64_t num_blocks, int64_t tile_stride, int32_t max_len,
             void* k_out, void* v_out, hipStream_t s) {
  const int64_t total = (int64_t)num_seqs * num_kv_heads * max_len * head_dim;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  hipLaunchKernelGGL(kv_gather_kernel<T>, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const T*>(k_cache), static_cast<const T*>(v_cache),
                     block_tables, seq_lens, total, num_kv_heads, head_dim, max_blocks,
                     num_blocks, tile_stride, max_len, static_cast<T*>(k_out),
                     static_cast<T*>(v_out));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// A pair's data is 2 * Hkv tiles (K and V of every KV head), taken as 16-byte pieces in
// the order K(g = 0), V(0), K(1), ... (ascending addresses in the interleaved layout).
// Workgroup (pair, part) moves pieces [part * 256, (part + 1) * 256), one per thread, with
// non-temporal loads and stores: copied blocks are not read again by this launch, and
// keeping them out of the caches measured faster than plain accesses and than several
// pieces in flight per thread.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(
    const int32_t* __restrict__ pairs, int32_t num_kv_heads, int64_t num_blocks,
    int32_t tile_shift, int32_t parts, int64_t tile_stride_bytes, uint8_t* k_cache,
    uint8_t* v_cache, float* k_scale, float* v_scale) {
  const int64_t p = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const int total = (2 * num_kv_heads) << tile_shift;
  const int c = part * 256 + (int)threadIdx.x;
  if (c < total) {
    const int t = c >> tile_shift;
    uint8_t* base = (t & 1) ? v_cache : k_cache;
    const int64_t off = (int64_t)(c & ((1 << tile_shift) - 1)) * 16;
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        base + kv_tile(src, t >> 1, num_kv_heads) * tile_stride_bytes + off));
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(
        base + kv_tile(dst, t >> 1, num_kv_heads) * tile_stride_bytes + off));
  }
  if (k_scale != nullptr && part == 0) {
    for (int g = threadIdx.x; g < num_kv_heads; g += 256) {
      k_scale[kv_tile(dst, g, num_kv_heads)] = k_scale[kv_tile(src, g, num_kv_heads)];
      v_scale[kv_tile(dst, g, num_kv_heads)] = v_scale[kv_tile(src, g, num_kv_heads)];
    }
  }
}

// e4m3 byte of an fp32 value (OCP format: bias 7, 3 mantissa bits, subnormals below 2^-6):
// round to nearest, ties to even, magnitudes at or above 448 saturate to 448; the sign bit
// is the value's own.  The power-of-two scalings are exact, so rintf does the rounding.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {             // subnormal grid m * 2^-9 (m = 8 is 2^-6)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;
    int r = (int)__builtin_rintf(ldexpf(a, 3 - e));   // 8 .. 16
    if (r == 16) {
      e += 1;
      r = 8;
    }
    code = (uint32_t)(((e + 7) << 3) | (r - 8));
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

template <int D, bool FP8>
__global__ __launch_bounds__(2 * D) void kv_append_quant_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ stage_rows,
    int32_t num_kv_heads, int64_t num_blocks, int32_t num_stage_rows, int64_t tile_stride,
    uint16_t* __restrict__ k_stage, uint16_t* __restrict__ v_stage, int8_t* __restrict__ k_cache,
    int8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale) {
  constexpr int TPT = D / 8;  // threads per token
  constexpr int NW = 2 * D / kWave;
  const int64_t i = blockIdx.x / num_kv_heads;
  const int g = (int)(blockIdx.x % num_kv_heads);
  const int64_t slot = slot_mapping[i];
  const int row = stage_rows[i];
  if (slot < 0 || slot >= num_blocks * kBlockTokens || row < 0 || row >= num_stage_rows) return;
  const int64_t blk = slot / kBlockTokens;
  const int off = (int)(slot % kBlockTokens);
  const int t = threadIdx.x / TPT;
  const int k0 = (threadIdx.x % TPT) * 8;
  const int64_t srow = (((int64_t)row * num_kv_heads + g) * kBlockTokens + t) * D + k0;
  const int64_t nrow = ((int64_t)i * num_kv_heads + g) * D + k0;

  // this thread's 8 dims of token t: from the staging row, or the new token itself
  u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
  if (t < off) {
    kw = *reinterpret_cast<const u32x4*>(k_stage + srow);
    vw = *reinterpret_cast<const u32x4*>(v_stage + srow);
  } else if (t == off) {
    kw = *reinterpret_cast<const u32x4*>(k_new + nrow);
    vw = *reinterpret_cast<const u32x4*>(v_new + nrow);
    *reinterpret_cast<u32x4*>(k_stage + srow) = kw;
    *reinterpret_cast<u32x4*>(v_stage + srow) = vw;
  }
  float kx[8], vx[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kx[2 * e] = bf16_bits_to_f32(kw[e] & 0xffffu);
    kx[2 * e + 1] = bf16_bits_to_f32(kw[e] >> 16);
    vx[2 * e] = bf16_bits_to_f32(vw[e] & 0xffffu);
    vx[2 * e + 1] = bf16_bits_to_f32(vw[e] >> 16);
  }
  // max |x| over the live tokens (tokens after `off` hold zeros here)
  float km = 0.f, vm = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    km = fmaxf(km, fabsf(kx[e]));
    vm = fmaxf(vm, fabsf(vx[e]));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    km = fmaxf(km, __shfl_xor(km, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
  }
  __shared__ float s_max[2][NW];
  const int wv = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s_max[0][wv] = km;
    s_max[1][wv] = vm;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    km = fmaxf(km, s_max[0][w]);
    vm = fmaxf(vm, s_max[1][w]);
  }
  constexpr float kMax = FP8 ? 448.f : 127.f;
  const float ks = km / kMax, vs = vm / kMax;  // correctly rounded fp32 divisions
  if (threadIdx.x == 0) {
    k_scale[kv_tile(blk, g, num_kv_heads)] = ks;
    v_scale[kv_tile(blk, g, num_kv_heads)] = vs;
  }
  if (t > off) return;
  const int64_t tile = kv_tile(blk, g, num_kv_heads) * tile_stride;
  // codes: int8 round-half-even(x / scale) clamped to +-127, or e4m3(x / scale); 0 for a
  // zero scale
  uint32_t kc[2] = {0u, 0u};
  int8_t* vt = v_cache + tile;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t ck = 0u, cv = 0u;
    if constexpr (FP8) {
      if (ks > 0.f) ck = e4m3_encode(kx[e] / ks);
      if (vs > 0.f) cv = e4m3_encode(vx[e] / vs);
    } else {
      float qk = ks > 0.f ? __builtin_rintf(kx[e] / ks) : 0.f;
      float qv = vs > 0.f ? __builtin_rintf(vx[e] / vs) : 0.f;
      qk = fminf(fmaxf(qk, -127.f), 127.f);
      qv = fminf(fmaxf(qv, -127.f), 127.f);
      ck = (uint32_t)(int32_t)qk & 0xffu;
      cv = (uint32_t)(int32_t)qv & 0xffu;
    }
    kc[e / 4] |= ck << (8 * (e % 4));
    vt[v_elem(t, k0 + e)] = (int8_t)(uint8_t)cv;
  }
  // the 8 dims are contiguous inside one 16-byte K column
  *reinterpret_cast<u32x2*>(k_cache + tile + k_elem<1>(t, k0)) = u32x2{kc[0], kc[1]};
}

}  // namespace

int launch_append_quant(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                        const int32_t* stage_rows, int32_t num_tokens, int32_t num_stage_rows,
                        int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                        int64_t tile_stride, bool fp8, void* k_stage, void* v_stage,
                        void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                        void* stream) {
  const int64_t grid = (int64_t)num_tokens * num_kv_heads;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto k8 = static_cast<int8_t*>(k_cache);
  auto v8 = static_cast<int8_t*>(v_cache);
  auto kn = static_cast<const uint16_t*>(k_new);
  auto vn = static_cast<const uint16_t*>(v_new);
  auto kst = static_cast<uint16_t*>(k_stage);
  auto vst = static_cast<uint16_t*>(v_stage);
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, s, kn, vn, slot_mapping,
                       stage_rows, num_kv_heads, num_blocks, num_stage_rows, tile_stride, kst, vst,
                       k8, v8, k_scale, v_scale);
  };
  if (head_dim == 64)
    fp8 ? go(kv_append_quant_kernel<64, true>, 128) : go(kv_append_quant_kernel<64, false>, 128);
  else
    fp8 ? go(kv_append_quant_kernel<128, true>, 256) : go(kv_append_quant_kernel<128, false>, 256);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_dim, int64_t num_blocks, int64_t tile_stride,
                       int elem_bytes, void* k_cache, void* v_cache, float* k_scale,
                       float* v_scale, void* stream) {
  // pieces per tile = head_dim * elem_bytes (a power of two: 64 or 128 dims, 1/2/4 bytes)
  int shift = 0;
  while ((1 << shift) < head_dim * elem_bytes) ++shift;
  const int64_t total = (int64_t)(2 * num_kv_heads) << shift;
  const int64_t parts = (total + 255) / 256;
  const int64_t grid = (int64_t)num_pairs * parts;
  if (grid > 0x7fffffff || total > 0x7fffffff) return PA_ERR_DIMS;
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), pairs, num_kv_heads, num_blocks, shift,
                     (int32_t)parts, tile_stride * elem_bytes, static_cast<uint8_t*>(k_cache),
                     static_cast<uint8_t*>(v_cache), k_scale, v_scale);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int64_t num_blocks, int64_t tile_stride, int elem_bytes, void* k_cache,
                  void* v_cache, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (elem_bytes == 4)
    return append_t<uint32_t>(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim,
                              num_blocks, tile_stride, k_cache, v_cache, s);
  return append_t<uint16_t>(k_new, v_new, slot_mapping, num_tokens, num_kv_heads, head_dim,
                            num_blocks, tile_stride, k_cache, v_cache, s);
}

int launch_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                  int32_t head_dim, int32_t max_blocks, int64_t num_blocks, int64_t tile_stride,
                  int32_t max_len, int elem_bytes, void* k_out, void* v_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (elem_bytes == 4)
    return gather_t<uint32_t>(k_cache, v_cache, block_tables, seq_lens, num_seqs, num_kv_heads,
                              head_dim, max_blocks, num_blocks, tile_stride, max_len, k_out,
                              v_out, s);
  if (elem_bytes == 2)
    return gather_t<uint16_t>(k_cache, v_cache, block_tables, seq_lens, num_seqs, num_kv_heads,
                              head_dim, max_blocks, num_blocks, tile_stride, max_len, k_out,
                              v_out, s);
  return gather_t<uint8_t>(k_cache, v_cache, block_tables, seq_lens, num_seqs, num_kv_heads,
                           head_dim, max_blocks, num_blocks, tile_stride, max_len, k_out,
                              v_out, s);
}

}  // namespace pa

// Device-side building blocks shared by the paged-attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;  // tokens per KV block (lecture 10: "e.g. 16")
constexpr int kWave = 64;         // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ---- block-table translation (the only place the paged address is formed) ----------
// Logical block j of sequence b lives in physical block tables[b * max_blocks + j]; a
// (physical block, KV head) tile of K or V is 16 * head_dim consecutive elements.
__device__ __forceinline__ int64_t kv_tile(int64_t phys, int g, int num_kv_heads) {
  return phys * num_kv_heads + g;
}
// Element offset of token `off` (0..15), dim k inside a K tile: the tile is stored as
// 16-byte columns, [k / x][off][k % x] with x = 16 / element bytes, so that the 16 tokens'
// bytes [16c, 16c + 16) are contiguous -- one lane's MFMA operand per 16 bytes, one load
// instruction per 1 KiB.
template <int kElemBytes>
__device__ __forceinline__ int k_elem(int off, int k) {
  constexpr int x = 16 / kElemBytes;
  return (k / x) * (kBlockTokens * x) + off * x + (k % x);
}
// ... and inside a V tile: [k][off]
__device__ __forceinline__ int v_elem(int off, int k) { return k * kBlockTokens + off; }

// ---- small numeric helpers ------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// 4 packed int8 codes -> 4 exact fp16 values.  Flipping the sign bit maps code x to the
// unsigned byte x + 128; placing that byte in the low mantissa bits of the fp16 pattern
// 0x64XX gives the value 1024 + (x + 128), and subtracting 1152 leaves x exactly.
__device__ __forceinline__ f16x4 i8x4_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
  return f16x4{a[0], a[1], b[0], b[1]};
}

// 4 packed int8 codes -> 4 exact bf16 values (|code| <= 128 needs 8 significant bits, which
// bf16 has): each byte is sign-extended into an fp32 (v_cvt_f32_i32 with a byte select) and
// pairs are packed to bf16 (v_cvt_pk_bf16_f32, exact for these integers).
__device__ __forceinline__ bf16x4 i8x4_to_bf16x4(uint32_t w) {
  const float a = (float)(int8_t)(w & 0xFFu);
  const float b = (float)(int8_t)((w >> 8) & 0xFFu);
  const float c = (float)(int8_t)((w >> 16) & 0xFFu);
  const float d = (float)(int8_t)(w >> 24);
  return bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

// Lanes l, l^16, l^32 and l^48 hold the same query row.  gfx950's permlane swaps exchange
// 16-lane rows (xor 16) and 32-lane halves (xor 32) on the VALU, without an LDS round trip:
// given two registers that both hold x, v_permlane16_swap leaves rows (0,0,2,2) of x in
// the first and rows (1,1,3,3) in the second, so every lane ends with its own value and
// its partner's; v_permlane32_swap does the same for the two halves.
// (The two results are copied to scalars before any bit cast: a bit cast applied directly
// to an element of the returned vector reads element 0.)
__device__ __forceinline__ void xor16_pair(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float xor16_pair_max(float x) {
  float a, b;
  xor16_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor32_pair_max(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor16_pair_sum(float x) {
  float a, b;
  xor16_pair(x, a, b);
  return a + b;
}
__device__ __forceinline__ float xor32_pair_sum(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return a + b;
}
// 4 x 4 transpose of 32-bit words across the four 16-lane rows: on entry row s holds
// M[s][0..3] in w0..w3, on exit row g holds M[0..3][g].  The xor-32 swaps exchange the
// off-diagonal 2 x 2 blocks between the halves, the xor-16 swaps transpose each block.
__device__ __forceinline__ void transpose_rows4(uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                                uint32_t& w3) {
  auto r02 = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
  auto r13 = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
  const uint32_t a0 = r02[0], a2 = r02[1], a1 = r13[0], a3 = r13[1];
  auto r01 = __builtin_amdgcn_permlane16_swap(a0, a1, false, false);
  auto r23 = __builtin_amdgcn_permlane16_swap(a2, a3, false, false);
  w0 = r01[0];
  w1 = r01[1];
  w2 = r23[0];
  w3 = r23[1];
}

__device__ __forceinline__ float wave_max_across_groups(float x) {
  return xor32_pair_max(xor16_pair_max(x));
}
__device__ __forceinline__ float wave_sum_across_groups(float x) {
  return xor32_pair_sum(xor16_pair_sum(x));
}

}  // namespace pa

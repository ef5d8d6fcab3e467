// Paged GQA decode / verify attention for gfx950 (CDNA4).
//
// What is computed (devpress tutorial section 2: softmax(q K^T / sqrt(d)) V; lecture 10
// "KV Cache 原理"; GQA sharing from lecture 10 "Grouped Query Attention"): every query
// row of a sequence attends over the sequence's cached tokens, reached through its block
// table (tutorial section 7).  A (sequence, KV head) pair serves nq * G query rows: the G
// heads of the group at each of the nq positions (nq = 1 for decode, K + 1 for the
// speculative verify forward of guide section 4.2).
//
// How, on CDNA4:
//  * The G-head group is the N side of matrix-core (MFMA) tiles, so each K/V tile that is
//    read from HBM is used by the whole group straight out of registers:
//      S^T[16 tokens x 16 rows] = K_tile[16 x d] * Q^T[d x 16 rows]
//      O^T[d x 16 rows]        += V_tile^T[d x 16 tokens] * P^T[16 tokens x 16 rows]
//    K tiles are stored as 16-byte token columns and V tiles dim-major, which is exactly
//    the register layout both MFMA A-operands want: each K load instruction reads 1 KiB
//    in lane order and each V load 512 contiguous bytes.
//  * Online softmax in the log2 domain: per row a running reference (max) and a running
//    sum; the output accumulators are rescaled only when a block's scores exceed some
//    row's reference by more than a fixed margin (the weights stay bounded meanwhile).
//  * P feeds the bf16 P*V MFMA in two 16-bit pieces (hi + lo) so the product keeps ~16
//    significant bits of the fp32 probabilities; the 8-bit (int8, fp8) paths round P once
//    to fp16 (11 bits) and the fp32 path uses fp32 MFMA directly.
//  * int8 / fp8 K/V are decoded in registers to exact bf16 (K, beside the bf16 q) and fp16
//    (V, beside the fp16 weights); the per-(block, head) K scale multiplies the scores and
//    the V scale is folded into P.
//  * Direct / split modes: a workgroup of W waves owns one (sequence, KV head, row group,
//    partition); its waves take interleaved blocks and are merged through LDS at the end
//    (same LSE identity as the cross-workgroup split).  Balanced mode: every wave streams
//    its own equal slice of the batch's flat block list (see paged_attn_balanced_kernel).
//  * Workgroup ids are remapped so that consecutive units (same KV head, neighbouring
//    sequences -- e.g. sequences sharing a prefix) land on the same XCD and its L2.
#include <hip/hip_runtime.h>
#include <type_traits>

#include "launch.hpp"
#include "pa_common.hpp"
#include "../../include/paged_attn.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Where a K/V tile is read once per call (decode: one row tile per sequence and KV head),
// its loads carry the non-temporal hint: on MI355X a streaming read of HBM reaches ~7.0
// TB/s with it and ~6.2 TB/s without.  Where several workgroups read the same tiles (the
// row tiles of multi-query rows), plain loads let the second and later reads hit L2: the
// hint kept them from it (candidate-tree verify read 2.6x its unique bytes from HBM).
template <typename T, bool NTL = true>
__device__ __forceinline__ T stream_load(const void* p) {
  if constexpr (NTL) return __builtin_nontemporal_load(static_cast<const T*>(p));
  else return *static_cast<const T*>(p);
}

// ---------------------------------------------------------------------------------------
// Element-type traits.  Lane l of a wave has row16 = l % 16 and grp = l / 16.
//   K operand (MFMA A, 16 tokens x d):  lane holds token row16, a grp-dependent d slice.
//   Q operand (MFMA B, d x 16 rows):    lane holds query row row16, the same d slice.
//   S^T result:                          lane holds tokens 4*grp + v (v = 0..3), row row16.
//   V operand (MFMA A, 16 d x 16 tok):   lane holds d = 16*t + row16, tokens 4*grp .. +3.
//   O^T accumulator:                     lane holds d = 16*t + 4*grp + v, row row16.
// ---------------------------------------------------------------------------------------
template <int D>
struct Bf16Kv {
  static constexpr int NK = D / 32;  // 16x16x32 bf16 steps for q.K
  static constexpr int ND = D / 16;  // d tiles of the output
  static constexpr int kElem = 2;
  static constexpr float kLazy = 8.f;  // weights below 2^8: far inside fp32 and bf16 range
  static constexpr int kQElem = 2;
  struct Q { bf16x8 v[NK]; };
  struct K { u32x4 v[NK]; };
  struct V { u32x2 v[ND]; };

  // d index of step kk, element j: 32*kk + 8*grp + j
  __device__ static void load_q(Q& q, const void* row, bool valid, int grp) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      u32x4 x = valid ? *reinterpret_cast<const u32x4*>(p + 32 * kk) : u32x4{0, 0, 0, 0};
      q.v[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // lane (token row16, grp) step kk: column 4*kk + grp of the K tile, at kk*1 KiB + lane*16
  template <bool NTL = true>
  __device__ static void load_k(K& k, const void* tile, int lane) {
    const uint8_t* p = static_cast<const uint8_t*>(tile) + lane * 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) k.v[kk] = stream_load<u32x4, NTL>(p + 1024 * kk);
  }
  template <bool NTL = true>
  __device__ static void load_v(V& v, const void* tile, int row16, int grp) {
    const uint16_t* p = static_cast<const uint16_t*>(tile) + row16 * 16 + 4 * grp;
#pragma unroll
    for (int t = 0; t < ND; ++t) v.v[t] = stream_load<u32x2, NTL>(p + t * 256);
  }
  // the loaded tiles are the MFMA operands already
  using KMat = K;
  using VMat = V;
  __device__ static const K& k_mat(const K& k) { return k; }
  __device__ static const V& v_mat(const V& v) { return v; }
  __device__ static f32x4 qk(const K& k, const Q& q) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k.v[kk]), q.v[kk],
                                                  c, 0, 0, 0);
    return c;
  }
  // zero V of tokens >= nvalid (poisoned tail slots must not reach the MFMA: 0 * NaN)
  __device__ static void mask_v(V& v, int nvalid, int grp) {
    const int t0 = 4 * grp;
    const uint32_t m0 = (t0 + 0 < nvalid ? 0x0000FFFFu : 0u) | (t0 + 1 < nvalid ? 0xFFFF0000u : 0u);
    const uint32_t m1 = (t0 + 2 < nvalid ? 0x0000FFFFu : 0u) | (t0 + 3 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int t = 0; t < ND; ++t) {
      v.v[t].x &= m0;
      v.v[t].y &= m1;
    }
  }
  // Decode-step append: the new token's K and V as this lane needs them to patch a tile --
  // the 16-byte K chunk of column 4u + grp (the lane's chunk at every step u) and V[16t +
  // row16] -- and the patch itself (token `off` of the tile).
  struct NewTok { u32x4 k[NK]; uint32_t v[ND]; };
  __device__ static void load_new(NewTok& n, const void* krow, const void* vrow, int row16,
                                  int grp) {
    const uint8_t* kp = static_cast<const uint8_t*>(krow) + 16 * grp;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) n.k[kk] = *reinterpret_cast<const u32x4*>(kp + 64 * kk);
    const uint16_t* vp = static_cast<const uint16_t*>(vrow) + row16;
#pragma unroll
    for (int t = 0; t < ND; ++t) n.v[t] = vp[16 * t];
  }
  __device__ static void patch(K& k, V& v, const NewTok& n, int off, int row16, int grp) {
    if (row16 == off) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) k.v[kk] = n.k[kk];
    }
    if (grp == (off >> 2)) {
      const bool hi_half = off & 1;
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        uint32_t w = (off & 2) ? v.v[t].y : v.v[t].x;
        w = hi_half ? ((w & 0x0000FFFFu) | (n.v[t] << 16)) : ((w & 0xFFFF0000u) | n.v[t]);
        if (off & 2) v.v[t].y = w; else v.v[t].x = w;
      }
    }
  }
  // the token's K row then V row, in k_new / v_new order, into LDS (see the kernel)
  __device__ static void stash_new(uint8_t* dst, const NewTok& n, int row16, int grp) {
    if (row16 == 0) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) *reinterpret_cast<u32x4*>(dst + (4 * kk + grp) * 16) = n.k[kk];
    }
    if (grp == 0) {
#pragma unroll
      for (int t = 0; t < ND; ++t)
        reinterpret_cast<uint16_t*>(dst + 2 * D)[16 * t + row16] = (uint16_t)n.v[t];
    }
  }
  // P = hi + lo (two bf16 terms, relative error below 2^-16) so that P.V keeps fp32-class
  // accuracy: hi is p cut to its top 16 bits (a bf16 value, exact), lo = p - hi (exact in
  // fp32) rounded to bf16; a byte permute packs two hi halves, a mask and a subtraction give
  // each lo.  FOLD: both terms go through one 16x16x32 MFMA, whose 32-long inner dimension
  // holds the lane's 4 tokens twice, against hi then lo (sum_k A B = sum_t v_t (hi_t + lo_t)):
  // half the MFMA cycles for the compute-bound multi-query rows, at the cost of a duplicated
  // operand (two more registers, which the register-tight balanced kernels do not have).
  // Otherwise two 16x16x16 MFMAs.
  template <bool FOLD = false>
  __device__ static void pv(f32x4* acc, const V& v, f32x4 p, float /*vfac*/) {
    // (the elements are copied to scalars before the bit casts: a bit cast applied directly
    // to a vector element reads element 0)
    const float pf[4] = {p[0], p[1], p[2], p[3]};
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = __builtin_bit_cast(uint32_t, pf[e]);
    bf16x2 lo01, lo23;
    lo01[0] = (__bf16)(pf[0] - __builtin_bit_cast(float, u[0] & 0xFFFF0000u));
    lo01[1] = (__bf16)(pf[1] - __builtin_bit_cast(float, u[1] & 0xFFFF0000u));
    lo23[0] = (__bf16)(pf[2] - __builtin_bit_cast(float, u[2] & 0xFFFF0000u));
    lo23[1] = (__bf16)(pf[3] - __builtin_bit_cast(float, u[3] & 0xFFFF0000u));
    const u32x2 hi = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                      __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
    const u32x2 lo = {__builtin_bit_cast(uint32_t, lo01), __builtin_bit_cast(uint32_t, lo23)};
    if constexpr (FOLD) {
      const u32x4 hl = {hi.x, hi.y, lo.x, lo.y};
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        const u32x4 a = {v.v[t].x, v.v[t].y, v.v[t].x, v.v[t].y};
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, hl), acc[t],
                                                         0, 0, 0);
      }
    } else {
      const s16x4 h = __builtin_bit_cast(s16x4, hi);
      const s16x4 l = __builtin_bit_cast(s16x4, lo);
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        const s16x4 a = __builtin_bit_cast(s16x4, v.v[t]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, h, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, l, acc[t], 0, 0, 0);
      }
    }
  }
};

template <int D>
struct F32Kv {
  static constexpr int NU = D / 16;  // float4 pieces per lane (d = 16*u + 4*grp + e)
  static constexpr int ND = D / 16;
  static constexpr int kElem = 4;
  static constexpr int kQElem = 4;
  static constexpr float kLazy = 8.f;
  struct Q { f32x4 v[NU]; };
  struct K { f32x4 v[NU]; };
  struct V { f32x4 v[ND]; };

  __device__ static void load_q(Q& q, const void* row, bool valid, int grp) {
    const float* p = static_cast<const float*>(row) + 4 * grp;
#pragma unroll
    for (int u = 0; u < NU; ++u)
      q.v[u] = valid ? *reinterpret_cast<const f32x4*>(p + 16 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  template <bool NTL = true>
  __device__ static void load_k(K& k, const void* tile, int lane) {
    const uint8_t* p = static_cast<const uint8_t*>(tile) + lane * 16;
#pragma unroll
    for (int u = 0; u < NU; ++u) k.v[u] = stream_load<f32x4, NTL>(p + 1024 * u);
  }
  template <bool NTL = true>
  __device__ static void load_v(V& v, const void* tile, int row16, int grp) {
    const float* p = static_cast<const float*>(tile) + row16 * 16 + 4 * grp;
#pragma unroll
    for (int t = 0; t < ND; ++t) v.v[t] = stream_load<f32x4, NTL>(p + t * 256);
  }
  using KMat = K;
  using VMat = V;
  __device__ static const K& k_mat(const K& k) { return k; }
  __device__ static const V& v_mat(const V& v) { return v; }
  __device__ static f32x4 qk(const K& k, const Q& q) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[u][e], q.v[u][e], c, 0, 0, 0);
    return c;
  }
  __device__ static void mask_v(V& v, int nvalid, int grp) {
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * grp + e >= nvalid) v.v[t][e] = 0.f;
  }
  template <bool FOLD = false>
  __device__ static void pv(f32x4* acc, const V& v, f32x4 p, float /*vfac*/) {
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.v[t][e], p[e], acc[t], 0, 0, 0);
  }
  // decode-step append (as in Bf16Kv): K chunk of column 4u + grp, V[16t + row16]
  struct NewTok { f32x4 k[NU]; float v[ND]; };
  __device__ static void load_new(NewTok& n, const void* krow, const void* vrow, int row16,
                                  int grp) {
    const uint8_t* kp = static_cast<const uint8_t*>(krow) + 16 * grp;
#pragma unroll
    for (int u = 0; u < NU; ++u) n.k[u] = *reinterpret_cast<const f32x4*>(kp + 64 * u);
    const float* vp = static_cast<const float*>(vrow) + row16;
#pragma unroll
    for (int t = 0; t < ND; ++t) n.v[t] = vp[16 * t];
  }
  __device__ static void patch(K& k, V& v, const NewTok& n, int off, int row16, int grp) {
    if (row16 == off) {
#pragma unroll
      for (int u = 0; u < NU; ++u) k.v[u] = n.k[u];
    }
    if (grp == (off >> 2)) {
      const int e = off & 3;
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        f32x4 x = v.v[t];
        x[0] = e == 0 ? n.v[t] : x[0];
        x[1] = e == 1 ? n.v[t] : x[1];
        x[2] = e == 2 ? n.v[t] : x[2];
        x[3] = e == 3 ? n.v[t] : x[3];
        v.v[t] = x;
      }
    }
  }
  __device__ static void stash_new(uint8_t* dst, const NewTok& n, int row16, int grp) {
    if (row16 == 0) {
#pragma unroll
      for (int u = 0; u < NU; ++u) *reinterpret_cast<f32x4*>(dst + (4 * u + grp) * 16) = n.k[u];
    }
    if (grp == 0) {
#pragma unroll
      for (int t = 0; t < ND; ++t) reinterpret_cast<float*>(dst + 4 * D)[16 * t + row16] = n.v[t];
    }
  }
};

template <int D>
struct I8Kv {
  static constexpr int NH = D / 64;  // 16-byte K loads per lane (d = 64*h + 16*grp + 8*s + j)
  static constexpr int ND = D / 16;
  static constexpr int kElem = 1;
  static constexpr int kQElem = 2;
  // weights below 2^3: times the V-scale factor (at most 4096) they stay inside fp16
  static constexpr float kLazy = 3.f;
  // q stays bf16 (any bf16 value, no narrowing): the codes are decoded to exact bf16 for
  // the q.K MFMA; only the P.V side uses fp16 operands
  struct Q { bf16x8 v[2 * NH]; };
  struct K { u32x4 v[NH]; };
  struct V { uint32_t v[ND]; };

  // d index of step 2h + s, element j: 64h + 16 grp + 8s + j
  __device__ static void load_q(Q& q, const void* row, bool valid, int grp) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + 16 * grp;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 x =
            valid ? *reinterpret_cast<const u32x4*>(p + 64 * h + 8 * s) : u32x4{0, 0, 0, 0};
        q.v[2 * h + s] = __builtin_bit_cast(bf16x8, x);
      }
  }
  template <bool NTL = true>
  __device__ static void load_k(K& k, const void* tile, int lane) {
    const uint8_t* p = static_cast<const uint8_t*>(tile) + lane * 16;
#pragma unroll
    for (int h = 0; h < NH; ++h) k.v[h] = stream_load<u32x4, NTL>(p + 1024 * h);
  }
  // V is loaded 16 bytes at a time: lane (row16, grp) takes all 16 tokens of dims
  // 16 * (TPG * grp + u) + row16 (u < TPG = ND / 4), one 16-byte row of the [d][16] tile
  // each, so word 4u + c holds tokens 4c .. 4c + 3 of those dims.  v_mat() moves word c of
  // row group s to row group c (transpose_rows4), which gives every lane the tokens
  // 4 * grp .. 4 * grp + 3 of dims 16 t + row16 that the MFMA operand wants.  (Four-byte
  // loads in the operand order issue four times as many load instructions; the 16-byte
  // form measured 3-6% faster on the 8-bit workloads.)
  static constexpr int TPG = ND / 4;
  template <bool NTL = true>
  __device__ static void load_v(V& v, const void* tile, int row16, int grp) {
    const uint8_t* p = static_cast<const uint8_t*>(tile) + (16 * TPG * grp + row16) * 16;
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      const u32x4 x = stream_load<u32x4, NTL>(p + 256 * u);
      v.v[4 * u] = x.x;
      v.v[4 * u + 1] = x.y;
      v.v[4 * u + 2] = x.z;
      v.v[4 * u + 3] = x.w;
    }
  }
  // the operand word of tile t = TPG * c + u after the transpose of set u
  __device__ static void v_words(const V& v, uint32_t* w) {
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      uint32_t a = v.v[4 * u], b = v.v[4 * u + 1], c = v.v[4 * u + 2], d = v.v[4 * u + 3];
      transpose_rows4(a, b, c, d);
      w[u] = a;
      w[TPG + u] = b;
      w[2 * TPG + u] = c;
      w[3 * TPG + u] = d;
    }
  }
  // int8 codes decoded once per block to exact MFMA operands (shared by all row tiles):
  // K to bf16 (beside the bf16 q), V to fp16 (beside the fp16 weights)
  struct KMat { bf16x8 v[2 * NH]; };
  struct VMat { f16x4 v[ND]; };
  __device__ static KMat k_mat(const K& k) {
    KMat m;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const bf16x4 a0 = i8x4_to_bf16x4(k.v[h].x), a1 = i8x4_to_bf16x4(k.v[h].y);
      const bf16x4 a2 = i8x4_to_bf16x4(k.v[h].z), a3 = i8x4_to_bf16x4(k.v[h].w);
      m.v[2 * h] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      m.v[2 * h + 1] = bf16x8{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
    }
    return m;
  }
  __device__ static VMat v_mat(const V& v) {
    uint32_t w[ND];
    v_words(v, w);
    VMat m;
#pragma unroll
    for (int t = 0; t < ND; ++t) m.v[t] = i8x4_to_f16x4(w[t]);
    return m;
  }
  __device__ static f32x4 qk(const KMat& k, const Q& q) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2 * NH; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.v[s], q.v[s], c, 0, 0, 0);
    return c;
  }
  __device__ static void mask_v(V&, int, int) {}  // codes are finite; P = 0 removes them
  // (no decode-step append into int8 caches: never instantiated)
  struct NewTok {};
  __device__ static void load_new(NewTok&, const void*, const void*, int, int) {}
  __device__ static void patch(K&, V&, const NewTok&, int, int, int) {}
  __device__ static void stash_new(uint8_t*, const NewTok&, int, int) {}
  // p is scaled by vfac = 256 * v_scale(block) / v_ref and rounded once to fp16 (relative
  // error <= 2^-11 per weight, so |error of out| <= 2^-11 * max|V|, inside the int8
  // tolerance); the factor 256 keeps small weights out of the fp16 subnormal range.
  template <bool FOLD = false>
  __device__ static void pv(f32x4* acc, const VMat& v, f32x4 p, float vfac) {
    f16x4 ph;
#pragma unroll
    for (int e = 0; e < 4; ++e) ph[e] = (_Float16)(p[e] * vfac);
#pragma unroll
    for (int t = 0; t < ND; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(v.v[t], ph, acc[t], 0, 0, 0);
  }
};

// fp8 e4m3 codes (OCP format) with the same per-(block, KV head) scales and tile layout as
// int8.  gfx950 converts two e4m3 bytes to two fp16 or two bf16 values in one instruction
// (v_cvt_scalef32_pk_{f16,bf16}_fp8, scale 1); every e4m3 value, subnormals included, is
// exact in both (4 significant bits, exponents 2^-9 .. 2^8), so the MFMA operands are exact
// as for int8: K in bf16 beside the bf16 q, V in fp16 beside the fp16 weights.  Unlike
// int8, any byte pattern of an unused slot may be a NaN code, so V codes past the sequence
// end are zeroed.
__device__ __forceinline__ f16x4 fp8x4_to_f16x4(uint32_t w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return f16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return bf16x4{a[0], a[1], b[0], b[1]};
}

template <int D>
struct Fp8Kv : I8Kv<D> {
  using Base = I8Kv<D>;
  using typename Base::K;
  using typename Base::V;
  using typename Base::KMat;
  using typename Base::VMat;
  static constexpr int NH = Base::NH;
  static constexpr int ND = Base::ND;
  __device__ static KMat k_mat(const K& k) {
    KMat m;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const bf16x4 a0 = fp8x4_to_bf16x4(k.v[h].x), a1 = fp8x4_to_bf16x4(k.v[h].y);
      const bf16x4 a2 = fp8x4_to_bf16x4(k.v[h].z), a3 = fp8x4_to_bf16x4(k.v[h].w);
      m.v[2 * h] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      m.v[2 * h + 1] = bf16x8{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
    }
    return m;
  }
  __device__ static VMat v_mat(const V& v) {
    uint32_t w[ND];
    Base::v_words(v, w);
    VMat m;
#pragma unroll
    for (int t = 0; t < ND; ++t) m.v[t] = fp8x4_to_f16x4(w[t]);
    return m;
  }
  // as loaded, word 4u + c holds tokens 4c .. 4c + 3 (one byte each)
  __device__ static void mask_v(V& v, int nvalid, int) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int keep = nvalid - 4 * c;
      const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : (1u << (8 * keep)) - 1u);
#pragma unroll
      for (int u = 0; u < Base::TPG; ++u) v.v[4 * u + c] &= m;
    }
  }
};

// 8-bit codes with per-(block, KV head) scales (int8 or fp8)
template <class KV> struct Scaled8 { static constexpr bool value = false; };
template <int D> struct Scaled8<I8Kv<D>> { static constexpr bool value = true; };
template <int D> struct Scaled8<Fp8Kv<D>> { static constexpr bool value = true; };

// ---------------------------------------------------------------------------------------
// Where a unit writes its rows.
enum OutMode { kDirect = 0, kSplit = 1, kBalanced = 2 };

// Candidate visibility of a wave's query rows (multi-query rows with a tree mask): the
// mask words of each of the lane's NT rows and the position of the first candidate.
template <int NT>
struct TreeRows {
  uint32_t w[NT][4];
  int base;
};

// Running online-softmax state of one wave's query rows (a tile of 16 * NT rows) over
// the blocks it has consumed: the output accumulators (O^T layout), and per row the
// running max (log2 domain, equal in the four lanes of a row) and this lane's share of the
// running sum.  For int8 the V scales are folded into P relative to v_ref.
template <class KV, int D, int NT>
struct Rows {
  static constexpr int ND = D / 16;
  static constexpr bool kScaled = Scaled8<KV>::value;
  f32x4 acc[NT][ND];
  float m[NT], l[NT];
  float nmu[NT];  // -m, or 0 while m is -inf: the exponent offset of the weights
  bool big;       // some reference of the wave is 2^20 or more in magnitude
  float v_ref, inv_vref256;

  __device__ __forceinline__ void reset(float vref) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = -INFINITY;
      nmu[nt] = 0.f;
      l[nt] = 0.f;
#pragma unroll
      for (int t = 0; t < ND; ++t) acc[nt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    big = false;
    v_ref = kScaled ? vref : 1.f;
    inv_vref256 = kScaled ? 256.f / vref : 1.f;
  }

  // One 16-token block whose first token is tok0: rows see tokens in [lo[nt], lim[nt])
  // (lim_min is the smallest limit over the wave's rows, lo_max the largest start: a
  // sliding window's); tokens >= hi are past the sequence end and their V may be poisoned.  sc = softmax scale * log2(e) (times the block's K scale for int8);
  // vs = the block's V scale (int8).
  // SW: a sliding window is in force (the lower bounds are tested at all).  TREE: the
  // tokens from tr.base on are candidates, each visible to a row only if its bit in the
  // row's mask words is set.
  template <bool SW, bool TREE = false, bool FOLD = false>
  __device__ __forceinline__ void update(const typename KV::Q* qop, const int* lim, int lim_min,
                                         const int* lo, int lo_max, const TreeRows<NT>& tr,
                                         int hi, typename KV::K& kk, typename KV::V& vv,
                                         int tok0, float sc, float vs, int grp) {
    f32x4 pr[NT];
    const auto& km = KV::k_mat(kk);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pr[nt] = KV::qk(km, qop[nt]);
    consume<SW, TREE, FOLD>(pr, lim, lim_min, lo, lo_max, tr, hi, vv, tok0, sc, vs, grp);
  }

  // The same for a block whose raw scores q.K (unscaled) are already in pr (they are
  // overwritten).
  template <bool SW, bool TREE = false, bool FOLD = false>
  __device__ __forceinline__ void consume(f32x4* pr, const int* lim, int lim_min, const int* lo,
                                          int lo_max, const TreeRows<NT>& tr, int hi,
                                          typename KV::V& vv, int tok0, float sc, float vs,
                                          int grp) {
    // The lane's maximum is taken first: inlined right after the MFMAs of update(), it sits
    // in their basic block, where the wait states a VALU read of an MFMA result needs are
    // counted exactly, while a first read placed behind a branch was seen to get too few
    // (stale maxima, run-to-run differences in the last bits).  Masked blocks take it again
    // after the masks.
    float lm[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      lm[nt] = fmaxf(fmaxf(pr[nt][0], pr[nt][1]), fmaxf(pr[nt][2], pr[nt][3]));
    float vfac = 1.f;
    if constexpr (kScaled) {
      vfac = vs * inv_vref256;
      if (vs > 0.f && (vfac > 4096.f || vfac < 16.f)) {
        // this block's V scale is more than 16x above or below the reference: move the
        // reference to it, so that p * vfac (p <= 2^kLazy) stays below the fp16 maximum and
        // weights down to 2^-18 stay above the fp16 subnormals (a reference stuck at an
        // outlier block's scale would leave the later blocks' weights there)
        const float r = v_ref / vs;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int t = 0; t < ND; ++t) acc[nt][t] *= r;
        v_ref = vs;
        inv_vref256 = 256.f / vs;
        vfac = 256.f;
      }
    }
    // (one uniform test: blocks inside every row's range skip the per-token masks)
    const bool need_mask = tok0 + kBlockTokens > lim_min || (SW && tok0 < lo_max);
    // The scores stay unscaled until the exponent: the scale (positive, so the maximum of
    // the scaled scores is the scaled maximum, rounding included) enters the row maximum
    // once per row and each weight through one fused multiply-add, exp2(s * sc - m).  A
    // zero scale (an 8-bit block whose K scale is 0) is raised to the smallest normal
    // float, which leaves every product with a finite score at 0 to fp32 precision and keeps
    // a masked score's -inf an -inf.  The fused form differs from the rounded product
    // minus m by less than an ulp of m, which stays far below 1 while every reference of
    // the wave is below 2^20 in magnitude; beyond that (scores at the fp32 limits) the
    // weights take the rounded product, as the maximum does, so that the largest weight
    // is exactly 1.
    const float scp = fmaxf(sc, 1.17549435e-38f);
    // Lazy reference: a row's reference m moves only when a score of the block exceeds it
    // by more than KV::kLazy (log2 units), so the weights exp2(s - m) stay below 2^kLazy
    // and most blocks skip the rescale of the accumulators.  Softmax does not depend on
    // the reference, so the result is the same up to rounding.  Whether the block moves
    // any reference is decided from each lane's own 4 scores; the row maximum is reduced
    // across the row's four lanes only when it does.
    bool move = false;
    // blocks inside every row's range skip the per-token tests (a wave-wide branch)
    if (__any(need_mask)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = tok0 + 4 * grp + e;
          bool hide = t >= lim[nt] || (SW && t < lo[nt]);
          if constexpr (TREE) {
            // candidates: visible only where the row's mask bit is set
            const int j = t - tr.base;
            if (j >= 0) {
              const uint32_t wd = j < 32 ? tr.w[nt][0]
                                         : (j < 64 ? tr.w[nt][1] : (j < 96 ? tr.w[nt][2] : tr.w[nt][3]));
              hide |= ((wd >> (j & 31)) & 1u) == 0u;
            }
          }
          if (hide) pr[nt][e] = -INFINITY;
        }
        lm[nt] = fmaxf(fmaxf(pr[nt][0], pr[nt][1]), fmaxf(pr[nt][2], pr[nt][3]));
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lm[nt] *= scp;
      move |= lm[nt] > m[nt] + KV::kLazy;
    }
    if (__any(move)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float mn = fmaxf(m[nt], wave_max_across_groups(lm[nt]));
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[nt] - mn);
        m[nt] = mn;
        nmu[nt] = mn == -INFINITY ? 0.f : -mn;
        l[nt] *= alpha;
#pragma unroll
        for (int t = 0; t < ND; ++t) acc[nt][t] *= alpha;
      }
      bool b = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b |= m[nt] != -INFINITY && fabsf(m[nt]) >= 1048576.f;
      big = __any(b);
    }
    if (!big) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[nt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(pr[nt][e], scp, nmu[nt]));
    } else {
      // (two roundings on purpose: the product must not be contracted into the addition)
#pragma clang fp contract(off)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = pr[nt][e] * scp;
          pr[nt][e] = __builtin_amdgcn_exp2f(x + nmu[nt]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l[nt] += (pr[nt][0] + pr[nt][1]) + (pr[nt][2] + pr[nt][3]);
    if (tok0 + kBlockTokens > hi) KV::mask_v(vv, hi - tok0, grp);
    const auto& vm = KV::v_mat(vv);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) KV::template pv<FOLD>(acc[nt], vm, pr[nt], vfac);
  }

  // After the last block: full row sums in every lane of the row; int8 scale undone.
  __device__ __forceinline__ void totals() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      l[nt] = wave_sum_across_groups(l[nt]);
      if (kScaled) {
        const float f = v_ref * (1.f / 256.f);
#pragma unroll
        for (int t = 0; t < ND; ++t) acc[nt][t] *= f;
      }
    }
  }
};

// First token a query row at causal limit lam (it sees tokens < lam) may attend: with a
// sliding window of W tokens ending at its own position, lam - W.
__device__ __forceinline__ int window_start(int lam, int window) {
  return window > 0 && lam > window ? lam - window : 0;
}

// Query rows of row tile rg for KV head g of sequence b: the MFMA B operand of each 16-row
// tile and the visible range of this lane's row (tokens [lo, lim); lim capped at hi).
// Returns the smallest limit over the tile's rows; lo_max receives the largest start.
// TREE: every row may see tokens < L, the candidates [L - nq, L) subject to the row's mask
// words (loaded into tr); the returned limit is then the first candidate, from which on
// blocks need the per-token test.
template <class KV, int D, int NT, bool SW, bool TREE = false>
__device__ __forceinline__ int load_rows(const AttnArgs& a, int b, int g, int rg, int L, int hi,
                                         typename KV::Q* qop, int* lim, int* lo, int& lo_max,
                                         TreeRows<NT>& tr, int row16, int grp) {
  const int row_base = rg * 16 * NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = row_base + nt * 16 + row16;
    const bool valid = r < a.rows;
    const int i = valid ? r / a.group : 0;
    const int h = g * a.group + (valid ? r % a.group : 0);
    const int64_t qoff = ((int64_t)(b * a.num_q_pos + i) * a.num_q_heads + h) * D;
    KV::load_q(qop[nt], static_cast<const uint8_t*>(a.q) + qoff * KV::kQElem, valid, grp);
    int lam = valid ? L - a.num_q_pos + 1 + i : L;
    lam = lam < 0 ? 0 : lam;
    if constexpr (TREE) {
      lam = L;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        tr.w[nt][k] = valid && k < a.mask_words
                          ? (uint32_t)a.tree_mask[((int64_t)b * a.num_q_pos + i) * a.mask_words + k]
                          : 0u;
    }
    lim[nt] = lam < hi ? lam : hi;
    lo[nt] = SW ? window_start(lam, a.window) : 0;
  }
  if constexpr (TREE) {
    tr.base = L - a.num_q_pos;
    const int first = tr.base < 0 ? 0 : tr.base;
    lo_max = 0;
    return first < hi ? first : hi;
  }
  lo_max = 0;
  if constexpr (SW) {  // the tile's last row has the largest start
    int r_last = row_base + 16 * NT - 1;
    r_last = r_last < a.rows ? r_last : a.rows - 1;
    int lam_last = L - a.num_q_pos + 1 + r_last / a.group;
    lam_last = lam_last < 0 ? 0 : lam_last;
    lo_max = window_start(lam_last, a.window);
  }
  const int i0 = row_base / a.group;
  int lam0 = L - a.num_q_pos + 1 + i0;
  lam0 = lam0 < 0 ? 0 : lam0;
  return lam0 < hi ? lam0 : hi;
}

// Normalise a wave's finished rows and write them: to out (direct mode, plus out_lse if
// given), to a partition slot (split mode) or to a partial id of the workspace (balanced).
template <class KV, int D, int NT>
__device__ __forceinline__ void write_rows(const AttnArgs& a, const Rows<KV, D, NT>& st,
                                           OutMode mode, int b, int g, int rg, int64_t slot,
                                           float* out_lse, int row16, int grp) {
  constexpr int ND = D / 16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rl = nt * 16 + row16;  // row within the row tile
    const int r = rg * 16 * NT + rl;
    if (r >= a.rows) continue;
    const int i = r / a.group;
    const int h = g * a.group + r % a.group;
    const float lsum = st.l[nt];
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse = lsum > 0.f ? (st.m[nt] + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
    const int64_t orow = (int64_t)(b * a.num_q_pos + i) * a.num_q_heads + h;
    float* dst;
    float* lse_dst = nullptr;
    if (mode == kDirect) {
      dst = a.out + orow * D;
      if (out_lse != nullptr) lse_dst = out_lse + orow;
    } else if (mode == kSplit) {
      dst = a.out + (orow * a.max_parts + slot) * D;
      lse_dst = a.part_lse + orow * a.max_parts + slot;
    } else {
      dst = a.ws_out + (slot * 16 * NT + rl) * D;
      lse_dst = a.ws_lse + slot * 16 * NT + rl;
    }
#pragma unroll
    for (int t = 0; t < ND; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * grp) = st.acc[nt][t] * inv;
    if (lse_dst != nullptr && grp == 0) *lse_dst = lse;
  }
}

// One unit of work: query rows [16*NT*rg, 16*NT*(rg+1)) of KV head g of sequence b, over
// that sequence's tokens [lo, hi) (lo a multiple of 16).  The W waves of the workgroup
// take interleaved blocks; their partial results are merged through LDS and wave 0
// writes the normalised rows (and, except in direct mode, their log-sum-exp).
// `slot` is the partition index (split mode).  SW: a sliding window is in force (each row
// also has a first visible token).  Every wave of the workgroup must call this together
// (it contains barriers).
template <class KV, int D, int NT, int W, int NBUF, bool SW, bool TREE = false, int RG = 1,
          bool REUSE = false>
__device__ __forceinline__ void attend_unit(const AttnArgs& a, OutMode mode, int b, int g, int rg,
                                            int L, int lo, int hi, int64_t slot) {
  constexpr int ND = D / 16;
  constexpr bool kScaled = Scaled8<KV>::value;
  constexpr int kStage = 64;  // table entries staged in LDS per wave
  constexpr int WS = W / RG;  // waves per row tile
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  // RG > 1: the workgroup serves RG row tiles (rg is then the index of that group of
  // tiles), WS waves each, which read the same blocks side by side (one HBM read of a
  // block serves them all); a tile past the last one reads nothing but keeps the barriers
  const int sub = w / WS, wl = w % WS;
  const int nrg = (a.rows + 16 * NT - 1) / (16 * NT);
  const int rt = rg * RG + sub;
  const bool live = rt < nrg;

  const int jb = lo / kBlockTokens;
  const int je = live ? (hi + kBlockTokens - 1) / kBlockTokens : jb;
  // this wave's blocks: jb + wl + WS * k for k in [0, nk)
  const int nk = je - jb - wl > 0 ? (je - jb - wl + WS - 1) / WS : 0;

  typename KV::Q qop[NT];
  int lim[NT], lo_row[NT], lo_max;
  TreeRows<NT> tr;
  const int lim_min = load_rows<KV, D, NT, SW, TREE>(a, b, g, live ? rt : 0, L, hi, qop, lim,
                                                     lo_row, lo_max, tr, row16, grp);

  const int64_t tile_bytes = a.tile_stride;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache);
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  // ---- per-wave LDS staging of block-table entries (and int8 scales) -------------------
  // Lane i fetches the entry of this wave's block k0 + i; the loop then reads them back
  // from LDS, so no dependent HBM load sits between consecutive tile loads.
  __shared__ int s_tbl[W][kStage];
  __shared__ float s_ks[W][kScaled ? kStage : 1];
  __shared__ float s_vs[W][kScaled ? kStage : 1];
  auto stage = [&](int k0) {
    const int k = k0 + lane;
    int ph = -1;
    if (k < nk) {
      ph = table[jb + wl + WS * k];
      if (ph < 0 || (int64_t)ph >= a.num_blocks) ph = -1;
    }
    s_tbl[w][lane] = ph;
    if constexpr (kScaled) {
      float ks = 0.f, vs = 0.f;
      if (ph >= 0) {
        ks = a.k_scale[kv_tile(ph, g, a.num_kv_heads)];
        vs = a.v_scale[kv_tile(ph, g, a.num_kv_heads)];
      }
      s_ks[w][lane] = ks;
      s_vs[w][lane] = vs;
    }
  };
  stage(0);
  auto lds_uniform_f = [](const float& x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
  };
  // block k of this wave: physical block (-1 = none) and, for int8, its K and V scales
  struct Slot {
    int ph;
    float ks, vs;
  };
  auto slot_at = [&](int k) -> Slot {
    Slot sl{-1, 0.f, 0.f};
    if (k < nk) {
      const int si = k & (kStage - 1);
      sl.ph = __builtin_amdgcn_readfirstlane(s_tbl[w][si]);
      if constexpr (kScaled) {
        sl.ks = lds_uniform_f(s_ks[w][si]);
        sl.vs = lds_uniform_f(s_vs[w][si]);
      }
    }
    return sl;
  };

  // int8: each block's V scale is folded into P relative to a reference scale
  float v_ref = 1.f;
  if constexpr (kScaled) {
    if (nk > 0) {
      const float s0 = lds_uniform_f(s_vs[w][0]);
      if (s0 > 0.f && s0 < 3.0e38f) v_ref = s0;
    }
  }
  Rows<KV, D, NT> st;
  st.reset(v_ref);

  // Loads are issued unconditionally: a slot with no block (past the end, or a table
  // entry outside the pool) reads tile (0, g), which is always inside the pool, and is
  // then not consumed.  Straight-line loads keep the wait counters exact, so NBUF - 1
  // blocks stay in flight while one is consumed.
  auto issue = [&](typename KV::K& kk, typename KV::V& vv, int ph) {
    const int64_t tl = kv_tile(ph >= 0 ? ph : 0, g, a.num_kv_heads);
    KV::template load_k<!REUSE>(kk, kbase + tl * tile_bytes, lane);
    KV::template load_v<!REUSE>(vv, vbase + tl * tile_bytes, row16, grp);
  };
  auto consume = [&](typename KV::K& kk, typename KV::V& vv, int kidx, const Slot& sl) {
    if (sl.ph < 0) return;
    const int tok0 = (jb + wl + WS * kidx) * kBlockTokens;
    st.template update<SW, TREE, true>(qop, lim, lim_min, lo_row, lo_max, tr, hi, kk, vv, tok0,
              a.scale_log2 * (kScaled ? sl.ks : 1.f), sl.vs, grp);
  };

  {
    typename KV::K kb[NBUF];
    typename KV::V vb[NBUF];
    Slot sb[NBUF];
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
      sb[s] = slot_at(s);
      issue(kb[s], vb[s], sb[s].ph);
    }
    for (int k = 0; k < nk; k += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const int kn = k + s + NBUF - 1;  // block issued now, consumed NBUF - 1 steps later
        const int sn = (s + NBUF - 1) % NBUF;
        if ((kn & (kStage - 1)) == 0 && kn < nk) stage(kn);
        sb[sn] = slot_at(kn);
        issue(kb[sn], vb[sn], sb[sn].ph);
        consume(kb[s], vb[s], k + s, sb[s]);
      }
    }
  }
  st.totals();

  // ---- merge the WS waves of each row tile through LDS (its wave 0 finishes) ----------
  if constexpr (WS > 1) {
    __shared__ float sm_m[RG][WS - 1][NT * 16];
    __shared__ float sm_l[RG][WS - 1][NT * 16];
    __shared__ f32x4 sm_acc[RG][WS - 1][NT][ND][kWave];
    if (wl > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (grp == 0) {
          sm_m[sub][wl - 1][nt * 16 + row16] = st.m[nt];
          sm_l[sub][wl - 1][nt * 16 + row16] = st.l[nt];
        }
#pragma unroll
        for (int t = 0; t < ND; ++t) sm_acc[sub][wl - 1][nt][t][lane] = st.acc[nt][t];
      }
    }
    __syncthreads();
    if (wl == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float M = st.m[nt];
#pragma unroll
        for (int x = 0; x < WS - 1; ++x) M = fmaxf(M, sm_m[sub][x][nt * 16 + row16]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        const float f0 = __builtin_amdgcn_exp2f(st.m[nt] - Mu);
        float lsum = st.l[nt] * f0;
#pragma unroll
        for (int t = 0; t < ND; ++t) st.acc[nt][t] *= f0;
#pragma unroll
        for (int x = 0; x < WS - 1; ++x) {
          const float fx = __builtin_amdgcn_exp2f(sm_m[sub][x][nt * 16 + row16] - Mu);
          lsum += sm_l[sub][x][nt * 16 + row16] * fx;
#pragma unroll
          for (int t = 0; t < ND; ++t) st.acc[nt][t] += sm_acc[sub][x][nt][t][lane] * fx;
        }
        st.m[nt] = M;
        st.l[nt] = lsum;
      }
    }
    __syncthreads();
    if (wl != 0) return;
  }
  if (!live) return;
  write_rows<KV, D, NT>(a, st, mode, b, g, rt, slot, mode == kDirect ? a.ws_out_lse : nullptr,
                        row16, grp);
}

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  return L < 0 ? 0 : (L > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : L);
}

// Workgroup id -> logical unit, so that consecutive units run on the same XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin).  gridDim.x is a multiple of 8.
__device__ __forceinline__ int64_t xcd_logical_id() {
  const int64_t per_xcd = gridDim.x / 8;
  return (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
}

// Occupancy the register allocation is asked to allow (waves per SIMD).  With a target
// above one wave the accumulators share the unified register file with the rest, which
// lets one row tile fit three waves per SIMD and two row tiles two.
// (fp32 tiles are twice as large, so they get one step less.)
template <class KV, int NT> struct WavesPerEU {
  static constexpr int value = (KV::kElem == 4 ? 2 : 3) - (NT == 1 ? 0 : 1);
};

// Direct and split modes: one unit per (KV head, sequence, row group, partition).
// TREE: multi-query rows whose candidates are filtered by a visibility mask (direct mode).
// RG > 1: each workgroup serves RG row tiles of its (sequence, KV head) (multi-query rows).
// REUSE: several workgroups read each tile (plain loads, which L2 keeps).
// The sequence of rank r in the batch ordered by decreasing length (ties by index), for
// batches of up to 64 sequences (one per lane; larger batches keep their order).  Units are
// dealt in rank order, so every XCD starts on its longest units and the short ones fill
// in behind them (longest-processing-time-first): with 4 to 32 sequences of uneven length
// the last workgroups otherwise ran alone for a fifth of the time.
constexpr int kRankedSeqs = 64;
__device__ __forceinline__ int seq_by_rank(const AttnArgs& a, int r) {
  const int B = a.num_seqs;
  if (B > kRankedSeqs) return r;
  const int lane = threadIdx.x & (kWave - 1);
  const int Li = lane < B ? clamp_len(a.seq_lens[lane], a.max_blocks) : -1;
  int rank = 0;
  for (int j = 0; j < B; ++j) {
    const int Lj = __builtin_amdgcn_readlane(Li, j);
    rank += (Lj > Li || (Lj == Li && j < lane)) ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < B && rank == r);
  return hit != 0 ? (int)__builtin_ctzll(hit) : r;
}

template <class KV, int D, int NT, int W, int NBUF, bool SW, bool TREE = false, int RG = 1,
          bool REUSE = false>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(WavesPerEU<KV, NT>::value)))
void paged_attn_kernel(AttnArgs a) {
  const int nrg = (a.rows + 16 * NT * RG - 1) / (16 * NT * RG);  // (groups of) row tiles
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * nrg * a.max_parts;
  const int64_t u = xcd_logical_id();
  if (u >= units) return;
  // (the grid, and so u, fits in int32: 32-bit divisions)
  const unsigned uu = (unsigned)u;
  const int p = (int)(uu % (unsigned)a.max_parts);
  unsigned rest = uu / (unsigned)a.max_parts;
  const int rg = (int)(rest % (unsigned)nrg);
  rest /= (unsigned)nrg;
  const int b = __builtin_amdgcn_readfirstlane(seq_by_rank(a, (int)(rest % (unsigned)a.num_seqs)));
  const int g = (int)(rest / (unsigned)a.num_seqs);
  const int L = clamp_len(a.seq_lens[b], a.max_blocks);
  int lo = 0, hi = L;
  if (a.split) {
    int nparts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 0;
    if (nparts > a.max_parts) nparts = a.max_parts;
    if (p >= nparts) return;
    lo = p * a.part_tokens;
    hi = (p == nparts - 1) ? L : lo + a.part_tokens;
  }
  // sliding window: no row of this sequence sees a block before the first row's window
  // (a partition wholly before it is left empty: zero rows, lse = -inf)
  if (SW) {
    int lam0 = L - a.num_q_pos + 1;
    lam0 = lam0 < 0 ? 0 : lam0;
    const int w0 = window_start(lam0, a.window) / kBlockTokens * kBlockTokens;
    lo = lo > w0 ? lo : w0;
    if (hi < lo) hi = lo;  // lo is a multiple of 16 here, so the unit reads no block
  }
  attend_unit<KV, D, NT, W, NBUF, SW, TREE, RG, REUSE>(a, a.split ? kSplit : kDirect, b, g, rg,
                                                       L, lo, hi, p);
}

// Balanced mode.  All (segment, block) pairs of the batch are laid out in one flat list --
// segment j = (KV head g, row group rg, sequence b) in order j = (g * nrg + rg) * B + b,
// holding ceil(L_b / 16) blocks -- and wave v (of num_workgroups * W) takes the contiguous
// slice [v * per, (v + 1) * per) with per = ceil(total / waves).  Every wave therefore
// streams the same number of blocks whatever the spread of sequence lengths, and it
// streams them without a break: its ring of tile loads runs on across segment boundaries,
// and the next segment's query rows are loaded while the current segment's last blocks
// are still being consumed.  A segment that lies wholly inside one slice is written out
// directly; otherwise each piece becomes a partial result at partial id v + j (unique:
// along the slices both v and j only grow) and the merge kernel combines the pieces.
//
// APP (decode step, nq = 1): the token at position L_b - 1 of every sequence is new this
// step.  Its K and V come from a.k_new / a.v_new [B][Hkv][d] rather than from the cache:
// the wave that consumes the tile holding it patches the token into the tile registers
// before the MFMAs, so one launch does the append and the attention.  The new-token rows
// are fetched together with the segment's query rows.  The slot itself is written at the
// end of the wave's slice (row group 0 only), from a copy kept in LDS: stores into the
// cache while the wave still streams cost ~5% (measured on MI355X), at the end ~0.4%.
//
// SW (sliding window): each sequence's list starts at the block that holds its first
// row's first visible token, so the blocks before the window are never dealt out.  The
// window is a separate instantiation because its bookkeeping cost 1-2% when compiled in.
// s_waitcnt immediate for vmcnt(0) with the other counters left open (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmem0 = 0x0F70;

// The balanced kernel runs at most two workgroups of W = 4 waves per compute unit (two
// waves per SIMD), so it may use the registers of two waves (fp32 with two row tiles:
// of one).
#ifndef PA_BAL_WAVES_PER_EU
#define PA_BAL_WAVES_PER_EU 2
#endif
#ifndef PA_BAL_PRIO
#define PA_BAL_PRIO 1
#endif
template <class KV, int NT> struct BalancedWavesPerEU {
  static constexpr int value = WavesPerEU<KV, NT>::value < PA_BAL_WAVES_PER_EU
                                   ? WavesPerEU<KV, NT>::value
                                   : PA_BAL_WAVES_PER_EU;
};

template <class KV, int D, int NT, int W, int NBUF, bool APP, bool SW>
__global__ __launch_bounds__(kWave* W)
__attribute__((amdgpu_waves_per_eu(BalancedWavesPerEU<KV, NT>::value)))
void paged_attn_balanced_kernel(AttnArgs a) {
  constexpr bool kScaled = Scaled8<KV>::value;
  constexpr int kStage = 64;
  __shared__ int s_pref[kMaxBalancedSeqs + 1];
  __shared__ int s_fb[SW ? kMaxBalancedSeqs : 1];  // first block a row of the sequence may see
  // The lengths stay in LDS: a global load of one at a segment switch would be counted with
  // the tile loads in flight, and waiting for it would drain the wave's ring.
  __shared__ int s_len[kMaxBalancedSeqs];
  const int64_t wid = xcd_logical_id();
  if (wid >= a.num_workgroups) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int B = a.num_seqs;

  // prefix over sequences of their block counts, by the whole workgroup.  With a sliding
  // window a sequence's list starts at the block holding its first row's first visible
  // token; the blocks before it are not dealt out at all.
  __shared__ int s_scan[kWave * W];
  // two row tiles: LDS slot w - 1 holds wave w's parked piece once its flag is set
  constexpr bool kComb = NT > 1;
  __shared__ int s_dflag[kComb ? W - 1 : 1];
  if (kComb && threadIdx.x < W - 1) s_dflag[threadIdx.x] = 0;
  int carry = 0;
  if (threadIdx.x == 0) s_pref[0] = 0;
  for (int c0 = 0; c0 < B; c0 += kWave * W) {
    const int bb = c0 + (int)threadIdx.x;
    int nb = 0;
    if (bb < B) {
      const int Lb = clamp_len(a.seq_lens[bb], a.max_blocks);
      s_len[bb] = Lb;
      int lam0 = Lb - a.num_q_pos + 1;
      lam0 = lam0 < 0 ? 0 : lam0;
      int fb = 0;
      if constexpr (SW) {
        fb = window_start(lam0, a.window) / kBlockTokens;
        s_fb[bb] = fb;
      }
      nb = (Lb + kBlockTokens - 1) / kBlockTokens - fb;
    }
    s_scan[threadIdx.x] = nb;
    __syncthreads();
    for (int off = 1; off < kWave * W; off <<= 1) {
      const int t = threadIdx.x >= (unsigned)off ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += t;
      __syncthreads();
    }
    if (bb < B) s_pref[bb + 1] = carry + s_scan[threadIdx.x];
    carry += s_scan[kWave * W - 1];
    __syncthreads();
  }
  if (wid == 0) {
    for (int k = threadIdx.x; k <= B; k += kWave * W) a.ws_prefix[k] = s_pref[k];
  }
  // (no barrier below this point: the waves are independent)

  // (the host keeps B * max_blocks * Hkv * nrg below 2^31, so flat positions are int32)
  const int nrg = (a.rows + 16 * NT - 1) / (16 * NT);
  const int T = __builtin_amdgcn_readfirstlane(s_pref[B]);
  const int total = T * a.num_kv_heads * nrg;
  const int per = (int)(((unsigned)total + (unsigned)a.num_workers - 1u) / (unsigned)a.num_workers);
  const int64_t v = wid * W + w;
  if (v * per >= total) return;
  const int x0 = (int)(v * per);
  const int x1 = total - x0 > per ? x0 + per : total;
  const int n = x1 - x0;  // blocks of this wave

  // segment of flat position x (uniform in the wave)
  struct Seg {
    int j, start, end;
    int b, g, rg;
    int fb;  // table index of the segment's first block
  };
  auto locate = [&](int x) -> Seg {
    Seg sg;
    const int gr = x / T;
    const int r = x - gr * T;
    int lo_b = 0, hi_b = B - 1;  // largest b with s_pref[b] <= r
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_pref[mid]) <= r) lo_b = mid; else hi_b = mid - 1;
    }
    sg.b = lo_b;
    sg.g = gr / nrg;
    sg.rg = gr % nrg;
    sg.j = gr * B + lo_b;
    sg.start = gr * T + __builtin_amdgcn_readfirstlane(s_pref[lo_b]);
    sg.end = gr * T + __builtin_amdgcn_readfirstlane(s_pref[lo_b + 1]);
    sg.fb = SW ? __builtin_amdgcn_readfirstlane(s_fb[lo_b]) : 0;
    return sg;
  };

  const int64_t tile_bytes = a.tile_stride;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache);

  // ---- per-wave LDS staging: tile index (physical block * Hkv + g, -1 = none) and int8
  // scales of this wave's blocks k0 .. k0 + 63; lane i resolves its own block's segment.
  __shared__ int s_tile[W][kStage];
  __shared__ float s_ks[W][kScaled ? kStage : 1];
  __shared__ float s_vs[W][kScaled ? kStage : 1];
  auto stage = [&](int k0) {
    const int k = k0 + lane;
    int tile = -1;
    float ks = 0.f, vs = 0.f;
    if (k < n) {
      const int x = x0 + k;
      const int gr = x / T;
      const int r = x - gr * T;
      int lo_b = 0, hi_b = B - 1;
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (s_pref[mid] <= r) lo_b = mid; else hi_b = mid - 1;
      }
      const int g = gr / nrg;
      const int ph = a.block_tables[(int64_t)lo_b * a.max_blocks + (r - s_pref[lo_b]) +
                                    (SW ? s_fb[lo_b] : 0)];
      if (ph >= 0 && (int64_t)ph < a.num_blocks) {
        tile = (int)kv_tile(ph, g, a.num_kv_heads);
        if constexpr (kScaled) {
          ks = a.k_scale[tile];
          vs = a.v_scale[tile];
        }
      }
    }
    s_tile[w][lane] = tile;
    if constexpr (kScaled) {
      s_ks[w][lane] = ks;
      s_vs[w][lane] = vs;
    }
  };
  auto lds_uniform_f = [](const float& x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
  };
  struct Slot {
    int tile;
    float ks, vs;
  };
  auto slot_at = [&](int k) -> Slot {
    Slot sl{-1, 0.f, 0.f};
    if (k < n) {
      const int si = k & (kStage - 1);
      sl.tile = __builtin_amdgcn_readfirstlane(s_tile[w][si]);
      if constexpr (kScaled) {
        sl.ks = lds_uniform_f(s_ks[w][si]);
        sl.vs = lds_uniform_f(s_vs[w][si]);
      }
    }
    return sl;
  };
  stage(0);

  // ---- current segment (being consumed) and the prefetched next one -----------------
  Seg cur;
  cur.end = x0;  // nothing consumed yet
  cur.j = -1;
  int L = 0, lim_min = 0, lim[NT], lo_row[NT], lo_max = 0;
  TreeRows<NT> no_tree;  // (the balanced kernel has causal rows only)
  typename KV::Q qop[NT], qnext[NT];
  int lim_next[NT], lim_min_next = 0, lo_next[NT], lo_max_next = 0;
  typename KV::NewTok tok, tok_next;  // APP: the new token of the current / next segment
  Seg nxt;                 // segment whose rows sit in qnext (valid while nxt.j >= 0)
  nxt.j = -1;
  int iss_end = x0;        // end of the segment of the newest issued block
  Rows<KV, D, NT> st;
  st.reset(1.f);

  // APP: new tokens whose slot this wave writes at the end: (tile, offset) and the rows
  constexpr int kAppCap = 8;
  constexpr int kRowBytes = APP ? 2 * D * KV::kElem : 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_appd[W][APP ? kAppCap : 1][kRowBytes];
  __shared__ int s_appm[W][APP ? kAppCap : 1][2];
  int napp = 0;
  auto drain = [&]() {
    for (int r = 0; r < napp; ++r) {
      const int tile = __builtin_amdgcn_readfirstlane(s_appm[w][r][0]);
      const int off = __builtin_amdgcn_readfirstlane(s_appm[w][r][1]);
      uint8_t* kt = const_cast<uint8_t*>(kbase) + (int64_t)tile * tile_bytes;
      uint8_t* vt = const_cast<uint8_t*>(vbase) + (int64_t)tile * tile_bytes;
      const uint8_t* src = s_appd[w][r];
      // K: 16-byte chunk c (x elements) of the row goes to column c, row off
      for (int c = lane; c < D * KV::kElem / 16; c += kWave)
        *reinterpret_cast<u32x4*>(kt + c * 256 + off * 16) =
            *reinterpret_cast<const u32x4*>(src + c * 16);
      // V: element d goes to [d][off]
      for (int d = lane; d < D; d += kWave) {
        if constexpr (KV::kElem == 4)
          reinterpret_cast<uint32_t*>(vt)[d * kBlockTokens + off] =
              reinterpret_cast<const uint32_t*>(src + 4 * D)[d];
        else
          reinterpret_cast<uint16_t*>(vt)[d * kBlockTokens + off] =
              reinterpret_cast<const uint16_t*>(src + 2 * D)[d];
      }
    }
    napp = 0;
  };

  auto rows_hi = [&](const Seg& sg, int Ls) {
    // tokens this wave may read in the segment: up to the end of its slice or the sequence
    const int last = sg.end < x1 ? sg.end : x1;
    const int hi_t = (last - sg.start + sg.fb) * kBlockTokens;
    return hi_t < Ls ? hi_t : Ls;
  };
  // ---- two row tiles: a segment cut between waves of one workgroup is combined on chip
  // (one partial result per workgroup instead of one per wave; with one row tile the
  // partials are small and the extra state cost registers for no gain): a wave whose
  // first segment began in an earlier wave's slice of the same workgroup (its "head
  // piece") parks its rows in LDS slot w - 1 and moves on without waiting; the first wave
  // of the workgroup that holds the segment -- for which the segment runs on past the end
  // of its slice, so this is its last one -- adds the parked rows to its own at the end of
  // its slice and writes the segment (if the workgroup holds all of it) or one partial
  // result for the merge kernel.  Each wave parks at most one piece, so each slot is used
  // once per launch.  The wait for a parked piece is bounded (kSpinLimit polls of ~100
  // cycles): a broken hand-over would end the kernel with wrong rows, not hang it.
  constexpr int ND = D / 16;
  constexpr int kSpinLimit = 1 << 20;
  constexpr int kSlots = kComb ? W - 1 : 1;
  __shared__ float s_dm[kSlots][kComb ? NT * 16 : 1];
  __shared__ float s_dl[kSlots][kComb ? NT * 16 : 1];
  __shared__ f32x4 s_dacc[kSlots][kComb ? NT : 1][kComb ? ND : 1][kComb ? kWave : 1];
  // workgroup's flat range and its waves' ids
  const int wv0 = (int)(wid * W);
  const int wx0 = (int)((int64_t)wv0 * per);
  const int wx1 = total - wx0 > W * per ? wx0 + W * per : total;
  // One row tile: a head piece (the slice's first segment, begun in an earlier slice) is
  // finished while the ring streams on; its rows are parked in LDS and written once the
  // wave has issued its last tile load (or after the loop), since global stores issued
  // mid-stream sit in the in-order memory counter in front of the next tiles' loads
  // (writing it at once cost the Llama-3-8B kernel ~1.4 us); stores behind every load
  // delay none.  (LDS rather than registers: the decode-step kernel has none to spare.)
  __shared__ f32x4 s_hacc[kComb ? 1 : W][kComb ? 1 : ND][kComb ? 1 : kWave];
  __shared__ float s_hml[kComb ? 1 : W][2][kComb ? 1 : 16];
  Seg held_seg;
  held_seg.j = -1;
  auto write_parked = [&]() {  // (write_rows' partial-result form, streamed from LDS)
    const int rl = row16;
    const int r = held_seg.rg * 16 + rl;
    const float lsum = s_hml[w][1][rl];
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int64_t slot = v + held_seg.j;
    if (r < a.rows) {
      float* dst = a.ws_out + (slot * 16 + rl) * D;
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        const f32x4 x = s_hacc[w][t][lane];
        *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * grp) = x * inv;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (grp == 0)
        a.ws_lse[slot * 16 + rl] =
            lsum > 0.f ? (s_hml[w][0][rl] + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
    }
    held_seg.j = -1;
  };
  auto finish = [&](auto at_end) {
    st.totals();
    const bool whole = cur.start >= x0 && cur.end <= x1;
    if constexpr (!kComb) {
      if (!decltype(at_end)::value && !whole) {
#pragma unroll
        for (int t = 0; t < ND; ++t) s_hacc[w][t][lane] = st.acc[0][t];
        if (grp == 0) {
          s_hml[w][0][row16] = st.m[0];
          s_hml[w][1][row16] = st.l[0];
        }
        held_seg = cur;
        return;
      }
      write_rows<KV, D, NT>(a, st, whole ? kDirect : kBalanced, cur.b, cur.g, cur.rg, v + cur.j,
                            a.ws_out_lse, row16, grp);
      return;
    }
    if (!whole && cur.start < x0 && w > 0) {  // park: the segment's first wave takes it
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (grp == 0) {
          s_dm[w - 1][nt * 16 + row16] = st.m[nt];
          s_dl[w - 1][nt * 16 + row16] = st.l[nt];
        }
#pragma unroll
        for (int t = 0; t < ND; ++t) s_dacc[w - 1][nt][t][lane] = st.acc[nt][t];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0)
        __hip_atomic_store(&s_dflag[w - 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return;
    }
    if constexpr (decltype(at_end)::value) {
      // the waves after this one in the workgroup that hold blocks of the segment
      int wl = w;
      if (cur.end > x1) {
        const int last = (int)((unsigned)(cur.end - 1) / (unsigned)per) - wv0;
        wl = last < W - 1 ? last : W - 1;
      }
      for (int sl = w; sl < wl; ++sl) {
#pragma unroll 1
        for (int i = 0; i < kSpinLimit; ++i) {
          if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                  &s_dflag[sl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0)
            break;
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float mp = s_dm[sl][nt * 16 + row16];
          const float M = fmaxf(mp, st.m[nt]);
          const float Mu = M == -INFINITY ? 0.f : M;
          const float fp = __builtin_amdgcn_exp2f(mp - Mu);
          const float fo = __builtin_amdgcn_exp2f(st.m[nt] - Mu);
          st.l[nt] = s_dl[sl][nt * 16 + row16] * fp + st.l[nt] * fo;
          st.m[nt] = M;
#pragma unroll
          for (int t = 0; t < ND; ++t) st.acc[nt][t] = s_dacc[sl][nt][t][lane] * fp + st.acc[nt][t] * fo;
        }
      }
    }
    const bool whole_wg = cur.start >= wx0 && cur.end <= wx1;
    write_rows<KV, D, NT>(a, st, whole_wg ? kDirect : kBalanced, cur.b, cur.g, cur.rg, v + cur.j,
                          a.ws_out_lse, row16, grp);
  };
  auto issue = [&](typename KV::K& kk, typename KV::V& vv, int kn, const Slot& sl) {
    const int x = x0 + kn;
    if (kn < n && x >= iss_end) {
      // first block of a new segment: fetch its query rows ahead of time
      const Seg sg = locate(x);
      iss_end = sg.end;
      if (nxt.j < 0) {
        nxt = sg;
        const int Ls = __builtin_amdgcn_readfirstlane(s_len[sg.b]);
        lim_min_next = load_rows<KV, D, NT, SW>(a, sg.b, sg.g, sg.rg, Ls, rows_hi(sg, Ls), qnext,
                                                lim_next, lo_next, lo_max_next, no_tree, row16,
                                                grp);
        if constexpr (APP) {
          const int64_t nrow = ((int64_t)sg.b * a.num_kv_heads + sg.g) * D * KV::kElem;
          KV::load_new(tok_next, static_cast<const uint8_t*>(a.k_new) + nrow,
                       static_cast<const uint8_t*>(a.v_new) + nrow, row16, grp);
        }
      }
    }
    const int64_t tl = sl.tile >= 0 ? sl.tile : 0;
    KV::load_k(kk, kbase + tl * tile_bytes, lane);
    KV::load_v(vv, vbase + tl * tile_bytes, row16, grp);
  };
  // Issue priority by progress: two waves sharing a SIMD (two workgroups per compute unit)
  // would otherwise be served oldest first, so the younger one streams far behind and ends
  // alone with half the loads in flight.  A wave's user priority drops by one at each
  // quarter of its slice, so whichever wave is behind is issued first.
  int quarter = -1;
  // quarter q of the slice starts at block ceil(q * n / 4)
  const int qt1 = (n + 3) / 4, qt2 = (2 * n + 3) / 4, qt3 = (3 * n + 3) / 4;
  auto set_priority = [&](int k) {
    if constexpr (PA_BAL_PRIO) {
      const int q4 = (k >= qt1 ? 1 : 0) + (k >= qt2 ? 1 : 0) + (k >= qt3 ? 1 : 0);
      if (q4 != quarter) {
        quarter = q4;
        if (q4 == 0) __builtin_amdgcn_s_setprio(3);
        else if (q4 == 1) __builtin_amdgcn_s_setprio(2);
        else if (q4 == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    }
  };
  auto consume = [&](typename KV::K& kk, typename KV::V& vv, int k, const Slot& sl) {
    if (k >= n) return;
    set_priority(k);
    const int x = x0 + k;
    if (x >= cur.end) {
      if (cur.j >= 0) finish(std::false_type{});
      const bool pre = nxt.j >= 0 && x >= nxt.start && x < nxt.end;
      cur = pre ? nxt : locate(x);
      L = __builtin_amdgcn_readfirstlane(s_len[cur.b]);
      const int hi = rows_hi(cur, L);
      if (pre) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          qop[nt] = qnext[nt];
          lim[nt] = lim_next[nt];
          lo_row[nt] = lo_next[nt];
        }
        lim_min = lim_min_next;
        lo_max = lo_max_next;
        if constexpr (APP) tok = tok_next;
        nxt.j = -1;
      } else {
        // (rare: two segments began within the blocks in flight) load the rows now and
        // wait for them here, so that no later wait has to allow for a pending query load
        lim_min = load_rows<KV, D, NT, SW>(a, cur.b, cur.g, cur.rg, L, hi, qop, lim, lo_row,
                                           lo_max, no_tree, row16, grp);
        if constexpr (APP) {
          const int64_t nrow = ((int64_t)cur.b * a.num_kv_heads + cur.g) * D * KV::kElem;
          KV::load_new(tok, static_cast<const uint8_t*>(a.k_new) + nrow,
                       static_cast<const uint8_t*>(a.v_new) + nrow, row16, grp);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
        if (nxt.j >= 0 && nxt.j <= cur.j) nxt.j = -1;
      }
      float vref = 1.f;
      if constexpr (kScaled) {
        if (sl.tile >= 0 && sl.vs > 0.f && sl.vs < 3.0e38f) vref = sl.vs;
      }
      st.reset(vref);
    }
    if (sl.tile < 0) return;
    const int tok0 = (x - cur.start + cur.fb) * kBlockTokens;
    const bool new_tok = APP && tok0 + kBlockTokens >= L;  // the tile holding token L - 1
    const int off = L - 1 - tok0;
    if constexpr (APP) {
      if (new_tok) KV::patch(kk, vv, tok, off, row16, grp);
    }
    st.template update<SW>(qop, lim, lim_min, lo_row, lo_max, no_tree, rows_hi(cur, L), kk, vv,
                           tok0, a.scale_log2 * (kScaled ? sl.ks : 1.f), sl.vs, grp);
    if constexpr (APP) {
      if (new_tok && cur.rg == 0) {  // keep the token for the store at the end
        if (napp == kAppCap) drain();
        KV::stash_new(s_appd[w][napp], tok, row16, grp);
        if (lane == 0) {
          s_appm[w][napp][0] = sl.tile;
          s_appm[w][napp][1] = off;
        }
        ++napp;
      }
    }
  };

  {
    typename KV::K kb[NBUF];
    typename KV::V vb[NBUF];
    Slot sb[NBUF];
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
      sb[s] = slot_at(s);
      issue(kb[s], vb[s], s, sb[s]);
    }
    for (int k = 0; k < n; k += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const int kn = k + s + NBUF - 1;  // block issued now, consumed NBUF - 1 steps later
        const int sn = (s + NBUF - 1) % NBUF;
        if ((kn & (kStage - 1)) == 0 && kn < n) stage(kn);
        sb[sn] = slot_at(kn);
        issue(kb[sn], vb[sn], kn, sb[sn]);
        if (!kComb && kn == n - 1 && held_seg.j >= 0) write_parked();
        consume(kb[s], vb[s], k + s, sb[s]);
      }
    }
  }
  if (cur.j >= 0) finish(std::true_type{});
  if (!kComb && held_seg.j >= 0) {
#pragma unroll
    for (int t = 0; t < ND; ++t) st.acc[0][t] = s_hacc[w][t][lane];
    st.m[0] = s_hml[w][0][row16];
    st.l[0] = s_hml[w][1][row16];
    write_rows<KV, D, NT>(a, st, kBalanced, held_seg.b, held_seg.g, held_seg.rg,
                          v + held_seg.j, a.ws_out_lse, row16, grp);
  }
  if constexpr (APP) drain();
}

template <class KV, int D, int NT, int W, int NBUF>
int launch_one(const AttnArgs& a, void* stream) {
  const int nrg = (a.rows + 16 * NT - 1) / (16 * NT);
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * nrg * a.max_parts;
  const int64_t grid = (units + 7) / 8 * 8;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  const dim3 gr((unsigned)grid), bl(kWave * W);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // several row tiles of a (sequence, KV head) read the same blocks (multi-query rows)
  const bool reuse = nrg > 1;
  if (a.window > 0) {
    if (reuse)
      hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, true, false, 1, true>), gr, bl, 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, true>), gr, bl, 0, st, a);
  } else {
    if (reuse)
      hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, false, false, 1, true>), gr, bl, 0, st, a);
    else
      hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, false>), gr, bl, 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <class KV, int D, int NT, int W, int NBUF, bool APP>
int launch_balanced_one(const AttnArgs& a, void* stream) {
  const int64_t grid = ((int64_t)a.num_workgroups + 7) / 8 * 8;
  if (a.window > 0)
    hipLaunchKernelGGL((paged_attn_balanced_kernel<KV, D, NT, W, NBUF, APP, true>),
                       dim3((unsigned)grid), dim3(kWave * W), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((paged_attn_balanced_kernel<KV, D, NT, W, NBUF, APP, false>),
                       dim3((unsigned)grid), dim3(kWave * W), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <class KV, int D, int NT, int W, int NBUF>
int occupancy_one() {
  int cus = 0, per_cu = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return PA_ERR_LAUNCH;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu,
          reinterpret_cast<const void*>(&paged_attn_balanced_kernel<KV, D, NT, W, NBUF, false, false>),
          kWave * W, 0) != hipSuccess)
    return PA_ERR_LAUNCH;
  // Measured on MI355X (Llama-3-8B decode, shared-prefix and 128K bf16 workloads; int8
  // verify): with one row tile a wave per SIMD (one workgroup per unit) streams fastest
  // (108 / 66 / 326 us against 110 / 73 / 347 us with two per unit); with two row tiles
  // (more compute per byte) two workgroups per unit hide it better (85 against 95 us), and
  // so they do for 8-bit tiles (half the bytes per block and an fp16 decode of each:
  // Llama-3-8B fp8 decode 48.4 against 49.7 us).
  const int want = NT == 1 && !Scaled8<KV>::value ? 1 : 2;
  const int64_t n = (int64_t)cus * (per_cu >= want ? want : (per_cu > 0 ? per_cu : 1));
  return n > 0x7fffffff ? 0x7fffffff : (int)n;
}

// waves per workgroup and register buffers per wave (build-time tunables)
#ifndef PA_WAVES
#define PA_WAVES 4
#endif
#ifndef PA_NBUF_1
#define PA_NBUF_1 2
#endif
#ifndef PA_NBUF_2
#define PA_NBUF_2 2
#endif

// multi-query rows with a candidate mask: two row tiles per wave, PA_TREE_RG such row
// tiles per workgroup (measured on MI355X, candidate-tree verify batch 32 x 64 rows: one
// tile 230 us, two 238 us, four 244 us, once plain loads let L2 serve the re-reads; two
// were faster while the loads bypassed it)
#ifndef PA_TREE_RG
#define PA_TREE_RG 1
#endif
#ifndef PA_MQ_NT
#define PA_MQ_NT 2
#endif
template <class KV, int D, int NBUF>
int launch_tree_one(const AttnArgs& a, void* stream) {
  constexpr int NT = PA_MQ_NT, W = PA_WAVES, RG = PA_TREE_RG;
  const int nrg = (a.rows + 16 * NT * RG - 1) / (16 * NT * RG);
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * nrg;
  const int64_t grid = (units + 7) / 8 * 8;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  if (nrg > 1)
    hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, false, true, RG, true>),
                       dim3((unsigned)grid), dim3(kWave * W), 0, static_cast<hipStream_t>(stream),
                       a);
  else
    hipLaunchKernelGGL((paged_attn_kernel<KV, D, NT, W, NBUF, false, true, RG>),
                       dim3((unsigned)grid), dim3(kWave * W), 0, static_cast<hipStream_t>(stream),
                       a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

enum Op { kLaunch, kLaunchBalanced, kLaunchBalancedAppend, kOccupancy, kLaunchTree };

template <template <int> class KVT, int D>
int dispatch_dim(const AttnArgs& a, Op op, void* stream) {
  constexpr int W = PA_WAVES;
  using KV = KVT<D>;
  constexpr bool kCanAppend = !Scaled8<KV>::value;
  if (op == kLaunchTree) return launch_tree_one<KV, D, PA_NBUF_2>(a, stream);
  if (a.rows <= 16) {
    if (op == kLaunch) return launch_one<KV, D, 1, W, PA_NBUF_1>(a, stream);
    if (op == kLaunchBalanced) return launch_balanced_one<KV, D, 1, W, PA_NBUF_1, false>(a, stream);
    if (op == kLaunchBalancedAppend) {
      if constexpr (kCanAppend) return launch_balanced_one<KV, D, 1, W, PA_NBUF_1, true>(a, stream);
      return PA_ERR_DTYPE;
    }
    return occupancy_one<KV, D, 1, W, PA_NBUF_1>();
  }
  if (op == kLaunch) return launch_one<KV, D, PA_MQ_NT, W, PA_MQ_NT == 1 ? PA_NBUF_1 : PA_NBUF_2>(a, stream);
  if (op == kLaunchBalanced) return launch_balanced_one<KV, D, 2, W, PA_NBUF_2, false>(a, stream);
  if (op == kLaunchBalancedAppend) {
    if constexpr (kCanAppend) return launch_balanced_one<KV, D, 2, W, PA_NBUF_2, true>(a, stream);
    return PA_ERR_DTYPE;
  }
  return occupancy_one<KV, D, 2, W, PA_NBUF_2>();
}

template <template <int> class KVT>
int dispatch_kv(const AttnArgs& a, Op op, void* stream) {
  return a.head_dim == 64 ? dispatch_dim<KVT, 64>(a, op, stream) : dispatch_dim<KVT, 128>(a, op, stream);
}

int dispatch(const AttnArgs& a, int q_dtype, int kv_dtype, Op op, void* stream) {
  if (q_dtype == PA_F32 && kv_dtype == PA_F32) return dispatch_kv<F32Kv>(a, op, stream);
  if (q_dtype == PA_BF16 && kv_dtype == PA_BF16) return dispatch_kv<Bf16Kv>(a, op, stream);
  if (q_dtype == PA_BF16 && kv_dtype == PA_I8) return dispatch_kv<I8Kv>(a, op, stream);
  if (q_dtype == PA_BF16 && kv_dtype == PA_FP8) return dispatch_kv<Fp8Kv>(a, op, stream);
  return PA_ERR_DTYPE;
}

}  // namespace

int launch_attention(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream) {
  return dispatch(a, q_dtype, kv_dtype, kLaunch, stream);
}

int launch_multi_query(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream) {
  return dispatch(a, q_dtype, kv_dtype, a.tree_mask != nullptr ? kLaunchTree : kLaunch, stream);
}

int balanced_row_tile(int32_t rows) { return rows <= 16 ? 16 : 32; }

int balanced_waves() { return PA_WAVES; }

int balanced_workgroups(int q_dtype, int kv_dtype, int head_dim, int32_t rows) {
  AttnArgs a{};
  a.head_dim = head_dim;
  a.rows = rows;
  return dispatch(a, q_dtype, kv_dtype, kOccupancy, nullptr);
}

int launch_balanced(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream) {
  return dispatch(a, q_dtype, kv_dtype, kLaunchBalanced, stream);
}

int launch_balanced_append(const AttnArgs& a, int q_dtype, int kv_dtype, void* stream) {
  return dispatch(a, q_dtype, kv_dtype, kLaunchBalancedAppend, stream);
}

}  // namespace pa

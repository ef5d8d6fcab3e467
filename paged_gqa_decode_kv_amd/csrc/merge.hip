// Log-sum-exp recombination of per-partition attention results (gfx950).
//
// Partition p of a row holds its normalised output o_p and lse_p = log of its softmax
// denominator.  With M = max_p lse_p and w_p = exp(lse_p - M) the full-context result is
// sum_p w_p o_p / sum_p w_p and its lse is M + log sum_p w_p: exact, because exp(lse_p)
// is partition p's share of the full denominator.  One wave per (sequence, query head)
// row.  The partition count of each sequence is derived from seq_lens exactly as the split
// attention kernel derives it.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "pa_common.hpp"
#include "../../include/paged_attn.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(kWave) void lse_merge_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int32_t num_q_heads, int32_t max_blocks,
    int32_t part_tokens, int32_t max_parts, float* __restrict__ out, float* __restrict__ out_lse) {
  // The wave splits into PG groups of D / 4 lanes: each group takes one partition's row per
  // step (four dims a lane) with its lse, U steps in flight, so one round trip covers PG * U
  // partitions.  The first round is issued before the sequence length arrives (partitions
  // past the sequence's count are masked afterwards; every slot below max_parts is inside
  // the caller's arrays), so a row with up to PG * U partitions costs one round trip after
  // the launch instead of one per partition.
  constexpr int LPR = D / 4;
  constexpr int PG = kWave / LPR;
  constexpr int U = 8;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int pg = lane / LPR, dl = lane % LPR;
  const int b = (int)(row / num_q_heads);
  const float* lse_row = part_lse + row * max_parts;
  const float* o = part_out + row * max_parts * D;
  int L = seq_lens[b];
  float M = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  int n = max_parts;  // partitions of this row; known once L has arrived
  for (int q0 = 0; q0 < n; q0 += PG * U) {
    float lp[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = q0 + u * PG + pg;
      lp[u] = -INFINITY;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p < n) {
        lp[u] = lse_row[p];
        v[u] = *reinterpret_cast<const f32x4*>(o + (int64_t)p * D + 4 * dl);
      }
    }
    if (q0 == 0) {
      L = L < 0 ? 0 : (L > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : L);
      const int np = L > 0 ? (L + part_tokens - 1) / part_tokens : 0;
      n = np > max_parts ? max_parts : np;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (q0 + u * PG + pg >= n) lp[u] = -INFINITY;
    // the chunk's maximum over all groups, then the rescaled sums
    float mc = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mc = fmaxf(mc, lp[u]);
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
    if (mc == -INFINITY) continue;
    if (M != -INFINITY && mc != M) {
      const float c = __builtin_amdgcn_exp2f((M - mc) * kLog2e);
      acc *= c;
      wsum *= c;
    }
    M = mc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wq = lp[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lp[u] - M) * kLog2e);
      if (wq != 0.f) acc += wq * v[u];
      wsum += wq;
    }
  }
  // the groups' partial sums (all groups share M)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
    wsum += __shfl_xor(wsum, off);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (pg == 0) *reinterpret_cast<f32x4*>(out + row * D + 4 * dl) = acc * inv;
  if (out_lse != nullptr && lane == 0)
    out_lse[row] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}


// Balanced mode: segment j (KV head g, row group rg, sequence b) occupies flat blocks
// [S_j, S_{j+1}) with S_j = (g * nrg + rg) * T + prefix[b]; attention wave w covered
// [w * per, (w + 1) * per), so the waves that held blocks of segment j are
// w0 = S_j / per .. w1 = (S_{j+1} - 1) / per.  With two row tiles the attention kernel
// combines the pieces of one workgroup (W consecutive waves) on chip, so there is one
// partial per workgroup, at partial id w + j for the first of its waves w in [w0, w1]
// (with one row tile W counts as 1 here: one partial per wave, at w + j).  A segment
// inside one workgroup (one wave) was written out by the attention kernel and is skipped
// here; an empty segment gets zeros.
// This form serves one row tile (up to 16 rows): one wave per query row of the segment's
// row tile, one workgroup per segment (the blockIdx.y split below covers larger tiles,
// which balanced_merge_rows_kernel takes instead).
template <int D>
__global__ __launch_bounds__(1024) void balanced_merge_kernel(AttnArgs a, int row_tile,
                                                              float* __restrict__ out,
                                                              float* __restrict__ out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int nwv = blockDim.x / kWave;
  // (flat block positions fit in int32, as the host checks: 32-bit divisions here)
  const int j = blockIdx.x;
  const int B = a.num_seqs;
  const int nrg = (a.rows + row_tile - 1) / row_tile;
  const int gr = j / B;
  const int b = j - gr * B;
  const int g = gr / nrg;
  const int rg = gr - g * nrg;

  const int T = a.ws_prefix[B];
  const int total = T * a.num_kv_heads * nrg;
  const int per = (int)(((unsigned)total + (unsigned)a.num_workers - 1u) / (unsigned)a.num_workers);
  const int s0 = gr * T + a.ws_prefix[b];
  const int s1 = gr * T + a.ws_prefix[b + 1];
  const int w0 = s1 > s0 ? (int)((unsigned)s0 / (unsigned)per) : 0;
  const int w1 = s1 > s0 ? (int)((unsigned)(s1 - 1) / (unsigned)per) : -1;
  // waves per attention workgroup whose pieces were combined (the two-tile launches use
  // balanced_merge_rows_kernel; kept general here)
  const int W = row_tile > 16 ? a.num_workers / a.num_workgroups : 1;
  const int k0 = w0 / W;                           // first and last workgroup
  const int k1 = s1 > s0 ? w1 / W : -1;            // (none for an empty segment)
  if (s1 > s0 && k0 == k1) return;   // written by the attention kernel

  // Within a row's wave the lanes split into PG groups of D / 4 lanes: each group takes one
  // piece per step, each lane four dims of it; U steps are in flight at once.  The pieces'
  // lse values arrive with their rows, so the maximum is a running one (one round trip for
  // up to PG * U pieces; a further chunk rescales what is summed so far).
  constexpr int LPR = D / 4;
  constexpr int PG = kWave / LPR;
  constexpr int U = 8;   // (16 spills: a 1024-thread workgroup leaves 128 VGPRs a lane)
  const int pg = lane / LPR, dl = lane % LPR;
  const int64_t npc = k1 - k0 + 1;  // pieces (0 for an empty segment)
  // workgroup y of the segment takes rows y * nwv .. of its row tile, one per wave
  for (int rl = blockIdx.y * nwv + wv; rl < row_tile && rl < (int)(blockIdx.y + 1) * nwv;
       rl += nwv) {
    const int r = rg * row_tile + rl;
    if (r >= a.rows) break;
    const int i = r / a.group;
    const int h = g * a.group + r % a.group;
    const int64_t orow = (int64_t)(b * a.num_q_pos + i) * a.num_q_heads + h;
    float M = -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int64_t q0 = 0; q0 < npc; q0 += PG * U) {
      float lp[U];
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t q = q0 + u * PG + pg;
        lp[u] = -INFINITY;
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (q < npc) {  // (no load for the slots past the last piece)
          const int64_t pid = (q == 0 ? w0 : (k0 + q) * W) + j;
          lp[u] = a.ws_lse[pid * row_tile + rl];
          v[u] = *reinterpret_cast<const f32x4*>(a.ws_out + (pid * row_tile + rl) * D + 4 * dl);
        }
      }
      // the chunk's maximum over all PG groups
      float mc = M;
#pragma unroll
      for (int u = 0; u < U; ++u) mc = fmaxf(mc, lp[u]);
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
      if (mc == -INFINITY) continue;
      if (M != -INFINITY && mc != M) {
        const float c = __builtin_amdgcn_exp2f((M - mc) * kLog2e);
        acc *= c;
        wsum *= c;
      }
      M = mc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wq = lp[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lp[u] - M) * kLog2e);
        if (wq != 0.f) acc += wq * v[u];
        wsum += wq;
      }
    }
    // the PG groups' partial sums (all groups share M)
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
      wsum += __shfl_xor(wsum, off);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (pg == 0) *reinterpret_cast<f32x4*>(out + orow * D + 4 * dl) = acc * inv;
    if (out_lse != nullptr && lane == 0)
      out_lse[orow] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
  }
}

// The same merge for two row tiles, whose segments have few pieces (one per attention
// workgroup): each lane group of D / 4 lanes owns RPG rows and loads U / RPG pieces of each
// per round trip, so a wave merges PG * RPG rows and a 24-row segment needs 6 waves rather
// than 24 (the launch of the waves, not their work, set the one-row-per-wave merge's time
// there).  Every lane of a group reads the same lse values, so no lane exchanges anything.
template <int D, int RPG>
__global__ __launch_bounds__(512) void balanced_merge_rows_kernel(AttnArgs a, int row_tile,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int j = blockIdx.x;
  const int B = a.num_seqs;
  const int nrg = (a.rows + row_tile - 1) / row_tile;
  const int gr = j / B;
  const int b = j - gr * B;
  const int g = gr / nrg;
  const int rg = gr - g * nrg;

  const int T = a.ws_prefix[B];
  const int total = T * a.num_kv_heads * nrg;
  const int per = (int)(((unsigned)total + (unsigned)a.num_workers - 1u) / (unsigned)a.num_workers);
  const int s0 = gr * T + a.ws_prefix[b];
  const int s1 = gr * T + a.ws_prefix[b + 1];
  const int w0 = s1 > s0 ? (int)((unsigned)s0 / (unsigned)per) : 0;
  const int w1 = s1 > s0 ? (int)((unsigned)(s1 - 1) / (unsigned)per) : -1;
  // waves per attention workgroup whose pieces were combined (two row tiles), else 1
  const int W = row_tile > 16 ? a.num_workers / a.num_workgroups : 1;
  const int k0 = w0 / W;
  const int k1 = s1 > s0 ? w1 / W : -1;
  if (s1 > s0 && k0 == k1) return;  // written by the attention kernel

  constexpr int LPR = D / 4;
  constexpr int PG = kWave / LPR;
  constexpr int U = 8;
  constexpr int UR = U / RPG;  // pieces of one row per round trip
  const int pg = lane / LPR, dl = lane % LPR;
  const int npc = k1 - k0 + 1;  // pieces (0 for an empty segment)
  int rl[RPG];
  bool live[RPG];
  float M[RPG], wsum[RPG];
  f32x4 acc[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    rl[i] = (wv * PG + pg) * RPG + i;
    live[i] = rl[i] < row_tile && rg * row_tile + rl[i] < a.rows;
    M[i] = -INFINITY;
    wsum[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int q0 = 0; q0 < npc; q0 += UR) {
    float lp[RPG][UR];
    f32x4 v[RPG][UR];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int q = q0 + u;
        lp[i][u] = -INFINITY;
        v[i][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (live[i] && q < npc) {
          const int64_t pid = (int64_t)(q == 0 ? w0 : (k0 + q) * W) + j;
          lp[i][u] = a.ws_lse[pid * row_tile + rl[i]];
          v[i][u] = *reinterpret_cast<const f32x4*>(a.ws_out + (pid * row_tile + rl[i]) * D + 4 * dl);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      float mc = M[i];
#pragma unroll
      for (int u = 0; u < UR; ++u) mc = fmaxf(mc, lp[i][u]);
      if (mc == -INFINITY) continue;
      if (M[i] != -INFINITY && mc != M[i]) {
        const float c = __builtin_amdgcn_exp2f((M[i] - mc) * kLog2e);
        acc[i] *= c;
        wsum[i] *= c;
      }
      M[i] = mc;
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float wq = lp[i][u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lp[i][u] - mc) * kLog2e);
        if (wq != 0.f) acc[i] += wq * v[i][u];
        wsum[i] += wq;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    if (!live[i]) continue;
    const int r = rg * row_tile + rl[i];
    const int qi = r / a.group;
    const int h = g * a.group + r % a.group;
    const int64_t orow = (int64_t)(b * a.num_q_pos + qi) * a.num_q_heads + h;
    const float inv = wsum[i] > 0.f ? 1.f / wsum[i] : 0.f;
    *reinterpret_cast<f32x4*>(out + orow * D + 4 * dl) = acc[i] * inv;
    if (out_lse != nullptr && dl == 0)
      out_lse[orow] = wsum[i] > 0.f ? M[i] + __builtin_amdgcn_logf(wsum[i]) * kLn2 : -INFINITY;
  }
}

}  // namespace

int launch_balanced_merge(const AttnArgs& a, float* out, float* out_lse, void* stream) {
  const int rt = balanced_row_tile(a.rows);
  const int nrg = (a.rows + rt - 1) / rt;
  const int64_t grid = (int64_t)a.num_kv_heads * nrg * a.num_seqs;
  if (grid > 0x7fffffff) return PA_ERR_DIMS;
  const int rows_in_tile = a.rows < rt ? a.rows : rt;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // two row tiles (one piece per attention workgroup): one workgroup per segment, PG * RPG
  // rows per wave (RPG = 2).  (Used for one row tile as well when segments span at most 4
  // slices, it gained nothing on the Llama-3-8B step and cost the fp8 decode step 1.3 us:
  // ~5 pieces a row take two round trips at 4 per trip.)
  if (rt > 16) {
    const int rpw = 2 * (kWave / (a.head_dim / 4));
    const int waves = (rows_in_tile + rpw - 1) / rpw;
    if (a.head_dim == 64)
      hipLaunchKernelGGL((balanced_merge_rows_kernel<64, 2>), dim3((unsigned)grid),
                         dim3(kWave * waves), 0, s, a, rt, out, out_lse);
    else
      hipLaunchKernelGGL((balanced_merge_rows_kernel<128, 2>), dim3((unsigned)grid),
                         dim3(kWave * waves), 0, s, a, rt, out, out_lse);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  // one wave per row of the tile: up to 16 per workgroup, more rows over more workgroups
  const int ysplit = (rows_in_tile + 15) / 16;
  const int waves = (rows_in_tile + ysplit - 1) / ysplit;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(balanced_merge_kernel<64>, dim3((unsigned)grid, ysplit),
                       dim3(kWave * waves), 0, s, a, rt, out, out_lse);
  else
    hipLaunchKernelGGL(balanced_merge_kernel<128>, dim3((unsigned)grid, ysplit),
                       dim3(kWave * waves), 0, s, a, rt, out, out_lse);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_merge(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                 int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_blocks,
                 int32_t part_tokens, int32_t max_parts, float* out, float* out_lse,
                 void* stream) {
  const int64_t rows = (int64_t)num_seqs * num_q_heads;
  if (rows > 0x7fffffff) return PA_ERR_DIMS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3((unsigned)rows), dim3(kWave), 0, s, part_out,
                       part_lse, seq_lens, num_q_heads, max_blocks, part_tokens, max_parts, out,
                       out_lse);
  else
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3((unsigned)rows), dim3(kWave), 0, s, part_out,
                       part_lse, seq_lens, num_q_heads, max_blocks, part_tokens, max_parts, out,
                       out_lse);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa

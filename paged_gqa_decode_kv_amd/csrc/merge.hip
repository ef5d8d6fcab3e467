// Log-sum-exp recombination of per-partition attention results (gfx950).
//
// Partition p of a row holds its normalised output o_p and lse_p = log of its softmax
// denominator.  With M = max_p lse_p and w_p = exp(lse_p - M) the full-context result is
// sum_p w_p o_p / sum_p w_p and its lse is M + log sum_p w_p: exact, because exp(lse_p)
// is partition p's share of the full denominator.  One wave per (sequence, query head)
// row; lane k owns dims k, k + 64, ...  The partition count of each sequence is derived
// from seq_lens exactly as the split attention kernel derives it.
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
  constexpr int PER = D / kWave;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = (int)(row / num_q_heads);
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : L);
  int n = L > 0 ? (L + part_tokens - 1) / part_tokens : 0;
  n = n > max_parts ? max_parts : n;

  const float* lse_row = part_lse + row * max_parts;
  // max over the occupied partitions (lanes stride over p, then a wave reduction)
  float M = -INFINITY;
  for (int p = lane; p < n; p += kWave) M = fmaxf(M, lse_row[p]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    const float* o = part_out + row * max_parts * D;
    for (int p = 0; p < n; ++p) {
      const float lp = lse_row[p];
      if (lp == -INFINITY) continue;
      const float wgt = __builtin_amdgcn_exp2f((lp - M) * kLog2e);
      wsum += wgt;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += wgt * o[(int64_t)p * D + lane + k * kWave];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[row * D + lane + k * kWave] = acc[k] * inv;
  if (out_lse != nullptr && lane == 0)
    out_lse[row] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

}  // namespace

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

// LSE merge of partial attention results over disjoint key sets.
//
// Per row, with M = max_p lse_p and w_p = exp(lse_p - M):
//   O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p
// (the STAGE_D.md page's "O rescale (kt>0)" workaround merge).  Parts whose
// LSE is -inf carry no weight and their O is never read, so a split that saw
// no key may leave its partial output unwritten.  One wavefront per row.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kCombineRowsPerBlock = 4;

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kCombineRowsPerBlock + w;
  if (row >= p.rows) return;
  const int r1 = row / p.n2, r2 = row - r1 * p.n2;
  const float *lp = p.lse_parts + r1 * p.lse_r1 + r2 * p.lse_r2;
  const float *op = p.o_parts + r1 * p.o_r1 + r2 * p.o_r2;

  // max over parts, lanes striding over the parts
  float mx = kNegInf;
  for (int i = lane; i < p.n_parts; i += 64) mx = fmaxf(mx, lp[i * p.lse_part_stride]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));

  uint16_t *out = p.o_out + r1 * p.out_r1 + r2 * p.out_r2;
  float lse_out = kNegInf;
  if (mx == kNegInf) {  // no part saw a key: empty row
    for (int t = lane * 4; t < p.d; t += 256) {
      u32x2 z = {0u, 0u};
      *reinterpret_cast<u32x2 *>(out + t) = z;
    }
  } else {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // d <= 512: two f32x4 per lane
    float wsum = 0.0f;
    for (int i = 0; i < p.n_parts; ++i) {
      const float li = lp[i * p.lse_part_stride];
      if (li == kNegInf) continue;
      const float wgt = __expf(li - mx);
      wsum += wgt;
      const float *oi = op + i * p.o_part_stride;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = lane * 4 + u * 256;
        if (t < p.d) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(oi + t);
          acc[4 * u + 0] += wgt * x[0];
          acc[4 * u + 1] += wgt * x[1];
          acc[4 * u + 2] += wgt * x[2];
          acc[4 * u + 3] += wgt * x[3];
        }
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane * 4 + u * 256;
      if (t < p.d) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[4 * u + 0] * inv, acc[4 * u + 1] * inv);
        v[1] = pack_bf16x2(acc[4 * u + 2] * inv, acc[4 * u + 3] * inv);
        *reinterpret_cast<u32x2 *>(out + t) = v;
      }
    }
    lse_out = mx + __logf(wsum);
  }
  if (p.lse_out != nullptr && lane == 0) p.lse_out[r1 * p.lse_out_r1 + r2 * p.lse_out_r2] = lse_out;
}

inline hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
  const int blocks = (p.rows + kCombineRowsPerBlock - 1) / kCombineRowsPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(64 * kCombineRowsPerBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

// LSE merge of partial attention results over disjoint key sets.
//
// Per row, with M = max_p lse_p and w_p = exp(lse_p - M):
//   O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p
// (the STAGE_D.md page's "O rescale (kt>0)" workaround merge).  Parts whose
// LSE is -inf carry no weight and their O is never read, so a split that saw
// no key may leave its partial output unwritten.
//
// One thread per 8 consecutive output columns of a row: the part loop reads
// one 16-byte (bf16) or 32-byte (fp32) vector per part, four parts at a time.
#pragma once

#include "common.hpp"

namespace attn {

template <typename PT>
__device__ __forceinline__ void load8(const PT *p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float (&v)[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

template <typename PT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int cpr = p.d / 8;  // 8-column chunks per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.rows * cpr) return;
  const int row = (int)(gid / cpr), ch = (int)(gid - (int64_t)row * cpr);
  const int r1 = row / p.n2, r2 = row - r1 * p.n2;
  const float *lp = p.lse_parts + r1 * p.lse_r1 + r2 * p.lse_r2;
  const PT *op = reinterpret_cast<const PT *>(p.o_parts) + r1 * p.o_r1 + r2 * p.o_r2 + ch * 8;

  float mx = kNegInf;
  for (int i = 0; i < p.n_parts; ++i) mx = fmaxf(mx, lp[i * p.lse_part_stride]);

  uint16_t *out = p.o_out + r1 * p.out_r1 + r2 * p.out_r2 + ch * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  if (mx != kNegInf) {
    int i = 0;
    for (; i + 4 <= p.n_parts; i += 4) {
      float li[4], v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) li[u] = lp[(i + u) * p.lse_part_stride];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (li[u] != kNegInf) load8<PT>(op + (int64_t)(i + u) * p.o_part_stride, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (li[u] == kNegInf) continue;
        const float wgt = __expf(li[u] - mx);
        wsum += wgt;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wgt * v[u][e];
      }
    }
    for (; i < p.n_parts; ++i) {
      const float li = lp[i * p.lse_part_stride];
      if (li == kNegInf) continue;
      float v[8];
      load8<PT>(op + (int64_t)i * p.o_part_stride, v);
      const float wgt = __expf(li - mx);
      wsum += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * v[e];
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  u32x4 res;
#pragma unroll
  for (int q = 0; q < 4; ++q) res[q] = pack_bf16x2(acc[2 * q] * inv, acc[2 * q + 1] * inv);
  *reinterpret_cast<u32x4 *>(out) = res;
  if (p.lse_out != nullptr && ch == 0)
    p.lse_out[r1 * p.lse_out_r1 + r2 * p.lse_out_r2] = wsum > 0.0f ? mx + __logf(wsum) : kNegInf;
}

template <typename PT>
inline hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.rows * (p.d / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel<PT>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

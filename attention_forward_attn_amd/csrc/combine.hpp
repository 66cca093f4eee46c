// LSE merge of partial attention results over disjoint key sets.
//
// Per row, with M = max_p lse_p and w_p = exp(lse_p - M):
//   O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p
// (the STAGE_D.md page's "O rescale (kt>0)" workaround merge).  Parts whose
// LSE is -inf carry no weight: their O is loaded but never used, so a split
// that saw no key may leave its partial output unwritten (any bit pattern,
// NaN included).
//
// One thread per 8 consecutive output columns of a row: each part gives it
// one 16-byte (bf16) or 32-byte (fp32) vector.
#pragma once

#include "common.hpp"

namespace attn {

// Raw 8-column vector of one part (fp32 or bf16) and its widening to fp32.
template <typename PT>
struct Vec8;
template <>
struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const f32x4 *>(p);
    b = *reinterpret_cast<const f32x4 *>(p + 4);
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};
template <>
struct Vec8<uint16_t> {
  u32x4 a;
  __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? __uint_as_float(a[e >> 1] & 0xffff0000u) : __uint_as_float(a[e >> 1] << 16);
  }
};

// Merge of one 8-column chunk of one row over n parts: lse_at(i) gives part
// i's LSE and vec_at(i) its 8-column vector (a Vec8); writes 8 bf16 to out
// and, if lse_out is not NULL, the LSE.  Parts are taken PB at a time.  The
// partial vectors of a batch are loaded together with their LSEs (not after
// them: a part's LSE only decides whether its vector is used), so a batch
// costs one memory round trip; the running (max, weight sum, accumulator) is
// rescaled once per batch to the batch's new maximum.
template <typename PT, int PB, typename LseAt, typename VecAt>
__device__ __forceinline__ void merge_parts(int n, LseAt &&lse_at, VecAt &&vec_at, uint16_t *out,
                                            float *lse_out) {
  float mx = kNegInf, wsum = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n; i += PB) {
    float li[PB];
    Vec8<PT> v[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      li[u] = kNegInf;
      if (i + u < n) {
        li[u] = lse_at(i + u);
        v[u] = vec_at(i + u);
      }
    }
    float bm = li[0];
#pragma unroll
    for (int u = 1; u < PB; ++u) bm = fmaxf(bm, li[u]);
    if (bm == kNegInf) continue;
    const float nm = fmaxf(mx, bm);
    const float sc = mx == kNegInf ? 0.0f : __expf(mx - nm);
    wsum *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (li[u] == kNegInf) continue;  // such a part's vector may be unwritten: never use it
      const float wgt = __expf(li[u] - nm);
      wsum += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * v[u].get(e);
    }
    mx = nm;
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  u32x4 res;
#pragma unroll
  for (int q = 0; q < 4; ++q) res[q] = pack_bf16x2(acc[2 * q] * inv, acc[2 * q + 1] * inv);
  *reinterpret_cast<u32x4 *>(out) = res;
  if (lse_out != nullptr) *lse_out = wsum > 0.0f ? mx + __logf(wsum) : kNegInf;
}

// The same with plain loads: LSE at lp[i*ls], vector at op[i*os].
template <typename PT, int PB>
__device__ __forceinline__ void merge_chunk(const float *lp, int64_t ls, const PT *op, int64_t os, int n,
                                            uint16_t *out, float *lse_out) {
  merge_parts<PT, PB>(
      n, [&](int i) { return lp[i * ls]; },
      [&](int i) {
        Vec8<PT> v;
        v.load(op + (int64_t)i * os);
        return v;
      },
      out, lse_out);
}

// bf16 parts come 16 to a batch (every split of an 8192-key sequence at 512
// keys per split in one trip), fp32 parts 8.
template <typename PT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int PB = sizeof(PT) == 2 ? 16 : 8;
  const int cpr = p.d / 8;  // 8-column chunks per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.rows * cpr) return;
  const int row = (int)(gid / cpr), ch = (int)(gid - (int64_t)row * cpr);
  const int r1 = row / p.n2, r2 = row - r1 * p.n2;
  int n = p.n_parts;
  if (p.kv_len != nullptr) {
    const int L = p.kv_len[r1];
    n = min(n, L > 0 ? (L - 1) / p.split + 1 : 1);
  }
  merge_chunk<PT, PB>(p.lse_parts + r1 * p.lse_r1 + r2 * p.lse_r2, p.lse_part_stride,
                      reinterpret_cast<const PT *>(p.o_parts) + r1 * p.o_r1 + r2 * p.o_r2 + ch * 8,
                      p.o_part_stride, n, p.o_out + r1 * p.out_r1 + r2 * p.out_r2 + ch * 8,
                      p.lse_out != nullptr && ch == 0 ? p.lse_out + r1 * p.lse_out_r1 + r2 * p.lse_out_r2
                                                      : nullptr);
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

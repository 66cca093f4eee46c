// Split-KV decode: one workgroup per (key split, kv head, head block, sequence).
//
// A decode step has one query token per sequence, so a single sequence gives
// an MMA only one row -- unless the query heads that share a kv head are
// stacked as the rows.  Here they are: the workgroup's BM rows are BM query
// heads of one kv group (all 128 heads of an MQA model), every K/V tile is
// read once from HBM and used by all of them (the DSV4 status page's
// "head-packed MQA/GQA", row D2, with MQA as kv head stride 0).  Each split
// covers a fixed run of keys; its normalised fp32 partial output and LSE are
// merged afterwards by the combine kernel (the LSE merge of the STAGE_D.md
// page).  With one query row the bottom-right causal mask admits every cached
// key, so only the tail of a split is masked.
#pragma once

#include "tile.hpp"

namespace attn {

template <int D, int NW, int BN, int OCC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_split_kernel(DecodeParams p) {
  using T = Tile<D, NW, BN>;
  constexpr int BM = T::BM;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * T::STAGE_BYTES / 2];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 31, hi = lane >> 5;

  const int split = blockIdx.x;
  const int g = blockIdx.y / p.n_hblk, hb = blockIdx.y - g * p.n_hblk;
  const int bi = blockIdx.z;
  const int L = p.kv_len[bi];
  const int kbeg = split * p.split;
  const int kend = min(kbeg + p.split, L);

  const int hig = hb * BM + w * 32 + lr;  // head inside the kv group
  const bool row_ok = hig < p.ratio;
  const int head = g * p.ratio + min(hig, p.ratio - 1);
  const int64_t part = ((int64_t)bi * p.h_q + head) * p.n_split + split;

  if (kbeg >= kend && split != 0) {  // nothing in this split: zero weight in the merge
    if (row_ok && hi == 0) p.lse_part[part] = kNegInf;
    return;
  }

  const int64_t start = p.kv_start[bi];
  const uint16_t *kbase = p.k + (start + kbeg) * p.k_st + g * p.k_sh;
  const uint16_t *vbase = p.v + (start + kbeg) * p.v_st + g * p.v_sh;
  const int n_keys = max(kend - kbeg, 0);
  const int n_tiles = (n_keys + BN - 1) / BN;
  const bool wave_ok = hb * BM + w * 32 < p.ratio;
  typename T::Lane ln;
  T::init_lane(ln, smem, p.k_st, p.v_st, w, lane);
  if (n_tiles > 0) T::dma(ln, smem, kbase, p.k_st, vbase, p.v_st, 0, n_keys, w);

  u32x4 qreg[T::NKK];
  {
    const uint16_t *qp = p.q + bi * p.q_sb + (int64_t)head * p.q_sh + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < T::NKK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
  }

  float m = kNegInf, l = 0.0f;
  if (p.sinks != nullptr && split == 0) {  // the sink belongs to exactly one part
    m = p.sinks[head] * kLog2e;
    l = hi == 0 ? 1.0f : 0.0f;
  }
  f32x16 o[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) o[db] = f32x16{};

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < n_tiles)
      T::dma(ln, smem + (cur ^ 1) * (T::STAGE_BYTES / 2), kbase, p.k_st, vbase, p.v_st, (t + 1) * BN,
             n_keys, w);
    const int j0 = t * BN;
    const uint32_t stage_off = cur * T::STAGE_BYTES;
    if (wave_ok) {
      f32x16 s[T::NKB];
      T::scores(s, qreg, ln, stage_off);
      if (j0 + BN > n_keys) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (j0 + T::key_of(kb, i, hi) >= n_keys) s[kb][i] = kNegInf;
      }
      u32x4 pk[T::NPV];
      T::softmax_step(s, pk, o, m, l, p.c);
      T::values(o, pk, ln, stage_off);
    }
  }

  const float lt = sum_across_halves(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    float *op = p.o_part + part * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 val = {o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv, o[db][4 * gi + 2] * inv,
                     o[db][4 * gi + 3] * inv};
        *reinterpret_cast<f32x4 *>(op + db * 32 + 8 * gi) = val;
      }
    if (hi == 0) p.lse_part[part] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, int NW, int BN, int OCC>
hipError_t launch_decode_split(const DecodeParams &p, hipStream_t stream) {
  dim3 grid(p.n_split, p.h_kv * p.n_hblk, p.B);
  hipLaunchKernelGGL((decode_split_kernel<D, NW, BN, OCC>), grid, dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

// Split-KV decode: one workgroup per (key split, kv head, head block, sequence).
//
// A decode step has one query token per sequence, so a single sequence gives
// an MMA only one row -- unless the query heads that share a kv head are
// stacked as the rows.  Here they are: the workgroup's 128 rows are 128 query
// heads of one kv group (all the heads of an MQA model), and every K/V tile is
// read once from HBM and used by all of them (the DSV4 status page's
// "head-packed MQA/GQA", row D2, with MQA as kv head stride 0).  Each split
// covers a fixed run of keys; its normalised partial output (bf16) and LSE
// (fp32) are
// merged afterwards by the combine kernel (the LSE merge of the STAGE_D.md
// page).  With one query row the bottom-right causal mask admits every cached
// key, so only the tail of a split is masked.
//
// Decode streams K/V once, so the kernel is built to keep bytes in flight:
// 8 waves = 4 head groups x 2 key groups (each wave takes 32 of the 64 keys of
// every tile, with its own running max/sum/O), and an LDS ring of STAGES tiles
// of which STAGES-1 are being loaded while one is consumed.  Every iteration
// issues exactly one tile's loads (tiles past the end get an empty buffer
// descriptor and load nothing), so the wait count is a constant.  At the end
// the two key groups of each head group are merged in LDS by their running
// maxima, exactly like two disjoint key sets.
#pragma once

#include "tile.hpp"

namespace attn {

// HG head groups of 32 heads x KG key groups of BN/KG keys = HG*KG waves.
template <int D, int HG, int KG, int BN, int STAGES, int OCC>
__global__ __launch_bounds__(HG * KG * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_split_kernel(DecodeParams p) {
  constexpr int NW = HG * KG;
  using TD = Tile<D, NW, BN>;       // DMA geometry: all waves load one BN-key tile
  using TC = Tile<D, NW, BN / KG>;  // MMA view: each wave computes on BN/KG keys of it
  constexpr int BM = 32 * HG;       // query heads per workgroup
  constexpr int NDB = TC::NDB;
  constexpr int MERGE_BYTES = KG > 1 ? HG * (NDB * 4 + 1) * 64 * 16 : 0;
  constexpr int RING_BYTES = STAGES * TD::STAGE_BYTES;
  constexpr int SMEM_BYTES = RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES;
  static_assert(STAGES >= 2 && (KG == 1 || KG == 2) && (BN / KG) % 32 == 0, "decode shape");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_BYTES / 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int hgrp = wave % HG, kgrp = wave / HG;

  const int split = blockIdx.x;
  const int g = blockIdx.y / p.n_hblk, hb = blockIdx.y - g * p.n_hblk;
  const int bi = blockIdx.z;
  const int L = p.kv_len[bi];
  const int kbeg = split * p.split;
  const int kend = min(kbeg + p.split, L);

  const int hig = hb * BM + hgrp * 32 + lr;  // head inside the kv group
  const bool row_ok = hig < p.ratio;
  const int head = g * p.ratio + min(hig, p.ratio - 1);
  const int64_t part = ((int64_t)bi * p.h_q + head) * p.n_split + split;

  if (kbeg >= kend && split != 0) {  // nothing in this split: zero weight in the merge
    if (row_ok && hi == 0 && kgrp == 0) p.lse_part[part] = kNegInf;
    return;
  }

  const int64_t start = p.kv_start[bi];
  const uint16_t *kbase = p.k + (start + kbeg) * p.k_st + g * p.k_sh;
  const uint16_t *vbase = p.v + (start + kbeg) * p.v_st + g * p.v_sh;
  const int n_keys = max(kend - kbeg, 0);
  const int n_tiles = (n_keys + BN - 1) / BN;
  const bool wave_ok = hb * BM + hgrp * 32 < p.ratio;

  typename TD::Lane dl;
  TD::init_dma(dl, p.k_st, p.v_st, wave, lane);
  typename TC::Lane ml;
  const uint32_t base = lds_offset(smem);
  TC::init_mma(ml, base + kgrp * (BN / KG) * D * 2, base + TD::TILE_BYTES + kgrp * (BN / KG) * D * 2, lane);

  // Prologue: tiles 0 .. STAGES-2 in flight.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    TD::dma(dl, smem + s * (TD::STAGE_BYTES / 2), kbase, p.k_st, vbase, p.v_st, s * BN, n_keys, wave);

  u32x4 qreg[TC::NKK];
  {
    const uint16_t *qp = p.q + bi * p.q_sb + (int64_t)head * p.q_sh + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < TC::NKK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
  }

  float m = kNegInf, l = 0.0f;
  if (p.sinks != nullptr && split == 0 && kgrp == 0) {  // the sink belongs to exactly one part
    m = p.sinks[head] * kLog2e;
    l = hi == 0 ? 1.0f : 0.0f;
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};

  for (int t = 0; t < n_tiles; ++t) {
    wait_vmcnt<(STAGES - 2) * 2 * TD::LOADS>();  // this wave's loads of tile t have landed
    __syncthreads();                              // everyone's have; tile t-1's stage is free
    const int nxt = t + STAGES - 1;
    TD::dma(dl, smem + (nxt % STAGES) * (TD::STAGE_BYTES / 2), kbase, p.k_st, vbase, p.v_st, nxt * BN,
            n_keys, wave);
    const uint32_t stage_off = (t % STAGES) * TD::STAGE_BYTES;
    const int j0 = t * BN + kgrp * (BN / KG);  // first key of this wave's part of the tile
    if (wave_ok && j0 < n_keys) {
      f32x16 s[TC::NKB];
      TC::scores(s, qreg, ml, stage_off);
      if (j0 + BN / KG > n_keys) {
#pragma unroll
        for (int kb = 0; kb < TC::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (j0 + TC::key_of(kb, i, hi) >= n_keys) s[kb][i] = kNegInf;
      }
      u32x4 pk[TC::NPV];
      TC::softmax_step(s, pk, o, m, l, p.c);
      TC::values(o, pk, ml, stage_off);
    }
  }

  // Merge the two key groups of each head group: (m, l, O) of key group 1
  // goes through LDS to key group 0, which rescales both to the larger max.
  wait_vmcnt<0>();
  if constexpr (KG > 1) {
  __syncthreads();
  f32x4 *xb = reinterpret_cast<f32x4 *>(smem) + hgrp * (NDB * 4 + 1) * 64;
  if (kgrp == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        xb[(db * 4 + q4) * 64 + lane] = f32x4{o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2],
                                               o[db][4 * q4 + 3]};
    xb[NDB * 4 * 64 + lane] = f32x4{m, l, 0.0f, 0.0f};
  }
  __syncthreads();
  if (kgrp == 1) return;
  {
    const f32x4 ml2 = xb[NDB * 4 * 64 + lane];
    const float mb = ml2[0], lb = ml2[1];
    const float mm = fmaxf(m, mb);
    const float fa = (m == kNegInf) ? 0.0f : fast_exp2(m - mm);
    const float fb = (mb == kNegInf) ? 0.0f : fast_exp2(mb - mm);
    m = mm;
    l = l * fa + lb * fb;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = xb[(db * 4 + q4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][4 * q4 + e] = o[db][4 * q4 + e] * fa + v[e] * fb;
      }
  }
  }

  const float lt = sum_across_halves(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    // normalised partial output, bf16 (its rounding is far below the final
    // bf16 rounding of O after the merge)
    uint16_t *op = p.o_part + part * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 val;
        val[0] = pack_bf16x2(o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv);
        val[1] = pack_bf16x2(o[db][4 * gi + 2] * inv, o[db][4 * gi + 3] * inv);
        *reinterpret_cast<u32x2 *>(op + db * 32 + 8 * gi) = val;
      }
    if (hi == 0) p.lse_part[part] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, int HG, int KG, int BN, int STAGES, int OCC>
hipError_t launch_decode_split(const DecodeParams &p, hipStream_t stream) {
  dim3 grid(p.n_split, p.h_kv * p.n_hblk, p.B);
  hipLaunchKernelGGL((decode_split_kernel<D, HG, KG, BN, STAGES, OCC>), grid, dim3(HG * KG * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

// Split-KV decode: one workgroup per unit (key split, sequence, kv head, head
// block of HG*32 query heads), and the LSE merge of the splits in the same
// launch.
//
// A decode step has one query token per sequence, so a single sequence gives
// an MMA only one row -- unless the query heads that share a kv head are
// stacked as the rows.  Here they are: the workgroup's 128 rows are 128 query
// heads of one kv group (all the heads of an MQA model), and every K/V tile is
// read once from HBM and used by all of them (the DSV4 status page's
// "head-packed MQA/GQA", row D2, with MQA as kv head stride 0).  Each split
// covers a fixed run of keys and writes its normalised partial output (bf16)
// and LSE (fp32); the splits of a row are then merged by the LSE merge of the
// STAGE_D.md page.  With one query row the bottom-right causal mask admits
// every cached key, so only the tail of a split is masked.
//
// Work placement.  Sequence lengths live on the device, so the grid is sized
// for max_kv_len and every workgroup first works out which unit it owns: the
// units that hold keys are numbered split-major (split 0 of every sequence,
// then split 1 of every sequence that reaches it, ...) and workgroup u takes
// unit u; workgroups past the last unit exit at once.  Consecutive workgroups
// are dispatched to consecutive XCDs, so this numbering hands every XCD the
// same number of units, and the same number of full 512-key splits up to one
// per split level -- with lengths spread over a range, numbering units per
// sequence instead leaves some XCDs with twice the bytes of others.  Empty
// splits never launch; the merge reads only the splits a sequence has.
//
// Decode streams K/V once, so the kernel is built to keep bytes in flight:
// an LDS ring of STAGES tiles of which STAGES-1 are being loaded while one is
// consumed.  The loads carry the non-temporal hint (kStreamOnce): lines read
// once take no retention priority in L2 (about 3 % faster at d = 128 and 6 %
// at d = 256).  Every iteration issues exactly one tile's loads (tiles past the
// end get an empty buffer descriptor and load nothing), so the wait count is a
// constant.
//
// Merge in the same launch.  The grid ends with one merge workgroup per
// (sequence, kv head, slice of decode_merge_heads(D) query heads).  Workgroups
// are dispatched in index order, so every unit is resident or done before a
// merge workgroup takes a slot, and a merge workgroup only ever waits for
// units.  A unit publishes its partial rows with device-coherent stores (sc1:
// written through the XCD's L2, which other XCDs do not see), waits until they
// are complete, and then counts itself in the arrival counter of each slice of
// its head block (a device-scope atomic).  The merge workgroup of a slice
// waits until its counter has counted every split of the sequence, resets it
// to zero for the next call, reads the partials with device-coherent loads and
// writes O and the LSE.  No cache-wide write-back or invalidate is involved.
// The counters sit 64 bytes apart when the workspace header has room: polls
// of many waiting workgroups on shared lines slowed the whole launch by 8 %
// (they queue at the memory channel that holds the line).
// The wait is bounded (kMergeSpin sleeps), so the launch always ends, even
// over counters that were not zero when it started.
#pragma once

#include "fp8.hpp"
#include "tile.hpp"

namespace attn {

// Splits of sequence b that form a unit: one per started chunk of keys, and
// split 0 even for an empty sequence (it carries the sink and the -inf LSE).
// Lengths beyond max_kv_len are clamped to the splits the grid was sized for.
__device__ __forceinline__ int decode_splits_len(int L, int split, int n_split) {
  const int n = L > 0 ? (L - 1) / split + 1 : 1;
  return min(n, n_split);
}
__device__ __forceinline__ int decode_splits_of(const int32_t *kv_len, int split, int n_split, int b) {
  return decode_splits_len(kv_len[b], split, n_split);
}

// Unit u: (split, sequence bi, kv head g, head block hb).  The (split,
// sequence, kv head) triples that hold keys are numbered split-major (q); the
// head blocks of one triple go to the same XCD (u % 8), one after another in
// dispatch order, so the K/V they share is fetched into one L2 once:
//   u = ((q / 8) * n_hblk + hb) * 8 + q % 8.
// Returns false past the last unit.  Every lane of the wave gets the same
// answer.  The scan walks the split levels with one ballot per level and per
// 64 sequences; it stops at u's level, so it is short for the early (full)
// units and at most n_split levels long.  len0 is kv_len[lane] (lanes below
// B), loaded by the caller.
__device__ bool decode_unit(const DecodeParams &p, int u, int lane, int len0, int &split, int &bi, int &g,
                            int &hb) {
  const int r8 = u >> 3;
  hb = r8 % p.n_hblk;
  const int q = (r8 / p.n_hblk) * 8 + (u & 7);
  const int nb0 = lane < p.B ? decode_splits_len(len0, p.split, p.n_split) : 0;
  auto count_above = [&](int s) {  // sequences with more than s splits
    int c = __popcll(__ballot(nb0 > s));
    for (int b0 = 64; b0 < p.B; b0 += 64) {
      const bool has = b0 + lane < p.B && decode_splits_of(p.kv_len, p.split, p.n_split, b0 + lane) > s;
      c += __popcll(__ballot(has));
    }
    return c;
  };
  int r = q;  // rank of the unit within its split level
  int s = 0;
  for (;; ++s) {
    if (s >= p.n_split) return false;
    const int c = count_above(s) * p.h_kv;
    if (r < c) break;
    r -= c;
  }
  split = s;
  g = r % p.h_kv;
  r /= p.h_kv;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const bool has = b < p.B && (b0 == 0 ? nb0 : decode_splits_of(p.kv_len, p.split, p.n_split, b)) > s;
    const uint64_t m = __ballot(has);
    const int cnt = __popcll(m);
    if (r < cnt) {
      const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      bi = b0 + __builtin_ctzll(__ballot(has && pre == r));
      return true;
    }
    r -= cnt;
  }
  return false;  // not reached: r is below the count of level s
}

// Sleeps a merge workgroup waits at most for its splits (s_sleep 2 is about
// 128 clocks: tens of milliseconds in all, far beyond any unit's run time).
constexpr int kMergeSpin = 1 << 20;

// Merge workgroup m: the splits of (sequence b, kv head g, heads
// [mb*MH, mb*MH + MH) of the group), one thread per 8 output columns of a head.
template <int D>
__device__ void decode_merge(const DecodeParams &p, int m) {
  constexpr int MH = decode_merge_heads(D);
  constexpr int CPR = D / 8;  // 8-column chunks per row
  static_assert(MH * CPR == 256, "one chunk per thread");
  const int per_b = p.h_kv * p.n_mblk;
  const int b = m / per_b;
  const int g = (m - b * per_b) / p.n_mblk;
  const int mb = m - b * per_b - g * p.n_mblk;
  const int n = decode_splits_of(p.kv_len, p.split, p.n_split, b);
  if (threadIdx.x == 0) {
    uint32_t *cnt = p.arrive + (int64_t)m * p.arrive_stride;
    int it = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)n && ++it < kMergeSpin)
      __builtin_amdgcn_s_sleep(2);
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int h0 = mb * MH;  // first head of the slice inside the kv group
  const int nh = min(MH, p.ratio - h0);
  const int r = threadIdx.x / CPR, ch = threadIdx.x % CPR;
  if (r >= nh) return;
  const int64_t row0 = (int64_t)b * p.h_q + g * p.ratio + h0;  // the slice's first head
  // Partial rows are split-major per sequence: split i of head h at row
  // (b * n_split + i) * h_q + h, so split i of this slice sits i * h_q rows on.
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.o_part + ((int64_t)b * p.n_split * p.h_q + g * p.ratio + h0) * D,
                (uint32_t)(((int64_t)(n - 1) * p.h_q + nh) * D * 2));
  const uint32_t off = (uint32_t)(r * D * 2 + ch * 16);
  const uint32_t split_bytes = (uint32_t)(p.h_q * D * 2);
  const float *lp = p.lse_part + (row0 + r) * p.n_split;
  const int head = g * p.ratio + h0 + r;
  merge_parts<uint16_t, 16>(
      n, [&](int i) { return __hip_atomic_load(lp + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
      [&](int i) {
        Vec8<uint16_t> v;
        v.a = __builtin_amdgcn_raw_buffer_load_b128(rs, off + (uint32_t)i * split_bytes, 0, kDeviceCoherent);
        return v;
      },
      p.o_out + b * p.o_sb + (int64_t)head * p.o_sh + ch * 8,
      p.lse_out != nullptr && ch == 0 ? p.lse_out + b * p.lse_sb + head : nullptr);
}

// HG head groups of 32 heads = HG waves.
// PAGED: K/V are read through the block table (one descriptor per DMA load,
// see Tile::dma1_paged) instead of from a per-sequence contiguous range.
// FP8: K/V are E4M3 codes with a per-kv-head scale (see fp8.hpp); with PAGED
// as well, the codes are read through the block table.
template <int D, int HG, int BN, int STAGES, int OCC, bool PAGED = false, bool FP8 = false>
__global__ __launch_bounds__(HG * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_split_kernel(DecodeParams p) {
  constexpr int NW = HG;
  using TD = Tile<D, NW, BN>;  // DMA geometry: all waves load one BN-key tile
  using TC = TD;               // MMA view: each wave computes on the whole tile for its heads
  using F8 = Fp8Tile<FP8 ? D : 128, NW, FP8 ? BN : 32>;
  constexpr int BM = 32 * HG;  // query heads per workgroup
  constexpr int NDB = TC::NDB;
  constexpr int RING_BYTES = STAGES * (FP8 ? F8::STAGE_BYTES : TD::STAGE_BYTES);
  constexpr int STORE_BYTES = BM * D * 2;  // partial tile staged for the whole-row stores
  constexpr int SMEM_BYTES = RING_BYTES > STORE_BYTES ? RING_BYTES : STORE_BYTES;
  static_assert(STAGES >= 2 && BN % 32 == 0, "decode shape");
  static_assert(HG * 64 == 256 && BM % decode_merge_heads(D) == 0, "merge slices inside one head block");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_BYTES / 2];

  if ((int)blockIdx.x >= p.unit_grid) {
    decode_merge<D>(p, (int)blockIdx.x - p.unit_grid);
    return;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int hgrp = wave;

  // Lengths and starts of the first 64 sequences are loaded once, side by
  // side, so the unit scan and this unit's key range wait for one load.
  const int len0 = lane < p.B ? p.kv_len[lane] : 0;
  const int64_t start0 = !PAGED && lane < p.B ? p.kv_start[lane] : 0;
  int split_, bi_, g_, hb_;
  if (!decode_unit(p, blockIdx.x, lane, len0, split_, bi_, g_, hb_)) return;
  const int split = __builtin_amdgcn_readfirstlane(split_);
  const int bi = __builtin_amdgcn_readfirstlane(bi_);
  const int g = __builtin_amdgcn_readfirstlane(g_);
  const int hb = __builtin_amdgcn_readfirstlane(hb_);
  const int L = bi < 64 ? __builtin_amdgcn_readlane(len0, bi) : p.kv_len[bi];
  const int kbeg = split * p.split;
  const int kend = min(kbeg + p.split, L);

  const int hig = hb * BM + hgrp * 32 + lr;  // head inside the kv group
  const bool row_ok = hig < p.ratio;
  const int head = g * p.ratio + min(hig, p.ratio - 1);
  const int64_t part = ((int64_t)bi * p.h_q + head) * p.n_split + split;

  const int64_t start =
      PAGED ? 0
      : bi < 64 ? (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(start0 >> 32), bi) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)start0, bi))
                : p.kv_start[bi];
  // Dense: the split's first key.  Paged: the kv head's base; the pages of
  // this split (at most 64) are read once into lane-wise registers.
  const uint16_t *kbase = p.k + (PAGED ? 0 : (start + kbeg) * p.k_st) + g * p.k_sh;
  const uint16_t *vbase = p.v + (PAGED ? 0 : (start + kbeg) * p.v_st) + g * p.v_sh;
  // FP8: the cache is addressed in bytes (strides count bytes).
  const uint8_t *kbase8 = reinterpret_cast<const uint8_t *>(p.k) + (PAGED ? 0 : (start + kbeg) * p.k_st) + g * p.k_sh;
  const uint8_t *vbase8 = reinterpret_cast<const uint8_t *>(p.v) + (PAGED ? 0 : (start + kbeg) * p.v_st) + g * p.v_sh;
  const int n_keys = max(kend - kbeg, 0);
  int pg = 0;
  if constexpr (PAGED) {
    const int n_pg = (n_keys + (1 << p.page_shift) - 1) >> p.page_shift;
    if (lane < n_pg) pg = p.block_table[(int64_t)bi * p.bt_stride + (kbeg >> p.page_shift) + lane];
  }
  const int n_tiles = (n_keys + BN - 1) / BN;
  const bool wave_ok = hb * BM + hgrp * 32 < p.ratio;

  typename TD::Lane dl;
  typename F8::Lane fl;
  if constexpr (PAGED) TD::init_dma_paged(dl, p.k_st, p.v_st, wave, lane);
  else TD::init_dma(dl, p.k_st, p.v_st, wave, lane);
  auto load_tile = [&](uint16_t *stage, int t) {
    uint8_t *stage8 = reinterpret_cast<uint8_t *>(stage);
    if constexpr (FP8 && PAGED)
      F8::template dma_paged<kStreamOnce>(fl, stage8, kbase8, p.k_st, p.k_ps, vbase8, p.v_st, p.v_ps, pg,
                                          p.page_shift, p.n_pages, t * BN, n_keys, wave);
    else if constexpr (FP8)
      F8::template dma<kStreamOnce>(fl, stage8, kbase8, p.k_st, vbase8, p.v_st, t * BN, n_keys, wave);
    else if constexpr (PAGED)
      TD::template dma_paged<kStreamOnce>(dl, stage, kbase, p.k_st, p.k_ps, vbase, p.v_st, p.v_ps, pg,
                                          p.page_shift, p.n_pages, t * BN, n_keys, wave);
    else
      TD::template dma<kStreamOnce>(dl, stage, kbase, p.k_st, vbase, p.v_st, t * BN, n_keys, wave);
  };
  typename TC::Lane ml;
  const uint32_t base = lds_offset(smem);
  if constexpr (FP8) {
    F8::init(fl, p.k_st, p.v_st, wave, lane, base, base + F8::TILE_BYTES);
    if constexpr (PAGED) F8::init_dma_paged(fl, p.k_st, p.v_st, wave, lane);
  } else {
    TC::init_mma(ml, base, base + TD::TILE_BYTES, lane);
  }

  constexpr int STG = FP8 ? F8::STAGE_BYTES : TD::STAGE_BYTES;  // bytes per ring stage
  constexpr int NLD = FP8 ? F8::LOADS : TD::LOADS;              // loads per wave per K or V tile
  // Prologue: tiles 0 .. STAGES-2 in flight.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) load_tile(smem + s * (STG / 2), s);

  u32x4 qreg[TC::NKK];
  {
    const uint16_t *qp = p.q + bi * p.q_sb + (int64_t)head * p.q_sh + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < TC::NKK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
  }

  float m = kNegInf, l = 0.0f;
  if (p.sinks != nullptr && split == 0) {  // the sink belongs to exactly one part
    m = p.sinks[head] * kLog2e;
    l = hi == 0 ? 1.0f : 0.0f;
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  // FP8: the K scale multiplies every logit, so it joins the exp2 factor.
  const float c = FP8 ? p.c * p.k_scale[g] : p.c;

  for (int t = 0; t < n_tiles; ++t) {
    wait_vmcnt<(STAGES - 2) * 2 * NLD>();  // this wave's loads of tile t have landed
    barrier_nofence();                      // everyone's have; tile t-1's stage is free
    const int nxt = t + STAGES - 1;
    load_tile(smem + (nxt % STAGES) * (STG / 2), nxt);
    const uint32_t stage_off = (t % STAGES) * STG;
    const int j0 = t * BN;  // first key of the tile
    if (wave_ok) {
      f32x16 s[TC::NKB];
      if constexpr (FP8) F8::scores(s, qreg, fl, stage_off);
      else TC::scores(s, qreg, ml, stage_off);
      if (j0 + BN > n_keys) {
#pragma unroll
        for (int kb = 0; kb < TC::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (j0 + TC::key_of(kb, i, hi) >= n_keys) s[kb][i] = kNegInf;
      }
      u32x4 pk[TC::NPV];
      TC::softmax_step(s, pk, o, m, l, c);
      if constexpr (FP8) F8::values(o, pk, fl, stage_off);
      else TC::values(o, pk, ml, stage_off);
    }
  }
  wait_vmcnt<0>();

  const float lt = sum_across_halves(l);
  // FP8: the V scale multiplies every output column.
  const float inv = lt > 0.0f ? (FP8 ? p.v_scale[g] : 1.0f) / lt : 0.0f;
  if (row_ok && hi == 0)
    __hip_atomic_store(p.lse_part + part, lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  // Normalised partial output, bf16 (its rounding is far below the final bf16
  // rounding of O after the merge).  A lane holds pieces of one head's row,
  // so a store straight from the accumulators would touch 32 rows 8 bytes at
  // a time; the tile goes through the (now idle) K/V ring instead, with 16-byte
  // chunks XOR-swizzled by row, and every store then writes whole rows.
  constexpr int NC = D / 8;              // 16-byte chunks per row
  constexpr int SW = NC < 16 ? NC : 16;  // swizzle span
  constexpr int RPI = 64 / NC;           // rows per store instruction
  static_assert(STORE_BYTES <= SMEM_BYTES, "partial tile must fit in LDS");
  __syncthreads();  // every wave is done with the last stage
  char *xw = reinterpret_cast<char *>(smem) + hgrp * 32 * D * 2;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      u32x2 val;
      val[0] = pack_bf16x2(o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv);
      val[1] = pack_bf16x2(o[db][4 * gi + 2] * inv, o[db][4 * gi + 3] * inv);
      const int chunk = db * 4 + gi;
      *reinterpret_cast<u32x2 *>(xw + lr * D * 2 + (chunk ^ (lr % SW)) * 16 + 8 * hi) = val;
    }
  __syncthreads();
  // The head block's partial rows of this split, device-coherent and
  // contiguous (split-major rows, (bi * n_split + split) * h_q + head): the
  // unit writes one run of nh * D * 2 bytes.
  const int nh = min(BM, p.ratio - hb * BM);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.o_part + (((int64_t)bi * p.n_split + split) * p.h_q + g * p.ratio + hb * BM) * D,
                (uint32_t)(nh * D * 2));
  const int cc = lane % NC;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / NC;
    const u32x4 val = *reinterpret_cast<const u32x4 *>(xw + r * D * 2 + (cc ^ (r % SW)) * 16);
    const int hr = hgrp * 32 + r;  // head inside the head block
    if (hr < nh)
      __builtin_amdgcn_raw_buffer_store_b128(val, rs, (uint32_t)(hr * D * 2 + cc * 16), 0, kDeviceCoherent);
  }
  // Arrival: once every wave's partial stores are complete, count this split
  // in the counter of each merge slice of the head block.
  if (p.arrive == nullptr) return;  // merged by a second kernel
  wait_vmcnt<0>();
  __syncthreads();
  if (wave == 0) {
    constexpr int SPB = BM / decode_merge_heads(D);  // merge slices per head block
    const int mb0 = hb * SPB;
    if (lane < SPB && mb0 + lane < p.n_mblk)
      __hip_atomic_fetch_add(p.arrive + (((int64_t)bi * p.h_kv + g) * p.n_mblk + mb0 + lane) * p.arrive_stride, 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Grid: the units (decode_grid_size), then the merge workgroups.
template <int D, int HG, int BN, int STAGES, int OCC, bool PAGED = false, bool FP8 = false>
hipError_t launch_decode_split(const DecodeParams &p, hipStream_t stream) {
  const int64_t merges = (int64_t)p.B * p.h_kv * p.n_mblk;
  dim3 grid((unsigned)(p.unit_grid + merges));
  hipLaunchKernelGGL((decode_split_kernel<D, HG, BN, STAGES, OCC, PAGED, FP8>), grid, dim3(HG * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

// FP8 (E4M3) K/V tiles for the split-KV decode at head dim 128.
//
// The cache holds 8-bit codes; a tile is BN keys x D bytes in LDS, rows of D
// bytes whose 16-byte chunks are XOR-swizzled by row (chunk ^ ((r ^ r>>2) & 7),
// which keeps both operand read patterns below at two LDS passes per
// instruction, the minimum for 512 bytes).  Operands are widened to bf16 in
// registers after the LDS read (v_cvt_scalef32_pk_bf16_fp8 with scale 1;
// every E4M3 value is exactly a bf16 value) and the MMAs are the bf16 ones of
// the tile engine, so only the K/V byte traffic changes.  The per-kv-head
// scales are applied outside the MMAs: k_scale folds into the exp2 argument
// factor, v_scale into the final 1/l.
#pragma once

#include "tile.hpp"

namespace attn {

template <int OFF>
__device__ __forceinline__ u32x2 ds_read_b64(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Transposed byte read: inside each 16-lane group, lanes 2e and 2e+1 point at
// the two 8-byte halves of a 16-byte row e (e = 0..7) and lane j receives
// byte j of every row, row e in byte e (measured on the box with an
// in-bounds probe).
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr8(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Eight E4M3 codes (byte e of v = element e) to eight bf16, element order kept.
__device__ __forceinline__ u32x4 widen_fp8x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true));
  return r;
}

template <int D, int NW, int BN>
struct Fp8Tile {
  static_assert(D == 128 && BN == 32, "FP8 tiles: head dim 128, 32-key tiles");
  static constexpr int CH = D / 16;  // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K + V
  static constexpr int LOADS = TILE_BYTES / 1024 / NW;  // 1-KiB DMA loads per wave per tile
  static_assert(LOADS * 1024 * NW == TILE_BYTES, "tile must split into whole 1-KiB wave loads");
  static constexpr int NKB = BN / 32, NDB = D / 32, NKK = D / 16, NPV = BN / 16;
  __device__ static __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & 7; }

  struct Lane {
    uint32_t kg[LOADS], vg[LOADS];  // global byte offsets of this lane's DMA chunks (tile-relative)
    uint32_t kl[NKK];               // LDS address of the K operand of k-step kk
    uint32_t vl[NDB][2];            // LDS address of the V^T operand of block db, 16-key step parity
  };

  // kbase/vbase: LDS byte addresses of the K and V tiles of stage 0.
  __device__ static __forceinline__ void init(Lane &ln, int64_t k_rs, int64_t v_rs, int w, int lane,
                                              uint32_t kbase, uint32_t vbase) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int pch = (u * NW + w) * 64 + lane;  // physical chunk this lane writes
      const int r = pch / CH, c = (pch % CH) ^ swz(r);
      ln.kg[u] = (uint32_t)(r * k_rs) + (uint32_t)(c * 16);
      ln.vg[u] = (uint32_t)(r * v_rs) + (uint32_t)(c * 16);
    }
    // K: lane (key lr, half hi) reads head-dim bytes 16kk + 8hi .. +7 of key lr.
    const int lr = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) ln.kl[kk] = kbase + lr * D + ((kk ^ swz(lr)) * 16) + 8 * hi;
    // V: in 16-lane group g, lane 2e+h points at half h of the 16 bytes of
    // head-dim columns 32db + 16(g&1) .. +15 of the key that the P operand
    // holds in k slot 8(g>>1) + e: 16T + 8(e>>2) + 4(g>>1) + (e&3).
    const int g = lane >> 4, i = lane & 15, e = i >> 1, h = i & 1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key = 16 * p + 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        ln.vl[db][p] = vbase + key * D + (((2 * db + (g & 1)) ^ swz(key)) * 16) + 8 * h;
    }
  }

  // This wave's DMA share of the tile of keys [j0, j0 + BN) into `stage`
  // (K tile then V tile); rows at or past nkeys read as zero.
  __device__ static __forceinline__ void dma(const Lane &ln, uint8_t *stage, const uint8_t *kbase, int64_t k_rs,
                                             const uint8_t *vbase, int64_t v_rs, int j0, int nkeys, int w) {
    const int rows = min(nkeys - j0, BN);
    const uint32_t kb = rows > 0 ? (uint32_t)((rows - 1) * k_rs + D) : 0u;
    const uint32_t vb = rows > 0 ? (uint32_t)((rows - 1) * v_rs + D) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(rows > 0 ? kbase + j0 * k_rs : kbase, kb);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(rows > 0 ? vbase + j0 * v_rs : vbase, vb);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(stage + (u * NW + w) * 1024), 16, ln.kg[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(stage + TILE_BYTES + (u * NW + w) * 1024), 16,
                                               ln.vg[u], 0, 0, 0);
  }

  // S^T = K . Q^T for the staged tile (all reads issued, then consumed in order).
  __device__ static __forceinline__ void scores(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK], const Lane &ln,
                                                uint32_t stage_off) {
    u32x2 a[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) a[kk] = ds_read_b64<0>(ln.kl[kk] + stage_off);
    s[0] = f32x16{};
    score_step<0>(s, qreg, a);
  }
  template <int KK>
  __device__ static __forceinline__ void score_step(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK], u32x2 (&a)[NKK]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(NKK - 1 - KK));
    asm volatile("" : "+v"(a[KK]));
    s[0] = mfma32(widen_fp8x8(a[KK]), qreg[KK], s[0]);
    if constexpr (KK + 1 < NKK) score_step<KK + 1>(s, qreg, a);
  }

  // O^T += V^T . P^T for the staged tile.
  __device__ static __forceinline__ void values(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], const Lane &ln,
                                                uint32_t stage_off) {
    u32x2 v[NPV * NDB];
#pragma unroll
    for (int t = 0; t < NPV; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        v[t * NDB + db] = ds_read_tr8<0>(ln.vl[db][t & 1] + stage_off + (t >> 1) * 32 * D);
    value_step<0>(o, pk, v);
  }
  template <int U>
  __device__ static __forceinline__ void value_step(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                    u32x2 (&v)[NPV * NDB]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(NPV * NDB - 1 - U));
    asm volatile("" : "+v"(v[U]));
    o[U % NDB] = mfma32(widen_fp8x8(v[U]), pk[U / NDB], o[U % NDB]);
    if constexpr (U + 1 < NPV * NDB) value_step<U + 1>(o, pk, v);
  }
};

}  // namespace attn

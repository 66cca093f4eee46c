// FP8 (E4M3) K/V tiles for the split-KV decode at head dims 128 and 256.
//
// The cache holds 8-bit codes; a tile is BN keys x D bytes in LDS, rows of D
// bytes whose 16-byte chunks are XOR-swizzled by row (chunk ^ ((r ^ r>>2) &
// (D/16 - 1)), which keeps both operand read patterns below at two LDS passes
// per instruction, the minimum for 512 bytes).  Operands are widened to bf16 in
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
  static_assert((D == 128 || D == 256) && BN == 32, "FP8 tiles: head dim 128 or 256, 32-key tiles");
  static constexpr int CH = D / 16;  // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K + V
  static constexpr int LOADS = TILE_BYTES / 1024 / NW;  // 1-KiB DMA loads per wave per tile
  static_assert(LOADS * 1024 * NW == TILE_BYTES, "tile must split into whole 1-KiB wave loads");
  static constexpr int NKB = BN / 32, NDB = D / 32, NKK = D / 16, NPV = BN / 16;
  static constexpr int WIN = 8;  // LDS operand reads in flight
  // Chunk swizzle of row r: both read patterns below then take two LDS passes
  // per instruction, the minimum for 512 bytes (a CPU count of bank use over
  // 64 banks of 4 bytes; at D = 256 a 3-bit swizzle would take four).
  __device__ static __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & (CH - 1); }

  // Operand addresses are formed per read from a row base and the row's
  // swizzle (the chunk index kk ^ swizzle has no per-lane constant stride).
  struct Lane {
    uint32_t kg[LOADS], vg[LOADS];  // global byte offsets of this lane's DMA chunks (tile-relative)
    uint32_t krow;                  // LDS address of this lane's K row (half hi), chunk 0
    uint32_t ksw;                   // its swizzle
    uint32_t vrow[2], vsw[2];       // V^T operand: key row address and swizzle per 16-key step parity
    uint32_t vcol;                  // 16-byte column group (g & 1) of this lane
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
    ln.krow = kbase + lr * D + 8 * hi;
    ln.ksw = (uint32_t)swz(lr);
    // V: in 16-lane group g, lane 2e+h points at half h of the 16 bytes of
    // head-dim columns 32db + 16(g&1) .. +15 of the key that the P operand
    // holds in k slot 8(g>>1) + e: 16T + 8(e>>2) + 4(g>>1) + (e&3).
    const int g = lane >> 4, i = lane & 15, e = i >> 1, h = i & 1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key = 16 * p + 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
      ln.vrow[p] = vbase + key * D + 8 * h;
      ln.vsw[p] = (uint32_t)swz(key);
    }
    ln.vcol = (uint32_t)(g & 1);
  }
  __device__ static __forceinline__ uint32_t kaddr(const Lane &ln, int kk, uint32_t stage_off) {
    return ln.krow + ((((uint32_t)kk ^ ln.ksw)) << 4) + stage_off;
  }
  __device__ static __forceinline__ uint32_t vaddr(const Lane &ln, int db, int t, uint32_t stage_off) {
    return ln.vrow[t & 1] + ((((uint32_t)(2 * db) + ln.vcol) ^ ln.vsw[t & 1]) << 4) + stage_off;
  }

  // This wave's DMA share of the tile of keys [j0, j0 + BN) into `stage`
  // (K tile then V tile); rows at or past nkeys read as zero.  CP is the
  // loads' cache-policy operand.
  template <int CP = 0>
  __device__ static __forceinline__ void dma(const Lane &ln, uint8_t *stage, const uint8_t *kbase, int64_t k_rs,
                                             const uint8_t *vbase, int64_t v_rs, int j0, int nkeys, int w) {
    const int rows = min(nkeys - j0, BN);
    const uint32_t kb = rows > 0 ? (uint32_t)((rows - 1) * k_rs + D) : 0u;
    const uint32_t vb = rows > 0 ? (uint32_t)((rows - 1) * v_rs + D) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(rows > 0 ? kbase + j0 * k_rs : kbase, kb);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(rows > 0 ? vbase + j0 * v_rs : vbase, vb);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(stage + (u * NW + w) * 1024), 16, ln.kg[u], 0, 0, CP);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(stage + TILE_BYTES + (u * NW + w) * 1024), 16,
                                               ln.vg[u], 0, 0, CP);
  }

  // Paged caches: a 1-KiB load holds RPL whole rows, which always sit in one
  // page (pages hold at least 16 rows), so each load gets its own descriptor
  // and the lane offsets count from the load's first row.
  static constexpr int RPL = 1024 / D;  // rows per load
  __device__ static __forceinline__ void init_dma_paged(Lane &ln, int64_t k_rs, int64_t v_rs, int w, int lane) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int pch = (u * NW + w) * 64 + lane;
      const int r = pch / CH, rl = lane / CH;  // row in the tile, row in the load
      const int c = (pch % CH) ^ swz(r);
      ln.kg[u] = (uint32_t)(rl * k_rs) + (uint32_t)(c * 16);
      ln.vg[u] = (uint32_t)(rl * v_rs) + (uint32_t)(c * 16);
    }
  }
  // This wave's loads of the tile whose first key is jt (keys counted from
  // the start of a run of pages): key j of the run is row j % 2^shift of page
  // readlane(pg, j >> shift), at head + page * page_rs + row * rs (bytes).
  // Rows at or past nkeys, and pages outside [0, n_pages), read as zero
  // without touching memory.
  template <int CP = 0>
  __device__ static __forceinline__ void dma_paged(const Lane &ln, uint8_t *stage, const uint8_t *khead,
                                                   int64_t k_rs, int64_t k_page_rs, const uint8_t *vhead,
                                                   int64_t v_rs, int64_t v_page_rs, int pg, int shift, int n_pages,
                                                   int jt, int nkeys, int w) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = jt + (u * NW + w) * RPL;
      const int nv = min(nkeys - key, RPL);
      const int page = __builtin_amdgcn_readlane(pg, min(key >> shift, 63));
      const bool ok = nv > 0 && (uint32_t)page < (uint32_t)n_pages;
      const int64_t slot = key & ((1 << shift) - 1);
      const uint8_t *kb = khead + (int64_t)page * k_page_rs + slot * k_rs;
      const uint8_t *vb = vhead + (int64_t)page * v_page_rs + slot * v_rs;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(ok ? kb : khead, ok ? (uint32_t)((nv - 1) * k_rs + D) : 0u),
                                               (lds_void *)(stage + (u * NW + w) * 1024), 16, ln.kg[u], 0, 0, CP);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(ok ? vb : vhead, ok ? (uint32_t)((nv - 1) * v_rs + D) : 0u),
                                               (lds_void *)(stage + TILE_BYTES + (u * NW + w) * 1024), 16,
                                               ln.vg[u], 0, 0, CP);
    }
  }

  // S^T = K . Q^T for the staged tile; WIN operand reads stay in flight.
  __device__ static __forceinline__ void scores(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK], const Lane &ln,
                                                uint32_t stage_off) {
    u32x2 a[NKK];
#pragma unroll
    for (int kk = 0; kk < (NKK < WIN ? NKK : WIN); ++kk) a[kk] = ds_read_b64<0>(kaddr(ln, kk, stage_off));
    s[0] = f32x16{};
    score_step<0>(s, qreg, a, ln, stage_off);
  }
  template <int KK>
  __device__ static __forceinline__ void score_step(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK], u32x2 (&a)[NKK],
                                                    const Lane &ln, uint32_t stage_off) {
    constexpr int ISSUED = KK + WIN < NKK ? KK + WIN : NKK;  // reads issued before this step's wait
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(ISSUED - 1 - KK));
    asm volatile("" : "+v"(a[KK]));
    if constexpr (KK + WIN < NKK) a[KK + WIN] = ds_read_b64<0>(kaddr(ln, KK + WIN, stage_off));
    s[0] = mfma32(widen_fp8x8(a[KK]), qreg[KK], s[0]);
    if constexpr (KK + 1 < NKK) score_step<KK + 1>(s, qreg, a, ln, stage_off);
  }

  // O^T += V^T . P^T for the staged tile; read U serves head-dim block U % NDB
  // of value k-step U / NDB.
  static constexpr int NVR = NPV * NDB;
  __device__ static __forceinline__ void values(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], const Lane &ln,
                                                uint32_t stage_off) {
    u32x2 v[NVR];
#pragma unroll
    for (int u = 0; u < (NVR < WIN ? NVR : WIN); ++u) v[u] = ds_read_tr8<0>(vaddr(ln, u % NDB, u / NDB, stage_off));
    value_step<0>(o, pk, v, ln, stage_off);
  }
  template <int U>
  __device__ static __forceinline__ void value_step(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], u32x2 (&v)[NVR],
                                                    const Lane &ln, uint32_t stage_off) {
    constexpr int ISSUED = U + WIN < NVR ? U + WIN : NVR;
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(ISSUED - 1 - U));
    asm volatile("" : "+v"(v[U]));
    if constexpr (U + WIN < NVR)
      v[U + WIN] = ds_read_tr8<0>(vaddr(ln, (U + WIN) % NDB, (U + WIN) / NDB, stage_off));
    o[U % NDB] = mfma32(widen_fp8x8(v[U]), pk[U / NDB], o[U % NDB]);
    if constexpr (U + 1 < NVR) value_step<U + 1>(o, pk, v, ln, stage_off);
  }
};

}  // namespace attn

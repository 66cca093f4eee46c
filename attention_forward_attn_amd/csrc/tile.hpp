// The streaming-softmax tile engine shared by the prefill and decode kernels.
//
// Work split of one workgroup: NW wavefronts, each owning 32 query rows (in
// decode: 32 query heads of one kv head), so a workgroup covers BM = 32*NW
// rows and walks the visible keys in tiles of BN keys staged in LDS.
//
// Both products run transposed so that one lane ends up owning one query row:
//
//   score MMA   S^T (keys x rows) = K (keys x d)  . Q^T (d x rows)
//   value MMA   O^T (d x rows)   += V^T (d x keys) . P^T (keys x rows)
//
// With the 32x32x16 bf16 MFMA, lane l owns query row l%32 and, of the 32 keys
// of a block, the 16 keys {8a + 4*(l/32) + b : a < 4, b < 4}.  The row max then
// needs one cross-lane step (lanes l and l^32, a permlane32 swap) per tile, the
// row sum none until the end, and the O rescale is a per-lane scalar multiply.
// This is the planner page's state machine (section A1; executable steps 2, 3
// and 8: a score MMA and a value MMA with the max / rescale / exp between them,
// O divided by the row sum only once at the end), laid out for 64-wide
// wavefronts and a register-resident accumulator instead of Blackwell's TMEM.
//
// K and V tiles are copied HBM -> LDS by direct-to-LDS loads (no register
// staging), row-major.  The score MMA reads its K operand as one 16-byte row
// segment per lane; the value MMA needs V transposed and gets it from the
// gfx950 LDS transpose read (ds_read_b64_tr_b16: inside each 16-lane group,
// lane 4a+b points at 4 consecutive head-dim elements of key row a, and lane i
// receives head-dim element i of the 4 keys).  Each access pattern has its own
// XOR swizzle of the 16-byte chunks of a row so that the lanes serviced
// together touch distinct LDS banks; the direct-to-LDS load writes each wave's
// 1 KiB contiguously and applies the swizzle on the global side instead.
//
// The rescale is lazy: the running max used as the exponent base only moves
// when some row of the wave sees its max grow by more than 2^8.  O and the row
// sum always share that base, so the result is unchanged; the numerators stay
// below 2^8, far inside fp32 and bf16 range.
#pragma once

#include "common.hpp"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt with vmcnt = n (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  const __attribute__((address_space(3))) char *q = (const __attribute__((address_space(3))) char *)p;
  return (uint32_t)(uintptr_t)q;
}

// ds_read_b64_tr_b16 issued through inline assembly.  The compiler cannot
// attach a memory operand to the transpose read, so it would otherwise wait for
// every outstanding direct-to-LDS load (including the next tile's prefetch)
// before it.  The read's completion is handled explicitly by lds_wait_all.
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// Wait for all outstanding LDS reads of this wave; the results are routed
// through the statement so that no use can be scheduled above the wait.
template <int N>
__device__ __forceinline__ void lds_wait_all(u32x2 (&a)[N], u32x2 (&b)[N]) {
  if constexpr (N == 1) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]));
  } else if constexpr (N == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]));
  } else if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]), "+v"(a[2]), "+v"(b[2]),
                   "+v"(a[3]), "+v"(b[3]));
  } else {
    static_assert(N == 8, "unsupported count");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(b[0]), "+v"(a[1]), "+v"(b[1]), "+v"(a[2]), "+v"(b[2]),
                   "+v"(a[3]), "+v"(b[3]), "+v"(a[4]), "+v"(b[4]), "+v"(a[5]), "+v"(b[5]),
                   "+v"(a[6]), "+v"(b[6]), "+v"(a[7]), "+v"(b[7]));
  }
}

template <int D, int NW, int BN>
struct Tile {
  static constexpr int NT = NW * 64;   // threads per workgroup
  static constexpr int BM = NW * 32;   // query rows per workgroup
  static constexpr int CH = D / 8;     // 16-byte chunks per K / V row
  static constexpr int NKB = BN / 32;  // 32-key blocks per tile (score accumulators)
  static constexpr int NDB = D / 32;   // 32-wide head-dim blocks (O accumulators)
  static constexpr int NKK = D / 16;   // k-steps of the score MMA
  static constexpr int NPV = BN / 16;  // k-steps of the value MMA
  static constexpr int TILE_ELEMS = BN * D;                // one K or V tile, bf16 elements
  static constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;       // K + V
  static constexpr int LOADS = TILE_ELEMS / 8 / 64 / NW;   // 1-KiB DMA loads per wave per tile
  static constexpr int ROWS_PER_256 = 256 / (2 * D) > 0 ? 256 / (2 * D) : 1;
  static constexpr float kLazy = 8.0f;  // log2 of the growth that forces a rescale
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(LOADS * 64 * NW * 8 == TILE_ELEMS, "tile must split into whole 1-KiB wave loads");

  // Chunk swizzle for the score MMA's K reads: 16 lanes read one chunk of 16
  // consecutive rows.
  __device__ static __forceinline__ int kswz(int r) {
    return D == 64 ? ((r >> 1) & 7) : (r & 15);
  }
  // Chunk swizzle for the value MMA's transposed V reads: 16 lanes read 4
  // chunks of 4 consecutive rows.
  __device__ static __forceinline__ int vswz(int r) { return 4 * ((r / ROWS_PER_256) & 3) & (CH - 1); }

  // Issue this wave's share of the DMA loads of one K or V tile: rows
  // [j0, j0 + BN) of `base` (row stride `rs`), rows past `jmax` clamped to it
  // (their contents are masked out or multiplied by zero).
  template <bool IS_V>
  __device__ static __forceinline__ void dma(uint16_t *lds_tile, const uint16_t *base, int64_t rs,
                                             int j0, int jmax, int w, int lane) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int blk = u * NW + w;            // which 1-KiB block of the tile
      const int pch = blk * 64 + lane;       // physical 16-byte chunk written by this lane
      const int r = pch / CH;
      const int c = (pch % CH) ^ (IS_V ? vswz(r) : kswz(r));
      const int j = min(j0 + r, jmax);
      const uint16_t *src = base + (int64_t)j * rs + c * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds_tile + blk * 512), 16, 0, 0);
    }
  }

  // S^T block accumulators of this wave for the staged tile.  The K operands
  // of k-step kk+1 are read while the MMAs of step kk run.
  __device__ static __forceinline__ u32x4 kread(const uint16_t *lk, int kb, int kk, int lr, int hi) {
    const int r = kb * 32 + lr;
    return *reinterpret_cast<const u32x4 *>(lk + r * D + (((2 * kk + hi) ^ kswz(r)) * 8));
  }
  __device__ static __forceinline__ void scores(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                const uint16_t *lk, int lr, int hi) {
    u32x4 a[2][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      a[0][kb] = kread(lk, kb, 0, lr, hi);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) a[(kk + 1) & 1][kb] = kread(lk, kb, kk + 1, lr, hi);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(a[kk & 1][kb], qreg[kk], s[kb]);
    }
  }

  // Byte offset of (row, col) of a V tile in LDS, swizzled for the transposed read.
  __device__ static __forceinline__ uint32_t vaddr(const uint16_t *lv, int row, int col) {
    const int c = (col >> 3) ^ vswz(row);
    return lds_offset(lv + row * D + c * 8 + (col & 7));
  }

  // O^T += V^T . P^T with P given as packed bf16 (one u32x4 of 8 keys per k-step).
  // The k-slot order of P (8*hi + j <-> key 16t + 8*(j/4) + 4*hi + j%4) is
  // matched by reading keys 16t + 4*hi + {0..3} and 16t + 8 + 4*hi + {0..3}.
  // The transposed reads of one k-step are issued together and waited for
  // once (see ds_read_tr16).
  __device__ static __forceinline__ void values(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                const uint16_t *lv, int lane) {
    const int grp = lane >> 4, s = lane & 15;
    const int krow = 4 * (grp >> 1) + (s >> 2);       // key row inside a 16-key step
    const int dcol = 16 * (grp & 1) + 4 * (s & 3);    // head-dim column inside a 32-block
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      u32x2 lo[NDB], hi2[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        lo[db] = ds_read_tr16(vaddr(lv, 16 * t + krow, db * 32 + dcol));
        hi2[db] = ds_read_tr16(vaddr(lv, 16 * t + 8 + krow, db * 32 + dcol));
      }
      lds_wait_all(lo, hi2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4 a = {lo[db][0], lo[db][1], hi2[db][0], hi2[db][1]};
        o[db] = mfma32(a, pk[t], o[db]);
      }
    }
  }

  // Key index (relative to the tile start) held by accumulator register i of block kb.
  __device__ static __forceinline__ int key_of(int kb, int i, int hi) {
    return kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
  }

  // One online-softmax step on this wave's scores (already masked to -inf).
  // m is the exponent base in base-2 units, l this lane's partial row sum.
  __device__ static __forceinline__ void softmax_step(f32x16 (&s)[NKB], u32x4 (&pk)[NPV],
                                                      f32x16 (&o)[NDB], float &m, float &l,
                                                      float c) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_across_halves(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {  // wave-uniform
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == kNegInf) ? 0.0f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    const float base = (m == kNegInf) ? 0.0f : m;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(fmaf(s[kb][i], c, -base));
        s[kb][i] = e;
        rs += e;
      }
    l += rs;
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      const int kb = t >> 1, r0 = (t & 1) * 8;
      u32x4 x;
      x[0] = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
      x[1] = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
      x[2] = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
      x[3] = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
      pk[t] = x;
    }
  }
};

}  // namespace attn

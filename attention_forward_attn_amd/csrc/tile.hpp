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
// K and V tiles are copied HBM -> LDS by direct-to-LDS buffer loads (no
// register staging), row-major.  Each tile gets its own buffer descriptor
// whose base is the tile's first key and whose size ends at the last valid key,
// so the per-lane byte offsets are fixed for the whole kernel and the hardware
// range check zero-fills rows past the end of the keys.  The score MMA reads
// its K operand as one 16-byte row segment per lane; the value MMA needs V
// transposed and gets it from the gfx950 LDS transpose read (ds_read_b64_tr_b16:
// inside each 16-lane group, lane 4a+b points at 4 consecutive head-dim
// elements of key row a, and lane i receives head-dim element i of the 4
// keys).  Each access pattern has its own XOR swizzle of the 16-byte chunks of
// a row so that the lanes serviced together touch distinct LDS banks; the
// direct-to-LDS load writes each wave's 1 KiB contiguously and applies the
// swizzle on the global side instead.  All LDS read addresses are per-lane
// constants plus immediate offsets.
//
// The rescale is lazy: the running max used as the exponent base only moves
// when some row of the wave sees its max grow by more than 2^8.  O and the row
// sum always share that base, so the result is unchanged; the numerators stay
// below 2^8, far inside fp32 and bf16 range.
#pragma once

#include "common.hpp"

namespace attn {

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with vmcnt = n (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Three-input maximum.  fmaxf on MMA results makes the compiler quiet possible
// signalling NaNs first (an extra v_max_f32 x, x, x per input); the NaN-
// propagating maximum needs no such step and becomes one v_maximum3_f32.  The
// two differ only on NaN and on the order of -0 and +0, and the scores are
// finite or -inf, where a signed zero maximum gives the same exponentials.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// Maximum of N values by a tree of three-input maxima (N/2 instructions).
template <int N>
__device__ __forceinline__ float max_tree(const float *v) {
  if constexpr (N == 1) {
    return v[0];
  } else if constexpr (N <= 3) {
    return max3f(v[0], v[1], v[N - 1]);
  } else {
    constexpr int T3 = N / 3, M = T3 + N % 3;  // triples of this level, plus the leftovers
    float w[M];
#pragma unroll
    for (int k = 0; k < T3; ++k) w[k] = max3f(v[3 * k], v[3 * k + 1], v[3 * k + 2]);
#pragma unroll
    for (int k = 0; k < N % 3; ++k) w[T3 + k] = v[3 * T3 + k];
    return max_tree<M>(w);
  }
}

__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier without __syncthreads' memory fence.  The tile loops
// publish LDS data only through direct-to-LDS loads, whose completion every
// wave awaits itself (wait_vmcnt) before the barrier, and every LDS read of a
// stage is consumed by an MMA (so it has completed) before the barrier that
// frees the stage.  The fence would add a wait for all outstanding loads,
// including the prefetch of later tiles.
__device__ __forceinline__ void barrier_nofence() { __builtin_amdgcn_s_barrier(); }

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  const __attribute__((address_space(3))) char *q = (const __attribute__((address_space(3))) char *)p;
  return (uint32_t)(uintptr_t)q;
}

// Cache-policy operand of the buffer load/store builtins that sets sc1: the
// access is coherent at device scope (a store is written through the XCD's
// L2, a load does not take a line another XCD may have changed from it).
constexpr int kDeviceCoherent = 16;
// Cache-policy operand that sets nt: the data is streamed through once (the
// decode's K/V), so its lines get no retention priority in the caches.
constexpr int kStreamOnce = 2;

// Buffer descriptor over [base, base + bytes) (gfx9 raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS reads issued through inline assembly with an immediate offset.  The
// compiler cannot attach a memory operand to the transpose read and would
// otherwise wait for every outstanding direct-to-LDS load (including the next
// tile's prefetch) before it; completion is handled by lds_wait below.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// s_waitcnt lgkmcnt(N): LDS reads of one wave complete in order, so this
// guarantees every read issued before the last N has landed.  The registers
// of those reads are routed through the statement (and through empty
// statements after it, which keep their order) so that no use can be
// scheduled above the wait.  No scalar memory loads are in flight inside the
// tile loops, which would otherwise share the counter.
template <typename V>
__device__ __forceinline__ void tie8(V *a, int m) {
  if (m >= 8) {
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]));
  } else if (m >= 4) {
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
    if (m > 4) tie8(a + 4, m - 4);
  } else {
    for (int i = 0; i < m; ++i) asm volatile("" : "+v"(a[i]));
  }
}
template <int N, typename V, int M>
__device__ __forceinline__ void lds_wait(V (&a)[M]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
#pragma unroll
  for (int i = 0; i < M; i += 8) tie8(a + i, M - i < 8 ? M - i : 8);
}

// Eight independent 2^x (v_exp_f32, the instruction behind fast_exp2) issued
// back to back.  Left to itself the compiler pairs every exp with the FMA
// that feeds it, so a single wave stalls on each pair; here all eight
// arguments are computed first.  The trailing s_nop gives the wait state a
// vector instruction needs before reading a transcendental result (one is
// required, two are given), which the compiler cannot see through the asm
// statement.
__device__ __forceinline__ void exp2_x8(float (&e)[8], const float (&t)[8]) {
  asm volatile(
      "v_exp_f32 %0, %8\n v_exp_f32 %1, %9\n v_exp_f32 %2, %10\n v_exp_f32 %3, %11\n"
      "v_exp_f32 %4, %12\n v_exp_f32 %5, %13\n v_exp_f32 %6, %14\n v_exp_f32 %7, %15\n s_nop 1"
      : "=&v"(e[0]), "=&v"(e[1]), "=&v"(e[2]), "=&v"(e[3]), "=&v"(e[4]), "=&v"(e[5]), "=&v"(e[6]), "=&v"(e[7])
      : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(t[4]), "v"(t[5]), "v"(t[6]), "v"(t[7]));
}

// 2^x of N values in place, N a multiple of 8: every argument is computed
// before the first v_exp_f32 and every result is used after the last one, so
// the exponentials of a whole tile issue back to back and each consumer finds
// its input long done (a transcendental takes far longer to deliver its
// result than to issue: with eight in flight a lone wave waits on each group).
// The s_nop is the wait state a vector instruction needs before reading a
// transcendental result, which the compiler cannot see through the asm.
template <int N>
__device__ __forceinline__ void exp2_all(float (&x)[N]) {
  static_assert(N % 8 == 0, "groups of eight");
#pragma unroll
  for (int g = 0; g < N; g += 8) tie8(x + g, 8);
#pragma unroll
  for (int g = 0; g < N; g += 8)
    asm volatile(
        "v_exp_f32 %0, %0\n v_exp_f32 %1, %1\n v_exp_f32 %2, %2\n v_exp_f32 %3, %3\n"
        "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n v_exp_f32 %6, %6\n v_exp_f32 %7, %7"
        : "+v"(x[g]), "+v"(x[g + 1]), "+v"(x[g + 2]), "+v"(x[g + 3]), "+v"(x[g + 4]), "+v"(x[g + 5]),
          "+v"(x[g + 6]), "+v"(x[g + 7]));
  asm volatile("s_nop 1");
#pragma unroll
  for (int g = 0; g < N; g += 8) tie8(x + g, 8);
}

// DS is the head-dim slice a wave works on: DS = D normally; for D = 512 two
// waves share the same query rows and each takes one 256-wide half, for the
// partial scores as well as for the output columns (see prefill.hpp).
// XS: one swizzle for both read patterns, so that a tile read row-wise (score
// MMA) and transposed (value MMA) is staged once (the backward's tiles).
template <int D, int NW, int BN, int DS = D, bool XS = false>
struct Tile {
  static constexpr int NT = NW * 64;   // threads per workgroup
  static constexpr int SPLIT = D / DS; // waves sharing one block of query rows
  static constexpr int BM = NW * 32 / SPLIT;  // query rows per workgroup
  static constexpr int CH = D / 8;     // 16-byte chunks per K / V row
  static constexpr int NKB = BN / 32;  // 32-key blocks per tile (score accumulators)
  static constexpr int NDB = DS / 32;  // 32-wide head-dim blocks of this wave's slice (O accumulators)
  static constexpr int NKK = DS / 16;  // k-steps of the score MMA over this wave's slice
  static constexpr int NPV = BN / 16;  // k-steps of the value MMA
  static constexpr int TILE_ELEMS = BN * D;                // one K or V tile, bf16 elements
  static constexpr int TILE_BYTES = TILE_ELEMS * 2;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;       // K + V
  static constexpr int LOADS_EXACT = TILE_ELEMS / 8 / 64 / NW;
  static constexpr int LOADS = LOADS_EXACT > 0 ? LOADS_EXACT : 1;  // 1-KiB DMA loads per wave per tile
  static constexpr int ROWS_PER_256 = 256 / (2 * D) > 0 ? 256 / (2 * D) : 1;
  static constexpr float kLazy = 8.0f;  // log2 of the growth that forces a rescale
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(STAGE_BYTES <= 65536, "LDS immediate offsets must stay below 64 KiB");
  static_assert(!XS || CH >= 8, "the shared swizzle needs rows of at least 8 chunks");

  // Chunk swizzle for the score MMA's K reads: 16 lanes read one chunk of 16
  // consecutive rows.
  __device__ static __forceinline__ int kswz(int r) {
    if constexpr (XS) return xswz(r);
    return D == 64 ? ((r >> 1) & 7) : (r & 15);
  }
  // Chunk swizzle for the value MMA's transposed V reads: 16 lanes read 4
  // chunks of 4 consecutive rows.
  __device__ static __forceinline__ int vswz(int r) {
    if constexpr (XS) return xswz(r);
    return 4 * ((r / ROWS_PER_256) & 3) & (CH - 1);
  }
  // The shared swizzle.  Rows of 256 bytes or more start on bank 0: the
  // row-wise reads want 16 distinct values over any 16 aligned rows, the
  // transposed reads 4 distinct values of swz >> 2 over any 4 aligned rows;
  // 4 (r mod 4) + (r / 4 mod 4) gives both.  At D = 64 two rows share the 64
  // banks: the row-wise reads want 8 distinct values over the even rows of 16
  // aligned ones (and over the odd ones), the transposed reads distinct swz >> 2
  // for rows 4m and 4m + 2; 4 (r / 2 mod 2) + (r / 4 mod 4) gives both.  Either
  // way rows r and r + 8 differ by 2 (bit 5 of the byte address) and rows r and
  // r + 16 not at all.
  __device__ static __forceinline__ int xswz(int r) {
    return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
  }

  // Per-lane constants: global byte offsets of this lane's DMA chunks inside a
  // tile, and LDS byte addresses (stage 0) of its MMA operands.
  // Both swizzles only touch the low 4 bits of a chunk index, so chunks 16
  // apart stay 256 bytes apart: k-step kk+8 and head-dim block db+4 reuse the
  // address of kk and db with an immediate offset of 256 bytes, and a lane
  // keeps at most 8 + 4 LDS addresses.
  static constexpr int NKL = NKK < 8 ? NKK : 8;
  static constexpr int NVL = NDB < 4 ? NDB : 4;
  // At D = 512 one 1-KiB load is exactly one row (64 chunks), so a load's
  // offsets are lane * 16 XOR the row's swizzle plus the row's (wave-uniform)
  // start; they are formed when the load issues and the lane keeps only
  // lane * 16, which frees 2 * LOADS - 1 VGPRs for the wide head dim.  The
  // row start stays in the vector offset: the buffer range check, which
  // zero-fills rows past the end of the keys, does not see the scalar offset.
  static constexpr bool ROW_DMA = CH == 64;
  struct Lane {
    uint32_t kg[LOADS], vg[LOADS];  // global byte offsets (tile-relative); unused with ROW_DMA
    uint32_t l16;                   // lane * 16 (ROW_DMA only)
    uint32_t kl[NKL];               // LDS address of the K operand of k-step kk (mod 8), key block 0
    uint32_t vl[NVL];               // LDS address of the V^T operand of head-dim block db (mod 4), k-step 0
  };

  // DMA offsets: wave w of the NW loading waves, writing a BN x D tile.
  __device__ static __forceinline__ void init_dma(Lane &ln, int64_t k_rs, int64_t v_rs, int w, int lane) {
    static_assert(LOADS_EXACT * 64 * NW * 8 == TILE_ELEMS, "tile must split into whole 1-KiB wave loads");
    if constexpr (ROW_DMA) {
      ln.l16 = (uint32_t)lane * 16;
    } else {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int pch = (u * NW + w) * 64 + lane;  // physical 16-byte chunk written by this lane
        const int r = pch / CH;
        ln.kg[u] = (uint32_t)(r * k_rs * 2) + (uint32_t)(((pch % CH) ^ kswz(r)) * 16);
        ln.vg[u] = (uint32_t)(r * v_rs * 2) + (uint32_t)(((pch % CH) ^ vswz(r)) * 16);
      }
    }
  }

  // MMA operand addresses for the K tile at LDS byte address kbase and the V
  // tile at vbase (row-major, D columns, swizzled as above; the first row of
  // each must sit at a multiple of 16 rows of its tile), head-dim slice `slice`.
  __device__ static __forceinline__ void init_mma(Lane &ln, uint32_t kbase, uint32_t vbase, int lane,
                                                  int slice = 0) {
    const int lr = lane & 31, hi = lane >> 5;
    static_assert(NKK <= NKL || (DS / 8) % 16 == 0, "slices must start on a 16-chunk boundary");
#pragma unroll
    for (int kk = 0; kk < NKL; ++kk)
      ln.kl[kk] = kbase + lr * D * 2 + (((slice * (DS / 8) + 2 * kk + hi) ^ kswz(lr)) * 16);
    const int grp = lane >> 4, s = lane & 15;
    const int krow = 4 * (grp >> 1) + (s >> 2);     // key row inside a 16-key step
    const int dcol = 16 * (grp & 1) + 4 * (s & 3);  // head-dim column inside a 32-block
#pragma unroll
    for (int db = 0; db < NVL; ++db) {
      const int col = slice * DS + db * 32 + dcol;
      ln.vl[db] = vbase + krow * D * 2 + (((col >> 3) ^ vswz(krow)) * 16) + (col & 7) * 2;
    }
  }

  __device__ static __forceinline__ void init_lane(Lane &ln, const uint16_t *smem, int64_t k_rs,
                                                   int64_t v_rs, int w, int lane, int slice = 0) {
    init_dma(ln, k_rs, v_rs, w, lane);
    const uint32_t base = lds_offset(smem);
    init_mma(ln, base, base + TILE_BYTES, lane, slice);
  }

  // Issue this wave's share of the DMA loads of the BN-row tile of `base`
  // (row stride rs) that starts at key j0, into the LDS tile at `dst`; rows at
  // or past `nkeys` read as zero.  The descriptor ends exactly at the end of
  // the last valid row; a tile entirely past the end gets an empty descriptor,
  // so its loads touch no memory and only write zeros to LDS.  Byte offsets
  // inside a tile must fit in 32 bits (row strides below 2^24 elements,
  // checked by the host).
  // (is_v selects the V lane offsets; a constant at every call.)  CP is the
  // loads' cache-policy operand.
  template <int CP = 0>
  __device__ static __forceinline__ void dma1(const Lane &ln, bool is_v, uint16_t *dst, const uint16_t *base,
                                              int64_t rs, int j0, int nkeys, int w) {
    const int rows = min(nkeys - j0, BN);
    const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * rs * 2 + D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(rows > 0 ? base + j0 * rs : base, bytes);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      uint32_t off;
      if constexpr (ROW_DMA) {
        const int row = u * NW + w;  // the tile row this load writes
        uint32_t l16 = ln.l16;
        asm volatile("" : "+v"(l16));  // keep the offsets from being hoisted into registers held all loop
        off = (l16 ^ (uint32_t)((is_v ? vswz(row) : kswz(row)) * 16)) + (uint32_t)(row * rs * 2);
      } else {
        off = is_v ? ln.vg[u] : ln.kg[u];
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (u * NW + w) * 512), 16, off, 0, 0, CP);
    }
  }
  __device__ static __forceinline__ void dma_k(const Lane &ln, uint16_t *dst, const uint16_t *base,
                                               int64_t rs, int j0, int nkeys, int w) {
    dma1(ln, false, dst, base, rs, j0, nkeys, w);
  }
  __device__ static __forceinline__ void dma_v(const Lane &ln, uint16_t *dst, const uint16_t *base,
                                               int64_t rs, int j0, int nkeys, int w) {
    dma1(ln, true, dst, base, rs, j0, nkeys, w);
  }
  // K and V tiles of one key range into a stage laid out as [K tile][V tile].
  template <int CP = 0>
  __device__ static __forceinline__ void dma(const Lane &ln, uint16_t *stage, const uint16_t *kbase,
                                             int64_t k_rs, const uint16_t *vbase, int64_t v_rs,
                                             int j0, int nkeys, int w) {
    dma1<CP>(ln, false, stage, kbase, k_rs, j0, nkeys, w);
    dma1<CP>(ln, true, stage + TILE_ELEMS, vbase, v_rs, j0, nkeys, w);
  }
  // Paged caches: a load's 64/CH consecutive tile rows always sit in one page
  // (pages hold at least 16 rows), so each load gets its own descriptor and
  // the lane offsets are taken from the load's first row.
  __device__ static __forceinline__ void init_dma_paged(Lane &ln, int64_t k_rs, int64_t v_rs, int w, int lane) {
    static_assert(LOADS_EXACT * 64 * NW * 8 == TILE_ELEMS && 64 % CH == 0, "whole loads of whole rows");
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int pch = (u * NW + w) * 64 + lane;
      const int r = pch / CH, rl = lane / CH;  // row in the tile, row in the load
      ln.kg[u] = (uint32_t)(rl * k_rs * 2) + (uint32_t)(((pch % CH) ^ kswz(r)) * 16);
      ln.vg[u] = (uint32_t)(rl * v_rs * 2) + (uint32_t)(((pch % CH) ^ vswz(r)) * 16);
    }
  }
  // This wave's loads of the tile whose first key is jt (keys counted from the
  // start of a run of pages): key j of the run is row j % 2^shift of page
  // readlane(pg, j >> shift) at `head` + page * page_rs + row * rs.  Rows at or
  // past nkeys, and pages outside [0, n_pages), read as zero without touching
  // memory.  jt and w must be wave-uniform.
  template <int CP = 0>
  __device__ static __forceinline__ void dma1_paged(const Lane &ln, bool is_v, uint16_t *dst, const uint16_t *head,
                                                    int64_t rs, int64_t page_rs, int pg, int shift, int n_pages,
                                                    int jt, int nkeys, int w) {
    constexpr int RPL = 64 / CH;  // rows per load
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = jt + (u * NW + w) * RPL;
      const int nv = min(nkeys - key, RPL);
      const int page = __builtin_amdgcn_readlane(pg, min(key >> shift, 63));
      const bool ok = nv > 0 && (uint32_t)page < (uint32_t)n_pages;
      const uint16_t *base = head + (int64_t)page * page_rs + (int64_t)(key & ((1 << shift) - 1)) * rs;
      const uint32_t bytes = ok ? (uint32_t)((nv - 1) * rs * 2 + D * 2) : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(ok ? base : head, bytes),
                                               (lds_void *)(dst + (u * NW + w) * 512), 16,
                                               is_v ? ln.vg[u] : ln.kg[u], 0, 0, CP);
    }
  }
  template <int CP = 0>
  __device__ static __forceinline__ void dma_paged(const Lane &ln, uint16_t *stage, const uint16_t *khead,
                                                   int64_t k_rs, int64_t k_page_rs, const uint16_t *vhead,
                                                   int64_t v_rs, int64_t v_page_rs, int pg, int shift,
                                                   int n_pages, int jt, int nkeys, int w) {
    dma1_paged<CP>(ln, false, stage, khead, k_rs, k_page_rs, pg, shift, n_pages, jt, nkeys, w);
    dma1_paged<CP>(ln, true, stage + TILE_ELEMS, vhead, v_rs, v_page_rs, pg, shift, n_pages, jt, nkeys, w);
  }
  // The same loads, issued from inside an MMA schedule: step<G>() issues the
  // K share after MMA group GK and the V share after group GV.
  template <int GK, int GV>
  struct DmaHook {
    const Lane &ln;
    uint16_t *stage;
    const uint16_t *kbase, *vbase;
    int64_t k_rs, v_rs;
    int j0, nkeys, w;
    template <int G>
    __device__ __forceinline__ void step() {
      if constexpr (G == GK) dma_k(ln, stage, kbase, k_rs, j0, nkeys, w);
      if constexpr (G == GV) dma_v(ln, stage + TILE_ELEMS, vbase, v_rs, j0, nkeys, w);
    }
  };

  // S^T block accumulators of this wave for the staged tile.  The K operands
  // of k-step kk+1 are in flight while the MMAs of step kk run.
  template <int KK>
  __device__ static __forceinline__ void kreads(u32x4 (&a)[NKB], const Lane &ln, uint32_t stage_off) {
    const uint32_t ad = ln.kl[KK % NKL] + stage_off;
    constexpr int KO = (KK / NKL) * 256;
    a[0] = ds_read_b128<KO>(ad);
    if constexpr (NKB > 1) a[1] = ds_read_b128<KO + 1 * 32 * D * 2>(ad);
    if constexpr (NKB > 2) a[2] = ds_read_b128<KO + 2 * 32 * D * 2>(ad);
    if constexpr (NKB > 3) a[3] = ds_read_b128<KO + 3 * 32 * D * 2>(ad);
    static_assert(NKB <= 4, "at most 128 keys per tile");
  }
  struct NoHook {
    template <int KK>
    __device__ __forceinline__ void step() {}
  };
  // After the MMAs of k-step KK are issued, hook.step<KK>() runs: independent
  // VALU work placed there overlaps the in-flight MMAs.  K operands are read
  // two k-steps ahead of their MMAs (three register buffers rotate).
  template <int KK, bool MMA, typename Hook>
  __device__ static __forceinline__ void score_steps(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                     u32x4 (&cur)[NKB], u32x4 (&nx1)[NKB], u32x4 (&nx2)[NKB],
                                                     const Lane &ln, uint32_t stage_off, Hook &hook) {
    if constexpr (MMA) {
      if constexpr (KK + 2 < NKK) {
        kreads<KK + 2>(nx2, ln, stage_off);
        lds_wait<2 * NKB>(cur);
      } else if constexpr (KK + 1 < NKK) {
        lds_wait<NKB>(cur);
      } else {
        lds_wait<0>(cur);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(cur[kb], qreg[KK], s[kb]);
    }
    hook.template step<KK>();
    if constexpr (KK + 1 < NKK) score_steps<KK + 1, MMA>(s, qreg, nx1, nx2, cur, ln, stage_off, hook);
  }
  // Score MMAs of one tile with a hook between k-steps (MMA = false runs the
  // hook alone, for a tile this wave does not see).
  template <typename Hook>
  __device__ static __forceinline__ void scores_hooked(bool mma, f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                       const Lane &ln, uint32_t stage_off, Hook &hook) {
    if (mma)
      scores<true>(s, qreg, ln, stage_off, hook);
    else
      scores<false>(s, qreg, ln, stage_off, hook);
  }
  template <bool MMA = true, typename Hook = NoHook>
  __device__ static __forceinline__ void scores(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                const Lane &ln, uint32_t stage_off, Hook &&hook = Hook{}) {
    u32x4 a[NKB], b[NKB], c[NKB];
    if constexpr (MMA) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
      kreads<0>(a, ln, stage_off);
      if constexpr (NKK > 1) kreads<1>(b, ln, stage_off);
    }
    score_steps<0, MMA>(s, qreg, a, b, c, ln, stage_off, hook);
  }
  // The score MMAs in two halves, so that other work (the value MMA of the
  // previous tile) can run while the first K operands are in flight:
  // scores_issue reads the operands of k-steps 0 and 1 into a and b,
  // scores_run later runs all k-steps from them.
  struct KPre {
    u32x4 a[NKB], b[NKB];
  };
  __device__ static __forceinline__ void scores_issue(KPre &pre, const Lane &ln, uint32_t stage_off) {
    kreads<0>(pre.a, ln, stage_off);
    if constexpr (NKK > 1) kreads<1>(pre.b, ln, stage_off);
  }
  __device__ static __forceinline__ void scores_run(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK], KPre &pre,
                                                    const Lane &ln, uint32_t stage_off) {
    u32x4 c[NKB];
    NoHook hook;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    score_steps<0, true>(s, qreg, pre.a, pre.b, c, ln, stage_off, hook);
  }

  // O^T += V^T . P^T, one k-step of 16 keys at a time, with P packed bf16
  // (8 keys per lane).  The k-slot order of P (8*hi + j <-> key
  // 16T + 8*(j/4) + 4*hi + j%4) is matched by reading keys 16T + 4*hi + {0..3}
  // and 16T + 8 + 4*hi + {0..3}.  Work goes in units of (k-step, group of up
  // to 4 head-dim blocks), 8 transpose reads each, and the reads of unit U+1
  // are in flight while the MMAs of unit U run.
  // head-dim blocks per unit: 4, or 2 at wide head dims where registers are short
  static constexpr int VG = NDB < 4 ? NDB : (NDB >= 8 ? 2 : 4);
  static constexpr int VUNITS = NPV * (NDB / VG);
  template <int U>
  __device__ static __forceinline__ void vreads(u32x2 (&v)[2 * VG], const Lane &ln, uint32_t stage_off) {
    constexpr int T_ = U / (NDB / VG), G = U % (NDB / VG);
    constexpr int OFF_LO = T_ * 16 * D * 2;
    constexpr int OFF_HI = OFF_LO + 8 * D * 2;
    vread_blocks<OFF_LO, OFF_HI, G * VG, 0>(v, ln, stage_off);
  }
  template <int OFF_LO, int OFF_HI, int DB0, int I>
  __device__ static __forceinline__ void vread_blocks(u32x2 (&v)[2 * VG], const Lane &ln, uint32_t stage_off) {
    constexpr int DB = DB0 + I;
    constexpr int XO = (DB / NVL) * 256;
    const uint32_t a = ln.vl[DB % NVL] + stage_off;
    v[2 * I] = ds_read_tr16<OFF_LO + XO>(a);
    // under the shared swizzle the rows 8 further sit at chunk ^ 2: address bit 5
    // (stage offsets are multiples of 64 bytes, row strides of 256)
    v[2 * I + 1] = ds_read_tr16<OFF_HI + XO>(XS ? (a ^ 32u) : a);
    if constexpr (I + 1 < VG) vread_blocks<OFF_LO, OFF_HI, DB0, I + 1>(v, ln, stage_off);
  }
  // After the MMAs of the last unit of k-step T are issued, hook.vstep<T>() runs.
  template <int U, typename Hook>
  __device__ static __forceinline__ void value_steps(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                     u32x2 (&cur)[2 * VG], u32x2 (&nxt)[2 * VG],
                                                     const Lane &ln, uint32_t stage_off, Hook &hook) {
    constexpr int T_ = U / (NDB / VG), G = U % (NDB / VG);
    if constexpr (U + 1 < VUNITS) {
      vreads<U + 1>(nxt, ln, stage_off);
      lds_wait<2 * VG>(cur);
    } else {
      lds_wait<0>(cur);
    }
#pragma unroll
    for (int i = 0; i < VG; ++i) {
      const u32x4 a = {cur[2 * i][0], cur[2 * i][1], cur[2 * i + 1][0], cur[2 * i + 1][1]};
      o[G * VG + i] = mfma32(a, pk[T_], o[G * VG + i]);
    }
    if constexpr (G + 1 == NDB / VG) hook.template vstep<T_>();
    if constexpr (U + 1 < VUNITS) value_steps<U + 1>(o, pk, nxt, cur, ln, stage_off, hook);
  }
  struct NoVHook {
    template <int T_>
    __device__ __forceinline__ void vstep() {}
  };
  template <typename Hook = NoVHook>
  __device__ static __forceinline__ void values(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                const Lane &ln, uint32_t stage_off, Hook &&hook = Hook{}) {
    u32x2 a[2 * VG], b[2 * VG];
    vreads<0>(a, ln, stage_off);
    value_steps<0>(o, pk, a, b, ln, stage_off, hook);
  }
  // values() with the reads of unit 0 already issued into vpre.
  __device__ static __forceinline__ void values_from(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                     u32x2 (&vpre)[2 * VG], const Lane &ln, uint32_t stage_off) {
    u32x2 b[2 * VG];
    NoVHook hook;
    value_steps<0>(o, pk, vpre, b, ln, stage_off, hook);
  }

  // Value MMA of one tile interleaved with the score MMA of the next, for the
  // ping-pong prefill: value unit u (4 MMAs over one 16-key step) alternates
  // with score k-steps 2u and 2u+1, and every operand group is read one group
  // ahead, so each LDS read has the MMAs of two groups to land while at most
  // 12 reads are in flight.  The reads of value unit 0 (vpre) are issued by
  // the caller before the workgroup barrier that opens the phase.
  static constexpr bool PV_S_FUSED = (VUNITS * 2 == NKK) && (VG == NDB);
  __device__ static __forceinline__ void values_issue0(u32x2 (&vpre)[2 * VG], const Lane &ln, uint32_t v_off) {
    vreads<0>(vpre, ln, v_off);
  }
  template <int U>
  __device__ static __forceinline__ void pv_s_step(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], f32x16 (&s)[NKB],
                                                   const u32x4 (&qreg)[NKK], u32x2 (&vcur)[2 * VG],
                                                   u32x2 (&vnxt)[2 * VG], u32x4 (&kcur)[2][NKB],
                                                   u32x4 (&knxt)[2][NKB], const Lane &ln, uint32_t v_off,
                                                   uint32_t k_off) {
    constexpr int KR = 2 * NKB;  // reads of one pair of score k-steps
    lds_wait<KR>(vcur);          // value unit U landed (the k pair U behind it may not have)
#pragma unroll
    for (int i = 0; i < VG; ++i) {
      const u32x4 a = {vcur[2 * i][0], vcur[2 * i][1], vcur[2 * i + 1][0], vcur[2 * i + 1][1]};
      o[i] = mfma32(a, pk[U], o[i]);
    }
    if constexpr (U + 1 < VUNITS) {
      vreads<U + 1>(vnxt, ln, v_off);
      lds_wait<2 * VG>(kcur[0]);
      tie8(kcur[1], NKB);
    } else {
      lds_wait<0>(kcur[0]);
      tie8(kcur[1], NKB);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(kcur[0][kb], qreg[2 * U], s[kb]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(kcur[1][kb], qreg[2 * U + 1], s[kb]);
    if constexpr (U + 1 < VUNITS) {
      kreads<2 * U + 2>(knxt[0], ln, k_off);
      kreads<2 * U + 3>(knxt[1], ln, k_off);
      pv_s_step<U + 1>(o, pk, s, qreg, vnxt, vcur, knxt, kcur, ln, v_off, k_off);
    }
  }
  __device__ static __forceinline__ void pv_scores(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], f32x16 (&s)[NKB],
                                                   const u32x4 (&qreg)[NKK], u32x2 (&vpre)[2 * VG],
                                                   const Lane &ln, uint32_t v_off, uint32_t k_off) {
    static_assert(PV_S_FUSED, "fused value/score schedule needs NKK == 2 * value units and one head-dim group");
    u32x2 vb[2 * VG];
    u32x4 ka[2][NKB], kb2[2][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    kreads<0>(ka[0], ln, k_off);
    kreads<1>(ka[1], ln, k_off);
    pv_s_step<0>(o, pk, s, qreg, vpre, vb, ka, kb2, ln, v_off, k_off);
  }

  // Finer version of the same schedule: 2*NKK groups of two MMAs alternate a
  // value half-unit (two head-dim blocks of one 16-key step) with one score
  // k-step, and the operands of group g+3 are read before group g waits, so
  // every LDS read has the MMAs of three groups to land (at most 12 reads in
  // flight).  Groups 0 and 2 (value unit 0) come from vpre, read before the
  // barrier; the reads are issued in the order 0, 2, 1, 3, 4, 5, ...
  static constexpr bool PV_S_FINE = PV_S_FUSED && NDB == 4 && NKK == 8;
  static constexpr int fine_n(int g) { return (g & 1) ? NKB : 4; }  // reads of group g
  static constexpr int fine_pos(int g) { return g == 1 ? 2 : g == 2 ? 1 : g; }  // issue position
  // reads issued after group g's, once group g+3 (if any) has been issued
  static constexpr int fine_after(int g) {
    int c = 0;
    const int last = g + 3 < 2 * NKK ? g + 3 : 2 * NKK - 1;
    for (int k = 0; k <= last; ++k)
      if (fine_pos(k) > fine_pos(g)) c += fine_n(k);
    return c;
  }
  struct FineBufs {
    u32x2 pv[3][4];
    u32x4 sk[3][NKB];
  };
  template <int G>
  __device__ static __forceinline__ void fine_issue(FineBufs &fb, u32x2 (&vpre)[8], const Lane &ln,
                                                    uint32_t v_off, uint32_t k_off) {
    if constexpr (G & 1) {
      kreads<G / 2>(fb.sk[(G / 2) % 3], ln, k_off);
    } else {
      constexpr int H = G / 2, T_ = H / 2, B0 = 2 * (H & 1);
      static_assert(H >= 2, "value half-units 0 and 1 come from vpre");
      constexpr int OFF_LO = T_ * 16 * D * 2, OFF_HI = OFF_LO + 8 * D * 2;
      u32x2 (&v)[4] = fb.pv[(H - 2) % 3];
      v[0] = ds_read_tr16<OFF_LO>(ln.vl[B0] + v_off);
      v[1] = ds_read_tr16<OFF_HI>(ln.vl[B0] + v_off);
      v[2] = ds_read_tr16<OFF_LO>(ln.vl[B0 + 1] + v_off);
      v[3] = ds_read_tr16<OFF_HI>(ln.vl[B0 + 1] + v_off);
    }
  }
  template <int G, typename Hook>
  __device__ static __forceinline__ void fine_step(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV], f32x16 (&s)[NKB],
                                                   const u32x4 (&qreg)[NKK], u32x2 (&vpre)[8], FineBufs &fb,
                                                   const Lane &ln, uint32_t v_off, uint32_t k_off, Hook &hook) {
    if constexpr (G + 3 < 2 * NKK) fine_issue<G + 3>(fb, vpre, ln, v_off, k_off);
    constexpr int W = fine_after(G);
    if constexpr (G & 1) {
      u32x4 (&k)[NKB] = fb.sk[(G / 2) % 3];
      lds_wait<W>(k);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(k[kb], qreg[G / 2], s[kb]);
    } else {
      constexpr int H = G / 2, T_ = H / 2, B0 = 2 * (H & 1);
      u32x2 *v = H < 2 ? vpre + 4 * H : fb.pv[(H - 2 + 3) % 3];
      asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(W));
      tie8(v, 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 a = {v[2 * j][0], v[2 * j][1], v[2 * j + 1][0], v[2 * j + 1][1]};
        o[B0 + j] = mfma32(a, pk[T_], o[B0 + j]);
      }
    }
    hook.template step<G>();
    if constexpr (G + 1 < 2 * NKK) fine_step<G + 1>(o, pk, s, qreg, vpre, fb, ln, v_off, k_off, hook);
  }
  // hook.step<G>() runs after the MMAs of group G are issued.
  template <typename Hook = NoHook>
  __device__ static __forceinline__ void pv_scores_fine(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                        f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                        u32x2 (&vpre)[8], const Lane &ln, uint32_t v_off,
                                                        uint32_t k_off, Hook &&hook = Hook{}) {
    static_assert(PV_S_FINE, "fine schedule shape");
    FineBufs fb;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    fine_issue<1>(fb, vpre, ln, v_off, k_off);  // groups 0 and 2 are in vpre
    fine_step<0>(o, pk, s, qreg, vpre, fb, ln, v_off, k_off, hook);
  }

  // Output epilogue of one wave: its 32 x DS tile of O, normalised by inv and
  // rounded to bf16, goes to memory through LDS.  A lane holds 8-byte pieces of
  // one row (columns db*32 + 8*gi + 4*hi .. +3), so stores straight from the
  // accumulators would touch 32 rows per instruction; stage_out puts the
  // pieces into a 32 x DS tile at xw (16-byte chunks XOR-swizzled by row),
  // and store_out then writes whole 16-byte chunks of consecutive row
  // segments.  Row r goes to dst + r * row_stride; rows at or past n_rows are
  // not written.  Between the two calls the workgroup must pass a barrier (the
  // tile is read back by other lanes), and xw must not be in use by any load.
  static constexpr int OUT_BYTES = 32 * DS * 2;  // LDS bytes of one wave's staged tile
  // Staging pays at slices up to 128 columns; at 256 the kernels already hold
  // (nearly) all 256 VGPRs and its registers spill into the tile loop, so
  // those store straight from the accumulators (store_direct).
  static constexpr bool STAGED_OUT = DS <= 128;
  __device__ static __forceinline__ void store_direct(const f32x16 (&o)[NDB], float inv, uint16_t *dst_row,
                                                      int lane) {
    uint16_t *op = dst_row + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 val;
        val[0] = pack_bf16x2(o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv);
        val[1] = pack_bf16x2(o[db][4 * gi + 2] * inv, o[db][4 * gi + 3] * inv);
        *reinterpret_cast<u32x2 *>(op + db * 32 + 8 * gi) = val;
      }
  }
  __device__ static __forceinline__ void stage_out(const f32x16 (&o)[NDB], float inv, char *xw, int lane) {
    constexpr int NC = DS / 8;             // 16-byte chunks per row segment
    constexpr int SW = NC < 16 ? NC : 16;  // swizzle span
    const int lr = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 val;
        val[0] = pack_bf16x2(o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv);
        val[1] = pack_bf16x2(o[db][4 * gi + 2] * inv, o[db][4 * gi + 3] * inv);
        *reinterpret_cast<u32x2 *>(xw + lr * DS * 2 + ((db * 4 + gi) ^ (lr % SW)) * 16 + 8 * hi) = val;
      }
  }
  __device__ static __forceinline__ void store_out(const char *xw, int lane, uint16_t *dst, int64_t row_stride,
                                                   int n_rows) {
    constexpr int NC = DS / 8;
    constexpr int SW = NC < 16 ? NC : 16;
    constexpr int RPI = 64 / NC;  // rows per store instruction
    static_assert(64 % NC == 0 && NC <= 64, "whole row segments per store");
    const int c = lane % NC;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / NC;
      const u32x4 val = *reinterpret_cast<const u32x4 *>(xw + r * DS * 2 + (c ^ (r % SW)) * 16);
      if (r < n_rows) *reinterpret_cast<u32x4 *>(dst + r * row_stride + c * 8) = val;
    }
  }

  // Key index (relative to the tile start) held by accumulator register i of block kb.
  __device__ static __forceinline__ int key_of(int kb, int i, int hi) {
    return kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
  }

  // Online-softmax update, first half: running max over this tile (scores
  // already masked to -inf), lazy rescale of l and O; returns the exponent base.
  __device__ static __forceinline__ float softmax_max(const f32x16 (&s)[NKB], f32x16 (&o)[NDB], float &m,
                                                      float &l, float c) {
    float v[16 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * kb + i] = s[kb][i];
    const float mx = max_across_halves(max_tree<16 * NKB>(v)) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {  // wave-uniform
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == kNegInf) ? 0.0f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    return (m == kNegInf) ? 0.0f : m;
  }
  // Second half: numerators 2^(c*s - base) of the tile, packed to bf16 into pk
  // (value k-step T takes the 16 keys of block T/2, registers 8(T mod 2) ..
  // +7), their fp32 sum added to rs.  GROUPED: the exponentials go in groups of
  // eight, each group's results used before the next group's arguments are
  // formed; otherwise all exponentials of the tile issue back to back (faster
  // for a lone wave; the ping-pong kernels keep the groups, whose softmax phase
  // then stays as long as the other group's MMA phase that it overlaps).
  template <bool GROUPED>
  __device__ static __forceinline__ void softmax_exp_all(const f32x16 (&s)[NKB], u32x4 (&pk)[NPV], float &rs,
                                                         float c, float base) {
    float e[16 * NKB];
    auto pack_sum = [&](int t) {
      const float *et = e + 8 * t;
      u32x4 x;
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = pack_bf16x2(et[2 * q], et[2 * q + 1]);
      pk[t] = x;
      rs += ((et[0] + et[1]) + (et[2] + et[3])) + ((et[4] + et[5]) + (et[6] + et[7]));
    };
    if constexpr (GROUPED) {
#pragma unroll
      for (int t = 0; t < NPV; ++t) {
        float g[8], r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = fmaf(s[t >> 1][8 * (t & 1) + j], c, -base);
        exp2_x8(r, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) e[8 * t + j] = r[j];
        pack_sum(t);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) e[16 * kb + i] = fmaf(s[kb][i], c, -base);
      exp2_all(e);
#pragma unroll
      for (int t = 0; t < NPV; ++t) pack_sum(t);
    }
  }
  // The whole update on one tile (no overlap with other work).
  template <bool GROUPED = false>
  __device__ static __forceinline__ void softmax_step(f32x16 (&s)[NKB], u32x4 (&pk)[NPV],
                                                      f32x16 (&o)[NDB], float &m, float &l,
                                                      float c) {
    const float base = softmax_max(s, o, m, l, c);
    float rs = 0.0f;
    softmax_exp_all<GROUPED>(s, pk, rs, c, base);
    l += rs;
  }
};

}  // namespace attn

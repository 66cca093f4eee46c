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
// needs one cross-lane step (lanes l and l^32) per tile, the row sum none until
// the end, and the O rescale is a per-lane scalar multiply.  This is the
// planner page's state machine (section A1; executable steps 2, 3 and 8: a
// score MMA and a value MMA with the max / rescale / exp between them, O
// divided by the row sum only once at the end), laid out for 64-wide
// wavefronts instead of Blackwell's TMEM.
//
// LDS holds, per pipeline stage, K row-major (the score MMA's A operand reads
// 16 contiguous bytes of one key row) and V transposed (the value MMA's A
// operand reads 8 keys of one head-dim column).  The key order inside V^T is
// permuted per 16-key group so that those 8 keys are contiguous and match, slot
// for slot, the keys that the lane's score accumulators hold (the contraction
// order of P.V is free).  16-byte chunks are XOR-swizzled per row so that 16
// consecutive lanes reading the same logical chunk of 16 different rows hit
// 16 different bank groups.
#pragma once

#include "common.hpp"

namespace attn {

template <int D, int NW, int BN>
struct Tile {
  static constexpr int NT = NW * 64;   // threads per workgroup
  static constexpr int BM = NW * 32;   // query rows per workgroup
  static constexpr int KCH = D / 8;    // 16-byte chunks per K row
  static constexpr int VCH = BN / 8;   // 16-byte chunks per V^T row
  static constexpr int NKB = BN / 32;  // 32-key blocks per tile (score accumulators)
  static constexpr int NDB = D / 32;   // 32-wide head-dim blocks (O accumulators)
  static constexpr int NKK = D / 16;   // k-steps of the score MMA
  static constexpr int NPV = BN / 16;  // k-steps of the value MMA
  static constexpr int KLOADS = BN * KCH / NT;       // K chunks staged per thread
  static constexpr int VITEMS = (BN / 4) * KCH / NT;  // (4 keys x 8 dims) V items per thread
  static constexpr int STAGE_ELEMS = 2 * BN * D;      // K + V^T, bf16 elements
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(KLOADS * NT == BN * KCH, "K tile must split evenly over the threads");
  static_assert(VITEMS * NT == (BN / 4) * KCH, "V tile must split evenly over the threads");

  // Swizzle of the 16-byte chunk index within a K row / V^T row.
  __device__ static __forceinline__ int kswz(int r) { return D == 64 ? ((r >> 1) & 7) : (r & 15); }
  __device__ static __forceinline__ int vswz(int d) {
    constexpr int rows_per_256 = 256 / (BN * 2) > 0 ? 256 / (BN * 2) : 1;
    constexpr int mask = VCH < 16 ? VCH - 1 : 15;
    return (d / rows_per_256) & mask;
  }
  // Position, inside its 16-key group, where key offset kk (0..15) is stored in V^T.
  __device__ static __forceinline__ int vpos16(int kk) {
    return 8 * ((kk >> 2) & 1) + 4 * (kk >> 3) + (kk & 3);
  }

  struct Stage {
    u32x4 k[KLOADS];
    u32x4 v[VITEMS][4];
  };

  // Global -> registers for keys [j0, j0 + BN); keys >= jend load as zero.
  __device__ static __forceinline__ void load(Stage &st, const uint16_t *kb, int64_t k_rs,
                                              const uint16_t *vb, int64_t v_rs, int j0, int jend,
                                              int tid) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int id = tid + u * NT;
      const int r = id / KCH, c = id % KCH;
      const int j = j0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < jend) x = *reinterpret_cast<const u32x4 *>(kb + (int64_t)j * k_rs + c * 8);
      st.k[u] = x;
    }
#pragma unroll
    for (int u = 0; u < VITEMS; ++u) {
      const int id = tid + u * NT;
      const int kg = id % (BN / 4), dg = id / (BN / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * kg + i;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (j < jend) x = *reinterpret_cast<const u32x4 *>(vb + (int64_t)j * v_rs + dg * 8);
        st.v[u][i] = x;
      }
    }
  }

  // Registers -> LDS stage (K row-major, V transposed with the key permutation).
  __device__ static __forceinline__ void store(const Stage &st, uint16_t *lk, uint16_t *lv,
                                               int tid) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int id = tid + u * NT;
      const int r = id / KCH, c = id % KCH;
      *reinterpret_cast<u32x4 *>(lk + r * D + ((c ^ kswz(r)) * 8)) = st.k[u];
    }
#pragma unroll
    for (int u = 0; u < VITEMS; ++u) {
      const int id = tid + u * NT;
      const int kg = id % (BN / 4), dg = id / (BN / 4);
      const int p0 = 16 * (kg >> 2) + vpos16(4 * (kg & 3));  // multiple of 4
      const u32x4 r0 = st.v[u][0], r1 = st.v[u][1], r2 = st.v[u][2], r3 = st.v[u][3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo, hi;
        if ((e & 1) == 0) {
          lo = (r0[w] & 0xffffu) | (r1[w] << 16);
          hi = (r2[w] & 0xffffu) | (r3[w] << 16);
        } else {
          lo = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
          hi = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
        }
        const int d = dg * 8 + e;
        u32x2 val = {lo, hi};
        *reinterpret_cast<u32x2 *>(lv + d * BN + (((p0 >> 3) ^ vswz(d)) * 8) + (p0 & 7)) = val;
      }
    }
  }

  // S^T block accumulators of this wave for the staged tile.
  __device__ static __forceinline__ void scores(f32x16 (&s)[NKB], const u32x4 (&qreg)[NKK],
                                                const uint16_t *lk, int lr, int hi) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = kb * 32 + lr;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(lk + r * D + (((2 * kk + hi) ^ kswz(r)) * 8));
        s[kb] = mfma32(a, qreg[kk], s[kb]);
      }
    }
  }

  // O^T += V^T . P^T with P given as packed bf16 (one u32x4 of 8 keys per k-step).
  __device__ static __forceinline__ void values(f32x16 (&o)[NDB], const u32x4 (&pk)[NPV],
                                                const uint16_t *lv, int lr, int hi) {
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dr = db * 32 + lr;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(lv + dr * BN + (((2 * t + hi) ^ vswz(dr)) * 8));
        o[db] = mfma32(a, pk[t], o[db]);
      }
    }
  }

  // Key index (relative to the tile start) held by accumulator register i of block kb.
  __device__ static __forceinline__ int key_of(int kb, int i, int hi) {
    return kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
  }

  // One online-softmax step on this wave's scores (already masked to -inf):
  // update the running max m (base-2 units), rescale l and O by
  // alpha = 2^(m_old - m_new), turn the scores into bf16 numerators P.
  __device__ static __forceinline__ void softmax_step(f32x16 (&s)[NKB], u32x4 (&pk)[NPV],
                                                      f32x16 (&o)[NDB], float &m, float &l,
                                                      float c) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float base = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - base);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
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

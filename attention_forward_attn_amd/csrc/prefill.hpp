// Prefill kernel: one workgroup per (batch, query head, tile of BM query rows).
//
// Masks follow the planner page's executable step 7: key tiles outside the
// visible range [kbeg, kend) of the workgroup are never loaded, tiles fully
// inside every row's visible range skip the element mask, and only tiles that
// cross a diagonal, a window edge or the end of the keys are masked
// element by element.  Causal masking is bottom-right aligned (o = s_k - s_q).
// A sink (status page row D5c) enters as the initial state of the running
// softmax: max = sigma * log2(e) and sum = 1, with nothing added to O.
//
// Head dim 512 (the STAGE_D.md page's hd=512 case): the two waves of a pair
// own the same 32 query rows and split the head dim into two 256-wide halves.
// Each wave computes the partial scores over its half of Q and K; the pair
// swaps the partials through LDS and adds them, so the score is summed in
// logit space (S = S_0 + S_1) before any softmax; both waves then run the
// same softmax and each multiplies P by its own 256 columns of V.
//
#pragma once

#include "tile.hpp"

namespace attn {

template <int D, int NW, int BN, bool CAUSAL, bool WINDOW, int OCC, int DS = D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void prefill_kernel(PrefillParams p) {
  using T = Tile<D, NW, BN, DS>;
  constexpr int BM = T::BM;
  constexpr int SPLIT = T::SPLIT;
  constexpr int XBYTES = SPLIT > 1 ? NW * T::NKB * 16 * 64 * 4 : 0;  // partial-score exchange
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(2 * T::STAGE_BYTES + XBYTES) / 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int w = wave / SPLIT;      // row block of this wave
  const int slice = wave % SPLIT;  // head-dim slice of this wave

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
  // range of work units so that the query tiles sharing one head's K/V run on
  // the same L2.  Inside a head, the longest (last) query tiles go first.
  const int n_units = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = n_units >> 3, rem = n_units & 7;
  const int unit = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int bh = unit / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (unit - bh * p.n_qtiles);
  const int bi = bh / p.h_q, h = bh - bi * p.h_q;
  const int g = h / p.ratio;
  const int q0 = qt * BM;
  const int off = p.s_k - p.s_q;

  // Keys visible to any row of this workgroup.
  const int i_last = min(p.s_q, q0 + BM) - 1;
  int kend = p.s_k;
  if (CAUSAL) kend = max(0, min(kend, i_last + off + 1));
  int kbeg = 0;
  if (WINDOW) kbeg = max(0, q0 + off - p.window + 1);
  const int t_begin = kbeg / BN;
  const int t_end = kbeg < kend ? (kend + BN - 1) / BN : t_begin;

  // This wave's rows.
  const int w_lo = q0 + w * 32;
  const int w_hi = min(w_lo + 31, p.s_q - 1);
  const int row = w_lo + lr;
  const bool row_ok = row < p.s_q;

  const uint16_t *kbase = p.k + bi * p.k_sb + g * p.k_sh;
  const uint16_t *vbase = p.v + bi * p.v_sb + g * p.v_sh;

  u32x4 qreg[T::NKK];
  {
    const uint16_t *qp = p.q + bi * p.q_sb + h * p.q_sh + (int64_t)min(row, p.s_q - 1) * p.q_ss +
                         slice * DS + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < T::NKK; ++kk) qreg[kk] = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
  }

  float m = kNegInf, l = 0.0f;
  if (p.sinks != nullptr) {
    m = p.sinks[h] * kLog2e;
    l = hi == 0 ? 1.0f : 0.0f;
  }
  f32x16 o[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) o[db] = f32x16{};

  // Does this wave's row block see any key of tile t, and must it be masked?
  auto active = [&](int t) {
    const int j0 = t * BN;
    bool a = w_lo < p.s_q;
    if (CAUSAL) a = a && j0 <= w_hi + off;
    if (WINDOW) a = a && j0 + BN - 1 >= w_lo + off - p.window + 1;
    return a;
  };
  auto mask = [&](f32x16 (&s)[T::NKB], int t) {
    const int j0 = t * BN;
    bool need = j0 + BN > p.s_k;
    if (CAUSAL) need = need || (j0 + BN - 1 > w_lo + off);
    if (WINDOW) need = need || (j0 < w_hi + off - p.window + 1);
    if (need) {
      const int lim_hi = CAUSAL ? min(row + off, p.s_k - 1) : p.s_k - 1;
      const int lim_lo = WINDOW ? row + off - p.window + 1 : 0;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + T::key_of(kb, i, hi);
          if (j > lim_hi || j < lim_lo) s[kb][i] = kNegInf;
        }
    }
  };

  if constexpr (SPLIT == 1) {
    // Two LDS stages of [K tile][V tile].  At the top of iteration t the
    // wave waits for its own loads of tile t and the barrier publishes the
    // tile (and guarantees every wave is done with tile t-1's stage); the loads
    // of tile t+1 into the other stage then run under the MMAs of tile t.
    typename T::Lane ln;
    T::init_lane(ln, smem, p.k_ss, p.v_ss, wave, lane);
    if (t_begin < t_end) T::dma(ln, smem, kbase, p.k_ss, vbase, p.v_ss, t_begin * BN, p.s_k, wave);
    for (int t = t_begin; t < t_end; ++t) {
      const int cur = (t - t_begin) & 1;
      wait_vmcnt<0>();
      __syncthreads();
      if (t + 1 < t_end)
        T::dma(ln, smem + (cur ^ 1) * (T::STAGE_BYTES / 2), kbase, p.k_ss, vbase, p.v_ss, (t + 1) * BN,
               p.s_k, wave);
      const uint32_t stage_off = cur * T::STAGE_BYTES;
      if (active(t)) {
        f32x16 s[T::NKB];
        T::scores(s, qreg, ln, stage_off);
        mask(s, t);
        u32x4 pk[T::NPV];
        T::softmax_step(s, pk, o, m, l, p.c);
        T::values(o, pk, ln, stage_off);
      }
    }
  } else {
    // Head dim split over wave pairs (no cross-tile pipelining): two LDS
    // stages of [K tile][V tile].
    typename T::Lane ln;
    T::init_lane(ln, smem, p.k_ss, p.v_ss, wave, lane, slice);
    if (t_begin < t_end) T::dma(ln, smem, kbase, p.k_ss, vbase, p.v_ss, t_begin * BN, p.s_k, wave);
    for (int t = t_begin; t < t_end; ++t) {
      const int cur = (t - t_begin) & 1;
      wait_vmcnt<0>();
      __syncthreads();
      if (t + 1 < t_end)
        T::dma(ln, smem + (cur ^ 1) * (T::STAGE_BYTES / 2), kbase, p.k_ss, vbase, p.v_ss, (t + 1) * BN,
               p.s_k, wave);
      const uint32_t stage_off = cur * T::STAGE_BYTES;
      const bool act = active(t);
      // Both waves of a pair take part in the exchange (and its barrier); the
      // pair's activity is decided together, inactive pairs skip the MMAs.
      f32x16 s[T::NKB];
      if (act) T::scores(s, qreg, ln, stage_off);
      f32x4 *xb = reinterpret_cast<f32x4 *>(reinterpret_cast<char *>(smem) + 2 * T::STAGE_BYTES);
      if (act) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {s[kb][4 * q4], s[kb][4 * q4 + 1], s[kb][4 * q4 + 2], s[kb][4 * q4 + 3]};
            xb[(wave * T::NKB * 4 + kb * 4 + q4) * 64 + lane] = v;
          }
      }
      __syncthreads();
      if (act) {
        const int partner = wave ^ 1;
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = xb[(partner * T::NKB * 4 + kb * 4 + q4) * 64 + lane];
            s[kb][4 * q4] += v[0];
            s[kb][4 * q4 + 1] += v[1];
            s[kb][4 * q4 + 2] += v[2];
            s[kb][4 * q4 + 3] += v[3];
          }
        mask(s, t);
        u32x4 pk[T::NPV];
        T::softmax_step(s, pk, o, m, l, p.c);
        T::values(o, pk, ln, stage_off);
      }
    }
  }

  // Epilogue: O / l once, bf16 round-to-nearest-even; LSE = ln2 * (m + log2 l).
  const float lt = sum_across_halves(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    uint16_t *op = p.o + bi * p.o_sb + h * p.o_sh + (int64_t)row * p.o_ss + slice * DS + 4 * hi;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 val;
        val[0] = pack_bf16x2(o[db][4 * gi + 0] * inv, o[db][4 * gi + 1] * inv);
        val[1] = pack_bf16x2(o[db][4 * gi + 2] * inv, o[db][4 * gi + 3] * inv);
        *reinterpret_cast<u32x2 *>(op + db * 32 + 8 * gi) = val;
      }
    if (p.lse != nullptr && hi == 0 && slice == 0)
      p.lse[bi * p.lse_sb + h * p.lse_sh + row] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

// Host-side launcher of one instantiation.
template <int D, int NW, int BN, bool CAUSAL, bool WINDOW, int OCC, int DS = D>
hipError_t launch_prefill(const PrefillParams &p, int n_units, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, NW, BN, CAUSAL, WINDOW, OCC, DS>), dim3(n_units), dim3(NW * 64),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

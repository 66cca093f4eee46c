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
// Head dim 512 (the STAGE_D.md page's hd=512 case): SPLIT consecutive waves
// own the same 32 query rows and split the head dim into SPLIT slices (two
// 256-wide halves as on the page).  Each wave computes the partial scores
// over its slice of Q and K; the pair swaps the partials through LDS and adds
// them, so the score is summed in logit space (S = S_0 + S_1) before any
// softmax; both waves then run the same softmax and multiply P by their own
// slice of V's columns.  The two halves of the workgroup take turns, so that
// one wave's softmax runs beside the other's score MMAs on every SIMD.
//
#pragma once

#include <type_traits>

#include "combine.hpp"
#include "tile.hpp"

namespace attn {

// Work unit of workgroup v: (batch x query head bh, query tile qt).
// Workgroups are dealt round-robin to the 8 XCDs (v % 8).  When the kv heads
// divide evenly, every query head of kv head bkv is placed on XCD bkv % 8, so
// the query tiles and heads that read the same K/V share one L2; with fewer
// than 8 kv heads, each gets its own group of 8 / (b * h_kv) XCDs.  The order
// inside an XCD depends on the mask: with a plain causal mask (LONGEST_FIRST)
// the later query tiles see the most keys, so units go out in levels of
// decreasing qt and the short ones fill in behind the long ones; otherwise
// all units are alike and one head's query tiles run together, which keeps
// the K/V working set of an XCD to a few heads.
template <bool LONGEST_FIRST>
__device__ __forceinline__ void prefill_unit(const PrefillParams &p, int v, int &bh, int &qt) {
  const int BH = p.b * p.h_q;
  const int nq = p.n_qtiles;
  if (((p.b * p.h_kv) & 7) == 0) {
    const int xcd = v & 7, slot = v >> 3;  // slot inside the XCD's (BH / 8) x nq units
    int j;                                 // head index inside the XCD
    if (LONGEST_FIRST) {
      const int level = slot / (BH >> 3);
      j = slot - level * (BH >> 3);
      qt = nq - 1 - level;
    } else {
      j = slot / nq;
      qt = nq - 1 - (slot - j * nq);
    }
    const int bkv = xcd + 8 * (j / p.ratio);
    bh = bkv * p.ratio + (j - (j / p.ratio) * p.ratio);
  } else if ((8 % (p.b * p.h_kv)) == 0 && ((int64_t)BH * nq) % 8 == 0) {
    // fewer than 8 kv heads: each gets 8 / (b * h_kv) XCDs of its own
    const int G = 8 / (p.b * p.h_kv);
    const int xcd = v & 7, slot = v >> 3;
    const int bkv = xcd / G;
    const int j = slot * G + (xcd - bkv * G);  // unit inside the kv head: ratio x nq of them
    const int lvl = j / p.ratio;
    bh = bkv * p.ratio + (j - lvl * p.ratio);
    qt = LONGEST_FIRST ? nq - 1 - lvl : lvl;
  } else if (LONGEST_FIRST) {
    const int level = v / BH;
    bh = v - level * BH;
    qt = nq - 1 - level;
  } else {
    bh = v / nq;
    qt = nq - 1 - (v - bh * nq);
  }
}

// One key chunk of a query tile whose key range is split (KSPLIT): the tile's
// visible key tiles [t_begin, t_end) are cut into chunks of `tiles` key tiles;
// chunk `index` is processed, and when the tile has more than one chunk the
// normalised partial O (bf16) and its natural-log LSE go to slot `part` of the
// partial buffers, to be merged by prefill_merge_kernel.
struct KeyChunk {
  int index, tiles;
  int64_t part;
  uint16_t *o_part;
  float *lse_part;
};

template <int D, int NW, int BN, bool CAUSAL, bool WINDOW, int DS, bool KSPLIT>
__device__ __forceinline__ void prefill_body(const PrefillParams &p, int bh, int qt, const KeyChunk &kc) {
  using T = Tile<D, NW, BN, DS>;
  constexpr int BM = T::BM;
  constexpr int SPLIT = T::SPLIT;
  constexpr int XBYTES = SPLIT > 1 ? NW * T::NKB * 16 * 64 * 4 : 0;  // partial-score exchange
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(2 * T::STAGE_BYTES + XBYTES) / 2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int w = wave / SPLIT;      // row block of this wave
  const int slice = wave % SPLIT;  // head-dim slice of this wave

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
  int t_begin = kbeg / BN;
  int t_end = kbeg < kend ? (kend + BN - 1) / BN : t_begin;
  bool partial = false;  // this chunk is one of several: write a partial result
  if constexpr (KSPLIT) {
    const int nt = t_end - t_begin;
    partial = nt > kc.tiles;
    t_begin += kc.index * kc.tiles;
    t_end = min(t_end, t_begin + kc.tiles);
  }

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
  if (p.sinks != nullptr && (!KSPLIT || kc.index == 0)) {  // the sink joins one chunk only
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
    // Head dim split over wave pairs, in two groups that take turns.  Waves
    // w and w + 4 share a SIMD; waves 0-3 (row blocks 0, 1) form group 0 and
    // waves 4-7 (row blocks 2, 3) group 1.  Two workgroup barriers per
    // iteration, A_i and X_i:
    //
    //   after A_i:  group 0: partial S(i) -> exchange   group 1: sum, softmax, P.V of tile i-1
    //   after X_i:  group 0: sum, softmax, P.V of i      group 1: partial S(i) -> exchange
    //
    // so on every SIMD one wave's softmax runs beside the other's score MMAs.
    // Tile i sits in stage (i - t_begin) mod 2 as [K][V].  V(i-1) is still
    // read in the first half of iteration i, so the loads go in two parts:
    // K(i+1) after A_i (K(i-1)'s slot, last read by group 1 before A_i) and
    // V(i+1) after X_i (V(i-1)'s slot, last read by group 1 before X_i).
    // Before A_i a wave needs its loads of K(i), and V(i), issued after them,
    // may stay in flight; before X_i it needs V(i), and K(i+1) may stay in
    // flight.  Each wave writes only its own exchange slots: group 0 writes
    // them after A_i and reads its pair's after X_i, group 1 writes after X_i
    // and reads after A_{i+1}.  Measured 125.5 -> 121.5 us on the causal
    // b1 h4 s4096 d512 workload against every wave running the same phase.
    static_assert(SPLIT == 2 && NW == 8, "two groups of two wave pairs");
    typename T::Lane ln;
    T::init_lane(ln, smem, p.k_ss, p.v_ss, wave, lane, slice);
    const int grp = wave >> 2;
    f32x4 *xb = reinterpret_cast<f32x4 *>(reinterpret_cast<char *>(smem) + 2 * T::STAGE_BYTES);
    auto stage = [&](int t) { return (t - t_begin) & 1; };
    auto score_half = [&](int t) {
      if (active(t)) {
        f32x16 s[T::NKB];
        T::scores(s, qreg, ln, stage(t) * T::STAGE_BYTES);
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {s[kb][4 * q4], s[kb][4 * q4 + 1], s[kb][4 * q4 + 2], s[kb][4 * q4 + 3]};
            xb[(wave * T::NKB * 4 + kb * 4 + q4) * 64 + lane] = v;
          }
      }
    };
    auto value_half = [&](int t) {
      if (active(t)) {
        // S = S_0 + S_1, in slice order in both waves of the pair (bit-identical scores)
        const int w0 = wave - slice;
        f32x16 s[T::NKB];
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = xb[(w0 * T::NKB * 4 + kb * 4 + q4) * 64 + lane] +
                            xb[((w0 + 1) * T::NKB * 4 + kb * 4 + q4) * 64 + lane];
            s[kb][4 * q4] = v[0];
            s[kb][4 * q4 + 1] = v[1];
            s[kb][4 * q4 + 2] = v[2];
            s[kb][4 * q4 + 3] = v[3];
          }
        mask(s, t);
        u32x4 pk[T::NPV];
        T::softmax_step(s, pk, o, m, l, p.c);
        T::values(o, pk, ln, stage(t) * T::STAGE_BYTES);
      }
    };
    if (t_begin < t_end) {
      T::dma_k(ln, smem, kbase, p.k_ss, t_begin * BN, p.s_k, wave);
      T::dma_v(ln, smem + T::TILE_ELEMS, vbase, p.v_ss, t_begin * BN, p.s_k, wave);
      // One loop per group (the group is fixed for the whole unit), each half
      // of an iteration straight-line: a branch between the two roles inside
      // one loop body made the compiler spill the Q operands.
      auto sync_a = [&](int i) {  // wait for K(i), barrier A_i, then load K(i+1)
        if (i < t_end)
          wait_vmcnt<T::LOADS>();  // V(i), issued after K(i), may be in flight
        else
          wait_vmcnt<0>();
        __syncthreads();
        if (i + 1 < t_end)
          T::dma_k(ln, smem + stage(i + 1) * (T::STAGE_BYTES / 2), kbase, p.k_ss, (i + 1) * BN, p.s_k, wave);
      };
      auto sync_x = [&](int i) {  // wait for V(i), barrier X_i, then load V(i+1)
        if (i + 1 < t_end)
          wait_vmcnt<T::LOADS>();  // K(i+1), issued after V(i), may be in flight
        else
          wait_vmcnt<0>();
        __syncthreads();
        if (i + 1 < t_end)
          T::dma_v(ln, smem + stage(i + 1) * (T::STAGE_BYTES / 2) + T::TILE_ELEMS, vbase, p.v_ss, (i + 1) * BN,
                   p.s_k, wave);
      };
      if (grp == 0) {
        for (int i = t_begin; i <= t_end; ++i) {
          sync_a(i);
          if (i < t_end) score_half(i);
          sync_x(i);
          if (i < t_end) value_half(i);
        }
      } else {
        for (int i = t_begin; i <= t_end; ++i) {
          sync_a(i);
          if (i > t_begin) value_half(i - 1);
          sync_x(i);
          if (i < t_end) score_half(i);
        }
      }
    }
  }

  // Epilogue: O / l once, bf16 round-to-nearest-even; LSE = ln2 * (m + log2 l).
  // A partial chunk writes the same two quantities into its slot instead.
  const float lt = sum_across_halves(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  // Staged: the output tile goes through the (now idle) K/V stages, and every
  // wave passes both barriers.
  const bool part_out = KSPLIT && partial;
  uint16_t *const dst = part_out ? kc.o_part + (kc.part * BM + (w_lo - q0)) * D + slice * DS
                                 : p.o + bi * p.o_sb + h * p.o_sh + (int64_t)w_lo * p.o_ss + slice * DS;
  const int64_t dst_rs = part_out ? (int64_t)D : p.o_ss;
  if constexpr (T::STAGED_OUT) {
    static_assert(NW * T::OUT_BYTES <= 2 * T::STAGE_BYTES, "staged output must fit in the K/V stages");
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the last stage
    char *xw = reinterpret_cast<char *>(smem) + wave * T::OUT_BYTES;
    T::stage_out(o, inv, xw, lane);
    __syncthreads();
    T::store_out(xw, lane, dst, dst_rs, max(0, min(32, p.s_q - w_lo)));
  } else if (row_ok) {
    T::store_direct(o, inv, dst + (row - w_lo) * dst_rs, lane);
  }
  if (part_out) {
    if (row_ok && hi == 0 && slice == 0)
      kc.lse_part[kc.part * BM + (row - q0)] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  } else if (p.lse != nullptr && row_ok && hi == 0 && slice == 0) {
    p.lse[bi * p.lse_sb + h * p.lse_sh + row] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, int NW, int BN, bool CAUSAL, bool WINDOW, int OCC, int DS = D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void prefill_kernel(PrefillParams p) {
  int bh, qt;
  prefill_unit<CAUSAL && !WINDOW>(p, blockIdx.x, bh, qt);
  prefill_body<D, NW, BN, CAUSAL, WINDOW, DS, false>(p, bh, qt, KeyChunk{});
}

// Causal prefill with the key ranges of long query tiles cut into chunks, so
// that the work units are of similar length when there are too few query
// tiles to keep the chip busy (the d = 512 shapes: 128-row tiles, one
// 8-wave workgroup per CU).  Unit v is (rank v / (b*h_q), head v % (b*h_q)); the rank
// table, built on the host, lists the (query tile, chunk) pairs longest first.
template <int D, int NW, int BN, int OCC, int DS = D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void prefill_chunked_kernel(PrefillParams p, PrefillChunks ck) {
  const int BH = p.b * p.h_q;
  const int rank = blockIdx.x / BH, bh = blockIdx.x - rank * BH;
  const uint32_t e = ck.rank[rank];
  const int qt = (int)(e >> 8), c = (int)(e & 255u);
  KeyChunk kc;
  kc.index = c;
  kc.tiles = ck.chunk_tiles;
  kc.part = qt >= ck.qt0 ? ((int64_t)bh * (p.n_qtiles - ck.qt0) + (qt - ck.qt0)) * ck.max_chunks + c : 0;
  kc.o_part = ck.o_part;
  kc.lse_part = ck.lse_part;
  prefill_body<D, NW, BN, true, false, DS, true>(p, bh, qt, kc);
}

// LSE merge of the chunk partials of the split query tiles (qt >= qt0): one
// thread per row and 8 output columns, parts merged as in the decode combine.
template <int D, int BM, int BN>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p, PrefillChunks ck) {
  constexpr int CPR = D / 8;
  const int nsq = p.n_qtiles - ck.qt0;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)p.b * p.h_q * nsq * BM * CPR) return;
  const int ch = (int)(gid % CPR);
  const int64_t rr = gid / CPR;
  const int r = (int)(rr % BM);
  const int64_t tq = rr / BM;  // bh * nsq + (qt - qt0)
  const int qt = ck.qt0 + (int)(tq % nsq);
  const int bh = (int)(tq / nsq);
  const int row = qt * BM + r;
  if (row >= p.s_q) return;
  // Chunks of this query tile (the kernel's own visible-range arithmetic).
  const int i_last = min(p.s_q, qt * BM + BM) - 1;
  const int kend = max(0, min(p.s_k, i_last + (p.s_k - p.s_q) + 1));
  const int nt = (kend + BN - 1) / BN;
  const int n = (nt + ck.chunk_tiles - 1) / ck.chunk_tiles;
  const int bi = bh / p.h_q, h = bh - bi * p.h_q;
  const int64_t part0 = tq * ck.max_chunks;
  merge_chunk<uint16_t, 16>(ck.lse_part + part0 * BM + r, BM, ck.o_part + (part0 * BM + r) * D + ch * 8,
                            (int64_t)BM * D, n, p.o + bi * p.o_sb + h * p.o_sh + (int64_t)row * p.o_ss + ch * 8,
                            p.lse != nullptr && ch == 0 ? p.lse + bi * p.lse_sb + h * p.lse_sh + row : nullptr);
}

// Ping-pong prefill (SPLIT == 1 head dims): 8 waves in two groups of 4 that
// share every staged K/V tile.  Waves w and w+4 run on the same SIMD, so the
// two groups can take turns: while one group runs its MMAs (the value MMA of
// the previous tile and the score MMA of the current one), the other runs the
// softmax of its current tile on the vector ALU.  Group 1 runs half an
// iteration behind group 0; one workgroup barrier A_i per iteration:
//
//   after A_i:  group 0: P(i-1).V(i-1), S(i) = K(i).Q   group 1: softmax(i-1)
//      then:    group 0: softmax(i)                     group 1: P(i-1).V(i-1), S(i)
//
// Each group goes from its first half to its second without a barrier: the
// halves keep their order because each half of one group is about as long
// as the other group's half that it overlaps, and no LDS access depends on
// the switch (below).  Row blocks are interleaved between the groups (group g
// owns blocks g, g+2, g+4, g+6 of the 256-row query tile) so that both see
// nearly the same causal and window extents.  A ring of STAGES LDS stages
// holds [K tile][V tile]; between A_i and A_{i+1} the waves read only the
// stages of tiles i-1 and i, and write (by DMA) only the stage of tile i-2,
// which takes tile i+STAGES-2 and whose last reads were consumed by MMAs
// before A_i.  Every wave's loads of tile i+1 are waited for before A_{i+1},
// so they have a full iteration or more to land.  The value operands of a tile are read ahead at
// the end of the softmax, so the MMA phase is mostly MMA issue.
struct NoUnitHook {
  __device__ void operator()() const {}
};
// on_loop_end() runs in every thread right after the tile loop, before the
// output epilogue (the work queue takes its next ticket there).
template <int D, int BN, bool CAUSAL, bool WINDOW, int STAGES, typename Hook = NoUnitHook>
__device__ __forceinline__ void pp_unit(const PrefillParams &p, int bh, int qt, Hook on_loop_end = Hook{}) {
  using T = Tile<D, 8, BN>;
  constexpr int BM = T::BM;
  static_assert(T::SPLIT == 1 && BM == 256 && STAGES >= 3, "ping-pong shape");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * T::STAGE_BYTES / 2];

  // In the work-queue loop the thread index is made opaque: the compiler would
  // otherwise hoist the per-lane address set-up of every unit out of the loop
  // and hold it in registers across the whole launch (spilling).
  int tid = threadIdx.x;
  if constexpr (!std::is_same<Hook, NoUnitHook>::value) asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int grp = wave >> 2;
  const int rb = 2 * (wave & 3) + grp;  // 32-row block of this wave inside the query tile

  const int bi = bh / p.h_q, h = bh - bi * p.h_q;
  const int g = h / p.ratio;
  const int q0 = qt * BM;
  const int off = p.s_k - p.s_q;

  const int i_last = min(p.s_q, q0 + BM) - 1;
  int kend = p.s_k;
  if (CAUSAL) kend = max(0, min(kend, i_last + off + 1));
  int kbeg = 0;
  if (WINDOW) kbeg = max(0, q0 + off - p.window + 1);
  const int t_begin = kbeg / BN;
  const int t_end = kbeg < kend ? (kend + BN - 1) / BN : t_begin;
  const int nt = t_end - t_begin;
  const int lim = min(p.s_k, t_end * BN);  // keys loaded: tiles at or past t_end stay empty

  const int w_lo = q0 + rb * 32;
  const int w_hi = min(w_lo + 31, p.s_q - 1);
  const int row = w_lo + (lane & 31);
  const bool row_ok = row < p.s_q;

  const uint16_t *kbase = p.k + bi * p.k_sb + g * p.k_sh;
  const uint16_t *vbase = p.v + bi * p.v_sb + g * p.v_sh;

  typename T::Lane ln;
  T::init_lane(ln, smem, p.k_ss, p.v_ss, wave, lane);
#pragma unroll
  for (int s = 0; s < STAGES - 2; ++s)
    T::dma(ln, smem + s * (T::STAGE_BYTES / 2), kbase, p.k_ss, vbase, p.v_ss, (t_begin + s) * BN, lim, wave);

  u32x4 qreg[T::NKK];
  {
    const uint16_t *qp = p.q + bi * p.q_sb + h * p.q_sh + (int64_t)min(row, p.s_q - 1) * p.q_ss + 8 * hi;
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

  f32x16 s[T::NKB];
  u32x4 pk[T::NPV];
  u32x2 vpre[2 * T::VG];  // value operands of unit 0, read ahead across the barrier
  // This wave's share of the loads of tile i+STAGES-2, into the stage of tile
  // i-2 (free once barrier A_i has passed), issued once per iteration: with
  // the fine schedule right after the last MMAs of the wave's MMA phase
  // (measured 3 % faster than at the start of the softmax phase, and than
  // between the first MMA groups, where the loads hold up the MMA issue);
  // otherwise at the start of the wave's softmax phase.  Before A_{i+1} a
  // wave has exactly one later tile in flight.
  auto load_ahead = [&](int i) {
    T::dma(ln, smem + ((i + STAGES - 2) % STAGES) * (T::STAGE_BYTES / 2), kbase, p.k_ss, vbase, p.v_ss,
           (t_begin + i + STAGES - 2) * BN, lim, wave);
  };
  constexpr bool DMA_IN_MMA = T::PV_S_FINE;
  // MMA phase of iteration i: value MMA of tile i-1 (its first operands are
  // already in flight) fused with the score MMA of tile i.  The wave raises
  // its issue priority so that the other group's softmax fills the gaps
  // between its MMAs rather than the other way round.
  auto mma_phase = [&](int i) {
    const bool pv = i > 0 && active(t_begin + i - 1);
    const bool sc = i < nt && active(t_begin + i);
    const uint32_t v_off = ((i + STAGES - 1) % STAGES) * T::STAGE_BYTES;
    const uint32_t k_off = (i % STAGES) * T::STAGE_BYTES;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (T::PV_S_FUSED) {
      if (pv && sc) {
        if constexpr (T::PV_S_FINE)
          T::pv_scores_fine(o, pk, s, qreg, vpre, ln, v_off, k_off,
                            typename T::template DmaHook<15, 15>{
                                ln, smem + ((i + STAGES - 2) % STAGES) * (T::STAGE_BYTES / 2), kbase, vbase,
                                p.k_ss, p.v_ss, (t_begin + i + STAGES - 2) * BN, lim, wave});
        else
          T::pv_scores(o, pk, s, qreg, vpre, ln, v_off, k_off);
      } else {
        if (DMA_IN_MMA) load_ahead(i);
        if (pv) T::values_from(o, pk, vpre, ln, v_off);
        else if (sc) T::scores(s, qreg, ln, k_off);
      }
    } else {  // registers are short (d = 256): no operands read ahead
      if (pv) T::values(o, pk, ln, v_off);
      if (sc) T::scores(s, qreg, ln, k_off);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Softmax of tile i, which ends by reading the first value operands of
  // tile i for the next MMA phase.
  auto softmax_phase = [&](int i) {
    if (i >= 0 && active(t_begin + i)) {
      mask(s, t_begin + i);
      T::template softmax_step<true>(s, pk, o, m, l, p.c);
      if constexpr (T::PV_S_FUSED) T::values_issue0(vpre, ln, (i % STAGES) * T::STAGE_BYTES);
    }
  };

  if (nt > 0) {
    for (int i = 0; i <= nt; ++i) {
      wait_vmcnt<(STAGES - 3) * 2 * T::LOADS>();  // this wave's loads of tile i have landed
      barrier_nofence();                           // A_i: tile i published, tile i-2's stage free
      if (grp == 0) {
        mma_phase(i);
        if (!DMA_IN_MMA) load_ahead(i);
        if (i < nt) softmax_phase(i);
      } else {
        if (!DMA_IN_MMA) load_ahead(i);
        if (i > 0) softmax_phase(i - 1);
        mma_phase(i);
      }
    }
  }
  wait_vmcnt<0>();  // every load into the ring (empty tiles included) has landed
  on_loop_end();

  const float lt = sum_across_halves(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  // Staged: the output tile goes through the idle ring, and every wave passes
  // both barriers.
  uint16_t *const dst = p.o + bi * p.o_sb + h * p.o_sh + (int64_t)w_lo * p.o_ss;
  if constexpr (T::STAGED_OUT) {
    static_assert(8 * T::OUT_BYTES <= STAGES * T::STAGE_BYTES, "staged output must fit in the ring");
    __syncthreads();  // every wave is done with the ring
    char *xw = reinterpret_cast<char *>(smem) + wave * T::OUT_BYTES;
    T::stage_out(o, inv, xw, lane);
    __syncthreads();
    T::store_out(xw, lane, dst, p.o_ss, max(0, min(32, p.s_q - w_lo)));
  } else if (row_ok) {
    T::store_direct(o, inv, dst + (int64_t)(row - w_lo) * p.o_ss, lane);
  }
  if (p.lse != nullptr && row_ok && hi == 0)
    p.lse[bi * p.lse_sb + h * p.lse_sh + row] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : kNegInf;
}

template <int D, int BN, bool CAUSAL, bool WINDOW, int STAGES>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_pp_kernel(PrefillParams p) {
  int bh, qt;
  prefill_unit<CAUSAL && !WINDOW>(p, blockIdx.x, bh, qt);
  pp_unit<D, BN, CAUSAL, WINDOW, STAGES>(p, bh, qt);
}

// Work-queue form of the ping-pong prefill.  The grid has one workgroup per
// compute unit.  The units are those of the fixed placement (unit v belongs to
// XCD v % 8, which keeps a kv head's query tiles on one XCD and its K/V in one
// L2; prefill_unit), held in one double-ended queue per XCD in the same order
// (longest first under a plain causal mask): queue x holds units x, x + 8,
// x + 16, ...  A workgroup takes units from the front of the queue of the XCD
// it runs on (read from the XCC_ID hardware register); once that is empty it
// takes from the back of the others, i.e. their shortest units, so when the
// XCDs of a chip settle at different clocks the fast ones finish the slow
// ones' last tiles instead of waiting for them, without taking the long units
// the owners would run next.  Each queue is one 64-bit word, front count in
// the low half and back count in the high half: a claim is valid when
// front + back was below the queue's size at its atomic, so front and back
// claims never overlap.  Claims are returning atomics, so a workgroup
// increments the exit counter only after its last claim has been counted; the
// workgroup that exits last therefore sees no claim after it and resets every
// counter to zero for the next launch.  queue must be zero before the first
// launch, and launches sharing a queue must not overlap.
constexpr int kQueueXcds = 8;
constexpr int kQueueExit = 32;                 // uint32 index of the exit counter (after 8 x 16 bytes)
constexpr uint32_t kQueueDone = 0xffffffffu;  // no unit left in any queue
constexpr uint32_t kQueueRetry = 0xfffffffeu; // none taken: look again (from the other queues)
template <int D, int BN, bool CAUSAL, bool WINDOW, int STAGES>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_pp_queue_kernel(PrefillParams p, uint32_t *queue) {
  __shared__ uint32_t s_unit;
  unsigned long long *q64 = reinterpret_cast<unsigned long long *>(queue);  // queue x at q64[2x]
  const uint32_t n_units = (uint32_t)(p.b * p.h_q * p.n_qtiles);
  const int home = __builtin_amdgcn_s_getreg((31 << 11) | 20) & (kQueueXcds - 1);  // XCC_ID
  auto qsize = [&](int x) -> uint32_t { return n_units > (uint32_t)x ? (n_units - 1 - x) / kQueueXcds + 1 : 0; };
  bool stealing = false;  // the home queue is empty
  // Thread 0 only: the next unit, kQueueRetry when none has been taken yet.
  uint32_t ahead = kQueueRetry;
  auto home_ticket = [&]() -> uint32_t {
    const unsigned long long w = atomicAdd(q64 + 2 * home, 1ull);
    const uint32_t f = (uint32_t)w, b = (uint32_t)(w >> 32);
    return (uint64_t)f + b < qsize(home) ? (uint32_t)home + kQueueXcds * f : kQueueRetry;
  };
  // The back (shortest) unit of another queue that still has some (all eight
  // words read in one round trip; a queue that looks empty is not touched);
  // kQueueRetry after a lost race, kQueueDone when every queue is empty.
  auto steal_ticket = [&]() -> uint32_t {
    unsigned long long c[kQueueXcds];
#pragma unroll
    for (int j = 0; j < kQueueXcds; ++j)
      c[j] = __hip_atomic_load(q64 + 2 * j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int x = -1;
#pragma unroll
    for (int j = 1; j <= kQueueXcds; ++j) {
      const int y = (home + j) & (kQueueXcds - 1);
      if (x < 0 && (uint64_t)(uint32_t)c[y] + (uint32_t)(c[y] >> 32) < qsize(y)) x = y;
    }
    if (x < 0) return kQueueDone;
    const unsigned long long w = atomicAdd(q64 + 2 * x, 1ull << 32);
    const uint32_t f = (uint32_t)w, b = (uint32_t)(w >> 32);
    const uint32_t size = qsize(x);
    return (uint64_t)f + b < size ? (uint32_t)x + kQueueXcds * (size - 1 - b) : kQueueRetry;
  };
  for (;;) {
    if (threadIdx.x == 0) s_unit = ahead != kQueueRetry ? ahead : stealing ? steal_ticket() : home_ticket();
    __syncthreads();
    const uint32_t u = s_unit;
    __syncthreads();  // every wave has read the unit before thread 0 takes the next
    if (u == kQueueDone) break;
    if (u == kQueueRetry) {  // the home queue is empty, or a steal lost its race
      stealing = true;
      continue;
    }
    ahead = kQueueRetry;
    int bh, qt;
    prefill_unit<CAUSAL && !WINDOW>(p, (int)u, bh, qt);
    // The home queue's next unit is claimed when this unit's tile loop ends,
    // so the atomic's round trip overlaps the output epilogue (its wait would
    // otherwise also wait for the epilogue's stores).
    pp_unit<D, BN, CAUSAL, WINDOW, STAGES>(p, bh, qt, [&] {
      if (threadIdx.x == 0 && !stealing) ahead = home_ticket();
    });
    __syncthreads();  // the LDS ring is free before the next tile's loads
  }
  if (threadIdx.x == 0 && atomicAdd(queue + kQueueExit, 1u) == gridDim.x - 1) {
    for (int x = 0; x < kQueueXcds; ++x) atomicExch(q64 + 2 * x, 0ull);
    atomicExch(queue + kQueueExit, 0u);
  }
}

template <int D, int BN, bool CAUSAL, bool WINDOW, int STAGES>
hipError_t launch_prefill_pp(const PrefillParams &p, int n_units, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_pp_kernel<D, BN, CAUSAL, WINDOW, STAGES>), dim3(n_units), dim3(512), 0, stream, p);
  return hipGetLastError();
}

// n_wg: workgroups of the grid (one per compute unit); queue: two zeroed uint32.
template <int D, int BN, bool CAUSAL, bool WINDOW, int STAGES>
hipError_t launch_prefill_pp_queue(const PrefillParams &p, int n_units, int n_wg, uint32_t *queue,
                                   hipStream_t stream) {
  const int grid = n_units < n_wg ? n_units : n_wg;
  hipLaunchKernelGGL((prefill_pp_queue_kernel<D, BN, CAUSAL, WINDOW, STAGES>), dim3(grid), dim3(512), 0, stream, p,
                     queue);
  return hipGetLastError();
}

// Host-side launcher of one instantiation.
template <int D, int NW, int BN, bool CAUSAL, bool WINDOW, int OCC, int DS = D>
hipError_t launch_prefill(const PrefillParams &p, int n_units, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, NW, BN, CAUSAL, WINDOW, OCC, DS>), dim3(n_units), dim3(NW * 64),
                     0, stream, p);
  return hipGetLastError();
}

// Host-side launcher of the chunked causal prefill and its merge.
template <int D, int NW, int BN, int OCC, int DS = D>
hipError_t launch_prefill_chunked(const PrefillParams &p, const PrefillChunks &ck, hipStream_t stream) {
  using T = Tile<D, NW, BN, DS>;
  const int64_t units = (int64_t)ck.n_rank * p.b * p.h_q;
  hipLaunchKernelGGL((prefill_chunked_kernel<D, NW, BN, OCC, DS>), dim3((unsigned)units), dim3(NW * 64), 0,
                     stream, p, ck);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)p.b * p.h_q * (p.n_qtiles - ck.qt0) * T::BM * (D / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_merge_kernel<D, T::BM, BN>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, p, ck);
  return hipGetLastError();
}

}  // namespace attn

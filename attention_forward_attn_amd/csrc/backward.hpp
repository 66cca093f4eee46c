// Attention backward at head dims 64, 128 and 256: dQ, dK, dV for an incoming dO, from the
// forward's O and LSE, under no mask, a causal mask or a causal sliding window,
// deterministic (no atomics).  A sink only enters through the forward's LSE
// (P = exp(scale*S - LSE) already carries its share of the normalisation), so
// dQ, dK and dV need nothing more; the sink logit's own gradient,
// d sigma_h = -sum_{b,i} exp(sigma_h - LSE_i) D_i, is summed per query tile by
// the dQ kernel and over the tiles and the batch, in a fixed order, by a small
// third kernel.
//
// Two kernels, both built from the forward's tile engine:
//   * dQ (one workgroup per NW x 32 query rows, NW waves x 32 rows): the forward
//     layout S^T = K.Q^T (rows in lanes, keys in registers), plus
//     dP^T = V.dO^T, then dQ^T += K^T.dS^T with dS = P * (dP - D).  It also
//     writes D_i = sum_t dO[i,t] O[i,t] and the row's LSE in base 2 (+inf
//     for a row with no key, so that P = exp2(S*c - L) needs no test) for
//     the second kernel.  Tiles whose keys every row of a wave sees skip the
//     per-key mask in both kernels.
//   * dK/dV (one workgroup per NW x 32 keys of one kv head, NW waves x 32 keys):
//     the same shapes with the roles of queries and keys swapped: S = Q.K^T
//     and dP = dO.V^T with keys in lanes and query rows in registers, then
//     dV^T += dO^T.P and dK^T += Q^T.dS, summed over every query head of the
//     kv group (a workgroup owns its keys, so no atomics are needed).
// A streamed tile is needed both row-wise (score-like MMA, A operand from
// 16-byte row segments) and transposed (value-like MMA, transpose reads); the
// tile engine's shared swizzle serves both read patterns without bank
// conflicts, so each tile is staged once.
#pragma once

#include "tile.hpp"

namespace attn {

// Packs eight f32 values of accumulator block (T>>1), registers 8(T&1)..+7,
// into the bf16 operand of value-MMA k-step T (the order softmax_exp uses).
template <int NKB, int NPV>
__device__ __forceinline__ void pack_operand(const f32x16 (&x)[NKB], u32x4 (&pk)[NPV]) {
#pragma unroll
  for (int t = 0; t < NPV; ++t) {
    const int kb = t >> 1, r0 = (t & 1) * 8;
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(x[kb][r0 + 2 * q], x[kb][r0 + 2 * q + 1]);
    pk[t] = v;
  }
}

// Loads the 32 x D bf16 block of rows r0.. (row stride rs) as the B operand
// of the score MMA (lane: row r0 + lane%32, 8 columns per k-step); rows past
// n_rows read row n_rows-1 (their results are never used).
template <int NKK>
__device__ __forceinline__ void load_b_rows(u32x4 (&reg)[NKK], const uint16_t *base, int64_t rs, int r,
                                            int n_rows, int hi) {
  const uint16_t *pr = base + (int64_t)min(r, n_rows - 1) * rs + 8 * hi;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) reg[kk] = *reinterpret_cast<const u32x4 *>(pr + kk * 16);
}

// N 16-byte LDS reads at addr + 32*I (I = 0..N-1) into f32x4 values.
template <int I, int N>
__device__ __forceinline__ void lds_row4(f32x4 (&v)[N], uint32_t addr) {
  v[I] = __builtin_bit_cast(f32x4, ds_read_b128<32 * I>(addr));
  if constexpr (I + 1 < N) lds_row4<I + 1>(v, addr);
}

// Hooks that run element-wise work between the MMAs of a score product
// (step<KK>, after k-step KK) or of a value product (vstep<T>, after k-step
// T): that vector work then executes while the MMAs just issued are in
// flight.  G groups of work are spread evenly over the N steps: step K runs
// groups ceil(K G / N) .. ceil((K+1) G / N) - 1 (G / N each when N divides G,
// one every N / G steps when G divides N).
template <int G, int N, typename F>
struct GroupHook {
  F &f;
  template <int K>
  __device__ __forceinline__ void run() {
    constexpr int lo = (K * G + N - 1) / N, hi = ((K + 1) * G + N - 1) / N;
#pragma unroll
    for (int g = lo; g < hi; ++g) f(g);
  }
  template <int KK>
  __device__ __forceinline__ void step() { run<KK>(); }
  template <int T_>
  __device__ __forceinline__ void vstep() { run<T_>(); }
};

// Wait before consuming tile n of a ring of NS stages, whose loads run NS - 1
// tiles ahead (LPT loads per tile issued by this wave): when the NS - 2 tiles
// after n are all in flight, only n's own loads need to have landed; near the
// end, with fewer in flight, everything is waited for.
template <int NS, int LPT>
__device__ __forceinline__ void ring_wait(bool later_in_flight) {
  if constexpr (NS <= 2) {
    wait_vmcnt<0>();
  } else {
    if (later_in_flight)
      wait_vmcnt<(NS - 2) * LPT>();
    else
      wait_vmcnt<0>();
  }
}

// Stores a transposed accumulator (lane = row, registers = head-dim columns)
// times f as bf16 rows.
template <int NDB>
__device__ __forceinline__ void store_rows(uint16_t *op, const f32x16 (&a)[NDB], float f) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      u32x2 val;
      val[0] = pack_bf16x2(a[db][4 * gi + 0] * f, a[db][4 * gi + 1] * f);
      val[1] = pack_bf16x2(a[db][4 * gi + 2] * f, a[db][4 * gi + 3] * f);
      *reinterpret_cast<u32x2 *>(op + db * 32 + 8 * gi) = val;
    }
}

// ---------------------------------------------------------------------------
// dQ (and D).  NS: stages of the K/V ring.
// With one wave per SIMD (NW = 4) P is computed between the dP MMAs; with two
// the other wave hides the exponentials and the hook measured slower.
template <int NW>
constexpr bool kDqPHook = NW == 4;
template <int D, int BN, bool CAUSAL, bool WINDOW, int NW, int NS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void bwd_dq_kernel(BwdParams p) {
  using T = Tile<D, NW, BN, D, true>;
  constexpr int BM = 32 * NW;
  constexpr int STAGE = 2 * T::TILE_BYTES;  // [K][V]
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE / 2];
  __shared__ float s_red[NW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int n_qt = (p.s_q + BM - 1) / BM;
  // Under a causal mask later query tiles see more keys: hand them out first.
  const int nbh = p.b * p.h_q;
  const int lvl = blockIdx.x / nbh, bh = blockIdx.x - lvl * nbh;
  const int qt = CAUSAL ? n_qt - 1 - lvl : lvl;
  const int bi = bh / p.h_q, h = bh - bi * p.h_q;
  const int g = h / p.ratio;
  const int q0 = qt * BM;
  const int off = p.s_k - p.s_q;
  const int i_last = min(p.s_q, q0 + BM) - 1;
  const int kend = CAUSAL ? max(0, min(p.s_k, i_last + off + 1)) : p.s_k;
  const int n_tiles = (kend + BN - 1) / BN;
  // A window: the first key any row of the tile sees.
  const int t0 = WINDOW ? min(n_tiles, max(0, q0 + off - p.window + 1) / BN) : 0;

  const int w_lo = q0 + wave * 32;
  const int w_hi = min(w_lo + 31, p.s_q - 1);
  const int row = w_lo + lr;
  const bool row_ok = row < p.s_q;

  const uint16_t *kbase = p.k + bi * p.k_sb + g * p.k_sh;
  const uint16_t *vbase = p.v + bi * p.k_sb + g * p.k_sh;
  const int64_t qrow0 = bi * p.q_sb + h * p.q_sh;  // q, o, do, dq share the row layout

  u32x4 qreg[T::NKK], dreg[T::NKK];
  load_b_rows(qreg, p.q + qrow0, p.q_ss, row, p.s_q, hi);
  load_b_rows(dreg, p.d_o + qrow0, p.q_ss, row, p.s_q, hi);
  // D = rowsum(dO * O) over this lane's half of the columns, then both halves.
  float dsum = 0.0f;
  {
    u32x4 oreg[T::NKK];
    load_b_rows(oreg, p.o + qrow0, p.q_ss, row, p.s_q, hi);
#pragma unroll
    for (int kk = 0; kk < T::NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = oreg[kk][e], b = dreg[kk][e];
        dsum = fmaf(__uint_as_float(a << 16), __uint_as_float(b << 16), dsum);
        dsum = fmaf(__uint_as_float(a & 0xffff0000u), __uint_as_float(b & 0xffff0000u), dsum);
      }
  }
  const float dd = sum_across_halves(dsum);
  const float lse = row_ok ? p.lse[bi * p.lse_sb + h * p.lse_sh + row] : kNegInf;
  // A row that saw no key has P = 0: exp2(s*c - inf) = 0.
  const float lse2 = lse == kNegInf ? -kNegInf : lse * kLog2e;
  if (row_ok && hi == 0) {
    p.dsum[(bi * p.h_q + h) * (int64_t)p.s_q + row] = dd;
    p.lse2[(bi * p.h_q + h) * (int64_t)p.s_q + row] = lse2;
  }

  f32x16 acc[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};

  typename T::Lane ln;
  T::init_dma(ln, p.k_ss, p.k_ss, wave, lane);  // K and V share the row stride (checked on the host)
  const uint32_t base = lds_offset(smem);
  T::init_mma(ln, base, base, lane);  // K read row-wise and transposed from one copy
  auto load = [&](int buf, int t) {
    uint16_t *st = smem + buf * (STAGE / 2);
    T::dma1(ln, false, st, kbase, p.k_ss, t * BN, p.s_k, wave);
    T::dma1(ln, false, st + T::TILE_ELEMS, vbase, p.k_ss, t * BN, p.s_k, wave);
  };
#pragma unroll
  for (int k = 0; k < NS - 1; ++k)
    if (t0 + k < n_tiles) load(k, t0 + k);
  int cur = 0;  // stage of tile t
  for (int t = t0; t < n_tiles; ++t, cur = cur + 1 == NS ? 0 : cur + 1) {
    ring_wait<NS, 2 * T::LOADS>(t + NS - 2 < n_tiles);
    __syncthreads();  // also: every wave is done with tile t - 1, whose stage is refilled next
    if (t + NS - 1 < n_tiles) load(cur == 0 ? NS - 1 : cur - 1, t + NS - 1);
    const int j0 = t * BN;
    if (w_lo < p.s_q && (!CAUSAL || j0 <= w_hi + off) &&
        (!WINDOW || j0 + BN - 1 >= w_lo + off - p.window + 1)) {
      const uint32_t so = cur * STAGE;
      f32x16 s[T::NKB], dp[T::NKB];
      T::scores(s, qreg, ln, so);
      // Every key of the tile visible to every row of the wave: no per-key test.
      const bool full = j0 + BN <= p.s_k && (!CAUSAL || j0 + BN - 1 <= w_lo + off) &&
                        (!WINDOW || j0 >= w_hi + off - p.window + 1);
      if constexpr (kDqPHook<NW>) {
        // P = exp(scale*S - LSE) in groups of four between the MMAs of dP (a
        // lone wave per SIMD has no other wave to hide its exponentials behind),
        // then dS = P * (dP - D).
        const int lim = CAUSAL ? min(row + off, p.s_k - 1) : p.s_k - 1;
        const int lo = WINDOW ? row + off - p.window + 1 : 0;
        // Full tiles and masked tiles run separate copies of the dP product
        // (a per-group branch inside one hook makes the compiler merge both
        // versions of every group with register copies).
        auto p_full = [&](int gi) {
          const int kb = gi >> 2, q4 = gi & 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][4 * q4 + e] = fast_exp2(fmaf(s[kb][4 * q4 + e], p.c, -lse2));
        };
        auto p_masked = [&](int gi) {
          const int kb = gi >> 2, q4 = gi & 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            const float pv = fast_exp2(fmaf(s[kb][i], p.c, -lse2));
            const int j = j0 + T::key_of(kb, i, hi);
            s[kb][i] = (j > lim || j < lo) ? 0.0f : pv;
          }
        };
        if (full) {
          GroupHook<4 * T::NKB, T::NKK, decltype(p_full)> hp{p_full};
          T::scores(dp, dreg, ln, so + T::TILE_BYTES, hp);
        } else {
          GroupHook<4 * T::NKB, T::NKK, decltype(p_masked)> hp{p_masked};
          T::scores(dp, dreg, ln, so + T::TILE_BYTES, hp);
        }
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] *= dp[kb][i] - dd;
      } else {
        T::scores(dp, dreg, ln, so + T::TILE_BYTES);
        if (full) {
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], p.c, -lse2)) * (dp[kb][i] - dd);
        } else {
          const int lim = CAUSAL ? min(row + off, p.s_k - 1) : p.s_k - 1;
          const int lo = WINDOW ? row + off - p.window + 1 : 0;
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = j0 + T::key_of(kb, i, hi);
              const float pv = (j > lim || j < lo) ? 0.0f : fast_exp2(fmaf(s[kb][i], p.c, -lse2));
              s[kb][i] = pv * (dp[kb][i] - dd);  // dS
            }
        }
      }
      u32x4 pk[T::NPV];
      pack_operand(s, pk);
      T::values(acc, pk, ln, so);  // dQ^T += K^T . dS^T (K read transposed)
    }
  }
  if (row_ok) store_rows(p.dq + qrow0 + (int64_t)row * p.q_ss + 4 * hi, acc, p.scale);
  if (p.dsink_part != nullptr) {
    // this tile's share of d sigma_h: -sum over its rows of exp(sigma_h - LSE_i) D_i
    float cs = (row_ok && hi == 0 && lse != kNegInf) ? -__expf(p.sinks[h] - lse) * dd : 0.0f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
    if (lane == 0) s_red[wave] = cs;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += s_red[w];
      p.dsink_part[(int64_t)bh * n_qt + qt] = tot;
    }
  }
}

// d sigma_h = sum over the batch and the query tiles of the dQ kernel's
// partials, in a fixed order (one thread per query head).
__global__ __launch_bounds__(256) void bwd_dsink_kernel(BwdParams p, int n_qt) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= p.h_q) return;
  float tot = 0.0f;
  for (int bi = 0; bi < p.b; ++bi)
    for (int qt = 0; qt < n_qt; ++qt) tot += p.dsink_part[((int64_t)bi * p.h_q + h) * n_qt + qt];
  p.d_sinks[h] = tot;
}

// ---------------------------------------------------------------------------
// dK, dV.  Reads D written by bwd_dq_kernel.  NS: stages of the Q/dO ring.
template <int D, int BN, bool CAUSAL, bool WINDOW, int NW, int NS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void bwd_dkdv_kernel(BwdParams p) {
  using T = Tile<D, NW, BN, D, true>;  // here the streamed "keys" of the engine are query rows
  constexpr int BK = 32 * NW;  // keys per workgroup
  // [Q][dO][LSE of the BN rows][D of the BN rows]
  constexpr int STAGE = 2 * T::TILE_BYTES + 2 * BN * 4;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE / 2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const int n_kt = (p.s_k + BK - 1) / BK;
  // Under a causal mask earlier key blocks are seen by more rows: hand them out first.
  const int nbg = p.b * p.h_kv;
  const int kt = blockIdx.x / nbg, bg = blockIdx.x - kt * nbg;
  const int bi = bg / p.h_kv, g = bg - bi * p.h_kv;
  const int off = p.s_k - p.s_q;
  const int w_key0 = kt * BK + wave * 32;
  const int key = w_key0 + lr;
  const bool key_ok = key < p.s_k;

  const int64_t krow0 = bi * p.k_sb + g * p.k_sh;  // k, v, dk, dv share the row layout
  u32x4 kreg[T::NKK], vreg[T::NKK];
  load_b_rows(kreg, p.k + krow0, p.k_ss, key, p.s_k, hi);
  load_b_rows(vreg, p.v + krow0, p.k_ss, key, p.s_k, hi);

  f32x16 dk[T::NDB], dv[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dk[db] = dv[db] = f32x16{};

  // Query rows that see any key of this workgroup: i + off >= first key.
  const int r_begin = CAUSAL ? max(0, kt * BK - off) : 0;
  // A window: rows past k1 - off + W - 1 (k1 the workgroup's last key) see none of its keys.
  const int r_end = WINDOW ? max(0, min(p.s_q, kt * BK + BK - 1 - off + p.window)) : p.s_q;
  const int t_begin = r_begin / BN;
  const int t_end = (r_end + BN - 1) / BN;
  const int n_tiles = t_begin < t_end ? t_end - t_begin : 0;

  typename T::Lane ln;
  T::init_dma(ln, p.q_ss, p.q_ss, wave, lane);  // Q and dO share the row stride (checked on the host)
  const uint32_t base = lds_offset(smem);
  T::init_mma(ln, base, base, lane);  // each tile read row-wise and transposed from one copy

  for (int h = g * p.ratio; h < (g + 1) * p.ratio; ++h) {
    const int64_t qrow0 = bi * p.q_sb + h * p.q_sh;
    const uint16_t *qbase = p.q + qrow0, *dobase = p.d_o + qrow0;
    const float *lse_h = p.lse2 + (bi * p.h_q + h) * (int64_t)p.s_q;  // LSE * log2(e), +inf for no key
    const float *d_h = p.dsum + (bi * p.h_q + h) * (int64_t)p.s_q;
    auto load = [&](int buf, int t) {
      uint16_t *st = smem + buf * (STAGE / 2);
      T::dma1(ln, false, st, qbase, p.q_ss, t * BN, p.s_q, wave);
      T::dma1(ln, false, st + T::TILE_ELEMS, dobase, p.q_ss, t * BN, p.s_q, wave);
      // LSE and D of the tile's rows, 4 bytes per lane; rows past s_q read as
      // zero.  A direct-to-LDS load writes at lane * 4 for every active lane,
      // so with tiles shorter than a wave only the first BN lanes take part.
      static_assert(BN <= 64, "one LSE and one D load per tile");
      if (wave == 0 && lane < BN) {
        const int r0 = t * BN, nr = max(0, min(BN, p.s_q - r0));
        uint16_t *aux = st + 2 * T::TILE_ELEMS;
        const uint32_t bytes = (uint32_t)(nr * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(nr > 0 ? lse_h + r0 : lse_h, bytes), (lds_void *)aux, 4,
                                                 lane * 4, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(nr > 0 ? d_h + r0 : d_h, bytes),
                                                 (lds_void *)(aux + 2 * BN), 4, lane * 4, 0, 0, 0);
      }
    };
    __syncthreads();  // the previous head's last tile is consumed
#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
      if (k < n_tiles) load(k, t_begin + k);
    int cur = 0;  // stage of tile n
    for (int n = 0; n < n_tiles; ++n, cur = cur + 1 == NS ? 0 : cur + 1) {
      const int t = t_begin + n;
      // wave 0 also loads the tile's LSE and D
      if (wave == 0)
        ring_wait<NS, 2 * T::LOADS + 2>(n + NS - 2 < n_tiles);
      else
        ring_wait<NS, 2 * T::LOADS>(n + NS - 2 < n_tiles);
      __syncthreads();  // also: every wave is done with tile n - 1, whose stage is refilled next
      if (n + NS - 1 < n_tiles) load(cur == 0 ? NS - 1 : cur - 1, t + NS - 1);
      const int i0 = t * BN;
      // this wave has keys, and (causal) the tile's last row reaches its first key
      if (w_key0 < p.s_k && (!CAUSAL || min(i0 + BN, p.s_q) - 1 + off >= w_key0) &&
          (!WINDOW || i0 <= min(w_key0 + 31, p.s_k - 1) - off + p.window - 1)) {
        {
          const uint32_t so = cur * STAGE;
          // LSE and D of the rows this lane's registers hold (4 consecutive
          // rows per read; index 4rb + q4: rows 32rb + 8q4 + 4hi .. +3), read
          // first: LDS reads complete in order, so they have landed once the
          // score product's own operand waits have passed.
          const uint32_t aux = base + so + 2 * T::TILE_BYTES + (4 * hi) * 4;
          f32x4 lv[4 * T::NKB], dv4[4 * T::NKB];
          lds_row4<0>(lv, aux);
          lds_row4<0>(dv4, aux + BN * 4);
          f32x16 s[T::NKB], dp[T::NKB];
          T::scores(s, kreg, ln, so);  // S = Q.K^T: rows in registers, keys in lanes
          tie8(lv, 4 * T::NKB);        // behind the last operand wait of the product above
          tie8(dv4, 4 * T::NKB);
          // Group g = 4rb + q4 of a lane's values: rows i0 + 32rb + 8q4 + 4hi + e
          // in registers 4q4 + e of block rb.
          auto visible = [&](int r) {
            return r < p.s_q && key_ok && (!CAUSAL || key <= r + off) && (!WINDOW || key >= r + off - p.window + 1);
          };
          // Every row of the tile sees every key of the wave: no per-pair test.
          const bool full = i0 + BN <= p.s_q && w_key0 + 32 <= p.s_k && (!CAUSAL || w_key0 + 31 <= i0 + off) &&
                            (!WINDOW || w_key0 >= i0 + BN - 1 + off - p.window + 1);
          // P = exp(scale*S - LSE), into s: over every pair (p_full), or
          // over the visible pairs only (p_masked).  The two run in separate
          // copies of the dP product: one hook that branched per group made
          // the compiler merge both versions of every group with register
          // copies (64 per tile).
          auto p_full = [&](int g) {
            const int rb = g >> 2, q4 = g & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) s[rb][4 * q4 + e] = fast_exp2(fmaf(s[rb][4 * q4 + e], p.c, -lv[g][e]));
          };
          auto p_masked = [&](int g) {
            const int rb = g >> 2, q4 = g & 3, r4 = i0 + 32 * rb + 8 * q4 + 4 * hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = fast_exp2(fmaf(s[rb][4 * q4 + e], p.c, -lv[g][e]));
              s[rb][4 * q4 + e] = visible(r4 + e) ? pv : 0.0f;
            }
          };
          auto ds_group = [&](int g) {  // dS = P * (dP - D), into dp
            const int rb = g >> 2, q4 = g & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[rb][4 * q4 + e] = s[rb][4 * q4 + e] * (dp[rb][4 * q4 + e] - dv4[g][e]);
          };
          // dP = dO.V^T, with P computed between its MMAs
          if (full) {
            GroupHook<4 * T::NKB, T::NKK, decltype(p_full)> hp{p_full};
            T::scores(dp, vreg, ln, so + T::TILE_BYTES, hp);
          } else {
            GroupHook<4 * T::NKB, T::NKK, decltype(p_masked)> hp{p_masked};
            T::scores(dp, vreg, ln, so + T::TILE_BYTES, hp);
          }
          u32x4 pp[T::NPV], pd[T::NPV];
          pack_operand(s, pp);
          // dV^T += dO^T . P, with dS computed between its MMAs
          GroupHook<4 * T::NKB, T::NPV, decltype(ds_group)> hd{ds_group};
          T::values(dv, pp, ln, so + T::TILE_BYTES, hd);
          pack_operand(dp, pd);
          T::values(dk, pd, ln, so);  // dK^T += Q^T . dS
        }
      }
    }
  }
  if (key_ok) {
    store_rows(p.dk + krow0 + (int64_t)key * p.k_ss + 4 * hi, dk, p.scale);
    store_rows(p.dv + krow0 + (int64_t)key * p.k_ss + 4 * hi, dv, 1.0f);
  }
}

// NWQ waves per dQ workgroup (NWQ x 32 query rows), NWK per dK/dV workgroup
// (NWK x 32 keys); NSQ and NSK stages in their rings; BNQ keys per dQ tile,
// BN query rows per dK/dV tile.
template <int D, int BN, bool CAUSAL, bool WINDOW, int NWQ, int NWK, int NSQ, int NSK, int BNQ = BN>
hipError_t launch_backward(const BwdParams &p, hipStream_t stream) {
  const int n_qt = (p.s_q + 32 * NWQ - 1) / (32 * NWQ), n_kt = (p.s_k + 32 * NWK - 1) / (32 * NWK);
  if (n_qt > 0) {  // dQ (zero when there are no keys), D and the sink partials
    hipLaunchKernelGGL((bwd_dq_kernel<D, BNQ, CAUSAL, WINDOW, NWQ, NSQ>), dim3(p.b * p.h_q * n_qt), dim3(NWQ * 64), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.d_sinks != nullptr) {  // zero when there are no query rows
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3((p.h_q + 255) / 256), dim3(256), 0, stream, p, n_qt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_kt > 0) {  // dK, dV (zero when there are no rows)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BN, CAUSAL, WINDOW, NWK, NSK>), dim3(p.b * p.h_kv * n_kt), dim3(NWK * 64), 0,
                       stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace attn

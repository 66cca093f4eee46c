// Shared device-side types and helpers of the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Device-side parameters of the prefill kernel (derived from attn_prefill_args).
struct PrefillParams {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  const float *sinks;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t lse_sb, lse_sh;
  int32_t b, h_q, h_kv, s_q, s_k;
  int32_t ratio;     // h_q / h_kv
  int32_t window;    // 0 = none
  int32_t n_qtiles;  // ceil(s_q / BM)
  float c;           // scale * log2(e): logits in base-2 units
};

// Chunked causal prefill: the (query tile, key chunk) pairs in launch order and
// the partial buffers of the query tiles that have more than one chunk
// (qt >= qt0): partial (bh, qt, c) is slot (bh*(n_qtiles-qt0) + qt-qt0)*max_chunks + c,
// holding BM rows of d bf16 values in o_part and BM fp32 LSEs in lse_part.
constexpr int kMaxChunkRanks = 384;
struct PrefillChunks {
  uint16_t *o_part;
  float *lse_part;
  int32_t chunk_tiles;  // key tiles per chunk
  int32_t qt0;          // first query tile with more than one chunk
  int32_t max_chunks;   // chunks of the longest query tile
  int32_t n_rank;       // entries of rank[] in use
  uint32_t rank[kMaxChunkRanks];  // (qt << 8) | chunk, longest first
};

// Device-side parameters of the backward kernels.  q, o, d_o and dq share one
// [b, h_q, s_q, d] layout (q strides); k, v, dk and dv share one [b, h_kv,
// s_k, d] layout (k strides); dsum and lse2 are fp32 [b, h_q, s_q] scratch.
struct BwdParams {
  const uint16_t *q, *k, *v, *o, *d_o;
  const float *lse;
  uint16_t *dq, *dk, *dv;
  float *dsum;
  float *lse2;  // fp32 [b, h_q, s_q] scratch: LSE * log2(e), +inf for a row with no key
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t lse_sb, lse_sh;
  int32_t b, h_q, h_kv, s_q, s_k, ratio;
  float c;      // scale * log2(e)
  float scale;
  int32_t window;        // 0 = none (a window requires the causal mask)
  const float *sinks;    // [h_q] sink logits, read only when d_sinks is set
  float *dsink_part;     // [b][h_q][query tiles of the dQ kernel] partial sink gradients
  float *d_sinks;        // [h_q] sink gradient summed over the batch; NULL = not wanted
};

// Device-side parameters of the split-KV decode kernel.
struct DecodeParams {
  const uint16_t *q, *k, *v;
  const int64_t *kv_start;
  const int32_t *kv_len;
  const float *sinks;
  uint16_t *o_part;  // [B][n_split][h_q][D] bf16, normalised partial outputs
  float *lse_part;  // [B][h_q][n_split] fp32, natural-log LSE of each part
  int64_t q_sb, q_sh;
  int64_t k_st, k_sh;
  int64_t v_st, v_sh;
  int32_t B, h_q, h_kv, ratio;
  int32_t n_split, split;
  int32_t n_hblk;  // head blocks per kv group: ceil(ratio / BM)
  // Paged cache only: token j of sequence b is row j % 2^page_shift of page
  // block_table[b * bt_stride + j >> page_shift], at k + page * k_ps + row * k_st
  // (+ g * k_sh); kv_start is unused.
  const int32_t *block_table;
  int64_t bt_stride;
  int64_t k_ps, v_ps;
  int32_t page_shift, n_pages;
  // FP8 cache only: E4M3 codes times these per-kv-head scales.
  const float *k_scale, *v_scale;
  float c;
  // Merge in the same launch: workgroups from unit_grid on merge the splits
  // of (sequence, kv head, slice of decode_merge_heads(D) heads) m once its
  // arrival counter arrive[m * arrive_stride] (m = (b * h_kv + g) * n_mblk +
  // slice) has counted every split, and write o_out / lse_out.
  uint32_t *arrive;
  uint16_t *o_out;
  float *lse_out;
  int64_t o_sb, o_sh, lse_sb;
  int32_t n_mblk, unit_grid;
  int32_t arrive_stride;  // 16 (one counter per 64-byte line) when they fit, else 1
};

// Query heads whose merge one 256-thread workgroup takes (8 columns a thread).
__host__ __device__ constexpr int decode_merge_heads(int d) { return 2048 / d; }

// Workgroups the split-KV decode launches for these sizes (its unit numbering
// needs the slots in whole groups of 8): every (split, sequence, kv head) slot,
// rounded up to a multiple of 8, times the head blocks.
__host__ __device__ inline int64_t decode_grid_size(int64_t n_split, int64_t B, int64_t h_kv, int64_t n_hblk) {
  return (n_split * B * h_kv + 7) / 8 * 8 * n_hblk;
}

// Device-side parameters of the LSE-merge kernel.  Rows are addressed as
// (r1, r2) with r2 < n2, so both flat rows (n2 = 1) and [B][h] rows work.
struct CombineParams {
  const void *o_parts;  // fp32 (public entry point) or bf16 (decode partials)
  const float *lse_parts;
  uint16_t *o_out;
  float *lse_out;
  int32_t n_parts, rows, n2, d;
  int64_t o_part_stride, o_r1, o_r2;
  int64_t lse_part_stride, lse_r1, lse_r2;
  int64_t out_r1, out_r2;
  int64_t lse_out_r1, lse_out_r2;
  // Decode: parts of row (r1, r2) are the splits of sequence r1 that hold
  // keys, min(n_parts, max(1, ceil(kv_len[r1] / split))); NULL = all n_parts.
  const int32_t *kv_len;
  int32_t split;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 of two values packed in one dword
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 MFMA, fp32 accumulate: D = A(32x16) * B(16x32) + C.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; the
// accumulator register i of lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

}  // namespace attn

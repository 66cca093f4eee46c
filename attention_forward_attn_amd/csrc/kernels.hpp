// Host-visible entry points of the kernel translation units.
#pragma once

#include "common.hpp"

namespace attn {

// Mask kinds of the prefill kernel.
enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskCausalWindow = 2 };

// Query rows per prefill workgroup for head dim d and mask kind (0 if unsupported).
int prefill_block_rows(int d, int mask);
// Enqueue the prefill kernel for head dim d; n_units = b * h_q * n_qtiles.
hipError_t prefill_d64(const PrefillParams &p, int mask, int n_units, hipStream_t s);
hipError_t prefill_d128(const PrefillParams &p, int mask, int n_units, hipStream_t s);
hipError_t prefill_d256(const PrefillParams &p, int mask, int n_units, hipStream_t s);
hipError_t prefill_d512(const PrefillParams &p, int mask, int n_units, hipStream_t s);
// Work-queue form of the ping-pong prefill at d = 256: n_wg workgroups take
// query tiles from the per-XCD counters at queue (a 256-byte header, zero
// before the first launch, left zero by every launch).
hipError_t prefill_d256_queue(const PrefillParams &p, int mask, int n_units, int n_wg, uint32_t *queue,
                              hipStream_t s);
// Key tiles per step of the prefill kernel for head dim d and mask kind.
int prefill_block_keys(int d, int mask);
// Causal d = 512 prefill with chunked key ranges (ck filled by the host) and the merge of the partials.
hipError_t prefill_d512_chunked(const PrefillParams &p, const PrefillChunks &ck, hipStream_t s);

// Query heads per decode workgroup (0 if unsupported).
int decode_block_rows(int d);
// Split-KV decode and the merge of its splits, one launch: p.unit_grid unit
// workgroups (decode_grid_size) then B * h_kv * n_mblk merge workgroups; the
// p.arrive counters must be zero at launch and are left zero.  With
// p.arrive = NULL and n_mblk = 0 only the partials are written (merged by
// combine_bf16).
hipError_t decode_split(int d, const DecodeParams &p, hipStream_t s);
// The same over a paged cache (p.block_table, p.page_shift, p.k_ps, p.v_ps set).
hipError_t decode_split_paged(int d, const DecodeParams &p, hipStream_t s);
// The same over an FP8 (E4M3) cache with per-kv-head scales (p.k_scale, p.v_scale); d = 128 or 256.
hipError_t decode_split_fp8(int d, const DecodeParams &p, hipStream_t s);
// The same over a paged FP8 cache (paged addressing in bytes); d = 128 or 256.
hipError_t decode_split_paged_fp8(int d, const DecodeParams &p, hipStream_t s);

// Attention backward (dQ, dK, dV, and the sink gradient when p.d_sinks is set) at
// head dim 64 or 128; p.dsum is scratch of b*h_q*s_q floats, p.dsink_part of
// b*h_q*ceil(s_q / backward_block_rows()) floats.  A window (p.window > 0)
// requires causal.
int backward_block_rows();
hipError_t backward(int d, const BwdParams &p, bool causal, hipStream_t s);

// LSE merge of fp32 partials (public entry point) / of bf16 partials (decode
// shapes with more merge workgroups than the workspace header has counters).
hipError_t combine(const CombineParams &p, hipStream_t s);
hipError_t combine_bf16(const CombineParams &p, hipStream_t s);

}  // namespace attn

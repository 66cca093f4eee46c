/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * One operation, in two launch shapes plus a merge:
 *
 *   O = softmax(scale * Q K^T + mask) V,   LSE = ln(sum over visible keys of exp(logit))
 *
 * computed with a streaming (online) softmax: per query row a running max,
 * a running sum and an O accumulator that is rescaled whenever the max grows,
 * and divided by the sum only at the very end.  That state machine is the
 * one the FA4 planner page ("b200-flash-attention4-planner", section A1
 * "Streaming online softmax" and executable steps 1-8) lays out; the masks,
 * sink and per-row LSE are rows D3, D4, D5b and D5c of the DSV4 status page
 * ("archived_plans/2026-05-28_STATUS.md"); the merge of partial results by
 * their LSE is the workaround paragraph "O rescale (kt>0)" of the STAGE_D.md
 * page (nvfp4-megamoe-kernel).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    keeps no pointer after a call returns, allocates no device memory and
 *    never synchronises the host: work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL means the default stream) and runs asynchronously.
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (uint16).  Strides are in
 *    ELEMENTS, int64, and the head-dim stride is always 1.
 *  - Arguments are validated on the host before any HIP call.  A non-zero
 *    status means nothing was enqueued; attn_last_error() then returns a
 *    thread-local message naming the offending argument.  ATTN_ERR_HIP means a
 *    launch was rejected by the runtime.  Faults inside a running kernel are
 *    reported by the stream, not by these calls.  No C++ exception crosses
 *    the ABI.
 *  - Alignment: every bf16 base pointer and every bf16 sequence/head/batch
 *    stride must be a multiple of 16 bytes (8 elements); fp32 pointers must be
 *    4-byte aligned.
 *  - Reentrancy: there is no global mutable state besides the thread-local
 *    error text and a thread-local memo of the last chunk plan (a pure
 *    function of the shape), so calls from several host threads are safe as
 *    long as they do not write the same output buffers.
 *  - Every output row is written, including rows that see no key.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_FWD_ABI_VERSION 10

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  ATTN_ERR_STRIDE = 3,      /* a stride is negative or not a multiple of 8 elements */
  ATTN_ERR_ALIGN = 4,       /* a base pointer is misaligned */
  ATTN_ERR_UNSUPPORTED = 5, /* a valid request this build has no kernel for */
  ATTN_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  ATTN_ERR_HIP = 7          /* the HIP runtime rejected a launch */
} attn_status;

/*
 * Prefill: one fused forward pass over [b, h_q, s_q] query rows.
 *
 * Element (bi, hi, si, t) of q lives at q + bi*q_sb + hi*q_sh + si*q_ss + t,
 * and likewise for k, v (with h_kv heads and s_k rows) and o (h_q heads, s_q
 * rows).  A [b, h, s, d] contiguous tensor has sb = h*s*d, sh = s*d, ss = d;
 * a [b, s, h, d] one has sb = s*h*d, sh = d, ss = h*d.  MQA may be expressed
 * either as h_kv = 1 or as h_kv = h_q with k_sh = v_sh = 0.
 *
 * Semantics (planner page, executable steps 1, 2 and 7; status page D2-D5c):
 *  - query head h reads kv head h / (h_q / h_kv): contiguous GQA groups;
 *  - logit(i, j) = scale * sum_t q[i, t] k[j, t]; scale must be finite and > 0;
 *  - causal = 1 masks with bottom-right alignment: key j is visible to row i
 *    iff j <= i + (s_k - s_q);
 *  - window = W > 0 (only together with causal) also requires
 *    j >= i + (s_k - s_q) - W + 1, i.e. W keys including the diagonal;
 *  - sinks, if not NULL, holds h_q fp32 logits: each acts as one extra
 *    softmax column with zero value, its logit taken as is (not scaled);
 *  - lse, if not NULL, receives the natural-log log-sum-exp of each row's
 *    scaled logits (sink included) at lse + bi*lse_sb + hi*lse_sh + si;
 *  - a row that sees no key and has no sink gets O = 0 and LSE = -inf.
 *
 * Supported: d in {64, 128, 256, 512}; b, h_q, h_kv >= 1; s_q, s_k >= 0
 * (s_q = 0 is a no-op); every index must fit in 31 bits.
 */
typedef struct {
  const void *q;      /* bf16 */
  const void *k;      /* bf16 */
  const void *v;      /* bf16 */
  void *o;            /* bf16 output */
  float *lse;         /* fp32 output [b, h_q, s_q] via lse_sb, lse_sh; NULL = not wanted */
  const float *sinks; /* fp32 [h_q]; NULL = no sink */
  int32_t b, h_q, h_kv, s_q, s_k, d;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t lse_sb, lse_sh;
  float scale;
  int32_t causal; /* 0 or 1 */
  int32_t window; /* 0 = none; W > 0 requires causal */
} attn_prefill_args;

/*
 * Decode: one query token per sequence against a KV cache that is contiguous
 * per sequence (the MQA/GQA decode of status-page row D2, with the multi-tile
 * key range handled by split-KV plus the LSE merge of the STAGE_D.md page).
 *
 * q: bf16, element (bi, hi, t) at q + bi*q_sb + hi*q_sh + t.
 * k, v: bf16; token tok of sequence bi, kv head g is at
 *       k + (kv_start[bi] + tok)*k_st + g*k_sh (v: v_st, v_sh); head strides
 *       may be 0 (MQA).
 * kv_start: DEVICE int64 [B]; kv_len: DEVICE int32 [B], each in [0, max_kv_len].
 * max_kv_len: host-side upper bound on every kv_len; it sizes the grid and the
 *       workspace, so no device-to-host copy is needed.
 * o: bf16 output (bi, hi, t) at o + bi*o_sb + hi*o_sh + t;
 * lse: fp32 output at lse + bi*lse_sb + hi (NULL = not wanted); sinks as in
 *       prefill.
 * split_size: keys per split (a multiple of 64, >= 64).  Split c of sequence
 *       bi covers keys [c*split_size, min((c+1)*split_size, kv_len[bi])).
 *
 * One kernel runs on `stream`: its split workgroups write normalised partial
 * outputs (rounded to bf16) and their fp32 LSE into the workspace, and its
 * merge workgroups, one per (sequence, kv head, slice of 2048/d query heads),
 * wait until every split of their rows has arrived and merge them in fp32
 * into o and lse.  The arrival counters sit in the first
 * ATTN_DECODE_WORKSPACE_HEADER bytes of the workspace, at fixed places for
 * every size: that header must be zero before the first call that uses the
 * workspace, and every call leaves it zero, so one zeroed workspace serves any
 * sequence of calls of any sizes that fit it.  (Over a header that is not
 * zero the merge may read splits that have not arrived; its wait is bounded,
 * so the kernel still ends.)  Shapes with more than ATTN_DECODE_WORKSPACE_HEADER
 * / 4 merge workgroups (B * h_kv * ceil((h_q / h_kv) / (2048 / d))) are merged
 * by a second kernel instead and do not use the header.  The workspace is
 * owned by the caller, must be 16-byte aligned, must stay allocated until the
 * stream has run the call's kernels, and must not be shared by calls that may
 * overlap.  Supported: d in {64, 128, 256}; B, h_q, h_kv >= 1, h_q % h_kv == 0.
 */
typedef struct {
  const void *q;
  const void *k;
  const void *v;
  const int64_t *kv_start;
  const int32_t *kv_len;
  void *o;
  float *lse;
  const float *sinks;
  int32_t B, h_q, h_kv, d;
  int32_t max_kv_len;
  int32_t split_size;
  int64_t q_sb, q_sh;
  int64_t k_st, k_sh;
  int64_t v_st, v_sh;
  int64_t o_sb, o_sh;
  int64_t lse_sb;
  float scale;
} attn_decode_args;

/*
 * Decode over a paged KV cache: the same operation, split kernel and combine
 * as attn_fwd_decode; only the addressing of K and V differs.  The pages ask
 * for paged and dense caches to get kernels of their own (optimize-fa4-blackwell
 * skill page, hard rules) and list a paged cache in the serving infrastructure
 * (DSV4 status page, KV cache infrastructure row) without fixing a layout; the one
 * taken here is a pool of pages of page_size tokens, with row bi of a block
 * table listing the pages of sequence bi in token order.  Token tok of
 * sequence bi, kv head g is at
 *     k + block_table[bi*bt_stride + tok/page_size]*k_ps + (tok % page_size)*k_ts + g*k_sh
 * (v: v_ps, v_ts, v_sh).
 *
 * block_table: DEVICE int32; row bi must list ceil(kv_len[bi]/page_size) page
 *       indices in [0, n_pages); entries past those are not read.  A page index
 *       outside [0, n_pages) is never dereferenced: its tokens read as zeros
 *       (a wrong result, not a fault).
 * page_size: a power of two in [16, split_size] that divides split_size, with
 *       split_size/page_size <= 64 (so every split starts on a page boundary);
 *       bt_stride >= ceil(max_kv_len/page_size).
 * Other fields, the workspace (attn_fwd_decode_workspace_size with the same
 * sizes), its ownership and the supported sizes are those of attn_fwd_decode.
 */
typedef struct {
  const void *q;
  const void *k;
  const void *v;
  const int32_t *block_table;
  const int32_t *kv_len;
  void *o;
  float *lse;
  const float *sinks;
  int32_t B, h_q, h_kv, d;
  int32_t max_kv_len;
  int32_t split_size;
  int32_t page_size;
  int32_t n_pages;
  int64_t bt_stride;
  int64_t q_sb, q_sh;
  int64_t k_ps, k_ts, k_sh;
  int64_t v_ps, v_ts, v_sh;
  int64_t o_sb, o_sh;
  int64_t lse_sb;
  float scale;
} attn_decode_paged_args;

/*
 * Decode over an FP8 KV cache: the same operation, split kernel and combine as
 * attn_fwd_decode, with K and V held as 8-bit codes.  The pages plan a KV
 * cache in fewer bits that is widened again on chip (DSV4 status page,
 * priority 7) without fixing a format; the one taken here is OCP FP8 E4M3
 * ("e4m3fn": bias 7, no infinities, 0x7f/0xff NaN) with one fp32 scale per kv
 * head for K and one for V: key element = value(code) * k_scale[g], value
 * element = value(code) * v_scale[g].  The kernel widens codes to bf16
 * exactly after the LDS read and applies the scales outside the MMAs.
 *
 * k, v: uint8 codes; token tok of sequence bi, kv head g at
 *       k + (kv_start[bi] + tok)*k_st + g*k_sh bytes (v: v_st, v_sh); token
 *       and head strides multiples of 16 bytes (head stride 0 = MQA).
 * k_scale, v_scale: DEVICE fp32 [h_kv].
 * Supported: d = 128 or 256.  Other fields, the workspace (attn_fwd_decode_workspace_size)
 * and its ownership are those of attn_fwd_decode.
 */
typedef struct {
  const void *q;
  const uint8_t *k;
  const uint8_t *v;
  const float *k_scale;
  const float *v_scale;
  const int64_t *kv_start;
  const int32_t *kv_len;
  void *o;
  float *lse;
  const float *sinks;
  int32_t B, h_q, h_kv, d;
  int32_t max_kv_len;
  int32_t split_size;
  int64_t q_sb, q_sh;
  int64_t k_st, k_sh;
  int64_t v_st, v_sh;
  int64_t o_sb, o_sh;
  int64_t lse_sb;
  float scale;
} attn_decode_fp8_args;

/*
 * Decode over a paged FP8 KV cache: the paged addressing of
 * attn_fwd_decode_paged (pages of page_size tokens, a block table per
 * sequence, the same rules on page_size, n_pages, bt_stride and indices
 * outside [0, n_pages)) over the E4M3 codes and per-kv-head scales of
 * attn_fwd_decode_fp8.  Token tok of sequence bi, kv head g is at
 *     k + block_table[bi*bt_stride + tok/page_size]*k_ps + (tok % page_size)*k_ts + g*k_sh
 * bytes (v: v_ps, v_ts, v_sh); every cache stride a non-negative multiple of
 * 16 bytes.  Supported: d = 128 or 256.  Other fields, the workspace
 * (attn_fwd_decode_workspace_size) and its ownership are those of
 * attn_fwd_decode.
 */
typedef struct {
  const void *q;
  const uint8_t *k;
  const uint8_t *v;
  const float *k_scale;
  const float *v_scale;
  const int32_t *block_table;
  const int32_t *kv_len;
  void *o;
  float *lse;
  const float *sinks;
  int32_t B, h_q, h_kv, d;
  int32_t max_kv_len;
  int32_t split_size;
  int32_t page_size;
  int32_t n_pages;
  int64_t bt_stride;
  int64_t q_sb, q_sh;
  int64_t k_ps, k_ts, k_sh;
  int64_t v_ps, v_ts, v_sh;
  int64_t o_sb, o_sh;
  int64_t lse_sb;
  float scale;
} attn_decode_paged_fp8_args;

/*
 * Backward of the prefill: dQ, dK, dV for an incoming gradient dO of O, from
 * the forward's O and LSE.  The pages list backward kernels and a
 * deterministic backward among the gaps to fill (SM120 research page) and
 * leave the algorithm to a design of its own (FA4 planner page, boundaries);
 * the one taken here is the chain rule through the softmax, with
 * P = exp(scale*QK^T - LSE), D_i = sum_t dO[i,t] O[i,t], dS = P*(dP - D),
 * dQ = scale*dS K, dK = scale*dS^T Q, dV = P^T dO (dK and dV summed over the
 * query heads of each kv head), under the forward's masks: none, causal, or a
 * causal sliding window of `window` keys (status page rows D3/D4).  A sink
 * (row D5c) enters only through the forward's LSE, which must be the one
 * computed with the same sinks; its logit's own gradient,
 * d_sinks[h] = -sum over the batch and rows of exp(sinks[h] - LSE_i) * D_i, is
 * written when d_sinks is not NULL.  The LSE gets no gradient.  Deterministic:
 * no atomics, every output element is written by exactly one thread in a fixed
 * order.
 *
 * q, o, d_o, dq: bf16 [b, h_q, s_q, d], one shared stride set (q_sb, q_sh,
 *       q_ss); k, v, dk, dv: bf16 [b, h_kv, s_k, d], one shared stride set
 *       (k_*); lse: fp32 (bi, h, i) at lse + bi*lse_sb + h*lse_sh + i.
 * q, o, d_o, lse and dq may be NULL when s_q = 0, k, v, dk and dv when s_k = 0.
 * window: 0 = none; W > 0 (only with causal) keeps keys j >= i + s_k - s_q - W + 1.
 * sinks: fp32 [h_q], the forward's sink logits (read only for d_sinks);
 * d_sinks: fp32 [h_q] output, NULL = not wanted (then sinks may be NULL).
 * workspace: attn_bwd_workspace_size(b, h_q, s_q) bytes, 16-byte aligned,
 *       caller-owned (row sums D and the rows' LSE in base 2 between the
 *       kernels, and the sink gradient's per-tile partials).
 * Kernels run on `stream`: dQ and D, the sink gradient (if wanted), then dK/dV.
 * Supported: d = 64, 128 or 256; causal (bottom-right) or not; h_q % h_kv == 0.
 */
typedef struct {
  const void *q, *k, *v, *o, *d_o;
  const float *lse;
  void *dq, *dk, *dv;
  int32_t b, h_q, h_kv, s_q, s_k, d;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t lse_sb, lse_sh;
  float scale;
  int32_t causal;
  int32_t window;
  const float *sinks;
  float *d_sinks;
} attn_bwd_args;

/* Bytes of device workspace attn_bwd needs at any supported d (0 on invalid
 * sizes): two fp32 values per query row, each array 256-byte aligned, then one
 * fp32 sink-gradient partial per 128 query rows of each (batch, head). */
size_t attn_bwd_workspace_size(int32_t b, int32_t h_q, int32_t s_q);

/*
 * Merge n_parts partial attention results computed over DISJOINT key sets
 * (STAGE_D.md page, "O rescale (kt>0)" workaround): per row, with
 * M = max_p lse_p and w_p = exp(lse_p - M),
 *     O = sum_p w_p O_p / sum_p w_p,   LSE = M + ln sum_p w_p.
 * A part with lse = -inf has zero weight: its O is loaded (so o_parts must be
 * allocated for every part) but never used, and may hold any bits, NaN
 * included; a row whose parts are all -inf gets O = 0, LSE = -inf.  It must not be used to merge
 * partial dot products over the same keys (head-dim sub-tiles add in logit
 * space; STAGE_D.md page, section 2).
 *
 * o_parts: fp32, element (p, r, t) at o_parts + p*o_part_stride + r*o_row_stride + t;
 * lse_parts: fp32 (p, r) at lse_parts + p*lse_part_stride + r*lse_row_stride;
 * o_out: bf16 (r, t) at o_out + r*o_out_row_stride + t;
 * lse_out: fp32 at lse_out + r (NULL = not wanted).
 * Supported: n_parts in [1, 1024], rows >= 0, d a multiple of 8 in [8, 512];
 * fp32 strides non-negative multiples of 4 elements, bf16 row stride a
 * multiple of 8 elements.
 */
typedef struct {
  const float *o_parts;
  const float *lse_parts;
  void *o_out;
  float *lse_out;
  int32_t n_parts, rows, d;
  int64_t o_part_stride, o_row_stride;
  int64_t lse_part_stride, lse_row_stride;
  int64_t o_out_row_stride;
} attn_combine_args;

/* Bytes of device workspace attn_fwd_decode needs for these sizes (0 on invalid
 * sizes), the ATTN_DECODE_WORKSPACE_HEADER bytes of arrival counters included. */
#define ATTN_DECODE_WORKSPACE_HEADER ((size_t)64 << 10)
size_t attn_fwd_decode_workspace_size(int32_t B, int32_t h_q, int32_t d, int32_t max_kv_len,
                                      int32_t split_size);

attn_status attn_fwd_prefill(const attn_prefill_args *args, void *stream);

/*
 * Scheduled prefill: the same operation and arguments as attn_fwd_prefill,
 * with a caller workspace that lets the library schedule the work better.
 *
 * Chunked causal prefill (head dim 512, causal, no window, too few query tiles
 * to fill the chip evenly; the STAGE_D.md page's hd=512 case: 128-row tiles,
 * one 8-wave workgroup per compute unit).  The visible key range of each long
 * query tile is cut into chunks whose length the host picks by simulating the
 * launch (units dealt to the 8 XCDs in grid order, each starting on the first
 * free compute unit of its XCD) for lengths around one compute unit's share of
 * the work and keeping the shortest makespan; each chunk runs as its own work
 * unit, longest first, and writes its normalised partial output (rounded to
 * bf16) and fp32 LSE into the workspace; a second kernel merges the chunks of
 * each row by their LSEs (the per-segment merge of the same page's "O rescale
 * (kt>0)" workaround).  A sink enters the first chunk only.  Results equal
 * attn_fwd_prefill's up to rounding (the partials pass through bf16), not bit
 * for bit.
 *
 * Work-queue prefill (head dim 256): one workgroup per compute unit takes
 * query tiles from counters in the workspace, one queue per XCD holding the
 * tiles attn_fwd_prefill would place on that XCD (longest first under a plain
 * causal mask); a workgroup takes from the front of its own XCD's queue and
 * then from the back (the shortest tiles) of the others, so XCDs that run at a
 * lower clock take fewer tiles.
 * Each tile is computed exactly as by attn_fwd_prefill: results are
 * bit-identical.
 *
 * The workspace starts with a 256-byte header holding the work-queue counters
 * (the chunk partials follow it).  The header must be zero before the first
 * call that uses the workspace; every call leaves it zero, and a call that
 * fails to launch does not touch it.  A workspace must not be shared by calls
 * that may overlap, and must stay allocated until the stream has run the
 * call's kernels.
 *
 * attn_fwd_prefill_chunked_workspace_size returns the bytes of workspace a
 * call with these arguments needs, or 0 when neither schedule applies (head
 * dim 64 or 128, head dim 512 without a causal mask, with a window or with
 * enough query tiles already) or the arguments are invalid;
 * with 0, workspace may be NULL and the call runs exactly attn_fwd_prefill.
 * Otherwise the workspace must be at least that large and 256-byte aligned
 * (ATTN_ERR_WORKSPACE / ATTN_ERR_ALIGN) and is owned by the caller.  The
 * returned size depends on every field that shapes the work (b, h_q, s_q, s_k,
 * d, causal, window), so query it with the same arguments.
 */
size_t attn_fwd_prefill_chunked_workspace_size(const attn_prefill_args *args);
attn_status attn_fwd_prefill_chunked(const attn_prefill_args *args, void *workspace, size_t workspace_bytes,
                                     void *stream);

attn_status attn_fwd_decode(const attn_decode_args *args, void *workspace, size_t workspace_bytes,
                            void *stream);
/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory or take a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same operation, kernels and
 * results as attn_fwd_decode; the workspace (arrival counters and split
 * partials) is a fixed region of ATTN_DECODE_SCRATCH_BYTES that the library
 * holds in device memory on every GPU it runs on, from the moment the
 * library's device code is loaded until the process ends.  Sizes whose partials need more
 * (attn_fwd_decode_workspace_size above ATTN_DECODE_SCRATCH_BYTES) are
 * rejected with ATTN_ERR_WORKSPACE; 72 MiB holds B = 64 sequences of up to
 * 8192 keys with h_q = 128 and d = 256 in 512-key splits.  The caller still
 * owns q, k, v, kv_start, kv_len, o, lse and sinks.  All calls on one GPU
 * share its region: calls that may overlap on one GPU (on different streams,
 * or from different host threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  The region starts zeroed
 * (static storage) and every call leaves its arrival counters zero.  The
 * first call on a device looks up the region's
 * address with that device current (hipGetSymbolAddress; ATTN_ERR_HIP if it
 * fails).
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)72 << 20)
attn_status attn_fwd_decode_noalloc(const attn_decode_args *args, void *stream);
attn_status attn_fwd_decode_paged(const attn_decode_paged_args *args, void *workspace,
                                  size_t workspace_bytes, void *stream);
attn_status attn_fwd_decode_fp8(const attn_decode_fp8_args *args, void *workspace, size_t workspace_bytes,
                                void *stream);
attn_status attn_fwd_decode_paged_fp8(const attn_decode_paged_fp8_args *args, void *workspace,
                                      size_t workspace_bytes, void *stream);
attn_status attn_combine(const attn_combine_args *args, void *stream);
attn_status attn_bwd(const attn_bwd_args *args, void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *attn_status_str(attn_status s);
/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char *attn_last_error(void);
/* ATTN_FWD_ABI_VERSION of the built library. */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */

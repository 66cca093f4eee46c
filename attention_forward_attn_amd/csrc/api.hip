// C ABI of the attention forward library: argument validation, instance
// selection, grid sizing and launch.  Every check runs on the host before any
// HIP call, so a rejected call has no side effect.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <vector>
#include <functional>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/attn_fwd.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

attn_status ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool bf16_stride_ok(int64_t s) { return s >= 0 && (s % 8) == 0; }
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;
// Key/value row strides are bounded so that byte offsets inside one tile of
// up to 128 rows fit the 32-bit buffer offsets of the kernels.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

// Largest element offset reachable through (extent, stride) pairs, plus the row length.
int64_t span(std::initializer_list<std::pair<int64_t, int64_t>> dims, int64_t last) {
  int64_t s = last;
  for (auto &d : dims)
    if (d.first > 0) s += (d.first - 1) * d.second;
  return s;
}

attn_status hip_fail(hipError_t e, const char *what) {
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Page geometry and block-table checks of the paged decode entry points
// (split_size already checked).
attn_status check_pages(int32_t ps, int32_t split_size, int32_t n_pages, int64_t bt_stride, int32_t max_kv_len) {
  if (ps < 16 || (ps & (ps - 1)) != 0 || ps > split_size || split_size / ps > 64)
    return fail(ATTN_ERR_SHAPE,
                "page_size must be a power of two in [16, split_size] with at most 64 pages per split (got %d)", ps);
  // Every split must start on a page boundary: the kernel maps key j of a
  // split to slot j % page_size of the split's (j / page_size)-th page.
  if (split_size % ps != 0)
    return fail(ATTN_ERR_SHAPE, "split_size (%d) must be a multiple of page_size (%d)", split_size, ps);
  if (n_pages < 1) return fail(ATTN_ERR_SHAPE, "n_pages must be >= 1");
  const int64_t max_pages = ((int64_t)max_kv_len + ps - 1) / ps;
  if (bt_stride < max_pages)
    return fail(ATTN_ERR_STRIDE, "bt_stride (%lld) must be >= ceil(max_kv_len / page_size) = %lld",
                (long long)bt_stride, (long long)max_pages);
  return ATTN_OK;
}

// Shared tail of the dense, paged and FP8 decode entry points (arguments
// already validated; p carries the K/V addressing; kind 0 = contiguous bf16
// cache, 1 = paged, 2 = FP8, 3 = paged FP8): grid check, workspace layout and
// the one launch of the split kernel with its merge.
attn_status run_decode(attn::DecodeParams &p, const int32_t *kv_len, const float *sinks, void *o, float *lse,
                       int32_t B, int32_t h_q, int32_t h_kv, int32_t d, int32_t max_kv_len, int32_t split_size,
                       int64_t q_sb, int64_t q_sh, int64_t o_sb, int64_t o_sh, int64_t lse_sb, float scale,
                       int kind, void *workspace, void *stream) {
  const int bm = attn::decode_block_rows(d);
  const int ratio = h_q / h_kv;
  const int64_t n_split = max_kv_len > 0 ? (max_kv_len + split_size - 1) / split_size : 1;
  const int64_t n_hblk = (ratio + bm - 1) / bm;
  const int64_t mh = attn::decode_merge_heads(d);
  const int64_t n_mblk = (ratio + mh - 1) / mh;
  const int64_t unit_grid = attn::decode_grid_size(n_split, B, h_kv, n_hblk);
  if (unit_grid + (int64_t)B * h_kv * n_mblk > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "decode grid too large: splits x B x kv heads x head blocks must fit in int32");
  // The merge addresses one sequence's partial rows through a 32-bit buffer range.
  if ((int64_t)h_q * n_split * d * 2 > (int64_t)UINT32_MAX)
    return fail(ATTN_ERR_SHAPE, "too many splits (%lld): h_q x splits x d x 2 must fit in 32 bits",
                (long long)n_split);

  const int64_t parts = (int64_t)B * h_q * n_split;
  char *ws = static_cast<char *>(workspace);
  const int64_t header = (int64_t)ATTN_DECODE_WORKSPACE_HEADER;
  // One arrival counter per merge workgroup in the fixed header; beyond that
  // many, the splits are merged by a second kernel instead.
  const int64_t n_merge = (int64_t)B * h_kv * n_mblk;
  const bool fused = n_merge <= header / 4;
  p.arrive = fused ? reinterpret_cast<uint32_t *>(ws) : nullptr;
  p.arrive_stride = n_merge * 64 <= header ? 16 : 1;  // a 64-byte line per counter when they fit
  p.o_part = reinterpret_cast<uint16_t *>(ws + header);
  p.lse_part = reinterpret_cast<float *>(ws + header + (parts * d * 2 + 255) / 256 * 256);
  p.kv_len = kv_len;
  p.sinks = sinks;
  p.q_sb = q_sb; p.q_sh = q_sh;
  p.B = B; p.h_q = h_q; p.h_kv = h_kv; p.ratio = ratio;
  p.n_split = (int32_t)n_split;
  p.split = split_size;
  p.n_hblk = (int32_t)n_hblk;
  p.c = scale * attn::kLog2e;
  p.o_out = static_cast<uint16_t *>(o);
  p.lse_out = lse;
  p.o_sb = o_sb; p.o_sh = o_sh; p.lse_sb = lse_sb;
  p.n_mblk = fused ? (int32_t)n_mblk : 0;  // no merge workgroups when the combine kernel merges
  p.unit_grid = (int32_t)unit_grid;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = kind == 1   ? attn::decode_split_paged(d, p, s)
                 : kind == 2 ? attn::decode_split_fp8(d, p, s)
                 : kind == 3 ? attn::decode_split_paged_fp8(d, p, s)
                             : attn::decode_split(d, p, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (fused) return ok();

  attn::CombineParams c;
  c.o_parts = p.o_part;
  c.lse_parts = p.lse_part;
  c.o_out = static_cast<uint16_t *>(o);
  c.lse_out = lse;
  c.n_parts = (int32_t)n_split;
  c.rows = B * h_q;
  c.n2 = h_q;
  c.d = d;
  c.o_part_stride = (int64_t)h_q * d;  // split-major partial rows
  c.o_r1 = (int64_t)n_split * h_q * d;
  c.o_r2 = d;
  c.lse_part_stride = 1;
  c.lse_r1 = (int64_t)h_q * n_split;
  c.lse_r2 = n_split;
  c.out_r1 = o_sb;
  c.out_r2 = o_sh;
  c.lse_out_r1 = lse_sb;
  c.lse_out_r2 = 1;
  c.kv_len = kv_len;
  c.split = split_size;
  e = attn::combine_bf16(c, s);
  if (e != hipSuccess) return hip_fail(e, "decode combine launch");
  return ok();
}

}  // namespace

extern "C" {

int32_t attn_abi_version(void) { return ATTN_FWD_ABI_VERSION; }

const char *attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_STRIDE: return "ATTN_ERR_STRIDE";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_ERR_UNKNOWN";
}

const char *attn_last_error(void) { return g_err; }

namespace {

// Plan of the chunked causal prefill (d = 512; see attn_fwd_prefill_chunked).
// The key range of each query tile is cut into chunks of `chunk_tiles` key
// tiles; the (query tile, chunk) pairs are launched longest first.  The chunk
// length is chosen by simulating that launch for each candidate length and
// keeping the shortest makespan: unit v of the grid goes to XCD v % 8 and, on
// its XCD, starts on whichever of the 32 compute units frees first (one
// workgroup per compute unit at d = 512); a unit costs its key tiles plus
// kUnitFixedTiles, the per-unit cost of its prologue, epilogue and share of
// the merge, measured in key tiles (with it the simulated makespan tracked the
// measured time of eight chunk lengths on the b1 h4 s4096 workload to within
// 1 us).  Candidates run from three quarters to twice the even share of the
// work per compute unit (never below kMinChunkTiles), at most
// kMaxChunkCandidates of them evenly spaced, so a first call plans in well
// under a millisecond; ties go to the longer chunk (fewer partials to merge).
constexpr int kChunkTargetCUs = 256;
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
constexpr int kMinChunkTiles = 8;
constexpr int64_t kUnitFixedTiles = 10;
constexpr int64_t kMaxChunkCandidates = 64;  // lengths simulated at most (evenly spaced)

struct ChunkPlan {
  int chunk_tiles = 0, qt0 = 0, max_chunks = 0, n_rank = 0;
  uint32_t rank[attn::kMaxChunkRanks];
  int64_t o_bytes = 0, lse_bytes = 0;  // partial buffers; o_bytes is a multiple of 256
};

struct ChunkUnit { int64_t len, qt, ch; };

// Units of chunk length c in launch order (longest first, later query tiles
// first among equals); false if the plan exceeds the rank table or 255 chunks.
bool chunk_units(const std::vector<int64_t> &T, int64_t c, std::vector<ChunkUnit> &es) {
  es.clear();
  for (int64_t qt = 0; qt < (int64_t)T.size(); ++qt) {
    const int64_t n = T[qt] > 0 ? (T[qt] + c - 1) / c : 1;
    if (n > 255) return false;
    for (int64_t ch = 0; ch < n; ++ch) es.push_back({T[qt] > 0 ? std::min(c, T[qt] - ch * c) : 0, qt, ch});
  }
  if ((int64_t)es.size() > attn::kMaxChunkRanks) return false;
  std::stable_sort(es.begin(), es.end(), [](const ChunkUnit &x, const ChunkUnit &y) {
    return x.len != y.len ? x.len > y.len : x.qt > y.qt;
  });
  return true;
}

// Simulated makespan (key tiles) of the launch of es, each rank repeated for
// the bh heads (grid index = rank * bh + head).
int64_t chunk_makespan(const std::vector<ChunkUnit> &es, int64_t bh) {
  std::vector<int64_t> cu[kXcds];
  for (auto &v : cu) v.assign(kCusPerXcd, 0);
  int64_t v = 0, mk = 0;
  for (const ChunkUnit &e : es)
    for (int64_t j = 0; j < bh; ++j, ++v) {
      std::vector<int64_t> &h = cu[v % kXcds];  // min-heap of finish times
      std::pop_heap(h.begin(), h.end(), std::greater<int64_t>());
      h.back() += e.len + kUnitFixedTiles;
      mk = std::max(mk, h.back());
      std::push_heap(h.begin(), h.end(), std::greater<int64_t>());
    }
  return mk;
}

struct PlanMemo {  // the last plan this thread made, keyed by the shape
  bool valid = false, chunked = false;
  int64_t b, h_q, s_q, s_k, d;
  ChunkPlan pl;
};
thread_local PlanMemo g_plan_memo;

// Fills pl and returns true when the call would be chunked; false leaves the
// single-pass kernel in charge.  Arguments must already be valid.
bool plan_chunks(const attn_prefill_args *a, ChunkPlan &pl) {
  if (a->d != 512 || !a->causal || a->window > 0 || a->s_q == 0 || a->s_k == 0) return false;
  PlanMemo &mm = g_plan_memo;
  if (mm.valid && mm.b == a->b && mm.h_q == a->h_q && mm.s_q == a->s_q && mm.s_k == a->s_k && mm.d == a->d) {
    if (mm.chunked) pl = mm.pl;
    return mm.chunked;
  }
  mm.valid = false;
  const int bm = attn::prefill_block_rows(512, attn::kMaskCausal);
  const int bn = attn::prefill_block_keys(512, attn::kMaskCausal);
  const int64_t nq = (a->s_q + bm - 1) / bm;
  const int64_t off = (int64_t)a->s_k - a->s_q;
  const int64_t bh = (int64_t)a->b * a->h_q;
  std::vector<int64_t> T(nq);
  int64_t total = 0, tmax = 0;
  for (int64_t qt = 0; qt < nq; ++qt) {
    const int64_t i_last = std::min<int64_t>(a->s_q, (qt + 1) * bm) - 1;
    const int64_t kend = std::max<int64_t>(0, std::min<int64_t>(a->s_k, i_last + off + 1));
    T[qt] = (kend + bn - 1) / bn;
    total += T[qt];
    tmax = std::max(tmax, T[qt]);
  }
  total *= bh;
  const int64_t c0 = std::max<int64_t>(kMinChunkTiles, (total + kChunkTargetCUs - 1) / kChunkTargetCUs);
  bool chunked = false;
  std::vector<ChunkUnit> es, best;
  if (c0 < tmax && nq < (1 << 23)) {
    int64_t best_c = 0, best_mk = 0;
    const int64_t lo = std::max<int64_t>(kMinChunkTiles, c0 * 3 / 4), hi = std::min(tmax - 1, 2 * c0);
    const int64_t step = std::max<int64_t>(1, (hi - lo) / (kMaxChunkCandidates - 1));
    for (int64_t c = lo; c <= hi; c += step) {
      if (!chunk_units(T, c, es) || (int64_t)es.size() * bh > kMaxIndex) continue;
      const int64_t mk = chunk_makespan(es, bh);
      if (best_c == 0 || mk <= best_mk) best_c = c, best_mk = mk, best = es;
    }
    if (best_c > 0) {
      chunked = true;
      pl.chunk_tiles = (int)best_c;
      pl.n_rank = (int)best.size();
      for (int i = 0; i < pl.n_rank; ++i) pl.rank[i] = (uint32_t)(best[i].qt << 8) | (uint32_t)best[i].ch;
      int64_t qt0 = nq;
      while (qt0 > 0 && T[qt0 - 1] > best_c) --qt0;  // T is non-decreasing in qt
      pl.qt0 = (int)qt0;
      pl.max_chunks = (int)((tmax + best_c - 1) / best_c);
      const int64_t rows = bh * (nq - qt0) * pl.max_chunks * bm;
      pl.o_bytes = (rows * a->d * 2 + 255) / 256 * 256;
      pl.lse_bytes = rows * 4;
    }
  }
  mm.b = a->b; mm.h_q = a->h_q; mm.s_q = a->s_q; mm.s_k = a->s_k; mm.d = a->d;
  mm.chunked = chunked;
  if (chunked) mm.pl = pl;
  mm.valid = true;
  return chunked;
}

// Workspace of the scheduled prefill: a 256-byte header holding the work-queue
// counters (two uint32; zero before first use, left zero by every call), then
// the chunk partials of a chunked plan.
constexpr size_t kQueueBytes = 256;
// Shapes whose scheduled form takes query tiles from the work queue: the
// ping-pong kernel at d = 256 (b1 h8 s16384 causal: 1180 -> 1015..1036 us).
// At d = 128 the queued form of the same kernel measured 1-7 % slower than
// the fixed placement, so d = 128 keeps it.
bool queue_shape(int d, int mask) {
  (void)mask;
  return d == 256;
}

// Validation and parameter block of a prefill call; on success *done is set
// when there is nothing to launch (s_q == 0).
attn_status prepare_prefill(const attn_prefill_args *a, attn::PrefillParams &p, int &mask, int64_t &n_units,
                            bool &done) {
  done = false;
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->b < 1 || a->h_q < 1 || a->h_kv < 1 || a->s_q < 0 || a->s_k < 0)
    return fail(ATTN_ERR_SHAPE, "need b, h_q, h_kv >= 1 and s_q, s_k >= 0 (got b=%d h_q=%d h_kv=%d s_q=%d s_k=%d)",
                a->b, a->h_q, a->h_kv, a->s_q, a->s_k);
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 64 && a->d != 128 && a->d != 256 && a->d != 512)
    return fail(ATTN_ERR_SHAPE, "d must be 64, 128, 256 or 512 (got %d)", a->d);
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERR_SHAPE, "causal must be 0 or 1");
  if (a->window < 0) return fail(ATTN_ERR_SHAPE, "window must be >= 0");
  if (a->window > 0 && !a->causal) return fail(ATTN_ERR_SHAPE, "a window requires causal = 1");
  if (a->s_q == 0) {
    done = true;
    return ok();
  }
  if (!a->q || !a->o || (a->s_k > 0 && (!a->k || !a->v)))
    return fail(ATTN_ERR_NULL, "q, o (and k, v when s_k > 0) must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->o) || (a->s_k > 0 && (!aligned16(a->k) || !aligned16(a->v))))
    return fail(ATTN_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if ((a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return fail(ATTN_ERR_ALIGN, "lse and sinks must be 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->q_ss, a->k_sb, a->k_sh, a->k_ss,
                        a->v_sb, a->v_sh, a->v_ss, a->o_sb, a->o_sh, a->o_ss};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  if (a->lse && (a->lse_sb < 0 || a->lse_sh < 0)) return fail(ATTN_ERR_STRIDE, "lse strides must be >= 0");
  if (a->k_ss >= kMaxRowStride || a->v_ss >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "k/v sequence strides must be below 2^24 elements");
  const int64_t bmax = span({{a->b, a->q_sb}, {a->h_q, a->q_sh}, {a->s_q, a->q_ss}}, a->d);
  const int64_t kmax = span({{a->b, a->k_sb}, {a->h_kv, a->k_sh}, {a->s_k, a->k_ss}}, a->d);
  const int64_t vmax = span({{a->b, a->v_sb}, {a->h_kv, a->v_sh}, {a->s_k, a->v_ss}}, a->d);
  const int64_t omax = span({{a->b, a->o_sb}, {a->h_q, a->o_sh}, {a->s_q, a->o_ss}}, a->d);
  if (bmax > (int64_t(1) << 40) || kmax > (int64_t(1) << 40) || vmax > (int64_t(1) << 40) ||
      omax > (int64_t(1) << 40))
    return fail(ATTN_ERR_SHAPE, "tensor extent exceeds 2^40 elements");

  mask = a->window > 0 ? attn::kMaskCausalWindow : (a->causal ? attn::kMaskCausal : attn::kMaskNone);
  const int bm = attn::prefill_block_rows(a->d, mask);
  const int64_t n_qtiles = (a->s_q + bm - 1) / bm;
  n_units = n_qtiles * a->b * a->h_q;
  if (n_units > kMaxIndex) return fail(ATTN_ERR_SHAPE, "too many work units (%lld)", (long long)n_units);

  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.o = static_cast<uint16_t *>(a->o);
  p.lse = a->lse;
  p.sinks = a->sinks;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_ss = a->q_ss;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_ss = a->k_ss;
  p.v_sb = a->v_sb; p.v_sh = a->v_sh; p.v_ss = a->v_ss;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_ss = a->o_ss;
  p.lse_sb = a->lse_sb; p.lse_sh = a->lse_sh;
  p.b = a->b; p.h_q = a->h_q; p.h_kv = a->h_kv; p.s_q = a->s_q; p.s_k = a->s_k;
  p.ratio = a->h_q / a->h_kv;
  p.window = a->window;
  p.n_qtiles = (int32_t)n_qtiles;
  p.c = a->scale * attn::kLog2e;
  return ok();
}

attn_status launch_prefill(const attn_prefill_args *a, const attn::PrefillParams &p, int mask, int64_t n_units,
                           void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (a->d) {
    case 64: e = attn::prefill_d64(p, mask, (int)n_units, s); break;
    case 128: e = attn::prefill_d128(p, mask, (int)n_units, s); break;
    case 256: e = attn::prefill_d256(p, mask, (int)n_units, s); break;
    default: e = attn::prefill_d512(p, mask, (int)n_units, s); break;
  }
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

}  // namespace

attn_status attn_fwd_prefill(const attn_prefill_args *a, void *stream) {
  attn::PrefillParams p;
  int mask;
  int64_t n_units;
  bool done;
  attn_status st = prepare_prefill(a, p, mask, n_units, done);
  if (st != ATTN_OK || done) return st;
  return launch_prefill(a, p, mask, n_units, stream);
}

size_t attn_fwd_prefill_chunked_workspace_size(const attn_prefill_args *a) {
  attn::PrefillParams p;
  int mask;
  int64_t n_units;
  bool done;
  if (prepare_prefill(a, p, mask, n_units, done) != ATTN_OK || done) return 0;
  static thread_local ChunkPlan pl;
  if (plan_chunks(a, pl)) return kQueueBytes + (size_t)(pl.o_bytes + pl.lse_bytes);
  return queue_shape(a->d, mask) ? kQueueBytes : 0;
}

attn_status attn_fwd_prefill_chunked(const attn_prefill_args *a, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  attn::PrefillParams p;
  int mask;
  int64_t n_units;
  bool done;
  attn_status st = prepare_prefill(a, p, mask, n_units, done);
  if (st != ATTN_OK || done) return st;
  static thread_local ChunkPlan pl;
  const bool chunked = plan_chunks(a, pl);
  const bool queued = !chunked && queue_shape(a->d, mask);
  if (!chunked && !queued) return launch_prefill(a, p, mask, n_units, stream);
  const size_t need = kQueueBytes + (chunked ? (size_t)(pl.o_bytes + pl.lse_bytes) : 0);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "scheduled prefill needs %zu workspace bytes (got %zu%s)", need,
                workspace_bytes, workspace == nullptr ? ", NULL" : "");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (queued) {
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "device query");
    uint32_t *queue = static_cast<uint32_t *>(workspace);
    e = attn::prefill_d256_queue(p, mask, (int)n_units, std::max(n_cu, 1), queue, s);
    if (e != hipSuccess) return hip_fail(e, "queued prefill launch");
    return ok();
  }
  char *parts = static_cast<char *>(workspace) + kQueueBytes;
  attn::PrefillChunks ck;
  ck.o_part = reinterpret_cast<uint16_t *>(parts);
  ck.lse_part = reinterpret_cast<float *>(parts + pl.o_bytes);
  ck.chunk_tiles = pl.chunk_tiles;
  ck.qt0 = pl.qt0;
  ck.max_chunks = pl.max_chunks;
  ck.n_rank = pl.n_rank;
  std::memcpy(ck.rank, pl.rank, sizeof(uint32_t) * pl.n_rank);
  std::memset(ck.rank + pl.n_rank, 0, sizeof(uint32_t) * (attn::kMaxChunkRanks - pl.n_rank));
  hipError_t e = attn::prefill_d512_chunked(p, ck, s);
  if (e != hipSuccess) return hip_fail(e, "chunked prefill launch");
  return ok();
}

size_t attn_fwd_decode_workspace_size(int32_t B, int32_t h_q, int32_t d, int32_t max_kv_len,
                                      int32_t split_size) {
  if (B < 1 || h_q < 1 || d < 1 || max_kv_len < 0 || split_size < 64 || split_size % 64 != 0) return 0;
  const int64_t n_split = max_kv_len > 0 ? (max_kv_len + split_size - 1) / split_size : 1;
  const int64_t parts = (int64_t)B * h_q * n_split;
  const int64_t o_bytes = parts * d * 2;  // bf16 partial outputs
  const int64_t o_aligned = (o_bytes + 255) / 256 * 256;
  return ATTN_DECODE_WORKSPACE_HEADER + (size_t)(o_aligned + parts * 4);
}

}  // extern "C"

namespace {

// Host-side checks of a contiguous-cache decode call, everything but the workspace.
attn_status check_decode_args(const attn_decode_args *a) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->B < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(ATTN_ERR_SHAPE, "need B, h_q, h_kv >= 1");
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 64 && a->d != 128 && a->d != 256)
    return fail(ATTN_ERR_SHAPE, "decode d must be 64, 128 or 256 (got %d)", a->d);
  if (a->max_kv_len < 0) return fail(ATTN_ERR_SHAPE, "max_kv_len must be >= 0");
  if (a->split_size < 64 || a->split_size % 64 != 0)
    return fail(ATTN_ERR_SHAPE, "split_size must be a positive multiple of 64 (got %d)", a->split_size);
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!a->q || !a->k || !a->v || !a->o || !a->kv_start || !a->kv_len)
    return fail(ATTN_ERR_NULL, "q, k, v, o, kv_start and kv_len must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(ATTN_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(a->kv_start) & 7u) || !aligned4(a->kv_len) ||
      (a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return fail(ATTN_ERR_ALIGN, "kv_start must be 8-byte and kv_len, lse, sinks 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->k_st, a->k_sh, a->v_st, a->v_sh, a->o_sb, a->o_sh};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  if (a->lse && a->lse_sb < 0) return fail(ATTN_ERR_STRIDE, "lse_sb must be >= 0");
  if (a->k_st >= kMaxRowStride || a->v_st >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "k/v token strides must be below 2^24 elements");
  return ATTN_OK;
}

// Split kernel + combine of a checked contiguous-cache decode call, partials in `workspace`.
attn_status launch_decode(const attn_decode_args *a, void *workspace, void *stream) {
  attn::DecodeParams p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.kv_start = a->kv_start;
  p.k_st = a->k_st; p.k_sh = a->k_sh;
  p.v_st = a->v_st; p.v_sh = a->v_sh;
  return run_decode(p, a->kv_len, a->sinks, a->o, a->lse, a->B, a->h_q, a->h_kv, a->d, a->max_kv_len,
                    a->split_size, a->q_sb, a->q_sh, a->o_sb, a->o_sh, a->lse_sb, a->scale, 0, workspace,
                    stream);
}

}  // namespace

// Device memory of attn_fwd_decode_noalloc: the split partials of every call
// on a GPU go here.  Each GPU the library runs on holds its own copy from
// module load until the process ends.  In host code this name is only a
// handle for hipGetSymbolAddress, never a device address.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
attn_status scratch_address(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd_decode(const attn_decode_args *a, void *workspace, size_t workspace_bytes,
                            void *stream) {
  const attn_status st = check_decode_args(a);
  if (st != ATTN_OK) return st;
  const size_t need = attn_fwd_decode_workspace_size(a->B, a->h_q, a->d, a->max_kv_len, a->split_size);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  return launch_decode(a, workspace, stream);
}

attn_status attn_fwd_decode_noalloc(const attn_decode_args *a, void *stream) {
  const attn_status st = check_decode_args(a);
  if (st != ATTN_OK) return st;
  const size_t need = attn_fwd_decode_workspace_size(a->B, a->h_q, a->d, a->max_kv_len, a->split_size);
  if (need > ATTN_DECODE_SCRATCH_BYTES)
    return fail(ATTN_ERR_WORKSPACE, "these sizes need %zu bytes of partials, above the %zu-byte scratch of "
                "attn_fwd_decode_noalloc (use attn_fwd_decode with a workspace)", need,
                (size_t)ATTN_DECODE_SCRATCH_BYTES);
  void *ptr = nullptr;
  const attn_status sst = scratch_address(&ptr);
  if (sst != ATTN_OK) return sst;
  return launch_decode(a, ptr, stream);
}

attn_status attn_fwd_decode_fp8(const attn_decode_fp8_args *a, void *workspace, size_t workspace_bytes,
                                void *stream) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->B < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(ATTN_ERR_SHAPE, "need B, h_q, h_kv >= 1");
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 128 && a->d != 256) return fail(ATTN_ERR_SHAPE, "FP8 decode supports d = 128 or 256 (got %d)", a->d);
  if (a->max_kv_len < 0) return fail(ATTN_ERR_SHAPE, "max_kv_len must be >= 0");
  if (a->split_size < 64 || a->split_size % 64 != 0)
    return fail(ATTN_ERR_SHAPE, "split_size must be a positive multiple of 64 (got %d)", a->split_size);
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!a->q || !a->k || !a->v || !a->o || !a->kv_start || !a->kv_len || !a->k_scale || !a->v_scale)
    return fail(ATTN_ERR_NULL, "q, k, v, o, kv_start, kv_len, k_scale and v_scale must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(ATTN_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(a->kv_start) & 7u) || !aligned4(a->kv_len) || !aligned4(a->k_scale) ||
      !aligned4(a->v_scale) || (a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return fail(ATTN_ERR_ALIGN, "kv_start must be 8-byte and kv_len, scales, lse, sinks 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->o_sb, a->o_sh};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  const int64_t cst[] = {a->k_st, a->k_sh, a->v_st, a->v_sh};
  for (int64_t s : cst)
    if (s < 0 || s % 16 != 0) return fail(ATTN_ERR_STRIDE, "FP8 cache strides must be non-negative multiples of 16 bytes");
  if (a->lse && a->lse_sb < 0) return fail(ATTN_ERR_STRIDE, "lse_sb must be >= 0");
  if (a->k_st >= kMaxRowStride || a->v_st >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "k/v token strides must be below 2^24 bytes");
  const size_t need = attn_fwd_decode_workspace_size(a->B, a->h_q, a->d, a->max_kv_len, a->split_size);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");

  attn::DecodeParams p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = reinterpret_cast<const uint16_t *>(a->k);  // byte addressing inside the kernel
  p.v = reinterpret_cast<const uint16_t *>(a->v);
  p.kv_start = a->kv_start;
  p.k_st = a->k_st; p.k_sh = a->k_sh;
  p.v_st = a->v_st; p.v_sh = a->v_sh;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  return run_decode(p, a->kv_len, a->sinks, a->o, a->lse, a->B, a->h_q, a->h_kv, a->d, a->max_kv_len,
                    a->split_size, a->q_sb, a->q_sh, a->o_sb, a->o_sh, a->lse_sb, a->scale, 2, workspace,
                    stream);
}

attn_status attn_fwd_decode_paged(const attn_decode_paged_args *a, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->B < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(ATTN_ERR_SHAPE, "need B, h_q, h_kv >= 1");
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 64 && a->d != 128 && a->d != 256)
    return fail(ATTN_ERR_SHAPE, "decode d must be 64, 128 or 256 (got %d)", a->d);
  if (a->max_kv_len < 0) return fail(ATTN_ERR_SHAPE, "max_kv_len must be >= 0");
  if (a->split_size < 64 || a->split_size % 64 != 0)
    return fail(ATTN_ERR_SHAPE, "split_size must be a positive multiple of 64 (got %d)", a->split_size);
  const int ps = a->page_size;
  const attn_status pst = check_pages(ps, a->split_size, a->n_pages, a->bt_stride, a->max_kv_len);
  if (pst != ATTN_OK) return pst;
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!a->q || !a->k || !a->v || !a->o || !a->block_table || !a->kv_len)
    return fail(ATTN_ERR_NULL, "q, k, v, o, block_table and kv_len must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(ATTN_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if (!aligned4(a->block_table) || !aligned4(a->kv_len) || (a->lse && !aligned4(a->lse)) ||
      (a->sinks && !aligned4(a->sinks)))
    return fail(ATTN_ERR_ALIGN, "block_table, kv_len, lse and sinks must be 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->k_ps, a->k_ts, a->k_sh, a->v_ps, a->v_ts, a->v_sh, a->o_sb, a->o_sh};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  if (a->lse && a->lse_sb < 0) return fail(ATTN_ERR_STRIDE, "lse_sb must be >= 0");
  if (a->k_ts >= kMaxRowStride || a->v_ts >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "k/v token strides must be below 2^24 elements");
  const size_t need = attn_fwd_decode_workspace_size(a->B, a->h_q, a->d, a->max_kv_len, a->split_size);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");

  attn::DecodeParams p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.k_ps = a->k_ps; p.k_st = a->k_ts; p.k_sh = a->k_sh;
  p.v_ps = a->v_ps; p.v_st = a->v_ts; p.v_sh = a->v_sh;
  p.page_shift = __builtin_ctz((unsigned)ps);
  p.n_pages = a->n_pages;
  return run_decode(p, a->kv_len, a->sinks, a->o, a->lse, a->B, a->h_q, a->h_kv, a->d, a->max_kv_len,
                    a->split_size, a->q_sb, a->q_sh, a->o_sb, a->o_sh, a->lse_sb, a->scale, 1, workspace,
                    stream);
}

attn_status attn_fwd_decode_paged_fp8(const attn_decode_paged_fp8_args *a, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->B < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(ATTN_ERR_SHAPE, "need B, h_q, h_kv >= 1");
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 128 && a->d != 256) return fail(ATTN_ERR_SHAPE, "FP8 decode supports d = 128 or 256 (got %d)", a->d);
  if (a->max_kv_len < 0) return fail(ATTN_ERR_SHAPE, "max_kv_len must be >= 0");
  if (a->split_size < 64 || a->split_size % 64 != 0)
    return fail(ATTN_ERR_SHAPE, "split_size must be a positive multiple of 64 (got %d)", a->split_size);
  const int ps = a->page_size;
  const attn_status pst = check_pages(ps, a->split_size, a->n_pages, a->bt_stride, a->max_kv_len);
  if (pst != ATTN_OK) return pst;
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  if (!a->q || !a->k || !a->v || !a->o || !a->block_table || !a->kv_len || !a->k_scale || !a->v_scale)
    return fail(ATTN_ERR_NULL, "q, k, v, o, block_table, kv_len, k_scale and v_scale must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(ATTN_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if (!aligned4(a->block_table) || !aligned4(a->kv_len) || !aligned4(a->k_scale) || !aligned4(a->v_scale) ||
      (a->lse && !aligned4(a->lse)) || (a->sinks && !aligned4(a->sinks)))
    return fail(ATTN_ERR_ALIGN, "block_table, kv_len, scales, lse and sinks must be 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->o_sb, a->o_sh};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  const int64_t cst[] = {a->k_ps, a->k_ts, a->k_sh, a->v_ps, a->v_ts, a->v_sh};
  for (int64_t s : cst)
    if (s < 0 || s % 16 != 0) return fail(ATTN_ERR_STRIDE, "FP8 cache strides must be non-negative multiples of 16 bytes");
  if (a->lse && a->lse_sb < 0) return fail(ATTN_ERR_STRIDE, "lse_sb must be >= 0");
  if (a->k_ts >= kMaxRowStride || a->v_ts >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "k/v token strides must be below 2^24 bytes");
  const size_t need = attn_fwd_decode_workspace_size(a->B, a->h_q, a->d, a->max_kv_len, a->split_size);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");

  attn::DecodeParams p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = reinterpret_cast<const uint16_t *>(a->k);  // byte addressing inside the kernel
  p.v = reinterpret_cast<const uint16_t *>(a->v);
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.k_ps = a->k_ps; p.k_st = a->k_ts; p.k_sh = a->k_sh;
  p.v_ps = a->v_ps; p.v_st = a->v_ts; p.v_sh = a->v_sh;
  p.page_shift = __builtin_ctz((unsigned)ps);
  p.n_pages = a->n_pages;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  return run_decode(p, a->kv_len, a->sinks, a->o, a->lse, a->B, a->h_q, a->h_kv, a->d, a->max_kv_len,
                    a->split_size, a->q_sb, a->q_sh, a->o_sb, a->o_sh, a->lse_sb, a->scale, 3, workspace,
                    stream);
}

// Backward workspace: D = rowsum(dO * O) [b][h_q][s_q] fp32, then (256-byte
// aligned) LSE * log2(e) [b][h_q][s_q] fp32, then (256-byte aligned) the
// sink-gradient partials [b][h_q][query tiles of the dQ kernel].
size_t attn_bwd_workspace_size(int32_t b, int32_t h_q, int32_t s_q) {
  if (b < 1 || h_q < 1 || s_q < 0) return 0;
  const size_t rows = (size_t)b * h_q * (size_t)(s_q > 0 ? s_q : 1);
  const size_t br = (size_t)attn::backward_block_rows();
  const size_t tiles = (size_t)b * h_q * (((size_t)s_q + br - 1) / br);
  return 2 * ((rows * 4 + 255) / 256 * 256) + tiles * 4;
}

attn_status attn_bwd(const attn_bwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->b < 1 || a->h_q < 1 || a->h_kv < 1 || a->s_q < 0 || a->s_k < 0)
    return fail(ATTN_ERR_SHAPE, "need b, h_q, h_kv >= 1 and s_q, s_k >= 0");
  if (a->h_q % a->h_kv != 0)
    return fail(ATTN_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if (a->d != 64 && a->d != 128 && a->d != 256)
    return fail(ATTN_ERR_SHAPE, "backward supports d = 64, 128 or 256 (got %d)", a->d);
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERR_SHAPE, "causal must be 0 or 1");
  if (a->window < 0) return fail(ATTN_ERR_SHAPE, "window must be >= 0");
  if (a->window > 0 && !a->causal) return fail(ATTN_ERR_SHAPE, "a window requires causal = 1");
  if (!(std::isfinite(a->scale) && a->scale > 0.0f))
    return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
  // A tensor with no element may be NULL (a zero-length torch tensor has no storage).
  if (a->s_q > 0 && (!a->q || !a->o || !a->d_o || !a->lse || !a->dq))
    return fail(ATTN_ERR_NULL, "q, o, d_o, lse and dq must be non-NULL when s_q > 0");
  if (a->s_k > 0 && (!a->k || !a->v || !a->dk || !a->dv))
    return fail(ATTN_ERR_NULL, "k, v, dk and dv must be non-NULL when s_k > 0");
  if (a->d_sinks && !a->sinks) return fail(ATTN_ERR_NULL, "d_sinks needs sinks");
  if ((a->sinks && !aligned4(a->sinks)) || (a->d_sinks && !aligned4(a->d_sinks)))
    return fail(ATTN_ERR_ALIGN, "sinks and d_sinks must be 4-byte aligned");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) || !aligned16(a->d_o) ||
      !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv) || !aligned4(a->lse))
    return fail(ATTN_ERR_ALIGN, "bf16 tensors must be 16-byte aligned, lse 4-byte aligned");
  const int64_t st[] = {a->q_sb, a->q_sh, a->q_ss, a->k_sb, a->k_sh, a->k_ss};
  for (int64_t s : st)
    if (!bf16_stride_ok(s)) return fail(ATTN_ERR_STRIDE, "bf16 strides must be non-negative multiples of 8 elements");
  if (a->lse_sb < 0 || a->lse_sh < 0) return fail(ATTN_ERR_STRIDE, "lse strides must be >= 0");
  if (a->q_ss >= kMaxRowStride || a->k_ss >= kMaxRowStride)
    return fail(ATTN_ERR_STRIDE, "row strides must be below 2^24 elements");
  if ((int64_t)a->b * a->h_q * ((a->s_q + 127) / 128) > INT32_MAX ||
      (int64_t)a->b * a->h_kv * ((a->s_k + 127) / 128) > INT32_MAX)
    return fail(ATTN_ERR_SHAPE, "backward grid too large");
  const size_t need = attn_bwd_workspace_size(a->b, a->h_q, a->s_q);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (a->s_q == 0 && a->s_k == 0 && a->d_sinks == nullptr) return ok();

  attn::BwdParams p;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.o = static_cast<const uint16_t *>(a->o);
  p.d_o = static_cast<const uint16_t *>(a->d_o);
  p.lse = a->lse;
  p.dq = static_cast<uint16_t *>(a->dq);
  p.dk = static_cast<uint16_t *>(a->dk);
  p.dv = static_cast<uint16_t *>(a->dv);
  p.dsum = static_cast<float *>(workspace);
  const size_t rows = (size_t)a->b * a->h_q * (size_t)(a->s_q > 0 ? a->s_q : 1);
  const size_t rows_bytes = (rows * 4 + 255) / 256 * 256;
  p.lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + rows_bytes);
  p.window = a->window;
  p.sinks = a->sinks;
  p.d_sinks = a->d_sinks;
  p.dsink_part = a->d_sinks ? reinterpret_cast<float *>(static_cast<char *>(workspace) + 2 * rows_bytes) : nullptr;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_ss = a->q_ss;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_ss = a->k_ss;
  p.lse_sb = a->lse_sb; p.lse_sh = a->lse_sh;
  p.b = a->b; p.h_q = a->h_q; p.h_kv = a->h_kv; p.s_q = a->s_q; p.s_k = a->s_k;
  p.ratio = a->h_q / a->h_kv;
  p.c = a->scale * attn::kLog2e;
  p.scale = a->scale;
  hipError_t e = attn::backward(a->d, p, a->causal != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

attn_status attn_combine(const attn_combine_args *a, void *stream) {
  if (a == nullptr) return fail(ATTN_ERR_NULL, "args is NULL");
  if (a->n_parts < 1 || a->n_parts > 1024) return fail(ATTN_ERR_SHAPE, "n_parts must be in [1, 1024]");
  if (a->rows < 0) return fail(ATTN_ERR_SHAPE, "rows must be >= 0");
  if (a->d < 8 || a->d > 512 || a->d % 8 != 0) return fail(ATTN_ERR_SHAPE, "d must be a multiple of 8 in [8, 512]");
  if (a->rows == 0) return ok();
  if (!a->o_parts || !a->lse_parts || !a->o_out) return fail(ATTN_ERR_NULL, "o_parts, lse_parts and o_out must be non-NULL");
  if (!aligned16(a->o_parts) || !aligned16(a->o_out) || !aligned4(a->lse_parts) ||
      (a->lse_out && !aligned4(a->lse_out)))
    return fail(ATTN_ERR_ALIGN, "o_parts and o_out must be 16-byte aligned, LSE pointers 4-byte aligned");
  if (a->o_part_stride < 0 || a->o_row_stride < 0 || a->o_part_stride % 4 || a->o_row_stride % 4)
    return fail(ATTN_ERR_STRIDE, "o_parts strides must be non-negative multiples of 4 elements");
  if (a->lse_part_stride < 0 || a->lse_row_stride < 0) return fail(ATTN_ERR_STRIDE, "LSE strides must be >= 0");
  if (!bf16_stride_ok(a->o_out_row_stride)) return fail(ATTN_ERR_STRIDE, "o_out_row_stride must be a non-negative multiple of 8");

  attn::CombineParams c;
  c.kv_len = nullptr;  // every row merges all n_parts
  c.split = 0;
  c.o_parts = a->o_parts;
  c.lse_parts = a->lse_parts;
  c.o_out = static_cast<uint16_t *>(a->o_out);
  c.lse_out = a->lse_out;
  c.n_parts = a->n_parts;
  c.rows = a->rows;
  c.n2 = 1;
  c.d = a->d;
  c.o_part_stride = a->o_part_stride;
  c.o_r1 = a->o_row_stride;
  c.o_r2 = 0;
  c.lse_part_stride = a->lse_part_stride;
  c.lse_r1 = a->lse_row_stride;
  c.lse_r2 = 0;
  c.out_r1 = a->o_out_row_stride;
  c.out_r2 = 0;
  c.lse_out_r1 = 1;
  c.lse_out_r2 = 0;
  hipError_t e = attn::combine(c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

}  // extern "C"

namespace attn {
// d = 128 and 256 run the 8-wave ping-pong kernel on 256 rows and d = 64 the
// 8-wave single-group kernel on 256 rows, except that a sliding window at
// d = 64 and 128 keeps the 4-wave kernel on 128 rows: with the window's two
// masked edges, the smaller tile wastes less of each tile range.
int prefill_block_rows(int d, int mask) {
  switch (d) {
    case 64: return mask == kMaskCausalWindow ? 128 : 256;
    case 128: return mask == kMaskCausalWindow ? 128 : 256;
    case 256: return 256;
    case 512: return 128;
    default: return 0;
  }
}

int prefill_block_keys(int d, int mask) {
  (void)mask;
  switch (d) {
    case 64: case 128: return 64;
    case 256: return 32;
    case 512: return 32;
    default: return 0;
  }
}
}  // namespace attn

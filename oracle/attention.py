"""Plain fp64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library and imports nothing from the
``attention_forward_attn_amd`` package.

What it computes, and where the pages define it:

* ``attention_ref`` -- O = softmax(scale * Q K^T + mask) V with an optional
  per-row log-sum-exp.  It materialises the score matrix, so it is the plain
  definition that the streaming algorithm of the FA4 planner page
  ("b200-flash-attention4-planner", section A1 "Streaming online softmax" and
  Executable step 2 "Define the streaming state") must reproduce exactly up
  to rounding.  Masks: causal (planner page, step 7 "Implement mask/GQA"),
  sliding window combined with causal (DSV4 status page
  "archived_plans/2026-05-28_STATUS.md", rows D3 and D4), attention sink
  (same page, row D5c) and GQA/MQA head mapping (planner page step 7; status
  page row D2 "head-packed MQA/GQA").  The per-row LSE is row D5b of the
  status page.
* ``online_softmax_ref`` -- the streaming recurrence itself, taken block by
  block in the order the planner page's section A1 lists its steps: score,
  new row max, rescale of the old row sum and O, numerator, accumulate, and
  the division by the row sum only at the very end.
* ``merge_ref`` -- combining results over disjoint key sets by their
  per-segment LSE (STAGE_D.md page of nvfp4-megamoe-kernel, the "O rescale
  (kt>0)" workaround paragraph, and its section 2 "External k_sub Merge is
  Mathematically Impossible", which limits it to disjoint token sets).
* ``decode_ref`` / ``decode_split_ref`` -- single-token decode over a packed
  per-sequence KV cache, unsplit and split into fixed-size key chunks.
* ``decode_paged_ref`` -- the same decode over a paged KV cache addressed
  through a block table (reading of the layout stated in its docstring).
* ``attention_backward_ref`` -- dQ, dK, dV of the attention output for an
  incoming gradient dO (reading stated in its docstring).
* ``decode_fp8_ref`` -- the same decode over an FP8 (E4M3) KV cache with a
  per-kv-head scale for K and for V (``fp8_e4m3_value`` decodes the codes from
  the format's definition).

Readings taken where the pages are silent or garbled (each is stated again
where it is used):

* LSE is the natural log of the softmax denominator of the *scaled* logits,
  including the sink column.
* Causal masking is bottom-right aligned: with o = s_k - s_q, key j is
  visible to query row i iff j <= i + o.
* A window of W keys keeps keys j >= i + o - W + 1 (W keys including the
  diagonal); a window is only defined together with the causal mask.
* A sink is one extra softmax column per query head whose logit sigma_h is
  taken as is (not multiplied by ``scale``) and whose value row is zero.
* GQA maps query head h to kv head floor(h / (h_q / h_kv)).
* A row with no visible key and no sink has O = 0 and LSE = -inf.

Arithmetic is float64 throughout; the only library primitives used are
matrix products, ``exp``, ``log`` and reductions.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    """Convert a numpy array or torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor: upcast exactly, then hand to numpy
        x = x.detach().to("cpu")
        import torch  # local import: torch is optional for pure-numpy callers

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def visible_keys(s_q: int, s_k: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [s_q, s_k] matrix: True where key j is visible to query row i.

    Causal masking is bottom-right aligned (o = s_k - s_q): key j is visible
    iff j <= i + o.  A window W > 0 further requires j >= i + o - W + 1, so a
    full row sees exactly W keys including its diagonal.  Planner page,
    executable step 7 (causal tiles), and the DSV4 status page rows D3/D4
    (sliding-window length mask, combined with causal).
    """
    if window < 0:
        raise ValueError("window must be >= 0")
    if window > 0 and not causal:
        raise ValueError("a sliding window is only defined together with the causal mask")
    o = s_k - s_q
    i = np.arange(s_q)[:, None]
    j = np.arange(s_k)[None, :]
    vis = np.ones((s_q, s_k), dtype=bool)
    if causal:
        vis &= j <= i + o
    if window > 0:
        vis &= j >= i + o - window + 1
    return vis


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [b, h, s, d]")
    b, h_q, _, d = q.shape
    bk, h_kv, s_k, dk = k.shape
    if k.shape != v.shape or bk != b or dk != d:
        raise ValueError("k and v must be [b, h_kv, s_k, d] matching q")
    if h_kv <= 0 or h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    return b, h_q, h_kv, s_k, d


def attention_ref(q, k, v, scale: float, causal: bool = False, window: int = 0,
                  sinks=None, row_chunk: int = 1024):
    """Plain attention: returns (O [b,h_q,s_q,d], LSE [b,h_q,s_q]) in float64.

    For every batch b, query head h (kv head g = h // (h_q // h_kv)) and query
    row i, with the visible key set V(i) from ``visible_keys``:

        s_ij  = scale * sum_t Q[b,h,i,t] * K[b,g,j,t]
        m     = max(max_{j in V(i)} s_ij, sigma_h if a sink is present)
        Z     = sum_{j in V(i)} exp(s_ij - m) + [sink] exp(sigma_h - m)
        O_i   = sum_{j in V(i)} exp(s_ij - m) V[b,g,j,:] / Z
        LSE_i = m + ln Z

    A row with an empty visible set and no sink gets O_i = 0, LSE_i = -inf.
    Rows are processed in chunks of ``row_chunk`` to bound memory; the chunks
    are independent (no blocking over keys).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    b, h_q, h_kv, s_k, d = _check_shapes(q, k, v)
    s_q = q.shape[2]
    ratio = h_q // h_kv
    sig = None if sinks is None else _as_f64(sinks).reshape(-1)
    if sig is not None and sig.shape[0] != h_q:
        raise ValueError("sinks must hold one logit per query head")
    vis = visible_keys(s_q, s_k, causal, window)
    out = np.zeros((b, h_q, s_q, d))
    lse = np.full((b, h_q, s_q), NEG_INF)
    for bi in range(b):
        for h in range(h_q):
            g = h // ratio
            kg = k[bi, g]
            vg = v[bi, g]
            for i0 in range(0, s_q, row_chunk):
                i1 = min(s_q, i0 + row_chunk)
                s = scale * (q[bi, h, i0:i1] @ kg.T)
                s = np.where(vis[i0:i1], s, NEG_INF)
                m = s.max(axis=1) if s_k > 0 else np.full(i1 - i0, NEG_INF)
                if sig is not None:
                    m = np.maximum(m, sig[h])
                finite = np.isfinite(m)
                m_safe = np.where(finite, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                z = e.sum(axis=1)
                if sig is not None:
                    z = z + np.exp(sig[h] - m_safe)
                num = e @ vg
                nonempty = z > 0
                out[bi, h, i0:i1] = np.where(nonempty[:, None],
                                             num / np.where(nonempty, z, 1.0)[:, None], 0.0)
                lse[bi, h, i0:i1] = np.where(nonempty, m_safe + np.log(np.where(nonempty, z, 1.0)),
                                             NEG_INF)
    return out, lse


def online_softmax_ref(q, k, v, scale: float, causal: bool = False, window: int = 0,
                       sinks=None, block_n: int = 64):
    """The streaming (online-softmax) recurrence, one key block at a time, fp64.

    Follows the planner page's section A1 "Streaming online softmax" in its
    own order.  Per query row the running state is (m, l, acc), initialised
    to (-inf, 0, 0) -- or to (sigma_h, 1, 0) when a sink column with zero
    value is present.  For every block of ``block_n`` keys:

        S      = scale * Q K_blk^T, masked to -inf outside the visible set
        m_new  = max(m, rowmax(S))
        alpha  = exp(m - m_new)            (rescales the old l and acc)
        P      = exp(S - m_new)
        l      = alpha * l + rowsum(P)
        acc    = alpha * acc + P V_blk
        m      = m_new

    and only after the last block O = acc / l, LSE = m + ln l.  Natural exp
    is used here; the equivalent exp2 form only rescales the exponent.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    b, h_q, h_kv, s_k, d = _check_shapes(q, k, v)
    s_q = q.shape[2]
    ratio = h_q // h_kv
    sig = None if sinks is None else _as_f64(sinks).reshape(-1)
    vis = visible_keys(s_q, s_k, causal, window)
    out = np.zeros((b, h_q, s_q, d))
    lse = np.full((b, h_q, s_q), NEG_INF)
    for bi in range(b):
        for h in range(h_q):
            g = h // ratio
            if sig is None:
                m = np.full(s_q, NEG_INF)
                l = np.zeros(s_q)
            else:
                m = np.full(s_q, sig[h])
                l = np.ones(s_q)
            acc = np.zeros((s_q, d))
            for j0 in range(0, s_k, block_n):
                j1 = min(s_k, j0 + block_n)
                s = scale * (q[bi, h] @ k[bi, g, j0:j1].T)
                s = np.where(vis[:, j0:j1], s, NEG_INF)
                m_new = np.maximum(m, s.max(axis=1))
                # rows whose running max is still -inf have seen nothing yet:
                # their state stays (l=0, acc=0) and the exponent base is 0
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                p = np.exp(s - base[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[bi, g, j0:j1]
                m = m_new
            nonempty = l > 0
            out[bi, h] = np.where(nonempty[:, None], acc / np.where(nonempty, l, 1.0)[:, None], 0.0)
            lse[bi, h] = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)), NEG_INF)
    return out, lse


def merge_ref(o_parts, lse_parts):
    """Merge results computed over DISJOINT key sets by their per-part LSE.

    ``o_parts`` is [n, ..., d] (each part already normalised), ``lse_parts``
    is [n, ...] (natural log).  With M = max_i lse_i and w_i = exp(lse_i - M):

        O   = sum_i w_i O_i / sum_i w_i
        LSE = M + ln sum_i w_i

    A part with lse = -inf has weight zero (its O is never read); if every
    part is -inf the row is empty: O = 0, LSE = -inf.  This is the merge of
    the STAGE_D.md page ("O rescale (kt>0)" workaround paragraph).  It is NOT
    valid for partial dot products over the same keys (that page's section 2).
    """
    o = _as_f64(o_parts)
    l = _as_f64(lse_parts)
    m = l.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - m_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    o_safe = np.where(np.isfinite(l)[..., None], o, 0.0)
    num = (w[..., None] * o_safe).sum(axis=0)
    nonempty = wsum > 0
    out = np.where(nonempty[..., None], num / np.where(nonempty, wsum, 1.0)[..., None], 0.0)
    lse = np.where(nonempty, m_safe + np.log(np.where(nonempty, wsum, 1.0)), NEG_INF)
    return out, lse


def decode_ref(q, k, v, kv_start, kv_len, scale: float, sinks=None):
    """Single-token decode: query b attends to keys [kv_start[b], kv_start[b]+kv_len[b]).

    q is [B, h_q, d]; k and v are a packed cache [T, h_kv, d] (token-major,
    contiguous per sequence).  Every cached key is visible (bottom-right
    causal alignment with one query row).  Returns O [B,h_q,d], LSE [B,h_q].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    starts = np.asarray(kv_start, dtype=np.int64).reshape(-1)
    lens = np.asarray(kv_len, dtype=np.int64).reshape(-1)
    B, h_q, d = q.shape
    out = np.zeros((B, h_q, d))
    lse = np.zeros((B, h_q))
    for bi in range(B):
        s0, n = int(starts[bi]), int(lens[bi])
        kb = np.transpose(k[s0:s0 + n], (1, 0, 2))[None]
        vb = np.transpose(v[s0:s0 + n], (1, 0, 2))[None]
        o, l = attention_ref(q[bi][None, :, None, :], kb, vb, scale, sinks=sinks)
        out[bi] = o[0, :, 0]
        lse[bi] = l[0, :, 0]
    return out, lse


def decode_split_ref(q, k, v, kv_start, kv_len, scale: float, split: int, sinks=None):
    """Split-KV decode: per-chunk partial results, then their LSE merge.

    Chunk c of sequence b holds keys [c*split, min((c+1)*split, L_b)).  Each
    chunk gives a normalised partial O_c and LSE_c (chunks past L_b give
    LSE = -inf); a sink, if present, enters the merge once as an extra part
    with zero output and LSE = sigma_h.  Returns (O, LSE, parts_o, parts_lse)
    where the parts are [n_chunks, B, h_q, (d)].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    starts = np.asarray(kv_start, dtype=np.int64).reshape(-1)
    lens = np.asarray(kv_len, dtype=np.int64).reshape(-1)
    B, h_q, d = q.shape
    n_chunks = max(1, int(math.ceil(int(lens.max()) / split)))
    po = np.zeros((n_chunks, B, h_q, d))
    pl = np.full((n_chunks, B, h_q), NEG_INF)
    for bi in range(B):
        for c in range(n_chunks):
            j0 = c * split
            j1 = min(int(lens[bi]), j0 + split)
            if j1 <= j0:
                continue
            s0 = int(starts[bi])
            kb = np.transpose(k[s0 + j0:s0 + j1], (1, 0, 2))[None]
            vb = np.transpose(v[s0 + j0:s0 + j1], (1, 0, 2))[None]
            o, l = attention_ref(q[bi][None, :, None, :], kb, vb, scale)
            po[c, bi] = o[0, :, 0]
            pl[c, bi] = l[0, :, 0]
    if sinks is not None:
        sig = _as_f64(sinks).reshape(-1)
        po = np.concatenate([po, np.zeros((1, B, h_q, d))], axis=0)
        pl = np.concatenate([pl, np.broadcast_to(sig[None, None, :], (1, B, h_q))], axis=0)
    o, l = merge_ref(po, pl)
    return o, l, po, pl


def gather_pages(cache, block_table_row, n_tokens: int, page_size: int) -> np.ndarray:
    """Tokens 0..n_tokens-1 of one sequence out of a paged cache, in order.

    cache is [n_pages, page_size, h_kv, d]; token t lives in page
    block_table_row[t // page_size] at slot t % page_size.  Only the pages
    that hold one of the n_tokens tokens are touched.  Returns [n_tokens, h_kv, d].
    """
    cache = _as_f64(cache)
    table = np.asarray(block_table_row, dtype=np.int64).reshape(-1)
    out = np.zeros((n_tokens,) + cache.shape[2:])
    for t0 in range(0, n_tokens, page_size):
        n = min(page_size, n_tokens - t0)
        out[t0:t0 + n] = cache[int(table[t0 // page_size]), :n]
    return out


def decode_paged_ref(q, k_cache, v_cache, block_table, kv_len, page_size: int, scale: float,
                     sinks=None):
    """Single-token decode over a paged KV cache (block table), fp64.

    The pages ask for paged and dense caches to get kernels of their own
    (hard rules of the optimize-fa4-blackwell skill page) and list a paged
    cache in the serving infrastructure (DSV4 status page, the KV cache
    infrastructure row), but fix no layout.  Reading used: the cache is a pool of fixed-size pages
    [n_pages, page_size, h_kv, d]; row b of block_table lists the pages of
    sequence b in token order, so token t of the sequence is slot
    t % page_size of page block_table[b][t // page_size].  The attention is
    then exactly decode_ref over the gathered keys and values.
    Returns O [B,h_q,d], LSE [B,h_q].
    """
    q = _as_f64(q)
    lens = np.asarray(kv_len, dtype=np.int64).reshape(-1)
    B, h_q, d = q.shape
    out = np.zeros((B, h_q, d))
    lse = np.zeros((B, h_q))
    table = np.asarray(block_table)
    for bi in range(B):
        n = int(lens[bi])
        kb = np.transpose(gather_pages(k_cache, table[bi], n, page_size), (1, 0, 2))[None]
        vb = np.transpose(gather_pages(v_cache, table[bi], n, page_size), (1, 0, 2))[None]
        o, l = attention_ref(q[bi][None, :, None, :], kb, vb, scale, sinks=sinks)
        out[bi] = o[0, :, 0]
        lse[bi] = l[0, :, 0]
    return out, lse


def fp8_e4m3_value(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 ("e4m3fn") codes, float64.

    The format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; an
    all-zero exponent is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7
    is NaN; there are no infinities, so the largest finite value is 448.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def decode_fp8_ref(q, k_codes, v_codes, k_scale, v_scale, kv_start, kv_len, scale: float, sinks=None):
    """Decode over an FP8 KV cache: keys and values are E4M3 codes times a per-kv-head scale.

    The pages plan a KV cache in fewer bits that is widened again in on-chip
    memory for a deeper load pipeline (DSV4 status page, priority 7); they fix
    neither the format nor the scaling.  Reading used: 8-bit E4M3 codes [T, h_kv, d] with one fp32
    scale per kv head for K and one for V, K = code value * k_scale[g],
    V = code value * v_scale[g]; the attention is then exactly decode_ref on
    those values.  Returns O [B,h_q,d], LSE [B,h_q].
    """
    ks = _as_f64(k_scale).reshape(-1)
    vs = _as_f64(v_scale).reshape(-1)
    k = fp8_e4m3_value(np.asarray(k_codes)) * ks[None, :, None]
    v = fp8_e4m3_value(np.asarray(v_codes)) * vs[None, :, None]
    return decode_ref(q, k, v, kv_start, kv_len, scale, sinks=sinks)


def attention_backward_ref(q, k, v, d_o, scale: float, causal: bool = False, window: int = 0, sinks=None):
    """Gradients of the attention output: (dQ, dK, dV) in float64, shapes of q, k, v.

    The pages name the backward kernels and ask for a deterministic one (SM120
    research page, feature-parity and tuning notes) but define no algorithm
    beyond the forward; the planner page says a backward needs its own design.
    Reading used: the gradients of L = sum(dO * O) for O of attention_ref
    (no incoming gradient on the LSE), by the chain rule through the softmax,
    per batch b and query head h (kv head g), with the visible keys of
    ``visible_keys`` (causal and sliding-window masks):

        P    = softmax_j(scale * Q K^T + mask)          (rows that see no key: 0)
        dV_g = sum_{h in g} P^T dO
        dP   = dO V^T
        D_i  = sum_t dO[i,t] O[i,t]   (= sum_j P_ij dP_ij)
        dS   = P * (dP - D)
        dQ   = scale * dS K,   dK_g = sum_{h in g} scale * dS^T Q

    A sink sigma_h (DSV4 status page row D5c: one more softmax column per query
    head, logit taken as is, zero value row) enters the normalisation of P, so
    the formulas above hold with P over the real keys only; its own column has
    dP = 0, hence d sigma_h = sum_{b,i} P_i,sink * (0 - D_i), summed over the
    batch because the sink is shared by every sequence.  With ``sinks`` the
    result is (dQ, dK, dV, d_sinks [h_q]).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    d_o = _as_f64(d_o)
    b, h_q, h_kv, s_k, d = _check_shapes(q, k, v)
    s_q = q.shape[2]
    ratio = h_q // h_kv
    sig = None if sinks is None else _as_f64(sinks).reshape(-1)
    vis = visible_keys(s_q, s_k, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsig = np.zeros(h_q)
    for bi in range(b):
        for h in range(h_q):
            g = h // ratio
            s = scale * (q[bi, h] @ k[bi, g].T)
            s = np.where(vis, s, NEG_INF)
            m = s.max(axis=1) if s_k > 0 else np.full(s_q, NEG_INF)
            if sig is not None:
                m = np.maximum(m, sig[h])
            m_safe = np.where(np.isfinite(m), m, 0.0)
            num = np.exp(s - m_safe[:, None])
            z = num.sum(axis=1)
            if sig is not None:
                z = z + np.exp(sig[h] - m_safe)
            p = num / np.where(z > 0, z, 1.0)[:, None]
            o = p @ v[bi, g]
            dp = d_o[bi, h] @ v[bi, g].T
            dd = (d_o[bi, h] * o).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[bi, h] = scale * (ds @ k[bi, g])
            dk[bi, g] += scale * (ds.T @ q[bi, h])
            dv[bi, g] += p.T @ d_o[bi, h]
            if sig is not None:
                p_sink = np.exp(sig[h] - m_safe) / np.where(z > 0, z, 1.0)
                dsig[h] += (p_sink * (0.0 - dd)).sum()
    if sig is not None:
        return dq, dk, dv, dsig
    return dq, dk, dv


def attention_flops(b: int, h_q: int, s_q: int, s_k: int, d: int, causal: bool,
                    window: int = 0) -> int:
    """Algorithmic flop count: 4 * d per visible (query row, key) pair.

    Two multiply-adds per pair and head-dim element: one for Q K^T and one
    for P V.  Non-causal this is 4*b*h*s_q*s_k*d, the count the SM120 research
    page's forward TFLOPS table is computed with; causal and windowed runs
    count only visible pairs.
    """
    o = s_k - s_q
    pairs = 0
    for i in range(s_q):
        hi = s_k - 1 if not causal else min(s_k - 1, i + o)
        lo = 0 if window <= 0 else max(0, i + o - window + 1)
        if hi >= lo:
            pairs += hi - lo + 1
    return 4 * d * pairs * b * h_q

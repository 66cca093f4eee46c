"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes an oracle module (the real ``oracle.attention``,
or a copy with a planted mistake) and raises AssertionError when the oracle
disagrees with:

* hand-derived closed-form instances (``tests/golden/hand_cases.json``),
* an independent brute force in 50-digit ``decimal`` arithmetic, enumerating
  visible keys one by one with no max subtraction,
* closed forms and invariants: single key, identical keys (prefix mean),
  causal row 0, logit-shift invariance, the sink's sigmoid/logaddexp form,
  window limits, GQA = MHA on repeated heads, hard attention through a
  permutation, empty rows, the flop count,
* a textbook routine: torch's CPU fp64 ``scaled_dot_product_attention``,
* the paged-cache decode against the brute force on the keys it scattered,
* the backward gradients against torch's fp64 autograd,
* the FP8 E4M3 decoder against torch's float8_e4m3fn type on all 256 codes,
  and the FP8 decode against the brute force on torch-dequantized values,
* the streaming recurrence and the split/merge reformulation, and the
  negative result that merging head-dim halves is NOT attention.

The pages define the operation in the FA4 planner page (section A1 and
executable steps 2, 7, 9), the DSV4 status page (rows D2-D5c) and the
STAGE_D.md page (per-segment LSE merge; head-dim sub-tiles add in logit
space).
"""

from __future__ import annotations

import json
import math
import os
from decimal import Decimal, localcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
TOL = 1e-12


def _arr(x):
    """Nested lists from the JSON fixtures ("-inf" strings allowed) to float64."""
    return np.array(_conv(x), dtype=np.float64)


def _conv(x):
    if isinstance(x, list):
        return [_conv(e) for e in x]
    if isinstance(x, str):
        return float(x)  # "-inf"
    return x


def _close(got, want, tol=TOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    same_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    with np.errstate(invalid="ignore"):
        diff = np.where(same_inf, 0.0, np.abs(got - want))
    diff = np.where(np.isnan(diff), np.inf, diff)
    assert float(diff.max(initial=0.0)) <= tol, f"{what}: max abs diff {diff.max()} > {tol}"


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, scale, causal, window, sinks):
    """Attention by direct enumeration in 50-digit decimal arithmetic.

    Written independently of the oracle: keys are admitted one at a time by
    the visibility rule, weights are exp(logit) with no max subtraction, and
    every sum is an exact-ish decimal sum.
    """
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    out = np.zeros((b, h_q, s_q, d))
    lse = np.zeros((b, h_q, s_q))
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        for bi in range(b):
            for h in range(h_q):
                g = (h * h_kv) // h_q  # kv group of query head h
                for i in range(s_q):
                    terms = []
                    for j in range(s_k):
                        back = i + (s_k - s_q) - j  # how far key j lies behind the diagonal
                        if causal and back < 0:
                            continue
                        if window and back >= window:
                            continue
                        dot = sum(Decimal(float(q[bi, h, i, t])) * Decimal(float(k[bi, g, j, t]))
                                  for t in range(d))
                        terms.append(((sc * dot).exp(), j))
                    z = sum((w for w, _ in terms), Decimal(0))
                    if sinks is not None:
                        z += Decimal(float(sinks[h])).exp()
                    if z == 0:
                        out[bi, h, i] = 0.0
                        lse[bi, h, i] = -math.inf
                        continue
                    for t in range(d):
                        num = sum((w * Decimal(float(v[bi, g, j, t])) for w, j in terms), Decimal(0))
                        out[bi, h, i, t] = float(num / z)
                    lse[bi, h, i] = float(z.ln())
    return out, lse


BRUTE_CASES = [
    # b, h_q, h_kv, s_q, s_k, d, causal, window, sink, seed
    (1, 1, 1, 5, 5, 3, False, 0, False, 1),
    (2, 2, 1, 4, 6, 2, False, 0, False, 2),
    (1, 4, 2, 6, 6, 4, True, 0, False, 3),
    (1, 2, 2, 3, 7, 3, True, 0, True, 4),   # s_q < s_k, causal, sink
    (1, 2, 1, 7, 3, 2, True, 0, False, 5),  # s_q > s_k: leading empty rows
    (2, 3, 3, 6, 6, 2, True, 2, False, 6),  # window 2
    (1, 4, 1, 5, 8, 3, True, 3, True, 7),   # MQA + window + sink, s_q < s_k
    (1, 2, 2, 4, 4, 5, True, 9, False, 8),  # window wider than s_k
]


def pin_brute_force(orc):
    for (b, h_q, h_kv, s_q, s_k, d, causal, window, sink, seed) in BRUTE_CASES:
        rng = _rng(seed)
        q = rng.standard_normal((b, h_q, s_q, d))
        k = rng.standard_normal((b, h_kv, s_k, d))
        v = rng.standard_normal((b, h_kv, s_k, d))
        sinks = rng.standard_normal(h_q) * 2 if sink else None
        scale = 0.7 / math.sqrt(d)
        o, l = orc.attention_ref(q, k, v, scale, causal=causal, window=window, sinks=sinks)
        bo, bl = brute_force(q, k, v, scale, causal, window, sinks)
        tag = f"brute case seed={seed}"
        _close(o, bo, 1e-12, tag + " O")
        _close(l, bl, 1e-12, tag + " LSE")


# ---------------------------------------------------------------- golden

def pin_golden_hand_cases(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)
    for c in cases["attention"]:
        sinks = None if c["sinks"] is None else np.array(c["sinks"], dtype=np.float64)
        o, l = orc.attention_ref(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]), c["scale"],
                                 causal=c["causal"], window=c["window"], sinks=sinks)
        _close(o, _arr(c["o"]), 1e-12, c["name"] + " O")
        _close(l, _arr(c["lse"]), 1e-12, c["name"] + " LSE")
    for c in cases["merge"]:
        o, l = orc.merge_ref(_arr(c["o_parts"]), _arr(c["lse_parts"]))
        _close(o, _arr(c["o"]), 1e-12, c["name"] + " O")
        _close(l, _arr(c["lse"]), 1e-12, c["name"] + " LSE")


# ---------------------------------------------------------------- closed forms

def pin_single_key(orc):
    """One key: O = V_0 and LSE = scale * q.k_0 exactly."""
    rng = _rng(11)
    q = rng.standard_normal((2, 3, 4, 8))
    k = rng.standard_normal((2, 3, 1, 8))
    v = rng.standard_normal((2, 3, 1, 8))
    scale = 0.35
    o, l = orc.attention_ref(q, k, v, scale)
    _close(o, np.broadcast_to(v, o.shape), 1e-14, "single key O")
    want = scale * np.einsum("bhid,bhjd->bhi", q, k)
    _close(l, want, 1e-13, "single key LSE")


def pin_identical_keys_prefix_mean(orc):
    """All keys equal: O_i is the mean of the visible V rows (prefix mean if causal)."""
    rng = _rng(12)
    s, d = 9, 4
    q = rng.standard_normal((1, 2, s, d))
    k = np.broadcast_to(rng.standard_normal((1, 2, 1, d)), (1, 2, s, d)).copy()
    v = rng.standard_normal((1, 2, s, d))
    o, l = orc.attention_ref(q, k, v, 0.5, causal=False)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-13, "mean")
    o, l = orc.attention_ref(q, k, v, 0.5, causal=True)
    counts = np.arange(1, s + 1, dtype=np.float64)[None, None, :, None]
    _close(o, np.cumsum(v, axis=2) / counts, 1e-13, "prefix mean")
    logit = 0.5 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0])
    _close(l, logit + np.log(np.arange(1, s + 1))[None, None], 1e-13, "prefix LSE")


def pin_causal_row0(orc):
    """Causal with s_q = s_k: row 0 sees only key 0, so O_0 = V_0, LSE_0 = scale q_0.k_0."""
    rng = _rng(13)
    q = rng.standard_normal((1, 2, 6, 5))
    k = rng.standard_normal((1, 2, 6, 5))
    v = rng.standard_normal((1, 2, 6, 5))
    o, l = orc.attention_ref(q, k, v, 0.8, causal=True)
    _close(o[:, :, 0], v[:, :, 0], 1e-14, "causal row 0 O")
    _close(l[:, :, 0], 0.8 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-13,
           "causal row 0 LSE")


def pin_shift_invariance(orc):
    """Adding the same constant to every logit of a row leaves O and shifts LSE.

    The constant enters through one extra head-dim element: q gets a and every
    key gets c, adding scale*a*c to each logit of the row.
    """
    rng = _rng(14)
    q = rng.standard_normal((1, 2, 5, 3))
    k = rng.standard_normal((1, 2, 7, 3))
    v = rng.standard_normal((1, 2, 7, 3))
    a, c, scale = 3.0, -2.5, 0.6
    q2 = np.concatenate([q, np.full((1, 2, 5, 1), a)], axis=-1)
    k2 = np.concatenate([k, np.full((1, 2, 7, 1), c)], axis=-1)
    v2 = np.concatenate([v, rng.standard_normal((1, 2, 7, 1))], axis=-1)
    for causal in (False, True):
        o, l = orc.attention_ref(q, k, v, scale, causal=causal)
        o2, l2 = orc.attention_ref(q2, k2, v2, scale, causal=causal)
        _close(o2[..., :3], o, 1e-13, "shift O")
        _close(l2, l + scale * a * c, 1e-13, "shift LSE")


def pin_sink_closed_form(orc):
    """A zero-value sink column: O_s = O * sigmoid(LSE - sigma), LSE_s = logaddexp(LSE, sigma)."""
    rng = _rng(15)
    q = rng.standard_normal((2, 4, 6, 4))
    k = rng.standard_normal((2, 2, 6, 4))
    v = rng.standard_normal((2, 2, 6, 4))
    sig = np.array([-3.0, 0.0, 1.5, 4.0])
    for causal, window in ((False, 0), (True, 0), (True, 3)):
        o, l = orc.attention_ref(q, k, v, 0.5, causal=causal, window=window)
        os_, ls = orc.attention_ref(q, k, v, 0.5, causal=causal, window=window, sinks=sig)
        s = sig[None, :, None]
        _close(os_, o / (1.0 + np.exp(s - l))[..., None], 1e-13, "sink O")
        _close(ls, np.logaddexp(l, s), 1e-13, "sink LSE")
    # a sink at -inf is no sink
    o0, l0 = orc.attention_ref(q, k, v, 0.5, causal=True)
    o1, l1 = orc.attention_ref(q, k, v, 0.5, causal=True, sinks=np.full(4, -np.inf))
    _close(o1, o0, 1e-15, "sink -inf O")
    _close(l1, l0, 1e-15, "sink -inf LSE")


def pin_window_limits(orc):
    """W >= s_k is plain causal; W = 1 keeps only the diagonal key."""
    rng = _rng(16)
    s_q, s_k = 5, 8
    q = rng.standard_normal((1, 2, s_q, 3))
    k = rng.standard_normal((1, 2, s_k, 3))
    v = rng.standard_normal((1, 2, s_k, 3))
    oc, lc = orc.attention_ref(q, k, v, 0.4, causal=True)
    ow, lw = orc.attention_ref(q, k, v, 0.4, causal=True, window=s_k)
    _close(ow, oc, 1e-15, "wide window O")
    _close(lw, lc, 1e-15, "wide window LSE")
    o1, l1 = orc.attention_ref(q, k, v, 0.4, causal=True, window=1)
    off = s_k - s_q
    diag = np.arange(s_q) + off
    _close(o1, v[:, :, diag], 1e-14, "W=1 O")
    _close(l1, 0.4 * np.einsum("bhid,bhid->bhi", q, k[:, :, diag]), 1e-13, "W=1 LSE")


def pin_gqa_equals_mha_repeat(orc):
    """GQA with ratio r equals MHA on K, V with every kv head repeated r times."""
    rng = _rng(17)
    q = rng.standard_normal((2, 6, 5, 4))
    k = rng.standard_normal((2, 2, 7, 4))
    v = rng.standard_normal((2, 2, 7, 4))
    kr = np.repeat(k, 3, axis=1)
    vr = np.repeat(v, 3, axis=1)
    for causal in (False, True):
        o, l = orc.attention_ref(q, k, v, 0.5, causal=causal)
        o2, l2 = orc.attention_ref(q, kr, vr, 0.5, causal=causal)
        _close(o, o2, 1e-15, "gqa O")
        _close(l, l2, 1e-15, "gqa LSE")


def pin_hard_attention_permutation(orc):
    """One-hot keys and permuted one-hot queries: a closed form that catches a transposed operand.

    K = I, Q_i = alpha * e_pi(i): row i has logit alpha at key pi(i) and 0
    elsewhere, so O_i = (e^alpha V_pi(i) + sum_{j != pi(i)} V_j) / (e^alpha + n - 1)
    and LSE_i = ln(e^alpha + n - 1).  pi is not an involution, so Q K^T and
    K Q^T differ.
    """
    n = 6
    pi = np.array([2, 0, 5, 1, 3, 4])
    alpha = 2.0
    q = (alpha * np.eye(n)[pi])[None, None]
    k = np.eye(n)[None, None]
    v = _rng(18).standard_normal((1, 1, n, n))
    o, l = orc.attention_ref(q, k, v, 1.0)
    total = v[0, 0].sum(axis=0)
    ea = math.exp(alpha)
    want = np.stack([(ea * v[0, 0, pi[i]] + total - v[0, 0, pi[i]]) / (ea + n - 1) for i in range(n)])
    _close(o[0, 0], want, 1e-13, "hard attention O")
    _close(l[0, 0], np.full(n, math.log(ea + n - 1)), 1e-13, "hard attention LSE")


def pin_empty_rows(orc):
    """Causal with s_q > s_k: the first s_q - s_k rows see nothing (O = 0, LSE = -inf)."""
    rng = _rng(19)
    q = rng.standard_normal((1, 1, 6, 2))
    k = rng.standard_normal((1, 1, 2, 2))
    v = rng.standard_normal((1, 1, 2, 2))
    o, l = orc.attention_ref(q, k, v, 1.0, causal=True)
    assert np.all(o[0, 0, :4] == 0.0)
    assert np.all(np.isneginf(l[0, 0, :4]))
    assert np.all(np.isfinite(l[0, 0, 4:]))
    _close(o[0, 0, 4], v[0, 0, 0], 1e-14, "first non-empty row")


def pin_textbook_sdpa(orc):
    """torch's CPU float64 scaled_dot_product_attention (dense, causal, GQA)."""
    import torch
    import torch.nn.functional as F

    rng = _rng(20)
    for (b, h_q, h_kv, s_q, s_k, d) in ((2, 4, 4, 7, 7, 8), (1, 8, 2, 5, 9, 4), (1, 4, 1, 9, 9, 6)):
        q = rng.standard_normal((b, h_q, s_q, d))
        k = rng.standard_normal((b, h_kv, s_k, d))
        v = rng.standard_normal((b, h_kv, s_k, d))
        for causal in (False, True):
            mask = None
            if causal:
                mask = torch.ones(s_q, s_k, dtype=torch.bool).tril(diagonal=s_k - s_q)
            want = F.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
                scale=0.3, enable_gqa=(h_q != h_kv)).numpy()
            o, _ = orc.attention_ref(q, k, v, 0.3, causal=causal)
            _close(o, want, 1e-12, f"sdpa {b},{h_q},{h_kv},{s_q},{s_k},{d} causal={causal}")


# ---------------------------------------------------------------- reformulations

def pin_online_equals_plain(orc):
    """The block-by-block streaming recurrence equals plain softmax to 1e-12."""
    rng = _rng(21)
    q = rng.standard_normal((1, 4, 13, 5)) * 2
    k = rng.standard_normal((1, 2, 17, 5)) * 2
    v = rng.standard_normal((1, 2, 17, 5))
    sig = rng.standard_normal(4)
    for causal, window, sinks in ((False, 0, None), (True, 0, None), (True, 4, sig), (False, 0, sig)):
        o, l = orc.attention_ref(q, k, v, 0.9, causal=causal, window=window, sinks=sinks)
        for bn in (1, 3, 8, 64):
            o2, l2 = orc.online_softmax_ref(q, k, v, 0.9, causal=causal, window=window,
                                            sinks=sinks, block_n=bn)
            _close(o2, o, 1e-12, f"online O bn={bn}")
            _close(l2, l, 1e-12, f"online LSE bn={bn}")


def _decode_case(seed, B=4, h_q=4, h_kv=2, d=4, lens=(1, 5, 12, 9)):
    rng = _rng(seed)
    lens = np.array(lens[:B])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    T = int(lens.sum()) + 3  # the cache may hold tokens past the last sequence
    q = rng.standard_normal((B, h_q, d))
    k = rng.standard_normal((T, h_kv, d))
    v = rng.standard_normal((T, h_kv, d))
    return q, k, v, starts, lens


def pin_decode_matches_brute(orc):
    """Decode over a packed cache equals the brute force on each sequence alone."""
    q, k, v, starts, lens = _decode_case(22)
    sig = np.array([0.5, -1.0, 2.0, 0.0])
    for sinks in (None, sig):
        o, l = orc.decode_ref(q, k, v, starts, lens, 0.45, sinks=sinks)
        for bi in range(len(lens)):
            kb = np.transpose(k[starts[bi]:starts[bi] + lens[bi]], (1, 0, 2))[None]
            vb = np.transpose(v[starts[bi]:starts[bi] + lens[bi]], (1, 0, 2))[None]
            bo, bl = brute_force(q[bi][None, :, None, :], kb, vb, 0.45, False, 0, sinks)
            _close(o[bi], bo[0, :, 0], 1e-12, "decode O")
            _close(l[bi], bl[0, :, 0], 1e-12, "decode LSE")


def pin_paged_decode_matches_brute(orc):
    """Decode through a block table equals the brute force on each sequence's own keys.

    The keys and values are drawn per sequence, then scattered to randomly
    chosen physical pages of a pool whose other slots hold NaN, so reading a
    wrong page or slot shows up as NaN or as a wrong value.
    """
    rng = _rng(25)
    B, h_q, h_kv, d = 3, 4, 2, 4
    lens = [7, 1, 12]
    sig = np.array([0.5, -1.0, 2.0, 0.0])
    for P in (1, 3, 4, 16):
        n_pages = sum(-(-L // P) for L in lens) + 5
        kc = np.full((n_pages, P, h_kv, d), np.nan)
        vc = np.full((n_pages, P, h_kv, d), np.nan)
        perm = rng.permutation(n_pages)
        table = np.full((B, max(-(-L // P) for L in lens)), -1, dtype=np.int64)
        q = rng.standard_normal((B, h_q, d))
        keys, vals, used = [], [], 0
        for bi, L in enumerate(lens):
            kb = rng.standard_normal((L, h_kv, d))
            vb = rng.standard_normal((L, h_kv, d))
            keys.append(kb)
            vals.append(vb)
            for pg in range(-(-L // P)):
                phys = int(perm[used])
                used += 1
                table[bi, pg] = phys
                n = min(P, L - pg * P)
                kc[phys, :n] = kb[pg * P:pg * P + n]
                vc[phys, :n] = vb[pg * P:pg * P + n]
        for sinks in (None, sig):
            o, l = orc.decode_paged_ref(q, kc, vc, table, np.array(lens), P, 0.45, sinks=sinks)
            for bi in range(B):
                kb = np.transpose(keys[bi], (1, 0, 2))[None]
                vb = np.transpose(vals[bi], (1, 0, 2))[None]
                bo, bl = brute_force(q[bi][None, :, None, :], kb, vb, 0.45, False, 0, sinks)
                _close(o[bi], bo[0, :, 0], 1e-12, f"paged decode O (page size {P})")
                _close(l[bi], bl[0, :, 0], 1e-12, f"paged decode LSE (page size {P})")


def pin_fp8_codes_match_library(orc):
    """All 256 E4M3 codes decode to torch's float8_e4m3fn values (NaN where torch gives NaN)."""
    import torch

    codes = np.arange(256)
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.fp8_e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN codes differ"
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), "E4M3 values differ"


def pin_fp8_decode_matches_brute(orc):
    """FP8 decode equals the brute force on values dequantized through torch's float8 type."""
    import torch

    rng = _rng(26)
    B, h_q, h_kv, d = 3, 4, 2, 4
    lens = np.array([5, 1, 9])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    T = int(lens.sum())
    q = rng.standard_normal((B, h_q, d))
    kc = torch.from_numpy(np.clip(rng.standard_normal((T, h_kv, d)) * 3, -448, 448)).to(torch.float8_e4m3fn)
    vc = torch.from_numpy(np.clip(rng.standard_normal((T, h_kv, d)) * 3, -448, 448)).to(torch.float8_e4m3fn)
    ks, vs = np.array([0.75, 1.5]), np.array([2.0, 0.25])
    kd = kc.to(torch.float64).numpy() * ks[None, :, None]
    vd = vc.to(torch.float64).numpy() * vs[None, :, None]
    sig = np.array([0.5, -1.0, 2.0, 0.0])
    for sinks in (None, sig):
        o, l = orc.decode_fp8_ref(q, kc.view(torch.uint8).numpy(), vc.view(torch.uint8).numpy(), ks, vs,
                                  starts, lens, 0.45, sinks=sinks)
        for bi in range(B):
            kb = np.transpose(kd[starts[bi]:starts[bi] + lens[bi]], (1, 0, 2))[None]
            vb = np.transpose(vd[starts[bi]:starts[bi] + lens[bi]], (1, 0, 2))[None]
            bo, bl = brute_force(q[bi][None, :, None, :], kb, vb, 0.45, False, 0, sinks)
            _close(o[bi], bo[0, :, 0], 1e-12, "fp8 decode O")
            _close(l[bi], bl[0, :, 0], 1e-12, "fp8 decode LSE")


def pin_backward_matches_autograd(orc):
    """dQ, dK, dV (and the sink gradient) equal torch's fp64 autograd through its textbook
    attention: GQA by repeated heads, the window as a band mask, the sink as a concatenated
    column of zero value."""
    import torch

    rng = _rng(27)
    for (b, h_q, h_kv, s_q, s_k, d, causal, window, with_sink) in [
            (1, 2, 2, 5, 5, 4, False, 0, False), (2, 4, 2, 6, 6, 3, True, 0, False),
            (1, 4, 1, 4, 7, 5, True, 0, False), (1, 2, 1, 7, 3, 2, True, 0, False),
            (2, 2, 1, 9, 9, 3, True, 3, False), (1, 2, 2, 6, 8, 4, True, 2, True),
            (2, 4, 2, 5, 5, 3, False, 0, True), (1, 2, 1, 7, 3, 2, True, 0, True)]:
        q = rng.standard_normal((b, h_q, s_q, d))
        k = rng.standard_normal((b, h_kv, s_k, d))
        v = rng.standard_normal((b, h_kv, s_k, d))
        do = rng.standard_normal((b, h_q, s_q, d))
        sig = rng.standard_normal(h_q) if with_sink else None
        res = orc.attention_backward_ref(q, k, v, do, 0.6, causal, window, sig)
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        r = h_q // h_kv
        kk = tk.repeat_interleave(r, dim=1)
        vv = tv.repeat_interleave(r, dim=1)
        s = 0.6 * tq @ kk.transpose(-1, -2)
        off = s_k - s_q
        keep = torch.ones(s_q, s_k, dtype=torch.bool)
        if causal:
            keep &= torch.arange(s_k)[None, :] <= torch.arange(s_q)[:, None] + off
        if window:
            keep &= torch.arange(s_k)[None, :] >= torch.arange(s_q)[:, None] + off - window + 1
        s = s.masked_fill(~keep, float("-inf"))
        if with_sink:
            ts = torch.tensor(sig, requires_grad=True)
            col = ts[None, :, None, None].expand(b, h_q, s_q, 1)
            p = torch.softmax(torch.cat([s, col], dim=-1), dim=-1)[..., :s_k]
        else:
            p = torch.softmax(s, dim=-1).nan_to_num(0.0)  # rows that see no key: zero
        o = p @ vv
        (o * torch.tensor(do)).sum().backward()
        _close(res[0], tq.grad.numpy(), 1e-10, "dQ")
        _close(res[1], tk.grad.numpy(), 1e-10, "dK")
        _close(res[2], tv.grad.numpy(), 1e-10, "dV")
        if with_sink:
            _close(res[3], ts.grad.numpy(), 1e-10, "d sinks")
        else:
            assert len(res) == 3


def pin_split_merge_equals_unsplit(orc):
    """Split-KV partials merged by LSE equal the unsplit decode (disjoint key sets)."""
    q, k, v, starts, lens = _decode_case(23)
    sig = np.array([0.5, -1.0, 2.0, 0.0])
    for sinks in (None, sig):
        o, l = orc.decode_ref(q, k, v, starts, lens, 0.45, sinks=sinks)
        for split in (1, 2, 4, 5, 64):
            o2, l2, po, pl = orc.decode_split_ref(q, k, v, starts, lens, 0.45, split, sinks=sinks)
            _close(o2, o, 1e-12, f"split {split} O")
            _close(l2, l, 1e-12, f"split {split} LSE")
            n_real = int(math.ceil(lens.max() / split))
            for bi, L in enumerate(lens):
                n_b = int(math.ceil(L / split))
                assert np.all(np.isfinite(pl[:n_b, bi])), "non-empty chunk with -inf LSE"
                assert np.all(np.isneginf(pl[n_b:n_real, bi])), "chunk past L_b not empty"


def pin_head_dim_halves_do_not_merge(orc):
    """Merging attention over the two halves of the head dim is NOT attention over all of it.

    The halves add in logit space (S = S_0 + S_1); the LSE merge applies only to
    disjoint key sets, so using it here must miss by far more than the 2e-2
    tolerance (STAGE_D.md page, section 2).
    """
    rng = _rng(24)
    q = rng.standard_normal((1, 2, 16, 8)) * 1.5
    k = rng.standard_normal((1, 2, 16, 8)) * 1.5
    v = rng.standard_normal((1, 2, 16, 8))
    o, l = orc.attention_ref(q, k, v, 0.5)
    lo = np.concatenate([np.ones(4), np.zeros(4)])  # keeps head-dim elements 0..3
    o0, l0 = orc.attention_ref(q * lo, k, v, 0.5)
    o1, l1 = orc.attention_ref(q * (1.0 - lo), k, v, 0.5)
    om, lm = orc.merge_ref(np.stack([o0, o1]), np.stack([l0, l1]))
    assert float(np.abs(om - o).max()) > 0.1, "head-dim halves merged like disjoint key sets"
    # logit-space accumulation of the two halves is exact
    s = 0.5 * (q[..., :4] @ np.swapaxes(k[..., :4], -1, -2) + q[..., 4:] @ np.swapaxes(k[..., 4:], -1, -2))
    p = np.exp(s - s.max(-1, keepdims=True))
    _close((p / p.sum(-1, keepdims=True)) @ v, o, 1e-12, "logit-space sum")


def pin_flop_count(orc):
    """4*d per visible pair: non-causal 4 b h s_q s_k d; causal square s(s+1)/2 pairs."""
    assert orc.attention_flops(2, 16, 4096, 4096, 128, False) == 4 * 2 * 16 * 4096 * 4096 * 128
    assert orc.attention_flops(1, 3, 100, 100, 64, True) == 4 * 64 * 3 * (100 * 101 // 2)
    # window W on a square causal problem: rows i < W see i+1 keys, later rows W keys
    s, W = 50, 7
    pairs = sum(min(i + 1, W) for i in range(s))
    assert orc.attention_flops(1, 1, s, s, 8, True, W) == 4 * 8 * pairs
    # every visible pair counted: compare with the mask
    assert orc.attention_flops(1, 1, 9, 13, 2, True, 4) == 4 * 2 * int(orc.visible_keys(9, 13, True, 4).sum())


PINS = [
    pin_brute_force,
    pin_golden_hand_cases,
    pin_single_key,
    pin_identical_keys_prefix_mean,
    pin_causal_row0,
    pin_shift_invariance,
    pin_sink_closed_form,
    pin_window_limits,
    pin_gqa_equals_mha_repeat,
    pin_hard_attention_permutation,
    pin_empty_rows,
    pin_textbook_sdpa,
    pin_online_equals_plain,
    pin_decode_matches_brute,
    pin_paged_decode_matches_brute,
    pin_fp8_codes_match_library,
    pin_fp8_decode_matches_brute,
    pin_backward_matches_autograd,
    pin_split_merge_equals_unsplit,
    pin_head_dim_halves_do_not_merge,
    pin_flop_count,
]

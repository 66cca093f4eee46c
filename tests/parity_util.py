"""Helpers of the GPU parity tests: oracle calls on the same bf16 inputs and the tolerance check.

Tolerances (stated for bf16 inputs and outputs): max |O_gpu - O_oracle| <= 2e-2
and max |LSE_gpu - LSE_oracle| <= 1e-3, with -inf LSE required to match exactly.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

O_TOL = 2e-2
LSE_TOL = 1e-3


def to_np(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def check(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o = to_np(o_gpu)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err_o = float(np.abs(o - o_ref).max(initial=0.0))
    assert err_o <= O_TOL, f"{what}: max |dO| = {err_o}"
    err_l = 0.0
    if lse_gpu is not None:
        l = to_np(lse_gpu)
        assert l.shape == lse_ref.shape
        ninf_g, ninf_r = np.isneginf(l), np.isneginf(lse_ref)
        assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf LSE rows differ"
        fin = ~ninf_r
        assert np.all(np.isfinite(l[fin])), f"{what}: non-finite LSE"
        err_l = float(np.abs(l[fin] - lse_ref[fin]).max(initial=0.0))
        assert err_l <= LSE_TOL, f"{what}: max |dLSE| = {err_l}"
    return err_o, err_l


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))


def oracle_rows(q, k, v, scale, causal, window, sinks, picks):
    """Oracle O and LSE of selected query rows (b, h, i) of a prefill problem.

    A row's result only depends on its own visible keys, so each picked row is
    an s_q = 1 problem over the keys up to its (bottom-right) diagonal; with
    s_q = 1 the causal/window rule then keeps exactly the row's visible keys.
    """
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    ratio = h_q // h_kv
    off = s_k - s_q
    o_out = np.zeros((len(picks), d))
    l_out = np.zeros(len(picks))
    sig_all = None if sinks is None else sinks.detach().cpu().double().numpy()
    for n, (bi, h, i) in enumerate(picks):
        g = h // ratio
        hi = s_k if not causal else max(0, min(s_k, i + off + 1))
        qi = q[bi, h, i:i + 1][None, None]
        kk = k[bi, g, :hi][None, None]
        vv = v[bi, g, :hi][None, None]
        sig = None if sig_all is None else sig_all[h:h + 1]
        o, l = oracle.attention_ref(qi, kk, vv, scale, causal=causal, window=window, sinks=sig)
        o_out[n] = o[0, 0, 0]
        l_out[n] = l[0, 0, 0]
    return o_out, l_out

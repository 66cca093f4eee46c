"""Helpers of the GPU parity tests: oracle calls on the same bf16 inputs and the tolerance check.

Tolerances (stated for bf16 inputs and outputs): max |O_gpu - O_oracle| <= 2e-2
and max |LSE_gpu - LSE_oracle| <= 1e-3, with -inf LSE required to match exactly.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


def oracle_full(q, k, v, scale, causal, window, sinks, workers=None):
    """Oracle O and LSE of every row of a prefill problem, one (batch, head) slice per task.

    The slices are independent problems, so each is handed to
    ``oracle.attention_ref`` unchanged; the tasks run on a thread pool (numpy
    releases the interpreter lock inside its kernels) with one BLAS thread per
    worker.
    """
    from threadpoolctl import threadpool_limits

    b, h_q, s_q, d = q.shape
    ratio = h_q // k.shape[1]
    qn, kn, vn = (t.detach().cpu().to(torch.float64).numpy() for t in (q, k, v))
    sig = None if sinks is None else sinks.detach().cpu().double().numpy()
    o_out = np.empty((b, h_q, s_q, d))
    l_out = np.empty((b, h_q, s_q))

    def one(bh):
        bi, h = divmod(bh, h_q)
        g = h // ratio
        o, l = oracle.attention_ref(qn[bi:bi + 1, h:h + 1], kn[bi:bi + 1, g:g + 1], vn[bi:bi + 1, g:g + 1],
                                    scale, causal=causal, window=window,
                                    sinks=None if sig is None else sig[h:h + 1])
        o_out[bi, h] = o[0, 0]
        l_out[bi, h] = l[0, 0]

    workers = workers or min(16, os.cpu_count() or 1)
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(b * h_q)))
    return o_out, l_out

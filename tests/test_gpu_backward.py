"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle.

Tolerance (the pages state none for the backward): max-abs error per tensor
within 2e-2 * max(1, max |reference|), the forward's O tolerance scaled by
the gradient's magnitude, since gradients are not bounded by 1 like O.
"""

import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as afa
import oracle
from attention_forward_attn_amd.inputs import prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def grad_check(got, want, what):
    g = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - want).max()
    tol = 2e-2 * max(1.0, np.abs(want).max())
    print(f"{what}: max-abs error {err:.2e} (tolerance {tol:.2e}, max |ref| {np.abs(want).max():.2f})")
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.3e}"


def run_case(b, h_q, h_kv, s_q, s_k, causal, seed, d=128):
    inp = prefill_inputs(b, h_q, h_kv, s_q, s_k, d, seed)
    gen = torch.Generator("cpu").manual_seed(seed + 99)
    d_o = torch.randn(b, h_q, s_q, d, generator=gen).to(torch.bfloat16)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    o, lse = afa.prefill(q, k, v, causal=causal)
    dq, dk, dv = afa.backward(q, k, v, o, d_o.to(DEV), lse, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward_ref(inp["q"], inp["k"], inp["v"], d_o, 1 / math.sqrt(d), causal)
    return (dq, dk, dv), (rq, rk, rv)


CASES = [
    # b, h_q, h_kv, s_q, s_k, causal
    (1, 2, 2, 100, 100, False),
    (2, 4, 2, 300, 300, True),
    (1, 4, 1, 129, 257, True),   # s_q < s_k
    (1, 2, 1, 257, 129, True),   # s_q > s_k: leading rows see no key
    (1, 2, 2, 64, 64, False),
    (1, 8, 2, 512, 512, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_small(case, d):
    print(f"backward case {case} d={d}", flush=True)
    got, want = run_case(*case, seed=51, d=d)
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        grad_check(g, w, f"{case} d={d} {name}")


def test_backward_long_heads():
    """Two heads at 2048 tokens: many key and row tiles, every output compared."""
    print("backward b1 h2 s2048 causal", flush=True)
    got, want = run_case(1, 2, 2, 2048, 2048, True, seed=52)
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        grad_check(g, w, name)


def test_backward_deterministic():
    inp = prefill_inputs(1, 4, 2, 300, 300, 128, 53)
    d_o = torch.randn(1, 4, 300, 128).to(torch.bfloat16).to(DEV)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    o, lse = afa.prefill(q, k, v, causal=True)
    r1 = afa.backward(q, k, v, o, d_o, lse, causal=True)
    r2 = afa.backward(q, k, v, o, d_o, lse, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))

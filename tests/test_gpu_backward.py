"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle.

Tolerance (the pages state none for the backward; derived from the
arithmetic).  bf16 keeps 8 significant bits, so each rounding is at most 2^-9
of the value rounded.  The kernels round P and dS to bf16 before the products
and round the gradients to bf16 at the end; the products sum many terms whose
rounding errors have random signs, so the error of every element stays within
a few 2^-9 of the tensor's scale.  Per tensor:

  * |got - ref| <= 8e-3 * max |ref| + e_D elementwise (about 4 * 2^-9 of the scale),
  * RMS(got - ref) <= r * RMS(ref), r = 5e-3 + RMS(e_D) / RMS(ref)   (about 2.5 * 2^-9),
  * cosine(got, ref) >= 1 - r^2 / 2 (what that RMS bound implies; 0.9999875 when e_D is 0).

e_D is the part of the error that comes from D: the kernels take
D_i = sum_t dO[i,t] O[i,t] from the forward's bf16 O (the oracle from its exact
O), so |D_gpu - D| <= delta_i = 2^-8 * sum_t |dO[i,t] O[i,t]|, which enters
dS = P (dP - D): e_D = scale * sum_j P_ij delta_i |K[j,t]| for dQ, the same sum
over the rows of every query head of the group with |Q[i,t]| for dK, and 0 for
dV.  It matters only where dP - D cancels (a row that sees one key, say).

Measured on the cases below: max-abs at most 3.6e-3 of max |ref| where e_D is
negligible, relative RMS 2.3e-3 to 2.7e-3, cosine at least 0.999996 (0.99999 for
a one-key window, where e_D dominates).
"""

import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as afa
import oracle
from attention_forward_attn_amd.inputs import WORKLOADS, backward_inputs, prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


MAX_REL = 8e-3    # max-abs error over max |ref|
RMS_REL = 5e-3    # RMS error over RMS of the reference


def grad_check(got, want, what, e_d=0.0):
    g = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    e = g - want
    scale = np.abs(want).max()
    bound = MAX_REL * scale + e_d
    worst = float((np.abs(e) / bound).max())
    ref_rms = max(float(np.sqrt((want * want).mean())), 1e-300)
    rms = float(np.sqrt((e * e).mean())) / ref_rms
    r = RMS_REL + float(np.sqrt(np.mean(np.square(e_d)))) / ref_rms
    cos = float((g * want).sum() / max(np.sqrt((g * g).sum() * (want * want).sum()), 1e-300))
    print(f"{what}: max-abs {np.abs(e).max():.2e}, worst error / bound {worst:.3f}, rel RMS {rms:.2e} (<= {r:.2e}), "
          f"cosine {cos:.7f}")
    assert worst <= 1.0, f"{what}: error above its bound (worst ratio {worst:.3f})"
    assert rms <= r, f"{what}: relative RMS error {rms:.3e} > {r:.3e}"
    assert cos >= 1.0 - 0.5 * r * r, f"{what}: cosine {cos:.7f} < {1.0 - 0.5 * r * r:.7f}"


def d_error_terms(inp, d_o, scale, causal, window, sinks):
    """e_D of dQ and dK (see the module docstring), from the oracle's forward in fp64."""
    q, k = inp["q"].double().numpy(), inp["k"].double().numpy()
    o, lse = oracle.attention_ref(inp["q"], inp["k"], inp["v"], scale, causal=causal, window=window, sinks=sinks)
    dn = 2.0 ** -8 * np.abs(d_o.double().numpy() * o).sum(-1)  # delta_i, [b, h_q, s_q]
    b, h_q, s_q, _ = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    vis = oracle.visible_keys(s_q, s_k, causal, window)
    eq = np.zeros_like(q)
    ek = np.zeros_like(k)
    for bi in range(b):
        for h in range(h_q):
            g = h // (h_q // h_kv)
            s = scale * q[bi, h] @ k[bi, g].T
            fin = np.isfinite(lse[bi, h])[:, None]
            pm = np.where(vis & fin, np.exp(np.where(vis, s, 0.0) - np.where(fin, lse[bi, h][:, None], 0.0)), 0.0)
            w = pm * dn[bi, h][:, None]
            eq[bi, h] = scale * w @ np.abs(k[bi, g])
            ek[bi, g] += scale * w.T @ np.abs(q[bi, h])
    return eq, ek


def run_case(b, h_q, h_kv, s_q, s_k, causal, seed, d=128, window=0, sink=False):
    """GPU gradients, oracle gradients and the e_D terms (dQ, dK, dV) of one problem."""
    inp = prefill_inputs(b, h_q, h_kv, s_q, s_k, d, seed, with_sinks=sink)
    gen = torch.Generator("cpu").manual_seed(seed + 99)
    d_o = torch.randn(b, h_q, s_q, d, generator=gen).to(torch.bfloat16)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    sd = inp["sinks"].to(DEV) if sink else None
    o, lse = afa.prefill(q, k, v, causal=causal, window=window, sinks=sd)
    got = afa.backward(q, k, v, o, d_o.to(DEV), lse, causal=causal, window=window, sinks=sd)
    torch.cuda.synchronize()
    sig = inp["sinks"] if sink else None
    want = oracle.attention_backward_ref(inp["q"], inp["k"], inp["v"], d_o, 1 / math.sqrt(d), causal, window, sig)
    eq, ek = d_error_terms(inp, d_o, 1 / math.sqrt(d), causal, window, sig)
    return got, want, (eq, ek, 0.0)


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
@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_small(case, d):
    print(f"backward case {case} d={d}", flush=True)
    got, want, ed = run_case(*case, seed=51, d=d)
    for name, g, w, e in zip(("dQ", "dK", "dV"), got, want, ed):
        grad_check(g, w, f"{case} d={d} {name}", e)


WINDOWED = [
    # b, h_q, h_kv, s_q, s_k, window, sink
    (1, 4, 2, 700, 700, 100, False),
    (2, 4, 1, 300, 500, 64, True),    # s_k > s_q, MQA, sink
    (1, 2, 2, 257, 129, 1, True),     # s_q > s_k, one-key window: leading rows see only the sink
    (1, 8, 2, 1100, 1100, 1024, True),
]


@pytest.mark.parametrize("case", WINDOWED, ids=[str(c) for c in WINDOWED])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_window_and_sink(case, d):
    """Sliding window and sink: dQ, dK, dV and the sink gradient against the oracle."""
    b, h_q, h_kv, s_q, s_k, window, sink = case
    print(f"backward window case {case} d={d}", flush=True)
    got, want, ed = run_case(b, h_q, h_kv, s_q, s_k, True, 54, d=d, window=window, sink=sink)
    for name, g, w, e in zip(("dQ", "dK", "dV"), got[:3], want[:3], ed):
        grad_check(g, w, f"{case} d={d} {name}", e)
    if sink:
        # d sigma_h sums terms exp(sigma_h - LSE_i) * D_i over the batch and the rows; the
        # bf16 inputs of each term (O, dO) bound its error, so the tolerance is
        # MAX_REL times the sum of the terms' magnitudes (from the oracle's forward).
        inp = prefill_inputs(b, h_q, h_kv, s_q, s_k, d, 54, with_sinks=True)
        d_o = torch.randn(b, h_q, s_q, d, generator=torch.Generator("cpu").manual_seed(54 + 99)).to(torch.bfloat16)
        o_ref, l_ref = oracle.attention_ref(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(d), causal=True,
                                            window=window, sinks=inp["sinks"])
        sig = inp["sinks"].double().numpy()
        p_sink = np.exp(sig[None, :, None] - l_ref)
        do_o = d_o.double().numpy() * o_ref
        terms = p_sink * do_o.sum(-1)
        # each term's own error, plus the D error delta_i carried by P_sink
        bound = (MAX_REL * np.abs(terms) + p_sink * 2.0 ** -8 * np.abs(do_o).sum(-1)).sum(axis=(0, 2))
        ds = got[3].cpu().double().numpy()
        err = np.abs(ds - want[3])
        print(f"{case} d={d} d_sinks: max-abs {err.max():.2e}, worst err/bound {(err / bound).max():.3f}")
        assert np.all(err <= bound), f"d_sinks error {err} above {bound}"


def test_backward_sink_gradient_without_rows():
    """s_q = 0: the sink gradient is zero (nothing else is written)."""
    q = torch.zeros(1, 4, 0, 128, dtype=torch.bfloat16, device=DEV)  # no storage: NULL pointers
    k = torch.randn(1, 4, 10, 128, device=DEV).to(torch.bfloat16)
    lse = torch.zeros(1, 4, 0, dtype=torch.float32, device=DEV)
    sinks = torch.randn(4, device=DEV)
    got = afa.backward(q, k, k, q, q, lse, causal=True, sinks=sinks)
    torch.cuda.synchronize()
    assert torch.equal(got[3], torch.zeros(4, device=DEV))
    assert torch.equal(got[1], torch.zeros_like(k)) and torch.equal(got[2], torch.zeros_like(k))


@pytest.mark.parametrize("d", [128, 256])
def test_backward_long_heads(d):
    """Two heads at 2048 tokens: many key and row tiles, every output compared."""
    print(f"backward b1 h2 s2048 causal d={d}", flush=True)
    got, want, ed = run_case(1, 2, 2, 2048, 2048, True, seed=52, d=d)
    for name, g, w, e in zip(("dQ", "dK", "dV"), got, want, ed):
        grad_check(g, w, f"d={d} {name}", e)


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.kind == "backward"])
def test_backward_workload_full_size(name):
    """A backward workload at its full size, in the bench's call: outputs pre-filled with NaN (a
    row never written fails), every element finite, and every element of two whole heads (the
    first of the first batch, the last of the last) against the oracle, which sees the same
    bf16 inputs for that head alone (MHA: a kv head's gradients come from its one query head)."""
    w = WORKLOADS[name]
    assert w.h_q == w.h_kv, "one query head per kv head"
    print(f"backward workload {name}", flush=True)
    inp = backward_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed)
    q, k, v, d_o = (inp[n].to(DEV) for n in ("q", "k", "v", "d_o"))
    o, lse = afa.prefill(q, k, v, causal=w.causal)
    nan = float("nan")
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(k, nan)
    afa.backward(q, k, v, o, d_o, lse, causal=w.causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for nm, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name}: {nm} has unwritten or non-finite elements"
    scale = 1 / math.sqrt(w.d)
    for bi, h in ((0, 0), (w.b - 1, w.h_q - 1)):
        one = {n: inp[n][bi:bi + 1, h:h + 1].contiguous() for n in ("q", "k", "v", "d_o")}
        want = oracle.attention_backward_ref(one["q"], one["k"], one["v"], one["d_o"], scale, w.causal, 0, None)
        eq, ek = d_error_terms(one, one["d_o"], scale, w.causal, 0, None)
        got = (dq[bi:bi + 1, h:h + 1], dk[bi:bi + 1, h:h + 1], dv[bi:bi + 1, h:h + 1])
        for nm, g, wt, e in zip(("dQ", "dK", "dV"), got, want, (eq, ek, 0.0)):
            grad_check(g, wt, f"{name} b={bi} h={h} {nm}", e)


@pytest.mark.parametrize("d", [128, 256])
def test_backward_deterministic(d):
    inp = prefill_inputs(1, 4, 2, 300, 300, d, 53)
    d_o = torch.randn(1, 4, 300, d).to(torch.bfloat16).to(DEV)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    o, lse = afa.prefill(q, k, v, causal=True)
    r1 = afa.backward(q, k, v, o, d_o, lse, causal=True)
    r2 = afa.backward(q, k, v, o, d_o, lse, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))

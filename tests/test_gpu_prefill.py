"""GPU parity of the prefill kernel against the fp64 oracle (through the C ABI).

Small problems are compared element by element over every output; they span
several query and key tiles and end in ragged tails.  The full-size workloads
run in the launch configuration the bench times and are compared on every row,
element by element, with NaN-filled outputs so that an unwritten row fails.
"""

import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as afa
import oracle
from attention_forward_attn_amd.inputs import WORKLOADS, prefill_inputs
from parity_util import check, oracle_full

pytestmark = pytest.mark.gpu

DEV = "cuda"


def run_case(b, h_q, h_kv, s_q, s_k, d, causal=False, window=0, sink=False, seed=7, scale=None,
             layout="bhsd", q_mul=1.0, chunked=True):
    inp = prefill_inputs(b, h_q, h_kv, s_q, s_k, d, seed, with_sinks=sink)
    q, k, v, sinks = inp["q"], inp["k"], inp["v"], inp["sinks"]
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if layout == "bshd":  # strided views of [b, s, h, d] storage
        qd = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
        kd = k.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
        vd = v.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    else:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = sinks.to(DEV) if sinks is not None else None
    out = torch.full((b, h_q, s_q, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((b, h_q, s_q), float("nan"), dtype=torch.float32, device=DEV)
    afa.prefill(qd, kd, vd, scale=scale, causal=causal, window=window, sinks=sd, out=out, lse=lse,
                chunked=chunked)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, causal=causal, window=window, sinks=sinks)
    return out, lse, o_ref, l_ref


SMALL = [
    # b, h_q, h_kv, s_q, s_k, d, causal, window, sink
    (1, 1, 1, 256, 256, 64, False, 0, False),   # the tiny single-head workload shape
    (1, 2, 2, 300, 300, 64, True, 0, False),
    (2, 4, 2, 257, 513, 128, False, 0, False),
    (1, 4, 4, 513, 257, 128, True, 0, False),   # s_q > s_k: leading empty rows
    (1, 4, 1, 384, 384, 128, True, 100, True),  # MQA + window + sink
    (2, 8, 2, 200, 777, 128, True, 64, False),
    (1, 2, 2, 129, 129, 256, False, 0, True),
    (1, 4, 2, 300, 300, 256, True, 0, False),
    (1, 2, 1, 1, 1000, 128, True, 0, False),    # one query row
    (1, 2, 1, 1000, 1, 64, False, 0, False),    # one key
    (1, 2, 2, 1, 1, 128, False, 0, False),
    (1, 4, 4, 65, 65, 64, True, 1, False),      # window of one key: O = V on the diagonal
    (1, 32, 1, 130, 130, 128, True, 0, True),   # GQA ratio 32
    (1, 2, 2, 200, 200, 512, False, 0, False),  # head dim 512: halves summed in logit space
    (1, 4, 2, 257, 300, 512, True, 0, True),
    (1, 2, 1, 150, 150, 512, True, 40, False),
    (1, 2, 2, 70, 33, 512, True, 0, False),     # s_q > s_k
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_prefill_small(case):
    b, h_q, h_kv, s_q, s_k, d, causal, window, sink = case
    print(f"prefill case {case}", flush=True)
    out, lse, o_ref, l_ref = run_case(b, h_q, h_kv, s_q, s_k, d, causal, window, sink)
    check(out, lse, o_ref, l_ref, str(case))


def chunked_workspace(b, h_q, h_kv, s_q, s_k, d, causal, window=0):
    """Workspace bytes the library's chunk plan asks for (0: single pass)."""
    q = torch.empty((b, h_q, s_q, d), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((b, h_kv, s_k, d), dtype=torch.bfloat16, device=DEV)
    a = afa._binding.prefill_args(q, k, k, q, None, None, 1.0 / math.sqrt(d), causal, window)
    return int(afa.load_library().attn_fwd_prefill_chunked_workspace_size(afa._binding.ctypes.byref(a)))


# d = 512 causal shapes whose key ranges the library cuts into chunks
# (key tiles of 32; the chunk length is the one the host plan's launch simulation picks)
CHUNKED = [
    # b, h_q, h_kv, s_q, s_k, sink
    (1, 1, 1, 1024, 1024, False),  # 8-tile chunks, up to 4 per 128-row query tile
    (1, 2, 1, 1000, 1100, True),   # GQA, s_k > s_q, ragged tail, sink in the first chunk only (8-tile chunks)
    (1, 2, 2, 700, 500, False),    # s_q > s_k: leading rows see no key, later chunks partly empty
    (2, 2, 2, 640, 640, True),
    (1, 3, 3, 3000, 3000, False),  # 16-tile chunks, up to 6 per query tile, ragged last query tile
    (2, 4, 4, 1536, 2048, False),  # 18-tile chunks, s_k > s_q
    (1, 8, 8, 2048, 2048, True),   # 20-tile chunks
]


@pytest.mark.parametrize("case", CHUNKED, ids=[str(c) for c in CHUNKED])
def test_prefill_chunked(case):
    b, h_q, h_kv, s_q, s_k, sink = case
    print(f"chunked prefill case {case}", flush=True)
    assert chunked_workspace(b, h_q, h_kv, s_q, s_k, 512, True) > 0, "shape is not chunked"
    out, lse, o_ref, l_ref = run_case(b, h_q, h_kv, s_q, s_k, 512, True, 0, sink)
    check(out, lse, o_ref, l_ref, f"chunked {case}")
    one, one_lse, _, _ = run_case(b, h_q, h_kv, s_q, s_k, 512, True, 0, sink, chunked=False)
    check(one, one_lse, o_ref, l_ref, f"single pass {case}")


EDGE_LENGTHS = [1, 17, 63, 64, 65, 255, 257, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("s", EDGE_LENGTHS)
def test_prefill_edge_lengths(s, d, causal):
    # lengths around the 64-key tiles and the 128/256-row query tiles
    out, lse, o_ref, l_ref = run_case(1, 2, 1, s, s, d, causal=causal, seed=s + d)
    check(out, lse, o_ref, l_ref, f"s={s} d={d} causal={causal}")


@pytest.mark.parametrize("ratio", [1, 2, 4, 8, 16, 32])
def test_prefill_gqa_ratios(ratio):
    out, lse, o_ref, l_ref = run_case(1, 32, 32 // ratio, 300, 300, 128, causal=True, seed=ratio)
    check(out, lse, o_ref, l_ref, f"ratio {ratio}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [1, 1024, 5000])
def test_prefill_window_sizes(window, d):
    # a one-key window, one shorter than the sequence, one longer than it
    out, lse, o_ref, l_ref = run_case(1, 2, 2, 1100, 1100, d, causal=True, window=window, sink=True,
                                      seed=window + d)
    check(out, lse, o_ref, l_ref, f"window {window} d={d}")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_prefill_strided_bshd(d):
    out, lse, o_ref, l_ref = run_case(2, 4, 2, 200, 200, d, causal=True, layout="bshd")
    check(out, lse, o_ref, l_ref, "bshd")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_prefill_extreme_logits(d):
    # Q x 30: near one-hot attention rows stress the running-max rescale
    out, lse, o_ref, l_ref = run_case(1, 2, 2, 200, 333, d, causal=True, q_mul=30.0)
    check(out, lse, o_ref, l_ref, "extreme")


@pytest.mark.parametrize("sig", [-1e4, 0.0, 20.0])
def test_prefill_sink_values(sig):
    inp = prefill_inputs(1, 4, 2, 150, 150, 128, 9)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    sinks = torch.full((4,), sig, dtype=torch.float32)
    out, lse = afa.prefill(q, k, v, causal=True, sinks=sinks.to(DEV))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(128),
                                        causal=True, sinks=sinks)
    check(out, lse, o_ref, l_ref, f"sink {sig}")


def test_gqa_matches_repeated_heads_bitwise():
    inp = prefill_inputs(1, 8, 2, 190, 190, 128, 11)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = afa.prefill(q, k, v, causal=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = afa.prefill(q, kr, vr, causal=True)
    # MQA through head stride 0: h_kv = h_q with a broadcast view
    o3, l3 = afa.prefill(q[:, :4], k[:, :1].expand(1, 4, 190, 128), v[:, :1].expand(1, 4, 190, 128),
                         causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1[:, :4], o3) and torch.equal(l1[:, :4], l3)


def test_prefill_deterministic_and_fully_written():
    inp = prefill_inputs(2, 4, 4, 333, 333, 128, 12, with_sinks=True)
    q, k, v, s = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), inp["sinks"].to(DEV)
    outs = []
    for fill in (float("nan"), 7.0):
        out = torch.full_like(q, fill)
        lse = torch.full((2, 4, 333), fill, dtype=torch.float32, device=DEV)
        afa.prefill(q, k, v, causal=True, window=50, sinks=s, out=out, lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0][0].float()).all() and torch.isfinite(outs[0][1]).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_prefill_empty_keys():
    q = torch.randn(1, 2, 40, 128, device=DEV).to(torch.bfloat16)
    k = torch.zeros(1, 2, 0, 128, device=DEV, dtype=torch.bfloat16)
    out, lse = afa.prefill(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_prefill_shift_invariance_exact():
    """Adding one head-dim element a to Q and b to every key adds scale*a*b to each logit."""
    d = 128
    inp = prefill_inputs(1, 2, 2, 160, 160, d, 13)
    q, k, v = inp["q"].clone(), inp["k"].clone(), inp["v"]
    q[..., -1] = 0
    k[..., -1] = 0
    o0, l0 = afa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    q[..., -1] = 4.0
    k[..., -1] = 2.0
    o1, l1 = afa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o0.float()).abs().max().item() <= 2e-2
    assert abs(((l1 - l0) - 8.0 / math.sqrt(d)).abs().max().item()) <= 1e-3


FULL = [n for n, w in WORKLOADS.items() if w.kind == "prefill"]


@pytest.mark.parametrize("name", FULL)
def test_prefill_full_size(name):
    """Every row of every prefill workload against the oracle, element by element.

    The call is the one the bench times: the scheduled entry point with a
    zeroed workspace (work queues at d = 256, the chunk plan at d = 512).  O
    and LSE start as NaN, so a row that no tile writes fails the check.
    """
    w = WORKLOADS[name]
    print(f"full-size prefill {name}", flush=True)
    inp = prefill_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed, w.sinks)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    sd = inp["sinks"].to(DEV) if inp["sinks"] is not None else None
    scale = 1.0 / math.sqrt(w.d)
    out = torch.full((w.b, w.h_q, w.s_q, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.b, w.h_q, w.s_q), float("nan"), dtype=torch.float32, device=DEV)
    need = chunked_workspace(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.causal, w.window)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    afa.prefill(q, k, v, scale=scale, causal=w.causal, window=w.window, sinks=sd, out=out, lse=lse,
                workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(inp["q"], inp["k"], inp["v"], scale, w.causal, w.window, inp["sinks"])
    err_o, err_l = check(out, lse, o_ref, l_ref, name)
    print(f"  {name}: max |dO| = {err_o:.3e}, max |dLSE| = {err_l:.3e} over {w.b * w.h_q * w.s_q} rows",
          flush=True)
    assert int(ws[:256].count_nonzero()) == 0  # the work-queue header is left zero


# Work-queue schedule of the d = 256 ping-pong kernel (per-XCD queues with stealing)
QUEUE = [
    # b, h_q, h_kv, s_q, s_k, d, causal, window
    (1, 8, 8, 16384, 16384, 256, True, 0),  # the long-context workload: 512 query tiles
    (1, 4, 2, 1000, 1200, 256, False, 0),
    (1, 2, 2, 300, 300, 256, True, 0),      # fewer query tiles than compute units
    (1, 8, 4, 2048, 2048, 256, True, 512),
    (3, 5, 5, 777, 900, 256, True, 0),      # unit count not a multiple of 8: ragged per-XCD queues
]


@pytest.mark.parametrize("case", QUEUE, ids=[str(c) for c in QUEUE])
def test_prefill_queue_bitwise(case):
    """Each tile is computed as by the single-pass launch; the queue header is left zero."""
    b, h_q, h_kv, s_q, s_k, d, causal, window = case
    print(f"queued prefill case {case}", flush=True)
    g = torch.Generator().manual_seed(11)
    q = torch.randn(b, h_q, s_q, d, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(b, h_kv, s_k, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(b, h_kv, s_k, d, generator=g).to(torch.bfloat16).to(DEV)
    small = (q[:, :1, :200].contiguous(), k[:, :1, :230].contiguous(), v[:, :1, :230].contiguous())
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    o0, l0 = afa.prefill(q, k, v, causal=causal, window=window, chunked=False)
    s0, sl0 = afa.prefill(*small, causal=causal, window=window, chunked=False)
    for rep in range(2):  # each call finds the header as the previous one left it
        o1, l1 = afa.prefill(q, k, v, causal=causal, window=window, workspace=ws)
        s1, sl1 = afa.prefill(*small, causal=causal, window=window, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(l1, l0), f"rep {rep}"
        assert torch.equal(s1, s0) and torch.equal(sl1, sl0), f"small, rep {rep}"
        assert int(ws[:256].count_nonzero()) == 0


def test_prefill_queue_graph_replays():
    """The d = 256 work-queue prefill captured in a HIP graph: every replay equals the eager call.

    The queue counters are reset by the kernel itself (no memset node), so each
    replay starts from the zero header the previous one left; eager launches on
    the same workspace run between the replays.
    """
    print("queued prefill under graph capture", flush=True)
    g = torch.Generator().manual_seed(13)
    b, h, s, d = 1, 4, 1536, 256
    q = torch.randn(b, h, s, d, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(b, h, s, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(b, h, s, d, generator=g).to(torch.bfloat16).to(DEV)
    ref_o, ref_l = afa.prefill(q, k, v, causal=True, chunked=False)
    ws = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(b, h, s, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch recommends
        afa.prefill(q, k, v, causal=True, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        afa.prefill(q, k, v, causal=True, out=out, lse=lse, workspace=ws)
    for rep in range(3):
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        assert int(ws[:256].count_nonzero()) == 0
        eo, el = afa.prefill(q, k, v, causal=True, workspace=ws)  # eager work on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(eo, ref_o) and torch.equal(el, ref_l)

"""attn_fwd_decode_noalloc (the decode that allocates nothing) against attn_fwd_decode.

Two calls in a row on the same GPU, the second with a smaller input, each
compared with the workspace entry point on the same inputs (bit for bit: the
same kernels run, only the partials' address differs) and with the oracle.
"""

import math

import pytest
import torch

import attention_forward_attn_amd as afa
import oracle
from attention_forward_attn_amd.inputs import WORKLOADS, decode_inputs
from parity_util import check

pytestmark = pytest.mark.gpu

DEV = "cuda"


def both(inp, max_len, split, sinks=None):
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "kv_start", "kv_len")]
    sd = None if sinks is None else sinks.to(DEV)
    outs = []
    for fn in (afa.decode, afa.decode_noalloc):
        out = torch.full(args[0].shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full(args[0].shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        fn(*args, max_len, sinks=sd, split_size=split, out=out, lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


def test_noalloc_decode_two_calls_second_smaller():
    w = WORKLOADS["mqa_decode_B64_hq128_d256"]  # the largest decode workload: 64.5 MiB of partials
    print(f"no-alloc decode, call 1: {w.name}", flush=True)
    inp = decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed)
    (o_ws, l_ws), (o_na, l_na) = both(inp, w.len_hi, w.split)
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                     1 / math.sqrt(w.d))
    check(o_na, l_na, o_ref, l_ref, "no-alloc call 1")

    print("no-alloc decode, call 2: B=5 h_q=16 h_kv=4 d=128 with sinks", flush=True)
    inp2 = decode_inputs(5, 16, 4, 128, 1, 900, 77, with_sinks=True)
    max2 = int(inp2["kv_len"].max())
    (o_ws2, l_ws2), (o_na2, l_na2) = both(inp2, max2, 128, inp2["sinks"])
    assert torch.equal(o_na2, o_ws2) and torch.equal(l_na2, l_ws2)
    o_ref2, l_ref2 = oracle.decode_ref(inp2["q"], inp2["k"], inp2["v"], inp2["kv_start"], inp2["kv_len"],
                                       1 / math.sqrt(128), sinks=inp2["sinks"])
    check(o_na2, l_na2, o_ref2, l_ref2, "no-alloc call 2")

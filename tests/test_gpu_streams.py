"""Calls on a caller-given stream: the binding allocates its outputs and workspaces on that stream."""

import pytest
import torch

import attention_forward_attn_amd as afa
from attention_forward_attn_amd.inputs import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_prefill_work_queue_on_side_stream():
    """d = 256 work-queue prefill with the zeroed queue header allocated by the binding, on a side stream."""
    print("prefill d=256 on a side stream", flush=True)
    inp = prefill_inputs(1, 4, 4, 1536, 1536, 256, 17)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    ref_o, ref_l = afa.prefill(q, k, v, causal=True, chunked=False)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [afa.prefill(q, k, v, causal=True, stream=side) for _ in range(3)]
    outs.append(afa.prefill(q, k, v, causal=True, stream=side.cuda_stream))  # raw handle
    side.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_decode_on_side_stream():
    print("decode on a side stream", flush=True)
    inp = decode_inputs(8, 128, 1, 128, 100, 3000, 18)
    args = [inp[n].to(DEV) for n in ("q", "k", "v", "kv_start", "kv_len")]
    max_len = int(inp["kv_len"].max())
    ref_o, ref_l = afa.decode(*args, max_len)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [afa.decode(*args, max_len, stream=side) for _ in range(3)]
    side.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)

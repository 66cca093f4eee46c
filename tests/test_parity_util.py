"""CPU checks of the parity helpers the GPU tests use."""

import numpy as np
import torch

import oracle
from attention_forward_attn_amd.inputs import prefill_inputs
from parity_util import oracle_full


def test_oracle_full_equals_one_call():
    """Slicing by (batch, head) on a thread pool gives the oracle's own result (GQA, window, sink)."""
    inp = prefill_inputs(2, 6, 2, 70, 90, 32, 5, with_sinks=True)
    o1, l1 = oracle_full(inp["q"], inp["k"], inp["v"], 0.3, True, 40, inp["sinks"], workers=3)
    o2, l2 = oracle.attention_ref(inp["q"], inp["k"], inp["v"], 0.3, causal=True, window=40, sinks=inp["sinks"])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_oracle_full_no_sink_noncausal():
    inp = prefill_inputs(1, 3, 3, 33, 17, 16, 6)
    o1, l1 = oracle_full(inp["q"], inp["k"], inp["v"], 0.25, False, 0, None, workers=2)
    o2, l2 = oracle.attention_ref(inp["q"], inp["k"], inp["v"], 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert isinstance(inp["q"], torch.Tensor)

"""GPU parity of split-KV decode and of the LSE-merge kernel against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as afa
import oracle
from attention_forward_attn_amd.inputs import (WORKLOADS, decode_inputs, fp8_decode_inputs, paged_decode_inputs,
                                               paged_fp8_decode_inputs)
from parity_util import check

pytestmark = pytest.mark.gpu

DEV = "cuda"


def poisoned_ws(nbytes):
    """A decode workspace of NaN bytes (partials) behind the zeroed counter header."""
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV)
    ws[: afa.DECODE_WORKSPACE_HEADER].zero_()
    return ws


def header_left_zero(ws):
    return not bool(ws[: afa.DECODE_WORKSPACE_HEADER].any())


def run_decode(inp, max_len, split=512, sinks=None, d=None, ws=None):
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    ks, kl = inp["kv_start"].to(DEV), inp["kv_len"].to(DEV)
    d = q.shape[-1]
    if ws is None:
        ws = poisoned_ws(afa.decode_workspace_size(q.shape[0], q.shape[1], d, max_len, split))
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    sd = None if sinks is None else sinks.to(DEV)
    afa.decode(q, k, v, ks, kl, max_len, sinks=sd, split_size=split, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert header_left_zero(ws)
    return out, lse


def make(B, h_q, h_kv, d, lens, seed):
    gen = torch.Generator("cpu").manual_seed(seed)
    lens_t = torch.tensor(lens, dtype=torch.int64)
    starts = torch.zeros(B, dtype=torch.int64)
    starts[1:] = torch.cumsum(lens_t, 0)[:-1]
    T = int(lens_t.sum()) + 5
    q = torch.randn(B, h_q, d, generator=gen).to(torch.bfloat16)
    k = torch.randn(T, h_kv, d, generator=gen).to(torch.bfloat16)
    v = torch.randn(T, h_kv, d, generator=gen).to(torch.bfloat16)
    return {"q": q, "k": k, "v": v, "kv_start": starts, "kv_len": lens_t.to(torch.int32)}


SMALL = [
    # B, h_q, h_kv, d, lens, split
    (4, 128, 1, 128, [1, 511, 512, 513], 512),
    (3, 128, 1, 256, [1000, 64, 1537], 512),
    (5, 16, 4, 64, [1, 2, 63, 64, 700], 128),
    (2, 8, 8, 128, [300, 5], 64),
    (2, 256, 2, 128, [129, 1030], 256),  # 128 query heads per kv head, two kv heads
    (3, 6, 2, 128, [17, 0, 90], 64),     # an empty sequence
    (2, 320, 1, 128, [700, 1500], 512),  # three head blocks, the last one of 64 heads
    (2, 96, 2, 256, [513, 40], 256),     # 48 heads per kv head: partial head block and merge slices
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
@pytest.mark.parametrize("with_sink", [False, True])
def test_decode_small(case, with_sink):
    B, h_q, h_kv, d, lens, split = case
    print(f"decode case {case} sink={with_sink}", flush=True)
    inp = make(B, h_q, h_kv, d, lens, 21)
    sinks = torch.randn(h_q, generator=torch.Generator().manual_seed(3)) if with_sink else None
    out, lse = run_decode(inp, max(max(lens), 1), split, sinks)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                     1 / math.sqrt(d), sinks=sinks)
    check(out, lse, o_ref, l_ref, str(case))


def test_decode_head_stride_zero_matches_mqa():
    inp = make(3, 16, 1, 128, [100, 700, 1], 22)
    out1, lse1 = run_decode(inp, 700, 128)
    # the same cache seen as 16 kv heads with head stride 0
    k = inp["k"].to(DEV).expand(-1, 16, -1)
    v = inp["v"].to(DEV).expand(-1, 16, -1)
    out2, lse2 = afa.decode(inp["q"].to(DEV), k, v, inp["kv_start"].to(DEV), inp["kv_len"].to(DEV),
                            700, split_size=128)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("B,h_q,h_kv,d,split", [(70, 16, 2, 128, 256), (133, 8, 1, 64, 128),
                                                (65, 32, 1, 256, 512),
                                                (300, 16, 4, 128, 256)])  # 1200 merges: counters 4 bytes apart
def test_decode_many_sequences(B, h_q, h_kv, d, split):
    # more sequences than a wave has lanes, empty sequences, and a max_kv_len
    # above every length (trailing splits hold no keys)
    print(f"decode many sequences B={B} h_q={h_q} h_kv={h_kv} d={d} split={split}", flush=True)
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 1300, size=B)
    lens[::7] = 0
    lens[1] = split
    inp = make(B, h_q, h_kv, d, lens.tolist(), 24)
    out, lse = run_decode(inp, 2048, split)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                     1 / math.sqrt(d))
    check(out, lse, o_ref, l_ref, f"B={B}")


def test_decode_workspace_reused_across_sizes():
    # one workspace, calls of different sizes in turn: the arrival counters sit
    # at fixed places, so every call finds them zero and leaves them zero
    big = make(70, 16, 2, 128, np.random.default_rng(5).integers(0, 2048, size=70).tolist(), 25)
    small = make(3, 128, 1, 256, [700, 1, 1500], 26)
    nbytes = max(afa.decode_workspace_size(70, 16, 128, 2048, 256), afa.decode_workspace_size(3, 128, 256, 1500, 256))
    ws = poisoned_ws(nbytes)
    for inp, max_len in ((big, 2048), (small, 1500), (big, 2048)):
        d = inp["q"].shape[-1]
        print(f"reused workspace B={inp['q'].shape[0]} d={d}", flush=True)
        out, lse = run_decode(inp, max_len, 256, ws=ws)
        o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                         1 / math.sqrt(d))
        check(out, lse, o_ref, l_ref, f"B={inp['q'].shape[0]}")


def test_decode_more_merges_than_counters():
    # B * h_kv merge workgroups above the header's 16384 counters: the splits
    # are merged by the second kernel instead
    B, h = 1040, 16
    assert B * h > afa.DECODE_WORKSPACE_HEADER // 4
    lens = np.random.default_rng(6).integers(0, 200, size=B)
    lens[::9] = 0
    inp = make(B, h, h, 64, lens.tolist(), 27)
    print("decode with the combine kernel, B=1040 h=16 d=64", flush=True)
    out, lse = run_decode(inp, 200, 64)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"], 1 / 8.0)
    check(out, lse, o_ref, l_ref, "B=1040")


def test_decode_split_size_invariance():
    inp = make(4, 128, 1, 128, [1500, 3000, 64, 2049], 23)
    o1, l1 = run_decode(inp, 3000, 512)
    o2, l2 = run_decode(inp, 3000, 4096)  # a single split per sequence
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items()
                                  if w.kind == "decode" and not w.page_size and not w.fp8])
def test_decode_full_size(name):
    w = WORKLOADS[name]
    print(f"full-size decode {name}", flush=True)
    inp = decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed)
    out, lse = run_decode(inp, w.len_hi, w.split)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                     1 / math.sqrt(w.d))
    check(out, lse, o_ref, l_ref, name)


@pytest.mark.parametrize("n,rows,d", [(1, 5, 64), (7, 33, 128), (16, 100, 256), (3, 10, 512)])
def test_combine_matches_merge(n, rows, d):
    gen = torch.Generator().manual_seed(n * 100 + rows)
    o_parts = torch.randn(n, rows, d, generator=gen)
    lse_parts = torch.randn(n, rows, generator=gen) * 3
    lse_parts[0, 0] = float("-inf")          # one empty part: its vector is loaded, never used
    o_parts[0, 0] = float("nan")
    if rows > 2:
        lse_parts[:, 1] = float("-inf")      # one empty row
        o_parts[:, 1] = float("nan")         # never read
    out, lse = afa.combine(o_parts.to(DEV), lse_parts.to(DEV))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge_ref(np.nan_to_num(o_parts.double().numpy()), lse_parts.double().numpy())
    check(out, lse, o_ref, l_ref, "combine")


# --- paged KV cache -------------------------------------------------------

def run_paged(inp, max_len, split=512, sinks=None, table=None):
    q = inp["q"].to(DEV)
    kc, vc = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    bt = (inp["block_table"] if table is None else table).to(DEV)
    kl = inp["kv_len"].to(DEV)
    d = q.shape[-1]
    ws = poisoned_ws(afa.decode_workspace_size(q.shape[0], q.shape[1], d, max_len, split))
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    sd = None if sinks is None else sinks.to(DEV)
    afa.decode_paged(q, kc, vc, bt, kl, max_len, sinks=sd, split_size=split, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert header_left_zero(ws)
    return out, lse


PAGED = [
    # B, h_q, h_kv, d, len_lo, len_hi, page_size, split
    (4, 128, 1, 128, 1, 1500, 16, 512),
    (3, 128, 1, 256, 1, 1100, 64, 512),
    (5, 16, 4, 64, 1, 700, 32, 128),
    (4, 8, 8, 128, 0, 300, 256, 256),      # empty sequences possible
    (3, 256, 2, 128, 100, 1030, 128, 1024),
    (2, 32, 1, 128, 200, 2100, 16, 1024),  # 64 pages per split
    (3, 64, 1, 128, 1, 1500, 128, 384),    # three pages per split (split not a power of two)
]


@pytest.mark.parametrize("case", PAGED, ids=[str(c) for c in PAGED])
@pytest.mark.parametrize("with_sink", [False, True])
def test_decode_paged_small(case, with_sink):
    B, h_q, h_kv, d, lo, hi, page, split = case
    print(f"paged decode case {case} sink={with_sink}", flush=True)
    inp = paged_decode_inputs(B, h_q, h_kv, d, lo, hi, page, 31, with_sink, spare=3, poison=True)
    out, lse = run_paged(inp, hi, split, inp["sinks"])
    o_ref, l_ref = oracle.decode_paged_ref(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                                           inp["kv_len"], page, 1 / math.sqrt(d), sinks=inp["sinks"])
    check(out, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("d,page", [(64, 16), (128, 64), (256, 32)])
def test_decode_paged_equals_dense_bitwise(d, page):
    """The same keys read through a block table give bit-identical results."""
    inp = paged_decode_inputs(6, 32, 2, d, 1, 1800, page, 32, True, spare=2, poison=True)
    out_p, lse_p = run_paged(inp, 1800, 512, inp["sinks"])
    out_d, lse_d = run_decode(inp, 1800, 512, inp["sinks"])
    assert torch.equal(out_p, out_d) and torch.equal(lse_p, lse_d)


def test_decode_paged_bad_page_reads_zero():
    """A page index outside [0, n_pages) is not dereferenced: its tokens read as zeros."""
    inp = paged_decode_inputs(3, 16, 1, 128, 300, 600, 64, 33, poison=True)
    n_pages = inp["k_cache"].shape[0]
    table = inp["block_table"].clone()
    table[0, 1] = n_pages       # one past the pool
    table[2, 0] = -5
    out, lse = run_paged(inp, 600, 256, table=table)
    # expected: the same pages pointed at an all-zero page appended to the pool
    zero = torch.zeros((1,) + tuple(inp["k_cache"].shape[1:]), dtype=torch.bfloat16)
    kc = torch.cat([inp["k_cache"], zero])
    vc = torch.cat([inp["v_cache"], zero])
    t2 = table.clone()
    t2[0, 1] = n_pages
    t2[2, 0] = n_pages
    o_ref, l_ref = oracle.decode_paged_ref(inp["q"], kc, vc, t2, inp["kv_len"], 64, 1 / math.sqrt(128))
    check(out, lse, o_ref, l_ref, "bad page")


def test_decode_paged_full_size():
    w = WORKLOADS["mqa_decode_paged_B64_hq128_d128_p64"]
    print(f"full-size paged decode {w.name}", flush=True)
    inp = paged_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed)
    out, lse = run_paged(inp, w.len_hi, w.split)
    o_ref, l_ref = oracle.decode_ref(inp["q"], inp["k"], inp["v"], inp["kv_start"], inp["kv_len"],
                                     1 / math.sqrt(w.d))
    check(out, lse, o_ref, l_ref, w.name)


# --- FP8 (E4M3) KV cache --------------------------------------------------

def run_fp8(inp, max_len, split=512, sinks=None):
    q = inp["q"].to(DEV)
    k8, v8 = inp["k8"].to(DEV), inp["v8"].to(DEV)
    ksc, vsc = inp["k_scale"].to(DEV), inp["v_scale"].to(DEV)
    ks, kl = inp["kv_start"].to(DEV), inp["kv_len"].to(DEV)
    d = q.shape[-1]
    ws = poisoned_ws(afa.decode_workspace_size(q.shape[0], q.shape[1], d, max_len, split))
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    sd = None if sinks is None else sinks.to(DEV)
    afa.decode_fp8(q, k8, v8, ksc, vsc, ks, kl, max_len, sinks=sd, split_size=split, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert header_left_zero(ws)
    return out, lse


FP8 = [
    # B, h_q, h_kv, d, len_lo, len_hi, split
    (4, 128, 1, 128, 1, 1500, 512),
    (5, 16, 4, 128, 0, 700, 128),
    (3, 256, 2, 128, 100, 1030, 256),
    (2, 8, 8, 128, 1, 300, 64),
    (4, 128, 1, 256, 1, 1500, 512),
    (5, 16, 4, 256, 0, 700, 128),
    (2, 8, 8, 256, 1, 300, 64),
]


@pytest.mark.parametrize("case", FP8, ids=[str(c) for c in FP8])
@pytest.mark.parametrize("with_sink", [False, True])
def test_decode_fp8_small(case, with_sink):
    B, h_q, h_kv, d, lo, hi, split = case
    print(f"fp8 decode case {case} sink={with_sink}", flush=True)
    inp = fp8_decode_inputs(B, h_q, h_kv, d, lo, hi, 41, with_sink)
    out, lse = run_fp8(inp, hi, split, inp["sinks"])
    o_ref, l_ref = oracle.decode_fp8_ref(inp["q"], inp["k8"].numpy(), inp["v8"].numpy(), inp["k_scale"],
                                         inp["v_scale"], inp["kv_start"], inp["kv_len"], 1 / math.sqrt(d),
                                         sinks=inp["sinks"])
    check(out, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("d", [128, 256])
def test_decode_fp8_equals_bf16_on_exact_values(d):
    """Power-of-two scales make every dequantized value a bf16 value: the FP8 path
    then matches the bf16 decode on the dequantized cache bit for bit."""
    inp = fp8_decode_inputs(5, 64, 2, d, 1, 1500, 42, True)
    inp["k_scale"] = torch.tensor([2.0 ** -6, 2.0 ** -7])
    inp["v_scale"] = torch.tensor([2.0 ** -5, 2.0 ** -8])
    for n in ("k", "v"):
        vals = inp[n + "8"].view(torch.float8_e4m3fn).to(torch.float32) * inp[n + "_scale"][None, :, None]
        inp[n] = vals.to(torch.bfloat16)
        assert torch.equal(inp[n].to(torch.float32), vals)
    out8, lse8 = run_fp8(inp, 1500, 512, inp["sinks"])
    outb, lseb = run_decode(inp, 1500, 512, inp["sinks"])
    assert torch.equal(out8, outb) and torch.equal(lse8, lseb)


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items()
                                  if w.kind == "decode" and w.fp8 and not w.page_size])
def test_decode_fp8_full_size(name):
    w = WORKLOADS[name]
    print(f"full-size fp8 decode {w.name}", flush=True)
    inp = fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed)
    out, lse = run_fp8(inp, w.len_hi, w.split)
    o_ref, l_ref = oracle.decode_fp8_ref(inp["q"], inp["k8"].numpy(), inp["v8"].numpy(), inp["k_scale"],
                                         inp["v_scale"], inp["kv_start"], inp["kv_len"], 1 / math.sqrt(w.d))
    check(out, lse, o_ref, l_ref, w.name)



# --- paged FP8 KV cache ----------------------------------------------------

def run_paged_fp8(inp, max_len, split=512, sinks=None, table=None):
    q = inp["q"].to(DEV)
    kc, vc = inp["k8_cache"].to(DEV), inp["v8_cache"].to(DEV)
    ksc, vsc = inp["k_scale"].to(DEV), inp["v_scale"].to(DEV)
    bt = (inp["block_table"] if table is None else table).to(DEV)
    kl = inp["kv_len"].to(DEV)
    d = q.shape[-1]
    ws = poisoned_ws(afa.decode_workspace_size(q.shape[0], q.shape[1], d, max_len, split))
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    sd = None if sinks is None else sinks.to(DEV)
    afa.decode_paged_fp8(q, kc, vc, ksc, vsc, bt, kl, max_len, sinks=sd, split_size=split, workspace=ws, out=out,
                         lse=lse)
    torch.cuda.synchronize()
    assert header_left_zero(ws)
    return out, lse


PAGED_FP8 = [
    # B, h_q, h_kv, d, len_lo, len_hi, page_size, split
    (4, 128, 1, 128, 1, 1500, 16, 512),
    (5, 16, 4, 128, 0, 700, 32, 128),      # empty sequences possible
    (3, 64, 1, 128, 1, 1500, 128, 384),    # three pages per split
    (4, 128, 1, 256, 1, 1500, 64, 512),
    (3, 8, 8, 256, 1, 300, 16, 1024),      # 64 pages per split
]


@pytest.mark.parametrize("case", PAGED_FP8, ids=[str(c) for c in PAGED_FP8])
@pytest.mark.parametrize("with_sink", [False, True])
def test_decode_paged_fp8_small(case, with_sink):
    B, h_q, h_kv, d, lo, hi, page, split = case
    print(f"paged fp8 decode case {case} sink={with_sink}", flush=True)
    inp = paged_fp8_decode_inputs(B, h_q, h_kv, d, lo, hi, page, 43, with_sink, spare=3)
    out, lse = run_paged_fp8(inp, hi, split, inp["sinks"])
    # the pages hold the codes of the contiguous draw, token for token
    o_ref, l_ref = oracle.decode_fp8_ref(inp["q"], inp["k8"].numpy(), inp["v8"].numpy(), inp["k_scale"],
                                         inp["v_scale"], inp["kv_start"], inp["kv_len"], 1 / math.sqrt(d),
                                         sinks=inp["sinks"])
    check(out, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("d,page", [(128, 64), (256, 16)])
def test_decode_paged_fp8_equals_contiguous_bitwise(d, page):
    """The same codes read through a block table give bit-identical results."""
    inp = paged_fp8_decode_inputs(6, 32, 2, d, 1, 1800, page, 44, True, spare=2)
    out_p, lse_p = run_paged_fp8(inp, 1800, 512, inp["sinks"])
    out_c, lse_c = run_fp8(inp, 1800, 512, inp["sinks"])
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)


def test_decode_paged_fp8_bad_page_reads_zero():
    """A page index outside [0, n_pages) is not dereferenced: its tokens read as zero codes."""
    inp = paged_fp8_decode_inputs(3, 16, 1, 128, 300, 600, 64, 45)
    n_pages = inp["k8_cache"].shape[0]
    table = inp["block_table"].clone()
    table[0, 1] = n_pages       # one past the pool
    table[2, 0] = -5
    out, lse = run_paged_fp8(inp, 600, 256, table=table)
    # expected: the contiguous codes with those two pages' tokens set to code 0 (+0.0)
    k8, v8 = inp["k8"].clone(), inp["v8"].clone()
    starts = inp["kv_start"]
    for b, pg in ((0, 1), (2, 0)):
        lo = int(starts[b]) + pg * 64
        hi = min(int(starts[b]) + int(inp["kv_len"][b]), lo + 64)
        k8[lo:hi] = 0
        v8[lo:hi] = 0
    o_ref, l_ref = oracle.decode_fp8_ref(inp["q"], k8.numpy(), v8.numpy(), inp["k_scale"], inp["v_scale"],
                                         inp["kv_start"], inp["kv_len"], 1 / math.sqrt(128))
    check(out, lse, o_ref, l_ref, "bad page")


def test_decode_paged_fp8_full_size():
    w = WORKLOADS["mqa_decode_paged_fp8_B64_hq128_d128_p64"]
    print(f"full-size paged fp8 decode {w.name}", flush=True)
    inp = paged_fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed)
    out, lse = run_paged_fp8(inp, w.len_hi, w.split)
    o_ref, l_ref = oracle.decode_fp8_ref(inp["q"], inp["k8"].numpy(), inp["v8"].numpy(), inp["k_scale"],
                                         inp["v_scale"], inp["kv_start"], inp["kv_len"], 1 / math.sqrt(w.d))
    check(out, lse, o_ref, l_ref, w.name)

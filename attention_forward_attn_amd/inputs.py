"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws random tensors and
lays them out.  Both the HIP path and the fp64 oracle receive exactly the
tensors produced here (the oracle upcasts the bf16 values exactly).

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw order is decode
lengths first (decode only), then Q, K, V, then sink logits.  Values are fp32
N(0, 1) rounded to bf16 with round-to-nearest-even; sinks stay fp32 N(0, 1).
Prefill tensors are [b, h, s, d] contiguous; the decode KV cache is packed
token-major, [sum_b L_b, h_kv, d], contiguous per sequence, with ``kv_start``
the exclusive prefix sum of the lengths.  A paged cache holds the same draw
in pages of ``page_size`` tokens, [n_pages, page_size, h_kv, d]; the pages of
all sequences (plus ``spare`` unused ones) are placed in a random order drawn
from a second generator (seed + 7919), so the values match the packed draw.  An FP8
cache holds the same draw as OCP E4M3 codes: per kv head, scale = max |x| / 448
and code = E4M3(x / scale) (torch's round-to-nearest-even cast).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

BASE_SEED = 1234


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, mask and the seed its inputs use."""

    name: str
    kind: str  # "prefill", "decode" or "backward"
    seed: int
    d: int
    h_q: int
    h_kv: int
    b: int = 1
    s_q: int = 0
    s_k: int = 0
    causal: bool = False
    window: int = 0
    sinks: bool = False
    # decode only
    len_lo: int = 0
    len_hi: int = 0
    split: int = 512
    page_size: int = 0  # paged KV cache (0 = contiguous per sequence)
    fp8: bool = False   # KV cache as E4M3 codes with per-kv-head scales
    notes: dict = field(default_factory=dict, compare=False)


def _w(*args, **kw) -> Workload:
    return Workload(*args, **kw)


# The five workload families; seed = BASE_SEED + family index.
WORKLOADS = {
    w.name: w
    for w in [
        # family 0: tiny single head
        _w("tiny_b1_h1_s256_d64", "prefill", BASE_SEED + 0, 64, 1, 1, b=1, s_q=256, s_k=256),
        # family 1: dense MHA prefill, both masks
        _w("mha_b2_h16_s4096_d128", "prefill", BASE_SEED + 1, 128, 16, 16, b=2, s_q=4096, s_k=4096),
        _w("mha_b2_h16_s4096_d128_causal", "prefill", BASE_SEED + 1, 128, 16, 16, b=2, s_q=4096,
           s_k=4096, causal=True),
        _w("mha_b1_h16_s8192_d128", "prefill", BASE_SEED + 1, 128, 16, 16, b=1, s_q=8192, s_k=8192),
        _w("mha_b1_h16_s8192_d128_causal", "prefill", BASE_SEED + 1, 128, 16, 16, b=1, s_q=8192,
           s_k=8192, causal=True),
        _w("mha_b4_h32_s2048_d64", "prefill", BASE_SEED + 1, 64, 32, 32, b=4, s_q=2048, s_k=2048),
        _w("mha_b4_h32_s2048_d64_causal", "prefill", BASE_SEED + 1, 64, 32, 32, b=4, s_q=2048,
           s_k=2048, causal=True),
        # family 2: GQA causal with LSE; sliding window + sink variant
        _w("gqa_b2_hq32_hkv8_s4096_d128_causal", "prefill", BASE_SEED + 2, 128, 32, 8, b=2,
           s_q=4096, s_k=4096, causal=True),
        _w("gqa_b2_hq32_hkv8_s4096_d128_swa1024_sink", "prefill", BASE_SEED + 2, 128, 32, 8, b=2,
           s_q=4096, s_k=4096, causal=True, window=1024, sinks=True),
        # family 3: MQA decode, split-KV in chunks of 512
        _w("mqa_decode_B64_hq128_d128", "decode", BASE_SEED + 3, 128, 128, 1, b=64,
           len_lo=1024, len_hi=8192),
        _w("mqa_decode_B64_hq128_d256", "decode", BASE_SEED + 3, 256, 128, 1, b=64,
           len_lo=1024, len_hi=8192),
        # the same draw quantized to an FP8 (E4M3) cache
        _w("mqa_decode_fp8_B64_hq128_d128", "decode", BASE_SEED + 3, 128, 128, 1, b=64,
           len_lo=1024, len_hi=8192, fp8=True),
        _w("mqa_decode_fp8_B64_hq128_d256", "decode", BASE_SEED + 3, 256, 128, 1, b=64,
           len_lo=1024, len_hi=8192, fp8=True),
        # the same draw held in a paged cache of 64-token pages
        _w("mqa_decode_paged_B64_hq128_d128_p64", "decode", BASE_SEED + 3, 128, 128, 1, b=64,
           len_lo=1024, len_hi=8192, page_size=64),
        # the FP8 codes of that draw in the same pages
        _w("mqa_decode_paged_fp8_B64_hq128_d128_p64", "decode", BASE_SEED + 3, 128, 128, 1, b=64,
           len_lo=1024, len_hi=8192, page_size=64, fp8=True),
        # backward of the dense causal MHA prefill (incoming dO ~ N(0,1), drawn after Q, K, V)
        _w("bwd_mha_b2_h16_s4096_d128_causal", "backward", BASE_SEED + 1, 128, 16, 16, b=2, s_q=4096,
           s_k=4096, causal=True),
        # family 4: large head dims, long context
        _w("long_b1_h8_s16384_d256_causal", "prefill", BASE_SEED + 4, 256, 8, 8, b=1,
           s_q=16384, s_k=16384, causal=True),
        _w("wide_b1_h4_s4096_d512_causal", "prefill", BASE_SEED + 4, 512, 4, 4, b=1,
           s_q=4096, s_k=4096, causal=True),
        # backward at d = 256: the d = 128 backward's shape with half the heads (same flops)
        _w("bwd_mha_b2_h8_s4096_d256_causal", "backward", BASE_SEED + 4, 256, 8, 8, b=2, s_q=4096,
           s_k=4096, causal=True),
    ]
}


def _randn_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def prefill_inputs(b: int, h_q: int, h_kv: int, s_q: int, s_k: int, d: int, seed: int,
                   with_sinks: bool = False):
    """Return dict(q, k, v, sinks) on the CPU: bf16 [b,h,s,d] and fp32 [h_q] (or None)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn_bf16((b, h_q, s_q, d), gen)
    k = _randn_bf16((b, h_kv, s_k, d), gen)
    v = _randn_bf16((b, h_kv, s_k, d), gen)
    sinks = torch.randn(h_q, generator=gen, dtype=torch.float32) if with_sinks else None
    return {"q": q, "k": k, "v": v, "sinks": sinks}


def decode_inputs(B: int, h_q: int, h_kv: int, d: int, len_lo: int, len_hi: int, seed: int,
                  with_sinks: bool = False):
    """Return dict(q, k, v, kv_start, kv_len, sinks) on the CPU.

    Lengths are uniform integers in [len_lo, len_hi]; q is bf16 [B,h_q,d];
    k and v are bf16 [sum L, h_kv, d]; kv_start int64 [B]; kv_len int32 [B].
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    kv_len = torch.randint(len_lo, len_hi + 1, (B,), generator=gen, dtype=torch.int64)
    kv_start = torch.zeros(B, dtype=torch.int64)
    if B > 1:
        kv_start[1:] = torch.cumsum(kv_len, 0)[:-1]
    total = int(kv_len.sum())
    q = _randn_bf16((B, h_q, d), gen)
    k = _randn_bf16((total, h_kv, d), gen)
    v = _randn_bf16((total, h_kv, d), gen)
    sinks = torch.randn(h_q, generator=gen, dtype=torch.float32) if with_sinks else None
    return {"q": q, "k": k, "v": v, "kv_start": kv_start, "kv_len": kv_len.to(torch.int32),
            "sinks": sinks}


def workload_inputs(w: Workload):
    """Inputs of a named workload (see WORKLOADS)."""
    if w.kind == "prefill":
        return prefill_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed, w.sinks)
    if w.kind == "backward":
        return backward_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed)
    if w.fp8 and w.page_size:
        return paged_fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed, w.sinks)
    if w.fp8:
        return fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed, w.sinks)
    if w.page_size:
        return paged_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed, w.sinks)
    return decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed, w.sinks)


def paged_decode_inputs(B: int, h_q: int, h_kv: int, d: int, len_lo: int, len_hi: int, page_size: int,
                        seed: int, with_sinks: bool = False, spare: int = 0, poison: bool = False):
    """The draw of decode_inputs laid out in a paged cache.

    Returns decode_inputs' dict plus k_cache, v_cache (bf16 [n_pages,
    page_size, h_kv, d]), block_table (int32 [B, ceil(len_hi / page_size)];
    entries past a sequence's pages are -1) and page_size.  Slots that hold no token are
    zero, or NaN with poison=True (so that reading one shows).
    """
    inp = decode_inputs(B, h_q, h_kv, d, len_lo, len_hi, seed, with_sinks)
    lens = [int(x) for x in inp["kv_len"]]
    starts = [int(x) for x in inp["kv_start"]]
    n_used = sum(-(-L // page_size) for L in lens)
    n_pages = max(1, n_used + spare)
    perm = torch.randperm(n_pages, generator=torch.Generator("cpu").manual_seed(seed + 7919))
    fill = float("nan") if poison else 0.0
    kc = torch.full((n_pages, page_size, h_kv, d), fill, dtype=torch.bfloat16)
    vc = torch.full((n_pages, page_size, h_kv, d), fill, dtype=torch.bfloat16)
    max_pages = max(1, -(-len_hi // page_size))  # the table is sized for the longest possible sequence
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    used = 0
    for b, (s0, L) in enumerate(zip(starts, lens)):
        for pg in range(-(-L // page_size)):
            phys = int(perm[used])
            used += 1
            table[b, pg] = phys
            n = min(page_size, L - pg * page_size)
            kc[phys, :n] = inp["k"][s0 + pg * page_size:s0 + pg * page_size + n]
            vc[phys, :n] = inp["v"][s0 + pg * page_size:s0 + pg * page_size + n]
    inp.update(k_cache=kc, v_cache=vc, block_table=table, page_size=page_size)
    return inp


def fp8_decode_inputs(B: int, h_q: int, h_kv: int, d: int, len_lo: int, len_hi: int, seed: int,
                      with_sinks: bool = False):
    """The draw of decode_inputs with K and V stored as E4M3 codes and per-kv-head scales.

    Returns decode_inputs' dict plus k8, v8 (uint8 [T, h_kv, d]) and k_scale,
    v_scale (fp32 [h_kv]).
    """
    inp = decode_inputs(B, h_q, h_kv, d, len_lo, len_hi, seed, with_sinks)
    for name in ("k", "v"):
        x = inp[name].to(torch.float32)
        amax = x.abs().amax(dim=(0, 2)).clamp_min(1e-30)
        sc = (amax / 448.0).to(torch.float32)
        codes = (x / sc[None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        inp[name + "8"] = codes.contiguous()
        inp[name + "_scale"] = sc
    return inp


def paged_fp8_decode_inputs(B: int, h_q: int, h_kv: int, d: int, len_lo: int, len_hi: int, page_size: int,
                            seed: int, with_sinks: bool = False, spare: int = 0):
    """The codes and scales of fp8_decode_inputs laid out in a paged cache.

    Returns fp8_decode_inputs' dict plus k8_cache, v8_cache (uint8 [n_pages,
    page_size, h_kv, d]), block_table and page_size, with the page order of
    paged_decode_inputs for the same seed; slots that hold no token are 0xff
    (an E4M3 NaN, so that reading one shows).
    """
    inp = fp8_decode_inputs(B, h_q, h_kv, d, len_lo, len_hi, seed, with_sinks)
    lens = [int(x) for x in inp["kv_len"]]
    starts = [int(x) for x in inp["kv_start"]]
    n_used = sum(-(-L // page_size) for L in lens)
    n_pages = max(1, n_used + spare)
    perm = torch.randperm(n_pages, generator=torch.Generator("cpu").manual_seed(seed + 7919))
    kc = torch.full((n_pages, page_size, h_kv, d), 255, dtype=torch.uint8)
    vc = torch.full((n_pages, page_size, h_kv, d), 255, dtype=torch.uint8)
    max_pages = max(1, -(-len_hi // page_size))
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    used = 0
    for b, (s0, L) in enumerate(zip(starts, lens)):
        for pg in range(-(-L // page_size)):
            phys = int(perm[used])
            used += 1
            table[b, pg] = phys
            n = min(page_size, L - pg * page_size)
            kc[phys, :n] = inp["k8"][s0 + pg * page_size:s0 + pg * page_size + n]
            vc[phys, :n] = inp["v8"][s0 + pg * page_size:s0 + pg * page_size + n]
    inp.update(k8_cache=kc, v8_cache=vc, block_table=table, page_size=page_size)
    return inp


def backward_inputs(b: int, h_q: int, h_kv: int, s_q: int, s_k: int, d: int, seed: int):
    """prefill_inputs plus an incoming gradient d_o (bf16 [b, h_q, s_q, d], N(0,1)) drawn after them."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn_bf16((b, h_q, s_q, d), gen)
    k = _randn_bf16((b, h_kv, s_k, d), gen)
    v = _randn_bf16((b, h_kv, s_k, d), gen)
    d_o = _randn_bf16((b, h_q, s_q, d), gen)
    return {"q": q, "k": k, "v": v, "d_o": d_o, "sinks": None}


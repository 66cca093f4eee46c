"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP call.

Every call here is invalid on purpose (so no kernel is ever launched): the
pointers are fake, non-NULL integers.
"""

import ctypes
import os
import re

import pytest

import attention_forward_attn_amd as afa
from attention_forward_attn_amd._binding import (BwdArgs, CombineArgs, DecodeArgs, DecodeFp8Args,
                                                 DecodePagedArgs, DecodePagedFp8Args, PrefillArgs)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fwd.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("attn_fwd_prefill", "attn_fwd_prefill_chunked", "attn_fwd_prefill_chunked_workspace_size",
                 "attn_fwd_decode", "attn_fwd_decode_paged", "attn_fwd_decode_fp8",
                 "attn_combine", "attn_bwd", "attn_bwd_workspace_size",
                 "attn_fwd_decode_workspace_size", "attn_fwd_decode_noalloc", "attn_status_str",
                 "attn_last_error", "attn_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = afa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in attn_fwd.h but not exported"
    assert lib.attn_abi_version() == 10


def test_status_strings():
    lib = afa.load_library()
    for code, name in enumerate(["ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_STRIDE",
                                 "ATTN_ERR_ALIGN", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE",
                                 "ATTN_ERR_HIP"]):
        assert lib.attn_status_str(code).decode() == name


def good_prefill(**over):
    a = PrefillArgs()
    a.q = a.k = a.v = a.o = FAKE
    a.lse = None
    a.sinks = None
    a.b, a.h_q, a.h_kv, a.s_q, a.s_k, a.d = 1, 2, 1, 64, 64, 128
    a.q_sb, a.q_sh, a.q_ss = 2 * 64 * 128, 64 * 128, 128
    a.k_sb, a.k_sh, a.k_ss = 64 * 128, 64 * 128, 128
    a.v_sb, a.v_sh, a.v_ss = 64 * 128, 64 * 128, 128
    a.o_sb, a.o_sh, a.o_ss = 2 * 64 * 128, 64 * 128, 128
    a.scale = 0.088
    a.causal = 0
    a.window = 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


PREFILL_BAD = [
    ("null q", dict(q=None), 1),
    ("null o", dict(o=None), 1),
    ("d=96", dict(d=96), 2),
    ("d=0", dict(d=0), 2),
    ("b=0", dict(b=0), 2),
    ("h_kv=0", dict(h_kv=0), 2),
    ("ratio not integral", dict(h_q=3, h_kv=2), 2),
    ("negative s_k", dict(s_k=-1), 2),
    ("zero scale", dict(scale=0.0), 2),
    ("negative scale", dict(scale=-1.0), 2),
    ("nan scale", dict(scale=float("nan")), 2),
    ("window without causal", dict(window=16), 2),
    ("negative window", dict(causal=1, window=-1), 2),
    ("causal=2", dict(causal=2), 2),
    ("odd seq stride", dict(q_ss=130), 3),
    ("negative stride", dict(k_sh=-8), 3),
    ("huge key stride", dict(k_ss=1 << 24), 3),
    ("misaligned q", dict(q=FAKE + 2), 4),
    ("misaligned v", dict(v=FAKE + 8), 4),
    ("misaligned lse", dict(lse=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", PREFILL_BAD, ids=[c[0] for c in PREFILL_BAD])
def test_prefill_rejects(name, over, code):
    lib = afa.load_library()
    a = good_prefill(**over)
    st = lib.attn_fwd_prefill(ctypes.byref(a), None)
    assert st == code, (st, lib.attn_last_error())
    assert lib.attn_last_error().decode() != ""


@pytest.mark.parametrize("name,over,code", PREFILL_BAD, ids=[c[0] for c in PREFILL_BAD])
def test_prefill_chunked_rejects(name, over, code):
    lib = afa.load_library()
    a = good_prefill(**over)
    st = lib.attn_fwd_prefill_chunked(ctypes.byref(a), None, 0, None)
    assert st == code, (st, lib.attn_last_error())
    assert lib.attn_fwd_prefill_chunked_workspace_size(ctypes.byref(a)) == 0


def wide_prefill(**over):
    """b=1, h=4, s=4096, d=512 causal, BHSD-contiguous strides."""
    s, d = over.pop("s", 4096), 512
    h = over.get("h_q", 4)
    base = dict(b=1, h_q=h, h_kv=h, s_q=s, s_k=s, d=d, causal=1,
                q_sb=h * s * d, q_sh=s * d, q_ss=d, k_sb=h * s * d, k_sh=s * d, k_ss=d,
                v_sb=h * s * d, v_sh=s * d, v_ss=d, o_sb=h * s * d, o_sh=s * d, o_ss=d)
    base.update(over)
    return good_prefill(**base)


def _chunk_plan_rows(b, h, s_q, s_k, bm=128, bn=32, fixed=10, xcds=8, cus=32, target=256, min_tiles=8):
    """The chunk plan's rule restated: partial rows of the chunk length whose simulated launch ends first."""
    import heapq
    nq = -(-s_q // bm)
    T = [-(-max(0, min(s_k, min(s_q, (qt + 1) * bm) - 1 + s_k - s_q + 1)) // bn) for qt in range(nq)]
    bh, tmax = b * h, max(T)
    c0 = max(min_tiles, -(-sum(T) * bh // target))
    if c0 >= tmax:
        return 0
    best = None
    lo, hi = max(min_tiles, c0 * 3 // 4), min(tmax - 1, 2 * c0)
    for c in range(lo, hi + 1, max(1, (hi - lo) // 63)):
        units = sorted(((min(c, T[qt] - ch * c), qt) for qt in range(nq) for ch in range(-(-T[qt] // c))),
                       key=lambda u: (-u[0], -u[1]))
        heaps = [[0] * cus for _ in range(xcds)]
        mk, v = 0, 0
        for length, _ in units:
            for _ in range(bh):
                t = heapq.heappop(heaps[v % xcds]) + length + fixed
                heapq.heappush(heaps[v % xcds], t)
                mk, v = max(mk, t), v + 1
        if best is None or mk <= best[0]:
            best = (mk, c)
    c = best[1]
    qt0 = sum(1 for t in T if t <= c)
    return bh * (nq - qt0) * -(-tmax // c) * bm


def test_prefill_chunked_plan_sizes():
    lib = afa.load_library()
    size = lambda a: lib.attn_fwd_prefill_chunked_workspace_size(ctypes.byref(a))
    # 32 query tiles of 128 rows; tile qt sees 4(qt+1) key tiles of 32.  The
    # simulated launch ends first with 36-tile chunks: tiles 9..31 (40..128 key
    # tiles) get 2..4 chunks (parts: 4 heads x 23 tiles x 4 chunk slots x 128 rows).
    rows = 4 * 23 * 4 * 128
    assert _chunk_plan_rows(1, 4, 4096, 4096) == rows
    assert size(wide_prefill()) == 256 + rows * 512 * 2 + rows * 4  # queue header, then the partials
    for s in (1024, 2048, 3000, 8192, 16384):  # at s = 16384 the candidates are spaced
        r = _chunk_plan_rows(1, 4, s, s)
        want = 256 + (r * 512 * 2 + 255) // 256 * 256 + r * 4 if r else 0
        assert size(wide_prefill(s=s)) == want, s
    # nothing to balance, or not a chunked shape: 0
    assert size(wide_prefill(causal=0)) == 0
    assert size(wide_prefill(window=1024)) == 0
    assert size(wide_prefill(h_q=64)) == 0   # 4096 query tiles: enough units already
    assert size(wide_prefill(s=0)) == 0
    a = good_prefill(causal=1, s_q=4096, s_k=4096, q_ss=128, k_ss=128, v_ss=128, o_ss=128,
                     q_sh=4096 * 128, k_sh=4096 * 128, v_sh=4096 * 128, o_sh=4096 * 128,
                     q_sb=2 * 4096 * 128, k_sb=4096 * 128, v_sb=4096 * 128, o_sb=2 * 4096 * 128)
    assert size(a) == 0                      # head dim 128 runs the single-pass kernel


def test_prefill_chunked_workspace_checks():
    lib = afa.load_library()
    a = wide_prefill()
    need = lib.attn_fwd_prefill_chunked_workspace_size(ctypes.byref(a))
    assert need > 0
    assert lib.attn_fwd_prefill_chunked(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_fwd_prefill_chunked(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_fwd_prefill_chunked(ctypes.byref(a), ctypes.c_void_p(FAKE + 16), need, None) == 4
    e = wide_prefill(s=0)
    assert lib.attn_fwd_prefill_chunked(ctypes.byref(e), None, 0, None) == 0
    # the work-queue shapes (d = 256, any mask) check their 256-byte header the same way
    for d in (256,):
        q = good_prefill(causal=1, s_q=1024, s_k=1024, d=d, q_ss=d, k_ss=d, v_ss=d, o_ss=d, q_sh=1024 * d,
                         k_sh=1024 * d, v_sh=1024 * d, o_sh=1024 * d, q_sb=1024 * d, k_sb=1024 * d,
                         v_sb=1024 * d, o_sb=1024 * d)
        assert lib.attn_fwd_prefill_chunked_workspace_size(ctypes.byref(q)) == 256
        assert lib.attn_fwd_prefill_chunked(ctypes.byref(q), None, 256, None) == 6
        assert lib.attn_fwd_prefill_chunked(ctypes.byref(q), ctypes.c_void_p(FAKE), 255, None) == 6
        assert lib.attn_fwd_prefill_chunked(ctypes.byref(q), ctypes.c_void_p(FAKE + 16), 256, None) == 4


def test_prefill_null_args():
    lib = afa.load_library()
    assert lib.attn_fwd_prefill(None, None) == 1


def test_prefill_empty_query_is_noop():
    # s_q = 0 is valid and returns before any HIP call
    lib = afa.load_library()
    a = good_prefill(s_q=0)
    assert lib.attn_fwd_prefill(ctypes.byref(a), None) == 0


def good_decode(**over):
    a = DecodeArgs()
    a.q = a.k = a.v = a.o = FAKE
    a.kv_start = a.kv_len = FAKE
    a.lse = None
    a.sinks = None
    a.B, a.h_q, a.h_kv, a.d = 4, 128, 1, 128
    a.max_kv_len, a.split_size = 8192, 512
    a.q_sb, a.q_sh = 128 * 128, 128
    a.k_st, a.k_sh, a.v_st, a.v_sh = 128, 0, 128, 0
    a.o_sb, a.o_sh = 128 * 128, 128
    a.lse_sb = 128
    a.scale = 0.088
    for k, v in over.items():
        setattr(a, k, v)
    return a


DECODE_BAD = [
    ("null kv_len", dict(kv_len=None), 1),
    ("null q", dict(q=None), 1),
    ("d=512", dict(d=512), 2),
    ("ratio", dict(h_q=6, h_kv=4), 2),
    ("split 100", dict(split_size=100), 2),
    ("split 0", dict(split_size=0), 2),
    ("negative max len", dict(max_kv_len=-1), 2),
    ("zero scale", dict(scale=0.0), 2),
    ("odd token stride", dict(k_st=12), 3),
    ("huge token stride", dict(v_st=1 << 24), 3),
    ("misaligned k", dict(k=FAKE + 4), 4),
    ("misaligned kv_start", dict(kv_start=FAKE + 4), 4),
]


@pytest.mark.parametrize("name,over,code", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_rejects(name, over, code):
    lib = afa.load_library()
    a = good_decode(**over)
    st = lib.attn_fwd_decode(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None)
    assert st == code, (st, lib.attn_last_error())


@pytest.mark.parametrize("name,over,code", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_noalloc_rejects(name, over, code):
    """The no-allocation decode checks its arguments like attn_fwd_decode, before any HIP call."""
    lib = afa.load_library()
    a = good_decode(**over)
    st = lib.attn_fwd_decode_noalloc(ctypes.byref(a), None)
    assert st == code, (st, lib.attn_last_error())


def test_decode_rejects_partials_beyond_a_32_bit_range():
    """The merge reads one sequence's partial rows through a 32-bit buffer range."""
    lib = afa.load_library()
    # h_q 128 x d 128 x 2 bytes x splits > 2^32 from 131073 splits of 64 keys
    a = good_decode(split_size=64, max_kv_len=131073 * 64)
    assert lib.attn_fwd_decode(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None) == 2
    assert b"too many splits" in lib.attn_last_error()


def test_decode_noalloc_rejects_sizes_beyond_its_scratch():
    lib = afa.load_library()
    # B = 64, h_q = 128, d = 256, 16384 keys in 512-key splits: 128 MiB of partials
    a = good_decode(B=64, h_q=128, d=256, max_kv_len=16384)
    need = lib.attn_fwd_decode_workspace_size(64, 128, 256, 16384, 512)
    assert need > 72 << 20
    assert lib.attn_fwd_decode_noalloc(ctypes.byref(a), None) == 6
    assert b"scratch" in lib.attn_last_error()
    # the largest decode workload (d = 256, 8192 keys) fits
    assert lib.attn_fwd_decode_workspace_size(64, 128, 256, 8192, 512) <= 72 << 20


def good_paged(**over):
    a = DecodePagedArgs()
    a.q = a.k = a.v = a.o = FAKE
    a.block_table = a.kv_len = FAKE
    a.lse = None
    a.sinks = None
    a.B, a.h_q, a.h_kv, a.d = 4, 128, 1, 128
    a.max_kv_len, a.split_size = 8192, 512
    a.page_size, a.n_pages = 64, 1000
    a.bt_stride = 128
    a.q_sb, a.q_sh = 128 * 128, 128
    a.k_ps, a.k_ts, a.k_sh = 64 * 128, 128, 0
    a.v_ps, a.v_ts, a.v_sh = 64 * 128, 128, 0
    a.o_sb, a.o_sh = 128 * 128, 128
    a.lse_sb = 128
    a.scale = 0.088
    for k, v in over.items():
        setattr(a, k, v)
    return a


PAGED_BAD = [
    ("null block table", dict(block_table=None), 1),
    ("null kv_len", dict(kv_len=None), 1),
    ("d=512", dict(d=512), 2),
    ("ratio", dict(h_q=6, h_kv=4), 2),
    ("page 8", dict(page_size=8), 2),
    ("page 48", dict(page_size=48), 2),
    ("page above split", dict(page_size=1024), 2),
    ("65 pages per split", dict(split_size=1024 + 64, page_size=16), 2),
    ("split 384, page 256", dict(split_size=384, page_size=256), 2),  # splits would start mid-page
    ("split 192, page 128", dict(split_size=192, page_size=128), 2),
    ("no pages", dict(n_pages=0), 2),
    ("table too narrow", dict(bt_stride=127), 3),
    ("odd page stride", dict(k_ps=12), 3),
    ("huge token stride", dict(v_ts=1 << 24), 3),
    ("misaligned v", dict(v=FAKE + 8), 4),
    ("misaligned block table", dict(block_table=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", PAGED_BAD, ids=[c[0] for c in PAGED_BAD])
def test_decode_paged_rejects(name, over, code):
    lib = afa.load_library()
    a = good_paged(**over)
    st = lib.attn_fwd_decode_paged(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None)
    assert st == code, (st, lib.attn_last_error())


def good_paged_fp8(**over):
    a = DecodePagedFp8Args()
    a.q = a.k = a.v = a.o = FAKE
    a.k_scale = a.v_scale = FAKE
    a.block_table = a.kv_len = FAKE
    a.lse = None
    a.sinks = None
    a.B, a.h_q, a.h_kv, a.d = 4, 128, 1, 128
    a.max_kv_len, a.split_size = 8192, 512
    a.page_size, a.n_pages = 64, 1000
    a.bt_stride = 128
    a.q_sb, a.q_sh = 128 * 128, 128
    a.k_ps, a.k_ts, a.k_sh = 64 * 128, 128, 0  # bytes
    a.v_ps, a.v_ts, a.v_sh = 64 * 128, 128, 0
    a.o_sb, a.o_sh = 128 * 128, 128
    a.lse_sb = 128
    a.scale = 0.088
    for k, v in over.items():
        setattr(a, k, v)
    return a


PAGED_FP8_BAD = [
    ("null k_scale", dict(k_scale=None), 1),
    ("null block table", dict(block_table=None), 1),
    ("d=64", dict(d=64), 2),
    ("d=512", dict(d=512), 2),
    ("ratio", dict(h_q=6, h_kv=4), 2),
    ("page 8", dict(page_size=8), 2),
    ("split 384, page 256", dict(split_size=384, page_size=256), 2),
    ("no pages", dict(n_pages=0), 2),
    ("table too narrow", dict(bt_stride=127), 3),
    ("page stride 8 bytes", dict(k_ps=8), 3),
    ("token stride 24 bytes", dict(v_ts=24), 3),
    ("huge token stride", dict(k_ts=1 << 24), 3),
    ("misaligned v", dict(v=FAKE + 8), 4),
    ("misaligned scale", dict(k_scale=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", PAGED_FP8_BAD, ids=[c[0] for c in PAGED_FP8_BAD])
def test_decode_paged_fp8_rejects(name, over, code):
    lib = afa.load_library()
    a = good_paged_fp8(**over)
    st = lib.attn_fwd_decode_paged_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None)
    assert st == code, (st, lib.attn_last_error())


def test_decode_paged_fp8_workspace_checks():
    lib = afa.load_library()
    a = good_paged_fp8(d=256)
    need = lib.attn_fwd_decode_workspace_size(4, 128, 256, 8192, 512)
    assert lib.attn_fwd_decode_paged_fp8(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_fwd_decode_paged_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_fwd_decode_paged_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), need, None) == 4


def test_decode_paged_workspace_checks():
    lib = afa.load_library()
    a = good_paged()
    need = lib.attn_fwd_decode_workspace_size(4, 128, 128, 8192, 512)
    assert lib.attn_fwd_decode_paged(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_fwd_decode_paged(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_fwd_decode_paged(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), need, None) == 4


def good_fp8(**over):
    a = DecodeFp8Args()
    a.q = a.k = a.v = a.o = FAKE
    a.k_scale = a.v_scale = FAKE
    a.kv_start = a.kv_len = FAKE
    a.lse = None
    a.sinks = None
    a.B, a.h_q, a.h_kv, a.d = 4, 128, 1, 128
    a.max_kv_len, a.split_size = 8192, 512
    a.q_sb, a.q_sh = 128 * 128, 128
    a.k_st, a.k_sh, a.v_st, a.v_sh = 128, 0, 128, 0
    a.o_sb, a.o_sh = 128 * 128, 128
    a.lse_sb = 128
    a.scale = 0.088
    for k, v in over.items():
        setattr(a, k, v)
    return a


FP8_BAD = [
    ("null k_scale", dict(k_scale=None), 1),
    ("null v_scale", dict(v_scale=None), 1),
    ("d=64", dict(d=64), 2),
    ("d=512", dict(d=512), 2),
    ("ratio", dict(h_q=6, h_kv=4), 2),
    ("split 100", dict(split_size=100), 2),
    ("token stride 8 bytes", dict(k_st=8), 3),
    ("head stride 24 bytes", dict(v_sh=24), 3),
    ("huge token stride", dict(k_st=1 << 24), 3),
    ("misaligned k", dict(k=FAKE + 8), 4),
    ("misaligned scale", dict(v_scale=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", FP8_BAD, ids=[c[0] for c in FP8_BAD])
def test_decode_fp8_rejects(name, over, code):
    lib = afa.load_library()
    a = good_fp8(**over)
    st = lib.attn_fwd_decode_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None)
    assert st == code, (st, lib.attn_last_error())


def test_decode_fp8_workspace_checks():
    lib = afa.load_library()
    a = good_fp8()
    need = lib.attn_fwd_decode_workspace_size(4, 128, 128, 8192, 512)
    assert lib.attn_fwd_decode_fp8(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_fwd_decode_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_fwd_decode_fp8(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), need, None) == 4


def test_decode_workspace_header_constant_matches_c_header():
    text = open(os.path.join(ROOT, "include", "attn_fwd.h")).read()
    m = re.search(r"#define ATTN_DECODE_WORKSPACE_HEADER \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == afa.DECODE_WORKSPACE_HEADER


def test_decode_workspace_checks():
    lib = afa.load_library()
    a = good_decode()
    need = lib.attn_fwd_decode_workspace_size(4, 128, 128, 8192, 512)
    # the counter header, then 4 sequences x 128 heads x 16 splits x (128 bf16 outputs + 1 fp32 LSE)
    assert need == afa.DECODE_WORKSPACE_HEADER + 4 * 128 * 16 * (128 * 2 + 4)
    assert lib.attn_fwd_decode(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_fwd_decode(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_fwd_decode(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), need, None) == 4
    assert lib.attn_fwd_decode_workspace_size(0, 128, 128, 8192, 512) == 0
    assert lib.attn_fwd_decode_workspace_size(4, 128, 128, 8192, 100) == 0


def good_combine(**over):
    a = CombineArgs()
    a.o_parts = a.lse_parts = a.o_out = FAKE
    a.lse_out = None
    a.n_parts, a.rows, a.d = 4, 16, 128
    a.o_part_stride, a.o_row_stride = 16 * 128, 128
    a.lse_part_stride, a.lse_row_stride = 16, 1
    a.o_out_row_stride = 128
    for k, v in over.items():
        setattr(a, k, v)
    return a


COMBINE_BAD = [
    ("null parts", dict(o_parts=None), 1),
    ("zero parts", dict(n_parts=0), 2),
    ("too many parts", dict(n_parts=5000), 2),
    ("d=12", dict(d=12), 2),
    ("d=1024", dict(d=1024), 2),
    ("part stride", dict(o_part_stride=6), 3),
    ("out stride", dict(o_out_row_stride=12), 3),
    ("misaligned out", dict(o_out=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", COMBINE_BAD, ids=[c[0] for c in COMBINE_BAD])
def test_combine_rejects(name, over, code):
    lib = afa.load_library()
    a = good_combine(**over)
    assert lib.attn_combine(ctypes.byref(a), None) == code, lib.attn_last_error()


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        afa.prefill(q, q, q)


def good_bwd(**over):
    a = BwdArgs()
    a.q = a.k = a.v = a.o = a.d_o = a.lse = a.dq = a.dk = a.dv = FAKE
    a.b, a.h_q, a.h_kv, a.s_q, a.s_k, a.d = 2, 16, 16, 4096, 4096, 128
    a.q_sb, a.q_sh, a.q_ss = 16 * 4096 * 128, 4096 * 128, 128
    a.k_sb, a.k_sh, a.k_ss = 16 * 4096 * 128, 4096 * 128, 128
    a.lse_sb, a.lse_sh = 16 * 4096, 4096
    a.scale = 0.088
    a.causal = 1
    for k, v in over.items():
        setattr(a, k, v)
    return a


BWD_BAD = [
    ("null lse", dict(lse=None), 1),
    ("null dv", dict(dv=None), 1),
    ("d=512", dict(d=512), 2),
    ("d=96", dict(d=96), 2),
    ("ratio", dict(h_q=6, h_kv=4), 2),
    ("causal 2", dict(causal=2), 2),
    ("zero scale", dict(scale=0.0), 2),
    ("odd row stride", dict(q_ss=100), 3),
    ("huge row stride", dict(k_ss=1 << 24), 3),
    ("misaligned dq", dict(dq=FAKE + 8), 4),
    ("misaligned lse", dict(lse=FAKE + 2), 4),
    ("window without causal", dict(causal=0, window=16), 2),
    ("negative window", dict(window=-1), 2),
    ("d_sinks without sinks", dict(d_sinks=FAKE), 1),
    ("null q with rows", dict(q=None), 1),
    ("null dk with keys", dict(dk=None), 1),
    ("misaligned d_sinks", dict(sinks=FAKE, d_sinks=FAKE + 2), 4),
]


@pytest.mark.parametrize("name,over,code", BWD_BAD, ids=[c[0] for c in BWD_BAD])
def test_bwd_rejects(name, over, code):
    lib = afa.load_library()
    a = good_bwd(**over)
    st = lib.attn_bwd(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None)
    assert st == code, (st, lib.attn_last_error())


def test_bwd_empty_sides_may_be_null():
    """s_q = 0 and s_k = 0: nothing to compute and no pointer needed, returns before any HIP call."""
    lib = afa.load_library()
    a = good_bwd(s_q=0, s_k=0, q=None, o=None, d_o=None, lse=None, dq=None, k=None, v=None, dk=None, dv=None)
    assert lib.attn_bwd(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 20, None) == 0, lib.attn_last_error()


def test_bwd_workspace_checks():
    lib = afa.load_library()
    a = good_bwd()
    need = lib.attn_bwd_workspace_size(2, 16, 4096)
    # D and the base-2 LSE per row, then the sink-gradient partials per 128 query rows (the
    # dQ kernel's shortest query tile, at d = 256)
    assert need == 2 * (2 * 16 * 4096 * 4) + 2 * 16 * (4096 // 128) * 4
    assert lib.attn_bwd_workspace_size(1, 1, 129) == 2 * 768 + 2 * 4  # 516 bytes of rows aligned to 768
    assert lib.attn_bwd(ctypes.byref(a), None, need, None) == 6
    assert lib.attn_bwd(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 1, None) == 6
    assert lib.attn_bwd(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), need, None) == 4


"""ctypes binding of ``libattnfwd.so`` (C ABI declared in include/attn_fwd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch tensors are used as device memory and for the
current stream; there is no fallback of any kind -- if the library is missing
or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattnfwd.so")

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_STRIDE",
    4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_UNSUPPORTED", 6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_HIP",
}


class AttnError(RuntimeError):
    """A non-OK status returned by the C ABI."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("b", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("s_q", ctypes.c_int32), ("s_k", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_ss", ctypes.c_int64),
        ("k_sb", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("k_ss", ctypes.c_int64),
        ("v_sb", ctypes.c_int64), ("v_sh", ctypes.c_int64), ("v_ss", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64), ("o_ss", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64), ("lse_sh", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_start", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("split_size", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_st", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v_st", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class DecodePagedArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("split_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("bt_stride", ctypes.c_int64),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_ps", ctypes.c_int64), ("k_ts", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v_ps", ctypes.c_int64), ("v_ts", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class DecodeFp8Args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("kv_start", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("split_size", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_st", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v_st", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class DecodePagedFp8Args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("split_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("bt_stride", ctypes.c_int64),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_ps", ctypes.c_int64), ("k_ts", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v_ps", ctypes.c_int64), ("v_ts", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("d_o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("b", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("s_q", ctypes.c_int32), ("s_k", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_ss", ctypes.c_int64),
        ("k_sb", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("k_ss", ctypes.c_int64),
        ("lse_sb", ctypes.c_int64), ("lse_sh", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("sinks", ctypes.c_void_p), ("d_sinks", ctypes.c_void_p),
    ]


class CombineArgs(ctypes.Structure):
    _fields_ = [
        ("o_parts", ctypes.c_void_p), ("lse_parts", ctypes.c_void_p),
        ("o_out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p),
        ("n_parts", ctypes.c_int32), ("rows", ctypes.c_int32), ("d", ctypes.c_int32),
        ("o_part_stride", ctypes.c_int64), ("o_row_stride", ctypes.c_int64),
        ("lse_part_stride", ctypes.c_int64), ("lse_row_stride", ctypes.c_int64),
        ("o_out_row_stride", ctypes.c_int64),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (there is no fallback path)")
    lib = ctypes.CDLL(path)
    lib.attn_fwd_prefill.argtypes = [ctypes.POINTER(PrefillArgs), ctypes.c_void_p]
    lib.attn_fwd_prefill.restype = ctypes.c_int
    lib.attn_fwd_prefill_chunked.argtypes = [ctypes.POINTER(PrefillArgs), ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]
    lib.attn_fwd_prefill_chunked.restype = ctypes.c_int
    lib.attn_fwd_prefill_chunked_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.attn_fwd_prefill_chunked_workspace_size.restype = ctypes.c_size_t
    lib.attn_fwd_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
    lib.attn_fwd_decode.restype = ctypes.c_int
    lib.attn_fwd_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
    lib.attn_fwd_decode_noalloc.restype = ctypes.c_int
    lib.attn_fwd_decode_paged.argtypes = [ctypes.POINTER(DecodePagedArgs), ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]
    lib.attn_fwd_decode_paged.restype = ctypes.c_int
    lib.attn_fwd_decode_fp8.argtypes = [ctypes.POINTER(DecodeFp8Args), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
    lib.attn_fwd_decode_fp8.restype = ctypes.c_int
    lib.attn_fwd_decode_paged_fp8.argtypes = [ctypes.POINTER(DecodePagedFp8Args), ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]
    lib.attn_fwd_decode_paged_fp8.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int32] * 3
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_combine.argtypes = [ctypes.POINTER(CombineArgs), ctypes.c_void_p]
    lib.attn_combine.restype = ctypes.c_int
    lib.attn_fwd_decode_workspace_size.argtypes = [ctypes.c_int32] * 5
    lib.attn_fwd_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = load_library()
        raise AttnError(status, lib.attn_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, ctypes.c_void_p):
        return stream
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on_stream(fn):
    """Run a binding call with its ``stream`` as torch's current stream.

    Outputs and workspaces the call allocates are then allocated on the stream
    the kernels run on, so the caching allocator orders any reuse of that
    memory after those kernels, and a workspace zeroed here is zeroed on that
    stream before the kernels read it.  The inputs must already be ready on
    that stream (as with any torch op issued there).  ``stream`` may be a
    torch stream, a raw hipStream_t handle (int) or None (torch's current
    stream).
    """
    import functools

    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        import torch

        if stream is None:
            return fn(*args, stream=None, **kw)
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(stream.cuda_stream if hasattr(stream, "cuda_stream")
                                               else int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)

    return call


def _require_cuda_bf16(name, t, ndim):
    import torch

    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in the head dim")


def prefill_args(q, k, v, out, lse, sinks, scale, causal, window) -> PrefillArgs:
    """Fill the C argument struct from [b, h, s, d]-indexed tensors (any strides)."""
    b, h_q, s_q, d = q.shape
    _, h_kv, s_k, _ = k.shape
    a = PrefillArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.b, a.h_q, a.h_kv, a.s_q, a.s_k, a.d = b, h_q, h_kv, s_q, s_k, d
    a.q_sb, a.q_sh, a.q_ss = q.stride(0), q.stride(1), q.stride(2)
    a.k_sb, a.k_sh, a.k_ss = k.stride(0), k.stride(1), k.stride(2)
    a.v_sb, a.v_sh, a.v_ss = v.stride(0), v.stride(1), v.stride(2)
    a.o_sb, a.o_sh, a.o_ss = out.stride(0), out.stride(1), out.stride(2)
    if lse is not None:
        a.lse_sb, a.lse_sh = lse.stride(0), lse.stride(1)
    a.scale = scale
    a.causal = 1 if causal else 0
    a.window = int(window)
    return a


@_on_stream
def prefill(q, k, v, *, scale: float | None = None, causal: bool = False, window: int = 0,
            sinks=None, out=None, lse=None, return_lse: bool = True, chunked: bool = True,
            workspace=None, stream=None):
    """Fused attention forward over [b, h, s, d]-indexed bf16 device tensors.

    q is [b, h_q, s_q, d]; k and v are [b, h_kv, s_k, d] (any strides with a
    unit head-dim stride, e.g. a transposed [b, s, h, d] view).  Returns
    (O, LSE): O bf16 shaped like q, LSE fp32 [b, h_q, s_q] (None when
    ``return_lse`` is False and no ``lse`` buffer is given).

    With ``chunked`` (the default) the call goes through the scheduled
    attn_fwd_prefill_chunked: long causal key ranges cut into chunks when the
    library's plan says so (d = 512), or query tiles taken from per-XCD work
    queues (d = 256); ``workspace`` (uint8 device tensor
    whose first 256 bytes are zero before its first use, as every call leaves
    them) is then used if given, else allocated zeroed.  ``chunked=False``
    always runs the single-pass attn_fwd_prefill.
    """
    import torch

    lib = load_library()
    _require_cuda_bf16("q", q, 4)
    _require_cuda_bf16("k", k, 4)
    _require_cuda_bf16("v", v, 4)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    b, h_q, s_q, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, h_q, s_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    if lse is not None and lse.stride(-1) != 1:
        raise ValueError("lse must have unit stride along the sequence")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 device tensor")
    a = prefill_args(q, k, v, out, lse, sinks, scale, causal, window)
    need = int(lib.attn_fwd_prefill_chunked_workspace_size(ctypes.byref(a))) if chunked else 0
    if need == 0:
        _check(lib.attn_fwd_prefill(ctypes.byref(a), _stream(stream)))
        return out, lse
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # zeroed queue header
    _check(lib.attn_fwd_prefill_chunked(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse



# ATTN_DECODE_WORKSPACE_HEADER: the leading bytes of a decode workspace that
# hold the merge's arrival counters (zero before the first call, left zero).
DECODE_WORKSPACE_HEADER = 64 << 10


def decode_workspace_size(B: int, h_q: int, d: int, max_kv_len: int, split_size: int = 512) -> int:
    return int(load_library().attn_fwd_decode_workspace_size(B, h_q, d, max_kv_len, split_size))


def new_decode_workspace(nbytes: int, device):
    """A decode workspace of nbytes with its counter header zeroed (the rest is left as allocated)."""
    import torch

    ws = torch.empty(max(nbytes, DECODE_WORKSPACE_HEADER), dtype=torch.uint8, device=device)
    ws[:DECODE_WORKSPACE_HEADER].zero_()
    return ws


def _decode_args(q, k, v, kv_start, kv_len, max_kv_len, scale, sinks, split_size, out, lse, return_lse):
    """Check the tensors of a contiguous-cache decode and fill the C argument struct (and outputs)."""
    import torch

    _require_cuda_bf16("q", q, 3)
    _require_cuda_bf16("k", k, 3)
    _require_cuda_bf16("v", v, 3)
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32:
        raise ValueError("kv_start must be int64 and kv_len int32")
    B, h_q, d = q.shape
    h_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, h_q), dtype=torch.float32, device=q.device)
    if lse is not None and lse.stride(-1) != 1:
        raise ValueError("lse must have unit stride along the heads")
    a = DecodeArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.kv_start, a.kv_len = kv_start.data_ptr(), kv_len.data_ptr()
    a.o = out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.B, a.h_q, a.h_kv, a.d = B, h_q, h_kv, d
    a.max_kv_len, a.split_size = int(max_kv_len), int(split_size)
    a.q_sb, a.q_sh = q.stride(0), q.stride(1)
    a.k_st, a.k_sh = k.stride(0), k.stride(1)
    a.v_st, a.v_sh = v.stride(0), v.stride(1)
    a.o_sb, a.o_sh = out.stride(0), out.stride(1)
    a.lse_sb = lse.stride(0) if lse is not None else 0
    a.scale = scale
    return a, out, lse


@_on_stream
def decode(q, k, v, kv_start, kv_len, max_kv_len: int, *, scale: float | None = None, sinks=None,
           split_size: int = 512, workspace=None, out=None, lse=None, return_lse: bool = True,
           stream=None):
    """Single-token decode over a per-sequence contiguous KV cache (split-KV + LSE merge).

    q: bf16 [B, h_q, d]; k, v: bf16 [T, h_kv, d] (token-major cache; any token
    and head strides with a unit head-dim stride); kv_start: int64 [B];
    kv_len: int32 [B]; max_kv_len: host upper bound on kv_len.
    Returns (O bf16 [B, h_q, d], LSE fp32 [B, h_q] or None).
    """
    import torch

    lib = load_library()
    a, out, lse = _decode_args(q, k, v, kv_start, kv_len, max_kv_len, scale, sinks, split_size, out, lse,
                               return_lse)
    need = int(lib.attn_fwd_decode_workspace_size(a.B, a.h_q, a.d, a.max_kv_len, a.split_size))
    if workspace is None:
        workspace = new_decode_workspace(need, q.device)
    _check(lib.attn_fwd_decode(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


@_on_stream
def decode_noalloc(q, k, v, kv_start, kv_len, max_kv_len: int, *, scale: float | None = None, sinks=None,
                   split_size: int = 512, out=None, lse=None, return_lse: bool = True, stream=None):
    """decode() through attn_fwd_decode_noalloc: no workspace, the library's fixed scratch region.

    Calls that may overlap on one GPU race (they share the region).  The
    outputs are allocated here unless ``out`` (and ``lse``) are given.
    """
    lib = load_library()
    a, out, lse = _decode_args(q, k, v, kv_start, kv_len, max_kv_len, scale, sinks, split_size, out, lse,
                               return_lse)
    _check(lib.attn_fwd_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out, lse


@_on_stream
def decode_paged(q, k_cache, v_cache, block_table, kv_len, max_kv_len: int, *, scale: float | None = None,
                 sinks=None, split_size: int = 512, workspace=None, out=None, lse=None,
                 return_lse: bool = True, stream=None):
    """Single-token decode over a paged KV cache (block table), split-KV + LSE merge.

    q: bf16 [B, h_q, d]; k_cache, v_cache: bf16 [n_pages, page_size, h_kv, d]
    (any page, token and head strides with a unit head-dim stride);
    block_table: int32 [B, max_pages] (row b lists the pages of sequence b in
    token order); kv_len: int32 [B]; max_kv_len: host upper bound on kv_len.
    Returns (O bf16 [B, h_q, d], LSE fp32 [B, h_q] or None).
    """
    import torch

    lib = load_library()
    _require_cuda_bf16("q", q, 3)
    _require_cuda_bf16("k_cache", k_cache, 4)
    _require_cuda_bf16("v_cache", v_cache, 4)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, max_pages] with unit column stride")
    if kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    B, h_q, d = q.shape
    n_pages, page_size, h_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.attn_fwd_decode_workspace_size(B, h_q, d, max_kv_len, split_size))
    if workspace is None:
        workspace = new_decode_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, h_q), dtype=torch.float32, device=q.device)
    if lse is not None and lse.stride(-1) != 1:
        raise ValueError("lse must have unit stride along the heads")
    a = DecodePagedArgs()
    a.q, a.k, a.v = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.block_table, a.kv_len = block_table.data_ptr(), kv_len.data_ptr()
    a.o = out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.B, a.h_q, a.h_kv, a.d = B, h_q, h_kv, d
    a.max_kv_len, a.split_size = int(max_kv_len), int(split_size)
    a.page_size, a.n_pages = int(page_size), int(n_pages)
    a.bt_stride = block_table.stride(0)
    a.q_sb, a.q_sh = q.stride(0), q.stride(1)
    a.k_ps, a.k_ts, a.k_sh = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    a.v_ps, a.v_ts, a.v_sh = v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)
    a.o_sb, a.o_sh = out.stride(0), out.stride(1)
    a.lse_sb = lse.stride(0) if lse is not None else 0
    a.scale = scale
    _check(lib.attn_fwd_decode_paged(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


@_on_stream
def decode_fp8(q, k8, v8, k_scale, v_scale, kv_start, kv_len, max_kv_len: int, *, scale: float | None = None,
               sinks=None, split_size: int = 512, workspace=None, out=None, lse=None,
               return_lse: bool = True, stream=None):
    """Single-token decode over an FP8 (E4M3) KV cache with per-kv-head scales.

    q: bf16 [B, h_q, d]; k8, v8: uint8 E4M3 codes [T, h_kv, d] (token and head
    strides multiples of 16 bytes, unit head-dim stride); k_scale, v_scale:
    fp32 [h_kv]; kv_start: int64 [B]; kv_len: int32 [B].
    Returns (O bf16 [B, h_q, d], LSE fp32 [B, h_q] or None).
    """
    import torch

    lib = load_library()
    _require_cuda_bf16("q", q, 3)
    for name, t in (("k8", k8), ("v8", v8)):
        if not t.is_cuda or t.dtype != torch.uint8 or t.dim() != 3 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a uint8 device tensor [T, h_kv, d] with unit last stride")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32:
        raise ValueError("kv_start must be int64 and kv_len int32")
    B, h_q, d = q.shape
    h_kv = k8.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.attn_fwd_decode_workspace_size(B, h_q, d, max_kv_len, split_size))
    if workspace is None:
        workspace = new_decode_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, h_q), dtype=torch.float32, device=q.device)
    if lse is not None and lse.stride(-1) != 1:
        raise ValueError("lse must have unit stride along the heads")
    a = DecodeFp8Args()
    a.q, a.k, a.v = q.data_ptr(), k8.data_ptr(), v8.data_ptr()
    a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    a.kv_start, a.kv_len = kv_start.data_ptr(), kv_len.data_ptr()
    a.o = out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.B, a.h_q, a.h_kv, a.d = B, h_q, h_kv, d
    a.max_kv_len, a.split_size = int(max_kv_len), int(split_size)
    a.q_sb, a.q_sh = q.stride(0), q.stride(1)
    a.k_st, a.k_sh = k8.stride(0), k8.stride(1)
    a.v_st, a.v_sh = v8.stride(0), v8.stride(1)
    a.o_sb, a.o_sh = out.stride(0), out.stride(1)
    a.lse_sb = lse.stride(0) if lse is not None else 0
    a.scale = scale
    _check(lib.attn_fwd_decode_fp8(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


@_on_stream
def decode_paged_fp8(q, k8_cache, v8_cache, k_scale, v_scale, block_table, kv_len, max_kv_len: int, *,
                     scale: float | None = None, sinks=None, split_size: int = 512, workspace=None, out=None,
                     lse=None, return_lse: bool = True, stream=None):
    """Single-token decode over a paged FP8 (E4M3) KV cache with per-kv-head scales.

    q: bf16 [B, h_q, d]; k8_cache, v8_cache: uint8 E4M3 codes [n_pages,
    page_size, h_kv, d] (page, token and head strides multiples of 16 bytes,
    unit head-dim stride); k_scale, v_scale: fp32 [h_kv]; block_table: int32
    [B, max_pages]; kv_len: int32 [B].  Returns (O bf16 [B, h_q, d], LSE fp32
    [B, h_q] or None).
    """
    import torch

    lib = load_library()
    _require_cuda_bf16("q", q, 3)
    for name, t in (("k8_cache", k8_cache), ("v8_cache", v8_cache)):
        if not t.is_cuda or t.dtype != torch.uint8 or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a uint8 device tensor [n_pages, page_size, h_kv, d] with unit last stride")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, max_pages] with unit column stride")
    if kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32")
    if k8_cache.shape != v8_cache.shape:
        raise ValueError("k8_cache and v8_cache must have the same shape")
    B, h_q, d = q.shape
    n_pages, page_size, h_kv = k8_cache.shape[0], k8_cache.shape[1], k8_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.attn_fwd_decode_workspace_size(B, h_q, d, max_kv_len, split_size))
    if workspace is None:
        workspace = new_decode_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, h_q), dtype=torch.float32, device=q.device)
    if lse is not None and lse.stride(-1) != 1:
        raise ValueError("lse must have unit stride along the heads")
    a = DecodePagedFp8Args()
    a.q, a.k, a.v = q.data_ptr(), k8_cache.data_ptr(), v8_cache.data_ptr()
    a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    a.block_table, a.kv_len = block_table.data_ptr(), kv_len.data_ptr()
    a.o = out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.B, a.h_q, a.h_kv, a.d = B, h_q, h_kv, d
    a.max_kv_len, a.split_size = int(max_kv_len), int(split_size)
    a.page_size, a.n_pages = int(page_size), int(n_pages)
    a.bt_stride = block_table.stride(0)
    a.q_sb, a.q_sh = q.stride(0), q.stride(1)
    a.k_ps, a.k_ts, a.k_sh = k8_cache.stride(0), k8_cache.stride(1), k8_cache.stride(2)
    a.v_ps, a.v_ts, a.v_sh = v8_cache.stride(0), v8_cache.stride(1), v8_cache.stride(2)
    a.o_sb, a.o_sh = out.stride(0), out.stride(1)
    a.lse_sb = lse.stride(0) if lse is not None else 0
    a.scale = scale
    _check(lib.attn_fwd_decode_paged_fp8(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def backward_workspace_size(b: int, h_q: int, s_q: int) -> int:
    """Bytes of device workspace backward() needs."""
    return int(load_library().attn_bwd_workspace_size(b, h_q, s_q))


@_on_stream
def backward(q, k, v, o, d_o, lse, *, scale: float | None = None, causal: bool = False, window: int = 0,
             sinks=None, dq=None, dk=None, dv=None, d_sinks=None, workspace=None, stream=None):
    """dQ, dK, dV of the prefill for an incoming gradient d_o, from the forward's o and lse.

    q, o, d_o: bf16 [b, h_q, s_q, d] with identical strides; k, v: bf16
    [b, h_kv, s_k, d] with identical strides; lse: fp32 [b, h_q, s_q] (unit
    stride along s); causal and window as in the forward.  Returns (dq, dk, dv)
    laid out like q, k and v; with ``sinks`` (the forward's fp32 [h_q] sink
    logits) also d_sinks, the sink gradient summed over the batch.
    """
    import torch

    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o)):
        _require_cuda_bf16(name, t, 4)
    if o.stride() != q.stride() or d_o.stride() != q.stride() or o.shape != q.shape or d_o.shape != q.shape:
        raise ValueError("o and d_o must have q's shape and strides")
    if v.stride() != k.stride() or v.shape != k.shape:
        raise ValueError("v must have k's shape and strides")
    if lse.dtype != torch.float32 or lse.dim() != 3 or lse.stride(-1) != 1:
        raise ValueError("lse must be float32 [b, h_q, s_q] with unit stride along s")
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty_strided(q.shape, q.stride(), dtype=torch.bfloat16, device=q.device)
    if dk is None:
        dk = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    if dv is None:
        dv = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=q.device)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != k.stride():
        raise ValueError("dq must have q's strides, dk and dv k's strides")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 device tensor")
    if sinks is not None and d_sinks is None:
        d_sinks = torch.empty(h_q, dtype=torch.float32, device=q.device)
    need = int(lib.attn_bwd_workspace_size(b, h_q, s_q))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a = BwdArgs()
    a.q, a.k, a.v, a.o, a.d_o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), d_o.data_ptr()
    a.lse = lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.b, a.h_q, a.h_kv, a.s_q, a.s_k, a.d = b, h_q, h_kv, s_q, s_k, d
    a.q_sb, a.q_sh, a.q_ss = q.stride(0), q.stride(1), q.stride(2)
    a.k_sb, a.k_sh, a.k_ss = k.stride(0), k.stride(1), k.stride(2)
    a.lse_sb, a.lse_sh = lse.stride(0), lse.stride(1)
    a.scale = scale
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.d_sinks = d_sinks.data_ptr() if d_sinks is not None else None
    _check(lib.attn_bwd(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                        workspace.numel() * workspace.element_size(), _stream(stream)))
    if sinks is not None:
        return dq, dk, dv, d_sinks
    return dq, dk, dv


@_on_stream
def combine(o_parts, lse_parts, *, out=None, lse=None, return_lse: bool = True, stream=None):
    """Merge partial results over disjoint key sets: o_parts fp32 [n, rows, d], lse_parts fp32 [n, rows]."""
    import torch

    lib = load_library()
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be float32")
    if o_parts.dim() != 3 or lse_parts.dim() != 2 or o_parts.stride(-1) != 1:
        raise ValueError("o_parts must be [n, rows, d] with unit last stride, lse_parts [n, rows]")
    n, rows, d = o_parts.shape
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None and return_lse:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    a = CombineArgs()
    a.o_parts, a.lse_parts = o_parts.data_ptr(), lse_parts.data_ptr()
    a.o_out = out.data_ptr()
    a.lse_out = lse.data_ptr() if lse is not None else None
    a.n_parts, a.rows, a.d = n, rows, d
    a.o_part_stride, a.o_row_stride = o_parts.stride(0), o_parts.stride(1)
    a.lse_part_stride, a.lse_row_stride = lse_parts.stride(0), lse_parts.stride(1)
    a.o_out_row_stride = out.stride(0)
    _check(lib.attn_combine(ctypes.byref(a), _stream(stream)))
    return out, lse

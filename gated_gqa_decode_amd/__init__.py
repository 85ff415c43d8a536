"""Gated grouped-query attention for AMD Instinct MI355X (gfx950).

Python binding of ``libgated_attn.so`` (C ABI declared in
``include/gated_attn.h``).  This module only marshals arguments: it checks
tensor dtypes, shapes and devices, allocates outputs and workspaces with torch
(device memory and streams are torch's job here), and calls the library.  Every
step of the computation runs in the library's HIP kernels; there is no other
code path, and importing fails loudly when the library has not been built.

    out = bf16( bf16(softmax(q K^T * scale) V) * bf16(sigmoid(gate)) )

Entry points: :func:`decode` (paged split-KV decode, two kernel launches),
:func:`prefill` (dense causal/non-causal MFMA prefill, one launch),
:func:`decode_plan` / :func:`decode_workspace_size`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgated_attn.so")

GA_OK = 0
GA_ERR_INVALID_ARGUMENT = 1
GA_ERR_UNSUPPORTED = 2
GA_ERR_WORKSPACE_TOO_SMALL = 3
GA_ERR_HIP = 4

# Every symbol include/gated_attn.h declares.
EXPORTED_SYMBOLS = (
    "gated_attn_decode_plan",
    "gated_attn_decode_workspace_size",
    "gated_attn_decode",
    "gated_attn_decode_ex",
    "gated_attn_decode_fp8kv",
    "gated_attn_decode_csr",
    "gated_attn_decode_noalloc",
    "gated_attn_decode_fp8kv_csr",
    "gated_attn_prefill",
    "gated_attn_prefill_ex",
    "gated_attn_qk_norm_rope",
    "gated_attn_stream_read",
    "gated_attn_status_string",
    "gated_attn_last_hip_error",
)


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class DecodePlan(ctypes.Structure):
    _fields_ = [
        ("tokens_per_split", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class PrefillDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class QkNormRopeDims(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class AttnOptions(ctypes.Structure):
    """ga_attn_options: sinks, lse output, prefill key lengths, window."""
    _fields_ = [
        ("sinks", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("kv_lens", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


def _load_library() -> ctypes.CDLL:
    # torch ships its own HIP runtime (same SONAME, libamdhip64.so.7).  Loading
    # torch first makes the library bind to that runtime instead of pulling a
    # second one into the process: one runtime, one view of devices, streams
    # and memory.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python gated_gqa_decode_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.gated_attn_decode_plan.restype = ctypes.c_int
    lib.gated_attn_decode_plan.argtypes = [ctypes.POINTER(DecodeDims), ctypes.POINTER(DecodePlan)]
    lib.gated_attn_decode_workspace_size.restype = sz
    lib.gated_attn_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeDims)]
    lib.gated_attn_decode.restype = ctypes.c_int
    lib.gated_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                      ctypes.POINTER(DecodeDims), vp, sz]
    lib.gated_attn_decode_noalloc.restype = ctypes.c_int
    lib.gated_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                              ctypes.POINTER(DecodeDims)]
    lib.gated_attn_decode_ex.restype = ctypes.c_int
    lib.gated_attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                         ctypes.POINTER(DecodeDims), vp, sz,
                                         ctypes.POINTER(AttnOptions)]
    lib.gated_attn_decode_fp8kv.restype = ctypes.c_int
    lib.gated_attn_decode_fp8kv.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                            ctypes.c_float, vp, vp, ctypes.POINTER(DecodeDims),
                                            vp, sz, ctypes.POINTER(AttnOptions)]
    lib.gated_attn_decode_csr.restype = ctypes.c_int
    lib.gated_attn_decode_csr.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_float,
                                          vp, vp, ctypes.POINTER(DecodeDims), vp, sz,
                                          ctypes.POINTER(AttnOptions)]
    lib.gated_attn_decode_fp8kv_csr.restype = ctypes.c_int
    lib.gated_attn_decode_fp8kv_csr.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                                ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                vp, vp, ctypes.POINTER(DecodeDims), vp, sz,
                                                ctypes.POINTER(AttnOptions)]
    lib.gated_attn_qk_norm_rope.restype = ctypes.c_int
    lib.gated_attn_qk_norm_rope.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                            vp, vp, ctypes.POINTER(QkNormRopeDims)]
    lib.gated_attn_prefill_ex.restype = ctypes.c_int
    lib.gated_attn_prefill_ex.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_int, vp, vp,
                                          ctypes.POINTER(PrefillDims),
                                          ctypes.POINTER(AttnOptions)]
    lib.gated_attn_prefill.restype = ctypes.c_int
    lib.gated_attn_prefill.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_int, vp, vp,
                                       ctypes.POINTER(PrefillDims)]
    lib.gated_attn_stream_read.restype = ctypes.c_int
    lib.gated_attn_stream_read.argtypes = [vp, sz, vp, vp]
    lib.gated_attn_status_string.restype = ctypes.c_char_p
    lib.gated_attn_status_string.argtypes = [ctypes.c_int]
    lib.gated_attn_last_hip_error.restype = ctypes.c_int
    lib.gated_attn_last_hip_error.argtypes = []
    return lib


lib = _load_library()


class GatedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        name = lib.gated_attn_status_string(status).decode()
        msg = f"{where}: {name}"
        if status == GA_ERR_HIP:
            msg += f" (hipError_t {lib.gated_attn_last_hip_error()})"
        super().__init__(msg)
        self.status = status


class InvalidArgument(GatedAttnError, ValueError):
    pass


class Unsupported(GatedAttnError, NotImplementedError):
    pass


class WorkspaceTooSmall(GatedAttnError, ValueError):
    pass


def check(status: int, where: str) -> None:
    """Raise the typed exception for a non-OK status."""
    if status == GA_OK:
        return
    cls = {GA_ERR_INVALID_ARGUMENT: InvalidArgument, GA_ERR_UNSUPPORTED: Unsupported,
           GA_ERR_WORKSPACE_TOO_SMALL: WorkspaceTooSmall}.get(status, GatedAttnError)
    raise cls(status, where)


@dataclass
class Plan:
    tokens_per_split: int
    num_splits: int
    workspace_bytes: int


def decode_dims(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq,
                num_pages) -> DecodeDims:
    return DecodeDims(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq,
                      num_pages)


def decode_plan(dims: DecodeDims) -> Plan:
    p = DecodePlan()
    check(lib.gated_attn_decode_plan(ctypes.byref(dims), ctypes.byref(p)), "gated_attn_decode_plan")
    return Plan(p.tokens_per_split, p.num_splits, p.workspace_bytes)


def decode_workspace_size(dims: DecodeDims) -> int:
    return int(lib.gated_attn_decode_workspace_size(ctypes.byref(dims)))


# ---------------------------------------------------------------------------
# torch-facing wrappers (marshalling only)
# ---------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _need(t, name, dtype, ndim, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def decode_dims_for(q, k_pool, block_table) -> DecodeDims:
    B, Hq, D = q.shape
    P, ps, Hkv, _ = k_pool.shape
    return decode_dims(B, Hq, Hkv, D, ps, block_table.shape[1], P)


def _options(sinks, window, lse, kv_lens, Hq, dev):
    """AttnOptions for the _ex entry points, or None for plain attention."""
    torch = _torch()
    if sinks is None and lse is None and kv_lens is None and not window:
        return None
    o = AttnOptions()
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1, dev)
        if sinks.shape[0] != Hq:
            raise ValueError("sinks must hold one logit per query head")
        o.sinks = sinks.data_ptr()
    if lse is not None:
        o.lse = lse.data_ptr()
    if kv_lens is not None:
        o.kv_lens = kv_lens.data_ptr()
    o.window = int(window) if window and window > 0 else 0
    return o


def decode(q, gate, k_pool, v_pool, block_table, seq_lens, scale, *, out=None, workspace=None,
           stream=None, sinks=None, window=0, lse=None, return_lse=False, k_descale=None,
           v_descale=None):
    """Gated GQA decode over a paged pool; returns ``out`` [B, H_q, D] bf16.

    q, gate: [B, H_q, D] bf16; k_pool, v_pool: [P, 16, H_kv, D] bf16;
    block_table: [B, W] int32; seq_lens: [B] int32 (<= 0: padded slot).
    ``workspace`` (uint8, >= decode_workspace_size bytes) is allocated when
    not given; pass one to keep the call allocation-free (e.g. under graph
    capture).  Work is enqueued on ``stream`` (default: torch's current stream).
    Options (gated_attn_decode_ex): ``sinks`` fp32 [H_q] sink logits,
    ``window`` > 0 keeps the last ``window`` keys, ``lse`` fp32 [B, H_q] to
    receive the natural-log log-sum-exp (or ``return_lse=True`` to allocate
    it; the call then returns ``(out, lse)``).
    FP8 pools (gated_attn_decode_fp8kv): ``k_pool`` / ``v_pool`` of dtype
    float8_e4m3fn (or uint8 holding e4m3 codes) with per-tensor factors
    ``k_descale`` / ``v_descale`` (K = k_descale * code value).
    """
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(gate, "gate", torch.bfloat16, 3, dev)
    fp8 = k_pool.dtype in (torch.uint8, torch.float8_e4m3fn)
    pool_dtype = k_pool.dtype if fp8 else torch.bfloat16
    _need(k_pool, "k_pool", pool_dtype, 4, dev)
    _need(v_pool, "v_pool", pool_dtype, 4, dev)
    if fp8 and (k_descale is None or v_descale is None):
        raise ValueError("FP8 pools need k_descale and v_descale")
    if not fp8 and (k_descale is not None or v_descale is not None):
        raise ValueError("k_descale / v_descale apply to FP8 pools only")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    if gate.shape != q.shape or v_pool.shape != k_pool.shape:
        raise ValueError("gate must match q and v_pool must match k_pool")
    B, Hq, D = q.shape
    if k_pool.shape[3] != D or block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("inconsistent shapes")
    dims = decode_dims_for(q, k_pool, block_table)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3, dev)
        if out.shape != q.shape:
            raise ValueError("out must match q")
    need = decode_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if lse.shape != (B, Hq):
            raise ValueError("lse must be [B, H_q]")
    opts = _options(sinks, window, lse, None, Hq, dev)
    args = (q.data_ptr(), gate.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
            block_table.data_ptr(), seq_lens.data_ptr(), float(scale), out.data_ptr(),
            _stream_handle(stream, dev), ctypes.byref(dims), workspace.data_ptr(),
            workspace.numel())
    if fp8:
        args = args[:7] + (float(k_descale), float(v_descale)) + args[7:]
        check(lib.gated_attn_decode_fp8kv(*args, None if opts is None else ctypes.byref(opts)),
              "gated_attn_decode_fp8kv")
    elif opts is None:
        check(lib.gated_attn_decode(*args), "gated_attn_decode")
    else:
        check(lib.gated_attn_decode_ex(*args, ctypes.byref(opts)), "gated_attn_decode_ex")
    return (out, lse) if return_lse else out


def prefill(q, gate, k, v, scale, causal=True, *, out=None, stream=None, kv_lens=None,
            sinks=None, window=0, lse=None, return_lse=False):
    """Gated dense prefill; q, gate: [B, S, H_q, D]; k, v: [B, S, H_kv, D] bf16.

    Options (gated_attn_prefill_ex): ``kv_lens`` int32 [B] key lengths,
    ``sinks`` fp32 [H_q], ``window`` > 0 (row i sees keys j > i - window),
    ``lse`` fp32 [B, S, H_q] (or ``return_lse=True``; returns ``(out, lse)``).
    """
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, 4, dev)
    _need(gate, "gate", torch.bfloat16, 4, dev)
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if gate.shape != q.shape or k.shape != (B, S, Hkv, D) or v.shape != k.shape:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
        if out.shape != q.shape:
            raise ValueError("out must match q")
    dims = PrefillDims(B, S, Hq, Hkv, D)
    if kv_lens is not None:
        _need(kv_lens, "kv_lens", torch.int32, 1, dev)
        if kv_lens.shape[0] != B:
            raise ValueError("kv_lens must be [B]")
    if return_lse and lse is None:
        lse = torch.empty((B, S, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, dev)
        if lse.shape != (B, S, Hq):
            raise ValueError("lse must be [B, S, H_q]")
    opts = _options(sinks, window, lse, kv_lens, Hq, dev)
    args = (q.data_ptr(), gate.data_ptr(), k.data_ptr(), v.data_ptr(), float(scale),
            int(bool(causal)), out.data_ptr(), _stream_handle(stream, dev), ctypes.byref(dims))
    if opts is None:
        check(lib.gated_attn_prefill(*args), "gated_attn_prefill")
    else:
        check(lib.gated_attn_prefill_ex(*args, ctypes.byref(opts)), "gated_attn_prefill_ex")
    return (out, lse) if return_lse else out


def qk_norm_rope(q, k, v, *, w_q=None, w_k=None, eps=1e-6, cos=None, sin=None,
                 slot_mapping=None, k_pool=None, v_pool=None, q_out=None, stream=None):
    """QK-RMSNorm + partial rotate-half RoPE on q [T, H_q, D] and k [T, H_kv, D]
    (bf16), one kernel launch (gated_attn_qk_norm_rope).

    ``w_q`` / ``w_k``: bf16 [D] norm weights (both or neither); ``cos`` /
    ``sin``: bf16 [T, R] tables (R = 0 without them).  With ``slot_mapping``
    (int64 [T], < 0 skips) K and V are written into ``k_pool`` / ``v_pool``
    ([P, 16, H_kv, D], in place) and ``(q_out, k_pool, v_pool)`` is returned;
    otherwise ``(q_out, k_out, v_out)`` with dense K / V outputs.
    """
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (T, Hkv, D) or v.shape != k.shape:
        raise ValueError("inconsistent shapes")
    if (w_q is None) != (w_k is None):
        raise ValueError("give both norm weights or neither")
    for name, w in (("w_q", w_q), ("w_k", w_k)):
        if w is not None:
            _need(w, name, torch.bfloat16, 1, dev)
    R = 0
    if cos is not None or sin is not None:
        _need(cos, "cos", torch.bfloat16, 2, dev)
        _need(sin, "sin", torch.bfloat16, 2, dev)
        if cos.shape[0] != T or sin.shape != cos.shape:
            raise ValueError("cos / sin must be [T, rope_dim]")
        R = cos.shape[1]
    if q_out is None:
        q_out = torch.empty_like(q)
    P = 0
    if slot_mapping is not None:
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
        _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
        P = k_pool.shape[0]
        k_out, v_out = k_pool, v_pool
    else:
        k_out, v_out = torch.empty_like(k), torch.empty_like(v)
    dims = QkNormRopeDims(T, Hq, Hkv, D, R, 16, 0, P)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.gated_attn_qk_norm_rope(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr(w_q), ptr(w_k), float(eps), ptr(cos),
        ptr(sin), ptr(slot_mapping), q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(),
        _stream_handle(stream, dev), ctypes.byref(dims))
    check(st, "gated_attn_qk_norm_rope")
    return q_out, k_out, v_out


def decode_csr(q, gate, k_pool, v_pool, kv_indptr, kv_indices, scale, *, max_seq_len,
               out=None, workspace=None, stream=None, sinks=None, window=0, lse=None,
               return_lse=False, k_descale=None, v_descale=None):
    """Gated GQA decode with CSR token indexing (page size 1,
    gated_attn_decode_csr): k_pool, v_pool [N, 1, H_kv, D] bf16 (or [N, H_kv, D]);
    kv_indptr int32 [B + 1]; kv_indices int32 [capacity]; ``max_seq_len`` is
    the per-sequence capacity in tokens that fixes the plan.  Pools of e4m3
    codes (float8_e4m3fn or uint8) with ``k_descale`` / ``v_descale`` go to
    gated_attn_decode_fp8kv_csr.  Options as :func:`decode`."""
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(gate, "gate", torch.bfloat16, 3, dev)
    if k_pool.dim() == 3:
        k_pool, v_pool = k_pool.unsqueeze(1), v_pool.unsqueeze(1)
    fp8 = k_pool.dtype in (torch.uint8, torch.float8_e4m3fn)
    pool_dtype = k_pool.dtype if fp8 else torch.bfloat16
    if fp8 != (k_descale is not None and v_descale is not None):
        raise ValueError("e4m3 pools take k_descale and v_descale; bf16 pools take neither")
    _need(k_pool, "k_pool", pool_dtype, 4, dev)
    _need(v_pool, "v_pool", pool_dtype, 4, dev)
    _need(kv_indptr, "kv_indptr", torch.int32, 1, dev)
    _need(kv_indices, "kv_indices", torch.int32, 1, dev)
    B, Hq, D = q.shape
    N, one, Hkv, _ = k_pool.shape
    if one != 1 or kv_indptr.shape[0] != B + 1 or gate.shape != q.shape:
        raise ValueError("inconsistent shapes")
    dims = decode_dims(B, Hq, Hkv, D, 1, int(max_seq_len), N)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    opts = _options(sinks, window, lse, None, Hq, dev)
    head = [q.data_ptr(), gate.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
            kv_indptr.data_ptr(), kv_indices.data_ptr(), kv_indices.numel(), float(scale)]
    tail = [out.data_ptr(), _stream_handle(stream, dev), ctypes.byref(dims), workspace.data_ptr(),
            workspace.numel(), None if opts is None else ctypes.byref(opts)]
    if fp8:
        st = lib.gated_attn_decode_fp8kv_csr(*head, float(k_descale), float(v_descale), *tail)
        check(st, "gated_attn_decode_fp8kv_csr")
    else:
        st = lib.gated_attn_decode_csr(*head, *tail)
        check(st, "gated_attn_decode_csr")
    return (out, lse) if return_lse else out


"""CPU oracle for gated grouped-query attention (fp64) -- test infrastructure.

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain
C, built by ``oracle/build.py``) with ctypes and numpy; it does not import the
GPU package and the GPU package does not import it.

All bf16 tensors cross this interface as ``numpy.uint16`` arrays of bit
patterns.  See ``gqa_oracle.c`` for the definition that is computed and the
passages of the pages it follows.

Parity status of each function (what pins it is in tests/test_oracle_*.py):
  bf16_rne, bf16_value, sigmoid_bf16, gate_output : pinned (exact-rational
      rounding, 40-digit decimal sigmoid over all 65,536 gates, closed forms)
  decode, prefill : pinned (closed forms, invariants, 50-digit brute force)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import compare  # noqa: F401  (tolerance helpers, re-exported)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from .build import build

        build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_bf16_rne_array.argtypes = [_f64p, _u16p, ctypes.c_int64]
    lib.oracle_sigmoid_bf16.restype = ctypes.c_uint16
    lib.oracle_sigmoid_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_sigmoid_table.restype = None
    lib.oracle_sigmoid_table.argtypes = [_u16p]
    lib.oracle_gate_output.restype = ctypes.c_uint16
    lib.oracle_gate_output.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [
        _u16p, _u16p, _u16p, _u16p, _i32p, _i32p, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, _u16p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.oracle_decode_ex.restype = ctypes.c_int
    lib.oracle_decode_ex.argtypes = [
        _u16p, _u16p, _u16p, _u16p, _i32p, _i32p, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, _f64p, ctypes.c_int, _u16p, _f64p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_fp8.restype = ctypes.c_int
    lib.oracle_decode_fp8.argtypes = [
        _u16p, _u16p, ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint8), _i32p, _i32p,
        ctypes.c_double, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, _f64p, ctypes.c_int, _u16p, _f64p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.oracle_prefill_ex.restype = ctypes.c_int
    lib.oracle_prefill_ex.argtypes = [
        _u16p, _u16p, _u16p, _u16p, ctypes.c_double, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _i32p, _f64p, ctypes.c_int,
        _i32p, ctypes.c_int, _u16p, _f64p, _f64p, _f64p, ctypes.c_int,
    ]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [
        _u16p, _u16p, _u16p, _u16p, ctypes.c_double, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _i32p, ctypes.c_int, _u16p, _f64p, _f64p, ctypes.c_int,
    ]
    _lib = lib
    return lib


def affinity_cores() -> int:
    """Cores in this process's affinity mask."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_share() -> int:
    """The CPU share granted to this process: OMP_NUM_THREADS when the
    environment sets it (a machine shared between GPUs grants each GPU's
    process a fixed number of cores), else the whole affinity mask."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    return n if n > 0 else affinity_cores()


def default_threads() -> int:
    """Host threads the oracle uses: every core of the affinity mask, within
    the process's CPU share."""
    return max(1, min(affinity_cores(), cpu_share()))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or '' if unknown."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


# --------------------------------------------------------------------------
# Scalar / table routines
# --------------------------------------------------------------------------
def bf16_value(bits) -> np.ndarray:
    """fp64 values of bf16 bit patterns (exact)."""
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_value(int(b)) for b in bits.ravel()],
                    dtype=np.float64).reshape(bits.shape)


def bf16_rne(x) -> np.ndarray:
    """Round fp64 values to bf16 (ties to even), as uint16 bit patterns."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_bf16_rne_array(_ptr(x, ctypes.c_double), _ptr(out, ctypes.c_uint16), x.size)
    return out


def sigmoid_bf16(gate_bits: int) -> int:
    return int(_load().oracle_sigmoid_bf16(int(gate_bits)))


def sigmoid_table() -> np.ndarray:
    """The 65,536-entry map gate bits -> bf16 bits of sigmoid(gate)."""
    t = np.empty(65536, dtype=np.uint16)
    _load().oracle_sigmoid_table(_ptr(t, ctypes.c_uint16))
    return t


def gate_output(ob_bits: int, sigma_bits: int) -> int:
    return int(_load().oracle_gate_output(int(ob_bits), int(sigma_bits)))


def e4m3_value(code: int) -> float:
    """fp64 value of an OCP float8 e4m3 code (NaN for 0x7F / 0xFF)."""
    return float(_load().oracle_e4m3_value(int(code) & 0xFF))


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
class OracleError(RuntimeError):
    pass


def _sinks(sinks, Hq):
    if sinks is None:
        return None, None
    sk = np.ascontiguousarray(sinks, dtype=np.float64).reshape(-1)
    assert sk.shape == (Hq,), "one sink logit per query head"
    return sk, _ptr(sk, ctypes.c_double)


def decode(q, gate, k_pool, v_pool, block_table, seq_lens, scale, nthreads=None, *,
           sinks=None, window=0, return_lse=False, k_descale=1.0, v_descale=1.0):
    """Gated GQA decode over a paged pool.

    q, gate: [B, H_q, D] bf16 bits; k_pool, v_pool: [P, page, H_kv, D];
    block_table: [B, W] int32; seq_lens: [B] int32.
    sinks: optional [H_q] sink logits; window > 0 keeps the last `window` keys.
    Returns (out bits [B,H_q,D], O fp64 [B,H_q,D], Mref fp64 [B,H_q,D]) and,
    with return_lse, also lse fp64 [B, H_q] (natural log of the softmax
    denominator, -inf for a row with no visible key and no sink).
    uint8 pools hold e4m3 codes: K = k_descale * e4m3(code), V likewise.
    """
    lib = _load()
    fp8 = np.asarray(k_pool).dtype == np.uint8
    q, gate = _u16(q), _u16(gate)
    if fp8:
        k_pool = np.ascontiguousarray(k_pool, dtype=np.uint8)
        v_pool = np.ascontiguousarray(v_pool, dtype=np.uint8)
    else:
        k_pool, v_pool = _u16(k_pool), _u16(v_pool)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, D = q.shape
    P, page, Hkv, D2 = k_pool.shape
    assert D2 == D and v_pool.shape == k_pool.shape and gate.shape == q.shape
    W = block_table.shape[1] if block_table.ndim == 2 else 0
    out = np.zeros((B, Hq, D), dtype=np.uint16)
    o = np.zeros((B, Hq, D), dtype=np.float64)
    mref = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    sk, sk_p = _sinks(sinks, Hq)
    tail = (B, Hq, Hkv, D, page, W, P, sk_p, int(window),
            _ptr(out, ctypes.c_uint16), _ptr(o, ctypes.c_double), _ptr(mref, ctypes.c_double),
            _ptr(lse, ctypes.c_double), nthreads or default_threads())
    if fp8:
        st = lib.oracle_decode_fp8(
            _ptr(q, ctypes.c_uint16), _ptr(gate, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint8), _ptr(v_pool, ctypes.c_uint8),
            _ptr(block_table, ctypes.c_int32), _ptr(seq_lens, ctypes.c_int32),
            float(scale), float(k_descale), float(v_descale), *tail)
    else:
        st = lib.oracle_decode_ex(
            _ptr(q, ctypes.c_uint16), _ptr(gate, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(block_table, ctypes.c_int32), _ptr(seq_lens, ctypes.c_int32),
            float(scale), *tail)
    if st != 0:
        raise OracleError(f"oracle_decode failed with status {st}")
    if return_lse:
        return out, o, mref, lse
    return out, o, mref


def prefill(q, gate, k, v, scale, causal=True, rows=None, nthreads=None, *, seq_lens=None,
            sinks=None, window=0, return_lse=False):
    """Gated dense prefill.  q, gate: [B,S,H_q,D]; k, v: [B,S,H_kv,D].

    rows: optional int array [n, 2] of (b, i) query positions; results are
    then [n, H_q, D].  Without rows, results are [B, S, H_q, D].
    seq_lens: optional [B] key lengths (keys j >= seq_lens[b] are masked);
    sinks: optional [H_q] sink logits; window > 0: row i sees keys j > i - window.
    With return_lse also returns lse fp64 ([n, H_q] or [B, S, H_q]).
    """
    lib = _load()
    q, gate, k, v = (_u16(a) for a in (q, gate, k, v))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape and gate.shape == q.shape
    if rows is None:
        n = B * S
        rows_p = None
        shape = (B, S, Hq, D)
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        n = rows.shape[0]
        rows_p = _ptr(rows, ctypes.c_int32)
        shape = (n, Hq, D)
    out = np.zeros(shape, dtype=np.uint16)
    o = np.zeros(shape, dtype=np.float64)
    mref = np.zeros(shape, dtype=np.float64)
    lse = np.zeros(shape[:-1], dtype=np.float64)
    sl_p = None
    if seq_lens is not None:
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32).reshape(-1)
        assert seq_lens.shape == (B,)
        sl_p = _ptr(seq_lens, ctypes.c_int32)
    sk, sk_p = _sinks(sinks, Hq)
    st = lib.oracle_prefill_ex(
        _ptr(q, ctypes.c_uint16), _ptr(gate, ctypes.c_uint16),
        _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        float(scale), int(bool(causal)), B, S, Hq, Hkv, D, sl_p, sk_p, int(window), rows_p, n,
        _ptr(out, ctypes.c_uint16), _ptr(o, ctypes.c_double), _ptr(mref, ctypes.c_double),
        _ptr(lse, ctypes.c_double), nthreads or default_threads())
    if st != 0:
        raise OracleError(f"oracle_prefill failed with status {st}")
    if return_lse:
        return out, o, mref, lse
    return out, o, mref


# --------------------------------------------------------------------------
# QK-RMSNorm + partial RoPE + K/V slot write
# --------------------------------------------------------------------------
def qk_norm_rope(q, k, v, w_q, w_k, eps, cos, sin, slot_mapping=None, k_pool=None,
                 v_pool=None):
    """q [T,H_q,D], k, v [T,H_kv,D] bf16 bits; w_q, w_k [D] or None; cos, sin [T,R].

    Without slot_mapping returns (q_out, k_out, v_out, qz, qmag, kz, kmag) with
    dense k_out / v_out [T,H_kv,D]; with slot_mapping [T] (int64, < 0 skips),
    k_pool / v_pool ([P, page, H_kv, D]) are copied, written and returned in
    place of the dense outputs.  qz / kz: fp64 values before the rounding;
    qmag / kmag: the magnitudes they were formed from.
    """
    lib = _load()
    if not hasattr(lib, "_qknr"):
        lib.oracle_qk_norm_rope.restype = ctypes.c_int
        lib.oracle_qk_norm_rope.argtypes = [
            _u16p, _u16p, _u16p, _u16p, _u16p, ctypes.c_double, _u16p, _u16p,
            ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int64, _u16p, _u16p, _u16p,
            _f64p, _f64p, _f64p, _f64p]
        lib._qknr = True
    q, k, v = (_u16(a) for a in (q, k, v))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    cos, sin = _u16(cos), _u16(sin)
    R = cos.shape[1] if cos.ndim == 2 else 0
    wq = None if w_q is None else _u16(w_q)
    wk = None if w_k is None else _u16(w_k)
    q_out = np.zeros_like(q)
    qz = np.zeros(q.shape, np.float64)
    qmag = np.zeros(q.shape, np.float64)
    kz = np.zeros(k.shape, np.float64)
    kmag = np.zeros(k.shape, np.float64)
    if slot_mapping is None:
        k_out = np.zeros_like(k)
        v_out = np.zeros_like(v)
        sm, nslots = None, 0
    else:
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        k_out = _u16(k_pool).copy()
        v_out = _u16(v_pool).copy()
        nslots = k_out.shape[0] * k_out.shape[1]
    st = lib.oracle_qk_norm_rope(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        None if wq is None else _ptr(wq, ctypes.c_uint16),
        None if wk is None else _ptr(wk, ctypes.c_uint16), float(eps),
        _ptr(cos, ctypes.c_uint16) if R else None, _ptr(sin, ctypes.c_uint16) if R else None,
        None if sm is None else _ptr(sm, ctypes.c_int64), T, Hq, Hkv, D, R, nslots,
        _ptr(q_out, ctypes.c_uint16), _ptr(k_out, ctypes.c_uint16), _ptr(v_out, ctypes.c_uint16),
        _ptr(qz, ctypes.c_double), _ptr(qmag, ctypes.c_double), _ptr(kz, ctypes.c_double),
        _ptr(kmag, ctypes.c_double))
    if st != 0:
        raise OracleError(f"oracle_qk_norm_rope failed with status {st}")
    return q_out, k_out, v_out, qz, qmag, kz, kmag

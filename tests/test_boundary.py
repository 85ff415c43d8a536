"""The C ABI on the host: symbols, split plans, and every argument check that
returns before anything touches a GPU.  No call here reaches a launch: each
one carries at least one invalid argument (fake device addresses are never
dereferenced), or has batch 0.
"""
import ctypes
import os
import re

import pytest

import gated_gqa_decode_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gated_attn.h")

FAKE = 0x7f0000000000  # 16-byte aligned, never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gated_attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    declared = header_functions()
    assert declared == sorted(ga.EXPORTED_SYMBOLS)
    raw = ctypes.CDLL(ga.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_status_strings():
    for st, name in [(0, "GA_OK"), (1, "GA_ERR_INVALID_ARGUMENT"), (2, "GA_ERR_UNSUPPORTED"),
                     (3, "GA_ERR_WORKSPACE_TOO_SMALL"), (4, "GA_ERR_HIP")]:
        assert ga.lib.gated_attn_status_string(st).decode() == name
    assert ga.lib.gated_attn_last_hip_error() == 0


def _dims(**kw):
    base = dict(batch=64, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=16,
                max_pages_per_seq=256, num_pages=16384)
    base.update(kw)
    return ga.decode_dims(**base)


@pytest.mark.parametrize("B,W", [(1, 32), (4, 32), (64, 256), (224, 384), (2, 2048), (65535, 1),
                                 (1, 1), (3, 100000), (70000, 3), (1 << 20, 2)])
def test_plan_covers_capacity(B, W):
    p = ga.decode_plan(_dims(batch=B, max_pages_per_seq=W))
    cap = W * 16
    t_max = 16384 if B * 2 < 256 else 4096
    assert p.tokens_per_split % 64 == 0 and 64 <= p.tokens_per_split <= t_max
    assert p.num_splits * p.tokens_per_split >= cap
    assert (p.num_splits - 1) * p.tokens_per_split < cap
    rows = B * 16 * p.num_splits
    assert p.workspace_bytes >= rows * 258 * 4 and p.workspace_bytes % 256 == 0
    assert ga.decode_workspace_size(_dims(batch=B, max_pages_per_seq=W)) == p.workspace_bytes


@pytest.mark.parametrize("G", list(range(1, 17)))
def test_supported_groups_plan(G):
    """Every group size uses one workgroup per (sequence, kv head, split): the
    split plan does not depend on the group."""
    d = _dims(batch=64, num_q_heads=2 * G, num_kv_heads=2, max_pages_per_seq=256)
    p = ga.decode_plan(d)
    units = 64 * 2
    t = -(-(4096 * units) // 256)
    t = min(max(-(-t // 64) * 64, 64), 16384)
    assert p.tokens_per_split == t
    assert p.workspace_bytes >= 64 * 2 * G * p.num_splits * 258 * 4


@pytest.mark.parametrize("B,Hkv,W,page,t_want,ns_want", [
    (64, 2, 2048, 16, 16384, 2),   # 128 pairs, capacity 32,768: two long splits
    (128, 2, 2048, 16, 4096, 8),   # 256 pairs: splits of at most 4,096 tokens
    (224, 2, 384, 16, 4096, 2),    # the serving shape
    (64, 2, 32768, 1, 2048, 16),   # page size 1: the token slots of a split fit LDS
    (1, 2, 2048, 16, 256, 128),    # one sequence: about 256 workgroups
])
def test_split_cap(B, Hkv, W, page, t_want, ns_want):
    """The largest split: 16,384 tokens with 16-token pages while the
    (sequence, kv head) pairs are fewer than the 256 target workgroups, else
    4,096; always 2,048 at page size 1."""
    p = ga.decode_plan(_dims(batch=B, num_q_heads=8 * Hkv, num_kv_heads=Hkv, page_size=page,
                             max_pages_per_seq=W, num_pages=max(16384, W)))
    assert (p.tokens_per_split, p.num_splits) == (t_want, ns_want)


def test_oversize_stage1_grid_is_declined():
    """B * H_kv * splits beyond one launch's grid: declined before any launch."""
    d = _dims(batch=65535, num_q_heads=64, num_kv_heads=8, max_pages_per_seq=4096)
    p = ga.DecodePlan()
    assert ga.lib.gated_attn_decode_plan(ctypes.byref(d), ctypes.byref(p)) == ga.GA_ERR_UNSUPPORTED
    assert ga.decode_workspace_size(d) == 0


def test_plan_depends_on_capacity_not_lengths():
    a = ga.decode_plan(_dims(batch=64, max_pages_per_seq=256))
    b = ga.decode_plan(_dims(batch=64, max_pages_per_seq=256, num_pages=1 << 30))
    assert a == b


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=128), ga.GA_ERR_UNSUPPORTED),
    (dict(num_q_heads=34), ga.GA_ERR_UNSUPPORTED),         # group of 17
    (dict(num_q_heads=64, num_kv_heads=2), ga.GA_ERR_UNSUPPORTED),  # group of 32
    (dict(num_q_heads=15), ga.GA_ERR_INVALID_ARGUMENT),    # not a multiple of H_kv
    (dict(page_size=32), ga.GA_ERR_UNSUPPORTED),
    (dict(page_size=0), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(batch=70000, max_pages_per_seq=16384), ga.GA_ERR_UNSUPPORTED),  # 8.96e6 workgroups
    (dict(num_pages=0), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(max_pages_per_seq=0), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(num_kv_heads=0), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=0), ga.GA_ERR_INVALID_ARGUMENT),
])
def test_bad_dims_are_declined(kw, status):
    d = _dims(**kw)
    p = ga.DecodePlan()
    assert ga.lib.gated_attn_decode_plan(ctypes.byref(d), ctypes.byref(p)) == status
    assert ga.decode_workspace_size(d) == 0
    st = ga.lib.gated_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, FAKE, None,
                                  ctypes.byref(d), FAKE, 1 << 40)
    assert st == status


def _call(q=FAKE, gate=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, scale=0.0625, out=FAKE,
          ws=FAKE, wsb=1 << 40, dims=None):
    d = dims or _dims()
    return ga.lib.gated_attn_decode(q, gate, k, v, bt, sl, scale, out, None, ctypes.byref(d),
                                    ws, wsb)


@pytest.mark.parametrize("field", ["q", "gate", "k", "v", "bt", "sl", "out", "ws"])
def test_null_pointers_are_rejected(field):
    assert _call(**{field: None}) == ga.GA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field,off", [("q", 8), ("gate", 2), ("k", 4), ("v", 8), ("out", 2),
                                       ("ws", 4), ("bt", 2), ("sl", 1)])
def test_misaligned_pointers_are_rejected(field, off):
    assert _call(**{field: FAKE + off}) == ga.GA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan")])
def test_bad_scale_is_rejected(scale):
    assert _call(scale=scale) == ga.GA_ERR_INVALID_ARGUMENT


def test_small_workspace_is_rejected():
    need = ga.decode_workspace_size(_dims())
    assert _call(wsb=need - 1) == ga.GA_ERR_WORKSPACE_TOO_SMALL


def _call_ex(opts, dims=None, batch=None):
    d = dims or _dims(**({} if batch is None else dict(batch=batch)))
    return ga.lib.gated_attn_decode_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, FAKE, None,
                                       ctypes.byref(d), FAKE, 1 << 40, opts)


@pytest.mark.parametrize("kw", [dict(flags=1), dict(sinks=FAKE + 2), dict(lse=FAKE + 1),
                                dict(kv_lens=FAKE)])
def test_decode_ex_bad_options_are_rejected(kw):
    """Reserved flags, misaligned option pointers, and prefill-only key lengths."""
    o = ga.AttnOptions(**kw)
    assert _call_ex(ctypes.byref(o)) == ga.GA_ERR_INVALID_ARGUMENT
    assert _call_ex(ctypes.byref(o), batch=0) == ga.GA_ERR_INVALID_ARGUMENT


def test_decode_ex_null_or_zero_options_behave_like_plain_decode():
    """No device here: the plain and _ex calls fail the same way, after the
    same argument checks, and a batch of 0 succeeds for both."""
    plain = _call()
    assert _call_ex(None) == plain
    assert _call_ex(ctypes.byref(ga.AttnOptions())) == plain
    assert _call_ex(ctypes.byref(ga.AttnOptions(window=-5))) == plain
    assert _call_ex(ctypes.byref(ga.AttnOptions(window=7, sinks=FAKE, lse=FAKE)), batch=0) == \
        ga.GA_OK


@pytest.mark.parametrize("kw,status", [(dict(flags=2), ga.GA_ERR_INVALID_ARGUMENT),
                                       (dict(kv_lens=FAKE + 2), ga.GA_ERR_INVALID_ARGUMENT),
                                       (dict(kv_lens=FAKE, window=3), ga.GA_OK)])
def test_prefill_ex_options(kw, status):
    d = ga.PrefillDims(0, 128, 16, 2, 256)  # batch 0: validated, then nothing to do
    o = ga.AttnOptions(**kw)
    assert ga.lib.gated_attn_prefill_ex(FAKE, FAKE, FAKE, FAKE, 0.0625, 1, FAKE, None,
                                        ctypes.byref(d), ctypes.byref(o)) == status


@pytest.mark.parametrize("kd,vd", [(0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0),
                                   (1.0, float("nan"))])
def test_fp8kv_bad_factors_are_rejected(kd, vd):
    d = _dims()
    assert ga.lib.gated_attn_decode_fp8kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, kd, vd, FAKE,
                                          None, ctypes.byref(d), FAKE, 1 << 40,
                                          None) == ga.GA_ERR_INVALID_ARGUMENT


def test_fp8kv_shares_the_decode_checks():
    d = _dims(head_dim=128)
    assert ga.lib.gated_attn_decode_fp8kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, 0.01, 0.01,
                                          FAKE, None, ctypes.byref(d), FAKE, 1 << 40,
                                          None) == ga.GA_ERR_UNSUPPORTED
    d = _dims(batch=0)
    assert ga.lib.gated_attn_decode_fp8kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, 0.01, 0.01,
                                          FAKE, None, ctypes.byref(d), FAKE, 1 << 40,
                                          None) == ga.GA_OK


def _rope_call(dims, eps=1e-6, wq=FAKE, wk=FAKE, cos=FAKE, sin=FAKE, slots=None, v_out=FAKE,
               q=FAKE):
    return ga.lib.gated_attn_qk_norm_rope(q, FAKE, FAKE, wq, wk, eps, cos, sin, slots, FAKE,
                                          FAKE, v_out, None, ctypes.byref(dims))


@pytest.mark.parametrize("kw,call_kw,status", [
    (dict(head_dim=128), {}, ga.GA_ERR_UNSUPPORTED),
    (dict(rope_dim=12), {}, ga.GA_ERR_UNSUPPORTED),        # not a multiple of 8
    (dict(rope_dim=7), {}, ga.GA_ERR_INVALID_ARGUMENT),    # odd
    (dict(rope_dim=264), {}, ga.GA_ERR_INVALID_ARGUMENT),  # > D
    (dict(num_tokens=-1), {}, ga.GA_ERR_INVALID_ARGUMENT),
    ({}, dict(eps=-1.0), ga.GA_ERR_INVALID_ARGUMENT),
    ({}, dict(eps=float("nan")), ga.GA_ERR_INVALID_ARGUMENT),
    ({}, dict(wk=None), ga.GA_ERR_INVALID_ARGUMENT),        # one weight only
    ({}, dict(cos=None), ga.GA_ERR_INVALID_ARGUMENT),       # R > 0 without tables
    ({}, dict(q=FAKE + 4), ga.GA_ERR_INVALID_ARGUMENT),     # misaligned
    ({}, dict(q=FAKE + 8), ga.GA_ERR_INVALID_ARGUMENT),     # rows are read in 16-byte pieces
    ({}, dict(cos=FAKE + 8), ga.GA_ERR_INVALID_ARGUMENT),
    ({}, dict(slots=FAKE, v_out=None), ga.GA_ERR_INVALID_ARGUMENT),  # pools need v_out
    (dict(page_size=8), dict(slots=FAKE), ga.GA_ERR_UNSUPPORTED),
    (dict(num_pages=0), dict(slots=FAKE), ga.GA_ERR_INVALID_ARGUMENT),
    (dict(num_tokens=0), {}, ga.GA_OK),
])
def test_qk_norm_rope_argument_checks(kw, call_kw, status):
    base = dict(num_tokens=4, num_q_heads=16, num_kv_heads=2, head_dim=256, rope_dim=64,
                page_size=16, reserved=0, num_pages=10)
    base.update(kw)
    assert _rope_call(ga.QkNormRopeDims(**base), **call_kw) == status


def test_null_dims_rejected():
    assert ga.lib.gated_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0625, FAKE, None,
                                    None, FAKE, 1 << 40) == ga.GA_ERR_INVALID_ARGUMENT
    assert ga.lib.gated_attn_prefill(FAKE, FAKE, FAKE, FAKE, 0.0625, 1, FAKE, None,
                                     None) == ga.GA_ERR_INVALID_ARGUMENT


def test_empty_batch_is_a_no_op():
    # batch 0 returns before any pointer is examined or any HIP call is made
    assert _call(dims=_dims(batch=0), q=None, ws=None, wsb=0) == ga.GA_OK
    d = ga.PrefillDims(0, 128, 16, 2, 256)
    assert ga.lib.gated_attn_prefill(None, None, None, None, 0.0625, 1, None, None,
                                     ctypes.byref(d)) == ga.GA_OK
    d = ga.PrefillDims(2, 0, 16, 2, 256)
    assert ga.lib.gated_attn_prefill(None, None, None, None, 0.0625, 1, None, None,
                                     ctypes.byref(d)) == ga.GA_OK


@pytest.mark.parametrize("dims,status", [
    ((2, 128, 16, 2, 128), ga.GA_ERR_UNSUPPORTED),
    ((2, 128, 34, 2, 256), ga.GA_ERR_UNSUPPORTED),  # group of 17
    ((2, 128, 66, 2, 256), ga.GA_ERR_UNSUPPORTED),
    ((2, 128, 15, 2, 256), ga.GA_ERR_INVALID_ARGUMENT),
    ((-1, 128, 16, 2, 256), ga.GA_ERR_INVALID_ARGUMENT),
    ((2, -5, 16, 2, 256), ga.GA_ERR_INVALID_ARGUMENT),
    # one sequence's K rows (S * H_kv * D * 2 bytes) past one buffer descriptor's 2^31 - 1
    ((1, 1 << 21, 16, 2, 256), ga.GA_ERR_UNSUPPORTED),
    ((1, 1 << 18, 128, 16, 256), ga.GA_ERR_UNSUPPORTED),
    # more than 2^22 workgroups: B * H_kv * parts * ceil(S / 16)
    ((4097, 16384, 16, 2, 256), ga.GA_ERR_UNSUPPORTED),
    ((2049, 16384, 32, 2, 256), ga.GA_ERR_UNSUPPORTED),  # group 16: two parts
])
def test_prefill_bad_dims(dims, status):
    d = ga.PrefillDims(*dims)
    assert ga.lib.gated_attn_prefill(FAKE, FAKE, FAKE, FAKE, 0.0625, 1, FAKE, None,
                                     ctypes.byref(d)) == status


@pytest.mark.parametrize("field", range(5))
def test_prefill_null_or_misaligned(field):
    d = ga.PrefillDims(2, 128, 16, 2, 256)
    for bad in (None, FAKE + 2):
        args = [FAKE] * 5
        args[field] = bad
        q, g, k, v, o = args
        assert ga.lib.gated_attn_prefill(q, g, k, v, 0.0625, 1, o, None,
                                         ctypes.byref(d)) == ga.GA_ERR_INVALID_ARGUMENT


def test_prefill_bad_scale():
    d = ga.PrefillDims(2, 128, 16, 2, 256)
    assert ga.lib.gated_attn_prefill(FAKE, FAKE, FAKE, FAKE, float("nan"), 1, FAKE, None,
                                     ctypes.byref(d)) == ga.GA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("src,nbytes,sink", [
    (None, 1 << 20, FAKE), (FAKE + 8, 1 << 20, FAKE), (FAKE, (1 << 20) + 4, FAKE),
    (FAKE, 1 << 20, None), (FAKE, 1 << 20, FAKE + 2)])
def test_stream_read_argument_checks(src, nbytes, sink):
    """The measurement hook rejects NULL / misaligned pointers and sizes that
    are not whole 16-byte loads before any HIP call."""
    assert ga.lib.gated_attn_stream_read(src, nbytes, sink, None) == ga.GA_ERR_INVALID_ARGUMENT


def test_fp8kv_csr_checks():
    """The e4m3 CSR entry point: null row pointers or indices, and page
    sizes other than 1, are declined before anything is enqueued."""
    f = ga.lib.gated_attn_decode_fp8kv_csr
    d1 = _dims(page_size=1)
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1024, 0.0625, 0.01, 0.01, FAKE, None,
             ctypes.byref(d1), FAKE, 1 << 40, None) == ga.GA_ERR_INVALID_ARGUMENT
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1024, 0.0625, 0.01, 0.01, FAKE, None,
             ctypes.byref(d1), FAKE, 1 << 40, None) == ga.GA_ERR_INVALID_ARGUMENT
    d16 = _dims()
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 0.0625, 0.01, 0.01, FAKE, None,
             ctypes.byref(d16), FAKE, 1 << 40, None) == ga.GA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 0.0625, 0.0, 0.01, FAKE, None,
             ctypes.byref(d1), FAKE, 1 << 40, None) == ga.GA_ERR_INVALID_ARGUMENT


def test_noalloc_declines_before_touching_a_gpu():
    """gated_attn_decode_noalloc: invalid dims and partials larger than its
    scratch array (B = 4096 at a 4,096-token capacity: 64 MiB) are declined
    before any device call; batch 0 is a no-op."""
    f = ga.lib.gated_attn_decode_noalloc
    args = [FAKE] * 6 + [0.0625, FAKE, None]
    big = _dims(batch=4096, max_pages_per_seq=256, num_pages=1 << 20)
    assert ga.decode_workspace_size(big) > (16 << 20)
    assert f(*args, ctypes.byref(big)) == ga.GA_ERR_WORKSPACE_TOO_SMALL
    assert f(*args, ctypes.byref(_dims(head_dim=128))) == ga.GA_ERR_UNSUPPORTED
    assert f(*args, ctypes.byref(_dims(num_q_heads=15))) == ga.GA_ERR_INVALID_ARGUMENT
    assert f(*args, None) == ga.GA_ERR_INVALID_ARGUMENT
    assert f(*args, ctypes.byref(_dims(batch=0))) == ga.GA_OK

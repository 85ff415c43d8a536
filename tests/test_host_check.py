"""The C ABI's host logic linked against stand-ins for the HIP runtime and
the kernel launchers (csrc/host_stub.cpp), so the paths that end in a launch
run without a GPU: the device-arch decision (cuDNN "Gated Attention Block",
Requirements and limits: a device the library does not serve is declined with
a typed error), the launch descriptors the plan produces, and the
no-allocation entry point's scratch lookup.  Fake device addresses are only
recorded, never dereferenced.
"""
import ctypes
import importlib.util
import os
import shutil

import pytest

import gated_gqa_decode_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_SCRATCH = 0x7e0000000000
Q, GATE, K, V, BT, SL, OUT, WS = (0x7f0000000000 + (i << 24) for i in range(8))


@pytest.fixture(scope="module")
def host_lib(tmp_path_factory):
    spec = importlib.util.spec_from_file_location(
        "_ga_build", os.path.join(ROOT, "gated_gqa_decode_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = str(tmp_path_factory.mktemp("hostcheck") / "libgated_attn_hostcheck.so")
    return mod.build_host_check(out=out)


def _load(path, tmp_path, arch):
    """A fresh instance of the library (its own device-arch cache) whose fake
    device reports `arch`."""
    copy = tmp_path / f"lib_{arch.split(':')[0]}.so"
    shutil.copy(path, copy)
    lib = ctypes.CDLL(str(copy))
    lib.ga_stub_set_arch(arch.encode())
    vp, f = ctypes.c_void_p, ctypes.c_float
    lib.gated_attn_decode.argtypes = [vp] * 6 + [f, vp, vp, ctypes.POINTER(ga.DecodeDims), vp,
                                                 ctypes.c_size_t]
    lib.gated_attn_decode_noalloc.argtypes = [vp] * 6 + [f, vp, vp, ctypes.POINTER(ga.DecodeDims)]
    lib.gated_attn_decode_fp8kv.argtypes = [vp] * 6 + [f, f, f, vp, vp,
                                                       ctypes.POINTER(ga.DecodeDims), vp,
                                                       ctypes.c_size_t, vp]
    lib.gated_attn_decode_csr.argtypes = [vp] * 6 + [ctypes.c_int64, f, vp, vp,
                                                     ctypes.POINTER(ga.DecodeDims), vp,
                                                     ctypes.c_size_t, vp]
    lib.gated_attn_prefill.argtypes = [vp] * 4 + [f, ctypes.c_int, vp, vp,
                                                  ctypes.POINTER(ga.PrefillDims)]
    lib.gated_attn_qk_norm_rope.argtypes = [vp] * 5 + [f] + [vp] * 7 + [
        ctypes.POINTER(ga.QkNormRopeDims)]
    lib.gated_attn_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    return lib


def _counts(lib):
    c = (ctypes.c_int * 4)()
    lib.ga_stub_launch_counts(c)
    return list(c)


def _last_decode(lib):
    i8 = (ctypes.c_int32 * 8)()
    p3 = (ctypes.c_uint64 * 3)()
    f3 = (ctypes.c_float * 3)()
    lib.ga_stub_last_decode(i8, p3, f3)
    keys = ("tokens_per_split", "num_splits", "split_target", "batch", "page_size", "kv_fp8",
            "window", "num_q_heads")
    d = dict(zip(keys, list(i8)))
    d.update(part_acc=p3[0], part_ml=p3[1], out=p3[2], scale=f3[0], k_descale=f3[1],
             v_descale=f3[2])
    return d


def _dims(**kw):
    base = dict(batch=64, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=16,
                max_pages_per_seq=256, num_pages=16384)
    base.update(kw)
    return ga.decode_dims(**base)


def _calls(lib):
    """One valid call of every entry point that launches."""
    d = _dims()
    ws = ga.decode_workspace_size(d)
    pd = ga.PrefillDims(2, 128, 16, 2, 256)
    rd = ga.QkNormRopeDims(4, 16, 2, 256, 64, 16, 0, 8)
    return {
        "decode": lambda: lib.gated_attn_decode(Q, GATE, K, V, BT, SL, 0.0625, OUT, None,
                                                ctypes.byref(d), WS, ws),
        "decode_noalloc": lambda: lib.gated_attn_decode_noalloc(Q, GATE, K, V, BT, SL, 0.0625,
                                                                OUT, None, ctypes.byref(d)),
        "decode_fp8kv": lambda: lib.gated_attn_decode_fp8kv(Q, GATE, K, V, BT, SL, 0.0625, 0.5,
                                                            0.25, OUT, None, ctypes.byref(d), WS,
                                                            ws, None),
        "decode_csr": lambda: lib.gated_attn_decode_csr(
            Q, GATE, K, V, BT, SL, 1 << 20, 0.0625, OUT, None,
            ctypes.byref(_dims(page_size=1, max_pages_per_seq=4096, num_pages=1 << 20)), WS,
            ga.decode_workspace_size(_dims(page_size=1, max_pages_per_seq=4096,
                                           num_pages=1 << 20)), None),
        "prefill": lambda: lib.gated_attn_prefill(Q, GATE, K, V, 0.0625, 1, OUT, None,
                                                  ctypes.byref(pd)),
        "qk_norm_rope": lambda: lib.gated_attn_qk_norm_rope(Q, K, V, GATE, GATE, 1e-6, BT, SL,
                                                            WS, OUT, K, V, None,
                                                            ctypes.byref(rd)),
        "stream_read": lambda: lib.gated_attn_stream_read(Q, 1 << 20, SL, None),
    }


def test_other_device_is_declined_before_any_launch(host_lib, tmp_path):
    lib = _load(host_lib, tmp_path, "gfx942:sramecc+:xnack-")
    for name, call in _calls(lib).items():
        assert call() == ga.GA_ERR_UNSUPPORTED, name
    assert _counts(lib) == [0, 0, 0, 0]
    assert lib.ga_stub_device_calls() > 0  # the arch query was made


def test_gfx950_reaches_every_launch(host_lib, tmp_path):
    lib = _load(host_lib, tmp_path, "gfx950:sramecc+:xnack-")
    calls = _calls(lib)
    for name, call in calls.items():
        assert call() == ga.GA_OK, name
    # decode, noalloc, fp8kv and csr launch decode; then prefill, rope, read
    assert _counts(lib) == [4, 1, 1, 1]


def test_invariant_divisor_division(host_lib, tmp_path):
    """The launchers' division by a divisor fixed per launch (one high
    multiply, an add and two shifts; the rope kernel's token index) equals
    n // d: every divisor up to 300 and every power of two and its neighbours
    up to 2^32 - 1, against numerators at 0, around multiples of d, at the top
    of the range, and seeded random ones."""
    import random
    lib = _load(host_lib, tmp_path, "gfx950")
    lib.ga_stub_divu32.restype = ctypes.c_uint32
    lib.ga_stub_divu32.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    top = (1 << 32) - 1
    rng = random.Random(32)
    divisors = list(range(1, 301))
    for k in range(9, 33):
        divisors += [(1 << k) - 1, min(1 << k, top), (1 << k) + 1]
    divisors += [rng.randrange(1, top + 1) for _ in range(200)]
    for d in sorted(set(x for x in divisors if 1 <= x <= top)):
        ns = {0, 1, d - 1, d, d + 1, top, top - 1, top - top % d, (top - top % d) - 1}
        ns |= {m * d + e for m in (1, 2, 3, 1000, top // d) for e in (-1, 0, 1)}
        ns |= {rng.randrange(0, top + 1) for _ in range(40)}
        for n in ns:
            if 0 <= n <= top:
                assert lib.ga_stub_divu32(n, d) == n // d, (n, d)


def test_prefill_size_limits(host_lib, tmp_path):
    """q, gate and out past 2^31 elements are served (the kernel addresses them
    with 64-bit offsets); the two real limits -- one sequence's K or V rows in
    one 2^31 - 1 byte buffer descriptor, at most 2^22 workgroups -- are
    declined before any launch, right at their edges."""
    lib = _load(host_lib, tmp_path, "gfx950")

    def call(B, S, Hq, Hkv):
        d = ga.PrefillDims(B, S, Hq, Hkv, 256)
        return lib.gated_attn_prefill(Q, GATE, K, V, 0.0625, 1, OUT, None, ctypes.byref(d))

    served = [
        (65, 2048, 64, 8),              # B*S*H_q*D = 2.18e9 elements > 2^31
        (1, (1 << 21) - 2, 16, 2),      # K rows of one sequence: 2^31 - 2048 bytes
        (2048, 16384, 16, 2),           # exactly 2^22 workgroups
        (1024, 16384, 32, 2),           # group 16 (two parts): exactly 2^22
    ]
    for i, shape in enumerate(served):
        assert call(*shape) == ga.GA_OK, shape
        assert _counts(lib)[1] == i + 1, shape
    for shape in [(1, 1 << 21, 16, 2), (2049, 16384, 16, 2), (1025, 16384, 32, 2)]:
        assert call(*shape) == ga.GA_ERR_UNSUPPORTED, shape
    assert _counts(lib)[1] == len(served)


def test_decode_size_limits(host_lib, tmp_path):
    """The batch is bounded only by one launch's grid (at most 2^32 threads):
    2^22 stage-1 workgroups of 512 threads (B * H_kv * num_splits) and 2^25
    (sequence, query head) rows for stage 2 (one 64-thread workgroup per row).  Served
    past 65,535 sequences and right at both limits; declined one past them,
    before any launch."""
    lib = _load(host_lib, tmp_path, "gfx950")

    def call(B, Hq, Hkv, W):
        d = _dims(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, max_pages_per_seq=W,
                  num_pages=1 << 20)
        return lib.gated_attn_decode(Q, GATE, K, V, BT, SL, 0.0625, OUT, None, ctypes.byref(d),
                                     WS, 1 << 62), d

    served = [
        (65536, 16, 2, 4),        # past the 16-bit grid dimension
        (70000, 16, 2, 3),
        (1 << 21, 16, 2, 1),      # 2^22 stage-1 workgroups (one split each), 2^25 rows
        (1 << 21, 16, 1, 1),      # 2^25 rows at a group of 16
        (1 << 19, 16, 2, 1024),   # 2^20 (sequence, kv head) pairs x 4 splits of 4,096
    ]
    for i, (B, Hq, Hkv, W) in enumerate(served):
        st, d = call(B, Hq, Hkv, W)
        assert st == ga.GA_OK, (B, Hq, Hkv, W)
        assert _counts(lib)[0] == i + 1
        p = ga.decode_plan(d)
        r = _last_decode(lib)
        assert (r["batch"], r["num_splits"]) == (B, p.num_splits)
        assert B * Hkv * p.num_splits <= 1 << 22 and B * Hq <= 1 << 25
    for B, Hq, Hkv, W in [((1 << 21) + 1, 2, 2, 1),      # stage-1 workgroups only
                          ((1 << 21) + 1, 16, 1, 1),     # stage-2 rows only
                          ((1 << 19) + 1, 16, 2, 1024)]:  # workgroups, 4 splits each
        st, d = call(B, Hq, Hkv, W)
        assert st == ga.GA_ERR_UNSUPPORTED, (B, Hq, Hkv, W)
        assert ga.decode_workspace_size(d) == 0
    assert _counts(lib)[0] == len(served)


def test_decode_launch_follows_the_plan(host_lib, tmp_path):
    lib = _load(host_lib, tmp_path, "gfx950")
    for B, W in ((1, 32), (4, 32), (64, 256), (224, 384)):
        d = _dims(batch=B, max_pages_per_seq=W)
        p = ga.decode_plan(d)
        st = lib.gated_attn_decode(Q, GATE, K, V, BT, SL, 0.0625, OUT, None, ctypes.byref(d), WS,
                                   p.workspace_bytes)
        assert st == ga.GA_OK
        r = _last_decode(lib)
        assert (r["tokens_per_split"], r["num_splits"], r["batch"]) == (p.tokens_per_split,
                                                                       p.num_splits, B)
        rows = B * 16 * p.num_splits
        assert r["part_acc"] == WS and r["part_ml"] == WS + rows * 256 * 4
        assert rows * 258 * 4 <= p.workspace_bytes
        assert r["out"] == OUT and r["scale"] == 0.0625 and r["k_descale"] == 1.0
        # one byte short of the plan's workspace: declined, nothing launched
        n = _counts(lib)[0]
        assert lib.gated_attn_decode(Q, GATE, K, V, BT, SL, 0.0625, OUT, None, ctypes.byref(d),
                                     WS, p.workspace_bytes - 1) == ga.GA_ERR_WORKSPACE_TOO_SMALL
        assert _counts(lib)[0] == n


def test_noalloc_uses_the_device_scratch_address(host_lib, tmp_path):
    lib = _load(host_lib, tmp_path, "gfx950")
    for B, W in ((64, 256), (1, 32), (224, 384)):
        d = _dims(batch=B, max_pages_per_seq=W)
        p = ga.decode_plan(d)
        assert lib.gated_attn_decode_noalloc(Q, GATE, K, V, BT, SL, 0.0625, OUT, None,
                                             ctypes.byref(d)) == ga.GA_OK
        r = _last_decode(lib)
        rows = B * 16 * p.num_splits
        assert r["part_acc"] == FAKE_SCRATCH
        assert r["part_ml"] == FAKE_SCRATCH + rows * 256 * 4
    n = _counts(lib)[0]
    big = _dims(batch=4096, max_pages_per_seq=256, num_pages=1 << 20)
    assert lib.gated_attn_decode_noalloc(Q, GATE, K, V, BT, SL, 0.0625, OUT, None,
                                         ctypes.byref(big)) == ga.GA_ERR_WORKSPACE_TOO_SMALL
    assert _counts(lib)[0] == n


def test_fp8_factors_reach_the_launch(host_lib, tmp_path):
    lib = _load(host_lib, tmp_path, "gfx950")
    d = _dims()
    ws = ga.decode_workspace_size(d)
    assert lib.gated_attn_decode_fp8kv(Q, GATE, K, V, BT, SL, 0.0625, 0.5, 0.25, OUT, None,
                                       ctypes.byref(d), WS, ws, None) == ga.GA_OK
    r = _last_decode(lib)
    assert (r["kv_fp8"], r["k_descale"], r["v_descale"]) == (1, 0.5, 0.25)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.gated_attn_decode_fp8kv(Q, GATE, K, V, BT, SL, 0.0625, bad, 0.25, OUT, None,
                                           ctypes.byref(d), WS, ws,
                                           None) == ga.GA_ERR_INVALID_ARGUMENT

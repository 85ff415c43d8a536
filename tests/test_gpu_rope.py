"""GPU parity of gated_attn_qk_norm_rope against the CPU oracle.

The GPU normalises and rotates in fp32 (a few 2^-24 relative to the
magnitudes involved) and rounds once to bf16; the oracle does the same in
fp64.  Rule, every element: |gpu - oracle| <= 1 bf16 ulp of max(|z|, mag),
mag being the magnitude the rotated value is formed from (|y_i cos| +
|y_p sin|; |y| for unrotated dims), so a rotation that cancels is judged
against its terms.  V is copied and must match bit for bit, as must rows
with no norm under the identity or the exact quarter-turn tables.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, to_dev, to_np
from oracle.compare import bf16_bits_to_f64, bf16_ulp

import gated_gqa_decode_amd as ga

pytestmark = pytest.mark.gpu


def _check(got, ref, z, mag, name):
    g, r = bf16_bits_to_f64(got), bf16_bits_to_f64(ref)
    tol = bf16_ulp(np.maximum(np.abs(z), mag))
    err = np.abs(g - r)
    ok = err <= tol
    print(f"[rope] {name}: n={got.size} bit-exact={int(np.sum(got == ref))} "
          f"max_err/ulp={float(np.max(err / tol)):.3f}", flush=True)
    assert np.all(ok), f"{name}: {int(np.sum(~ok))} elements off"


def _gpu(c, norm=True, slots=None, k_pool=None, v_pool=None, cos=None, sin=None):
    cos = c.cos if cos is None else cos
    sin = c.sin if sin is None else sin
    R = cos.shape[1]
    out = ga.qk_norm_rope(
        to_dev(c.q), to_dev(c.k), to_dev(c.v),
        w_q=to_dev(c.w_q) if norm else None, w_k=to_dev(c.w_k) if norm else None, eps=c.eps,
        cos=to_dev(cos) if R else None, sin=to_dev(sin) if R else None,
        slot_mapping=None if slots is None else torch.tensor(slots, dtype=torch.int64,
                                                            device=DEV),
        k_pool=None if k_pool is None else to_dev(k_pool),
        v_pool=None if v_pool is None else to_dev(v_pool))
    torch.cuda.synchronize()
    return [to_np(x) for x in out]


# rope_dim 16..128 in steps of 16 take the RoPE partners from the partner lane
# (DPP row shifts of 1..8 lanes); 8, 200 and 256 load them from memory (200:
# partner groups split in two)
@pytest.mark.parametrize("R", [0, 8, 16, 48, 64, 128, 200, 256])
@pytest.mark.parametrize("norm", [True, False])
def test_dense_parity(R, norm):
    c = workloads.make_rope(f"rope_R{R}", 37, seed=20 + R, rope_dim=R)
    qo, ko, vo = _gpu(c, norm)
    w = (c.w_q, c.w_k) if norm else (None, None)
    rq, rk, rv, qz, qmag, kz, kmag = oracle.qk_norm_rope(c.q, c.k, c.v, *w, c.eps, c.cos, c.sin)
    _check(qo, rq, qz, qmag, f"q R={R} norm={norm}")
    _check(ko, rk, kz, kmag, f"k R={R} norm={norm}")
    assert np.array_equal(vo, c.v)
    if not norm and R == 0:
        assert np.array_equal(qo, c.q) and np.array_equal(ko, c.k)


@pytest.mark.parametrize("R", [16, 64, 128, 200])
def test_quarter_turn_is_bit_exact(R):
    c = workloads.make_rope(f"rope_qt{R}", 9, seed=30 + R, rope_dim=R)
    cos = np.zeros_like(c.cos)
    sin = np.full_like(c.sin, 0x3F80)
    qo, ko, _ = _gpu(c, norm=False, cos=cos, sin=sin)
    rq, rk, _, _, _, _, _ = oracle.qk_norm_rope(c.q, c.k, c.v, None, None, 0.0, cos, sin)
    assert np.array_equal(qo, rq) and np.array_equal(ko, rk)


@pytest.mark.parametrize("Hq,Hkv", [(32, 2), (12, 4), (8, 8)])
def test_head_geometries(Hq, Hkv):
    c = workloads.make_rope(f"rope_{Hq}_{Hkv}", 21, seed=31 + Hq, num_q_heads=Hq,
                            num_kv_heads=Hkv, rope_dim=64)
    qo, ko, vo = _gpu(c)
    rq, rk, _, qz, qmag, kz, kmag = oracle.qk_norm_rope(c.q, c.k, c.v, c.w_q, c.w_k, c.eps,
                                                        c.cos, c.sin)
    _check(qo, rq, qz, qmag, f"q {Hq}/{Hkv}")
    _check(ko, rk, kz, kmag, f"k {Hq}/{Hkv}")
    assert np.array_equal(vo, c.v)


def test_slot_writes():
    """Slots scattered over a poisoned pool, with skipped (-1) and
    out-of-pool slots; every other pool row must stay untouched."""
    T, P = 12, 5
    c = workloads.make_rope("rope_slots", T, seed=33, rope_dim=64)
    kp = np.full((P, 16, 2, 256), workloads.NAN_BF16, np.uint16)
    vp = np.full((P, 16, 2, 256), workloads.NAN_BF16, np.uint16)
    slots = np.array([3, 79, -1, 16, 0, 40, 41, 500, 17, 63, -9, 5], np.int64)
    qo, kpo, vpo = _gpu(c, slots=slots, k_pool=kp, v_pool=vp)
    valid = np.where(slots < P * 16, slots, -1)
    rq, rkp, rvp, qz, qmag, kz, kmag = oracle.qk_norm_rope(
        c.q, c.k, c.v, c.w_q, c.w_k, c.eps, c.cos, c.sin, slot_mapping=valid, k_pool=kp,
        v_pool=vp)
    _check(qo, rq, qz, qmag, "q slots")
    fk, frk, fv, frv = (x.reshape(-1, 2, 256) for x in (kpo, rkp, vpo, rvp))
    for t, s in enumerate(valid):
        if s >= 0:
            _check(fk[s], frk[s], kz[t], kmag[t], f"k slot {s}")
    untouched = np.setdiff1d(np.arange(P * 16), valid[valid >= 0])
    assert np.array_equal(fk[untouched], frk[untouched])
    assert np.array_equal(fv, frv)


def test_decode_after_norm_rope_append():
    """The step before attention then attention: the new token of every
    sequence is normed, rotated and written at position L - 1 of its pages,
    then decode runs on the normed, rotated q.  Compared with the oracle doing
    the same two steps."""
    lens = [1, 17, 300, 64, 999, 0]
    c = workloads.make_decode("rope_pipeline", lens, seed=34, poison=True, max_pages_per_seq=64)
    B = len(lens)
    r = workloads.make_rope("rope_pipeline_new", B, seed=35, rope_dim=64)
    L = np.asarray(lens)
    slots = np.array([c.block_table[b, (l - 1) // 16] * 16 + (l - 1) % 16 if l > 0 else -1
                      for b, l in enumerate(L)], np.int64)
    # GPU: norm/rope/append into the device pools, then decode
    kp, vp = to_dev(c.k_pool), to_dev(c.v_pool)
    q_new, _, _ = ga.qk_norm_rope(to_dev(r.q), to_dev(r.k), to_dev(r.v), w_q=to_dev(r.w_q),
                                  w_k=to_dev(r.w_k), eps=r.eps, cos=to_dev(r.cos),
                                  sin=to_dev(r.sin),
                                  slot_mapping=torch.tensor(slots, dtype=torch.int64, device=DEV),
                                  k_pool=kp, v_pool=vp)
    out = ga.decode(q_new, to_dev(c.gate), kp, vp, to_dev(c.block_table), to_dev(c.seq_lens),
                    c.scale)
    torch.cuda.synchronize()
    got_q = to_np(q_new)
    # oracle: the same two steps
    rq, rkp, rvp, qz, qmag, _, _ = oracle.qk_norm_rope(r.q, r.k, r.v, r.w_q, r.w_k, r.eps, r.cos,
                                                       r.sin, slot_mapping=slots,
                                                       k_pool=c.k_pool, v_pool=c.v_pool)
    _check(got_q, rq, qz, qmag, "pipeline q")
    # decode parity on the GPU's own q (the rope step is checked just above)
    ref, o, mref = oracle.decode(got_q, c.gate, to_np(kp), to_np(vp), c.block_table, c.seq_lens,
                                 c.scale)
    from oracle.compare import check_outputs
    res = check_outputs(to_np(out), ref, o, mref, oracle.sigmoid_table()[c.gate])
    assert res["ok"], res
    # and the pools the GPU wrote hold the oracle's rows at the appended slots
    fk, frk = to_np(kp).reshape(-1, 2, 256), rkp.reshape(-1, 2, 256)
    for s in slots[slots >= 0]:
        d = np.abs(bf16_bits_to_f64(fk[s]) - bf16_bits_to_f64(frk[s]))
        assert np.all(d <= bf16_ulp(np.abs(bf16_bits_to_f64(frk[s]))) * 2)


def test_graph_replay_with_changed_inputs():
    """The decode step's norm/rope/append captured into a HIP graph (slot
    mode, caller-owned q_out and pools: nothing is allocated inside), replayed
    with new rows and slots: every replay equals an eager call, bit for bit."""
    T, P = 24, 4
    c = workloads.make_rope("rope_graph", T, seed=36, rope_dim=64)
    t = {n: to_dev(getattr(c, n)) for n in ("q", "k", "v", "w_q", "w_k", "cos", "sin")}
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    kp = torch.zeros((P, 16, 2, 256), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    q_out = torch.empty_like(t["q"])

    def call(kpool, vpool, qo):
        ga.qk_norm_rope(t["q"], t["k"], t["v"], w_q=t["w_q"], w_k=t["w_k"], eps=c.eps,
                        cos=t["cos"], sin=t["sin"], slot_mapping=slots, k_pool=kpool,
                        v_pool=vpool, q_out=qo)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(kp, vp, q_out)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(kp, vp, q_out)
    rng = np.random.default_rng(7)
    for it in range(4):
        for i, n in enumerate(("q", "k", "v")):
            t[n].copy_(to_dev(workloads.normal_bf16(400 + 10 * it + i, 1, getattr(c, n).shape)))
        perm = rng.permutation(P * 16)[:T]
        perm[rng.integers(0, T)] = -1  # one skipped token
        slots.copy_(torch.from_numpy(perm.astype(np.int64)).to(DEV))
        kp.zero_()
        vp.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = [to_np(x) for x in (q_out, kp, vp)]
        kp2, vp2, qo2 = torch.zeros_like(kp), torch.zeros_like(vp), torch.empty_like(q_out)
        call(kp2, vp2, qo2)
        torch.cuda.synchronize()
        for a, b in zip(got, (to_np(qo2), to_np(kp2), to_np(vp2))):
            assert np.array_equal(a, b), it

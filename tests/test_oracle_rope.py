"""Pins for the oracle's QK-RMSNorm + partial RoPE + K/V slot write.

Closed forms and exact constructions, not a retyped formula: the identity
(no norm, no rotation, cos 1 / sin 0), the exact quarter turn (cos 0, sin 1:
a signed swap of the two halves), a constant row (its norm is sign(c) * w),
power-of-two scale invariance of the norm, preserved pair norms under a
rotation, slot placement in the pools, and a 50-digit decimal brute force.
"""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle.compare import bf16_bits_to_f64
from test_oracle_bf16 import grid_round

B16 = np.uint16


def _tabs(T, R, c_bits, s_bits):
    return np.full((T, R), c_bits, B16), np.full((T, R), s_bits, B16)


def test_no_norm_no_rotation_is_identity():
    c = workloads.make_rope("id", 5, seed=1, rope_dim=0)
    for cos, sin, R in ((c.cos, c.sin, 0), _tabs(5, 64, 0x3F80, 0x0000) + (64,)):
        qo, ko, vo, qz, _, _, _ = oracle.qk_norm_rope(c.q, c.k, c.v, None, None, 1e-6, cos, sin)
        assert np.array_equal(qo, c.q) and np.array_equal(ko, c.k) and np.array_equal(vo, c.v)
        assert np.array_equal(qz, bf16_bits_to_f64(c.q))


@pytest.mark.parametrize("R", [8, 64, 256])
def test_quarter_turn_swaps_halves_with_sign(R):
    """cos 0, sin 1: z_i = -y_{i+R/2}, z_{i+R/2} = y_i, dims >= R untouched."""
    c = workloads.make_rope("qt", 3, seed=2, rope_dim=0)
    cos, sin = _tabs(3, R, 0x0000, 0x3F80)
    qo, ko, _, _, _, _, _ = oracle.qk_norm_rope(c.q, c.k, c.v, None, None, 1e-6, cos, sin)
    h = R // 2
    for x, o in ((c.q, qo), (c.k, ko)):
        assert np.array_equal(o[..., :h], x[..., h:R] ^ 0x8000)
        assert np.array_equal(o[..., h:R], x[..., :h])
        assert np.array_equal(o[..., R:], x[..., R:])


def test_constant_row_normalises_to_the_weight():
    """x_d = c for every d, eps = 0: y = sign(c) * w exactly."""
    c = workloads.make_rope("cr", 4, seed=3, rope_dim=0)
    q = np.empty_like(c.q)
    consts = np.array([0x3F80, 0xC040, 0x3A80, 0x4700], B16)  # 1, -3, 2^-10 * 1, 32768
    for t in range(4):
        q[t] = consts[t]
    qo, _, _, _, _, _, _ = oracle.qk_norm_rope(q, c.k, c.v, c.w_q, c.w_k, 0.0, c.cos, c.sin)
    for t in range(4):
        want = c.w_q ^ (0x8000 if consts[t] & 0x8000 else 0)
        assert np.array_equal(qo[t, 0], want), t


def test_norm_is_invariant_under_power_of_two_scaling():
    c = workloads.make_rope("sc", 6, seed=4)
    base = oracle.qk_norm_rope(c.q, c.k, c.v, c.w_q, c.w_k, 0.0, c.cos, c.sin)
    x = bf16_bits_to_f64(c.q) * 2.0 ** -5
    q2 = oracle.bf16_rne(x)
    assert np.array_equal(bf16_bits_to_f64(q2), x)
    r = oracle.qk_norm_rope(q2, c.k, c.v, c.w_q, c.w_k, 0.0, c.cos, c.sin)
    assert np.array_equal(r[0], base[0]) and np.array_equal(r[3], base[3])


def test_rotation_preserves_pair_norms():
    """Both halves use the same (cos, sin): z_i^2 + z_p^2 = (y_i^2 + y_p^2)(c^2 + s^2)."""
    c = workloads.make_rope("pn", 8, seed=5, rope_dim=64)
    _, _, _, qz, _, _, _ = oracle.qk_norm_rope(c.q, c.k, c.v, None, None, 0.0, c.cos, c.sin)
    y = bf16_bits_to_f64(c.q)
    cs, sn = bf16_bits_to_f64(c.cos)[:, None, :32], bf16_bits_to_f64(c.sin)[:, None, :32]
    lhs = qz[..., :32] ** 2 + qz[..., 32:64] ** 2
    rhs = (y[..., :32] ** 2 + y[..., 32:64] ** 2) * (cs ** 2 + sn ** 2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-300)
    assert np.array_equal(qz[..., 64:], y[..., 64:])


def test_slots_receive_the_rows_and_nothing_else():
    c = workloads.make_rope("sl", 6, seed=6)
    dense = oracle.qk_norm_rope(c.q, c.k, c.v, c.w_q, c.w_k, c.eps, c.cos, c.sin)
    P = 3
    kp = np.full((P, 16, 2, 256), 0x1234, B16)
    vp = np.full((P, 16, 2, 256), 0x4321, B16)
    slots = np.array([17, -1, 0, 47, 5, -7], np.int64)
    r = oracle.qk_norm_rope(c.q, c.k, c.v, c.w_q, c.w_k, c.eps, c.cos, c.sin, slot_mapping=slots,
                            k_pool=kp, v_pool=vp)
    assert np.array_equal(r[0], dense[0])
    fk, fv = r[1].reshape(-1, 2, 256), r[2].reshape(-1, 2, 256)
    written = set()
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(fk[s], dense[1][t]) and np.array_equal(fv[s], c.v[t])
            written.add(int(s))
    for s in range(P * 16):
        if s not in written:
            assert np.all(fk[s] == 0x1234) and np.all(fv[s] == 0x4321)


def _dec(bits):
    return Decimal(float(bf16_bits_to_f64(np.array([bits], B16))[0]))


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_tiny(seed):
    """D = 16, R = 8, eps = 1e-3, 50-digit decimal arithmetic, one rounding."""
    D, R, eps = 16, 8, 1e-3
    c = workloads.make_rope("bf", 2, seed=10 + seed, num_q_heads=2, num_kv_heads=1, head_dim=D,
                            rope_dim=R)
    qo, ko, _, _, _, _, _ = oracle.qk_norm_rope(c.q, c.k, c.v, c.w_q, c.w_k, eps, c.cos, c.sin)
    with localcontext() as ctx:
        ctx.prec = 50
        for x, w, o in ((c.q, c.w_q, qo), (c.k, c.w_k, ko)):
            for t in range(2):
                for h in range(x.shape[1]):
                    xs = [_dec(b) for b in x[t, h]]
                    r = 1 / (sum(a * a for a in xs) / D + Decimal(eps)).sqrt()
                    y = [a * r * _dec(wb) for a, wb in zip(xs, w)]
                    z = list(y)
                    for i in range(R // 2):
                        p = i + R // 2
                        z[i] = y[i] * _dec(c.cos[t, i]) - y[p] * _dec(c.sin[t, i])
                        z[p] = y[p] * _dec(c.cos[t, p]) + y[i] * _dec(c.sin[t, p])
                    assert list(o[t, h]) == [grid_round(Fraction(v)) for v in z], (t, h)

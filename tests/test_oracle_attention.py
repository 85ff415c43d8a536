"""Pins for the oracle's attention: closed forms, invariants, brute force.

None of these re-types the oracle's formula at the same precision:
  * closed forms whose answer is fixed by the mathematics (a single key, equal
    scores, a dominating key, a two-key softmax = the logistic function from
    scipy, constant values per kv head, gate 0 / +40, padded rows);
  * invariants (page permutation, score shift, masked-future independence);
  * a 50-digit decimal brute force on tiny shapes.
Each is chosen so a plausible slip in the oracle (wrong page/slot/head index,
dropped key, missing scale, flipped sign, off-by-one causal mask, a missing
normalisation) fails at least one of them.
"""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads
from oracle.compare import bf16_bits_to_f64
from test_oracle_bf16 import grid_round, _decimal_sigmoid_bits

B16 = np.uint16


def _f2b(x):
    """float -> bf16 bits for values that are exactly representable."""
    x = np.asarray(x, dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    back = bf16_bits_to_f64(bits).reshape(x.shape)
    assert np.array_equal(back, x.astype(np.float64)), "not exact in bf16"
    return bits


def _case(lens, seed=0, Hq=16, Hkv=2, D=256, W=None, poison=True, shuffle=True, extra=0):
    return workloads.make_decode("t", lens, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv,
                                 head_dim=D, max_pages_per_seq=W, poison=poison,
                                 shuffle=shuffle, extra_pages=extra)


def _run(c):
    return oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale)


def _kv_row(c, pool, b, j, g):
    page = c.block_table[b, j // workloads.PAGE_SIZE]
    return pool[page, j % workloads.PAGE_SIZE, g]


def _sig_table():
    return oracle.sigmoid_table()


# --------------------------------------------------------------------------
def test_single_key_output_is_gated_value():
    """L = 1: softmax weight 1, so O = V_0 exactly and out = bf16(V_0 * sigma_b)."""
    c = _case([1, 1, 1], seed=5)
    out, o, mref = _run(c)
    sig = _sig_table()
    for b in range(3):
        for h in range(16):
            v = _kv_row(c, c.v_pool, b, 0, h // 8)
            assert np.array_equal(o[b, h], bf16_bits_to_f64(v))
            exp = [oracle.gate_output(int(vb), int(sig[gb])) for vb, gb in zip(v, c.gate[b, h])]
            assert np.array_equal(out[b, h], np.array(exp, dtype=B16))


@pytest.mark.parametrize("jstar", [0, 1, 15, 16, 17, 31, 32, 36])
def test_dominating_key_selects_its_value(jstar):
    """One key aligned with 64*q scores ~1000 above the rest: every other weight
    underflows to exactly 0 in fp64, so O = V[j*] -- pins the page/slot gather."""
    c = _case([37, 40], seed=9)
    b, h = 1, 11
    g = h // 8
    qv = bf16_bits_to_f64(c.q[b, h])
    assert float(qv @ qv) > 200.0
    page = c.block_table[b, jstar // 16]
    c.k_pool[page, jstar % 16, g] = _f2b(64.0 * qv)
    out, o, _ = _run(c)
    assert np.array_equal(o[b, h], bf16_bits_to_f64(_kv_row(c, c.v_pool, b, jstar, g)))
    # the other sequence is unaffected and finite
    assert np.all(np.isfinite(o[0]))


@pytest.mark.parametrize("L", [32, 37, 64])
def test_equal_scores_give_mean_of_values(L):
    """All keys identical: equal scores, O = mean_j V_j (exact sum / L) and the
    reference magnitude Mref = mean_j |V_j|."""
    c = _case([L], seed=3)
    for j in range(L):
        for g in range(2):
            page = c.block_table[0, j // 16]
            c.k_pool[page, j % 16, g] = c.k_pool[c.block_table[0, 0], 0, g]
    _, o, mref = _run(c)
    for h in (0, 7, 8, 15):
        g = h // 8
        vals = [bf16_bits_to_f64(_kv_row(c, c.v_pool, 0, j, g)) for j in range(L)]
        for d in (0, 1, 100, 255):
            exact = Fraction(sum(Fraction(float(v[d])) for v in vals), L)
            assert o[0, h, d] == float(exact), (h, d)
            mag = Fraction(sum(abs(Fraction(float(v[d]))) for v in vals), L)
            assert mref[0, h, d] == float(mag), (h, d)


@pytest.mark.parametrize("delta_raw", [0.5, -1.25, 3.0, 24.0])
def test_two_key_softmax_is_logistic(delta_raw):
    """Two keys whose scores differ by scale * q0 * (k0 - k1): the weight of key 0
    is expit(difference) -- pins the scale, the exponent's sign and base e."""
    c = _case([2], seed=4)
    b, h, g = 0, 3, 0
    q = np.zeros(256, np.float32)
    q[0] = 2.0
    c.q[b, h] = _f2b(q)
    k0 = np.zeros(256, np.float32)
    k1 = np.zeros(256, np.float32)
    k0[0] = delta_raw * 16 / 2.0  # scale = 1/16, q0 = 2
    c.k_pool[c.block_table[0, 0], 0, g] = _f2b(k0)
    c.k_pool[c.block_table[0, 0], 1, g] = _f2b(k1)
    _, o, _ = _run(c)
    w0 = expit(delta_raw)
    v0 = bf16_bits_to_f64(_kv_row(c, c.v_pool, 0, 0, g))
    v1 = bf16_bits_to_f64(_kv_row(c, c.v_pool, 0, 1, g))
    np.testing.assert_allclose(o[b, h], w0 * v0 + (1 - w0) * v1, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (4, 2), (8, 1), (6, 3)])
def test_gqa_head_map_is_contiguous_groups(Hq, Hkv):
    """V constant 2^g on kv head g (a power of two, so the weighted mean is
    exact): query head h must see 2^(h // (Hq/Hkv))."""
    c = _case([20, 5], seed=6, Hq=Hq, Hkv=Hkv, D=16)
    for g in range(Hkv):
        c.v_pool[:, :, g, :] = _f2b(np.float32(2.0 ** g))
    _, o, _ = _run(c)
    for h in range(Hq):
        assert np.all(o[:, h, :] == 2.0 ** (h // (Hq // Hkv))), h


def test_page_permutation_invariance():
    """The same logical KV under two different page permutations: identical bits."""
    a = _case([100, 77, 3], seed=12, extra=5)
    b = _case([100, 77, 3], seed=12, extra=5)
    rng = np.random.default_rng(1)
    perm = rng.permutation(a.k_pool.shape[0]).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    b.k_pool = a.k_pool[inv].copy()   # new page p holds old page inv[p]
    b.v_pool = a.v_pool[inv].copy()
    b.block_table = np.where(a.block_table >= 0, perm[np.clip(a.block_table, 0, None)], -1)
    ra, rb = _run(a), _run(b)
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])


def test_poisoned_tails_and_pages_do_not_leak():
    c = _case([17, 1, 33, 0], seed=2, extra=3)
    out, o, mref = _run(c)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(mref))
    assert not np.any((out & 0x7F80) == 0x7F80)


def test_score_shift_invariance():
    """Adding the same amount to every score leaves O unchanged (softmax is
    shift invariant); an oracle that forgot the normalisation would not be."""
    a = _case([50], seed=8, poison=False)
    b = _case([50], seed=8, poison=False)
    a.q[:, :, 255] = _f2b(np.float32(8.0))
    b.q[:, :, 255] = _f2b(np.float32(8.0))
    a.k_pool[:, :, :, 255] = 0
    b.k_pool[:, :, :, 255] = _f2b(np.float32(32.0))  # +8*32/16 = +16 on every score
    _, oa, _ = _run(a)
    _, ob, _ = _run(b)
    np.testing.assert_allclose(ob, oa, rtol=1e-12, atol=1e-14)


def test_padded_rows_are_positive_zero():
    c = _case([0, 9, -3], seed=1)
    out, o, _ = _run(c)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(o[0] == 0)
    assert np.any(out[1] != 0)


def test_mref_equals_abs_o_for_nonnegative_values():
    c = _case([40], seed=10)
    c.v_pool &= 0x7FFF  # clear sign bits (NaN poison stays NaN but is never read)
    _, o, mref = _run(c)
    assert np.array_equal(o, mref)


def test_gate_closed_forms_on_attention():
    """gate = 0 -> out = bf16(O)/2 (exact), gate = +40 -> out = bf16(O)."""
    c = _case([70, 33], seed=13)
    c.gate[0] = 0x0000
    c.gate[1] = 0x4220
    out, o, _ = _run(c)
    ob = oracle.bf16_rne(o)
    half = bf16_bits_to_f64(ob[0]) / 2
    assert np.array_equal(bf16_bits_to_f64(out[0]), half)
    assert np.array_equal(out[1], ob[1])


# --------------------------------------------------------------------------
# 50-digit brute force on tiny shapes
# --------------------------------------------------------------------------
def _dec(bits):
    return Decimal(float(bf16_bits_to_f64(np.array([bits], dtype=B16))[0]))


def _brute_row(qrow, keys, vals, gate_row, scale):
    """Decimal (50 digits) softmax, then exact-rational bf16 roundings."""
    with localcontext() as ctx:
        ctx.prec = 50
        s = [Decimal(scale) * sum(_dec(a) * _dec(b) for a, b in zip(qrow, k)) for k in keys]
        m = max(s)
        p = [(x - m).exp() for x in s]
        den = sum(p)
        outs = []
        for d in range(len(qrow)):
            o = sum(pj * _dec(v[d]) for pj, v in zip(p, vals)) / den
            ob = grid_round(Fraction(o))
            sb = _decimal_sigmoid_bits(int(gate_row[d]))
            prod = Fraction(float(bf16_bits_to_f64(np.array([ob], B16))[0])) * \
                Fraction(float(bf16_bits_to_f64(np.array([sb], B16))[0]))
            outs.append(grid_round(prod))
    return outs


@pytest.mark.parametrize("seed", range(6))
def test_decode_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, 10, size=3)]
    c = workloads.make_decode("tiny", lens, seed=100 + seed, num_q_heads=4, num_kv_heads=2,
                              head_dim=8, poison=True, extra_pages=2)
    out, _, _ = _run(c)
    for b, L in enumerate(lens):
        for h in range(4):
            g = h // 2
            keys = [_kv_row(c, c.k_pool, b, j, g) for j in range(L)]
            vals = [_kv_row(c, c.v_pool, b, j, g) for j in range(L)]
            ref = _brute_row(c.q[b, h], keys, vals, c.gate[b, h], c.scale)
            assert list(out[b, h]) == ref, (b, h)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_brute_force_tiny(causal):
    c = workloads.make_prefill("tiny", 2, 6, seed=21, num_q_heads=4, num_kv_heads=2,
                               head_dim=8, causal=causal)
    out, _, _ = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, causal=causal)
    for b in range(2):
        for i in range(6):
            L = i + 1 if causal else 6
            for h in range(4):
                g = h // 2
                ref = _brute_row(c.q[b, i, h], [c.k[b, j, g] for j in range(L)],
                                 [c.v[b, j, g] for j in range(L)], c.gate[b, i, h], c.scale)
                assert list(out[b, i, h]) == ref, (b, i, h)


def test_causal_row_ignores_the_future_and_sees_the_diagonal():
    c = workloads.make_prefill("t", 1, 40, seed=5, num_q_heads=4, num_kv_heads=2, head_dim=32)
    i = 17
    rows = np.array([[0, i]], np.int32)
    base = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, True, rows=rows)[1]
    k2, v2 = c.k.copy(), c.v.copy()
    k2[0, i + 1:] = 0x7FC0  # NaN in every future position
    v2[0, i + 1:] = 0x7FC0
    fut = oracle.prefill(c.q, c.gate, k2, v2, c.scale, True, rows=rows)[1]
    assert np.array_equal(base, fut)
    v3 = c.v.copy()
    v3[0, i] = 0x7FC0       # the diagonal key is visible
    diag = oracle.prefill(c.q, c.gate, c.k, v3, c.scale, True, rows=rows)[1]
    assert np.all(np.isnan(diag))


def test_prefill_rows_subset_matches_full():
    c = workloads.make_prefill("t", 2, 24, seed=6, num_q_heads=4, num_kv_heads=2, head_dim=16)
    full = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, True)
    rows = np.array([[1, 0], [0, 23], [1, 13]], np.int32)
    sub = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, True, rows=rows)
    for r, (b, i) in enumerate(rows):
        assert np.array_equal(sub[0][r], full[0][b, i])
        assert np.array_equal(sub[1][r], full[1][b, i])


def test_oracle_rejects_bad_page_ids():
    c = _case([20], seed=1)
    c.block_table[0, 1] = c.k_pool.shape[0] + 4
    with pytest.raises(oracle.OracleError):
        _run(c)

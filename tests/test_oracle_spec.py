"""Pins for the oracle's attention-spec options: sliding window, attention
sinks, the log-sum-exp output and per-sequence key lengths in prefill.

The readings these pin (the pages name the options without defining them):
  * a window w > 0 keeps the w most recent visible keys (decode: j >= L - w;
    prefill row i: j > i - w);
  * a sink is a per-head logit that joins the softmax denominator only, i.e. a
    key with score sink_h and an all-zero value row;
  * lse = ln(sum_visible exp(s_j) + exp(sink_h)), natural log, -inf when the
    row has no visible key and no sink;
  * prefill key lengths mask keys j >= len[b] (query rows are not dropped);
    a row with no visible key is dead: out = +0.
None of the checks re-types the oracle's formula at the same precision: they
use closed forms (one key, identical keys, the logistic two-term softmax),
constructions that turn an option into plain attention on other inputs (a
window into a shorter sequence, a sink into an extra zero-value key, a prefill
row into a decode), and a 50-digit decimal brute force.
"""
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
PS = workloads.PAGE_SIZE


def _val(bits):
    return bf16_bits_to_f64(np.asarray(bits, dtype=B16))


def _kv_row(c, pool, b, j, g):
    return pool[c.block_table[b, j // PS], j % PS, g]


def _exact_score(qrow, krow, scale):
    """scale * q.k as an exact rational, rounded once to fp64."""
    dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(_val(qrow), _val(krow)))
    return float(Fraction(scale) * dot)


def _dense_pool(k_rows, v_rows):
    """Pack [L, H_kv, D] token rows into a contiguous paged pool."""
    L, Hkv, D = k_rows.shape
    P = max(1, -(-L // PS))
    kp = np.zeros((P, PS, Hkv, D), dtype=B16)
    vp = np.zeros((P, PS, Hkv, D), dtype=B16)
    kp.reshape(P * PS, Hkv, D)[:L] = k_rows
    vp.reshape(P * PS, Hkv, D)[:L] = v_rows
    return kp, vp, np.arange(P, dtype=np.int32)[None, :]


def _tokens(c, b, j0, j1):
    """K and V rows [j1 - j0, H_kv, D] of tokens j0..j1-1 of sequence b."""
    ks = np.stack([c.k_pool[c.block_table[b, j // PS], j % PS] for j in range(j0, j1)])
    vs = np.stack([c.v_pool[c.block_table[b, j // PS], j % PS] for j in range(j0, j1)])
    return ks, vs


# --------------------------------------------------------------------------
# sliding window (decode)
# --------------------------------------------------------------------------
def test_window_of_one_selects_the_last_value():
    """w = 1: one visible key, so O = V_{L-1} exactly, out = bf16(V * sigma_b)
    and lse = s_{L-1}."""
    c = workloads.make_decode("w1", [1, 37, 160], seed=11)
    out, o, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                   c.scale, window=1, return_lse=True)
    sig = oracle.sigmoid_table()
    Hq = c.q.shape[1]
    G = Hq // c.k_pool.shape[2]
    for b, L in enumerate(c.seq_lens):
        for h in range(Hq):
            v = _kv_row(c, c.v_pool, b, L - 1, h // G)
            assert np.array_equal(o[b, h], _val(v))
            want = [oracle.gate_output(int(x), int(sig[gg])) for x, gg in zip(v, c.gate[b, h])]
            assert list(out[b, h]) == want
            s = _exact_score(c.q[b, h], _kv_row(c, c.k_pool, b, L - 1, h // G), c.scale)
            assert abs(lse[b, h] - s) <= 1e-12 * max(1.0, abs(s))


@pytest.mark.parametrize("w", [5, 16, 37, 100])
def test_window_equals_the_truncated_sequence(w):
    """Decode with window w == plain decode over the last w tokens alone
    (repacked into a fresh pool), bit for bit: same keys, same order."""
    lens = [300, 40, 7, 101]
    c = workloads.make_decode("wt", lens, seed=12)
    out, o, mref, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                                      c.seq_lens, c.scale, window=w, return_lse=True)
    for b, L in enumerate(lens):
        j0 = max(0, L - w)
        ks, vs = _tokens(c, b, j0, L)
        kp, vp, bt = _dense_pool(ks, vs)
        r = oracle.decode(c.q[b:b + 1], c.gate[b:b + 1], kp, vp, bt,
                          np.array([L - j0], np.int32), c.scale, return_lse=True)
        assert np.array_equal(out[b], r[0][0])
        assert np.array_equal(o[b], r[1][0])
        assert np.array_equal(mref[b], r[2][0])
        assert np.array_equal(lse[b], r[3][0])


def test_window_not_shorter_than_the_sequence_changes_nothing():
    c = workloads.make_decode("wn", [50, 64, 65], seed=13)
    base = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                         return_lse=True)
    for w in (65, 66, 1000):
        r = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                          window=w, return_lse=True)
        for x, y in zip(base, r):
            assert np.array_equal(x, y)
    r = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                      window=64, return_lse=True)
    assert np.array_equal(r[1][:2], base[1][:2])       # L <= 64: unchanged
    assert not np.array_equal(r[1][2], base[1][2])     # L = 65 loses its first key


# --------------------------------------------------------------------------
# sinks (decode)
# --------------------------------------------------------------------------
def test_sink_with_one_key_is_the_logistic_weight():
    """L = 1: O = V_0 * e^s / (e^s + e^sink) = V_0 * expit(s - sink) and
    lse = logaddexp(s, sink)."""
    c = workloads.make_decode("s1", [1, 1], seed=14)
    Hq = c.q.shape[1]
    G = Hq // c.k_pool.shape[2]
    sinks = np.linspace(-3.0, 2.5, Hq)
    _, o, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                 c.scale, sinks=sinks, return_lse=True)
    for b in range(2):
        for h in range(Hq):
            s = _exact_score(c.q[b, h], _kv_row(c, c.k_pool, b, 0, h // G), c.scale)
            v = _val(_kv_row(c, c.v_pool, b, 0, h // G))
            np.testing.assert_allclose(o[b, h], v * expit(s - sinks[h]), rtol=1e-14, atol=0)
            assert abs(lse[b, h] - np.logaddexp(s, sinks[h])) <= 1e-14 * max(1, abs(lse[b, h]))


def test_sink_is_an_extra_key_with_a_zero_value_row():
    """q_h = c_h * e_0 makes every score scale * c_h * k_j[0]; appending a key
    with k[0] = 12 and V = 0 then adds the logit sink_h = scale * 12 * c_h to
    the denominator only.  Plain decode over the L + 1 keys must equal decode
    with those sinks over the first L keys (up to fp64 summation order)."""
    L, Hq, Hkv, D = 45, 8, 2, 256
    c = workloads.make_decode("sx", [L + 1], seed=15, num_q_heads=Hq, num_kv_heads=Hkv,
                              shuffle=False, poison=False)
    coef = np.array([1.0, 0.5, 2.0, -1.0, 0.25, -0.5, 1.5, 3.0])
    c.q[:] = 0
    c.q[0, :, 0] = (coef.astype(np.float32).view(np.uint32) >> 16).astype(B16)
    flat_k = c.k_pool.reshape(-1, Hkv, D)
    flat_v = c.v_pool.reshape(-1, Hkv, D)
    flat_k[L] = 0
    flat_k[L, :, 0] = 0x4140  # 12.0
    flat_v[L] = 0
    sinks = c.scale * 12.0 * coef
    plain = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                          return_lse=True)
    with_sink = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                              np.array([L], np.int32), c.scale, sinks=sinks, return_lse=True)
    assert np.array_equal(plain[0], with_sink[0])
    np.testing.assert_allclose(with_sink[1], plain[1], rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(with_sink[3], plain[3], rtol=1e-14)


def test_sink_of_minus_infinity_is_no_sink():
    c = workloads.make_decode("sn", [33, 1, 0], seed=16)
    base = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                         return_lse=True)
    r = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                      sinks=np.full(c.q.shape[1], -np.inf), return_lse=True)
    for x, y in zip(base, r):
        assert np.array_equal(x, y)


def test_dead_rows_output_zero_and_their_lse_is_the_sink():
    c = workloads.make_decode("sd", [0, -3, 5], seed=17)
    Hq = c.q.shape[1]
    out, o, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                   c.scale, return_lse=True)
    assert not np.any(out[:2]) and not np.any(o[:2])
    assert np.all(np.isneginf(lse[:2]))
    sinks = np.arange(Hq, dtype=np.float64) - 4.0
    out, o, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                   c.scale, sinks=sinks, return_lse=True)
    assert not np.any(out[:2])
    assert np.array_equal(lse[0], sinks) and np.array_equal(lse[1], sinks)


# --------------------------------------------------------------------------
# lse closed form
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L", [1, 2, 17, 300])
def test_lse_of_identical_keys_is_score_plus_log_length(L):
    c = workloads.make_decode("li", [L], seed=18, poison=False)
    c.k_pool[:] = c.k_pool[0, 0]
    _, _, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                 c.scale, return_lse=True)
    Hq = c.q.shape[1]
    G = Hq // c.k_pool.shape[2]
    for h in range(Hq):
        s = _exact_score(c.q[0, h], c.k_pool[0, 0, h // G], c.scale)
        assert abs(lse[0, h] - (s + np.log(L))) <= 1e-12 * max(1.0, abs(s))


# --------------------------------------------------------------------------
# 50-digit brute force with window, sinks and lse
# --------------------------------------------------------------------------
def _dec(bits):
    return Decimal(float(_val(np.array([bits], dtype=B16))[0]))


def _brute(qrow, keys, vals, gate_row, scale, sink):
    with localcontext() as ctx:
        ctx.prec = 50
        s = [Decimal(scale) * sum(_dec(a) * _dec(b) for a, b in zip(qrow, k)) for k in keys]
        terms = list(s) + ([Decimal(sink)] if sink is not None else [])
        if not terms:
            return [0] * len(qrow), float("-inf")
        m = max(terms)
        p = [(x - m).exp() for x in s]
        den = sum(p) + ((Decimal(sink) - m).exp() if sink is not None else 0)
        lse = float(m + den.ln())
        if not keys:
            return [0] * len(qrow), lse
        outs = []
        for d in range(len(qrow)):
            o = sum(pj * _dec(v[d]) for pj, v in zip(p, vals)) / den
            ob = grid_round(Fraction(o))
            sb = _decimal_sigmoid_bits(int(gate_row[d]))
            prod = Fraction(float(_val(np.array([ob], B16))[0])) * \
                Fraction(float(_val(np.array([sb], B16))[0]))
            outs.append(grid_round(prod))
    return outs, lse


@pytest.mark.parametrize("seed", range(4))
def test_decode_brute_force_window_sinks_lse(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 12, size=3)]
    w = int(rng.integers(1, 6))
    c = workloads.make_decode("bf", lens, seed=200 + seed, num_q_heads=4, num_kv_heads=2,
                              head_dim=8, poison=True, extra_pages=2, max_pages_per_seq=1)
    sinks = rng.normal(0.0, 1.0, size=4)
    out, _, _, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                   c.scale, sinks=sinks, window=w, return_lse=True)
    for b, L in enumerate(lens):
        for h in range(4):
            g = h // 2
            js = range(max(0, L - w), L)
            ref, ref_lse = _brute(c.q[b, h], [_kv_row(c, c.k_pool, b, j, g) for j in js],
                                  [_kv_row(c, c.v_pool, b, j, g) for j in js], c.gate[b, h],
                                  c.scale, float(sinks[h]))
            assert list(out[b, h]) == ref, (b, h)
            assert abs(lse[b, h] - ref_lse) <= 1e-14 * max(1.0, abs(ref_lse)), (b, h)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_brute_force_lengths_window_sinks(causal):
    S, w = 7, 3
    c = workloads.make_prefill("bfp", 2, S, seed=31, num_q_heads=4, num_kv_heads=2,
                               head_dim=8, causal=causal)
    lens = np.array([5, 0], np.int32)
    sinks = np.array([0.3, -1.2, 2.0, -0.1])
    out, _, _, lse = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, causal=causal,
                                    seq_lens=lens, sinks=sinks, window=w, return_lse=True)
    for b in range(2):
        for i in range(S):
            js = [j for j in range(S) if j < lens[b] and (not causal or j <= i) and j > i - w]
            for h in range(4):
                g = h // 2
                ref, ref_lse = _brute(c.q[b, i, h], [c.k[b, j, g] for j in js],
                                      [c.v[b, j, g] for j in js], c.gate[b, i, h], c.scale,
                                      float(sinks[h]))
                assert list(out[b, i, h]) == ref, (b, i, h)
                assert abs(lse[b, i, h] - ref_lse) <= 1e-14 * max(1.0, abs(ref_lse))


# --------------------------------------------------------------------------
# prefill rows == decode rows with the same visible keys
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("w", [0, 9])
def test_prefill_rows_match_decode(causal, w):
    """Each prefill row (b, i) equals a decode of q[b, i] over sequence b's
    keys: L = min(len, i + 1) under the causal mask (else len), and the window
    rebased onto that L.  Exercises the prefill visibility rules (key length,
    causal, window) against the decode ones, which the tests above pin."""
    S = 40
    c = workloads.make_prefill("pd", 2, S, seed=41, num_q_heads=4, num_kv_heads=2,
                               head_dim=32, causal=causal)
    lens = np.array([29, S], np.int32)
    sinks = np.array([0.5, -0.25, 1.0, 0.0])
    out, o, _, lse = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, causal=causal,
                                    seq_lens=lens, sinks=sinks, window=w, return_lse=True)
    for b in range(2):
        kp, vp, bt = _dense_pool(c.k[b], c.v[b])
        for i in range(S):
            L = min(int(lens[b]), i + 1) if causal else int(lens[b])
            lo = i - w + 1 if w > 0 else 0       # first key the window keeps
            wd = L - max(lo, 0)                  # keys left in [lo, L)
            if w > 0 and wd <= 0:
                assert not np.any(out[b, i]) and np.allclose(lse[b, i], sinks), (b, i)
                continue
            # keys [max(lo, 0), L): a decode window of wd keys ending at L - 1
            r = oracle.decode(c.q[b, i][None], c.gate[b, i][None], kp, vp, bt,
                              np.array([L], np.int32), c.scale, sinks=sinks,
                              window=(wd if w > 0 else 0), return_lse=True)
            assert np.array_equal(out[b, i], r[0][0]), (b, i)
            assert np.array_equal(o[b, i], r[1][0]), (b, i)
            assert np.array_equal(lse[b, i], r[3][0]), (b, i)


def test_prefill_key_lengths_hide_poisoned_keys_and_dead_rows_are_zero():
    c = workloads.make_prefill("pk", 3, 24, seed=42, num_q_heads=4, num_kv_heads=2,
                               head_dim=16, causal=True)
    lens = np.array([10, 0, 24], np.int32)
    base = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, True, seq_lens=lens,
                          return_lse=True)
    k2, v2 = c.k.copy(), c.v.copy()
    k2[0, 10:] = 0x7FC0
    v2[0, 10:] = 0x7FC0
    k2[1] = 0x7FC0
    v2[1] = 0x7FC0
    pois = oracle.prefill(c.q, c.gate, k2, v2, c.scale, True, seq_lens=lens, return_lse=True)
    for x, y in zip(base, pois):
        assert np.array_equal(x, y)
    assert not np.any(base[0][1]) and np.all(np.isneginf(base[3][1]))
    full = oracle.prefill(c.q, c.gate, c.k, c.v, c.scale, True, return_lse=True)
    assert np.array_equal(base[0][2], full[0][2])

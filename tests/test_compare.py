"""The tolerance checks of oracle.compare, on outputs built from the oracle's
own fp64 O with planted attention-output errors (no GPU)."""
import numpy as np

import oracle
import workloads
from oracle.compare import ETA, bf16_bits_to_f64, check_outputs


def _case():
    c = workloads.make_decode("cmp", [4096, 300, 0, 17], seed=7, max_pages_per_seq=256)
    ref, o, mref = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                 c.scale)
    return c, ref, o, mref, oracle.sigmoid_table()[c.gate]


def _gated(o_perturbed, sig_bits):
    ob = bf16_bits_to_f64(oracle.bf16_rne(o_perturbed))
    return oracle.bf16_rne(ob * bf16_bits_to_f64(sig_bits))


def test_oracle_output_passes_both_checks():
    _, ref, o, mref, sig = _case()
    res = check_outputs(ref, ref, o, mref, sig)
    assert res["ok"] and res["n_fail_model"] == 0 and res["n_bit_exact"] == ref.size


def test_error_inside_the_model_passes():
    """Every O moved by half the stated bound, alternating in sign."""
    _, ref, o, mref, sig = _case()
    sgn = np.where(np.arange(o.size).reshape(o.shape) % 2 == 0, 1.0, -1.0)
    got = _gated(o + sgn * 0.5 * ETA * mref, sig)
    res = check_outputs(got, ref, o, mref, sig)
    assert res["ok"], res


def test_error_past_the_model_fails_where_the_floored_rule_passes():
    """O moved by 4x the stated bound (2^-8 of Mref): within the floored rule
    (2 ulp of sigma_b Mref, i.e. up to 2^-6 Mref) on every element, but
    outside the model interval on many -- the check the floored rule lacks."""
    _, ref, o, mref, sig = _case()
    got = _gated(o + 4 * ETA * mref, sig)
    res = check_outputs(got, ref, o, mref, sig)
    assert res["n_fail_floor"] == 0
    assert res["n_fail_model"] > 1000
    assert not res["ok"]
    live = mref > 0
    assert res["n_fail_model"] <= int(np.count_nonzero(live))


def test_eta_none_is_the_floored_rule_alone():
    _, ref, o, mref, sig = _case()
    got = _gated(o + 4 * ETA * mref, sig)
    assert check_outputs(got, ref, o, mref, sig, eta=None)["ok"]

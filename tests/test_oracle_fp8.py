"""Pins for the oracle's FP8 (e4m3) KV path.

  * The e4m3 decoder against torch's float8_e4m3fn conversion, all 256 codes
    (an independent implementation of the OCP format).
  * FP8 decode == bf16 decode of the same values: e4m3 values times a power of
    two are exact in bf16, so the plain (already pinned) path on the re-encoded
    pools must give the same bits.
  * A non-power-of-two k factor equals folding it into the score scale, and a
    v factor equals scaling O (up to fp64 rounding order).
  * NaN codes in page tails and unused pages do not leak.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.compare import bf16_bits_to_f64


def test_e4m3_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 for 0x80
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def _as_bf16_pool(pool8, factor):
    """bf16 bits of factor * e4m3(code) (exact when factor is a power of two)."""
    vals = torch.from_numpy(pool8).view(torch.float8_e4m3fn).to(torch.float64) * factor
    t = vals.to(torch.float32)
    assert torch.equal(t.to(torch.float64), vals) or torch.isnan(vals).any()
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("factor", [1.0, 2.0 ** -6, 2.0 ** 3])
def test_fp8_decode_equals_bf16_decode_of_the_same_values(factor):
    c = workloads.make_decode("f8", [1, 33, 300, 0], seed=51, kv_dtype="fp8", kv_descale=factor,
                              poison=False)
    r8 = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                       k_descale=factor, v_descale=factor, return_lse=True)
    kb, vb = _as_bf16_pool(c.k_pool, factor), _as_bf16_pool(c.v_pool, factor)
    assert np.array_equal(bf16_bits_to_f64(kb),
                          torch.from_numpy(c.k_pool).view(torch.float8_e4m3fn).double()
                          .numpy() * factor)
    rb = oracle.decode(c.q, c.gate, kb, vb, c.block_table, c.seq_lens, c.scale, return_lse=True)
    for x, y in zip(r8, rb):
        assert np.array_equal(x, y)


def test_fp8_factors_fold_into_scale_and_output():
    """k factor kd: scores scale * q.(kd k) = (scale kd) * q.k; v factor vd:
    O = vd * O(codes).  Non-power-of-two factors, fp64 rounding order only."""
    kd, vd = 0.0137, 0.0291
    c = workloads.make_decode("f8s", [5, 200, 1000], seed=52, kv_dtype="fp8", poison=False)
    _, o, mref, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                    c.scale, k_descale=kd, v_descale=vd, return_lse=True)
    kb, vb = _as_bf16_pool(c.k_pool, 1.0), _as_bf16_pool(c.v_pool, 1.0)
    _, o1, mref1, lse1 = oracle.decode(c.q, c.gate, kb, vb, c.block_table, c.seq_lens,
                                       c.scale * kd, return_lse=True)
    # fp64 rounding of a sum is relative to the magnitude it was formed from
    assert np.all(np.abs(o - vd * o1) <= 1e-13 * vd * mref1)
    np.testing.assert_allclose(mref, vd * mref1, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse, lse1, rtol=1e-13)


def test_fp8_poisoned_tails_do_not_leak():
    c = workloads.make_decode("f8p", [7, 16, 17, 250], seed=53, kv_dtype="fp8", poison=True,
                              extra_pages=3)
    out, o, _ = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                              k_descale=c.k_descale, v_descale=c.v_descale)
    assert np.all(np.isfinite(o))
    assert np.any(c.k_pool == workloads.NAN_E4M3)

"""GPU parity of gated_attn_decode_fp8kv (e4m3 K / V pools) against the CPU
oracle's FP8 path.

The codes are decoded exactly on both sides (every e4m3 value is a bf16
value), the products q * k are exact in fp32 and the K factor only changes the
score scale, so the arithmetic and its error are those of the bf16 decode: the
same floored two-ulp rule applies.  With power-of-two factors and a single key
the result is exact and must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, to_dev, to_np
from oracle.compare import check_outputs

import gated_gqa_decode_amd as ga

pytestmark = pytest.mark.gpu


def _run(c, **opts):
    sk = opts.pop("sinks", None)
    sinks_t = None if sk is None else torch.tensor(sk, dtype=torch.float32, device=DEV)
    out, lse = ga.decode(to_dev(c.q), to_dev(c.gate), to_dev(c.k_pool), to_dev(c.v_pool),
                         to_dev(c.block_table), to_dev(c.seq_lens), c.scale,
                         k_descale=c.k_descale, v_descale=c.v_descale, sinks=sinks_t,
                         return_lse=True, **opts)
    torch.cuda.synchronize()
    return to_np(out), to_np(lse)


def _parity(c, **opts):
    got, got_lse = _run(c, **dict(opts))
    ref, o, mref, lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                                      c.seq_lens, c.scale, k_descale=c.k_descale,
                                      v_descale=c.v_descale, return_lse=True, **opts)
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] {c.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.all(np.abs(got_lse[fin] - lse[fin]) <= 2e-4 + 1e-6 * np.abs(lse[fin]))
    return res


def test_fp8_full_size_b64_l4096():
    c = workloads.make_decode("decode_b64_l4096_fp8", [4096] * 64, seed=2, kv_dtype="fp8",
                              max_pages_per_seq=256)
    _parity(c)


def test_fp8_serving_shape_b224():
    c = workloads.make_decode("decode_b224_fp8", workloads.config3_lengths(), seed=3,
                              kv_dtype="fp8", max_pages_per_seq=384)
    _parity(c)


def test_fp8_ragged_poisoned():
    lens = [1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 257, 640, 0]
    c = workloads.make_decode("fp8_ragged", lens, seed=61, kv_dtype="fp8",
                              max_pages_per_seq=48, extra_pages=5)
    _parity(c)


@pytest.mark.parametrize("descale", [2.0 ** -6, 0.0093])
def test_fp8_factors(descale):
    c = workloads.make_decode("fp8_f", [100, 3000], seed=62, kv_dtype="fp8", kv_descale=descale,
                              max_pages_per_seq=200)
    _parity(c)


def test_fp8_options_and_groups():
    for hq in (16, 32, 6):
        c = workloads.make_decode(f"fp8_opt_{hq}", [2000, 9, 0, 700], seed=63 + hq,
                                  num_q_heads=hq, num_kv_heads=2, kv_dtype="fp8",
                                  max_pages_per_seq=160)
        sinks = np.linspace(-1.0, 1.0, hq).astype(np.float32).astype(np.float64)
        _parity(c, sinks=sinks, window=333)


def test_fp8_single_key_is_bit_exact():
    c = workloads.make_decode("fp8_L1", [1] * 24, seed=64, kv_dtype="fp8", kv_descale=2.0 ** -4)
    got, _ = _run(c)
    ref, _, _ = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                              c.scale, k_descale=c.k_descale, v_descale=c.v_descale)
    assert np.array_equal(got, ref)


def test_page_size_one_block_table():
    """e4m3 pools at page size 1: every token its own pool row at a shuffled
    slot (spare slots NaN codes), the block table holding token slots.  Within
    the rule against the oracle on that layout, and bit-identical to the same
    tokens in 16-token pages (the two layouts get the same split plan here)."""
    lens = [700, 1, 33, 0, 2049, 16]
    c = workloads.make_decode("fp8_tok", lens, seed=142, kv_dtype="fp8", max_pages_per_seq=160)
    k1, v1, _, _, table = workloads.csr_layout(c, seed=143)
    c1 = workloads.DecodeCase(c.name + "_p1", c.q, c.gate, k1, v1, table, c.seq_lens, c.scale,
                              c.k_descale, c.v_descale)
    p16 = ga.decode_plan(ga.decode_dims(**c.dims))
    p1 = ga.decode_plan(ga.decode_dims(**c1.dims))
    assert p1.tokens_per_split == p16.tokens_per_split
    got, _ = _run(c1)
    _parity(c1)
    paged, _ = _run(c)
    assert np.array_equal(got, paged)


def test_csr_indexing():
    """gated_attn_decode_fp8kv_csr: the same tokens addressed by CSR row
    pointers and indices.  Within the rule against the oracle and bit-identical
    to the page-size-1 block table over the same slots."""
    c = workloads.make_decode("fp8_csr", [700, 1, 33, 0, 2049, 16], seed=144, kv_dtype="fp8",
                              max_pages_per_seq=160)
    k1, v1, indptr, idx, table = workloads.csr_layout(c, seed=145)
    c1 = workloads.DecodeCase(c.name + "_p1", c.q, c.gate, k1, v1, table, c.seq_lens, c.scale,
                              c.k_descale, c.v_descale)
    out = ga.decode_csr(to_dev(c.q), to_dev(c.gate), to_dev(k1), to_dev(v1), to_dev(indptr),
                        to_dev(idx), c.scale, max_seq_len=table.shape[1],
                        k_descale=c.k_descale, v_descale=c.v_descale)
    torch.cuda.synchronize()
    got = to_np(out)
    ref, o, mref = oracle.decode(c1.q, c1.gate, c1.k_pool, c1.v_pool, c1.block_table,
                                 c1.seq_lens, c1.scale, k_descale=c1.k_descale,
                                 v_descale=c1.v_descale)
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] {c.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    assert np.array_equal(got, _run(c1)[0])

"""GPU parity of the attention-spec options (gated_attn_decode_ex /
gated_attn_prefill_ex): sliding window, sinks, the lse output and prefill key
lengths, against the CPU oracle.

out: the floored two-ulp rule of oracle/compare.py, as for plain attention.
lse (fp32 on the GPU, fp64 in the oracle): the GPU forms each score as an fp32
sum of 256 exact bf16 products (error at most 256 * 2^-24 * scale * sum|q_d k_d|,
about 1.5e-4 for N(0, 1) data at scale 1/16, typically 1e-5), then the log of
an fp32 sum of positive terms (relative error a few 2^-24 per term) and one
fp32 multiply by ln 2.  The bound below, 2e-4 + 1e-6 |lse|, covers that worst
case; a dropped split, a missing sink term or a wrong log base is off by 1e-2
or more.
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


def _check_lse(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{name}: -inf rows differ"
    err = np.abs(got[~ninf] - ref[~ninf])
    tol = 2e-4 + 1e-6 * np.abs(ref[~ninf])
    worst = float(err.max()) if err.size else 0.0
    print(f"[lse] {name}: n={err.size} max_abs_err={worst:.3e}", flush=True)
    assert np.all(err <= tol), f"{name}: lse error {worst}"


def _decode_case_parity(c, sinks=None, window=0):
    sk = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device=DEV)
    out, lse = ga.decode(to_dev(c.q), to_dev(c.gate), to_dev(c.k_pool), to_dev(c.v_pool),
                         to_dev(c.block_table), to_dev(c.seq_lens), c.scale, sinks=sk,
                         window=window, return_lse=True)
    torch.cuda.synchronize()
    got = to_np(out)
    ref, o, mref, ref_lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                                          c.seq_lens, c.scale, sinks=sinks, window=window,
                                          return_lse=True)
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] {c.name} window={window} sinks={sinks is not None}: n={res['n']} "
          f"bit-exact={res['n_bit_exact']} max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    _check_lse(to_np(lse), ref_lse, c.name)


@pytest.mark.parametrize("window", [0, 1, 7, 16, 100, 1000, 2049])
@pytest.mark.parametrize("with_sinks", [False, True])
def test_decode_window_sinks_lse(window, with_sinks):
    """Windows below, at and across step (8), page (16) and split boundaries,
    over ragged lengths (0 = padded slot) and a long row spanning splits."""
    lens = [1, 5, 16, 17, 300, 0, 2050, 4096]
    c = workloads.make_decode("spec", lens, seed=90 + window, max_pages_per_seq=256)
    sinks = None
    if with_sinks:
        sinks = np.random.default_rng(window).normal(0.0, 2.0, size=c.q.shape[1])
        sinks = sinks.astype(np.float32).astype(np.float64)  # the values the GPU gets
    _decode_case_parity(c, sinks, window)


def test_decode_sinks_dominating_and_negligible():
    """Sinks far above every score (O -> 0 but not underflowing to a wrong
    value) and far below (no effect)."""
    c = workloads.make_decode("sink_ext", [40, 3000], seed=95, max_pages_per_seq=256)
    Hq = c.q.shape[1]
    sinks = np.where(np.arange(Hq) % 2 == 0, 40.0, -60.0)
    _decode_case_parity(c, sinks, 0)


def test_decode_options_group16_and_group6():
    for hq in (32, 12):
        c = workloads.make_decode(f"spec_hq{hq}", [2000, 9, 0, 700], seed=96 + hq,
                                  num_q_heads=hq, num_kv_heads=2, max_pages_per_seq=160)
        sinks = np.linspace(-1.0, 1.0, hq).astype(np.float32).astype(np.float64)
        _decode_case_parity(c, sinks, 333)


def test_decode_options_full_size():
    """B = 64, L = 4096 with a 1000-token window, sinks and lse."""
    c = workloads.make_decode("decode_b64_l4096_spec", [4096] * 64, seed=97,
                              max_pages_per_seq=256)
    sinks = np.full(16, 0.5)
    _decode_case_parity(c, sinks, 1000)


def test_decode_plain_entry_matches_ex_with_zero_options():
    c = workloads.make_decode("plain_vs_ex", [700, 33, 0], seed=98, max_pages_per_seq=64)
    args = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
    a = to_np(ga.decode(*args, c.scale))
    b, _ = ga.decode(*args, c.scale, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(a, to_np(b))


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------
def _prefill_parity(p, kv_lens=None, sinks=None, window=0, rows=None):
    kl = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    sk = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device=DEV)
    # outputs poisoned with NaN first: an element the kernel never writes fails
    out = torch.full(p.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(p.q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    ga.prefill(to_dev(p.q), to_dev(p.gate), to_dev(p.k), to_dev(p.v), p.scale,
               causal=p.causal, kv_lens=kl, sinks=sk, window=window, out=out, lse=lse)
    torch.cuda.synchronize()
    got, got_lse = to_np(out), to_np(lse)
    ref, o, mref, ref_lse = oracle.prefill(p.q, p.gate, p.k, p.v, p.scale, causal=p.causal,
                                           rows=rows, seq_lens=kv_lens, sinks=sinks,
                                           window=window, return_lse=True)
    gate = p.gate
    if rows is not None:
        got, got_lse = got[rows[:, 0], rows[:, 1]], got_lse[rows[:, 0], rows[:, 1]]
        gate = p.gate[rows[:, 0], rows[:, 1]]
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[gate])
    print(f"[parity] {p.name} lens={kv_lens} window={window} sinks={sinks is not None}: "
          f"n={res['n']} bit-exact={res['n_bit_exact']} max_ulp_floor={res['max_ulp_floor']:.4f} "
          f"strict_fail={res['n_fail_strict']} model_fail={res['n_fail_model']}", flush=True)
    assert res["ok"], res
    _check_lse(got_lse, ref_lse, p.name)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [0, 1, 50, 64, 130])
def test_prefill_lengths_window_sinks_lse(causal, window):
    p = workloads.make_prefill("pspec", 4, 200, seed=110 + window, causal=causal)
    lens = [200, 150, 0, 37]
    sinks = np.random.default_rng(window).normal(0.0, 1.5, size=16)
    sinks = sinks.astype(np.float32).astype(np.float64)
    _prefill_parity(p, lens, sinks, window)


def test_prefill_options_groups():
    for hq, hkv in ((32, 2), (6, 3)):
        p = workloads.make_prefill(f"pspec_{hq}_{hkv}", 2, 130, seed=120 + hq, causal=True,
                                   num_q_heads=hq, num_kv_heads=hkv)
        _prefill_parity(p, [130, 77], np.linspace(-2.0, 2.0, hq).astype(np.float32)
                        .astype(np.float64), 40)


def test_prefill_options_full_size_every_element():
    """B = 2, S = 2048 causal with key lengths (2048, 1500), a 512-key window,
    sinks and lse, in the benchmark's launch configuration: every one of the
    16.8 M outputs and 65,536 lse values against the oracle, out and lse
    NaN-poisoned before the call."""
    p = workloads.workload(4)
    _prefill_parity(p, [2048, 1500], np.full(16, -0.5), 512)

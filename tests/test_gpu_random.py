"""Seeded random shapes and options through the C-ABI against the CPU oracle.

Each case draws its own GQA geometry (groups 1..16 over 1..8 kv heads),
batch, ragged lengths (dead rows included), block-table capacity, sliding
window and sinks from a fixed seed, so a failure names a case that replays
exactly.  Pass criterion: the floored two-ulp rule of oracle/compare.py on
every output element and the lse bound of test_gpu_spec.py.
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

GEOMETRIES = [(16, 2), (8, 1), (6, 3), (4, 2), (3, 1), (2, 2), (1, 1), (7, 1), (12, 2),
              (32, 2), (10, 1), (40, 8), (5, 5), (14, 1), (9, 1), (26, 2), (33, 3), (15, 1)]


def _lse_ok(got, ref, name):
    got = np.asarray(got, dtype=np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{name}: -inf rows differ"
    err = np.abs(got[~ninf] - ref[~ninf])
    assert np.all(err <= 2e-4 + 1e-6 * np.abs(ref[~ninf])), f"{name}: lse error {err.max()}"


def _decode_case(seed):
    rng = np.random.default_rng(1000 + seed)
    hq, hkv = GEOMETRIES[int(rng.integers(len(GEOMETRIES)))]
    batch = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 3000, size=batch)]
    if rng.random() < 0.5:
        lens[int(rng.integers(batch))] = 0  # a dead row
    if rng.random() < 0.3:
        lens[int(rng.integers(batch))] = int(rng.integers(1, 17))  # within one page
    need = max(1, (max(lens) + 15) // 16)
    cap = need + int(rng.integers(0, 3 * need + 1))  # capacity at or above the longest
    window = int(rng.integers(1, 2500)) if rng.random() < 0.5 else 0
    sinks = (rng.normal(0.0, 2.0, size=hq).astype(np.float32).astype(np.float64)
             if rng.random() < 0.5 else None)
    c = workloads.make_decode(f"rand{seed}_{hq}_{hkv}", lens, seed=2000 + seed, num_q_heads=hq,
                              num_kv_heads=hkv, max_pages_per_seq=cap,
                              extra_pages=int(rng.integers(0, 9)))
    return c, window, sinks


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    c, window, sinks = _decode_case(seed)
    print(f"[case] {c.name} lens={c.seq_lens.tolist()} cap={c.block_table.shape[1]} "
          f"window={window} sinks={sinks is not None}", flush=True)
    sk = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device=DEV)
    out, lse = ga.decode(to_dev(c.q), to_dev(c.gate), to_dev(c.k_pool), to_dev(c.v_pool),
                         to_dev(c.block_table), to_dev(c.seq_lens), c.scale, sinks=sk,
                         window=window, return_lse=True)
    torch.cuda.synchronize()
    ref, o, mref, ref_lse = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                                          c.seq_lens, c.scale, sinks=sinks, window=window,
                                          return_lse=True)
    res = check_outputs(to_np(out), ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] {c.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    _lse_ok(to_np(lse), ref_lse, c.name)


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill(seed):
    rng = np.random.default_rng(3000 + seed)
    hq, hkv = GEOMETRIES[int(rng.integers(len(GEOMETRIES)))]
    batch = int(rng.integers(1, 3))
    S = int(rng.integers(1, 400))
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, S + 40)) if rng.random() < 0.4 else 0
    kv_lens = [int(x) for x in rng.integers(0, S + 1, size=batch)] if rng.random() < 0.4 else None
    sinks = (rng.normal(0.0, 2.0, size=hq).astype(np.float32).astype(np.float64)
             if rng.random() < 0.4 else None)
    p = workloads.make_prefill(f"prand{seed}_{hq}_{hkv}", batch, S, seed=4000 + seed,
                               num_q_heads=hq, num_kv_heads=hkv, causal=causal)
    print(f"[case] {p.name} B={batch} S={S} causal={causal} window={window} "
          f"kv_lens={kv_lens} sinks={sinks is not None}", flush=True)
    kl = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    sk = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device=DEV)
    out, lse = ga.prefill(to_dev(p.q), to_dev(p.gate), to_dev(p.k), to_dev(p.v), p.scale,
                          causal=causal, kv_lens=kl, sinks=sk, window=window, return_lse=True)
    torch.cuda.synchronize()
    ref, o, mref, ref_lse = oracle.prefill(p.q, p.gate, p.k, p.v, p.scale, causal=causal,
                                           seq_lens=kv_lens, sinks=sinks, window=window,
                                           return_lse=True)
    res = check_outputs(to_np(out), ref, o, mref, oracle.sigmoid_table()[p.gate])
    print(f"[parity] {p.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    _lse_ok(to_np(lse), ref_lse, p.name)

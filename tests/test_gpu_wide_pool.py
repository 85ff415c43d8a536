"""Page-size-1 decode over pools whose rows span more than 4 GiB.

At page size 1 stage 1 addresses a token's row by a 32-bit byte offset from
the pool's start; a pool larger than that takes the 64-bit address form, which
the library selects from num_pages alone.  These tests build real pools of
4.25 GiB each on the device (bf16 and e4m3), place a small workload's tokens at
seeded rows spread over the whole pool -- some forced just below and just past
the 4 GiB offset and at the last row -- and compare against the oracle on the
same tokens in a compact pool.  The same tokens in a compact device pool (the
32-bit form) must give the identical bits.
"""
import numpy as np
import pytest
import torch

import gated_gqa_decode_amd as ga
import oracle
import workloads
from gpu_helpers import DEV, to_dev, to_np
from oracle.compare import check_outputs

pytestmark = pytest.mark.gpu

LENS = [700, 1, 33, 0, 2049, 16]
FOUR_GIB = 1 << 32


def _big_rows(n_small: int, n_big: int, row_bytes: int, seed: int) -> np.ndarray:
    """Distinct big-pool rows for the compact rows 0..n_small-1: seeded, spread
    over [0, n_big), with rows at the 4 GiB seam and the last row included."""
    seam = FOUR_GIB // row_bytes
    forced = np.array([seam - 1, seam, seam + 1, n_big - 1, 0], dtype=np.int64)
    rng = np.random.default_rng(seed)
    rest = rng.choice(n_big - 1, size=n_small + len(forced), replace=False).astype(np.int64)
    rest = rest[~np.isin(rest, forced)][: n_small - len(forced)]
    rows = np.concatenate([forced, rest])
    rng.shuffle(rows)
    assert len(np.unique(rows)) == n_small and rows.max() < n_big
    return rows


def _run_case(kv_dtype: str, use_csr: bool, seed: int):
    c = workloads.make_decode(f"wide_{kv_dtype}", LENS, seed=seed, kv_dtype=kv_dtype,
                              max_pages_per_seq=160)
    k1, v1, indptr, idx, table = workloads.csr_layout(c, seed=seed + 1)
    n_small, _, hkv, d = k1.shape
    row_bytes = hkv * d * k1.dtype.itemsize
    n_big = FOUR_GIB // row_bytes + FOUR_GIB // row_bytes // 16  # 4.25 GiB per pool
    assert n_big * row_bytes > FOUR_GIB
    rows = _big_rows(n_small, n_big, row_bytes, seed + 2)
    tdtype = torch.uint8 if c.fp8 else torch.bfloat16

    def big_pool(small):
        pool = torch.empty((n_big, 1, hkv, d), dtype=tdtype, device=DEV)
        pool[torch.from_numpy(rows).to(DEV)] = to_dev(small).view(tdtype)
        return pool

    kb, vb = big_pool(k1), big_pool(v1)
    big_table = np.where(table >= 0, rows[np.maximum(table, 0)], -1).astype(np.int32)
    big_idx = rows[idx].astype(np.int32)
    fp8 = dict(k_descale=c.k_descale, v_descale=c.v_descale) if c.fp8 else {}
    q, gate = to_dev(c.q), to_dev(c.gate)
    if use_csr:
        out = ga.decode_csr(q, gate, kb, vb, to_dev(indptr), to_dev(big_idx), c.scale,
                            max_seq_len=table.shape[1], **fp8)
        small = ga.decode_csr(q, gate, to_dev(k1).view(tdtype), to_dev(v1).view(tdtype),
                              to_dev(indptr), to_dev(idx), c.scale,
                              max_seq_len=table.shape[1], **fp8)
    else:
        out = ga.decode(q, gate, kb, vb, to_dev(big_table), to_dev(c.seq_lens), c.scale, **fp8)
        small = ga.decode(q, gate, to_dev(k1).view(tdtype), to_dev(v1).view(tdtype),
                          to_dev(table), to_dev(c.seq_lens), c.scale, **fp8)
    torch.cuda.synchronize()
    got, got_small = to_np(out), to_np(small)
    del kb, vb
    torch.cuda.empty_cache()
    kw = dict(k_descale=c.k_descale, v_descale=c.v_descale) if c.fp8 else {}
    ref, o, mref = oracle.decode(c.q, c.gate, k1, v1, table, c.seq_lens, c.scale, **kw)
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] wide pool {kv_dtype} csr={use_csr}: n={res['n']} "
          f"bit-exact={res['n_bit_exact']} max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res
    assert np.array_equal(got, got_small), "64-bit and 32-bit copy forms differ"


@pytest.mark.parametrize("use_csr", [False, True])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_pool_rows_past_4gib(kv_dtype, use_csr):
    _run_case(kv_dtype, use_csr, seed=170 + 2 * int(use_csr) + (10 if kv_dtype == "fp8" else 0))

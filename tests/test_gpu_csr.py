"""GPU parity of decode at page size 1: CSR indexing (gated_attn_decode_csr)
and a page-size-1 block table (gated_attn_decode with page_size 1), against
the oracle on the equivalent token table.  Same floored two-ulp rule; the
layout must not change a single bit relative to 16-token pages."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, gpu_decode, to_dev, to_np
from oracle.compare import check_outputs

import gated_gqa_decode_amd as ga

pytestmark = pytest.mark.gpu


def _csr_gpu(c, k1, v1, indptr, idx, **kw):
    cap = c.block_table.shape[1] * c.k_pool.shape[1]
    r = ga.decode_csr(to_dev(c.q), to_dev(c.gate), to_dev(k1), to_dev(v1), to_dev(indptr),
                      to_dev(idx), c.scale, max_seq_len=cap, **kw)
    torch.cuda.synchronize()
    return r


def _parity(c, got, table, k1, v1, **kw):
    ref, o, mref = oracle.decode(c.q, c.gate, k1, v1, table, c.seq_lens, c.scale, **kw)
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
    print(f"[parity] {c.name} (page size 1): n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res


@pytest.mark.parametrize("lens,cap", [([512], 512), ([512, 495, 478, 461], 512),
                                      ([1, 2, 7, 8, 9, 15, 16, 17, 300, 0, 1000], 1024),
                                      ([4096] * 64, 4096)])
def test_csr_parity(lens, cap):
    c = workloads.make_decode(f"csr_{len(lens)}x{max(lens)}", lens, seed=82 + len(lens),
                              max_pages_per_seq=cap // 16)
    k1, v1, indptr, idx, table = workloads.csr_layout(c, seed=len(lens))
    got = to_np(_csr_gpu(c, k1, v1, indptr, idx))
    _parity(c, got, table, k1, v1)
    # the same tokens in 16-token pages: identical bits
    assert np.array_equal(got, gpu_decode(c))


def test_page_size_one_block_table():
    c = workloads.make_decode("tok_table", [700, 33, 0, 2049], seed=90, max_pages_per_seq=160)
    k1, v1, _, _, table = workloads.csr_layout(c, seed=9)
    got = to_np(ga.decode(to_dev(c.q), to_dev(c.gate), to_dev(k1), to_dev(v1), to_dev(table),
                          to_dev(c.seq_lens), c.scale))
    torch.cuda.synchronize()
    _parity(c, got, table, k1, v1)


def test_csr_with_options():
    c = workloads.make_decode("csr_opts", [3000, 5, 0, 640], seed=91, max_pages_per_seq=192)
    k1, v1, indptr, idx, table = workloads.csr_layout(c, seed=10)
    sinks = np.linspace(-1.5, 1.5, 16).astype(np.float32).astype(np.float64)
    out, lse = _csr_gpu(c, k1, v1, indptr, idx,
                        sinks=torch.tensor(sinks, dtype=torch.float32, device=DEV), window=777,
                        return_lse=True)
    _parity(c, to_np(out), table, k1, v1, sinks=sinks, window=777)
    ref_lse = oracle.decode(c.q, c.gate, k1, v1, table, c.seq_lens, c.scale, sinks=sinks,
                            window=777, return_lse=True)[3]
    g = to_np(lse).astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.all(np.abs(g[fin] - ref_lse[fin]) <= 2e-4 + 1e-6 * np.abs(ref_lse[fin]))

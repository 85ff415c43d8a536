"""Pin for the oracle at page size 1 (the CSR serving layout): the same
tokens laid out one per pool row at shuffled slots give the same bits as the
16-token pages, with and without window, sinks and lse."""
import numpy as np

import oracle
import workloads


def test_page_size_one_equals_sixteen_token_pages():
    c = workloads.make_decode("p1", [1, 16, 17, 300, 0, 77], seed=81, extra_pages=2)
    k1, v1, indptr, idx, table = workloads.csr_layout(c, seed=81)
    assert np.array_equal(np.diff(indptr), np.clip(c.seq_lens, 0, None))
    for kw in ({}, dict(window=20, sinks=np.linspace(-1, 1, 16), return_lse=True)):
        a = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                          **kw)
        b = oracle.decode(c.q, c.gate, k1, v1, table, c.seq_lens, c.scale, **kw)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    # the CSR rows are the table's rows
    for bb in range(len(c.seq_lens)):
        n = indptr[bb + 1] - indptr[bb]
        assert np.array_equal(idx[indptr[bb]:indptr[bb + 1]], table[bb, :n])

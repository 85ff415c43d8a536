"""Calls in flight together on separate streams do not interfere.

The decode and prefill entry points keep no state of their own between calls
(the cuDNN "Gated Attention Block" page, Forward: one caller-owned workspace,
nothing allocated by the library): each call reads only its arguments and
writes only its outputs and its workspace.  Several calls enqueued on three
streams without synchronisation between them must each give the bits of the
same call made alone.
"""
import numpy as np
import pytest
import torch

import gated_gqa_decode_amd as ga
import workloads
from gpu_helpers import DEV, to_dev, to_np

pytestmark = pytest.mark.gpu


def _decode_case(name, lens, seed):
    c = workloads.make_decode(name, lens, seed=seed, max_pages_per_seq=96)
    args = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
    dims = ga.decode_dims_for(args[0], args[2], args[4])
    ws = torch.empty(ga.decode_workspace_size(dims), dtype=torch.uint8, device=DEV)
    return c, args, ws


def test_concurrent_streams_match_serial_calls():
    ca, aa, wa = _decode_case("streams_a", [1500, 3, 0, 700, 1536, 64], seed=91)
    cb, ab, wb = _decode_case("streams_b", [1, 1200, 511, 1536], seed=92)
    p = workloads.make_prefill("streams_p", 2, 300, seed=93, causal=True)
    pa = [to_dev(x) for x in (p.q, p.gate, p.k, p.v)]

    # each call alone, in order, with a synchronisation after each
    ref_a = to_np(ga.decode(*aa, ca.scale, workspace=wa))
    torch.cuda.synchronize()
    ref_b = to_np(ga.decode(*ab, cb.scale, workspace=wb))
    torch.cuda.synchronize()
    ref_p = to_np(ga.prefill(*pa, p.scale, causal=True))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in range(3)]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs_a = [torch.empty_like(aa[0]) for _ in range(4)]
    outs_b = [torch.empty_like(ab[0]) for _ in range(4)]
    outs_p = [torch.empty_like(pa[0]) for _ in range(4)]
    # the workspaces are per stream: calls on one stream run in order, so
    # they may share it; the other stream has its own
    for it in range(4):
        with torch.cuda.stream(streams[0]):
            ga.decode(*aa, ca.scale, out=outs_a[it], workspace=wa)
        with torch.cuda.stream(streams[1]):
            ga.decode(*ab, cb.scale, out=outs_b[it], workspace=wb)
        with torch.cuda.stream(streams[2]):
            ga.prefill(*pa, p.scale, causal=True, out=outs_p[it])
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for it in range(4):
        assert np.array_equal(to_np(outs_a[it]), ref_a), ("decode a", it)
        assert np.array_equal(to_np(outs_b[it]), ref_b), ("decode b", it)
        assert np.array_equal(to_np(outs_p[it]), ref_p), ("prefill", it)

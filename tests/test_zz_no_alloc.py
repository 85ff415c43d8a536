"""gated_attn_decode_noalloc (the decode entry point that allocates nothing
and takes no workspace) through the C ABI, against gated_attn_decode with a
caller-owned workspace: two calls in a row, the second on a smaller input
(stale partials of the first stay in the library's scratch array), each
bit-identical to the workspace entry point and within the rule against the
oracle."""
import ctypes

import numpy as np
import pytest
import torch

import gated_gqa_decode_amd as ga
import oracle
import workloads
from gpu_helpers import DEV, to_dev, to_np
from oracle.compare import check_outputs

pytestmark = pytest.mark.gpu


def _noalloc(c, tensors, out):
    q, gate, kp, vp, bt, sl = tensors
    dims = ga.decode_dims(**c.dims)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return ga.lib.gated_attn_decode_noalloc(q.data_ptr(), gate.data_ptr(), kp.data_ptr(),
                                            vp.data_ptr(), bt.data_ptr(), sl.data_ptr(),
                                            ctypes.c_float(c.scale), out.data_ptr(), stream,
                                            ctypes.byref(dims))


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # B=64 L=4096 (2 MiB of partials), then B=4 ragged L 512..461 (smaller)
    for c in (workloads.workload(2), workloads.workload(1)):
        t = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
        ref_gpu = to_np(ga.decode(*t, c.scale))
        out = torch.full(c.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        st = _noalloc(c, t, out)
        assert st == ga.GA_OK, ga.lib.gated_attn_status_string(st)
        torch.cuda.synchronize()
        got = to_np(out)
        print(f"[noalloc] {c.name}: identical={np.array_equal(got, ref_gpu)}", flush=True)
        assert np.array_equal(got, ref_gpu)
        ref, o, mref = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table,
                                     c.seq_lens, c.scale)
        res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[c.gate])
        assert res["ok"], res


def test_noalloc_declines_partials_past_its_scratch():
    """B = 4096 at a 4,096-token capacity needs 64 MiB of partials: declined
    with GA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued."""
    c = workloads.make_decode("noalloc_big", [16] * 4096, seed=3, max_pages_per_seq=256)
    assert ga.decode_workspace_size(ga.decode_dims(**c.dims)) > (16 << 20)
    t = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
    out = torch.full(c.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    assert _noalloc(c, t, out) == ga.GA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert np.all(np.isnan(out.float().cpu().numpy()))

"""GPU parity of gated_attn_decode against the CPU oracle (gfx950 only).

Pass criterion (the floored two-ulp rule in oracle/compare.py) on every
element; where the computation is exact by construction (a single key,
identical K and V rows, the gate epilogue given the same bf16 O) the GPU must
match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, decode_parity, gpu_decode, to_dev, to_np
from oracle.compare import check_outputs

import gated_gqa_decode_amd as ga

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [0, 1, 2, 3])
def test_workload_parity(wl):
    """The four decode workloads at full size, every output element."""
    c = workloads.workload(wl)
    res = decode_parity(c)
    assert res["ok"], res
    if wl == 3:
        pad = c.seq_lens <= 0
        assert pad.sum() == 11


@pytest.mark.parametrize("Hq,Hkv", [(32, 2), (24, 2), (20, 2), (12, 2), (14, 2), (8, 2),
                                     (2, 2), (7, 1), (6, 3), (40, 8), (3, 1), (16, 1),
                                     (9, 1), (22, 2), (15, 1), (39, 3)])
def test_gqa_group_sizes(Hq, Hkv):
    """Groups 1..16 (idle MFMA columns past the group), over ragged lengths,
    several splits and a dead row."""
    lens = [700, 1, 2049, 0, 64, 333]
    c = workloads.make_decode(f"gqa_{Hq}_{Hkv}", lens, seed=70 + Hq + Hkv, num_q_heads=Hq,
                              num_kv_heads=Hkv, max_pages_per_seq=160)
    res = decode_parity(c)
    assert res["ok"], res


def test_group16_full_size():
    """H_q = 32, H_kv = 2 at B = 64, L = 4096, every output element."""
    c = workloads.make_decode("decode_b64_l4096_hq32", [4096] * 64, seed=72, num_q_heads=32,
                              num_kv_heads=2, max_pages_per_seq=256)
    res = decode_parity(c)
    assert res["ok"], res


def test_ragged_lengths_across_steps_pages_and_splits():
    lens = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 513, 640]
    c = workloads.make_decode("ragged", lens, seed=31, max_pages_per_seq=48, extra_pages=7)
    res = decode_parity(c)
    assert res["ok"], res


def test_long_sequences_largest_split():
    """Capacity 32768 tokens at batch 64 gives the largest split (16,384
    tokens: each wave copies 128 tiles, so its page ids fill both per-lane
    registers); the short sequences run as few splits of their own size."""
    lens = [32768, 1, 1025, 32767, 0, 4096] + [17] * 58
    c = workloads.make_decode("long", lens, seed=32, max_pages_per_seq=2048)
    plan = ga.decode_plan(ga.decode_dims(**c.dims))
    assert (plan.tokens_per_split, plan.num_splits) == (16384, 2)
    res = decode_parity(c)
    assert res["ok"], res


def test_long_sequences_many_pairs():
    """256 (sequence, kv head) pairs in a capacity of 32,768 tokens: splits of
    4,096 tokens (8 per sequence); long, page-ragged and short sequences, so
    most of the short sequences' splits are empty."""
    lens = [32768, 1, 4097, 32767, 0, 8192] + [17] * 122
    c = workloads.make_decode("long_many", lens, seed=46, max_pages_per_seq=2048)
    plan = ga.decode_plan(ga.decode_dims(**c.dims))
    assert (plan.tokens_per_split, plan.num_splits) == (4096, 8)
    res = decode_parity(c)
    assert res["ok"], res


def test_batch_past_65535_sampled_sequences():
    """70,000 sequences (past a 16-bit grid dimension: 140,000 stage-1
    workgroups and 1.12 M stage-2 rows) with ragged lengths 0..48 in a
    three-page capacity, pages shuffled over the pool.  Inputs are seeded
    draws on the device (torch's generator).  The NaN-poisoned output must be
    written everywhere, padded slots must be +0, and sampled sequences -- the
    first and last ones, the ones around index 65,535 and random ones -- match
    the oracle on their inputs copied back."""
    B, Hq, Hkv, D, W = 70000, 16, 2, 256, 3
    P = B * W + 5
    gen = torch.Generator(device=DEV)
    gen.manual_seed(65536)

    def draw(shape, std):
        return (torch.randn(shape, generator=gen, device=DEV) * std).to(torch.bfloat16)

    q = draw((B, Hq, D), 1.0)
    gate = draw((B, Hq, D), 2.0)
    k_pool = torch.empty((P, 16, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.empty_like(k_pool)
    for lo in range(0, P, 16384):  # fp32 temporaries stay small
        hi = min(P, lo + 16384)
        k_pool[lo:hi] = draw((hi - lo, 16, Hkv, D), 1.0)
        v_pool[lo:hi] = draw((hi - lo, 16, Hkv, D), 1.0)
    perm = torch.randperm(P, generator=gen, device=DEV)
    block_table = perm[:B * W].view(B, W).to(torch.int32).contiguous()
    lens = torch.randint(0, W * 16 + 1, (B,), generator=gen, device=DEV, dtype=torch.int32)
    for i, n in ((0, 0), (1, 1), (2, 48), (65534, 16), (65535, 17), (65536, 0), (B - 2, 0),
                 (B - 1, 48)):
        lens[i] = n
    out = torch.full_like(q, float("nan"))
    ga.decode(q, gate, k_pool, v_pool, block_table, lens, 1.0 / 16, out=out)
    torch.cuda.synchronize()
    bits = out.view(torch.int16)
    assert not bool(((bits & 0x7F80) == 0x7F80).any()), "non-finite (unwritten?) output"
    dead = lens <= 0
    assert int(dead.sum()) > 0 and not bool(bits[dead].any()), "padded slot not +0"

    rng = np.random.default_rng(65536)
    idx = sorted(set(range(24)) | set(range(65520, 65552)) | set(range(B - 24, B))
                 | set(int(x) for x in rng.integers(0, B, 96)))
    sel = torch.tensor(idx, device=DEV)
    pages = block_table[sel].reshape(-1).long()
    c_q, c_gate = to_np(q[sel]), to_np(gate[sel])
    c_k, c_v = to_np(k_pool[pages]), to_np(v_pool[pages])
    c_bt = np.arange(len(idx) * W, dtype=np.int32).reshape(len(idx), W)
    c_lens = to_np(lens[sel])
    ref, o, mref = oracle.decode(c_q, c_gate, c_k, c_v, c_bt, c_lens, 1.0 / 16)
    res = check_outputs(to_np(out[sel]), ref, o, mref, oracle.sigmoid_table()[c_gate])
    print(f"[parity] decode_b70000 sampled {len(idx)} sequences: n={res['n']} "
          f"bit-exact={res['n_bit_exact']} max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
    assert res["ok"], res


def test_single_key_is_bit_exact():
    c = workloads.make_decode("L1", [1] * 24, seed=33)
    got = gpu_decode(c)
    ref, _, _ = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale)
    assert np.array_equal(got, ref)


def test_identical_kv_rows_are_bit_exact():
    """Every key and value row equal: O = v exactly in fp32 as well."""
    c = workloads.make_decode("same_kv", [1, 5, 16, 100, 700, 2000], seed=34, poison=False)
    c.k_pool[:] = c.k_pool[0, 0]
    c.v_pool[:] = c.v_pool[0, 0]
    got = gpu_decode(c)
    ref, _, _ = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale)
    assert np.array_equal(got, ref)


def test_every_gate_bit_pattern_through_the_api():
    """L = 1 and V = 1.0: out = bf16(sigmoid(gate)) for all 65,536 gate values,
    which must equal the oracle's correctly rounded table bit for bit."""
    B = 16
    c = workloads.make_decode("all_gates", [1] * B, seed=35)
    c.v_pool[:] = 0x3F80
    c.gate = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(B, 16, 256)
    got = gpu_decode(c)
    table = oracle.sigmoid_table()
    exp = table[c.gate]
    nan = (exp & 0x7F80) == 0x7F80
    nan &= (exp & 0x7F) != 0
    assert np.array_equal(got[~nan], exp[~nan])
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))


def test_gate_epilogue_zero_and_forty():
    """Same attention, gate 0 vs gate +40: sigma_b = 0.5 and 1.0, so the two
    outputs differ by exactly a factor of two (the product is bit-exact given
    the same bf16 O)."""
    c = workloads.make_decode("gate_c", [300, 17, 4096], seed=36)
    c.gate[:] = 0x4220
    out40 = gpu_decode(c)
    c.gate[:] = 0x0000
    out0 = gpu_decode(c)
    vals40 = oracle.compare.bf16_bits_to_f64(out40)
    vals0 = oracle.compare.bf16_bits_to_f64(out0)
    normal = np.abs(vals40) >= 2.0 ** -125
    assert np.array_equal(vals0[normal], vals40[normal] / 2)
    res = decode_parity(c, out0)
    assert res["ok"], res


def test_page_layout_does_not_change_bits():
    """Contiguous pages, one shuffle, another shuffle: bit-identical outputs."""
    lens = [512, 495, 478, 461]
    a = workloads.make_decode("contig", lens, seed=37, shuffle=False)
    outs = [gpu_decode(a)]
    for seed in (1, 2):
        perm = np.random.default_rng(seed).permutation(a.k_pool.shape[0]).astype(np.int32)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size, dtype=np.int32)
        b = workloads.make_decode("contig", lens, seed=37, shuffle=False)
        b.k_pool = a.k_pool[inv].copy()
        b.v_pool = a.v_pool[inv].copy()
        b.block_table = np.where(a.block_table >= 0, perm[np.clip(a.block_table, 0, None)], -1)
        outs.append(gpu_decode(b))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_batch_permutation_permutes_outputs():
    lens = [100, 2000, 37, 0, 1500]
    c = workloads.make_decode("perm", lens, seed=38)
    out = gpu_decode(c)
    order = np.array([3, 1, 4, 0, 2])
    c.q, c.gate = c.q[order].copy(), c.gate[order].copy()
    c.block_table, c.seq_lens = c.block_table[order].copy(), c.seq_lens[order].copy()
    assert np.array_equal(gpu_decode(c), out[order])


def test_padded_slots_are_positive_zero_and_nan_does_not_leak():
    c = workloads.make_decode("pad", [0, 33, 0, 1, 4094], seed=39, extra_pages=4)
    got = gpu_decode(c)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    finite = (got & 0x7F80) != 0x7F80
    assert finite.all()
    assert decode_parity(c, got)["ok"]


def test_inputs_are_not_modified_and_output_is_fully_written():
    c = workloads.make_decode("ro", [700, 3], seed=40)
    ins = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
    before = [t.clone() for t in ins]
    out = torch.full_like(ins[0], float("nan"))
    ga.decode(*ins, c.scale, out=out)
    torch.cuda.synchronize()
    for a, b in zip(ins, before):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
    assert not torch.isnan(out.float()).any()


def test_graph_replay_with_changed_inputs():
    """Capture one call into a HIP graph with a caller-owned workspace, then
    replay it with new q / gate / lengths; every replay equals an eager call."""
    c = workloads.make_decode("graph", [1024, 777, 16, 2048], seed=41, max_pages_per_seq=128)
    args = [to_dev(x) for x in (c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens)]
    dims = ga.decode_dims_for(args[0], args[2], args[4])
    ws = torch.empty(ga.decode_workspace_size(dims), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(args[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ga.decode(*args, c.scale, out=out, workspace=ws)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ga.decode(*args, c.scale, out=out, workspace=ws)
    rng = np.random.default_rng(5)
    for it in range(4):
        nq = workloads.normal_bf16(100 + it, 1, c.q.shape)
        ng = workloads.normal_bf16(200 + it, 2, c.gate.shape, std=2.0)
        nl = c.seq_lens.copy()
        # a new length may only use pages the block table already holds
        i = int(rng.integers(0, 4))
        nl[i] = int(rng.integers(0, int(c.seq_lens[i]) + 1))
        args[0].copy_(to_dev(nq))
        args[1].copy_(to_dev(ng))
        args[5].copy_(to_dev(nl))
        graph.replay()
        torch.cuda.synchronize()
        replayed = to_np(out)
        eager = to_np(ga.decode(*args, c.scale))
        torch.cuda.synchronize()
        assert np.array_equal(replayed, eager), it

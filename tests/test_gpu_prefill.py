"""GPU parity of gated_attn_prefill against the CPU oracle (gfx950 only)."""
import numpy as np
import pytest

import oracle
import workloads
import torch

import gated_gqa_decode_amd as ga
from gpu_helpers import DEV, gpu_prefill, to_dev, to_np
from oracle.compare import check_outputs

pytestmark = pytest.mark.gpu


def _parity(p, got, rows=None):
    ref, o, mref = oracle.prefill(p.q, p.gate, p.k, p.v, p.scale, causal=p.causal, rows=rows)
    gate = p.gate if rows is None else p.gate[rows[:, 0], rows[:, 1]]
    if rows is not None:
        got = got[rows[:, 0], rows[:, 1]]
    res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[gate])
    print(f"[parity] {p.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f} strict_fail={res['n_fail_strict']} "
          f"max_ulp_strict={res['max_ulp_strict']:.3f} model_fail={res['n_fail_model']}", flush=True)
    return res


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [1, 15, 16, 17, 64, 65, 100, 200])
def test_small_prefill_parity(S, causal):
    p = workloads.make_prefill(f"pf_S{S}_c{int(causal)}", 2, S, seed=50 + S, causal=causal)
    res = _parity(p, gpu_prefill(p))
    assert res["ok"], res


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(32, 2), (12, 2), (20, 2), (4, 2), (2, 2), (7, 1), (6, 3),
                                     (9, 1), (22, 2), (15, 1), (39, 3)])
def test_gqa_group_sizes(Hq, Hkv, causal):
    """Groups below 8 (idle waves only stage K/V) and groups 9..16 (two
    workgroups per kv head, ceil(G/2) and floor(G/2) heads); S = 130 spans
    three key tiles and a ragged tail."""
    p = workloads.make_prefill(f"pf_gqa_{Hq}_{Hkv}", 2, 130, seed=80 + Hq + Hkv, causal=causal,
                               num_q_heads=Hq, num_kv_heads=Hkv)
    res = _parity(p, gpu_prefill(p))
    assert res["ok"], res


def test_workload4_full_size_every_element():
    """B=2, S=2048 causal, in the launch configuration the benchmark times:
    every one of the 16.8 M outputs against the oracle.  The output is
    NaN-poisoned before the call, so a query tile the kernel never writes (or
    writes elsewhere) fails."""
    p = workloads.workload(4)
    out = torch.full(p.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    ga.prefill(to_dev(p.q), to_dev(p.gate), to_dev(p.k), to_dev(p.v), p.scale, causal=True,
               out=out)
    torch.cuda.synchronize()
    got = to_np(out)
    assert not np.any((got & 0x7F80) == 0x7F80), "non-finite (unwritten?) output"
    res = _parity(p, got)
    assert res["ok"], res


def test_identical_kv_rows_bit_exact():
    p = workloads.make_prefill("pf_same", 1, 130, seed=60, causal=True)
    p.k[:] = p.k[0, 0, 0]
    p.v[:] = p.v[0, 0, 0]
    got = gpu_prefill(p)
    ref, _, _ = oracle.prefill(p.q, p.gate, p.k, p.v, p.scale, causal=True)
    assert np.array_equal(got, ref)


def test_causal_first_row_is_gated_first_value():
    """Row 0 under the causal mask sees one key: out = bf16(V_0 * sigma_b)."""
    p = workloads.make_prefill("pf_row0", 2, 48, seed=61, causal=True)
    got = gpu_prefill(p)
    ref, _, _ = oracle.prefill(p.q, p.gate, p.k, p.v, p.scale, causal=True)
    assert np.array_equal(got[:, 0], ref[:, 0])


def test_every_gate_bit_pattern_through_prefill():
    """V = 1.0 everywhere, so O = 1 exactly and out = bf16(sigmoid(gate)):
    all 65,536 gate values (S = 16 rows x 16 heads x 256 dims) must equal the
    oracle's correctly rounded table bit for bit, as through decode."""
    p = workloads.make_prefill("pf_all_gates", 1, 16, seed=62, causal=True)
    p.v[:] = 0x3F80
    p.gate = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(p.gate.shape)
    got = gpu_prefill(p)
    exp = oracle.sigmoid_table()[p.gate]
    nan = ((exp & 0x7F80) == 0x7F80) & ((exp & 0x7F) != 0)
    assert np.array_equal(got[~nan], exp[~nan])
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))


def _every_row_written(got):
    assert not np.any((got & 0x7F80) == 0x7F80), "non-finite (unwritten?) output"


@pytest.mark.parametrize("B,S,Hq,Hkv", [
    (1, 8192, 16, 2),   # 512 query tiles per (sequence, kv head); 2 slices, 4 XCDs each
    (4, 520, 32, 4),    # 16 slices: several slices per XCD; a ragged last query tile
])
def test_long_and_many_slice_prefill_sampled_rows(B, S, Hq, Hkv):
    """Shapes past the other tests' (query tiles per slice, slices per XCD):
    the NaN-poisoned output must be written everywhere, and sampled rows --
    first and last positions, tile and key-tile boundaries, seeded picks --
    match the oracle."""
    p = workloads.make_prefill(f"pf_B{B}_S{S}", B, S, seed=90 + S, causal=True, num_q_heads=Hq,
                               num_kv_heads=Hkv)
    out = torch.full(p.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    ga.prefill(to_dev(p.q), to_dev(p.gate), to_dev(p.k), to_dev(p.v), p.scale, causal=True,
               out=out)
    torch.cuda.synchronize()
    got = to_np(out)
    _every_row_written(got)
    rng = np.random.default_rng(S)
    pos = {0, 1, 15, 16, 17, 63, 64, 65, S // 2, S - 17, S - 16, S - 2, S - 1}
    pos |= set(int(x) for x in rng.integers(0, S, size=24))
    rows = np.array([(b, s) for b in range(B) for s in sorted(pos)], dtype=np.int64)
    res = _parity(p, got, rows=rows)
    assert res["ok"], res


def test_prefill_graph_replay_with_changed_inputs():
    """A prefill call captured into a HIP graph, replayed with new q / gate /
    k / v: every replay equals an eager call, bit for bit."""
    p = workloads.make_prefill("pf_graph", 2, 200, seed=95, causal=True)
    args = [to_dev(x) for x in (p.q, p.gate, p.k, p.v)]
    out = torch.empty_like(args[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ga.prefill(*args, p.scale, causal=True, out=out)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ga.prefill(*args, p.scale, causal=True, out=out)
    for it in range(4):
        for i, (x, std) in enumerate(((p.q, 1.0), (p.gate, 2.0), (p.k, 1.0), (p.v, 1.0))):
            args[i].copy_(to_dev(workloads.normal_bf16(300 + 10 * it + i, 1, x.shape, std=std)))
        graph.replay()
        torch.cuda.synchronize()
        replayed = to_np(out)
        eager = to_np(ga.prefill(*args, p.scale, causal=True))
        torch.cuda.synchronize()
        assert np.array_equal(replayed, eager), it


def test_prefill_past_2_31_elements_sampled_rows():
    """q, gate and out of 2.18e9 elements each (B=65, S=2048, H_q=64, H_kv=8),
    so the last sequence's rows sit past element 2^31 and past byte 2^32
    (where a 32-bit element or byte offset would wrap onto sequence 0).  The
    inputs are seeded draws on the device (torch's generator), every sequence
    its own; the NaN-poisoned output must be written everywhere, and sampled
    rows of the first, a middle and the last sequences match the oracle on
    those sequences' inputs copied back."""
    B, S, Hq, Hkv, D = 65, 2048, 64, 8, 256
    assert B * S * Hq * D > 2 ** 31
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2031)

    def draw(shape, std):
        x = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)
        return (x * std).to(torch.bfloat16)

    # drawn in per-sequence slabs (fp32 temporaries stay small)
    q = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV)
    gate = torch.empty_like(q)
    k = torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    for b in range(B):
        q[b] = draw((S, Hq, D), 1.0)
        gate[b] = draw((S, Hq, D), 2.0)
        k[b] = draw((S, Hkv, D), 1.0)
        v[b] = draw((S, Hkv, D), 1.0)
    out = torch.full_like(q, float("nan"))
    scale = 1.0 / 16
    ga.prefill(q, gate, k, v, scale, causal=True, out=out)
    torch.cuda.synchronize()
    bits = out.view(torch.int16)
    assert not bool(((bits & 0x7F80) == 0x7F80).any()), "non-finite (unwritten?) output"
    rng = np.random.default_rng(2031)
    for b in (0, 32, B - 1):
        pos = {0, 1, 15, 16, 1023, 1024, S - 2, S - 1} | set(int(x) for x in rng.integers(0, S, 6))
        rows = np.array([(0, s) for s in sorted(pos)], dtype=np.int64)
        qb, gb, kb, vb = (to_np(x[b:b + 1]) for x in (q, gate, k, v))
        ref, o, mref = oracle.prefill(qb, gb, kb, vb, scale, causal=True, rows=rows)
        got = to_np(out[b:b + 1])[rows[:, 0], rows[:, 1]]
        res = check_outputs(got, ref, o, mref, oracle.sigmoid_table()[gb[rows[:, 0], rows[:, 1]]])
        print(f"[parity] pf_2_31 sequence {b}: n={res['n']} bit-exact={res['n_bit_exact']} "
              f"max_ulp_floor={res['max_ulp_floor']:.4f}", flush=True)
        assert res["ok"], (b, res)

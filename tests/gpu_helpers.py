"""Helpers for the GPU tests: host <-> device marshalling and parity reports."""
import numpy as np
import torch

import gated_gqa_decode_amd as ga
import oracle
from oracle.compare import check_outputs

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def gpu_decode(c, **kw) -> np.ndarray:
    out = ga.decode(to_dev(c.q), to_dev(c.gate), to_dev(c.k_pool), to_dev(c.v_pool),
                    to_dev(c.block_table), to_dev(c.seq_lens), c.scale, **kw)
    torch.cuda.synchronize()
    return to_np(out)


def gpu_prefill(p, causal=None) -> np.ndarray:
    out = ga.prefill(to_dev(p.q), to_dev(p.gate), to_dev(p.k), to_dev(p.v), p.scale,
                     causal=p.causal if causal is None else causal)
    torch.cuda.synchronize()
    return to_np(out)


def decode_parity(c, got=None) -> dict:
    if got is None:
        got = gpu_decode(c)
    ref, o, mref = oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                 c.scale)
    sig = oracle.sigmoid_table()[c.gate]
    res = check_outputs(got, ref, o, mref, sig)
    res["name"] = c.name
    print(f"[parity] {c.name}: n={res['n']} bit-exact={res['n_bit_exact']} "
          f"max_ulp_floor={res['max_ulp_floor']:.4f} strict_fail={res['n_fail_strict']} "
          f"max_ulp_strict={res['max_ulp_strict']:.3f} model_fail={res['n_fail_model']}", flush=True)
    return res

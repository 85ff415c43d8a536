"""Seeded synthetic inputs for gated GQA decode and prefill.

This module is shared by the test suite, the benchmark and the smoke check.  It
only draws random numbers and lays them out (paged pools, block tables,
lengths); it performs none of the attention arithmetic and imports neither the
GPU package nor the oracle.

Value recipe (the same for every workload): q, K, V ~ N(0, 1) and gate ~ N(0, 2)
(standard deviation 2), drawn in float32 from numpy's PCG64 -- chunk i of the
tensor with stream id s comes from ``SeedSequence([seed, s, i])`` -- then
rounded to bf16 by torch's float32 -> bfloat16 conversion.  The rounding of the inputs does not affect
parity: the GPU and the oracle receive the identical bits.

Paged layout: pools are [num_pages][16][H_kv][D]; sequence b owns
ceil(L_b / 16) pages whose ids are a seeded permutation of [0, num_pages),
assigned in logical order (or the identity for a contiguous workload).  Unused
block-table entries hold -1.  With ``poison=True`` the slots past L_b in each
sequence's last page and every unused page hold NaN (bf16 0x7FC0), so a kernel
that reads past a sequence's end produces NaN instead of a plausible number.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 16
NAN_BF16 = 0x7FC0
NAN_E4M3 = 0x7F
E4M3_MAX = 448.0
# default per-tensor dequantisation factor of FP8 pools: N(0, 1) values up to
# 6.5 map onto the whole e4m3 range
E4M3_DESCALE = float(np.float32(6.5 / E4M3_MAX))

# Stream ids for SeedSequence([seed, stream]).
_S_Q, _S_GATE, _S_K, _S_V, _S_LEN, _S_PERM, _S_PAD = range(1, 8)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(seed: int, stream: int, shape, std: float = 1.0, chunk: int = 1 << 22) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws.

    The array is cut into fixed chunks; chunk i comes from its own generator
    SeedSequence([seed, stream, i]), so the values do not depend on how many
    threads fill them (generation runs on a small thread pool)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)

    def fill(i: int) -> None:
        s, e = i * chunk, min(n, (i + 1) * chunk)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream), i])))
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = _f32_to_bf16_bits(x)

    nchunks = (n + chunk - 1) // chunk
    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        from concurrent.futures import ThreadPoolExecutor

        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normal_e4m3(seed: int, stream: int, shape, descale: float, chunk: int = 1 << 22) -> np.ndarray:
    """e4m3 codes (uint8) of N(0, 1) draws divided by ``descale``, clipped to
    the finite range, encoded by torch's float32 -> float8_e4m3fn conversion.
    Same chunked, thread-count independent streams as normal_bf16."""
    import torch

    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint8)
    inv = np.float32(1.0 / descale)

    def fill(i: int) -> None:
        s, e = i * chunk, min(n, (i + 1) * chunk)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream), i])))
        x = np.clip(rng.standard_normal(e - s, dtype=np.float32) * inv, -E4M3_MAX, E4M3_MAX)
        t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
        out[s:e] = t.numpy()

    nchunks = (n + chunk - 1) // chunk
    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        from concurrent.futures import ThreadPoolExecutor

        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclasses.dataclass
class DecodeCase:
    name: str
    q: np.ndarray            # [B, H_q, D] uint16 (bf16 bits)
    gate: np.ndarray         # [B, H_q, D]
    k_pool: np.ndarray       # [P, 16, H_kv, D]
    v_pool: np.ndarray       # [P, 16, H_kv, D]
    block_table: np.ndarray  # [B, W] int32, -1 where unused
    seq_lens: np.ndarray     # [B] int32, 0 for padded slots
    scale: float
    k_descale: float = 1.0   # FP8 pools (uint8 e4m3 codes): K = k_descale * e4m3(code)
    v_descale: float = 1.0

    @property
    def fp8(self) -> bool:
        return self.k_pool.dtype == np.uint8

    @property
    def dims(self):
        B, Hq, D = self.q.shape
        P, ps, Hkv, _ = self.k_pool.shape
        return dict(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                    max_pages_per_seq=self.block_table.shape[1], num_pages=P)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes a decode call reads: sum_b L_b * H_kv * D * elem * 2
        (elem = 2 bytes for bf16 pools, 1 for e4m3)."""
        _, _, Hkv, D = self.k_pool.shape
        elem = self.k_pool.dtype.itemsize
        return int(np.clip(self.seq_lens, 0, None).astype(np.int64).sum()) * Hkv * D * elem * 2


@dataclasses.dataclass
class PrefillCase:
    name: str
    q: np.ndarray      # [B, S, H_q, D]
    gate: np.ndarray   # [B, S, H_q, D]
    k: np.ndarray      # [B, S, H_kv, D]
    v: np.ndarray      # [B, S, H_kv, D]
    scale: float
    causal: bool


def make_decode(name: str, seq_lens: Sequence[int], *, seed: int, num_q_heads: int = 16,
                num_kv_heads: int = 2, head_dim: int = 256, max_pages_per_seq: Optional[int] = None,
                shuffle: bool = True, poison: bool = True, extra_pages: int = 0,
                scale: Optional[float] = None, gate_std: float = 2.0, kv_dtype: str = "bf16",
                kv_descale: float = E4M3_DESCALE) -> DecodeCase:
    """kv_dtype "fp8": K and V pools of e4m3 codes with per-tensor factor kv_descale."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    B = lens.shape[0]
    npages = (np.clip(lens, 0, None).astype(np.int64) + PAGE_SIZE - 1) // PAGE_SIZE
    W = int(max_pages_per_seq if max_pages_per_seq is not None else max(1, int(npages.max(initial=1))))
    assert np.all(npages <= W), "a sequence needs more pages than the block table holds"
    used = int(npages.sum())
    P = used + int(extra_pages)
    if shuffle:
        ids = _rng(seed, _S_PERM).permutation(P).astype(np.int32)
    else:
        ids = np.arange(P, dtype=np.int32)
    block_table = np.full((B, W), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        n = int(npages[b])
        block_table[b, :n] = ids[cursor:cursor + n]
        cursor += n
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    q = normal_bf16(seed, _S_Q, (B, Hq, D))
    gate = normal_bf16(seed, _S_GATE, (B, Hq, D), std=gate_std)
    pool_shape = (max(P, 1), PAGE_SIZE, Hkv, D)
    if kv_dtype == "fp8":
        k_pool = normal_e4m3(seed, _S_K, pool_shape, kv_descale)
        v_pool = normal_e4m3(seed, _S_V, pool_shape, kv_descale)
        nan = NAN_E4M3
    else:
        assert kv_dtype == "bf16", kv_dtype
        k_pool = normal_bf16(seed, _S_K, pool_shape)
        v_pool = normal_bf16(seed, _S_V, pool_shape)
        nan = NAN_BF16
    if poison:
        for b in range(B):
            n = int(npages[b])
            tail = int(lens[b]) - (n - 1) * PAGE_SIZE if n > 0 else PAGE_SIZE
            if n > 0 and tail < PAGE_SIZE:
                last = block_table[b, n - 1]
                k_pool[last, tail:] = nan
                v_pool[last, tail:] = nan
        if extra_pages or P == 0:
            unused = ids[used:] if P else np.array([0])
            k_pool[unused] = nan
            v_pool[unused] = nan
    fp8 = kv_dtype == "fp8"
    return DecodeCase(name, q, gate, k_pool, v_pool, block_table, lens,
                      float(scale if scale is not None else 1.0 / np.sqrt(D)),
                      k_descale=float(kv_descale) if fp8 else 1.0,
                      v_descale=float(kv_descale) if fp8 else 1.0)


def make_prefill(name: str, batch: int, seq_len: int, *, seed: int, num_q_heads: int = 16,
                 num_kv_heads: int = 2, head_dim: int = 256, causal: bool = True,
                 scale: Optional[float] = None, gate_std: float = 2.0) -> PrefillCase:
    B, S, Hq, Hkv, D = batch, seq_len, num_q_heads, num_kv_heads, head_dim
    return PrefillCase(
        name,
        normal_bf16(seed, _S_Q, (B, S, Hq, D)),
        normal_bf16(seed, _S_GATE, (B, S, Hq, D), std=gate_std),
        normal_bf16(seed, _S_K, (B, S, Hkv, D)),
        normal_bf16(seed, _S_V, (B, S, Hkv, D)),
        float(scale if scale is not None else 1.0 / np.sqrt(D)),
        causal,
    )


# --------------------------------------------------------------------------
# The five workloads.  Workload i is generated with seed i.
# --------------------------------------------------------------------------
WORKLOADS = {
    0: "decode B=1 L=512 contiguous pages",
    1: "decode B=4 L=512/495/478/461 paged shuffled",
    2: "decode B=64 L=4096 paged shuffled",
    3: "decode B=224 L~U[4094,6142] paged shuffled, 11 padded slots",
    4: "prefill B=2 S=2048 causal",
}


def config3_lengths(seed: int = 3, batch: int = 224, lo: int = 4094, hi: int = 6142,
                    pad_fraction: float = 0.05) -> np.ndarray:
    lens = _rng(seed, _S_LEN).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    npad = int(round(pad_fraction * batch))
    pad = _rng(seed, _S_PAD).choice(batch, size=npad, replace=False)
    lens[pad] = 0
    return lens


def workload(i: int, *, poison: bool = True):
    """Build workload i (0..4) with seed i."""
    if i == 0:
        return make_decode("decode_b1_l512_contiguous", [512], seed=0, shuffle=False,
                           poison=poison, max_pages_per_seq=32)
    if i == 1:
        return make_decode("decode_b4_l512_495_478_461_paged", [512, 495, 478, 461], seed=1,
                           poison=poison, max_pages_per_seq=32)
    if i == 2:
        return make_decode("decode_b64_l4096_paged", [4096] * 64, seed=2, poison=poison,
                           max_pages_per_seq=256)
    if i == 3:
        return make_decode("decode_b224_l4094_6142_pad11_paged", config3_lengths(), seed=3,
                           poison=poison, max_pages_per_seq=384)
    if i == 4:
        return make_prefill("prefill_b2_s2048_causal", 2, 2048, seed=4, causal=True)
    raise ValueError(f"no workload {i}")


@dataclasses.dataclass
class RopeCase:
    """Inputs of the QK-RMSNorm + partial-RoPE + K/V-write step for T tokens."""
    name: str
    q: np.ndarray       # [T, H_q, D] bf16 bits
    k: np.ndarray       # [T, H_kv, D]
    v: np.ndarray       # [T, H_kv, D]
    w_q: np.ndarray     # [D] norm weights
    w_k: np.ndarray     # [D]
    cos: np.ndarray     # [T, R] bf16 bits, rotate-half (both halves hold the same angles)
    sin: np.ndarray     # [T, R]
    positions: np.ndarray  # [T] int64
    eps: float


def rope_tables(positions: np.ndarray, rope_dim: int, base: float = 1.0e7):
    """bf16 cos / sin tables [T, rope_dim] for the given positions: angle
    pos * base^(-2i / rope_dim) for i < rope_dim / 2, repeated for the second
    half (rotate-half layout), computed in fp64 and rounded by torch."""
    import torch

    half = rope_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rope_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    to16 = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16).copy()
    return to16(np.cos(ang)), to16(np.sin(ang))


def make_rope(name: str, num_tokens: int, *, seed: int, num_q_heads: int = 16,
              num_kv_heads: int = 2, head_dim: int = 256, rope_dim: int = 64,
              max_position: int = 8192, eps: float = 1e-6) -> RopeCase:
    """q, k, v ~ N(0, 1); norm weights 1 + 0.1 N(0, 1); random positions."""
    import torch

    T, Hq, Hkv, D = num_tokens, num_q_heads, num_kv_heads, head_dim
    pos = _rng(seed, _S_LEN).integers(0, max_position, size=T).astype(np.int64)
    w = _rng(seed, _S_PAD).standard_normal((2, D)).astype(np.float32) * np.float32(0.1) + 1
    w16 = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    cos, sin = rope_tables(pos, rope_dim) if rope_dim else (np.zeros((T, 0), np.uint16),) * 2
    return RopeCase(name, normal_bf16(seed, _S_Q, (T, Hq, D)), normal_bf16(seed, _S_K, (T, Hkv, D)),
                    normal_bf16(seed, _S_V, (T, Hkv, D)), w16[0].copy(), w16[1].copy(), cos, sin,
                    pos, float(eps))


def csr_layout(case: DecodeCase, seed: int, extra_slots: int = 7, poison: bool = True):
    """The same tokens at page size 1: every token of every sequence gets its
    own pool row, at a seeded random slot, addressed by CSR row pointers and
    indices (sequence b's tokens are indices[indptr[b] : indptr[b + 1]]).
    Also returns the equivalent page-size-1 block table [B, capacity] (-1
    where unused).  Unused slots hold NaN when ``poison``.

    Returns (k_pool [N, 1, H_kv, D], v_pool, indptr [B + 1], indices, table)."""
    lens = np.clip(case.seq_lens.astype(np.int64), 0, None)
    B = lens.shape[0]
    cap = case.block_table.shape[1] * case.k_pool.shape[1]
    total = int(lens.sum())
    N = total + int(extra_slots)
    slots = _rng(seed, _S_PERM + 16).permutation(N)[:total].astype(np.int32)
    _, _, Hkv, D = case.k_pool.shape
    nan = NAN_E4M3 if case.fp8 else NAN_BF16
    k1 = np.full((max(N, 1), 1, Hkv, D), nan if poison else 0, dtype=case.k_pool.dtype)
    v1 = np.full_like(k1, nan if poison else 0)
    indptr = np.zeros(B + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(lens)
    table = np.full((B, cap), -1, dtype=np.int32)
    ps = case.k_pool.shape[1]
    seq = np.repeat(np.arange(B), lens)                  # sequence of each token
    j = np.arange(total) - np.repeat(indptr[:-1], lens)  # position in its sequence
    page = case.block_table[seq, j // ps]
    k1[slots, 0] = case.k_pool[page, j % ps]
    v1[slots, 0] = case.v_pool[page, j % ps]
    table[seq, j] = slots
    return k1, v1, indptr, slots.copy(), table


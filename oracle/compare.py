"""Tolerance check of GPU bf16 outputs against the oracle -- test infrastructure.

Stated tolerance (floored two-ulp rule).  For an oracle output y with fp64
attention output O, reference magnitude Mref = sum_j p_j |V_j| / sum_j p_j and
sigma_b = bf16(sigmoid(gate)):

    |gpu - y| <= 2 * ulp_bf16( max(|y|, sigma_b * Mref) )

with ulp_bf16(x) = 2^(max(floor(log2 x), -126) - 7) and ulp_bf16(0) = 2^-133.
Where O does not come from cancellation (|O| comparable to Mref) this is the
plain "2 bf16 ulp of the oracle output"; where the weighted sum cancels, the
ulp is taken at the size of the terms summed, the only scale an fp32
accumulation error can be bounded by.  The strict count (ulp of |y| alone) is
reported beside it.

Error-model check (asserted beside the floored rule).  The GPU's fp32 paths
have an attention output within eta * Mref of the fp64 O, eta = 2^-10: the
scores sum 256 exact products in fp32 (error <= 255 * 2^-24 * scale *
sum_d |q_d k_d| <= 2^-12.1 for the seeded N(0, 1) inputs at D = 256 and scale
1/16, whose largest |scale * q.k| sums stay below 15), a relative error rho
of every softmax weight moves O by at most 2 rho Mref (numerator and
denominator), and the accumulation, exp2 and split-P errors add less than
2^-14 -- 2^-11.0 in all, taken twice for margin.  Rounding is monotone and
sigma_b >= 0, so the GPU output must then lie in

    [ bf16(bf16(O - eta Mref) * sigma_b),  bf16(bf16(O + eta Mref) * sigma_b) ]

exactly, with no ulp allowance.  This bounds the error of every element by
the size of the terms summed -- also where O cancels and the strict rule
cannot hold -- at 2^-10 of them, 16x tighter than the floored rule's 2^-6.
It is also what bounds the strict-rule violations: where |O| >= Mref / 2
(no cancellation to speak of), eta * Mref is below half a bf16 ulp of O, the
interval holds at most the two bf16 neighbours of O (times sigma_b, rounded),
and an output more than one or two ulp from the oracle's fails.  A strict
violation can only pass on an element whose |O| / Mref is below 1/2, and
there only by as many ulp of |O| as the cancellation allows.
"""
from __future__ import annotations

import numpy as np

TWO_M133 = 2.0 ** -133
ETA = 2.0 ** -10  # stated bound of |O_gpu - O| / Mref (module docstring)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^-133 at and below the subnormal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(a.shape, TWO_M133)
    nz = (a > 0) & np.isfinite(a)
    e = np.floor(np.log2(a[nz]))
    # guard log2 rounding at exact powers of two and just below them
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a[nz], e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a[nz], e + 1, e)
    e = np.maximum(e, -126.0)
    out[nz] = np.ldexp(1.0, (e - 7).astype(np.int64))
    return out


def model_interval(o_f64, mref, sigma_bits, eta: float = ETA):
    """The values the gated output may take when the attention output is
    within eta * Mref of O: (lowest, highest), fp64 arrays."""
    from . import bf16_rne

    o = np.asarray(o_f64, dtype=np.float64)
    e = eta * np.asarray(mref, dtype=np.float64)
    sig = bf16_bits_to_f64(sigma_bits)
    with np.errstate(invalid="ignore"):
        lo = bf16_bits_to_f64(bf16_rne(bf16_bits_to_f64(bf16_rne(o - e)) * sig))
        hi = bf16_bits_to_f64(bf16_rne(bf16_bits_to_f64(bf16_rne(o + e)) * sig))
    return lo, hi


def check_outputs(gpu_bits, ref_bits, o_f64, mref, sigma_bits, ulps: float = 2.0,
                  eta: float = ETA) -> dict:
    """Compare GPU output bits against the oracle's under the floored rule and
    the error-model interval (``eta=None`` skips the latter).

    All arrays share one shape.  Returns a dict with the counts; ``ok`` is the
    verdict of both checks on every element (NaN must match NaN).
    """
    gpu = bf16_bits_to_f64(gpu_bits)
    ref = bf16_bits_to_f64(ref_bits)
    sig = bf16_bits_to_f64(sigma_bits)
    mref = np.asarray(mref, dtype=np.float64)
    ref_nan = np.isnan(ref)
    gpu_nan = np.isnan(gpu)
    nan_mismatch = int(np.count_nonzero(ref_nan != gpu_nan))
    both = ~(ref_nan | gpu_nan)
    diff = np.zeros(ref.shape)
    with np.errstate(invalid="ignore"):
        diff[both] = np.abs(gpu[both] - ref[both])
    floor_scale = np.maximum(np.abs(np.where(both, ref, 0.0)), sig * mref)
    u_floor = bf16_ulp(floor_scale)
    u_strict = bf16_ulp(np.where(both, ref, 0.0))
    r_floor = diff / u_floor
    r_strict = diff / u_strict
    n_fail_floor = int(np.count_nonzero(r_floor > ulps)) + nan_mismatch
    strict_bad = r_strict > ulps
    n_fail_model = 0
    if eta is not None:
        lo, hi = model_interval(o_f64, mref, sigma_bits, eta)
        chk = both & np.isfinite(lo) & np.isfinite(hi)
        outside = np.zeros(ref.shape, dtype=bool)
        outside[chk] = (gpu[chk] < lo[chk]) | (gpu[chk] > hi[chk])
        n_fail_model = int(np.count_nonzero(outside))
    res = {
        "n": int(ref.size),
        "ok": n_fail_floor == 0 and n_fail_model == 0,
        "n_fail_model": n_fail_model,
        "eta": eta,
        "n_fail_floor": n_fail_floor,
        "max_ulp_floor": float(r_floor.max()) if r_floor.size else 0.0,
        "n_fail_strict": int(np.count_nonzero(strict_bad)) + nan_mismatch,
        "max_ulp_strict": float(r_strict.max()) if r_strict.size else 0.0,
        "n_bit_exact": int(np.count_nonzero(np.asarray(gpu_bits) == np.asarray(ref_bits))),
        "nan_mismatch": nan_mismatch,
    }
    if n_fail_model:
        o = np.asarray(o_f64, dtype=np.float64)
        res["model_violators"] = [
            {"index": [int(i) for i in ix], "gpu": float(gpu[tuple(ix)]),
             "lo": float(lo[tuple(ix)]), "hi": float(hi[tuple(ix)]),
             "O": float(o[tuple(ix)]), "Mref": float(mref[tuple(ix)])}
            for ix in np.argwhere(outside)[:8]]
    if np.any(strict_bad):
        o = np.asarray(o_f64, dtype=np.float64)
        idx = np.argwhere(strict_bad)[:8]
        res["strict_violators"] = [
            {"index": [int(i) for i in ix],
             "ulp_strict": float(r_strict[tuple(ix)]),
             "abs_O_over_Mref": float(abs(o[tuple(ix)]) / mref[tuple(ix)]) if mref[tuple(ix)] > 0 else None}
            for ix in idx
        ]
    return res

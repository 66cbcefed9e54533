"""Comparison helpers for GPU-vs-oracle parity tests."""
import numpy as np

import oracle

# Tolerance on bf16 outputs against the fp64 oracle: max-abs 1e-2 and
# mean-abs 1e-3.  Where the oracle value is so large that rounding alone
# can exceed 1e-2 (|o| >= 4: half a bf16 ulp is 2^-6 there), an element may
# be off by half an ulp of the oracle value plus 2^-10 |o| for the kernel's
# fp32 arithmetic before its final rounding -- a correctly rounded fp32
# result lands there, a result one whole ulp off does not.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
FP32_REL = 2.0 ** -10


def bf16_bits_to_f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.ldexp(1.0, (e - 7).astype(int)), 0.0)


def check_bf16(got_bits, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """got_bits: uint16 bf16 patterns; ref: fp64 oracle values (NaN = skip)."""
    got = bf16_bits_to_f64(got_bits)
    sel = ~np.isnan(ref)
    g, r = got[sel], ref[sel]
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    allow = np.maximum(max_abs, 0.5 * ulp_bf16(r) + FP32_REL * np.abs(r))
    bad = err > allow
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond tolerance, "
                           f"max err {err.max():.3g} at ref {r[np.argmax(err)]:.4g}")
    m = err.mean() if err.size else 0.0
    assert m <= mean_abs, f"{what}: mean abs err {m:.3g} > {mean_abs}"
    # error against the correctly rounded oracle isolates kernel error
    rr = oracle.bf16_round(r)
    return {"max_abs": float(err.max()) if err.size else 0.0, "mean_abs": float(m),
            "max_abs_vs_rounded": float(np.abs(g - rr).max()) if err.size else 0.0,
            "n": int(err.size)}

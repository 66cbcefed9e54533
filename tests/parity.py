"""Comparison helpers for GPU-vs-oracle parity tests."""
import numpy as np

import oracle

# Tolerance on bf16 outputs against the fp64 oracle: max-abs 1e-2 and
# mean-abs 1e-3.  An element whose oracle value is large enough that one
# bf16 ulp exceeds 1e-2 (|o| >= 2) may be off by that ulp: a correct fp32
# result can round either way near a tie.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


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
    allow = np.maximum(max_abs, ulp_bf16(r))
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

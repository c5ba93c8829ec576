"""The quotient rounding the quantizer kernels use, checked on the CPU.

The kernels compute rint_half_even(w / s) for bf16 w and s without a full
IEEE division: y0 = w * r with r a reciprocal of s within 1 ulp, the exact
residual e = w - y0 * s (an fma), y1 = y0 + e * r (an fma), then rint(y1).
This emulates those fp32 steps exactly in numpy (each fma is an exact
product and sum rounded once to fp32) and compares the integers with what
IEEE fp32 division followed by rint gives ("Quantization basics: from FP32
to INT4" §2.2 and §5: the quotient is rounded half to even), over every
bf16 s of one binade (the steps are invariant under scaling s and w by
a power of two), every bf16 w from 2^-30 s to 32 s of both signs plus
constructed ties, and every float within 1 ulp of 1/s as r.  The GPU
kernels themselves are checked bit for bit against the oracle by the
quantizer parity tests.
"""

import numpy as np


def _bf16_values(exps, signs=(1.0, -1.0)):
    m = np.arange(128, dtype=np.float64)
    return np.concatenate([sg * (1 + m / 128) * 2.0 ** e for e in exps for sg in signs])


def _f32_of_exact_sum(a, b):
    """fp32 rounding of the exact a + b (float64 inputs)."""
    S = a + b
    bb = S - a
    err = (a - (S - bb)) + (b - bb)            # S + err == a + b exactly
    c = S.astype(np.float32)
    up = np.nextafter(c, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(c, np.float32(-np.inf)).astype(np.float64)
    c64 = c.astype(np.float64)
    res = c64.copy()
    # S on an fp32 midpoint: the sign of err decides
    at_up = (S == (up + c64) / 2) & (err > 0)
    at_dn = (S == (dn + c64) / 2) & (err < 0)
    res[at_up] = up[at_up]
    res[at_dn] = dn[at_dn]
    return res.astype(np.float32)


def test_corrected_reciprocal_rounds_like_ieee_division():
    mismatches = 0
    for s in _bf16_values([0], signs=(1.0,)):
        s32 = np.float32(s)
        w = np.concatenate([_bf16_values(range(-30, 5)), [0.0, 0.5 * s, -0.5 * s, 2.5 * s]])
        w32 = w.astype(np.float32)
        ref = np.rint(w32 / s32)
        rc = np.float32(1) / s32
        for r in (rc, np.nextafter(rc, np.float32(0)), np.nextafter(rc, np.float32(np.inf))):
            if abs(float(r) - 1.0 / float(s)) >= float(np.spacing(rc)):
                continue                        # not within 1 ulp of 1/s
            y0 = (w32.astype(np.float64) * float(r)).astype(np.float32)
            e = (w32.astype(np.float64) - y0.astype(np.float64) * float(s32)).astype(np.float32)
            y1 = _f32_of_exact_sum(y0.astype(np.float64), e.astype(np.float64) * float(r))
            mismatches += int(np.sum(np.rint(y1) != ref))
    assert mismatches == 0

"""The low-bit quantizer's code rule on the device, checked in float32 on the
CPU: codes from a reciprocal multiply with an IEEE-divide fallback near
half-integers give exactly the codes of the divide (the oracle's step-3
definition). No GPU and no HIP code: the rule is restated here in numpy."""
import numpy as np


def test_divide_free_code_rule_matches_ieee_division():
    """The HIP quantizer finds rint(fl((x - z) / s)) as rint((x - z) * r) with
    r a reciprocal of s within 1 ulp, and falls back to the IEEE divide when
    the product is within 2^-16 (2^-13 for 8-bit codes) of a half-integer,
    tested as |fma(x - z, r, -rint(y))| >= 1/2 - margin (the exact product's
    distance from the code, rounded once to float32). Check that rule in
    float32
    over random fp16 groups (the oracle's step-3 setting, scale from the
    group's range) with r = the rounded reciprocal and its neighbours one ulp
    away: wherever the margin test passes, the code equals the divide's."""
    rng = np.random.default_rng(20260)
    checked = 0
    for bits in (8, 4, 2):
        margin = np.float32(2.0 ** -13 if bits == 8 else 2.0 ** -16)
        qmax = np.float32((1 << bits) - 1)
        for scale in (1.0, 20.0, 1e-3):
            x = (rng.standard_normal((4000, 64)) * scale).astype(np.float16).astype(np.float32)
            mn, mx = x.min(1, keepdims=True), x.max(1, keepdims=True)
            s = ((mx - mn) / qmax).astype(np.float32).astype(np.float16).astype(np.float32)
            ok = (s > 0)[:, 0]
            x, mn, s = x[ok], mn[ok], s[ok]
            a = (x - mn).astype(np.float32)
            ref = np.rint((a / s).astype(np.float32))
            r0 = (np.float32(1.0) / s).astype(np.float32)
            for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
                y = (a * r).astype(np.float32)
                t = np.rint(y)
                # fma: the float64 product of two float32 values is exact
                d = (a.astype(np.float64) * r.astype(np.float64) - t).astype(np.float32)
                far = np.abs(d) < np.float32(0.5) - margin
                assert np.array_equal(t[far], ref[far])
                checked += int(far.sum())
    assert checked > 1_000_000

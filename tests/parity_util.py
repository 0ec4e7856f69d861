"""Comparison helpers shared by the GPU parity tests."""
import numpy as np

P99_TOL = 1e-3          # 99th-percentile relative error vs the oracle's walk at the same theta
MEDIAN_SLACK = 1e-3     # GPU median error vs direct may exceed the oracle's by this fraction
FP32_FLOOR = 2e-6       # relative-error floor of fp32 sums (about 16 ulp), for theta -> 0


def rel_err(got, ref):
    """Per-target relative errors of the acceleration vector and of |phi|.
    Targets whose reference acceleration is zero are excluded (NaN)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    an = np.linalg.norm(ref[:, :3], axis=1)
    ea = np.linalg.norm(got[:, :3] - ref[:, :3], axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        acc = np.where(an > 0, ea / an, np.nan)
        pot = np.where(ref[:, 3] != 0, np.abs(got[:, 3] - ref[:, 3]) / np.abs(ref[:, 3]), np.nan)
    return acc, pot


def bracketed_err(got, ref_modes, ties):
    """Relative error per target against the nearest of the oracle's results
    (as computed, near-ties forced open, near-ties forced accepted) for
    targets that met a near-tie; plain error for the rest."""
    acc0, pot0 = rel_err(got, ref_modes[0])
    if ties is None or not np.any(ties > 0):
        return acc0, pot0
    acc1, pot1 = rel_err(got, ref_modes[1])
    acc2, pot2 = rel_err(got, ref_modes[2])
    t = ties > 0
    acc = acc0.copy()
    pot = pot0.copy()
    acc[t] = np.fmin(acc0[t], np.fmin(acc1[t], acc2[t]))
    pot[t] = np.fmin(pot0[t], np.fmin(pot1[t], pot2[t]))
    return acc, pot


def pct(x, q):
    x = x[np.isfinite(x)]
    return float(np.percentile(x, q)) if x.size else 0.0


def assert_walk_parity(got, oracle_modes, ties, label=""):
    acc, pot = bracketed_err(got, oracle_modes, ties)
    p99a, p99p = pct(acc, 99), pct(pot, 99)
    assert np.all(np.isfinite(got)), label + ": non-finite GPU output"
    assert p99a <= P99_TOL, "%s: p99 acceleration error %.3g" % (label, p99a)
    assert p99p <= P99_TOL, "%s: p99 potential error %.3g" % (label, p99p)
    return p99a, p99p


def assert_median_vs_direct(got, bh_ref, direct_ref, label=""):
    g, _ = rel_err(got, direct_ref)
    o, _ = rel_err(bh_ref, direct_ref)
    mg, mo = pct(g, 50), pct(o, 50)
    assert mg <= mo * (1 + MEDIAN_SLACK) + FP32_FLOOR, "%s: median vs direct %.4g > oracle %.4g" % (
        label, mg, mo)
    return mg, mo

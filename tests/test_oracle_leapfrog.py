"""Pins of the oracle's leapfrog and conserved-quantity definitions against
closed forms and the properties of the kick-drift-kick scheme (CPU only)."""
import numpy as np
import pytest

import workloads as W


def f4(xyz, m):
    xyz = np.asarray(xyz, np.float64)
    return np.concatenate([xyz, np.broadcast_to(np.asarray(m, np.float64).reshape(-1, 1),
                                                (xyz.shape[0], 1))], 1).astype(np.float32)


def test_free_particle_moves_in_a_straight_line(orc):
    p = f4([[0.25, -1.5, 3.0]], 2.0)
    v = np.array([[0.5, 0.25, -1.0]], np.float32)
    x, vv, a = orc.leapfrog(p, v, 0.125, 16, 0.5, 1.0, 0.0)
    assert np.array_equal(a, np.zeros((1, 4)))
    assert np.allclose(x, p[:, :3].astype(np.float64) + 2.0 * v, rtol=0, atol=1e-14)
    assert np.array_equal(vv, v.astype(np.float64))


def _circular_pair():
    # two bodies of mass 1/2 at separation 1 (G = 1): relative speed 1, each
    # body at speed 1/2 about the centre of mass, period 2 pi
    p = f4([[-0.5, 0.0, 0.0], [0.5, 0.0, 0.0]], 0.5)
    v = np.array([[0.0, -0.5, 0.0], [0.0, 0.5, 0.0]], np.float32)
    return p, v


def test_circular_two_body_orbit_closes(orc):
    p, v = _circular_pair()
    steps = 2000
    dt = 2.0 * np.pi / steps
    x, vv, a = orc.leapfrog(p, v, dt, steps, 0.0, 1.0, 0.0)
    assert np.max(np.abs(x - p[:, :3])) < 1e-3
    d0 = orc.diagnostics(p[:, :3], p[:, 3], v, [-0.5, -0.5])
    d1 = orc.diagnostics(x, p[:, 3], vv, a[:, 3])
    # closed forms: E = -G m1 m2 / (2 d) = -1/8, L_z = 2 * m * r * v = 1/4
    assert d0["kinetic"] + d0["potential"] == pytest.approx(-0.125, abs=1e-7)
    assert d0["angular_momentum"][2] == pytest.approx(0.25, abs=1e-7)
    e1 = d1["kinetic"] + d1["potential"]
    assert abs(e1 + 0.125) < 1e-5
    # a central force conserves L exactly; the forces here are evaluated at the
    # fp32-rounded positions, which leaves ~1e-9 of drift after 2000 steps
    assert abs(d1["angular_momentum"][2] - 0.25) < 1e-8
    assert np.all(np.abs(d1["momentum"]) < 1e-12)


def test_energy_error_is_second_order(orc):
    # an eccentric pair: the largest energy error over a fixed time falls by
    # about 4 when dt halves
    p = f4([[-0.5, 0.0, 0.0], [0.5, 0.0, 0.0]], 0.5)
    v = np.array([[0.0, -0.3, 0.0], [0.0, 0.3, 0.0]], np.float32)
    errs = []
    for steps in (400, 800):
        dt = 4.0 / steps
        x = p[:, :3].astype(np.float64)
        vv = v.astype(np.float64)
        e0 = None
        worst = 0.0
        for k in range(8):
            x, vv, a = orc.leapfrog(f4(x, 0.5), vv, dt, steps // 8, 0.0, 1.0, 0.0)
            d = orc.diagnostics(x, p[:, 3], vv, a[:, 3])
            e = d["kinetic"] + d["potential"]
            if e0 is None:
                d0 = orc.diagnostics(p[:, :3], p[:, 3], v, [-0.5, -0.5])
                e0 = d0["kinetic"] + d0["potential"]
            worst = max(worst, abs(e - e0))
        errs.append(worst)
    assert 3.0 < errs[0] / errs[1] < 5.0


def test_time_reversible(orc):
    rng = np.random.default_rng(21)
    p = W.plummer(500, seed=22)
    v = (0.3 * rng.standard_normal((500, 3))).astype(np.float32)
    x1, v1, _ = orc.leapfrog(p, v, 0.01, 20, 0.5, 1.0, 0.05, leaf_cap=4)
    x2, v2, _ = orc.leapfrog(f4(x1, p[:, 3]), -v1, 0.01, 20, 0.5, 1.0, 0.05, leaf_cap=4)
    # x1 is rounded to fp32 to restart; positions come back to that rounding
    assert np.max(np.abs(x2 - p[:, :3])) < 1e-6
    assert np.max(np.abs(v2 + v)) < 1e-5


def test_momentum_conserved_with_pairwise_forces(orc):
    rng = np.random.default_rng(23)
    p = W.plummer(300, seed=24)
    v = (0.2 * rng.standard_normal((300, 3))).astype(np.float32)
    x, vv, _ = orc.leapfrog(p, v, 0.01, 10, 0.0, 1.0, 0.02)
    m = p[:, 3].astype(np.float64)
    p0 = (m[:, None] * v).sum(0)
    p1 = (m[:, None] * vv).sum(0)
    # with theta = 0 every pair force is computed twice with opposite signs, so
    # the total momentum changes by rounding only
    assert np.max(np.abs(p1 - p0)) < 1e-13


def test_tree_forces_track_direct_forces(orc):
    rng = np.random.default_rng(25)
    p = W.plummer(2000, seed=26)
    v = (0.2 * rng.standard_normal((2000, 3))).astype(np.float32)
    xb, vb, _ = orc.leapfrog(p, v, 0.01, 10, 0.4, 1.0, 0.02)
    xd, vd, _ = orc.leapfrog(p, v, 0.01, 10, 0.0, 1.0, 0.02)
    disp = np.linalg.norm(xd - p[:, :3], axis=1)
    assert np.percentile(np.linalg.norm(xb - xd, axis=1) / disp, 99) < 1e-2


def test_diagnostics_unequal_masses_by_hand(orc):
    """Each conserved quantity of two bodies of unequal mass, worked out by
    hand: masses 1 and 3 at (1, 0, 0) and (0, 2, 0), velocities (0, 1, 0) and
    (2, 0, 1), potentials -3/sqrt(5) and -1/sqrt(5) (each body's potential
    from the other at separation sqrt(5), G = 1).  A sum that drops or
    misplaces the mass weight, the factor 1/2 or an operand of the cross
    product gives another number."""
    x = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    m = np.array([1.0, 3.0])
    v = np.array([[0.0, 1.0, 0.0], [2.0, 0.0, 1.0]])
    r5 = np.sqrt(5.0)
    d = orc.diagnostics(x, m, v, [-3.0 / r5, -1.0 / r5])
    assert d["mass"] == 4.0
    # (1 * 1 + 3 * (4 + 1)) / 2
    assert d["kinetic"] == 8.0
    # (1 * (-3 / sqrt 5) + 3 * (-1 / sqrt 5)) / 2
    assert d["potential"] == pytest.approx(-3.0 / r5, rel=1e-15)
    # 1 * (0, 1, 0) + 3 * (2, 0, 1)
    assert list(d["momentum"]) == [6.0, 1.0, 3.0]
    # 1 * (1,0,0) x (0,1,0) + 3 * (0,2,0) x (2,0,1) = (0, 0, 1) + 3 * (2, 0, -4)
    assert list(d["angular_momentum"]) == [6.0, 0.0, -11.0]

"""Pins for the CPU oracle: each check compares the oracle with something other
than itself (closed forms, invariants, exact rational geometry, brute-force
enumeration, values fixed by the pages), so that a dropped term, a wrong sign,
index or operand in oracle.c fails at least one of them."""
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f4(xyz, m):
    xyz = np.asarray(xyz, dtype=np.float64)
    out = np.zeros((xyz.shape[0], 4), np.float32)
    out[:, :3] = xyz
    out[:, 3] = m
    return out


def fib_sphere(n, radius):
    """Fibonacci lattice on a sphere: a nearly uniform shell."""
    k = np.arange(n) + 0.5
    z = 1.0 - 2.0 * k / n
    phi = np.pi * (1.0 + 5 ** 0.5) * k
    s = np.sqrt(1.0 - z * z)
    return radius * np.stack([s * np.cos(phi), s * np.sin(phi), z], axis=1)


# --------------------------------------------------------------------------
# bounding box
# --------------------------------------------------------------------------
def test_bbox_matches_numpy_minmax(orc):
    p = W.plummer(20000, seed=7)
    lo, hi, L = orc.Tree(p).bbox()
    assert np.array_equal(lo, p[:, :3].min(0).astype(np.float64))
    assert np.array_equal(hi, p[:, :3].max(0).astype(np.float64))
    assert L == max(float(hi[a]) - float(lo[a]) for a in range(3))


# --------------------------------------------------------------------------
# keys
# --------------------------------------------------------------------------
def _golden_octants():
    rows = []
    with open(os.path.join(GOLDEN, "octant_order.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


@pytest.mark.parametrize("bits", [63, 30])
def test_key_top_digit_follows_page_octant_order(orc, bits):
    # Two anchor particles fix the root cube to [0, 1]^3; the probe sits at the
    # centre of one level-1 octant.  The key's top 3-bit digit must be the
    # page's child index for that octant.
    for ux, uy, uz, child in _golden_octants():
        probe = [0.25 + 0.5 * ux, 0.25 + 0.5 * uy, 0.25 + 0.5 * uz]
        p = f4([[0, 0, 0], [1, 1, 1], probe], 1.0)
        k = orc.Tree(p, key_bits=bits, leaf_cap=1).keys()
        assert int(k[2]) >> (bits - 3) == child


@pytest.mark.parametrize("bits", [63, 30])
def test_key_corners(orc, bits):
    p = f4([[-2.0, 3.0, 1.0], [5.0, 4.0, 2.0], [1.0, 3.5, 1.5]], 1.0)
    k = orc.Tree(p, key_bits=bits).keys()
    assert int(k[0]) == 0                      # the min corner
    # the max extent is along x; x = hi clamps to the top cell, y and z do not reach it
    assert int(k[1]) & int("001" * (bits // 3), 2) == int("001" * (bits // 3), 2)


def test_key_all_ones_at_max_corner(orc):
    p = f4([[0, 0, 0], [1, 1, 1]], 1.0)
    assert int(orc.Tree(p, key_bits=63).keys()[1]) == (1 << 63) - 1
    assert int(orc.Tree(p, key_bits=30).keys()[1]) == (1 << 30) - 1


def _descend_exact(x, lo, L, bits):
    """Octant digits of a point by exact rational bisection of the root cube
    (upper half when the coordinate is at or above the midpoint), clamped at
    the max face.  Independent of the oracle's quantise-and-interleave."""
    key = 0
    lo_c = [Fraction(v) for v in lo]
    size = Fraction(L)
    for _ in range(bits):
        size /= 2
        digit = 0
        for a in range(3):
            mid = lo_c[a] + size
            if Fraction(float(x[a])) >= mid and Fraction(float(x[a])) < lo[a] + Fraction(L):
                digit |= 1 << a
                lo_c[a] = mid
            elif Fraction(float(x[a])) >= lo[a] + Fraction(L):   # max face clamps up
                digit |= 1 << a
                lo_c[a] = mid
        key = (key << 3) | digit
    return key


def test_keys_match_exact_rational_bisection(orc):
    p = W.plummer(200, seed=11)
    t = orc.Tree(p, key_bits=63)
    lo, _, L = t.bbox()
    keys = t.keys()
    for i in range(p.shape[0]):
        assert int(keys[i]) == _descend_exact(p[i, :3], lo, L, 21), i


def test_keys_30bit_are_the_top_of_63bit(orc):
    p = W.plummer(5000, seed=12)
    k63 = orc.Tree(p, key_bits=63).keys()
    k30 = orc.Tree(p, key_bits=30).keys()
    assert np.array_equal(k30, k63 >> np.uint64(33))


# --------------------------------------------------------------------------
# order
# --------------------------------------------------------------------------
def test_perm_is_stable_sort_of_keys(orc):
    # a coarse lattice with duplicated points forces equal keys
    p = W.lattice(8, shuffled=True, seed=3)
    p = np.concatenate([p, p[::3]])
    t = orc.Tree(p, key_bits=30)
    keys, perm = t.keys(), t.perm()
    assert np.array_equal(np.sort(perm), np.arange(p.shape[0]))
    ks = keys[perm]
    assert np.all(ks[1:] >= ks[:-1])
    eq = ks[1:] == ks[:-1]
    assert np.all(perm[1:][eq] > perm[:-1][eq])
    assert np.array_equal(perm, np.argsort(keys, kind="stable"))


# --------------------------------------------------------------------------
# tree topology
# --------------------------------------------------------------------------
def _brute_force_cells(keys, bits, leaf_cap):
    """Every (level, prefix) cell by enumeration; a cell exists when its parent
    exists, holds more than B particles and is above the finest level."""
    b = bits // 3
    cells = {}
    for lev in range(b + 1):
        pref, cnt = np.unique(keys >> np.uint64(3 * (b - lev)), return_counts=True)
        for pr, c in zip(pref.tolist(), cnt.tolist()):
            if lev == 0 or (cells.get((lev - 1, pr >> 3), (0, 0))[0] > leaf_cap
                            and (lev - 1, pr >> 3) in cells):
                cells[(lev, pr)] = (c, int(c <= leaf_cap or lev == b))
    return cells


@pytest.mark.parametrize("n,leaf_cap,bits,dup", [(40, 1, 63, False), (64, 4, 63, True),
                                                  (100, 2, 30, True), (300, 16, 63, False)])
def test_tree_matches_brute_force_enumeration(orc, n, leaf_cap, bits, dup):
    p = W.plummer(n, seed=n)
    if dup:
        p = np.concatenate([p, p[:5], p[:2]])
    t = orc.Tree(p, key_bits=bits, leaf_cap=leaf_cap)
    c = t.cells()
    got = {(int(l), int(pr)): (int(cn), int(lf)) for l, pr, cn, lf in
           zip(c["level"], c["prefix"], c["count"], c["is_leaf"])}
    assert got == _brute_force_cells(t.keys(), bits, leaf_cap)


def test_tree_invariants_and_preorder(orc):
    p = W.plummer(30000, seed=21)
    B = 8
    t = orc.Tree(p, key_bits=63, leaf_cap=B)
    c, keys, perm = t.cells(), t.keys(), t.perm()
    sk = keys[perm]
    lev, start, count = c["level"], c["start"], c["count"]
    assert count[0] == p.shape[0] and lev[0] == 0
    for i in range(len(lev)):
        # members form the contiguous sorted range [start, start + count)
        shift = np.uint64(3 * (21 - lev[i]))
        seg = sk[start[i]:start[i] + count[i]] >> shift
        assert np.all(seg == c["prefix"][i])
        if start[i] > 0:
            assert (sk[start[i] - 1] >> shift) != c["prefix"][i]
        if c["is_leaf"][i]:
            assert count[i] <= B or lev[i] == 21
            assert c["n_children"][i] == 0
        else:
            assert count[i] > B
    # pre-order: sorted by (start, level), children of a cell sum to its count
    order = np.lexsort((lev, start))
    assert np.array_equal(order, np.arange(len(lev)))
    total_child = np.zeros(len(lev), np.int64)
    stack = []
    for i in range(len(lev)):
        while stack and lev[stack[-1]] >= lev[i]:
            stack.pop()
        if stack:
            assert lev[stack[-1]] == lev[i] - 1
            total_child[stack[-1]] += count[i]
        stack.append(i)
    internal = c["is_leaf"] == 0
    assert np.array_equal(total_child[internal], count[internal])


def test_coincident_particles_stop_at_finest_level(orc):
    p = f4(np.concatenate([np.zeros((10, 3)), np.ones((1, 3))]), 0.5)
    c = orc.Tree(p, key_bits=30, leaf_cap=2).cells()
    deep = (c["is_leaf"] == 1) & (c["count"] == 10)
    assert deep.sum() == 1 and c["level"][deep][0] == 10


# --------------------------------------------------------------------------
# centre of mass
# --------------------------------------------------------------------------
def test_com_cube_corners_is_centre(orc):
    corners = np.array([[x, y, z] for z in (0, 1) for y in (0, 1) for x in (0, 1)], float)
    c = orc.Tree(f4(corners, 0.125), leaf_cap=8).cells()
    assert c["mass"][0] == 1.0
    assert np.allclose(c["com"][0], [0.5, 0.5, 0.5], rtol=0, atol=1e-15)


def test_com_matches_weighted_means(orc):
    rng = np.random.default_rng(5)
    p = W.plummer(3000, seed=5)
    p[:, 3] = rng.uniform(0.1, 2.0, p.shape[0]).astype(np.float32)
    t = orc.Tree(p, leaf_cap=4)
    c, perm = t.cells(), t.perm()
    P = p.astype(np.float64)
    for i in range(0, len(c["level"]), 7):
        mem = perm[c["start"][i]:c["start"][i] + c["count"][i]]
        m = P[mem, 3]
        assert np.isclose(c["mass"][i], m.sum(), rtol=1e-13, atol=0)
        assert np.allclose(c["com"][i], (m[:, None] * P[mem, :3]).sum(0) / m.sum(),
                           rtol=1e-12, atol=1e-13)


def test_massless_cell_takes_its_centre(orc):
    p = f4([[0, 0, 0], [1, 1, 1], [0.1, 0.1, 0.1]], 0.0)
    p[1, 3] = 1.0
    c = orc.Tree(p, leaf_cap=1).cells()
    lev1 = [i for i in range(len(c["level"])) if c["level"][i] == 1 and c["prefix"][i] == 0]
    assert np.allclose(c["com"][lev1[0]], [0.25, 0.25, 0.25])


def test_node_hmax_from_key_membership(orc):
    """Per-cell hmax against cell membership taken from the keys alone (a
    particle belongs to a level-l cell when its key's top 3l bits are the
    cell's prefix), so a wrong range, permutation or order fails."""
    rng = np.random.default_rng(17)
    base = W.plummer(300, seed=17)
    p = np.concatenate([base, base[:40]])               # coincident pairs too
    h = rng.uniform(0.01, 1.0, p.shape[0]).astype(np.float32)
    for bits, B in ((63, 1), (63, 3), (30, 2)):
        t = orc.Tree(p, key_bits=bits, leaf_cap=B)
        c, keys = t.cells(), t.keys()
        got = orc.node_hmax(t, h)
        b3 = bits // 3
        for i in range(len(c["level"])):
            shift = np.uint64(3 * (b3 - int(c["level"][i])))
            mem = (keys >> shift) == c["prefix"][i]
            assert mem.sum() == c["count"][i]
            assert got[i] == h[mem].max()


def test_node_hmax_invariants(orc):
    rng = np.random.default_rng(18)
    p = W.plummer(20000, seed=18)
    h = rng.exponential(0.1, p.shape[0]).astype(np.float32)
    t = orc.Tree(p, leaf_cap=16)
    c = t.cells()
    got = orc.node_hmax(t, h)
    assert got[0] == h.max()                              # the root holds everything
    lev = c["level"]
    for i in range(1, len(lev)):                         # a cell's parent precedes it
        j = i - 1
        while lev[j] >= lev[i]:
            j -= 1
        assert lev[j] == lev[i] - 1 and got[j] >= got[i]


# --------------------------------------------------------------------------
# forces: direct sum and the walk
# --------------------------------------------------------------------------
@pytest.mark.parametrize("eps", [0.0, 0.05])
def test_two_body_closed_form(orc, eps):
    p = f4([[0.1, -0.2, 0.3], [0.6, 0.4, -0.2]], 0.0)
    p[:, 3] = [0.75, 2.5]
    G = 1.7
    P = p.astype(np.float64)
    d = P[1, :3] - P[0, :3]
    r2 = d @ d + eps * eps
    a0 = G * P[1, 3] * d / r2 ** 1.5
    a1 = -G * P[0, 3] * d / r2 ** 1.5
    want = np.array([[*a0, -G * P[1, 3] / r2 ** 0.5], [*a1, -G * P[0, 3] / r2 ** 0.5]])
    assert np.allclose(orc.direct(p, G, eps), want, rtol=1e-14, atol=0)
    # theta up to 0.5 opens the root (at theta = 1 the root, self included,
    # would pass the test: the walk has no guard for a cell holding the target)
    for theta in (0.0, 0.3, 0.5):
        out, ni, _ = orc.Tree(p, leaf_cap=1).gravity(theta, G, eps)
        assert np.allclose(out, want, rtol=1e-14, atol=0)
        assert ni.tolist() == [1, 1]


def test_direct_net_force_vanishes(orc):
    p = W.plummer(3000, seed=8)
    out = orc.direct(p, 1.0, 0.01)
    m = p[:, 3].astype(float)
    net = (m[:, None] * out[:, :3]).sum(0)
    scale = (m[:, None] * np.abs(out[:, :3])).sum(0)
    assert np.all(np.abs(net) <= 1e-12 * scale)


def test_shell_theorem(orc):
    R, M, n = 0.8, 1.0, 20000
    src = f4(fib_sphere(n, R), M / n)
    dirs = fib_sphere(7, 1.0)
    outside = 2.5 * R * dirs
    inside = 0.3 * R * dirs
    q = f4(np.concatenate([outside, inside]), 0.0)
    d = orc.direct(src, 1.0, 0.0, targets=q)
    r = np.linalg.norm(outside, axis=1)
    assert np.allclose(d[:7, :3], -M * outside / r[:, None] ** 3, rtol=2e-3, atol=1e-6)
    assert np.allclose(d[:7, 3], -M / r, rtol=1e-4)
    assert np.all(np.linalg.norm(d[7:, :3], axis=1) < 2e-3 * M / R ** 2)
    assert np.allclose(d[7:, 3], -M / R, rtol=1e-4)
    bh, _, _ = orc.Tree(src, leaf_cap=8).gravity(0.3, 1.0, 0.0, targets=q)
    # the walk approximates: its own error at theta = 0.3 is well under 1%
    assert np.allclose(bh[:7, :3], d[:7, :3], rtol=5e-3, atol=1e-4)
    assert np.all(np.linalg.norm(bh[7:, :3], axis=1) < 1e-2 * M / R ** 2)
    assert np.allclose(bh[:, 3], d[:, 3], rtol=1e-2)


def test_uniform_ball_interior_field(orc):
    R, h = 1.0, 0.04
    g = np.arange(-R, R + h / 2, h)
    x, y, z = np.meshgrid(g, g, g, indexing="ij")
    pts = np.stack([x.ravel(), y.ravel(), z.ravel()], 1)
    pts = pts[np.linalg.norm(pts, axis=1) < R]
    M = 1.0
    src = f4(pts, M / pts.shape[0])
    # probes at lattice cell centres, where the nearest points cancel by symmetry
    probe = np.array([[0.30, 0.18, -0.06], [-0.18, 0.38, 0.10]])
    d = orc.direct(src, 1.0, 0.0, targets=f4(probe, 0.0))
    assert np.allclose(d[:, :3], -M * probe / R ** 3, rtol=0.03, atol=0.01)


def test_theta_zero_reproduces_direct(orc):
    p = W.uniform_cube(2048, seed=9)
    out, ni, _ = orc.Tree(p, leaf_cap=4).gravity(0.0, 1.0, 1e-3)
    d = orc.direct(p, 1.0, 1e-3)
    assert np.allclose(out, d, rtol=1e-12, atol=1e-12 * np.abs(d).max())
    assert ni.sum() == p.shape[0] * (p.shape[0] - 1)


def test_theta_infinite_is_one_root_monopole(orc):
    p = W.plummer(4000, seed=10)
    eps, G = 0.02, 1.3
    out, ni, _ = orc.Tree(p, leaf_cap=16).gravity(np.inf, G, eps)
    P = p.astype(np.float64)
    M = P[:, 3].sum()
    X = (P[:, 3:4] * P[:, :3]).sum(0) / M
    d = X - P[:, :3]
    r2 = (d * d).sum(1) + eps * eps
    want = G * M * d / r2[:, None] ** 1.5
    err = np.linalg.norm(out[:, :3] - want, axis=1) / np.linalg.norm(want, axis=1)
    assert err.max() < 1e-12
    assert np.allclose(out[:, 3], -G * M / r2 ** 0.5, rtol=1e-12)
    assert np.all(ni == 1)


def _golden_mac():
    rows = []
    with open(os.path.join(GOLDEN, "mac_cases.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                v = line.split()
                rows.append(([float(v[0]), float(v[1]), float(v[2])], int(v[3]), int(v[4])))
    return rows


def test_opening_test_hand_cases(orc):
    src = f4([[0, 0, 0], [0.25, 0, 0], [1, 1, 1]], 1.0)
    t = orc.Tree(src, key_bits=63, leaf_cap=1)
    for target, accepted, n_inter in _golden_mac():
        q = f4([target], 0.0)
        out, ni, _ = t.gravity(0.5, 1.0, 0.0, targets=q)
        exact = orc.direct(src, 1.0, 0.0, targets=q)[0]
        x = q[0, :3].astype(float)
        # C used whole: a monopole of mass 2 at (0.125, 0, 0) plus s3 exactly
        mono = np.zeros(4)
        for m, xs in ((2.0, [0.125, 0, 0]), (1.0, [1, 1, 1])):
            d = np.array(xs) - x
            r = np.linalg.norm(d)
            mono[:3] += m * d / r ** 3
            mono[3] -= m / r
        want = mono if accepted else exact
        assert np.allclose(out[0], want, rtol=1e-13, atol=0), target
        assert not np.allclose(mono, exact, rtol=1e-3)
        assert ni[0] == n_inter


def test_plummer_mean_radial_field(orc):
    n = 1 << 15
    p = W.plummer(n, seed=13)
    t = orc.Tree(p, leaf_cap=16)
    out, _, _ = t.gravity(0.3, 1.0, 0.0)
    x = p[:, :3].astype(float)
    r = np.linalg.norm(x, axis=1)
    ar = (out[:, :3] * x).sum(1) / r
    umax = (400.0 / 401.0) ** 1.5
    for lo_r, hi_r in ((2.0, 3.0), (3.0, 5.0)):
        sel = (r > lo_r) & (r < hi_r)
        rr = r[sel]
        enclosed = np.minimum(rr ** 3 / (rr ** 2 + 1.0) ** 1.5 / umax, 1.0)
        assert abs(np.mean(ar[sel] / (-enclosed / rr ** 2)) - 1.0) < 0.02


def test_bh_error_shrinks_with_theta(orc):
    p = W.uniform_cube(4096, seed=1)
    t = orc.Tree(p, leaf_cap=16)
    d = orc.direct(p, 1.0, 1e-3)
    dn = np.linalg.norm(d[:, :3], axis=1)
    med = []
    for theta in (0.3, 0.5, 0.7):
        out, _, _ = t.gravity(theta, 1.0, 1e-3)
        med.append(np.median(np.linalg.norm(out[:, :3] - d[:, :3], axis=1) / dn))
    assert med[0] < med[1] < med[2] < 0.02


def test_near_tie_bracket_modes(orc):
    # A lattice aligned with the cells (16 points per axis at i/15, root cube
    # [0,1]^3) puts each level-2 centre of mass at (8k+3)/30 per axis; targets
    # half a unit away in x sit at r^2 = 0.25 = w^2/theta^2 for theta = 0.5,
    # an exact tie in real arithmetic.  The forced modes must bracket the
    # default and differ from it only at near-ties.
    g = np.arange(16) / 15.0
    z, y, x = np.meshgrid(g, g, g, indexing="ij")
    src = f4(np.stack([x.ravel(), y.ravel(), z.ravel()], 1), 1.0 / 4096)
    com = (8 * np.array([[0, 0, 0], [1, 0, 1], [2, 3, 1]]) + 3) / 30.0
    q = f4(np.concatenate([com + [0.5, 0, 0], [[0.11, 0.52, 0.33]]]), 0.0)
    t = orc.Tree(src, leaf_cap=8)
    base, n0, ties = t.gravity(0.5, 1.0, 1e-3, targets=q, tie_mode=0)
    op, n1, _ = t.gravity(0.5, 1.0, 1e-3, targets=q, tie_mode=1)
    ac, n2, _ = t.gravity(0.5, 1.0, 1e-3, targets=q, tie_mode=2)
    assert np.all(ties[:3] > 0)
    assert np.all(n1 >= n0) and np.all(n0 >= n2) and np.all(n1[:3] > n2[:3])
    assert np.any(op[:3] != ac[:3])
    untied = ties == 0
    assert np.array_equal(base[untied], op[untied]) and np.array_equal(base[untied], ac[untied])


# ---------------------------------------------------------------------------
# the warp vote ([GASPHiA] 性能瓶颈分析): groups of consecutive sorted targets
# ---------------------------------------------------------------------------
def test_vote_group_of_one_is_the_per_particle_walk(orc):
    p = W.plummer(3000, seed=12)
    t = orc.Tree(p, leaf_cap=8)
    ref, n_ref, _ = t.gravity(0.6, 1.0, 0.01)
    out, n_v, _, members = t.gravity_vote(0.6, 1.0, 0.01, group=1)
    assert np.array_equal(out, ref) and np.array_equal(n_v, n_ref)
    assert np.array_equal(np.sort(members), np.arange(3000))


def test_vote_never_uses_a_cell_the_member_would_open(orc):
    # every member sees at least the per-particle walk's interactions, and a
    # member of a group whose other members open more sees strictly more
    p = W.uniform_cube(4096, seed=1)
    t = orc.Tree(p, leaf_cap=16)
    _, n_ref, _ = t.gravity(0.5, 1.0, 1e-3)
    for group in (2, 64, 4096):
        _, n_v, _, _ = t.gravity_vote(0.5, 1.0, 1e-3, group=group)
        assert np.all(n_v >= n_ref)
        assert n_v.sum() > n_ref.sum()
    # one group of everything: every member uses the same cells, so all
    # counts are equal except for the self pair
    _, n_all, _, _ = t.gravity_vote(0.5, 1.0, 1e-3, group=4096)
    assert n_all.max() - n_all.min() <= 1


def test_vote_theta_limits(orc):
    p = W.plummer(2000, seed=13)
    t = orc.Tree(p, leaf_cap=4)
    d = orc.direct(p, 1.0, 0.02)
    out, n_v, _, _ = t.gravity_vote(0.0, 1.0, 0.02, group=64)
    assert np.all(n_v == 1999)
    assert np.allclose(out, d, rtol=1e-10, atol=1e-12)
    ref, _, _ = t.gravity(float("inf"), 1.0, 0.02)
    out, n_v, _, _ = t.gravity_vote(float("inf"), 1.0, 0.02, group=64)
    assert np.array_equal(out, ref) and np.all(n_v == 1)


def test_vote_groups_are_independent(orc):
    p = W.plummer(5000, seed=14)
    t = orc.Tree(p, leaf_cap=16)
    full, n_full, _, _ = t.gravity_vote(0.5, 1.0, 0.01, group=64)
    out, n_sub, _, members = t.gravity_vote(0.5, 1.0, 0.01, group=64, groups=[3, 40, 78])
    assert members.shape == (64 * 2 + 5000 - 78 * 64,)
    assert np.array_equal(out[members], full[members])
    assert np.array_equal(n_sub[members], n_full[members])


def test_vote_is_more_accurate_than_the_per_particle_walk(orc):
    p = W.uniform_cube(4096, seed=1)
    t = orc.Tree(p, leaf_cap=16)
    d = orc.direct(p, 1.0, 1e-3)
    dn = np.linalg.norm(d[:, :3], axis=1)
    ref, _, _ = t.gravity(0.5, 1.0, 1e-3)
    out, _, _, _ = t.gravity_vote(0.5, 1.0, 1e-3, group=64)
    e_ref = np.linalg.norm(ref[:, :3] - d[:, :3], axis=1) / dn
    e_v = np.linalg.norm(out[:, :3] - d[:, :3], axis=1) / dn
    assert np.median(e_v) < 0.5 * np.median(e_ref)


# ---------------------------------------------------------------------------
# stochastic Barnes-Hut ([SBH] 方法, 关键设计) and its random numbers
# ---------------------------------------------------------------------------
def test_philox_known_answers(orc):
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = [line.split() for line in open(path) if line.strip() and not line.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        assert orc.philox4x32_10(w[:4], w[4:6]).tolist() == w[6:10]


def test_target_order_matches_source_order_and_clamps(orc):
    p = W.plummer(3000, seed=31)
    t = orc.Tree(p)
    assert np.array_equal(t.target_order(p), t.perm())
    lo, hi, L = t.bbox()
    top = lo + L   # the root cube's upper corner
    q = f4([lo - 1.0, top + 1.0, lo, top], 0.0)   # below, above, at the two corners
    order = t.target_order(q)
    # below the cube and at its low corner both quantise to key 0, above and
    # at the high corner to the top key: the stable order is 0, 2, 1, 3
    assert order.tolist() == [0, 2, 1, 3]


def test_sbh_exact_cases(orc):
    # one source: the estimate is the exact pair term for any seed
    p = f4([[0.3, -0.2, 0.7]], 2.5)
    q = f4([[1.0, 1.0, 1.0], [-2.0, 0.5, 0.0]], 0.0)
    d = orc.direct(p, 1.0, 0.0, targets=q)
    for seed in (1, 2):
        out, _, _ = orc.Tree(p, leaf_cap=1).sbh(q, d=2, seed=seed)
        assert np.allclose(out, d, rtol=1e-14, atol=0)
    # one source per octant of the root: every stratum is a leaf, so the
    # estimate is the exact sum
    g = np.array([[x, y, z] for z in (0.1, 0.9) for y in (0.2, 0.8) for x in (0.15, 0.85)])
    p = f4(g, np.arange(1, 9) / 8.0)
    q = f4([[0.5, 0.5, 0.5], [2.0, -1.0, 0.3]], 0.0)
    d = orc.direct(p, 1.3, 0.0, targets=q)
    for dd in (2, 4):
        out, _, _ = orc.Tree(p, leaf_cap=1).sbh(q, d=dd, seed=9, G=1.3)
        assert np.allclose(out, d, rtol=1e-12, atol=0)


@pytest.mark.parametrize("d", [2, 4])
def test_sbh_is_unbiased(orc, d):
    src = W.surface_sources(1 << 11, seed=12)
    rng = np.random.default_rng(32)
    q = f4(rng.uniform(-1, 1, (8, 3)), 0.0)
    exact = orc.direct(src, 1.0, 0.0, targets=q)
    t = orc.Tree(src, leaf_cap=1)
    S = 20000
    out, sq, _ = t.sbh(q, d=d, samples=S, seed=77)
    se = np.sqrt(np.maximum(sq - out[:, 3] ** 2, 0.0) / S)
    z = (out[:, 3] - exact[:, 3]) / se
    assert np.all(np.abs(z) < 4.5), z
    assert np.all(se > 0)
    # the acceleration is estimated on the same paths: close to exact on average
    rel = np.linalg.norm(out[:, :3] - exact[:, :3], axis=1) / np.linalg.norm(exact[:, :3], axis=1)
    assert np.median(rel) < 0.02


def test_sbh_far_field_is_nearly_exact(orc):
    src = W.surface_sources(1 << 11, seed=13)
    q = f4([[40.0, -30.0, 25.0], [-60.0, 5.0, 10.0]], 0.0)
    exact = orc.direct(src, 1.0, 0.0, targets=q)
    out, _, _ = orc.Tree(src, leaf_cap=1).sbh(q, d=2, seed=5)
    assert np.max(np.abs(out[:, 3] / exact[:, 3] - 1.0)) < 1e-4


def test_sbh_group_shares_random_numbers(orc):
    src = W.surface_sources(1 << 10, seed=14)
    q = f4(np.repeat([[0.1, 0.2, 0.3]], 3, axis=0), 0.0)
    out, _, _ = orc.Tree(src, leaf_cap=1).sbh(q, d=2, seed=3)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])
    # queries one group apart draw other numbers
    out2, _, _ = orc.Tree(src, leaf_cap=1).sbh(q, d=2, seed=3, group=1)
    assert not np.array_equal(out2[0], out2[1])


# ---------------------------------------------------------------------------
# Hilbert keys (Skilling's transpose algorithm) and the tree in Hilbert order
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("side,bits", [(8, 63), (16, 63), (8, 30)])
def test_hilbert_keys_walk_the_grid_one_step_at_a_time(orc, side, bits):
    # points at i/(side-1) fall one per cell of the side^3 grid of the root
    # cube [0, 1]^3, so the top digits of their keys are the curve's index of
    # that cell: the curve must visit every cell once, start at the origin and
    # move to a face neighbour at every step
    g = np.arange(side) / (side - 1.0)
    z, y, x = np.meshgrid(g, g, g, indexing="ij")
    p = f4(np.stack([x.ravel(), y.ravel(), z.ravel()], 1), 1.0)
    t = orc.Tree(p, key_bits=bits, leaf_cap=1, curve="hilbert")
    levels = int(np.log2(side))
    top = t.keys() >> np.uint64(3 * (bits // 3 - levels))
    assert np.array_equal(np.sort(top), np.arange(side ** 3, dtype=np.uint64))
    cells = np.stack([np.round(x.ravel() * (side - 1)), np.round(y.ravel() * (side - 1)),
                      np.round(z.ravel() * (side - 1))], 1).astype(np.int64)
    path = cells[np.argsort(top)]
    assert np.array_equal(path[0], [0, 0, 0])
    assert np.all(np.abs(np.diff(path, axis=0)).sum(1) == 1)


@pytest.mark.parametrize("case,B", [("uniform4096", 16), ("plummer5000", 4), ("dups", 1)])
def test_hilbert_tree_has_the_morton_cells(orc, case, B):
    p = {"uniform4096": lambda: W.uniform_cube(4096, seed=1),
         "plummer5000": lambda: W.plummer(5000, seed=15),
         "dups": lambda: np.concatenate([W.uniform_cube(700, seed=16)] * 2)}[case]()
    tm = orc.Tree(p, leaf_cap=B, curve="morton")
    th = orc.Tree(p, leaf_cap=B, curve="hilbert")

    def cellset(t):
        c = t.cells()
        perm = t.perm()
        return {(int(l), int(pre), int(lf), int(cnt), tuple(sorted(perm[s:s + cnt].tolist())))
                for l, pre, lf, s, cnt in zip(c["level"], c["prefix"], c["is_leaf"], c["start"],
                                              c["count"])}
    assert cellset(tm) == cellset(th)
    # the same cells in another order: forces agree to rounding
    a, na, _ = tm.gravity(0.5, 1.0, 1e-3)
    b, nb, _ = th.gravity(0.5, 1.0, 1e-3)
    assert np.array_equal(na, nb)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)

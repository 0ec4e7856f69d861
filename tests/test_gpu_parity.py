"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bit-exact: bounding box, Morton keys, the sorted permutation, the tree
(every node's level, start, count, leaf flag, in pre-order).  Tolerance:
node masses and centres of mass (fp32 sums), and accelerations/potentials
(99th-percentile relative error <= 1e-3 vs the oracle's walk at the same
theta; median error vs the direct sum no worse than the oracle's own)."""
import numpy as np
import pytest

import workloads as W
from parity_util import P99_TOL, assert_median_vs_direct, assert_walk_parity, pct, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import barnes_hut_tree_amd  # noqa: F401  (must load: no fallback)
    barnes_hut_tree_amd.load_library()


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def log(*a):
    print(*a, flush=True)


def make_tree(p, key_bits=63, leaf_cap=16, max_targets=0, node_capacity=0, curve="morton"):
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(max(p.shape[0], 1), max_targets, key_bits, leaf_cap, node_capacity,
                     curve=curve)
    t.build(torch.from_numpy(p).cuda())
    t.sync()
    return t


# ---------------------------------------------------------------------------
# keys, order, bounding box: bit-exact
# ---------------------------------------------------------------------------
def _dup(p):
    return np.concatenate([p, p[:100], p[:7]])


def _clusters(sizes, radius, seed, background=0):
    """Tight balls of sources (radius relative to a unit root cube) plus two
    corners that fix the cube: many sources then share the top 40 bits of
    their 63-bit keys, the long runs the sort finishes in a workgroup."""
    rng = np.random.default_rng(seed)
    parts = [np.array([[0.0, 0.0, 0.0], [1.0, 1.0, 1.0]])]
    for k, m in enumerate(sizes):
        c = rng.uniform(0.2, 0.8, 3)
        d = rng.standard_normal((m, 3))
        d *= (radius * rng.uniform(0, 1, (m, 1)) ** (1 / 3)) / np.linalg.norm(d, axis=1, keepdims=True)
        parts.append(c + d)
    if background:
        parts.append(rng.uniform(0, 1, (background, 3)))
    xyz = np.concatenate(parts)
    xyz = xyz[rng.permutation(xyz.shape[0])]
    return np.concatenate([xyz, np.full((xyz.shape[0], 1), 1.0 / xyz.shape[0])], 1).astype(np.float32)


KEY_CASES = {
    "uniform4096": lambda: W.uniform_cube(4096, seed=1),
    "plummer65536": lambda: W.plummer(1 << 16, seed=3),
    "lattice_shuffled": lambda: W.lattice(100, shuffled=True, seed=2),
    "duplicates": lambda: _dup(W.uniform_cube(5000, seed=4)),
    "ragged4097": lambda: W.plummer(4097, seed=6),
    "ragged65": lambda: W.uniform_cube(65, seed=7),
    "single": lambda: W.uniform_cube(1, seed=8),
    # above the size from which the sort takes its larger tiles; every key twice
    "large_ragged": lambda: W.uniform_cube((1 << 22) + 777, seed=11),
    "large_duplicates": lambda: np.concatenate([W.plummer((1 << 21) + 5, seed=12)] * 2),
    # runs of 65..4096 sources sharing their top key bits (sorted in LDS) and
    # longer ones (counting passes), among short runs
    "clusters_mid": lambda: _clusters([70, 300, 1000, 4000], 1e-5, 13, background=30000),
    "clusters_long": lambda: _clusters([20000, 5000], 1e-5, 14, background=1000),
    "cluster_duplicates": lambda: np.concatenate([_clusters([9000], 1e-6, 15)] * 2),
    # many runs of 65..1100 sources starting in the same tiles (sorted a wave
    # per run), beside longer ones
    "clusters_many": lambda: _clusters([65, 66, 100, 127, 128, 129, 300, 511, 512, 513, 700,
                                        1023, 1024, 1025, 1100] * 4 + [3000], 1e-5, 16,
                                       background=2000),
    # several long runs to a tile beside runs longer than the LDS sort takes
    "clusters_heavy_long": lambda: _clusters([65, 80, 100, 120] * 8 + [20000, 6000], 1e-5, 17,
                                             background=500),
}


@pytest.mark.parametrize("bits", [63, 30])
@pytest.mark.parametrize("case", list(KEY_CASES))
def test_keys_perm_bbox_bitexact(orc, case, bits):
    p = KEY_CASES[case]()
    log("keys", case, bits, p.shape[0])
    t = make_tree(p, key_bits=bits)
    ref = orc.Tree(p, key_bits=bits, leaf_cap=16)
    lo, hi, L = t.bbox()
    rlo, rhi, rL = ref.bbox()
    assert lo == list(rlo) and hi == list(rhi) and L == rL
    k, perm = t.keys()
    rk = ref.keys()
    rperm = ref.perm()
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), rperm)
    assert np.array_equal(k.cpu().numpy().view(np.uint64), rk[rperm])
    t.close()


@pytest.mark.parametrize("case", ["clusters_many", "clusters_heavy_long", "cluster_duplicates",
                                  "plummer65536"])
def test_clustered_keys_sorted_in_all_passes_bitexact(orc, case):
    """A sort that finds several runs of more than 64 equal top key bits
    starting in one tile flags the context; its next builds sort all 63 bits
    in eight passes instead of five passes and the runs' kernel.  Keys and
    order stay bit-exact over repeated builds, whichever way each build took
    (the first of each case takes the runs' kernel; Plummer's runs never
    reach 65, so it always does)."""
    p = KEY_CASES[case]()
    log("clustered keys", case, p.shape[0])
    ref = orc.Tree(p, key_bits=63, leaf_cap=16)
    rk, rperm = ref.keys(), ref.perm()
    t = make_tree(p, key_bits=63)
    src = torch.from_numpy(p).cuda()
    for b in range(3):
        if b:
            t.build(src)
        k, perm = t.keys()   # waits for the build, so the next one sees its flag
        assert np.array_equal(perm.cpu().numpy().astype(np.int64), rperm), "build %d" % b
        assert np.array_equal(k.cpu().numpy().view(np.uint64), rk[rperm]), "build %d" % b
    t.close()


# ---------------------------------------------------------------------------
# tree: topology exact, centres of mass within fp32 tolerance
# ---------------------------------------------------------------------------
def _expected_skip(level):
    n = len(level)
    skip = np.full(n, n, dtype=np.int64)
    stack = []
    for i in range(n):
        while stack and level[stack[-1]] >= level[i]:
            skip[stack.pop()] = i
        stack.append(i)
    return skip


TREE_CASES = [("uniform4096", 63, 16), ("uniform4096", 63, 1), ("plummer65536", 63, 16),
              ("plummer65536", 30, 8), ("duplicates", 63, 4), ("lattice_shuffled", 63, 16),
              ("ragged65", 63, 3), ("single", 63, 16), ("plummer65536", 63, 256),
              # leaf capacities either side of 64, where the leaf-start search changes
              # from one wave row either side to a scan of the window
              ("plummer65536", 63, 33), ("ragged4097", 63, 63), ("plummer65536", 63, 64),
              ("ragged4097", 63, 64), ("plummer65536", 63, 65), ("duplicates", 30, 64),
              ("ragged65", 63, 64)]


@pytest.mark.parametrize("case,bits,B", TREE_CASES)
def test_tree_topology_and_com(orc, case, bits, B):
    import barnes_hut_tree_amd as bh
    p = KEY_CASES[case]()
    log("tree", case, bits, B, p.shape[0])
    t = make_tree(p, key_bits=bits, leaf_cap=B)
    g = bh.nodes_numpy(t.nodes())
    c = orc.Tree(p, key_bits=bits, leaf_cap=B).cells()
    assert len(g["level"]) == len(c["level"])
    assert np.array_equal(g["level"], c["level"])
    assert np.array_equal(g["start"].astype(np.int64), c["start"])
    assert np.array_equal(g["count"].astype(np.int64), c["count"])
    assert np.array_equal(g["is_leaf"], c["is_leaf"])
    assert np.array_equal(g["skip"].astype(np.int64), _expected_skip(c["level"]))
    assert np.allclose(g["mass"], c["mass"], rtol=2e-6, atol=0)
    _, _, L = t.bbox()
    err = np.abs(g["com"] - c["com"]).max(axis=1)
    assert err.max() <= 4e-6 * max(L, 1e-30) + 1e-6 * np.abs(c["com"]).max()
    t.close()


@pytest.mark.parametrize("curve", ["morton", "hilbert"])
@pytest.mark.parametrize("case,bits,B", [("uniform4096", 63, 1), ("plummer65536", 63, 16),
                                         ("plummer65536", 30, 8), ("duplicates", 63, 4),
                                         ("ragged65", 63, 3), ("single", 63, 16)])
def test_cells_level_prefix_count(orc, case, bits, B, curve):
    """bh_get_cells: every cell's level, place on its level's grid (key prefix)
    and source count, in pre-order, equal to the oracle's cells."""
    p = KEY_CASES[case]()
    t = make_tree(p, key_bits=bits, leaf_cap=B, curve=curve)
    g = t.cells()
    c = orc.Tree(p, key_bits=bits, leaf_cap=B, curve=curve).cells()
    assert g["level"].shape[0] == len(c["level"]) == t.node_count()
    assert np.array_equal(g["level"].cpu().numpy().astype(np.int32), c["level"])
    assert np.array_equal(g["prefix"].cpu().numpy().view(np.uint64), c["prefix"])
    assert np.array_equal(g["count"].cpu().numpy().view(np.uint32).astype(np.int64), c["count"])
    t.close()


def test_context_interaction_counter(orc):
    """bh_set_counting / bh_get_interactions: the context's own counter holds
    the count of the last walk (cleared at each call), equal to the caller's
    counter of bh_gravity_counted, and is refused once a walk did not count."""
    import barnes_hut_tree_amd as bh
    p = W.uniform_cube(4096, seed=1)
    t = make_tree(p)
    want = t.count_interactions(0.5, 1e-3)
    t.set_counting(True)
    for _ in range(2):
        t.gravity(0.5, 1.0, 1e-3)
        assert t.interactions() == want
    t.gravity(0.0, 1.0, 1e-3)
    assert t.interactions() == 4096 * 4095
    t.set_counting(False)
    t.gravity(0.5, 1.0, 1e-3)
    with pytest.raises(bh.BHError):
        t.interactions()
    t.close()


def test_headline_interaction_count_matches_oracle(orc):
    """The numerator of the benchmark's interactions/s: the GPU's count for
    the whole Plummer 2^20 step (Hilbert keys, theta = 0.5, eps = 0.01, leaf
    capacity 16) inside the oracle's full count bracket (near-ties forced
    accepted .. forced open), and within 1e-5 of its count as computed."""
    p = W.plummer(1 << 20, seed=3)
    t = make_tree(p, curve="hilbert")
    t.set_counting(True)
    t.gravity(0.5, 1.0, 0.01)
    got = t.interactions()
    t.close()
    ref = orc.Tree(p, leaf_cap=16, curve="hilbert")
    counts = [int(ref.gravity(0.5, 1.0, 0.01, tie_mode=m)[1].sum()) for m in (0, 1, 2)]
    log("  interactions gpu %d oracle %d (bracket %d .. %d)" % (got, counts[0], counts[2],
                                                                 counts[1]))
    assert counts[2] <= got <= counts[1]
    assert abs(got - counts[0]) <= 1e-5 * counts[0]


# ---------------------------------------------------------------------------
# gravity: the full 4096-particle cube against both oracles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B", [16, 1])
@pytest.mark.parametrize("theta", [0.3, 0.5, 0.7])
def test_gravity_uniform4096(orc, theta, B):
    p = W.uniform_cube(4096, seed=1)
    eps = 1e-3
    log("gravity uniform4096", theta, B)
    t = make_tree(p, leaf_cap=B)
    got = t.gravity(theta, 1.0, eps).cpu().numpy()
    cnt = t.count_interactions(theta, eps)
    ref = orc.Tree(p, leaf_cap=B)
    modes = [ref.gravity(theta, 1.0, eps, tie_mode=m) for m in (0, 1, 2)]
    ties = modes[0][2]
    p99a, p99p = assert_walk_parity(got, [m[0] for m in modes], ties, "uniform4096")
    direct = orc.direct(p, 1.0, eps)
    mg, mo = assert_median_vs_direct(got, modes[0][0], direct, "uniform4096")
    log("  p99 acc %.3g pot %.3g  median vs direct gpu %.4g oracle %.4g" % (p99a, p99p, mg, mo))
    lo_c, hi_c = modes[2][1].sum(), modes[1][1].sum()
    assert lo_c <= cnt <= hi_c, (cnt, lo_c, hi_c)
    t.close()


def test_theta_zero_is_direct_sum(orc):
    p = W.uniform_cube(4096, seed=1)
    t = make_tree(p, leaf_cap=16)
    got = t.gravity(0.0, 1.0, 1e-3).cpu().numpy()
    assert t.count_interactions(0.0, 1e-3) == 4096 * 4095
    d = orc.direct(p, 1.0, 1e-3)
    acc, pot = rel_err(got, d)
    # fp32 sums of 4095 terms; the worst targets are those whose terms nearly cancel
    assert pct(acc, 99) < 1e-5 and pct(acc, 100) < 2e-4
    assert pct(pot, 100) < 2e-5
    t.close()


def test_theta_infinite_is_root_monopole(orc):
    p = W.plummer(5000, seed=10)
    t = make_tree(p)
    got = t.gravity(float("inf"), 1.3, 0.02).cpu().numpy()
    ref, ni, _ = orc.Tree(p).gravity(float("inf"), 1.3, 0.02)
    acc, pot = rel_err(got, ref)
    assert pct(acc, 100) < 1e-4 and pct(pot, 100) < 1e-5
    assert t.count_interactions(float("inf")) == p.shape[0]
    t.close()


@pytest.mark.parametrize("case", ["tiny_cube", "huge_theta"])
def test_thresholds_below_the_exponent_step(orc, case):
    """(L / theta)^2 below 2^-83, where stepping the exponent by 2 per level
    would leave the normal range: the walk computes the level thresholds with
    ldexp instead.  A Plummer sphere scaled to a 7e-14 cube at theta = 0.5
    (tree levels down to a few 1e-16) with masses scaled by the square of the
    length scale, so accelerations stay of order one and m r^-3 stays inside the
    fp32 range, and a unit-scale one at theta = 1e16."""
    p = W.plummer(1 << 12, seed=12)
    if case == "tiny_cube":
        s = 2e-15
        p = p.copy()
        p[:, :3] *= np.float32(s)
        p[:, 3] *= np.float32(s * s)
        theta, eps = 0.5, 2e-17
    else:
        theta, eps = 1e16, 0.01
    log("exact thresholds", case)
    t = make_tree(p)
    got = t.gravity(theta, 1.0, eps).cpu().numpy()
    ref = orc.Tree(p)
    modes = [ref.gravity(theta, 1.0, eps, tie_mode=m) for m in (0, 1, 2)]
    assert_walk_parity(got, [m[0] for m in modes], modes[0][2], case)
    cnt = t.count_interactions(theta, eps)
    lo_c, hi_c = modes[2][1].sum(), modes[1][1].sum()
    assert lo_c <= cnt <= hi_c, (cnt, lo_c, hi_c)
    t.close()


def test_zero_softening_coincident_pairs(orc):
    # eps = 0 with coincident particles: such pairs must add nothing
    base = W.uniform_cube(600, seed=11)
    p = np.concatenate([base, base[:50]])
    t = make_tree(p, leaf_cap=4)
    got = t.gravity(0.5, 1.0, 0.0).cpu().numpy()
    ref = orc.Tree(p, leaf_cap=4)
    modes = [ref.gravity(0.5, 1.0, 0.0, tie_mode=m) for m in (0, 1, 2)]
    assert_walk_parity(got, [m[0] for m in modes], modes[0][2], "coincident eps=0")
    t.close()


def test_repeat_runs_bit_identical():
    p = W.plummer(1 << 16, seed=3)
    t = make_tree(p)
    a = t.gravity(0.5, 1.0, 0.01).cpu().numpy()
    t.build(torch.from_numpy(p).cuda())
    b = t.gravity(0.5, 1.0, 0.01).cpu().numpy()
    assert np.array_equal(a, b)
    t.close()


# ---------------------------------------------------------------------------
# full-size workloads, in the benchmark's launch configuration, on a sample
# of targets the oracle evaluates one by one
# ---------------------------------------------------------------------------
def _sampled_parity(orc, p, theta, eps, B, n_sample, seed, label, key_bits=63, direct=True,
                    curve="morton"):
    t = make_tree(p, key_bits=key_bits, leaf_cap=B, curve=curve)
    got = t.gravity(theta, 1.0, eps).cpu().numpy()
    assert np.all(np.isfinite(got)), label
    which = np.sort(np.random.default_rng(seed).choice(p.shape[0], n_sample, replace=False))
    ref = orc.Tree(p, key_bits=key_bits, leaf_cap=B, curve=curve)
    modes = [ref.gravity(theta, 1.0, eps, which=which, tie_mode=m) for m in (0, 1, 2)]
    ties = modes[0][2]
    p99a, p99p = assert_walk_parity(got[which], [m[0] for m in modes], ties, label)
    msg = "  %s: p99 acc %.3g pot %.3g, near-tie targets %d" % (label, p99a, p99p,
                                                                 int((ties > 0).sum()))
    if direct:
        d = orc.direct(p, 1.0, eps, which=which)
        mg, mo = assert_median_vs_direct(got[which], modes[0][0], d, label)
        msg += ", median vs direct gpu %.4g oracle %.4g" % (mg, mo)
    log(msg)
    t.close()
    return got


@pytest.mark.parametrize("theta", [0.3, 0.5, 0.7])
def test_plummer_2p20_random_order(orc, theta):
    p = W.plummer(1 << 20, seed=3)
    log("plummer 2^20 theta", theta)
    _sampled_parity(orc, p, theta, 0.01, 16, 2048, 31, "plummer2^20")


def test_plummer_2p20_sorted_order_same_result(orc):
    p = W.plummer(1 << 20, seed=3)
    order = orc.Tree(p).perm()
    t = make_tree(p)
    a = t.gravity(0.5, 1.0, 0.01).cpu().numpy()
    t.build(torch.from_numpy(np.ascontiguousarray(p[order])).cuda())
    b = t.gravity(0.5, 1.0, 0.01).cpu().numpy()
    assert np.array_equal(a[order], b)
    t.close()


@pytest.mark.parametrize("shuffled", [False, True])
def test_lattice_1m(orc, shuffled):
    p = W.lattice(100, shuffled=shuffled, seed=2)
    log("lattice 1M shuffled", shuffled)
    _sampled_parity(orc, p, 0.5, 1e-3, 16, 2048, 32, "lattice")


def test_galaxy_pair_5m(orc):
    p, _ = W.galaxy_pair()
    log("galaxy pair 5M")
    _sampled_parity(orc, p, 0.5, 0.02, 16, 1024, 33, "galaxy5M")


@pytest.mark.parametrize("seed", [10, 11])
@pytest.mark.parametrize("m_src", [1 << 15, 1 << 17, 1 << 20])
@pytest.mark.parametrize("queries", ["grid", "box"])
def test_surface_sources_separate_queries(orc, m_src, queries, seed):
    """Sources on spheres and tori, evaluated at the 100^3 grid or at 10^6
    uniform queries (theta = 0.5, eps = 0), on 2048 sampled queries: p99
    against the oracle's walk, the median acceleration error against the
    direct sum no worse than the oracle walk's, and the absolute potential
    errors (mean, median, max) the stochastic Barnes-Hut notes tabulate."""
    import barnes_hut_tree_amd as bh
    src = W.surface_sources(m_src, seed=seed)
    q = W.grid_queries() if queries == "grid" else W.box_queries()
    log("surface", m_src, queries, "seed", seed)
    t = bh.BarnesHut(src.shape[0], q.shape[0], 63, 16)
    t.build(torch.from_numpy(src).cuda())
    got = t.gravity(0.5, 1.0, 0.0, targets=torch.from_numpy(q).cuda()).cpu().numpy()
    t.sync()
    which = np.sort(np.random.default_rng(34 + seed).choice(q.shape[0], 2048, replace=False))
    ref = orc.Tree(src, leaf_cap=16)
    modes = [ref.gravity(0.5, 1.0, 0.0, targets=q, which=which, tie_mode=m) for m in (0, 1, 2)]
    p99a, p99p = assert_walk_parity(got[which], [m[0] for m in modes], modes[0][2], "surface")
    d = orc.direct(src, 1.0, 0.0, targets=q, which=which)
    mg, mo = assert_median_vs_direct(got[which], modes[0][0], d, "surface")
    abs_err = np.abs(got[which, 3] - d[:, 3])
    log("  p99 acc %.3g pot %.3g; median acc err vs direct gpu %.4g oracle %.4g; "
        "|phi| abs err vs direct mean %.3g median %.3g max %.3g" % (
            p99a, p99p, mg, mo, abs_err.mean(), np.median(abs_err), abs_err.max()))
    t.close()


# ---------------------------------------------------------------------------
# edge cases and device-detected errors
# ---------------------------------------------------------------------------
def test_empty_and_tiny_inputs(orc):
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(8, 4, 63, 16)
    t.build(torch.zeros((0, 4), device="cuda"))
    assert t.gravity(0.5).shape == (0, 4)
    none = torch.zeros((0, 4), device="cuda")
    assert t.gravity(0.5, targets=none).shape == (0, 4)
    q = torch.tensor([[0.5, 0.5, 0.5, 0.0]], device="cuda")
    assert torch.all(t.gravity(0.5, targets=q) == 0)
    t.sync()
    one = torch.tensor([[0.2, 0.3, 0.4, 1.0]], device="cuda")
    t.build(one)
    assert torch.all(t.gravity(0.5, eps=0.1) == 0)
    assert torch.all(t.gravity(0.5, eps=0.0) == 0)
    two = np.array([[0.1, -0.2, 0.3, 0.75], [0.6, 0.4, -0.2, 2.5]], np.float32)
    t.build(torch.from_numpy(two).cuda())
    got = t.gravity(0.5, 1.7, 0.05).cpu().numpy()
    want = orc.direct(two, 1.7, 0.05)
    assert np.allclose(got, want, rtol=2e-6)
    t.sync()
    t.close()


def test_all_coincident(orc):
    p = np.tile(np.array([[0.3, 0.3, 0.3, 0.01]], np.float32), (300, 1))
    for eps in (0.0, 0.1):
        t = make_tree(p, leaf_cap=8)
        got = t.gravity(0.5, 1.0, eps).cpu().numpy()
        ref, _, _ = orc.Tree(p, leaf_cap=8).gravity(0.5, 1.0, eps)
        assert np.allclose(got, ref, rtol=1e-5, atol=0)
        t.close()


def test_end_record_after_the_last_node(orc):
    """Every build writes an end record right after its last node (NaN centre,
    zero mass, an empty leaf starting at n, leaf bit set, level 0, skip
    pointing at itself, so a record fetched at its skip stays inside the
    array): every lane still walking opens it, which ends the walk's loop.  A second, smaller build
    in the same context writes its own at the lower index, and the walk then
    matches the oracle on that tree."""
    import ctypes
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(5000, 0, 63, 16)
    for n in (5000, 300):
        p = W.uniform_cube(n, seed=7)
        t.build(torch.from_numpy(p).cuda())
        nn = t.node_count()
        buf = torch.empty((nn + 1, 8), dtype=torch.int32, device="cuda")
        st = bh.load_library().bh_get_nodes(t._h, ctypes.c_void_p(buf.data_ptr()), nn + 1,
                                            bh._stream())
        assert st == 0
        f = bh.nodes_numpy(buf)
        assert np.all(np.isnan(f["com"][nn])) and f["mass"][nn] == 0.0
        assert f["start"][nn] == n and f["count"][nn] == 0 and f["skip"][nn] == nn
        assert f["is_leaf"][nn] == 1 and f["level"][nn] == 0
        assert np.all(np.isfinite(f["com"][:nn]))
        got = t.gravity(0.5, 1.0, 1e-3).cpu().numpy()
        ref = orc.Tree(p, leaf_cap=16)
        modes = [ref.gravity(0.5, 1.0, 1e-3, tie_mode=m) for m in (0, 1, 2)]
        assert_walk_parity(got, [m[0] for m in modes], modes[0][2], "end record n=%d" % n)
    t.close()


def test_nonfinite_input_is_reported():
    import barnes_hut_tree_amd as bh
    p = W.uniform_cube(1000, seed=2)
    p[17, 1] = np.nan
    t = bh.BarnesHut(1000, 0, 63, 16)
    t.build(torch.from_numpy(p).cuda())
    assert t.status() == bh.BH_ERR_NONFINITE
    with pytest.raises(bh.BHError):
        t.gravity(0.5)
    p[17, 1] = 0.5
    t.build(torch.from_numpy(p).cuda())
    t.sync()
    assert torch.all(torch.isfinite(t.gravity(0.5)))
    t.close()


def test_node_capacity_overflow_is_reported():
    import barnes_hut_tree_amd as bh
    p = W.uniform_cube(4096, seed=1)
    t = bh.BarnesHut(4096, 0, 63, 1, node_capacity=1000)
    t.build(torch.from_numpy(p).cuda())
    assert t.status() == bh.BH_ERR_CAPACITY
    t.close()


def test_targets_outside_the_root_cube(orc):
    import barnes_hut_tree_amd as bh
    src = W.plummer(20000, seed=5)
    q = np.array([[100.0, -50.0, 3.0, 0], [-80.0, 0.0, 0.0, 0], [0.1, 0.2, 0.3, 0]], np.float32)
    t = bh.BarnesHut(src.shape[0], 3, 63, 16)
    t.build(torch.from_numpy(src).cuda())
    got = t.gravity(0.5, 1.0, 0.01, targets=torch.from_numpy(q).cuda()).cpu().numpy()
    ref, _, _ = orc.Tree(src).gravity(0.5, 1.0, 0.01, targets=q)
    acc, pot = rel_err(got, ref)
    assert pct(acc, 100) < P99_TOL and pct(pot, 100) < P99_TOL
    t.close()


def test_invalid_arguments():
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(100, 0, 63, 16)
    with pytest.raises(bh.BHError):
        t.gravity(0.5)            # not built
    p = torch.from_numpy(W.uniform_cube(100)).cuda()
    t.build(p)
    with pytest.raises(bh.BHError):
        t.gravity(-1.0)
    with pytest.raises(bh.BHError):
        t.gravity(0.5, eps=-1.0)
    with pytest.raises(bh.BHError):
        t.gravity(0.5, targets=p)  # no target capacity
    big = torch.from_numpy(W.uniform_cube(101)).cuda()
    with pytest.raises(bh.BHError):
        t.build(big)
    # a target count that only matches the source count modulo 2^32, and NaN theta
    import ctypes
    L = bh.load_library()
    out = torch.empty((100, 4), dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o = ctypes.c_void_p(out.data_ptr())
    assert L.bh_gravity(t._h, None, (1 << 32) + 100, 0.5, 1.0, 0.0, o, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity(t._h, None, 100, float("nan"), 1.0, 0.0, o, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity(t._h, None, 100, 0.5, float("inf"), 0.0, o, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity(t._h, None, 100, 0.5, 1.0, 0.0, o, s) == bh.BH_OK
    t.close()


# ---------------------------------------------------------------------------
# other build parameters: 30-bit keys, very small and very large leaves
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key_bits,B", [(30, 16), (63, 2), (63, 64), (63, 65), (63, 256), (30, 256)])
def test_gravity_other_build_parameters(orc, key_bits, B):
    p = W.plummer(1 << 16, seed=12)
    log("gravity plummer 2^16 key_bits", key_bits, "B", B)
    _sampled_parity(orc, p, 0.5, 0.01, B, 2048, 35, "plummer2^16 bits=%d B=%d" % (key_bits, B),
                    key_bits=key_bits)


def test_separate_targets_30bit_keys(orc):
    import barnes_hut_tree_amd as bh
    src = W.surface_sources(1 << 15, seed=13)
    q = W.box_queries()[:100003]
    t = bh.BarnesHut(src.shape[0], q.shape[0], 30, 16)
    t.build(torch.from_numpy(src).cuda())
    got = t.gravity(0.5, 1.0, 0.0, targets=torch.from_numpy(q).cuda()).cpu().numpy()
    t.sync()
    which = np.sort(np.random.default_rng(36).choice(q.shape[0], 2048, replace=False))
    ref = orc.Tree(src, key_bits=30, leaf_cap=16)
    modes = [ref.gravity(0.5, 1.0, 0.0, targets=q, which=which, tie_mode=m) for m in (0, 1, 2)]
    p99a, p99p = assert_walk_parity(got[which], [m[0] for m in modes], modes[0][2], "30-bit queries")
    log("  30-bit keys, separate queries: p99 acc %.3g pot %.3g" % (p99a, p99p))
    t.close()

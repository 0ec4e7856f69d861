"""Contexts built with Hilbert keys (BH_CURVE_HILBERT) against the oracle's
tree in the same curve order: keys and permutation bit-exact, the tree
bit-exact in pre-order, centres of mass to fp32 tolerance (massless cells
take their centre), gravity at the oracle's tolerance, and the stochastic
estimator with queries grouped along the curve."""
import numpy as np
import pytest

import workloads as W
from parity_util import assert_walk_parity
from test_gpu_parity import KEY_CASES, _expected_skip, _sampled_parity, log, make_tree

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import barnes_hut_tree_amd
    barnes_hut_tree_amd.load_library()


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def _massless():
    p = W.uniform_cube(4096, seed=17)
    p[p[:, 0] < 0.3, 3] = 0.0   # a slab of massless sources: cells there take their centre
    return p


CASES = dict(KEY_CASES, massless=_massless,
             uniform_2p20=lambda: W.uniform_box(1 << 20, seed=5))


@pytest.mark.parametrize("bits", [63, 30])
@pytest.mark.parametrize("case", ["uniform4096", "plummer65536", "duplicates", "ragged65",
                                  "single", "uniform_2p20", "large_ragged"])
def test_hilbert_keys_perm_bitexact(orc, case, bits):
    p = CASES[case]()
    log("hilbert keys", case, bits)
    t = make_tree(p, key_bits=bits, curve="hilbert")
    ref = orc.Tree(p, key_bits=bits, leaf_cap=16, curve="hilbert")
    k, perm = t.keys()
    rperm = ref.perm()
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), rperm)
    assert np.array_equal(k.cpu().numpy().view(np.uint64), ref.keys()[rperm])
    t.close()


@pytest.mark.parametrize("curve", ["hilbert", "morton"])
@pytest.mark.parametrize("case,bits,B", [("uniform4096", 63, 16), ("plummer65536", 63, 16),
                                         ("plummer65536", 30, 4), ("duplicates", 63, 4),
                                         ("lattice_shuffled", 63, 16), ("massless", 63, 8)])
def test_tree_in_curve_order(orc, case, bits, B, curve):
    import barnes_hut_tree_amd as bh
    p = CASES[case]()
    log("tree", curve, case, bits, B)
    t = make_tree(p, key_bits=bits, leaf_cap=B, curve=curve)
    g = bh.nodes_numpy(t.nodes())
    c = orc.Tree(p, key_bits=bits, leaf_cap=B, curve=curve).cells()
    assert np.array_equal(g["level"], c["level"])
    assert np.array_equal(g["start"].astype(np.int64), c["start"])
    assert np.array_equal(g["count"].astype(np.int64), c["count"])
    assert np.array_equal(g["is_leaf"], c["is_leaf"])
    assert np.array_equal(g["skip"].astype(np.int64), _expected_skip(c["level"]))
    assert np.allclose(g["mass"], c["mass"], rtol=2e-6, atol=0)
    _, _, L = t.bbox()
    err = np.abs(g["com"] - c["com"]).max(axis=1)
    assert err.max() <= 4e-6 * max(L, 1e-30) + 1e-6 * np.abs(c["com"]).max()
    if case == "massless":
        assert np.any(c["mass"] == 0)
    t.close()


@pytest.mark.parametrize("theta", [0.3, 0.5, 0.7])
def test_hilbert_gravity_uniform4096(orc, theta):
    p = W.uniform_cube(4096, seed=1)
    t = make_tree(p, curve="hilbert")
    got = t.gravity(theta, 1.0, 1e-3).cpu().numpy()
    ref = orc.Tree(p, leaf_cap=16, curve="hilbert")
    modes = [ref.gravity(theta, 1.0, 1e-3, tie_mode=m) for m in (0, 1, 2)]
    assert_walk_parity(got, [m[0] for m in modes], modes[0][2], "hilbert uniform4096")
    # the same interactions as the Morton tree (the same cells)
    tm = make_tree(p)
    assert t.count_interactions(theta, 1e-3) == tm.count_interactions(theta, 1e-3)
    t.close()
    tm.close()


@pytest.mark.parametrize("theta", [0.3, 0.5, 0.7])
def test_hilbert_plummer_2p20(orc, theta):
    """The benchmark's workload and curve at each opening angle of the
    Plummer configuration, on 2048 sampled targets, with the median error
    against the direct sum on the same targets."""
    p = W.plummer(1 << 20, seed=3)
    log("hilbert plummer 2^20 theta", theta)
    _sampled_parity(orc, p, theta, 0.01, 16, 2048, 37, "hilbert plummer2^20 theta=%g" % theta,
                    curve="hilbert")


def test_hilbert_sbh_matches_oracle(orc):
    import barnes_hut_tree_amd as bh
    src = W.surface_sources(1 << 15, seed=10)
    q = W.grid_queries()
    t = bh.BarnesHut(src.shape[0], q.shape[0], 63, 1, curve="hilbert")
    t.build(torch.from_numpy(src).cuda())
    got = t.sbh(torch.from_numpy(q).cuda(), d=2, samples=1, seed=99).cpu().numpy()
    t.sync()
    which = np.sort(np.random.default_rng(72).choice(q.shape[0], 1024, replace=False))
    ref, _, near = orc.Tree(src, leaf_cap=1, curve="hilbert").sbh(q, d=2, samples=1, seed=99,
                                                                  which=which)
    clean = near == 0
    ep = np.abs(got[which, 3] - ref[:, 3]) / np.abs(ref[:, 3])
    assert clean.sum() >= 0.95 * len(which)
    assert np.percentile(ep[clean], 99) < 1e-3
    t.close()


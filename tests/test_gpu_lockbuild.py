"""The lock-based dense build (bh_build_locked) against the oracle's
leaf-capacity-1 octree: the same internal cells (level, key prefix) and the
same leaves with the same member sources, bit-exact, whatever order the
threads won their locks in."""
import numpy as np
import pytest

import workloads as W
from locktree_util import locked_tree_sets, oracle_tree_sets

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


def log(*a):
    print(*a, flush=True)


def _dups():
    base = W.uniform_cube(3000, seed=4)
    return np.concatenate([base, base, base[:11]])


CASES = {
    "uniform4096": lambda: W.uniform_cube(4096, seed=1),
    "plummer65536": lambda: W.plummer(1 << 16, seed=3),
    "lattice_shuffled": lambda: W.lattice(40, shuffled=True, seed=2),
    "duplicates": _dups,
    "ragged4097": lambda: W.plummer(4097, seed=6),
    "single": lambda: W.uniform_cube(1, seed=8),
    "two_coincident": lambda: np.repeat(W.uniform_cube(1, seed=9), 2, axis=0),
}


def lock_build(p, key_bits):
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(p.shape[0], 0, key_bits, 1)
    t.build_locked(torch.from_numpy(p).cuda())
    assert t.status() == bh.BH_OK
    child, level, nxt, cap = t.locked_tree()
    res = child.cpu().numpy(), level.cpu().numpy(), nxt.cpu().numpy(), cap
    return t, res


@pytest.mark.parametrize("bits", [63, 30])
@pytest.mark.parametrize("case", list(CASES))
def test_lock_build_equals_oracle_tree(orc, case, bits):
    p = CASES[case]()
    log("lock build", case, bits)
    t, (child, level, nxt, cap) = lock_build(p, bits)
    got = locked_tree_sets(child, level, nxt, cap, p.shape[0])
    want = oracle_tree_sets(orc.Tree(p, key_bits=bits, leaf_cap=1))
    if p.shape[0] == 1:
        # one source: the oracle's root is that leaf; the dense tree keeps an
        # empty root cell with the source in its octant
        assert len(got[1]) == 1 and list(got[1].values()) == [(0,)]
    else:
        assert got[0] == want[0]
        assert got[1] == want[1]
    t.close()


def test_lock_build_plummer_2p20(orc):
    p = W.plummer(1 << 20, seed=3)
    log("lock build plummer 2^20")
    t, (child, level, nxt, cap) = lock_build(p, 63)
    got = locked_tree_sets(child, level, nxt, cap, p.shape[0])
    want = oracle_tree_sets(orc.Tree(p, key_bits=63, leaf_cap=1))
    assert got[0] == want[0] and got[1] == want[1]
    t.close()


def test_lock_build_replaces_the_tree_and_reports_nonfinite():
    import barnes_hut_tree_amd as bh
    p = W.uniform_cube(1000, seed=5)
    t = bh.BarnesHut(1000, 0, 63, 1)
    src = torch.from_numpy(p).cuda()
    t.build(src)
    t.build_locked(src)
    with pytest.raises(bh.BHError):
        t.gravity(0.5)            # the sorted tree is gone until bh_build runs again
    t.build(src)
    assert torch.isfinite(t.gravity(0.5, 1.0, 1e-3)).all()
    bad = p.copy()
    bad[17, 1] = np.nan
    t.build_locked(torch.from_numpy(bad).cuda())
    assert t.status() == bh.BH_ERR_NONFINITE
    t.close()

"""The node bound of the allocation-free step (bh_gravity_static sizes its tree
from it): a tree over n sources with leaf capacity B and `bits` levels below
the root has at most bits * floor(n / (B + 1)) + n nodes, because at each
level the split cells (more than B sources each) are disjoint and the leaves
are disjoint non-empty cells.  Checked on the oracle's trees for inputs built
to come close to it (CPU only)."""
import numpy as np
import pytest

import workloads as W


def bound(n, bits, B):
    return bits * (n // (B + 1)) + n


def near_pairs(n_pairs, offset, seed):
    rng = np.random.default_rng(seed)
    base = rng.random((n_pairs, 3))
    other = base + offset * rng.choice([-1.0, 1.0], size=(n_pairs, 3))
    p = np.concatenate([base, other])
    m = np.full((2 * n_pairs, 1), 1.0 / (2 * n_pairs))
    return np.concatenate([p, m], 1).astype(np.float32)


CASES = {
    # pairs one or two key quanta apart: chains of single-child cells almost to
    # the deepest level, the pattern that approaches the bound at B = 1
    "near_pairs": lambda: near_pairs(2048, 6e-7, 51),
    "near_pairs_wider": lambda: near_pairs(2048, 4e-5, 52),
    # a coincident cluster with one far source, and a plain Plummer sphere
    "coincident": lambda: np.concatenate([np.tile(np.float32([[0.3, 0.3, 0.3, 1e-3]]), (999, 1)),
                                          np.float32([[0.9, 0.1, 0.5, 1e-3]])]),
    "plummer": lambda: W.plummer(1 << 14, seed=53),
}


@pytest.mark.parametrize("key_bits,B", [(63, 1), (63, 2), (63, 16), (30, 1)])
@pytest.mark.parametrize("case", list(CASES))
def test_tree_fits_the_static_node_bound(orc, case, key_bits, B):
    p = CASES[case]()
    n = p.shape[0]
    cells = orc.Tree(p, key_bits=key_bits, leaf_cap=B).cells()
    nc = len(cells["level"])
    bits = key_bits // 3
    assert nc <= bound(n, bits, B)
    # the two parts of the bound separately
    internal = int((cells["is_leaf"] == 0).sum())
    for lvl in range(bits):
        assert int(((cells["is_leaf"] == 0) & (cells["level"] == lvl)).sum()) <= n // (B + 1)
    assert nc - internal <= n
    if case == "near_pairs" and key_bits == 63 and B == 1:
        # this input really comes near the bound (well above the n * 2 a
        # uniform cloud needs)
        assert nc > 0.6 * bound(n, bits, B)

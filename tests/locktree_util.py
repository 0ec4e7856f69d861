"""Host-side reading of the lock-based dense tree (bh_get_locked_tree) and
its comparison with the oracle's leaf-capacity-1 octree."""
import numpy as np


def locked_tree_sets(child, level, nxt, cap, n):
    """(internal cells as {(level, prefix)}, leaves as {(level, prefix): sorted
    particle tuple}) of a dense tree; prefixes are the top 3*level key bits."""
    n_cells = child.shape[0]
    first = cap - n_cells
    cells, leaves = set(), {}
    stack = [(cap - 1, 0, 0)]
    while stack:
        cid, lev, pre = stack.pop()
        row = cid - first
        assert 0 <= row < n_cells, "cell id out of range"
        assert level[row] == lev, "cell level mismatch"
        cells.add((lev, pre))
        for o in range(8):
            v = int(child[row, o])
            if v == -1:
                continue
            assert v != -2, "a slot is still locked"
            if v >= n:
                stack.append((v - n, lev + 1, pre * 8 + o))
            else:
                members = []
                while v != -1:
                    members.append(v)
                    v = int(nxt[v])
                    assert len(members) <= n, "chain cycle"
                leaves[(lev + 1, pre * 8 + o)] = tuple(sorted(members))
    return cells, leaves


def oracle_tree_sets(tree):
    c = tree.cells()
    perm_part = None
    cells, leaves = set(), {}
    # member particles of a leaf: the keys-sorted order agrees with the
    # partition at cell granularity, so a leaf's members are perm[start:start+count]
    perm = tree.perm()
    for lev, leaf, pre, st, cnt in zip(c["level"], c["is_leaf"], c["prefix"], c["start"],
                                       c["count"]):
        if leaf:
            leaves[(int(lev), int(pre))] = tuple(sorted(int(x) for x in perm[st:st + cnt]))
        else:
            cells.add((int(lev), int(pre)))
    del perm_part
    return cells, leaves

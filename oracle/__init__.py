"""ctypes loader for the fp64 CPU oracle (oracle.c).

Test infrastructure only: the tests, the smoke check and the CPU baseline leg
of the benchmark use it.  The product path (barnes_hut_tree_amd) never
imports it.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=False):
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_build.restype = P
        L.orc_build.argtypes = [P, i64, ctypes.c_int, ctypes.c_int]
        L.orc_build_curve.restype = P
        L.orc_build_curve.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_free.argtypes = [P]
        L.orc_bbox.argtypes = [P, P, P, P]
        L.orc_keys.argtypes = [P, P]
        L.orc_perm.argtypes = [P, P]
        L.orc_ncells.restype = i64
        L.orc_ncells.argtypes = [P]
        L.orc_cells.argtypes = [P] + [P] * 8
        L.orc_bh.argtypes = [P, P, P, i64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                             ctypes.c_int, P, P, P]
        L.orc_direct.argtypes = [P, i64, P, P, i64, ctypes.c_double, ctypes.c_double, P]
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_target_order.restype = ctypes.c_int
        L.orc_target_order.argtypes = [P, P, i64, P]
        L.orc_sbh.restype = ctypes.c_int
        L.orc_sbh.argtypes = [P, P, P, i64, P, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                              ctypes.c_double, ctypes.c_double, P, P, P]
        L.orc_bh_vote.restype = ctypes.c_int
        L.orc_bh_vote.argtypes = [P, i64, P, i64, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_int, P, P, P]
        L.orc_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f4(pos_mass):
    a = np.ascontiguousarray(pos_mass, dtype=np.float32)
    if a.ndim != 2 or a.shape[1] != 4:
        raise ValueError("expected an (n, 4) float32 array of x, y, z, m")
    return a


class Tree:
    """The oracle's octree over fp32 (x, y, z, m) sources, built in fp64."""

    CURVES = {"morton": 0, "hilbert": 1}

    def __init__(self, pos_mass, key_bits=63, leaf_cap=16, curve="morton"):
        self.src = _f4(pos_mass)  # kept alive: the C side keeps a pointer to it
        self.n = self.src.shape[0]
        self.key_bits = key_bits
        self.leaf_cap = leaf_cap
        self.curve = curve
        self._h = lib().orc_build_curve(_ptr(self.src), self.n, key_bits, leaf_cap,
                                        self.CURVES[curve])
        if not self._h:
            raise ValueError("invalid oracle build arguments")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_free(h)
            self._h = None

    def bbox(self):
        lo = np.zeros(3)
        hi = np.zeros(3)
        L = np.zeros(1)
        lib().orc_bbox(self._h, _ptr(lo), _ptr(hi), _ptr(L))
        return lo, hi, float(L[0])

    def keys(self):
        k = np.zeros(self.n, dtype=np.uint64)
        lib().orc_keys(self._h, _ptr(k))
        return k

    def perm(self):
        p = np.zeros(self.n, dtype=np.int64)
        lib().orc_perm(self._h, _ptr(p))
        return p

    def cells(self):
        nc = lib().orc_ncells(self._h)
        out = dict(
            level=np.zeros(nc, np.int32), is_leaf=np.zeros(nc, np.int32),
            prefix=np.zeros(nc, np.uint64), start=np.zeros(nc, np.int64),
            count=np.zeros(nc, np.int64), n_children=np.zeros(nc, np.int32),
            mass=np.zeros(nc), com=np.zeros((nc, 3)))
        lib().orc_cells(self._h, *[_ptr(out[k]) for k in
                                   ("level", "is_leaf", "prefix", "start", "count",
                                    "n_children", "mass", "com")])
        return out

    def gravity(self, theta, G=1.0, eps=0.0, targets=None, which=None, tie_mode=0):
        """(n_t, 4) fp64 (ax, ay, az, phi), interactions and near-ties per target.

        targets=None: the sources are the targets, self excluded.  which selects
        a subset of targets by index."""
        t = None if targets is None else _f4(targets)
        w = None if which is None else np.ascontiguousarray(which, dtype=np.int64)
        nt = (self.n if t is None else t.shape[0]) if w is None else w.shape[0]
        out = np.zeros((nt, 4))
        ni = np.zeros(nt, np.int64)
        nties = np.zeros(nt, np.int64)
        lib().orc_bh(self._h, _ptr(t), _ptr(w), nt, float(theta), float(G), float(eps),
                     int(tie_mode), _ptr(out), _ptr(ni), _ptr(nties))
        return out, ni, nties

    def target_order(self, targets):
        """Stable Morton order of separate query points on this tree's root cube."""
        q = _f4(targets)
        order = np.zeros(q.shape[0], np.int64)
        if lib().orc_target_order(self._h, _ptr(q), q.shape[0], _ptr(order)) != 0:
            raise MemoryError("orc_target_order")
        return order

    def sbh(self, targets, d=2, samples=1, seed=0, G=1.0, eps=0.0, which=None, group=64):
        """Stochastic Barnes-Hut estimate at separate query points (the tree
        must have leaf capacity 1): (n, 4) fp64 ax, ay, az, phi averaged over
        `samples`, the mean square of the per-sample potential, and the number
        of roulette draws within 1e-5 of their probability per query.  Queries
        share random numbers in groups of `group` consecutive queries of the
        Morton order."""
        q = _f4(targets)
        rank = np.empty(q.shape[0], np.int64)
        rank[self.target_order(q)] = np.arange(q.shape[0])
        w = np.arange(q.shape[0], dtype=np.int64) if which is None else \
            np.ascontiguousarray(which, dtype=np.int64)
        grp = np.ascontiguousarray(rank[w] // group, dtype=np.int64)
        out = np.zeros((w.shape[0], 4))
        sq = np.zeros(w.shape[0])
        near = np.zeros(w.shape[0], np.int64)
        rc = lib().orc_sbh(self._h, _ptr(q), _ptr(w), w.shape[0], _ptr(grp), int(d),
                           int(samples), int(seed) & 0xFFFFFFFFFFFFFFFF, float(G), float(eps),
                           _ptr(out), _ptr(sq), _ptr(near))
        if rc != 0:
            raise ValueError("orc_sbh: bad arguments")
        return out, sq, near

    def gravity_vote(self, theta, G=1.0, eps=0.0, group=64, groups=None, tie_mode=0):
        """Self-gravity by the warp vote over groups of `group` consecutive sorted
        sources: (n, 4) fp64 in the caller's order, interactions and near-ties
        per source, and the caller indices of the evaluated groups' members
        (all sources when groups is None)."""
        g = None if groups is None else np.ascontiguousarray(groups, dtype=np.int64)
        ng = 0 if g is None else g.shape[0]
        out = np.zeros((self.n, 4))
        ni = np.zeros(self.n, np.int64)
        nties = np.zeros(self.n, np.int64)
        rc = lib().orc_bh_vote(self._h, int(group), _ptr(g), ng, float(theta), float(G),
                               float(eps), int(tie_mode), _ptr(out), _ptr(ni), _ptr(nties))
        if rc != 0:
            raise ValueError("orc_bh_vote failed (%d)" % rc)
        perm = self.perm()
        if g is None:
            members = perm
        else:
            members = np.concatenate([perm[k * group:(k + 1) * group] for k in g])
        return out, ni, nties, members


def philox4x32_10(ctr, key):
    """The four output words of Philox4x32-10 for a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def direct(pos_mass, G=1.0, eps=0.0, targets=None, which=None):
    """The O(N^2) direct sum in fp64: (n_t, 4) (ax, ay, az, phi)."""
    src = _f4(pos_mass)
    t = None if targets is None else _f4(targets)
    w = None if which is None else np.ascontiguousarray(which, dtype=np.int64)
    nt = (src.shape[0] if t is None else t.shape[0]) if w is None else w.shape[0]
    out = np.zeros((nt, 4))
    lib().orc_direct(_ptr(src), src.shape[0], _ptr(t), _ptr(w), nt, float(G), float(eps),
                     _ptr(out))
    return out


def threads():
    return lib().orc_threads()


# ---------------------------------------------------------------------------
# Time stepping.  The pages advance their 5M-particle galaxy collision in time
# ([GASPHiA], page header) without naming the integrator; the reading taken is
# the kick-drift-kick leapfrog with the tree rebuilt every step.  The state is
# fp64; the tree of each step is built from the positions rounded to fp32,
# the precision sources are given in.
# ---------------------------------------------------------------------------
def _forces(x, m, theta, G, eps, key_bits, leaf_cap):
    p32 = np.concatenate([x, m[:, None]], axis=1).astype(np.float32)
    out, _, _ = Tree(p32, key_bits, leaf_cap).gravity(theta, G, eps)
    return out


def leapfrog(pos_mass, vel, dt, steps, theta, G=1.0, eps=0.0, key_bits=63, leaf_cap=16):
    """Kick-drift-kick leapfrog: per step v += a dt/2, x += v dt, a = a(x),
    v += a dt/2.  pos_mass (n, 4): x, y, z, m; vel (n, >= 3).  Returns fp64
    positions (n, 3), velocities (n, 3) and the last (n, 4) accelerations and
    potentials."""
    x = np.asarray(pos_mass, dtype=np.float64)[:, :3].copy()
    m = np.asarray(pos_mass, dtype=np.float64)[:, 3].copy()
    v = np.asarray(vel, dtype=np.float64)[:, :3].copy()
    a = _forces(x, m, theta, G, eps, key_bits, leaf_cap)
    for _ in range(steps):
        v += 0.5 * dt * a[:, :3]
        x += dt * v
        a = _forces(x, m, theta, G, eps, key_bits, leaf_cap)
        v += 0.5 * dt * a[:, :3]
    return x, v, a


def diagnostics(x, m, v, phi):
    """Conserved quantities, by their definitions: total mass, kinetic energy
    sum m v^2 / 2, potential energy sum m phi / 2 (phi: each particle's
    potential from all others), momentum sum m v and angular momentum
    sum m x cross v."""
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    m = np.asarray(m, np.float64)
    phi = np.asarray(phi, np.float64)
    return dict(mass=m.sum(), kinetic=0.5 * np.sum(m * np.sum(v * v, axis=1)),
                potential=0.5 * np.sum(m * phi), momentum=(m[:, None] * v).sum(axis=0),
                angular_momentum=(m[:, None] * np.cross(x, v)).sum(axis=0))


def node_hmax(tree, h):
    """Per cell of `tree` (pre-order, the order of Tree.cells), the largest h
    among its particles: the hmax the tree of [Tree] (树结构, 粒子领域搜索)
    keeps for its SPH neighbour search, by its definition.  h is given in the
    input order of the particles."""
    h = np.asarray(h, np.float32)
    c = tree.cells()
    perm = tree.perm()
    out = np.empty(len(c["level"]), np.float32)
    for k, (s, n) in enumerate(zip(c["start"], c["count"])):
        out[k] = h[perm[s:s + n]].max()
    return out

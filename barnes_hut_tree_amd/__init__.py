"""Barnes-Hut octree self-gravity for AMD MI355X (gfx950).

A thin ctypes binding over libbh.so (include/bh.h): argument marshalling only,
every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams.

    import torch, barnes_hut_tree_amd as bh
    tree = bh.BarnesHut(max_sources=n, key_bits=63, leaf_cap=16)
    tree.build(pos_mass)                  # (n, 4) float32 cuda tensor: x, y, z, m
    out = tree.gravity(theta=0.5, G=1.0, eps=1e-3)   # (n, 4): ax, ay, az, phi
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbh.so")

BH_OK = 0
BH_ERR_INVALID = -1
BH_ERR_OOM = -2
BH_ERR_HIP = -3
BH_ERR_CAPACITY = -4
BH_ERR_NONFINITE = -5
BH_ERR_NOT_BUILT = -6
BH_ERR_CONTENTION = -7

WALK_VOTE = 1        # BH_WALK_VOTE
WALK_UNSORTED = 2    # BH_WALK_UNSORTED

EXPORTS = ("bh_create", "bh_build", "bh_gravity", "bh_gravity_counted", "bh_gravity_ex", "bh_sbh", "bh_build_locked",
           "bh_get_locked_tree", "bh_direct", "bh_kick_drift",
           "bh_leapfrog_step", "bh_diagnostics", "bh_sync", "bh_destroy",
           "bh_status_string", "bh_get_keys", "bh_get_node_count", "bh_get_nodes", "bh_get_bbox",
           "bh_set_profiling", "bh_get_profile", "bh_node_hmax", "bh_get_cells",
           "bh_set_counting", "bh_get_interactions", "bh_gravity_static", "bh_get_walk_runs")

NODE_DTYPE_FIELDS = [("com_x", "f4"), ("com_y", "f4"), ("com_z", "f4"), ("mass", "f4"),
                     ("start", "u4"), ("count", "u4"), ("skip", "u4"), ("meta", "u4")]


class BHError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))


class _Params(ctypes.Structure):
    _fields_ = [("key_bits", ctypes.c_int32), ("leaf_cap", ctypes.c_int32),
                ("node_capacity", ctypes.c_int64), ("key_curve", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


CURVES = {"morton": 0, "hilbert": 1}   # BH_CURVE_MORTON, BH_CURVE_HILBERT


_lib = None


def load_library():
    """Load libbh.so (built in-tree).  Fails loudly when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbh.so is not built: run `python -m barnes_hut_tree_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sigs = {
        "bh_create": [ctypes.POINTER(P), i64, i64, ctypes.POINTER(_Params)],
        "bh_build": [P, P, i64, P],
        "bh_gravity": [P, P, i64, f32, f32, f32, P, P],
        "bh_gravity_counted": [P, P, i64, f32, f32, f32, P, P, P],
        "bh_gravity_ex": [P, P, i64, f32, f32, f32, ctypes.c_uint32, P, P, P],
        "bh_sbh": [P, P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, f32, f32, P, P],
        "bh_build_locked": [P, P, i64, P],
        "bh_get_locked_tree": [P, ctypes.POINTER(i64), ctypes.POINTER(i64), P, P, P, P],
        "bh_direct": [P, i64, P, i64, f32, f32, P, P],
        "bh_kick_drift": [P, P, P, i64, f32, f32, P],
        "bh_leapfrog_step": [P, P, P, P, i64, f32, f32, f32, f32, P],
        "bh_diagnostics": [P, P, P, P, i64, P, P],
        "bh_sync": [P],
        "bh_destroy": [P],
        "bh_get_keys": [P, P, P, P],
        "bh_get_node_count": [P, ctypes.POINTER(i64), P],
        "bh_get_nodes": [P, P, i64, P],
        "bh_get_bbox": [P, P, P, P, P],
        "bh_set_profiling": [P, i32],
        "bh_get_profile": [P, P, i32],
        "bh_node_hmax": [P, P, i64, P, i64, P],
        "bh_get_cells": [P, ctypes.POINTER(i64), P, P, P, P],
        "bh_set_counting": [P, i32],
        "bh_get_interactions": [P, ctypes.POINTER(ctypes.c_uint64)],
        "bh_gravity_static": [P, i64, ctypes.POINTER(_Params), f32, f32, f32, P, P],
        "bh_get_walk_runs": [P, P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.bh_status_string.argtypes = [ctypes.c_int]
    L.bh_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status):
    return load_library().bh_status_string(int(status)).decode()


def _check(status, where):
    if status != BH_OK:
        raise BHError(status, where)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
        raise TypeError("%s must be a float32 CUDA tensor" % name)
    if t.dim() != 2 or t.shape[1] != 4 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous (n, 4) tensor" % name)
    return t


def _counter(t):
    """An interaction counter must be one int64 element of device memory on
    the current device (the walk adds to it with a device atomic)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.int64:
        raise TypeError("interactions must be an int64 CUDA tensor")
    if t.numel() != 1 or not t.is_contiguous():
        raise ValueError("interactions must be a contiguous 1-element tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError("interactions must be on the current device")
    return t


class BarnesHut:
    """One octree context (bh_ctx) on the current device."""

    def __init__(self, max_sources, max_targets=0, key_bits=63, leaf_cap=16, node_capacity=0,
                 curve="morton"):
        L = load_library()
        self._h = ctypes.c_void_p()
        p = _Params(int(key_bits), int(leaf_cap), int(node_capacity), CURVES[curve], 0)
        _check(L.bh_create(ctypes.byref(self._h), int(max_sources), int(max_targets),
                           ctypes.byref(p)), "bh_create")
        self.max_sources = int(max_sources)
        self.max_targets = int(max_targets)
        self.key_bits = int(key_bits)
        self.leaf_cap = int(leaf_cap)
        self.curve = curve
        self.n = 0

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            load_library().bh_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def build(self, pos_mass):
        t = _rows(pos_mass, "pos_mass")
        _check(load_library().bh_build(self._h, ctypes.c_void_p(t.data_ptr()), t.shape[0],
                                       _stream()), "bh_build")
        self.n = t.shape[0]

    def gravity(self, theta, G=1.0, eps=0.0, targets=None, out=None, interactions=None,
                flags=0):
        """(n_targets, 4) float32: ax, ay, az, phi in the caller's order.

        targets=None: the built sources, each excluding itself.
        interactions: optional uint64 (int64) CUDA tensor of 1 element that the
        interaction count is added to.  flags: WALK_VOTE / WALK_UNSORTED."""
        import torch
        if targets is not None:
            targets = _rows(targets, "targets")
            nt = targets.shape[0]
            tp = ctypes.c_void_p(targets.data_ptr())
        else:
            nt = self.n
            tp = ctypes.c_void_p()
        if out is None:
            out = torch.empty((nt, 4), dtype=torch.float32, device="cuda")
        else:
            _rows(out, "out")
            if out.shape[0] != nt:
                raise ValueError("out must have %d rows" % nt)
        if interactions is not None:
            _counter(interactions)
        if targets is not None and nt == 0:
            # an empty tensor's data pointer is NULL, which would mean "self"
            return out
        L = load_library()
        if flags:
            cp = ctypes.c_void_p() if interactions is None else ctypes.c_void_p(
                interactions.data_ptr())
            st = L.bh_gravity_ex(self._h, tp, nt, float(theta), float(G), float(eps), int(flags),
                                 ctypes.c_void_p(out.data_ptr()), cp, _stream())
        elif interactions is None:
            st = L.bh_gravity(self._h, tp, nt, float(theta), float(G), float(eps),
                              ctypes.c_void_p(out.data_ptr()), _stream())
        else:
            st = L.bh_gravity_counted(self._h, tp, nt, float(theta), float(G), float(eps),
                                      ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(interactions.data_ptr()), _stream())
        _check(st, "bh_gravity")
        return out

    def build_locked(self, pos_mass):
        """The lock-based dense build (bh_build_locked); replaces the tree."""
        t = _rows(pos_mass, "pos_mass")
        _check(load_library().bh_build_locked(self._h, ctypes.c_void_p(t.data_ptr()), t.shape[0],
                                              _stream()), "bh_build_locked")
        self.n = t.shape[0]

    def locked_tree(self):
        """(child (n_cells, 8), level (n_cells,), next (n,), cap) of the last
        lock-based build as CUDA int32 tensors; row r is cell cap - n_cells + r."""
        import torch
        L = load_library()
        nc, cap = ctypes.c_int64(), ctypes.c_int64()
        _check(L.bh_get_locked_tree(self._h, ctypes.byref(nc), ctypes.byref(cap), None, None, None,
                                    _stream()), "bh_get_locked_tree")
        child = torch.empty((max(nc.value, 1), 8), dtype=torch.int32, device="cuda")
        level = torch.empty(max(nc.value, 1), dtype=torch.int32, device="cuda")
        nxt = torch.empty(max(self.n, 1), dtype=torch.int32, device="cuda")
        _check(L.bh_get_locked_tree(self._h, ctypes.byref(nc), ctypes.byref(cap),
                                    ctypes.c_void_p(child.data_ptr()),
                                    ctypes.c_void_p(level.data_ptr()),
                                    ctypes.c_void_p(nxt.data_ptr()), _stream()),
               "bh_get_locked_tree")
        return child[:nc.value], level[:nc.value], nxt[:self.n], cap.value

    def sbh(self, targets, d=2, samples=1, seed=0, G=1.0, eps=0.0, out=None):
        """Stochastic Barnes-Hut estimate at separate targets (bh_sbh; the
        context needs leaf_cap=1): (n_targets, 4) float32 in the caller's order."""
        import torch
        targets = _rows(targets, "targets")
        nt = targets.shape[0]
        if out is None:
            out = torch.empty((nt, 4), dtype=torch.float32, device="cuda")
        else:
            _rows(out, "out")
        if nt == 0:
            return out
        _check(load_library().bh_sbh(self._h, ctypes.c_void_p(targets.data_ptr()), nt, int(d),
                                     int(samples), int(seed) & 0xFFFFFFFFFFFFFFFF, float(G),
                                     float(eps), ctypes.c_void_p(out.data_ptr()), _stream()),
               "bh_sbh")
        return out

    def count_interactions(self, theta, eps=0.0, targets=None, flags=0):
        import torch
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.gravity(theta, 1.0, eps, targets=targets, interactions=cnt, flags=flags)
        return int(cnt.item())

    def set_counting(self, on=True):
        """Count interactions of every following gravity() call that has no
        counter of its own (bh_set_counting); read with interactions()."""
        _check(load_library().bh_set_counting(self._h, int(bool(on))), "bh_set_counting")

    def walk_runs(self):
        """(uneven, starts) of the last per-target walk (bh_get_walk_runs):
        whether it walked XCD runs balanced on an earlier walk's times, and
        then the first group of each of the eight runs plus the group count."""
        import numpy as np
        starts = np.zeros(9, np.uint32)
        uneven = ctypes.c_int32()
        _check(load_library().bh_get_walk_runs(self._h, ctypes.c_void_p(starts.ctypes.data),
                                               ctypes.byref(uneven), None), "bh_get_walk_runs")
        return bool(uneven.value), (starts.tolist() if uneven.value else None)

    def walk_split(self):
        """How many groups the last per-target walk walked as four waves of 16
        targets each (bh_get_walk_runs)."""
        uneven, split = ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().bh_get_walk_runs(self._h, None, ctypes.byref(uneven),
                                               ctypes.byref(split)), "bh_get_walk_runs")
        return int(split.value)

    def interactions(self):
        """Interactions of the last counted gravity() call (bh_get_interactions)."""
        v = ctypes.c_uint64()
        _check(load_library().bh_get_interactions(self._h, ctypes.byref(v)),
               "bh_get_interactions")
        return v.value

    def cells(self):
        """Per node in pre-order (bh_get_cells): level (uint8), key prefix of
        the cell's place on its level's grid (int64 view of uint64) and source
        count (int32 view of uint32), as CUDA tensors."""
        import torch
        L = load_library()
        nn = ctypes.c_int64()
        _check(L.bh_get_cells(self._h, ctypes.byref(nn), None, None, None, _stream()),
               "bh_get_cells")
        k = max(nn.value, 1)
        level = torch.empty(k, dtype=torch.uint8, device="cuda")
        prefix = torch.empty(k, dtype=torch.int64, device="cuda")
        count = torch.empty(k, dtype=torch.int32, device="cuda")
        _check(L.bh_get_cells(self._h, ctypes.byref(nn), ctypes.c_void_p(level.data_ptr()),
                              ctypes.c_void_p(prefix.data_ptr()),
                              ctypes.c_void_p(count.data_ptr()), _stream()), "bh_get_cells")
        m = nn.value
        return dict(level=level[:m], prefix=prefix[:m], count=count[:m])

    def sync(self):
        _check(load_library().bh_sync(self._h), "bh_sync")

    def status(self):
        return load_library().bh_sync(self._h)

    def keys(self):
        """Sorted Morton keys (int64 view of uint64) and the sorted permutation."""
        import torch
        k = torch.empty(self.n, dtype=torch.int64, device="cuda")
        p = torch.empty(self.n, dtype=torch.int32, device="cuda")
        _check(load_library().bh_get_keys(self._h, ctypes.c_void_p(k.data_ptr()),
                                          ctypes.c_void_p(p.data_ptr()), _stream()), "bh_get_keys")
        return k, p

    def node_count(self):
        n = ctypes.c_int64()
        _check(load_library().bh_get_node_count(self._h, ctypes.byref(n), _stream()),
               "bh_get_node_count")
        return n.value

    def nodes(self):
        """Node records as an (n_nodes, 8) int32 CUDA tensor (bh_node layout)."""
        import torch
        nn = self.node_count()
        buf = torch.empty((max(nn, 1), 8), dtype=torch.int32, device="cuda")
        _check(load_library().bh_get_nodes(self._h, ctypes.c_void_p(buf.data_ptr()), nn,
                                           _stream()), "bh_get_nodes")
        return buf[:nn]

    def node_hmax(self, h):
        """Largest h among each node's sources (bh_node_hmax): h is a float32
        CUDA tensor of the built sources' smoothing lengths in their order;
        returns a float32 CUDA tensor with one value per node (node order)."""
        import torch
        if not isinstance(h, torch.Tensor) or h.device.type != "cuda" or h.dtype != torch.float32:
            raise TypeError("h must be a float32 CUDA tensor")
        if h.dim() != 1 or not h.is_contiguous():
            raise ValueError("h must be a contiguous 1-D tensor")
        nn = self.node_count() if h.shape[0] > 0 else 0
        out = torch.empty(max(nn, 1), dtype=torch.float32, device="cuda")
        _check(load_library().bh_node_hmax(self._h, ctypes.c_void_p(h.data_ptr()), h.shape[0],
                                           ctypes.c_void_p(out.data_ptr()), nn, _stream()),
               "bh_node_hmax")
        return out[:nn]

    def bbox(self):
        lo = (ctypes.c_double * 3)()
        hi = (ctypes.c_double * 3)()
        L = ctypes.c_double()
        _check(load_library().bh_get_bbox(self._h, lo, hi, ctypes.byref(L), _stream()),
               "bh_get_bbox")
        return list(lo), list(hi), L.value

    def leapfrog_step(self, pos_mass, vel, acc_pot, dt, theta, G=1.0, eps=0.0):
        """One kick-drift-kick step in place (bh_leapfrog_step); acc_pot must
        hold the forces at the current positions."""
        pos_mass = _rows(pos_mass, "pos_mass")
        vel = _rows(vel, "vel")
        acc_pot = _rows(acc_pot, "acc_pot")
        n = pos_mass.shape[0]
        if vel.shape[0] != n or acc_pot.shape[0] != n:
            raise ValueError("pos_mass, vel and acc_pot need the same number of rows")
        _check(load_library().bh_leapfrog_step(
            self._h, ctypes.c_void_p(pos_mass.data_ptr()), ctypes.c_void_p(vel.data_ptr()),
            ctypes.c_void_p(acc_pot.data_ptr()), n, float(dt), float(theta), float(G),
            float(eps), _stream()), "bh_leapfrog_step")
        self.n = n

    def diagnostics(self, pos_mass, vel, acc_pot):
        """dict of fp64 conserved quantities (bh_diagnostics); waits for them."""
        import torch
        pos_mass = _rows(pos_mass, "pos_mass")
        vel = _rows(vel, "vel")
        acc_pot = _rows(acc_pot, "acc_pot")
        out = torch.empty(10, dtype=torch.float64, device="cuda")
        _check(load_library().bh_diagnostics(
            self._h, ctypes.c_void_p(pos_mass.data_ptr()), ctypes.c_void_p(vel.data_ptr()),
            ctypes.c_void_p(acc_pot.data_ptr()), pos_mass.shape[0],
            ctypes.c_void_p(out.data_ptr()), _stream()), "bh_diagnostics")
        o = out.cpu().tolist()
        return dict(mass=o[0], kinetic=o[1], potential=o[2], momentum=o[3:6],
                    angular_momentum=o[6:9], count=o[9])

    def set_profiling(self, on=True):
        _check(load_library().bh_set_profiling(self._h, int(bool(on))), "bh_set_profiling")

    def profile(self):
        """Device ms of [bbox+keys, sort, tree with centres of mass, walk]."""
        ms = (ctypes.c_float * 4)()
        _check(load_library().bh_get_profile(self._h, ms, 4), "bh_get_profile")
        return list(ms)


def direct(src, G=1.0, eps=0.0, targets=None, out=None):
    """All-pairs direct sum (bh_direct): (n_targets, 4) float32 ax, ay, az, phi.
    targets=None: the sources themselves, each excluding itself."""
    import torch
    src = _rows(src, "src")
    if targets is not None:
        targets = _rows(targets, "targets")
        nt, tp = targets.shape[0], ctypes.c_void_p(targets.data_ptr())
    else:
        nt, tp = src.shape[0], ctypes.c_void_p()
    if out is None:
        out = torch.empty((nt, 4), dtype=torch.float32, device="cuda")
    else:
        _rows(out, "out")
    if nt == 0:   # an empty tensor's data pointer is NULL, which would mean "self"
        return out
    _check(load_library().bh_direct(ctypes.c_void_p(src.data_ptr()), src.shape[0], tp, nt,
                                    float(G), float(eps), ctypes.c_void_p(out.data_ptr()),
                                    _stream()), "bh_direct")
    return out


def gravity_static(pos_mass, theta, G=1.0, eps=0.0, key_bits=63, leaf_cap=16, curve="morton",
                   out=None):
    """One self-gravity step (build + walk) that allocates no device memory in
    the library (bh_gravity_static): its scratch is a static device array.
    Returns (n, 4) float32 ax, ay, az, phi in the caller's order."""
    import torch
    pos_mass = _rows(pos_mass, "pos_mass")
    n = pos_mass.shape[0]
    if out is None:
        out = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    else:
        _rows(out, "out")
        if out.shape[0] != n:
            raise ValueError("out must have %d rows" % n)
    p = _Params(int(key_bits), int(leaf_cap), 0, CURVES[curve], 0)
    _check(load_library().bh_gravity_static(ctypes.c_void_p(pos_mass.data_ptr()), n,
                                            ctypes.byref(p), float(theta), float(G), float(eps),
                                            ctypes.c_void_p(out.data_ptr()), _stream()),
           "bh_gravity_static")
    return out


def kick_drift(pos_mass, vel, acc_pot, dt_kick, dt_drift):
    """vel += acc dt_kick; pos += vel dt_drift, in place (bh_kick_drift)."""
    vel = _rows(vel, "vel")
    n = vel.shape[0]
    pp = ctypes.c_void_p() if pos_mass is None else ctypes.c_void_p(_rows(pos_mass, "pos_mass")
                                                                     .data_ptr())
    ap = ctypes.c_void_p() if acc_pot is None else ctypes.c_void_p(_rows(acc_pot, "acc_pot")
                                                                    .data_ptr())
    _check(load_library().bh_kick_drift(pp, ctypes.c_void_p(vel.data_ptr()), ap, n,
                                        float(dt_kick), float(dt_drift), _stream()),
           "bh_kick_drift")


def nodes_numpy(node_tensor):
    """Split an (n, 8) int32 node tensor (on any device) into named numpy fields."""
    import numpy as np
    a = node_tensor.cpu().numpy()
    f = a[:, :4].view(np.float32)
    u = a[:, 4:].view(np.uint32)
    meta = u[:, 3]
    return dict(com=f[:, :3].copy(), mass=f[:, 3].copy(), start=u[:, 0].copy(),
                count=u[:, 1].copy(), skip=u[:, 2].copy(), level=(meta & 0xff).astype(np.int32),
                is_leaf=((meta >> 8) & 1).astype(np.int32))

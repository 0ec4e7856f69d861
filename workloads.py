"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds only input generation (no part of the gravity method's
arithmetic).  Both the HIP path's tests/benchmark and the CPU oracle take
their inputs from here, so the two sides always see identical bytes.

Every array is generated in fp64 with numpy's PCG64 (`default_rng(seed)`)
and then cast to fp32 float4 rows (x, y, z, m).

Workloads (the shapes come from the pages; sizes and seeds are fixed here):
  uniform_cube   N=4096 particles uniform in the unit cube, m = 1/N
  lattice        the 100^3 regular cube lattice of [GASPHiA] 性能测试与对比,
                 cell-centred (i + 0.5)/100, equal masses; lattice or shuffled order
  plummer        a Plummer sphere (scale a = 1, truncated at 20a), equal masses;
                 the 1M-particle random-vs-sorted and theta-sweep runs of
                 [GASPHiA] 排序算法 / 精度与加速比验证
  galaxy_pair    two galaxies (Hernquist halo 80% of mass + exponential sech^2
                 disk 20%), standing in for the DICE initial conditions of the
                 5M-particle collision on the [GASPHiA] page (not available)
  surface_sources / grid_queries / box_queries
                 area-uniform point masses on a seeded union of spheres and tori
                 with grid or random queries, standing in for the 116-mesh set
                 of the stochastic Barnes-Hut notes (not available)
"""
import numpy as np

PLUMMER_TRUNC = 20.0          # Plummer radius truncation, in units of a
HERNQUIST_A = 5.0             # assumed halo scale length
HERNQUIST_TRUNC = 20.0        # halo truncation, in units of a_h
DISK_RD, DISK_Z0 = 1.0, 0.1   # disk scale length and sech^2 scale height


def _float4(xyz, m):
    out = np.empty((xyz.shape[0], 4), dtype=np.float32)
    out[:, :3] = xyz
    out[:, 3] = m
    return out


def _isotropic(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def uniform_cube(n=4096, seed=1):
    rng = np.random.default_rng(seed)
    return _float4(rng.random((n, 3)), 1.0 / n)


def lattice(side=100, shuffled=False, seed=2):
    """side^3 particles at cell centres (i + 0.5)/side, index ix + side*iy + side^2*iz."""
    i = (np.arange(side) + 0.5) / side
    iz, iy, ix = np.meshgrid(i, i, i, indexing="ij")
    xyz = np.stack([ix.ravel(), iy.ravel(), iz.ravel()], axis=1)
    n = xyz.shape[0]
    out = _float4(xyz, 1.0 / n)
    if shuffled:
        out = out[np.random.default_rng(seed).permutation(n)]
    return out


def plummer(n=1 << 20, a=1.0, seed=3):
    """Equal-mass Plummer sphere: r = a / sqrt(u^(-2/3) - 1), u the enclosed mass
    fraction, drawn up to the fraction inside PLUMMER_TRUNC * a."""
    rng = np.random.default_rng(seed)
    c = PLUMMER_TRUNC
    umax = (c * c / (c * c + 1.0)) ** 1.5
    u = rng.uniform(0.0, 1.0, n) * umax
    u = np.where(u <= 0.0, np.finfo(float).tiny, u)
    r = a / np.sqrt(u ** (-2.0 / 3.0) - 1.0)
    xyz = r[:, None] * _isotropic(rng, n)
    return _float4(xyz, 1.0 / n)


def _hernquist(rng, n, a):
    c = HERNQUIST_TRUNC
    umax = (c / (c + 1.0)) ** 2
    s = np.sqrt(rng.uniform(0.0, 1.0, n) * umax)
    r = a * s / (1.0 - s)
    return r[:, None] * _isotropic(rng, n)


def _exp_disk(rng, n, rd, z0):
    R = np.empty(0)
    while R.size < n:
        x = rng.gamma(2.0, rd, 2 * n)
        R = np.concatenate([R, x[x < 10.0 * rd]])
    R = R[:n]
    z = np.empty(0)
    while z.size < n:
        x = z0 * np.arctanh(2.0 * rng.uniform(0.0, 1.0, 2 * n) - 1.0)
        z = np.concatenate([z, x[np.abs(x) < 10.0 * z0]])
    z = z[:n]
    phi = rng.uniform(0.0, 2.0 * np.pi, n)
    return np.stack([R * np.cos(phi), R * np.sin(phi), z], axis=1)


def galaxy_pair(n=5_000_000, seed=4, offset=20.0, rel_speed=0.5):
    """Two galaxies of unit mass each, 80% halo / 20% disk particles of equal
    mass, centred at (+-offset/2, 0, 0).  Returns (float4 pos+mass, velocities);
    the velocities (+-rel_speed/2 along y) are not used by a gravity step."""
    rng = np.random.default_rng(seed)
    per = n // 2
    n_halo = (per * 4) // 5
    n_disk = per - n_halo
    parts, vel = [], []
    for sign in (-1.0, 1.0):
        g = np.concatenate([_hernquist(rng, n_halo, HERNQUIST_A),
                            _exp_disk(rng, n_disk, DISK_RD, DISK_Z0)])
        g[:, 0] += sign * offset / 2.0
        parts.append(g)
        v = np.zeros_like(g)
        v[:, 1] = sign * rel_speed / 2.0
        vel.append(v)
    xyz = np.concatenate(parts)
    return _float4(xyz, 2.0 / xyz.shape[0]), np.concatenate(vel).astype(np.float32)


def _random_rotation(rng):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def surface_shapes(seed):
    """3-6 spheres/tori with disjoint bounding spheres inside [-0.9, 0.9]^3."""
    rng = np.random.default_rng(seed)
    k = int(rng.integers(3, 7))
    shapes = []
    while len(shapes) < k:
        if rng.random() < 0.5:
            s = dict(kind="sphere", radius=rng.uniform(0.15, 0.4))
            bound = s["radius"]
        else:
            s = dict(kind="torus", major=rng.uniform(0.2, 0.45), minor=rng.uniform(0.05, 0.15),
                     rot=_random_rotation(rng))
            bound = s["major"] + s["minor"]
        for _ in range(1000):
            c = rng.uniform(-0.9 + bound, 0.9 - bound, 3) if bound < 0.9 else np.zeros(3)
            if all(np.linalg.norm(c - o["centre"]) > bound + o["bound"] for o in shapes):
                s["centre"], s["bound"] = c, bound
                shapes.append(s)
                break
        else:
            break
    return shapes


def _area(s):
    if s["kind"] == "sphere":
        return 4.0 * np.pi * s["radius"] ** 2
    return 4.0 * np.pi ** 2 * s["major"] * s["minor"]


def _sample_surface(rng, s, n):
    if s["kind"] == "sphere":
        return s["centre"] + s["radius"] * _isotropic(rng, n)
    R, r = s["major"], s["minor"]
    pts = np.empty((0, 3))
    while pts.shape[0] < n:
        u = rng.uniform(0.0, 2.0 * np.pi, 2 * n)
        v = rng.uniform(0.0, 2.0 * np.pi, 2 * n)
        keep = rng.uniform(0.0, R + r, 2 * n) < R + r * np.cos(v)
        u, v = u[keep], v[keep]
        p = np.stack([(R + r * np.cos(v)) * np.cos(u), (R + r * np.cos(v)) * np.sin(u),
                      r * np.sin(v)], axis=1)
        pts = np.concatenate([pts, p])
    return s["centre"] + pts[:n] @ s["rot"].T


def surface_sources(m_sources=1 << 20, seed=10):
    """m_sources area-uniform points on surface_shapes(seed); each mass is the
    total area over m_sources (area weights)."""
    shapes = surface_shapes(seed)
    rng = np.random.default_rng(seed + 1000)
    areas = np.array([_area(s) for s in shapes])
    counts = rng.multinomial(m_sources, areas / areas.sum())
    xyz = np.concatenate([_sample_surface(rng, s, c) for s, c in zip(shapes, counts)])
    xyz = xyz[rng.permutation(xyz.shape[0])]
    return _float4(xyz, areas.sum() / m_sources)


def grid_queries(side=100):
    g = np.linspace(-1.0, 1.0, side)
    z, y, x = np.meshgrid(g, g, g, indexing="ij")
    return _float4(np.stack([x.ravel(), y.ravel(), z.ravel()], axis=1), 0.0)


def box_queries(n=1_000_000, seed=20):
    rng = np.random.default_rng(seed)
    return _float4(rng.uniform(-1.0, 1.0, (n, 3)), 0.0)


def uniform_box(n, seed=5):
    """Uniform random particles in the unit cube, for size sweeps."""
    rng = np.random.default_rng(seed)
    return _float4(rng.random((n, 3)), 1.0 / max(n, 1))

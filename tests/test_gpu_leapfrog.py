"""Time stepping through the C ABI (bh_kick_drift, bh_leapfrog_step,
bh_diagnostics) against the oracle's fp64 leapfrog and the definitions of the
conserved quantities."""
import numpy as np
import pytest

import workloads as W

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


def vel4(v):
    v = np.asarray(v, np.float32)
    return np.concatenate([v[:, :3], np.zeros((v.shape[0], 1), np.float32)], 1)


def test_kick_drift_elementwise():
    import barnes_hut_tree_amd as bh
    rng = np.random.default_rng(60)
    n = 100003
    p = rng.standard_normal((n, 4)).astype(np.float32)
    v = rng.standard_normal((n, 4)).astype(np.float32)
    a = rng.standard_normal((n, 4)).astype(np.float32)
    tp, tv, ta = (torch.from_numpy(x).cuda() for x in (p, v, a))
    bh.kick_drift(tp, tv, ta, 0.015625, 0.03125)
    gv, gp = tv.cpu().numpy(), tp.cpu().numpy()
    ev = (v[:, :3].astype(np.float64) + a[:, :3].astype(np.float64) * 0.015625).astype(np.float32)
    ep = (p[:, :3].astype(np.float64) + gv[:, :3].astype(np.float64) * 0.03125).astype(np.float32)
    # one fused multiply-add per component: exact up to the final rounding
    assert np.allclose(gv[:, :3], ev, rtol=2e-7, atol=1e-30)
    assert np.allclose(gp[:, :3], ep, rtol=2e-7, atol=1e-30)
    assert np.array_equal(gv[:, 3], v[:, 3]) and np.array_equal(gp[:, 3], p[:, 3])
    # kick only (positions untouched, may be absent), drift only (forces absent)
    bh.kick_drift(None, tv, ta, 0.5, 0.0)
    bh.kick_drift(tp, tv, None, 0.0, 0.25)
    torch.cuda.synchronize()


@pytest.mark.parametrize("theta,B", [(0.5, 16), (0.7, 4)])
def test_leapfrog_matches_oracle(orc, theta, B):
    import barnes_hut_tree_amd as bh
    p, v = W.galaxy_pair(n=20000, seed=4)
    eps, dt, steps = 0.02, 0.05, 10
    log("leapfrog galaxy 2e4 theta", theta, "B", B)
    t = bh.BarnesHut(p.shape[0], 0, 63, B)
    tp = torch.from_numpy(p.copy()).cuda()
    tv = torch.from_numpy(vel4(v)).cuda()
    t.build(tp)
    ta = t.gravity(theta, 1.0, eps)
    for _ in range(steps):
        t.leapfrog_step(tp, tv, ta, dt, theta, 1.0, eps)
    t.sync()
    gx, gv = tp.cpu().numpy()[:, :3].astype(np.float64), tv.cpu().numpy()[:, :3].astype(np.float64)
    ox, ov, oa = orc.leapfrog(p, v, dt, steps, theta, 1.0, eps, leaf_cap=B)
    x0, v0 = p[:, :3].astype(np.float64), v[:, :3].astype(np.float64)
    ex = np.linalg.norm(gx - ox, axis=1) / np.linalg.norm(ox - x0, axis=1)
    ev = np.linalg.norm(gv - ov, axis=1) / np.linalg.norm(ov - v0, axis=1)
    log("  displacement rel err p99 %.3g max %.3g; velocity change p99 %.3g max %.3g" % (
        np.percentile(ex, 99), ex.max(), np.percentile(ev, 99), ev.max()))
    assert np.percentile(ex, 99) < 1e-3 and np.percentile(ev, 99) < 1e-3
    # the final forces too
    ga = ta.cpu().numpy().astype(np.float64)
    ea = np.linalg.norm(ga[:, :3] - oa[:, :3], axis=1) / np.linalg.norm(oa[:, :3], axis=1)
    assert np.percentile(ea, 99) < 1e-3
    t.close()


def test_diagnostics_match_definitions(orc):
    import barnes_hut_tree_amd as bh
    p, v = W.galaxy_pair(n=300001, seed=4)
    rng = np.random.default_rng(61)
    v = v + 0.1 * rng.standard_normal(v.shape).astype(np.float32)
    t = bh.BarnesHut(p.shape[0], 0, 63, 16)
    tp = torch.from_numpy(p).cuda()
    tv = torch.from_numpy(vel4(v)).cuda()
    t.build(tp)
    ta = t.gravity(0.5, 1.0, 0.02)
    d = t.diagnostics(tp, tv, ta)
    a = ta.cpu().numpy()
    ref = orc.diagnostics(p[:, :3], p[:, 3], v, a[:, 3])
    assert d["count"] == p.shape[0]
    for k in ("mass", "kinetic", "potential"):
        assert d[k] == pytest.approx(ref[k], rel=1e-12), k
    scale_p = np.sum(p[:, 3].astype(np.float64) * np.linalg.norm(v, axis=1))
    assert np.max(np.abs(np.array(d["momentum"]) - ref["momentum"])) < 1e-12 * scale_p
    scale_l = np.sum(p[:, 3].astype(np.float64) * np.linalg.norm(p[:, :3], axis=1) *
                     np.linalg.norm(v, axis=1))
    assert np.max(np.abs(np.array(d["angular_momentum"]) - ref["angular_momentum"])) < \
        1e-12 * scale_l
    # deterministic order
    assert t.diagnostics(tp, tv, ta) == d
    t.close()


def test_galaxy_pair_5m_conserves(orc):
    # the benchmark's system: a few steps at full size keep energy and
    # momentum to the level the tree's force errors allow
    import barnes_hut_tree_amd as bh
    p, v = W.galaxy_pair()
    t = bh.BarnesHut(p.shape[0], 0, 63, 16)
    tp = torch.from_numpy(p).cuda()
    tv = torch.from_numpy(vel4(v)).cuda()
    t.build(tp)
    ta = t.gravity(0.5, 1.0, 0.02)
    d0 = t.diagnostics(tp, tv, ta)
    for _ in range(5):
        t.leapfrog_step(tp, tv, ta, 0.05, 0.5, 1.0, 0.02)
    d1 = t.diagnostics(tp, tv, ta)
    t.sync()
    e0 = d0["kinetic"] + d0["potential"]
    e1 = d1["kinetic"] + d1["potential"]
    dp = np.abs(np.array(d1["momentum"]) - np.array(d0["momentum"]))
    log("  5M galaxy, 5 steps: dE/E %.3g, |dP| %s, K %.5g -> %.5g" % (
        (e1 - e0) / abs(e0), dp, d0["kinetic"], d1["kinetic"]))
    assert d1["mass"] == pytest.approx(d0["mass"], rel=1e-12)
    assert abs(e1 - e0) < 1e-3 * abs(e0)
    assert np.all(dp < 1e-4)
    assert d1["kinetic"] > d0["kinetic"]   # the cold halos start to fall in
    t.close()


def test_leapfrog_argument_errors():
    import ctypes

    import barnes_hut_tree_amd as bh
    L = bh.load_library()
    t = bh.BarnesHut(64, 0, 63, 16)
    x = torch.zeros((64, 4), device="cuda")
    P = ctypes.c_void_p
    xp = P(x.data_ptr())
    assert L.bh_leapfrog_step(t._h, xp, xp, xp, 65, 0.1, 0.5, 1.0, 0.0, None) == bh.BH_ERR_INVALID
    assert L.bh_leapfrog_step(t._h, xp, xp, xp, 64, float("nan"), 0.5, 1.0, 0.0, None) == \
        bh.BH_ERR_INVALID
    assert L.bh_kick_drift(None, xp, None, 64, 0.1, 0.0, None) == bh.BH_ERR_INVALID
    assert L.bh_kick_drift(None, xp, xp, 64, 0.1, 0.1, None) == bh.BH_ERR_INVALID
    assert L.bh_diagnostics(t._h, xp, xp, xp, 64, None, None) == bh.BH_ERR_INVALID
    t.close()

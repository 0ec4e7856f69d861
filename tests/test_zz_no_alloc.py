"""bh_gravity_static, the step that allocates nothing (its scratch is a static
device array of the library), against the context path it varies, bh_build +
bh_gravity on a context with the same parameters: bit-identical outputs on two
calls in a row, the second with a smaller input (the array then holds the
larger tree of the first call); the size limit and the argument checks."""
import ctypes

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


def context_step(p, key_bits, leaf_cap, curve, theta, G, eps):
    import barnes_hut_tree_amd as bh
    t = bh.BarnesHut(p.shape[0], 0, key_bits, leaf_cap, curve=curve)
    t.build(torch.from_numpy(p).cuda())
    out = t.gravity(theta, G, eps).cpu().numpy()
    t.sync()
    t.close()
    return out


@pytest.mark.parametrize("key_bits,leaf_cap,curve,n_big", [
    (63, 16, "morton", 200000), (63, 16, "hilbert", 150000), (63, 1, "hilbert", 70000),
    (30, 8, "morton", 100000)])
def test_static_step_matches_context_twice(key_bits, leaf_cap, curve, n_big):
    import barnes_hut_tree_amd as bh
    cases = [(W.plummer(n_big, seed=41), 0.5, 1.0, 0.01), (W.uniform_cube(4097, seed=42), 0.7, 1.3, 1e-3)]
    side = torch.cuda.Stream()
    for k, (p, theta, G, eps) in enumerate(cases):
        print("static step", key_bits, leaf_cap, curve, "n", p.shape[0], flush=True)
        src = torch.from_numpy(p).cuda()
        if k == 0:
            got = bh.gravity_static(src, theta, G, eps, key_bits, leaf_cap, curve)
        else:   # the second call on another stream of the same device
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                got = bh.gravity_static(src, theta, G, eps, key_bits, leaf_cap, curve)
            side.synchronize()
        got = got.cpu().numpy()
        want = context_step(p, key_bits, leaf_cap, curve, theta, G, eps)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, want)


def test_static_step_limits_and_arguments():
    import barnes_hut_tree_amd as bh
    L = bh.load_library()
    s = bh._stream()
    p = torch.from_numpy(W.uniform_cube(90000, seed=43)).cuda()
    out = torch.empty_like(p)
    P = lambda kb, B, cap=0, curve=0, res=0: ctypes.byref(bh._Params(kb, B, cap, curve, res))  # noqa: E731
    sp, op = ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(out.data_ptr())
    # 90000 sources at leaf capacity 1 need more than the static array
    assert L.bh_gravity_static(sp, 90000, P(63, 1), 0.5, 1.0, 0.0, op, s) == bh.BH_ERR_CAPACITY
    assert L.bh_gravity_static(sp, 90000, P(63, 16), 0.5, 1.0, 0.0, op, s) == bh.BH_OK
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    assert L.bh_gravity_static(sp, 100, P(63, 16, cap=1000), 0.5, 1.0, 0.0, op, s) == \
        bh.BH_ERR_INVALID
    assert L.bh_gravity_static(sp, 100, P(31, 16), 0.5, 1.0, 0.0, op, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity_static(sp, 100, P(63, 0), 0.5, 1.0, 0.0, op, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity_static(None, 100, None, 0.5, 1.0, 0.0, op, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity_static(sp, 100, None, -0.5, 1.0, 0.0, op, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity_static(sp, -1, None, 0.5, 1.0, 0.0, op, s) == bh.BH_ERR_INVALID
    assert L.bh_gravity_static(None, 0, None, 0.5, 1.0, 0.0, None, s) == bh.BH_OK
    # defaults (NULL params): 63-bit Morton keys, leaf capacity 16
    q = W.plummer(3000, seed=44)
    tq = torch.from_numpy(q).cuda()
    oq = torch.empty_like(tq)
    assert L.bh_gravity_static(ctypes.c_void_p(tq.data_ptr()), 3000, None, 0.5, 1.0, 0.01,
                               ctypes.c_void_p(oq.data_ptr()), s) == bh.BH_OK
    assert np.array_equal(oq.cpu().numpy(), context_step(q, 63, 16, "morton", 0.5, 1.0, 0.01))

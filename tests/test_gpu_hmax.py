"""bh_node_hmax against the oracle's per-cell maximum of h: exact (a maximum
does not round), node for node in the pre-order both sides produce."""
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


CASES = [
    ("uniform4096", lambda: W.uniform_cube(4096, seed=1), 63, 16, "morton"),
    ("plummer65536", lambda: W.plummer(1 << 16, seed=3), 63, 16, "hilbert"),
    ("plummer65536_B1", lambda: W.plummer(1 << 16, seed=3), 63, 1, "morton"),
    ("duplicates_B4", _dups, 63, 4, "morton"),
    ("plummer_30bit_B8", lambda: W.plummer(1 << 16, seed=3), 30, 8, "hilbert"),
    ("ragged65_B3", lambda: W.uniform_cube(65, seed=7), 63, 3, "morton"),
    ("single", lambda: W.uniform_cube(1, seed=8), 63, 16, "morton"),
    ("ragged4097_B64", lambda: W.plummer(4097, seed=6), 63, 64, "morton"),
    ("plummer65536_B256", lambda: W.plummer(1 << 16, seed=3), 63, 256, "morton"),
]


def _h(n, seed):
    return np.random.default_rng(seed).exponential(0.05, n).astype(np.float32)


@pytest.mark.parametrize("name,make,bits,B,curve", CASES, ids=[c[0] for c in CASES])
def test_node_hmax_matches_oracle(orc, name, make, bits, B, curve):
    import barnes_hut_tree_amd as bh
    p = make()
    h = _h(p.shape[0], 21)
    log("hmax", name, p.shape[0], bits, B, curve)
    t = bh.BarnesHut(p.shape[0], 0, bits, B, curve=curve)
    t.build(torch.from_numpy(p).cuda())
    got = t.node_hmax(torch.from_numpy(h).cuda()).cpu().numpy()
    want = orc.node_hmax(orc.Tree(p, key_bits=bits, leaf_cap=B, curve=curve), h)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    t.close()


def test_node_hmax_plummer_2p20(orc):
    import barnes_hut_tree_amd as bh
    p = W.plummer(1 << 20, seed=3)
    h = _h(p.shape[0], 22)
    log("hmax plummer 2^20")
    t = bh.BarnesHut(p.shape[0], 0, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(p).cuda())
    got = t.node_hmax(torch.from_numpy(h).cuda()).cpu().numpy()
    want = orc.node_hmax(orc.Tree(p, key_bits=63, leaf_cap=16, curve="hilbert"), h)
    assert np.array_equal(got, want)
    t.close()


def test_node_hmax_arguments():
    import barnes_hut_tree_amd as bh
    L = bh.load_library()
    p = W.uniform_cube(1000, seed=5)
    t = bh.BarnesHut(1000, 0, 63, 16)
    h = torch.ones(1000, dtype=torch.float32, device="cuda")
    with pytest.raises(bh.BHError):
        t.node_hmax(h)                      # not built yet
    t.build(torch.from_numpy(p).cuda())
    nn = t.node_count()
    out = torch.empty(nn, dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hp, op = ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(out.data_ptr())
    assert L.bh_node_hmax(t._h, hp, 999, op, nn, s) == bh.BH_ERR_INVALID       # n != built n
    assert L.bh_node_hmax(t._h, hp, 1000, op, nn - 1, s) == bh.BH_ERR_INVALID  # buffer too small
    assert L.bh_node_hmax(t._h, None, 1000, op, nn, s) == bh.BH_ERR_INVALID
    assert L.bh_node_hmax(None, hp, 1000, op, nn, s) == bh.BH_ERR_INVALID
    assert L.bh_node_hmax(t._h, hp, 1000, op, nn, s) == bh.BH_OK
    torch.cuda.synchronize()
    assert torch.all(out == 1.0)
    # an empty build gives an empty result
    t.build(torch.empty((0, 4), dtype=torch.float32, device="cuda"))
    assert t.node_hmax(torch.empty(0, dtype=torch.float32, device="cuda")).numel() == 0
    t.close()

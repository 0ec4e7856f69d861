"""The per-target walk's XCD runs, balanced on an earlier walk's per-group
times, and its heaviest groups walked as four waves of 16 targets (through
bh_gravity; bh_get_walk_runs reports the runs and the split groups used).

Each XCD walks one contiguous run of the groups of 64 targets.  Every fourth
walk of the same groups stores its per-group times; when those show the equal
runs more than 8% out of balance (and the waves long-lived), later walks move
the runs' ends so that their sums of those times are equal.  Which XCD walks a
group changes nothing in that group's arithmetic, so every call must give the
same bits as the first, and as the caller-order walk (which keeps equal runs
and, lane by lane, the same walk).  Outputs are filled with NaN before each
call, so a group that no workgroup walked shows up."""
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


def log(*a):
    print(*a, flush=True)


def _nan_out(n):
    return torch.full((n, 4), float("nan"), dtype=torch.float32, device="cuda")


def _walk(t, n, eps, targets=None, flags=0):
    out = _nan_out(n)
    t.gravity(0.5, 1.0, eps, targets=targets, out=out, flags=flags)
    return out.cpu().numpy()


CASES = {
    "plummer65536": lambda: W.plummer(1 << 16, seed=3),
    "plummer_ragged100003": lambda: W.plummer(100003, seed=9),
    "galaxy_pair200000": lambda: W.galaxy_pair(200_000, seed=4)[0],
    "uniform300": lambda: W.uniform_cube(300, seed=7),
    "uniform65": lambda: W.uniform_cube(65, seed=8),
    "single": lambda: W.uniform_cube(1, seed=1),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_balanced_runs_walk_every_group_once(case):
    import barnes_hut_tree_amd as bh
    p = CASES[case]()
    n = p.shape[0]
    eps = 0.01
    log("balanced runs", case, n)
    t = bh.BarnesHut(n, 0, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(p).cuda())
    first = _walk(t, n, eps)
    assert np.all(np.isfinite(first)) or n == 1
    for k in range(3):
        again = _walk(t, n, eps)
        assert np.array_equal(again, first, equal_nan=True), "call %d" % (k + 2)
    # a rebuild of the same sources keeps the groups (and the history)
    t.build(torch.from_numpy(p).cuda())
    assert np.array_equal(_walk(t, n, eps), first, equal_nan=True)
    caller_order = _walk(t, n, eps, flags=bh.WALK_UNSORTED)
    assert np.array_equal(caller_order, first, equal_nan=True)
    t.close()


def test_history_follows_the_grouping():
    """Self-gravity and separate targets of another count alternate on one
    context: each walk's result equals that of a fresh context."""
    import barnes_hut_tree_amd as bh
    src = W.plummer(1 << 15, seed=5)
    q = W.box_queries(50001, seed=21)
    n, m = src.shape[0], q.shape[0]
    qt = torch.from_numpy(q).cuda()
    fresh = bh.BarnesHut(n, m, 63, 16, curve="hilbert")
    fresh.build(torch.from_numpy(src).cuda())
    ref_self = _walk(fresh, n, 0.01)
    fresh.close()
    fresh = bh.BarnesHut(n, m, 63, 16, curve="hilbert")
    fresh.build(torch.from_numpy(src).cuda())
    ref_q = _walk(fresh, m, 0.01, targets=qt)
    fresh.close()
    t = bh.BarnesHut(n, m, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(src).cuda())
    for k in range(3):
        log("alternating walks, round", k)
        assert np.array_equal(_walk(t, n, 0.01), ref_self)
        assert np.array_equal(_walk(t, n, 0.01), ref_self)
        assert np.array_equal(_walk(t, m, 0.01, targets=qt), ref_q)
        assert np.array_equal(_walk(t, m, 0.01, targets=qt), ref_q)
        # a vote walk between them leaves the per-target walk's history alone
        t.gravity(0.5, 1.0, 0.01, flags=bh.WALK_VOTE)
    t.close()


def test_fewer_sources_on_a_larger_context():
    """A context built for more sources, rebuilt with fewer: the groups change,
    so the walk starts again from equal runs, and then balances again."""
    import barnes_hut_tree_amd as bh
    big = W.plummer(1 << 16, seed=3)
    small = W.plummer(20000, seed=6)
    t = bh.BarnesHut(big.shape[0], 0, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(big).cuda())
    for _ in range(2):
        _walk(t, big.shape[0], 0.01)
    ref = bh.BarnesHut(small.shape[0], 0, 63, 16, curve="hilbert")
    ref.build(torch.from_numpy(small).cuda())
    want = _walk(ref, small.shape[0], 0.01)
    ref.close()
    t.build(torch.from_numpy(small).cuda())
    for k in range(3):
        log("smaller rebuild, call", k)
        assert np.array_equal(_walk(t, small.shape[0], 0.01), want)
    t.close()


def test_uneven_runs_walk_every_group_once():
    """The galaxy pair: its groups' walk times differ by far more than 8%
    between eighths of the key order, and its waves live long, so after a few
    walks the XCD runs become uneven.  Every call, rebuilt like a time step,
    gives the first call's bits; the runs are contiguous, cover every group
    and stay within the grid's room of 1.25 equal shares."""
    import barnes_hut_tree_amd as bh
    p = W.galaxy_pair(500_000, seed=4)[0]
    n = p.shape[0]
    groups = (n + 63) // 64
    cap = (groups + 7) // 8 + (groups + 31) // 32
    src = torch.from_numpy(p).cuda()
    t = bh.BarnesHut(n, 0, 63, 16, curve="hilbert")
    t.build(src)
    first = _walk(t, n, 0.02)
    uneven_calls = 0
    for k in range(12):
        t.build(src)
        got = _walk(t, n, 0.02)
        assert np.array_equal(got, first), "call %d" % (k + 2)
        uneven, starts = t.walk_runs()
        log("galaxy pair call", k + 2, "uneven runs" if uneven else "equal runs", starts)
        if uneven:
            uneven_calls += 1
            s = np.array(starts, np.int64)
            assert s[0] == 0 and s[8] == groups
            assert np.all(np.diff(s) >= 0) and np.all(np.diff(s) <= cap)
            assert not np.array_equal(s, [x * (groups // 8) + min(x, groups % 8) for x in range(9)])
    assert uneven_calls >= 4
    # the caller-order walk keeps equal runs: the same bits again
    assert np.array_equal(_walk(t, n, 0.02, flags=bh.WALK_UNSORTED), first)
    t.close()


@pytest.mark.parametrize("m_queries", [1_000_000, 999_983])
def test_heavy_groups_split_walk_every_target_once(m_queries):
    """Separate queries around dense surfaces: a few groups of 64 queries take
    far longer than the mean (queries on a surface open many leaves), so after
    the first recorded walk the heaviest are walked as four waves of 16
    queries each (also with a ragged last group).  Every call gives the first
    call's bits (outputs filled with NaN before each), and so does the
    caller-order walk."""
    import barnes_hut_tree_amd as bh
    src = torch.from_numpy(W.surface_sources(1 << 20, seed=10)).cuda()
    q = torch.from_numpy(np.ascontiguousarray(W.grid_queries()[:m_queries])).cuda()
    m = q.shape[0]
    t = bh.BarnesHut(src.shape[0], m, 63, 16, curve="hilbert")
    t.build(src)
    first = _walk(t, m, 0.0, targets=q)
    assert np.all(np.isfinite(first))
    split = []
    for k in range(10):
        assert np.array_equal(_walk(t, m, 0.0, targets=q), first), "call %d" % (k + 2)
        split.append(t.walk_split())
    log("split groups per call", split)
    limit = 2 * ((((m + 63) // 64) + 63) // 64)
    assert max(split) > 0 and all(0 <= s <= limit for s in split)
    assert np.array_equal(_walk(t, m, 0.0, targets=q, flags=bh.WALK_UNSORTED), first)
    t.close()


def test_plummer_groups_not_split():
    """Plummer self-gravity: group times differ by less than the split ratio,
    so no group is split."""
    import barnes_hut_tree_amd as bh
    p = W.plummer(1 << 18, seed=3)
    n = p.shape[0]
    t = bh.BarnesHut(n, 0, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(p).cuda())
    for _ in range(8):
        _walk(t, n, 0.01)
        assert t.walk_split() == 0
    t.close()


def test_self_gravity_split_walk_every_target_once():
    """Self-gravity with 20000 coincident sources in a uniform background:
    they share one leaf far over the capacity (no key bit separates them), so
    each of their groups sums that leaf whole and takes far longer than the
    rest; those groups are walked as four waves of 16 targets each, whose
    leaf holds their own targets (the self pair masked per lane).  Every call
    gives the first call's bits, and so does the caller-order walk."""
    import barnes_hut_tree_amd as bh
    rng = np.random.default_rng(21)
    bg = rng.uniform(-1.0, 1.0, (200_000, 3))
    xyz = np.concatenate([bg, np.full((20_000, 3), 0.3)])[rng.permutation(220_000)]
    p = np.concatenate([xyz, np.full((xyz.shape[0], 1), 1.0 / xyz.shape[0])], 1).astype(np.float32)
    n = p.shape[0]
    t = bh.BarnesHut(n, 0, 63, 16, curve="hilbert")
    t.build(torch.from_numpy(p).cuda())
    first = _walk(t, n, 1e-4)
    assert np.all(np.isfinite(first))
    split = []
    for k in range(10):
        assert np.array_equal(_walk(t, n, 1e-4), first), "call %d" % (k + 2)
        split.append(t.walk_split())
    log("self-gravity split groups per call", split)
    assert max(split) > 0
    assert np.array_equal(_walk(t, n, 1e-4, flags=bh.WALK_UNSORTED), first)
    t.close()

"""Benchmark: one gravity step = tree build + tree walk over all particles.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload plummer]

Default workload: an equal-mass Plummer sphere of N = 2^20 particles (scale
radius 1, truncated at 20), fp32 float4, theta = 0.5, G = 1, Plummer
softening eps = 0.01, leaf capacity 16, 63-bit keys on the Hilbert curve
(--curve morton for the Z-order of the pages; the same tree cells), fed in
random (generation) order.  Inputs are synthetic (workloads.py) and resident in
device memory before timing starts.  One step = bh_build + bh_gravity (keys,
sort, tree, centre of mass, walk), from caller-order input to caller-order
output.  Prints one JSON line.

value = interactions per second of the whole step (interactions = accepted
nodes + particle pairs of the walk, counted by the library in an untimed
pass).  The roofline object describes the walk kernel (the dominant one),
counted at 20 flops per interaction against the fp32 vector peak, and in its
"build" member bh_build's algorithmic bytes against the HBM peak.
config.morton_keys times the same step with Morton keys (the pages' order).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per gravity step + interactions/s at N=2^20, θ=0.5, fp32 (1 GPU)"
FLOPS_PER_INTERACTION = 20
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_BYTES = 8e12
PROFILES = os.path.join(ROOT, "profiles")


def make_workload(name):
    import workloads as W
    if name == "plummer":
        return W.plummer(1 << 20, seed=3), dict(theta=0.5, G=1.0, eps=0.01), \
            "plummer_n1048576_random_order"
    if name == "lattice":
        return W.lattice(100, shuffled=True, seed=2), dict(theta=0.5, G=1.0, eps=1e-3), \
            "lattice_n1000000_shuffled"
    if name == "galaxy":
        return W.galaxy_pair()[0], dict(theta=0.5, G=1.0, eps=0.02), "galaxy_pair_n5000000"
    if name == "uniform":
        return W.uniform_cube(4096, seed=1), dict(theta=0.5, G=1.0, eps=1e-3), "uniform_n4096"
    if name.startswith("uniform_2p"):
        n = 1 << int(name[len("uniform_2p"):])
        return W.uniform_box(n, seed=5), dict(theta=0.5, G=1.0, eps=1e-3), "uniform_n%d" % n
    raise SystemExit("unknown workload " + name)


def build_alg_bytes(n, n_nodes, n_leaves, key_bits):
    """Algorithmic HBM bytes of one bh_build over n sources giving n_nodes
    nodes and n_leaves leaves: bounding box 16n read; keys 16n read and 12n
    written; per sort pass an 8n histogram read and a 12n + 12n scatter; the
    16-byte rows gathered in sorted order (16n + 16n), with 63-bit keys by the
    kernel that finishes the runs of equal top 40 bits after five passes
    (which also moves the keys and indices once more, 12n + 12n), with 30-bit
    keys by the last of four passes; count 26n read and 2n written; emit 18n
    read, 16 bytes per node and 40 per leaf written; ranges 84 bytes read and
    32 written per node."""
    if key_bits > 40:
        sort = ((key_bits - 24 + 7) // 8) * 32 * n + 56 * n
    else:
        sort = ((key_bits + 7) // 8) * 32 * n + 32 * n
    return (16 * n + 28 * n + sort + 28 * n + 18 * n
            + 16 * n_nodes + 40 * n_leaves + 116 * n_nodes)


def walk_source_hash():
    """Hash of the walk kernel's sources (the walk and its pair interaction):
    counter summaries taken for another version of the kernel are not
    reported."""
    h = hashlib.sha256()
    for f in ("traverse.hip", "interaction.h"):
        h.update(open(os.path.join(ROOT, "barnes_hut_tree_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload, curve):
    """HBM bytes per walk launch from the committed rocprofv3 counter summary,
    or None when absent, taken for a different walk kernel source, or for the
    other key curve."""
    path = os.path.join(PROFILES, "walk_%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("walk_source_sha256_16") != walk_source_hash() or vals.get("key_curve") != curve:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, prm, key_bits, leaf_cap, curve, budget_s=8.0):
    """The oracle (fp64, OpenMP) on the host: full tree build plus the walk
    for a random sample of targets sized to about budget_s seconds, scaled to
    the whole step.  Returns the baseline record and the oracle's interaction
    count for the step: exact when the sample is every target, else scaled
    from the sample (the label says which)."""
    import numpy as np

    import oracle
    n = p.shape[0]
    t0 = time.perf_counter()
    tree = oracle.Tree(p, key_bits, leaf_cap, curve=curve)
    t_build = time.perf_counter() - t0
    rng = np.random.default_rng(99)
    m = min(n, 1 << 13)
    which = np.sort(rng.choice(n, m, replace=False))
    t0 = time.perf_counter()
    _, ni, _ = tree.gravity(prm["theta"], prm["G"], prm["eps"], which=which)
    t_walk = time.perf_counter() - t0
    if t_walk < budget_s and m < n:
        m = int(min(n, m * budget_s / max(t_walk, 1e-3)))
        which = np.sort(rng.choice(n, m, replace=False))
        t0 = time.perf_counter()
        _, ni, _ = tree.gravity(prm["theta"], prm["G"], prm["eps"], which=which)
        t_walk = time.perf_counter() - t0
    per_target = t_walk / m
    t_step = t_build + per_target * n
    inter = float(ni.sum()) * n / m
    rec = {
        "value": inter / t_step, "unit": "interactions/s", "cores": oracle.threads(),
        "kind": "oracle",
        "sample": "full fp64 tree build (%.2f s) + walk of %d random targets of %d (%.2f s), "
                  "scaled to all targets: %.2f s per step" % (t_build, m, n, t_walk, t_step),
    }
    count = {"interactions": int(ni.sum()) if m == n else int(round(inter)),
             "kind": "exact: every target walked" if m == n else
                     "scaled from %d of %d targets" % (m, n)}
    return rec, count


def theta_sweep(args):
    """Accuracy and speed-up of the walk against the GPU direct sum over a
    range of opening angles, in the layout of the pages' table ([GASPHiA]
    精度与加速比验证): walk time, max and mean relative error of the
    acceleration vector, speed-up over the direct sum.  One JSON line per
    theta, then a summary line."""
    import torch

    import barnes_hut_tree_amd as bh
    p, prm, wname = make_workload(args.workload)
    n = p.shape[0]
    src = torch.from_numpy(p).cuda()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ref = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    direct_ms = timed(lambda: bh.direct(src, prm["G"], prm["eps"], out=ref), 2)
    ref64 = ref.double()
    ref_norm = ref64[:, :3].norm(dim=1)
    pairs = n * (n - 1)
    print(json.dumps({"kernel": "direct", "workload": wname, "n": n, "ms": round(direct_ms, 3),
                      "pairs_per_s": pairs / (direct_ms * 1e-3),
                      "tflops_at_20_per_pair": round(20 * pairs / (direct_ms * 1e-3) / 1e12, 2)}),
          flush=True)

    tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap, curve=args.curve)
    build_ms = timed(lambda: tree.build(src), 5)
    tree.sync()
    out = torch.empty_like(ref)
    rows = []
    thetas = [0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8] if args.theta is None else [args.theta]
    for th in thetas:
        walk_ms = timed(lambda: tree.gravity(th, prm["G"], prm["eps"], out=out), 3)
        err = (out.double()[:, :3] - ref64[:, :3]).norm(dim=1) / ref_norm
        perr = ((out.double()[:, 3] - ref64[:, 3]) / ref64[:, 3]).abs()
        row = {"theta": th, "walk_ms": round(walk_ms, 3), "build_ms": round(build_ms, 3),
               "max_rel_err": float(err.max()), "mean_rel_err": float(err.mean()),
               "pot_max_rel_err": float(perr.max()), "pot_mean_rel_err": float(perr.mean()),
               "interactions": tree.count_interactions(th, prm["eps"]),
               "speedup_walk": round(direct_ms / walk_ms, 1),
               "speedup_step": round(direct_ms / (walk_ms + build_ms), 1)}
        rows.append(row)
        print(json.dumps(row), flush=True)
    tree.close()
    print(json.dumps({"sweep": wname, "n": n, "eps": prm["eps"], "leaf_cap": args.leaf_cap,
                      "key_curve": args.curve,
                      "direct_ms": round(direct_ms, 3), "rows": len(rows)}), flush=True)


def ablations(args):
    """The pages' design comparisons on MI355X, one JSON line each.

    Target order ([GASPHiA] 排序算法 compares a random order, a regular lattice
    order and the tree-sorted order on 1M particles): the 1M lattice walked in
    the caller's order, shuffled and in lattice order, against the Morton-ordered
    walk.  Warp vote ([GASPHiA] 性能瓶颈分析): the default workload with the
    per-target walk and with the vote, time, interactions and accuracy against
    the GPU direct sum."""
    import numpy as np
    import torch

    import barnes_hut_tree_amd as bh
    import workloads as W

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    theta, eps = 0.5, 1e-3
    for shuffled in (True, False):
        p = W.lattice(100, shuffled=shuffled, seed=2)
        n = p.shape[0]
        src = torch.from_numpy(p).cuda()
        out = torch.empty((n, 4), dtype=torch.float32, device="cuda")
        tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap)
        tree.build(src)
        tree.sync()
        modes = [("caller_order", bh.WALK_UNSORTED)] + ([("morton_order", 0)] if shuffled else [])
        for name, flags in modes:
            ms = timed(lambda: tree.gravity(theta, 1.0, eps, out=out, flags=flags))
            inter = tree.count_interactions(theta, eps, flags=flags)
            print(json.dumps({"ablation": "target_order", "workload": "lattice_n1000000_" +
                              ("shuffled" if shuffled else "lattice_order"), "walk": name,
                              "theta": theta, "eps": eps, "walk_ms": round(ms, 3),
                              "interactions": inter}), flush=True)
        tree.close()

    # tree build: the pages' lock-based dense build against the sorted-key build
    builds = [("lattice_n1000000_shuffled", W.lattice(100, shuffled=True, seed=2)),
              ("lattice_n1000000_lattice_order", W.lattice(100, shuffled=False, seed=2)),
              ("plummer_n1048576_random_order", W.plummer(1 << 20, seed=3)),
              ("galaxy_pair_n5000000", W.galaxy_pair()[0])]
    for wl, p in builds:
        n = p.shape[0]
        src = torch.from_numpy(p).cuda()
        t1 = bh.BarnesHut(n, 0, args.key_bits, 1)
        ms_lock = timed(lambda: t1.build_locked(src))
        t1.sync()
        ms_sorted1 = timed(lambda: t1.build(src))
        t1.sync()
        t1.close()
        t16 = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap)
        ms_sorted16 = timed(lambda: t16.build(src))
        t16.close()
        print(json.dumps({"ablation": "tree_build", "workload": wl, "n": n,
                          "lock_based_dense_b1_ms": round(ms_lock, 3),
                          "sorted_key_b1_ms": round(ms_sorted1, 3),
                          "sorted_key_b%d_ms" % args.leaf_cap: round(ms_sorted16, 3)}),
              flush=True)
        del src

    p, prm, wname = make_workload("plummer")
    n = p.shape[0]
    src = torch.from_numpy(p).cuda()
    ref = bh.direct(src, prm["G"], prm["eps"]).double()
    ref_n = ref[:, :3].norm(dim=1)
    tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap)
    tree.build(src)
    out = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    for th in (0.3, 0.5, 0.7):
        for name, flags in (("per_target", 0), ("vote", bh.WALK_VOTE)):
            ms = timed(lambda: tree.gravity(th, prm["G"], prm["eps"], out=out, flags=flags))
            inter = tree.count_interactions(th, prm["eps"], flags=flags)
            err = ((out.double()[:, :3] - ref[:, :3]).norm(dim=1) / ref_n).cpu().numpy()
            print(json.dumps({"ablation": "warp_vote", "workload": wname, "walk": name,
                              "theta": th, "walk_ms": round(ms, 3), "interactions": inter,
                              "interactions_per_s": inter / (ms * 1e-3),
                              "median_rel_err": float(np.median(err)),
                              "mean_rel_err": float(err.mean()), "max_rel_err": float(err.max())}),
                  flush=True)
    tree.close()


def leapfrog(args):
    """Time stepping of the 5M galaxy pair ([GASPHiA] page header): kick-drift-
    kick leapfrog with the tree rebuilt every step (bh_leapfrog_step), timed
    over --steps steps after --warmup steps; the conserved quantities before
    and after.  One JSON line."""
    import numpy as np
    import torch

    import barnes_hut_tree_amd as bh
    import workloads as W
    p, v = W.galaxy_pair()
    n = p.shape[0]
    theta = 0.5 if args.theta is None else args.theta
    eps, dt = 0.02, 0.05
    tp = torch.from_numpy(p).cuda()
    tv = torch.from_numpy(np.concatenate([v, np.zeros((n, 1), np.float32)], 1)).cuda()
    tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap, curve=args.curve)
    tree.build(tp)
    ta = tree.gravity(theta, 1.0, eps)
    for _ in range(args.warmup):
        tree.leapfrog_step(tp, tv, ta, dt, theta, 1.0, eps)
    d0 = tree.diagnostics(tp, tv, ta)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tree.leapfrog_step(tp, tv, ta, dt, theta, 1.0, eps)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    d1 = tree.diagnostics(tp, tv, ta)
    tree.sync()
    e0, e1 = d0["kinetic"] + d0["potential"], d1["kinetic"] + d1["potential"]
    print(json.dumps({
        "leapfrog": "galaxy_pair_n5000000", "n": n, "theta": theta, "eps": eps, "dt": dt,
        "key_curve": args.curve,
        "steps": args.steps, "warmup_steps": args.warmup, "ms_per_step": round(ms, 3),
        "energy_before": e0, "energy_after": e1, "rel_energy_change": (e1 - e0) / abs(e0),
        "kinetic_before": d0["kinetic"], "kinetic_after": d1["kinetic"],
        "momentum_before": d0["momentum"], "momentum_after": d1["momentum"],
        "angular_momentum_before": d0["angular_momentum"],
        "angular_momentum_after": d1["angular_momentum"]}), flush=True)
    tree.close()


def sbh_compare(args):
    """Stochastic Barnes-Hut against the per-target Barnes-Hut walk at separate
    query points ([SBH] 实验结果's table): sources on 3-6 spheres and tori
    (area weights), M = 2^15, 2^17, 2^20, 10^6 queries on a 100^3 grid or
    uniform in [-1, 1]^3, G = 1, eps = 0, potential errors against the GPU
    direct sum, 8 source seeds (10-17), mean and spread over the seeds.  BH:
    theta = 0.5 (far-field ratio 2), leaf capacity 16; SBH: S = 1 sample per
    stratum, leaf capacity 1, d = 4 and d = 2; Morton keys.  Times are device times of the
    query call (the target ordering included), mean of 5; the build is listed
    apart.  One JSON line per (M, queries, method)."""
    import numpy as np
    import torch

    import barnes_hut_tree_amd as bh
    import workloads as W

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    seeds = list(range(10, 18))
    sizes = [1 << 15, 1 << 17, 1 << 20]
    qsets = {"grid100": W.grid_queries(), "uniform1e6": W.box_queries()}
    for qname, qa in qsets.items():
        q = torch.from_numpy(qa).cuda()
        nq = q.shape[0]
        out = torch.empty((nq, 4), dtype=torch.float32, device="cuda")
        for m in sizes:
            res = {k: [] for k in ("bh", "sbh_d4", "sbh_d2")}
            for sd in seeds:
                src = torch.from_numpy(W.surface_sources(m, seed=sd)).cuda()
                exact = bh.direct(src, 1.0, 0.0, targets=q)[:, 3].double()
                t16 = bh.BarnesHut(m, nq, args.key_bits, 16)
                build16 = timed(lambda: t16.build(src))
                ms = timed(lambda: t16.gravity(0.5, 1.0, 0.0, targets=q, out=out))
                err = (out[:, 3].double() - exact).abs()
                res["bh"].append((ms, build16, err))
                t16.close()
                t1 = bh.BarnesHut(m, nq, args.key_bits, 1)
                build1 = timed(lambda: t1.build(src))
                for d in (4, 2):
                    ms = timed(lambda: t1.sbh(q, d=d, samples=1, seed=sd, out=out))
                    err = (out[:, 3].double() - exact).abs()
                    res["sbh_d%d" % d].append((ms, build1, err))
                t1.close()
            for meth, rows in res.items():
                ms = np.array([r[0] for r in rows])
                bms = np.array([r[1] for r in rows])
                mean = np.array([float(r[2].mean()) for r in rows])
                med = np.array([float(r[2].median()) for r in rows])
                mx = np.array([float(r[2].max()) for r in rows])
                print(json.dumps({
                    "compare": "sbh_vs_bh", "sources": "surfaces", "m": m, "queries": qname,
                    "method": meth, "seeds": len(seeds),
                    "ms_mean": round(float(ms.mean()), 4), "ms_sd": round(float(ms.std()), 4),
                    "build_ms_mean": round(float(bms.mean()), 4),
                    "mean_abs_err": [float(mean.mean()), float(mean.std())],
                    "median_abs_err": [float(med.mean()), float(med.std())],
                    "max_abs_err": [float(mx.mean()), float(mx.std())]}), flush=True)


def cpu_oracle_row(p, q, prm, key_bits, leaf_cap, curve, budget_s=4.0, direct_targets=1 << 14):
    """CPU baselines of one configuration, both from the oracle (fp64, OpenMP)
    on the host: its tree build plus its walk for a random sample of the
    targets sized to about budget_s seconds, scaled to all targets; and its
    direct sum on direct_targets random targets, scaled to all targets."""
    import numpy as np

    import oracle
    n = p.shape[0]
    nt = n if q is None else q.shape[0]
    rng = np.random.default_rng(98)
    t0 = time.perf_counter()
    tree = oracle.Tree(p, key_bits, leaf_cap, curve=curve)
    t_build = time.perf_counter() - t0
    m = min(nt, 1 << 11)
    for _ in range(2):
        which = np.sort(rng.choice(nt, m, replace=False))
        t0 = time.perf_counter()
        tree.gravity(prm["theta"], prm["G"], prm["eps"], targets=q, which=which)
        t_walk = time.perf_counter() - t0
        if t_walk >= budget_s / 4 or m == nt:
            break
        m = int(min(nt, m * budget_s / max(t_walk, 1e-3)))
    del tree
    md = min(nt, direct_targets)
    which = np.sort(rng.choice(nt, md, replace=False))
    t0 = time.perf_counter()
    oracle.direct(p, prm["G"], prm["eps"], targets=q, which=which)
    t_direct = time.perf_counter() - t0
    return {"cpu_cores": oracle.threads(),
            "cpu_bh_s": round(t_build + t_walk * nt / m, 3),
            "cpu_bh_sample": "tree build %.2f s + walk of %d of %d targets %.2f s, scaled"
                             % (t_build, m, nt, t_walk),
            "cpu_direct_s": round(t_direct * nt / md, 3),
            "cpu_direct_sample": "%d of %d targets %.2f s, scaled" % (md, nt, t_direct)}


def configs_table(args):
    """One JSON line per measured configuration: the 4096 uniform cube against
    the direct sum; the 1M lattice shuffled and in lattice order; the Plummer
    sphere at theta 0.3/0.5/0.7 in random and in Morton-sorted input order;
    the 5M galaxy pair; the surface sources at M = 2^15, 2^17, 2^20 with grid
    and box queries.  Per line: build and walk device ms (HIP events, mean of
    --steps), interactions, the walk's fraction of the fp32 vector peak at 20
    flops per interaction, the build's algorithmic bytes against 8 TB/s,
    whether the timed walks took uneven XCD runs, and the oracle's CPU times
    (tree walk and direct sum, both scaled from samples) unless
    --no-cpu-baseline.  Six warm-up steps per line, each waited for."""
    import numpy as np
    import torch

    import barnes_hut_tree_amd as bh
    import workloads as W

    def morton_sorted(p):
        t = bh.BarnesHut(p.shape[0], 0, args.key_bits, args.leaf_cap, curve="morton")
        t.build(torch.from_numpy(p).cuda())
        _, perm = t.keys()
        t.close()
        return np.ascontiguousarray(p[perm.cpu().numpy()])

    rows = [("uniform_n4096", lambda: W.uniform_cube(4096, seed=1), None, [0.5], 1e-3),
            ("lattice_n1000000_shuffled", lambda: W.lattice(100, shuffled=True, seed=2), None,
             [0.5], 1e-3),
            ("lattice_n1000000_lattice_order", lambda: W.lattice(100, shuffled=False, seed=2),
             None, [0.5], 1e-3),
            ("plummer_n1048576_random_order", lambda: W.plummer(1 << 20, seed=3), None,
             [0.3, 0.5, 0.7], 0.01),
            ("plummer_n1048576_morton_sorted", lambda: morton_sorted(W.plummer(1 << 20, seed=3)),
             None, [0.3, 0.5, 0.7], 0.01),
            ("galaxy_pair_n5000000", lambda: W.galaxy_pair()[0], None, [0.5], 0.02)]
    for m in (1 << 15, 1 << 17, 1 << 20):
        for qn, qf in (("grid100", W.grid_queries), ("uniform1e6", W.box_queries)):
            rows.append(("surfaces_m%d_%s" % (m, qn),
                         (lambda m=m: W.surface_sources(m, seed=10)), qf, [0.5], 0.0))
    for wname, pf, qf, thetas, eps in rows:
        p = pf()
        q = None if qf is None else qf()
        n = p.shape[0]
        nt = n if q is None else q.shape[0]
        src = torch.from_numpy(p).cuda()
        tq = None if q is None else torch.from_numpy(q).cuda()
        out = torch.empty((nt, 4), dtype=torch.float32, device="cuda")
        tree = bh.BarnesHut(n, 0 if q is None else nt, args.key_bits, args.leaf_cap,
                            curve=args.curve)
        for th in thetas:
            # warm-up steps, each waited for: the walk balances its XCD runs on
            # earlier walks' times (bh_get_walk_runs), whose verdict the host
            # reads between calls
            for _ in range(6):
                tree.build(src)
                tree.gravity(th, 1.0, eps, targets=tq, out=out)
                torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                   for _ in range(args.steps)]
            for e in evs:
                e[0].record(stream)
                tree.build(src)
                e[1].record(stream)
                tree.gravity(th, 1.0, eps, targets=tq, out=out)
                e[2].record(stream)
            torch.cuda.synchronize()
            tree.sync()
            uneven_runs = tree.walk_runs()[0]   # the last timed walk's XCD runs
            build_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
            walk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / len(evs)
            inter = tree.count_interactions(th, eps, targets=tq)
            nodes = tree.nodes()
            nn = int(nodes.shape[0])
            nl = int(((nodes[:, 7] & (1 << 8)) != 0).sum().item())
            bbytes = build_alg_bytes(n, nn, nl, args.key_bits)
            row = {"config": wname, "n_sources": n, "n_targets": nt, "theta": th, "eps": eps,
                   "leaf_cap": args.leaf_cap, "key_curve": args.curve,
                   "uneven_xcd_runs": uneven_runs,
                   "build_ms": round(build_ms, 4), "walk_ms": round(walk_ms, 4),
                   "step_ms": round(build_ms + walk_ms, 4), "interactions": inter,
                   "walk_alu_frac": round(FLOPS_PER_INTERACTION * inter / (walk_ms * 1e-3)
                                          / (FP32_PEAK_TFLOPS * 1e12), 4),
                   "nodes": nn, "leaves": nl, "build_alg_bytes": bbytes,
                   "build_hbm_frac": round(bbytes / (build_ms * 1e-3) / HBM_PEAK_BYTES, 4)}
            if not args.no_cpu_baseline:
                row.update(cpu_oracle_row(p, q, dict(theta=th, G=1.0, eps=eps), args.key_bits,
                                          args.leaf_cap, args.curve))
            print(json.dumps(row), flush=True)
        tree.close()
        del src, tq, out


def build_only(args):
    """bh_build alone (bounding box, keys, sort with the sorted-source gather,
    tree, centres of mass), timed with HIP events on the launch stream; the
    per-kernel split comes from rocprofv3 on this mode."""
    import torch

    import barnes_hut_tree_amd as bh
    p, _, wname = make_workload(args.workload)
    n = p.shape[0]
    src = torch.from_numpy(p).cuda()
    tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap, curve=args.curve)
    for _ in range(args.warmup):
        tree.build(src)
    tree.sync()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        tree.build(src)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    tree.sync()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    nodes = tree.nodes()
    n_nodes = int(nodes.shape[0])
    n_leaves = int(((nodes[:, 7] & (1 << 8)) != 0).sum().item())
    tree.close()
    print(json.dumps({"mode": "build_only", "workload": wname, "n": n,
                      "n_nodes": n_nodes, "n_leaves": n_leaves,
                      "leaf_cap": args.leaf_cap, "key_bits": args.key_bits,
                      "key_curve": args.curve, "steps": args.steps,
                      "build_ms_median": ms[len(ms) // 2], "build_ms_min": ms[0]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="plummer")
    ap.add_argument("--leaf-cap", type=int, default=16)
    ap.add_argument("--key-bits", type=int, default=63)
    ap.add_argument("--curve", default="hilbert", choices=["morton", "hilbert"],
                    help="key curve of the tree (sort order of the sources and targets); "
                         "the same cells either way, Hilbert waves walk fewer nodes")
    ap.add_argument("--theta", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="theta sweep against the GPU direct sum instead of the step benchmark")
    ap.add_argument("--ablations", action="store_true",
                    help="the pages' design comparisons (target order, warp vote)")
    ap.add_argument("--leapfrog", action="store_true",
                    help="time-step the 5M galaxy pair (kick-drift-kick, rebuild every step)")
    ap.add_argument("--sbh", action="store_true",
                    help="stochastic Barnes-Hut vs the tree walk at separate query points")
    ap.add_argument("--configs", action="store_true",
                    help="one line per measured configuration (uniform 4096, lattice, Plummer "
                         "theta and input order, galaxy pair, surfaces M sweep)")
    ap.add_argument("--build-only", action="store_true",
                    help="time bh_build alone on the workload (keys, sort, tree, centres of "
                         "mass) and print its JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (3 times), "
                         "the reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the walk has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import barnes_hut_tree_amd as bh
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written":
                          nbytes, "copies": 3}), file=sys.stderr, flush=True)
        del a, b

    if args.sweep:
        theta_sweep(args)
        return
    if args.ablations:
        ablations(args)
        return
    if args.leapfrog:
        leapfrog(args)
        return
    if args.sbh:
        sbh_compare(args)
        return

    if args.build_only:
        build_only(args)
        return
    if args.configs:
        configs_table(args)
        return

    p, prm, wname = make_workload(args.workload)
    if args.theta is not None:
        prm["theta"] = args.theta
    n = p.shape[0]
    src = torch.from_numpy(p).cuda()
    out = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    tree = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap, curve=args.curve)

    def step():
        tree.build(src)
        tree.gravity(prm["theta"], prm["G"], prm["eps"], out=out)

    for _ in range(args.warmup):
        step()
    tree.sync()
    interactions = tree.count_interactions(prm["theta"], prm["eps"])

    # per-phase device times: the median of five profiled steps outside the
    # timed region
    tree.set_profiling(True)
    runs = []
    for _ in range(5):
        step()
        runs.append(tree.profile())
    tree.set_profiling(False)
    tree.sync()
    phases = [sorted(r[k] for r in runs)[len(runs) // 2] for k in range(len(runs[0]))]

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for k in range(args.steps):
        evb[k].record(stream)
        tree.build(src)
        ev[k][0].record(stream)
        tree.gravity(prm["theta"], prm["G"], prm["eps"], out=out)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tree.sync()
    ms_step = (t1 - t0) * 1e3 / args.steps
    walk_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    build_ms = sum(evb[k].elapsed_time(ev[k][0]) for k in range(args.steps)) / args.steps
    nodes = tree.nodes()
    n_nodes = int(nodes.shape[0])
    n_leaves = int(((nodes[:, 7] & (1 << 8)) != 0).sum().item())
    del nodes
    build_bytes = build_alg_bytes(n, n_nodes, n_leaves, args.key_bits)
    value = interactions / (ms_step * 1e-3)

    achieved = FLOPS_PER_INTERACTION * interactions / (walk_ms * 1e-3) / 1e12
    roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4),
                "traffic": read_traffic(wname, args.curve),
                # the build (all of bh_build's kernels): algorithmic bytes
                # against the HBM peak
                "build": {"bound": "hbm",
                          "achieved": round(build_bytes / (build_ms * 1e-3) / 1e9, 1),
                          "peak": HBM_PEAK_BYTES / 1e9, "unit": "GB/s",
                          "frac": round(build_bytes / (build_ms * 1e-3) / HBM_PEAK_BYTES, 4),
                          "bytes_per_call": build_bytes, "ms": round(build_ms, 4)}}

    rec = {
        "metric": METRIC, "value": value, "unit": "interactions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wname, "n": n, "theta": prm["theta"], "G": prm["G"],
                   "eps": prm["eps"], "leaf_cap": args.leaf_cap, "key_bits": args.key_bits,
                   "key_curve": args.curve,
                   "interactions_per_step": interactions,
                   "walk_ms": round(walk_ms, 4),
                   "phase_ms": {k: round(v, 4) for k, v in zip(
                       ("bbox_keys", "sort", "tree_com", "walk"), phases)}},
        "roofline": roofline,
    }
    tree.close()
    if args.curve != "morton":
        # the same step on Morton keys (the pages' order; the same cells), timed
        # the same way after the timed region, so the curve's effect can be read
        # off this line
        tm = bh.BarnesHut(n, 0, args.key_bits, args.leaf_cap, curve="morton")
        for _ in range(args.warmup):
            tm.build(src)
            tm.gravity(prm["theta"], prm["G"], prm["eps"], out=out)
        tm.sync()
        evm = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in evm:
            e[0].record(stream)
            tm.build(src)
            e[1].record(stream)
            tm.gravity(prm["theta"], prm["G"], prm["eps"], out=out)
            e[2].record(stream)
        torch.cuda.synchronize()
        tm.sync()
        rec["config"]["morton_keys"] = {
            "ms_per_step": round(sum(e[0].elapsed_time(e[2]) for e in evm) / len(evm), 4),
            "walk_ms": round(sum(e[1].elapsed_time(e[2]) for e in evm) / len(evm), 4),
            "interactions_per_step": tm.count_interactions(prm["theta"], prm["eps"])}
        tm.close()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], oc = cpu_baseline(p, prm, args.key_bits, args.leaf_cap, args.curve)
        # the numerator checked against the oracle's own count (fp64 opening
        # decisions: near-ties may flip against the GPU's fp32 ones)
        rec["config"]["interactions_oracle"] = oc["interactions"]
        rec["config"]["interactions_oracle_kind"] = oc["kind"]
        rec["config"]["interactions_rel_diff"] = (interactions - oc["interactions"]) / max(
            oc["interactions"], 1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

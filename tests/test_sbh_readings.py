"""The exact-variance study of the stochastic estimator (oracle/sbh_readings.py)
pinned to the oracle's own Monte Carlo estimator ([SBH] 方法, 关键设计 2-4): for
the readings the oracle implements (d = 2 and d = 4 per axis, strata = the
root's children) the analytic mean is the direct sum and the analytic variance
of one sample matches the sample variance of 20000 seeded samples."""
import numpy as np

import oracle
import workloads as W
from oracle.sbh_readings import Levels


def test_exact_variance_matches_oracle_samples():
    p = W.surface_sources(1 << 12, seed=10)
    q = W.box_queries(4, seed=21)
    t1 = oracle.Tree(p, 63, 1)
    exact = -oracle.direct(p, 1.0, 0.0, targets=q)[:, 3]
    for d, b in ((2, 3), (4, 6)):
        lv = Levels(p, b)
        out, sq, _ = t1.sbh(q, d=d, samples=20000, seed=5)
        for k in range(q.shape[0]):
            e, mu, v, work = lv.stratum_variance(q[k, :3].astype(np.float64), 1)
            assert abs(e - exact[k]) <= 1e-12 * exact[k]
            assert abs(mu - e) <= 1e-12 * e
            vmc = sq[k] - out[k, 3] ** 2
            assert 0.85 < vmc / v < 1.15, (d, k, v, vmc)
            assert work >= (8 if d == 2 else 64)


def test_children_per_node_readings_are_unbiased():
    p = W.surface_sources(1 << 11, seed=11)
    q = W.grid_queries(5)[::17]
    for b in (1, 2):
        lv = Levels(p, b)
        for k in range(q.shape[0]):
            e, mu, v, _ = lv.stratum_variance(q[k, :3].astype(np.float64), 1)
            assert abs(mu - e) <= 1e-12 * e and v >= 0.0

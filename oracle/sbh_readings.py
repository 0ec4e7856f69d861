"""Exact variance of the stochastic Barnes-Hut estimator under alternative
readings of its tree ([SBH] 方法, 关键设计 2-4).  Test infrastructure: CPU only,
fp64, built on the oracle's keys; nothing here is used by the library.

The estimator (one path per stratum per sample): a path starts at its
stratum's node T_0 with the source index I drawn uniformly from the stratum's
sources, and goes down the nodes T_1, T_2, ... holding I.  It adds the
stratum's monopole, and the exchange term Delta_T = (sum over T's children of
m_c f(p_c, q)) - m_T f(p_T, q) of each node T_{k-1} it reaches with K >= k,
scaled by 1 / (P(I in T_{k-1}) P(K >= k)); P(K >= k) is the product of the
continuation probabilities p_j = min(1, max(1, b_j) / b_{j+1}), b_j the
far-field ratio |q - p_{T_j}| / |B_{T_j}| (box edge) of the path's node at
depth j.  With f = m / r (the potential's magnitude, G = 1, no softening),
the mean is the exact sum and, for a fixed path index I, the second moment
over K is sum_k a_k^2 P_k + 2 sum_{k<l} a_k a_l P_l with a_k the scaled
exchange term of step k and P_k = P(K >= k).  So the variance of a stratum's
sample is the mean over its sources of that second moment minus the square
of the mean: no sampling noise.

Readings compared (the notes give d as the branching factor per dimension and
use d = 2 for their Barnes-Hut tree, d = 4 for theirs; the strata are the
root's children):
  * bits per level b of the Morton key (x, y, z interleaved): b = 3 is the
    octree (d = 2 per axis, 8 children), b = 6 two octree levels per step
    (d = 4 per axis, 64 children), b = 1 a binary tree and b = 2 a 4-ary one
    (d read as children per node);
  * strata: the nodes at depth 1 (the root's children) or at depth 2.
Boxes are the cells' boxes: a cell of bit depth t has edge L 2^-floor(t/3)
(its longest edge).  Tight source boxes are not a reading here: a singleton
node's tight box has size zero, its far-field ratio is infinite and the
continuation into it has probability zero, which would bias the estimator.

    python3 oracle/sbh_readings.py [--queries 200] [--m 15,17]
"""
import argparse
import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_HERE))

import oracle  # noqa: E402


class Levels:
    """The cells of the radix tree over sorted Morton keys with b bits per
    level: level j holds the runs of keys sharing their top min(j b, bits)
    bits (bits = 3 * (key_bits // 3))."""

    def __init__(self, p, b, key_bits=63):
        t = oracle.Tree(p, key_bits, 1, curve="morton")
        keys = t.keys()
        perm = t.perm()
        lo, _, L = t.bbox()
        del t
        bits = 3 * (key_bits // 3)
        keys = keys[perm].astype(np.uint64)
        q = p[perm].astype(np.float64)
        self.n = n = p.shape[0]
        self.pos, self.m = q[:, :3], q[:, 3]
        self.levels = []
        depth = 0
        while True:
            sh = np.uint64(bits - depth)
            pref = keys >> sh if depth > 0 else np.zeros(n, np.uint64)
            starts = np.flatnonzero(np.r_[True, pref[1:] != pref[:-1]])
            counts = np.diff(np.r_[starts, n])
            cid = np.repeat(np.arange(starts.size), counts)
            mass = np.add.reduceat(self.m, starts)
            com = np.add.reduceat(self.m[:, None] * self.pos, starts, axis=0) / mass[:, None]
            edge = L * 2.0 ** -(depth // 3)
            self.levels.append(dict(starts=starts, counts=counts, cid=cid, mass=mass, com=com,
                                    edge=edge, depth=depth))
            if depth >= bits or counts.max() == 1:
                break
            depth = min(depth + b, bits)
        # parent of each cell of level j + 1 in level j
        for j in range(len(self.levels) - 1):
            self.levels[j + 1]["parent"] = self.levels[j]["cid"][self.levels[j + 1]["starts"]]

    def stratum_variance(self, qpt, s_level):
        """(exact sum, sum over strata of the variance of one path, mean
        number of child evaluations of one sample) at query point qpt."""
        lv = self.levels
        nl = len(lv)
        phi, beta, delta = [], [], []
        for j in range(nl):
            r = np.linalg.norm(lv[j]["com"] - qpt, axis=1)
            phi.append(lv[j]["mass"] / r)
            beta.append(r / lv[j]["edge"])
        nchild = []
        for j in range(nl):
            if j + 1 < nl:
                s = np.bincount(lv[j + 1]["parent"], weights=phi[j + 1],
                                minlength=lv[j]["starts"].size)
                c = np.bincount(lv[j + 1]["parent"], minlength=lv[j]["starts"].size)
                d = s - phi[j]
                d[lv[j]["counts"] == 1] = 0.0
                delta.append(d)
                nchild.append(c)
            else:
                delta.append(np.zeros_like(phi[j]))
                nchild.append(np.zeros(lv[j]["starts"].size, np.int64))
        exact = float(np.sum(self.m / np.linalg.norm(self.pos - qpt, axis=1)))
        # per source I: its path from the stratum node down
        st = lv[s_level]["cid"]
        n_s = lv[s_level]["counts"][st].astype(np.float64)
        P = np.ones(self.n)
        A = np.zeros(self.n)       # sum of the a_k so far
        E1 = np.zeros(self.n)
        E2 = np.zeros(self.n)
        cost = np.zeros(self.n)
        for j in range(s_level, nl - 1):
            c0 = lv[j]["cid"]
            c1 = lv[j + 1]["cid"]
            b0 = beta[j][c0]
            b1 = beta[j + 1][c1]
            p = np.minimum(1.0, np.maximum(1.0, b0) / b1)
            P = P * p
            qT = lv[j]["counts"][c0] / n_s
            dT = delta[j][c0]
            live = P > 0
            a = np.where(live, dT / (qT * np.where(live, P, 1.0)), 0.0)
            E1 += a * P
            E2 += a * a * P + 2.0 * a * A * P
            A += a
            cost += P * nchild[j][c0] * (dT != 0.0)
        # base term: the stratum's monopole, deterministic
        ns = lv[s_level]["starts"].size
        w = 1.0 / lv[s_level]["counts"][st]
        m1 = np.bincount(st, weights=E1 * w, minlength=ns)
        m2 = np.bincount(st, weights=E2 * w, minlength=ns)
        var = float(np.sum(np.maximum(m2 - m1 * m1, 0.0)))
        mean = float(np.sum(phi[s_level]) + np.sum(m1))
        work = float(np.bincount(st, weights=cost * w, minlength=ns).sum()) + ns
        return exact, mean, var, work


def main():
    import workloads as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--queries", type=int, default=200)
    ap.add_argument("--m", default="15,17")
    ap.add_argument("--seed", type=int, default=10)
    args = ap.parse_args()
    rng = np.random.default_rng(7)
    grid = W.grid_queries()
    qsets = {"grid100": grid[rng.choice(grid.shape[0], args.queries, replace=False)],
             "uniform": W.box_queries(args.queries, seed=21)}
    readings = [(3, 1), (6, 1), (1, 1), (2, 1), (3, 2)]
    print("# columns: M, query set, reading (b bits per level, depth of the strata), median and "
          "mean over queries of the standard deviation of one sample (S = 1), the same of the "
          "walk's |error| (theta 0.5, leaf capacity 16), median over queries of sd / |walk "
          "error|, child evaluations per query of one sample, walk interactions per query, "
          "largest |mean - exact| / exact")
    for lm in [int(x) for x in args.m.split(",")]:
        p = W.surface_sources(1 << lm, seed=args.seed)
        bh = oracle.Tree(p, 63, 16)
        lvs = {b: Levels(p, b) for b in sorted({b for b, _ in readings})}
        for qn, qa in qsets.items():
            out, ni, _ = bh.gravity(0.5, 1.0, 0.0, targets=qa)
            ex = oracle.direct(p, 1.0, 0.0, targets=qa)[:, 3]
            bh_err = np.abs(out[:, 3] - ex)
            for b, sl in readings:
                sds, works, bias = [], [], []
                for k in range(qa.shape[0]):
                    e, mu, v, wk = lvs[b].stratum_variance(qa[k, :3].astype(np.float64), sl)
                    sds.append(np.sqrt(v))
                    works.append(wk)
                    bias.append(abs(mu - e) / e)
                sds = np.array(sds)
                print("2^%d %-8s b=%d strata@%d  %.3e %.3e  %.3e %.3e  %7.1f  %8.0f  %6.0f  %.1e" % (
                    lm, qn, b, sl, np.median(sds), sds.mean(), np.median(bh_err), bh_err.mean(),
                    np.median(sds / np.maximum(bh_err, 1e-300)), np.mean(works), ni.mean(),
                    max(bias)), flush=True)


if __name__ == "__main__":
    main()

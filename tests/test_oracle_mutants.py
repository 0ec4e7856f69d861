"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (a text substitution; the
oracle itself is untouched), compiles it on the CPU, and runs the pin tests of
test_oracle.py against it in a child process: at least one pin must fail.  A
planted mistake can make the C code write out of bounds (no depth limit,
unclamped keys), so the mutated library is never loaded into the test process
itself; a child that dies counts as caught.  CPU only."""
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text in oracle.c, planted mistake)
MUTANTS = [
    ("pair_sign", "d[a] = xs[a] - w->x[a];", "d[a] = w->x[a] - xs[a];"),
    ("potential_sign", "w->phi -= w->G * m * inv_r;", "w->phi += w->G * m * inv_r;"),
    ("dropped_softening", "double d[3], r2 = w->eps_sq;", "double d[3], r2 = 0.0;"),
    ("inverse_square_power", "double inv_r3 = inv_r * inv_r * inv_r;\n    for (int a = 0; a < 3; ++a) w->acc",
     "double inv_r3 = inv_r * inv_r;\n    for (int a = 0; a < 3; ++a) w->acc"),
    ("half_edge_w", "double width = ldexp(t->L, -cell->level);",
     "double width = ldexp(t->L, -cell->level - 1);"),
    ("mac_non_strict", "int accept = threshold < r_sq;", "int accept = threshold <= r_sq;"),
    ("mac_to_cell_centre", "double d = cell->com[a] - w->x[a];",
     "double d = t->lo[a] + ldexp(t->L, -cell->level) * ((double)cell->corner[a] + 0.5) - w->x[a];"),
    ("self_not_excluded", "if (p == w->self) continue;", "if (p == -7) continue;"),
    ("octant_bit_order", "return ox + 2 * oy + 4 * oz;", "return oz + 2 * oy + 4 * ox;"),
    ("key_axis_order", "key |= ((qa >> k) & 1u) << (3 * k + a);",
     "key |= ((qa >> k) & 1u) << (3 * k + (2 - a));"),
    ("leaf_rule_le", "if (count <= t->leaf_cap || level == t->bits) {",
     "if (count < t->leaf_cap || level == t->bits) {"),
    ("no_max_depth", "if (count <= t->leaf_cap || level == t->bits) {",
     "if (count <= t->leaf_cap || level == t->bits + 1) {"),
    ("com_unweighted", "s[a] += mp * (double)t->src[4 * p + a];", "s[a] += (double)t->src[4 * p + a];"),
    ("bbox_extent_min", "if (ext > t->L) t->L = ext;", "if (ext < t->L || t->L == 0.0) t->L = ext;"),
    ("key_no_clamp", "uint64_t qa = (f >= (double)top) ? top : (uint64_t)f;",
     "uint64_t qa = (uint64_t)f & top;"),
    ("unstable_order", "return (a > b) - (a < b);", "return (a < b) - (a > b);"),
    ("direct_self_pair", "if (j == self) continue;", "if (j == -7) continue;"),
    ("direct_sign", "d[a] = (double)src[4 * j + a] - x[a];", "d[a] = x[a] - (double)src[4 * j + a];"),
    ("vote_first_member_decides", "if (!accept) any_open = 1;",
     "if (k == 0) any_open = !accept;"),
    ("vote_all_must_open", "if (!accept) any_open = 1;\n    }",
     "if (!accept) any_open += 1;\n    }\n    any_open = any_open == g->m;"),
    ("vote_leaf_self_kept", "            int64_t p = t->idx[cell->off + q];\n            if (p == w->self) continue;",
     "            int64_t p = t->idx[cell->off + q];"),
    ("sbh_no_count_ratio", "const double scale = w * (double)c->count / (double)cell->count;",
     "const double scale = w;"),
    ("sbh_no_roulette_weight", "w /= pk;", "w /= 1.0;"),
    ("sbh_exchange_sign", "est[a] -= scale * f[a];", "est[a] += scale * f[a];"),
    ("sbh_roulette_inverted", "if (!(u < pk)) break;", "if (u < pk) break;"),
    ("philox_multiplier", "(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F55u * c0"),
    ("target_clamp_low", "uint64_t qa = !(f >= 0.0) ? 0 :", "uint64_t qa = !(f >= 0.0) ? top :"),
    ("hilbert_no_gray_code", "for (int i = 1; i < 3; ++i) X[i] ^= X[i - 1];",
     "for (int i = 1; i < 3; ++i) X[i] ^= 0;"),
    ("hilbert_half_exchange", "                X[0] ^= t;\n                X[i] ^= t;",
     "                X[0] ^= t;"),
    ("partition_by_octant_not_digit", "digit_count[digit_of(t, t->idx[off + k], level + 1)]++;",
     "digit_count[octant_of(t, t->idx[off + k], level + 1)]++;"),
    ("vote_leaf_monopole", "            interact(&g->w[k], cell->mass, cell->com);",
     "            interact(&g->w[k], cell->mass, g->w[k].x);"),
]

PIN_TESTS = [name for name in dir(pins) if name.startswith("test_")]


def _build_mutant(name, old, new, workdir):
    text = open(SRC).read()
    assert old in text, "mutation site not found in oracle.c: %s" % name
    path = os.path.join(workdir, "oracle_%s.c" % name)
    with open(path, "w") as fh:
        fh.write(text.replace(old, new, 1))
    lib = os.path.join(workdir, "liboracle_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", lib, path, "-lm"], check=True)
    return lib


def _run_pins_against(lib_path):
    """Run every pin with the oracle module pointed at lib_path; return the
    names of the pins that failed."""
    saved = oracle._lib
    failed = []
    try:
        oracle._lib = None
        real_lib = oracle._LIB
        oracle._LIB = lib_path
        # load through the module's own loader (it checks mtimes: skip building)
        orig_build = oracle.build
        oracle.build = lambda force=False: lib_path
        try:
            oracle.lib()
            for name in PIN_TESTS:
                fn = getattr(pins, name)
                params = getattr(fn, "pytestmark", [])
                cases = [()]
                for mark in params:
                    if mark.name == "parametrize":
                        argnames, values = mark.args[0], mark.args[1]
                        argnames = [a.strip() for a in argnames.split(",")] if isinstance(
                            argnames, str) else list(argnames)
                        new = []
                        for c in cases:
                            for v in values:
                                v = v if isinstance(v, tuple) else (v,)
                                new.append(c + tuple(zip(argnames, v)))
                        cases = new
                for case in cases:
                    try:
                        fn(oracle, **dict(case))
                    except Exception:  # an assertion, or a crash the mistake causes
                        failed.append(name)
                        break
        finally:
            oracle.build = orig_build
            oracle._LIB = real_lib
    finally:
        oracle._lib = saved
    return failed


_CHILD = """
import json, sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import test_oracle_mutants as m
print("FAILED_PINS " + json.dumps(m._run_pins_against(sys.argv[1])), flush=True)
"""


def _pins_in_child(lib_path):
    """Failed pin names from a child process, or None when the child died."""
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _CHILD, lib_path, here, os.path.dirname(here)],
                       capture_output=True, text=True, timeout=600, env=env)
    for line in r.stdout.splitlines():
        if line.startswith("FAILED_PINS "):
            return json.loads(line[len("FAILED_PINS "):])
    return None


@pytest.fixture(scope="module")
def mutant_results(orc):
    """Every mutant (and the unmutated control) built and run, four at a time."""
    from concurrent.futures import ThreadPoolExecutor
    cases = [("control", "", "")] + MUTANTS
    with tempfile.TemporaryDirectory() as d:
        def one(case):
            return case[0], _pins_in_child(_build_mutant(case[0], case[1], case[2], d))
        with ThreadPoolExecutor(max_workers=4) as pool:
            return dict(pool.map(one, cases))


def test_unmutated_copy_passes_every_pin(mutant_results):
    """Control: the harness itself makes no pin fail, and the child runs to its end."""
    assert mutant_results["control"] == [], mutant_results["control"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant_results, name, old, new):
    failed = mutant_results[name]
    assert failed is None or failed, "no pin caught the planted mistake %r" % name

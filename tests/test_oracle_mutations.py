"""Plant plausible mistakes in a copy of the oracle and require the pins to catch each.

Every mutant is built on the CPU from a patched copy of oracle.c in a
temporary directory; the pin suite then runs against it in a subprocess and
must fail.  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement) -- the first occurrence is replaced
MUTANTS = [
    ("mean divides by block size", "o[c] = s / (double)(t1 - t0);", "o[c] = s / (double)bs;"),
    ("score sign", "cand[j - c0].s = s;", "cand[j - c0].s = -s;"),
    ("tie-break reversed", "return (x->j > y->j) - (x->j < y->j);",
     "return (x->j < y->j) - (x->j > y->j);"),
    ("group drops heads", "for (int32_t h = (int32_t)kvh * g; h < (int32_t)kvh * g + g; ++h)",
     "for (int32_t h = (int32_t)kvh * g; h < (int32_t)kvh * g + 1; ++h)"),
    ("no 1/sqrt(d) scale", "z[t] = s * scale;", "z[t] = s;"),
    ("softmax exponent sign", "z[t] = exp(z[t] - zmax);", "z[t] = exp(zmax - z[t]);"),
    ("K and V swapped", "rows, rows, k, v, NULL, NULL, scale, z,\n                      out",
     "rows, rows, v, k, NULL, NULL, scale, z,\n                      out"),
    ("wrong GQA head map", "int64_t b = bh / Hq, h = bh % Hq, kvh = h / g;",
     "int64_t b = bh / Hq, h = bh % Hq, kvh = h % Hkv;"),
    ("local range off by one", "int32_t l_beg = nb - n_local > 0 ? nb - n_local : 0;",
     "int32_t l_beg = nb - n_local - 1 > 0 ? nb - n_local - 1 : 0;"),
    ("keep ratio rounded up", "floor(keep_ratio * (double)nb + 0.5)", "ceil(keep_ratio * (double)nb)"),
    ("window off by one", "int32_t t0 = p - window + 1 > 0 ? p - window + 1 : 0;",
     "int32_t t0 = p - window > 0 ? p - window : 0;"),
    ("tile pools one query", "int32_t i1 = i0 + q_tile < C ? i0 + q_tile : C;",
     "int32_t i1 = i0 + 1;"),
    ("branch average", "for (int32_t c = 0; c < d; ++c) dst[c] /= 3.0;",
     "for (int32_t c = 0; c < d; ++c) dst[c] /= 2.0;"),
    ("concat drops the query's own token", "for (int32_t t = t0; t <= p; ++t) rka[na++]",
     "for (int32_t t = t0; t < p; ++t) rka[na++]"),
    ("concat reads K as V for the dense entries", ": t < src[1] ? (double)v128[rka[t] + c]",
     ": t < src[1] ? (double)k128[rka[t] + c]"),
    ("sink logit sign", "double den = has_sink ? exp(zs - zmax) : 0.0;",
     "double den = has_sink ? exp(zmax - zs) : 0.0;"),
    ("adaptive threshold from the lowest anchor",
     "double tau = fixed > 0 ? a_max + margin * (a_max - a_min) : -INFINITY;",
     "double tau = fixed > 0 ? a_min + margin * (a_max - a_min) : -INFINITY;"),
    ("adaptive counts scores equal to the threshold", "if (sc[j] > tau) ++above;",
     "if (sc[j] >= tau) ++above;"),
    ("adaptive anchors skip the local blocks", "      if (j < c0 || j >= c1) {\n        if (sc[j] > a_max)",
     "      if (j < c0) {\n        if (sc[j] > a_max)"),
    ("adaptive k ignores the lower bound",
     "int32_t k = above < k_lo ? k_lo : (above > k_hi ? k_hi : above);",
     "int32_t k = above > k_hi ? k_hi : above;"),
    ("e4m3 ties away from zero", "double r = rint(a / ldexp(1.0, E - 3));",
     "double r = floor(a / ldexp(1.0, E - 3) + 0.5);"),
    ("e4m3 exponent bias 8", "double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);",
     "double v = e ? ldexp(1.0 + m / 8.0, e - 8) : ldexp(m / 8.0, -7);"),
    ("fp8 scale for the E4M3 max of the FNUZ variant", "float sc = amax / 448.0f;",
     "float sc = amax / 240.0f;"),
    ("fp8 values use the key scale", "vs[n] = (double)vscales[p * sstride + blk];",
     "vs[n] = (double)kscales[p * sstride + blk];"),
    ("branch sink uses the wrong lse", "double keep = has_sink ? 1.0 / (1.0 + exp(zs - l[br])) : 1.0;",
     "double keep = has_sink ? 1.0 / (1.0 + exp(zs - l[0])) : 1.0;"),
    ("bf16 ties away from zero", "double ri = rint(s);", "double ri = floor(s + 0.5);"),
    ("dense branch reads K as V", "E128, rk, rk, NULL, NULL, k128, v128,",
     "E128, rk, rk, NULL, NULL, k128, k128,"),
    ("lse drops the max", "return zmax + log(l);", "return log(l);"),
    ("weights not normalised", "double p = z[t] / l;", "double p = z[t];"),
    ("fp32 summary accumulates in fp64", "        float s = 0.0f;\n        for (int32_t t = t0; t < t1; ++t)\n          s = s + (float)bf(",
     "        double s = 0.0;\n        for (int32_t t = t0; t < t1; ++t)\n          s = s + (float)bf("),
    ("fp32 summary adds the tokens last to first", "        for (int32_t t = t0; t < t1; ++t)\n          s = s + (float)bf(",
     "        for (int32_t t = t1 - 1; t >= t0; --t)\n          s = s + (float)bf("),
    ("fp32 summary multiplies by a rounded reciprocal", "o[c] = s / (float)(t1 - t0);",
     "o[c] = s * (1.0f / (float)(t1 - t0));"),
    ("fp8 attention ignores the key scale",
     "sdot += bf(q[bh * d + c]) * (ks * lut[kr[c]]);", "sdot += bf(q[bh * d + c]) * (lut[kr[c]]);"),
    ("fp8 keys take the first block's scale", "double ks = (double)kscales[p * sstride + blk];",
     "double ks = (double)kscales[p * sstride];"),
    ("branch A keys are the unrounded means",
     "k4[i] = (float)bf(oracle_round_bf16(ks_exact[i]));", "k4[i] = (float)ks_exact[i];"),
    ("branch A values are the unrounded means",
     "v4[i] = (float)bf(oracle_round_bf16(tmp4[i]));", "v4[i] = (float)tmp4[i];"),
    ("branch B keys are the unrounded means",
     "k128[i] = (float)bf(oracle_round_bf16(tmp128[i]));", "k128[i] = (float)tmp128[i];"),
    ("branch B values are the unrounded means",
     "v128[i] = (float)bf(oracle_round_bf16(tmp128[i]));", "v128[i] = (float)tmp128[i];"),
    ("pooled query skips a dimension", "for (int32_t c = 0; c < d; ++c) qbar[c] += bf(q[(b * Hq + h)",
     "for (int32_t c = 1; c < d; ++c) qbar[c] += bf(q[(b * Hq + h)"),
    ("indexer scores the exact means", "const double* keys = indexer == 0 ? ks_b16 : ks_exact;",
     "const double* keys = ks_exact;"),
    ("indexer rounds the exact mean", "ks_b16[i] = bf(oracle_round_bf16((double)f32[i]));",
     "ks_b16[i] = bf(oracle_round_bf16(ks_exact[i]));"),
    ("indexer keys are the unrounded fp32 means", "ks_b16[i] = bf(oracle_round_bf16((double)f32[i]));",
     "ks_b16[i] = (double)f32[i];"),
]


# mutants the randomised properties (test_oracle_properties.py) must catch on their own
PROPERTY_MUTANTS = ["mean divides by block size", "score sign", "tie-break reversed",
                    "group drops heads", "no 1/sqrt(d) scale", "K and V swapped",
                    "wrong GQA head map", "local range off by one", "lse drops the max",
                    "weights not normalised", "indexer scores the exact means",
                    "indexer rounds the exact mean", "indexer keys are the unrounded fp32 means"]

SUITES = {"pins": "test_oracle_pins.py", "properties": "test_oracle_properties.py"}


def run_mutant(suite, name, workdir):
    """Build oracle.c with mutant `name` in `workdir` and run the `suite` against it in a
    subprocess; returns (return code, the end of its output)."""
    old, new = next((o, n) for m, o, n in MUTANTS if m == name)
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
    cfile = os.path.join(workdir, "oracle.c")
    with open(cfile, "w") as f:
        f.write(src.replace(old, new, 1))
    with open(os.path.join(workdir, "oracle.h"), "w") as f:
        f.write(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = os.path.join(workdir, "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    cfile, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, BSA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", SUITES[suite])],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


_ALL = None


def result(suite, name, tmp_path):
    """The mutant's run.  In a serial session every mutant's run is started on first use,
    several at a time (each is its own process); under pytest-xdist each test runs its own."""
    global _ALL
    if os.environ.get("PYTEST_XDIST_WORKER"):
        return run_mutant(suite, name, str(tmp_path))
    if _ALL is None:
        jobs = [("pins", m[0]) for m in MUTANTS] + [("properties", m) for m in PROPERTY_MUTANTS]
        base = tempfile.mkdtemp(prefix="oracle_mutants_")
        dirs = {}
        for i, job in enumerate(jobs):
            dirs[job] = os.path.join(base, str(i))
            os.makedirs(dirs[job])
        try:
            with ThreadPoolExecutor(max_workers=max(1, min(6, (os.cpu_count() or 2) - 1))) as ex:
                futs = {job: ex.submit(run_mutant, job[0], job[1], dirs[job]) for job in jobs}
                _ALL = {job: f.result() for job, f in futs.items()}
        finally:
            shutil.rmtree(base, ignore_errors=True)
    return _ALL[(suite, name)]


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name):
    rc, out = result("pins", name, tmp_path)
    assert rc != 0, f"pins did not catch mutant '{name}'\n{out}"


@pytest.mark.parametrize("name", PROPERTY_MUTANTS)
def test_properties_catch_mutant(tmp_path, name):
    rc, out = result("properties", name, tmp_path)
    assert rc != 0, f"properties did not catch mutant '{name}'\n{out}"

"""The oracle's pins must catch plausible mistakes: each case below plants one
mistake in a copy of oracle/oracle.c (a dropped term, a wrong constant, sign,
order or index, a missing check), builds it, and runs the pin tests
(tests/test_oracle.py) against that build. Every mutant must make at least
one pin fail; a surviving mutant names a part of the oracle the pins do not
hold. CPU only; the planted mistakes live in temporary copies."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("first moment: beta1 decay dropped",
     "float m_old = 0.9f * m[i];", "float m_old = m[i];"),
    ("first moment: (1 - beta1) factor dropped",
     "float m_new_part = 0.1f * gp;", "float m_new_part = gp;"),
    ("first moment: beta1 = 0.99",
     "float m_old = 0.9f * m[i];", "float m_old = 0.99f * m[i];"),
    ("second moment: square dropped",
     "float gsq = gp * gp;", "float gsq = gp;"),
    ("second moment: (1 - beta2) factor is 0.01",
     "float v_new_part = 0.001f * gsq;", "float v_new_part = 0.01f * gsq;"),
    ("bias correction: beta1 used for v",
     "*bc2 = (float)(1.0 - pow(0.999, (double)t));", "*bc2 = (float)(1.0 - pow(0.9, (double)t));"),
    ("bias correction: t + 1",
     "*bc1 = (float)(1.0 - pow(0.9, (double)t));", "*bc1 = (float)(1.0 - pow(0.9, (double)t + 1.0));"),
    ("bias correction of v dropped",
     "float vh = vi / bc2;", "float vh = vi;"),
    ("epsilon inside the square root",
     "float root = sqrtf(vh);\n        float den = root + 1e-8f;",
     "float root = sqrtf(vh + 1e-8f);\n        float den = root;"),
    ("epsilon 1e-6",
     "float den = root + 1e-8f;", "float den = root + 1e-6f;"),
    ("decay applied after the step",
     "w[i] = decayed - stepv;", "w[i] = (w[i] - stepv) * decay;"),
    ("step added instead of subtracted",
     "w[i] = decayed - stepv;", "w[i] = decayed + stepv;"),
    ("decay ignores the learning rate",
     "*decay = (float)(1.0 - (double)lr * (double)wd);", "*decay = (float)(1.0 - (double)wd);"),
    ("step uses the uncorrected first moment",
     "float num = lr * mh;", "float num = lr * mi;"),
    ("clip applied below the threshold",
     "if (norm > (double)clip) return", "if (norm < (double)clip) return"),
    ("clip factor inverted",
     "return (float)((double)clip / norm);", "return (float)(norm / (double)clip);"),
    ("clip factor ignored in the update",
     "float gp = g[i] * s;", "float gp = g[i];"),
    ("norm without the square root",
     "return sqrt(oracle_sumsq_finish(st));", "return oracle_sumsq_finish(st);"),
    ("norm sums absolute values",
     "double x = (double)g[i] * (double)g[i];", "double x = fabs((double)g[i]);"),
    ("norm squares in float32",
     "double x = (double)g[i] * (double)g[i];", "double x = (double)(g[i] * g[i]);"),
    ("norm compensation dropped",
     "return state[0] + state[1];", "return state[0];"),
    ("non-finite norm not skipped by the update",
     "    if (!isfinite(norm)) return ORACLE_SKIPPED;\n    float s = oracle_clip_scale(norm, clip);\n"
     "    float bc1",
     "    float s = oracle_clip_scale(norm, clip);\n    float bc1"),
    ("micro-batch scale ignored",
     "for (int64_t i = 0; i < n; ++i) g[i] = g[i] * scale;", "(void)scale;"),
    ("header fields swapped",
     "put_i32_le(buf + 0, step);\n    put_i32_le(buf + 4, (int32_t)n);",
     "put_i32_le(buf + 0, (int32_t)n);\n    put_i32_le(buf + 4, step);"),
    ("m and v regions swapped in the pack",
     "uint8_t *pw = buf + 8, *pm = buf + 8 + 4 * n, *pv = buf + 8 + 8 * n;",
     "uint8_t *pw = buf + 8, *pv = buf + 8 + 4 * n, *pm = buf + 8 + 8 * n;"),
    ("big-endian integers",
     "p[0] = (uint8_t)(u & 0xffu);\n    p[1] = (uint8_t)((u >> 8) & 0xffu);\n"
     "    p[2] = (uint8_t)((u >> 16) & 0xffu);\n    p[3] = (uint8_t)((u >> 24) & 0xffu);",
     "p[3] = (uint8_t)(u & 0xffu);\n    p[2] = (uint8_t)((u >> 8) & 0xffu);\n"
     "    p[1] = (uint8_t)((u >> 16) & 0xffu);\n    p[0] = (uint8_t)((u >> 24) & 0xffu);"),
    ("size omits the header",
     "return 8 + 12 * n;", "return 12 * n;"),
    ("unpack accepts a different n",
     "if (n_expected > 0 && (int64_t)n != n_expected) return ORACLE_EHEADER;", ""),
    ("unpack accepts a longer buffer",
     "if (len != 8 + 12 * (int64_t)n) return ORACLE_ESIZE;",
     "if (len < 8 + 12 * (int64_t)n) return ORACLE_ESIZE;"),
    ("unpack accepts a negative step",
     "if (n <= 0 || step < 0) return ORACLE_EHEADER;", "if (n <= 0) return ORACLE_EHEADER;"),
    ("unpack swaps m and v",
     "m[i] = get_f32_le(pm + 4 * i);\n        v[i] = get_f32_le(pv + 4 * i);",
     "m[i] = get_f32_le(pv + 4 * i);\n        v[i] = get_f32_le(pm + 4 * i);"),
    ("float64 definition: square dropped",
     "v[i] = beta2 * v[i] + (1.0 - beta2) * (gi * gi);", "v[i] = beta2 * v[i] + (1.0 - beta2) * gi;"),
    ("float64 definition: bias correction with t + 1",
     "const double corr1 = 1.0 - pow(beta1, (double)t);",
     "const double corr1 = 1.0 - pow(beta1, (double)t + 1.0);"),
    ("float64 definition: decay applied after the step",
     "w[i] = keep * w[i] - lr * m_hat / (sqrt(v_hat) + eps);",
     "w[i] = keep * (w[i] - lr * m_hat / (sqrt(v_hat) + eps));"),
    ("float64 definition: clip factor inverted",
     "const double scale = (norm > clip) ? clip / norm : 1.0;",
     "const double scale = (norm > clip) ? norm / clip : 1.0;"),
    ("float64 definition: moments not carried between updates",
     "m[i] = beta1 * m[i] + (1.0 - beta1) * gi;", "m[i] = (1.0 - beta1) * gi;"),
]


def _kill(tmp, idx, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name!r}: its text must occur exactly once"
    mutated = src.replace(old, new)
    d = os.path.join(tmp, f"m{idx}")
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, "oracle.c")
    so = os.path.join(d, "liboracle.so")
    open(c, "w").write(mutated)
    r = subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                        "-shared", c, "-o", so, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        return name, "does not compile: " + r.stderr[-300:]
    env = dict(os.environ, RCS_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], capture_output=True, text=True,
                       env=env, cwd=ROOT, timeout=300)
    return name, ("killed" if r.returncode != 0 else "SURVIVED")


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(lambda a: _kill(str(tmp_path), *a),
                              [(i, *m) for i, m in enumerate(MUTANTS)]))
    bad = [(name, how) for name, how in results if how != "killed"]
    assert not bad, bad


def test_the_unmutated_oracle_passes_its_pins(tmp_path):
    """Control: the same harness with no mistake planted passes."""
    so = tmp_path / "liboracle.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", SRC, "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, RCS_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], capture_output=True, text=True,
                       env=env, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]

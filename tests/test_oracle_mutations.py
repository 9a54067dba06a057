"""Plant mistakes in the oracle (on the CPU) and check that its pins catch
each one: the oracle source is copied, one plausible slip is introduced,
the copy is built into a temporary library, and the pin suite is run
against it in a subprocess; it must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "dropped correction factor":
        ("d = d * corr + exp(v - m_new);", "d = d + exp(v - m_new);"),
    "exponent sign flipped":
        ("double t = (v == -INFINITY) ? 0.0 : exp(v - m);",
         "double t = (v == -INFINITY) ? 0.0 : exp(m - v);"),
    "row stride replaced by N":
        ("double v = load_elem(x, dtype, i * ld + j);",
         "double v = load_elem(x, dtype, i * N + j);"),
    "identity guard lost":
        ("if (m == -INFINITY) {", "if (0) {"),
    "merge rescale of b dropped":
        ("*d_out = da * exp(ma - m) + db * exp(mb - m);",
         "*d_out = da * exp(ma - m) + db;"),
    "lse without m":
        ("if (lse_out) lse_out[i] = m + logd;",
         "if (lse_out) lse_out[i] = logd;"),
    "log-softmax without log d":
        ("y[i * N + j] = (load_elem(x, dtype, i * ld + j) - m) - logd;",
         "y[i * N + j] = (load_elem(x, dtype, i * ld + j) - m);"),
    "log-softmax without m":
        ("y[i * N + j] = (load_elem(x, dtype, i * ld + j) - m) - logd;",
         "y[i * N + j] = load_elem(x, dtype, i * ld + j) - logd;"),
    "cross-entropy sign of the label term":
        ("loss[i] = (m - load_elem(x, dtype, i * ld + c)) + logd;",
         "loss[i] = (m + load_elem(x, dtype, i * ld + c)) + logd;"),
    "log d takes the max's own term":
        ("*logd_out = isfinite(m) ? log1p(s) : log(d);",
         "*logd_out = isfinite(m) ? log1p(d) : log(d);"),
    "log d keeps every instance of the max":
        ("            found = 1;          /* the max's own 1, left out of s */\n            continue;",
         "            found = 1;          /* the max's own 1, left out of s */"),
    "cross-entropy mean counts ignored rows":
        ("            loss[i] = 0.0;\n            continue;",
         "            loss[i] = 0.0;\n            count = count + 1;\n            continue;"),
    "masked columns read":
        ("row_stats(x, dtype, base, n, &m, &d, &logd);",
         "row_stats(x, dtype, base, N, &m, &d, &logd);"),
    "causal offset off by one":
        ("if (causal >= 0 && i + causal + 1 < n) n = i + causal + 1;",
         "if (causal >= 0 && i + causal < n) n = i + causal;"),
    "attention scale dropped":
        ("    return scale * dot;", "    return dot;"),
    "attention key row stride replaced by the query's":
        ("load_elem(k, dtype, j * ldk + c);", "load_elem(k, dtype, j * ldq + c);"),
    "attention probabilities not normalised":
        ("double p = t / l;", "double p = t;"),
    "attention value rows reversed":
        ("p * load_elem(v, dtype, j * ldv + c);",
         "p * load_elem(v, dtype, (n - 1 - j) * ldv + c);"),
    "attention causal mask off by one":
        ("return (last + 1 < Sk) ? last + 1 : Sk;",
         "return (last < Sk) ? last : Sk;"),
    "attention lse without max":
        ("if (lse) lse[r] = m + log(l);", "if (lse) lse[r] = log(l);"),
    "online output rescale dropped":
        ("for (int64_t c = 0; c < D; ++c) acc[c] = alpha * acc[c];",
         "for (int64_t c = 0; c < D; ++c) acc[c] = acc[c];"),
    "pass 2 with a state: exponent sign flipped":
        ("log_form ? (v - m) - log(d) : exp(v - m) / d;",
         "log_form ? (v - m) - log(d) : exp(m - v) / d;"),
    "pass 2 with a state: log form without log d":
        ("log_form ? (v - m) - log(d) : exp(v - m) / d;",
         "log_form ? (v - m) : exp(v - m) / d;"),
    "online normaliser rescale dropped":
        ("            l = alpha * l;", "            l = l;"),
}

PIN_FILES = ("test_oracle.py", "test_oracle_attention.py")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old}"
    mutated = tmp_path / "oracle.c"
    mutated.write_text(src.replace(old, new))
    (tmp_path / "oracle.h").write_text(
        open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                    "-ffp-contract=off", "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x",
                        "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"

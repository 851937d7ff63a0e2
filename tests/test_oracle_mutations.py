"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle source, plants one mistake (a dropped term, a
wrong sign, bound, index or tie rule), builds the copy, and runs the CPU pin
tests against it (test_oracle_*.py, in a child process with LSA_ORACLE_LIB
pointing at the mutant).  The pins pass on the real oracle; every mutant must
make at least one of them fail."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "lsa_oracle.c")
PINS = [os.path.join(HERE, f) for f in ("test_oracle_formats.py", "test_oracle_score.py",
                                        "test_oracle_select.py", "test_oracle_labels.py",
                                        "test_oracle_fetch.py", "test_oracle_attention.py",
                                        "test_oracle_lightning.py")]

# (name, exact snippet of lsa_oracle.c, planted replacement)
MUTANTS = [
    ("bf16 decode shift", "uint32_t w = (uint32_t)bits << 16;", "uint32_t w = (uint32_t)bits << 15;"),
    ("bf16 rounds down", "double r = nearbyint(ldexp(m, -ulp_exp));", "double r = floor(ldexp(m, -ulp_exp));"),
    ("e4m3 exponent bias", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3 subnormal scale", "v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    ("softplus without |x|", "return fmax(x, 0.0) + log1p(exp(-fabs(x)));", "return fmax(x, 0.0) + log1p(exp(-x));"),
    ("sigmoid sign", "double lsa_or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }",
     "double lsa_or_sigmoid(double x) { return 1.0 / (1.0 + exp(x)); }"),
    ("projection reads h reversed", "lsa_or_bf16_to_double(h[d]);\n    q[j]",
     "lsa_or_bf16_to_double(h[D - 1 - d]);\n    q[j]"),
    ("gate without softplus", "g[hh] = (float)lsa_or_softplus(a);", "g[hh] = (float)a;"),
    ("score drops the gate", "      z += (double)g[hh] * dot;\n    }\n    z_out[i]",
     "      z += dot;\n    }\n    z_out[i]"),
    ("score drops the key scale", "z_out[i] = z * sigma + bias;", "z_out[i] = z + bias;"),
    ("score bias sign", "z_out[i] = z * sigma + bias;", "z_out[i] = z * sigma - bias;"),
    ("score transposed key index", "*\n               key_value(key_dtype, keys, s * dI + d)",
     "*\n               key_value(key_dtype, keys, d * (int64_t)N + s)"),
    ("threshold exclusive", "sel[i] = (z[i] >= 0.0) ? 1 : 0;", "sel[i] = (z[i] > 0.0) ? 1 : 0;"),
    ("union reads only layer 0", "if (sel[(int64_t)l * N + s]) any = 1;",
     "if (sel[(int64_t)l * N + s] && l == 0) any = 1;"),
    ("merged logit is a min", "zmax = fmax(zmax, z[(int64_t)l * N + s]);",
     "zmax = fmin(zmax, z[(int64_t)l * N + s]);"),
    ("top-k ascending", "if (!an && a->z != b->z) return (a->z > b->z) ? -1 : 1;",
     "if (!an && a->z != b->z) return (a->z > b->z) ? 1 : -1;"),
    ("top-k ties to the higher index", "  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);\n}\n\nstatic int cmp_int_asc",
     "  return (a->idx > b->idx) ? -1 : (a->idx < b->idx);\n}\n\nstatic int cmp_int_asc"),
    ("fetch skips eviction", "if (e >= 0 && !is_surv[e]) {", "if (e >= 0 && !is_surv[e] && 0) {"),
    ("fetch copies the slot's cold row", "cold + (int64_t)s * row_bytes", "cold + (int64_t)j * row_bytes"),
    ("fetch takes the highest free slot", "int64_t j = 0;\n  for (int64_t i = 0; i < n; ++i) {\n    int32_t s = surv[i];\n    if (slot_of[s] >= 0) continue;\n    while (j < S && entry_of[j] >= 0) ++j;\n    if (j >= S) break;",
     "int64_t j = S - 1;\n  for (int64_t i = 0; i < n; ++i) {\n    int32_t s = surv[i];\n    if (slot_of[s] >= 0) continue;\n    while (j >= 0 && entry_of[j] >= 0) --j;\n    if (j < 0) break;"),
    ("fetch re-copies resident rows", "    if (slot_of[s] >= 0) continue;\n    while",
     "    if (slot_of[s] >= 0) {\n      memcpy(rows + (int64_t)slot_of[s] * row_bytes, cold + (int64_t)s * row_bytes, (size_t)row_bytes);\n      continue;\n    }\n    while"),
    ("gather pads with ones", "memset(hot + j * row_bytes, 0, (size_t)row_bytes);",
     "memset(hot + j * row_bytes, 1, (size_t)row_bytes);"),
    ("nucleus keeps at mass == p", "    if (A < top_p) {", "    if (A <= top_p) {"),
    ("nucleus drops the crossing entry", "    if (mass_ahead) mass_ahead[s] = A;\n    if (A < top_p) {",
     "    if (mass_ahead) mass_ahead[s] = A;\n    A += e[s] / S;\n    if (A < top_p) {"),
    ("nucleus ties to the higher index", "  if (a->x != b->x) return (a->x > b->x) ? -1 : 1;\n  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);",
     "  if (a->x != b->x) return (a->x > b->x) ? -1 : 1;\n  return (a->idx > b->idx) ? -1 : (a->idx < b->idx);"),
    ("vote exclusive", "label[s] = (c >= theta) ? 1 : 0;", "label[s] = (c > theta) ? 1 : 0;"),
    ("focal derivative sign", "*dz = dbce + sgn * dfl_du;", "*dz = dbce - sgn * dfl_du;"),
    ("focal term dropped from the loss", "loss_sum += bce + fl;", "loss_sum += bce;"),
    ("gradient drops the gate", "acc += g[t * H + hh] * G[t * dI + d] * h[(int64_t)t * D + c];",
     "acc += G[t * dI + d] * h[(int64_t)t * D + c];"),
    ("mean over N only", "const double inv = 1.0 / ((double)Q * (double)N);", "const double inv = 1.0 / (double)N;"),
    ("trigger phase", "return (t % tau) == 0;", "return (t % tau) == 1;"),
    ("attention without the max shift", "      s[j] = exp(s[j] - m);", "      s[j] = exp(s[j]);"),
    ("attention unnormalised", "    double p = s[j] / sum;", "    double p = s[j];"),
    ("attention scale applied twice", "      s[j] = scale * dot;", "      s[j] = scale * scale * dot;"),
    ("attention transposed row index", "               lsa_or_bf16_to_double(rows[j * D + d]);\n      s[j]",
     "               lsa_or_bf16_to_double(rows[(int64_t)d * n + j]);\n      s[j]"),
    ("attention value from the query", "        double v = lsa_or_bf16_to_double(rows[j * D + d]);",
     "        double v = lsa_or_bf16_to_double(q[(int64_t)hh * D + d]);"),
    ("lightning without the relu", "acc += (double)w[hh] * fmax(0.0, dot * sigma);",
     "acc += (double)w[hh] * (dot * sigma);"),
    ("lightning without the head weight", "acc += (double)w[hh] * fmax(0.0, dot * sigma);",
     "acc += fmax(0.0, dot * sigma);"),
    ("lightning scores the list position", "    const int64_t s = idx[i];\n    const double sigma = (key_dtype == 1 && scale)",
     "    const int64_t s = i;\n    const double sigma = (key_dtype == 1 && scale)"),
    ("attention drops the last row", "    for (int64_t j = 0; j < n; ++j) {\n      double p = s[j] / sum;",
     "    for (int64_t j = 0; j + 1 < n; ++j) {\n      double p = s[j] / sum;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"snippet for '{name}' must occur exactly once"
    d = tmp_path / name.replace(" ", "_")
    d.mkdir()
    c = d / "lsa_oracle.c"
    c.write_text(src.replace(old, new))
    so = d / "liblsa_oracle_mutant.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-I", os.path.join(ROOT, "oracle"), str(c), "-o",
                    str(so), "-lm"], check=True)
    return str(so)


def _run_pins(lib):
    env = dict(os.environ, LSA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-400:]


def test_pins_pass_on_the_real_oracle(tmp_path):
    lib = _build_mutant(tmp_path, "unchanged", "int lsa_or_num_threads(void) {",
                        "int lsa_or_num_threads(void) {")
    code, out = _run_pins(lib)
    assert code == 0, out


def test_every_planted_mistake_is_caught(tmp_path):
    libs = [(name, _build_mutant(tmp_path, name, old, new)) for name, old, new in MUTANTS]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda nl: (nl[0], *_run_pins(nl[1])), libs))
    missed = [(name, out) for name, code, out in results if code != 1]
    assert not missed, "pins did not catch: " + "; ".join(f"{n}: {o}" for n, o in missed)

"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a private copy of the oracle's C source (or,
marked "py", of its Python module)
(a dropped term, a wrong sign or index, a wrong rounding rule, a wrong bit order,
...), rebuilds that copy with gcc in a temporary directory and runs the pin suite
against it.  Every mutant must make at least one pin fail.  The real oracle is
never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "shrink exponent p instead of p-1": ("pow(ax, p - 1.0)", "pow(ax, p)"),
    "shrink without 1/beta": ("pow(ax, p - 1.0) / beta", "pow(ax, p - 1.0)"),
    "z update adds W_e": ("(w[k] - we[k]) * inv_s", "(w[k] + we[k]) * inv_s"),
    "z update drops W_e": ("(w[k] - we[k]) * inv_s", "(w[k]) * inv_s"),
    "z update divides by g-1": ("return acc / (double)g;", "return acc / (double)(g - 1);"),
    "residual sign of z": ("r[k] = w[k] - s * (q[k] - z)", "r[k] = w[k] - s * (q[k] + z)"),
    "init z sign": ("*z = -mn * (*inv_s);", "*z = mn * (*inv_s);"),
    "min-max skips last element": ("for (int k = 1; k < g; ++k) {\n    if (w[k] < mn)",
                                   "for (int k = 1; k < g - 1; ++k) {\n    if (w[k] < mn)"),
    "stop only on strict increase": ("int improves = e < best_e;", "int improves = e <= best_e;"),
    "return the rejected z": ("if (early_stop && !improves) break;",
                              "if (early_stop && !improves) { best_z = z; "
                              "for (int k = 0; k < g; ++k) best_q[k] = q[k]; break; }"),
    "stop step off by one": ("t_star = t;", "t_star = t > 0 ? t - 1 : 0;"),
    "beta never updated": ("beta = kappa * beta;", "beta = beta;"),
    "round half away from zero": ("double q = nearbyint(x);", "double q = round(x);"),
    "later decisions in binary32": ("  double x = w * inv_s + z;\n  double q = nearbyint(x);",
                                    "  double x = (double)(float)(w * inv_s + z);\n  double q = nearbyint(x);"),
    "init decision in binary32": ("double q = oracle_round_ratio((w - mn) * (double)qmax, mx - mn);",
                                  "double q = nearbyint((double)(float)(((w - mn) * (double)qmax) / (mx - mn)));"),
    "init decision through fp64 1/s": ("q[k] = t == 0 ? oracle_quantize_init_value(w[k], mn, mx, qmax)",
                                       "q[k] = t < 0 ? oracle_quantize_init_value(w[k], mn, mx, qmax)"),
    "ratio midpoint rounds up": ("return fmod(k, 2.0) == 0.0 ? k : k + 1.0;", "return k + 1.0;"),
    "ratio midpoint rounds down": ("if (rem2 < den) return k;", "if (rem2 <= den) return k;"),
    "no upper clamp": ("if (q > (double)qmax) q = (double)qmax;", ""),
    "error of squared residual": ("pow(fabs(r[k]), err_pow)", "pow(r[k] * r[k], err_pow)"),
    "pack MSB first": ("out[bit >> 3] |= (uint8_t)(1u << (bit & 7));",
                       "out[bit >> 3] |= (uint8_t)(0x80u >> (bit & 7));"),
    "binary16 truncates": ("double n = nearbyint(ldexp(a, 10 - e));",
                           "double n = floor(ldexp(a, 10 - e));"),
    "groups read column-major": ("const uint16_t* src = W_f16 + gi * group_size;",
                                 "const uint16_t* src = W_f16 + ((gi % rows) * cols + "
                                 "(gi / rows) * group_size);"),
    "dequant adds z": ("s * ((double)c - z)", "s * ((double)c + z)"),
    "tensor stop on non-increase": ("if (!(total[t] < best)) break;",
                                    "if (!(total[t] <= best)) break;"),
    "tensor stop keeps the global best": ("if (!(total[t] < best)) break;",
                                          "if (!(total[t] < best)) continue;"),
    "tensor stop one step late": ("    t_star = t;\n  }\n  if (E)", "    t_star = t + (t < iters);\n  }\n  if (E)"),
    "tensor total skips the last group": ("for (int t = 0; t <= iters; ++t) total[t] += trace[t];",
                                          "if (gi + 1 < ngroups) for (int t = 0; t <= iters; ++t) "
                                          "total[t] += trace[t];"),
    "meta 256 levels": ("(oracle_f16_to_f64(values[i]) - mn) * 255.0, d);",
                        "(oracle_f16_to_f64(values[i]) - mn) * 256.0, d);"),
    "meta decision in binary32": ("c = oracle_round_ratio((oracle_f16_to_f64(values[i]) - mn) * 255.0, d);",
                                  "c = nearbyint((double)(float)(((oracle_f16_to_f64(values[i]) - mn) * 255.0) / d));"),
    "meta round half away from zero": ("c = oracle_round_ratio((oracle_f16_to_f64(values[i]) - mn) * 255.0, d);",
                                       "c = round(((oracle_f16_to_f64(values[i]) - mn) * 255.0) / d);"),
    "meta offset is the max": ("offset16[ng] = oracle_f64_to_f16(mn);",
                               "offset16[ng] = oracle_f64_to_f16(mx);"),
    "meta scale over 256": ("d > 0.0 ? d / 255.0 : 1.0", "d > 0.0 ? d / 256.0 : 1.0"),
    "meta constant group scale 0": ("d > 0.0 ? d / 255.0 : 1.0", "d / 255.0"),
    "meta min-max skips last element": ("for (int64_t i = g0 + 1; i < g1; ++i) {",
                                        "for (int64_t i = g0 + 1; i < g1 - 1; ++i) {"),
    "meta dequant subtracts": ("oracle_f16_to_f64(offset16[gi]) +",
                               "oracle_f16_to_f64(offset16[gi]) -"),
    "meta dequant group off by one": ("const int64_t gi = i / gs;",
                                      "const int64_t gi = (i + 1) / gs;"),
    "matmul drops the zero-point": ("acc += (x * s) * ((double)c - z);",
                                    "acc += (x * s) * ((double)c);"),
    "matmul adds the zero-point": ("acc += (x * s) * ((double)c - z);",
                                   "acc += (x * s) * ((double)c + z);"),
    "matmul reads the weight transposed": ("const int64_t elem = n * K + k;",
                                           "const int64_t elem = k * N + n;"),
    "matmul group along the wrong axis": ("const int64_t gi = n * gpr + k / group_size;",
                                          "const int64_t gi = (k / group_size) * N + n % gpr;"),
    "matmul code bits reversed": ("const int64_t bit = elem * nbits + b;",
                                  "const int64_t bit = elem * nbits + (nbits - 1 - b);"),
    "residual adds the zero-point": ("dW[i] = oracle_f16_to_f64(W_f16[i]) - s * ((double)c - z);",
                                     "dW[i] = oracle_f16_to_f64(W_f16[i]) - s * ((double)c + z);"),
    "residual group off by one": ("    const int64_t gi = i / group_size;\n    const double s = oracle_f16_to_f64(scale_f16[gi]);\n    const double z = oracle_f16_to_f64(zero_f16[gi]);\n    dW[i]",
                                  "    const int64_t gi = (i + 1) / group_size % (n / group_size);\n    const double s = oracle_f16_to_f64(scale_f16[gi]);\n    const double z = oracle_f16_to_f64(zero_f16[gi]);\n    dW[i]"),
    "py: lowrank B without Sigma": ("B = U * (S * flip)", "B = U * flip", "py"),
    "py: lowrank keeps the smallest": ("U, S, Vt = U[:, :r], sig[:r], Vt[:r]",
                                       "U, S, Vt = U[:, -r:], sig[-r:], Vt[-r:]", "py"),
    "py: lowrank A is V": ("A = Vt * flip[:, None]", "A = (Vt.T * flip).T[::-1]", "py"),
    "matmul skips the last k": ("for (int64_t k = 0; k < K; ++k) {\n        const int64_t elem",
                                "for (int64_t k = 0; k < K - 1; ++k) {\n        const int64_t elem"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    before, after = MUTANTS[name][:2]
    target = "__init__.py" if MUTANTS[name][2:] == ("py",) else "hqq_oracle.c"
    for sub in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src_path = tmp_path / "oracle" / target
    src = src_path.read_text()
    assert src.count(before) >= 1, f"mutation site for {name!r} not found"
    src_path.write_text(src.replace(before, after, 1))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_meta_pins.py",
                        "tests/test_oracle_matmul_pins.py", "tests/test_oracle_lowrank_pins.py"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode != 0, f"mutant {name!r} survived the pins:\n{r.stdout[-2000:]}"

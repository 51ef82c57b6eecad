"""The pins catch planted mistakes.

Each case plants one plausible slip into a copy of the oracle's C source
(on the CPU, in a temporary directory), builds it, and runs the pin tests
against that build in a subprocess.  At least one pin must fail for every
slip.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = {
    "silu_on_up": ("h[r] = silu(a) * b;", "h[r] = a * silu(b);"),
    "down_transposed": ("acc += widen(wd, dtype, woff_dn + (int64_t)c * f + r) * h[r];",
                        "acc += widen(wd, dtype, woff_dn + (int64_t)r * d + c) * h[r];"),
    "drop_shared": ("for (int c = 0; c < d; ++c) yt[c] += o[c];", ";"),
    "tie_to_higher_index": ("return a < b;", "return a > b;"),
    "no_renorm": ("gates[j] = renorm ? s[id[j]] / denom : s[id[j]];", "gates[j] = s[id[j]];"),
    "sigmoid_sign": ("s[e] = 1.0 / (1.0 + exp(-l[e]));", "s[e] = 1.0 / (1.0 + exp(l[e]));"),
    "dispatch_unstable": ("for (int64_t p = 0; p < P; ++p) {", "for (int64_t p = P - 1; p >= 0; --p) {"),
    "softmax_denominator": ("s[e] = exp(l[e] - m); z += s[e];", "s[e] = exp(l[e] - m); z += s[e] * 1.0000001;"),
    "logit_index": ("widen(w_r, dtype, (int64_t)e * d + c)", "widen(w_r, dtype, (int64_t)c * E + e)"),
    "bias_space_ignored": ("key[e] = bias ? (bias_on_scores ? s[e] : l[e]) + bias[e] : l[e];",
                           "key[e] = bias ? l[e] + bias[e] : l[e];"),
    "capacity_off_by_one": ("(cap < 0 || c < cap)", "(cap < 0 || c <= cap)"),
    "dropped_pair_counted": ("if (keep && !keep[i * k + j]) continue;", ";"),
    "gate_from_key": ("denom += s[id[j]];", "denom += key[id[j]];"),
    "dsilu_dropped_term": ("double dsilu = sig * (1.0 + a[r] * (1.0 - sig));        /* d/da of a * sigmoid(a) */",
                           "double dsilu = sig;"),
    "renorm_jacobian_sign": ("dgj_dlm = dse_dlm / S - s[e] * dS_dlm / (S * S);",
                             "dgj_dlm = dse_dlm / S + s[e] * dS_dlm / (S * S);"),
    "router_grad_transposed": ("dxt[c] += widen(w_r, dtype, (int64_t)m * d + c) * dl[m];",
                               "dxt[c] += widen(w_r, dtype, (int64_t)c * E + m) * dl[m];"),
    "backward_ignores_drops": ("            if (keep && !keep[t * k + j]) {", "            if (0) {"),
    "shared_grad_ungated_missing": ("for (int r = 0; r < f_s; ++r) dsd[(int64_t)c * f_s + r] += dyt[c] * h[r];",
                                    "for (int r = 0; r < f_s; ++r) dsd[(int64_t)c * f_s + r] += 0.5 * dyt[c] * h[r];"),
    "expert_rows_row_index": ("swiglu_one(d, f, x, (int64_t)rows[i] * d,", "swiglu_one(d, f, x, (int64_t)i * d,"),
    "expert_rows_h_shifted": ("if (h_out) memcpy(h_out + i * f, h, sizeof(double) * f);",
                              "if (h_out) memcpy(h_out + i * f, h + 1, sizeof(double) * (f - 1));"),
    "logits_row_offset": ("int64_t t = t0 + tt;", "int64_t t = tt;"),
}
PIN_FILES = ["test_oracle_pins.py", "test_oracle_next.py", "test_oracle_backward.py"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    a, b = MUTATIONS[name]
    src = open(SRC).read()
    assert a in src, f"mutation site for {name} not found"
    (tmp_path / "moe_oracle.c").write_text(src.replace(a, b))
    lib = tmp_path / "liboracle.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(tmp_path / "moe_oracle.c"),
                           "-o", str(lib), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *(os.path.join(ROOT, "tests", f) for f in PIN_FILES)],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0, f"no pin failed for planted mistake {name}:\n{r.stdout[-2000:]}"

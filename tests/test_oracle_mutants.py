"""The pins must catch plausible slips in the oracle.

Each case plants one mistake in a copy of the oracle's C source (here, on the
CPU), builds it, and runs the pin suite against it in a subprocess: at least
one pin must fail.  The unmodified source must pass the same run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linattn_oracle.c")

MUTANTS = {
    "phi_drops_plus_one": ("x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x : exp(x)"),
    "phi_branch_flipped": ("x > 0.0 ? x + 1.0 : exp(x)", "x < 0.0 ? x + 1.0 : exp(x)"),
    "state_update_transposed": ("for (c = 0; c < d; ++c) Z[j * d + c] += f[j] * (double)vt[c];\n"
                                "                S[j] += f[j];\n            }\n            if (!out)",
                                "for (c = 0; c < d; ++c) Z[c * d + j] += f[j] * (double)vt[c];\n"
                                "                S[j] += f[j];\n            }\n            if (!out)"),
    "key_sum_without_phi": ("                S[j] += f[j];\n            }\n            if (!out)",
                            "                S[j] += (double)kt[j];\n            }\n            if (!out)"),
    "eps_dropped": ("                den += eps;\n                for (c = 0; c < d; ++c) {\n                    double num = 0.0;\n                    for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];\n                    ot[c]",
                    "                den += 0.0;\n                for (c = 0; c < d; ++c) {\n                    double num = 0.0;\n                    for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];\n                    ot[c]"),
    "readout_transposed": ("for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];\n                    ot[c] = num / den;\n                }\n            }\n        }",
                           "for (j = 0; j < d; ++j) num += g[j] * Z[c * d + j];\n                    ot[c] = num / den;\n                }\n            }\n        }"),
    "query_uses_key": ("for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);\n            {",
                       "for (j = 0; j < d; ++j) g[j] = phi((double)kt[j]);\n            {"),
    "state_in_ignored": ("if (z_in) memcpy(Z, z_in + h * d * d, (size_t)(d * d) * sizeof(double));\n"
                         "        if (s_in) memcpy(S, s_in + h * d, (size_t)d * sizeof(double));\n"
                         "        for (t = 0; t < N; ++t) {\n            const float *kt = k + (h * N + t) * d;\n"
                         "            const float *vt = v + (h * N + t) * d;\n            const float *qt",
                         "if (0) memcpy(Z, z_in + h * d * d, (size_t)(d * d) * sizeof(double));\n"
                         "        if (s_in) memcpy(S, s_in + h * d, (size_t)d * sizeof(double));\n"
                         "        for (t = 0; t < N; ++t) {\n            const float *kt = k + (h * N + t) * d;\n"
                         "            const float *vt = v + (h * N + t) * d;\n            const float *qt"),
    "exclusive_causality": ("            const float *kt = k + (h * N + t) * d;\n            const float *vt = v + (h * N + t) * d;\n            const float *qt = q + (h * N + t) * d;",
                            "            const float *kt = k + (h * N + t) * d;\n            const float *vt = v + (h * N + t) * d;\n            const float *qt = q + (h * N + (t + 1 < N ? t + 1 : t)) * d;"),
    "decode_skips_key_sum": ("            Sh[j] += fj;", "            Sh[j] += 0.0 * fj;"),
    "noncausal_sum_stops_early": ("        for (t = 0; t < N; ++t) {\n            const float *kt = k + (h * N + t) * d;\n            const float *vt = v + (h * N + t) * d;\n            for (j = 0; j < d; ++j) {\n                double fj",
                                  "        for (t = 0; t + 1 < N; ++t) {\n            const float *kt = k + (h * N + t) * d;\n            const float *vt = v + (h * N + t) * d;\n            for (j = 0; j < d; ++j) {\n                double fj"),
    "memory_read_without_norm_term": ("for (i = 0; i < d; ++i) retrieved_norm += fq[i] * norm[i];",
                                      "for (i = 0; i < d; ++i) retrieved_norm += fq[i];"),
    "memory_update_without_phi": ("const double fk = phi((double)krow[i]);", "const double fk = (double)krow[i];"),
    "memory_read_map_is_x_plus_one": ("for (i = 0; i < d; ++i) fq[i] = phi((double)qrow[i]);",
                                      "for (i = 0; i < d; ++i) fq[i] = (double)qrow[i] + 1.0;"),
    "memory_in_ignored": ("if (z_in) memcpy(mem,", "if (0) memcpy(mem,"),
    "memory_read_transposed": ("retrieved += fq[i] * mem[i * d + c];", "retrieved += fq[i] * mem[c * d + i];"),
    "unnormalized_update_without_phi": ("for (a = 0; a < d; ++a) phik[a] = phi((double)krow[a]);",
                                        "for (a = 0; a < d; ++a) phik[a] = (double)krow[a];"),
    "unnormalized_context_in_ignored": ("if (w_in) memcpy(W,", "if (0) memcpy(W,"),
    "unnormalized_read_transposed": ("acc += phiq[a] * W[a * d + b];", "acc += phiq[a] * W[b * d + a];"),
}

# planted in the backward pass (oracle_causal_bwd); checked by its own pins
BACKWARD_MUTANTS = {
    "bwd_phi_derivative_is_one": ("static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }",
                                  "static double dphi(double x) { return x > 0.0 ? 1.0 : 1.0; }"),
    "bwd_phi_derivative_is_exp": ("static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }",
                                  "static double dphi(double x) { return exp(x); }"),
    "bwd_normaliser_term_dropped": ("dD[t] = -dodo / den;", "dD[t] = 0.0 * dodo;"),
    "bwd_normaliser_sign_flipped": ("dD[t] = -dodo / den;", "dD[t] = dodo / den;"),
    "bwd_dq_misses_key_sum": ("double acc = S[j] * dD[t];", "double acc = 0.0 * S[j] * dD[t];"),
    "bwd_dq_uses_key_derivative": ("dq[(h * N + t) * d + j] = acc * dphi((double)qt[j]);",
                                   "dq[(h * N + t) * d + j] = acc * dphi((double)kt[j]);"),
    "bwd_dk_adjoint_transposed": ("for (c = 0; c < d; ++c) acc += R[j * d + c] * (double)vt[c];",
                                  "for (c = 0; c < d; ++c) acc += R[c * d + j] * (double)vt[c];"),
    "bwd_dv_adjoint_transposed": ("for (j = 0; j < d; ++j) acc += R[j * d + c] * f[j];",
                                  "for (j = 0; j < d; ++j) acc += R[c * d + j] * f[j];"),
    "bwd_dk_misses_key_sum_adjoint": ("                double acc = r[j];", "                double acc = 0.0 * r[j];"),
    "bwd_adjoint_excludes_own_token": (
        "            for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);\n            for (j = 0; j < d; ++j) {\n"
        "                for (c = 0; c < d; ++c) R[j * d + c] += g[j] * dn[t * d + c];",
        "            for (j = 0; j < d; ++j) g[j] = t + 1 < N ? phi((double)qt[j + d]) : 0.0;\n"
        "            for (j = 0; j < d; ++j) {\n"
        "                for (c = 0; c < d; ++c) R[j * d + c] += g[j] * (t + 1 < N ? dn[(t + 1) * d + c] : 0.0);"),
    "bwd_final_state_gradient_ignored": ("if (dz_out) memcpy(R,", "if (0) memcpy(R,"),
}


def _build(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(so), str(c), "-lm"],
                   check=True)
    return str(so)


def _run_pins(lib, pins="test_oracle_pins.py"):
    env = dict(os.environ, LINATTN_ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_oracle_passes_pins(tmp_path):
    lib = _build(tmp_path, "clean", open(SRC).read())
    for pins in ("test_oracle_pins.py", "test_oracle_backward_pins.py"):
        rc, out = _run_pins(lib, pins)
        assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    lib = _build(tmp_path, name, src.replace(old, new))
    rc, out = _run_pins(lib)
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = BACKWARD_MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    lib = _build(tmp_path, name, src.replace(old, new))
    rc, out = _run_pins(lib, "test_oracle_backward_pins.py")
    assert rc != 0, f"mutant {name} passed every backward pin:\n{out}"

"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant is a copy of oracle/vq_oracle.c with one plausible mistake (a
dropped term, a wrong sign or index, a reversed tie rule, a skipped step),
built into a temporary library and run against every pin in a child process.
A mutant that passes every pin would mean the pins do not constrain that part
of the oracle.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vq_oracle.c")

MUTANTS = {
    "distance_drops_weight": [("acc += om[t] * sq;", "acc += sq;")],
    "distance_not_squared": [("double sq = diff * diff;", "double sq = diff;")],
    "score_not_squared": [("float s = h[j] * sq;", "float s = h[j] * w;")],
    "score_ignores_h": [("float s = h[j] * sq;", "float s = sq;")],
    "select_ties_to_larger_index": [
        ("if (x->lin < y->lin) return -1;\n    if (x->lin > y->lin) return 1;",
         "if (x->lin < y->lin) return 1;\n    if (x->lin > y->lin) return -1;")],
    "select_off_by_one": [("for (long long e = 0; e < nnz; ++e) keep[all[e].lin] = 0;",
                           "for (long long e = 1; e < nnz; ++e) keep[all[e].lin] = 0;")],
    "nnz_rounds_up": [("(long long)floor(p * (double)(M * N))", "(long long)ceil(p * (double)(M * N))")],
    "assign_ties_to_highest": [("if (v < best) { best = v; arg = k; }", "if (v <= best) { best = v; arg = k; }")],
    "weight_wrong_column": [("long long j = (s % nb) * d + t;", "long long j = t;")],
    "weight_ignores_row": [("if (rho) w = w * (double)rho[i];", "(void)rho;")],
    "weight_ignores_mask": [("if (keep && keep[i * N + j] == 0) return 0.0;", "(void)keep;")],
    "update_unweighted_mean": [
        ("num += w * (double)X[(size_t)s * (size_t)d + (size_t)t];",
         "num += (double)X[(size_t)s * (size_t)d + (size_t)t];"),
        ("den += w;", "den += 1.0;")],
    "update_empty_to_zero": [
        ("if (den > 0.0) C[(size_t)k * (size_t)d + (size_t)t] = (float)(num / den);",
         "C[(size_t)k * (size_t)d + (size_t)t] = (float)(den > 0.0 ? num / den : 0.0);")],
    "update_J_after_update": [
        ("    double J = orc_objective(X, hcol, rho, keep, M, N, d, C, idx);\n", ""),
        ("    free(start);\n    free(order);\n    free(fill);\n    return J;",
         "    free(start);\n    free(order);\n    free(fill);\n"
         "    return orc_objective(X, hcol, rho, keep, M, N, d, C, idx);")],
    "init_no_dedupe": [("if (dup) continue;", "(void)dup;")],
    "binorm_rho_not_squared": [("rho[i] = (float)(ri * ri);", "rho[i] = (float)(ri);")],
    "binorm_hcol_one_factor": [("hcol[j] = (float)((double)h[j] * cj * cj);", "hcol[j] = (float)((double)h[j] * cj);")],
    "binorm_multiplies": [("Wp[i * N + j] = W[i * N + j] / ri;", "Wp[i * N + j] = W[i * N + j] * ri;")],
    "binorm_mean_not_rms": [("            double w = (double)W[i * N + j];\n            acc += w * w;",
                             "            double w = (double)W[i * N + j];\n            acc += w * w * w * w;")],
    "residual_sign": [("R[s * d + t] = X[s * d + t] - C", "R[s * d + t] = X[s * d + t] + C")],
    "reconstruct_drops_stage2": [("if (C2) v = v + C2", "if (0) v = v + C2")],
    "reconstruct_wrong_col_scale": [("if (c) v = v * c[j];", "if (c) v = v * c[(j + 1) % N];")],
    "reconstruct_drops_row_scale": [("if (r) v = v * r[i];", "if (0) v = v * r[i];")],
    "reconstruct_no_overwrite": [("if (row_ptr)\n            for", "if (0)\n            for")],
    "subvec_score_ignores_h": [("float term = h[j] * sq;", "float term = sq;")],
    "subvec_wrong_block": [("long long j = b * d + t;\n            float w = W[i * N + j];",
                            "long long j = t;\n            float w = W[i * N + j];")],
    "residual_ignores_keep": [("        if (keep[e] == 0) continue;\n        float r", "        float r")],
    "residual_not_squared": [("float sq = r * r;", "float sq = r;")],
    "residual_takes_one_more": [("for (long long e = 0; e < n_sel && e < n; ++e)",
                                 "for (long long e = 0; e <= n_sel && e < n; ++e)")],
    "keep_to_csr_skips_row0": [("int* row_ptr, int* col, float* val)\n{\n    long long pos = 0;\n    row_ptr[0] = 0;\n"
                                "    for (long long i = 0;",
                                "int* row_ptr, int* col, float* val)\n{\n    long long pos = 0;\n    row_ptr[0] = 0;\n"
                                "    for (long long i = 1;")],
    "vptq_error_not_scaled": [("E[m * N + n] = (Wk[m * N + n] - (double)What[m * N + n]) / unn;",
                               "E[m * N + n] = (Wk[m * N + n] - (double)What[m * N + n]);")],
    "vptq_boundary_skips_column": [("for (long long j = s_end; j < N; ++j) {\n                double acc",
                                    "for (long long j = s_end + 1; j < N; ++j) {\n                double acc")],
    "vptq_inblock_sign": [("Wk[m * N + j] -= E[m * N + n] * unj;", "Wk[m * N + j] += E[m * N + n] * unj;")],
    "vptq_quantizes_original": [("double diff = Wk[(v * V + t) * N + n] -", "double diff = (double)W[(v * V + t) * N + n] -")],
    "vptq_inblock_reaches_past_block": [("for (long long j = n + 1; j < s_end; ++j) {\n                double unj",
                                         "for (long long j = n + 1; j < N; ++j) {\n                double unj")],
    "grouped_outliers_smallest_h": [("if (x->score > y->score) return -1;\n    if (x->score < y->score) return 1;\n    return (x->lin > y->lin)",
                                     "if (x->score > y->score) return 1;\n    if (x->score < y->score) return -1;\n    return (x->lin > y->lin)")],
    "grouped_scatter_shifted": [("What[i * N + cols[c0 + q]] = Wg[i * Ng + q];",
                                 "What[i * N + cols[(c0 + q + 1) % N]] = Wg[i * Ng + q];")],
    "grouped_h_not_gathered": [("hg[q] = hc[j];", "hg[q] = hc[q];")],
    "grouped_outlier_group_uses_main_d": [("int dg = outlier ? d0 : d,", "int dg = outlier ? d : d,")],
    "qgemv_wrong_row": [("acc += (double)What[i * N + j] * (double)x[j];",
                         "acc += (double)What[((i + 1) % M) * N + j] * (double)x[j];")],
    "qgemv_float_accumulation": [("            double acc = 0.0;\n            for (long long j = 0; j < N; ++j) acc +=",
                                  "            float acc = 0.0f;\n            for (long long j = 0; j < N; ++j) acc +=")],
    "qgemv_token_stride": [("const float* x = X + b * N;", "const float* x = X;")],
    "lloyd_no_final_assign": [
        ("    orc_assign(X, hcol, rho, keep, M, N, d, C, K, NULL, 0, idx, NULL, nthreads);\n    J[T] =",
         "    J[T] =")],
    "fit_residual_uses_W": [("orc_init(R, n_sub, d, perm2, K2, C2)", "orc_init(Wp, n_sub, d, perm2, K2, C2)")],
}

RUNNER = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load({lib!r})
res = {{}}
for pin in ALL_PINS:
    try:
        pin(lib); res[pin.__name__] = "pass"
    except AssertionError:
        res[pin.__name__] = "FAIL"
    except Exception as e:
        res[pin.__name__] = "ERROR " + type(e).__name__
print(json.dumps(res))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    import oracle
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, "mutation anchor not unique/absent: %r" % old
        src = src.replace(old, new)
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src)
    lib = oracle.build(out_path=str(tmp_path / "libmutant.so"), src=str(msrc))
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if p.returncode != 0:
        # a crash of the broken copy also counts as caught
        return
    res = json.loads(p.stdout.strip().splitlines()[-1])
    caught = [k for k, v in res.items() if v != "pass"]
    assert caught, "mutant %s passed every pin" % name

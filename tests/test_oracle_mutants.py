"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is the oracle source with one plausible error substituted (a
dropped term, a wrong sign, a wrong index, a transposed operand, ...), built
with gcc into a temporary directory.  This shows that the pins constrain
every part of the oracle.  CPU only; the real oracle is not modified.
"""
import os

import pytest

import oracle
from pins import PINS
from pins_backward import BACKWARD_PINS
from pins_ex import EX_PINS
from pins_rowsparse import ROWSPARSE_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "sse_oracle.c")

MUTANTS = {
    "no_shared_partition": ("for (int r = 0; r <= k; r++) {", "for (int r = 0; r < k; r++) {"),
    "decay_sign": ("alpha[j] = exp(la[j]);", "alpha[j] = exp(-la[j]);"),
    "decay_on_columns": ("Sp[(int64_t)j * d + m] = alpha[j] * Sp",
                         "Sp[(int64_t)j * d + m] = alpha[m % c] * Sp"),
    "no_write_gate": ("+ w * kappa[j] * v[m];", "+ kappa[j] * v[m];"),
    "no_read_gate": ("o[m] += w * acc;", "o[m] += acc;"),
    "renormalised_gate": ("double w = (r < k) ? e[part] : 1.0;",
                          "double w = (r < k) ? e[part] / e[sel[0]] : 1.0;"),
    "raw_key_logits": ("softmax(kl, c, kappa);",
                       "for (int j = 0; j < c; j++) kappa[j] = kl[j];"),
    "ties_to_higher_index": ("z[i] > z[best]", "z[i] >= z[best]"),
    "read_before_write": ("acc += q[j] * Sp[(int64_t)j * d + m];",
                          "acc += q[j] * (Sp[(int64_t)j * d + m] - w * kappa[j] * v[m]) / alpha[j];"),
    "unselected_decay": ("    for (int r = 0; r <= k; r++) {",
                         "    for (int p = 0; p < N; p++) for (int64_t x = 0; x < cd; x++) "
                         "S[p * cd + x] *= alpha[x / d];\n    for (int r = 0; r <= k; r++) {"),
    "shared_gets_router_weight": ("double w = (r < k) ? e[part] : 1.0;",
                                  "double w = (r < k) ? e[part] : e[sel[0]];"),
    "key_transposed": ("+ w * kappa[j] * v[m];", "+ w * kappa[m % c] * v[j % d];"),
    "query_dropped_row": ("for (int j = 0; j < c; j++)\n                acc += q[j]",
                          "for (int j = 1; j < c; j++)\n                acc += q[j]"),
    "output_row_shift": ("S, o + lt * d, selr", "S, o + (lt > 0 ? lt - 1 : 0) * d, selr"),
    "grouping_reversed_time": ("for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; t++)",
                               "for (int64_t t = cu_seqlens[s + 1] - 1; t >= cu_seqlens[s]; t--)"),
    "state_reset_missing": ("memset(S, 0, sizeof(double) * (size_t)st);", "(void)0;"),
    "init_ignored": ("memcpy(S, J->init + (int64_t)u * st, sizeof(double) * (size_t)st);",
                     "memset(S, 0, sizeof(double) * (size_t)st);"),
    # row-sparse key variant
    "rowsparse_unselected_decay": ("double a = (sel[j] || !identity_unselected) ? exp(ll[j]) : 1.0;",
                                   "double a = exp(ll[j]);"),
    "rowsparse_softmax_over_all_rows": ("kappa[j] = sel[j] ? exp(kk[j] - mx) / z : 0.0;",
                                        "kappa[j] = sel[j] ? exp(kk[j] - mx) / (z + 1.0) : 0.0;"),
    "rowsparse_dense_key": ("kappa[j] = sel[j] ? exp(kk[j] - mx) / z : 0.0;",
                            "kappa[j] = exp(kk[j] - mx) / z;"),
    "rowsparse_selected_rows_no_decay": ("double a = (sel[j] || !identity_unselected) ? exp(ll[j]) : 1.0;",
                                         "double a = (!sel[j] && !identity_unselected) ? exp(ll[j]) : 1.0;"),
    # general form (own shared q/k, read sets)
    "ex_shared_uses_routed_key": ("const double *key = (r < k) ? kap : kaps;",
                                  "const double *key = kap;"),
    "ex_shared_uses_routed_query": ("const double *qv = (r < krr) ? qq : qs;",
                                    "const double *qv = qq;"),
    "ex_read_with_write_weight": ("double w = (r < krr) ? er[part] : 1.0;",
                                  "double w = (r < krr) ? e[part] : 1.0;"),
    "ex_read_set_is_write_set": ("top_k(zr, N, krr, R);             /* read set */",
                                 "top_k(z, N, krr, R);"),
    "ex_no_shared_read": ("for (int r = 0; r <= krr; r++) {", "for (int r = 0; r < krr; r++) {"),
    # backward
    "bwd_adjoint_not_decayed": ("                    Ap[(int64_t)j * d + m] *= alpha[j];",
                                "                    (void)0;"),
    "bwd_no_read_gate_gradient": ("                dw += y[m] * dot[m];",
                                  "                dw += 0.0 * y[m] * dot[m];"),
    "bwd_key_softmax_jacobian_sign": ("gk[j] = kap[j] * (dkap[j] - kd);",
                                      "gk[j] = kap[j] * (dkap[j] + kd);"),
    "bwd_decay_gradient_without_alpha": ("gl[j] += alpha[j] * as;", "gl[j] += as;"),
    "bwd_query_gradient_before_write": (
        "const double snew = alpha[j] * Sb[(int64_t)j * d + m] + w * kap[j] * vv[m];",
        "const double snew = Sb[(int64_t)j * d + m];"),
    "bwd_router_jacobian_no_mean": ("dz[lt * N + i] = e[i] * (de[i] - ed);",
                                    "dz[lt * N + i] = e[i] * de[i];"),
    "bwd_read_adjoint_missing_gate": ("Ap[(int64_t)j * d + m] += w * qq[j] * dot[m];",
                                      "Ap[(int64_t)j * d + m] += qq[j] * dot[m];"),
    "rowsparse_read_before_write": ("            o[(t - t0) * d + m] = acc;",
                                    "            o[(t - t0) * d + m] = acc - qq[0] * kappa[0] * vv[m];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} must occur exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = oracle.build(str(mpath), str(tmp_path / "libmutant.so"),
                      extra_flags=("-Wno-error", "-w"))
    lib = oracle.load(so)
    failed = []
    for pin in PINS + ROWSPARSE_PINS + EX_PINS + BACKWARD_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"

"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Every case below edits one line of ``oracle/ssm_oracle.c`` in a temporary copy (a
dropped term, a wrong sign, a wrong index, a transposed operand, a wrong order),
compiles it with the oracle's own flags, swaps it in for the real library and runs
the pins. A mutant that passes every pin would mean the pins cannot tell that
mistake from the correct loop.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

MUTANTS = {
    "sign_of_input_term": ("h[n] = dA * h[n] + dB * xv;", "h[n] = dA * h[n] - dB * xv;"),
    "sign_of_A": ("const double dA = exp(dv * A[d * N + n]);\n                    const double dB", "const double dA = exp(-dv * A[d * N + n]);\n                    const double dB"),
    "dropped_dt_in_B": ("A[d * N + n]);\n                    const double dB = dv * B[s + n];",
                        "A[d * N + n]);\n                    const double dB = B[s + n];"),
    "B_for_C": ("h[n] = dA * h[n] + dB * xv;\n                    acc = acc + C[s + n] * h[n];", "h[n] = dA * h[n] + dB * xv;\n                    acc = acc + B[s + n] * h[n];"),
    "dropped_skip": ("double yv = acc + Dv[d] * xv;\n                if (z) yv = yv * silu(z[i]);\n                y[i] = yv;\n            }\n            if (h_final)\n                for (int64_t n = 0; n < N; ++n) h_final",
                     "double yv = acc;\n                if (z) yv = yv * silu(z[i]);\n                y[i] = yv;\n            }\n            if (h_final)\n                for (int64_t n = 0; n < N; ++n) h_final"),
    "gate_without_sigmoid": ("static double silu(double z) { return z / (1.0 + exp(-z)); }",
                             "static double silu(double z) { return z; }"),
    "transposed_A_index": ("const double dA = exp(dv * A[d * N + n]);\n                    const double dB", "const double dA = exp(dv * A[n * Dn + d]);\n                    const double dB"),
    "output_from_old_state": ("h[n] = dA * h[n] + dB * xv;\n                    acc = acc + C[s + n] * h[n];",
                              "acc = acc + C[s + n] * h[n];\n                    h[n] = dA * h[n] + dB * xv;"),
    "h0_ignored": ("h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;\n            for (int64_t t = 0; t < L; ++t) {\n                const int64_t i = (b * L + t) * Dn + d;   /* (b, t, d) */",
                   "h[n] = 0.0;\n            for (int64_t t = 0; t < L; ++t) {\n                const int64_t i = (b * L + t) * Dn + d;   /* (b, t, d) */"),
    "decode_sign": ("hs[n] = dA * hs[n] + dB * xv;", "hs[n] = dA * hs[n] - dB * xv;"),
    "complex_decode_A_layer_index": ("const double *Ad = A + (l * Dn + d) * N * 2;", "const double *Ad = A + d * N * 2;"),
    "decode_A_layer_index": ("const double *Ad = A + (l * Dn + d) * N;\n                const double xv = x[i], dv = dt[i];\n                double acc", "const double *Ad = A + d * N;\n                const double xv = x[i], dv = dt[i];\n                double acc"),
    "complex_rotation_sense": ("const double ni = (dAr * hi[n] + dAi * hr[n]) + dBi * xv;",
                               "const double ni = (dAr * hi[n] - dAi * hr[n]) + dBi * xv;"),
    "complex_conjugated_C": ("acc = acc + (C[(s + n) * 2 + 0] * hr[n] - C[(s + n) * 2 + 1] * hi[n]);",
                             "acc = acc + (C[(s + n) * 2 + 0] * hr[n] + C[(s + n) * 2 + 1] * hi[n]);"),
    "complex_sin_cos_swapped": ("const double dAr = mag * cos(dv * aim);\n                    const double dAi = mag * sin(dv * aim);",
                                "const double dAr = mag * sin(dv * aim);\n                    const double dAi = mag * cos(dv * aim);"),
    "complex_decay_dropped": ("const double mag = exp(dv * are);", "const double mag = 1.0;"),
    "complex_decode_sign": ("const double nr = (dAr * hs[2 * n] - dAi * hs[2 * n + 1]) + dBr * xv;",
                            "const double nr = (dAr * hs[2 * n] + dAi * hs[2 * n + 1]) + dBr * xv;"),
    "state_bytes_factor": ("return n_layers * channels * d_state * bytes_per_value;",
                           "return n_layers * channels * d_state * 4;"),
    "conv_taps_flipped": ("acc = acc + w[d * K + k] * conv_input", "acc = acc + w[d * K + (K - 1 - k)] * conv_input"),
    "conv_off_by_one": ("conv_input(x, state0, b, t - (K - 1) + k, d, L, Dn, K)",
                        "conv_input(x, state0, b, t - K + k, d, L, Dn, K)"),
    "conv_bias_dropped": ("double acc = cb ? cb[d] : 0.0;", "double acc = 0.0;"),
    "conv_without_silu": ("u[(b * L + t) * Dn + d] = silu(acc);", "u[(b * L + t) * Dn + d] = acc;"),
    "conv_state_reversed": ("return state0[(b * (K - 1) + (K - 1 + s)) * Dn + d];",
                            "return state0[(b * (K - 1) + (-1 - s)) * Dn + d];"),
    "conv_state_out_shifted": ("conv_input(x, state0, b, L - (K - 1) + j, d, L, Dn, K);",
                               "conv_input(x, state0, b, L - K + j, d, L, Dn, K);"),
    "softplus_sign": ("return fmax(v, 0.0) + log1p(exp(-fabs(v)));", "return fmax(v, 0.0) + log1p(exp(fabs(v)));"),
    "softplus_no_max": ("return fmax(v, 0.0) + log1p(exp(-fabs(v)));", "return log1p(exp(-fabs(v)));"),
    "dt_bias_dropped": ("softplus(raw[i * Dn + d] + (bias ? bias[d] : 0.0));", "softplus(raw[i * Dn + d]);"),
    "dt_bias_row_index": ("softplus(raw[i * Dn + d] + (bias ? bias[d] : 0.0));",
                          "softplus(raw[i * Dn + d] + (bias ? bias[i % Dn] : 0.0));"),
    "bwd_ddt_without_decay_term": ("gdt += lt * (xv * B[s + n] + A[d * N + n] * a * hp);", "gdt += lt * (xv * B[s + n]);"),
    "bwd_dA_from_new_state": ("dA[d * N + n] += lt * dv * a * hp;", "dA[d * N + n] += lt * dv * a * hs[(t + 1) * N + n];"),
    "bwd_adjoint_not_decayed": ("lam[n] = a * lt;", "lam[n] = lt;"),
    "bwd_gate_derivative": ("(sg * (1.0 + z[i] * (1.0 - sg)))", "(sg)"),
    "bwd_dC_from_old_state": ("dC[s + n] += dout * hs[(t + 1) * N + n];", "dC[s + n] += dout * hs[t * N + n];"),
    "bwd_dx_skip_dropped": ("double gx = dout * Dv[d], gdt = 0.0;", "double gx = 0.0, gdt = 0.0;"),
    "bwd_dD_ungated": ("dD[d] += dout * xv;", "dD[d] += dy[i] * xv;"),
    "bwd_dh_final_ignored": ("lam[n] = dh_final ? dh_final[(b * Dn + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    "bwd_dB_without_dt": ("dB[s + n] += lt * dv * xv;", "dB[s + n] += lt * xv;"),
    "trap_prev_not_decayed": ("h[n] = dA * h[n] + (wp * (dA * prev) + wc * (B[s + n] * xv));",
        "h[n] = dA * h[n] + (wp * prev + wc * (B[s + n] * xv));"),
    "trap_default_weight_is_euler": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = lam ? lam[i] : 1.0;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_older_weight_full": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv;\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_older_weight_without_dt": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_weights_swapped": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * (1.0 - lv), wp = dv * lv;\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_lambda_ignored": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_lambda_of_next_step": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
        "const double lv = lam ? lam[(b * L + (t + 1) % L) * Dn + d] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "trap_decode_lambda_ignored": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * Ad[n]);",
        "const double lv = 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * Ad[n]);"),
    "trap_decode_weights_swapped": ("const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * lv, wp = dv * (1.0 - lv);\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * Ad[n]);",
        "const double lv = lam ? lam[i] : 0.5;\n                const double wc = dv * (1.0 - lv), wp = dv * lv;\n                double acc = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * Ad[n]);"),
    "trap_prev_input_not_advanced": ("                xp = xv;\n", ""),
    "trap_prev_B_row_ahead": ("                Bp = B + s;", "                Bp = B + s + N;"),
    "trap_first_prev_ignored": ("double xp = has_prev ? x_prev[b * Dn + d] : 0.0;", "double xp = 0.0;"),
    "trap_decode_prev_is_current_B": ("const double prev = has_prev ? B_prev[s + n] * x_prev[i] : 0.0;",
                                      "const double prev = has_prev ? B[s + n] * x_prev[i] : 0.0;"),
    "trap_decode_prev_not_decayed": ("hs[n] = dA * hs[n] + (wp * (dA * prev) + wc * (B[s + n] * xv));",
                                     "hs[n] = dA * hs[n] + (wp * prev + wc * (B[s + n] * xv));"),
    "mimo_B_transposed": ("const double dA = exp(dv * A[d * N + n]);\n                    double u = 0.0;\n                    for (int64_t r = 0; r < R; ++r) u = u + (dv * Bt[n * R + r]) * xv[r];",
                          "const double dA = exp(dv * A[d * N + n]);\n                    double u = 0.0;\n                    for (int64_t r = 0; r < R; ++r) u = u + (dv * Bt[r * N + n]) * xv[r];"),
    "mimo_dt_dropped_from_input": ("const double dA = exp(dv * A[d * N + n]);\n                    double u = 0.0;\n                    for (int64_t r = 0; r < R; ++r) u = u + (dv * Bt[n * R + r]) * xv[r];",
                                   "const double dA = exp(dv * A[d * N + n]);\n                    double u = 0.0;\n                    for (int64_t r = 0; r < R; ++r) u = u + Bt[n * R + r] * xv[r];"),
    "mimo_C_transposed": ("acc[r] = acc[r] + Ct[n * R + r] * h[n];", "acc[r] = acc[r] + Ct[r * N + n] * h[n];"),
    "mimo_skip_reads_first_input": ("double yv = acc[r] + Dv[d] * xv[r];", "double yv = acc[r] + Dv[d] * xv[0];"),
    "mimo_gate_reads_first_input": ("double yv = acc[r] + Dv[d] * xv[r];\n                    if (z) yv = yv * silu(z[i * R + r]);",
                                    "double yv = acc[r] + Dv[d] * xv[r];\n                    if (z) yv = yv * silu(z[i * R]);"),
    "mimo_x_row_stride": ("const double *xv = x + i * R;                 /* (b, t, d, 0) */",
                          "const double *xv = x + i;                 /* (b, t, d, 0) */"),
    "mimo_B_row_stride": ("const double *Bt = B + (b * L + t) * N * R;   /* (b, t, 0, 0) */",
                          "const double *Bt = B + (b * L + t) * N;   /* (b, t, 0, 0) */"),
    "mimo_h0_ignored": ("h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;\n            for (int64_t t = 0; t < L; ++t) {\n                const int64_t i = (b * L + t) * Dn + d;        /* (b, t, d) of dt */",
                        "h[n] = 0.0;\n            for (int64_t t = 0; t < L; ++t) {\n                const int64_t i = (b * L + t) * Dn + d;        /* (b, t, d) of dt */"),
    "mimo_outputs_accumulate_across_steps": ("for (int64_t r = 0; r < R; ++r) acc[r] = 0.0;\n                for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);",
                                             "for (int64_t n = 0; n < N; ++n) {\n                    const double dA = exp(dv * A[d * N + n]);"),
    "mimo_decode_B_layer_dropped": ("const double *Bt = B + (l * n_seq + q) * N * R;", "const double *Bt = B + q * N * R;"),
    "mimo_decode_output_from_old_state": ("hs[n] = dA * hs[n] + u;\n                    for (int64_t r = 0; r < R; ++r) acc[r] = acc[r] + Ct[n * R + r] * hs[n];",
                                          "for (int64_t r = 0; r < R; ++r) acc[r] = acc[r] + Ct[n * R + r] * hs[n];\n                    hs[n] = dA * hs[n] + u;"),
    "input_bwd_silu_derivative_truncated": ("const double da = du[e] * sg * (1.0 + pre * (1.0 - sg));",
                                            "const double da = du[e] * sg;"),
    "input_bwd_filter_flipped": ("if (s >= 0) dx[(b * L + s) * Dn + d] += w[d * K + k] * da;",
                                 "if (s >= 0) dx[(b * L + s) * Dn + d] += w[d * K + (K - 1 - k)] * da;"),
    "input_bwd_softplus_derivative_sign": ("dr[e] = ddt[e] / (1.0 + exp(-v));", "dr[e] = ddt[e] / (1.0 + exp(v));"),
    "input_bwd_state_positions_reversed": ("else if (dstate0) dstate0[(b * H + (H + s)) * Dn + d] += w[d * K + k] * da;",
                                           "else if (dstate0) dstate0[(b * H + (-1 - s)) * Dn + d] += w[d * K + k] * da;"),
    "input_bwd_bias_gradient_dropped": ("if (dcb) dcb[d] += da;", "if (dcb) dcb[d] += 0.0 * da;"),
}


def _run_all_pins():
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(oracle)
        except AssertionError as e:
            failures.append(str(e))
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", str(so), str(path), "-lm"], check=True)
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fname in ("oracle_scan_f64", "oracle_scan_c128", "oracle_step_f64", "oracle_step_c128",
                  "oracle_state_bytes", "oracle_conv_silu_f64", "oracle_softplus_f64",
                  "oracle_scan_bwd_f64", "oracle_scan_trap_f64", "oracle_step_trap_f64",
                  "oracle_scan_mimo_f64", "oracle_step_mimo_f64", "oracle_input_stage_bwd_f64"):
        f, g = getattr(lib, fname), getattr(real, fname)
        f.argtypes, f.restype = g.argtypes, g.restype
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = _run_all_pins()
    assert failures, f"mutant {name} passed every pin"

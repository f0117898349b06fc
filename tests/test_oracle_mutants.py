"""Planted mistakes in the oracle must be caught by its pins.

Each case below copies ttt_oracle.c, plants one plausible mistake in the copy
(a wrong sign, a transposed operand, a dropped factor, the readout taken
before the update, ...), compiles it with gcc into a temporary library and
runs the pin battery from test_oracle.py against it.  At least one pin must
fail for every mutant; the unmodified source must pass them all.  Everything
here runs on the CPU.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle as pins
import test_oracle_backward as bpins
import test_oracle_momentum as mpins
import test_oracle_prologue as ppins
import test_oracle_prologue_backward as pbpins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ttt_oracle.c")

MUTANTS = {
    "residual_sign": ("r[j] = acc - vt[j];\n            }\n            /* G += k^T r",
                      "r[j] = vt[j] - acc;\n            }\n            /* G += k^T r"),
    "gradient_transposed": ("G[i * d + j] += kt[i] * r[j];", "G[i * d + j] += kt[j] * r[i];"),
    "prediction_transposed": ("acc += kt[i] * Wc[i * d + j];\n                r[j] = acc - vt[j];\n            }\n            /* G += k^T r",
                              "acc += kt[i] * Wc[j * d + i];\n                r[j] = acc - vt[j];\n            }\n            /* G += k^T r"),
    "readout_before_update": ("readout after the update) */\n            for (long j = 0; j < d; ++j) {\n                double acc = 0.0;\n                for (long i = 0; i < d; ++i)\n                    acc += qt[i] * Wt[i * d + j];",
                              "readout after the update) */\n            for (long j = 0; j < d; ++j) {\n                double acc = 0.0;\n                for (long i = 0; i < d; ++i)\n                    acc += qt[i] * Wc[i * d + j];"),
    "missing_half": ("                Wt[x] = Wc[x] - eta * G[x];\n            /* y_t",
                     "                Wt[x] = Wc[x] - 2.0 * eta * G[x];\n            /* y_t"),
    "gradient_not_accumulated": ("G[i * d + j] += kt[i] * r[j];", "G[i * d + j] = kt[i] * r[j];"),
    "silu_grad_sign": ("return s * (1.0 + x * (1.0 - s));", "return s * (1.0 - x * (1.0 - s));"),
    "silu_is_sigmoid": ("static double silu(double x) { return x * sigmoid(x); }",
                        "static double silu(double x) { return sigmoid(x); }"),
    "mlp_w2_grad_uses_preactivation": ("w->G2[p * d + j] += w->a[p] * w->e[j];",
                                       "w->G2[p * d + j] += w->h[p] * w->e[j];"),
    "mlp_w1_grad_drops_activation_grad": ("w->dh[p] = acc * silu_grad(w->h[p]);",
                                          "w->dh[p] = acc;"),
    "mlp_readout_old_w2": ("acc += w->aq[p] * w->W2t[p * d + j];",
                           "acc += w->aq[p] * w->A2c[p * d + j];"),
    "decode_sign": ("Wu[i * d + j] -= eta[h] * g;", "Wu[i * d + j] += eta[h] * g;"),
    "decode_residual_uses_query": ("acc += kt[i] * Wu[i * d + j];", "acc += qt[i] * Wu[i * d + j];"),
    # backward of the linear scan
    "bwd_state_adjoint_sign": ("w->Gb[x] -= eta * w->Wtb[x];", "w->Gb[x] += eta * w->Wtb[x];"),
    "bwd_dv_sign": ("dv[t * d + j] = -w->rb[j];\n        }\n        /* the chunk-start weights",
                    "dv[t * d + j] = w->rb[j];\n        }\n        /* the chunk-start weights"),
    "bwd_drops_final_state_adjoint": ("dy[t * d + j]\n                                        + (t == e - 1 ? w->Wb[i * d + j] : 0.0);",
                                      "dy[t * d + j]\n                                        + 0.0;"),
    "bwd_dk_transposed": ("vb_t = -rb_t */\n            for (long i = 0; i < d; ++i) {\n                double acc = 0.0;\n                for (long j = 0; j < d; ++j)\n                    acc += w->rb[j] * Wc[i * d + j];",
                          "vb_t = -rb_t */\n            for (long i = 0; i < d; ++i) {\n                double acc = 0.0;\n                for (long j = 0; j < d; ++j)\n                    acc += w->rb[j] * Wc[j * d + i];"),
    "bwd_eta_sign": ("eb -= w->Wtb[x] * G[x];", "eb += w->Wtb[x] * G[x];"),
    "bwd_prefix_not_accumulated": ("(t > s ? G[i * d + j - dd] : 0.0) + k[t * d + i] * r[j];",
                                   "k[t * d + i] * r[j];"),
    "bwd_dq_uses_chunk_start": ("acc += dy[t * d + j] * w->Wt[i * d + j];",
                                "acc += dy[t * d + j] * Wc[i * d + j];"),
    # prologue: per-token step size and LayerNorm
    "tok_eta_dropped": ("G[i * d + j] += eta_t[t] * kt[i] * r[j];", "G[i * d + j] += kt[i] * r[j];"),
    "tok_eta_of_chunk_start": ("G[i * d + j] += eta_t[t] * kt[i] * r[j];",
                               "G[i * d + j] += eta_t[s] * kt[i] * r[j];"),
    "chunk_start_read_uses_updated": ("const double* Wr = read_start ? Wc : Wt;",
                                      "const double* Wr = read_start ? Wt : Wt;"),
    "ln_no_mean_in_variance": ("var += (x[j] - mean) * (x[j] - mean);\n        var /= (double)d;\n        const double inv = 1.0 / sqrt(var + eps);\n        for (long j = 0; j < d; ++j)\n            x[j] =",
                               "var += x[j] * x[j];\n        var /= (double)d;\n        const double inv = 1.0 / sqrt(var + eps);\n        for (long j = 0; j < d; ++j)\n            x[j] ="),
    "ln_gamma_beta_swapped": ("x[j] = (x[j] - mean) * inv * gamma[h * d + j] + beta[h * d + j];",
                              "x[j] = (x[j] - mean) * inv * beta[h * d + j] + gamma[h * d + j];"),
    "ln_eps_dropped": ("const double inv = 1.0 / sqrt(var + eps);\n        for (long j = 0; j < d; ++j)\n            x[j] =",
                       "const double inv = 1.0 / sqrt(var);\n        for (long j = 0; j < d; ++j)\n            x[j] ="),
    "bwd_state_adjoint_not_passed": ("previous chunk */\n        memcpy(w->Wb, w->Wcb, (size_t)dd * sizeof(double));",
                                     "previous chunk */\n        memcpy(w->Wb, w->Wtb, (size_t)dd * sizeof(double));"),
    # backward through the prologue
    "tokbwd_deta_drops_key": ("et_b += k[t * d + i] * acc;", "et_b += acc;"),
    "tokbwd_dk_missing_eta": ("dk[t * d + i] = eta_t[t] * acc;", "dk[t * d + i] = acc;"),
    "tokbwd_rb_missing_eta": ("w->rb[j] = eta_t[t] * acc;", "w->rb[j] = acc;"),
    "tokbwd_start_read_adjoint_dropped": ("w->Wcb[i * d + j] += qy;", "w->Wcb[i * d + j] += 0.0;"),
    "tokbwd_dq_reads_updated": ("const double* Wr = read_start ? Wc : w->Wt;",
                                "const double* Wr = w->Wt;"),
    "tokbwd_state_adjoint_not_passed": ("memcpy(w->Wb, w->Wcb, (size_t)dd * sizeof(double));\n    }\n    memcpy(dw0, w->Wb, (size_t)dd * sizeof(double));\n}\n\n/* dQ, dK, dV: [B][H][T][d]; dW0 per chain [B][H][d][d]; deta_tok",
                                        "memcpy(w->Wb, w->Wtb, (size_t)dd * sizeof(double));\n    }\n    memcpy(dw0, w->Wb, (size_t)dd * sizeof(double));\n}\n\n/* dQ, dK, dV: [B][H][T][d]; dW0 per chain [B][H][d][d]; deta_tok"),
    "lnbwd_drops_mean_term": ("g[j] = (dxh[j] - m1 - xh[j] * m2) * inv;", "g[j] = (dxh[j] - xh[j] * m2) * inv;"),
    "lnbwd_drops_projection": ("g[j] = (dxh[j] - m1 - xh[j] * m2) * inv;", "g[j] = (dxh[j] - m1) * inv;"),
    "lnbwd_dgamma_of_raw_rows": ("dgb[(2 * h) * d + j] += g[j] * xh[j];", "dgb[(2 * h) * d + j] += g[j] * x[j];"),
    "lnbwd_dbeta_scaled": ("dgb[(2 * h + 1) * d + j] += g[j];",
                           "dgb[(2 * h + 1) * d + j] += g[j] * gamma[h * d + j];"),
    # momentum GD (exact token steps and chunk-start gradients)
    "mom_beta_scales_gradient": ("M[i * d + j] = beta * M[i * d + j] + kt[i] * r[j];",
                                 "M[i * d + j] = beta * (M[i * d + j] + kt[i] * r[j]);"),
    "mom_step_uses_gradient": ("W[i * d + j] -= eta * M[i * d + j];",
                               "W[i * d + j] -= eta * kt[i] * r[j];"),
    "mom_gradient_point_swapped": ("const double* Wg = grad_mode ? Wc : W;",
                                   "const double* Wg = grad_mode ? W : Wc;"),
    "mom_initial_momentum_dropped": ("    if (m_init)\n        memcpy(M, m_init,",
                                     "    if (0)\n        memcpy(M, m_init,"),
    "mom_gradient_transposed": ("M[i * d + j] = beta * M[i * d + j] + kt[i] * r[j];",
                                "M[i * d + j] = beta * M[i * d + j] + kt[j] * r[i];"),
    "mom_chunk_start_off_by_one": ("if (t % b == 0)\n            memcpy(Wc, W,",
                                   "if (t % b == 1 || b == 1)\n            memcpy(Wc, W,"),
}


def _battery():
    """Run the pins; return the names of those that fail."""
    failed = []
    checks = [
        ("worked_examples", lambda: pins.test_worked_examples_exact(oracle)),
        ("eta_zero_linear", lambda: pins.test_eta_zero_linear(oracle)),
        ("autograd_linear_b1", lambda: pins.test_autograd_minibatch_linear(oracle, 1)),
        ("autograd_linear_b4", lambda: pins.test_autograd_minibatch_linear(oracle, 4)),
        ("linear_attention", lambda: pins.test_zero_init_is_causal_linear_attention(oracle, 16, 16)),
        ("eta_zero_mlp", lambda: pins.test_eta_zero_mlp(oracle)),
        ("mlp_kernel_attention", lambda: pins.test_mlp_zero_second_layer_is_kernel_linear_attention(oracle)),
        ("autograd_mlp_b4", lambda: pins.test_autograd_minibatch_mlp(oracle, 4)),
        ("mlp_fd", lambda: pins.test_mlp_gradient_matches_finite_differences(oracle)),
        ("decode_vs_scan", lambda: pins.test_decode_steps_equal_b1_scan(oracle)),
        ("decode_example", lambda: pins.test_decode_worked_example(oracle)),
        ("bwd_fd", lambda: bpins.test_backward_matches_finite_differences(oracle, 2, 2, 7, 3, 3, False)),
        ("bwd_autograd_b4", lambda: bpins.test_backward_matches_double_autograd(oracle, 4)),
        ("bwd_eta_zero", lambda: bpins.test_backward_eta_zero_closed_form(oracle, 4)),
        ("bwd_linear_attention", lambda: bpins.test_backward_linear_attention(oracle, 11, 16)),
        ("bwd_chain_rule", lambda: bpins.test_backward_chain_rule_across_calls(oracle)),
        ("ln_torch", lambda: ppins.test_layernorm_matches_torch(oracle, 1e-2)),
        ("tok_eta_head", lambda: ppins.test_constant_token_eta_is_head_eta(oracle, 4)),
        ("tok_eta_autograd", lambda: ppins.test_token_eta_matches_autograd(oracle, 3)),
        ("tok_eta_zero", lambda: ppins.test_zero_token_eta_freezes_the_state(oracle)),
        ("start_read_la", lambda: ppins.test_chunk_start_read_is_block_causal_linear_attention(oracle, 13, 8)),
        ("start_read_b1", lambda: ppins.test_chunk_start_read_b1_is_online_gd_read_before_update(oracle)),
        ("pbwd_off", lambda: pbpins.test_prologue_off_is_linear_backward(oracle, 2, 3, 37, 16, False)),
        ("pbwd_fd", lambda: pbpins.test_matches_finite_differences(oracle, 7, 3, 3, True, True)),
        ("pbwd_autograd", lambda: pbpins.test_matches_torch_autograd(oracle, 4, False)),
        ("pbwd_autograd_start", lambda: pbpins.test_matches_torch_autograd(oracle, 4, True)),
        ("pbwd_token_sum", lambda: pbpins.test_token_eta_gradients_sum_to_head_gradient(oracle, False)),
        ("mom_worked", lambda: mpins.test_momentum_worked_examples_exact(oracle)),
        ("mom_heavy_ball", lambda: mpins.test_heavy_ball_closed_form(oracle, 0.1, 0.5)),
        ("mom_beta0_online", lambda: mpins.test_beta_zero_exact_steps_is_online_gd(oracle, 5)),
        ("mom_beta0_minibatch", lambda: mpins.test_beta_zero_chunk_start_is_minibatch(oracle, 4)),
        ("mom_autograd_exact", lambda: mpins.test_momentum_matches_autograd(oracle, 0, 6)),
        ("mom_autograd_start", lambda: mpins.test_momentum_matches_autograd(oracle, 1, 6)),
    ]
    for name, fn in checks:
        try:
            with np.errstate(all="ignore"):
                fn()
        except AssertionError:
            failed.append(name)
    return failed


def _build_variant(src_text, tmpdir, tag):
    c = os.path.join(tmpdir, f"oracle_{tag}.c")
    so = os.path.join(tmpdir, f"liboracle_{tag}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", c, "-o", so, "-lm"],
                   check=True, capture_output=True)
    return so


def _with_library(so):
    import ctypes
    saved = oracle._lib
    oracle._lib = None
    real = oracle._LIB
    oracle._LIB = so
    try:
        oracle._load()
        return _battery()
    finally:
        oracle._lib = saved
        oracle._LIB = real
        del ctypes


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


def test_unmodified_source_passes_battery(source):
    with tempfile.TemporaryDirectory() as td:
        so = _build_variant(source, td, "clean")
        assert _with_library(so) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    with tempfile.TemporaryDirectory() as td:
        so = _build_variant(source.replace(old, new), td, name)
        failed = _with_library(so)
    assert failed, f"mutant {name} passed every pin"

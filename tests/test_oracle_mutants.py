"""Plant plausible mistakes in copies of the oracle (on the CPU) and require the
pins to catch every one of them.  This shows the pins constrain each term of
the definition: the decay and its sign, the dt on the input, the readout order,
B versus C, the D skip, the gate and its order, the group index, the B/C
layout, the initial state and the final state; and each term of the backward
(the adjoint's decay, the state each gradient uses, the gate derivative, the
upstream state gradient); the trapezoid's previous-token term and each
term of its backward; and the rotary step on B and C (the angle's sign
and running sum, the rotation, the pairing of states, the group, the per-head
angles, the starting angle, C's rotation)."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, [(old, new), ...]) -- every ``old`` must occur in oracle.c.
MUTANTS = [
    ("decay_sign", [("exp(dl * A[d * dstate + n])", "exp(-dl * A[d * dstate + n])")]),
    ("no_dt_on_input", [("h[n] = abar * h[n] + dl * B[j] * x;", "h[n] = abar * h[n] + B[j] * x;")]),
    ("readout_before_update", [(
        "h[n] = abar * h[n] + dl * B[j] * x;\n                    acc += C[j] * h[n];",
        "acc += C[j] * h[n];\n                    h[n] = abar * h[n] + dl * B[j] * x;")]),
    ("b_c_swapped", [("dl * B[j] * x", "dl * C[j] * x"), ("acc += C[j] * h[n];", "acc += B[j] * h[n];")]),
    ("no_dskip", [("if (Dskip) acc += Dskip[d] * x;", "")]),
    ("sigmoid_gate", [("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));")]),
    ("gate_before_dskip", [(
        "if (Dskip) acc += Dskip[d] * x;\n                if (z) acc *= silu(z[i]);",
        "if (z) acc *= silu(z[i]);\n                if (Dskip) acc += Dskip[d] * x;")]),
    ("group_index", [("const int64_t g = d / dpg;", "const int64_t g = d % ngroups;")]),
    ("bc_layout_transposed", [("((b * ngroups + g) * dstate + n) * seqlen + t",
                               "((b * ngroups + g) * seqlen + t) * dstate + n")]),
    ("h0_ignored", [("h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;", "h[n] = 0.0;")]),
    ("dt_times_a_off_by_one", [("const double dl = delta[i];",
                                "const double dl = delta[t + 1 < seqlen ? i + 1 : i];")]),
    ("ssd_decay_sign", [("exp(d * A[hd])", "exp(-d * A[hd])")]),
    ("ssd_no_dt_on_input", [("*hp = alpha * *hp + d * Bt[n] * xv;", "*hp = alpha * *hp + Bt[n] * xv;")]),
    ("ssd_no_dskip", [("if (Dskip) acc += Dskip[hd] * xv;", "")]),
    ("ssd_wrong_state_index", [("double *hp = &H[p * dstate + n];", "double *hp = &H[n * headdim + p];")]),
    ("ssd_group_index", [("const int64_t g = hd / hpg;", "const int64_t g = hd % ngroups;")]),
    ("ssd_h0_ignored", [("H[k] = h0 ? h0[(b * nheads + hd) * headdim * dstate + k] : 0.0;", "H[k] = 0.0;")]),
    ("trap_no_beta_term", [("H[k] = alpha * H[k] + beta * prev[k] + gamma * bx;",
                            "H[k] = alpha * H[k] + gamma * bx;")]),
    ("trap_beta_without_decay", [("const double beta = (d - gamma) * alpha;", "const double beta = d - gamma;")]),
    ("trap_gamma_ignores_lam", [("const double gamma = lm * d;", "const double gamma = d;")]),
    ("trap_prev_updated_first", [("H[k] = alpha * H[k] + beta * prev[k] + gamma * bx;\n                        prev[k] = bx;",
                                  "prev[k] = bx;\n                        H[k] = alpha * H[k] + beta * prev[k] + gamma * bx;")]),
    ("trap_prev_ignored", [("prev[p * dstate + n] = x_prev ?", "prev[p * dstate + n] = 0 ?")]),
    ("trap_prev_group_index", [("B_prev[(b * ngroups + g) * dstate + n]",
                                "B_prev[(b * ngroups + hd % ngroups) * dstate + n]")]),
    ("trap_prev_head_index", [("x_prev[(b * nheads + hd) * headdim + p]",
                               "x_prev[(b * nheads + g) * headdim + p]")]),
    ("bwd_no_decay_in_adjoint", [("lam[n] = abar * l;", "lam[n] = l;")]),
    ("bwd_dA_uses_new_state", [("dA[d * dstate + n] += l * dl * abar * hprev;",
                                "dA[d * dstate + n] += l * dl * abar * hs[(t + 1) * dstate + n];")]),
    ("bwd_ddelta_no_decay_term", [("ddl += l * (B[j] * x + a * abar * hprev);", "ddl += l * (B[j] * x);")]),
    ("bwd_dC_uses_old_state", [("dC[j] += dyh * hs[(t + 1) * dstate + n];", "dC[j] += dyh * hs[t * dstate + n];")]),
    ("bwd_gate_derivative", [("dz[i] = dy[i] * yhat[t] * s * (1.0 + z[i] * (1.0 - s));",
                              "dz[i] = dy[i] * yhat[t] * s;")]),
    ("bwd_readout_ungated", [("const double l = lam[n] + dyh * C[j];", "const double l = lam[n] + dy[i] * C[j];")]),
    ("bwd_dh_last_ignored", [("lam[n] = dh_last ? dh_last[(b * dim + d) * dstate + n] : 0.0;", "lam[n] = 0.0;")]),
    ("bwd_dD_ungated", [("dD[d] += dyh * x;", "dD[d] += dy[i] * x;")]),
    ("ssd_bwd_no_decay_in_adjoint", [("                        lam[k] = alpha * l;", "                        lam[k] = l;")]),
    ("ssd_bwd_dC_uses_old_state", [("dCt[n] += S[(t + 1) * PN + k] * dyh[p];", "dCt[n] += S[t * PN + k] * dyh[p];")]),
    ("ssd_bwd_dA_without_decay", [("dA[hd] += l * d * alpha * S[t * PN + k];", "dA[hd] += l * d * S[t * PN + k];")]),
    ("ssd_bwd_ddt_no_input_term", [("ddl += l * (x[i] * Bt[n] + A[hd] * alpha * S[t * PN + k]);",
                                    "ddl += l * (A[hd] * alpha * S[t * PN + k]);")]),
    ("ssd_bwd_dx_no_dt", [("dxp += l * d * Bt[n];", "dxp += l * Bt[n];")]),
    ("ssd_bwd_gate_derivative", [("dz[i] = dy[i] * yhat[t * headdim + p] * sg * (1.0 + z[i] * (1.0 - sg));",
                                  "dz[i] = dy[i] * yhat[t * headdim + p] * sg;")]),
    ("ssd_bwd_dh_last_ignored", [("lam[k] = dh_last ? dh_last[(b * nheads + hd) * PN + k] : 0.0;", "lam[k] = 0.0;")]),
    ("ssd_bwd_group_index", [("            const int64_t g = hd / hpg;\n            /* forward, keeping every state",
                              "            const int64_t g = hd % ngroups;\n            /* forward, keeping every state")]),
    ("trap_bwd_no_next_beta", [("const double dq = gamma * l + beta_next * Ln[k];", "const double dq = gamma * l;")]),
    ("trap_bwd_dlam_sign", [("dlam[it] = d * (dga - alpha * dbe);", "dlam[it] = d * (dga + alpha * dbe);")]),
    ("trap_bwd_ddt_no_gamma_term", [(" + lm * dga;", ";")]),
    ("trap_bwd_ddt_beta_decay_dropped", [("(1.0 - lm) * alpha * (1.0 + d * A[hd]) * dbe", "(1.0 - lm) * alpha * dbe")]),
    ("trap_bwd_dA_no_beta", [("dA[hd] += d * (alpha * dal + beta * dbe);", "dA[hd] += d * alpha * dal;")]),
    ("trap_bwd_prev_uses_alpha", [("const double dp = seqlen > 0 ? beta_next * Ln[p * dstate + n] : 0.0;",
                                   "const double dp = seqlen > 0 ? alpha_next * Ln[p * dstate + n] : 0.0;")]),
    ("trap_bwd_dB_prev_not_summed", [("dbq[n] += dp * xp[p];", "dbq[n] = dp * xp[p];")]),
    ("trap_bwd_adjoint_no_decay", [("double l = dyh[p] * Ct[n] + alpha_next * Ln[k];", "double l = dyh[p] * Ct[n] + Ln[k];")]),
    ("trap_bwd_dbeta_uses_current_input", [("dbe += l * (Bq ? Bq[n] * xq : 0.0);", "dbe += l * Bt[n] * x[i];")]),
    ("softplus_overflows", [("return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));", "return log1p(exp(v));")]),
    ("softplus_bias_dropped", [("out[i] = softplus(raw[i] + bv);", "out[i] = softplus(raw[i]);")]),
    ("softplus_bias_index", [("bias[(i / inner) % nb]", "bias[i % nb]")]),
    ("softplus_grad_sign", [("grad_in[i] * sigmoid(raw[i] + bv)", "grad_in[i] * sigmoid(-(raw[i] + bv))")]),
    ("sigmoid_sign", [("return 1.0 / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(v));")]),
    ("rope_angle_sign", [("phi -= dt[(b * seqlen + t) * nheads + h]", "phi += dt[(b * seqlen + t) * nheads + h]")]),
    ("rope_exclusive_sum", [(
        "phi -= dt[(b * seqlen + t) * nheads + h] * theta[((b * seqlen + t) * theta_heads + th) * half + k];\n"
        "          const double c = cos(phi), s = sin(phi);",
        "const double c = cos(phi), s = sin(phi);\n"
        "          phi -= dt[(b * seqlen + t) * nheads + h] * theta[((b * seqlen + t) * theta_heads + th) * half + k];")]),
    ("rope_rotation_sign", [("B_rot[dst + k + half] = b1 * s + b2 * c;", "B_rot[dst + k + half] = -b1 * s + b2 * c;")]),
    ("rope_pairs_adjacent", [("const double b1 = B[src + k], b2 = B[src + k + half];",
                              "const double b1 = B[src + 2 * k], b2 = B[src + 2 * k + 1];"),
                             ("const double c1 = C[src + k], c2 = C[src + k + half];",
                              "const double c1 = C[src + 2 * k], c2 = C[src + 2 * k + 1];"),
                             ("B_rot[dst + k] = b1", "B_rot[dst + 2 * k] = b1"),
                             ("B_rot[dst + k + half] = b1", "B_rot[dst + 2 * k + 1] = b1"),
                             ("C_rot[dst + k] = c1", "C_rot[dst + 2 * k] = c1"),
                             ("C_rot[dst + k + half] = c1", "C_rot[dst + 2 * k + 1] = c1")]),
    ("rope_group_index", [("const int64_t g = h / hpg;", "const int64_t g = h % ngroups;")]),
    ("rope_theta_head", [("const int64_t th = theta_heads == 1 ? 0 : h;", "const int64_t th = 0;")]),
    ("rope_angle0_ignored", [("double phi = angle0 ? angle0[(b * nheads + h) * half + k] : 0.0;", "double phi = 0.0;")]),
    ("rope_c_unrotated", [("C_rot[dst + k] = c1 * c - c2 * s;", "C_rot[dst + k] = c1;"),
                          ("C_rot[dst + k + half] = c1 * s + c2 * c;", "C_rot[dst + k + half] = c2;")]),
    # the rotary step's backward
    ("rope_bwd_angle_grad_sign", [("dphi[t] = -gb1 * rb2 + gb2 * rb1", "dphi[t] = gb1 * rb2 - gb2 * rb1")]),
    ("rope_bwd_not_transposed", [("dB[src + k + half] += -gb1 * s + gb2 * c;", "dB[src + k + half] += gb1 * s + gb2 * c;"),
                                 ("dB[src + k] += gb1 * c + gb2 * s;", "dB[src + k] += gb1 * c - gb2 * s;")]),
    ("rope_bwd_exclusive_suffix", [(
        "R += dphi[t];\n          const int64_t it = (b * seqlen + t) * nheads + h;",
        "const int64_t it = (b * seqlen + t) * nheads + h;"),
        ("ddt[it] += -theta[ith] * R;\n        }", "ddt[it] += -theta[ith] * R;\n          R += dphi[t];\n        }")]),
    ("rope_bwd_dangle_last_ignored", [("double R = dangle_last ? dangle_last[(b * nheads + h) * half + k] : 0.0;",
                                       "double R = 0.0;")]),
    ("rope_bwd_dtheta_without_dt", [("dtheta[ith] += -dt[it] * R;", "dtheta[ith] += -R;")]),
    ("rope_bwd_c_angle_term_dropped", [("- gc1 * rc2 + gc2 * rc1;", ";")]),
]


def _build(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutant {name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", *oracle._CFLAGS, str(c), "-o", str(so), "-lm"])
    return oracle.Oracle(str(so))


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    orc = _build(tmp_path, name, edits)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"

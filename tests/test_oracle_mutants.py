"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutant is a copy of ``oracle/selscan_ref.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a transposed or swapped operand),
compiled with gcc into a temporary directory and run through every pin. CPU
only; the built oracle itself is untouched.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "selscan_ref.c")

# (name, original text, replacement). Every original must occur in the source.
MUTANTS = [
    ("decay_sign", "exp(dl * Ad[n])", "exp(-dl * Ad[n])"),
    ("decay_no_delta", "exp(dl * Ad[n])", "exp(Ad[n])"),
    ("input_no_delta", "dl * Bb[n * L + t] * x[t]", "Bb[n * L + t] * x[t]"),
    ("B_transposed", "dl * Bb[n * L + t] * x[t]", "dl * Bb[t * N + n] * x[t]"),
    ("readout_uses_B", "acc += Cb[n * L + t] * h[n];", "acc += Bb[n * L + t] * h[n];"),
    ("C_time_shift", "acc += Cb[n * L + t] * h[n];",
     "acc += Cb[n * L + (t > 0 ? t - 1 : 0)] * h[n];"),
    ("no_D_skip", "double yv = acc + Dd * x[t];", "double yv = acc;"),
    ("D_outside_gate", "yv *= g;", "yv = acc * g + Dd * x[t];"),
    ("gate_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("softplus_sign", "log1p(exp(-fabs(u)))", "log1p(exp(fabs(u)))"),
    ("softplus_no_max", "fmax(u, 0.0) + log1p", "log1p"),
    ("bias_dropped", "softplus(dr[t] + bias)", "softplus(dr[t])"),
    ("bias_outside", "softplus(dr[t] + bias)", "(softplus(dr[t]) + bias)"),
    ("A_row_index", "j->A + d * N", "j->A + b * N"),
    ("h0_ignored", "h[n] = j->h0 ? j->h0[row * N + n] : 0.0;", "h[n] = 0.0;"),
    ("state_no_decay", "h[n] = abar * h[n] + bx;", "h[n] = h[n] + bx;"),
    ("scale_no_decay", "habs[n] = abar * habs[n] + fabs(bx);", "habs[n] = habs[n] + fabs(bx);"),
    ("scale_no_D", "double sv = acc_abs + fabs(Dd * x[t]);", "double sv = acc_abs;"),
    ("last_state_scale_swap", "if (j->last_state) j->last_state[i * N + n] = h[n];",
     "if (j->last_state) j->last_state[i * N + n] = habs[n];"),
    ("step_decay_index", "exp(dl * A[d * N + n])", "exp(dl * A[n])"),
    ("step_no_delta", "dl * B[b * N + n] * xv", "B[b * N + n] * xv"),
    ("step_readout_B", "acc += C[b * N + n] * h[n];", "acc += B[b * N + n] * h[n];"),
    ("step_no_D", "double yv = acc + Dd * xv;", "double yv = acc;"),
    ("step_no_gate", "yv *= g;\n                sv *= fabs(g);\n            }\n            y[row] = yv;",
     "sv *= fabs(g);\n            }\n            y[row] = yv;"),
    ("step_softplus_dropped", "const double dl = softplus(delta[row]);",
     "const double dl = delta[row];"),
    ("conv_taps_reversed", "pre += w[d * K + k] * xv;", "pre += w[d * K + (K - 1 - k)] * xv;"),
    ("conv_window_off_by_one", "const int64_t s = t - (K - 1) + k;", "const int64_t s = t - K + k;"),
    ("conv_not_causal", "const int64_t s = t - (K - 1) + k;", "const int64_t s = t + k;"),
    ("conv_prev_order", "(pr ? pr[K - 1 + s] : 0.0);\n                    pre +=",
     "(pr ? pr[-1 - s] : 0.0);\n                    pre +="),
    ("conv_bias_dropped", "double pre = bias ? bias[d] : 0.0;\n                double sc",
     "double pre = 0.0;\n                double sc"),
    ("conv_no_silu", "out[row * seqlen + t] = silu(pre);", "out[row * seqlen + t] = pre;"),
    ("conv_scale_signed", "sc += fabs(w[d * K + k] * xv);", "sc += w[d * K + k] * xv;"),
    ("conv_last_wrong", "x_last[row * (K - 1) + k] = s >= 0 ? xr[s]", "x_last[row * (K - 1) + k] = s > 0 ? xr[s]"),
    ("conv_step_shift_wrong", "for (int64_t k = 0; k + 1 < K - 1; ++k) st[k] = st[k + 1];",
     "for (int64_t k = 0; k + 1 < K - 1; ++k) st[k + 1] = st[k];"),
    ("conv_step_newest_tap", "pre += w[d * K + K - 1] * x[row];", "pre += w[d * K] * x[row];"),
    ("bwd_dA_sign", "j->pA[(b * dim + d) * N + n] += q * dl;", "j->pA[(b * dim + d) * N + n] -= q * dl;"),
    ("bwd_carry_no_decay", "carry[n] = abar * dh;", "carry[n] = dh;"),
    ("bwd_q_uses_h_t", "const double q = dh * abar * hp[n];", "const double q = dh * abar * h[n];"),
    ("bwd_dB_no_dl", "dBb[n * L + t] += dh * dl * x[t];", "dBb[n * L + t] += dh * x[t];"),
    ("bwd_dC_prev_state", "dCb[n * L + t] += ds * h[n];", "dCb[n * L + t] += ds * hp[n];"),
    ("bwd_ddelta_no_sigmoid", "j->ddelta[row * L + t] = ddl * sg;", "j->ddelta[row * L + t] = ddl;"),
    ("bwd_dx_no_D", "j->dx[row * L + t] = ds * Dd + dl * accB;", "j->dx[row * L + t] = dl * accB;"),
    ("bwd_dz_uses_silu", "j->dz[row * L + t] = dy[t] * s * gp;", "j->dz[row * L + t] = dy[t] * s * g;"),
    ("bwd_ds_no_gate", "const double ds = dy[t] * g, dsa = fabs(ds);", "const double ds = dy[t], dsa = fabs(ds);"),
    ("bwd_decay_term_dropped", "ddl += q * Ad[n];", "ddl += 0.0 * Ad[n];"),
    ("bwd_dD_ungated", "dD += ds * x[t];", "dD += dy[t] * x[t];"),
    ("bwd_dt_bias_no_sigmoid", "dT += ddl * sg;", "dT += ddl;"),
    ("conv_bwd_no_silu_grad", "g[t] = dr[t] * sg * (1.0 + pre * (1.0 - sg));", "g[t] = dr[t] * sg;"),
    ("conv_bwd_tap_reversed", "if (t >= 0 && t < L) { v += wd[k] * g[t];", "if (t >= 0 && t < L) { v += wd[K - 1 - k] * g[t];"),
    ("conv_bwd_dw_shift", "dw[d * K + k] += g[t] * XX(t - H + k);", "dw[d * K + k] += g[t] * XX(t - H + k - 1);"),
    ("ssd_decay_no_delta", "const double a = exp(dl * Ah);", "const double a = exp(Ah);"),
    ("ssd_input_no_delta", "const double in = dl * Bt[n] * xt[p];", "const double in = Bt[n] * xt[p];"),
    ("ssd_h0_ignored", "S[k] = j->h0 ? j->h0[i * N * P + k] : 0.0;", "S[k] = 0.0;"),
    ("ssd_readout_B", "acc += Ct[n] * S[n * P + p];", "acc += Bt[n] * S[n * P + p];"),
    ("ssd_no_D", "yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    ("ssd_head_index", "const double dl = softplus(j->delta[(b * L + t) * H + h] + bias);",
     "const double dl = softplus(j->delta[(b * L + t) * H] + bias);"),
    ("ssd_state_transposed", "S[n * P + p] = a * S[n * P + p] + in;", "S[n * P + p] = a * S[p * N + n % P] + in;"),
    ("bwd_h0_ignored", "H[n] = j->h0 ? j->h0[row * N + n] : 0.0;", "H[n] = 0.0;"),
    ("bwd_dlast_ignored", "carry[n] = j->dlast ? j->dlast[row * N + n] : 0.0;", "carry[n] = 0.0;"),
    ("bwd_dh0_scale_swap", "j->dh0[row * N + n] = carry[n];", "j->dh0[row * N + n] = carry_abs[n];"),
    ("bwd_dx_scale_no_D", "j->sdx[row * L + t] = fabs(ds * Dd) + dl * accBa;", "j->sdx[row * L + t] = dl * accBa;"),
]


@pytest.mark.parametrize("name,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, repl):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(orig, repl, 1)
    c = tmp_path / f"{name}.c"
    c.write_text(mutated)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(c), "-o",
                    str(so), "-lm"], check=True)
    O = oracle.Oracle(str(so))
    caught = []
    for pname, fn in PINS.items():
        try:
            fn(O)
        except (AssertionError, FloatingPointError, ValueError, RuntimeError):
            caught.append(pname)
    assert caught, f"mutant {name} passed every pin"

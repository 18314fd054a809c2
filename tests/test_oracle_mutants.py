"""The pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a temporary copy of the oracle's C
source (a dropped term, a wrong sign, a transposed operand, an off-by-one
index), compiles it on the CPU, and checks that at least one pin rejects it.
The real oracle is never modified.
"""
import os

import pytest

import oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "cfc_oracle.c")

MUTANTS = {
    "forward_transposed_w_rec": ("s += w_rec[(size_t)i * H + j] * h[j];",
                                 "s += w_rec[(size_t)j * H + i] * h[j];"),
    "forward_drops_bias": ("double s = bias[i];", "double s = 0.0;"),
    "forward_gate_sign": ("g[i] = oracle_sigmoid(-sp[i] * s * dt);",
                          "g[i] = oracle_sigmoid(sp[i] * s * dt);"),
    "forward_gate_roles_swapped": ("h_next[i] = g[i] * h[i] + (1.0 - g[i]) * c[i];",
                                   "h_next[i] = (1.0 - g[i]) * h[i] + g[i] * c[i];"),
    "softplus_wrong_branch": ("return log1p(exp(-fabs(w))) + (w > 0.0 ? w : 0.0);",
                              "return log1p(exp(-fabs(w))) + (w < 0.0 ? w : 0.0);"),
    "backward_drops_gate_term": ("- dz[i] * sp[i] * dt;", ";"),
    "backward_dz_sign": ("dz[i] = delta[i] * (hp[i] - c[i]) * g[i] * (1.0 - g[i]);",
                         "dz[i] = delta[i] * (c[i] - hp[i]) * g[i] * (1.0 - g[i]);"),
    "backward_tanh_derivative": ("(1.0 - c[i] * c[i]) - dz[i] * sp[i] * dt;", "(1.0 - c[i]) - dz[i] * sp[i] * dt;"),
    "backward_transposed_w_rec": ("s += w_rec[(size_t)i * H + j] * da[i];",
                                  "s += w_rec[(size_t)j * H + i] * da[i];"),
    "backward_drops_direct_path": ("double s = delta[j] * g[j];", "double s = 0.0;"),
    "backward_h_prev_off_by_one": ("h_seq + ((size_t)b * K + (k - 1)) * H;",
                                   "h_seq + ((size_t)b * K + k) * H;"),
    "backward_dw_tau_missing_sigmoid": ("g_wtau[i] += dz[i] * (-a[i] * dt) * sw[i];",
                                        "g_wtau[i] += dz[i] * (-a[i] * dt);"),
    "backward_dw_rec_uses_x": ("g_wrec[(size_t)i * H + j] += da[i] * hp[j];",
                               "g_wrec[(size_t)i * H + j] += da[i] * hn[j];"),
    "backward_no_scratch_clear": ("row[j] = 0.0;", "row[j] = row[j];"),
    "reduce_skips_first_row": ("for (long long b = 0; b < B; ++b)\n        for (long long j = 0; j < N; ++j)\n            out[j] += in[b * N + j];",
                               "for (long long b = 1; b < B; ++b)\n        for (long long j = 0; j < N; ++j)\n            out[j] += in[b * N + j];"),
    "loss_seed_sign": ("delta[i] = hK[i] - y[(size_t)b * H + i];",
                       "delta[i] = y[(size_t)b * H + i] - hK[i];"),
    "grad_x_transposed_w_in": ("t += w_in[(size_t)i * n_in + j] * da[i];",
                               "t += w_in[(size_t)j * n_in + i] * da[i];"),
    "grad_x_uses_dz": ("t += w_in[(size_t)i * n_in + j] * da[i];",
                       "t += w_in[(size_t)i * n_in + j] * dz[i];"),
    "grad_x_steps_reversed": ("double *gx = grad_x + ((size_t)b * K + k) * n_in;",
                              "double *gx = grad_x + ((size_t)b * K + (K - 1 - k)) * n_in;"),
    "tau_decay_product": ("sp[i] = exp(-dt / tau_eff);", "sp[i] = exp(-dt * tau_eff);"),
    "tau_guard_inverted": ("sw[i] = w_tau[i] > ORACLE_TAU_EPS ? dt / (tau_eff * tau_eff) : 0.0;",
                           "sw[i] = w_tau[i] > ORACLE_TAU_EPS ? 0.0 : dt / (tau_eff * tau_eff);"),
    "tau_da_drops_one_minus_decay": ("da[i] = delta[i] * (1.0 - g[i]) * (1.0 - c[i] * c[i]);\n",
                                     "da[i] = delta[i] * (1.0 - c[i] * c[i]);\n"),
    "tau_dtau_missing_decay": ("g_wtau[i] += dz[i] * g[i] * sw[i];", "g_wtau[i] += dz[i] * sw[i];"),
    "tau_dz_sign": ("dz[i] = delta[i] * (hp[i] - c[i]);", "dz[i] = delta[i] * (c[i] - hp[i]);"),
    "grad_h0_before_last_step": ("            memcpy(delta, delta_prev, sizeof(double) * H);\n        }\n        /* after step 0",
                                 "            if (k > 0) memcpy(delta, delta_prev, sizeof(double) * H);\n        }\n        /* after step 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    O.build_oracle(str(mutated), so)
    lib = O.load_oracle(so)
    caught = []
    for pin_name, pin in P.ALL_PINS.items():
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"no pin caught mutant {name}"

"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Each mutant is the oracle's C source with one fragment replaced, compiled into a temporary
library. A mutant must break at least one pin; the fragment must occur exactly once in the
source, so the list stays in step with the oracle.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "decay_dropped": ("S[(size_t)i * dk + j] = alpha * s_proj + beta * v[i] * k[j];",
                      "S[(size_t)i * dk + j] = s_proj + beta * v[i] * k[j];"),
    "decay_on_write_term": ("S[(size_t)i * dk + j] = alpha * s_proj + beta * v[i] * k[j];",
                            "S[(size_t)i * dk + j] = alpha * (s_proj + beta * v[i] * k[j]);"),
    "projector_sign": ("S[(size_t)i * dk + j] - beta * Sk[i] * k[j];",
                       "S[(size_t)i * dk + j] + beta * Sk[i] * k[j];"),
    "write_without_beta": ("alpha * s_proj + beta * v[i] * k[j]", "alpha * s_proj + v[i] * k[j]"),
    "state_transposed_in_Sk": ("acc += S[(size_t)i * dk + j] * k[j];",
                               "acc += S[(size_t)j * dk + i] * k[j];"),
    "readout_with_k": ("acc += S[(size_t)i * dk + j] * (scale * q[j]);",
                       "acc += S[(size_t)i * dk + j] * (scale * k[j]);"),
    "readout_without_scale": ("(scale * q[j])", "(q[j])"),
    "gates_swapped": ("alpha[g], beta[g], scale", "beta[g], alpha[g], scale"),
    "conv_taps_reversed": ("acc += w[i] * u[t + i];", "acc += w[3 - i] * u[t + i];"),
    "conv_window_shifted": ("acc += w[i] * u[t + i];", "acc += w[i] * u[t + i - (t > 0)];"),
    "silu_dropped": ("y[(size_t)t * C + c] = acc * logistic(acc);", "y[(size_t)t * C + c] = acc;"),
    "conv_bias_dropped": ("if (conv_b) acc += conv_b[c];", "if (0) acc += conv_b[c];"),
    "conv_state_not_rolled": ("cs[0] = u[T]; cs[1] = u[T + 1]; cs[2] = u[T + 2];",
                              "cs[0] = u[0]; cs[1] = u[1]; cs[2] = u[2];"),
    "l2_norm_without_sqrt": ("double nq = sqrt(sq + l2_eps), nk = sqrt(sk + l2_eps);",
                             "double nq = (sq + l2_eps), nk = sqrt(sk + l2_eps);"),
    "q_k_blocks_swapped": ("const double* yq = yt + (size_t)h * dk;",
                           "const double* yq = yt + (size_t)H * dk + (size_t)h * dk;"),
    "beta_sign": ("beta[g] = logistic(b_logit[g]);", "beta[g] = logistic(-b_logit[g]);"),
    "alpha_sign": ("alpha[g] = exp(-softplus(a_logit[g]));",
                   "alpha[g] = exp(softplus(a_logit[g]));"),
    "softplus_without_log1p": ("return m + log1p(exp(-fabs(x)));", "return m + exp(-fabs(x));"),
    "lowrank_old_writes_not_decayed": ("ch[s] = alpha[g] * ch[s];", "ch[s] = ch[s];"),
    "lowrank_new_write_decayed": ("ch[p] = 1.0;", "ch[p] = alpha[g];"),
    "lowrank_slot_not_advanced": ("p = (p + 1) % r;", "p = p % r;"),
    "lowrank_newest_evicted": ("p = (p + 1) % r;", "p = (p + r - 1) % r;"),
    "lowrank_evict_before_write": ("/* 1-2: the write against the state before the token */",
                                   "ch[p] = 0.0;"),
    "lowrank_readout_before_update": (
        "/* 5: readout with the updated state */\n                lowrank_form_state(r, dk, dv, Uh, Kh, ch, S);",
        "/* 5 */"),
    "lowrank_key_from_q": ("Kh[(size_t)p * dk + j] = kt[j];", "Kh[(size_t)p * dk + j] = qt[j];"),
    "lowrank_write_without_alpha": ("delta[i] = beta[g] * (vt[i] - alpha[g] * acc);",
                                    "delta[i] = beta[g] * (vt[i] - acc);"),
    "lowrank_form_transposed_key": (
        "S[(size_t)i * dk + j] += c[s] * U[(size_t)s * dv + i] * K[(size_t)s * dk + j];",
        "S[(size_t)i * dk + j] += c[s] * U[(size_t)s * dv + i] * K[(size_t)s * dk + (dk - 1 - j)];"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"fragment for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    lib_path = oracle.build(str(src), str(tmp_path / f"lib{name}.so"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_build_passes_every_pin(source, tmp_path):
    src = tmp_path / "same.c"
    src.write_text(source)
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libsame.so")))
    for pin in oracle_pins.ALL_PINS:
        pin(lib)

"""Plant plausible mistakes in copies of the oracle source and check that the
pins in test_oracle_pins.py catch every one (CPU only).

Each mutant is built with gcc from a textually edited copy of
oracle/kda_oracle.c in a temporary directory; the real oracle is untouched.
"""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import kda_oracle

SRC = os.path.join(os.path.dirname(kda_oracle.__file__), "kda_oracle.c")

TOKEN_STEP_DECAY_AFTER_WRITE = """
static void token_step(double *S, int64_t dk, int64_t dv, const double *qb,
                       const double *kb, const float *v, const float *g,
                       double beta, double *vh, double *o) {
    for (int64_t j = 0; j < dv; ++j) vh[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) vh[j] += S[i * dv + j] * kb[i];
    for (int64_t j = 0; j < dv; ++j) vh[j] = beta * ((double)v[j] - vh[j]);
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kb[i] * vh[j];
    for (int64_t i = 0; i < dk; ++i) {
        double a = exp((double)g[i]);
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) o[j] += S[i * dv + j] * qb[i];
}
"""

TOKEN_STEP_READ_BEFORE_WRITE = """
static void token_step(double *S, int64_t dk, int64_t dv, const double *qb,
                       const double *kb, const float *v, const float *g,
                       double beta, double *vh, double *o) {
    for (int64_t i = 0; i < dk; ++i) {
        double a = exp((double)g[i]);
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) o[j] += S[i * dv + j] * qb[i];
    for (int64_t j = 0; j < dv; ++j) vh[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) vh[j] += S[i * dv + j] * kb[i];
    for (int64_t j = 0; j < dv; ++j) vh[j] = beta * ((double)v[j] - vh[j]);
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kb[i] * vh[j];
}
"""


def _replace_token_step(src: str, body: str) -> str:
    a = src.index("static void token_step(")
    b = src.index("static void run_unit_recurrence(")
    return src[:a] + body.strip() + "\n\n" + src[b:]


# (name, function of the source text -> mutated text)
MUTANTS = [
    ("delta sign flipped",
     lambda s: s.replace("vh[j] = beta * ((double)v[j] - vh[j]);",
                         "vh[j] = beta * ((double)v[j] + vh[j]);")),
    ("beta dropped",
     lambda s: s.replace("vh[j] = beta * ((double)v[j] - vh[j]);",
                         "vh[j] = ((double)v[j] - vh[j]);")),
    ("write uses q instead of k",
     lambda s: s.replace("S[i * dv + j] += kb[i] * vh[j];", "S[i * dv + j] += qb[i] * vh[j];")),
    ("prediction uses q instead of k",
     lambda s: s.replace("vh[j] += S[i * dv + j] * kb[i];", "vh[j] += S[i * dv + j] * qb[i];")),
    ("read-out uses k instead of q",
     lambda s: s.replace("o[j] += S[i * dv + j] * qb[i];", "o[j] += S[i * dv + j] * kb[i];")),
    ("decay sign flipped",
     lambda s: s.replace("double a = exp((double)g[i]);", "double a = exp(-(double)g[i]);")),
    ("decay dropped",
     lambda s: s.replace("double a = exp((double)g[i]);", "double a = 1.0;")),
    ("decay on the value axis",
     lambda s: s.replace("for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;",
                         "for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= "
                         "exp((double)g[j < dk ? j : 0]) + 0.0 * a;")),
    ("decay after the write", lambda s: _replace_token_step(s, TOKEN_STEP_DECAY_AFTER_WRITE)),
    ("read-out before the write", lambda s: _replace_token_step(s, TOKEN_STEP_READ_BEFORE_WRITE)),
    ("no L2 normalisation",
     lambda s: s.replace("double inv = 1.0 / sqrt(ss + eps);", "double inv = 1.0;")),
    ("eps outside the square root",
     lambda s: s.replace("double inv = 1.0 / sqrt(ss + eps);",
                         "double inv = 1.0 / (sqrt(ss) + eps);")),
    ("scale dropped",
     lambda s: s.replace("load_vec(qb, J->q + th * dk, dk, J->l2norm, J->eps, J->scale);",
                         "load_vec(qb, J->q + th * dk, dk, J->l2norm, J->eps, 1.0);")),
    ("initial state ignored",
     lambda s: s.replace("S[e] = J->s0 ? (double)J->s0[so + e] : 0.0;", "S[e] = 0.0;")),
    ("state not reset between sequences",
     lambda s: s.replace("S[e] = J->s0 ? (double)J->s0[so + e] : 0.0;",
                         "S[e] = (J->s0 && n == 0) ? (double)J->s0[so + e] : S[e] * (n == 0);")),
]

# every pin, with one parameter set each where parametrised
PIN_CALLS = [
    ("hand example", lambda o: pins.test_hand_worked_example(o)),
    ("P1", lambda o: pins.test_p1_delta_write_recalls_value(o)),
    ("P2", lambda o: pins.test_p2_beta0_g0_is_identity(o)),
    ("P3", lambda o: pins.test_p3_beta0_pure_channel_decay(o)),
    ("P5", lambda o: pins.test_p5_matches_explicit_unrolling(o, 5, 12, 4, 3)),
    ("P6", lambda o: pins.test_p6_orthonormal_keys_reduce_to_causal_linear_attention(o)),
    ("P7a", lambda o: pins.test_p7a_repeated_key_converges_without_stacking(o, 0.3)),
    ("P7b", lambda o: pins.test_p7b_scalar_gate_geometric_series(o)),
    ("P8", lambda o: pins.test_p8_norm_growth_bounded_by_the_write(o)),
    ("P10", lambda o: pins.test_p10_chunk_form_equals_recurrence(o, 16)),
    ("varlen", lambda o: pins.test_varlen_packing_equals_separate_runs(o)),
    ("null state", lambda o: pins.test_null_initial_state_is_zero(o)),
    ("l2/scale", lambda o: pins.test_l2norm_makes_qk_scale_free_and_scale_is_linear(o)),
    ("decode=prefill", lambda o: pins.test_decode_steps_equal_prefill(o)),
]


def _caught_by(oracle_mod) -> list:
    caught = []
    for name, call in PIN_CALLS:
        try:
            with np.errstate(all="ignore"):
                call(oracle_mod)
        except (AssertionError, RuntimeError, FloatingPointError):
            caught.append(name)
    return caught


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,mutate", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle, source, name, mutate):
    mutated = mutate(source)
    assert mutated != source, f"mutation '{name}' did not apply"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mut.c")
        so = os.path.join(td, "libmut.so")
        with open(c, "w") as f:
            f.write(mutated)
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                        "-shared", "-w", "-o", so, c, "-lpthread", "-lm"], check=True)
        with kda_oracle.using_library(so):
            caught = _caught_by(kda_oracle)
    assert caught, f"planted mistake '{name}' survived every pin"


def test_unmutated_oracle_passes_every_pin(oracle):
    assert _caught_by(kda_oracle) == []

"""CPU tests: the oracle against its pins, and the pins against planted mistakes.

The mutation test copies the oracle's C source, plants one plausible mistake
(a dropped term, an off-by-one, a wrong sign or index, a multiply-by-zero
reset), builds the copy with gcc, and requires at least one pin to fail.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

import oracle as oracle_mod
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_finite_differences_no_gate_no_skip_no_bias(orc):
    oc.check_finite_differences(orc, gate=False, skip=False, bias=False, seed=21, lengths=(1, 5, 2))


def test_finite_differences_single_token_sequences(orc):
    oc.check_finite_differences(orc, seed=22, lengths=(1, 1, 3, 1))


# (function, text as written, planted mistake)
MUTATIONS = [
    ("conv: tap kept one step too early", "if (k <= pos[t]) acc += w", "if (k < pos[t]) acc += w"),
    ("conv: taps in reverse order", "w[(int64_t)d * W + (W - 1 - k)] * x[(t - k) * D + d];\n            if (v)",
     "w[(int64_t)d * W + k] * x[(t - k) * D + d];\n            if (v)"),
    ("scan: skip term dropped", "if (Dp) acc += Dp[d] * uu;\n            if (y)", "if (y)"),
    ("scan: reset multiplies by zero", "h[n] = bu;\n                } else {\n                    const double a = exp(dt * A[(int64_t)d * N + n]);\n                    h[n] = a * h[n] + bu;",
     "h[n] = exp(dt * A[(int64_t)d * N + n]) * (0.0 * h[n]) + bu;\n                } else {\n                    const double a = exp(dt * A[(int64_t)d * N + n]);\n                    h[n] = a * h[n] + bu;"),
    ("scan: decay sign flipped", "const double a = exp(dt * A[(int64_t)d * N + n]);\n                    h[n] = a * h[n] + bu;",
     "const double a = exp(-dt * A[(int64_t)d * N + n]);\n                    h[n] = a * h[n] + bu;"),
    ("scan: no reset at heads", "const int head = pos[t] == 0;\n            const double dt = delta_eff(delta[t * D + d], dbias, d, sp);\n            const double uu = u[t * D + d];\n            double acc = 0.0;\n            for (int32_t n = 0; n < N; ++n) {\n                const double bu = dt * B[t * N + n] * uu;\n                if (head) {\n                    h[n] = bu;",
     "const int head = t == 0;\n            const double dt = delta_eff(delta[t * D + d], dbias, d, sp);\n            const double uu = u[t * D + d];\n            double acc = 0.0;\n            for (int32_t n = 0; n < N; ++n) {\n                const double bu = dt * B[t * N + n] * uu;\n                if (head) {\n                    h[n] = bu;"),
    ("bwd: dA loses the delta factor", "dA_d[n] += term(dh * dt * a * hp);", "dA_d[n] += term(dh * a * hp);"),
    ("bwd: carry crosses heads", "ddt += term(dh * (Bn * uu));\n                    c[n] = 0.0;",
     "ddt += term(dh * (Bn * uu));\n                    c[n] = dh;"),
    ("bwd: previous state index off by one", "const double hp = hs[(t - 1) * N + n];", "const double hp = hs[t * N + n];"),
    ("bwd: dz uses the wrong sigmoid derivative", "s * (1.0 + zz * (1.0 - s))", "s * (1.0 + zz * s)"),
    ("bwd: dB misses u", "dB[t * N + n] += term(dh * dt * uu);", "dB[t * N + n] += term(dh * dt);"),
    ("bwd: dC uses the previous state", "dC[t * N + n] += term(g * hs[t * N + n]);",
     "dC[t * N + n] += term(g * (t > 0 ? hs[(t - 1) * N + n] : 0.0));"),
    ("conv bwd: reverse rule off by one", "if (s + k < T && k <= pos[s + k])", "if (s + k < T && k < pos[s + k])"),
    ("conv bwd: dw tap index transposed", "dw[(int64_t)d * W + (W - 1 - k)] = acc;", "dw[(int64_t)d * W + k] = acc;"),
    ("conv bwd: silu derivative drops a term", "gv[t] = term(g * s * (1.0 + v * (1.0 - s)));", "gv[t] = term(g * s);"),
    ("pack: heads off by one", "pos[t] = (int32_t)(t - cu[s]);", "pos[t] = (int32_t)(t - cu[s] + (s > 0));"),
    ("step map: softplus loses its log1p tail", "return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));",
     "return (v > 0.0 ? v : 0.0);"),
    ("step map: bias read for the wrong channel", "const double v = raw + (bias ? bias[d] : 0.0);",
     "const double v = raw + (bias ? bias[0] : 0.0);"),
    ("step map: backward misses the softplus slope", "return sp ? sigmoid(raw + (bias ? bias[d] : 0.0)) : 1.0;",
     "return 1.0;"),
    ("gate floor: forward drops it", "acc * (z[t * D + d] * sigmoid(z[t * D + d]) + gate_floor)",
     "acc * (z[t * D + d] * sigmoid(z[t * D + d]))"),
    ("gate floor: backward drops it", "g = term(go) * (term(zz * s) + gate_floor);", "g = term(go) * (term(zz * s));"),
    ("step map: bias gradient keeps only one token", "ddb_acc += term(ddraw);", "ddb_acc = term(ddraw);"),
    ("state: initial state ignored", "for (int32_t n = 0; n < N; ++n) h[n] = h0 ? h0[((int64_t)s * D + d) * N + n] : 0.0;",
     "for (int32_t n = 0; n < N; ++n) h[n] = 0.0;"),
    ("state: final state transposed", "for (int32_t n = 0; n < N; ++n) hT[((int64_t)s * D + d) * N + n] = h[n];",
     "for (int32_t n = 0; n < N; ++n) hT[((int64_t)s * N + n) * D + d] = h[n];"),
    ("state bwd: final-state gradient ignored", "c[n] = dhT ? term(dhT[((int64_t)s * D + d) * N + n]) : 0.0;",
     "c[n] = 0.0;"),
    ("state bwd: previous state at the head taken as zero",
     "const double hp = (t == cu[s]) ? hinit[n] : hs[(t - 1) * N + n];",
     "const double hp = (t == cu[s]) ? 0.0 : hs[(t - 1) * N + n];"),
    ("state bwd: replay ignores the initial state",
     "const double hp = (t == cu[s]) ? (h0 ? term(h0[((int64_t)s * D + d) * N + n]) : 0.0)",
     "const double hp = (t == cu[s]) ? 0.0"),
    ("state bwd: initial-state gradient for the wrong sequence",
     "for (int32_t n = 0; n < N; ++n) dh0[((int64_t)s * D + d) * N + n] = c[n];",
     "for (int32_t n = 0; n < N; ++n) dh0[((int64_t)(nseq - 1 - s) * D + d) * N + n] = c[n];"),
    ("conv context: oldest and newest swapped", "const int64_t j = i - ((int64_t)cu[s] - (W - 1));",
     "const int64_t j = (int64_t)cu[s] - 1 - i;"),
    ("conv context: final context drops the initial one",
     "conv_input(x, xc0, cu, s, (int64_t)cu[s + 1] - (W - 1) + j, D, W, d);",
     "conv_input(x, NULL, cu, s, (int64_t)cu[s + 1] - (W - 1) + j, D, W, d);"),
    ("conv context bwd: gradient not passed through short sequences",
     "if (dxcT && jt >= 0 && jt < W - 1) acc +=", "if (dxcT && jt >= 0 && jt < W - 1 && i >= a) acc +="),
    ("conv context bwd: dw misses the context",
     "if (t - k < cu[s] && !xc0) continue;\n                    acc += term(gv[t]",
     "if (t - k < cu[s]) continue;\n                    acc += term(gv[t]"),
]


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


# Lines that the reset-only functions and the state-carrying ones share are
# planted in each: (name, text, planted, k) plants in the k-th of exactly two
# occurrences (0: the reset-only function, 1: the state-carrying one).
_SHARED = [
    ("bwd: dA loses the delta factor", "dA_d[n] += term(dh * dt * a * hp);", "dA_d[n] += term(dh * a * hp);"),
    ("bwd: dB misses u", "dB[t * N + n] += term(dh * dt * uu);", "dB[t * N + n] += term(dh * dt);"),
    ("bwd: dC uses the wrong state", "dC[t * N + n] += term(g * hs[t * N + n]);",
     "dC[t * N + n] += term(g * hs[(t > 0 ? t - 1 : t) * N + n]);"),
    ("conv bwd: dw tap index transposed", "dw[(int64_t)d * W + (W - 1 - k)] = acc;", "dw[(int64_t)d * W + k] = acc;"),
    ("gate floor: forward drops it", "acc * (z[t * D + d] * sigmoid(z[t * D + d]) + gate_floor)",
     "acc * (z[t * D + d] * sigmoid(z[t * D + d]))"),
    ("step map: bias gradient keeps only one token", "ddb_acc += term(ddraw);", "ddb_acc = term(ddraw);"),
]
MUTATIONS = [m for m in MUTATIONS if m[1] not in {sh[1] for sh in _SHARED}]
MUTATIONS = [m + (None,) for m in MUTATIONS] + [
    (f"{name} [{which}]", orig, planted, k) for name, orig, planted in _SHARED
    for k, which in ((0, "reset"), (1, "states"))]


@pytest.mark.parametrize("name,orig,planted,nth", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(mutant_dir, name, orig, planted, nth):
    src = open(oracle_mod._SRC).read()
    if nth is None:
        assert src.count(orig) == 1, f"mutation anchor not unique/found: {name}"
        mutated = src.replace(orig, planted)
    else:
        assert src.count(orig) == 2, f"shared anchor not found exactly twice: {name}"
        at = src.index(orig)
        if nth == 1:
            at = src.index(orig, at + 1)
        mutated = src[:at] + planted + src[at + len(orig):]
    idx = MUTATIONS.index((name, orig, planted, nth))
    c_path = os.path.join(mutant_dir, f"m{idx}.c")
    so_path = os.path.join(mutant_dir, f"m{idx}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", c_path, "-o", so_path, "-lm"],
                   check=True)
    mut = oracle_mod.Oracle(so_path)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(mut)
        except AssertionError:
            failed.append(check.__name__)
        except (ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"

"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source to a temporary directory, plants one
mistake (a dropped term, a wrong sign, index or operand) inside one function,
compiles the copy and runs the pins against it: at least one pin must fail.
The committed oracle is never modified.
"""
from __future__ import annotations

import os

import pytest

import oracle
import test_oracle_pins as pins

# (name, function, original text, planted text)
MUTANTS = [
    ("ser: duplicate targets not merged", "oracle_ser_forward",
     "if (cand_m[e] == m) { found = e; break; }", "if (0) { found = e; break; }"),
    ("ser: ties go to the higher index", "oracle_ser_forward",
     "cand_m[e] < cand_m[best]", "cand_m[e] > cand_m[best]"),
    ("ser: leg 2 read at the source row", "oracle_ser_forward",
     "size_t r2 = row(b, j, h, n, hkv);", "size_t r2 = row(b, i, h, n, hkv);"),
    ("ser: path weight summed, not multiplied", "oracle_ser_forward",
     "cand_acc[found] += x * y;", "cand_acc[found] += x + y;"),
    ("ser: zero-weight candidates fill slots", "oracle_ser_forward",
     "if (taken[e] || !(cand_key[e] > 0.0f)) continue;", "if (taken[e]) continue;"),
    ("sea: edge expert (ln w) dropped", "oracle_sea_forward",
     "l[t] = scale * dot + log(wt);", "l[t] = scale * dot;"),
    ("sea: score not scaled", "oracle_sea_forward",
     "l[t] = scale * dot + log(wt);", "l[t] = dot + log(wt);"),
    ("sea: interleaved GQA head mapping", "oracle_sea_forward",
     "int head = h * G + g;", "int head = g * hkv + h;"),
    ("sea: probability reported at the next slot", "oracle_sea_forward",
     "if (pv) pv[t] = p;", "if (pv) pv[(t + 1) % s] = p;"),
    ("sea bwd: softmax backward sign", "oracle_sea_backward",
     "double dl = p[t] * (gt[t] - gbar);", "double dl = p[t] * (gt[t] + gbar);"),
    ("sea bwd: dk without the score scale", "oracle_sea_backward",
     "dk[src + c] += scale * dl * qv[c];", "dk[src + c] += dl * qv[c];"),
    ("sea bwd: dw not divided by w", "oracle_sea_backward",
     "dw[r * s + t] += dl / wt;", "dw[r * s + t] += dl;"),
    ("sea bwd: dv weighted by dl instead of p", "oracle_sea_backward",
     "dv[src + c] += p[t] * dov[c];", "dv[src + c] += dl * dov[c];"),
    ("sea bwd: dq from v instead of k", "oracle_sea_backward",
     "dqv[c] += scale * dl * kv[c];", "dqv[c] += scale * dl * v[src + c];"),
    ("leg: mixing weight dropped", "oracle_leg_mix_forward",
     "cand_acc[found] += alpha[(size_t)h * K + k] * w[r * K + k];",
     "cand_acc[found] += w[r * K + k];"),
    ("leg: mixing weight of the wrong head", "oracle_leg_mix_forward",
     "cand_acc[found] += alpha[(size_t)h * K + k] * w[r * K + k];",
     "cand_acc[found] += alpha[(size_t)(hkv - 1 - h) * K + k] * w[r * K + k];"),
    ("leg bwd: dalpha from the mixing weight", "oracle_leg_mix_backward",
     "dalpha[(size_t)h * K + k] += g * x;", "dalpha[(size_t)h * K + k] += g * a;"),
    ("refresh: ranking by the last head only", "oracle_dense_refresh",
     "for (int j = 0; j <= i; ++j) pbar[j] += exp(sc[j] - mx) / z / G;",
     "for (int j = 0; j <= i; ++j) pbar[j] = exp(sc[j] - mx) / z;"),
    ("refresh: unscaled scores", "oracle_dense_refresh",
     "sc[j] = scale * dot;", "sc[j] = dot;"),
    ("ser bwd: leg operands swapped", "oracle_ser_backward",
     "dw1[r1 * s2 + a] += gt * y;", "dw1[r1 * s2 + a] += gt * x;"),
    ("ser bwd: padding slots of A' pass gradient", "oracle_ser_backward",
     "if (!(w_out[r1 * s1 + t] > 0.0)) continue;", ""),
    ("ser bwd: leg-2 gradient to the source row", "oracle_ser_backward",
     "dw2[r2 * s3 + c] += gt * x;", "dw2[r1 * s3 + c] += gt * x;"),
]

PINS = [
    pins.test_ser_forward_tiny_config_dense,
    lambda o: pins.test_ser_forward_matches_dense_product(o, "mixed"),
    pins.test_ser_forward_pointer_chase_closed_form,
    pins.test_ser_forward_self_loops_closed_form,
    pins.test_ser_forward_invariants,
    pins.test_ser_backward_matches_dense,
    pins.test_ser_backward_finite_differences,
    pins.test_ser_backward_euler_identities,
    pins.test_sea_tiny_config_dense,
    pins.test_sea_forward_backward_match_dense,
    pins.test_sea_single_slot_closed_form,
    pins.test_sea_slot_probabilities_match_dense,
    pins.test_sea_zero_query_closed_form,
    pins.test_sea_constant_values_and_conservation,
    pins.test_sea_finite_differences,
    pins.test_ser_forward_1000_random_small_cases,
    pins.test_leg_mix_matches_dense_mixture,
    pins.test_leg_mix_single_slot_closed_form,
    pins.test_leg_mix_backward_matches_dense_and_differences,
    pins.test_dense_refresh_matches_dense_attention,
]


def _plant(src: str, func: str, old: str, new: str) -> str:
    start = src.index(f"int {func}(")
    end = src.find("\nint oracle_", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) == 1, f"{old!r} not unique in {func}"
    return src[:start] + body.replace(old, new) + src[end:]


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, func, old, new):
    with open(oracle.SRC) as f:
        src = f.read()
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(_plant(src, func, old, new))
    lib = oracle.build(path, os.path.join(tmp_path, "libmutant.so"))
    mutant = oracle.Oracle(lib)
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError):
            return
    pytest.fail(f"no pin caught the planted mistake: {name}")

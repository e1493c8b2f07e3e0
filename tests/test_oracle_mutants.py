"""Strength of the oracle's pins: copies of oracle/dla_oracle.c with one
planted mistake each (a dropped term, a wrong sign, index or tie-break, a
transposed operand) are compiled on the CPU and run through the same pins as
the oracle.  The unmodified source must pass every pin, and every mutant must
fail at least one.  Nothing here touches the GPU or the HIP library."""
import os
import traceback

import pytest

import oracle
from tests import test_oracle as P
from tests import test_oracle_state_score as Q

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dla_oracle.c")

# (name, text in dla_oracle.c, replacement).  Each text occurs exactly once.
MUTANTS = [
    ("score sign flipped",
     "return (float)(1.0 - d / sqrt(ab));", "return (float)(1.0 + d / sqrt(ab));"),
    ("score norm of the wrong key",
     "b += (double)kp[i] * (double)kp[i];", "b += (double)kt[i] * (double)kt[i];"),
    ("score without the square root",
     "return (float)(1.0 - d / sqrt(ab));", "return (float)(1.0 - d / ab);"),
    ("boundary rule with or",
     "!((s < tau) && (s_prev < tau))", "!((s < tau) || (s_prev < tau))"),
    ("boundary rule drops the previous token",
     "!((s < tau) && (s_prev < tau))", "!(s < tau)"),
    ("boundary at equality treated as low",
     "!((s < tau) && (s_prev < tau))", "!((s <= tau) && (s_prev <= tau))"),
    ("information of the previous token",
     "llrint(ldexp((double)s, 32))", "llrint(ldexp((double)s_prev, 32))"),
    ("ties go to the latest pair",
     "if (key < bestkey)", "if (key <= bestkey)"),
    ("largest pair merged",
     "if (key < bestkey)", "if (key > bestkey)"),
    ("merge keys use one state only",
     "int64_t key = I[i] + I[i + 1];", "int64_t key = I[i + 1];"),
    ("merge drops the later state's information",
     "I[best] += I[best + 1];", "(void)0;"),
    ("merge drops the later state's matrix",
     "for (size_t e = 0; e < SS; ++e) Sa[e] += Sb[e];", ""),
    ("merge keeps the later start",
     "/* st[best] is kept", "st[best] = st[best + 1]; /*"),
    ("merge drops the later state's count",
     "n[best] += n[best + 1];", "(void)0;"),
    ("merging one state early",
     "if (m > C) {", "if (m >= C && m > 1) {"),
    ("joining token's information dropped",
     "I[m - 1] += qs;", "(void)qs;"),
    ("joining token added to the oldest state",
     "double *Sl = S + (size_t)(m - 1) * SS;", "double *Sl = S;"),
    ("new state transposed",
     "Sn[(size_t)r * dk + c] = (double)vt[r] * (double)kt[c];",
     "Sn[(size_t)c * dv + r] = (double)vt[r] * (double)kt[c];"),
    ("joining update transposed",
     "Sl[(size_t)r * dk + c] += (double)vt[r] * (double)kt[c];",
     "Sl[(size_t)c * dv + r] += (double)vt[r] * (double)kt[c];"),
    ("read oldest state first",
     "const double *Sj = S + (size_t)(m - 1 - j) * SS;", "const double *Sj = S + (size_t)j * SS;"),
    ("read weights by the wrong slot",
     "const double w = (double)lt[j];", "const double w = (double)lt[m - 1 - j];"),
    ("read with the key instead of the query",
     "acc += Sj[(size_t)r * dk + c] * (double)qt[c];", "acc += Sj[(size_t)r * dk + c] * (double)kt[c];"),
    ("read drops the weight",
     "ot[r] += w * acc;", "ot[r] += acc;"),
    ("start counted from one",
     "st[m] = t_seen;", "st[m] = t_seen + 1;"),
    ("density ties go to the latest pair",
     "if (num * bden < bnum * den)", "if (num * bden <= bnum * den)"),
    ("density compares the numerators only",
     "if (num * bden < bnum * den)", "if (num < bnum)"),
    ("density cross-multiplied the wrong way",
     "if (num * bden < bnum * den)", "if (num * den < bnum * bden)"),
    ("density counts one state of the pair",
     "den = (__int128)n[i] + n[i + 1];", "den = (__int128)n[i];"),
    ("density rule ignored",
     "if (A->merge_rule == 1) {", "if (0) {"),
    # the state information score
    ("state score without the normalisation",
     "const double ra = sqrt(a2 / D), rc = sqrt(c2 / D);", "const double ra = 1.0, rc = 1.0;"),
    ("state score against the oldest state",
     "m > 0 ? S + (size_t)(m - 1) * SS : NULL", "m > 0 ? S : NULL"),
    ("state score drops the current state from the numerator",
     "diff += (na - ns) * (na - ns);", "diff += na * na;"),
    ("state score with a reversed key index",
     "const double na = (double)vt[r] * (double)kt[c] / ra;",
     "const double na = (double)vt[r] * (double)kt[dk - 1 - c] / ra;"),
    ("state score with eps = 1",
     "return (float)(sqrt(diff) / (sqrt(nc) + 1e-6));", "return (float)(sqrt(diff) / (sqrt(nc) + 1.0));"),
    ("state score of an empty cache is 1",
     "if (!Sc) return 2.0f;", "if (!Sc) return 1.0f;"),
    ("state score of a zero matrix is 0",
     "if (a2 == 0.0 || c2 == 0.0) return 2.0f;", "if (a2 == 0.0 || c2 == 0.0) return 0.0f;"),
    ("state boundary at equality treated as low",
     "bnd = (m == 0) || (s >= tau);", "bnd = (m == 0) || (s > tau);"),
    ("state rule keeps the two-low boundary rule",
     "bnd = (m == 0) || (s >= tau);", "bnd = (m == 0) || !((s < tau) && (s_prev < tau));"),
    ("state rule ignored",
     "if (A->score_rule == 1) {", "if (0) {"),
]


def _battery():
    """(name, thunk(lib)) for every pin, at fixed parameters."""
    out = [("score closed forms", P.pin_score_closed_forms)]
    for case in P._golden():
        out.append((f"golden {case['name']}", lambda lib, c=case: P.pin_hand_derived_schedule(c, lib)))
    for args in [(70, 4, 3, 3, 0.3, 8, 1), (60, 8, 8, 2, 0.3, 2, 2), (50, 2, 1, 4, 0.9, 1000, 3),
                 (64, 8, 3, 5, -1.0, 8, 4), (40, 4, 8, 1, 3.0, 2, 5), (70, 8, 8, 6, 0.3, 8, 6)]:
        out.append((f"brute force {args}", lambda lib, a=args: P.pin_brute_force_and_greedy(*a, lib=lib)))
    for args in [(90, 4, 3, 3, 0.3, 8, 7), (80, 8, 2, 4, 0.3, 30, 8), (60, 4, 1, 2, -1.0, 2, 9)]:
        out.append((f"density brute force {args}",
                    lambda lib, a=args: P.pin_brute_force_and_greedy(*a, lib=lib, merge_rule="density")))
    for tau, C in [(0.3, 3), (-1.0, 2)]:
        out.append((f"lambda one {tau} {C}", lambda lib, t=tau, c=C: P.pin_lambda_one(t, c, lib)))
    out.append(("single state", lambda lib: P.pin_single_state(0.3, lib)))
    out.append(("dense slot weighted", P.pin_dense_slot_weighted))
    out.append(("prefix sum", P.pin_prefix_sum))
    for args in [(120, 4, 3, 3, 0.3, 1), (100, 6, 6, 2, 0.3, 2), (80, 8, 5, 5, 0.15, 3)]:
        out.append((f"state score closed form {args}", lambda lib, a=args: Q.pin_state_closed_form(*a, lib=lib)))
    out.append(("state score special cases", Q.pin_state_special_cases))
    for case in Q._golden():
        out.append((f"state golden {case['name']}", lambda lib, c=case: Q.pin_state_golden(c, lib)))
    out.append(("state continuation", Q.pin_state_continuation))
    return out


def _failing_pins(lib):
    failed = []
    for name, pin in _battery():
        try:
            pin(lib)
        except AssertionError:
            failed.append(name)
    return failed


def _compile(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    return oracle.load_library(oracle.build(src=str(src), out=str(tmp_path / f"{name}.so")))


def test_unmodified_source_passes_every_pin(tmp_path):
    lib = _compile(tmp_path, "control", open(SRC).read())
    assert _failing_pins(lib) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    lib = _compile(tmp_path, "mutant", text.replace(old, new))
    try:
        failed = _failing_pins(lib)
    except Exception:                       # a crash of the mutant also counts as caught
        failed = ["raised: " + traceback.format_exc(limit=1)]
    assert failed, f"no pin catches the planted mistake '{name}'"

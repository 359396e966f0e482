"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case rewrites one line of an oracle function's source (a dropped term,
a wrong sign, a wrong reduction, the wrong logarithm), executes the mutant
in a scratch namespace and checks that at least one pin now fails. The real
oracle is never modified.
"""
import inspect
import math
import textwrap

import numpy as np
import pytest

from oracle import calibration as oc
from oracle import skip_softmax as osk
from synth import CONFIGS, bf16_bits_to_f32, make_inputs


def _mutant(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(vars(inspect.getmodule(fn)))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[fn.__name__]


@pytest.fixture(scope="module")
def small():
    cfg = CONFIGS["tiny"]
    x = make_inputs(cfg)
    f = {n: bf16_bits_to_f32(x[n][:256, :1]).astype(np.float64)[:, 0] for n in ("q", "k", "v")}
    return f


def _pins_hold(qblock_fn, f, golden):
    """Forward pins, applied to a (possibly mutated) Q-block function."""
    g = golden("two_tile_example.txt")
    q2, k2, v2 = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    for lam, skip in ((g["lambda_keep"], False), (g["lambda_skip"], True)):
        r = qblock_fn(q2, k2, v2, math.log2(lam), 2, math.log(2.0))
        want = np.array(g["o_skip"]) if skip else np.array(g["o_keep_num"]) / np.array(g["o_keep_den"])
        if bool(r["skip"][1]) != skip or not np.allclose(r["o"], want, atol=1e-12, rtol=0):
            return False
    scale = osk.default_sm_scale(64)
    exact = osk.attention_exact(f["q"], f["k"], f["v"], scale)
    for i in range(4):
        qb = f["q"][64 * i:64 * (i + 1)]
        dense = qblock_fn(qb, f["k"], f["v"], float("-inf"), 64, scale)
        if not np.allclose(dense["o"], exact[64 * i:64 * (i + 1)], atol=1e-10, rtol=0):
            return False
        for lam in (1e-3, 1e-1, 1.0):
            seq = qblock_fn(qb, f["k"], f["v"], math.log2(lam), 64, scale)
            fast = osk.skip_softmax_qblock_fast(qb, f["k"], f["v"], math.log2(lam), 64, scale)
            if not np.array_equal(seq["skip"], fast["skip"]) or not np.allclose(seq["o"], fast["o"], atol=1e-12):
                return False
    return True


def test_real_oracle_passes_the_pins(small, golden):
    assert _pins_hold(osk.skip_softmax_qblock, small, golden)


@pytest.mark.parametrize("old,new", [
    ("d = float(np.max(rowmax - m))", "d = float(np.min(rowmax - m))"),       # any-row vote
    ("d = float(np.max(rowmax - m))", "d = float(np.max(m - rowmax))"),       # sign flip
    ("skip = d < t", "skip = d <= t + 1.0"),                                  # wrong comparison
    ("alpha = np.exp2(m - m_new)", "alpha = np.exp2(m_new - m)"),             # rescale sign
    ("l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),               # dropped rescale
    ("p = np.exp2(s - m_new[:, None])", "p = np.exp(s - m_new[:, None])"),    # wrong base
    ("s = (qb @ k[j0:j1].T) * c", "s = (qb @ k[j0:j1].T) * sm_scale"),        # natural-log scores
])
def test_forward_mutants_are_caught(small, golden, old, new):
    assert not _pins_hold(_mutant(osk.skip_softmax_qblock, old, new), small, golden)


def test_fast_form_prefix_mutant_is_caught(small):
    bad = _mutant(osk.tile_stats_fast, "np.maximum.accumulate(tile_max, axis=1)[:, :-1]",
                  "np.maximum.accumulate(tile_max, axis=1)[:, 1:]")
    scale = osk.default_sm_scale(64)
    qb = small["q"][:64]
    d_ref = osk.skip_softmax_qblock(qb, small["k"], small["v"], -np.inf, 64, scale)["d"]
    d_bad, _ = bad(qb, small["k"], 64, scale)
    assert not np.allclose(d_ref, d_bad)


@pytest.mark.parametrize("old,new", [
    ("y = np.log(lam[use] * sk[use])", "y = np.log(lam[use])"),               # forgot seq_k
    ("b = float(np.sum((x - xm) * (y - ym)) / np.sum((x - xm) ** 2))",
     "b = float(np.sum((x - xm) * (y - ym)) / np.sum((y - ym) ** 2))"),      # swapped regression
])
def test_fit_mutants_are_caught(old, new):
    bad = _mutant(oc.fit_exponential_logspace, old, new)
    a, b, seq_k = 7.93, 8.61, 75600
    s = np.linspace(0.35, 0.85, 12)
    f = bad(a * np.exp(b * s) / seq_k, s, seq_k)
    assert not (math.isclose(f.a, a, rel_tol=1e-9) and math.isclose(f.b, b, rel_tol=1e-9))


def test_resolve_natural_log_mutant_is_caught(golden):
    g = golden("threshold_anchors.txt")
    bad = _mutant(oc.resolve_threshold, "return OK, 2.0 ** r, r", "return OK, math.exp(r), r")
    _, lam, _ = bad(oc.ThresholdSpec(raw_log2=g["raw_log2_example"]), 75600)
    assert abs(lam - g["fixed_lambda_example"]) > g["example_abs_tol"]

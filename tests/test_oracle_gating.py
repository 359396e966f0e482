"""Pins of the gating oracle (oracle/gating.py) against the pages."""
import numpy as np

from oracle import gating as og


def test_printed_schedule_table(golden):
    g = golden("unipc_40_steps.txt")
    t = og.flow_timesteps(int(g["n_steps"]), int(g["num_train_timesteps"]), g["flow_shift"])
    assert t.shape == (40,)
    assert np.all(np.diff(t) < 0) and t[0] < 1.0 and t[-1] > 0.0
    for c, d, k in zip(g["cutoffs"][0], g["dense_steps"][0], g["skip_steps"][0]):
        assert og.dense_steps(t, c) == int(d)
        assert 40 - og.dense_steps(t, c) == int(k)


def test_printed_example_timesteps(golden):
    g = golden("unipc_40_steps.txt")
    t = og.flow_timesteps(40, 1000, 3.0)
    assert abs(t[13] - g["t13_approx"]) <= g["approx_tol"]
    assert abs(t[14] - g["t14_approx"]) <= g["approx_tol"]
    # the cutoff 0.86 falls between them: 14 dense steps (i = 0 .. 13)
    assert t[13] >= 0.86 > t[14]


def test_shift_reduces_to_the_printed_form():
    # shift 3: shifted = 3 s / (1 + 2 s); shift 1 leaves the sigma unshifted
    T, n = 1000, 40
    s = 1.0 - np.arange(n) * (1.0 - 1.0 / T) / n
    keep = 1.0 - 1.0 / T
    assert np.allclose(og.flow_timesteps(n, T, 3.0) / keep, 3 * s / (1 + 2 * s), rtol=0, atol=1e-15)
    assert np.allclose(og.flow_timesteps(n, T, 1.0) / keep, s, rtol=0, atol=1e-15)


def test_other_conversions_fail_the_table(golden):
    # t = shifted sigma (no conversion) contradicts the printed rows for cutoffs 1.00 and 0.90
    g = golden("unipc_40_steps.txt")
    s = 1.0 - np.arange(40) * 0.999 / 40
    t_plain = 3 * s / (1 + 2 * s)
    got = [og.dense_steps(t_plain, c) for c in g["cutoffs"][0]]
    assert got != [int(d) for d in g["dense_steps"][0]]


def test_dense_steps_edges():
    t = og.flow_timesteps(40)
    assert og.dense_steps(t, None) == 0
    assert og.dense_steps(t, 0.0) == 40       # 0.0 is a cutoff, not "no cutoff"
    assert og.dense_steps([0.5, 0.5], 0.5) == 2  # equality is dense


def test_layer_matching_examples():
    # "blocks.0.attn1 matches transformer.blocks.0.attn1 and transformer_2.blocks.0.attn1"
    for name in ("transformer.blocks.0.attn1", "transformer_2.blocks.0.attn1", "blocks.0.attn1"):
        assert og.layer_matches(name, "blocks.0.attn1")
    assert not og.layer_matches("transformer.blocks.10.attn1", "blocks.0.attn1")
    assert not og.layer_matches("transformer.blocks.0.attn2", "blocks.0.attn1")
    assert og.layer_matches("transformer_blocks.0.attn", "transformer_blocks.0*")
    assert og.layer_matches("single_transformer_blocks.7.attn", "single_transformer_blocks*")
    assert not og.layer_matches("Transformer.blocks.0.attn1", "transformer.blocks.0.attn1")


def test_gate_rule_order():
    ign = ["blocks.0.attn1", "blocks.0.attn2"]
    ovr = [("transformer_blocks.0*", 0.0), ("single_transformer_blocks*", 8000.0), ("single_*", 1.0)]
    # timestep cutoff wins over everything; per-token timesteps reduce to their max
    assert og.gate_layer("x.blocks.5.attn1", [0.1, 0.85], 5000.0, cutoff=0.8) == (og.RULE_TIMESTEP, 0.0)
    assert og.gate_layer("x.blocks.5.attn1", [0.1, 0.79], 5000.0, cutoff=0.8) == (og.RULE_BASE, 5000.0)
    assert og.gate_layer("x.blocks.5.attn1", [0.8], 5000.0, cutoff=0.8) == (og.RULE_TIMESTEP, 0.0)
    # ignore before overrides
    assert og.gate_layer("transformer.blocks.0.attn1", [0.5], 5000.0, cutoff=0.8, ignore=ign,
                         overrides=[("*", 7.0)]) == (og.RULE_IGNORED, 0.0)
    # first matching override
    assert og.gate_layer("single_transformer_blocks.3.attn", [0.5], 5000.0, overrides=ovr) == (og.RULE_OVERRIDE, 8000.0)
    assert og.gate_layer("transformer_blocks.0.attn", [0.5], 5000.0, overrides=ovr) == (og.RULE_OVERRIDE, 0.0)
    assert og.gate_layer("transformer_blocks.1.attn", [0.5], 5000.0, overrides=ovr) == (og.RULE_BASE, 5000.0)
    assert og.gate_layer("a.b", [1.0], 3.0) == (og.RULE_BASE, 3.0)  # no cutoff: never disabled

"""Pins of the fp64 oracle's forward (CPU only).

Each test checks the oracle against something other than itself: the
textbook softmax definition and torch's CPU SDPA at lambda = 0, a hand-worked
two-tile example, brute-force agreement of two differently-built forms, and
the probability bounds the skip rule implies.
"""
import math

import numpy as np
import pytest
import torch

from oracle import skip_softmax as osk
from synth import CONFIGS, bf16_bits_to_f32, make_inputs
from synth.video_tokens import make_random_inputs

INF = float("inf")


@pytest.fixture(scope="module")
def tiny():
    cfg = CONFIGS["tiny"]
    x = make_inputs(cfg)
    return cfg, {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}, x["cu_seqlens"]


def _sdpa_fp64(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    return out[0, 0].numpy()


def test_dense_is_exact_softmax_and_never_skips(tiny):
    cfg, x, cu = tiny
    res = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block)
    assert res["skipped"].sum() == 0
    assert res["total"].sum() == cfg.num_heads * (1024 // 64) ** 2
    scale = osk.default_sm_scale(cfg.head_dim)
    for h in range(cfg.num_heads):
        ref_np = osk.attention_exact(x["q"][:, h], x["k"][:, h], x["v"][:, h], scale)
        ref_t = _sdpa_fp64(x["q"][:, h], x["k"][:, h], x["v"][:, h], scale)
        np.testing.assert_allclose(res["o"][:, h], ref_t, atol=1e-10, rtol=0)
        np.testing.assert_allclose(ref_np, ref_t, atol=1e-12, rtol=0)


def test_two_tile_worked_example(golden):
    g = golden("two_tile_example.txt")
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    scale = math.log(2.0)
    for lam, skip in ((g["lambda_keep"], False), (g["lambda_skip"], True)):
        r = osk.skip_softmax_qblock(q, k, v, math.log2(lam), 2, scale)
        assert r["d"][1] == pytest.approx(g["d_tile1"], abs=1e-12)
        assert bool(r["skip"][0]) is False
        assert bool(r["skip"][1]) is skip
        if skip:
            want = np.array(g["o_skip"])
        else:
            want = np.array(g["o_keep_num"]) / np.array(g["o_keep_den"])
        np.testing.assert_allclose(r["o"], want, atol=1e-12, rtol=0)


@pytest.mark.parametrize("lam", [1e-6, 1e-3, 1e-1, 0.7, 1.0])
def test_sequential_equals_fast_form(tiny, lam):
    cfg, x, cu = tiny
    t = math.log2(lam)
    seq = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block)
    fast = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block, fast=True)
    np.testing.assert_array_equal(seq["mask"], fast["mask"])
    np.testing.assert_allclose(seq["d"], fast["d"], atol=1e-9, rtol=0)
    np.testing.assert_allclose(seq["o"], fast["o"], atol=1e-12, rtol=0)


def test_skip_sets_nested_and_counts_monotone(tiny):
    cfg, x, cu = tiny
    lams = np.geomspace(1e-6, 1.0, 9)
    prev_mask, prev_count = None, -1
    for lam in lams:
        r = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, math.log2(lam), cfg.block, fast=True)
        m = r["mask"] == osk.TILE_SKIPPED
        if prev_mask is not None:
            assert np.all(m[prev_mask]), "skip set not nested"
        assert r["skipped"].sum() >= prev_count
        prev_mask, prev_count = m, r["skipped"].sum()
    assert prev_count > 0
    # the first KV tile of every Q-block is never skipped, even at lambda = 1
    assert np.all(prev_mask[..., 0] == False)  # noqa: E712


@pytest.mark.parametrize("lam", [1e-3, 1e-1, 1.0])
def test_dropped_probability_and_output_bounds(tiny, lam):
    """Every skipped score has exact softmax probability < lambda, and the
    output moves by at most 2 * (dropped mass) * max|V| per row."""
    cfg, x, cu = tiny
    scale = osk.default_sm_scale(cfg.head_dim)
    r = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, math.log2(lam), cfg.block)
    B = cfg.block
    worst = 0.0
    for h in range(cfg.num_heads):
        qh, kh, vh = x["q"][:, h], x["k"][:, h], x["v"][:, h]
        z = (qh @ kh.T) * scale
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        cols_skipped = np.repeat(r["mask"][0, h] == osk.TILE_SKIPPED, B, axis=1).repeat(B, axis=0)
        dropped = np.where(cols_skipped, p, 0.0)
        worst = max(worst, dropped.max())
        assert dropped.max() < lam
        delta = dropped.sum(1)
        exact = p @ vh
        dev = np.abs(r["o"][:, h] - exact).max(1)
        assert np.all(dev <= 2 * delta * np.abs(vh).max() + 1e-12)
    assert worst > 0.0


def test_ragged_batch_with_empty_sequence_dense():
    lens = [1, 63, 0, 65, 200]
    x = make_random_inputs(lens, 3, 64, seed=11)
    f = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    cu = x["cu_seqlens"]
    res = osk.skip_softmax_forward(f["q"], f["k"], f["v"], cu, -INF, 64)
    scale = osk.default_sm_scale(64)
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        for h in range(3):
            if s1 == s0:
                continue
            ref = _sdpa_fp64(f["q"][s0:s1, h], f["k"][s0:s1, h], f["v"][s0:s1, h], scale)
            np.testing.assert_allclose(res["o"][s0:s1, h], ref, atol=1e-10, rtol=0)
    assert res["total"][2].sum() == 0
    assert np.array_equal(res["total"][:, 0], [1, 1, 0, 4, 16])


def test_forced_mask_reproduces_decisions(tiny):
    cfg, x, cu = tiny
    t = math.log2(1e-2)
    r = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block)
    f = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block, forced_mask=r["mask"])
    np.testing.assert_array_equal(r["mask"], f["mask"])
    np.testing.assert_array_equal(r["o"], f["o"])


def test_fast_form_equals_sequential_under_forced_masks(tiny):
    """Under any forced decisions (first tile kept) both forms compute the
    softmax restricted to the kept tiles' keys: the sequential loop through
    its rescaled running sums, the fast form directly. Random masks include
    decisions the threshold would never take (a row's maximum tile skipped),
    so the equality does not lean on the lambda <= 1 lemma."""
    cfg, x, cu = tiny
    rng = np.random.default_rng(5)
    full = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block)
    for _ in range(3):
        forced = full["mask"].copy()
        real = forced != osk.TILE_NONE
        draw = rng.random(forced.shape) < 0.5
        forced[real & draw] = osk.TILE_SKIPPED
        forced[..., 0] = np.where(forced[..., 0] == osk.TILE_NONE, osk.TILE_NONE, osk.TILE_KEPT)
        seq = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block, forced_mask=forced)
        fast = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block, forced_mask=forced,
                                        fast=True)
        np.testing.assert_array_equal(seq["mask"], forced)
        np.testing.assert_allclose(seq["o"], fast["o"], atol=1e-12, rtol=0)
        # and both equal the textbook softmax over the kept keys, written out directly
        scale = osk.default_sm_scale(x["q"].shape[2])
        for h in range(x["q"].shape[1]):
            for i in range(forced.shape[2]):
                keep = np.repeat(forced[0, h, i] == osk.TILE_KEPT, cfg.block)
                rows = slice(i * cfg.block, (i + 1) * cfg.block)
                z = x["q"][rows, h] @ x["k"][:, h].T * scale
                z = np.where(keep[None, :], z, -np.inf)
                p = np.exp(z - z.max(1, keepdims=True))
                want = (p @ x["v"][:, h]) / p.sum(1, keepdims=True)
                np.testing.assert_allclose(seq["o"][rows, h], want, atol=1e-12, rtol=0)

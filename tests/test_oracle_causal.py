"""Pins of the oracle's causal (prefill) form (CPU only)."""
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


def _sdpa_causal_fp64(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale, is_causal=True)
    return out[0, 0].numpy()


def test_causal_dense_is_exact_causal_softmax(tiny):
    cfg, x, cu = tiny
    res = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block, causal=True)
    nq = 1024 // cfg.block
    assert res["skipped"].sum() == 0
    assert np.all(res["total"] == nq * (nq + 1) // 2)
    scale = osk.default_sm_scale(cfg.head_dim)
    for h in range(cfg.num_heads):
        ref_t = _sdpa_causal_fp64(x["q"][:, h], x["k"][:, h], x["v"][:, h], scale)
        ref_np = osk.attention_exact(x["q"][:, h], x["k"][:, h], x["v"][:, h], scale, causal=True)
        np.testing.assert_allclose(res["o"][:, h], ref_t, atol=1e-10, rtol=0)
        np.testing.assert_allclose(ref_np, ref_t, atol=1e-12, rtol=0)
    # tiles beyond the causal triangle are not visited
    m = res["mask"][0, 0]
    assert np.all(m[np.triu_indices(nq, 1)] == osk.TILE_NONE)
    assert np.all(m[np.tril_indices(nq)] == osk.TILE_KEPT)


def test_causal_ragged_dense():
    lens = [1, 63, 0, 65, 200]
    x = make_random_inputs(lens, 2, 64, seed=12)
    f = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    cu = x["cu_seqlens"]
    res = osk.skip_softmax_forward(f["q"], f["k"], f["v"], cu, -INF, 64, causal=True)
    scale = osk.default_sm_scale(64)
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        for h in range(2):
            if s1 == s0:
                continue
            ref = _sdpa_causal_fp64(f["q"][s0:s1, h], f["k"][s0:s1, h], f["v"][s0:s1, h], scale)
            np.testing.assert_allclose(res["o"][s0:s1, h], ref, atol=1e-10, rtol=0)
    assert np.array_equal(res["total"][:, 0], [1, 1, 0, 3, 10])


@pytest.mark.parametrize("lam", [1e-4, 1e-2, 0.5, 1.0])
def test_causal_sequential_equals_fast_form(tiny, lam):
    cfg, x, cu = tiny
    t = math.log2(lam)
    seq = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block, causal=True)
    fast = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block, fast=True, causal=True)
    np.testing.assert_array_equal(seq["mask"], fast["mask"])
    np.testing.assert_allclose(seq["d"], fast["d"], atol=1e-9, rtol=0)
    np.testing.assert_allclose(seq["o"], fast["o"], atol=1e-12, rtol=0)
    assert seq["skipped"].sum() > 0 or lam < 1e-3


@pytest.mark.parametrize("lam", [1e-2, 1.0])
def test_causal_dropped_probability_bound(tiny, lam):
    cfg, x, cu = tiny
    scale = osk.default_sm_scale(cfg.head_dim)
    r = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, math.log2(lam), cfg.block, causal=True)
    B = cfg.block
    for h in range(cfg.num_heads):
        qh, kh, vh = x["q"][:, h], x["k"][:, h], x["v"][:, h]
        z = (qh @ kh.T) * scale
        z = np.where(np.tril(np.ones(z.shape, bool)), z, -np.inf)
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        cols_skipped = np.repeat(r["mask"][0, h] == osk.TILE_SKIPPED, B, axis=1).repeat(B, axis=0)
        dropped = np.where(cols_skipped, p, 0.0)
        assert dropped.max() < lam
        dev = np.abs(r["o"][:, h] - p @ vh).max(1)
        assert np.all(dev <= 2 * dropped.sum(1) * np.abs(vh).max() + 1e-12)


def test_causal_calibration_counts_equal_forward(tiny):
    cfg, x, cu = tiny
    lams = np.geomspace(1e-5, 0.7, 6)
    cal = osk.calibration_counts(x["q"], x["k"], x["v"], cu, np.log2(lams), cfg.block, causal=True)
    for kk, lam in enumerate(lams):
        fwd = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, math.log2(lam), cfg.block, causal=True)
        per_wg = [(fwd["mask"][b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in cal["wg"]]
        np.testing.assert_array_equal(cal["counts"][:, kk], per_wg)
    assert np.array_equal(cal["tiles"], [i + 1 for (_, _, i) in cal["wg"]])


def test_diagonal_off_by_one_is_caught(tiny, monkeypatch):
    """A planted mistake (each query also masks itself) fails the causal SDPA pin."""
    cfg, x, cu = tiny
    orig = osk._causal_mask

    def wrong(s, row0, col0):
        if row0 is None:
            return s
        rows = row0 + np.arange(s.shape[0])[:, None]
        cols = col0 + np.arange(s.shape[1])[None, :]
        return np.where(cols < rows, s, np.where(cols == rows, s - 50.0, -np.inf))

    monkeypatch.setattr(osk, "_causal_mask", wrong)
    res = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block, causal=True)
    ref = _sdpa_causal_fp64(x["q"][:, 0], x["k"][:, 0], x["v"][:, 0], osk.default_sm_scale(cfg.head_dim))
    assert np.abs(res["o"][:, 0] - ref).max() > 1e-3
    monkeypatch.setattr(osk, "_causal_mask", orig)

"""Helpers for GPU-vs-oracle parity tests (not collected by pytest).

The GPU side is reached only through the C-ABI binding; the oracle side only
through `oracle/`; both consume the same `synth` bf16 inputs.
"""
from __future__ import annotations

import math
import os
import sys
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

from oracle import skip_softmax as osk
from synth import bf16_bits_to_f32

# Tolerances: skip bits exact outside a +-1e-3 (log2 units) band around the
# threshold; outputs within max-abs 2e-2 / mean-abs 2e-3 of the fp64 oracle
# run on the same bf16-rounded inputs.
MARGIN_BAND = 1e-3
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def gpu_forward(xd: Dict, cu, threshold, kind: str, block: int, mask: bool = True, causal: bool = False,
                block_scales=None, sm_scale: float = 0.0):
    """Run ssa_attn_fwd; return (o fp32 numpy [T,H,D], skipped [B,H], total [B,H], mask or None).
    `block_scales` = (q scales, k scales) selects block-scaled e4m3 q/k."""
    import torch
    import skip_softmax_video_amd as ssa
    B = len(cu) - 1
    T, H, D = xd["q"].shape
    skipped = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    total = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    tm = None
    if mask:
        prob, _ = ssa.make_problem(xd["q"], cu, block)
        nq, nk = ssa.tile_mask_dims(prob)
        tm = torch.empty((B, H, nq, nk), dtype=torch.uint8, device="cuda")
    o = ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, threshold, kind=kind, block=block, sm_scale=sm_scale,
                     skipped=skipped, total=total, tile_mask=tm, causal=causal, block_scales=block_scales)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), skipped.cpu().numpy().reshape(B, H), total.cpu().numpy().reshape(B, H),
            None if tm is None else tm.cpu().numpy())


def t_matrix(cu, H: int, threshold, kind: str) -> np.ndarray:
    """[B, H] log2 thresholds as the oracle reads them (fp64)."""
    B = len(cu) - 1
    vals = np.broadcast_to(np.atleast_1d(np.asarray(threshold, np.float64)), (H,))
    t = np.empty((B, H))
    for b in range(B):
        S = int(cu[b + 1] - cu[b])
        for h in range(H):
            v = float(vals[h])
            if kind == "lambda":
                lam = v
            elif kind == "scale_factor":
                lam = 0.0 if S == 0 else v / S
            else:
                t[b, h] = v
                continue
            t[b, h] = -math.inf if lam == 0 else math.log2(lam)
    return t


def compare_masks(gpu_mask: np.ndarray, ref: Dict, t_bh: np.ndarray, qblocks: Iterable[Tuple[int, int, int]]):
    """Skip bits must agree except where the oracle margin |d - t| <= MARGIN_BAND.

    Returns the number of band tiles and of band mismatches (reported, allowed).
    """
    band = mism = 0
    for (b, h, i) in qblocks:
        g = gpu_mask[b, h, i]
        r = ref["mask"][b, h, i]
        valid = r != osk.TILE_NONE
        assert np.all(g[~valid] == osk.TILE_NONE), f"tile mask written beyond the sequence at {(b, h, i)}"
        with np.errstate(invalid="ignore"):
            near = np.abs(ref["d"][b, h, i] - t_bh[b, h]) <= MARGIN_BAND
        bad = (g != r) & valid
        band += int(np.sum(near & valid))
        mism += int(np.sum(bad & near))
        hard = bad & ~near
        assert not np.any(hard), (f"skip decision mismatch outside the margin band at (b,h,i)={(b, h, i)} "
                                  f"tiles {np.nonzero(hard)[0][:8]} d={ref['d'][b, h, i][hard][:8]} t={t_bh[b, h]}")
    return band, mism


def compare_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, rows: Optional[np.ndarray] = None):
    """max-abs / mean-abs of the GPU output against the oracle over computed rows."""
    sel = ~np.isnan(o_ref)
    diff = np.abs(o_gpu[sel] - o_ref[sel])
    assert diff.size > 0
    mx, mean = float(diff.max()), float(diff.mean())
    assert np.all(np.isfinite(o_gpu[sel])), "non-finite GPU output"
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, f"output mismatch: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def compare_outputs_derived(o_gpu: np.ndarray, o_ref: np.ndarray, vmax: float, v_scale: float):
    """Output check for inputs whose V is drawn at scale `v_scale` (N(0, v_scale^2))
    and whose sharp rows push |O| up to max|V|, beyond the unit-scale video
    workloads the 2e-2 / 2e-3 bounds are stated for. Bound per element:
    - the bf16 rounding of P (2^-9 relative, times max|V|);
    - plus the rounding of O (2^-9 relative);
    - plus accumulation noise; each rounding term is taken twice for margin.
    Every error term is relative to V's magnitude, so the mean-abs bound is the
    stated 2e-3 times v_scale."""
    sel = ~np.isnan(o_ref)
    diff = np.abs(o_gpu[sel] - o_ref[sel])
    tol = 2.0 ** -8 * vmax + 2.0 ** -8 * np.abs(o_ref[sel]) + 1e-3
    assert np.all(np.isfinite(o_gpu[sel])), "non-finite GPU output"
    assert np.all(diff <= tol), f"output outside the derived bound: max-abs {diff.max():.3e}"
    assert diff.mean() <= O_MEAN_ABS * v_scale, f"mean-abs {diff.mean():.3e}"
    return float(diff.max()), float(diff.mean())


# ---- full-size oracle fixtures (tests/golden/fullsize_*.npz) ---------------------------
# Written by tests/golden/make_fullsize_fixtures.py, which calls only oracle/ and synth.
GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")


def load_fixture(name: str) -> Dict[str, np.ndarray]:
    with np.load(os.path.join(GOLDEN, f"fullsize_{name}.npz")) as z:
        return {k: z[k] for k in z.files}


def mask_workgroup_stats(mask: np.ndarray, cu, H: int, block: int) -> np.ndarray:
    """[n_wg, 3] int64 per work-group (the library's row order: sequence, head,
    Q-block): skipped tiles, sum of their indices j and of j^2, from a tile mask."""
    rows = []
    for b in range(len(cu) - 1):
        n = osk.n_tiles(int(cu[b + 1] - cu[b]), block)
        if n == 0:
            continue
        m = mask[b, :, :n, :n]
        assert np.all(m != osk.TILE_NONE), "a visited tile is marked as absent"
        sk = (m == osk.TILE_SKIPPED).astype(np.int64)
        j = np.arange(n, dtype=np.int64)
        rows.append(np.stack([sk.sum(-1), sk @ j, sk @ (j * j)], axis=-1).reshape(H * n, 3))
    return np.concatenate(rows)


def compare_workgroup_stats(stats: np.ndarray, fx: Dict[str, np.ndarray], col: int) -> Dict[str, int]:
    """GPU per-work-group skip statistics against fixture column `col`.

    A work-group with no tile in the decision band must match the oracle in
    count, sum j and sum j^2 (its skip bits tile for tile, barring a
    coincidence of all three sums); elsewhere the counts may differ by at most
    the number of band tiles."""
    band = fx["band"][:, col].astype(np.int64)
    sc = list(fx["sum_cols"]).index(col)
    want = np.stack([fx["count"][:, col], fx["sum_j"][:, sc], fx["sum_j2"][:, sc]], axis=-1).astype(np.int64)
    assert stats.shape == want.shape, f"{stats.shape} work-groups vs the fixture's {want.shape}"
    exact = band == 0
    off = exact & np.any(stats != want, axis=1)
    assert not off.any(), (f"{int(off.sum())} band-free work-groups differ from the oracle, e.g. row "
                           f"{int(np.nonzero(off)[0][0])}: gpu {stats[off][0]} oracle {want[off][0]}")
    diff = np.abs(stats[:, 0] - want[:, 0])
    over = diff > band
    assert not over.any(), f"count differs beyond the band at rows {np.nonzero(over)[0][:8]}"
    return {"band_workgroups": int((~exact).sum()), "band_tiles": int(band.sum()), "flipped": int(diff.sum())}


def compare_calibration_counts(counts: np.ndarray, tiles: np.ndarray, fx: Dict[str, np.ndarray],
                               cols: Sequence[int]) -> Dict[str, int]:
    """Calibration counts [n_wg, len(cols)] against the fixture columns: exact
    where no tile of the work-group lies in the band, else within the band."""
    np.testing.assert_array_equal(tiles, fx["tiles"])
    band = fx["band"][:, cols].astype(np.int64)
    want = fx["count"][:, cols].astype(np.int64)
    diff = np.abs(np.asarray(counts, np.int64) - want)
    assert np.all(diff[band == 0] == 0), f"{int((diff[band == 0] > 0).sum())} band-free counts differ"
    assert np.all(diff <= band), "calibration counts differ beyond the band"
    return {"band_tiles": int(band.sum()), "flipped": int(diff.sum()), "cells": int(diff.size)}


def sampled_outputs_vs_oracle(x: Dict, cu, o: np.ndarray, mask: np.ndarray, t_bh: np.ndarray, block: int,
                              qblocks: Sequence[Tuple[int, int, int]], sequential_every: int = 8):
    """Outputs of the sampled Q-blocks against the oracle under the GPU's own
    skip decisions (forced mask). Every `sequential_every`-th block runs the
    oracle's tile loop; the others its fast form, which equals the loop under
    any forced mask (pinned on the CPU). Returns (max-abs, mean-abs)."""
    scale = osk.default_sm_scale(x["q"].shape[2])
    worst, tot, n = 0.0, 0.0, 0
    cache = {}
    for idx, (b, h, i) in enumerate(qblocks):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if (b, h) not in cache:
            cache.clear()
            cache[(b, h)] = (to_f64(x["k"][s0:s1, h]), to_f64(x["v"][s0:s1, h]))
        kh, vh = cache[(b, h)]
        r0, r1 = i * block, min(s1 - s0, (i + 1) * block)
        qh = to_f64(x["q"][s0 + r0:s0 + r1, h])
        nk = osk.n_tiles(s1 - s0, block)
        forced = mask[b, h, i, :nk] == osk.TILE_SKIPPED
        fn = osk.skip_softmax_qblock if idx % sequential_every == 0 else osk.skip_softmax_qblock_fast
        ref = fn(qh, kh, vh, float(t_bh[b, h]), block, scale, forced_skip=forced)
        diff = np.abs(o[s0 + r0:s0 + r1, h] - ref["o"])
        assert np.all(np.isfinite(o[s0 + r0:s0 + r1, h])), f"non-finite output at {(b, h, i)}"
        worst = max(worst, float(diff.max()))
        tot += float(diff.sum())
        n += diff.size
    mean = tot / n
    assert worst <= O_MAX_ABS and mean <= O_MEAN_ABS, f"output mismatch max {worst:.3e} mean {mean:.3e}"
    return worst, mean


def sample_qblocks(cu, H: int, block: int, heads: Sequence[int], per_head: int, seed: int):
    """Deterministic sample of Q-blocks: first, last (often partial) and random ones."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(len(cu) - 1):
        nq = osk.n_tiles(int(cu[b + 1] - cu[b]), block)
        if nq == 0:
            continue
        for h in heads:
            picks = {0, nq - 1}
            while len(picks) < min(per_head, nq):
                picks.add(int(rng.integers(nq)))
            out += [(b, h, i) for i in sorted(picks)]
    return out


# ---- e4m3 (FP8) path ------------------------------------------------------------------
# The kernel rounds P to e4m3 for the P.V product. With P = 2^(s - m_base),
# where m_base lies within 2^8 of the row's running maximum, a value in the
# normal range moves by at most 2^-4 of itself. A subnormal value moves by at
# most 2^-10, and a flushed one by itself. So row r's output moves by at most
#   max|v| * sum_j max(2^-4 p_j, min(p_j, 2^-10)) / sum_j p_j,
# with p_j = 2^(s_j - max kept s) over the kept keys. On top of that come the
# bf16 rounding of O (2^-9 relative) and fp32 accumulation noise.
FP8_NOISE = 2e-3


def fp8_row_bound(qf: np.ndarray, kf: np.ndarray, vf: np.ndarray, kept_cols: np.ndarray, scale: float,
                  o_ref: np.ndarray, causal_row0=None) -> np.ndarray:
    """Per-row output bound of the e4m3 P.V product (see above), fp64.
    qf [R, D] rows, kf/vf [S, D] of one head (dequantized), kept_cols [S] bool."""
    s = (qf @ kf.T) * (scale / math.log(2.0))
    if causal_row0 is not None:
        rows = causal_row0 + np.arange(s.shape[0])[:, None]
        s = np.where(np.arange(s.shape[1])[None, :] <= rows, s, -np.inf)
    s = np.where(kept_cols[None, :], s, -np.inf)
    p = np.exp2(s - s.max(axis=1, keepdims=True))
    err = np.maximum(2.0 ** -4 * p, np.minimum(p, 2.0 ** -10))
    vmax = np.abs(vf).max()
    return vmax * err.sum(1) / p.sum(1) + 2.0 ** -8 * np.abs(o_ref).max(1) + FP8_NOISE

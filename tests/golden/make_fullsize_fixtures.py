"""Write the full-size oracle fixtures that the GPU parity tests compare against.

This script calls only the fp64 oracle (`oracle/`) and the seeded input
generator (`synth/`); no value in the fixtures comes from the HIP path.

Method: ModelOpt pull request "skip-softmax ... via dedicated Triton kernels",
sections "Changes / Triton kernels" and "Calibration"; ModelOpt README
"Skip-Softmax Sparse Attention for Diffusion Models", section "Threshold
Modes" (log2 comparison, lambda = scale_factor / seq_k).

For every KV tile j of every Q-block the oracle's fast form
(`oracle.skip_softmax.tile_stats_fast`) gives d_j, the largest margin of the
tile's row maxima over the running maxima; for lambda <= 1 it does not depend
on lambda, so one pass over the scores serves every threshold. A tile is
skipped at log2 threshold t when d_j < t, and it lies in the decision band
when |d_j - t| <= 1e-3 (either decision is accepted there).

Per work-group (one Q-block of one (sequence, head), in the library's row
order `oracle.skip_softmax.workgroups`) and per threshold, a fixture holds:
- count: skipped tiles;
- band: tiles in the decision band;
- sum_j, sum_j2 (forward columns only, listed in sum_cols): sums of the
  skipped tiles' indices j and j^2, so that a work-group with no band tile is
  checked tile by tile, not only by its count;
- tiles: tiles visited.
Plus, per config: the calibration config's log-space fit of the oracle's
own counts, and for the WAN-5B-like config the full skip and band bit masks.

Run from the repository root:  python tests/golden/make_fullsize_fixtures.py [name ...]
It takes about 10-15 minutes per 75,600-token config on 8 CPU cores.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import calibration as oc  # noqa: E402
from oracle import skip_softmax as osk  # noqa: E402
from synth import CONFIGS, bf16_bits_to_f32, make_inputs  # noqa: E402

OUT_DIR = os.path.dirname(os.path.abspath(__file__))
BAND = 1e-3
CALIB_LAMBDAS = np.geomspace(1e-6, 0.7, 16)

# name -> threshold columns. A column is ("lambda", value) for one lambda on
# every (sequence, head), or ("scale_factor", [H] values) with lambda_bh =
# sf_h / S_b. Calibration columns (the 16 log-spaced lambdas) keep counts and
# band counts; forward columns also keep the index sums.
_VARLEN_SF = np.full(40, 650.0)
_VARLEN_SF[:2] = 0.0
COLUMNS = {
    "wan5b": [("lambda", 1e-3)],
    "calib": [("lambda", x) for x in CALIB_LAMBDAS],
    "headline": [("lambda", x) for x in CALIB_LAMBDAS] + [("lambda", 8e-3), ("lambda", 1.0)],
    "varlen": [("scale_factor", _VARLEN_SF)],
}
FORWARD_COLUMNS = {"wan5b": [0], "calib": [], "headline": [16, 17], "varlen": [0]}

_X = {}  # inputs of the config being processed (inherited by the worker processes)


def _limit_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _head_d(task):
    """d [nQ, nK] of every Q-block of sequence b, head h (oracle fast form)."""
    b, h, block, scale = task
    cu = _X["cu"]
    s0, s1 = int(cu[b]), int(cu[b + 1])
    qh = bf16_bits_to_f32(_X["q"][s0:s1, h]).astype(np.float64)
    kh = bf16_bits_to_f32(_X["k"][s0:s1, h]).astype(np.float64)
    n = osk.n_tiles(s1 - s0, block)
    d = np.empty((n, n))
    for i in range(n):
        d[i], _ = osk.tile_stats_fast(qh[i * block:(i + 1) * block], kh, block, scale)
    return b, h, d


def _t_matrix(cu, H, col):
    kind, val = col
    B = len(cu) - 1
    t = np.empty((B, H))
    for b in range(B):
        S = int(cu[b + 1] - cu[b])
        for h in range(H):
            lam = val if kind == "lambda" else (float(val[h]) / S if S > 0 else 0.0)
            t[b, h] = oc.log2_threshold(lam)
    return t


def build(name: str, workers: int) -> str:
    cfg = CONFIGS[name]
    t0 = time.time()
    x = make_inputs(cfg)
    _X.update(q=x["q"], k=x["k"], cu=x["cu_seqlens"])
    cu = x["cu_seqlens"]
    H, blk = cfg.num_heads, cfg.block
    scale = osk.default_sm_scale(cfg.head_dim)
    print(f"[{name}] inputs ready in {time.time() - t0:.1f} s; {len(cu) - 1} sequences x {H} heads", flush=True)
    tasks = [(b, h, blk, scale) for b in range(len(cu) - 1) for h in range(H) if cu[b + 1] > cu[b]]
    ds = {}
    with mp.get_context("fork").Pool(workers, initializer=_limit_threads) as pool:
        for n, (b, h, d) in enumerate(pool.imap_unordered(_head_d, tasks), 1):
            ds[(b, h)] = d
            if n % 4 == 0 or n == len(tasks):
                print(f"[{name}] {n}/{len(tasks)} heads, {time.time() - t0:.0f} s", flush=True)
    wgs = osk.workgroups(cu, H, blk)
    cols = COLUMNS[name]
    nw, nc = len(wgs), len(cols)
    tmat = [_t_matrix(cu, H, c) for c in cols]
    fwd = FORWARD_COLUMNS[name]
    count = np.zeros((nw, nc), np.int16)
    band = np.zeros((nw, nc), np.int16)
    sum_j = np.zeros((nw, len(fwd)), np.int32)
    sum_j2 = np.zeros((nw, len(fwd)), np.int32)
    tiles = np.zeros(nw, np.int16)
    for r, (b, h, i) in enumerate(wgs):
        d = ds[(b, h)][i]
        j = np.arange(d.size)
        tiles[r] = d.size
        for c in range(nc):
            t = tmat[c][b, h]
            skip = d < t
            count[r, c] = skip.sum()
            band[r, c] = np.sum(np.abs(d - t) <= BAND)
            if c in fwd:
                sum_j[r, fwd.index(c)] = j[skip].sum()
                sum_j2[r, fwd.index(c)] = (j[skip] ** 2).sum()
    out = {"count": count, "band": band, "sum_j": sum_j, "sum_j2": sum_j2, "sum_cols": np.array(fwd, np.int32),
           "tiles": tiles,
           "cu_seqlens": cu, "num_heads": H, "head_dim": cfg.head_dim, "block": blk, "seed": cfg.seed,
           "band_width": BAND,
           "column_kind": np.array([c[0] for c in cols]),
           "column_value": np.array([c[1] if c[0] == "lambda" else np.nan for c in cols])}
    if any(c[0] == "scale_factor" for c in cols):
        out["scale_factor"] = np.stack([np.asarray(c[1], np.float64) for c in cols if c[0] == "scale_factor"])
    if name in ("calib", "headline"):
        # the oracle's own fit of its per-threshold tile sparsity (one sequence)
        S = int(cu[1] - cu[0])
        sp = count[:, :16].sum(0, dtype=np.int64) / tiles.sum(dtype=np.int64)
        fit = oc.fit_exponential_logspace(CALIB_LAMBDAS, sp, np.full(16, float(S)))
        out.update(sparsity=sp, fit_a=fit.a, fit_b=fit.b, fit_s_min=fit.s_min, fit_s_max=fit.s_max,
                   fit_n_used=fit.n_used)
        print(f"[{name}] sparsity {np.round(sp, 4)}; fit a={fit.a:.6g} b={fit.b:.6g}", flush=True)
    if name == "wan5b":
        t = tmat[0][0, 0]
        dd = np.stack([ds[(0, h)] for h in range(H)])
        out["skip_bits"] = np.packbits(dd < t)
        out["band_bits"] = np.packbits(np.abs(dd - t) <= BAND)
        out["skip_per_head"] = (dd < t).sum(axis=(1, 2))
        print(f"[{name}] per-head skipped tiles at lambda 1e-3: {out['skip_per_head'].tolist()}", flush=True)
    path = os.path.join(OUT_DIR, f"fullsize_{name}.npz")
    np.savez_compressed(path, **out)
    print(f"[{name}] wrote {path} ({os.path.getsize(path)} bytes) in {time.time() - t0:.0f} s", flush=True)
    _X.clear()
    return path


def main(argv):
    names = argv or list(COLUMNS)
    workers = min(8, os.cpu_count() or 1)
    for n in names:
        if n not in COLUMNS:
            raise SystemExit(f"unknown config {n}; choose from {list(COLUMNS)}")
        build(n, workers)


if __name__ == "__main__":
    main(sys.argv[1:])

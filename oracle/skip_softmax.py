"""Skip-softmax (BLASST) attention forward, fp64, written as the method's steps.

TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

Sources (web pages, cited by title and section):
* ModelOpt diffusers sparsity README "Skip-Softmax Sparse Attention for
  Diffusion Models", introduction: the FlashAttention loop leaves out KV
  tiles that would add almost nothing to the softmax; section "Threshold
  Modes": the kernel compares in log2 units against log2(lambda).
* ModelOpt pull request "skip-softmax ... via dedicated Triton kernels",
  section "Changes / Triton kernels": when a tile's largest score sits well
  under the running softmax maximum, the loop moves on to the next tile
  without fetching that tile's V, exponentiating its scores or adding to the
  output; the skipped tiles are counted at run time; the calibration kernel
  runs the full attention and, in the same pass, counts for N thresholds
  how many tiles each would have left out.
* ModelOpt pull request #1166 "Add the Skip softmax for diffusion", section
  "Usage": tiles are br x bc = 128 x 128, attention is non-causal.

Readings where the pages are silent (each one is listed with its reason in
the design notes):
* Scores are compared in log2 units: s = (q.k) * sm_scale * log2(e), against
  t = log2(lambda); lambda = 0 gives t = -inf (dense).
* The vote is per row: with rowmax_r the tile's maximum over valid keys of
  row r and m_r the running maximum BEFORE the tile,
  d = max over valid rows of (rowmax_r - m_r), with m_r = -inf giving +inf;
  the tile is skipped iff d < t (strict). The first tile is never skipped.
* KV tiles are visited in ascending order; invalid keys of a partial last
  tile take no part; query rows past the end of a sequence do not vote.
* A skipped tile changes nothing (m, l and the accumulator keep their values).

Array conventions: q, k, v are [T, H, D] (packed tokens of all sequences,
`cu_seqlens` [B+1] gives sequence b's token range); the oracle computes in
fp64 on whatever (bf16-rounded) values it is given.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

LOG2E = 1.0 / math.log(2.0)

# Tile-mask codes (shared meaning with the library's debug mask output).
TILE_KEPT = 0
TILE_SKIPPED = 1
TILE_NONE = 2  # no tile here (beyond the sequence) or not computed


def n_tiles(n: int, block: int) -> int:
    return (n + block - 1) // block


def default_sm_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _head(x: np.ndarray, s0: int, s1: int, h: int) -> np.ndarray:
    return np.asarray(x[s0:s1, h, :], dtype=np.float64)


# ---------------------------------------------------------------------------
# The textbook definition (dense attention).
# ---------------------------------------------------------------------------
def attention_exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                    causal: bool = False) -> np.ndarray:
    """softmax(q k^T * sm_scale) v for one head, q [R,D], k/v [S,D], fp64.

    causal: query r attends keys 0..r only (R == S). The exact result that
    dense mode (lambda = 0) must reproduce up to rounding. Pinned by torch's
    CPU scaled_dot_product_attention in fp64 (is_causal for the causal form).
    """
    z = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * sm_scale
    if causal:
        z = np.where(np.tril(np.ones(z.shape, dtype=bool)), z, -np.inf)
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.asarray(v, np.float64)


# ---------------------------------------------------------------------------
# Sequential form: the tile loop, one Q-block at a time.
# ---------------------------------------------------------------------------
def _causal_limit(S: int, block: int, causal_row0: Optional[int], R: int) -> Tuple[int, int]:
    """(number of KV tiles visited, key columns visible to the block)."""
    if causal_row0 is None:
        return n_tiles(S, block), S
    last = causal_row0 + R - 1            # position of the block's last query
    nk = last // block + 1
    return nk, min(S, nk * block)


def _causal_mask(s: np.ndarray, causal_row0: Optional[int], col0: int) -> np.ndarray:
    """Scores with keys after each row's query set to -inf (causal only)."""
    if causal_row0 is None:
        return s
    rows = causal_row0 + np.arange(s.shape[0])[:, None]
    cols = col0 + np.arange(s.shape[1])[None, :]
    return np.where(cols <= rows, s, -np.inf)


def skip_softmax_qblock(qb: np.ndarray, k: np.ndarray, v: np.ndarray, t: float, block: int,
                        sm_scale: float, forced_skip: Optional[np.ndarray] = None,
                        calib_ts: Optional[np.ndarray] = None,
                        causal_row0: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Run the skip-softmax tile loop for one Q-block of one head.

    qb: [R, D] valid query rows of the block; k, v: [S, D] the head's keys/values.
    t: log2 threshold (float('-inf') for dense). forced_skip: optional [nK]
    bool array that replaces the decisions (used to compare outputs under the
    GPU's own decisions). calib_ts: optional [N] log2 thresholds; when given,
    the loop never skips and counts, per threshold, the tiles with d < t_k.
    causal_row0: position of the block's first query for causal attention
    (query at position p sees keys 0..p; only tiles up to the one holding
    the block's last query are visited); None = non-causal.

    Returns dict(o [R,D], d [nK], skip [nK] bool, counts [N] (calibration)).
    Pinned by: the textbook definition at lambda=0, the fast form on small
    inputs, the two-tile worked example, the per-element dropped-probability
    bound and the output-deviation bound (tests/test_oracle_*.py).
    """
    qb = np.asarray(qb, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    R, D = qb.shape
    S = k.shape[0]
    nk, _ = _causal_limit(S, block, causal_row0, R)
    c = sm_scale * LOG2E

    m = np.full(R, -np.inf)        # running max (log2 units), before each tile
    l = np.zeros(R)                # running sum of 2^(s - m)
    acc = np.zeros((R, v.shape[1]))
    d_all = np.empty(nk)
    skip_all = np.zeros(nk, dtype=bool)
    counts = None if calib_ts is None else np.zeros(len(calib_ts), dtype=np.int64)

    for j in range(nk):
        j0, j1 = j * block, min(S, (j + 1) * block)
        s = (qb @ k[j0:j1].T) * c                 # scores of tile j, log2 units
        s = _causal_mask(s, causal_row0, j0)
        rowmax = s.max(axis=1)
        with np.errstate(invalid="ignore"):
            d = float(np.max(rowmax - m))         # m = -inf gives +inf
        d_all[j] = d
        if calib_ts is not None:
            counts += (d < np.asarray(calib_ts)).astype(np.int64)
            skip = False
        elif forced_skip is not None:
            skip = bool(forced_skip[j])
        else:
            skip = d < t
        skip_all[j] = skip
        if skip:
            continue                               # no V, no exp, no P.V
        m_new = np.maximum(m, rowmax)
        alpha = np.exp2(m - m_new)                 # 0 when m was -inf
        p = np.exp2(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    return {"o": acc / l[:, None], "d": d_all, "skip": skip_all, "counts": counts}


# ---------------------------------------------------------------------------
# Fast form (valid for lambda <= 1): decisions from the dense prefix maximum.
# ---------------------------------------------------------------------------
def tile_stats_fast(qb: np.ndarray, k: np.ndarray, block: int, sm_scale: float,
                    causal_row0: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """d_j for every KV tile of one Q-block, from the dense prefix maximum.

    For lambda <= 1 a skipped tile has rowmax_r < m_r in every row, so the
    running maximum before tile j always equals the prefix maximum over
    tiles 0..j-1 whatever was skipped; d_j therefore does not depend on the
    threshold. Returns (d [nK], scores [R, visible keys] in log2 units).
    Pinned by equality with the sequential form (tests).
    """
    qb = np.asarray(qb, np.float64)
    _, kv_end = _causal_limit(k.shape[0], block, causal_row0, qb.shape[0])
    s = (qb @ np.asarray(k, np.float64)[:kv_end].T) * (sm_scale * LOG2E)
    s = _causal_mask(s, causal_row0, 0)
    S = s.shape[1]
    starts = np.arange(0, S, block)
    tile_max = np.maximum.reduceat(s, starts, axis=1)            # [R, nK]
    prefix = np.full_like(tile_max, -np.inf)
    if tile_max.shape[1] > 1:
        prefix[:, 1:] = np.maximum.accumulate(tile_max, axis=1)[:, :-1]
    with np.errstate(invalid="ignore"):
        d = np.max(tile_max - prefix, axis=0)
    return d, s


def skip_softmax_qblock_fast(qb: np.ndarray, k: np.ndarray, v: np.ndarray, t: float, block: int,
                             sm_scale: float, forced_skip: Optional[np.ndarray] = None,
                             causal_row0: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Fast form of `skip_softmax_qblock` for t <= 0 (lambda <= 1).

    The output is the exact softmax restricted to the kept tiles' keys,
    renormalised: each row's overall maximum lies in a kept tile.
    """
    d, s = tile_stats_fast(qb, k, block, sm_scale, causal_row0)
    skip = (d < t) if forced_skip is None else np.asarray(forced_skip, bool)
    keep_cols = np.repeat(~skip, block)[: s.shape[1]]
    sk = np.where(keep_cols[None, :], s, -np.inf)
    mx = sk.max(axis=1, keepdims=True)
    p = np.exp2(sk - mx)
    o = (p @ np.asarray(v, np.float64)[: s.shape[1]]) / p.sum(axis=1, keepdims=True)
    return {"o": o, "d": d, "skip": skip}


# ---------------------------------------------------------------------------
# Whole-problem drivers over (sequence, head, Q-block).
# ---------------------------------------------------------------------------
def workgroups(cu_seqlens: Sequence[int], num_heads: int, block: int) -> List[Tuple[int, int, int]]:
    """(b, h, i) of every Q-block, sequence-major, then head, then Q-block.

    This is also the row order of the calibration count table.
    """
    out = []
    for b in range(len(cu_seqlens) - 1):
        S = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        for h in range(num_heads):
            for i in range(n_tiles(S, block)):
                out.append((b, h, i))
    return out


def skip_softmax_forward(q, k, v, cu_seqlens, t_bh, block: int, sm_scale: Optional[float] = None,
                         qblocks: Optional[Iterable[Tuple[int, int, int]]] = None,
                         forced_mask: Optional[np.ndarray] = None, fast: bool = False,
                         causal: bool = False) -> Dict[str, np.ndarray]:
    """Skip-softmax forward over a packed varlen batch (causal: prefill form).

    t_bh: [B, H] log2 thresholds. qblocks: optional subset of (b, h, i) to
    compute (others are left NaN / TILE_NONE). forced_mask: optional
    [B, H, nQmax, nKmax] tile mask whose skip bits replace the decisions.
    Returns dict(o [T,H,D] fp64 (NaN where not computed), mask, d
    [B,H,nQmax,nKmax], skipped [B,H], total [B,H]).
    """
    T, H, D = q.shape
    cu = [int(x) for x in cu_seqlens]
    B = len(cu) - 1
    scale = default_sm_scale(D) if sm_scale is None else sm_scale
    lens = [cu[b + 1] - cu[b] for b in range(B)]
    nmax = max([n_tiles(s, block) for s in lens] + [0])
    t_bh = np.broadcast_to(np.asarray(t_bh, np.float64), (B, H))
    o = np.full((T, H, D), np.nan)
    mask = np.full((B, H, nmax, nmax), TILE_NONE, dtype=np.uint8)
    dd = np.full((B, H, nmax, nmax), np.nan)
    skipped = np.zeros((B, H), dtype=np.int64)
    total = np.zeros((B, H), dtype=np.int64)
    todo = workgroups(cu, H, block) if qblocks is None else list(qblocks)
    heads_cache: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
    for (b, h, i) in todo:
        s0, s1 = cu[b], cu[b + 1]
        if (b, h) not in heads_cache:
            heads_cache.clear()
            heads_cache[(b, h)] = (_head(q, s0, s1, h), _head(k, s0, s1, h), _head(v, s0, s1, h))
        qh, kh, vh = heads_cache[(b, h)]
        r0, r1 = i * block, min(s1 - s0, (i + 1) * block)
        nk = i + 1 if causal else n_tiles(s1 - s0, block)
        forced = None if forced_mask is None else forced_mask[b, h, i, :nk] == TILE_SKIPPED
        fn = skip_softmax_qblock_fast if fast else skip_softmax_qblock
        res = fn(qh[r0:r1], kh, vh, float(t_bh[b, h]), block, scale, forced_skip=forced,
                 causal_row0=r0 if causal else None)
        o[s0 + r0:s0 + r1, h, :] = res["o"]
        mask[b, h, i, :nk] = np.where(res["skip"], TILE_SKIPPED, TILE_KEPT)
        dd[b, h, i, :nk] = res["d"]
        skipped[b, h] += int(res["skip"].sum())
        total[b, h] += nk
    return {"o": o, "mask": mask, "d": dd, "skipped": skipped, "total": total}


def calibration_counts(q, k, v, cu_seqlens, log2_ts: Sequence[float], block: int,
                       sm_scale: Optional[float] = None,
                       qblocks: Optional[Iterable[Tuple[int, int, int]]] = None,
                       causal: bool = False) -> Dict[str, np.ndarray]:
    """The calibration pass: dense attention plus, per Q-block (work-group)
    and per threshold t_k, the number of tiles that would be skipped (d < t_k).

    Returns dict(o [T,H,D] dense output, counts [nWG, N], tiles [nWG], wg
    list of (b,h,i)). Rows follow `workgroups` order; with `qblocks` only
    those rows are computed (others stay -1).
    Pinned by: counts equal the sequential forward's skip counts at each
    lambda_k, and monotone in lambda (tests).
    """
    T, H, D = q.shape
    cu = [int(x) for x in cu_seqlens]
    scale = default_sm_scale(D) if sm_scale is None else sm_scale
    wgs = workgroups(cu, H, block)
    index = {w: n for n, w in enumerate(wgs)}
    ts = np.asarray(log2_ts, np.float64)
    counts = np.full((len(wgs), len(ts)), -1, dtype=np.int64)
    tiles = np.full(len(wgs), -1, dtype=np.int64)
    o = np.full((T, H, D), np.nan)
    todo = wgs if qblocks is None else list(qblocks)
    cache: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
    for (b, h, i) in todo:
        s0, s1 = cu[b], cu[b + 1]
        if (b, h) not in cache:
            cache.clear()
            cache[(b, h)] = (_head(q, s0, s1, h), _head(k, s0, s1, h), _head(v, s0, s1, h))
        qh, kh, vh = cache[(b, h)]
        r0, r1 = i * block, min(s1 - s0, (i + 1) * block)
        res = skip_softmax_qblock(qh[r0:r1], kh, vh, float("-inf"), block, scale, calib_ts=ts,
                                  causal_row0=r0 if causal else None)
        n = index[(b, h, i)]
        counts[n] = res["counts"]
        tiles[n] = len(res["d"])
        o[s0 + r0:s0 + r1, h, :] = res["o"]
    return {"o": o, "counts": counts, "tiles": tiles, "wg": wgs}

"""Threshold conversion, exponential-model fit and threshold resolution, fp64.

TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

Sources (web pages, cited by title and section):
* ModelOpt diffusers sparsity README "Skip-Softmax Sparse Attention for
  Diffusion Models": the exponential model scale_factor = a * exp(b *
  target_sparsity), fitted in log space (introduction); section "Threshold
  Modes": fixed lambda goes to the kernel as log2(lambda); calibrated mode
  computes threshold = scale_factor / seq_k; the static default is
  lambda = 0.1; section "Known Issues": targets below the observed floor
  extrapolate and trigger a warning; the checkpoint (a, b) are used as
  a * exp(b * sparsity) with no further conversion.
* ModelOpt pull request "skip-softmax ... via dedicated Triton kernels",
  sections "Method" and "Calibration": priority raw threshold > calibrated
  scale_factor > static threshold; the log-space fit minimises relative
  error and records the observed sparsity range.
* TensorRT-LLM pull request "Add SkipSoftmax sparse attention support for
  visual generation", sections "Use Cases" and "Priority Order": a direct
  threshold_scale_factor wins over target_sparsity + formula; a target
  without a formula is an error; coefficients may come as a or log_a.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

STATIC_DEFAULT_LAMBDA = 0.1

# Status codes, same meaning as the library's.
OK = 0
WARN_EXTRAPOLATED = 1
ERR_INVALID_ARG = -1
ERR_THRESHOLD_RANGE = -3
ERR_NO_FORMULA = -4
ERR_FIT_DEGENERATE = -5


def log2_threshold(lam: float) -> float:
    """t = log2(lambda) for lambda in [0, 1]; lambda = 0 gives -inf (dense)."""
    if not (0.0 <= lam <= 1.0):
        raise ValueError("lambda must lie in [0, 1]")
    return float("-inf") if lam == 0.0 else math.log2(lam)


@dataclasses.dataclass
class Fit:
    a: float
    log_a: float
    b: float
    s_min: float
    s_max: float
    n_used: int


def fit_exponential_logspace(lambdas: Sequence[float], sparsities: Sequence[float],
                             seq_k: Sequence[float]) -> Fit:
    """Least-squares fit of ln(scale_factor) = ln(a) + b * sparsity.

    One point per measured (lambda_i, sparsity_i, seq_k_i); scale_factor_i =
    lambda_i * seq_k_i. Points with sparsity 0 or 1 carry no information about
    the curve (plateaus) and are left out. Ordinary least squares written out
    (closed-form normal equations), no library fit. Raises ValueError when
    fewer than two distinct sparsities remain.
    Pinned by exact recovery of (a, b) from points on a known curve, a
    hand-worked three-point fit and scipy.stats.linregress (tests).
    """
    lam = np.asarray(lambdas, np.float64)
    s = np.asarray(sparsities, np.float64)
    sk = np.broadcast_to(np.asarray(seq_k, np.float64), lam.shape)
    use = (s > 0.0) & (s < 1.0) & (lam > 0.0)
    x = s[use]
    y = np.log(lam[use] * sk[use])
    if x.size < 2 or np.unique(x).size < 2:
        raise ValueError("degenerate fit: fewer than two distinct usable sparsities")
    xm, ym = x.mean(), y.mean()
    b = float(np.sum((x - xm) * (y - ym)) / np.sum((x - xm) ** 2))
    log_a = float(ym - b * xm)
    return Fit(a=math.exp(log_a), log_a=log_a, b=b, s_min=float(x.min()), s_max=float(x.max()),
               n_used=int(x.size))


def _usable_points(lambdas, sparsities, seq_k):
    lam = np.asarray(lambdas, np.float64)
    s = np.asarray(sparsities, np.float64)
    sk = np.broadcast_to(np.asarray(seq_k, np.float64), lam.shape)
    use = (s > 0.0) & (s < 1.0) & (lam > 0.0)
    return s[use], lam[use] * sk[use]


def fit_exponential_linear(lambdas: Sequence[float], sparsities: Sequence[float],
                           seq_k: Sequence[float]) -> Fit:
    """Least-squares fit of scale_factor = a * exp(b * sparsity) in linear space.

    This is the calibrator's non-log option: fit_logspace = False, the
    ModelOpt default; the log-space fit is the one recommended for diffusion.
    It minimises sum_i (a e^{b s_i} - y_i)^2 with y_i = lambda_i * seq_k_i,
    over the same usable points as the log-space fit.

    Written as plain nonlinear least squares: scipy's Levenberg-Marquardt on
    the residuals r_i = exp(ln a + b s_i) - y_i with their exact Jacobian,
    parameterised by (ln a, b) so that a stays positive, started from the
    log-space fit. Raises ValueError for fewer than two distinct usable
    sparsities.

    Pinned by:
    - exact recovery of (a, b) from points on a known curve;
    - the zero gradient of the squared error at the returned (a, b), and no
      better neighbouring point;
    - scipy.optimize.curve_fit on noisy points (tests).
    """
    from scipy.optimize import least_squares

    x, y = _usable_points(lambdas, sparsities, seq_k)
    if x.size < 2 or np.unique(x).size < 2:
        raise ValueError("degenerate fit: fewer than two distinct usable sparsities")
    start = fit_exponential_logspace(lambdas, sparsities, seq_k)

    def residuals(p):
        return np.exp(p[0] + p[1] * x) - y

    def jacobian(p):
        e = np.exp(p[0] + p[1] * x)
        return np.stack([e, x * e], axis=1)

    sol = least_squares(residuals, [start.log_a, start.b], jac=jacobian, method="lm",
                        xtol=1e-15, ftol=1e-15, gtol=1e-15, max_nfev=20000)
    log_a, b = float(sol.x[0]), float(sol.x[1])
    return Fit(a=math.exp(log_a), log_a=log_a, b=b, s_min=float(x.min()), s_max=float(x.max()),
               n_used=int(x.size))


class CalibPool:
    """Calibration counts pooled over passes, one group per key length.

    Several samples of one shape pool into one group (multi-sample
    accumulation). Different shapes keep separate groups, whose points can be
    fitted together or apart. This addresses the resolution dependence the
    README lists under "Known Issues".

    Group sparsity at threshold k = sum of skipped tiles / sum of visited
    tiles over every sequence of that key length. This is the same
    tile-weighted ratio as one pass over all of those sequences.

    Pinned by: pooling two passes equals one pass over the union of their
    work-groups (tests).
    """

    def __init__(self, n_lambda: int):
        self.n_lambda = int(n_lambda)
        self.groups: Dict[int, List] = {}  # seq_k -> [skipped (n_lambda,), visited]; insertion order kept

    def add(self, counts, tiles, cu_seqlens, num_heads: int, block: int) -> None:
        counts = np.asarray(counts, np.int64).reshape(-1, self.n_lambda)
        tiles = np.asarray(tiles, np.int64).reshape(-1)
        w = 0
        for b in range(len(cu_seqlens) - 1):
            S = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
            nwg = -(-S // block) * num_heads
            if S > 0:
                g = self.groups.setdefault(S, [np.zeros(self.n_lambda, np.int64), 0])
                g[0] = g[0] + counts[w:w + nwg].sum(axis=0)
                g[1] += int(tiles[w:w + nwg].sum())
            w += nwg

    def points(self, lambdas: Sequence[float]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Flattened fit points (lambda, sparsity, seq_k), group-major."""
        lam, sp, sk = [], [], []
        for S, (skipped, visited) in self.groups.items():
            for k in range(self.n_lambda):
                lam.append(float(lambdas[k]))
                sp.append(skipped[k] / visited)
                sk.append(float(S))
        return np.array(lam), np.array(sp), np.array(sk)


@dataclasses.dataclass
class ThresholdSpec:
    """Optional threshold sources, applied in priority order (first set wins)."""

    raw_log2: Optional[float] = None
    lam: Optional[float] = None
    scale_factor: Optional[float] = None
    target_sparsity: Optional[float] = None
    a: Optional[float] = None
    log_a: Optional[float] = None
    b: Optional[float] = None
    s_min: Optional[float] = None
    s_max: Optional[float] = None


def resolve_threshold(spec: ThresholdSpec, seq_k: int):
    """Resolve a threshold spec into (status, lambda, log2 lambda).

    Priority: raw log2 > fixed lambda > scale_factor / seq_k > target sparsity
    with formula (scale_factor = a * exp(b * target), then / seq_k) > static
    lambda 0.1. Errors: target without formula; lambda outside [0, 1]; NaN.
    A target outside [s_min, s_max] resolves but returns WARN_EXTRAPOLATED.
    Pinned by the pages' printed anchors (raw -0.7 vs lambda 0.61557, static
    0.1, the formula's value at target 0 and its doubling step) (tests).
    """
    def finish(lam: float, status: int = OK):
        if not (lam == lam) or lam < 0.0 or lam > 1.0:
            return ERR_THRESHOLD_RANGE, float("nan"), float("nan")
        return status, lam, (float("-inf") if lam == 0.0 else math.log2(lam))

    if spec.raw_log2 is not None:
        r = float(spec.raw_log2)
        if r != r or r > 0.0:
            return ERR_THRESHOLD_RANGE, float("nan"), float("nan")
        return OK, 2.0 ** r, r
    if spec.lam is not None:
        return finish(float(spec.lam))
    if spec.scale_factor is not None:
        if seq_k < 1:
            return ERR_INVALID_ARG, float("nan"), float("nan")
        return finish(float(spec.scale_factor) / seq_k)
    if spec.target_sparsity is not None:
        tgt = float(spec.target_sparsity)
        if tgt != tgt or seq_k < 1:
            return ERR_INVALID_ARG, float("nan"), float("nan")
        if spec.b is None or (spec.a is None and spec.log_a is None):
            return ERR_NO_FORMULA, float("nan"), float("nan")
        log_a = spec.log_a if spec.log_a is not None else math.log(spec.a)
        sf = math.exp(log_a + spec.b * tgt)
        status = OK
        if spec.s_min is not None and spec.s_max is not None and not (spec.s_min <= tgt <= spec.s_max):
            status = WARN_EXTRAPOLATED
        return finish(sf / seq_k, status)
    return finish(STATIC_DEFAULT_LAMBDA)

"""Pins of the oracle's calibration counter, fit and threshold resolution (CPU only)."""
import math

import numpy as np
import pytest
import scipy.stats

from oracle import calibration as oc
from oracle import skip_softmax as osk
from synth import CONFIGS, bf16_bits_to_f32, make_inputs

INF = float("inf")


@pytest.fixture(scope="module")
def tiny():
    cfg = CONFIGS["tiny"]
    x = make_inputs(cfg)
    return cfg, {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}, x["cu_seqlens"]


def test_calibration_counts_equal_forward_skip_counts(tiny):
    cfg, x, cu = tiny
    lams = np.geomspace(1e-6, 0.7, 16)
    ts = np.log2(lams)
    cal = osk.calibration_counts(x["q"], x["k"], x["v"], cu, ts, cfg.block)
    wgs = cal["wg"]
    assert cal["counts"].shape == (len(wgs), 16)
    assert np.all(np.diff(cal["counts"], axis=1) >= 0), "counts must be monotone in lambda"
    for kk, t in enumerate(ts):
        fwd = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, t, cfg.block)
        per_wg = [(fwd["mask"][b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs]
        np.testing.assert_array_equal(cal["counts"][:, kk], per_wg)
    dense = osk.skip_softmax_forward(x["q"], x["k"], x["v"], cu, -INF, cfg.block)
    np.testing.assert_allclose(cal["o"], dense["o"], atol=1e-13, rtol=0)
    assert np.all(cal["tiles"] == 1024 // 64)


def test_fit_recovers_exact_curve():
    a, b, seq_k = 7.93, 8.61, 75600
    s = np.linspace(0.35, 0.85, 12)
    lam = a * np.exp(b * s) / seq_k
    f = oc.fit_exponential_logspace(lam, s, seq_k)
    assert f.a == pytest.approx(a, rel=1e-12)
    assert f.b == pytest.approx(b, rel=1e-12)
    assert (f.s_min, f.s_max, f.n_used) == (pytest.approx(0.35), pytest.approx(0.85), 12)


def test_fit_hand_worked_three_points():
    # ln(sf) = 0, 1, 3 at s = 0.2, 0.4, 0.6: x-mean 0.4, y-mean 4/3,
    # Sxy = (-0.2)(-4/3) + 0 + (0.2)(5/3) = 0.6, Sxx = 0.08, b = 7.5,
    # ln a = 4/3 - 7.5 * 0.4 = -5/3.
    s = [0.2, 0.4, 0.6]
    sf = [1.0, math.e, math.e ** 3]
    f = oc.fit_exponential_logspace([x / 1000.0 for x in sf], s, 1000.0)
    assert f.b == pytest.approx(7.5, rel=1e-12)
    assert f.log_a == pytest.approx(-5.0 / 3.0, rel=1e-12)


def test_fit_matches_linregress_and_drops_plateaus():
    rng = np.random.default_rng(5)
    s = np.concatenate([[0.0, 0.0], np.sort(rng.uniform(0.3, 0.9, 10)), [1.0]])
    lam = np.geomspace(1e-6, 0.7, s.size)
    f = oc.fit_exponential_logspace(lam, s, 32760)
    use = (s > 0) & (s < 1)
    ref = scipy.stats.linregress(s[use], np.log(lam[use] * 32760))
    assert f.b == pytest.approx(ref.slope, rel=1e-10)
    assert f.log_a == pytest.approx(ref.intercept, rel=1e-10, abs=1e-12)
    assert f.n_used == 10


def test_fit_degenerate():
    with pytest.raises(ValueError):
        oc.fit_exponential_logspace([1e-3, 1e-2], [0.5, 0.5], 100)
    with pytest.raises(ValueError):
        oc.fit_exponential_logspace([1e-3, 1e-2], [0.0, 1.0], 100)


def test_resolve_page_anchors(golden):
    g = golden("threshold_anchors.txt")
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(raw_log2=g["raw_log2_example"]), 75600)
    assert st == oc.OK and lam == pytest.approx(g["fixed_lambda_example"], abs=g["example_abs_tol"])
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(lam=g["fixed_lambda_example"]), 75600)
    assert st == oc.OK and t == pytest.approx(g["raw_log2_example"], abs=1e-4)
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(), 75600)
    assert st == oc.OK and lam == g["static_default_lambda"]
    # scale factor 5000 over 10000 keys is lambda 1/2 exactly, log2 = -1
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(scale_factor=g["direct_scale_factor"]), 10000)
    assert (st, lam, t) == (oc.OK, 0.5, -1.0)
    # over 1024 keys the same factor is lambda > 1: out of range
    st, _, _ = oc.resolve_threshold(oc.ThresholdSpec(scale_factor=g["direct_scale_factor"]), 1024)
    assert st == oc.ERR_THRESHOLD_RANGE
    # formula at target 0 is a itself; one step of ln2/b doubles it
    a, b = g["checkpoint_a"], g["checkpoint_b"]
    st, lam0, _ = oc.resolve_threshold(oc.ThresholdSpec(target_sparsity=0.0, a=a, b=b), 1000)
    assert st == oc.OK and lam0 == pytest.approx(a / 1000.0, rel=1e-15)
    _, lam1, _ = oc.resolve_threshold(oc.ThresholdSpec(target_sparsity=math.log(2) / b, a=a, b=b), 1000)
    assert lam1 == pytest.approx(2 * lam0, rel=1e-14)
    # log_a form equals a form
    _, lam2, _ = oc.resolve_threshold(
        oc.ThresholdSpec(target_sparsity=g["docs_target"], log_a=math.log(g["docs_a"]), b=g["docs_b"]), 75600)
    _, lam3, _ = oc.resolve_threshold(
        oc.ThresholdSpec(target_sparsity=g["docs_target"], a=g["docs_a"], b=g["docs_b"]), 75600)
    assert lam2 == pytest.approx(lam3, rel=1e-14)


def test_resolve_priority_and_errors():
    full = dict(raw_log2=-1.0, lam=0.25, scale_factor=100.0, target_sparsity=0.5, a=1.0, b=1.0)
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(**full), 1000)
    assert (st, t) == (oc.OK, -1.0)
    full.pop("raw_log2")
    assert oc.resolve_threshold(oc.ThresholdSpec(**full), 1000)[1] == 0.25
    full.pop("lam")
    assert oc.resolve_threshold(oc.ThresholdSpec(**full), 1000)[1] == 0.1
    full.pop("scale_factor")
    assert oc.resolve_threshold(oc.ThresholdSpec(**full), 1000)[1] == pytest.approx(math.exp(0.5) / 1000)
    # target without formula is an error, never a silent default
    assert oc.resolve_threshold(oc.ThresholdSpec(target_sparsity=0.5), 1000)[0] == oc.ERR_NO_FORMULA
    # extrapolation warning outside the observed range
    spec = oc.ThresholdSpec(target_sparsity=0.25, a=7.93, b=8.61, s_min=0.38, s_max=0.86)
    assert oc.resolve_threshold(spec, 75600)[0] == oc.WARN_EXTRAPOLATED
    spec.target_sparsity = 0.5
    assert oc.resolve_threshold(spec, 75600)[0] == oc.OK
    for bad in (-0.1, 1.5, float("nan")):
        assert oc.resolve_threshold(oc.ThresholdSpec(lam=bad), 10)[0] == oc.ERR_THRESHOLD_RANGE
    assert oc.resolve_threshold(oc.ThresholdSpec(raw_log2=0.5), 10)[0] == oc.ERR_THRESHOLD_RANGE
    st, lam, t = oc.resolve_threshold(oc.ThresholdSpec(lam=0.0), 10)
    assert (st, lam, t) == (oc.OK, 0.0, -INF)


# ---- linear-space fit and pooled calibration -------------------------------------
def test_linear_fit_recovers_exact_curve():
    a, b, seq_k = 7.93, 8.61, 75600
    s = np.linspace(0.35, 0.85, 12)
    f = oc.fit_exponential_linear(a * np.exp(b * s) / seq_k, s, seq_k)
    assert f.a == pytest.approx(a, rel=1e-12)
    assert f.b == pytest.approx(b, rel=1e-12)
    assert (f.s_min, f.s_max, f.n_used) == (pytest.approx(0.35), pytest.approx(0.85), 12)


def _noisy(seed, n=14, a=5e-3, b=25.0, sigma=0.3):
    rng = np.random.default_rng(seed)
    s = np.sort(rng.uniform(0.3, 0.9, n))
    y = a * np.exp(b * s) * np.exp(rng.normal(0, sigma, n))
    return s, y


@pytest.mark.parametrize("seed", range(4))
def test_linear_fit_is_a_stationary_point_of_the_squared_error(seed):
    s, y = _noisy(seed)
    f = oc.fit_exponential_linear(y / 1000.0, s, 1000.0)
    e = np.exp(f.b * s)
    r = f.a * e - y
    # dF/da = 2 sum r e, dF/db = 2 sum r a s e, relative to the size of the terms
    assert abs(np.sum(r * e)) <= 1e-9 * np.sum(np.abs(y * e))
    assert abs(np.sum(r * f.a * s * e)) <= 1e-9 * np.sum(np.abs(y * f.a * s * e))
    # and no nearby point does better
    F = np.sum(r * r)
    for da, db in ((1e-4, 0), (-1e-4, 0), (0, 1e-4), (0, -1e-4)):
        assert np.sum(((f.a * (1 + da)) * np.exp((f.b + db) * s) - y) ** 2) >= F


@pytest.mark.parametrize("seed", range(4))
def test_linear_fit_matches_scipy_curve_fit(seed):
    from scipy.optimize import curve_fit
    s, y = _noisy(seed)
    f = oc.fit_exponential_linear(y / 1000.0, s, 1000.0)
    lf = oc.fit_exponential_logspace(y / 1000.0, s, 1000.0)
    p, _ = curve_fit(lambda x, A, B: A * np.exp(B * x), s, y, p0=(lf.a, lf.b), maxfev=50000,
                     xtol=1e-15, ftol=1e-15, gtol=1e-15)
    assert f.a == pytest.approx(p[0], rel=1e-6)
    assert f.b == pytest.approx(p[1], rel=1e-6)
    # the two fits minimise different errors: on noisy data they differ
    assert abs(f.b - lf.b) > 1e-6


def test_linear_fit_degenerate():
    with pytest.raises(ValueError):
        oc.fit_exponential_linear([1e-3, 1e-2], [0.5, 0.5], 100.0)
    with pytest.raises(ValueError):
        oc.fit_exponential_linear([1e-3, 1e-2, 1e-1], [0.0, 0.5, 1.0], 100.0)


def test_pool_equals_one_pass_over_the_union(tiny):
    # Two calibration passes (a 2-sequence batch and a 1-sequence batch of
    # the same key length, plus one of another length) pooled by key length
    # give the same sparsities as one pass over all sequences together.
    cfg, x, cu = tiny
    S = int(cu[1])
    lams = np.geomspace(1e-4, 0.5, 6)
    ts = np.log2(lams)
    q, k, v = x["q"], x["k"], x["v"]
    half = S // 2
    cat = lambda parts: np.concatenate(parts, axis=0)
    # pass A: sequences [0, half) and [half, S); pass B: [0, half) again and [0, 3*half/2)
    qa, ka, va = q, k, v
    cua = [0, half, S]
    qb_, kb_, vb_ = cat([q[:half], q[:3 * half // 2]]), cat([k[:half], k[:3 * half // 2]]), cat([v[:half], v[:3 * half // 2]])
    cub = [0, half, half + 3 * half // 2]
    A = osk.calibration_counts(qa, ka, va, cua, ts, cfg.block)
    B = osk.calibration_counts(qb_, kb_, vb_, cub, ts, cfg.block)
    pool = oc.CalibPool(len(lams))
    pool.add(A["counts"], A["tiles"], cua, cfg.num_heads, cfg.block)
    pool.add(B["counts"], B["tiles"], cub, cfg.num_heads, cfg.block)
    assert list(pool.groups) == [half, 3 * half // 2]
    # the union as one varlen pass
    qu = cat([q[:half], q[half:S], q[:half], q[:3 * half // 2]])
    ku = cat([k[:half], k[half:S], k[:half], k[:3 * half // 2]])
    vu = cat([v[:half], v[half:S], v[:half], v[:3 * half // 2]])
    cuu = [0, half, S, S + half, S + half + 3 * half // 2]
    U = osk.calibration_counts(qu, ku, vu, cuu, ts, cfg.block)
    wgs = U["wg"]
    for key, seqs in ((half, (0, 1, 2)), (3 * half // 2, (3,))):
        rows = [n for n, (b, h, i) in enumerate(wgs) if b in seqs]
        skipped, visited = pool.groups[key]
        np.testing.assert_array_equal(skipped, U["counts"][rows].sum(0))
        assert visited == U["tiles"][rows].sum()
    lam_p, sp_p, sk_p = pool.points(lams)
    assert lam_p.size == 2 * len(lams) and set(sk_p) == {half, 3 * half // 2}

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Runs on an MI355X only (marker `gpu`). Inputs come from the seeded `synth`
generator; the oracle runs on the same bf16-rounded values.
"""
import math

import numpy as np
import pytest

from oracle import calibration as oc
from oracle import skip_softmax as osk
from synth import CONFIGS, make_inputs
from synth.video_tokens import VideoTokenConfig
from tests._parity import (compare_calibration_counts, compare_masks, compare_outputs, compare_outputs_derived,
                           compare_workgroup_stats, gpu_forward, load_fixture, log, mask_workgroup_stats,
                           sample_qblocks, sampled_outputs_vs_oracle, t_matrix, to_device, to_f64)

pytestmark = pytest.mark.gpu

# Small multi-tile ragged batch: 3072 / 300 / 0 / 129 / 64 tokens.
RAGGED = VideoTokenConfig("ragged", ((6, 16, 32), (3, 10, 10), (0, 1, 1), (1, 3, 43), (1, 8, 8)),
                          num_heads=3, head_dim=128, sigma=0.5, block=128, seed=7)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import skip_softmax_video_amd as ssa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ssa.load_library()
    log(f"device: {torch.cuda.get_device_name(0)}")


def _inputs(cfg, heads=None):
    x = make_inputs(cfg, heads=heads)
    xd = {n: to_device(x[n]) for n in ("q", "k", "v")}
    return x, xd, x["cu_seqlens"]


def _f64(x):
    return {n: to_f64(x[n]) for n in ("q", "k", "v")}


def _full_parity(cfg, threshold, kind="lambda", block=None, causal=False, sm_scale=None):
    """Whole batch on the GPU and in the oracle; sm_scale None = the default 1/sqrt(D)."""
    block = block or cfg.block
    x, xd, cu = _inputs(cfg)
    xf = _f64(x)
    H = cfg.num_heads
    log(f"[{cfg.name}] D={cfg.head_dim} block={block} threshold={threshold} kind={kind} causal={causal} "
        f"sm_scale={sm_scale}")
    o, sk, tot, mask = gpu_forward(xd, cu, threshold, kind, block, causal=causal, sm_scale=sm_scale or 0.0)
    t = t_matrix(cu, H, threshold, kind)
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, block, sm_scale=sm_scale, causal=causal)
    wgs = osk.workgroups(cu, H, block)
    band, mism = compare_masks(mask, ref, t, wgs)
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, block, sm_scale=sm_scale,
                                      forced_mask=mask, causal=causal)
    mx, mean = compare_outputs(o, forced["o"])
    np.testing.assert_array_equal(sk, (mask == osk.TILE_SKIPPED).sum(axis=(2, 3)))
    np.testing.assert_array_equal(tot, ref["total"])
    log(f"  skipped {sk.sum()}/{tot.sum()} band tiles {band} band mismatches {mism} "
        f"max-abs {mx:.2e} mean-abs {mean:.2e}")
    return sk, tot, mask, o


@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-1])
def test_tiny_parity(lam):
    sk, tot, _, _ = _full_parity(CONFIGS["tiny"], lam)
    if lam == 0.0:
        assert sk.sum() == 0
    else:
        assert sk.sum() > 0


@pytest.mark.parametrize("lam", [0.0, 1e-2, 1.0])
def test_ragged_d128_parity(lam):
    sk, tot, mask, _ = _full_parity(RAGGED, lam)
    assert tot[2].sum() == 0 and np.all(mask[2] == osk.TILE_NONE)
    if lam > 0:
        assert sk.sum() > 0


@pytest.mark.parametrize("head_dim,block", [(64, 128), (128, 64)])
def test_other_tile_shapes(head_dim, block):
    cfg = VideoTokenConfig("mixed", ((4, 13, 20), (1, 5, 9)), num_heads=2, head_dim=head_dim, sigma=0.5,
                           block=block, seed=9)
    sk, _, _, _ = _full_parity(cfg, 1e-1, block=block)
    assert sk.sum() > 0


def test_varlen_per_head_scale_factor():
    # per-head scale factors; heads 0-1 dense (sf = 0), lambda_bh = sf_h / S_b
    sf = [0.0, 0.0, 60.0]
    sk, tot, mask, _ = _full_parity(RAGGED, sf, kind="scale_factor")
    assert sk[:, :2].sum() == 0 and sk[:, 2].sum() > 0
    # 300 / 64 keys is lambda > 1 on the shortest sequence: refused, nothing launched
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    with pytest.raises(ssa.SSAError) as e:
        ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, [0.0, 0.0, 300.0], kind="scale_factor", block=128)
    assert e.value.status == ssa.SSA_ERR_THRESHOLD_RANGE


def test_calibration_counts_and_fit():
    import torch
    import skip_softmax_video_amd as ssa
    cfg = RAGGED
    x, xd, cu = _inputs(cfg)
    xf = _f64(x)
    lams = np.geomspace(1e-6, 0.7, 16)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block)
    torch.cuda.synchronize()
    counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
    wgs = osk.workgroups(cu, cfg.num_heads, cfg.block)
    # the calibration output is the dense output, bit for bit
    o0, _, _, _ = gpu_forward(xd, cu, 0.0, "lambda", cfg.block, mask=False)
    np.testing.assert_array_equal(o_cal.float().cpu().numpy(), o0)
    # counts equal the forward's skipped tiles at each lambda_k, exactly
    ts = np.log2(lams)
    ref_d = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, -math.inf, cfg.block, fast=True)["d"]
    cal_ref = osk.calibration_counts(xf["q"], xf["k"], xf["v"], cu, ts, cfg.block)
    np.testing.assert_array_equal(tiles, cal_ref["tiles"])
    total_band = 0
    for kk, lam in enumerate(lams):
        _, _, _, mask = gpu_forward(xd, cu, lam, "lambda", cfg.block)
        per_wg = np.array([(mask[b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs])
        np.testing.assert_array_equal(counts[:, kk], per_wg)
        band = np.array([np.sum(np.abs(ref_d[b, h, i] - ts[kk]) <= 1e-3) for (b, h, i) in wgs])
        assert np.all(np.abs(counts[:, kk] - cal_ref["counts"][:, kk]) <= band)
        total_band += band.sum()
    log(f"  calibration counts ok; band tiles over 16 thresholds: {total_band}")
    # per-sequence sparsity and the log-space fit through the C ABI
    sp = ssa.calibration_sparsity(cu, cfg.num_heads, cfg.head_dim, cfg.block, counts, tiles)
    nwg0 = cfg.num_heads * osk.n_tiles(int(cu[1] - cu[0]), cfg.block)  # the 3072-token sequence
    fit = ssa.calibration_fit(lams, sp[0], float(cu[1] - cu[0]))
    ref_sp = cal_ref["counts"][:nwg0].sum(0) / cal_ref["tiles"][:nwg0].sum()
    ref_fit = oc.fit_exponential_logspace(lams, ref_sp, float(cu[1] - cu[0]))
    assert fit.b == pytest.approx(ref_fit.b, rel=1e-3)
    assert fit.a == pytest.approx(ref_fit.a, rel=1e-3)


def test_determinism():
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    r1 = gpu_forward(xd, cu, 1e-2, "lambda", 128)
    r2 = gpu_forward(xd, cu, 1e-2, "lambda", 128)
    for a, b in zip(r1, r2):
        np.testing.assert_array_equal(a, b)
    c1 = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, [1e-4, 1e-2], block=128)
    c2 = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, [1e-4, 1e-2], block=128)
    torch.cuda.synchronize()
    for a, b in zip(c1, c2):
        assert torch.equal(a, b)


def _guarded(n, dtype, pad, fill):
    """A device buffer of n elements with `pad` canary elements on each side."""
    import torch
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n]


@pytest.mark.parametrize("causal", [False, True])
def test_canaries_around_counters_mask_and_calibration_outputs(causal):
    """Every output the kernels write (skipped/total counters, the tile mask,
    the output rows, calibration counts and tiles) sits between canary
    regions; after the forward and the calibration pass the canaries are
    unchanged, so no write lands outside the buffer the caller was asked for.
    The ragged batch includes an empty sequence and a single partial tile."""
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    T, H, D = xd["q"].shape
    B, blk = len(cu) - 1, RAGGED.block
    prob, _ = ssa.make_problem(xd["q"], cu, blk)
    nq, nk = ssa.tile_mask_dims(prob)
    nwg = ssa.calib_num_workgroups(prob)
    lams = np.geomspace(1e-6, 0.7, 16)
    c64 = -0x21524111  # 0xDEADBEEF-like pattern in each canary
    sk_buf, sk = _guarded(B * H, torch.int64, 8, c64)
    tt_buf, tt = _guarded(B * H, torch.int64, 8, c64)
    m_buf, m = _guarded(B * H * nq * nk, torch.uint8, 64, 0xA5)
    o_buf, o = _guarded(T * H * D, torch.bfloat16, 64, 3.0)
    c_buf, c = _guarded(nwg * lams.size, torch.int32, 16, c64)
    t_buf, tl = _guarded(nwg, torch.int32, 16, c64)
    ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, 1e-2, block=blk, out=o.view(T, H, D), skipped=sk, total=tt,
                 tile_mask=m.view(B, H, nq, nk), causal=causal)
    ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=blk, out=o.view(T, H, D),
                       counts=c.view(nwg, lams.size), tiles=tl, causal=causal)
    torch.cuda.synchronize()
    for name, buf, pad, fill in (("skipped", sk_buf, 8, c64), ("total", tt_buf, 8, c64), ("mask", m_buf, 64, 0xA5),
                                 ("out", o_buf, 64, 3.0), ("counts", c_buf, 16, c64), ("tiles", t_buf, 16, c64)):
        head, tail = buf[:pad], buf[buf.numel() - pad:]
        assert torch.all(head == fill) and torch.all(tail == fill), f"{name}: a canary was overwritten"
    # and the guarded buffers hold real results: totals per head, tiles per work-group
    nqs = [osk.n_tiles(int(cu[b + 1] - cu[b]), blk) for b in range(B)]
    want = [n * (n + 1) // 2 if causal else n * n for n in nqs]
    np.testing.assert_array_equal(tt.cpu().numpy().reshape(B, H), np.array([[w] * H for w in want]))
    assert int(tl.sum()) == sum(w * H for w in want)


@pytest.mark.parametrize("head_dim,block", [(64, 64), (128, 128)])
def test_untouched_memory_outside_valid_rows(head_dim, block):
    """Output rows of other heads / padding stay untouched (strided layout with a gap)."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg = VideoTokenConfig("gap", ((1, 10, 20),), num_heads=2, head_dim=head_dim, sigma=0.5, block=block, seed=3)
    x = make_inputs(cfg)
    T, H, D = x["q"].shape
    big = {}
    for n in ("q", "k", "v"):
        buf = torch.zeros((T, H + 1, D), dtype=torch.bfloat16, device="cuda")  # head slot H is padding
        buf[:, :H] = to_device(x[n])
        big[n] = buf[:, :H]
    out_buf = torch.full((T, H + 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    o = ssa.attn_fwd(big["q"], big["k"], big["v"], x["cu_seqlens"], 0.0, block=block, out=out_buf[:, :H])
    torch.cuda.synchronize()
    assert torch.all(out_buf[:, H] == 7.0)
    ref = osk.skip_softmax_forward(*(to_f64(x[n]) for n in ("q", "k", "v")), x["cu_seqlens"], -math.inf, block)
    compare_outputs(o.float().cpu().numpy(), ref["o"])


def _sampled_parity(cfg, lams, heads, per_head, causal=False, kind="lambda", counts_out=None):
    """Full-size launch; outputs and skip bits checked on sampled Q-blocks
    (first, last/partial and random ones) that the oracle computes one by one.
    Each entry of `lams` is one threshold for every head, or one per head, of `kind`.
    `counts_out`, if given, receives each launch's skipped-tile counts [B, H]."""
    x, xd, cu = _inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    scale = osk.default_sm_scale(cfg.head_dim)
    qbs = sample_qblocks(cu, H, blk, heads, per_head, seed=cfg.seed)
    fracs = []
    for lam in lams:
        log(f"[{cfg.name}] {kind}={np.unique(lam)} causal={causal}: GPU forward (full launch)")
        o, sk, tot, mask = gpu_forward(xd, cu, lam, kind, blk, causal=causal)
        t = t_matrix(cu, H, lam, kind)
        nqs = [osk.n_tiles(int(cu[b + 1] - cu[b]), blk) for b in range(len(cu) - 1)]
        want_tot = np.array([[n * (n + 1) // 2 if causal else n * n] * H for n in nqs])
        np.testing.assert_array_equal(tot, want_tot)
        np.testing.assert_array_equal(sk, (mask == osk.TILE_SKIPPED).sum(axis=(2, 3)))
        log(f"  oracle on {len(qbs)} sampled Q-blocks")
        band = mism = 0
        worst_max, sum_abs, n_abs = 0.0, 0.0, 0
        cache = {}
        for (b, h, i) in qbs:
            s0, s1 = int(cu[b]), int(cu[b + 1])
            if (b, h) not in cache:
                cache.clear()
                cache[(b, h)] = (to_f64(x["k"][s0:s1, h]), to_f64(x["v"][s0:s1, h]))
            kh, vh = cache[(b, h)]
            r0, r1 = i * blk, min(s1 - s0, (i + 1) * blk)
            qh = to_f64(x["q"][s0 + r0:s0 + r1, h])
            nk = i + 1 if causal else osk.n_tiles(s1 - s0, blk)
            d, _ = osk.tile_stats_fast(qh, kh, blk, scale, causal_row0=r0 if causal else None)
            ref_skip = d < t[b, h]
            gpu_skip = mask[b, h, i, :nk] == osk.TILE_SKIPPED
            assert np.all(mask[b, h, i, nk:] == osk.TILE_NONE)
            near = np.abs(d - t[b, h]) <= 1e-3
            hard = (gpu_skip != ref_skip) & ~near
            assert not np.any(hard), f"skip mismatch at {(b, h, i)} tiles {np.nonzero(hard)[0][:8]}"
            band += int(near.sum())
            mism += int(((gpu_skip != ref_skip) & near).sum())
            ref = osk.skip_softmax_qblock(qh, kh, vh, t[b, h], blk, scale, forced_skip=gpu_skip,
                                          causal_row0=r0 if causal else None)
            diff = np.abs(o[s0 + r0:s0 + r1, h] - ref["o"])
            worst_max = max(worst_max, float(diff.max()))
            sum_abs += float(diff.sum())
            n_abs += diff.size
        mean = sum_abs / n_abs
        assert worst_max <= 2e-2 and mean <= 2e-3, f"output mismatch max {worst_max:.3e} mean {mean:.3e}"
        frac = sk.sum() / tot.sum()
        log(f"  sparsity {frac:.4f} band {band} band-mismatch {mism} max-abs {worst_max:.2e} mean-abs {mean:.2e}")
        fracs.append(frac)
        if counts_out is not None:
            counts_out.append(sk)
    return fracs


# ---- full-size parity against the oracle's fixtures ------------------------------------
# tests/golden/fullsize_*.npz hold the oracle's per-work-group skip statistics
# for whole configs (written by tests/golden/make_fullsize_fixtures.py from
# oracle/ and synth only); the GPU runs the same configs at full size.
def _check_dense(cu, H, blk, sk, tot, mask):
    assert sk.sum() == 0
    nqs = [osk.n_tiles(int(cu[b + 1] - cu[b]), blk) for b in range(len(cu) - 1)]
    np.testing.assert_array_equal(tot, np.array([[n * n] * H for n in nqs]))
    for b, n in enumerate(nqs):
        assert np.all(mask[b, :, :n, :n] == osk.TILE_KEPT)


def test_wan5b_full_tile_mask_and_per_head_counts():
    """WAN-5B-like config (S=16,384, H=24) at lambda = 1e-3 and dense: the
    whole tile mask against the oracle's (mismatches only inside the 1e-3
    band), per-head skipped tiles reported and checked, and outputs of every
    head (4 Q-blocks each, the last one included) against the oracle."""
    cfg, fx = CONFIGS["wan5b"], load_fixture("wan5b")
    x, xd, cu = _inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    n = osk.n_tiles(int(cu[1]), blk)
    o0, sk0, tot0, m0 = gpu_forward(xd, cu, 0.0, "lambda", blk)
    _check_dense(cu, H, blk, sk0, tot0, m0)
    o, sk, tot, mask = gpu_forward(xd, cu, 1e-3, "lambda", blk)
    skip = mask[0] == osk.TILE_SKIPPED
    want = np.unpackbits(fx["skip_bits"])[:H * n * n].reshape(H, n, n).astype(bool)
    band = np.unpackbits(fx["band_bits"])[:H * n * n].reshape(H, n, n).astype(bool)
    hard = (skip != want) & ~band
    assert not hard.any(), f"{int(hard.sum())} tiles differ outside the band, first at {np.argwhere(hard)[0]}"
    per_head = skip.sum(axis=(1, 2))
    np.testing.assert_array_equal(sk[0], per_head)
    assert np.all(np.abs(per_head - fx["skip_per_head"]) <= band.sum(axis=(1, 2)))
    log(f"  per-head skipped tiles of {n * n} (GPU / oracle):")
    log("  " + " ".join(f"{h}:{int(a)}/{int(b)}" for h, (a, b) in enumerate(zip(per_head, fx["skip_per_head"]))))
    log(f"  band tiles {int(band.sum())}, differing inside the band {int((skip != want).sum())}")
    t = t_matrix(cu, H, 1e-3, "lambda")
    qbs = sample_qblocks(cu, H, blk, range(H), 4, seed=cfg.seed)
    mx, mean = sampled_outputs_vs_oracle(x, cu, o, mask, t, blk, qbs)
    mx0, mean0 = sampled_outputs_vs_oracle(x, cu, o0, m0, t_matrix(cu, H, 0.0, "lambda"), blk, qbs[::4])
    log(f"  outputs of {len(qbs)} Q-blocks: max-abs {mx:.2e} mean-abs {mean:.2e}; dense max-abs {mx0:.2e}")


def test_headline_forward_matches_oracle_fixture():
    """Headline config (S=75,600, H=40): at lambda = 8e-3 and lambda = 1 the
    skip statistics of all 23,640 work-groups against the oracle's (exact
    where no tile of a work-group lies in the 1e-3 band), per-head counts,
    dense mode, and outputs of every head (16 Q-blocks each at lambda = 8e-3,
    4 in dense mode, the partial last one included) against the oracle under
    the GPU's decisions."""
    cfg, fx = CONFIGS["headline"], load_fixture("headline")
    x, xd, cu = _inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    o0, sk0, tot0, m0 = gpu_forward(xd, cu, 0.0, "lambda", blk)
    _check_dense(cu, H, blk, sk0, tot0, m0)
    qbs = sample_qblocks(cu, H, blk, range(H), 16, seed=cfg.seed)
    for col, lam in ((16, 8e-3), (17, 1.0)):
        assert fx["column_value"][col] == lam
        o, sk, tot, mask = gpu_forward(xd, cu, lam, "lambda", blk)
        stats = mask_workgroup_stats(mask, cu, H, blk)
        res = compare_workgroup_stats(stats, fx, col)
        nq = osk.n_tiles(int(cu[1]), blk)
        per_head_gpu = stats[:, 0].reshape(H, nq).sum(1)
        per_head_ref = fx["count"][:, col].astype(np.int64).reshape(H, nq).sum(1)
        band_head = fx["band"][:, col].astype(np.int64).reshape(H, nq).sum(1)
        np.testing.assert_array_equal(sk[0], per_head_gpu)
        assert np.all(np.abs(per_head_gpu - per_head_ref) <= band_head)
        log(f"  lambda {lam}: sparsity {sk.sum() / tot.sum():.4f} (oracle {per_head_ref.sum() / tot.sum():.4f}); "
            f"{res}")
        if col == 16:
            mx, mean = sampled_outputs_vs_oracle(x, cu, o, mask, t_matrix(cu, H, lam, "lambda"), blk, qbs)
            log(f"  outputs of {len(qbs)} Q-blocks: max-abs {mx:.2e} mean-abs {mean:.2e}")
    qbs0 = sample_qblocks(cu, H, blk, range(H), 4, seed=cfg.seed + 1)
    mx0, mean0 = sampled_outputs_vs_oracle(x, cu, o0, m0, t_matrix(cu, H, 0.0, "lambda"), blk, qbs0)
    log(f"  dense outputs of {len(qbs0)} Q-blocks: max-abs {mx0:.2e} mean-abs {mean0:.2e}")


@pytest.mark.parametrize("name", ["calib", "headline"])
def test_headline_calibration_pass_matches_oracle_fixture(name):
    """Calibration pass at the headline shape with 16 thresholds log-spaced over
    [1e-6, 0.7] (the calibration config's own sample, and the headline sample):
    every work-group's 16 counts against the oracle's (exact where no tile of
    the work-group lies in the 1e-3 band), the fitted (a, b) through the C ABI
    within 1e-3 relative of the oracle's fit of its own counts, and the
    resolved lambdas for targets 0.25 / 0.5 / 0.7 against the oracle's resolve."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg, fx = CONFIGS[name], load_fixture(name)
    x, xd, cu = _inputs(cfg)
    lams = np.geomspace(1e-6, 0.7, 16)
    np.testing.assert_array_equal(fx["column_value"][:16], lams)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block)
    torch.cuda.synchronize()
    counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
    res = compare_calibration_counts(counts, tiles, fx, list(range(16)))
    S = int(cu[1] - cu[0])
    sp = ssa.calibration_sparsity(cu, cfg.num_heads, cfg.head_dim, cfg.block, counts, tiles)[0]
    np.testing.assert_allclose(sp, fx["sparsity"], rtol=0, atol=res["band_tiles"] / tiles.sum() + 1e-15)
    fit = ssa.calibration_fit(lams, sp, float(S))
    assert fit.a == pytest.approx(float(fx["fit_a"]), rel=1e-3)
    assert fit.b == pytest.approx(float(fx["fit_b"]), rel=1e-3)
    assert fit.n_used == int(fx["fit_n_used"])
    log(f"  [{name}] counts {res}; sparsity {np.round(sp, 4)}")
    log(f"  fit a={fit.a:.6g} (oracle {float(fx['fit_a']):.6g}) b={fit.b:.6g} (oracle {float(fx['fit_b']):.6g})")
    for tgt in (0.25, 0.5, 0.7):
        st, lam, _ = ssa.resolve_threshold(S, target_sparsity=tgt, a=fit.a, b=fit.b, s_min=fit.s_min,
                                           s_max=fit.s_max)
        ref = oc.resolve_threshold(oc.ThresholdSpec(target_sparsity=tgt, a=float(fx["fit_a"]),
                                                    b=float(fx["fit_b"]), s_min=float(fx["fit_s_min"]),
                                                    s_max=float(fx["fit_s_max"])), S)
        assert st == ref[0]
        assert lam == pytest.approx(ref[1], rel=2e-3)  # a (1e-3) and exp(b t) (<= 1e-3 * |b t|)
        log(f"  target {tgt}: lambda {lam:.6g} (oracle {ref[1]:.6g}) status {ssa.status_string(st)}")


def test_varlen_full_size_per_head_scale_factor():
    """The varlen batch at full size (75,600 / 32,760 / 8,190 tokens, H=40):
    per-head scale factors with heads 0-1 forced dense, lambda_bh = sf_h / S_b.
    sf = 650 puts lambda near 8.6e-3 on the longest sequence. All 36,440
    work-groups' skip statistics against the oracle's fixture, per-(sequence,
    head) counts, and outputs of every head of every sequence (2 Q-blocks
    each, the partial last ones included)."""
    cfg, fx = CONFIGS["varlen"], load_fixture("varlen")
    sf = np.full(cfg.num_heads, 650.0)
    sf[:2] = 0.0
    np.testing.assert_array_equal(fx["scale_factor"][0], sf)
    x, xd, cu = _inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    o, sk, tot, mask = gpu_forward(xd, cu, sf, "scale_factor", blk)
    stats = mask_workgroup_stats(mask, cu, H, blk)
    res = compare_workgroup_stats(stats, fx, 0)
    assert sk[:, :2].sum() == 0 and np.all(sk[:, 2:] > 0)
    w = 0
    for b in range(len(cu) - 1):
        nq = osk.n_tiles(int(cu[b + 1] - cu[b]), blk)
        ref_bh = fx["count"][w:w + H * nq, 0].astype(np.int64).reshape(H, nq).sum(1)
        band_bh = fx["band"][w:w + H * nq, 0].astype(np.int64).reshape(H, nq).sum(1)
        assert np.all(np.abs(sk[b] - ref_bh) <= band_bh)
        np.testing.assert_array_equal(tot[b], np.full(H, nq * nq))
        log(f"  sequence {b} (S={int(cu[b + 1] - cu[b])}): sparsity {sk[b].sum() / tot[b].sum():.4f} "
            f"(oracle {ref_bh.sum() / tot[b].sum():.4f})")
        w += H * nq
    log(f"  {res}")
    t = t_matrix(cu, H, sf, "scale_factor")
    qbs = sample_qblocks(cu, H, blk, range(H), 2, seed=cfg.seed)
    mx, mean = sampled_outputs_vs_oracle(x, cu, o, mask, t, blk, qbs)
    log(f"  outputs of {len(qbs)} Q-blocks: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_denoising_schedule_gating():
    """Gating feeds the forward: over a 40-step flow schedule with cutoff 0.86,
    the first 14 forwards run dense and the rest skip exactly the oracle's
    tiles at lambda = sf / S (sf from the layer's override)."""
    import skip_softmax_video_amd as ssa
    from oracle import gating as og
    cfg = CONFIGS["tiny"]
    x, xd, cu = _inputs(cfg)
    xf = _f64(x)
    S, H = int(cu[1]), cfg.num_heads
    sched = ssa.flow_timesteps(40, 1000, 3.0)
    layer, cutoff = "transformer.blocks.3.attn1", 0.86
    ovr = [("blocks.3.*", 0.1 * S)]  # lambda = 0.1 for this layer
    lam_ref = og.gate_layer(layer, [0.0], 0.0, cutoff, (), ovr)[1] / S
    t_ref = np.full((1, H), math.log2(lam_ref))
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t_ref, cfg.block)
    dense_ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, np.full((1, H), -math.inf), cfg.block)
    n_dense = 0
    for i, t in enumerate(sched):
        rule, sf = ssa.gate_layer(layer, [t], 0.0, cutoff, ["blocks.0.attn1"], ovr)
        assert (rule, sf) == og.gate_layer(layer, [t], 0.0, cutoff, ["blocks.0.attn1"], ovr)
        o, sk, tot, mask = gpu_forward(xd, cu, sf, "scale_factor", cfg.block)
        if rule == ssa.GATE_TIMESTEP:
            n_dense += 1
            assert sk.sum() == 0
            compare_outputs(o, dense_ref["o"])
        else:
            compare_masks(mask, ref, t_ref, osk.workgroups(cu, H, cfg.block))
            assert sk.sum() > 0
    assert n_dense == 14
    log(f"  40 forwards: {n_dense} dense, {40 - n_dense} skip-softmax")


def test_pooled_calibration_multi_sample_multi_shape():
    """Two calibration passes (three sequences of 1,024 tokens and one of 512,
    two samples) pooled by key length through the C ABI, then the log- and
    linear-space fits, against the oracle's pool of its own counts."""
    import torch
    import skip_softmax_video_amd as ssa
    second = VideoTokenConfig("tiny_b", ((4, 16, 16), (2, 16, 16), (4, 16, 16)), num_heads=2, head_dim=64,
                              sigma=0.5, block=64, seed=11)
    lams = np.geomspace(1e-6, 0.7, 16)
    ts = np.log2(lams)
    pool = ssa.CalibrationPool(16, max_groups=4)
    ref_pool = oc.CalibPool(16)
    band_by_key = {}
    for cfg in (CONFIGS["tiny"], second):
        x, xd, cu = _inputs(cfg)
        xf = _f64(x)
        log(f"[{cfg.name}] calibration pass, sequences {np.diff(cu).tolist()}")
        _, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block)
        torch.cuda.synchronize()
        counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
        pool.add(cu, cfg.num_heads, cfg.head_dim, cfg.block, counts, tiles)
        ref = osk.calibration_counts(xf["q"], xf["k"], xf["v"], cu, ts, cfg.block)
        ref_pool.add(ref["counts"], ref["tiles"], cu, cfg.num_heads, cfg.block)
        d = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, -math.inf, cfg.block, fast=True)["d"]
        for n, (b, h, i) in enumerate(osk.workgroups(cu, cfg.num_heads, cfg.block)):
            key = int(cu[b + 1] - cu[b])
            band_by_key.setdefault(key, np.zeros(16, np.int64))
            band_by_key[key] += np.array([np.sum(np.abs(d[b, h, i] - t) <= 1e-3) for t in ts])
    got, exp = pool.groups, ref_pool.groups
    assert list(got) == list(exp) == [1024, 512]
    for key in exp:
        assert got[key][1] == exp[key][1]
        assert np.all(np.abs(got[key][0] - exp[key][0]) <= band_by_key[key])
    lam_g, sp_g, sk_g = pool.points(lams)
    lam_r, sp_r, sk_r = ref_pool.points(lams)
    for space, ofit in (("log", oc.fit_exponential_logspace), ("linear", oc.fit_exponential_linear)):
        g = ssa.calibration_fit(lam_g, sp_g, sk_g, space=space)
        r = ofit(lam_r, sp_r, sk_r)
        log(f"  {space}: a={g.a:.5g} b={g.b:.5g} (oracle a={r.a:.5g} b={r.b:.5g}) points {g.n_used}")
        assert g.b == pytest.approx(r.b, rel=1e-3) and g.a == pytest.approx(r.a, rel=1e-3)


# ---- causal (prefill) form ---------------------------------------------------------
@pytest.mark.parametrize("lam", [0.0, 1e-2, 1.0])
def test_causal_tiny_parity(lam):
    sk, tot, mask, _ = _full_parity(CONFIGS["tiny"], lam, causal=True)
    nq = 1024 // 64
    assert np.all(tot == nq * (nq + 1) // 2)
    assert (sk.sum() == 0) == (lam == 0.0)


@pytest.mark.parametrize("lam", [0.0, 1e-2])
def test_causal_ragged_d128_parity(lam):
    _full_parity(RAGGED, lam, causal=True)


def _calibration_matches_forward(cfg, lams, causal):
    """Calibration pass: dense output bit-equal to the lambda = 0 forward,
    tiles per work-group as the oracle, counts equal to the forward's skipped
    tiles at each lambda exactly, and to the oracle's outside the 1e-3 band."""
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(cfg)
    xf = _f64(x)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block, causal=causal)
    torch.cuda.synchronize()
    counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
    wgs = osk.workgroups(cu, cfg.num_heads, cfg.block)
    ts = np.log2(lams)
    ref = osk.calibration_counts(xf["q"], xf["k"], xf["v"], cu, ts, cfg.block, causal=causal)
    np.testing.assert_array_equal(tiles, ref["tiles"])
    if causal:
        np.testing.assert_array_equal(tiles, [i + 1 for (_, _, i) in wgs])
    o0, _, _, _ = gpu_forward(xd, cu, 0.0, "lambda", cfg.block, mask=False, causal=causal)
    np.testing.assert_array_equal(o_cal.float().cpu().numpy(), o0)
    d = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, -math.inf, cfg.block, fast=True, causal=causal)["d"]
    for kk, lam in enumerate(lams):
        _, _, _, mask = gpu_forward(xd, cu, lam, "lambda", cfg.block, causal=causal)
        per_wg = np.array([(mask[b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs])
        np.testing.assert_array_equal(counts[:, kk], per_wg)
        with np.errstate(invalid="ignore"):
            band = np.array([np.sum(np.abs(d[b, h, i] - ts[kk]) <= 1e-3) for (b, h, i) in wgs])
        assert np.all(np.abs(counts[:, kk] - ref["counts"][:, kk]) <= band)
    return counts


def test_causal_calibration_counts():
    _calibration_matches_forward(RAGGED, np.geomspace(1e-5, 0.7, 8), causal=True)


def _shape_cfg(head_dim, block):
    # two sequences, 2080 and 45 tokens: several tiles, a ragged last tile, a one-tile sequence
    return VideoTokenConfig("shape", ((8, 13, 20), (1, 5, 9)), num_heads=2, head_dim=head_dim, sigma=0.5,
                            block=block, seed=11)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("head_dim,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_calibration_all_tile_shapes(head_dim, block, causal):
    counts = _calibration_matches_forward(_shape_cfg(head_dim, block), np.geomspace(1e-4, 1.0, 6), causal)
    assert counts.sum() > 0


def test_calibration_64_thresholds():
    """The largest threshold list (64: one per lane of a wave), including a
    repeated value: every column matches the forward at its lambda exactly."""
    lams = np.geomspace(1e-8, 1.0, 63)
    lams = np.sort(np.concatenate([lams, lams[40:41]]))
    assert lams.size == 64
    counts = _calibration_matches_forward(_shape_cfg(128, 128), lams, causal=False)
    np.testing.assert_array_equal(counts[:, 40], counts[:, 41])
    assert np.all(np.diff(counts, axis=1) >= 0) and counts[:, -1].sum() > counts[:, 0].sum()


@pytest.mark.parametrize("head_dim,block", [(64, 128), (128, 64)])
def test_causal_other_tile_shapes(head_dim, block):
    sk, tot, _, _ = _full_parity(_shape_cfg(head_dim, block), 1.0, causal=True)
    assert sk.sum() > 0


def test_causal_headline_sampled_parity():
    fr = _sampled_parity(CONFIGS["headline"], [0.0, 8e-3], heads=[0, 39], per_head=3, causal=True)
    assert fr[0] == 0.0 and fr[1] > 0.1


# ---- FP8 (e4m3) variant -------------------------------------------------------------
def _fp8_inputs(cfg):
    import torch
    from synth import e4m3_bits_to_f32, make_fp8_inputs
    x = make_inputs(cfg)
    f = make_fp8_inputs(x)
    xd = {n: torch.from_numpy(np.ascontiguousarray(f[n + "8"])).cuda() for n in ("q", "k", "v")}
    scales = (f["scale_q"], f["scale_k"], f["scale_v"])
    xf = {n: e4m3_bits_to_f32(f[n + "8"]).astype(np.float64) * f["scale_" + n] for n in ("q", "k", "v")}
    return xd, xf, scales, x["cu_seqlens"]


def _fp8_forward(xd, cu, lam, block, scales, causal=False, mask=True):
    import torch
    import skip_softmax_video_amd as ssa
    B = len(cu) - 1
    T, H, D = xd["q"].shape
    skipped = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    total = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    prob, _ = ssa.make_problem(xd["q"], cu, block, scales=scales)
    nq, nk = ssa.tile_mask_dims(prob)
    tm = torch.empty((B, H, nq, nk), dtype=torch.uint8, device="cuda") if mask else None
    o = ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, lam, block=block, skipped=skipped, total=total,
                     tile_mask=tm, causal=causal, scales=scales)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), skipped.cpu().numpy().reshape(B, H), total.cpu().numpy().reshape(B, H),
            None if tm is None else tm.cpu().numpy())


def _fp8_full_parity(cfg, lam, causal=False):
    from tests._parity import fp8_row_bound
    xd, xf, scales, cu = _fp8_inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    log(f"[{cfg.name} fp8] lambda={lam} causal={causal} scales={tuple(round(s, 6) for s in scales)}")
    o, sk, tot, mask = _fp8_forward(xd, cu, lam, blk, scales, causal=causal)
    t = t_matrix(cu, H, lam, "lambda")
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, causal=causal)
    band, mism = compare_masks(mask, ref, t, osk.workgroups(cu, H, blk))
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, forced_mask=mask, causal=causal)
    np.testing.assert_array_equal(sk, (mask == osk.TILE_SKIPPED).sum(axis=(2, 3)))
    np.testing.assert_array_equal(tot, ref["total"])
    scale = osk.default_sm_scale(cfg.head_dim)
    worst_ratio, mean_abs = 0.0, []
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for h in range(H):
            for i in range(osk.n_tiles(s1 - s0, blk)):
                r0, r1 = i * blk, min(s1 - s0, (i + 1) * blk)
                kept_tiles = mask[b, h, i] == osk.TILE_KEPT
                kept_cols = np.repeat(kept_tiles, blk)[: s1 - s0]
                o_ref = forced["o"][s0 + r0:s0 + r1, h]
                bound = fp8_row_bound(xf["q"][s0 + r0:s0 + r1, h], xf["k"][s0:s1, h], xf["v"][s0:s1, h],
                                      kept_cols, scale, o_ref, causal_row0=r0 if causal else None)
                err = np.abs(o[s0 + r0:s0 + r1, h] - o_ref).max(1)
                assert np.all(err <= bound), f"fp8 output outside its bound at {(b, h, i)}: {err.max():.3e}"
                worst_ratio = max(worst_ratio, float((err / bound).max()))
                mean_abs.append(np.abs(o[s0 + r0:s0 + r1, h] - o_ref).mean())
    log(f"  skipped {sk.sum()}/{tot.sum()} band {band} band-mismatch {mism} mean-abs {np.mean(mean_abs):.2e} "
        f"worst err/bound {worst_ratio:.3f}")
    return sk, tot


@pytest.mark.parametrize("lam", [0.0, 1e-2, 1.0])
def test_fp8_tiny_parity(lam):
    sk, tot = _fp8_full_parity(CONFIGS["tiny"], lam)
    assert (sk.sum() == 0) == (lam == 0.0)


@pytest.mark.parametrize("lam,causal", [(0.0, False), (1e-2, False), (1e-2, True)])
def test_fp8_ragged_d128_parity(lam, causal):
    _fp8_full_parity(RAGGED, lam, causal=causal)


def test_fp8_calibration_counts_match_forward():
    import torch
    import skip_softmax_video_amd as ssa
    xd, xf, scales, cu = _fp8_inputs(RAGGED)
    lams = np.geomspace(1e-5, 0.7, 6)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=RAGGED.block,
                                              scales=scales)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    wgs = osk.workgroups(cu, RAGGED.num_heads, RAGGED.block)
    o0, _, _, _ = _fp8_forward(xd, cu, 0.0, RAGGED.block, scales, mask=False)
    np.testing.assert_array_equal(o_cal.float().cpu().numpy(), o0)
    for kk, lam in enumerate(lams):
        _, _, _, mask = _fp8_forward(xd, cu, lam, RAGGED.block, scales)
        per_wg = np.array([(mask[b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs])
        np.testing.assert_array_equal(counts[:, kk], per_wg)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("head_dim,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_fp8_calibration_all_tile_shapes(head_dim, block, causal):
    """e4m3 calibration pass at every tile shape: counts equal the fp8
    forward's skipped tiles exactly and the oracle's (on the dequantized
    inputs) outside the 1e-3 band; the output equals the lambda = 0 forward."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg = _shape_cfg(head_dim, block)
    xd, xf, scales, cu = _fp8_inputs(cfg)
    lams = np.geomspace(1e-4, 1.0, 6)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=block, scales=scales,
                                              causal=causal)
    torch.cuda.synchronize()
    counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
    wgs = osk.workgroups(cu, cfg.num_heads, block)
    ts = np.log2(lams)
    ref = osk.calibration_counts(xf["q"], xf["k"], xf["v"], cu, ts, block, causal=causal)
    np.testing.assert_array_equal(tiles, ref["tiles"])
    o0, _, _, _ = _fp8_forward(xd, cu, 0.0, block, scales, causal=causal, mask=False)
    np.testing.assert_array_equal(o_cal.float().cpu().numpy(), o0)
    d = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, -math.inf, block, fast=True, causal=causal)["d"]
    for kk, lam in enumerate(lams):
        _, _, _, mask = _fp8_forward(xd, cu, lam, block, scales, causal=causal)
        per_wg = np.array([(mask[b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs])
        np.testing.assert_array_equal(counts[:, kk], per_wg)
        with np.errstate(invalid="ignore"):
            band = np.array([np.sum(np.abs(d[b, h, i] - ts[kk]) <= 1e-3) for (b, h, i) in wgs])
        assert np.all(np.abs(counts[:, kk] - ref["counts"][:, kk]) <= band)
    if not causal:  # causal 128-key tiles of this batch skip one tile at most (oracle)
        assert counts.sum() > 0


def test_fp8_headline_sampled_parity():
    """Full-size e4m3 launch at the headline shape; skip bits and outputs
    checked on sampled Q-blocks against the oracle on the dequantized inputs."""
    from tests._parity import fp8_row_bound
    cfg = CONFIGS["headline"]
    xd, xf, scales, cu = _fp8_inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    scale = osk.default_sm_scale(cfg.head_dim)
    qbs = sample_qblocks(cu, H, blk, [0, 39], 3, seed=cfg.seed)
    S = int(cu[1])
    for lam in (0.0, 8e-3):
        log(f"[headline fp8] lambda={lam}: GPU forward (full launch)")
        o, sk, tot, mask = _fp8_forward(xd, cu, lam, blk, scales)
        t = t_matrix(cu, H, lam, "lambda")
        assert np.all(tot == osk.n_tiles(S, blk) ** 2)
        worst = 0.0
        for (b, h, i) in qbs:
            kh, vh = xf["k"][:, h], xf["v"][:, h]
            r0, r1 = i * blk, min(S, (i + 1) * blk)
            qh = xf["q"][r0:r1, h]
            d, _ = osk.tile_stats_fast(qh, kh, blk, scale)
            near = np.abs(d - t[b, h]) <= 1e-3
            gpu_skip = mask[b, h, i] == osk.TILE_SKIPPED
            assert not np.any((gpu_skip != (d < t[b, h])) & ~near), f"skip mismatch at {(b, h, i)}"
            ref = osk.skip_softmax_qblock(qh, kh, vh, t[b, h], blk, scale, forced_skip=gpu_skip)
            kept_cols = np.repeat(~gpu_skip, blk)[:S]
            bound = fp8_row_bound(qh, kh, vh, kept_cols, scale, ref["o"])
            err = np.abs(o[r0:r1, h] - ref["o"]).max(1)
            assert np.all(err <= bound), f"fp8 output outside its bound at {(b, h, i)}: {err.max():.3e}"
            worst = max(worst, float((err / bound).max()))
        log(f"  sparsity {sk.sum() / tot.sum():.4f} worst err/bound {worst:.3f}")


# ---- launch splitting, limits and degenerate shapes ---------------------------------
def test_launch_splitting_many_sequences_per_head_thresholds():
    """40 sequences x 16 heads: more than 32 sequences and 512 (sequence, head)
    thresholds per launch, so the host splits the batch into several launches.
    Per-head scale factors (lambda = sf / S_b) make every launch's threshold
    table different; one sequence is empty."""
    from synth.video_tokens import make_random_inputs
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(64, 300, 40)]  # >= 64 keys: lambda = sf / S stays <= 1
    lens[17] = 0
    H, D, blk = 16, 64, 64
    x = make_random_inputs(lens, H, D, seed=22, scale=1.5)
    xd = {n: to_device(x[n]) for n in ("q", "k", "v")}
    xf = {n: to_f64(x[n]) for n in ("q", "k", "v")}
    cu = x["cu_seqlens"]
    sf = np.concatenate([[0.0], np.geomspace(0.5, 60.0, H - 1)])
    log(f"[split] B={len(lens)} H={H} total tokens {int(cu[-1])}")
    o, sk, tot, mask = gpu_forward(xd, cu, sf, "scale_factor", blk)
    t = t_matrix(cu, H, sf, "scale_factor")
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk)
    band, mism = compare_masks(mask, ref, t, osk.workgroups(cu, H, blk))
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, forced_mask=mask)
    mx, mean = compare_outputs(o, forced["o"])
    np.testing.assert_array_equal(tot, ref["total"])
    assert sk[:, 0].sum() == 0 and sk.sum() > 0
    log(f"  output max-abs {mx:.3e} mean-abs {mean:.3e}")
    log(f"  skipped {sk.sum()}/{tot.sum()} band {band} band-mismatch {mism}")


def test_max_heads_and_tiny_sequences():
    """512 heads (the limit), sequences of 1, 2 and 129 tokens."""
    from synth.video_tokens import make_random_inputs
    lens = [1, 2, 129]
    H, D, blk = 512, 64, 64
    x = make_random_inputs(lens, H, D, seed=23, scale=2.0)
    xd = {n: to_device(x[n]) for n in ("q", "k", "v")}
    xf = {n: to_f64(x[n]) for n in ("q", "k", "v")}
    cu = x["cu_seqlens"]
    o, sk, tot, mask = gpu_forward(xd, cu, 0.5, "lambda", blk)
    t = t_matrix(cu, H, 0.5, "lambda")
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, fast=True)
    compare_masks(mask, ref, t, osk.workgroups(cu, H, blk))
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, forced_mask=mask, fast=True)
    mx, mean = compare_outputs(o, forced["o"])
    np.testing.assert_array_equal(tot, ref["total"])
    log(f"  output max-abs {mx:.3e} mean-abs {mean:.3e}")
    import skip_softmax_video_amd as ssa
    with pytest.raises(ssa.SSAError):
        x2 = make_random_inputs([8], 513, 64, seed=1)
        d2 = {n: to_device(x2[n]) for n in ("q", "k", "v")}
        ssa.attn_fwd(d2["q"], d2["k"], d2["v"], x2["cu_seqlens"], 0.1, block=64)


def test_large_v_rounding_bound():
    """Separate large-|V| case (V ~ N(0, 4^2), sharp rows): |O| reaches max|V|,
    outside the range the 2e-2 bound is stated for, so the check is the bound
    derived from the bf16 roundings of P and O (2^-8 max|V| + 2^-8 |O| + 1e-3
    per element, mean-abs 2e-3 times V's scale)."""
    from synth.video_tokens import make_random_inputs
    lens = [1, 70, 129, 300]
    H, D, blk = 8, 64, 64
    x = make_random_inputs(lens, H, D, seed=24, scale=2.0, v_scale=4.0)
    xd = {n: to_device(x[n]) for n in ("q", "k", "v")}
    xf = {n: to_f64(x[n]) for n in ("q", "k", "v")}
    cu = x["cu_seqlens"]
    o, sk, tot, mask = gpu_forward(xd, cu, 0.25, "lambda", blk)
    t = t_matrix(cu, H, 0.25, "lambda")
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk)
    compare_masks(mask, ref, t, osk.workgroups(cu, H, blk))
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, forced_mask=mask)
    mx, mean = compare_outputs_derived(o, forced["o"], np.abs(xf["v"]).max(), v_scale=4.0)
    log(f"  max|V| {np.abs(xf['v']).max():.2f} output max-abs {mx:.3e} mean-abs {mean:.3e}")


@pytest.mark.parametrize("head_dim,block", [(64, 64), (64, 128), (128, 64)])
def test_fp8_other_tile_shapes(head_dim, block):
    cfg = VideoTokenConfig("mixed8", ((4, 13, 20), (1, 5, 9)), num_heads=2, head_dim=head_dim, sigma=0.5,
                           block=block, seed=9)
    sk, _ = _fp8_full_parity(cfg, 1e-1)
    assert sk.sum() > 0


@pytest.mark.parametrize("fp8", [False, True])
def test_headline_calibration_counts_equal_forward_skips(fp8):
    """At the full headline size the calibration pass counts exactly the tiles
    the forward skips, threshold by threshold (same arithmetic on both sides)."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg = CONFIGS["calib"]
    if fp8:
        xd, _, scales, cu = _fp8_inputs(cfg)
    else:
        x, xd, cu = _inputs(cfg)
        scales = None
    lams = np.geomspace(1e-6, 0.7, 16)
    _, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block, scales=scales)
    torch.cuda.synchronize()
    per_lam = counts.sum(0).cpu().numpy()
    H = cfg.num_heads
    skipped = torch.zeros(H, dtype=torch.int64, device="cuda")
    total = torch.zeros(H, dtype=torch.int64, device="cuda")
    for kk in (0, 5, 8, 12, 15):
        ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, lams[kk], block=cfg.block, skipped=skipped, total=total,
                     scales=scales)
        torch.cuda.synchronize()
        assert int(skipped.sum()) == int(per_lam[kk]), f"lambda {lams[kk]:.3g}: {int(skipped.sum())} vs {per_lam[kk]}"
        assert int(total.sum()) == int(tiles.sum())
    log(f"  fp8={fp8}: calibration counts equal forward skips at 5 of 16 thresholds "
        f"(sparsity {per_lam[0] / int(tiles.sum()):.3f} .. {per_lam[-1] / int(tiles.sum()):.3f})")


# ---- block-scaled (MXFP8) q/k with bf16 v ------------------------------------------------------
def _mx_inputs(cfg):
    """Device tensors (e4m3 q/k bytes, E8M0 block scales, bf16 v) and the
    oracle's fp64 inputs: q/k dequantized exactly, v as bf16."""
    import torch
    from synth import make_mxfp8_qk_inputs, mxfp8_dequantize
    x = make_inputs(cfg)
    m = make_mxfp8_qk_inputs(x)
    xd = {"q": torch.from_numpy(m["q8"]).cuda(), "k": torch.from_numpy(m["k8"]).cuda(), "v": to_device(x["v"])}
    bs = (torch.from_numpy(m["q_bscale"]).cuda(), torch.from_numpy(m["k_bscale"]).cuda())
    xf = {"q": mxfp8_dequantize(m["q8"], m["q_bscale"]), "k": mxfp8_dequantize(m["k8"], m["k_bscale"]),
          "v": to_f64(x["v"])}
    return xd, bs, xf, x["cu_seqlens"]


def _mx_full_parity(cfg, lam, causal=False):
    xd, bs, xf, cu = _mx_inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    log(f"[{cfg.name} mxfp8 q/k] D={cfg.head_dim} block={blk} lambda={lam} causal={causal}")
    o, sk, tot, mask = gpu_forward(xd, cu, lam, "lambda", blk, causal=causal, block_scales=bs)
    t = t_matrix(cu, H, lam, "lambda")
    ref = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, causal=causal)
    band, mism = compare_masks(mask, ref, t, osk.workgroups(cu, H, blk))
    forced = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, t, blk, forced_mask=mask, causal=causal)
    mx, mean = compare_outputs(o, forced["o"])
    np.testing.assert_array_equal(sk, (mask == osk.TILE_SKIPPED).sum(axis=(2, 3)))
    np.testing.assert_array_equal(tot, ref["total"])
    log(f"  skipped {sk.sum()}/{tot.sum()} band {band} band-mismatch {mism} max-abs {mx:.2e} mean-abs {mean:.2e}")
    return sk, tot


@pytest.mark.parametrize("lam", [0.0, 1e-2, 1.0])
def test_mx_tiny_parity(lam):
    sk, _ = _mx_full_parity(CONFIGS["tiny"], lam)
    assert (sk.sum() == 0) == (lam == 0.0)


@pytest.mark.parametrize("lam,causal", [(0.0, False), (1e-2, False), (1e-2, True)])
def test_mx_ragged_d128_parity(lam, causal):
    _mx_full_parity(RAGGED, lam, causal=causal)


@pytest.mark.parametrize("head_dim,block", [(64, 128), (128, 64)])
def test_mx_other_tile_shapes(head_dim, block):
    sk, _ = _mx_full_parity(_shape_cfg(head_dim, block), 1e-1)
    assert sk.sum() > 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("head_dim,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_mx_calibration_all_tile_shapes(head_dim, block, causal):
    """Counts equal the block-scaled forward's skipped tiles exactly and the
    oracle's outside the 1e-3 band; the output equals the lambda = 0 forward."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg = _shape_cfg(head_dim, block)
    xd, bs, xf, cu = _mx_inputs(cfg)
    lams = np.geomspace(1e-4, 1.0, 6)
    o_cal, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=block, causal=causal,
                                              block_scales=bs)
    torch.cuda.synchronize()
    counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
    wgs = osk.workgroups(cu, cfg.num_heads, block)
    ts = np.log2(lams)
    ref = osk.calibration_counts(xf["q"], xf["k"], xf["v"], cu, ts, block, causal=causal)
    np.testing.assert_array_equal(tiles, ref["tiles"])
    o0, _, _, _ = gpu_forward(xd, cu, 0.0, "lambda", block, mask=False, causal=causal, block_scales=bs)
    np.testing.assert_array_equal(o_cal.float().cpu().numpy(), o0)
    d = osk.skip_softmax_forward(xf["q"], xf["k"], xf["v"], cu, -math.inf, block, fast=True, causal=causal)["d"]
    for kk, lam in enumerate(lams):
        _, _, _, mask = gpu_forward(xd, cu, lam, "lambda", block, causal=causal, block_scales=bs)
        per_wg = np.array([(mask[b, h, i] == osk.TILE_SKIPPED).sum() for (b, h, i) in wgs])
        np.testing.assert_array_equal(counts[:, kk], per_wg)
        with np.errstate(invalid="ignore"):
            band = np.array([np.sum(np.abs(d[b, h, i] - ts[kk]) <= 1e-3) for (b, h, i) in wgs])
        assert np.all(np.abs(counts[:, kk] - ref["counts"][:, kk]) <= band)
    if not causal:
        assert counts.sum() > 0


def test_mx_headline_sampled_parity():
    """Full-size block-scaled q/k launch at the headline shape: skip bits and
    outputs on sampled Q-blocks against the oracle on the dequantized q/k."""
    cfg = CONFIGS["headline"]
    xd, bs, xf, cu = _mx_inputs(cfg)
    H, blk = cfg.num_heads, cfg.block
    scale = osk.default_sm_scale(cfg.head_dim)
    qbs = sample_qblocks(cu, H, blk, [0, 39], 3, seed=cfg.seed)
    S = int(cu[1])
    for lam in (0.0, 8e-3):
        log(f"[headline mxfp8 q/k] lambda={lam}: GPU forward (full launch)")
        o, sk, tot, mask = gpu_forward(xd, cu, lam, "lambda", blk, block_scales=bs)
        t = t_matrix(cu, H, lam, "lambda")
        assert np.all(tot == osk.n_tiles(S, blk) ** 2)
        worst, sum_abs, n_abs = 0.0, 0.0, 0
        for (b, h, i) in qbs:
            kh, vh = xf["k"][:, h], xf["v"][:, h]
            r0, r1 = i * blk, min(S, (i + 1) * blk)
            qh = xf["q"][r0:r1, h]
            d, _ = osk.tile_stats_fast(qh, kh, blk, scale)
            near = np.abs(d - t[b, h]) <= 1e-3
            gpu_skip = mask[b, h, i] == osk.TILE_SKIPPED
            assert not np.any((gpu_skip != (d < t[b, h])) & ~near), f"skip mismatch at {(b, h, i)}"
            ref = osk.skip_softmax_qblock(qh, kh, vh, t[b, h], blk, scale, forced_skip=gpu_skip)
            diff = np.abs(o[r0:r1, h] - ref["o"])
            worst = max(worst, float(diff.max()))
            sum_abs += float(diff.sum())
            n_abs += diff.size
        assert worst <= 2e-2 and sum_abs / n_abs <= 2e-3, f"output mismatch {worst:.3e} {sum_abs / n_abs:.3e}"
        log(f"  sparsity {sk.sum() / tot.sum():.4f} max-abs {worst:.2e} mean-abs {sum_abs / n_abs:.2e}")
        if lam > 0:
            assert sk.sum() > 0


@pytest.mark.parametrize("causal", [False, True])
def test_mx_strided_layout_matches_contiguous(causal):
    """q, k, v, o and both scale arrays as views with a padding head between
    rows (non-default token strides): the output equals the contiguous run
    bit for bit and the padding head's output rows stay untouched."""
    import torch
    import skip_softmax_video_amd as ssa
    xd, bs, xf, cu = _mx_inputs(RAGGED)
    T, H, D = xd["q"].shape
    big = {}
    for n in ("q", "k", "v"):
        buf = torch.zeros((T, H + 1, D), dtype=xd[n].dtype, device="cuda")
        buf[:, :H] = xd[n]
        big[n] = buf[:, :H]
    bbs = []
    for s in bs:
        buf = torch.full((T, H + 1, D // 32), 255, dtype=torch.uint8, device="cuda")  # padding: invalid scale
        buf[:, :H] = s
        bbs.append(buf[:, :H])
    out_buf = torch.full((T, H + 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    for lam in (0.0, 1e-2):
        o_ref = ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, lam, block=RAGGED.block, causal=causal, block_scales=bs)
        ssa.attn_fwd(big["q"], big["k"], big["v"], cu, lam, block=RAGGED.block, causal=causal,
                     block_scales=tuple(bbs), out=out_buf[:, :H])
        torch.cuda.synchronize()
        assert torch.equal(out_buf[:, :H], o_ref)
        assert torch.all(out_buf[:, H] == 7.0)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_strided_layout_matches_contiguous(causal):
    """e4m3 q, k, v and the bf16 output as views with a padding head between
    rows: the output equals the contiguous run bit for bit and the padding
    head's output rows stay untouched."""
    import torch
    import skip_softmax_video_amd as ssa
    xd, xf, scales, cu = _fp8_inputs(RAGGED)
    T, H, D = xd["q"].shape
    big = {}
    for n in ("q", "k", "v"):
        buf = torch.full((T, H + 1, D), 0x7E, dtype=torch.uint8, device="cuda")  # padding: e4m3 448
        buf[:, :H] = xd[n]
        big[n] = buf[:, :H]
    out_buf = torch.full((T, H + 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    for lam in (0.0, 1e-2):
        o_ref = ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, lam, block=RAGGED.block, causal=causal, scales=scales)
        ssa.attn_fwd(big["q"], big["k"], big["v"], cu, lam, block=RAGGED.block, causal=causal, scales=scales,
                     out=out_buf[:, :H])
        torch.cuda.synchronize()
        assert torch.equal(out_buf[:, :H], o_ref)
        assert torch.all(out_buf[:, H] == 7.0)


# ---- streams and graph capture -------------------------------------------------------------------
def test_side_stream_matches_default_stream():
    """Forward (with counters) and calibration enqueued on a non-default
    stream give the default-stream results bit for bit."""
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    B, H = len(cu) - 1, RAGGED.num_heads
    o0, sk0, tot0, _ = gpu_forward(xd, cu, 1e-2, "lambda", RAGGED.block, mask=False)
    _, c0, t0 = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, [1e-3, 1e-2], block=RAGGED.block)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sk = torch.full((B * H,), 99, dtype=torch.int64, device="cuda")
        tot = torch.full((B * H,), 99, dtype=torch.int64, device="cuda")
        o = ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, 1e-2, block=RAGGED.block, skipped=sk, total=tot)
        _, c, t = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, [1e-3, 1e-2], block=RAGGED.block)
    side.synchronize()
    np.testing.assert_array_equal(o.float().cpu().numpy(), o0)
    np.testing.assert_array_equal(sk.cpu().numpy().reshape(B, H), sk0)
    np.testing.assert_array_equal(tot.cpu().numpy().reshape(B, H), tot0)
    assert torch.equal(c, c0) and torch.equal(t, t0)


def test_graph_capture_replays_match_eager():
    """The forward with counters captured in a HIP graph: every replay (with
    eager work in between) equals the eager result, counters included, since
    the counters are cleared by a kernel, not a memset node."""
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    B, H = len(cu) - 1, RAGGED.num_heads
    o_e, sk_e, tot_e, _ = gpu_forward(xd, cu, 1e-2, "lambda", RAGGED.block, mask=False)
    o = torch.empty_like(xd["q"])
    sk = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    tot = torch.zeros(B * H, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, 1e-2, block=RAGGED.block, out=o, skipped=sk, total=tot)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssa.attn_fwd(xd["q"], xd["k"], xd["v"], cu, 1e-2, block=RAGGED.block, out=o, skipped=sk, total=tot)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(0.0)
        sk.fill_(12345)
        tot.fill_(12345)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        np.testing.assert_array_equal(o.float().cpu().numpy(), o_e)
        np.testing.assert_array_equal(sk.cpu().numpy().reshape(B, H), sk_e)
        np.testing.assert_array_equal(tot.cpu().numpy().reshape(B, H), tot_e)


def test_binding_rejects_wrong_output_buffers():
    """Counters, tile masks and calibration outputs of the wrong size, type or
    layout are refused before anything is launched (the library sees only
    their pointers)."""
    import torch
    import skip_softmax_video_amd as ssa
    x, xd, cu = _inputs(RAGGED)
    B, H = len(cu) - 1, RAGGED.num_heads
    q, k, v = xd["q"], xd["k"], xd["v"]
    prob, _ = ssa.make_problem(q, cu, RAGGED.block)
    nq, nk = ssa.tile_mask_dims(prob)
    nwg = ssa.calib_num_workgroups(prob)
    i64 = dict(dtype=torch.int64, device="cuda")
    bad_fwd = [
        dict(skipped=torch.zeros(B * H - 1, **i64)),
        dict(total=torch.zeros(B * H, dtype=torch.int32, device="cuda")),
        dict(skipped=torch.zeros(2 * B * H, **i64)[::2]),
        dict(skipped=torch.zeros(B * H, dtype=torch.int64)),
        dict(tile_mask=torch.empty((B, H, nq, nk - 1), dtype=torch.uint8, device="cuda")),
        dict(tile_mask=torch.empty((B, H, nq, nk), dtype=torch.int32, device="cuda")),
    ]
    for kw in bad_fwd:
        with pytest.raises(ValueError):
            ssa.attn_fwd(q, k, v, cu, 1e-2, block=RAGGED.block, **kw)
    bad_cal = [
        dict(counts=torch.empty((nwg, 1), dtype=torch.int32, device="cuda")),
        dict(counts=torch.empty((nwg, 2), dtype=torch.int64, device="cuda")),
        dict(tiles=torch.empty((nwg - 1,), dtype=torch.int32, device="cuda")),
    ]
    for kw in bad_cal:
        with pytest.raises(ValueError):
            ssa.attn_calibrate(q, k, v, cu, [1e-3, 1e-2], block=RAGGED.block, **kw)
    # exactly sized buffers, in either counter type torch offers, are accepted
    sk = torch.zeros((B, H), **i64)
    ssa.attn_fwd(q, k, v, cu, 1e-2, block=RAGGED.block, skipped=sk,
                 tile_mask=torch.empty((B, H, nq, nk), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    _, sk0, _, _ = gpu_forward(xd, cu, 1e-2, "lambda", RAGGED.block, mask=False)
    np.testing.assert_array_equal(sk.cpu().numpy(), sk0)


def test_resolved_lambda_sparsity_lies_between_calibration_points():
    """Calibrate, fit, resolve a target, run the forward at the resolved lambda.
    For lambda <= 1 the running maximum does not depend on lambda, so skip sets
    are nested and each sequence's sparsity at the resolved lambda lies between
    its calibrated sparsities at the neighbouring grid thresholds, exactly."""
    import torch
    import skip_softmax_video_amd as ssa
    cfg = RAGGED
    x, xd, cu = _inputs(cfg)
    B, H = len(cu) - 1, cfg.num_heads
    lams = np.geomspace(1e-6, 0.7, 16)
    _, counts, tiles = ssa.attn_calibrate(xd["q"], xd["k"], xd["v"], cu, lams, block=cfg.block)
    torch.cuda.synchronize()
    sp = ssa.calibration_sparsity(cu, H, cfg.head_dim, cfg.block, counts.cpu().numpy(), tiles.cpu().numpy())
    seq_k = float(cu[1] - cu[0])
    fit = ssa.calibration_fit(lams, sp[0], seq_k)
    for target in (0.05, 0.2):  # inside the 3,072-token sequence's calibrated range
        status, lam, _ = ssa.resolve_threshold(int(seq_k), target_sparsity=target, a=fit.a, b=fit.b,
                                               s_min=fit.s_min, s_max=fit.s_max)
        assert status == ssa.SSA_OK and lams[0] <= lam <= lams[-1]
        k = int(np.searchsorted(lams, lam, side="right")) - 1
        _, sk, tot, _ = gpu_forward(xd, cu, lam, "lambda", cfg.block, mask=False)
        for b in range(B):
            if tot[b].sum() == 0:
                continue
            s_b = sk[b].sum() / tot[b].sum()
            hi = sp[b][k + 1] if k + 1 < lams.size else 1.0
            assert sp[b][k] <= s_b <= hi, (target, b, sp[b][k], s_b, hi)
        s0 = sk[0].sum() / tot[0].sum()
        log(f"  target {target}: lambda {lam:.4g}, sequence 0 sparsity {s0:.4f} "
            f"(grid {sp[0][k]:.4f} .. {sp[0][min(k + 1, lams.size - 1)]:.4f})")


@pytest.mark.parametrize("sm_scale", [0.125, 0.03])
def test_custom_sm_scale_parity(sm_scale):
    """A caller-given softmax scale replaces 1/sqrt(D) in the scores, the skip
    test and the softmax alike (0.125 sharpens the rows, 0.03 flattens them)."""
    sk, tot, _, _ = _full_parity(RAGGED, 1e-2, sm_scale=sm_scale)
    sk0, _, _, _ = _full_parity(RAGGED, 1e-2)
    assert sk.sum() != sk0.sum()  # the scale reaches the skip test
    if sm_scale > 1 / math.sqrt(RAGGED.head_dim):
        assert sk.sum() > sk0.sum()


def test_log2_thresholds_equal_lambda_thresholds():
    """A raw log2 threshold is the kernel's own threshold: log2(lambda) given
    directly gives the lambda call's result bit for bit, and -inf is dense."""
    x, xd, cu = _inputs(RAGGED)
    lam = [1e-3, 1e-2, 0.5]
    o_l, sk_l, tot_l, m_l = gpu_forward(xd, cu, lam, "lambda", RAGGED.block)
    o_t, sk_t, tot_t, m_t = gpu_forward(xd, cu, list(np.log2(lam)), "log2", RAGGED.block)
    np.testing.assert_array_equal(o_t, o_l)
    np.testing.assert_array_equal(m_t, m_l)
    np.testing.assert_array_equal(sk_t, sk_l)
    assert sk_l.sum() > 0
    o_d, sk_d, _, _ = gpu_forward(xd, cu, 0.0, "lambda", RAGGED.block)
    o_i, sk_i, _, _ = gpu_forward(xd, cu, -math.inf, "log2", RAGGED.block)
    np.testing.assert_array_equal(o_i, o_d)
    assert sk_i.sum() == 0 and sk_d.sum() == 0

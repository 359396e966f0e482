"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side logic (threshold resolution, fit, calibration reduction,
argument validation) matches the oracle. No GPU call is made here: every
forward/calibrate call below fails validation before any HIP work."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import skip_softmax_video_amd as ssa
from skip_softmax_video_amd import _binding as bnd
from oracle import calibration as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    lib = ssa.load_library()
    decl = set()
    for name in os.listdir(os.path.join(ROOT, "include")):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            decl |= set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s+(ssa_\w+)\s*\(", text, re.M))
    assert decl, "no declarations found"
    assert decl == set(ssa.EXPORTED)
    for sym in decl:
        assert hasattr(lib, sym), sym


RESOLVE_CASES = [
    dict(raw_log2=-0.7), dict(lam=0.61557), dict(), dict(scale_factor=5000.0),
    dict(target_sparsity=0.5, a=7.93, b=8.61), dict(target_sparsity=0.7, log_a=math.log(7.93), b=8.61),
    dict(target_sparsity=0.25, a=7.93, b=8.61, s_min=0.38, s_max=0.86),
    dict(raw_log2=-1.0, lam=0.25, scale_factor=100.0), dict(lam=0.0), dict(raw_log2=-math.inf),
]


@pytest.mark.parametrize("case", RESOLVE_CASES)
@pytest.mark.parametrize("seq_k", [8190, 32760, 75600])
def test_resolve_matches_oracle(case, seq_k):
    okw = dict(case)
    if "lam" in okw:
        okw["lam"] = okw.pop("lam")
    want = oc.resolve_threshold(oc.ThresholdSpec(**okw), seq_k)
    got = ssa.resolve_threshold(seq_k, **case)
    assert got[0] == want[0]
    assert got[1] == pytest.approx(want[1], rel=1e-15, abs=0)
    assert got[2] == pytest.approx(want[2], rel=1e-15, abs=0) or (math.isinf(got[2]) and got[2] == want[2])


@pytest.mark.parametrize("case,status", [
    (dict(target_sparsity=0.5), ssa.SSA_ERR_NO_FORMULA),
    (dict(target_sparsity=0.5, b=1.0), ssa.SSA_ERR_NO_FORMULA),
    (dict(lam=1.5), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(lam=-0.1), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(lam=float("nan")), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(raw_log2=0.5), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(scale_factor=5000.0), ssa.SSA_ERR_THRESHOLD_RANGE),   # over 1024 keys: lambda 4.88
])
def test_resolve_errors(case, status):
    with pytest.raises(ssa.SSAError) as e:
        ssa.resolve_threshold(1024, **case)
    assert e.value.status == status
    want = oc.resolve_threshold(oc.ThresholdSpec(**case), 1024)[0]
    assert want == status


def test_fit_matches_oracle_and_degenerate():
    rng = np.random.default_rng(2)
    for trial in range(20):
        n = int(rng.integers(2, 17))
        s = np.concatenate([rng.uniform(0, 1, n), [0.0, 1.0]])
        lam = np.geomspace(1e-6, 0.7, s.size)
        sk = rng.choice([8190.0, 32760.0, 75600.0], size=s.size)
        try:
            want = oc.fit_exponential_logspace(lam, s, sk)
        except ValueError:
            with pytest.raises(ssa.SSAError):
                ssa.calibration_fit(lam, s, sk)
            continue
        got = ssa.calibration_fit(lam, s, sk)
        assert got.b == pytest.approx(want.b, rel=1e-10)
        assert got.log_a == pytest.approx(want.log_a, rel=1e-10, abs=1e-12)
        assert (got.s_min, got.s_max, got.n_used) == (want.s_min, want.s_max, want.n_used)
    with pytest.raises(ssa.SSAError) as e:
        ssa.calibration_fit([1e-3, 1e-2], [0.5, 0.5], 100.0)
    assert e.value.status == ssa.SSA_ERR_FIT_DEGENERATE
    # non-finite points are rejected, not fitted
    for lam, s, sk in (([1e-3, np.inf], [0.3, 0.6], 100.0), ([1e-3, 1e-2], [0.3, 0.6], np.inf),
                       ([1e-3, 1e-2], [0.3, np.nan], 100.0)):
        with pytest.raises(ssa.SSAError) as e:
            ssa.calibration_fit(lam, s, sk)
        assert e.value.status == ssa.SSA_ERR_INVALID_ARG


def test_calibration_sparsity_reduction():
    cu = [0, 1000, 1000, 129]
    cu = np.cumsum([0, 1000, 0, 129])
    H, blk, n = 3, 128, 4
    nwg = (8 + 0 + 2) * H
    rng = np.random.default_rng(0)
    tiles = np.array([8] * 24 + [2] * 6, dtype=np.int32)
    counts = np.sort(rng.integers(0, 3, size=(nwg, n)), axis=1).astype(np.int32)
    sp = ssa.calibration_sparsity(cu, H, 128, blk, counts, tiles)
    assert sp.shape == (3, n)
    np.testing.assert_allclose(sp[0], counts[:24].sum(0) / tiles[:24].sum())
    assert np.all(np.isnan(sp[1]))
    np.testing.assert_allclose(sp[2], counts[24:].sum(0) / tiles[24:].sum())


def _problem(**kw):
    cu = np.asarray(kw.pop("cu", [0, 256]), dtype=np.int32)
    base = dict(batch=len(cu) - 1, num_heads=2, head_dim=128, block=128,
                cu_seqlens=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                stride_token=256, stride_head=128, sm_scale=0.0)
    base.update(kw)
    return bnd.Problem(**base), cu


FAKE = 1 << 20  # aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,th,status", [
    (dict(head_dim=96), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(block=32), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(num_heads=0), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(num_heads=600, stride_token=600 * 128), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(cu=[0, 10, 5]), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(cu=[3, 10]), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(stride_token=100), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(sm_scale=-1.0), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(causal=2), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=3), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),           # unknown element type
    # block-scaled (MXFP8) q/k: the scale arrays are required, aligned to a row
    # of D / 32 bytes, strided in whole rows and addressable in 32 bits
    (dict(dtype=2), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE + 1, block_scale_stride_token=8,
          block_scale_stride_head=4), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=6,
          block_scale_stride_head=4), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=8,
          block_scale_stride_head=0), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),   # two heads on one row
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=8,
          block_scale_stride_head=4, stride_token=264, stride_head=136), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=1 << 30,
          block_scale_stride_head=4), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=8,
          block_scale_stride_head=4), (0, [1.5]), ssa.SSA_ERR_THRESHOLD_RANGE),  # scales fine, lambda not
    (dict(dtype=1, scale_q=1.0, scale_k=1.0, scale_v=0.0), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=1, scale_q=1.0, scale_k=float("inf"), scale_v=1.0), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=1, scale_q=1.0, scale_k=1.0, scale_v=1.0, stride_token=264, stride_head=136),
     (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),                          # e4m3 rows must be 16-byte aligned
    (dict(causal=-1), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    # a token step past 32-bit buffer offsets; a head step past any device range
    (dict(stride_token=1 << 33), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(stride_token=(1 << 62) + 128), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(stride_head=1 << 48), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(stride_head=-128), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=1 << 60,
          block_scale_stride_head=4), (0, [0.1]), ssa.SSA_ERR_UNSUPPORTED),
    (dict(dtype=2, block_scale_q=FAKE, block_scale_k=FAKE, block_scale_stride_token=8,
          block_scale_stride_head=1 << 60), (0, [0.1]), ssa.SSA_ERR_INVALID_ARG),
    (dict(), (0, [1.5]), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(), (0, [float("nan")]), ssa.SSA_ERR_THRESHOLD_RANGE),
    (dict(), (1, [0.25]), ssa.SSA_ERR_THRESHOLD_RANGE),            # raw log2 > 0
    (dict(), (2, [300.0]), ssa.SSA_ERR_THRESHOLD_RANGE),           # sf / 256 > 1
    (dict(), (0, [0.1, 0.1, 0.1]), ssa.SSA_ERR_INVALID_ARG),       # count not 1 or H
    (dict(), (7, [0.1]), ssa.SSA_ERR_INVALID_ARG),                 # unknown kind
])
def test_forward_argument_errors(kw, th, status):
    lib = ssa.load_library()
    prob, cu = _problem(**kw)
    vals = np.asarray(th[1], dtype=np.float64)
    t = bnd.Thresholds(kind=th[0], count=vals.size, values=vals.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    st = lib.ssa_attn_fwd(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, ctypes.byref(t), None, None, None, None)
    assert st == status, ssa.status_string(st)


def test_forward_null_and_misaligned_pointers():
    lib = ssa.load_library()
    prob, cu = _problem()
    vals = np.asarray([0.1])
    t = bnd.Thresholds(kind=0, count=1, values=vals.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    assert lib.ssa_attn_fwd(ctypes.byref(prob), None, FAKE, FAKE, FAKE, ctypes.byref(t), None, None, None, None) \
        == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_attn_fwd(ctypes.byref(prob), FAKE + 8, FAKE, FAKE, FAKE, ctypes.byref(t), None, None, None,
                            None) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, ctypes.byref(t), None, None, None, None) \
        == ssa.SSA_ERR_INVALID_ARG


@pytest.mark.parametrize("lams,status", [
    ([0.0, 0.1], ssa.SSA_ERR_THRESHOLD_RANGE),
    ([0.1, 1.5], ssa.SSA_ERR_THRESHOLD_RANGE),
    ([0.1, 0.01], ssa.SSA_ERR_INVALID_ARG),     # not ascending
    ([0.1] * 65, ssa.SSA_ERR_INVALID_ARG),      # more than 64 thresholds
    ([], ssa.SSA_ERR_INVALID_ARG),
])
def test_calibrate_argument_errors(lams, status):
    lib = ssa.load_library()
    prob, cu = _problem()
    lam = np.asarray(lams, dtype=np.float64)
    st = lib.ssa_attn_calibrate(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE,
                                lam.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), lam.size, FAKE, FAKE, None)
    assert st == status


def test_workgroup_and_mask_dims():
    prob, cu = _problem(cu=np.cumsum([0, 75600, 32760, 8190]).tolist(), num_heads=40, stride_token=40 * 128)
    assert ssa.calib_num_workgroups(prob) == 40 * (591 + 256 + 64)
    assert ssa.tile_mask_dims(prob) == (591, 591)


def test_status_strings():
    for code in (0, 1, -1, -2, -3, -4, -5, -6):
        assert ssa.status_string(code) and ssa.status_string(code) != "unknown status"
    assert ssa.status_string(99) == "unknown status"


# ---- timestep and layer gating --------------------------------------------------
from oracle import gating as og  # noqa: E402


@pytest.mark.parametrize("n,T,shift", [(40, 1000, 3.0), (50, 1000, 5.0), (1, 1000, 3.0), (30, 1, 1.0),
                                       (7, 20, 0.5)])
def test_flow_timesteps_match_oracle(n, T, shift):
    got = ssa.flow_timesteps(n, T, shift)
    ref = og.flow_timesteps(n, T, shift)
    assert np.allclose(got, ref, rtol=0, atol=1e-15)


def test_gate_dense_steps_match_oracle(golden):
    g = golden("unipc_40_steps.txt")
    t = ssa.flow_timesteps(40, 1000, 3.0)
    for c, d in zip(g["cutoffs"][0], g["dense_steps"][0]):
        assert ssa.gate_dense_steps(t, c) == og.dense_steps(t, c) == int(d)
    assert ssa.gate_dense_steps(t, None) == 0 and ssa.gate_dense_steps(t, 0.0) == 40
    assert ssa.gate_dense_steps([], 0.5) == 0


_NAMES = ["transformer.blocks.0.attn1", "transformer_2.blocks.0.attn1", "transformer.blocks.10.attn1",
          "blocks.0.attn2", "single_transformer_blocks.3.attn", "transformer_blocks.0.attn",
          "transformer_blocks.12.attn", "attn", "a.b.c.d"]
_PATTERNS = ["blocks.0.attn1", "blocks.0.*", "*attn2", "transformer_blocks.0*", "single_transformer_blocks*",
             "blocks.?.attn1", "blocks.[01].attn1", "blocks.[!0].attn1", "*", "b.c.*", "a.b.c.d", "nomatch"]


def test_gate_layer_matches_oracle():
    rng = np.random.default_rng(5)
    for _ in range(400):
        name = _NAMES[rng.integers(len(_NAMES))]
        ign = [_PATTERNS[i] for i in rng.choice(len(_PATTERNS), rng.integers(0, 3), replace=False)]
        ovr = [(_PATTERNS[i], float(rng.choice([0.0, 800.0, 8000.0])))
               for i in rng.choice(len(_PATTERNS), rng.integers(0, 4), replace=False)]
        cutoff = [None, 0.0, 0.6, 0.86, 1.0][rng.integers(5)]
        ts = rng.uniform(0, 1, rng.integers(1, 4))
        base = float(rng.choice([0.0, 5000.0, 123.5]))
        assert ssa.gate_layer(name, ts, base, cutoff, ign, ovr) == og.gate_layer(name, ts, base, cutoff, ign, ovr)


@pytest.mark.parametrize("kw", [dict(cutoff=1.5), dict(cutoff=-0.1), dict(base=-1.0), dict(base=math.nan),
                                dict(ts=[math.nan]), dict(ts=[]), dict(ovr=[("x", -2.0)])])
def test_gate_errors(kw):
    with pytest.raises(ssa.SSAError) as e:
        ssa.gate_layer("a.b", kw.get("ts", [0.5]), kw.get("base", 1.0), kw.get("cutoff"), (), kw.get("ovr", ()))
    assert e.value.status == ssa.SSA_ERR_INVALID_ARG
    for bad in (dict(n=0), dict(T=0), dict(shift=0.0), dict(shift=math.nan)):
        with pytest.raises(ssa.SSAError):
            ssa.flow_timesteps(bad.get("n", 4), bad.get("T", 1000), bad.get("shift", 3.0))
    with pytest.raises(ssa.SSAError):
        ssa.gate_dense_steps([0.5], 2.0)


# ---- linear-space fit and pooled calibration -------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_linear_fit_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(3, 30))
    s = np.sort(rng.uniform(0.2, 0.95, n))
    a, b = 10 ** rng.uniform(-6, 1), rng.uniform(5, 40)
    seq_k = rng.choice([8190.0, 32760.0, 75600.0], n)
    lam = np.minimum(a * np.exp(b * s) * np.exp(rng.normal(0, 0.25, n)) / seq_k, 1.0)
    got = ssa.calibration_fit(lam, s, seq_k, space="linear")
    ref = oc.fit_exponential_linear(lam, s, seq_k)
    # The library searches b on a grid and bisects dH/db; the oracle runs plain
    # Levenberg-Marquardt. Both must reach the same least-squares minimum. Along
    # its flat direction the squared error changes only at the 1e-15 level, so
    # the parameters agree to about 1e-7 while the minimum and the fitted
    # values agree to rounding.
    y = lam * seq_k
    err = lambda f: np.sum((f.a * np.exp(f.b * s) - y) ** 2)
    assert err(got) == pytest.approx(err(ref), rel=1e-12)
    np.testing.assert_allclose(got.a * np.exp(got.b * s), ref.a * np.exp(ref.b * s), rtol=1e-7)
    assert got.b == pytest.approx(ref.b, rel=1e-6)
    assert got.a == pytest.approx(ref.a, rel=1e-6)
    assert (got.s_min, got.s_max, got.n_used) == (ref.s_min, ref.s_max, ref.n_used)


def test_linear_fit_degenerate():
    with pytest.raises(ssa.SSAError) as e:
        ssa.calibration_fit([1e-3, 1e-2], [0.5, 0.5], 100.0, space="linear")
    assert e.value.status == ssa.SSA_ERR_FIT_DEGENERATE


def _random_pass(rng, H, block, n, lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    nwg = sum(-(-int(S) // block) * H for S in lengths)
    tiles = np.zeros(nwg, np.int32)
    w = 0
    for S in lengths:
        nt = -(-int(S) // block)
        tiles[w:w + nt * H] = nt
        w += nt * H
    counts = np.sort(rng.integers(0, np.maximum(tiles, 1)[:, None], (nwg, n)), axis=1).astype(np.int32)
    return cu, counts, tiles


def test_pool_matches_oracle():
    rng = np.random.default_rng(9)
    H, block, n = 3, 128, 5
    lams = np.geomspace(1e-5, 0.5, n)
    pool, ref = ssa.CalibrationPool(n, max_groups=8), oc.CalibPool(n)
    for lengths in ([300, 1000, 0, 300], [1000], [77, 300, 129]):
        cu, counts, tiles = _random_pass(rng, H, block, n, lengths)
        pool.add(cu, H, 128, block, counts, tiles)
        ref.add(counts, tiles, cu, H, block)
    got, exp = pool.groups, ref.groups
    assert list(got) == list(exp) == [300, 1000, 77, 129]
    for key in exp:
        np.testing.assert_array_equal(got[key][0], exp[key][0])
        assert got[key][1] == exp[key][1]
    for a, b in zip(pool.points(lams), ref.points(lams)):
        np.testing.assert_array_equal(a, b)


def test_pool_errors_leave_it_unchanged():
    rng = np.random.default_rng(3)
    pool = ssa.CalibrationPool(4, max_groups=2)
    cu, counts, tiles = _random_pass(rng, 2, 64, 4, [100, 200])
    pool.add(cu, 2, 128, 64, counts, tiles)
    before = {k: (v[0].copy(), v[1]) for k, v in pool.groups.items()}
    cu2, counts2, tiles2 = _random_pass(rng, 2, 64, 4, [100, 300])  # a third key length: pool full
    with pytest.raises(ssa.SSAError):
        pool.add(cu2, 2, 128, 64, counts2, tiles2)
    cu3, counts3, tiles3 = _random_pass(rng, 2, 64, 3, [100])  # wrong threshold count
    with pytest.raises(ssa.SSAError):
        pool.add(cu3, 2, 128, 64, counts3, tiles3)
    with pytest.raises(ssa.SSAError):  # cu_seqlens must start at 0
        pool.add(np.asarray(cu) + 5, 2, 128, 64, counts, tiles)
    after = pool.groups
    assert list(after) == list(before)
    for k in before:
        np.testing.assert_array_equal(after[k][0], before[k][0])
        assert after[k][1] == before[k][1]


def test_host_arrays_must_match_the_problem():
    """The C functions read counts[w * n + k] for every work-group w: the
    binding refuses host arrays of another shape before calling them."""
    rng = np.random.default_rng(4)
    cu, counts, tiles = _random_pass(rng, 2, 64, 4, [100, 200])
    with pytest.raises(ValueError):
        ssa.calibration_sparsity(cu, 2, 128, 64, counts[:-1], tiles)
    with pytest.raises(ValueError):
        ssa.calibration_sparsity(cu, 2, 128, 64, counts, tiles[:-1])
    with pytest.raises(ValueError):
        ssa.calibration_sparsity(cu, 2, 128, 64, counts.ravel(), tiles)
    pool = ssa.CalibrationPool(4, max_groups=2)
    with pytest.raises(ValueError):
        pool.add(cu, 2, 128, 64, counts[:-1], tiles[:-1])
    pool.add(cu, 2, 128, 64, counts, tiles)
    with pytest.raises(ValueError):
        pool.points(np.geomspace(1e-4, 0.5, 3))
    with pytest.raises(ValueError):
        ssa.CalibrationPool(0)
    with pytest.raises(ValueError):
        ssa.calibration_fit([1e-3, 1e-2, 1e-1], [0.3, 0.6], 100.0)


@pytest.mark.parametrize("cu, msg", [
    ([0, 64, 129], "past the tensors"),      # last offset beyond T = 128
    ([0, 96, 64], "never decrease"),
    ([5, 64, 128], "start at 0"),
    ([[0, 128]], "1-D"),
    ([0], "1-D"),
    ([0.0, 128.0], "integers"),
])
def test_cu_seqlens_refused_before_any_launch(cu, msg):
    """The library sees only pointers, so the binding checks cu_seqlens against
    the tensors' token count; a bad array raises before anything is launched
    (these tensors live on the CPU, so a launch could not even be attempted)."""
    import torch
    q = torch.zeros((128, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=msg):
        bnd.make_problem(q, cu, 128)
    with pytest.raises(ValueError, match=msg):
        bnd.check_cu_seqlens(cu, q.shape[0])


def test_cu_seqlens_accepts_shorter_batches_and_empty_sequences():
    import torch
    q = torch.zeros((128, 2, 128), dtype=torch.bfloat16)
    for cu in ([0, 128], [0, 0, 100], np.array([0, 64, 64, 120], dtype=np.int64), torch.tensor([0, 128])):
        prob, arr = bnd.make_problem(q, cu, 128)
        assert arr.dtype == np.int32 and prob.batch == len(arr) - 1

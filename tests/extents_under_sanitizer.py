"""Launch-plan extents, run only inside the sanitizer build (see
test_host_sanitized.py, which starts pytest on this file in a process with the
AddressSanitizer runtime preloaded and SSA_LIBRARY naming the host-only build).

That build replaces the kernel launchers with a checker that walks every
planned work-group through the kernels' own work-group mapping and records
the largest index each kernel would touch in each caller buffer. These tests
compare those extents with the buffer sizes the Python binding demands
(`_check_out`): the counters [B*H], the tile mask [B, H, nq, nk], the
calibration counts [num_wg, n] and tiles [num_wg], and the token rows
(cu_seqlens[-1] <= T). No pointer is ever dereferenced: the checker only
does index arithmetic.
"""
import ctypes

import numpy as np
import pytest

from skip_softmax_video_amd import _binding as bnd

FAKE = 1 << 20  # 16-byte aligned stand-in address; the checker never reads through it


@pytest.fixture(scope="module")
def lib():
    lib = bnd.load_library()
    if not hasattr(lib, "ssa_check_extents"):
        pytest.skip("needs the host-only sanitizer build (SSA_LIBRARY)")
    lib.ssa_check_extents.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    lib.ssa_check_extents.restype = ctypes.c_int
    return lib


def _extents(lib):
    out = (ctypes.c_int64 * 10)()
    assert lib.ssa_check_extents(out, 10) == 10
    keys = ("launches", "wgs", "bh", "mask", "counts", "tiles", "tokens", "fill64", "fill8", "unmapped")
    return dict(zip(keys, list(out)))


def _problem(lens, H, D, blk, causal=False):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    prob = bnd.Problem(batch=len(lens), num_heads=H, head_dim=D, block=blk,
                       cu_seqlens=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                       stride_token=H * D, stride_head=D, sm_scale=0.0, causal=1 if causal else 0,
                       dtype=bnd.DTYPE_BF16, scale_q=1.0, scale_k=1.0, scale_v=1.0)
    return prob, cu


CASES = [
    ([3072, 300, 0, 129, 64], 3, 128, 128),                     # ragged, an empty sequence
    ([int(x) for x in np.random.default_rng(21).integers(64, 300, 40)], 16, 64, 64),  # several launches
    ([1, 2, 129], 512, 64, 64),                                 # the head limit
    ([75600, 32760, 8190], 40, 128, 128),                       # the varlen batch
    ([5, 0], 2, 128, 64),                                       # empty last sequence
    ([75600], 40, 128, 128),                                    # the headline: whole XCD rounds and a tail
    ([256 * 128 + 1], 1, 64, 128),                              # one work-group past whole rounds of chunks
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens,H,D,blk", CASES)
def test_forward_extents_match_binding_buffers(lib, lens, H, D, blk, causal):
    prob, cu = _problem(lens, H, D, blk, causal)
    B = len(lens)
    nq, nk = bnd.tile_mask_dims(prob)
    vals = np.array([0.01], np.float64)
    th = bnd.Thresholds(kind=bnd.THRESH_LAMBDA, count=1, values=vals.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    _extents(lib)  # reset
    st = lib.ssa_attn_fwd(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, ctypes.byref(th), FAKE, FAKE, FAKE, None)
    assert st == bnd.SSA_OK
    e = _extents(lib)
    nwg = bnd.calib_num_workgroups(prob)
    last_bh = max(b * H + H - 1 for b in range(B) if lens[b] > 0)
    assert e["unmapped"] == 0
    assert e["wgs"] == nwg
    assert e["bh"] == last_bh and e["bh"] < B * H          # skipped/total hold B*H entries
    assert e["fill64"] == B * H
    assert e["fill8"] == B * H * nq * nk and e["mask"] < B * H * nq * nk
    assert e["tokens"] == int(cu[-1])                       # within T = cu[-1] rows
    assert e["counts"] == -1 and e["tiles"] == -1


@pytest.mark.parametrize("n", [1, 16, 64])
@pytest.mark.parametrize("lens,H,D,blk", CASES)
def test_calibration_extents_match_binding_buffers(lib, lens, H, D, blk, n):
    prob, cu = _problem(lens, H, D, blk)
    lams = np.geomspace(1e-6, 0.7, n)
    _extents(lib)
    st = lib.ssa_attn_calibrate(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE,
                                lams.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n, FAKE, FAKE, None)
    assert st == bnd.SSA_OK
    e = _extents(lib)
    nwg = bnd.calib_num_workgroups(prob)
    assert e["unmapped"] == 0 and e["wgs"] == nwg
    assert e["counts"] == nwg * n - 1 and e["tiles"] == nwg - 1   # counts [num_wg, n], tiles [num_wg]
    assert e["tokens"] == int(cu[-1])
    assert e["bh"] == -1 and e["mask"] == -1

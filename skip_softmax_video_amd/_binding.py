"""ctypes binding of libssa.so (the C ABI in include/ssa.h).

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels or its C host code. torch is used for device memory and
streams (tensor pointers and torch's current HIP stream). There is no CPU
fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libssa.so")

# ---- status codes (include/ssa.h) -------------------------------------------
SSA_OK = 0
SSA_WARN_EXTRAPOLATED = 1
SSA_ERR_INVALID_ARG = -1
SSA_ERR_UNSUPPORTED = -2
SSA_ERR_THRESHOLD_RANGE = -3
SSA_ERR_NO_FORMULA = -4
SSA_ERR_FIT_DEGENERATE = -5
SSA_ERR_HIP = -6

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
DTYPE_MXFP8_QK = 2

THRESH_LAMBDA = 0
THRESH_LOG2 = 1
THRESH_SCALE_FACTOR = 2
_KINDS = {"lambda": THRESH_LAMBDA, "log2": THRESH_LOG2, "scale_factor": THRESH_SCALE_FACTOR}

SPEC_RAW_LOG2 = 1 << 0
SPEC_LAMBDA = 1 << 1
SPEC_SCALE_FACTOR = 1 << 2
SPEC_TARGET = 1 << 3
SPEC_A = 1 << 4
SPEC_LOG_A = 1 << 5
SPEC_B = 1 << 6
SPEC_RANGE = 1 << 7

EXPORTED = (
    "ssa_attn_fwd", "ssa_tile_mask_dims", "ssa_attn_calibrate", "ssa_calib_num_workgroups",
    "ssa_calibration_sparsity", "ssa_calibration_fit", "ssa_resolve_threshold", "ssa_status_string",
    "ssa_gate_layer", "ssa_flow_timesteps", "ssa_gate_dense_steps",
    "ssa_calibration_fit_linear", "ssa_calibration_pool_add", "ssa_calibration_pool_points",
)

GATE_BASE = 0
GATE_TIMESTEP = 1
GATE_IGNORED = 2
GATE_OVERRIDE = 3


class SSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64), ("sm_scale", ctypes.c_double),
        ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale_q", ctypes.c_double), ("scale_k", ctypes.c_double), ("scale_v", ctypes.c_double),
        ("block_scale_q", ctypes.c_void_p), ("block_scale_k", ctypes.c_void_p),
        ("block_scale_stride_token", ctypes.c_int64), ("block_scale_stride_head", ctypes.c_int64),
    ]


class Thresholds(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("count", ctypes.c_int32), ("values", ctypes.POINTER(ctypes.c_double))]


class CalibResult(ctypes.Structure):
    _fields_ = [("a", ctypes.c_double), ("log_a", ctypes.c_double), ("b", ctypes.c_double),
                ("s_min", ctypes.c_double), ("s_max", ctypes.c_double), ("n_used", ctypes.c_int32)]


class ThresholdSpec(ctypes.Structure):
    _fields_ = [("set", ctypes.c_uint32), ("raw_log2", ctypes.c_double), ("lambda_", ctypes.c_double),
                ("scale_factor", ctypes.c_double), ("target_sparsity", ctypes.c_double),
                ("a", ctypes.c_double), ("log_a", ctypes.c_double), ("b", ctypes.c_double),
                ("s_min", ctypes.c_double), ("s_max", ctypes.c_double)]


class CalibPoolC(ctypes.Structure):
    _fields_ = [("n_lambda", ctypes.c_int32), ("max_groups", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("seq_k", ctypes.POINTER(ctypes.c_int64)), ("skipped", ctypes.POINTER(ctypes.c_int64)),
                ("visited", ctypes.POINTER(ctypes.c_int64))]


class LayerOverride(ctypes.Structure):
    _fields_ = [("pattern", ctypes.c_char_p), ("scale_factor", ctypes.c_double)]


class GateSpec(ctypes.Structure):
    _fields_ = [("disabled_until_timestep", ctypes.c_double), ("ignore", ctypes.POINTER(ctypes.c_char_p)),
                ("n_ignore", ctypes.c_int32), ("overrides", ctypes.POINTER(LayerOverride)),
                ("n_overrides", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libssa.so (built by skip_softmax_video_amd.build). Raises if absent.
    The environment variable SSA_LIBRARY names another build to load instead
    (the CPU sanitizer tests use it for their host-only build)."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("SSA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m skip_softmax_video_amd.build`; "
                           "there is no fallback implementation")
    lib = ctypes.CDLL(path)
    P, V = ctypes.POINTER, ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    sig = {
        "ssa_attn_fwd": [P(Problem), V, V, V, V, P(Thresholds), V, V, V, V],
        "ssa_tile_mask_dims": [P(Problem), P(i64), P(i64)],
        "ssa_attn_calibrate": [P(Problem), V, V, V, V, P(dbl), i32, V, V, V],
        "ssa_calib_num_workgroups": [P(Problem), P(i64)],
        "ssa_calibration_sparsity": [P(Problem), P(i32), P(i32), i32, P(dbl)],
        "ssa_calibration_fit": [P(dbl), P(dbl), P(dbl), i32, P(CalibResult)],
        "ssa_resolve_threshold": [P(ThresholdSpec), i64, P(dbl), P(dbl)],
        "ssa_calibration_fit_linear": [P(dbl), P(dbl), P(dbl), i32, P(CalibResult)],
        "ssa_calibration_pool_add": [P(Problem), P(i32), P(i32), i32, P(CalibPoolC)],
        "ssa_calibration_pool_points": [P(CalibPoolC), P(dbl), P(dbl), P(dbl), P(dbl), P(i32)],
        "ssa_gate_layer": [P(GateSpec), ctypes.c_char_p, P(dbl), i32, dbl, P(dbl), P(i32)],
        "ssa_flow_timesteps": [i32, i32, dbl, P(dbl)],
        "ssa_gate_dense_steps": [P(dbl), i32, dbl, P(i32)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ssa_status_string.argtypes = [ctypes.c_int]
    lib.ssa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssa_status_string(int(status)).decode()


def _check(status: int, where: str) -> int:
    if status < 0:
        raise SSAError(status, where)
    return status


# ---- problem marshalling -----------------------------------------------------
def check_cu_seqlens(cu_seqlens, num_tokens: int) -> np.ndarray:
    """cu_seqlens as the int32 host array the library reads, checked against
    the token count of the [T, H, D] tensors. The library sees only pointers,
    so a last offset past T would make the kernels read q/k/v and write o
    beyond the tensors: refused here, before any launch."""
    raw = np.asarray(cu_seqlens)
    if raw.ndim != 1 or raw.size < 2:
        raise ValueError("cu_seqlens must be a 1-D array of B + 1 >= 2 token offsets")
    if raw.dtype.kind not in "iu":
        raise ValueError("cu_seqlens must hold integers")
    wide = raw.astype(np.int64)
    if wide[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    if np.any(np.diff(wide) < 0):
        raise ValueError("cu_seqlens must never decrease")
    if wide[-1] > int(num_tokens):
        raise ValueError(f"cu_seqlens ends at {int(wide[-1])} tokens, past the tensors' {int(num_tokens)}")
    if wide[-1] > np.iinfo(np.int32).max:
        raise ValueError("cu_seqlens offsets must fit int32")
    return np.ascontiguousarray(wide.astype(np.int32))


def _is_fp8(t) -> bool:
    import torch
    return t.dtype in (torch.float8_e4m3fn, torch.uint8)


def make_problem(q, cu_seqlens, block: int, sm_scale: float = 0.0, causal: bool = False,
                 scales: Optional[Tuple[float, float, float]] = None,
                 block_scales=None) -> Tuple[Problem, np.ndarray]:
    """ssa_problem for a [T, H, D] tensor: bf16; e4m3 bytes with per-tensor
    `scales` = (scale_q, scale_k, scale_v); or e4m3 q/k bytes with
    `block_scales` = (q scales, k scales), uint8 E8M0 device tensors
    [T, H, D / 32] (MXFP8 q/k, bf16 v). Returns (struct, cu array kept alive)."""
    cu = check_cu_seqlens(cu_seqlens, q.shape[0])
    T, H, D = q.shape
    fp8 = _is_fp8(q)
    sq, sk, sv = scales if scales is not None else (1.0, 1.0, 1.0)
    dtype = DTYPE_MXFP8_QK if block_scales is not None else (DTYPE_FP8_E4M3 if fp8 else DTYPE_BF16)
    prob = Problem(batch=len(cu) - 1, num_heads=H, head_dim=D, block=block,
                   cu_seqlens=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                   stride_token=q.stride(0), stride_head=q.stride(1), sm_scale=float(sm_scale),
                   causal=1 if causal else 0, dtype=dtype,
                   scale_q=float(sq), scale_k=float(sk), scale_v=float(sv))
    if block_scales is not None:
        qs, ks = block_scales
        prob.block_scale_q, prob.block_scale_k = _ptr(qs), _ptr(ks)
        prob.block_scale_stride_token, prob.block_scale_stride_head = qs.stride(0), qs.stride(1)
    return prob, cu


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_out(t, name: str, dtypes, numel: int, device) -> None:
    """A caller-supplied output buffer must be exactly what the kernels write:
    the library sees only its pointer, so a short buffer would be overrun."""
    if t is None:
        return
    if t.dtype not in dtypes or t.device != device or not t.is_contiguous() or t.numel() != numel:
        kinds = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be a contiguous {kinds} tensor of {numel} elements on {device}")


def _counter_dtypes():
    import torch
    return tuple(d for d in (torch.int64, getattr(torch, "uint64", None)) if d is not None)


def _check_qkv(q, k, v, o, block_scales=None):
    import torch
    fp8 = _is_fp8(q)
    mx = block_scales is not None
    if mx and not fp8:
        raise ValueError("block_scales need e4m3 q and k (torch.float8_e4m3fn or uint8 bytes)")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        byte_typed = fp8 and (name in ("q", "k") or not mx) and name != "o"
        want = q.dtype if byte_typed else torch.bfloat16
        if t.dtype != want or not t.is_cuda or t.dim() != 3 or t.device != q.device:
            raise ValueError(f"{name} must be a 3-D {want} device tensor [T, H, D] on q's device")
        if t.shape != q.shape or t.stride() != q.stride():
            raise ValueError(f"{name} must match q's shape and strides")
    if mx:
        T, H, D = q.shape
        qs, ks = block_scales
        for name, t in (("q scales", qs), ("k scales", ks)):
            if (t.dtype != torch.uint8 or t.device != q.device or tuple(t.shape) != (T, H, D // 32)
                    or t.stride(2) != 1):
                raise ValueError(f"{name} must be a uint8 device tensor [T, H, D / 32] with contiguous last dim")
        if qs.stride() != ks.stride():
            raise ValueError("q and k block scales must share strides")


def tile_mask_dims(prob: Problem) -> Tuple[int, int]:
    nq, nk = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().ssa_tile_mask_dims(ctypes.byref(prob), ctypes.byref(nq), ctypes.byref(nk)),
           "ssa_tile_mask_dims")
    return nq.value, nk.value


def calib_num_workgroups(prob: Problem) -> int:
    n = ctypes.c_int64()
    _check(load_library().ssa_calib_num_workgroups(ctypes.byref(prob), ctypes.byref(n)),
           "ssa_calib_num_workgroups")
    return n.value


# ---- entry points -------------------------------------------------------------
def attn_fwd(q, k, v, cu_seqlens, threshold: Union[float, Sequence[float]], kind: str = "lambda",
             block: int = 128, sm_scale: float = 0.0, out=None, skipped=None, total=None,
             tile_mask=None, stream=None, causal: bool = False,
             scales: Optional[Tuple[float, float, float]] = None, block_scales=None):
    """ssa_attn_fwd on torch tensors; returns `out` (allocated when None).

    threshold: one value for every head, or H values (per head); `kind` is
    "lambda", "log2" (raw) or "scale_factor" (lambda = sf / S_b).
    skipped/total: optional uint64 device tensors [B*H]; tile_mask: optional
    uint8 device tensor [B, H, nq, nk]. q, k, v may be e4m3 (torch.float8_e4m3fn
    or uint8 bytes) with scales = (scale_q, scale_k, scale_v); or q, k e4m3
    with block_scales = (q scales, k scales) [T, H, D / 32] E8M0 and v bf16
    (MXFP8 q/k). out is bf16.
    """
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check_qkv(q, k, v, out, block_scales)
    prob, cu = make_problem(q, cu_seqlens, block, sm_scale, causal, scales, block_scales)
    bh = (len(cu) - 1) * q.shape[1]
    _check_out(skipped, "skipped", _counter_dtypes(), bh, q.device)
    _check_out(total, "total", _counter_dtypes(), bh, q.device)
    if tile_mask is not None:
        nq, nk = tile_mask_dims(prob)
        _check_out(tile_mask, "tile_mask", (torch.uint8,), bh * nq * nk, q.device)
    vals = np.ascontiguousarray(np.atleast_1d(np.asarray(threshold, dtype=np.float64)))
    th = Thresholds(kind=_KINDS[kind], count=vals.size, values=vals.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    st = load_library().ssa_attn_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(th),
                                     _ptr(skipped), _ptr(total), _ptr(tile_mask), _stream(stream))
    _check(st, "ssa_attn_fwd")
    return out


def attn_calibrate(q, k, v, cu_seqlens, lambdas: Sequence[float], block: int = 128, sm_scale: float = 0.0,
                   out=None, counts=None, tiles=None, stream=None, causal: bool = False,
                   scales: Optional[Tuple[float, float, float]] = None, block_scales=None):
    """ssa_attn_calibrate; returns (out, counts [num_wg, n] int32, tiles [num_wg] int32) on the device."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check_qkv(q, k, v, out, block_scales)
    prob, cu = make_problem(q, cu_seqlens, block, sm_scale, causal, scales, block_scales)
    lam = np.ascontiguousarray(np.asarray(lambdas, dtype=np.float64))
    nwg = calib_num_workgroups(prob)
    if counts is None:
        counts = torch.empty((nwg, lam.size), dtype=torch.int32, device=q.device)
    if tiles is None:
        tiles = torch.empty((nwg,), dtype=torch.int32, device=q.device)
    _check_out(counts, "counts", (torch.int32,), nwg * lam.size, q.device)
    _check_out(tiles, "tiles", (torch.int32,), nwg, q.device)
    st = load_library().ssa_attn_calibrate(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                           lam.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), lam.size,
                                           _ptr(counts), _ptr(tiles), _stream(stream))
    _check(st, "ssa_attn_calibrate")
    return out, counts, tiles


def _check_host_counts(prob: Problem, c: np.ndarray, t: np.ndarray) -> None:
    """Host copies of a calibration pass must hold one row per work-group."""
    nwg = calib_num_workgroups(prob)
    if c.ndim != 2 or c.shape[0] != nwg or c.shape[1] < 1 or t.shape != (nwg,):
        raise ValueError(f"counts must be [{nwg}, n] and tiles [{nwg}] for this problem "
                         f"(got {c.shape} and {t.shape})")


def calibration_sparsity(cu_seqlens, num_heads: int, head_dim: int, block: int, counts: np.ndarray,
                         tiles: np.ndarray) -> np.ndarray:
    """ssa_calibration_sparsity on host copies; returns [B, n] tile sparsity."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.int32))
    prob = Problem(batch=len(cu) - 1, num_heads=num_heads, head_dim=head_dim, block=block,
                   cu_seqlens=cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                   stride_token=num_heads * head_dim, stride_head=head_dim, sm_scale=0.0)
    _check_host_counts(prob, c, t)
    n = c.shape[1]
    out = np.empty((len(cu) - 1, n), dtype=np.float64)
    P = ctypes.POINTER
    _check(load_library().ssa_calibration_sparsity(
        ctypes.byref(prob), c.ctypes.data_as(P(ctypes.c_int32)), t.ctypes.data_as(P(ctypes.c_int32)), n,
        out.ctypes.data_as(P(ctypes.c_double))), "ssa_calibration_sparsity")
    return out


def calibration_fit(lambdas, sparsity, seq_k, space: str = "log") -> CalibResult:
    """ssa_calibration_fit (space="log") or ssa_calibration_fit_linear (space="linear"):
    fit of scale_factor = a * exp(b * s)."""
    lam = np.ascontiguousarray(np.asarray(lambdas, dtype=np.float64))
    sp = np.ascontiguousarray(np.asarray(sparsity, dtype=np.float64))
    if lam.ndim != 1 or sp.shape != lam.shape:
        raise ValueError("lambdas and sparsity must be 1-D arrays of the same length")
    sk = np.ascontiguousarray(np.broadcast_to(np.asarray(seq_k, dtype=np.float64), lam.shape))
    res = CalibResult()
    P = ctypes.POINTER
    name = {"log": "ssa_calibration_fit", "linear": "ssa_calibration_fit_linear"}[space]
    _check(getattr(load_library(), name)(lam.ctypes.data_as(P(ctypes.c_double)),
                                         sp.ctypes.data_as(P(ctypes.c_double)),
                                         sk.ctypes.data_as(P(ctypes.c_double)), lam.size, ctypes.byref(res)),
           name)
    return res


class CalibrationPool:
    """ssa_calib_pool owned from Python: add calibration passes, read fit points."""

    def __init__(self, n_lambda: int, max_groups: int = 64):
        if n_lambda < 1 or max_groups < 0:
            raise ValueError("a pool needs n_lambda >= 1 and max_groups >= 0")
        self._seq_k = np.zeros(max_groups, dtype=np.int64)
        self._skipped = np.zeros(max_groups * n_lambda, dtype=np.int64)
        self._visited = np.zeros(max_groups, dtype=np.int64)
        P = ctypes.POINTER
        self.c = CalibPoolC(n_lambda=n_lambda, max_groups=max_groups, n_groups=0,
                            seq_k=self._seq_k.ctypes.data_as(P(ctypes.c_int64)),
                            skipped=self._skipped.ctypes.data_as(P(ctypes.c_int64)),
                            visited=self._visited.ctypes.data_as(P(ctypes.c_int64)))

    def add(self, cu_seqlens, num_heads: int, head_dim: int, block: int, counts, tiles) -> None:
        """Add one calibration pass (host or device counts [num_wg, n] and tiles [num_wg])
        of a problem with these sequence lengths, heads, head_dim and block size."""
        if hasattr(counts, "cpu"):
            counts, tiles = counts.cpu().numpy(), tiles.cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        c = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        t = np.ascontiguousarray(np.asarray(tiles, dtype=np.int32))
        P = ctypes.POINTER
        prob = Problem(batch=len(cu) - 1, num_heads=num_heads, head_dim=head_dim, block=block,
                       cu_seqlens=cu.ctypes.data_as(P(ctypes.c_int32)), stride_token=num_heads * head_dim,
                       stride_head=head_dim, sm_scale=0.0)
        _check_host_counts(prob, c, t)
        _check(load_library().ssa_calibration_pool_add(ctypes.byref(prob), c.ctypes.data_as(P(ctypes.c_int32)),
                                                       t.ctypes.data_as(P(ctypes.c_int32)), c.shape[1],
                                                       ctypes.byref(self.c)), "ssa_calibration_pool_add")

    def points(self, lambdas) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        lam = np.ascontiguousarray(np.asarray(lambdas, dtype=np.float64))
        if lam.shape != (self.c.n_lambda,):
            raise ValueError(f"lambdas must hold the pool's {self.c.n_lambda} thresholds")
        m = self.c.n_groups * self.c.n_lambda
        outs = [np.empty(m, dtype=np.float64) for _ in range(3)]
        n = ctypes.c_int32()
        P = ctypes.POINTER
        _check(load_library().ssa_calibration_pool_points(
            ctypes.byref(self.c), lam.ctypes.data_as(P(ctypes.c_double)),
            *[o.ctypes.data_as(P(ctypes.c_double)) for o in outs], ctypes.byref(n)), "ssa_calibration_pool_points")
        return tuple(o[:n.value] for o in outs)

    @property
    def groups(self):
        g = self.c.n_groups
        return {int(self._seq_k[i]): (self._skipped[i * self.c.n_lambda:(i + 1) * self.c.n_lambda].copy(),
                                      int(self._visited[i])) for i in range(g)}


def resolve_threshold(seq_k: int, raw_log2=None, lam=None, scale_factor=None, target_sparsity=None,
                      a=None, log_a=None, b=None, s_min=None, s_max=None) -> Tuple[int, float, float]:
    """ssa_resolve_threshold; returns (status, lambda, log2 lambda). Errors raise SSAError."""
    spec = ThresholdSpec()
    for flag, name, val in ((SPEC_RAW_LOG2, "raw_log2", raw_log2), (SPEC_LAMBDA, "lambda_", lam),
                            (SPEC_SCALE_FACTOR, "scale_factor", scale_factor),
                            (SPEC_TARGET, "target_sparsity", target_sparsity), (SPEC_A, "a", a),
                            (SPEC_LOG_A, "log_a", log_a), (SPEC_B, "b", b)):
        if val is not None:
            spec.set |= flag
            setattr(spec, name, float(val))
    if s_min is not None and s_max is not None:
        spec.set |= SPEC_RANGE
        spec.s_min, spec.s_max = float(s_min), float(s_max)
    out_l, out_t = ctypes.c_double(), ctypes.c_double()
    st = load_library().ssa_resolve_threshold(ctypes.byref(spec), int(seq_k), ctypes.byref(out_l), ctypes.byref(out_t))
    _check(st, "ssa_resolve_threshold")
    return st, out_l.value, out_t.value


# ---- timestep and layer gating (host) -----------------------------------------
def gate_layer(layer: str, timesteps, base_scale_factor: float, cutoff: Optional[float] = None,
               ignore: Sequence[str] = (), overrides: Sequence[Tuple[str, float]] = ()) -> Tuple[int, float]:
    """ssa_gate_layer: (rule, effective threshold_scale_factor) of one layer at one forward."""
    ts = np.ascontiguousarray(np.atleast_1d(np.asarray(timesteps, dtype=np.float64)))
    ign = (ctypes.c_char_p * max(1, len(ignore)))(*[p.encode() for p in ignore])
    ovr = (LayerOverride * max(1, len(overrides)))(*[LayerOverride(p.encode(), float(v)) for p, v in overrides])
    spec = GateSpec(disabled_until_timestep=float("nan") if cutoff is None else float(cutoff),
                    ignore=ign, n_ignore=len(ignore), overrides=ovr, n_overrides=len(overrides))
    sf, rule = ctypes.c_double(), ctypes.c_int32()
    _check(load_library().ssa_gate_layer(ctypes.byref(spec), layer.encode(),
                                         ts.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ts.size,
                                         float(base_scale_factor), ctypes.byref(sf), ctypes.byref(rule)),
           "ssa_gate_layer")
    return rule.value, sf.value


def flow_timesteps(n_steps: int, num_train_timesteps: int = 1000, flow_shift: float = 3.0) -> np.ndarray:
    """ssa_flow_timesteps: normalized runtime timesteps of an n-step flow schedule."""
    t = np.empty(max(0, n_steps), dtype=np.float64)
    _check(load_library().ssa_flow_timesteps(int(n_steps), int(num_train_timesteps), float(flow_shift),
                                             t.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "ssa_flow_timesteps")
    return t


def gate_dense_steps(timesteps, cutoff: Optional[float]) -> int:
    """ssa_gate_dense_steps: count(t >= cutoff); None = no cutoff."""
    ts = np.ascontiguousarray(np.asarray(timesteps, dtype=np.float64))
    n = ctypes.c_int32()
    _check(load_library().ssa_gate_dense_steps(ts.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ts.size,
                                               float("nan") if cutoff is None else float(cutoff),
                                               ctypes.byref(n)),
           "ssa_gate_dense_steps")
    return n.value

"""Seeded 3D-grid video-token inputs for non-causal diffusion self-attention.

Stand-in for the WAN 2.2 self-attention workload that the TensorRT-LLM pull
request "Add SkipSoftmax sparse attention support for visual generation"
benchmarks (section "Benchmark": 720x1280, 81 frames, sequence length about
75K). No prompts, weights or datasets are used: the inputs are synthetic with
the same shapes and a distance-decaying logit structure, so that the
fraction of KV tiles that add almost nothing behaves like a video model's.

Recipe (the pages fix none of the constants; each is a stated choice):

* Token t of a sequence sits at grid point p = (f, r, c) of an F x Hg x Wg
  latent grid, frame-major: t = (f * Hg + r) * Wg + c.
* Per head, a locality length ell_h ~ U[2, 16] grid units and 8 frequency
  vectors w_k ~ N(0, ell_h^-2 I_3).
* phi(p) = A * [sin(w_1.p), cos(w_1.p), ..., sin(w_8.p), cos(w_8.p)] fills
  dims 0..15; dims 16..D-1 are zero. E[q.k] then decays like
  exp(-|dp|^2 / (2 ell^2)) with grid distance.
* q = sigma * N(0, I_D) + phi(p), k = sigma * N(0, I_D) + phi(p), v ~ N(0, I_D).
* A^2 = L * sqrt(D) / 8 with peak logit L = 40 nats: q.k / sqrt(D) reaches L
  for a token against itself, large enough that the strictest thresholds
  still skip roughly a third of the tiles, the floor the ModelOpt README
  ("Known Issues") reports for real diffusion models.
* numpy default_rng(seed); draws in a fixed order: ell for all heads, w for
  all heads, then per sequence and per head: q-noise, k-noise, v.
* Q/K/V are produced in fp32 and rounded to bf16 (round to nearest even);
  both the GPU path and the oracle consume exactly those bf16 values.

This module contains no attention arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

PEAK_LOGIT_NATS = 40.0
N_FREQ = 8  # 8 frequency vectors -> 16 sin/cos features


@dataclasses.dataclass(frozen=True)
class VideoTokenConfig:
    """One synthetic workload: B sequences, each on its own (F, Hg, Wg) grid."""

    name: str
    grids: Tuple[Tuple[int, int, int], ...]
    num_heads: int
    head_dim: int
    sigma: float
    block: int
    seed: int
    ell_range: Tuple[float, float] = (2.0, 16.0)
    peak_logit: float = PEAK_LOGIT_NATS

    @property
    def seq_lens(self) -> List[int]:
        return [f * h * w for (f, h, w) in self.grids]

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    def dense_flops(self) -> float:
        """Dense-equivalent FLOP of one forward: sum_b 4 * S_b^2 * H * D."""
        return float(sum(4.0 * s * s * self.num_heads * self.head_dim for s in self.seq_lens))


# The five workloads: tiny (oracle-sized), WAN-5B-like, the WAN-14B 720p
# headline, its calibration pass (same shape, its own seed), and a varlen
# batch of 720p / 480p / 240p-sized sequences.
CONFIGS: Dict[str, VideoTokenConfig] = {
    "tiny": VideoTokenConfig("tiny", ((4, 16, 16),), 2, 64, 0.5, 64, seed=0),
    "wan5b": VideoTokenConfig("wan5b", ((16, 32, 32),), 24, 128, 1.0, 128, seed=1),
    "headline": VideoTokenConfig("headline", ((21, 45, 80),), 40, 128, 0.5, 128, seed=2),
    "calib": VideoTokenConfig("calib", ((21, 45, 80),), 40, 128, 0.5, 128, seed=3),
    "varlen": VideoTokenConfig(
        "varlen", ((21, 45, 80), (21, 30, 52), (21, 15, 26)), 40, 128, 0.5, 128, seed=4
    ),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of each bf16 bit pattern."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


E4M3_MAX = 448.0


def e4m3_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of each OCP e4m3 ("e4m3fn") byte: 1 sign, 4 exponent (bias 7),
    3 mantissa bits, subnormals at exponent 0, NaN at S.1111.111, no infinities."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int32)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & ((b & 7) == 7), np.nan, val)
    return (sign * val).astype(np.float32)


_E4M3_POS = e4m3_bits_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)  # codes 0..126, ascending


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (ties to the even code), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)  # first code with value >= a
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_e4m3(values: np.ndarray):
    """Per-tensor e4m3 quantization: scale = max|x| / 448; returns (bytes, scale)."""
    amax = float(np.max(np.abs(values))) if values.size else 0.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    return f32_to_e4m3_bits(np.asarray(values, np.float64) / scale), scale


def make_fp8_inputs(x: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """e4m3 versions of bf16 inputs from `make_inputs`: q8/k8/v8 bytes [T,H,D]
    and their per-tensor dequantization scales (value = code * scale).
    Each bf16 bit pattern is converted once (a 65,536-entry table), which is
    the same as converting every element."""
    out = {"cu_seqlens": x["cu_seqlens"]}
    with np.errstate(invalid="ignore"):
        all_bf16 = bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float64)
    for n in ("q", "k", "v"):
        used = np.zeros(65536, dtype=bool)
        used[np.asarray(x[n]).ravel()] = True
        vals = all_bf16[used]
        amax = float(np.max(np.abs(vals[np.isfinite(vals)]))) if vals.size else 0.0
        scale = amax / E4M3_MAX if amax > 0 else 1.0
        lut = f32_to_e4m3_bits(np.where(np.isfinite(all_bf16), all_bf16, 0.0) / scale)
        out[n + "8"] = lut[x[n]]
        out["scale_" + n] = scale
    return out


# MXFP8 (OCP microscaling formats, MX E4M3): one E8M0 scale per block of
# MX_BLOCK consecutive elements along the head dimension.
MX_BLOCK = 32
E4M3_EMAX = 8  # exponent of the largest e4m3 normal: 448 = 1.75 * 2^8


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(code - 127) (code 255, NaN, is never produced here)."""
    return np.ldexp(1.0, np.asarray(codes, dtype=np.int32) - 127)


_BF16_TO_E4M3 = None


def _bf16_to_e4m3_table() -> np.ndarray:
    """e4m3 code (round to nearest even, saturating) of every finite bf16 bit pattern."""
    global _BF16_TO_E4M3
    if _BF16_TO_E4M3 is None:
        with np.errstate(invalid="ignore"):
            v = bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float64)
        _BF16_TO_E4M3 = f32_to_e4m3_bits(np.where(np.isfinite(v), v, 0.0))
    return _BF16_TO_E4M3


def quantize_mxfp8_bf16(bits: np.ndarray):
    """MX E4M3 quantization of bf16 bit patterns [..., D] along the last axis.

    Each block of 32 consecutive elements gets the shared scale
    X = 2^(floor(log2(amax)) - 8) (E8M0 code floor(log2(amax)) + 119, at
    least 0), and each element the e4m3 code of v / X, rounded to nearest
    even and saturated at +-448. Because X is a power of two, v / X is the
    bf16 value with its exponent field lowered by log2(X), so the code of a
    normal v comes from the bf16 -> e4m3 table; a scaled magnitude below the
    bf16 normal range gives +-0, zeros stay +-0, and bf16 subnormals are
    rounded directly. Returns (codes uint8 [..., D], scales uint8 [..., D / 32])."""
    b = np.asarray(bits, dtype=np.uint16)
    D = b.shape[-1]
    assert D % MX_BLOCK == 0
    lut = _bf16_to_e4m3_table()
    blk = b.reshape(b.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)).astype(np.int32)
    field = (blk & 0x7FFF) >> 7                      # bf16 exponent field of each element
    amax_field = field.max(axis=-1)                  # that of the block maximum
    scale = np.clip(amax_field - E4M3_EMAX, 0, 254)  # E8M0 code: (amax_field - 127) - 8 + 127
    e = (scale - 127)[..., None]                     # X = 2^e
    ok = (field >= 1) & ((field - e) >= 1)           # a normal v whose v / X is still a bf16 normal
    shifted = (blk - (e << 7)) & 0xFFFF
    codes = np.where(ok, lut[shifted], np.where(blk & 0x8000, 0x80, 0)).astype(np.uint8)
    sub = (field == 0) & ((blk & 0x7F) != 0)         # bf16 subnormals: round v / X directly
    if np.any(sub):
        v = bf16_bits_to_f32(blk[sub].astype(np.uint16)).astype(np.float64)
        codes[sub] = f32_to_e4m3_bits(v / np.ldexp(1.0, np.broadcast_to(e, blk.shape)[sub]))
    return codes.reshape(b.shape), scale.astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact fp64 values code * 2^(scale - 127) of MX E4M3 data [..., D]."""
    return e4m3_bits_to_f32(codes).astype(np.float64) * np.repeat(e8m0_to_f64(scales), MX_BLOCK, axis=-1)


def make_mxfp8_qk_inputs(x: Dict[str, np.ndarray], chunk: int = 4096) -> Dict[str, np.ndarray]:
    """MX E4M3 versions of q and k from `make_inputs` (v stays bf16):
    q8, k8 uint8 [T, H, D] and q_bscale, k_bscale uint8 [T, H, D / 32].
    Tokens are processed `chunk` at a time to bound host memory."""
    out = {"cu_seqlens": x["cu_seqlens"], "v": x["v"]}
    for n in ("q", "k"):
        src = np.asarray(x[n])
        T, H, D = src.shape
        codes = np.empty((T, H, D), dtype=np.uint8)
        scales = np.empty((T, H, D // MX_BLOCK), dtype=np.uint8)
        for t0 in range(0, T, chunk):
            codes[t0:t0 + chunk], scales[t0:t0 + chunk] = quantize_mxfp8_bf16(src[t0:t0 + chunk])
        out[n + "8"] = codes
        out[n + "_bscale"] = scales
    return out


def grid_positions(grid: Sequence[int]) -> np.ndarray:
    """(S, 3) float64 grid coordinates (f, r, c) in frame-major token order."""
    f, h, w = grid
    ff, rr, cc = np.meshgrid(np.arange(f), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([ff.ravel(), rr.ravel(), cc.ravel()], axis=1).astype(np.float64)


def fourier_amplitude(head_dim: int, peak_logit: float = PEAK_LOGIT_NATS) -> float:
    """A with 8 * A^2 / sqrt(D) = peak_logit (8 cos terms equal to 1 at zero distance)."""
    return math.sqrt(peak_logit * math.sqrt(head_dim) / N_FREQ)


def make_inputs(cfg: VideoTokenConfig, heads: Sequence[int] | None = None) -> Dict[str, np.ndarray]:
    """Generate bf16 Q, K, V for `cfg` as uint16 bit arrays of shape [T, H, D].

    `heads` restricts generation to a subset of heads (the others stay zero);
    the random stream is still consumed in full order so every generated head
    is identical to the full generation.
    Returns dict(q, k, v: uint16 [T,H,D]; cu_seqlens: int32 [B+1]; ell: [H]).
    """
    rng = np.random.default_rng(cfg.seed)
    H, D = cfg.num_heads, cfg.head_dim
    lo, hi = cfg.ell_range
    ell = rng.uniform(lo, hi, size=H)
    omega = rng.standard_normal((H, N_FREQ, 3)) / ell[:, None, None]
    amp = fourier_amplitude(D, cfg.peak_logit)
    want = set(range(H)) if heads is None else set(int(h) for h in heads)

    T = cfg.total_tokens
    out = {name: np.zeros((T, H, D), dtype=np.uint16) for name in ("q", "k", "v")}
    cu = cfg.cu_seqlens
    for b, grid in enumerate(cfg.grids):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        S = s1 - s0
        pos = grid_positions(grid)
        for h in range(H):
            qn = rng.standard_normal((S, D), dtype=np.float32)
            kn = rng.standard_normal((S, D), dtype=np.float32)
            vv = rng.standard_normal((S, D), dtype=np.float32)
            if h not in want:
                continue
            phase = pos @ omega[h].T  # (S, 8)
            feat = np.empty((S, 2 * N_FREQ), dtype=np.float64)
            feat[:, 0::2] = np.sin(phase)
            feat[:, 1::2] = np.cos(phase)
            feat *= amp
            q = cfg.sigma * qn
            k = cfg.sigma * kn
            q[:, : 2 * N_FREQ] += feat.astype(np.float32)
            k[:, : 2 * N_FREQ] += feat.astype(np.float32)
            out["q"][s0:s1, h, :] = f32_to_bf16_bits(q)
            out["k"][s0:s1, h, :] = f32_to_bf16_bits(k)
            out["v"][s0:s1, h, :] = f32_to_bf16_bits(vv)
    out["cu_seqlens"] = cu
    out["ell"] = ell
    return out


def make_random_inputs(seq_lens: Sequence[int], num_heads: int, head_dim: int, seed: int,
                       scale: float = 1.0, v_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Plain bf16 inputs for edge-case shapes (ragged lengths, empty sequences):
    Q, K ~ N(0, scale^2), which sharpens the softmax rows as scale grows, and
    V ~ N(0, v_scale^2), N(0, 1) as in every video configuration by default."""
    rng = np.random.default_rng(seed)
    T = int(sum(seq_lens))
    out = {}
    for name in ("q", "k", "v"):
        sd = v_scale if name == "v" else scale
        x = (sd * rng.standard_normal((T, num_heads, head_dim))).astype(np.float32)
        out[name] = f32_to_bf16_bits(x)
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int32)
    return out

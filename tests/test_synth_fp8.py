"""The e4m3 input encoder in `synth` against torch's float8_e4m3fn casts (CPU only)."""
import numpy as np
import torch

from synth import (CONFIGS, bf16_bits_to_f32, e4m3_bits_to_f32, f32_to_e4m3_bits, make_fp8_inputs, make_inputs,
                   quantize_e4m3)


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_bits_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.all((mine == ref) | both_nan)
    assert np.nanmax(mine) == 448.0 and np.nanmin(np.abs(mine[mine != 0])) == 2.0 ** -9


def test_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(300000) * np.exp2(rng.uniform(-14, 9, 300000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    # exact codes and the midpoints between neighbours (ties to even)
    vals = e4m3_bits_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, vals.astype(np.float32), mids, -mids])
    mine = f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_saturation_and_per_tensor_scale():
    assert e4m3_bits_to_f32(f32_to_e4m3_bits(np.array([1e6, -1e6, 449.0])))[0] == 448.0
    x = np.array([[0.5, -3.0], [1.5, 2.25]], dtype=np.float32)
    codes, scale = quantize_e4m3(x)
    assert scale == 3.0 / 448.0
    assert np.max(np.abs(e4m3_bits_to_f32(codes))) == 448.0
    rel = np.abs(e4m3_bits_to_f32(codes) * scale - x) / np.abs(x)
    assert np.all(rel <= 2.0 ** -4 + 1e-12)


def test_fp8_inputs_from_bf16_config():
    x = make_inputs(CONFIGS["tiny"])
    f = make_fp8_inputs(x)
    for n in ("q", "k", "v"):
        assert f[n + "8"].dtype == np.uint8 and f[n + "8"].shape == x[n].shape
        assert f["scale_" + n] > 0


# ---- block-scaled (MX E4M3) q/k inputs --------------------------------------------------------
from synth import (e8m0_to_f64, f32_to_bf16_bits, make_mxfp8_qk_inputs, mxfp8_dequantize,  # noqa: E402
                   quantize_mxfp8_bf16)


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_mx_scale_rule_and_saturation():
    """Shared scale 2^(floor(log2 amax) - 8) per 32 elements; codes of v / X,
    saturating at 448 (OCP MX: emax of e4m3 is 8)."""
    rows = np.zeros((4, 64), dtype=np.float32)
    rows[0, :32] = 448.0                 # amax 448: floor(log2) = 8 -> X = 1 (code 127)
    rows[1, 5] = 1.0                     # amax 1: X = 2^-8 (code 119); the rest of the block is 0
    rows[2, 0] = 7.9375                  # amax in [4, 8): X = 2^-6; 7.9375 / X = 508 saturates to 448
    rows[2, 1] = -0.75                   # -0.75 / 2^-6 = -48 exactly
    rows[3, 40] = 3.0e-30                # floor(log2) = -99: code 20
    rows[3, 0] = 1.0e-37                 # floor(log2) = -123: code -4, clipped at 0
    codes, scales = quantize_mxfp8_bf16(_bf16(rows))
    assert scales.shape == (4, 2)
    assert scales[0, 0] == 127 and scales[1, 0] == 119 and scales[2, 0] == 121
    assert scales[0, 1] == scales[1, 1] == scales[2, 1] == 0      # all-zero blocks
    assert scales[3, 1] == 20 and scales[3, 0] == 0
    deq = mxfp8_dequantize(codes, scales)
    assert np.all(deq[0, :32] == 448.0) and deq[1, 5] == 1.0
    assert deq[2, 0] == 448.0 * 2.0 ** -6 and deq[2, 1] == -0.75
    assert np.all(deq[:3, 32:] == 0.0)
    np.testing.assert_array_equal(e8m0_to_f64(np.array([0, 127, 254])), [2.0 ** -127, 1.0, 2.0 ** 127])


def test_mx_codes_equal_direct_rounding():
    """The bit-pattern path equals e4m3 round-to-nearest-even of v / X
    computed directly, element for element."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((512, 128)) * np.exp2(rng.uniform(-20, 12, (512, 1)))
         * np.exp2(rng.uniform(-6, 0, (512, 128)))).astype(np.float32)
    x[:, 7] = 0.0
    x[::7, 64:96] = 0.0                     # whole zero blocks
    x[1::9, 100] = -0.0
    x[2::11, 33] = np.float32(3e-39)        # bf16 subnormals
    x[3::13, 96:128] = np.float32(1e-36)    # tiny blocks: X = 2^-127, the scaled zeros must stay zero
    x[3::13, 97] = 0.0
    bits = _bf16(x)
    codes, scales = quantize_mxfp8_bf16(bits)
    v = bf16_bits_to_f32(bits).astype(np.float64)
    X = np.repeat(e8m0_to_f64(scales), 32, axis=-1)
    direct = f32_to_e4m3_bits(v / X)
    np.testing.assert_array_equal(codes, direct)
    assert np.all(mxfp8_dequantize(codes, scales)[v == 0] == 0.0)
    # every block whose scale is not clipped at 2^-127 has its maximum scaled
    # into [256, 512): the largest e4m3 binade, or saturation
    amax = np.abs(v).reshape(512, 4, 32).max(-1)
    nz = scales > 0
    ratio = amax[nz] / e8m0_to_f64(scales)[nz]
    assert np.all((ratio >= 256) & (ratio < 512))
    assert np.all(scales[3::13, 3] == 0)


def test_mx_dequantization_error_bound():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((256, 64)) * 3).astype(np.float32)
    bits = _bf16(x)
    codes, scales = quantize_mxfp8_bf16(bits)
    v = bf16_bits_to_f32(bits).astype(np.float64)
    X = np.repeat(e8m0_to_f64(scales), 32, axis=-1)
    deq = mxfp8_dequantize(codes, scales)
    sat = np.abs(v) / X > 448
    # round to nearest with 3 mantissa bits: half an ulp of the value's binade (subnormals: 2^-10 X)
    binade = np.exp2(np.floor(np.log2(np.maximum(np.abs(v) / X, 2.0 ** -6))))
    assert np.all(np.abs(deq - v)[~sat] <= (binade * 2.0 ** -4 * X)[~sat])
    np.testing.assert_array_equal(np.abs(deq[sat]), (448.0 * X)[sat])


def test_mx_inputs_from_bf16_config():
    x = make_inputs(CONFIGS["tiny"])
    m = make_mxfp8_qk_inputs(x, chunk=100)          # several chunks, a ragged last one
    T, H, D = x["q"].shape
    assert m["q8"].shape == (T, H, D) and m["k_bscale"].shape == (T, H, D // 32)
    assert m["v"] is x["v"]
    whole = make_mxfp8_qk_inputs(x, chunk=T)
    for n in ("q8", "k8", "q_bscale", "k_bscale"):
        np.testing.assert_array_equal(m[n], whole[n])
    deq = mxfp8_dequantize(m["q8"], m["q_bscale"])
    ref = bf16_bits_to_f32(x["q"]).astype(np.float64)
    rel = np.abs(deq - ref).max() / np.abs(ref).max()
    assert rel < 0.13          # bounded by saturation of block maxima (at most 1 - 448 / 512)

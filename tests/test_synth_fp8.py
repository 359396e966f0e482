"""The e4m3 input encoder in `synth` against torch's float8_e4m3fn casts (CPU only)."""
import numpy as np
import torch

from synth import e4m3_bits_to_f32, f32_to_e4m3_bits, make_fp8_inputs, make_inputs, quantize_e4m3, CONFIGS


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

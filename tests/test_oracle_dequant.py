"""The oracle's per-channel e4m3 -> bf16 weight dequant (the W8A16 arm's building block).

Pinned against torch: the float8_e4m3fn decode, a float32 multiply and the bfloat16 cast
(round half to even), computed independently here, on every code value and on random
rows; and the W8A16 linear built from it is the oracle's W8A16 counterfactual (the
activation never quantized).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def _torch_dequant(codes, ws):
    w = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32)
    return (w * torch.from_numpy(np.asarray(ws, np.float32)).reshape(-1, 1)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_every_code_at_random_scales():
    from oracle import dequant_channel_bf16
    rng = np.random.default_rng(3)
    codes = np.tile(np.arange(256, dtype=np.uint8), (64, 1))
    ws = rng.uniform(1e-4, 1e-1, 64).astype(np.float32)
    got, want = dequant_channel_bf16(codes, ws), _torch_dequant(codes, ws)
    nan = (codes & 0x7F) == 0x7F
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)             # NaN codes stay NaN


def test_synthetic_weight_rows():
    from oracle import dequant_channel_bf16
    from workloads import block_params
    p = block_params(0, 0)
    w, ws = p["out_w"][:256], p["out_w_scale"][:256]
    assert np.array_equal(dequant_channel_bf16(w, ws), _torch_dequant(w, ws))


def test_w8a16_linear_from_the_dequant():
    """x_bf16 @ dequant(W)^T is the oracle's W8A16 arm; it differs from W8A8 by the
    activation quantization alone."""
    from oracle import bf16_to_f64, dequant_channel_bf16, fp8_linear, quantize_static
    from workloads import linear_case
    a, w, ws, sa = linear_case(4, 256, 512, extra=2)
    w16 = bf16_to_f64(dequant_channel_bf16(w, ws))
    y16 = bf16_to_f64(a) @ w16.T
    y8 = fp8_linear(quantize_static(a, sa), w, ws, sa)
    rms = np.sqrt(np.mean(y8 ** 2))
    d = np.max(np.abs(y16 - y8)) / rms
    assert 1e-3 < d < 0.5                                    # a real but bounded difference

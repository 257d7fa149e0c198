"""The per-channel e4m3 -> bf16 weight dequant (W8A16 arm) on the GPU: bit-exact with the
oracle, and the W8A16 linear built from it against the oracle's W8A16 counterfactual."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nhm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_w8a8_linear_amd as m
    return m


def _same(got, want):
    nan = (want & 0x7FFF) > 0x7F80
    return np.array_equal(got[~nan], want[~nan]) and np.all((got[nan] & 0x7FFF) > 0x7F80)


def test_dequant_every_code(nhm):
    from oracle import dequant_channel_bf16
    from tests.gpu_util import dev, host
    rng = np.random.default_rng(11)
    codes = np.tile(np.arange(256, dtype=np.uint8), (96, 1))
    ws = rng.uniform(1e-5, 1.0, 96).astype(np.float32)
    got = host(nhm.fp8_dequant_channel_bf16(dev(codes), dev(ws)))
    torch.cuda.synchronize()
    assert _same(got, dequant_channel_bf16(codes, ws))


@pytest.mark.parametrize("n,k,pad_w,pad_o", [(10304, 2688, 0, 0), (2688, 4096, 0, 0), (7, 16, 16, 8), (300, 48, 0, 24)])
def test_dequant_weights(nhm, n, k, pad_w, pad_o):
    from oracle import dequant_channel_bf16
    from tests.gpu_util import dev
    from workloads import linear_case
    _, w, ws, _ = linear_case(1, n, k, extra=12)
    wp = np.zeros((n, k + pad_w), np.uint8)
    wp[:, :k] = w
    wd, sd = dev(wp), dev(ws)
    out = torch.full((n, k + pad_o), 0x1234, dtype=torch.int16, device="cuda")
    import ctypes as C                                       # row strides k + pad through the raw ABI
    st = nhm.lib.nhm_fp8_dequant_channel_bf16(C.c_void_p(wd.data_ptr()), C.c_void_p(sd.data_ptr()), n, k, k + pad_w,
                                              C.c_void_p(out.data_ptr()), k + pad_o,
                                              C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, nhm.lib.nhm_last_error()
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[:, :k], dequant_channel_bf16(w, ws))
    assert np.all(o[:, k:] == 0x1234)                        # the row padding is untouched


def test_w8a16_counterfactual_on_gpu(nhm):
    """The W8A16 arm (bf16 activation x dequantized weight, f32 accumulation by torch on the
    GPU) against the oracle's W8A16 linear, and its separation from the W8A8 linear."""
    from oracle import bf16_to_f64, dequant_channel_bf16, fp8_linear, quantize_static
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(8, 10304, 2688, extra=13)
    w16 = nhm.fp8_dequant_channel_bf16(dev(w), dev(ws))
    x = dev(a)
    y16 = (x.view(torch.bfloat16).float() @ w16.view(torch.bfloat16).float().T).cpu().numpy().astype(np.float64)
    ref16 = bf16_to_f64(a) @ bf16_to_f64(dequant_channel_bf16(w, ws)).T
    rms = np.sqrt(np.mean(ref16 ** 2))
    assert np.max(np.abs(y16 - ref16)) <= 1e-4 * rms         # f32 sums of exact bf16 products
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    y8 = bf16_to_f64(host(nhm.fp8_linear(x, W)))
    ref8 = fp8_linear(quantize_static(a, sa), w, ws, sa)
    sep = np.max(np.abs(ref16 - ref8)) / rms
    assert np.max(np.abs(y8 - ref8)) / rms <= 2e-2 < sep     # W8A8 matches its oracle, not W8A16
    print(f"W8A16 vs W8A8 separation {sep:.3f}")

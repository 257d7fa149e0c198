"""a1 / a9 parity: the HIP static quant is bit-exact with the oracle's E4M3(f32(x)/s)."""
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


ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("scale", [np.float32(4.0 / 448.0), np.float32(1.0), np.float32(0.37),
                                   np.float32(3.0e-3), np.float32(17.25), np.float32(1e-30)])
def test_quant_all_bf16_patterns_bit_exact(nhm, scale):
    from oracle import quantize_static
    from tests.gpu_util import dev, host
    x = ALL.reshape(256, 256)
    want = quantize_static(x, np.array([scale]))
    got = host(nhm.quantize_static(dev(x), dev(np.array([scale], np.float32))))
    torch.cuda.synchronize()
    assert got.shape == want.shape == (256, 256)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first x=0x{x[bad][0]:04x} got 0x{got[bad][0]:02x} want 0x{want[bad][0]:02x}"


@pytest.mark.parametrize("rows,cols", [(1, 2688), (8, 2688), (3, 13), (5, 4096), (17, 40), (0, 8)])
def test_quant_shapes_random_scales(nhm, rows, cols):
    from oracle import quantize_static
    from tests.gpu_util import dev, host
    from workloads import bf16_bits
    r = np.random.default_rng(rows * 1000 + cols)
    x = bf16_bits(r.standard_normal((rows, cols)).astype(np.float32) * 3)
    s = np.array([r.uniform(1e-3, 1.0)], np.float32)
    if rows == 0:
        q = torch.empty((0, cols), dtype=torch.uint8, device="cuda")
        nhm.quantize_static(dev(x), dev(s), q=q)
        return
    got = host(nhm.quantize_static(dev(x), dev(s)))
    assert np.array_equal(got, quantize_static(x, s))


def test_quant_strided_rows(nhm):
    """ld_x > cols and ld_q > cols through the raw ABI."""
    import ctypes as C
    from oracle import quantize_static
    from tests.gpu_util import dev, host
    from workloads import bf16_bits
    r = np.random.default_rng(5)
    xf = bf16_bits(r.standard_normal((6, 40)).astype(np.float32))
    xd = dev(xf)
    s = dev(np.array([0.05], np.float32))
    q = torch.full((6, 48), 0xAB, dtype=torch.uint8, device="cuda")
    st = nhm.lib.nhm_fp8_quantize_static(C.c_void_p(xd.data_ptr()), 6, 24, 40, C.c_void_p(s.data_ptr()),
                                         C.c_void_p(q.data_ptr()), 48, C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    got = host(q)
    assert np.array_equal(got[:, :24], quantize_static(xf[:, :24], np.array([0.05], np.float32)))
    assert np.all(got[:, 24:] == 0xAB)

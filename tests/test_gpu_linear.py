"""a2 / a10 parity: the HIP W8A8 GEMV / GEMM against the oracle's dequantize-then-matmul.

Bound (derived from the arithmetic): the kernel accumulates exact e4m3 products
in f32 and rounds the scaled result once to bf16, so
    |gpu - ref| <= 2^-8 |ref| + 2^-16 * S,   S = sum_k |a_k w_k| * s_a * ws_n,
one bf16 ulp plus a generous f32 accumulation term. The block tolerance
(max |d| <= 2e-2 RMS(ref)) is asserted as well.
"""
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


def _check(nhm, a_bf16, w, ws, sa, via_e4m3=False, ld_pad=0):
    from oracle import bf16_to_f64, e4m3_decode, fp8_linear, quantize_static
    from tests.gpu_util import dev, host, rel_max
    m, k = a_bf16.shape
    n = w.shape[0]
    q = quantize_static(a_bf16, sa)
    ref = fp8_linear(q, w, ws, sa)
    S = np.abs(e4m3_decode(q)) @ np.abs(e4m3_decode(w)).T * np.float64(sa[0]) * ws.astype(np.float64)[None, :]
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    a_in = dev(q) if via_e4m3 else dev(a_bf16)
    a_type = nhm.NHM_E4M3 if via_e4m3 else nhm.NHM_BF16
    out = torch.full((m, n + ld_pad), 0x7777, dtype=torch.int16, device="cuda")
    if ld_pad == 0:
        nhm.fp8_linear(a_in, W, out=out, a_type=a_type)
    else:                                 # row stride n + ld_pad through the raw ABI
        import ctypes as C
        need = nhm.fp8_linear_workspace_bytes(m, n, k, a_type)
        wsb = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        st = nhm.lib.nhm_fp8_linear(C.c_void_p(a_in.data_ptr()), a_type, m, k, C.byref(W.struct),
                                    C.c_void_p(out.data_ptr()), n + ld_pad, C.c_void_p(wsb.data_ptr()),
                                    wsb.numel(), C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, nhm.lib.nhm_last_error()
    torch.cuda.synchronize()
    o = host(out)
    got = bf16_to_f64(o[:, :n])
    if ld_pad:
        assert np.all(o[:, n:] == 0x7777)
    assert got.shape == ref.shape == (m, n) and got.size == m * n
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * S
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"
    assert rel_max(got, ref) <= 2e-2
    return o


@pytest.mark.parametrize("m,n,k", [(1, 10304, 2688), (8, 10304, 2688), (512, 10304, 2688),
                                   (1, 2688, 4096), (512, 2688, 4096), (64, 4096, 4096)])
def test_linear_sweep_shapes(nhm, m, n, k):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k)
    _check(nhm, a, w, ws, sa)


# m <= 16: GEMV; m <= 640: a ring kernel when it has >= 160 tiles -- 192 x 128 (384 x 10300
# x 2608: 162 tiles; 500 x 10000 x 2672: ragged m, n and k) or 256 x 128, whichever puts fewer
# operand bytes on a CU (600 x 10304: 205 tiles of 256 x 128 against 270 of 192 x 128) --
# else the 64 x 128 panel kernel; larger m: the 256 x 256 tile kernel
# when it has >= 160 tiles (the last two shapes), else the 128 x 128 one. The ragged shapes cut every kind of tile edge (2600 x 4100
# x 272: partial m and n tiles, n % 8 != 0, k ending inside a 64-byte ring stage).
@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (3, 100, 48), (16, 200, 272), (17, 130, 256),
                                   (130, 70, 144), (5, 1000, 4096), (200, 10304, 2688),
                                   (384, 10300, 2608), (500, 10000, 2672), (600, 10304, 2688), (641, 130, 256), (700, 520, 272),
                                   (2600, 4100, 272), (1030, 10304, 2688),
                                   (3, 520, 12288), (2, 130, 16384)])     # the GEMV's 16-wave variants
def test_linear_ragged(nhm, m, n, k):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=7)
    _check(nhm, a, w, ws, sa)


@pytest.mark.parametrize("m", [1, 8, 64])
def test_linear_prequantized_input(nhm, m):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, 2688, 4096, extra=3)
    _check(nhm, a, w, ws, sa, via_e4m3=True)


# A per-tensor weight scale (one scalar per projection) is the per-channel vector with every
# entry equal: through the GEMV, the 64 x 128 panel, the 192 x 128 ring and the 256 x 256 tile.
@pytest.mark.parametrize("m,n,k", [(8, 10304, 2688), (200, 10304, 2688), (512, 10304, 2688),
                                   (2600, 4100, 272)])
def test_linear_per_tensor_weight_scale(nhm, m, n, k):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=10, per_tensor=True)
    assert np.all(ws == ws[0])
    _check(nhm, a, w, ws, sa)


# The per-tensor form the checkpoint carries (w_scale_per_tensor = 1, one f32) against the same
# scale broadcast to a per-channel vector: bit-identical on every dispatch path -- the GEMV at
# both row classes, the 64 x 128 panel, the 192 x 128 ring, the split-k ring with its
# reduction, the 256 x 256 tile -- with bf16 and f32 output and with exact sums.
@pytest.mark.parametrize("m,n,k", [(1, 10304, 2688), (8, 2688, 4096), (200, 10304, 2688), (512, 10304, 2688),
                                   (64, 4096, 4096), (33, 1002, 4096), (2600, 4100, 272)])
def test_linear_per_tensor_scale_form(nhm, m, n, k):
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=11, per_tensor=True)
    wd, ad, sad = dev(w), dev(a), dev(sa)
    vec = nhm.Fp8Weight(wd, dev(ws), sad)
    one = nhm.Fp8Weight(wd, dev(ws[:1].copy()), sad)
    assert one.per_tensor and not vec.per_tensor
    for kw in (dict(), dict(out_type=nhm.NHM_F32), dict(exact=True)):
        ov = nhm.fp8_linear(ad, vec, **kw)
        o1 = nhm.fp8_linear(ad, one, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(host(ov), host(o1)), kw


# Narrow shapes whose panel launch would leave most of the chip idle: with the workspace the
# query reports, the 192 x 128 ring tile over S k ranges plus the reduction (33 x 1002: ragged
# m and n, n % 4 != 0 takes the reduction's element path); an e4m3 input with no workspace
# runs the unsplit 64 x 128 panel kernel. Both meet the bound, with bf16 and with f32 output.
@pytest.mark.parametrize("m,n,k", [(64, 4096, 4096), (48, 2688, 4096), (17, 4096, 4096), (33, 1002, 4096)])
@pytest.mark.parametrize("out_type", ["bf16", "f32"])
def test_linear_split_k_and_unsplit(nhm, m, n, k, out_type):
    import ctypes as C
    from oracle import bf16_to_f64, e4m3_decode, fp8_linear, quantize_static
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=11)
    q = quantize_static(a, sa)
    ref = fp8_linear(q, w, ws, sa)
    S = np.abs(e4m3_decode(q)) @ np.abs(e4m3_decode(w)).T * np.float64(sa[0]) * ws.astype(np.float64)[None, :]
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    need = nhm.fp8_linear_workspace_bytes(m, n, k, nhm.NHM_E4M3)
    assert need >= 2 * m * n * 4                         # room for the partials of at least two splits
    qd = dev(q)
    f32 = out_type == "f32"
    outs = []
    for wsb in (torch.zeros(need, dtype=torch.uint8, device="cuda"), None):
        out = torch.empty((m, n), dtype=torch.float32 if f32 else torch.int16, device="cuda")
        st = nhm.lib.nhm_fp8_linear_ex(C.c_void_p(qd.data_ptr()), nhm.NHM_E4M3, m, k, C.byref(W.struct),
                                       C.c_void_p(out.data_ptr()), nhm.NHM_F32 if f32 else nhm.NHM_BF16, n,
                                       None if wsb is None else C.c_void_p(wsb.data_ptr()),
                                       0 if wsb is None else wsb.numel(),
                                       C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, nhm.lib.nhm_last_error()
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64) if f32 else bf16_to_f64(host(out)))
    for got in outs:
        err = np.abs(got - ref)
        bound = (2.0 ** -22 if f32 else 2.0 ** -8) * np.abs(ref) + 2.0 ** -16 * S
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), f"at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"


# ld_pad 13 makes the row stride odd: the kernels fall back from 8-byte stores
@pytest.mark.parametrize("m", [2, 100, 700])
@pytest.mark.parametrize("ld_pad", [12, 13])
def test_linear_strided_output(nhm, m, ld_pad):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, 520, 512, extra=4)
    _check(nhm, a, w, ws, sa, ld_pad=ld_pad)


# (1024, 2688, 4096): 128 x 128 tiles; (4096, 2688, 4096): 176 tiles of 256 x 256
@pytest.mark.parametrize("m", [1024, 4096])
def test_linear_large_m(nhm, m):
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, 2688, 4096, extra=5)
    _check(nhm, a, w, ws, sa)


# the 256 x 256 tile kernel's output staging with a padded row stride: 4112 keeps 16-byte
# stores, 4113 takes the element path
@pytest.mark.parametrize("ld_pad", [12, 13])
def test_linear_strided_output_wide_tiles(nhm, ld_pad):
    from workloads import linear_case
    a, w, ws, sa = linear_case(2600, 4100, 272, extra=6)
    _check(nhm, a, w, ws, sa, ld_pad=ld_pad)


# f32 output (the D = f32 plan): the unrounded result, through every dispatch path -- GEMV
# (m <= 16), the 192 x 128 ring tile (384 x 10300, 500 x 10000), the panel kernel (200 x 10304,
# 130 x 70), the
# 128 x 128 tile (641 x 130, 1030 x 2688) and the 256 x 256 tile (2600 x 4100 x 272, ragged).
# Bound: the f32 accumulation term of the bf16 test without the bf16 rounding,
# |gpu - ref| <= 2^-22 |ref| + 2^-16 * S.
@pytest.mark.parametrize("m,n,k,via_e4m3,ld_pad", [(1, 10304, 2688, False, 0), (8, 2688, 4096, True, 0),
                                                   (13, 100, 48, False, 5), (200, 10304, 2688, False, 0),
                                                   (384, 10300, 2608, False, 0),
                                                   (130, 70, 144, False, 0), (500, 10000, 2672, False, 0),
                                                   (512, 2688, 4096, False, 0), (641, 130, 256, True, 0),
                                                   (1030, 2688, 4096, False, 4), (2600, 4100, 272, False, 0),
                                                   (2600, 4100, 272, False, 3)])
def test_linear_f32_output(nhm, m, n, k, via_e4m3, ld_pad):
    import ctypes as C
    from oracle import e4m3_decode, fp8_linear, quantize_static
    from tests.gpu_util import dev
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=8)
    q = quantize_static(a, sa)
    ref = fp8_linear(q, w, ws, sa)
    S = np.abs(e4m3_decode(q)) @ np.abs(e4m3_decode(w)).T * np.float64(sa[0]) * ws.astype(np.float64)[None, :]
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    a_in, a_type = (dev(q), nhm.NHM_E4M3) if via_e4m3 else (dev(a), nhm.NHM_BF16)
    out = torch.full((m, n + ld_pad), 12345.0, dtype=torch.float32, device="cuda")
    need = nhm.fp8_linear_workspace_bytes(m, n, k, a_type)
    wsb = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    st = nhm.lib.nhm_fp8_linear_ex(C.c_void_p(a_in.data_ptr()), a_type, m, k, C.byref(W.struct),
                                   C.c_void_p(out.data_ptr()), nhm.NHM_F32, n + ld_pad, C.c_void_p(wsb.data_ptr()),
                                   wsb.numel(), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, nhm.lib.nhm_last_error()
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, n:] == 12345.0)                       # the row padding is untouched
    got = o[:, :n].astype(np.float64)
    err = np.abs(got - ref)
    bound = 2.0 ** -22 * np.abs(ref) + 2.0 ** -16 * S
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"


def test_linear_f32_output_binding(nhm):
    """The binding's float32 output and the bf16 output agree up to the bf16 rounding."""
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(8, 10304, 2688, extra=9)
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    ad = dev(a)
    of = nhm.fp8_linear(ad, W, out_type=nhm.NHM_F32)
    ob = host(nhm.fp8_linear(ad, W))
    torch.cuda.synchronize()
    assert of.dtype == torch.float32
    rounded = of.to(torch.bfloat16).view(torch.int16).cpu().numpy()
    assert np.array_equal(rounded, ob.view(np.int16))


@pytest.mark.parametrize("m", [8, 200, 512, 700, 4096])
def test_linear_deterministic(nhm, m):
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, 10304, 2688)
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    ad = dev(a)
    o1 = host(nhm.fp8_linear(ad, W))
    o2 = host(nhm.fp8_linear(ad, W))
    assert np.array_equal(o1, o2)


def test_linear_zero_rows(nhm):
    from tests.gpu_util import dev
    from workloads import linear_case
    _, w, ws, sa = linear_case(1, 64, 128)
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    a = torch.empty((0, 128), dtype=torch.int16, device="cuda")
    out = nhm.fp8_linear(a, W)
    assert out.shape == (0, 64)


# nhm_fp8_linear_exact: every product summed in f32 on every dispatch path -- the GEMV (8 x
# 10304), the 64 x 128 panel (17 x 130, 200 x 10304), the 192 x 128 ring (384 x 10300 x 2608,
# 512 x 10304), the 256 x 128 ring (600 x 10304), the split-k ring with its reduction (64 x
# 4096 x 4096, 33 x 1002), the 128 x 128 tile (700 x 520 x 272) and the 256 x 256 tile (1030 x
# 10304, 2600 x 4100 x 272). Bound: one f32 rounding of the result and of each partial sum
# combined, |gpu - ref| <= 2^-22 |ref| + 2^-22 S (the e4m3 MFMA path needs 2^-16 S); the
# bf16 output is the f32 result rounded once (half a bf16 step, at most 2^-8 |ref|),
# |gpu - ref| <= 2^-8 |ref| + 2^-22 S.
@pytest.mark.parametrize("m,n,k", [(8, 10304, 2688), (17, 130, 256), (200, 10304, 2688), (384, 10300, 2608),
                                   (512, 10304, 2688), (600, 10304, 2688), (64, 4096, 4096), (33, 1002, 4096),
                                   (700, 520, 272), (1030, 10304, 2688), (2600, 4100, 272)])
def test_linear_exact(nhm, m, n, k):
    from oracle import bf16_to_f64, e4m3_decode, fp8_linear, quantize_static
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=12)
    q = quantize_static(a, sa)
    ref = fp8_linear(q, w, ws, sa)
    S = np.abs(e4m3_decode(q)) @ np.abs(e4m3_decode(w)).T * np.float64(sa[0]) * ws.astype(np.float64)[None, :]
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    ad = dev(a)
    of = nhm.fp8_linear(ad, W, out_type=nhm.NHM_F32, exact=True)
    ob = nhm.fp8_linear(ad, W, exact=True)
    torch.cuda.synchronize()
    for got, rel in ((of.cpu().numpy().astype(np.float64), 2.0 ** -22), (bf16_to_f64(host(ob)), 2.0 ** -8)):
        err = np.abs(got - ref)
        bound = rel * np.abs(ref) + 2.0 ** -22 * S
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), f"at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"
    # the bf16 output is the f32 output rounded once
    assert np.array_equal(of.to(torch.bfloat16).view(torch.int16).cpu().numpy(), host(ob).view(np.int16))
    print(f"exact {m}x{n}x{k}: max |d| / (2^-24 S) = {np.max(np.abs(of.cpu().numpy() - ref) / (2.0 ** -24 * S)):.3f}")


# The GEMV on the decode shapes (in_proj 10304 x 2688, out_proj 2688 x 4096) at every row count
# class it serves, against the oracle as test_linear_exact bounds it: the activation codes given
# at a row stride past k whose extra bytes hold large codes (e4m3 input through the raw ABI), and
# as bf16 (quantized by the library); both calls agree bit for bit, and the dispatch counters
# show the GEMV ran.
@pytest.mark.parametrize("m", [1, 5, 8, 9, 12, 16])
@pytest.mark.parametrize("n,k", [(10304, 2688), (2688, 4096)])
def test_gemv_decode_shapes(nhm, m, n, k):
    import ctypes as C
    from oracle import bf16_to_f64, e4m3_decode, fp8_linear, quantize_static
    from tests.gpu_util import dev, host
    from workloads import linear_case
    a, w, ws, sa = linear_case(m, n, k, extra=14)
    q = quantize_static(a, sa)
    ref = fp8_linear(q, w, ws, sa)
    S = np.abs(e4m3_decode(q)) @ np.abs(e4m3_decode(w)).T * np.float64(sa[0]) * ws.astype(np.float64)[None, :]
    W = nhm.Fp8Weight(dev(w), dev(ws), dev(sa))
    lda = k + 48
    qs = np.full((m, lda), 0x7E, dtype=np.uint8)            # past-k bytes hold large codes
    qs[:, :k] = q
    qd = dev(qs)
    out = torch.zeros((m, n), dtype=torch.int16, device="cuda")
    nhm.dispatch_counters(reset=True)
    st = nhm.lib.nhm_fp8_linear_exact(C.c_void_p(qd.data_ptr()), nhm.NHM_E4M3, m, lda, C.byref(W.struct),
                                      C.c_void_p(out.data_ptr()), nhm.NHM_BF16, n, None, 0,
                                      C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, nhm.lib.nhm_last_error()
    ob2 = nhm.fp8_linear(dev(a), W, exact=True)
    torch.cuda.synchronize()
    assert nhm.dispatch_counters(reset=True) == {"gemv": (2, 2 * m), "quant_vec8": (1, m)}
    for got in (bf16_to_f64(host(out)), bf16_to_f64(host(ob2))):
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * S
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), f"at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"
    assert np.array_equal(host(out), host(ob2))

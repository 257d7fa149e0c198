"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
refuses bad arguments on the host before anything is enqueued (no GPU needed:
every call here fails validation before a launch)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nhm.h")


@pytest.fixture(scope="module")
def nhm():
    import fp8_w8a8_linear_amd as m
    return m


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"NHM_API\s+[\w\s\*]+?\b(nhm_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(nhm):
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(nhm.lib, n), f"{n} not exported"


def test_dispatch_counters(nhm):
    """Every kernel has a named counter; refused calls launch nothing and count nothing."""
    n = nhm.lib.nhm_dispatch_counters(None, 0, 1)
    assert n >= 21
    arr = (nhm._DispatchCounter * n)()
    assert nhm.lib.nhm_dispatch_counters(arr, n, 0) == n
    names = [c.kernel.decode() for c in arr]
    assert len(set(names)) == n and "gemv" in names and "decode_ssm" in names and "ssd_out" in names
    assert all(c.launches == 0 and c.rows == 0 for c in arr)
    q = nhm.lib.nhm_fp8_quantize_static
    assert q(0x101, 2, 8, 8, 0x100, 0x200, 8, None) == 3
    assert nhm.dispatch_counters() == {}


def test_build_arch(nhm):
    assert nhm.lib.nhm_build_arch() == b"gfx950"
    assert nhm.lib.nhm_status_str(4) == b"NHM_ERR_UNSUPPORTED"


def test_layout_matches_oracle(nhm):
    from oracle import layout
    assert nhm.mixer_layout() == layout()


@pytest.mark.parametrize("field,value", [("head_dim", 32), ("d_state", 64), ("conv_width", 3), ("n_groups", 7),
                                         ("rms_eps", 0.0), ("hidden", 100), ("n_heads", 0)])
def test_unsupported_geometry(nhm, field, value):
    g = dict(nhm.GEOMETRY)
    g[field] = value
    with pytest.raises(nhm.NhmError) as e:
        nhm.mixer_layout(g)
    assert e.value.status == 4


def test_n_heads_not_multiple_of_8_refused(nhm):
    """in_proj rows (64 n_heads + conv_dim + n_heads bf16) are read 16 bytes at a time, so
    n_heads must be a multiple of 8 even where n_groups divides it."""
    for nh, ng in [(4, 2), (12, 4), (20, 4)]:
        g = dict(nhm.GEOMETRY, n_heads=nh, n_groups=ng, hidden=256)
        with pytest.raises(nhm.NhmError) as e:
            nhm.mixer_layout(g)
        assert e.value.status == 4 and b"multiple of 8" in nhm.lib.nhm_last_error()
    assert nhm.mixer_layout(dict(nhm.GEOMETRY, n_heads=8, n_groups=2, hidden=256))["d_in_proj"] % 8 == 0


def _w(nhm, w=0x1000, s=0x2000, a=0x3000, n=64, k=128, per_tensor=0):
    return nhm._Fp8Weight(w, s, a, n, k, per_tensor)


def _lin(nhm, a, a_type, m, lda, w, out, ld_out, ws, wsb):
    return nhm.lib.nhm_fp8_linear(a, a_type, m, lda, C.byref(w), out, ld_out, ws, wsb, None)


def test_linear_refusals(nhm):
    A, O, WS = 0x10000, 0x20000, 0x40000
    need = nhm.fp8_linear_workspace_bytes(32, 64, 128, nhm.NHM_BF16)
    assert need >= 32 * 128                                  # bf16 into the GEMM: an e4m3 copy
    cases = [
        (dict(a=None), 1), (dict(out=None), 1), (dict(w=_w(nhm, w=0)), 1),
        (dict(w=_w(nhm, k=100)), 2), (dict(w=_w(nhm, n=0)), 2), (dict(m=-1), 2), (dict(lda=64), 2),
        (dict(ld_out=10), 2), (dict(a=A + 2), 3), (dict(w=_w(nhm, w=0x1008)), 3), (dict(out=O + 1), 3),
        (dict(wsb=need - 1), 5), (dict(ws=None), 5), (dict(a_type=7), 4), (dict(ws=WS + 8), 3),
        (dict(w=_w(nhm, per_tensor=2)), 4), (dict(w=_w(nhm, per_tensor=-1)), 4),
    ]
    for over, status in cases:
        kw = dict(a=A, a_type=nhm.NHM_BF16, m=32, lda=128, w=_w(nhm), out=O, ld_out=64, ws=WS, wsb=need)
        kw.update(over)
        st = _lin(nhm, kw["a"], kw["a_type"], kw["m"], kw["lda"], kw["w"], kw["out"], kw["ld_out"], kw["ws"], kw["wsb"])
        assert st == status, (over, st, nhm.lib.nhm_last_error())
        assert nhm.lib.nhm_last_error() != b""


def test_linear_ex_refusals(nhm):
    """The output-type variant: its own checks (type, f32 alignment), then nhm_fp8_linear's."""
    A, O, WS = 0x10000, 0x20000, 0x40000
    need = nhm.fp8_linear_workspace_bytes(32, 64, 128, nhm.NHM_BF16)
    ex = nhm.lib.nhm_fp8_linear_ex
    w = _w(nhm)
    ok = dict(a=A, a_type=nhm.NHM_BF16, m=32, lda=128, out=O, out_type=nhm.NHM_F32, ld_out=64, ws=WS, wsb=need)
    cases = [(dict(out_type=nhm.NHM_E4M3), 4), (dict(out_type=9), 4), (dict(out=O + 2), 3), (dict(out=None), 1),
             (dict(ld_out=10), 2), (dict(a_type=7), 4), (dict(wsb=need - 1), 5)]
    for over, status in cases:
        kw = dict(ok)
        kw.update(over)
        st = ex(kw["a"], kw["a_type"], kw["m"], kw["lda"], C.byref(w), kw["out"], kw["out_type"], kw["ld_out"], kw["ws"],
                kw["wsb"], None)
        assert st == status, (over, st, nhm.lib.nhm_last_error())
    # a bf16 output only needs 2-byte alignment, as in nhm_fp8_linear
    assert ex(A, nhm.NHM_BF16, 0, 128, C.byref(w), O + 2, nhm.NHM_BF16, 64, WS, need, None) == 0


def test_linear_two_gib_operands_refused(nhm):
    """Operands of 2 GiB or more (32-bit buffer offsets) are refused on the host, before the
    quant of a bf16 input is enqueued, on the GEMV (m <= 16) and the tiled (m > 16) paths."""
    A, O, WS = 0x10000, 0x20000, 0x40000
    # (m, n, k, ld_a, input types): every case is refused (a bf16 input with a wide row
    # stride is quantized into [m, k] codes first, so only its e4m3 form is refused there)
    cases = [(8, 1 << 19, 4096, 4096, (nhm.NHM_BF16, nhm.NHM_E4M3)),
             (32, 1 << 19, 4096, 4096, (nhm.NHM_BF16, nhm.NHM_E4M3)),
             (1 << 19, 64, 4096, 4096, (nhm.NHM_BF16, nhm.NHM_E4M3)),
             (32, 64, 128, 1 << 26, (nhm.NHM_E4M3,))]
    for m, n, k, ld, types in cases:
        for a_type in types:
            st = _lin(nhm, A, a_type, m, ld, _w(nhm, n=n, k=k), O, n, WS, 1 << 62)
            assert st == 4, (m, n, k, ld, a_type, st, nhm.lib.nhm_last_error())
            assert b"2 GiB" in nhm.lib.nhm_last_error()


def test_linear_zero_rows_is_noop(nhm):
    assert _lin(nhm, None, nhm.NHM_BF16, 0, 128, _w(nhm), None, 64, None, 0) == 0


def test_dequant_refusals(nhm):
    d = nhm.lib.nhm_fp8_dequant_channel_bf16
    W, S, O = 0x10000, 0x20000, 0x30000
    assert d(None, None, 0, 16, 16, None, 16, None) == 0                 # empty is a no-op
    assert d(W, S, 4, 0, 16, O, 16, None) == 0
    assert d(None, S, 4, 16, 16, O, 16, None) == 1
    assert d(W, S, 4, 16, 16, None, 16, None) == 1
    assert d(W, S, -1, 16, 16, O, 16, None) == 2
    assert d(W, S, 4, 24, 32, O, 32, None) == 2                           # k % 16 != 0
    assert d(W, S, 4, 16, 8, O, 16, None) == 2                            # ld_w < k
    assert d(W + 8, S, 4, 16, 16, O, 16, None) == 3
    assert d(W, S, 4, 16, 24, O, 16, None) == 3                           # ld_w % 16 != 0
    assert d(W, S, 4, 16, 16, O + 4, 16, None) == 3


def test_quant_refusals(nhm):
    q = nhm.lib.nhm_fp8_quantize_static
    assert q(None, 0, 8, 8, None, None, 8, None) == 0                 # empty is a no-op
    assert q(None, 2, 8, 8, 0x100, 0x200, 8, None) == 1
    assert q(0x100, 2, 8, 4, 0x100, 0x200, 8, None) == 2
    assert q(0x101, 2, 8, 8, 0x100, 0x200, 8, None) == 3
    assert q(0x100, -1, 8, 8, 0x100, 0x200, 8, None) == 2


def _params(nhm, **over):
    g = nhm.Geometry(**nhm.GEOMETRY)
    lay = nhm.mixer_layout()
    d = dict(in_proj=_w(nhm, n=lay["d_in_proj"], k=2688), out_proj=_w(nhm, n=2688, k=4096), conv_w=0x5000,
             conv_b=0x6000, norm_w=0x7000, A_log=0x8000, D=0x9000, dt_bias=0xA000)
    d.update(over)
    return nhm._MixerParams(g, d["in_proj"], d["out_proj"], d["conv_w"], d["conv_b"], d["norm_w"], d["A_log"],
                            d["D"], d["dt_bias"])


def test_decode_refusals(nhm):
    dec = nhm.lib.nhm_mixer_decode
    need = nhm.decode_ws_layout(8)["total"]
    H, SL, SP, CP, O, WS = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000

    def call(p=None, hidden=H, batch=8, slots=SL, sp=SP, cp=CP, n_slots=64, out=O, ws=WS, wsb=need):
        p = p or _params(nhm)
        return dec(C.byref(p), hidden, batch, slots, sp, cp, n_slots, out, ws, wsb, None)

    assert call(batch=0) == 0
    assert call(hidden=None) == 1
    assert call(ws=None) == 1
    assert call(p=_params(nhm, conv_w=0)) == 1
    assert call(p=_params(nhm, in_proj=_w(nhm, n=10304, k=4096))) == 2      # wrong orientation
    assert call(p=_params(nhm, out_proj=_w(nhm, n=4096, k=2688))) == 2
    assert call(batch=-1) == 2
    assert call(n_slots=0) == 2
    assert call(hidden=H + 8) == 3
    assert call(p=_params(nhm, conv_w=0x5008)) == 3
    assert call(wsb=need - 1) == 5
    g = nhm.Geometry(**dict(nhm.GEOMETRY, rms_eps=0.0))
    p = _params(nhm)
    p.g = g
    assert call(p=p) == 4


def test_decode_q_refusals(nhm):
    """The pre-quantized decode: it needs the input (bf16 or codes), and out_q needs its scale."""
    f = nhm.lib.nhm_mixer_decode_q
    need = nhm.decode_ws_layout(8)["total"]
    H, Q, SL, SP, CP, O, OQ, S, WS = [0x100000 * i for i in range(1, 10)]
    p = _params(nhm)

    def call(hidden=H, hq=Q, out_q=OQ, scale=S, wsb=need):
        return f(C.byref(p), hidden, hq, 8, SL, SP, nhm.NHM_F32, CP, 64, O, out_q, scale, WS, wsb, None)

    assert call(hidden=None, hq=None) == 1
    assert call(scale=None) == 1
    assert call(hq=Q + 8) == 3
    assert call(out_q=OQ + 4) == 3
    assert call(scale=S + 2) == 3
    assert call(wsb=need - 1) == 5
    assert f(C.byref(p), H, Q, 0, SL, SP, nhm.NHM_F32, CP, 64, O, OQ, S, WS, need, None) == 0


def test_decode_noalloc_refusals(nhm):
    """The no-allocation decode validates like nhm_mixer_decode_ex and refuses a batch whose
    workspace exceeds its 16 MiB per-device scratch (300 rows at this geometry), before any
    device call."""
    f = nhm.lib.nhm_mixer_decode_noalloc
    H, SL, SP, CP, O = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    p = _params(nhm)
    assert f(C.byref(p), H, 0, SL, SP, nhm.NHM_F32, CP, 64, O, None) == 0
    assert nhm.decode_ws_layout(299)["total"] <= 16 << 20 < nhm.decode_ws_layout(300)["total"]
    assert f(C.byref(p), H, 300, SL, SP, nhm.NHM_F32, CP, 512, O, None) == 5
    assert b"scratch" in nhm.lib.nhm_last_error()
    assert f(C.byref(p), None, 8, SL, SP, nhm.NHM_F32, CP, 64, O, None) == 1
    assert f(C.byref(p), H, 8, SL, SP, nhm.NHM_F32, CP, 64, None, None) == 1
    assert f(C.byref(p), H + 8, 8, SL, SP, nhm.NHM_F32, CP, 64, O, None) == 3
    assert f(C.byref(p), H, 8, SL, SP, 7, CP, 64, O, None) == 4
    assert f(C.byref(p), H, -1, SL, SP, nhm.NHM_F32, CP, 64, O, None) == 2


def test_prefill_refusals(nhm):
    pre = nhm.lib.nhm_mixer_prefill
    need = nhm.prefill_ws_layout(512, 1)["total"]
    H, CU, SL, HI, SP, CP, O, WS = [0x100000 * i for i in range(1, 9)]

    def call(T=512, cu=CU, n=1, chunk=128, n_slots=4, ws=WS, wsb=need, hidden=H, hi=HI):
        return pre(C.byref(_params(nhm)), hidden, T, cu, n, SL, hi, chunk, SP, CP, n_slots, O, ws, wsb, None)

    assert call(T=0, n=0) == 0
    assert call(T=5, n=0) == 2
    assert call(chunk=64) == 4
    assert call(n=5, n_slots=4) == 2
    assert call(cu=None) == 1
    assert call(hi=None) == 1
    assert call(hidden=H + 4) == 3
    assert call(wsb=need - 1) == 5
    assert call(ws=WS + 16) == 3
    with pytest.raises(nhm.NhmError):
        nhm.prefill_ws_layout(512, 1, chunk=256)


def test_workspace_sizes_grow(nhm):
    a = nhm.prefill_ws_layout(512, 1)
    b = nhm.prefill_ws_layout(15360, 4)
    assert b["total"] > a["total"] > 0
    assert a["q_in"] < a["zxbcdt"] < a["xbc_conv"] < a["y"] < a["norm"] < a["q_out"] < a["total"]
    d = nhm.decode_ws_layout(8)
    assert d["q_out"] + 8 * 4096 <= d["total"]


def test_linear_workspace_split_partials(nhm):
    """The workspace query: a narrow shape that splits k reports room for its f32 partials
    (at least two splits of m x n), after the bf16 input's codes; other shapes report none."""
    need = nhm.fp8_linear_workspace_bytes(64, 4096, 4096, nhm.NHM_E4M3)
    assert need >= 2 * 64 * 4096 * 4 and need % 256 == 0
    assert nhm.fp8_linear_workspace_bytes(64, 4096, 4096, nhm.NHM_BF16) == 64 * 4096 + need
    for m, n, k in [(512, 10304, 2688), (512, 2688, 4096), (8, 10304, 2688), (4096, 2688, 4096)]:
        assert nhm.fp8_linear_workspace_bytes(m, n, k, nhm.NHM_E4M3) == 0
        assert nhm.fp8_linear_workspace_bytes(m, n, k, nhm.NHM_BF16) == (m * k + 255) // 256 * 256

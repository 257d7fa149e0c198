"""Python binding of libnhm, the FP8 W8A8 NemotronH Mamba2 mixer for MI355X (gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
``libnhm.so`` behind the C ABI declared in ``include/nhm.h``. torch supplies
device memory and the current stream. Importing this module fails loudly when
the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = ["lib", "LIB_PATH", "NhmError", "Geometry", "Layout", "WsLayout", "Fp8Weight", "MixerParams",
           "GEOMETRY", "mixer_layout", "quantize_static", "fp8_linear", "fp8_linear_workspace_bytes",
           "decode_ws_layout", "prefill_ws_layout", "mixer_decode", "mixer_prefill", "NHM_BF16", "NHM_E4M3",
           "NHM_F32", "fp8_dequant_channel_bf16", "mixer_decode_noalloc", "mixer_decode_q",
           "dispatch_counters"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnhm.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python fp8_w8a8_linear_amd/build.py` "
                      "(or __graft_entry__.build()); this package has no non-HIP fallback")
lib = C.CDLL(LIB_PATH)

NHM_BF16, NHM_E4M3, NHM_F32 = 0, 1, 2
_STATUS = {0: "NHM_OK", 1: "NHM_ERR_NULL", 2: "NHM_ERR_SHAPE", 3: "NHM_ERR_ALIGN", 4: "NHM_ERR_UNSUPPORTED",
           5: "NHM_ERR_WORKSPACE", 6: "NHM_ERR_HIP"}


class NhmError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


class Geometry(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32), ("d_state", C.c_int32),
                ("n_groups", C.c_int32), ("conv_width", C.c_int32), ("rms_eps", C.c_float)]


class Layout(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "d_inner", "conv_dim", "d_in_proj", "z_off", "z_width", "xbc_off", "xbc_width", "dt_off", "dt_width",
        "x_off", "x_width", "b_off", "b_width", "c_off", "c_width", "heads_per_group", "norm_group")]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("total", "q_in", "zxbcdt", "xbc_conv", "y", "norm", "q_out")]


class _DispatchCounter(C.Structure):
    _fields_ = [("kernel", C.c_char_p), ("launches", C.c_uint64), ("rows", C.c_uint64)]


class _Fp8Weight(C.Structure):
    _fields_ = [("w", C.c_void_p), ("w_scale", C.c_void_p), ("a_scale", C.c_void_p), ("n", C.c_int64),
                ("k", C.c_int64), ("w_scale_per_tensor", C.c_int32)]


class _MixerParams(C.Structure):
    _fields_ = [("g", Geometry), ("in_proj", _Fp8Weight), ("out_proj", _Fp8Weight), ("conv_w", C.c_void_p),
                ("conv_b", C.c_void_p), ("norm_w", C.c_void_p), ("A_log", C.c_void_p), ("D", C.c_void_p),
                ("dt_bias", C.c_void_p)]


_p, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_SIGS = {
    "nhm_status_str": (C.c_char_p, [C.c_int]),
    "nhm_last_error": (C.c_char_p, []),
    "nhm_build_arch": (C.c_char_p, []),
    "nhm_mixer_layout": (C.c_int, [C.POINTER(Geometry), C.POINTER(Layout)]),
    "nhm_fp8_quantize_static": (C.c_int, [_p, _i64, _i64, _i64, _p, _p, _i64, _p]),
    "nhm_fp8_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, C.c_int]),
    "nhm_fp8_dequant_channel_bf16": (C.c_int, [_p, _p, _i64, _i64, _i64, _p, _i64, _p]),
    "nhm_fp8_linear": (C.c_int, [_p, C.c_int, _i64, _i64, C.POINTER(_Fp8Weight), _p, _i64, _p, _sz, _p]),
    "nhm_fp8_linear_ex": (C.c_int, [_p, C.c_int, _i64, _i64, C.POINTER(_Fp8Weight), _p, C.c_int, _i64, _p, _sz, _p]),
    "nhm_fp8_linear_exact": (C.c_int, [_p, C.c_int, _i64, _i64, C.POINTER(_Fp8Weight), _p, C.c_int, _i64, _p, _sz,
                                       _p]),
    "nhm_mixer_decode_ws_layout": (C.c_int, [C.POINTER(Geometry), _i32, C.POINTER(WsLayout)]),
    "nhm_mixer_prefill_ws_layout": (C.c_int, [C.POINTER(Geometry), _i64, _i32, _i32, C.POINTER(WsLayout)]),
    "nhm_mixer_decode": (C.c_int, [C.POINTER(_MixerParams), _p, _i32, _p, _p, _p, _i32, _p, _p, _sz, _p]),
    "nhm_mixer_prefill": (C.c_int, [C.POINTER(_MixerParams), _p, _i64, _p, _i32, _p, _p, _i32, _p, _p, _i32, _p,
                                    _p, _sz, _p]),
    "nhm_mixer_decode_ex": (C.c_int, [C.POINTER(_MixerParams), _p, _i32, _p, _p, C.c_int, _p, _i32, _p, _p, _sz,
                                      _p]),
    "nhm_dispatch_counters": (C.c_int32, [C.POINTER(_DispatchCounter), C.c_int32, C.c_int32]),
    "nhm_mixer_decode_q": (C.c_int, [C.POINTER(_MixerParams), _p, _p, _i32, _p, _p, C.c_int, _p, _i32, _p, _p, _p,
                                     _p, _sz, _p]),
    "nhm_mixer_decode_noalloc": (C.c_int, [C.POINTER(_MixerParams), _p, _i32, _p, _p, C.c_int, _p, _i32, _p, _p]),
    "nhm_mixer_prefill_ex": (C.c_int, [C.POINTER(_MixerParams), _p, _i64, _p, _i32, _p, _p, _i32, _p, C.c_int, _p,
                                       _i32, _p, _p, _sz, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args


def _check(status):
    if status != 0:
        raise NhmError(status, lib.nhm_last_error().decode())


GEOMETRY = dict(hidden=2688, n_heads=64, head_dim=64, d_state=128, n_groups=8, conv_width=4, rms_eps=1e-5)


def _geom(g):
    return Geometry(**g) if isinstance(g, dict) else g


def mixer_layout(g=GEOMETRY):
    out = Layout()
    _check(lib.nhm_mixer_layout(C.byref(_geom(g)), C.byref(out)))
    return {n: getattr(out, n) for n, _ in Layout._fields_}


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev_tensor(x, name):
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


class Fp8Weight:
    """One FP8 W8A8 projection on the device: e4m3 codes [n, k] (uint8), f32 weight scale [n] (per
    output channel) or [1] (per tensor), f32 a_scale [1]."""

    def __init__(self, w, w_scale, a_scale):
        self.w = _dev_tensor(w, "w")
        self.w_scale = _dev_tensor(w_scale, "w_scale")
        self.a_scale = _dev_tensor(a_scale, "a_scale")
        self.n, self.k = int(w.shape[0]), int(w.shape[1])
        ns = int(self.w_scale.numel())
        if ns not in (1, self.n):
            raise ValueError(f"w_scale has {ns} entries: {self.n} (per channel) or 1 (per tensor)")
        self.per_tensor = ns == 1 and self.n != 1
        self._s = _Fp8Weight(self.w.data_ptr(), self.w_scale.data_ptr(), self.a_scale.data_ptr(), self.n, self.k,
                             1 if self.per_tensor else 0)

    @property
    def struct(self):
        return self._s


class MixerParams:
    """All parameters of one mixer block as device tensors (bf16 as int16/uint16 bit patterns)."""

    def __init__(self, in_proj: Fp8Weight, out_proj: Fp8Weight, conv_w, conv_b, norm_w, A_log, D, dt_bias,
                 g=GEOMETRY):
        self.in_proj, self.out_proj = in_proj, out_proj
        self.tensors = dict(conv_w=_dev_tensor(conv_w, "conv_w"), conv_b=_dev_tensor(conv_b, "conv_b"),
                            norm_w=_dev_tensor(norm_w, "norm_w"), A_log=_dev_tensor(A_log, "A_log"),
                            D=_dev_tensor(D, "D"), dt_bias=_dev_tensor(dt_bias, "dt_bias"))
        self.geometry = dict(g)
        t = self.tensors
        self._s = _MixerParams(_geom(g), in_proj.struct, out_proj.struct, t["conv_w"].data_ptr(),
                               t["conv_b"].data_ptr(), t["norm_w"].data_ptr(), t["A_log"].data_ptr(),
                               t["D"].data_ptr(), t["dt_bias"].data_ptr())

    @property
    def struct(self):
        return self._s


def quantize_static(x, scale, q=None, stream=None):
    """e4m3 codes of a bf16 [rows, cols] tensor (given as int16/uint16/bfloat16) with a device f32 scale [1]."""
    import torch
    x = _dev_tensor(x, "x")
    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _check(lib.nhm_fp8_quantize_static(_ptr(x), rows, cols, cols, _ptr(scale), _ptr(q), cols, _stream(stream)))
    return q


def fp8_linear_workspace_bytes(m, n, k, a_type):
    return int(lib.nhm_fp8_linear_workspace_bytes(m, n, k, a_type))


def fp8_linear(a, weight: Fp8Weight, out=None, ws=None, a_type=None, stream=None, out_type=None, exact=False):
    """[m, n] = W8A8(a [m, k], weight). a: bf16 bits (int16/uint16/bfloat16) or e4m3 codes (uint8).

    The output is bf16 bits (int16) unless out_type is NHM_F32 (or out is a float32 tensor).
    exact=True calls nhm_fp8_linear_exact (every product summed in f32 on every path)."""
    import torch
    a = _dev_tensor(a, "a")
    if a_type is None:
        a_type = NHM_E4M3 if a.dtype == torch.uint8 else NHM_BF16
    if out_type is None:
        out_type = NHM_F32 if out is not None and out.dtype == torch.float32 else NHM_BF16
    m = int(a.shape[0])
    if out is None:
        out = torch.empty((m, weight.n), dtype=torch.float32 if out_type == NHM_F32 else torch.int16, device=a.device)
    need = fp8_linear_workspace_bytes(m, weight.n, weight.k, a_type)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=a.device)
    fn = lib.nhm_fp8_linear_exact if exact else lib.nhm_fp8_linear_ex
    _check(fn(_ptr(a), a_type, m, a.shape[1], C.byref(weight.struct), _ptr(out), out_type, out.shape[1], _ptr(ws),
              0 if ws is None else ws.numel(), _stream(stream)))
    return out


def fp8_dequant_channel_bf16(w, w_scale, out=None, stream=None):
    """bf16 [n, k] = bf16(val(w) * w_scale[row]) of an e4m3 weight [n, k] (uint8)."""
    import torch
    w = _dev_tensor(w, "w")
    n, k = int(w.shape[0]), int(w.shape[1])
    if out is None:
        out = torch.empty((n, k), dtype=torch.int16, device=w.device)
    _check(lib.nhm_fp8_dequant_channel_bf16(_ptr(w), _ptr(w_scale), n, k, w.stride(0), _ptr(out), out.stride(0),
                                            _stream(stream)))
    return out


def decode_ws_layout(batch, g=GEOMETRY):
    out = WsLayout()
    _check(lib.nhm_mixer_decode_ws_layout(C.byref(_geom(g)), batch, C.byref(out)))
    return {n: int(getattr(out, n)) for n, _ in WsLayout._fields_}


def prefill_ws_layout(n_tokens, n_seqs, chunk=128, g=GEOMETRY):
    out = WsLayout()
    _check(lib.nhm_mixer_prefill_ws_layout(C.byref(_geom(g)), n_tokens, n_seqs, chunk, C.byref(out)))
    return {n: int(getattr(out, n)) for n, _ in WsLayout._fields_}


def _ssm_type(pool):
    """NHM_F32 for a float32 state pool, NHM_BF16 for bf16 bits (int16/uint16) or bfloat16."""
    import torch
    if pool.dtype == torch.float32:
        return NHM_F32
    if pool.dtype in (torch.int16, torch.uint16, torch.bfloat16):
        return NHM_BF16
    raise TypeError(f"SSM state pool of dtype {pool.dtype}: float32 or bf16 bits")


def mixer_decode(params: MixerParams, hidden, slot_idx, ssm_pool, conv_pool, out, ws, stream=None):
    """One decode token per sequence; pools updated in place (f32 or bf16 state pool).
    ws: uint8 device tensor of the layout size."""
    batch = int(hidden.shape[0])
    _check(lib.nhm_mixer_decode_ex(C.byref(params.struct), _ptr(hidden), batch, _ptr(slot_idx), _ptr(ssm_pool),
                                   _ssm_type(ssm_pool), _ptr(conv_pool), int(ssm_pool.shape[0]), _ptr(out), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    return out


def dispatch_counters(reset=False):
    """{kernel: (launches, rows)} of every kernel launched since the last reset (host-side
    counters; a launch captured into a graph counts once). reset=True zeroes them after reading."""
    n = int(lib.nhm_dispatch_counters(None, 0, 0))
    arr = (_DispatchCounter * n)()
    lib.nhm_dispatch_counters(arr, n, 1 if reset else 0)
    return {c.kernel.decode(): (int(c.launches), int(c.rows)) for c in arr if c.launches}


def mixer_decode_q(params: MixerParams, hidden, slot_idx, ssm_pool, conv_pool, out, ws, hidden_q=None, out_q=None,
                   out_q_scale=None, stream=None):
    """mixer_decode with a pre-quantized input (hidden_q: e4m3 codes under in_proj's a_scale; hidden
    may then be None) and/or the output's codes (out_q under out_q_scale, a device f32 [1])."""
    src = hidden if hidden is not None else hidden_q
    batch = int(src.shape[0])
    _check(lib.nhm_mixer_decode_q(C.byref(params.struct), _ptr(hidden), _ptr(hidden_q), batch, _ptr(slot_idx),
                                  _ptr(ssm_pool), _ssm_type(ssm_pool), _ptr(conv_pool), int(ssm_pool.shape[0]),
                                  _ptr(out), _ptr(out_q), _ptr(out_q_scale), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def mixer_decode_noalloc(params: MixerParams, hidden, slot_idx, ssm_pool, conv_pool, out, stream=None):
    """mixer_decode with the library's per-device scratch instead of a workspace (nothing is
    allocated by the call; calls that overlap on one GPU race)."""
    batch = int(hidden.shape[0])
    _check(lib.nhm_mixer_decode_noalloc(C.byref(params.struct), _ptr(hidden), batch, _ptr(slot_idx), _ptr(ssm_pool),
                                        _ssm_type(ssm_pool), _ptr(conv_pool), int(ssm_pool.shape[0]), _ptr(out),
                                        _stream(stream)))
    return out


def mixer_prefill(params: MixerParams, hidden, cu_seqlens, slot_idx, has_initial, ssm_pool, conv_pool, out, ws,
                  chunk=128, stream=None):
    """Varlen prefill of packed sequences; pools updated in place (f32 or bf16 state pool).
    ws: uint8 device tensor of the layout size."""
    n_tokens = int(hidden.shape[0])
    n_seqs = int(slot_idx.shape[0])
    _check(lib.nhm_mixer_prefill_ex(C.byref(params.struct), _ptr(hidden), n_tokens, _ptr(cu_seqlens), n_seqs,
                                    _ptr(slot_idx), _ptr(has_initial), chunk, _ptr(ssm_pool), _ssm_type(ssm_pool),
                                    _ptr(conv_pool), int(ssm_pool.shape[0]), _ptr(out), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return out

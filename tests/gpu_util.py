"""Helpers for the GPU parity tests: upload seeded inputs, read workspace regions, compare."""
import numpy as np
import torch

import fp8_w8a8_linear_amd as nhm

DEV = "cuda"


def dev(a):
    """numpy -> device tensor; uint16 (bf16 bits) travels as int16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.view(dtype)


def upload_params(p, g=nhm.GEOMETRY):
    inw = nhm.Fp8Weight(dev(p["in_w"]), dev(p["in_w_scale"]), dev(p["in_a_scale"]))
    outw = nhm.Fp8Weight(dev(p["out_w"]), dev(p["out_w_scale"]), dev(p["out_a_scale"]))
    return nhm.MixerParams(inw, outw, dev(p["conv_w"]), dev(p["conv_b"]), dev(p["norm_w"]), dev(p["A_log"]),
                           dev(p["D"]), dev(p["dt_bias"]), g)


def ws_region(ws, off, count, dtype):
    """A view of `count` elements of dtype at byte offset `off` of a uint8 workspace."""
    nbytes = count * np.dtype(dtype).itemsize
    b = ws[off:off + nbytes].cpu().numpy()
    return b.view(dtype)


def zeros_ws(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


from oracle.parity import block_parity, rel_l2, rel_max  # noqa: E402,F401

"""Seeded synthetic inputs with the shapes and distributions of the mixer workloads.

Every stream is a numpy PCG64 generator keyed by (workload id, tensor kind,
layer), so any tensor can be regenerated alone. Storage casts go through torch's
CPU casts (float32 -> bfloat16 and float32 -> float8_e4m3fn, both round half to
even); the weight codes are cast after an explicit clamp to +-448, which the
draw already satisfies by construction of the per-channel scale.

Workload ids: 0 one decode token through one block; 1 the W8A8 linear sweep;
2 paged decode B=8 through 23 blocks; 3 prefill of 512 tokens through one block;
4 ragged prefill of 8192+4096+2048+1024 tokens through 23 blocks.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = ["GEOM", "rng", "bf16_bits", "e4m3_weight", "block_params", "hidden",
           "ssm_pool", "conv_pool", "slots", "linear_case", "LINEAR_SHAPES",
           "RAGGED_LENGTHS", "KIND"]

GEOM = dict(hidden=2688, n_heads=64, head_dim=64, d_state=128, n_groups=8,
            conv_width=4, rms_eps=1e-5)
INNER = GEOM["n_heads"] * GEOM["head_dim"]                            # 4096
CONV_DIM = INNER + 2 * GEOM["n_groups"] * GEOM["d_state"]             # 6144
D_IN_PROJ = INNER + CONV_DIM + GEOM["n_heads"]                        # 10304

KIND = dict(param=1, hidden=2, ssm=3, conv=4, slot=5, act=6, weight=7)

# (m, n, k) of the standalone W8A8 linear sweep: in_proj / out_proj at decode,
# small-batch and prefill widths, plus a square control.
LINEAR_SHAPES = [(1, 10304, 2688), (8, 10304, 2688), (512, 10304, 2688),
                 (1, 2688, 4096), (512, 2688, 4096), (64, 4096, 4096)]
RAGGED_LENGTHS = [8192, 4096, 2048, 1024]


def rng(workload, kind, layer=0, extra=0):
    """Independent PCG64 stream for (workload, tensor kind, layer, extra)."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(workload), KIND[kind], int(layer), int(extra)])))


def bf16_bits(a):
    """bfloat16 bit patterns (uint16) of float32 data via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_weight(g, n, k, std=0.02, per_tensor=False):
    """W ~ N(0, std) [n, k]; per-output-channel scale amax/448 (per_tensor: one scale, the
    whole tensor's amax/448, repeated for every channel); codes of W/scale."""
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    amax = np.abs(w).max(axis=1)
    if per_tensor:
        amax = np.full_like(amax, amax.max() if amax.size else 0.0)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(w / scale[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scale


def _dims(g):
    """(d_inner, conv_dim, d_in_proj) of a geometry."""
    inner = g["n_heads"] * g["head_dim"]
    conv_dim = inner + 2 * g["n_groups"] * g["d_state"]
    return inner, conv_dim, inner + conv_dim + g["n_heads"]


def block_params(workload, layer, g=GEOM):
    """All parameters of one mixer block, drawn in a fixed order from one stream."""
    r = rng(workload, "param", layer)
    inner, conv_dim, d_in_proj = _dims(g)
    in_w, in_ws = e4m3_weight(r, d_in_proj, g["hidden"])
    out_w, out_ws = e4m3_weight(r, g["hidden"], inner)
    conv_w = bf16_bits(r.standard_normal((conv_dim, g["conv_width"]), dtype=np.float32) * np.float32(0.5))
    conv_b = bf16_bits(r.standard_normal(conv_dim, dtype=np.float32) * np.float32(0.1))
    H = g["n_heads"]
    A_log = r.uniform(0.0, np.log(16.0), H).astype(np.float32)
    dtv = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H))
    dt_bias = np.log(np.expm1(dtv)).astype(np.float32)     # inverse softplus of dtv
    D = (1.0 + 0.1 * r.standard_normal(H)).astype(np.float32)
    norm_w = bf16_bits(1.0 + 0.1 * r.standard_normal(inner).astype(np.float32))
    a_scale = np.array([4.0 / 448.0], dtype=np.float32)
    return dict(in_w=in_w, in_w_scale=in_ws, in_a_scale=a_scale.copy(),
                out_w=out_w, out_w_scale=out_ws, out_a_scale=a_scale.copy(),
                conv_w=conv_w, conv_b=conv_b, A_log=A_log, dt_bias=dt_bias, D=D,
                norm_w=norm_w)


def hidden(workload, T, g=GEOM, extra=0):
    """Block input, bf16 ~ N(0, 1), [T, hidden]."""
    return bf16_bits(rng(workload, "hidden", 0, extra).standard_normal((T, g["hidden"]), dtype=np.float32))


def ssm_pool(workload, layer, S, zero=False, g=GEOM):
    """f32 SSM state pool [S, H, P, N] ~ N(0, 0.1), or zeros."""
    shp = (S, g["n_heads"], g["head_dim"], g["d_state"])
    if zero:
        return np.zeros(shp, dtype=np.float32)
    return rng(workload, "ssm", layer).standard_normal(shp, dtype=np.float32) * np.float32(0.1)


def conv_pool(workload, layer, S, zero=False, g=GEOM):
    """bf16 conv window pool [S, W-1, conv_dim] ~ N(0, 1), oldest row first, or zeros."""
    shp = (S, g["conv_width"] - 1, _dims(g)[1])
    if zero:
        return np.zeros(shp, dtype=np.uint16)
    return bf16_bits(rng(workload, "conv", layer).standard_normal(shp, dtype=np.float32))


def slots(workload, count, S):
    """count distinct int32 slot indices drawn without replacement from [0, S)."""
    return rng(workload, "slot").choice(S, size=count, replace=False).astype(np.int32)


def linear_case(m, n, k, extra=0, per_tensor=False):
    """One W8A8 linear case: bf16 activations ~ N(0,1) [m,k]; weights as for a block
    (per_tensor: one weight scale for the whole tensor)."""
    a = bf16_bits(rng(1, "act", m * 100003 + n, extra).standard_normal((m, k), dtype=np.float32))
    w, ws = e4m3_weight(rng(1, "weight", n * 100003 + k, extra), n, k, per_tensor=per_tensor)
    return a, w, ws, np.array([4.0 / 448.0], dtype=np.float32)

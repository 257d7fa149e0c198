"""A plain float32 evaluation of the mixer block: the float-noise floor of the block tolerance.

Test infrastructure. Every stage runs in IEEE float32 numpy arithmetic and stores bf16
between stages, as an f32 implementation of the method does, with the two projections
summed exactly (float64 sums of the exact e4m3 products, rounded once to float32: the best
an f32-accumulating GEMM can deliver) and the recurrence advancing a float32 state one token
at a time. Its distance from the float64 oracle on the same input is what any correct
float32 implementation must expect; tests/test_oracle_noise_floor.py measures it.
"""
import numpy as np

import oracle.nhm_oracle as O

F = np.float32


def _f32_linear(q, w, ws, sa):
    acc = (O.e4m3_decode(q) @ O.e4m3_decode(w).T).astype(F)          # exact sum, rounded once
    return (acc * F(np.asarray(sa, F).reshape(-1)[0])) * np.asarray(ws, F)[None, :]


def _bf16(v):
    return O.bf16_from_f64(np.asarray(v, F).astype(np.float64))


def _val(bits):
    return O.bf16_to_f64(bits).astype(F)


def mixer_sequence_f32(p, hidden_bf16, window_bf16, state_f32, g=O.GEOMETRY):
    lay = O.layout(g)
    H, P, N, G = g["n_heads"], g["head_dim"], g["d_state"], g["n_groups"]
    T = hidden_bf16.shape[0]
    q_in = O.quantize_static(hidden_bf16, p["in_a_scale"])
    zx = _bf16(_f32_linear(q_in, p["in_w"], p["in_w_scale"], p["in_a_scale"]))
    z = zx[:, lay["z_off"]:lay["z_off"] + lay["z_width"]]
    xbc = zx[:, lay["xbc_off"]:lay["xbc_off"] + lay["xbc_width"]]
    dt_raw = zx[:, lay["dt_off"]:lay["dt_off"] + lay["dt_width"]]
    # conv + SiLU, taps in order, float32
    u = np.concatenate([_val(window_bf16), _val(xbc)], axis=0)
    w, b = _val(p["conv_w"]), _val(p["conv_b"])
    pre = np.broadcast_to(b, (T, b.shape[0])).astype(F)
    for j in range(w.shape[1]):
        pre = pre + w[:, j][None, :] * u[j:j + T, :]
    conv = _bf16(pre / (F(1) + np.exp(-pre)))
    x = _val(conv[:, lay["x_off"]:lay["x_off"] + lay["x_width"]]).reshape(T, H, P)
    Bm = _val(conv[:, lay["b_off"]:lay["b_off"] + lay["b_width"]]).reshape(T, G, N)
    Cm = _val(conv[:, lay["c_off"]:lay["c_off"] + lay["c_width"]]).reshape(T, G, N)
    uu = _val(dt_raw) + np.asarray(p["dt_bias"], F)
    dt = np.where(uu > F(20), uu, np.log1p(np.exp(np.minimum(uu, F(20))))).astype(F)
    dA = np.exp(dt * -np.exp(np.asarray(p["A_log"], F))).astype(F)
    D = np.asarray(p["D"], F)
    h = np.asarray(state_f32, F).copy()
    hpg = H // G
    y = np.empty((T, H, P), F)
    for t in range(T):
        Bh = np.repeat(Bm[t], hpg, axis=0)
        Ch = np.repeat(Cm[t], hpg, axis=0)
        h = dA[t][:, None, None] * h + (dt[t][:, None] * x[t])[:, :, None] * Bh[:, None, :]
        y[t] = np.einsum("hpn,hn->hp", h, Ch) + D[:, None] * x[t]
    y_bf = _bf16(y.reshape(T, H * P))
    yv, zv, nw = _val(y_bf), _val(z), _val(p["norm_w"])
    v = yv * (zv / (F(1) + np.exp(-zv)))
    vg = v.reshape(T, G, -1)
    r = F(1) / np.sqrt(np.mean(vg * vg, axis=-1, keepdims=True, dtype=F) + F(g["rms_eps"]))
    o_bf = _bf16((vg * r).reshape(T, -1) * nw)
    q_out = O.quantize_static(o_bf, p["out_a_scale"])
    out = _f32_linear(q_out, p["out_w"], p["out_w_scale"], p["out_a_scale"])
    return dict(out=out.astype(np.float64), q_out=q_out, norm_bf16=o_bf, state=h)


def mixer_prefill_f32(p, hidden_bf16, cu_seqlens, has_initial, windows, states, g=O.GEOMETRY):
    """Varlen form: sequence i uses windows[i] / states[i] when has_initial[i], else zeros."""
    lay = O.layout(g)
    outs, qs = [], []
    for i in range(len(cu_seqlens) - 1):
        t0, t1 = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        if t1 == t0:
            continue
        if has_initial[i]:
            win, st = windows[i], states[i]
        else:
            win = np.zeros((g["conv_width"] - 1, lay["conv_dim"]), np.uint16)
            st = np.zeros((g["n_heads"], g["head_dim"], g["d_state"]), np.float32)
        r = mixer_sequence_f32(p, hidden_bf16[t0:t1], win, st, g)
        outs.append(r["out"])
        qs.append(r["q_out"])
    return np.concatenate(outs), np.concatenate(qs)

"""Block-level invariants of the oracle and the armed counterfactuals of its tolerance.

The block has no external golden output, so it is pinned through its parts
(the other test_oracle_* files) and through invariants that must hold between
calls: carrying the state across a split of the sequence changes nothing, and
decode is prefill of length one from the pool row. The tolerance used for the
HIP path (max |d| <= 2e-2 * RMS of the reference) is shown to REJECT plausible
mistakes, each planted here in a copy of the oracle's composition.
"""
import numpy as np
import pytest

from oracle import (GEOMETRY, bf16_from_f64, bf16_to_f64, causal_conv1d_silu, dt_and_decay, e4m3_decode,
                    fp8_linear, gated_group_rmsnorm, layout, mixer_decode, mixer_prefill,
                    mixer_sequence, quantize_static, ssm_scan_sequential)
from workloads import block_params, conv_pool, hidden, ssm_pool

TOL = 2e-2


def rel_max(got, ref):
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref * ref)))


@pytest.fixture(scope="module")
def case():
    p = block_params(0, 0)
    return p, hidden(0, 6), ssm_pool(0, 0, 3), conv_pool(0, 0, 3)


def test_decode_is_prefill_of_length_one(case):
    p, h, sp, cp = case
    sp1, cp1 = sp.copy(), cp.copy()
    out_d, _ = mixer_decode(p, h[:2], np.array([2, 0]), sp1, cp1)
    sp2, cp2 = sp.copy(), cp.copy()
    out_p, _ = mixer_prefill(p, h[:2], np.array([0, 1, 2]), np.array([2, 0]), np.array([1, 1]), sp2, cp2)
    # equal up to the float64 summation order of the batched projection
    assert rel_max(out_d, out_p) < 1e-9
    assert np.max(np.abs(sp1 - sp2)) <= 1e-6 * np.max(np.abs(sp2)) and np.array_equal(cp1, cp2)
    assert not np.array_equal(sp1[2], sp[2]) and np.array_equal(sp1[1], sp[1])


def test_padded_decode_row_is_zero_and_untouched(case):
    p, h, sp, cp = case
    sp1, cp1 = sp.copy(), cp.copy()
    out, _ = mixer_decode(p, h[:2], np.array([-1, 1]), sp1, cp1)
    assert np.all(out[0] == 0) and np.array_equal(sp1[0], sp[0]) and np.array_equal(sp1[2], sp[2])


def test_carry_split_equals_whole(case):
    p, h, sp, cp = case
    whole = mixer_sequence(p, h, cp[0], sp[0])
    a = mixer_sequence(p, h[:2], cp[0], sp[0])
    b = mixer_sequence(p, h[2:], a["window"], a["state"])
    assert np.array_equal(np.concatenate([a["out_bf16"], b["out_bf16"]]), whole["out_bf16"]) or \
        rel_max(np.concatenate([a["out"], b["out"]]), whole["out"]) < 1e-6
    d = whole["state_f64"]
    assert np.linalg.norm(b["state"] - d) / np.linalg.norm(d) < 1e-6
    assert np.array_equal(b["window"], whole["window"])


def test_fresh_sequence_ignores_pool(case):
    p, h, sp, cp = case
    sp1, cp1 = sp.copy(), cp.copy()
    out, _ = mixer_prefill(p, h[:3], np.array([0, 3]), np.array([1]), np.array([0]), sp1, cp1)
    r = mixer_sequence(p, h[:3], np.zeros_like(cp[1]), np.zeros_like(sp[1]))
    assert np.array_equal(out, r["out"]) and np.array_equal(sp1[1], r["state"])


def test_block_output_scale(case):
    p, h, sp, cp = case
    r = mixer_sequence(p, h[:1], cp[0], sp[0])
    rms = np.sqrt(np.mean(r["out"] ** 2))
    assert 0.3 < rms < 3.0 and r["out"].shape == (1, 2688)


# --------------------------------------------------------------------------
# armed counterfactuals: each planted mistake must be rejected by the tolerance
# --------------------------------------------------------------------------

def _variant(p, hid, win, st, kind):
    g = GEOMETRY
    lay = layout(g)
    H, P, N, G = g["n_heads"], g["head_dim"], g["d_state"], g["n_groups"]
    T = hid.shape[0]
    if kind == "w8a16":        # activation never quantized: bf16 values straight into the GEMM
        A = bf16_to_f64(hid)
        W = e4m3_decode(p["in_w"]) * p["in_w_scale"].astype(np.float64)[:, None]
        zx = bf16_from_f64(A @ W.T)
    else:
        q = quantize_static(hid, p["in_a_scale"])
        ws = p["in_w_scale"]
        if kind == "per_tensor_wscale":
            ws = np.full_like(ws, ws.max())
        zx = bf16_from_f64(fp8_linear(q, p["in_w"], ws, p["in_a_scale"]))
    z = zx[:, :lay["xbc_off"]]
    xbc = zx[:, lay["xbc_off"]:lay["dt_off"]]
    dtr = zx[:, lay["dt_off"]:]
    if kind == "zero_carry":
        win = np.zeros_like(win)
        st = np.zeros_like(st)
    _, xc, _ = causal_conv1d_silu(xbc, win, p["conv_w"], p["conv_b"])
    xv = bf16_to_f64(xc[:, :lay["b_off"]]).reshape(T, H, P)
    Bv = bf16_to_f64(xc[:, lay["b_off"]:lay["c_off"]]).reshape(T, G, N)
    Cv = bf16_to_f64(xc[:, lay["c_off"]:]).reshape(T, G, N)
    if kind == "swap_bc":
        Bv, Cv = Cv, Bv
    dt, dA = dt_and_decay(dtr, p["dt_bias"], p["A_log"])
    y, _ = ssm_scan_sequential(xv, Bv, Cv, dt, dA, p["D"], st.astype(np.float64))
    yb = bf16_from_f64(y.reshape(T, H * P))
    if kind == "norm_then_gate":
        yv = bf16_to_f64(yb).reshape(T, G, -1)
        o = yv / np.sqrt(np.mean(yv * yv, axis=-1, keepdims=True) + g["rms_eps"])
        zz = bf16_to_f64(z)
        o = o.reshape(T, -1) * (zz / (1 + np.exp(-zz))) * bf16_to_f64(p["norm_w"])
        ob = bf16_from_f64(o)
    else:
        _, ob = gated_group_rmsnorm(yb, z, p["norm_w"], G, g["rms_eps"])
    qo = quantize_static(ob, p["out_a_scale"])
    return fp8_linear(qo, p["out_w"], p["out_w_scale"], p["out_a_scale"])


@pytest.mark.parametrize("kind", ["w8a16", "per_tensor_wscale", "zero_carry", "swap_bc", "norm_then_gate"])
def test_tolerance_rejects_planted_mistake(case, kind):
    p, h, sp, cp = case
    ref = mixer_sequence(p, h[:1], cp[0], sp[0])
    ok = _variant(p, h[:1], cp[0], sp[0], "none")
    assert rel_max(ok, ref["out"]) == 0.0          # the recomposition itself is faithful
    bad = _variant(p, h[:1], cp[0], sp[0], kind)
    sep = rel_max(bad, ref["out"])
    print(f"{kind}: separation {sep:.4f} vs tolerance {TOL}")
    assert sep > TOL

"""Plain, slow, CPU oracle of the NemotronH Mamba2 mixer with FP8 W8A8 projections.

TEST INFRASTRUCTURE. This module is the yardstick the HIP path is checked
against. It is imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product library never links, calls or
imports it, and it shares no code, constant table or helper with that library.

Sources. The method is described on five pull-request pages of one C++ LLM
inference project; they are cited by number and title:

  [PR1288] "feat(#810 A2-Q1): NemotronH's 23 Mamba2 blocks reach the device on
           the FP8 W8A8 seam (#517)"
  [PR1289] the same change re-filed as #1289 (conversation and commit log)
  [PR988]  "spec(#810 A2-Q): split the quantized arms into A2-Q1 and A2-Q2,
           because their blockers differ (#517)"
  [PR950]  "feat(#810 A2-R): NemotronH's dense weights reach the device, and the
           attention block that reads them is model-local (#517)"
  [PR972]  "refactor(VT-FP8-SHARED-SEAM): the FP8 W8A8 linear path becomes a
           seam a second model can reach (#940)"

The block, in the order [PR1288] "What it does" gives it:

  in_proj (FP8 W8A8) -> split z | xBC | dt -> causal conv1d + SiLU
  -> split x | B | C -> Mamba2 chunk scan -> gated group RMSNorm(n_groups)
  -> out_proj (FP8 W8A8)

Precision. Every stage computes in float64. Values are stored as bf16 between
stages, the recurrent SSM state is stored as float32 at rest, and the three
per-head SSM parameters are float32: [PR1288] "What it does" says the device
block keeps the host arm's dtypes and that the gathered state is an f32 working
buffer, and [PR950] "Review repairs" F2 counts 3 f32-by-contract SSM tensors of
64 heads per layer. The e4m3 activation code is a decision taken on the float32
quotient x / s, as the static per-tensor quant op defines it ([PR988] "The Thor
finding, measured": the quant op is its own kernel with an f32 scale).

Where the pages are silent, the plainest reading is taken (listed in the design doc):
OCP E4M3FN with saturation at +-448 and round-half-even; the gate is applied
before the group RMS; groups are contiguous; tap 3 of the conv meets the
current token; softplus(u) = u above 20; no dt clamp.

Parity status of each function is recorded in its docstring; every function
here is pinned by tests/test_oracle_*.py against values that do not come from
this module (closed forms, library routines, brute force, page facts).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GEOMETRY", "layout", "fp8_weight_elements",
    "bf16_from_f64", "bf16_to_f64", "e4m3_encode", "e4m3_decode",
    "quantize_static", "fp8_linear", "causal_conv1d_silu", "dt_and_decay",
    "ssm_scan_sequential", "ssd_chunked", "gated_group_rmsnorm",
    "mixer_sequence", "mixer_decode", "mixer_prefill",
    "mixer_decode_bf16_state", "mixer_prefill_bf16_state", "dequant_channel_bf16",
]

# NemotronH Mamba2 mixer geometry: hidden 2688, in_proj 2688 -> 10304 and
# out_proj 4096 -> 2688 ([PR1288] opening section; [PR988] "The Thor finding,
# measured", the six probe shapes); 64 heads ([PR950] "Review repairs" F2).
# head_dim 64, d_state 128, n_groups 8 and conv width 4 are the values that make
# the pages' widths add up: 64*64 = 4096 and 4096 + 2*8*128 = 6144 = conv_dim,
# 4096 + 6144 + 64 = 10304.
GEOMETRY = dict(hidden=2688, n_heads=64, head_dim=64, d_state=128,
                n_groups=8, conv_width=4, rms_eps=1e-5)


# ----------------------------------------------------------------------------
# Split indices
# ----------------------------------------------------------------------------

def layout(g=GEOMETRY):
    """Column offsets of the two splits of one in_proj row.

    [PR1289] commit log and [PR1288] "What it does": an in_proj row is z, xBC
    and dt as adjacent column ranges (widths I, conv_dim and n_heads, in that
    order), and a conv output row is x, B and C in that order.
    I = n_heads*head_dim, conv_dim = I + 2*n_groups*d_state.
    """
    inner = g["n_heads"] * g["head_dim"]
    gs = g["n_groups"] * g["d_state"]
    conv_dim = inner + 2 * gs
    return dict(
        d_inner=inner, conv_dim=conv_dim, d_in_proj=inner + conv_dim + g["n_heads"],
        z_off=0, z_width=inner,
        xbc_off=inner, xbc_width=conv_dim,
        dt_off=inner + conv_dim, dt_width=g["n_heads"],
        x_off=0, x_width=inner,          # offsets inside xBC
        b_off=inner, b_width=gs,
        c_off=inner + gs, c_width=gs,
        heads_per_group=g["n_heads"] // g["n_groups"],
        norm_group=inner // g["n_groups"],
    )


def fp8_weight_elements(n_layers, g=GEOMETRY):
    """fp8 weight elements of n_layers mixer blocks: n_layers*(in_proj + out_proj).

    [PR1288] opening section: the host arm re-expands this many elements per
    token (23 layers).
    """
    lay = layout(g)
    return n_layers * (lay["d_in_proj"] * g["hidden"] + g["hidden"] * lay["d_inner"])


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_from_f64(v):
    """Round float64 values to bfloat16 (round half to even), return the bit patterns.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits. A value v with
    frexp exponent e (v = m*2^e, 0.5 <= |m| < 1) has bf16 spacing 2^(e-8), and
    spacing 2^-133 in the subnormal range (e <= -126). NaN -> 0x7FC0 with sign.
    Pinned against torch's float32 -> bfloat16 cast in tests/test_oracle_formats.py.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e, -125)
    spacing = np.ldexp(1.0, e - 8)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(v / spacing) * spacing
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, v), r)
    r = np.where(np.isinf(v), v, r)
    with np.errstate(over="ignore", invalid="ignore"):
        bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        sign = (np.signbit(v).astype(np.uint16) << 15)
        bits = np.where(nan, sign | np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_to_f64(bits):
    """Exact value of bfloat16 bit patterns (the upper half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3_encode(v):
    """OCP FP8 E4M3FN code of float32 values, round half to even, saturating.

    Format: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
    NaN = S.1111.111, largest finite 448 = 1.75*2^8, normals down to 2^-6,
    subnormals m*2^-9. Readings: |v| >= 448 or +-inf -> +-448 (saturation);
    NaN -> 0x7F with the sign kept; a result of zero keeps the sign bit.
    Pinned: round trip over all finite codes, monotonicity, and equality with
    torch's float8_e4m3fn cast after clamping to +-448 (tests/test_oracle_formats.py).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    finite = np.isfinite(a)
    sat = (~finite) | (a >= 448.0)
    sub = finite & (a < 2.0 ** -6)
    nrm = finite & ~sub & ~sat
    # subnormal range: count of 2^-9 steps, rounded half to even (8 steps = 2^-6,
    # which is also the code of the smallest normal, so the codes stay contiguous)
    code = np.where(sub, np.rint(np.where(sub, a, 0.0) * 512.0).astype(np.int64), code)
    # normal range: a = m * 2^E with 1 <= m < 2; 3 mantissa bits
    m, e = np.frexp(np.where(nrm, a, 1.0))          # a = m*2^e, 0.5 <= m < 1
    E = e - 1
    frac = np.rint((m * 2.0 - 1.0) * 8.0).astype(np.int64)   # 0..8
    E = np.where(frac == 8, E + 1, E)
    frac = np.where(frac == 8, 0, frac)
    code = np.where(nrm, ((E + 7) << 3) | frac, code)
    code = np.where(sat, 0x7E, code)
    code = np.where(np.isnan(v), 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes):
    """Exact float64 value of OCP E4M3FN codes (0x7F / 0xFF -> NaN)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _e4m3_value_table():
    c = np.arange(256, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    f = c & 0x7
    mag = np.where(E == 0, f * 2.0 ** -9, (1.0 + f / 8.0) * np.ldexp(1.0, E - 7))
    mag = np.where((E == 0xF) & (f == 0x7), np.nan, mag)
    return s * mag


_E4M3_TABLE = _e4m3_value_table()   # value of each of the 256 codes


# ----------------------------------------------------------------------------
# a1 / a9: static per-tensor activation quant
# ----------------------------------------------------------------------------

def quantize_static(x_bf16, scale):
    """e4m3 code of every bf16 element: E(f32(x) / s), an IEEE float32 division.

    [PR988] "The Thor finding, measured" (the static activation quant op with one
    f32 scale); [PR1288] "The comparison is not bit-comparable, and that is the
    point" (W8A8 applies input_scale to the activation). Pinned through
    e4m3_encode plus a float64 check that the f32 quotient is the correctly
    rounded one.
    """
    x = bf16_to_f64(x_bf16).astype(np.float32)
    s = np.float32(np.asarray(scale, dtype=np.float32).reshape(-1)[0])
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        q = x / s                                  # float32 / float32, IEEE
    return e4m3_encode(q)


# ----------------------------------------------------------------------------
# a2 / a10: W8A8 GEMM
# ----------------------------------------------------------------------------

def fp8_linear(a_codes, w_codes, w_scale, a_scale):
    """out[m, n] = sum_k (val(a[m,k]) * s_a) * (val(W[n,k]) * ws[n]), float64.

    a_codes: e4m3 [M, K]; w_codes: e4m3 [N, K] in the [out, in] torch-Linear
    orientation ([PR950] "Review repairs" F2: GEMM consumers refuse any other);
    w_scale: f32 [N] per output channel; a_scale: f32 [1] static per tensor.
    The operands are dequantized first, then one float64 matmul (a library
    primitive) forms every dot product. Returns the unrounded float64 result;
    the block stores bf16(out). Pinned: brute-force triple loop and one-hot
    rows in tests/test_oracle_linear.py.
    """
    A = e4m3_decode(a_codes) * np.float64(np.asarray(a_scale, np.float32).reshape(-1)[0])
    W = e4m3_decode(w_codes) * np.asarray(w_scale, np.float32).astype(np.float64)[:, None]
    return A @ W.T


# ----------------------------------------------------------------------------
# a4: causal depthwise conv1d + SiLU
# ----------------------------------------------------------------------------

def causal_conv1d_silu(xbc_bf16, window_bf16, conv_w_bf16, conv_b_bf16):
    """Causal depthwise conv of one sequence, then SiLU.

    xbc_bf16: [T, C] pre-conv rows; window_bf16: [W-1, C] the previous W-1 rows,
    oldest first (zeros for a fresh sequence); conv_w: [C, W]; conv_b: [C].
    pre[t, c] = b[c] + sum_j w[c, j] * u[t - (W-1) + j, c] where u is the window
    followed by the new rows, so tap W-1 meets the current token; out = bf16(silu(pre)).
    The carried window after the call is the last W-1 rows of u.
    [PR1288] "What it does" (CausalConv1dFwd(silu)); [PR1289] commit log (the
    carried conv window). Pinned against torch conv1d in tests/test_oracle_conv.py.
    """
    x = bf16_to_f64(xbc_bf16)
    win = bf16_to_f64(window_bf16)
    w = bf16_to_f64(conv_w_bf16)
    b = bf16_to_f64(conv_b_bf16)
    T = x.shape[0]
    W = w.shape[1]
    u = np.concatenate([win, x], axis=0)            # [W-1+T, C]
    pre = np.broadcast_to(b, x.shape).copy()
    for j in range(W):
        pre += w[:, j][None, :] * u[j:j + T, :]
    out = pre / (1.0 + np.exp(-pre))
    new_window = np.asarray(np.concatenate([window_bf16, xbc_bf16], axis=0)[-(W - 1):])
    return out, bf16_from_f64(out), new_window.astype(np.uint16)


# ----------------------------------------------------------------------------
# a6: dt and decay
# ----------------------------------------------------------------------------

def dt_and_decay(dt_raw_bf16, dt_bias, A_log):
    """dt = softplus(f32(dt_raw) + dt_bias[h]); A = -exp(A_log[h]); dA = exp(dt*A).

    softplus(u) = log(1 + exp(u)), taken as u itself above 20 (reading). The
    three per-head parameters are float32 by contract ([PR950] "Review repairs"
    F2, three f32 SSM tensors of 64 heads per layer).
    """
    u = bf16_to_f64(dt_raw_bf16) + np.asarray(dt_bias, np.float32).astype(np.float64)
    dt = np.where(u > 20.0, u, np.log1p(np.exp(np.minimum(u, 20.0))))
    A = -np.exp(np.asarray(A_log, np.float32).astype(np.float64))
    return dt, np.exp(dt * A)


# ----------------------------------------------------------------------------
# a7: the recurrence
# ----------------------------------------------------------------------------

def ssm_scan_sequential(x, Bm, Cm, dt, dA, D, h0):
    """The Mamba2 recurrence, one token at a time.

    x: [T, H, P]; Bm, Cm: [T, G, N]; dt, dA: [T, H]; D: [H]; h0: [H, P, N].
    Head h reads group g = h // (H/G). For each token t:
        h[h,p,n] <- dA[t,h] * h[h,p,n] + (dt[t,h] * x[t,h,p]) * B[t,g,n]
        y[t,h,p]  = sum_n h[h,p,n] * C[t,g,n] + D[h] * x[t,h,p]
    Returns (y [T, H, P], h_final [H, P, N]) in float64.
    [PR1288] "What it does" (Mamba2ChunkScan advancing the state rows in place).
    Pinned by closed forms and by ssd_chunked (tests/test_oracle_ssm.py).
    """
    T, H, P = x.shape
    G = Bm.shape[1]
    hpg = H // G
    h = np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((T, H, P), dtype=np.float64)
    D = np.asarray(D, np.float64)
    for t in range(T):
        Bh = np.repeat(Bm[t], hpg, axis=0)          # [H, N]
        Ch = np.repeat(Cm[t], hpg, axis=0)
        h = dA[t][:, None, None] * h + (dt[t][:, None] * x[t])[:, :, None] * Bh[:, None, :]
        y[t] = np.einsum("hpn,hn->hp", h, Ch) + D[:, None] * x[t]
    return y, h


def ssd_chunked(x, Bm, Cm, dt, dA, D, h0, chunk):
    """The same recurrence evaluated by the chunked state-space-duality split.

    Used only by the invariant test "chunked == sequential". Within a chunk the
    cumulative log-decay cs_t = sum_{s<=t} log dA_s gives, for s <= t,
        y_t = sum_s (C_t . B_s) exp(cs_t - cs_s) dt_s x_s  +  exp(cs_t) C_t . H_in
    and the state leaving the chunk is exp(cs_end) H_in + sum_s exp(cs_end - cs_s)
    dt_s x_s (x) B_s (Dao & Gu 2024, "Transformers are SSMs", chunked SSD).
    """
    T, H, P = x.shape
    G = Bm.shape[1]
    hpg = H // G
    Hs = np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((T, H, P), dtype=np.float64)
    D = np.asarray(D, np.float64)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        L = c1 - c0
        logd = np.log(dA[c0:c1])                     # [L, H]
        cs = np.cumsum(logd, axis=0)                 # [L, H]
        Bh = np.repeat(Bm[c0:c1], hpg, axis=1)       # [L, H, N]
        Ch = np.repeat(Cm[c0:c1], hpg, axis=1)
        xs = x[c0:c1]                                # [L, H, P]
        dts = dt[c0:c1]                              # [L, H]
        CB = np.einsum("thn,shn->hts", Ch, Bh)       # [H, L, L]
        decay = np.exp(cs.T[:, :, None] - cs.T[:, None, :])   # [H, t, s]
        mask = np.tril(np.ones((L, L), dtype=bool))
        Lmat = np.where(mask[None], CB * decay, 0.0) * dts.T[:, None, :]
        y_diag = np.einsum("hts,shp->thp", Lmat, xs)
        y_off = np.exp(cs)[:, :, None] * np.einsum("thn,hpn->thp", Ch, Hs)
        y[c0:c1] = y_diag + y_off + D[None, :, None] * xs
        w = np.exp(cs[-1][None, :] - cs) * dts       # [L, H]
        S = np.einsum("sh,shp,shn->hpn", w, xs, Bh)
        Hs = np.exp(cs[-1])[:, None, None] * Hs + S
    return y, Hs


# ----------------------------------------------------------------------------
# a8: gated group RMSNorm
# ----------------------------------------------------------------------------

def gated_group_rmsnorm(y_bf16, z_bf16, norm_w_bf16, n_groups, eps):
    """o = (v * rsqrt(mean_group(v^2) + eps)) * w with v = y * silu(z).

    Groups are n_groups contiguous runs of channels; the gate is applied before
    the mean square (reading); eps is explicit and never defaulted to 0 ([PR950]
    "Not dense_attn::AttnBlock (#941)": a missing rms eps key silently became 0).
    [PR1288] "What it does" (RmsNormGatedGroup(n_groups)). Returns (o float64,
    bf16 bits). Pinned by closed forms in tests/test_oracle_norm.py.
    """
    y = bf16_to_f64(y_bf16)
    z = bf16_to_f64(z_bf16)
    w = bf16_to_f64(norm_w_bf16)
    v = y * (z / (1.0 + np.exp(-z)))
    shp = v.shape
    vg = v.reshape(shp[:-1] + (n_groups, shp[-1] // n_groups))
    r = 1.0 / np.sqrt(np.mean(vg * vg, axis=-1, keepdims=True) + eps)
    o = (vg * r).reshape(shp) * w
    return o, bf16_from_f64(o)


# ----------------------------------------------------------------------------
# The block
# ----------------------------------------------------------------------------

def mixer_sequence(p, hidden_bf16, window_bf16, state_f32, g=GEOMETRY):
    """One mixer block over the tokens of ONE sequence, from a given carried state.

    p: block parameters (dict of numpy arrays; see the design doc for names).
    hidden_bf16: [T, hidden]; window_bf16: [W-1, conv_dim]; state_f32: [H, P, N]
    (pass zeros for a fresh sequence). Returns a dict with the float64 block
    output ("out"), its bf16 bits ("out_bf16"), the new carried window and
    float32 state, and every intermediate the HIP path also stores.
    """
    lay = layout(g)
    H, P, N, G = g["n_heads"], g["head_dim"], g["d_state"], g["n_groups"]
    T = hidden_bf16.shape[0]
    q_in = quantize_static(hidden_bf16, p["in_a_scale"])                      # a1
    zxbcdt_f = fp8_linear(q_in, p["in_w"], p["in_w_scale"], p["in_a_scale"])  # a2
    zxbcdt = bf16_from_f64(zxbcdt_f)
    z = zxbcdt[:, lay["z_off"]:lay["z_off"] + lay["z_width"]]                # a3
    xbc = zxbcdt[:, lay["xbc_off"]:lay["xbc_off"] + lay["xbc_width"]]
    dt_raw = zxbcdt[:, lay["dt_off"]:lay["dt_off"] + lay["dt_width"]]
    _, xbc_conv, new_window = causal_conv1d_silu(xbc, window_bf16, p["conv_w"], p["conv_b"])  # a4
    xv = bf16_to_f64(xbc_conv[:, lay["x_off"]:lay["x_off"] + lay["x_width"]]).reshape(T, H, P)  # a5
    Bv = bf16_to_f64(xbc_conv[:, lay["b_off"]:lay["b_off"] + lay["b_width"]]).reshape(T, G, N)
    Cv = bf16_to_f64(xbc_conv[:, lay["c_off"]:lay["c_off"] + lay["c_width"]]).reshape(T, G, N)
    dt, dA = dt_and_decay(dt_raw, p["dt_bias"], p["A_log"])                  # a6
    y, h = ssm_scan_sequential(xv, Bv, Cv, dt, dA, p["D"],
                               np.asarray(state_f32, np.float32).astype(np.float64))  # a7
    y_bf16 = bf16_from_f64(y.reshape(T, H * P))
    o64, o_bf16 = gated_group_rmsnorm(y_bf16, z, p["norm_w"], G, g["rms_eps"])  # a8
    q_out = quantize_static(o_bf16, p["out_a_scale"])                         # a9
    out = fp8_linear(q_out, p["out_w"], p["out_w_scale"], p["out_a_scale"])   # a10
    return dict(out=out, out_bf16=bf16_from_f64(out), window=new_window,
                state=h.astype(np.float32), state_f64=h, q_in=q_in, zxbcdt=zxbcdt,
                xbc_conv=xbc_conv, y_bf16=y_bf16, y=y.reshape(T, H * P),
                norm=o64, norm_bf16=o_bf16, q_out=q_out)


def mixer_decode(p, hidden_bf16, slot_idx, ssm_pool, conv_pool, g=GEOMETRY):
    """One decode token for each of B sequences, state rows addressed by slot.

    hidden_bf16: [B, hidden]; slot_idx: [B] int (a negative slot marks a padded
    row whose output is zero and whose state is untouched); ssm_pool:
    [S, H, P, N] float32 and conv_pool: [S, W-1, conv_dim] bf16 are updated IN
    PLACE (copies are the caller's business). Decode always continues from the
    pool rows ([PR1288] "What it does": the paged arm advances gathered rows in
    place with has_initial = true). The rows are independent; the two
    projections are done for all rows at once (same arithmetic as row by row).
    Returns (out float64 [B, hidden], dict of per-row intermediates).
    """
    lay = layout(g)
    H, P, N, G = g["n_heads"], g["head_dim"], g["d_state"], g["n_groups"]
    B = hidden_bf16.shape[0]
    live = [b for b in range(B) if int(slot_idx[b]) >= 0]
    out = np.zeros((B, g["hidden"]), dtype=np.float64)
    res = dict(q_in=quantize_static(hidden_bf16, p["in_a_scale"]))
    zx = bf16_from_f64(fp8_linear(res["q_in"], p["in_w"], p["in_w_scale"], p["in_a_scale"]))   # a1, a2
    res["zxbcdt"] = zx
    xbc_conv = np.zeros((B, lay["conv_dim"]), dtype=np.uint16)
    y_bf16 = np.zeros((B, lay["d_inner"]), dtype=np.uint16)
    y64 = np.zeros((B, lay["d_inner"]), dtype=np.float64)
    for b in live:
        s = int(slot_idx[b])
        z = zx[b:b + 1, lay["z_off"]:lay["z_off"] + lay["z_width"]]
        xbc = zx[b:b + 1, lay["xbc_off"]:lay["xbc_off"] + lay["xbc_width"]]
        dt_raw = zx[b:b + 1, lay["dt_off"]:lay["dt_off"] + lay["dt_width"]]
        _, xc, conv_pool[s] = causal_conv1d_silu(xbc, conv_pool[s], p["conv_w"], p["conv_b"])   # a4
        xbc_conv[b] = xc[0]
        xv = bf16_to_f64(xc[:, lay["x_off"]:lay["x_off"] + lay["x_width"]]).reshape(1, H, P)   # a5
        Bv = bf16_to_f64(xc[:, lay["b_off"]:lay["b_off"] + lay["b_width"]]).reshape(1, G, N)
        Cv = bf16_to_f64(xc[:, lay["c_off"]:lay["c_off"] + lay["c_width"]]).reshape(1, G, N)
        dt, dA = dt_and_decay(dt_raw, p["dt_bias"], p["A_log"])                                # a6
        y, h = ssm_scan_sequential(xv, Bv, Cv, dt, dA, p["D"], ssm_pool[s].astype(np.float64))  # a7
        ssm_pool[s] = h.astype(np.float32)
        y64[b] = y.reshape(-1)
        y_bf16[b] = bf16_from_f64(y.reshape(-1))
    o64, o_bf16 = gated_group_rmsnorm(y_bf16, zx[:, lay["z_off"]:lay["z_off"] + lay["z_width"]],
                                    p["norm_w"], G, g["rms_eps"])                                # a8
    q_out = quantize_static(o_bf16, p["out_a_scale"])                                           # a9
    o = fp8_linear(q_out, p["out_w"], p["out_w_scale"], p["out_a_scale"])                       # a10
    out[live] = o[live]
    res.update(xbc_conv=xbc_conv, y=y64, y_bf16=y_bf16, norm=o64, norm_bf16=o_bf16, q_out=q_out)
    return out, res


def mixer_prefill(p, hidden_bf16, cu_seqlens, slot_idx, has_initial, ssm_pool, conv_pool,
                  g=GEOMETRY):
    """Varlen prefill: sequence i owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1.

    has_initial[i] = 0 starts sequence i from zero SSM state and zero conv
    window; 1 continues from pool row slot_idx[i]. The final state and window
    are written to that row IN PLACE. Sequences are independent. Returns
    (out float64 [T, hidden], list of per-sequence result dicts).
    """
    lay = layout(g)
    T = hidden_bf16.shape[0]
    out = np.zeros((T, g["hidden"]), dtype=np.float64)
    res = []
    for i in range(len(cu_seqlens) - 1):
        t0, t1 = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        s = int(slot_idx[i])
        if has_initial[i]:
            win, st = conv_pool[s], ssm_pool[s]
        else:
            win = np.zeros((g["conv_width"] - 1, lay["conv_dim"]), dtype=np.uint16)
            st = np.zeros((g["n_heads"], g["head_dim"], g["d_state"]), dtype=np.float32)
        if t1 == t0:
            res.append(None)
            if not has_initial[i]:
                ssm_pool[s] = st
                conv_pool[s] = win
            continue
        r = mixer_sequence(p, hidden_bf16[t0:t1], win, st, g)
        ssm_pool[s] = r["state"]
        conv_pool[s] = r["window"]
        out[t0:t1] = r["out"]
        res.append(r)
    return out, res


# ----------------------------------------------------------------------------
# bf16 SSM state pool
# ----------------------------------------------------------------------------

def _widen_state(ssm_pool_bf16):
    """The f32 working copy of a bf16 state pool (exact: every bf16 value is a float32)."""
    return bf16_to_f64(ssm_pool_bf16).astype(np.float32)


def mixer_decode_bf16_state(p, hidden_bf16, slot_idx, ssm_pool_bf16, conv_pool, g=GEOMETRY):
    """mixer_decode with the SSM state stored as bfloat16 [S, H, P, N] (bit patterns).

    [PR1288] "What it does": the gather widens the stored rows into an f32 working buffer
    and the result is narrowed back to the cache dtype, so a bf16 cache is a different
    computation from an f32 one. Read that way: widen the rows (exact), run the f32
    computation of mixer_decode unchanged (outputs come from the f32 state), then round
    each touched row's f32 state to bf16 (round half to even). Updates ssm_pool_bf16 and
    conv_pool in place; returns what mixer_decode returns.
    """
    work = _widen_state(ssm_pool_bf16)
    out, res = mixer_decode(p, hidden_bf16, slot_idx, work, conv_pool, g)
    for s in sorted({int(s) for s in slot_idx if int(s) >= 0}):
        ssm_pool_bf16[s] = bf16_from_f64(work[s])
    return out, res


def mixer_prefill_bf16_state(p, hidden_bf16, cu_seqlens, slot_idx, has_initial, ssm_pool_bf16, conv_pool,
                             g=GEOMETRY):
    """mixer_prefill with a bfloat16 state pool, read as mixer_decode_bf16_state: the
    initial rows are widened to f32, the call runs as mixer_prefill, and every sequence's
    final f32 state is rounded to bf16 into its row."""
    work = _widen_state(ssm_pool_bf16)
    out, res = mixer_prefill(p, hidden_bf16, cu_seqlens, slot_idx, has_initial, work, conv_pool, g)
    for s in sorted({int(s) for s in slot_idx}):
        ssm_pool_bf16[s] = bf16_from_f64(work[s])
    return out, res


# ----------------------------------------------------------------------------
# W8A16 weight dequant (debug / counterfactual arm)
# ----------------------------------------------------------------------------

def dequant_channel_bf16(w_codes, w_scale):
    """Per-output-channel e4m3 -> bf16 dequant: bf16(val(W[r, c]) * ws[r]) as bit patterns.

    [PR950] "What runs where, and why the line falls there" names the one standalone
    device dequant, per-channel FP8 -> bf16; [PR1288] "The comparison is not
    bit-comparable, and that is the point": the host arm it serves is W8A16, the weight
    dequantized to bf16 and the activation left unquantized. Read as the path's stage
    rule (f32 inside a stage, bf16 at its boundary): the product is formed in float32
    (IEEE, round to nearest) and rounded once to bf16 (half to even). NaN codes give NaN.
    """
    v = e4m3_decode(w_codes).astype(np.float32)          # exact: every e4m3 value is a float32
    prod = v * np.asarray(w_scale, np.float32).reshape(-1, 1)
    return bf16_from_f64(prod.astype(np.float64))

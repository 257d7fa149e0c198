"""Block parity: nhm_mixer_decode / nhm_mixer_prefill against the oracle.

Bars (oracle/parity.block_parity): e4m3 bytes bit-exact (a1 on identical input; a9 on the
GPU's own bf16 norm output); the stated block tolerance max|d| <= 2e-2 * RMS end to end on
every call of fewer than 128 tokens, and from 128 tokens on every row whose a9 codes equal
the oracle's (the float32 floor of tests/test_oracle_noise_floor.py misses the whole-call
bar there), with every row also held to it against the oracle's out_proj of the GPU's own
codes; the gated norm output elementwise within its derived bound (no element exempt); a9
codes that differ from the oracle's reachable and rare; f32 state ||d||/||ref|| <= 1e-3;
conv windows (bf16 copies) likewise; untouched pool rows bit-identical. Element counts are
asserted against the geometry.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL_OUT, TOL_STATE = 2e-2, 1e-3
# bf16 state pool: two f32 states within eps of each other round to bf16 values one ulp
# (2^-8 relative) apart on about eps / ulp of the elements, an RMS of sqrt(eps * 2^-8) =
# 2e-3 at the stated f32 bar eps = 1e-3; twice that is the bar
TOL_STATE_BF16 = 4e-3
H, I = 2688, 4096


@pytest.fixture(scope="module")
def nhm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_w8a8_linear_amd as m
    return m


@pytest.fixture(scope="module")
def block0():
    from workloads import block_params
    return block_params(0, 0)


def _gpu_decode(nhm, pd, hidden, slots, sp, cp):
    from tests.gpu_util import dev, host, zeros_ws
    B = hidden.shape[0]
    lay = nhm.decode_ws_layout(B)
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((B, H), dtype=torch.int16, device="cuda")
    nhm.mixer_decode(pd, dev(hidden), dev(slots), spd, cpd, out, ws)
    torch.cuda.synchronize()
    return host(out), host(spd), host(cpd), ws, lay


def _gpu_prefill(nhm, pd, hidden, cu, slots, has_init, sp, cp):
    from tests.gpu_util import dev, host, zeros_ws
    T = hidden.shape[0]
    lay = nhm.prefill_ws_layout(T, len(slots))
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    nhm.mixer_prefill(pd, dev(hidden), dev(np.asarray(cu, np.int32)), dev(np.asarray(slots, np.int32)),
                      dev(np.asarray(has_init, np.int32)), spd, cpd, out, ws)
    torch.cuda.synchronize()
    return host(out), host(spd), host(cpd), ws, lay


def _parity(out, ws, lay, rows, ref_out, ref_norm, ref_q, p):
    """Block parity on the given token rows, reading the GPU's a9 codes and norm output from ws."""
    from tests.gpu_util import block_parity, ws_region
    T = out.shape[0]
    q = ws_region(ws, lay["q_out"], T * I, np.uint8).reshape(T, I)[rows]
    nrm = ws_region(ws, lay["norm"], T * I, np.uint16).reshape(T, I)[rows]
    o = out[rows]
    assert o.shape == (len(rows), H) and q.shape == (len(rows), I)
    return block_parity(o, q, nrm, ref_out[rows] if ref_out.shape[0] == T else ref_out, ref_norm, ref_q, p)


def _check_states(sp_gpu, sp_ref, sp_before, touched):
    from tests.gpu_util import rel_l2
    worst = 0.0
    for s in range(sp_ref.shape[0]):
        if s in touched and not np.any(sp_ref[s]):       # a fresh empty sequence leaves zeros
            assert not np.any(sp_gpu[s]), f"slot {s} should be zero"
        elif s in touched:
            r = rel_l2(sp_gpu[s], sp_ref[s])
            worst = max(worst, r)
            assert r <= TOL_STATE, f"slot {s}: state rel l2 {r:.3g}"
        else:
            assert np.array_equal(sp_gpu[s], sp_before[s]), f"untouched slot {s} changed"
    return worst


def _check_windows(cp_gpu, cp_ref, cp_before, touched):
    from oracle import bf16_to_f64
    from tests.gpu_util import rel_l2, rel_max
    for s in range(cp_ref.shape[0]):
        if s in touched:
            a, b = bf16_to_f64(cp_gpu[s]), bf16_to_f64(cp_ref[s])
            if not np.any(b):
                assert not np.any(a)
                continue
            # copies of bf16 in_proj outputs: they differ only where the f32 and the f64
            # projection round to different bf16 neighbours
            assert rel_l2(a, b) <= TOL_STATE and rel_max(a, b) <= TOL_OUT, f"slot {s} window"
        else:
            assert np.array_equal(cp_gpu[s], cp_before[s])


def test_decode_one_block_one_token(nhm, block0):
    """One decode token through one block (m = 1), state from the pool."""
    from oracle import mixer_decode
    from tests.gpu_util import upload_params, ws_region
    from workloads import conv_pool, hidden, ssm_pool
    S = 4
    h = hidden(0, 1)
    sp, cp = ssm_pool(0, 0, S), conv_pool(0, 0, S)
    slots = np.array([2], np.int32)
    pd = upload_params(block0)
    out, spg, cpg, ws, lay = _gpu_decode(nhm, pd, h, slots, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_decode(block0, h, slots, spr, cpr)
    assert np.array_equal(ws_region(ws, lay["q_in"], H, np.uint8), res["q_in"].reshape(-1))   # a1
    m = _parity(out, ws, lay, [0], ref, res["norm"], res["q_out"], block0)
    st = _check_states(spg, spr, sp, {2})
    _check_windows(cpg, cpr, cp, {2})
    assert np.array_equal(cpg[2][:2], cp[2][1:])          # the two older rows shift exactly
    print(f"decode m=1: {m}, state rel l2 {st:.3e}")


# 20: in_proj and out_proj one GEMV per 16 rows; 33 and 64: both projections as one GEMM call
# each (in_proj summing exactly, out_proj with split k; 33: ragged m), the norm's hand-off
# counters zeroed by a launch of their own; 64 is the whole 64-slot pool in one call
@pytest.mark.parametrize("B,slot_list,S", [(8, None, 24), (3, [5, -1, 0], 24), (20, None, 24),
                                           (33, None, 48), (64, None, 64)])
def test_decode_batch(nhm, block0, B, slot_list, S):
    from oracle import mixer_decode
    from tests.gpu_util import upload_params, ws_region
    from workloads import conv_pool, hidden, slots, ssm_pool
    h = hidden(2, B, extra=B)
    sl = np.array(slot_list, np.int32) if slot_list else slots(2, B, S)
    sp, cp = ssm_pool(2, 0, S), conv_pool(2, 0, S)
    pd = upload_params(block0)
    nhm.dispatch_counters(reset=True)
    out, spg, cpg, ws, lay = _gpu_decode(nhm, pd, h, sl, sp, cp)
    path = nhm.dispatch_counters(reset=True)
    if B > 32:
        assert "gemv" not in path and path["clear"] == (1, B * 8) and path["decode_ssm"] == (1, B), path
        assert any(k.endswith("_exact") and v == (1, B) for k, v in path.items()), path
    else:
        assert path["gemv"][0] == 2 * ((B + 15) // 16) and "clear" not in path, path
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_decode(block0, h, sl, spr, cpr)
    # a1: the in_proj input codes kept in the workspace (the quant launch), every row, padded
    # ones too
    q_in = ws_region(ws, lay["q_in"], B * H, np.uint8).reshape(B, H)
    assert np.array_equal(q_in, res["q_in"].reshape(B, H))
    live = [b for b in range(B) if sl[b] >= 0]
    m = _parity(out, ws, lay, live, ref, res["norm"][live], res["q_out"][live], block0)
    pad = [b for b in range(B) if sl[b] < 0]
    assert np.all(out[pad] == 0)
    touched = {int(s) for s in sl if s >= 0}
    _check_states(spg, spr, sp, touched)
    _check_windows(cpg, cpr, cp, touched)
    print(f"decode B={B}: {m}")


def test_decode_stacked_layers(nhm):
    """Paged decode B=8 through 3 stacked blocks (bench.py checks layers of the full 23)."""
    from oracle import mixer_decode
    from tests.gpu_util import dev, host, upload_params, zeros_ws
    from workloads import block_params, conv_pool, hidden, slots, ssm_pool
    S, B, L = 64, 8, 3
    sl = slots(2, B, S)
    x = hidden(2, B)
    xd = dev(x)
    lay = nhm.decode_ws_layout(B)
    ws = zeros_ws(lay["total"])
    for layer in range(L):
        p = block_params(2, layer)
        sp, cp = ssm_pool(2, layer, S), conv_pool(2, layer, S)
        spd, cpd = dev(sp), dev(cp)
        out = torch.empty((B, H), dtype=torch.int16, device="cuda")
        nhm.mixer_decode(upload_params(p), xd, dev(sl), spd, cpd, out, ws)
        torch.cuda.synchronize()
        spr, cpr = sp.copy(), cp.copy()
        ref, res = mixer_decode(p, x, sl, spr, cpr)      # oracle on the same bf16 layer input
        got = host(out)
        m = _parity(got, ws, lay, list(range(B)), ref, res["norm"], res["q_out"], p)
        _check_states(host(spd), spr, sp, set(int(s) for s in sl))
        _check_windows(host(cpd), cpr, cp, set(int(s) for s in sl))
        print(f"layer {layer}: {m}")
        x, xd = got, out                                # next layer input: this layer's bf16 output


# 8 rows: the out_proj GEMV writes the codes in its epilogue; 40 rows: the tiled out_proj and a
# quant launch
@pytest.mark.parametrize("B", [8, 40])
def test_decode_chained_codes(nhm, B):
    """Three stacked blocks passing e4m3 codes (nhm_mixer_decode_q: each block's out_q, under
    the next block's in_proj scale, is the next block's hidden_q) against the same blocks through
    nhm_mixer_decode with bf16 input and output: outputs, state and conv pools bit-identical, and
    every out_q equal to the oracle's quantizer applied to the GPU's bf16 output."""
    from oracle import quantize_static
    from tests.gpu_util import dev, host, upload_params, zeros_ws
    from workloads import block_params, conv_pool, hidden, slots, ssm_pool
    S, L = 64, 3
    sl = dev(slots(2, B, S))
    x = dev(hidden(2, B, extra=70 + B))
    ps = [block_params(2, layer) for layer in range(L)]
    pds = [upload_params(p) for p in ps]
    ws = zeros_ws(nhm.decode_ws_layout(B)["total"])
    pools = [(ssm_pool(2, layer, S), conv_pool(2, layer, S)) for layer in range(L)]
    runs = []
    for chained in (False, True):
        xin, qin, outs, qs, st = x, None, [], [], []
        for layer in range(L):
            sp, cp = dev(pools[layer][0]), dev(pools[layer][1])
            out = torch.empty((B, H), dtype=torch.int16, device="cuda")
            if chained:
                oq = torch.full((B, H), 0x5A, dtype=torch.uint8, device="cuda") if layer + 1 < L else None
                nxt = pds[layer + 1].in_proj.a_scale if layer + 1 < L else None
                nhm.mixer_decode_q(pds[layer], xin if layer == 0 else None, sl, sp, cp, out, ws,
                                   hidden_q=qin, out_q=oq, out_q_scale=nxt)
                qin = oq
                qs.append(oq)
            else:
                nhm.mixer_decode(pds[layer], xin, sl, sp, cp, out, ws)
            torch.cuda.synchronize()
            outs.append(host(out))
            st.append((host(sp), host(cp)))
            xin = out
        runs.append((outs, st, qs))
    (o_plain, s_plain, _), (o_chain, s_chain, q_chain) = runs
    for layer in range(L):
        assert np.array_equal(o_plain[layer], o_chain[layer]), f"layer {layer}: outputs differ"
        assert np.array_equal(s_plain[layer][0], s_chain[layer][0]), f"layer {layer}: state pools differ"
        assert np.array_equal(s_plain[layer][1], s_chain[layer][1]), f"layer {layer}: conv pools differ"
        if layer + 1 < L:
            want = quantize_static(o_chain[layer], ps[layer + 1]["in_a_scale"])
            assert np.array_equal(host(q_chain[layer]), want), f"layer {layer}: out_q codes"


def test_decode_deterministic(nhm, block0):
    from tests.gpu_util import upload_params
    from workloads import conv_pool, hidden, ssm_pool
    h = hidden(0, 8)
    sp, cp = ssm_pool(0, 1, 8), conv_pool(0, 1, 8)
    sl = np.arange(8, dtype=np.int32)[::-1].copy()
    pd = upload_params(block0)
    a = _gpu_decode(nhm, pd, h, sl, sp, cp)
    b = _gpu_decode(nhm, pd, h, sl, sp, cp)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def _prefill_refs(res, lens):
    norm = np.concatenate([r["norm"] for r, L in zip(res, lens) if L > 0])
    q = np.concatenate([r["q_out"] for r, L in zip(res, lens) if L > 0])
    qin = np.concatenate([r["q_in"] for r, L in zip(res, lens) if L > 0])
    return norm, q, qin


def test_prefill_512_one_block(nhm, block0):
    """Prefill of one 512-token sequence (4 chunks) from a carried state."""
    from oracle import mixer_prefill
    from tests.gpu_util import upload_params, ws_region
    from workloads import conv_pool, hidden, ssm_pool
    S, T = 2, 512
    h = hidden(3, T)
    sp, cp = ssm_pool(3, 0, S), conv_pool(3, 0, S)
    pd = upload_params(block0)
    cu, sl, hi = [0, T], [1], [1]
    out, spg, cpg, ws, lay = _gpu_prefill(nhm, pd, h, cu, sl, hi, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(block0, h, cu, sl, hi, spr, cpr)
    norm, q, qin = _prefill_refs(res, [T])
    assert np.array_equal(ws_region(ws, lay["q_in"], T * H, np.uint8), qin.reshape(-1))     # a1
    m = _parity(out, ws, lay, list(range(T)), ref, norm, q, block0)
    st = _check_states(spg, spr, sp, {1})
    _check_windows(cpg, cpr, cp, {1})
    print(f"prefill 512: {m}, state rel l2 {st:.3e}")


@pytest.mark.parametrize("lens,has_init", [([5, 130, 1, 0, 260, 128], [1, 0, 1, 0, 1, 0]),
                                           ([2, 3], [1, 1]), ([17], [0])])
def test_prefill_ragged(nhm, block0, lens, has_init):
    from oracle import mixer_prefill
    from tests.gpu_util import upload_params
    from workloads import conv_pool, hidden, ssm_pool
    S = 8
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    h = hidden(4, T, extra=len(lens))
    sp, cp = ssm_pool(4, 0, S), conv_pool(4, 0, S)
    sl = np.array([7, 0, 3, 5, 1, 6][:len(lens)], np.int32)
    pd = upload_params(block0)
    out, spg, cpg, ws, lay = _gpu_prefill(nhm, pd, h, cu, sl, has_init, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(block0, h, cu, sl, has_init, spr, cpr)
    norm, q, _ = _prefill_refs(res, lens)
    m = _parity(out, ws, lay, list(range(T)), ref, norm, q, block0)
    touched = set(int(s) for s in sl)
    _check_states(spg, spr, sp, touched)
    _check_windows(cpg, cpr, cp, touched)
    print(f"prefill {lens}: {m}")


def test_mixed_batch_decode_rows_and_prefill_chunks(nhm, block0):
    """One prefill call carrying a mixed batch: 8 decode rows (one token each, continuing
    their pool rows) interleaved with two chunked-prefill continuations (300 and 129 tokens
    from a carried state) and one fresh 40-token prompt. A decode row is a length-1 sequence
    with has_initial 1, so the call needs no mode switch. Checked against the oracle's
    prefill of the same batch (every output, state and window), and the decode rows also
    against nhm_mixer_decode of the same 8 rows (the GEMV path)."""
    from oracle import bf16_to_f64, mixer_prefill
    from tests.gpu_util import rel_l2, rel_max, upload_params
    from workloads import conv_pool, hidden, ssm_pool
    S = 16
    lens = [1, 1, 300, 1, 1, 40, 1, 129, 1, 1, 1]
    has_init = [1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1]
    sl = np.array([9, 2, 14, 0, 5, 11, 7, 3, 12, 1, 15], np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    h = hidden(4, T, extra=31)
    sp, cp = ssm_pool(4, 2, S), conv_pool(4, 2, S)
    pd = upload_params(block0)
    out, spg, cpg, ws, lay = _gpu_prefill(nhm, pd, h, cu, sl, has_init, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(block0, h, cu, sl, has_init, spr, cpr)
    norm, q, _ = _prefill_refs(res, lens)
    m = _parity(out, ws, lay, list(range(T)), ref, norm, q, block0)
    touched = set(int(s) for s in sl)
    st = _check_states(spg, spr, sp, touched)
    _check_windows(cpg, cpr, cp, touched)
    # the decode rows through the decode entry point (GEMV projections, the per-token state
    # update) and through this prefill call (tiled GEMMs, the chunked scan) differ in float
    # rounding only: both are checked against the oracle, and their states and windows against
    # each other with the stated tolerances rather than bit equality
    dec = [i for i, L in enumerate(lens) if L == 1]
    rows = cu[dec]
    od, spd, cpd, wsd, layd = _gpu_decode(nhm, pd, h[rows], sl[dec], sp, cp)
    # the decode rows through nhm_mixer_decode against the oracle's results for the same rows
    md = _parity(od, wsd, layd, list(range(len(dec))), ref[rows], norm[rows], q[rows], block0)
    for s in sl[dec]:
        assert rel_l2(spd[s], spg[s]) <= TOL_STATE
        a, b = bf16_to_f64(cpd[s]), bf16_to_f64(cpg[s])
        assert rel_l2(a, b) <= TOL_STATE and rel_max(a, b) <= TOL_OUT
    print(f"mixed batch {lens}: {m}, state rel l2 {st:.3e}; its decode rows through nhm_mixer_decode: {md}")


def _check_states_bf16(sp_gpu, sp_ref, sp_before, touched):
    from oracle import bf16_to_f64
    from tests.gpu_util import rel_l2
    worst = 0.0
    for s in range(sp_ref.shape[0]):
        if s in touched and not np.any(sp_ref[s]):
            assert not np.any(sp_gpu[s]), f"slot {s} should be zero"
        elif s in touched:
            r = rel_l2(bf16_to_f64(sp_gpu[s]), bf16_to_f64(sp_ref[s]))
            worst = max(worst, r)
            assert r <= TOL_STATE_BF16, f"slot {s}: bf16 state rel l2 {r:.3g}"
        else:
            assert np.array_equal(sp_gpu[s], sp_before[s]), f"untouched slot {s} changed"
    return worst


def test_decode_bf16_state_two_steps(nhm, block0):
    """Decode B=8 (one padded row) for two steps on a bf16 state pool: the second step reads
    the state the first rounded. Outputs and every pool row against the oracle's bf16-state
    decode."""
    from oracle import mixer_decode_bf16_state
    from tests.gpu_util import upload_params
    from workloads import bf16_bits, conv_pool, hidden, slots, ssm_pool
    S, B = 16, 8
    sl = slots(2, B, S)
    sl[3] = -1
    sp = bf16_bits(ssm_pool(2, 3, S))
    cp = conv_pool(2, 3, S)
    pd = upload_params(block0)
    spr, cpr = sp.copy(), cp.copy()
    live = [b for b in range(B) if sl[b] >= 0]
    touched = {int(s) for s in sl if s >= 0}
    for step in range(2):
        h = hidden(2, B, extra=40 + step)
        out, spg, cpg, ws, lay = _gpu_decode(nhm, pd, h, sl, sp, cp)
        before = sp.copy()
        ref, res = mixer_decode_bf16_state(block0, h, sl, spr, cpr)
        m = _parity(out, ws, lay, live, ref, res["norm"][live], res["q_out"][live], block0)
        assert np.all(out[3] == 0)
        st = _check_states_bf16(spg, spr, before, touched)
        _check_windows(cpg, cpr, cp, touched)
        sp, cp = spg, cpg                       # the GPU's rounded state feeds the next step
        spr, cpr = spg.copy(), cpg.copy()       # and the oracle starts from the same rows
        print(f"decode bf16 state, step {step}: {m}, state rel l2 {st:.3e}")


@pytest.mark.parametrize("lens,has_init", [([5, 130, 1, 0, 260, 128], [1, 0, 1, 0, 1, 0])])
def test_prefill_bf16_state(nhm, block0, lens, has_init):
    from oracle import mixer_prefill_bf16_state
    from tests.gpu_util import upload_params
    from workloads import bf16_bits, conv_pool, hidden, ssm_pool
    S = 8
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    h = hidden(4, T, extra=50)
    sp, cp = bf16_bits(ssm_pool(4, 3, S)), conv_pool(4, 3, S)
    sl = np.array([7, 0, 3, 5, 1, 6][:len(lens)], np.int32)
    pd = upload_params(block0)
    out, spg, cpg, ws, lay = _gpu_prefill(nhm, pd, h, cu, sl, has_init, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill_bf16_state(block0, h, cu, sl, has_init, spr, cpr)
    norm, q, _ = _prefill_refs(res, lens)
    m = _parity(out, ws, lay, list(range(T)), ref, norm, q, block0)
    touched = set(int(s) for s in sl)
    st = _check_states_bf16(spg, spr, sp, touched)
    _check_windows(cpg, cpr, cp, touched)
    print(f"prefill bf16 state {lens}: {m}, state rel l2 {st:.3e}")


def test_decode_equals_prefill_of_one(nhm, block0):
    from oracle import bf16_to_f64
    from tests.gpu_util import rel_max, upload_params
    from workloads import conv_pool, hidden, ssm_pool
    h = hidden(0, 2)
    sp, cp = ssm_pool(0, 2, 4), conv_pool(0, 2, 4)
    sl = np.array([3, 1], np.int32)
    pd = upload_params(block0)
    od, spd, cpd, _, _ = _gpu_decode(nhm, pd, h, sl, sp, cp)
    op, spp, cpp, _, _ = _gpu_prefill(nhm, pd, h, [0, 1, 2], sl, [1, 1], sp, cp)
    assert rel_max(bf16_to_f64(od), bf16_to_f64(op)) <= TOL_OUT
    for s in (3, 1):
        assert np.linalg.norm(spd[s] - spp[s]) <= 1e-4 * np.linalg.norm(spp[s])
    assert np.array_equal(cpd, cpp)


def test_prefill_carry_split(nhm, block0):
    """prefill(T1) then prefill(T2) from the carried pool row == prefill(T1 + T2)."""
    from oracle import bf16_to_f64
    from tests.gpu_util import rel_l2, rel_max, upload_params
    from workloads import conv_pool, hidden, ssm_pool
    T1, T2 = 200, 77
    h = hidden(3, T1 + T2, extra=9)
    sp, cp = ssm_pool(3, 1, 2), conv_pool(3, 1, 2)
    pd = upload_params(block0)
    ow, spw, cpw, _, _ = _gpu_prefill(nhm, pd, h, [0, T1 + T2], [0], [1], sp, cp)
    o1, sp1, cp1, _, _ = _gpu_prefill(nhm, pd, h[:T1], [0, T1], [0], [1], sp, cp)
    o2, sp2, cp2, _, _ = _gpu_prefill(nhm, pd, h[T1:], [0, T2], [0], [1], sp1, cp1)
    assert rel_max(bf16_to_f64(np.concatenate([o1, o2])), bf16_to_f64(ow)) <= TOL_OUT
    assert rel_l2(sp2[0], spw[0]) <= TOL_STATE
    assert np.array_equal(cp2[0], cpw[0])


def test_prefill_zero_tokens(nhm, block0):
    """Only empty sequences: no token work, yet each pool row is carried through
    (has_initial 1) or reset to the zero state and window (has_initial 0), as the oracle."""
    from oracle import mixer_prefill
    from tests.gpu_util import upload_params
    from workloads import conv_pool, ssm_pool
    S = 8
    cu, sl, hi = [0, 0, 0], [6, 2], [1, 0]
    h = np.zeros((0, H), np.uint16)
    sp, cp = ssm_pool(4, 1, S), conv_pool(4, 1, S)
    pd = upload_params(block0)
    out, spg, cpg, _, _ = _gpu_prefill(nhm, pd, h, cu, sl, hi, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    mixer_prefill(block0, h, cu, sl, hi, spr, cpr)
    assert out.shape == (0, H)
    assert np.array_equal(spg, spr) and np.array_equal(cpg, cpr)
    assert np.array_equal(spg[6], sp[6]) and not np.any(spg[2]) and not np.any(cpg[2])


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_prefill_ragged_15360_23_blocks(nhm):
    """Ragged prefill of 4 sequences (8192, 4096, 2048, 1024 tokens, zero initial state)
    through 23 stacked blocks, each block's output the next one's input.

    Layer 0 is checked in full against the oracle (every token, every final state and
    window). Layers 11 and 22 are checked on the shortest sequence, with the oracle fed
    the GPU's own input to that layer, so each check covers one block (the tolerance is
    per block; the oracle and the GPU path would otherwise drift apart through 22 stacked
    blocks of bf16/e4m3 rounding).
    """
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from tests.gpu_util import dev, host, upload_params, ws_region, zeros_ws
    from tests.oracle_workers import prefill_sequence
    from workloads import RAGGED_LENGTHS, block_params, hidden, slots
    W, S, L = 4, 8, 23
    lens = list(RAGGED_LENGTHS)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    assert T == 15360 and len(lens) == 4
    sl = slots(W, len(lens), S)
    short = int(np.argmin(lens))
    rows_short = list(range(int(cu[short]), int(cu[short + 1])))
    x = hidden(W, T)
    lay = nhm.prefill_ws_layout(T, len(lens))
    ws = zeros_ws(lay["total"])
    cud, sld, hid = dev(cu), dev(sl), dev(np.zeros(len(lens), np.int32))
    check = {0: list(range(len(lens))), 11: [short], 22: [short]}
    got = {}
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=6, mp_context=ctx) as pool:
        jobs = {}
        xd = dev(x)
        for layer in range(L):
            if layer in check:
                xh = host(xd)
                for i in check[layer]:
                    jobs[(layer, i)] = pool.submit(prefill_sequence, (W, layer, xh[cu[i]:cu[i + 1]]))
            pd = upload_params(block_params(W, layer))
            spd = torch.zeros((S, 64, 64, 128), dtype=torch.float32, device="cuda")
            cpd = torch.zeros((S, 3, 6144), dtype=torch.int16, device="cuda")
            out = torch.empty((T, H), dtype=torch.int16, device="cuda")
            nhm.mixer_prefill(pd, xd, cud, sld, hid, spd, cpd, out, ws)
            torch.cuda.synchronize()
            if layer in check:
                got[layer] = dict(out=host(out), sp=host(spd), cp=host(cpd),
                                  q=ws_region(ws, lay["q_out"], T * I, np.uint8).reshape(T, I),
                                  norm=ws_region(ws, lay["norm"], T * I, np.uint16).reshape(T, I),
                                  q_in=ws_region(ws, lay["q_in"], T * H, np.uint8).reshape(T, H))
            xd = out
        refs = {key: f.result() for key, f in jobs.items()}

    from tests.gpu_util import block_parity, rel_l2, rel_max
    from oracle import bf16_to_f64
    failures = []
    for layer, seqs in check.items():
        g = got[layer]
        p = block_params(W, layer)
        rows = [r for i in seqs for r in range(int(cu[i]), int(cu[i + 1]))]
        ref_out = np.concatenate([refs[(layer, i)]["out"] for i in seqs])
        ref_norm = np.concatenate([refs[(layer, i)]["norm"] for i in seqs])
        ref_q = np.concatenate([refs[(layer, i)]["q_out"] for i in seqs])
        if layer == 0:
            ref_qin = np.concatenate([refs[(layer, i)]["q_in"] for i in seqs])
            assert np.array_equal(g["q_in"], ref_qin)                                        # a1, every token
        try:
            m = block_parity(g["out"][rows], g["q"][rows], g["norm"][rows], ref_out, ref_norm, ref_q, p)
        except AssertionError as e:
            m = f"FAILED: {e}"
            failures.append(f"layer {layer}: {e}")
        states = []
        for i in seqs:
            r = rel_l2(g["sp"][sl[i]], refs[(layer, i)]["state"])
            states.append(round(float(r), 7))
            if r > TOL_STATE:
                failures.append(f"layer {layer} sequence {i}: state rel l2 {r:.3g}")
            a, b = bf16_to_f64(g["cp"][sl[i]]), bf16_to_f64(refs[(layer, i)]["window"])
            if not (rel_l2(a, b) <= TOL_STATE and rel_max(a, b) <= TOL_OUT):
                failures.append(f"layer {layer} sequence {i} window")
        print(f"layer {layer} sequences {seqs} (rows {rows[0]}..{rows[-1]}): {m}, state rel l2 {states}")
    assert not failures, "; ".join(failures)


# Another geometry: hidden 256, 8 heads of 64 in 2 groups (4 heads per group), so the B and C
# channels sit at other offsets, the group's B/C windows are shared by 4 heads instead of 8,
# and the projections take other dispatch shapes (in_proj 1544 x 256, out_proj 256 x 512).
SMALL = dict(hidden=256, n_heads=8, head_dim=64, d_state=128, n_groups=2, conv_width=4, rms_eps=1e-5)


def _small_parity(out, ws, lay, rows, T, ref, ref_norm, ref_q, p):
    from tests.gpu_util import block_parity, ws_region
    inner = SMALL["n_heads"] * SMALL["head_dim"]
    q = ws_region(ws, lay["q_out"], T * inner, np.uint8).reshape(T, inner)[rows]
    nrm = ws_region(ws, lay["norm"], T * inner, np.uint16).reshape(T, inner)[rows]
    return block_parity(out[rows], q, nrm, ref[rows], ref_norm, ref_q, p)


def test_decode_small_geometry(nhm):
    """Decode at hidden 256, 8 heads in 2 groups, with a padded row."""
    from oracle import mixer_decode
    from tests.gpu_util import dev, host, upload_params, ws_region, zeros_ws
    from workloads import block_params, conv_pool, hidden, ssm_pool
    g, S, B = SMALL, 12, 6
    p = block_params(5, 0, g)
    h = hidden(5, B, g)
    sl = np.array([3, 0, -1, 11, 7, 5], np.int32)
    sp, cp = ssm_pool(5, 0, S, g=g), conv_pool(5, 0, S, g=g)
    pd = upload_params(p, g)
    lay = nhm.decode_ws_layout(B, g)
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((B, g["hidden"]), dtype=torch.int16, device="cuda")
    nhm.mixer_decode(pd, dev(h), dev(sl), spd, cpd, out, ws)
    torch.cuda.synchronize()
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_decode(p, h, sl, spr, cpr, g=g)
    q_in = ws_region(ws, lay["q_in"], B * g["hidden"], np.uint8).reshape(B, g["hidden"])
    assert np.array_equal(q_in, res["q_in"].reshape(B, g["hidden"]))
    o = host(out)
    live = [b for b in range(B) if sl[b] >= 0]
    m = _small_parity(o, ws, lay, live, B, ref, res["norm"][live], res["q_out"][live], p)
    assert np.all(o[2] == 0)
    touched = {int(s) for s in sl if s >= 0}
    _check_states(host(spd), spr, sp, touched)
    _check_windows(host(cpd), cpr, cp, touched)
    print(f"decode small geometry: {m}")


def test_prefill_small_geometry(nhm):
    """Varlen prefill at hidden 256, 8 heads in 2 groups: a two-chunk sequence from a carried
    state, a fresh one and a one-token continuation."""
    from oracle import mixer_prefill
    from tests.gpu_util import dev, host, upload_params, zeros_ws
    from workloads import block_params, conv_pool, hidden, ssm_pool
    g, S = SMALL, 10
    lens, has_init = [130, 5, 1], [1, 0, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    p = block_params(6, 0, g)
    h = hidden(6, T, g)
    sl = np.array([4, 9, 0], np.int32)
    sp, cp = ssm_pool(6, 0, S, g=g), conv_pool(6, 0, S, g=g)
    pd = upload_params(p, g)
    lay = nhm.prefill_ws_layout(T, len(lens), g=g)
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((T, g["hidden"]), dtype=torch.int16, device="cuda")
    nhm.mixer_prefill(pd, dev(h), dev(cu), dev(sl), dev(np.asarray(has_init, np.int32)), spd, cpd, out, ws)
    torch.cuda.synchronize()
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(p, h, cu, sl, has_init, spr, cpr, g=g)
    norm, q, _ = _prefill_refs(res, lens)
    m = _small_parity(host(out), ws, lay, list(range(T)), T, ref, norm, q, p)
    touched = {int(s) for s in sl}
    _check_states(host(spd), spr, sp, touched)
    _check_windows(host(cpd), cpr, cp, touched)
    print(f"prefill small geometry {lens}: {m}")


# A third geometry: hidden 256, 16 heads of 64 in one group, so every head shares one B/C
# group and a norm group spans 1,024 channels. The decode state kernel finishes norm groups of
# at most 512 channels itself; wider ones go to a launch of their own (with the B/C window
# shift), which these tests reach.
WIDE = dict(hidden=256, n_heads=16, head_dim=64, d_state=128, n_groups=1, conv_width=4, rms_eps=1e-5)


def _geom_parity(g, out, ws, lay, rows, T, ref, ref_norm, ref_q, p):
    from tests.gpu_util import block_parity, ws_region
    inner = g["n_heads"] * g["head_dim"]
    q = ws_region(ws, lay["q_out"], T * inner, np.uint8).reshape(T, inner)[rows]
    nrm = ws_region(ws, lay["norm"], T * inner, np.uint16).reshape(T, inner)[rows]
    return block_parity(out[rows], q, nrm, ref[rows], ref_norm, ref_q, p)


def test_decode_wide_group(nhm):
    """Decode with one 1,024-channel norm group (16 heads, hidden 256), with a padded row: the
    norm runs as its own launch."""
    from oracle import mixer_decode
    from tests.gpu_util import dev, host, upload_params, ws_region, zeros_ws
    from workloads import block_params, conv_pool, hidden, ssm_pool
    g, S, B = WIDE, 9, 5
    p = block_params(7, 0, g)
    h = hidden(7, B, g)
    sl = np.array([6, -1, 2, 8, 0], np.int32)
    sp, cp = ssm_pool(7, 0, S, g=g), conv_pool(7, 0, S, g=g)
    pd = upload_params(p, g)
    lay = nhm.decode_ws_layout(B, g)
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((B, g["hidden"]), dtype=torch.int16, device="cuda")
    nhm.dispatch_counters(reset=True)
    nhm.mixer_decode(pd, dev(h), dev(sl), spd, cpd, out, ws)
    torch.cuda.synchronize()
    path = nhm.dispatch_counters(reset=True)
    assert "gnorm_quant" in path and "decode_ssm" in path, path
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_decode(p, h, sl, spr, cpr, g=g)
    q_in = ws_region(ws, lay["q_in"], B * g["hidden"], np.uint8).reshape(B, g["hidden"])
    assert np.array_equal(q_in, res["q_in"].reshape(B, g["hidden"]))
    o = host(out)
    live = [b for b in range(B) if sl[b] >= 0]
    m = _geom_parity(g, o, ws, lay, live, B, ref, res["norm"][live], res["q_out"][live], p)
    assert np.all(o[1] == 0)
    touched = {int(s) for s in sl if s >= 0}
    _check_states(host(spd), spr, sp, touched)
    _check_windows(host(cpd), cpr, cp, touched)
    print(f"decode wide group: {m}, path {path}")


def test_prefill_wide_group(nhm):
    """Varlen prefill with one 1,024-channel norm group: a two-chunk sequence from a carried
    state, a fresh one and a one-token continuation."""
    from oracle import mixer_prefill
    from tests.gpu_util import dev, host, upload_params, zeros_ws
    from workloads import block_params, conv_pool, hidden, ssm_pool
    g, S = WIDE, 7
    lens, has_init = [131, 3, 1], [1, 0, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    p = block_params(8, 0, g)
    h = hidden(8, T, g)
    sl = np.array([5, 1, 3], np.int32)
    sp, cp = ssm_pool(8, 0, S, g=g), conv_pool(8, 0, S, g=g)
    pd = upload_params(p, g)
    lay = nhm.prefill_ws_layout(T, len(lens), g=g)
    ws = zeros_ws(lay["total"])
    spd, cpd = dev(sp), dev(cp)
    out = torch.empty((T, g["hidden"]), dtype=torch.int16, device="cuda")
    nhm.mixer_prefill(pd, dev(h), dev(cu), dev(sl), dev(np.asarray(has_init, np.int32)), spd, cpd, out, ws)
    torch.cuda.synchronize()
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(p, h, cu, sl, has_init, spr, cpr, g=g)
    norm, q, _ = _prefill_refs(res, lens)
    m = _geom_parity(g, host(out), ws, lay, list(range(T)), T, ref, norm, q, p)
    touched = {int(s) for s in sl}
    _check_states(host(spd), spr, sp, touched)
    _check_windows(host(cpd), cpr, cp, touched)
    print(f"prefill wide group {lens}: {m}")


def _edge_params():
    """Block 0's parameters with the method's corner cases switched on: heads 0-7 have
    dt_raw + dt_bias > 20 (softplus taken as its argument), head 8 A_log = 0 (A = -1) and head 9
    A_log = ln 16 (A = -16), the two ends of the A_log draw."""
    from workloads import block_params
    p = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in block_params(0, 0).items()}
    p["dt_bias"][:8] = np.float32(25.0)
    p["A_log"][8] = np.float32(0.0)
    p["A_log"][9] = np.float32(np.log(16.0))
    return p


def _edge_hidden(T, extra):
    """Block input with a tenth of its entries scaled to |x| in [4, 2000]: |x| / s >= 448 for
    the static scale s = 4/448, so those codes saturate at +-448."""
    from workloads import bf16_bits
    r = np.random.default_rng(9000 + extra)
    x = r.standard_normal((T, H)).astype(np.float32)
    big = r.random((T, H)) < 0.1
    x[big] = np.sign(x[big]) * r.uniform(4.0, 2000.0, int(big.sum())).astype(np.float32)
    return bf16_bits(x)


def test_decode_edge_cases(nhm):
    """Decode B=8 with the softplus linear branch, both ends of A_log and saturating inputs."""
    from oracle import mixer_decode, quantize_static
    from tests.gpu_util import upload_params, ws_region
    from workloads import conv_pool, ssm_pool, slots
    p = _edge_params()
    B, S = 8, 16
    h = _edge_hidden(B, 1)
    assert np.sum(quantize_static(h, p["in_a_scale"]) & 0x7f == 0x7e) > 1000     # saturated codes present
    sl = slots(2, B, S)
    sp, cp = ssm_pool(2, 5, S), conv_pool(2, 5, S)
    out, spg, cpg, ws, lay = _gpu_decode(nhm, upload_params(p), h, sl, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_decode(p, h, sl, spr, cpr)
    assert np.array_equal(ws_region(ws, lay["q_in"], B * H, np.uint8).reshape(B, H), res["q_in"].reshape(B, H))
    m = _parity(out, ws, lay, list(range(B)), ref, res["norm"], res["q_out"], p)
    st = _check_states(spg, spr, sp, set(int(s) for s in sl))
    _check_windows(cpg, cpr, cp, set(int(s) for s in sl))
    print(f"decode edge cases: {m}, state rel l2 {st:.3e}")


def test_prefill_edge_cases(nhm):
    """Prefill of a 100-token sequence from a carried state and a fresh 3-token one with the same
    corner cases (under 128 tokens: the whole-call bar applies)."""
    from oracle import mixer_prefill
    from tests.gpu_util import upload_params
    from workloads import conv_pool, ssm_pool
    p = _edge_params()
    lens, has_init, S = [100, 3], [1, 0], 4
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    h = _edge_hidden(T, 2)
    sl = np.array([2, 0], np.int32)
    sp, cp = ssm_pool(3, 5, S), conv_pool(3, 5, S)
    out, spg, cpg, ws, lay = _gpu_prefill(nhm, upload_params(p), h, cu, sl, has_init, sp, cp)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = mixer_prefill(p, h, cu, sl, has_init, spr, cpr)
    norm, q, qin = _prefill_refs(res, lens)
    from tests.gpu_util import ws_region
    assert np.array_equal(ws_region(ws, lay["q_in"], T * H, np.uint8), qin.reshape(-1))
    m = _parity(out, ws, lay, list(range(T)), ref, norm, q, p)
    st = _check_states(spg, spr, sp, set(int(s) for s in sl))
    _check_windows(cpg, cpr, cp, set(int(s) for s in sl))
    print(f"prefill edge cases: {m}, state rel l2 {st:.3e}")


def test_block_per_tensor_weight_scales(nhm, block0):
    """A block whose projections carry one weight scale each (the checkpoint's form, the
    per-tensor flag of nhm_fp8_weight) equals, bit for bit, the same block with those scales
    broadcast to per-channel vectors: decode (B = 8, the GEMV path) and prefill (the GEMM path),
    outputs, state pools and conv windows."""
    from tests.gpu_util import dev, host, zeros_ws
    from workloads import conv_pool, hidden, ssm_pool
    p = dict(block0)
    for key in ("in_w_scale", "out_w_scale"):
        p[key] = np.full_like(p[key], p[key][0])               # one scale per projection
    vec = nhm.MixerParams(nhm.Fp8Weight(dev(p["in_w"]), dev(p["in_w_scale"]), dev(p["in_a_scale"])),
                          nhm.Fp8Weight(dev(p["out_w"]), dev(p["out_w_scale"]), dev(p["out_a_scale"])),
                          dev(p["conv_w"]), dev(p["conv_b"]), dev(p["norm_w"]), dev(p["A_log"]), dev(p["D"]),
                          dev(p["dt_bias"]))
    one = nhm.MixerParams(nhm.Fp8Weight(dev(p["in_w"]), dev(p["in_w_scale"][:1].copy()), dev(p["in_a_scale"])),
                          nhm.Fp8Weight(dev(p["out_w"]), dev(p["out_w_scale"][:1].copy()), dev(p["out_a_scale"])),
                          dev(p["conv_w"]), dev(p["conv_b"]), dev(p["norm_w"]), dev(p["A_log"]), dev(p["D"]),
                          dev(p["dt_bias"]))
    sp, cp = ssm_pool(0, 3, 10), conv_pool(0, 3, 10)          # 10 slots: every index below is in range
    h = hidden(0, 8, extra=21)
    sl = np.array([9, 0, 4, 7, 2, 5, 1, 8], np.int32)
    res = []
    for prm in (vec, one):
        lay = nhm.decode_ws_layout(8)
        spd, cpd = dev(sp), dev(cp)
        out = torch.empty((8, H), dtype=torch.int16, device="cuda")
        nhm.mixer_decode(prm, dev(h), dev(sl), spd, cpd, out, zeros_ws(lay["total"]))
        torch.cuda.synchronize()
        res.append((host(out), host(spd), host(cpd)))
    for x, y in zip(*res):
        assert np.array_equal(x, y)
    hp = hidden(0, 300, extra=22)
    res = []
    for prm in (vec, one):
        lay = nhm.prefill_ws_layout(300, 2)
        spd, cpd = dev(sp), dev(cp)
        out = torch.empty((300, H), dtype=torch.int16, device="cuda")
        nhm.mixer_prefill(prm, dev(hp), dev(np.array([0, 170, 300], np.int32)), dev(np.array([3, 6], np.int32)),
                          dev(np.array([1, 0], np.int32)), spd, cpd, out, zeros_ws(lay["total"]))
        torch.cuda.synchronize()
        res.append((host(out), host(spd), host(cpd)))
    for x, y in zip(*res):
        assert np.array_equal(x, y)

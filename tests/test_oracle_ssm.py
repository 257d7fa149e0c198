"""Pins of the oracle's recurrence: brute-force chunked == sequential, closed forms, carry."""
import numpy as np
import pytest

from oracle import dt_and_decay, ssd_chunked, ssm_scan_sequential


def _tiny(T=7, H=4, G=2, P=3, N=5, seed=0, zero_h0=False):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H, P))
    Bm = r.standard_normal((T, G, N))
    Cm = r.standard_normal((T, G, N))
    dt = np.exp(r.uniform(np.log(1e-3), np.log(0.5), (T, H)))
    A = -np.exp(r.uniform(0, np.log(16), H))
    dA = np.exp(dt * A)
    D = 1 + 0.1 * r.standard_normal(H)
    h0 = np.zeros((H, P, N)) if zero_h0 else 0.1 * r.standard_normal((H, P, N))
    return x, Bm, Cm, dt, dA, D, h0


@pytest.mark.parametrize("T,Q", [(7, 4), (8, 4), (1, 4), (9, 3), (5, 8)])
@pytest.mark.parametrize("seed", [0, 1])
def test_chunked_equals_sequential(T, Q, seed):
    args = _tiny(T=T, seed=seed)
    y1, h1 = ssm_scan_sequential(*args)
    y2, h2 = ssd_chunked(*args, chunk=Q)
    assert y1.shape == y2.shape == (T, 4, 3) and h1.shape == (4, 3, 5)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * max(1.0, np.max(np.abs(y1)))
    assert np.max(np.abs(h1 - h2)) <= 1e-12 * max(1.0, np.max(np.abs(h1)))


def test_brute_force_by_hand_loops():
    x, Bm, Cm, dt, dA, D, h0 = _tiny(T=4, H=2, G=1, P=2, N=3, seed=5)
    y, hT = ssm_scan_sequential(x, Bm, Cm, dt, dA, D, h0)
    h = h0.copy()
    for t in range(4):
        for hh in range(2):
            for p in range(2):
                acc = 0.0
                for n in range(3):
                    h[hh, p, n] = dA[t, hh] * h[hh, p, n] + dt[t, hh] * x[t, hh, p] * Bm[t, 0, n]
                    acc += h[hh, p, n] * Cm[t, 0, n]
                assert abs(y[t, hh, p] - (acc + D[hh] * x[t, hh, p])) < 1e-12
    assert np.max(np.abs(hT - h)) < 1e-12


def test_no_decay_no_skip_is_prefix_sum():
    x, Bm, Cm, dt, _, _, h0 = _tiny(T=6, seed=2)
    _, dA = dt_and_decay(np.zeros((6, 4), np.uint16), np.zeros(4, np.float32), np.full(4, -np.inf, np.float32))
    assert np.all(dA == 1.0)
    Cm = np.zeros_like(Cm)
    Cm[:, :, 2] = 1.0                      # read state column n = 2
    y, _ = ssm_scan_sequential(x, Bm, Cm, dt, dA, np.zeros(4), h0)
    hpg = 2
    for hh in range(4):
        g = hh // hpg
        inc = dt[:, hh, None] * x[:, hh, :] * Bm[:, g, 2][:, None]       # [T, P]
        want = h0[hh, :, 2][None, :] + np.cumsum(inc, axis=0)
        assert np.max(np.abs(y[:, hh, :] - want)) < 1e-12


def test_single_token_from_zero_state():
    x, Bm, Cm, dt, dA, D, h0 = _tiny(T=1, seed=3, zero_h0=True)
    y, h = ssm_scan_sequential(x, Bm, Cm, dt, dA, D, h0)
    for hh in range(4):
        g = hh // 2
        want = dt[0, hh] * np.dot(Cm[0, g], Bm[0, g]) * x[0, hh] + D[hh] * x[0, hh]
        assert np.max(np.abs(y[0, hh] - want)) < 1e-12


def test_pure_decay_of_initial_state():
    x, Bm, Cm, dt, dA, D, h0 = _tiny(T=5, seed=4)
    x = np.zeros_like(x)
    y, h = ssm_scan_sequential(x, Bm, Cm, dt, dA, D, h0)
    decay = np.cumprod(dA, axis=0)          # [T, H]
    assert np.max(np.abs(h - decay[-1][:, None, None] * h0)) < 1e-14
    for t in range(5):
        for hh in range(4):
            want = decay[t, hh] * h0[hh] @ Cm[t, hh // 2]
            assert np.max(np.abs(y[t, hh] - want)) < 1e-14


def test_carry_split_equals_whole():
    x, Bm, Cm, dt, dA, D, h0 = _tiny(T=9, seed=6)
    y, h = ssm_scan_sequential(x, Bm, Cm, dt, dA, D, h0)
    for T1 in (1, 4, 8):
        ya, ha = ssm_scan_sequential(x[:T1], Bm[:T1], Cm[:T1], dt[:T1], dA[:T1], D, h0)
        yb, hb = ssm_scan_sequential(x[T1:], Bm[T1:], Cm[T1:], dt[T1:], dA[T1:], D, ha)
        assert np.max(np.abs(np.concatenate([ya, yb]) - y)) < 1e-12
        assert np.max(np.abs(hb - h)) < 1e-12


def test_dt_softplus_and_decay_closed_forms():
    from workloads import bf16_bits
    raw = bf16_bits(np.array([[0.0, 1.0, 25.0, -3.0]], np.float32))
    bias = np.array([0.0, 0.5, 0.0, 0.25], np.float32)
    A_log = np.array([0.0, np.log(2.0), 1.0, 0.0], np.float32)
    dt, dA = dt_and_decay(raw, bias, A_log)
    want = [np.log(2.0), np.log1p(np.exp(1.5)), 25.0, np.log1p(np.exp(-2.75))]
    assert np.max(np.abs(dt[0] - want)) < 1e-12
    A = -np.exp(A_log.astype(np.float64))
    assert np.max(np.abs(dA[0] - np.exp(np.array(want) * A))) < 1e-15
    assert dA[0, 0] == 0.5                   # softplus(0) = ln 2, A = -1

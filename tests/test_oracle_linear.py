"""Pins of the oracle's W8A8 GEMM: brute force on tiny shapes and one-hot rows."""
import numpy as np

from oracle import e4m3_decode, fp8_linear


def _codes(r, shape):
    c = r.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x38), c).astype(np.uint8)   # no NaN codes


def test_fp8_linear_brute_force():
    r = np.random.default_rng(11)
    M, N, K = 3, 5, 7
    a, w = _codes(r, (M, K)), _codes(r, (N, K))
    ws = r.uniform(0.1, 2.0, N).astype(np.float32)
    sa = np.array([0.25], np.float32)
    got = fp8_linear(a, w, ws, sa)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(e4m3_decode(a[m, k])) * float(e4m3_decode(w[n, k]))
            want = acc * float(sa[0]) * float(ws[n])
            assert abs(got[m, n] - want) <= 1e-12 * max(1.0, abs(want))


def test_fp8_linear_one_hot_rows_copy_scaled_columns():
    r = np.random.default_rng(12)
    M, N, K = 4, 6, 16
    a = _codes(r, (M, K))
    w = np.zeros((N, K), np.uint8)
    ks = [0, 3, 15, 7, 7, 9]
    for n, k in enumerate(ks):
        w[n, k] = 0x38            # 1.0
    ws = np.array([1, 2, 0.5, 3, -1, 0.125], np.float32)
    sa = np.array([4.0 / 448.0], np.float32)
    got = fp8_linear(a, w, ws, sa)
    for n, k in enumerate(ks):
        assert np.array_equal(got[:, n], e4m3_decode(a[:, k]) * np.float64(sa[0]) * np.float64(ws[n]))


def test_fp8_linear_orientation_is_out_in():
    # W is [N, K]; a transposed weight must not give the same answer
    r = np.random.default_rng(13)
    a = _codes(r, (2, 8))
    w = _codes(r, (8, 8))
    ws = np.ones(8, np.float32)
    sa = np.ones(1, np.float32)
    assert not np.allclose(fp8_linear(a, w, ws, sa), fp8_linear(a, w.T.copy(), ws, sa))

"""Pins of the oracle's causal depthwise conv: torch conv1d, one-hot taps, the carried window."""
import numpy as np
import torch

from oracle import bf16_from_f64, bf16_to_f64, causal_conv1d_silu
from workloads import bf16_bits


def _case(T, C, seed, W=4):
    r = np.random.default_rng(seed)
    x = bf16_bits(r.standard_normal((T, C)).astype(np.float32))
    win = bf16_bits(r.standard_normal((W - 1, C)).astype(np.float32))
    w = bf16_bits((0.5 * r.standard_normal((C, W))).astype(np.float32))
    b = bf16_bits((0.1 * r.standard_normal(C)).astype(np.float32))
    return x, win, w, b


def test_conv_matches_torch_conv1d_f64():
    T, C = 9, 24
    x, win, w, b = _case(T, C, 1)
    pre_out, out_bits, _ = causal_conv1d_silu(x, win, w, b)
    u = torch.from_numpy(np.concatenate([bf16_to_f64(win), bf16_to_f64(x)], 0).T[None].copy())
    ref = torch.nn.functional.conv1d(u, torch.from_numpy(bf16_to_f64(w)[:, None, :].copy()),
                                     torch.from_numpy(bf16_to_f64(b).copy()), groups=C)[0].T.numpy()
    ref = torch.nn.functional.silu(torch.from_numpy(ref)).numpy()
    assert pre_out.shape == (T, C)
    assert np.max(np.abs(pre_out - ref)) <= 1e-12
    assert np.array_equal(out_bits, bf16_from_f64(ref))


def test_conv_one_hot_current_tap_gives_silu():
    T, C = 5, 8
    x, win, _, _ = _case(T, C, 2)
    w = np.zeros((C, 4), np.uint16)
    w[:, 3] = 0x3F80          # 1.0 on the current-token tap
    b = np.zeros(C, np.uint16)
    out, _, _ = causal_conv1d_silu(x, win, w, b)
    xv = bf16_to_f64(x)
    assert np.max(np.abs(out - xv / (1 + np.exp(-xv)))) == 0.0


def test_conv_one_hot_oldest_tap_reads_window():
    T, C = 2, 8
    x, win, _, _ = _case(T, C, 3)
    w = np.zeros((C, 4), np.uint16)
    w[:, 0] = 0x3F80          # tap 0 sees the token three steps back
    b = np.zeros(C, np.uint16)
    out, _, _ = causal_conv1d_silu(x, win, w, b)
    u = bf16_to_f64(win)
    assert np.array_equal(out, u[:2] / (1 + np.exp(-u[:2])))


def test_conv_window_carry():
    T, C = 11, 16
    x, win, w, b = _case(T, C, 4)
    _, full, wfull = causal_conv1d_silu(x, win, w, b)
    for T1 in (1, 2, 3, 7):
        _, o1, w1 = causal_conv1d_silu(x[:T1], win, w, b)
        _, o2, w2 = causal_conv1d_silu(x[T1:], w1, w, b)
        assert np.array_equal(np.concatenate([o1, o2]), full)
        assert np.array_equal(w2, wfull)
    assert np.array_equal(wfull, x[-3:])
    # a sequence shorter than the window mixes the old window and the new rows
    _, _, wshort = causal_conv1d_silu(x[:1], win, w, b)
    assert np.array_equal(wshort, np.concatenate([win[1:], x[:1]]))

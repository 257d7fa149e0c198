"""The oracle's bf16 SSM state pool (widen to f32, compute, round back to bf16).

Pins: the narrowing is torch's float32 -> bfloat16 cast (round half to even) of the f32
computation's state, computed independently here; rows the call does not touch keep
their bits; on a pool whose values are already bf16 the outputs of one call equal the f32
pool's; and a second step from the rounded state differs from the f32 pool's second step
(the two caches are different computations), by no more than the state's bf16 rounding
can explain.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def _bf16_of_f32(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


@pytest.fixture(scope="module")
def case():
    from workloads import block_params, conv_pool, hidden, ssm_pool
    p = block_params(0, 0)
    sp32 = ssm_pool(0, 5, 4)
    sp16 = _bf16_of_f32(sp32)                               # a bf16 pool
    cp = conv_pool(0, 5, 4)
    h = hidden(0, 3, extra=5)
    return p, sp16, cp, h


def test_decode_bf16_state_narrowing_and_untouched_rows(case):
    from oracle import bf16_to_f64, mixer_decode, mixer_decode_bf16_state
    p, sp16, cp, h = case
    slots = np.array([2, -1, 0], np.int32)
    a16, ac = sp16.copy(), cp.copy()
    out16, _ = mixer_decode_bf16_state(p, h, slots, a16, ac)
    w32, wc = bf16_to_f64(sp16).astype(np.float32), cp.copy()   # the same values as an f32 pool
    out32, _ = mixer_decode(p, h, slots, w32, wc)
    assert np.array_equal(out16, out32)                        # one call: the same computation
    assert np.array_equal(ac, wc)
    for s in (0, 2):
        assert np.array_equal(a16[s], _bf16_of_f32(w32[s]))    # narrowed by round half to even
    for s in (1, 3):
        assert np.array_equal(a16[s], sp16[s])                 # untouched rows keep their bits


def test_bf16_state_is_a_different_computation(case):
    from oracle import bf16_to_f64, mixer_decode, mixer_decode_bf16_state
    p, sp16, cp, h = case
    slots = np.array([1], np.int32)
    a16, ac = sp16.copy(), cp.copy()
    w32, wc = bf16_to_f64(sp16).astype(np.float32), cp.copy()
    for t in range(2):
        o16, _ = mixer_decode_bf16_state(p, h[t:t + 1], slots, a16, ac)
        o32, _ = mixer_decode(p, h[t:t + 1], slots, w32, wc)
    d = np.linalg.norm(bf16_to_f64(a16[1]) - w32[1]) / np.linalg.norm(w32[1])
    assert 0 < d <= 2.0 ** -8                                   # the state's bf16 rounding, no more
    assert not np.array_equal(o16, o32)                        # the second step sees the rounded state
    # end to end the small state difference is amplified by the e4m3 re-quantization of the
    # out_proj input (a few codes flip, each moving every output): held to the end-to-end bound
    assert np.max(np.abs(o16 - o32)) <= 0.1 * np.sqrt(np.mean(o32 ** 2))


def test_prefill_bf16_state_narrowing(case):
    from oracle import bf16_to_f64, mixer_prefill, mixer_prefill_bf16_state
    p, sp16, cp, _ = case
    from workloads import hidden
    hh = hidden(3, 9, extra=6)
    cu, sl, hi = [0, 4, 4, 9], [3, 1, 0], [1, 0, 0]
    a16, ac = sp16.copy(), cp.copy()
    out16, _ = mixer_prefill_bf16_state(p, hh, cu, sl, hi, a16, ac)
    w32, wc = bf16_to_f64(sp16).astype(np.float32), cp.copy()
    out32, _ = mixer_prefill(p, hh, cu, sl, hi, w32, wc)
    assert np.array_equal(out16, out32) and np.array_equal(ac, wc)
    for s in (3, 1, 0):
        assert np.array_equal(a16[s], _bf16_of_f32(w32[s]))
    assert not np.any(a16[1])                                  # an empty fresh sequence: zero row
    assert np.array_equal(a16[2], sp16[2])

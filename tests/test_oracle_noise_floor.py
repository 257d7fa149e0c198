"""The float-noise floor of the block tolerance, measured on the CPU.

A plain float32 evaluation of the block (tests/f32_floor.py: the projections summed exactly
and rounded once to float32, the conv, the recurrence -- a float32 state advanced token by
token -- and the gated norm in float32, bf16 between stages) is compared end to end with
the float64 oracle on the inputs of two GPU parity tests. The a9 re-quantization turns the
two evaluations' rare one-step bf16 differences of the norm output into whole e4m3 steps,
each of which moves every output of its row by up to ~0.02 RMS. On the 512-token prefill and
on the 477-token mixed batch that float32 evaluation already misses the 2e-2 whole-call bar,
while on every row without a flipped code it agrees with the oracle to float32 rounding: the
whole-call bar is not attainable by a float32 implementation at these sizes, which is why the
GPU tests assert it per row (rows whose codes equal the oracle's) from 128 tokens per call.
"""
import numpy as np

import oracle.nhm_oracle as O
from tests.f32_floor import mixer_prefill_f32
from workloads import block_params, conv_pool, hidden, ssm_pool


def _floor(wl, lens, has_init, S, slots, extra=0, pool_layer=0):
    p = block_params(0, 0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    h = hidden(wl, int(cu[-1]), extra=extra)
    sp, cp = ssm_pool(wl, pool_layer, S), conv_pool(wl, pool_layer, S)
    spr, cpr = sp.copy(), cp.copy()
    ref, res = O.mixer_prefill(p, h, cu, slots, has_init, spr, cpr)
    refq = np.concatenate([r["q_out"] for r in res if r is not None])
    out, q = mixer_prefill_f32(p, h, cu, has_init, [cp[s] for s in slots], [sp[s] for s in slots])
    rms = np.sqrt(np.mean(ref ** 2))
    d = np.abs(out - ref) / rms
    flip_rows = np.any(q != refq, axis=1)
    return float(d.max()), float(d[~flip_rows].max()), float(np.mean(q != refq)), float(flip_rows.mean())


def test_f32_floor_prefill_512():
    """The inputs of the 512-token prefill parity test (one sequence from a carried state)."""
    e2e, clean, flips, rows = _floor(3, [512], [1], 2, [1])
    print(f"float32 floor, prefill 512: end to end {e2e:.4f}, flip-free rows {clean:.2e}, "
          f"a9 flips {flips:.2e} on {rows:.1%} of the rows")
    assert e2e > 2e-2            # the whole-call bar is out of reach of a float32 evaluation
    assert clean < 1e-4          # rows without a flipped code agree to float32 rounding
    assert 0 < flips < 1e-3


def test_f32_floor_mixed_batch():
    """The inputs of the mixed-batch parity test (8 decode rows, two continuations, a prompt)."""
    lens = [1, 1, 300, 1, 1, 40, 1, 129, 1, 1, 1]
    has_init = [1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1]
    slots = [9, 2, 14, 0, 5, 11, 7, 3, 12, 1, 15]
    e2e, clean, flips, rows = _floor(4, lens, has_init, 16, slots, extra=31, pool_layer=2)
    print(f"float32 floor, mixed batch: end to end {e2e:.4f}, flip-free rows {clean:.2e}, "
          f"a9 flips {flips:.2e} on {rows:.1%} of the rows")
    assert e2e > 2e-2
    assert clean < 1e-4
    assert 0 < flips < 1e-3

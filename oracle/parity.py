"""Comparison helpers for HIP-vs-oracle parity (test infrastructure, like the oracle).

Used by tests/ and by bench.py's parity sample; never by the product path.
"""
import numpy as np


def rel_max(got, ref):
    """max |got - ref| / RMS(ref): the block-output tolerance measure."""
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.sqrt(np.mean(ref * ref)))


def rel_l2(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / np.linalg.norm(ref))


def block_parity(out_bits, q_gpu, norm_gpu, ref_out, ref_norm, ref_q, p, tol=2e-2, e2e_sanity=0.1):
    """Parity of one block call, given the oracle's results on the same block input.

    The out_proj input codes (a9) are a decision that float noise upstream can
    tip either way near an e4m3 rounding boundary, so both neighbouring codes are
    correct there. What is unique is checked exactly or to a bound:
      1. the block output against the oracle's out_proj applied to the GPU's own
         codes: max |d| <= tol * RMS (the stated block tolerance);
      2. the codes against the oracle quantizer applied to the GPU's own bf16 norm
         output: bit-exact;
      3. the bf16 norm output against the oracle's float64 one: ||d|| / ||ref|| <=
         4e-3 (one bf16 ulp) and |d| <= 2^-7 |ref| + 0.05 RMS elementwise (up to one
         element per 1e7 outputs, rounded up, may exceed it, by at most 1.5x);
      4. every code that differs from the oracle's is reachable from a norm value
         within eta = 2^-7 |o| + 0.05 RMS of the oracle's o (the elementwise norm bound), and such codes are
         rare (<= 1 %).
    Bounds 3-4 are the float-noise floor: evaluating the oracle with float32
    accumulation in its projections (the pages' COMPUTE_32F) moves its own norm
    output by up to 0.025 RMS before rounding and flips ~0.03 % of its a9 codes
    (tests/test_oracle_noise_floor.py).
    The GPU's in_proj sums its e4m3 products in the MFMA's adder, coarser than f32
    (measured up to ~2^-17 of sum |a b| per 128 products), which adds to that floor:
    at 15,360 tokens (6.3e7 norm outputs) one element reached 1.02x the elementwise
    bound while the oracle's own float32 variant stays within 0.78x of it; with the
    32x32x64 instruction (up to ~166 vs ~111 x 2^-24 of sum |a b| per reduction, the same
    median) one of 4.2e6 outputs of a 1,024-token block reached 1.002x.
    The end-to-end difference to the oracle's output is returned and held to a
    sanity bound only: the same float32 variant of the oracle already differs
    from the float64 oracle by 0.0206 RMS end to end at T = 128.
    """
    from oracle import bf16_from_f64, bf16_to_f64, e4m3_decode, fp8_linear, quantize_static
    out = bf16_to_f64(out_bits)
    s = p["out_a_scale"]
    a10 = fp8_linear(q_gpu, p["out_w"], p["out_w_scale"], s)
    r1 = rel_max(out, a10)
    assert r1 <= tol, f"block output vs out_proj(GPU codes): {r1:.4g}"
    assert np.array_equal(q_gpu, quantize_static(norm_gpu, s)), "a9 codes are not E4M3(norm / s)"
    ng = bf16_to_f64(norm_gpu)
    rms_n = float(np.sqrt(np.mean(ref_norm * ref_norm)))
    r2 = rel_l2(ng, ref_norm)
    assert r2 <= 4e-3, f"gated norm output rel l2 {r2:.4g}"
    dn = np.abs(ng - ref_norm)
    bound_n = 2.0 ** -7 * np.abs(ref_norm) + 0.05 * rms_n
    bad = dn > bound_n
    # the bound is a floor measured over 5e5 elements, and any call may see its tail: at
    # most one element per 1e7 (rounded up) beyond it, none beyond 1.5x
    allowed = -(-dn.size // 10_000_000)
    worst = float(np.max(dn / bound_n)) if dn.size else 0.0
    if int(bad.sum()) > allowed or worst > 1.5:
        w = np.unravel_index(int(np.argmax(dn / bound_n)), dn.shape)
        raise AssertionError(f"{int(bad.sum())} norm outputs beyond the noise bound ({allowed} allowed); worst at "
                             f"{tuple(int(i) for i in w)}: gpu {ng[w]:.5g} oracle {ref_norm[w]:.5g} |d| {dn[w]:.4g} = "
                             f"{dn[w] / bound_n[w]:.3f} x bound (RMS {rms_n:.4g})")
    diff = q_gpu != ref_q
    frac = float(diff.mean())
    assert frac <= 0.01, f"{frac:.4%} of the a9 codes differ from the oracle's"
    if diff.any():
        o = ref_norm[diff]
        eta = 2.0 ** -7 * np.abs(o) + 0.05 * rms_n
        lo = e4m3_decode(quantize_static(bf16_from_f64(o - eta), s))
        hi = e4m3_decode(quantize_static(bf16_from_f64(o + eta), s))
        qv = e4m3_decode(q_gpu[diff])
        ok = (qv >= np.minimum(lo, hi)) & (qv <= np.maximum(lo, hi))
        assert ok.all(), f"{int((~ok).sum())} a9 codes not reachable from the oracle's norm output"
    r3 = rel_max(out, ref_out)
    assert r3 <= e2e_sanity, f"end-to-end {r3:.4g}"
    return dict(out_vs_a10=round(r1, 5), norm_l2=round(r2, 6), code_flips=round(frac, 6), end_to_end=round(r3, 5))

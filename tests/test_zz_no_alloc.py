"""nhm_mixer_decode_noalloc (the decode with the library's per-device scratch instead of a
workspace argument) against nhm_mixer_decode_ex with a caller's workspace: the same kernels
on the same inputs, so outputs, updated state rows and conv windows must match bit for bit.
Two calls in a row, the second with a smaller batch and a bf16 state pool, so the second
runs on scratch the first left full of its own intermediates."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nhm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_w8a8_linear_amd as m
    return m


def test_decode_noalloc_matches_decode_with_workspace(nhm):
    from tests.gpu_util import dev, host, upload_params, zeros_ws
    from workloads import bf16_bits, block_params, conv_pool, hidden, slots, ssm_pool
    p = upload_params(block_params(0, 0))
    S = 40
    for B, bf16_state, extra in ((33, False, 61), (6, True, 62)):
        print(f"noalloc decode: B={B}, bf16 state {bf16_state}", flush=True)
        h = dev(hidden(2, B, extra=extra))
        sl_host = slots(2, B, S)
        sl_host[1] = -1                                        # a padded row
        sl = dev(sl_host)
        sp0 = ssm_pool(2, extra, S)
        sp0 = bf16_bits(sp0) if bf16_state else sp0
        cp0 = conv_pool(2, extra, S)
        results = []
        for noalloc in (False, True):
            sp, cp = dev(sp0), dev(cp0)
            out = torch.full((B, 2688), 0x5555, dtype=torch.int16, device="cuda")
            if noalloc:
                nhm.mixer_decode_noalloc(p, h, sl, sp, cp, out)
            else:
                ws = zeros_ws(nhm.decode_ws_layout(B)["total"])
                nhm.mixer_decode(p, h, sl, sp, cp, out, ws)
            torch.cuda.synchronize()
            results.append((host(out), host(sp), host(cp)))
        (o1, s1, c1), (o2, s2, c2) = results
        assert np.array_equal(o1, o2), "outputs differ"
        assert np.all(o2[1] == 0)                              # the padded row's output is zero
        assert np.array_equal(s1, s2), "updated state pools differ"
        assert np.array_equal(c1, c2), "updated conv pools differ"
        assert not np.array_equal(s2, sp0)                     # the call did advance the state

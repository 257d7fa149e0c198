"""Oracle runs for the large GPU parity tests, one sequence per worker process.

The sequences of a varlen prefill are independent, so the oracle's sequential scan
of a ragged batch splits across processes. Workers are spawned (never forked from a
process that holds the GPU) and import only the oracle and the input generators.
"""
import numpy as np


def prefill_sequence(job):
    """Oracle prefill of one sequence from a zero state through block (workload, layer).

    job: (workload, layer, hidden_bf16 [T, hidden]). Returns the float64 block output,
    the bf16 norm output as float64, the a9 and a1 codes, and the final f32 state and
    bf16 conv window.
    """
    from threadpoolctl import threadpool_limits

    from oracle import GEOMETRY, layout, mixer_prefill
    from workloads import block_params

    workload, layer, h = job
    g = GEOMETRY
    conv_dim = layout(g)["conv_dim"]
    with threadpool_limits(limits=4):        # several workers share the host's cores
        p = block_params(workload, layer)
        T = h.shape[0]
        sp = np.zeros((1, g["n_heads"], g["head_dim"], g["d_state"]), np.float32)
        cp = np.zeros((1, g["conv_width"] - 1, conv_dim), np.uint16)
        out, res = mixer_prefill(p, h, [0, T], [0], [0], sp, cp)
    r = res[0]
    return {"out": out, "norm": r["norm"], "q_out": r["q_out"], "q_in": r["q_in"], "state": sp[0], "window": cp[0]}

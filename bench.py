#!/usr/bin/env python3
"""Mixer throughput on one MI355X: paged decode B=8 through 23 stacked blocks (the
headline line), the same step on bf16 state pools (decode_bf16_state), prefill of one
512-token sequence through one block, and one block of the ragged prefill (8192 + 4096 +
2048 + 1024 tokens).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--copy-probe]

A step is one decode token for each of 8 sequences through all 23 mixer blocks
(nhm_mixer_decode per block, state rows updated in place), replayed as one HIP
graph. Inputs are seeded synthetic tensors already resident in HBM. After all GPU
timing, layers 0 and 1 of one step from their seeded pools are checked against the
oracle (block parity and the updated f32 states); that same oracle run, timed on the
host cores, is the cpu_baseline. Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N_LAYERS, BATCH, SLOTS, HIDDEN, INNER = 23, 8, 64, 2688, 4096
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
WORKLOAD_DECODE = 2          # paged decode B=8, 23 blocks
WORKLOAD_PREFILL = 3         # prefill 512, one block
WORKLOAD_RAGGED = 4          # ragged prefill 8192 + 4096 + 2048 + 1024 tokens, zero initial state


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes_per_layer(B, state_bytes=4):
    """Algorithmic HBM bytes of one decode call: weights + scales + small params once,
    and per sequence the state row read+write (f32, or bf16 with state_bytes=2), the conv
    window read+write and the bf16 block input and output."""
    w = 10304 * 2688 + 2688 * 4096
    scales = 4 * (10304 + 2688 + 2)
    small = 6144 * 4 * 2 + 6144 * 2 + 4096 * 2 + 3 * 64 * 4
    per_seq = 2 * 64 * 64 * 128 * state_bytes + 2 * 3 * 6144 * 2 + 2 * 2688 * 2 + 4
    return w + scales + small + B * per_seq


# HBM bytes one launch of the roofline kernel actually moved, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, per dispatch) of `bench.py --copy-probe`, each scaled by what
# the same counter reads for the 256 MiB device copy of that run. Valid only for the kernel
# sources it was measured on: reported as null once their hash differs.
TRAFFIC = {"sources": ["fp8_w8a8_linear_amd/csrc/gemv.hip", "fp8_w8a8_linear_amd/csrc/nhm_device.h"],
           "sha256": "8dae69b3570025f3b938d1e67ab96b50ed884ab46609e6ec5bc3767951fe8aca",
           "bytes_per_launch": 28289270}


def measured_traffic():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return TRAFFIC["bytes_per_launch"] if h.hexdigest() == TRAFFIC["sha256"] else None


def gemv_bytes(m, n, k):
    """Algorithmic bytes of one W8A8 GEMV: weight + per-channel scales + e4m3 input + bf16 output."""
    return n * k + 4 * n + m * k + 2 * m * n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle parity sample and cpu_baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a 256 MiB device-to-device copy and negation (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the mixer shards by sequence with no "
              "collective, so an N-GPU figure is N independent copies of this one", file=sys.stderr)
        sys.exit(2)
    if args.steps <= 0:
        print("--steps must be positive", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_w8a8_linear_amd as nhm
    from workloads import block_params, conv_pool, hidden, slots, ssm_pool

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        src = torch.randn(64 << 20, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy probe: 3 x (copy_ + neg) of 256 MiB float32 done")
        del src, dst

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    # ------------------------------------------------------------ decode inputs
    t0 = time.time()
    params, host_params, spools, cpools, host_pools = [], [], [], [], {}
    for layer in range(N_LAYERS):
        p = block_params(WORKLOAD_DECODE, layer)
        sp, cp = ssm_pool(WORKLOAD_DECODE, layer, SLOTS), conv_pool(WORKLOAD_DECODE, layer, SLOTS)
        if layer < 2:
            host_params.append(p)
            host_pools[layer] = (sp, cp)
        params.append(nhm.MixerParams(nhm.Fp8Weight(up(p["in_w"]), up(p["in_w_scale"]), up(p["in_a_scale"])),
                                      nhm.Fp8Weight(up(p["out_w"]), up(p["out_w_scale"]), up(p["out_a_scale"])),
                                      up(p["conv_w"]), up(p["conv_b"]), up(p["norm_w"]), up(p["A_log"]),
                                      up(p["D"]), up(p["dt_bias"])))
        spools.append(up(sp))
        cpools.append(up(cp))
        if layer % 6 == 5:
            log(f"generated {layer + 1}/{N_LAYERS} blocks ({time.time() - t0:.0f} s)")
    sl_host = slots(WORKLOAD_DECODE, BATCH, SLOTS)
    x_host = hidden(WORKLOAD_DECODE, BATCH)
    sl = up(sl_host)
    x0 = up(x_host)
    lay = nhm.decode_ws_layout(BATCH)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=dev)
    acts = [x0] + [torch.empty((BATCH, HIDDEN), dtype=torch.int16, device=dev) for _ in range(N_LAYERS)]
    torch.cuda.synchronize()
    log(f"decode inputs resident ({time.time() - t0:.0f} s)")

    def step(stream=None):
        for l in range(N_LAYERS):
            nhm.mixer_decode(params[l], acts[l], sl, spools[l], cpools[l], acts[l + 1], ws, stream=stream)

    # ------------------------------------------------------------ graph capture and timing
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    if not ms_step > 0:
        print("refusing to report a rate over a non-positive window", file=sys.stderr)
        sys.exit(3)
    tok_s = BATCH / (ms_step * 1e-3)
    step_bytes = N_LAYERS * decode_bytes_per_layer(BATCH)
    log(f"decode step {ms_step * 1e3:.1f} us, {tok_s:.0f} tokens/s, step HBM {step_bytes / ms_step / 1e6:.0f} GB/s")

    # ------------------------------------------------------------ dominant kernel: in_proj GEMV, m=8
    s = torch.cuda.current_stream()
    qin = ws[lay["q_in"]:lay["q_in"] + BATCH * HIDDEN].view(BATCH, HIDDEN)
    gout = torch.empty((BATCH, 10304), dtype=torch.int16, device=dev)
    gws = torch.zeros(max(nhm.fp8_linear_workspace_bytes(BATCH, 10304, HIDDEN, nhm.NHM_E4M3), 256),
                      dtype=torch.uint8, device=dev)
    # one launch per layer's weights (890 MB cycle, far above the 256 MB MALL), captured as a
    # graph so the host's launch rate does not pace a ~10 us kernel
    for l in range(N_LAYERS):
        nhm.fp8_linear(qin, params[l].in_proj, out=gout, ws=gws, a_type=nhm.NHM_E4M3)
    torch.cuda.synchronize()
    rg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rg, stream=cap):
        for l in range(N_LAYERS):
            nhm.fp8_linear(qin, params[l].in_proj, out=gout, ws=gws, a_type=nhm.NHM_E4M3)
    for _ in range(3):
        rg.replay()
    torch.cuda.synchronize()
    passes = 20
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(s)
    for _ in range(passes):
        rg.replay()
    g1.record(s)
    torch.cuda.synchronize()
    gemv_us = g0.elapsed_time(g1) * 1e3 / (passes * N_LAYERS)
    gb = gemv_bytes(BATCH, 10304, HIDDEN)
    achieved = gb / (gemv_us * 1e-6) / 1e9
    log(f"in_proj GEMV m=8: {gemv_us:.2f} us/launch, {achieved:.0f} GB/s")

    # ------------------------------------------------------------ decode with a bf16 state pool
    # the same step on bf16 copies of the state pools (rows widened to f32 in the kernel and
    # rounded back on store): half the state bytes
    spools16 = [sp.to(torch.bfloat16).view(torch.int16) for sp in spools]
    torch.cuda.synchronize()

    def step16(stream=None):
        for l in range(N_LAYERS):
            nhm.mixer_decode(params[l], acts[l], sl, spools16[l], cpools[l], acts[l + 1], ws, stream=stream)

    with torch.cuda.stream(cap):
        step16()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph16 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph16, stream=cap):
        step16()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph16.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph16.replay()
    e1.record()
    torch.cuda.synchronize()
    ms16 = e0.elapsed_time(e1) / args.steps
    bytes16 = N_LAYERS * decode_bytes_per_layer(BATCH, state_bytes=2)
    dec16 = {"us_per_step": round(ms16 * 1e3, 1), "tokens_per_s": round(BATCH / (ms16 * 1e-3), 1), "bytes": bytes16,
             "achieved_GBs": round(bytes16 / (ms16 * 1e-3) / 1e9, 1),
             "frac": round(bytes16 / (ms16 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"decode step, bf16 state pools: {dec16}")
    del spools16, graph16

    # ------------------------------------------------------------ prefill 512, one block
    pp = block_params(WORKLOAD_PREFILL, 0)
    ppar = nhm.MixerParams(nhm.Fp8Weight(up(pp["in_w"]), up(pp["in_w_scale"]), up(pp["in_a_scale"])),
                           nhm.Fp8Weight(up(pp["out_w"]), up(pp["out_w_scale"]), up(pp["out_a_scale"])),
                           up(pp["conv_w"]), up(pp["conv_b"]), up(pp["norm_w"]), up(pp["A_log"]), up(pp["D"]),
                           up(pp["dt_bias"]))
    T = 512
    ph = up(hidden(WORKLOAD_PREFILL, T))
    psp, pcp = up(ssm_pool(WORKLOAD_PREFILL, 0, 2)), up(conv_pool(WORKLOAD_PREFILL, 0, 2))
    pcu, psl, phi = up(np.array([0, T], np.int32)), up(np.array([1], np.int32)), up(np.array([1], np.int32))
    pws = torch.zeros(nhm.prefill_ws_layout(T, 1)["total"], dtype=torch.uint8, device=dev)
    pout = torch.empty((T, HIDDEN), dtype=torch.int16, device=dev)

    def pstep():
        nhm.mixer_prefill(ppar, ph, pcu, psl, phi, psp, pcp, pout, pws)

    pg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        pstep()
    torch.cuda.synchronize()
    with torch.cuda.graph(pg, stream=cap):
        pstep()
    for _ in range(5):
        pg.replay()
    torch.cuda.synchronize()
    preps = 50
    e0.record()
    for _ in range(preps):
        pg.replay()
    e1.record()
    torch.cuda.synchronize()
    pre_us = e0.elapsed_time(e1) * 1e3 / preps
    # the two fp8 GEMMs of that block, alone, on the codes the block feeds them: bf16 ~ N(0,1)
    # activations (the block input; the gated norm's output is of the same scale) quantized by
    # the library with the projection's static scale
    from workloads import bf16_bits

    def act_codes(rows, k, w, seed):
        x = up(bf16_bits(np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32)))
        q = nhm.quantize_static(x, w.a_scale)
        torch.cuda.synchronize()
        return q

    gemm = {}
    for name, (n, k) in {"in_proj": (10304, 2688), "out_proj": (2688, 4096)}.items():
        w = ppar.in_proj if name == "in_proj" else ppar.out_proj
        a = act_codes(T, k, w, 7001 + k)
        o = torch.empty((T, n), dtype=torch.int16, device=dev)
        for _ in range(3):
            nhm.fp8_linear(a, w, out=o, a_type=nhm.NHM_E4M3)
        torch.cuda.synchronize()
        g0.record(s)
        for _ in range(50):
            nhm.fp8_linear(a, w, out=o, a_type=nhm.NHM_E4M3)
        g1.record(s)
        torch.cuda.synchronize()
        us = g0.elapsed_time(g1) * 1e3 / 50
        gemm[name] = {"us": round(us, 2), "tflops": round(2 * T * n * k / (us * 1e-6) / 1e12, 1)}
    # the same two projections at the ragged-prefill size (15,360 tokens), where the GEMM has
    # enough arithmetic per weight byte to be bound by the MFMA rather than by operand delivery
    TL = 15360
    gemm_large = {}
    for name, (n, k) in {"in_proj": (10304, 2688), "out_proj": (2688, 4096)}.items():
        w = ppar.in_proj if name == "in_proj" else ppar.out_proj
        a = act_codes(TL, k, w, 7101 + k)
        o = torch.empty((TL, n), dtype=torch.int16, device=dev)
        for _ in range(2):
            nhm.fp8_linear(a, w, out=o, a_type=nhm.NHM_E4M3)
        torch.cuda.synchronize()
        g0.record(s)
        for _ in range(10):
            nhm.fp8_linear(a, w, out=o, a_type=nhm.NHM_E4M3)
        g1.record(s)
        torch.cuda.synchronize()
        us = g0.elapsed_time(g1) * 1e3 / 10
        tf = 2 * TL * n * k / (us * 1e-6) / 1e12
        gemm_large[name] = {"us": round(us, 1), "tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
        del a, o
    log(f"GEMMs at m = {TL}: {gemm_large}")
    # one block of the ragged prefill (4 sequences, 15,360 tokens, zero initial state), replayed
    from workloads import RAGGED_LENGTHS
    rp = block_params(WORKLOAD_RAGGED, 0)
    rpar = nhm.MixerParams(nhm.Fp8Weight(up(rp["in_w"]), up(rp["in_w_scale"]), up(rp["in_a_scale"])),
                           nhm.Fp8Weight(up(rp["out_w"]), up(rp["out_w_scale"]), up(rp["out_a_scale"])),
                           up(rp["conv_w"]), up(rp["conv_b"]), up(rp["norm_w"]), up(rp["A_log"]), up(rp["D"]),
                           up(rp["dt_bias"]))
    rl = list(RAGGED_LENGTHS)
    RT = int(sum(rl))
    rh = up(hidden(WORKLOAD_RAGGED, RT))
    rsp = torch.zeros((8, 64, 64, 128), dtype=torch.float32, device=dev)
    rcp = torch.zeros((8, 3, 6144), dtype=torch.int16, device=dev)
    rcu = up(np.concatenate([[0], np.cumsum(rl)]).astype(np.int32))
    rsl = up(slots(WORKLOAD_RAGGED, len(rl), 8))
    rhi = up(np.zeros(len(rl), np.int32))
    rws = torch.zeros(nhm.prefill_ws_layout(RT, len(rl))["total"], dtype=torch.uint8, device=dev)
    rout = torch.empty((RT, HIDDEN), dtype=torch.int16, device=dev)
    rg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        nhm.mixer_prefill(rpar, rh, rcu, rsl, rhi, rsp, rcp, rout, rws)
    torch.cuda.synchronize()
    with torch.cuda.graph(rg, stream=cap):
        nhm.mixer_prefill(rpar, rh, rcu, rsl, rhi, rsp, rcp, rout, rws)
    for _ in range(2):
        rg.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        rg.replay()
    e1.record()
    torch.cuda.synchronize()
    rag_us = e0.elapsed_time(e1) * 1e3 / 10
    log(f"ragged prefill {rl}: {rag_us:.1f} us/block, {RT / (rag_us * 1e-6):.0f} tokens/s")
    del rh, rws, rout, rsp, rcp
    gemm_us = gemm["in_proj"]["us"] + gemm["out_proj"]["us"]
    gemm_tflops = 2 * T * 38707200 / (gemm_us * 1e-6) / 1e12
    log(f"prefill 512: {pre_us:.1f} us/block, {T / (pre_us * 1e-6):.0f} tokens/s; GEMMs {gemm}")

    # ------------------------------------------------------------ parity sample + cpu baseline
    # after every GPU measurement (the oracle's host threads cannot disturb them); layers 0-1
    # get their initial pools back, so the sample checks one step from the seeded state
    parity, cpu = None, None
    if not args.no_cpu:
        for layer in range(2):
            sp, cp = host_pools[layer]
            spools[layer].copy_(up(sp))
            cpools[layer].copy_(up(cp))
        torch.cuda.synchronize()
        from oracle import mixer_decode as oracle_decode
        from oracle.parity import block_parity, rel_l2
        import threadpoolctl
        parity = {}
        t_layers = []
        x_in = x_host
        for layer in range(2):
            nhm.mixer_decode(params[layer], acts[layer], sl, spools[layer], cpools[layer], acts[layer + 1], ws)
            torch.cuda.synchronize()
            out = acts[layer + 1].cpu().numpy().view(np.uint16)
            wsn = ws.cpu().numpy()
            q = wsn[lay["q_out"]:lay["q_out"] + BATCH * INNER].reshape(BATCH, INNER)
            nrm = wsn[lay["norm"]:lay["norm"] + BATCH * INNER * 2].view(np.uint16).reshape(BATCH, INNER)
            st_gpu = spools[layer].cpu().numpy()
            sp, cp = host_pools[layer]
            spr, cpr = sp.copy(), cp.copy()
            tc = time.perf_counter()
            ref, res = oracle_decode(host_params[layer], x_in, sl_host, spr, cpr)
            t_layers.append(time.perf_counter() - tc)
            st_err = max(rel_l2(st_gpu[s], spr[s]) for s in sl_host)
            assert st_err <= 1e-3, f"layer {layer}: state rel l2 {st_err}"
            entry = {"state_rel_l2_max": float(f"{st_err:.3e}")}
            entry.update(block_parity(out, q, nrm, ref, res["norm"], res["q_out"], host_params[layer]))
            parity[f"layer{layer}"] = entry
            x_in = out
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
        t_layer = float(np.mean(t_layers))
        cpu = {"value": round(BATCH / (N_LAYERS * t_layer), 4), "unit": "tokens/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"oracle decode of layers 0-1 of one B={BATCH} step ({t_layer:.2f} s/layer), scaled to 23 layers"}
        log(f"parity sample ok: {parity}; oracle {t_layer:.2f} s/layer on {cores} threads")

    line = {
        "metric": "Mamba2-mixer tokens/s (decode b=8, prefill 512) + % HBM / fp8-MFMA peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3xe4m3->f32 GEMMs, f32 SSM state, bf16 activations",
        "data": "synthetic (seeded; no checkpoint)",
        "config": {"workload": "paged decode, 8 sequences x 1 token through 23 stacked NemotronH Mamba2 mixer "
                               "blocks (hidden 2688, 64 heads x 64, d_state 128, 8 groups), pool of 64 slots",
                   "global_batch": BATCH, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "decode_step_hbm": {"bytes": step_bytes, "achieved_GBs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                            "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_bf16_state": dec16,
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel (in_proj 10304x2688, m=8)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "us_per_launch": round(gemv_us, 3), "bytes_per_launch": gb},
        "prefill_512": {"tokens_per_s": round(T / (pre_us * 1e-6), 1), "us_per_block": round(pre_us, 1),
                        "gemm": gemm, "gemm_bound": "mfma", "gemm_tflops": round(gemm_tflops, 1),
                        "gemm_frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4)},
        "gemm_m15360": gemm_large,
        "prefill_ragged_15360": {"lengths": rl, "us_per_block": round(rag_us, 1),
                                 "tokens_per_s": round(RT / (rag_us * 1e-6), 1)},
        "parity_sample": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Mixer throughput on one MI355X: paged decode B=8 through 23 stacked blocks (the
headline line), the same step on bf16 state pools (decode_bf16_state), prefill of one
512-token sequence through one block, one block of the ragged prefill (8192 + 4096 +
2048 + 1024 tokens), the W8A8 projections at the prefill sizes and the six-shape linear
sweep.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--copy-probe]

A step is one decode token for each of 8 sequences through all 23 mixer blocks, replayed
as one HIP graph: block 0 quantizes its bf16 input, and every block's out_proj also writes
the codes of its output under the next block's input scale, which the next block takes as
its pre-quantized input (nhm_mixer_decode_q); state rows are updated in place. Inputs are
seeded synthetic tensors already resident in HBM. Every timed figure is the median of at
least five repeats (the headline times exactly K steps, in five consecutive groups whose
median is reported beside it). The library's dispatch counters of one eager decode step and
one prefill call are printed and checked as path-taken evidence. After all GPU timing,
layers 0 and 1 of one step from their seeded pools are checked against the oracle (block
parity and the updated f32 states); that same oracle run, timed on the host, is the
cpu_baseline. Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N_LAYERS, BATCH, SLOTS, HIDDEN, INNER, D_IN_PROJ = 23, 8, 64, 2688, 4096, 10304
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0          # dense e4m3 MFMA
BF16_PEAK_TFLOPS = 2500.0         # dense bf16 MFMA (the exact-sum GEMMs run on it)
WORKLOAD_DECODE = 2          # paged decode B=8, 23 blocks
WORKLOAD_PREFILL = 3         # prefill 512, one block
WORKLOAD_RAGGED = 4          # ragged prefill 8192 + 4096 + 2048 + 1024 tokens, zero initial state
REPEATS = 5


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
           "sha256": "29ea381219b68867df2122ac520e40b26daf89e43e4b2adbee68087df9013864",
           "bytes_per_launch": 28208202}


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


def host_cpu():
    """(logical CPUs of the host, CPUs this process may run on, CPU model)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return os.cpu_count(), affinity, model


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
    from workloads import LINEAR_SHAPES, RAGGED_LENGTHS, bf16_bits, block_params, conv_pool, hidden, slots, ssm_pool

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

    def upload(p):
        return nhm.MixerParams(nhm.Fp8Weight(up(p["in_w"]), up(p["in_w_scale"]), up(p["in_a_scale"])),
                               nhm.Fp8Weight(up(p["out_w"]), up(p["out_w_scale"]), up(p["out_a_scale"])),
                               up(p["conv_w"]), up(p["conv_b"]), up(p["norm_w"]), up(p["A_log"]), up(p["D"]),
                               up(p["dt_bias"]))

    cap = torch.cuda.Stream()   # graphs are captured on this stream and replayed on the current one

    def time_repeats(fn, iters, repeats=REPEATS):
        """Median and all repeats of the per-iteration time (us) of fn(), each repeat timed with
        HIP events on the current stream, where fn's work runs (eager calls and graph replays)."""
        st = torch.cuda.current_stream()
        out = []
        for _ in range(repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for _ in range(iters):
                fn()
            b.record(st)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e3 / iters)
        if not min(out) > 0:
            print("refusing to report a rate over a non-positive window", file=sys.stderr)
            sys.exit(3)
        return float(np.median(out)), [round(x, 2) for x in out]

    def graph_of(fn):
        with torch.cuda.stream(cap):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    # ------------------------------------------------------------ decode inputs
    t0 = time.time()
    params, host_params, spools, cpools, host_pools = [], [], [], [], {}
    for layer in range(N_LAYERS):
        p = block_params(WORKLOAD_DECODE, layer)
        sp, cp = ssm_pool(WORKLOAD_DECODE, layer, SLOTS), conv_pool(WORKLOAD_DECODE, layer, SLOTS)
        if layer < 2:
            host_params.append(p)
            host_pools[layer] = (sp, cp)
        params.append(upload(p))
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
    codes = [None] + [torch.empty((BATCH, HIDDEN), dtype=torch.uint8, device=dev) for _ in range(N_LAYERS - 1)]
    torch.cuda.synchronize()
    log(f"decode inputs resident ({time.time() - t0:.0f} s)")

    def step(pools=None, stream=None):
        """One decode step: block 0 quantizes its bf16 input; each block's out_proj also emits the
        next block's input codes (under that block's in_proj scale)."""
        pools = pools or spools
        for l in range(N_LAYERS):
            nxt = params[l + 1].in_proj.a_scale if l + 1 < N_LAYERS else None
            nhm.mixer_decode_q(params[l], acts[l] if l == 0 else None, sl, pools[l], cpools[l], acts[l + 1], ws,
                               hidden_q=codes[l], out_q=codes[l + 1] if l + 1 < N_LAYERS else None,
                               out_q_scale=nxt, stream=stream)

    # path-taken evidence: the kernels one eager step launches
    torch.cuda.synchronize()
    nhm.dispatch_counters(reset=True)
    step()
    torch.cuda.synchronize()
    decode_path = nhm.dispatch_counters(reset=True)
    want = {"quant_vec8": (1, BATCH), "gemv": (2 * N_LAYERS, 2 * N_LAYERS * BATCH),
            "decode_ssm": (N_LAYERS, N_LAYERS * BATCH)}   # the gated norm runs inside decode_ssm
    assert decode_path == want, f"decode step dispatched {decode_path}, expected {want}"
    log(f"decode step path: {decode_path}")

    # ------------------------------------------------------------ headline: K graph-replayed steps
    graph = graph_of(step)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    groups = REPEATS if args.steps >= REPEATS else 1
    sizes = [args.steps // groups + (1 if i < args.steps % groups else 0) for i in range(groups)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    evs[0].record()
    for gi, n in enumerate(sizes):
        for _ in range(n):
            graph.replay()
        evs[gi + 1].record()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_step = total_ms / args.steps
    if not ms_step > 0:
        print("refusing to report a rate over a non-positive window", file=sys.stderr)
        sys.exit(3)
    group_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 / sizes[i] for i in range(groups)]
    tok_s = BATCH / (ms_step * 1e-3)
    step_bytes = N_LAYERS * decode_bytes_per_layer(BATCH)
    log(f"decode step {ms_step * 1e3:.1f} us (groups {[round(u, 1) for u in group_us]}), {tok_s:.0f} tokens/s, "
        f"step HBM {step_bytes / ms_step / 1e6:.0f} GB/s")

    # ------------------------------------------------------------ dominant kernel: in_proj GEMV, m=8
    qin = codes[1]   # block 1's input codes, as the step feeds them
    gout = torch.empty((BATCH, D_IN_PROJ), dtype=torch.int16, device=dev)
    gws = torch.zeros(max(nhm.fp8_linear_workspace_bytes(BATCH, D_IN_PROJ, HIDDEN, nhm.NHM_E4M3), 256),
                      dtype=torch.uint8, device=dev)

    def gemv_pass():   # one launch per layer's weights (890 MB cycle, far above the 256 MB MALL)
        for l in range(N_LAYERS):
            nhm.fp8_linear(qin, params[l].in_proj, out=gout, ws=gws, a_type=nhm.NHM_E4M3)

    rg = graph_of(gemv_pass)   # captured, so the host's launch rate does not pace a ~10 us kernel
    for _ in range(3):
        rg.replay()
    torch.cuda.synchronize()
    pass_us, pass_all = time_repeats(rg.replay, 4)
    gemv_us = pass_us / N_LAYERS
    gb = gemv_bytes(BATCH, D_IN_PROJ, HIDDEN)
    achieved = gb / (gemv_us * 1e-6) / 1e9
    log(f"in_proj GEMV m=8: {gemv_us:.2f} us/launch (median of {REPEATS}: "
        f"{[round(u / N_LAYERS, 2) for u in pass_all]}), {achieved:.0f} GB/s")
    del rg

    # ------------------------------------------------------------ decode with a bf16 state pool
    # the same step on bf16 copies of the state pools (rows widened to f32 in the kernel and
    # rounded back on store): half the state bytes
    spools16 = [sp.to(torch.bfloat16).view(torch.int16) for sp in spools]
    torch.cuda.synchronize()
    graph16 = graph_of(lambda: step(spools16))
    for _ in range(args.warmup):
        graph16.replay()
    torch.cuda.synchronize()
    us16, all16 = time_repeats(graph16.replay, max(args.steps // REPEATS, 1))
    bytes16 = N_LAYERS * decode_bytes_per_layer(BATCH, state_bytes=2)
    dec16 = {"us_per_step": round(us16, 1), "repeats_us": all16, "tokens_per_s": round(BATCH / (us16 * 1e-6), 1),
             "bytes": bytes16, "achieved_GBs": round(bytes16 / (us16 * 1e-6) / 1e9, 1),
             "frac": round(bytes16 / (us16 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"decode step, bf16 state pools: {dec16}")
    del spools16, graph16, graph

    # ------------------------------------------------------------ prefill 512, one block
    pp = block_params(WORKLOAD_PREFILL, 0)
    ppar = upload(pp)
    T = 512
    ph = up(hidden(WORKLOAD_PREFILL, T))
    psp, pcp = up(ssm_pool(WORKLOAD_PREFILL, 0, 2)), up(conv_pool(WORKLOAD_PREFILL, 0, 2))
    pcu, psl, phi = up(np.array([0, T], np.int32)), up(np.array([1], np.int32)), up(np.array([1], np.int32))
    pws = torch.zeros(nhm.prefill_ws_layout(T, 1)["total"], dtype=torch.uint8, device=dev)
    pout = torch.empty((T, HIDDEN), dtype=torch.int16, device=dev)

    def pstep():
        nhm.mixer_prefill(ppar, ph, pcu, psl, phi, psp, pcp, pout, pws)

    nhm.dispatch_counters(reset=True)
    pstep()
    torch.cuda.synchronize()
    prefill_path = nhm.dispatch_counters(reset=True)
    for k_ in ("quant_vec8", "gemm_ring192x128_exact", "conv_fwd", "ssd_state", "ssd_pass", "ssd_out", "gnorm_quant"):
        assert k_ in prefill_path, f"prefill 512 did not launch {k_}: {prefill_path}"
    assert not any(k_.startswith("gemv") for k_ in prefill_path), prefill_path
    log(f"prefill 512 path: {prefill_path}")
    pg = graph_of(pstep)
    for _ in range(5):
        pg.replay()
    torch.cuda.synchronize()
    pre_us, pre_all = time_repeats(pg.replay, 20)
    del pg

    # the projections of that block, alone, on the codes the block feeds them (bf16 ~ N(0,1)
    # activations quantized by the library with the projection's static scale): in_proj with
    # every product summed in f32, as the block runs it (bf16 MFMA), and both projections on the
    # e4m3 MFMA (nhm_fp8_linear)
    def act_codes(rows, k, w, seed):
        x = up(bf16_bits(np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32)))
        q = nhm.quantize_static(x, w.a_scale)
        torch.cuda.synchronize()
        return q

    def time_linear(m, w, seed, exact, iters):
        a = act_codes(m, w.k, w, seed)
        o = torch.empty((m, w.n), dtype=torch.int16, device=dev)
        wsl = torch.zeros(max(nhm.fp8_linear_workspace_bytes(m, w.n, w.k, nhm.NHM_E4M3), 256), dtype=torch.uint8,
                          device=dev)
        f = lambda: nhm.fp8_linear(a, w, out=o, ws=wsl, a_type=nhm.NHM_E4M3, exact=exact)  # noqa: E731
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        us, all_ = time_repeats(f, iters)
        tf = 2 * m * w.n * w.k / (us * 1e-6) / 1e12
        peak = BF16_PEAK_TFLOPS if exact else FP8_PEAK_TFLOPS
        return {"us": round(us, 2), "repeats_us": all_, "tflops": round(tf, 1),
                "mfma": "bf16 (codes converted exactly, f32 sums)" if exact else "e4m3",
                "frac_peak": round(tf / peak, 4)}

    gemm = {"in_proj": time_linear(T, ppar.in_proj, 7001 + HIDDEN, True, 50),
            "out_proj": time_linear(T, ppar.out_proj, 7001 + INNER, False, 50),
            "in_proj_e4m3": time_linear(T, ppar.in_proj, 7001 + HIDDEN, False, 50)}
    blk_gemm_us = gemm["in_proj"]["us"] + gemm["out_proj"]["us"]
    log(f"prefill 512: {pre_us:.1f} us/block {pre_all}, {T / (pre_us * 1e-6):.0f} tokens/s; GEMMs {gemm}")
    # the same at the ragged-prefill size (15,360 tokens), where the GEMMs have enough arithmetic
    # per weight byte to be bound by the MFMA rather than by operand delivery
    TL = 15360
    gemm_large = {"in_proj": time_linear(TL, ppar.in_proj, 7101 + HIDDEN, True, 3),
                  "out_proj": time_linear(TL, ppar.out_proj, 7101 + INNER, False, 3),
                  "in_proj_e4m3": time_linear(TL, ppar.in_proj, 7101 + HIDDEN, False, 3)}
    log(f"projections at m = {TL}: {gemm_large}")

    # ------------------------------------------------------------ the six-shape W8A8 linear sweep
    sweep = {}
    for (m, n, k) in LINEAR_SHAPES:
        w = ppar.in_proj if (n, k) == (D_IN_PROJ, HIDDEN) else ppar.out_proj if (n, k) == (HIDDEN, INNER) else None
        if w is None:   # the square control
            from workloads import linear_case
            _, wq, wsc, sa = linear_case(m, n, k)
            w = nhm.Fp8Weight(up(wq), up(wsc), up(sa))
        r = time_linear(m, w, 7201 + m + n, False, 50 if m < 4096 else 5)
        byts = gemv_bytes(m, n, k)
        r["GBs"] = round(byts / (r["us"] * 1e-6) / 1e9, 1)
        r["frac_hbm"] = round(r["GBs"] / HBM_PEAK_GBS, 4)
        r["bound"] = "hbm" if 2 * m * n * k / byts < 5e15 / 8e12 else "mfma"
        sweep[f"{m}x{n}x{k}"] = r
    log(f"linear sweep: { {s: (v['us'], v['bound']) for s, v in sweep.items()} }")

    # ------------------------------------------------------------ one block of the ragged prefill
    rp = block_params(WORKLOAD_RAGGED, 0)
    rpar = upload(rp)
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
    # the kernels one eager call launches (has_initial = 0: the call reads none of the pools
    # it writes, so the replays below compute the same block)
    nhm.dispatch_counters(reset=True)
    nhm.mixer_prefill(rpar, rh, rcu, rsl, rhi, rsp, rcp, rout, rws)
    torch.cuda.synchronize()
    ragged_path = nhm.dispatch_counters(reset=True)
    for k_ in ("quant_vec8", "gemm_ring256x256_exact", "gemm_ring256x256", "conv_fwd", "ssd_state", "ssd_pass",
               "ssd_out", "gnorm_quant"):
        assert k_ in ragged_path, f"the ragged prefill did not launch {k_}: {ragged_path}"
    log(f"ragged prefill path: {ragged_path}")
    rgr = graph_of(lambda: nhm.mixer_prefill(rpar, rh, rcu, rsl, rhi, rsp, rcp, rout, rws))
    for _ in range(2):
        rgr.replay()
    torch.cuda.synchronize()
    rag_us, rag_all = time_repeats(rgr.replay, 2)
    log(f"ragged prefill {rl}: {rag_us:.1f} us/block {rag_all}, {RT / (rag_us * 1e-6):.0f} tokens/s")
    del rh, rws, rout, rsp, rcp, rgr

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
        blas_threads = max([i.get("num_threads", 1) for i in info] + [1])
        n_cpu, affinity, model = host_cpu()
        t_layer = float(np.median(t_layers))
        cpu = {"value": round(BATCH / (N_LAYERS * t_layer), 4), "unit": "tokens/s", "cores": int(blas_threads),
               "kind": "oracle", "host_cpus": n_cpu, "cpus_available": affinity, "cpu_model": model,
               "sample": f"oracle decode of layers 0-1 of one B={BATCH} step ({t_layer:.2f} s/layer), scaled to 23 "
                         f"layers; cores = the BLAS threads its float64 matmuls used (the rest is single-threaded)"}
        log(f"parity sample ok: {parity}; oracle {t_layer:.2f} s/layer on {blas_threads} BLAS threads "
            f"({affinity} of {n_cpu} CPUs available, {model})")

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
        "dtype": "e4m3 x e4m3 projections (f32 sums), f32 SSM state, bf16 activations",
        "data": "synthetic (seeded; no checkpoint)",
        "config": {"workload": "paged decode, 8 sequences x 1 token through 23 stacked NemotronH Mamba2 mixer "
                               "blocks (hidden 2688, 64 heads x 64, d_state 128, 8 groups), pool of 64 slots",
                   "global_batch": BATCH, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "decode_step_groups_us": [round(u, 1) for u in group_us],
        "decode_step_median_us": round(float(np.median(group_us)), 1),
        "decode_step_hbm": {"bytes": step_bytes, "achieved_GBs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                            "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_path": decode_path,
        "decode_bf16_state": dec16,
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel (in_proj 10304x2688, m=8)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "us_per_launch": round(gemv_us, 3), "bytes_per_launch": gb,
                     "repeats_us_per_launch": [round(u / N_LAYERS, 3) for u in pass_all]},
        "prefill_512": {"tokens_per_s": round(T / (pre_us * 1e-6), 1), "us_per_block": round(pre_us, 1),
                        "repeats_us": pre_all, "path": prefill_path, "gemm": gemm,
                        "gemm_us": round(blk_gemm_us, 2),
                        "gemm_frac_of_block": round(blk_gemm_us / pre_us, 3)},
        "gemm_m15360": gemm_large,
        "linear_sweep": sweep,
        "prefill_ragged_15360": {"lengths": rl, "us_per_block": round(rag_us, 1), "repeats_us": rag_all,
                                 "tokens_per_s": round(RT / (rag_us * 1e-6), 1), "path": ragged_path},
        "parity_sample": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

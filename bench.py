#!/usr/bin/env python3
"""Throughput of the MoE gate_up hot path on one MI355X.

One step = one pass of the whole path over one batch of tokens of a routed-
expert gate_up layer (Gemma 4 26B-A4B shapes: hidden 2048, 128 experts,
top-8, 2 x 768 gate_up rows per expert):
    moe_route_permute_rotate -> moe_gateup_i8h_grouped (act out)
(the routing kernel rotates the activation rows of the tokens it routes).
For a few tokens everything runs as one launch (moe_route_gateup_i8h_decode);
for the FP8 block variant the step is moe_route_permute -> moe_gateup_fp8blk_grouped,
for the W8A8 int8 g128 form (workload w8a8, prefill sizes) moe_route_permute ->
moe_gateup_i8g_grouped.

Default workload: one decode token (T = 1). Inputs are seeded synthetic data
already resident in HBM; every step takes a different token (router logits
and activations) and a different copy of the layer's weights, so the touched
experts stream from HBM rather than from the 256 MB last-level cache. The
steps are captured in a HIP graph and replayed; the timed region is bracketed
by device synchronisations.

Printed: one JSON line with the step throughput (weight GB/s: bytes of the
touched experts' codes and scales per second), tokens/s, the roofline of the
dominant kernel (gate_up) timed with HIP events over graph replays of that
kernel alone, and the CPU oracle timed on a bounded sample of the same steps
(one thread, then every thread; the CPU model is recorded). The decode step
is the headline; the verify (T = 128) and prefill (T = 2048) steps are
measured in the same run and reported under "rows", each with its own
roofline (HBM, and the bf16 MFMA fraction). Each line (the headline and
every row) runs exactly --warmup untimed steps, then times exactly --steps
steps between device synchronisations: whole graphs of the step cycle, then
a graph of the remaining steps. The kernel-alone timings behind the
rooflines replay graphs for at least --min-ms. A plain HBM read probe
(libi8h_probe.so) runs first, and every roofline is also given as a fraction
of what it reaches on the same GPU.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

METRIC = "weight GB/s and tokens/s, MoE gate_up at M=1/128/2048; % HBM / MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512, help="timed steps of each line (exactly)")
    ap.add_argument("--warmup", type=int, default=64, help="untimed steps before them (exactly)")
    ap.add_argument("--min-ms", type=float, default=20.0,
                    help="least length of each kernel-alone timing (the rooflines' graph replays)")
    ap.add_argument("--workload", default="decode", choices=["decode", "verify", "prefill", "fp8", "w8a8"])
    ap.add_argument("--rows", default="auto",
                    help="comma list of further workloads measured in the same run and reported under 'rows' "
                         "(auto: verify,prefill for the decode headline, none otherwise; 'none': skip)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies cycled (0: enough to defeat caches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of each CPU oracle sample (one thread, then all threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the live HBM read-bandwidth probe")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm", "tall", "skinny"])
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 4 times (the reference kernel "
                         "whose FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic figures)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the HBM read-bandwidth probe (streaming and one-shot decode-sized reads) "
                         "and print its JSON line")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="only run the MFMA / VALU overlap probe (time per MFMA with N FMAs beside it, one and "
                         "two waves a SIMD) and print its JSON line")
    ap.add_argument("--two-launch", action="store_true",
                    help="decode: time moe_route_permute + moe_gateup_i8h_grouped_fused instead of the "
                         "one-launch moe_route_gateup_i8h_decode")
    ap.add_argument("--unfused", action="store_true",
                    help="rotate with hadamard128_rotate as a call of its own, then moe_gateup_i8h_grouped "
                         "(defaults: decode rotates inside the gate_up kernel, many tokens inside the routing "
                         "kernel, moe_route_permute_rotate)")
    ap.add_argument("--act-f32", action="store_true",
                    help="--stage down: float32 act rows, rounded to bf16 inside the call (default: bf16 rows, "
                         "as the gate_up calls' bf16 form hands them over)")
    ap.add_argument("--stage", default="gate_up", choices=["gate_up", "down", "linear"],
                    help="down: time the step after the path instead, moe_down_bf16_combine (bf16 grouped down "
                         "projection + weighted combine) on the workload's token count, with the routing "
                         "computed beforehand and synthetic float32 act rows; linear: the drafter's dense int8 "
                         "linear with f16 group scales (linear_i8f16) on its stand-in shape, 16 tokens x "
                         "K 2048 -> N 4096 (--workload is ignored)")
    return ap.parse_args()


def capture_graph(fn, S, dev):
    """fn(0..S-1) once eagerly on a side stream, then captured into one graph."""
    import torch
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(S):
            fn(i)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            fn(i)
    torch.cuda.synchronize(dev)
    return g


def timed_replays(g, S, args, dev, step):
    """Exactly args.warmup untimed steps, then exactly args.steps timed steps,
    bracketed by device synchronisations: whole replays of g (the cycle of S
    steps), then a graph of the remaining steps (steps 0 .. r - 1 of the
    cycle, captured beforehand from step). Returns (steps, warmup steps, wall
    seconds of the timed region, per-step ms from HIP events on the replay
    stream)."""
    import torch
    K, W = max(1, args.steps), max(0, args.warmup)
    tail_k = capture_graph(step, K % S, dev) if K % S else None
    tail_w = capture_graph(step, W % S, dev) if W % S else None
    for _ in range(W // S):
        g.replay()
    if tail_w is not None:
        tail_w.replay()
    st = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0.record(st)
    for _ in range(K // S):
        g.replay()
    if tail_k is not None:
        tail_k.replay()
    ev1.record(st)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    return K, W, wall, ev0.elapsed_time(ev1) / K


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the hot path is measured on one GPU; --gpus must be 1 "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_hadamard_domain_amd as i8h

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe > 0:
        a = torch.ones(args.copy_probe, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "copies": 4}))
        return
    if args.read_probe:
        print(json.dumps({"read_probe": read_probe(dev)}))
        return
    if args.overlap_probe:
        print(json.dumps({"overlap_probe": overlap_probe(dev)}))
        return
    i8h.lib()

    if args.stage == "down":
        bench_down(args, synth_layer(args.workload), dev)
        return
    if args.stage == "linear":
        bench_linear(args, dev)
        return

    probe = None if args.no_probe else read_probe(dev)
    head = measure_gate_up(args, args.workload, dev, probe, keep_inputs=not args.no_cpu_baseline)
    if args.rows == "auto":
        extra = ["verify", "prefill"] if args.workload == "decode" else []
    elif args.rows in ("", "none"):
        extra = []
    else:
        extra = [w for w in args.rows.split(",") if w]
    rows = {}
    for name in extra:
        torch.cuda.empty_cache()
        r = measure_gate_up(args, name, dev, probe, keep_inputs=False)
        r.pop("_cpu", None)
        rows[name] = r
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(*head.pop("_cpu"), args.cpu_seconds)
    head.pop("_cpu", None)
    out = {"metric": METRIC}
    out.update(head)
    out["cpu_baseline"] = cpu
    if rows:
        out["rows"] = rows
    if probe is not None:
        out["read_probe"] = probe
    print(json.dumps(out))


def synth_layer(name):
    import synth
    return synth.layer(name)


MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_I8_PEAK_TOPS = 5000.0


def measure_gate_up(args, name, dev, probe, keep_inputs):
    """One workload of the path: its step captured in HIP graphs and replayed.
    Returns the bench line's fields for it (value, steps, roofline ...)."""
    import torch
    import int8_hadamard_domain_amd as i8h
    import synth

    L = synth.layer(name)
    fp8 = name == "fp8"
    w8 = name == "w8a8"
    fused = (not fp8) and (not w8) and (not args.unfused) and args.path == "auto" and L.T <= 8
    one_launch = fused and not args.two_launch and L.P <= 64 and L.E <= 256 and L.K <= 4096
    per_copy_bytes = L.E * L.N * L.K * (1 + (2 / (128 * 128) if fp8 else 2 / 128))
    if args.copies > 0:
        copies = args.copies
    else:
        # keep several hundred MB between reuses of any copy
        touched = min(L.E, L.P) / L.E * per_copy_bytes
        copies = int(min(16, max(2, np.ceil(1.6e9 / max(touched, 1)))))
    # distinct token batches cycled by the steps
    nb = 64 if L.T == 1 else (8 if L.T <= 128 else 4)
    S = nb * copies // np.gcd(nb, copies)          # steps per captured graph: every (batch, copy) pair
    while S > 256:
        S //= 2

    t_setup = time.perf_counter()
    LB = synth.layer(name, T=L.T * nb)
    logits_np = synth.router_logits(LB).reshape(nb, L.T, L.E)
    x_np = synth.activations_bf16(LB).reshape(nb, L.T, L.K)
    if fp8:
        codes_np, sbits_np = synth.synthetic_fp8(L)
    else:
        codes_np, sbits_np = synth.synthetic_i8h(L)
    codes0 = torch.from_numpy(codes_np).to(dev)
    scales0 = torch.from_numpy(sbits_np.view(np.int16)).view(torch.bfloat16).to(dev)
    codes = [codes0] + [codes0.clone() for _ in range(copies - 1)]
    scales = [scales0] + [scales0.clone() for _ in range(copies - 1)]
    logits = torch.from_numpy(logits_np).to(dev)
    xs = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)

    k = L.topk
    route_bufs = [dict() for _ in range(S)]
    for b in route_bufs:
        b["topk_ids"] = torch.empty((L.T, k), dtype=torch.int32, device=dev)
        b["topk_w"] = torch.empty((L.T, k), dtype=torch.float32, device=dev)
        b["expert_off"] = torch.empty((L.E + 1,), dtype=torch.int32, device=dev)
        b["sorted_pairs"] = torch.empty((L.P,), dtype=torch.int32, device=dev)
        b["pair_pos"] = torch.empty((L.P,), dtype=torch.int32, device=dev)
        ws = i8h.lib().moe_route_permute_workspace_size(L.T, L.E, k)
        b["workspace"] = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    xr = torch.empty((L.T, L.K), dtype=torch.bfloat16, device=dev)
    act = torch.empty((L.P, L.N // 2), dtype=torch.float32, device=dev)
    fp8_ws = torch.empty((max(i8h.lib().moe_gateup_fp8blk_workspace_size(L.T, L.K), 1),),
                         dtype=torch.uint8, device=dev)
    i8g_ws = torch.empty((max(i8h.lib().moe_gateup_i8g_workspace_size(L.T, L.K), 1),),
                         dtype=torch.uint8, device=dev)
    fused_ws = torch.empty((max(i8h.lib().moe_gateup_i8h_fused_workspace_size(L.T, L.K), 1),),
                           dtype=torch.uint8, device=dev)

    def gate_up(i):
        b = route_bufs[i]
        c = i % copies
        if one_launch:
            i8h.moe_route_gateup_i8h_decode(logits[i % nb], xs[i % nb], codes[c], scales[c], k, gate_up=False,
                                            act=act, out=b)
        elif fp8:
            i8h.moe_gateup_fp8blk_grouped(xs[i % nb], codes[c], scales[c], k, b["expert_off"], b["sorted_pairs"],
                                          gate_up=False, act=act, workspace=fp8_ws, path=args.path)
        elif w8:
            i8h.moe_gateup_i8g_grouped(xs[i % nb], codes[c], scales[c], k, b["expert_off"], b["sorted_pairs"],
                                       gate_up=False, act=act, workspace=i8g_ws)
        elif fused:
            i8h.moe_gateup_i8h_grouped_fused(xs[i % nb], codes[c], scales[c], k, b["expert_off"],
                                             b["sorted_pairs"], gate_up=False, act=act, workspace=fused_ws)
        else:
            i8h.moe_gateup_i8h_grouped(xr, codes[c], scales[c], k, b["expert_off"], b["sorted_pairs"],
                                       gate_up=False, act=act, path=args.path)

    def step(i):
        if one_launch:           # routing is inside the kernel
            gate_up(i)
            return
        if not fp8 and not w8 and not fused:
            if args.unfused:     # the rotation as a call of its own
                i8h.moe_route_permute(logits[i % nb], k, out=route_bufs[i])
                i8h.hadamard128_rotate(xs[i % nb], out=xr)
            else:                # the routing kernel rotates the rows it routes
                i8h.moe_route_permute_rotate(logits[i % nb], xs[i % nb], k, out=route_bufs[i], x_rot=xr)
        else:
            i8h.moe_route_permute(logits[i % nb], k, out=route_bufs[i])
        gate_up(i)

    g_step = capture_graph(step, S, dev)
    # touched experts of every captured step (bookkeeping only, outside the timed region)
    touched = []
    for i in range(S):
        off = route_bufs[i]["expert_off"].cpu().numpy()
        touched.append(int(np.count_nonzero(np.diff(off))))
    setup_s = time.perf_counter() - t_setup

    bytes_per_expert = L.N * L.K + (L.N // 128) * L.G * 2 if fp8 else L.N * L.K + L.N * L.G * 2
    weight_bytes = np.array(touched, dtype=np.float64) * bytes_per_expert   # per step in the graph

    steps, warm, wall, step_ms_ev = timed_replays(g_step, S, args, dev, step)
    ms_per_step = wall / steps * 1e3
    value = weight_bytes.mean() * steps / wall / 1e9
    tokens_per_s = L.T * steps / wall

    # ---- dominant kernel: gate_up alone, HIP events around graph replays ----
    g_gu = capture_graph(gate_up, S, dev)
    reps = max(2, int(np.ceil(args.min_ms * 1e-3 / max(ms_per_step * 1e-3 * S, 1e-7))))
    for _ in range(2):
        g_gu.replay()
    st = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    ev0.record(st)
    for _ in range(reps):
        g_gu.replay()
    ev1.record(st)
    torch.cuda.synchronize(dev)
    kern_us = ev0.elapsed_time(ev1) * 1e3 / (reps * S)
    del g_gu, g_step
    # algorithmic bytes per launch: touched codes + scales, activations read once,
    # act written, routing lists read
    x_bytes = L.T * L.K * (1 if fp8 else 2)
    alg_bytes = weight_bytes.mean() + x_bytes + L.P * (L.N // 2) * 4 + L.P * 4 + (L.E + 1) * 4
    if one_launch:
        # the kernel also reads the logits and writes ids, weights and pair_pos
        alg_bytes += L.T * L.E * 4 + 3 * L.P * 4
    if fp8 or w8:
        alg_bytes += L.T * L.K * 2 + L.T * L.G * 4       # quantizer reads bf16 x, writes scales
    achieved = alg_bytes / (kern_us * 1e-6) / 1e9
    flops = 2.0 * L.P * L.N * L.K
    if one_launch:
        kernel_name, key = "k_route_gateup_decode (routing + rotation + gate_up)", "route_gateup_decode"
    elif w8:
        kernel_name, key = "k_gateup_i8g (+ k_i8_act_quant)", "i8g"
    elif fp8 and (args.path == "gemm" or (args.path == "auto" and L.P >= 32 * L.E)):
        kernel_name, key = "k_gateup_gemm<E4M3> (+ k_fp8_act_quant)", "gemm_e4m3"
    elif fp8:
        kernel_name, key = "k_gateup_fp8_skinny (+ k_fp8_act_quant)", "skinny_e4m3"
    elif args.path == "gemv" or (args.path == "auto" and L.T <= 8):
        kernel_name = "k_gateup_i8h_gemv" + ("<rotation fused>" if fused else "")
        key = "gemv_rot" if fused else "gemv"
    elif args.path == "tall" or (args.path == "auto" and L.P >= 32 * L.E):
        kernel_name, key = "k_gateup_gemm_tall (int8, 256-pair passes)", "gemm_tall"
    elif args.path == "gemm":
        kernel_name, key = "k_gateup_gemm<I8>", "gemm_i8"
    else:
        kernel_name, key = "k_gateup_i8h_skinny (int8, 64-pair passes)", "skinny"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(key, name),
                "kernel": kernel_name, "kernel_us": round(kern_us, 3), "alg_bytes_per_launch": int(alg_bytes)}
    if probe is not None:
        # against what a plain read reaches on this GPU: a one-shot read of the decode step's size for
        # the decode kernels, the sustained streaming rate for the others
        ref = probe["oneshot"]["gbs"] if L.T <= 8 else probe["stream"]["gbs"]
        roofline["probe_gbs"] = ref
        roofline["frac_of_probe"] = round(achieved / ref, 4)
    if w8:
        tops = flops / (kern_us * 1e-6) / 1e12
        roofline["mfma"] = {"achieved": round(tops, 1), "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s (int8)",
                            "frac": round(tops / MFMA_I8_PEAK_TOPS, 4)}
    else:
        tf = flops / (kern_us * 1e-6) / 1e12
        roofline["mfma"] = {"achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s (bf16)",
                            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}

    row = {
        "value": round(value, 2),
        "unit": "GB/s",
        "tokens_per_s": round(tokens_per_s, 1),
        "n_gpus": 1,
        "steps": int(steps),
        "warmup": int(warm),
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_events": round(step_ms_ev, 5),
        "timed_region_ms": round(wall * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3*bf16(exact)->f32" if fp8 else "i8*i8->i32->f32" if w8 else "i8*bf16->f32",
        "data": "synthetic",
        "config": {"workload": f"{name}: T={L.T} K={L.K} E={L.E} top-{k} N={L.N} (gate_up of Gemma 4 26B-A4B)",
                   "T": L.T, "K": L.K, "E": L.E, "topk": k, "N": L.N, "weight_copies": int(copies),
                   "steps_per_graph": int(S), "touched_experts_per_step": float(np.mean(touched)),
                   "steps_requested": int(args.steps), "warmup_requested": int(args.warmup),
                   "outputs": "act (fp32); gate_up not stored", "setup_s": round(setup_s, 1),
                   "step": ("route -> rotate -> gate_up in one launch" if one_launch else
                            "route -> gate_up (FP8 quantizer + product)" if fp8 else
                            "route -> gate_up (int8 activation quantizer + int8 product)" if w8 else
                            "route -> gate_up with the rotation fused" if fused else
                            "route -> rotate -> gate_up" if args.unfused else
                            "route + rotate (one kernel) -> gate_up")},
        "roofline": roofline,
    }
    if keep_inputs:
        row["_cpu"] = (L, nb, logits_np, x_np, codes_np, sbits_np, "fp8" if fp8 else "i8g" if w8 else "i8h",
                       bytes_per_expert)
    del codes, scales, codes0, scales0
    return row


def read_probe(dev):
    """HBM read bandwidth on this GPU with the plainest read kernel
    (libi8h_probe.so): a sustained stream over 2 GiB, and one-shot reads of
    the decode step's touched bytes (8 experts' codes and scales, 25.56 MB),
    16 buffers cycled in a graph of 64 launches so no read finds its buffer in
    the 256 MB last-level cache. Several grid sizes; the best of each."""
    import ctypes
    import torch
    here = os.path.dirname(os.path.abspath(__file__))
    P = ctypes.CDLL(os.path.join(here, "int8_hadamard_domain_amd", "lib", "libi8h_probe.so"))
    P.i8h_read_probe.restype = ctypes.c_int
    P.i8h_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32,
                                 ctypes.c_void_p, ctypes.c_void_p]
    key = 0x9E3779B9
    max_blocks = 65536
    sink = torch.zeros(max_blocks * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)

    def launch(buf, nbytes, blocks):
        # on the stream current at the call (the capturing one inside a graph capture)
        cur = torch.cuda.current_stream(dev).cuda_stream
        rc = P.i8h_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, key, ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(cur))
        if rc != 0:
            raise RuntimeError(f"i8h_read_probe failed ({rc})")

    def time_graph(fn, n_launch, reps):
        g = capture_graph(fn, n_launch, dev)
        for _ in range(2):
            g.replay()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        ev0.record(st)
        for _ in range(reps):
            g.replay()
        ev1.record(st)
        torch.cuda.synchronize(dev)
        return ev0.elapsed_time(ev1) * 1e-3 / (reps * n_launch)

    out = {}
    big = 2 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device=dev)
    best = None
    for per_thread in (8, 32, 128):
        blocks = min(max_blocks, -(-big // (16 * 256 * per_thread)))
        t = time_graph(lambda i: launch(buf, big, blocks), 4, 3)
        if best is None or t < best[0]:
            best = (t, blocks)
    out["stream"] = {"bytes": big, "us": round(best[0] * 1e6, 2), "gbs": round(big / best[0] / 1e9, 1),
                     "blocks": best[1], "frac_of_peak": round(big / best[0] / 1e9 / HBM_PEAK_GBS, 4)}
    del buf
    one = 8 * (1536 * 2048 + 1536 * 16 * 2)        # the decode step's touched weight bytes
    bufs = [torch.ones(one // 4, dtype=torch.int32, device=dev) for _ in range(16)]
    best = None
    for per_thread in (8, 16, 32):
        blocks = -(-one // (16 * 256 * per_thread))
        t = time_graph(lambda i: launch(bufs[i % 16], one, blocks), 64, 8)
        if best is None or t < best[0]:
            best = (t, blocks)
    out["oneshot"] = {"bytes": one, "us": round(best[0] * 1e6, 3), "gbs": round(one / best[0] / 1e9, 1),
                      "blocks": best[1], "frac_of_peak": round(one / best[0] / 1e9 / HBM_PEAK_GBS, 4),
                      "note": "per launch inside a graph of 64, 16 buffers cycled"}
    del bufs, sink
    torch.cuda.empty_cache()
    return out


def overlap_probe(dev):
    """How much VALU work hides under the MFMAs (libi8h_probe.so): a workgroup
    per CU, one or two waves a SIMD, four independent 32x32x16 bf16 MFMA
    chains a wave with N independent float FMAs after each MFMA. Per N: the
    time per MFMA and wave (best of 3 launches after one untimed), also in
    clocks at the nominal 2.4 GHz."""
    import ctypes
    import torch
    here = os.path.dirname(os.path.abspath(__file__))
    P = ctypes.CDLL(os.path.join(here, "int8_hadamard_domain_amd", "lib", "libi8h_probe.so"))
    P.i8h_overlap_probe.restype = ctypes.c_int
    P.i8h_overlap_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 20000
    out_buf = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev)
    res = {"cus": cus, "iters": iters, "mfma": "v_mfma_f32_32x32x16_bf16, 4 chains a wave", "valu": "v_fma_f32"}
    for threads in (256, 512):
        rows = {}
        for n in (0, 2, 4, 6, 8, 12, 16):
            best = None
            for rep in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                rc = P.i8h_overlap_probe(n, threads, cus, iters, ctypes.c_void_p(out_buf.data_ptr()),
                                         ctypes.c_void_p(st.cuda_stream))
                e1.record(st)
                if rc != 0:
                    raise RuntimeError(f"i8h_overlap_probe failed ({rc})")
                torch.cuda.synchronize(dev)
                if rep > 0:
                    t = e0.elapsed_time(e1) * 1e-3 / (4 * iters)
                    best = t if best is None else min(best, t)
            rows[str(n)] = {"ns_per_mfma": round(best * 1e9, 2), "clk_2p4ghz": round(best * 2.4e9, 1)}
        res[f"waves_per_simd_{threads // 256}"] = rows
    del out_buf
    return res


# device-code sources of each timed kernel: a traffic figure holds only for the sources it was
# measured on (launch.hpp only declares host launchers and is left out)
KERNEL_SOURCES = {
    "route_gateup_decode": ["gateup_i8h_gemv.hip", "topk.hpp", "xlane.hpp", "common.hpp"],
    "gemv": ["gateup_i8h_gemv.hip", "topk.hpp", "xlane.hpp", "common.hpp"],
    "gemv_rot": ["gateup_i8h_gemv.hip", "topk.hpp", "xlane.hpp", "common.hpp"],
    "gemm_i8": ["gateup_gemm.hip", "common.hpp"],
    "gemm_tall": ["gateup_gemm.hip", "common.hpp"],
    "gemm_e4m3": ["gateup_gemm.hip", "gateup_fp8.hip", "xlane.hpp", "common.hpp"],
    "down_gemv": ["down.hip", "xlane.hpp", "common.hpp"],
    "down_gemm": ["down.hip", "xlane.hpp", "common.hpp"],
    "linear": ["linear.hip", "common.hpp"],
    "skinny": ["gateup_skinny.hip", "common.hpp"],
    "skinny_e4m3": ["gateup_skinny.hip", "gateup_fp8.hip", "common.hpp"],
    "i8g": ["gateup_i8g.hip", "xlane.hpp", "common.hpp"],
}


def measured_traffic(key, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled) from profiles/hbm_traffic.txt, or None
    when there is no line for this kernel and workload or its sources changed since."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "int8_hadamard_domain_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    try:
        with open(os.path.join(here, "profiles", "hbm_traffic.txt")) as fh:
            for line in fh:
                f = line.split()
                if len(f) == 5 and not line.startswith("#") and f[0] == key and f[1] == workload and f[2] == sha:
                    return int(f[3]) + int(f[4])
    except OSError:
        pass
    return None


def bench_down(args, L, dev):
    """The step after the path on the workload's shapes: out[T, H] from the
    expert-sorted act rows [P, I] and W_down [E, H, I] bf16 (H = K). The act
    rows come in bf16, as the gate_up calls hand them over in their bf16 form
    (--act-f32: float32 rows, rounded inside the call)."""
    import torch
    import int8_hadamard_domain_amd as i8h
    import synth

    k, H, I = L.topk, L.K, L.I
    per_copy = L.E * H * I * 2
    copies = args.copies if args.copies > 0 else int(min(16, max(2, np.ceil(
        1.6e9 / max(min(L.E, L.P) / L.E * per_copy, 1)))))
    nb = 64 if L.T == 1 else (8 if L.T <= 128 else 4)
    S = nb * copies // np.gcd(nb, copies)
    while S > 256:
        S //= 2

    t_setup = time.perf_counter()
    LB = synth.layer(L.name, T=L.T * nb)
    logits_np = synth.router_logits(LB).reshape(nb, L.T, L.E)
    w_np = synth.down_weights_bf16(L)
    w0 = torch.from_numpy(w_np.view(np.int16)).view(torch.bfloat16).to(dev)
    ws_ = [w0] + [w0.clone() for _ in range(copies - 1)]
    act_np = synth.act_f32(LB).reshape(nb, L.P, I)
    acts = torch.from_numpy(act_np).to(dev)
    act16 = not args.act_f32
    if act16:
        acts = acts.to(torch.bfloat16)
    routes = [i8h.moe_route_permute(torch.from_numpy(logits_np[b]).to(dev), k) for b in range(nb)]
    out = torch.empty((L.T, H), dtype=torch.float32, device=dev)
    wsz = (i8h.lib().moe_down_bf16_act_bf16_workspace_size if act16 else
           i8h.lib().moe_down_bf16_workspace_size)(L.T, I, H, k)
    work = torch.empty((max(wsz, 1),), dtype=torch.uint8, device=dev)
    gemv = L.P <= 64

    def step(i):
        i8h.moe_down_bf16_combine(acts[i % nb], ws_[i % copies], routes[i % nb], out=out, workspace=work)

    g = capture_graph(step, S, dev)
    touched = [int(np.count_nonzero(np.diff(routes[i % nb]["expert_off"].cpu().numpy()))) for i in range(S)]
    setup_s = time.perf_counter() - t_setup
    wbytes = np.array(touched, dtype=np.float64) * H * I * 2

    steps, warm, wall, step_ms_ev = timed_replays(g, S, args, dev, step)
    call_us = step_ms_ev * 1e3
    value = wbytes.mean() * steps / wall / 1e9
    # algorithmic bytes per call: touched W_down, act read once, out written, routing lists
    alg = wbytes.mean() + L.P * I * (2 if act16 else 4) + L.T * H * 4 + L.P * 4 * 3 + (L.E + 1) * 4
    achieved = alg / (call_us * 1e-6) / 1e9
    flops = 2.0 * L.P * H * I
    key = "down_gemv" if gemv else "down_gemm"
    kernel = ("k_down_gemv_combine (one launch)" if gemv else
              "k_down_gemm + k_down_combine (the call)" if act16 else
              "k_f32_to_bf16 + k_down_gemm + k_down_combine (the call)")
    workload = "down-" + L.name + ("" if act16 else "-f32act")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(key, workload),
                "kernel": kernel, "kernel_us": round(call_us, 3), "alg_bytes_per_launch": int(alg),
                "mfma_tflops": round(flops / (call_us * 1e-6) / 1e12, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import down, router
        try:
            import threadpoolctl
            cores = max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] + [1])
        except Exception:
            cores = 1
        wf = synth.bf16_bits_to_f64(w_np)
        done, wb, tok = 0, 0.0, 0
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < args.cpu_seconds or done == 0:   # cycles through the batches
            r = router.route(logits_np[done % nb], k)
            down.down_combine(act_np[done % nb], wf, r["expert_off"], r["pair_pos"], r["weights"], k)
            wb += np.count_nonzero(np.diff(r["expert_off"])) * H * I * 2
            tok += L.T
            done += 1
        el = time.perf_counter() - c0
        cpu = {"value": round(wb / el / 1e9, 4), "unit": "GB/s", "tokens_per_s": round(tok / el, 3),
               "cores": int(cores), "kind": "oracle",
               "sample": f"{done} step(s) of the same workload (route + down projection + combine, fp64 "
                         f"NumPy), {el:.1f} s"}

    print(json.dumps({
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "tokens_per_s": round(L.T * steps / wall, 1),
        "n_gpus": 1,
        "steps": int(steps),
        "warmup": int(warm),
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16*bf16->f32",
        "data": "synthetic",
        "config": {"workload": f"{workload}: T={L.T} H={H} I={I} E={L.E} top-{k} (down projection + "
                               f"combine of Gemma 4 26B-A4B)",
                   "T": L.T, "H": H, "I": I, "E": L.E, "topk": k, "weight_copies": int(copies),
                   "steps_per_graph": int(S), "touched_experts_per_step": float(np.mean(touched)),
                   "setup_s": round(setup_s, 1),
                   "act": "bf16" if act16 else "float32",
                   "step": "moe_down_bf16_combine (" + ("one launch" if gemv else "GEMM, combine" if act16 else
                                                       "bf16 act, GEMM, combine") + ")"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }))


def bench_linear(args, dev):
    """The drafter's dense int8 linear with f16 group scales on its stand-in
    shape (16 tokens, K 2048, N 4096); weight copies cycled past the caches."""
    import torch
    import int8_hadamard_domain_amd as i8h
    import synth

    d = synth.DRAFTER
    T, K, N = d["T"], d["K"], d["N"]
    wbytes = N * K + N * (K // 128) * 2
    copies = args.copies if args.copies > 0 else int(min(256, max(2, np.ceil(1.6e9 / wbytes))))
    S = copies
    t_setup = time.perf_counter()
    q_np, s_np = synth.synthetic_i8f16(N, K, d["seed"])
    x_np = synth.drafter_activations_bf16(T, K, d["seed"])
    q0 = torch.from_numpy(q_np).to(dev)
    s0 = torch.from_numpy(s_np.view(np.int16)).view(torch.float16).to(dev)
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)

    def step(i):
        i8h.linear_i8f16(x, qs[i % copies], ss[i % copies], out=y)

    g = capture_graph(step, S, dev)
    setup_s = time.perf_counter() - t_setup
    steps, warm, wall, step_ms_ev = timed_replays(g, S, args, dev, step)
    call_us = step_ms_ev * 1e3
    alg = wbytes + T * K * 2 + T * N * 4
    achieved = alg / (call_us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import dense, numfmt
        try:
            import threadpoolctl
            cores = max([dd.get("num_threads", 1) for dd in threadpoolctl.threadpool_info()] + [1])
        except Exception:
            cores = 1
        xf, sf = synth.bf16_bits_to_f64(x_np), numfmt.f16_from_bits(s_np)
        done = 0
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < args.cpu_seconds or done == 0:
            dense.linear_i8_f16(xf, q_np, sf)
            done += 1
        el = time.perf_counter() - c0
        cpu = {"value": round(done * wbytes / el / 1e9, 4), "unit": "GB/s", "tokens_per_s": round(done * T / el, 3),
               "cores": int(cores), "kind": "oracle",
               "sample": f"{done} call(s) of the same linear (fp64 NumPy), {el:.1f} s"}
    print(json.dumps({
        "metric": METRIC,
        "value": round(wbytes * steps / wall / 1e9, 2),
        "unit": "GB/s",
        "tokens_per_s": round(T * steps / wall, 1),
        "n_gpus": 1,
        "steps": int(steps),
        "warmup": int(warm),
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8*bf16->f32",
        "data": "synthetic",
        "config": {"workload": f"drafter linear stand-in: T={T} K={K} N={N} (int8, f16 scale per row per 128)",
                   "T": T, "K": K, "N": N, "weight_copies": int(copies), "setup_s": round(setup_s, 1),
                   "step": "linear_i8f16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("linear", "drafter"),
                     "kernel": "k_linear_i8f16", "kernel_us": round(call_us, 3), "alg_bytes_per_launch": int(alg),
                     "mfma_tflops": round(2.0 * T * N * K / (call_us * 1e-6) / 1e12, 2)},
        "cpu_baseline": cpu,
    }))


def host_cpu():
    """CPU model and the threads this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, avail


def blas_threads():
    try:
        import threadpoolctl
        return max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline(L, nb, logits_np, x_np, codes_np, sbits_np, fmt, bytes_per_expert, budget_s):
    """The fp64 oracle, as it stands, on the same steps until the budget is
    spent: once restricted to one thread, once with every thread its BLAS
    uses on this host."""
    import threadpoolctl
    from oracle import gateup, hadamard, numfmt, quant, router, w8a8

    scales = numfmt.bf16_from_bits(sbits_np)

    def run(budget):
        done, wbytes, tokens = 0, 0.0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget or done == 0:      # cycles through the step batches
            lg = logits_np[done % nb]
            x = numfmt.bf16_from_bits(x_np[done % nb])
            r = router.route(lg, L.topk)
            if fmt == "fp8":
                qx, sx = quant.quantize_fp8_activations(x)
                gu = gateup.gateup_fp8blk(qx, sx, codes_np, scales, r["expert_off"], r["sorted_pairs"], L.topk)
            elif fmt == "i8g":
                qx, sx = w8a8.quantize_i8_activations(x)
                gu = w8a8.gateup_i8g(qx, sx, codes_np, scales, r["expert_off"], r["sorted_pairs"], L.topk)
            else:
                xr = hadamard.rotate_activations_bf16(x)
                gu = gateup.gateup_i8h(xr, codes_np, scales, r["expert_off"], r["sorted_pairs"], L.topk)
            gateup.epilogue(gu)
            done += 1
            wbytes += np.count_nonzero(np.diff(r["expert_off"])) * bytes_per_expert
            tokens += L.T
        el = time.perf_counter() - t0
        return done, wbytes / el / 1e9, tokens / el, el

    model, avail = host_cpu()
    with threadpoolctl.threadpool_limits(limits=1):
        d1, v1, t1, e1 = run(budget_s)
    threads = blas_threads()
    dn, vn, tn, en = run(budget_s)
    what = f"route + {'rotate' if fmt == 'i8h' else 'quantize'} + gate_up + epilogue, fp64 NumPy"
    return {"value": round(vn, 4), "unit": "GB/s", "tokens_per_s": round(tn, 3), "cores": int(threads),
            "kind": "oracle",
            "sample": f"{dn} step(s) of the same workload ({what}), {en:.1f} s, {threads} BLAS threads",
            "single_thread": {"value": round(v1, 4), "unit": "GB/s", "tokens_per_s": round(t1, 3), "cores": 1,
                              "sample": f"{d1} step(s), {e1:.1f} s"},
            "cpu_model": model, "cpus_available": int(avail)}


if __name__ == "__main__":
    main()

"""Benchmark of the routed expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one call of the layer's hot path on one batch of seeded synthetic
input already resident in HBM: for the forward workloads dispatch, W13 grouped
GEMM with the SwiGLU epilogue, W2 grouped GEMM and the score-weighted combine;
for "train" also the whole backward (router gradient, DGRAD, WGRAD, dX
combine); "train-mxfp8" is the same step on MXFP8 operands.  Timing uses HIP events on the stream the library launches on;
per-kernel durations come from the library's own event pairs around each
stage during the same timed region.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd TFLOP/s & tokens/s (1 MI355X), % MFMA peak; decode % HBM BW"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published

WORKLOADS = {
    # name: (config in inputs.CONFIGS, training, MXFP8)
    "prefill": ("prefill", False, False),
    "tiny": ("tiny", False, False),
    "train": ("train", True, False),
    "train-mxfp8": ("train", True, True),
    "decode1": ("decode1", False, False),
    "decode32": ("decode32", False, False),
    "mxfp8": ("mxfp8", False, True),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default run: leave out the decode and MXFP8 workloads reported beside prefill")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="before warm-up, run one plain device copy of BYTES (counter calibration)")
    ap.add_argument("--routed", action="store_true",
                    help="time moe_forward_routed instead: the workload's rows put in expert "
                         "order once outside the timed region, then W13 + SwiGLU and W2 on "
                         "them (no dispatch, no combine; forward workloads, BF16 or MXFP8)")
    ap.add_argument("--wgrad-accumulate", action="store_true",
                    help="train workload: the backward adds the weight gradients into the "
                         "existing dW13 / dW2 (plan option wgrad_accumulate)")
    ap.add_argument("--mega", action="store_true",
                    help="decode workloads: the fused one-launch decode (plan option mega: W13, "
                         "activation and W2 chunked over I, then the combine)")
    ap.add_argument("--recompute-h", action="store_true",
                    help="train workload: the forward keeps no h, the backward recomputes it "
                         "(plan option recompute_h)")
    ap.add_argument("--activation", default="swiglu", choices=("swiglu", "geglu", "reglu"),
                    help="gated activation of the W13 output (plan option activation)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor library's BF16 GEMMs (hipBLASLt through torch) on the "
                         "workload's expert-product shapes with uniform rows per expert, and a "
                         "square 8192 GEMM, then exit (context for the roofline)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc csv files and exit")
    return ap.parse_args()


KERNEL_OF_STAGE = {
    # stage name (library event pairs) -> substrings of the symbols (as rocprofv3 reports
    # them) of every kernel the stage launches
    "dispatch": ("dispatch_kernel",),
    "w13": ("grouped_gemm<0,", "fwd_fixup<0,"), "w2": ("grouped_gemm<1,", "fwd_fixup<1,"),
    "combine": ("combine_kernel",), "score_grad": ("score_grad_kernel", "score_grad_sum_kernel"),
    "dgrad_w2": ("grouped_gemm<2,",), "dgrad_w13": ("grouped_gemm<3,",),
    "wgrad_w2": ("grouped_gemm<4,", "wgrad_fixup<4>"), "wgrad_w13": ("grouped_gemm<5,", "wgrad_fixup<5>"),
    "quant_x": ("quantize_kernel", "route_scales_kernel"), "decode_w13": ("decode_w13",), "decode_w2": ("decode_w2",),
    "wgrad_rows": ("wgrad_rows_kernel",), "recompute_h": ("grouped_gemm<0,",),
    "mega": ("mega_decode", "mega_combine"),
}
# the MXFP8 workloads' GEMM stages run the block-scaled kernels
KERNEL_OF_STAGE_MX = dict(KERNEL_OF_STAGE, w13=("grouped_gemm_mx<0,",), w2=("grouped_gemm_mx<1,",),
                          recompute_h=("grouped_gemm_mx<0,",), dgrad_w2=("grouped_gemm_mx<2, 0, false, 0>",),
                          dgrad_w13=("grouped_gemm_mx<2, 0, false, 1>",),
                          wgrad_w2=("grouped_gemm_mx<3, 0, false, 0>",),
                          wgrad_w13=("grouped_gemm_mx<3, 0, false, 1>",), quant_do=("mx_scaled_rows_kernel",),
                          act_bwd=("mx_act_backward_kernel",), quant_t=("mx_transpose_quant_kernel",))
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash():
    """Hash of every kernel and host source of the library: traffic figures taken on
    other sources are stale."""
    import glob
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_routed_dispatch_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_of_stage(workload: str):
    return KERNEL_OF_STAGE_MX if WORKLOADS[workload][2] else KERNEL_OF_STAGE


def _load_traffic():
    try:
        with open(TRAFFIC_PATH) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def traffic_for(stage: str, workload: str):
    """HBM bytes (read + written) per call of the stage (all its kernels), from the
    committed rocprofv3 counter summary, if it was taken on the current sources for this
    workload."""
    tab = _load_traffic()
    if tab.get("source_hash") != source_hash():
        return None
    ent = tab.get("workloads", {}).get(workload, {}).get("stages", {}).get(stage)
    return None if ent is None else ent["read_bytes"] + ent["write_bytes"]


def _pmc_values(path: str, counter: str):
    """{kernel symbol: [counter value of each dispatch]} from a rocprofv3 --pmc csv."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def write_traffic(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) of
    `bench.py --copy-probe N` into bytes per launch for each kernel (median over its
    dispatches).  Each counter is scaled by the factor that makes the plain copy of N
    bytes read and write N bytes."""
    fetch = _pmc_values(fetch_csv, "FETCH_SIZE")
    write = _pmc_values(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copy" in k.lower() and "moe" not in k and k in write]
    if not copy:
        raise SystemExit("no copy kernel in %s" % fetch_csv)
    # the probe is the largest copy dispatch of the run
    ck = max(copy, key=lambda k: max(fetch[k]))
    f_fetch = copy_bytes / (max(fetch[ck]) * 1024.0)
    f_write = copy_bytes / (max(write[ck]) * 1024.0)
    # the median over a kernel's dispatches: the calls of one stage are alike, while a
    # kernel can also run once outside the steps (the quantizer prepares the weights)
    med = lambda v: sorted(v)[len(v) // 2]
    fetch = {k: med(v) for k, v in fetch.items()}
    write = {k: med(v) for k, v in write.items()}
    kernels, stages = {}, {}
    for stage, subs in kernel_of_stage(workload).items():
        names = sorted(k for k in fetch if k in write and any(sub in k for sub in subs))
        if not names:
            continue
        for k in names:
            kernels[k] = {"read_bytes": fetch[k] * 1024.0 * f_fetch, "write_bytes": write[k] * 1024.0 * f_write,
                          "fetch_kib_raw": fetch[k], "write_kib_raw": write[k]}
        # every kernel of the stage runs once per call of the stage
        stages[stage] = {"kernels": names,
                         "read_bytes": sum(kernels[k]["read_bytes"] for k in names),
                         "write_bytes": sum(kernels[k]["write_bytes"] for k in names)}
    # one file for every workload measured on the same sources
    tab = _load_traffic()
    if tab.get("source_hash") != source_hash():
        tab = {"source_hash": source_hash(), "workloads": {}}
    tab.setdefault("workloads", {})[workload] = {
        "copy_kernel": ck, "copy_bytes": copy_bytes, "fetch_factor": f_fetch,
        "write_factor": f_write, "stages": stages, "kernels": kernels}
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(tab, f, indent=1)
    return tab


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads():
    import oracle
    try:
        return int(oracle.num_threads())
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, training: bool, target_s: float, mx: bool = False):
    """The oracle as it stands, on a bounded token sample of the same batch.  MXFP8: the
    forward with x and a quantized (forward_tokens_mx, on the prepared weights'
    dequantized values, prepared once outside the timing); training: the oracle's MXFP8
    training step (train_mx) on the first n tokens, which also builds its weight images
    in every call."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    T, d, I, k = inp.T, inp.d, inp.I, inp.k
    flop_per_token = 6.0 * k * I * d * (3.0 if training else 1.0)
    if mx and not training:
        w13, w2 = (oracle.mx_dequantize(*oracle.mx_quantize(w)) for w in (inp.w13, inp.w2))
    else:
        w13, w2 = inp.w13, inp.w2
    n = min(T, 4)
    rng = np.random.default_rng(123)
    spent = 0.0
    while True:
        toks = np.sort(rng.choice(T, size=n, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        if mx and training:
            oracle.train_mx(inp.x[:n], inp.ids[:n], inp.scores[:n], w13, w2, inp.dy[:n])
        elif mx:
            oracle.forward_tokens_mx(inp.x, inp.ids, inp.scores, w13, w2, toks=toks)
        else:
            oracle.forward_tokens(inp.x, inp.ids, inp.scores, w13, w2, toks=toks)
            if training:
                oracle.backward_tokens(inp.x, inp.ids, inp.scores, w13, w2, inp.dy, toks=toks)
        dt = time.perf_counter() - t0
        spent += dt
        if dt >= target_s * 0.5 or n >= T or spent > 3 * target_s:
            break
        n = min(T, max(n + 1, int(n * min(8.0, target_s / max(dt, 1e-3)))))
    tflops = flop_per_token * n / dt / 1e12
    what = ("the MXFP8 training step (train_mx) on the first %d of %d tokens, weight images included"
            % (n, T) if mx and training else
            "%d of %d tokens of the same batch, %s" % (n, T, "forward + backward" if training else
                                                     ("MXFP8 forward" if mx else "forward")))
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": oracle_threads(),
        "cpu_model": cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": "%s in the fp64 C oracle (OpenMP over tokens / rows / experts), %.1f s; flop "
                  "counted as %d*k*I*d per token" % (what, dt, 18 if training else 6),
        "tokens_per_s": n / dt,
    }


def library_gemm(workload: str):
    """hipBLASLt (torch.bmm / torch.matmul, contiguous BF16 operands) on the shapes of the
    workload's two forward expert products with R / E rows per expert: no gather, no
    SwiGLU, no ragged tails, i.e. the plain batched GEMM the grouped kernels generalise;
    and one square 8192 GEMM, the chip's dense BF16 rate under its power limit."""
    import torch
    from mixture_experts_routed_dispatch_amd import inputs
    cfg = inputs.CONFIGS[WORKLOADS[workload][0]]
    E, d, I = cfg["E"], cfg["d"], cfg["I"]
    M = cfg["T"] * cfg["k"] // E

    def timed(fn, flop, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / n
        return {"us": round(us, 1), "tflops": round(flop / (us * 1e-6) / 1e12, 1)}

    g = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    out = {"library": "hipBLASLt via torch %s" % torch.__version__, "workload": workload,
           "rows_per_expert": M, "E": E, "d": d, "I": I}
    x, w13 = rnd(E, M, d), rnd(E, d, 2 * I)
    out["w13_bmm"] = timed(lambda: torch.bmm(x, w13), 2.0 * E * M * d * 2 * I)
    del x, w13
    a, w2 = rnd(E, M, I), rnd(E, I, d)
    out["w2_bmm"] = timed(lambda: torch.bmm(a, w2), 2.0 * E * M * I * d)
    del a, w2
    A, B = rnd(8192, 8192), rnd(8192, 8192)
    out["square_8192"] = timed(lambda: torch.matmul(A, B), 2.0 * 8192 ** 3, n=10)
    print(json.dumps(out))


def main():
    args = parse()
    if args.library_gemm:
        library_gemm(args.workload)
        return
    if args.traffic:
        tab = write_traffic(args.traffic[0], args.traffic[1], args.workload,
                            args.copy_probe or (1 << 30))
        print(json.dumps(tab, indent=1))
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; --gpus %d is not supported "
              "(no collectives, no sharding)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    out = measure(args, args.workload)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(out.pop("_inp"), WORKLOADS[args.workload][1], args.cpu_seconds,
                                           mx=WORKLOADS[args.workload][2])
    else:
        out.pop("_inp")
        out["cpu_baseline"] = None
    default_run = (args.workload == "prefill" and not args.routed and not args.wgrad_accumulate and not args.mega
                   and not args.recompute_h and args.activation == "swiglu" and not args.copy_probe
                   and not args.no_extra)
    if default_run:
        # the other headline workloads (decode at 1 and 32 tokens: HBM-bound; MXFP8: the
        # FP8 products; training in BF16 and MXFP8), a few steps each, reported beside the
        # prefill line
        import torch
        extra = {}
        for w, steps in (("decode1", 200), ("decode32", 50), ("mxfp8", 10), ("train", 10), ("train-mxfp8", 10)):
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**vars(args))
            sub.steps, sub.warmup = steps, 3
            o = measure(sub, w)
            o.pop("_inp")
            extra[w] = {key: o[key] for key in ("value", "unit", "ms_per_step", "dtype", "config", "stage_us",
                                                 "roofline", "decode", "tokens_per_s", "mfma_frac_layer",
                                                 "gemm_mfma_frac", "steps", "warmup", "weight_prepare_us") if key in o}
        out["other_workloads"] = extra
    print(json.dumps(out), flush=True)


def device_inputs(inp):
    """The seeded host arrays of one workload as device tensors (BF16 bit patterns kept)."""
    import numpy as np
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    out = dict(x=bf16(inp.x), w13=bf16(inp.w13), w2=bf16(inp.w2),
               ids=torch.from_numpy(inp.ids).to("cuda"), scores=torch.from_numpy(inp.scores).to("cuda"))
    if inp.dy is not None:
        out["dy"] = bf16(inp.dy)
    return out


def measure(args, workload):
    """Time args.steps steps of one workload; returns the JSON fields (and the host
    inputs under "_inp", for the CPU baseline)."""
    import numpy as np
    import torch
    from mixture_experts_routed_dispatch_amd import inputs, moe

    cfg_name, training, mx = WORKLOADS[workload]
    inp = inputs.generate_config(cfg_name, seed=0, with_dy=training)
    T, d, I, E, k = inp.T, inp.d, inp.I, inp.E, inp.k
    R = T * k
    t = device_inputs(inp)
    decode = cfg_name.startswith("decode")
    if (args.wgrad_accumulate or args.recompute_h) and not training:
        raise SystemExit("--wgrad-accumulate, --recompute-h: the train workload only")
    if args.mega and not decode:
        raise SystemExit("--mega: the decode workloads only")
    layer = moe.Layer(T, d, I, E, k, training=training,
                      precision=moe.MOE_MXFP8_E4M3 if mx else moe.MOE_BF16, mega=args.mega,
                      wgrad_accumulate=args.wgrad_accumulate, recompute_h=args.recompute_h,
                      activation=("swiglu", "geglu", "reglu").index(args.activation))
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    if training:
        dx = torch.empty_like(y)
        dw13 = torch.empty((E, 2 * I, d), dtype=torch.bfloat16, device="cuda")
        dw2 = torch.empty((E, d, I), dtype=torch.bfloat16, device="cuda")
        ds = torch.empty((T, k), dtype=torch.float32, device="cuda")

    # Per-step inputs.  Decode moves each active expert's weights once per call, so
    # consecutive calls must not find them in the 256 MB MALL: batch-one decode cycles
    # through 16 routings that split the experts into disjoint groups, and the 32-token
    # batch rotates over 4 copies of the whole weight set (1.2 GB each).
    ids_list = [t["ids"]]
    w_list = [(t["w13"], t["w2"])]
    w_scales = [(None, None)]
    bwd_w = None
    prep_us = None
    if mx:
        # weights prepared to MXFP8 once, outside the timed region (timed on their own)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w13q, w13s, w2q, w2s = layer.prepare_weights(t["w13"], t["w2"])
        if training:
            bwd_w = layer.prepare_weights_backward(t["w13"], t["w2"])
        torch.cuda.synchronize()
        e0.record()
        layer.prepare_weights(t["w13"], t["w2"])
        if training:
            layer.prepare_weights_backward(t["w13"], t["w2"])
        e1.record()
        torch.cuda.synchronize()
        prep_us = 1e3 * e0.elapsed_time(e1)
        w_list, w_scales = [(w13q, w2q)], [(w13s, w2s)]
        del t["w13"], t["w2"]
    if cfg_name == "decode1":
        rout = inputs.disjoint_routings(E, k, E // k, seed=1)
        ids_list = [torch.from_numpy(rout[i:i + 1]).to("cuda") for i in range(len(rout))]
    elif cfg_name == "decode32":
        for _ in range(3):
            w_list.append((t["w13"].clone(), t["w2"].clone()))
    n_active = []
    for ids_dev in ids_list:
        n_active.append(len(np.unique(ids_dev.cpu().numpy())))
    n_active_mean = float(np.mean(n_active))
    if len(w_scales) < len(w_list):
        w_scales = w_scales + [(None, None)] * (len(w_list) - len(w_scales))
    bw = [v.data_ptr() for v in bwd_w] if bwd_w is not None else [0, 0, 0, 0]
    wlist = [moe.weights(a.data_ptr(), b.data_ptr(), sa.data_ptr() if sa is not None else 0,
                         sb.data_ptr() if sb is not None else 0, *bw)
             for (a, b), (sa, sb) in zip(w_list, w_scales)]
    state = {"i": 0}

    if args.routed:
        if training or decode:
            raise SystemExit("--routed: forward workloads on the grouped-GEMM path only")
        # expert-major rows and m_indptr from the library's own dispatch, once
        m_ind, gath, _, _ = layer.dispatch(t["ids"], t["scores"])
        x_rows = t["x"][gath.long()].contiguous()
        out_rows = torch.empty((R, d), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()

    def step():
        if args.routed:
            moe.moe_forward_routed(layer.plan, x_rows.data_ptr(), m_ind.data_ptr(), wlist[0],
                                   out_rows.data_ptr(), sp)
            return
        i = state["i"]
        state["i"] = i + 1
        ids_dev = ids_list[i % len(ids_list)]
        w = wlist[i % len(wlist)]
        moe.moe_forward(layer.plan, t["x"].data_ptr(), ids_dev.data_ptr(),
                        t["scores"].data_ptr(), w, y.data_ptr(), sp)
        if training:
            moe.moe_backward(layer.plan, t["dy"].data_ptr(), t["x"].data_ptr(), w, dx.data_ptr(),
                             dw13.data_ptr(), dw2.data_ptr(), ds.data_ptr(), sp)

    if args.copy_probe:
        src_buf = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st, flags = layer.status()
    if flags:
        raise SystemExit("device routing flags set: %d" % flags)

    def timed(profile: bool):
        """Run args.steps steps back to back; returns (ms per step, wall s, stage table)."""
        if profile:
            moe.moe_profile(layer.plan, True)
            moe.moe_profile_read(layer.plan)       # drop anything recorded before
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # Hold the stream with a short spin so that the host has enqueued every timed step
        # before the first one starts: the steps then run back to back, whatever the host's
        # launch overhead (which matters for the few-microsecond decode calls).
        torch.cuda._sleep(int(2e6 + 2e5 * args.steps))
        wall0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - wall0
        tab = None
        if profile:
            moe.moe_profile(layer.plan, False)
            tab = moe.moe_profile_read(layer.plan)
        return ev0.elapsed_time(ev1) / args.steps, wall_s, tab

    # whole-step time without per-kernel events, then per-kernel times (library event
    # pairs around each kernel on the launch stream) in a second pass of the same length
    ms_step, wall, _ = timed(False)
    ms_step_profiled, _, stages = timed(True)

    fwd_flop = 6.0 * R * I * d
    flop = fwd_flop * (3.0 if training else 1.0)
    tflops = flop / (ms_step * 1e-3) / 1e12
    stage_us = {kname: 1e3 * ms / max(n, 1) for kname, (ms, n) in stages.items()}

    # dominant kernel: the longest stage
    dom = max(stage_us, key=stage_us.get)
    gemm_flop = {"w13": 4.0 * R * I * d, "w2": 2.0 * R * I * d, "recompute_h": 4.0 * R * I * d,
                 "dgrad_w2": 2.0 * R * I * d, "wgrad_w2": 2.0 * R * I * d,
                 "dgrad_w13": 4.0 * R * I * d, "wgrad_w13": 4.0 * R * I * d}
    # bytes each stage must move at least once
    min_bytes = {"combine": 2.0 * R * d + 2.0 * T * d + 8.0 * R,
                 "wgrad_rows": 4.0 * R * d + 4.0 * T * d + 8.0 * R,
                 "dispatch": 8.0 * R + 4.0 * (E + 1) + 12.0 * R,
                 "quant_x": T * d * (2.0 + 1.0 + 1.0 / 32),
                 "decode_w13": n_active_mean * 2 * I * d * 2.0 + 2.0 * T * d + 2.0 * R * I + 4.0 * R,
                 "decode_w2": n_active_mean * d * I * 2.0 + 2.0 * R * I + 2.0 * R * d + 2.0 * T * d
                 + 8.0 * R,
                 "mega": n_active_mean * 3 * I * d * 2.0 + 2.0 * T * d + 2.0 * T * d + 8.0 * R,
                 "quant_do": 2.0 * R * d + R * d * 33.0 / 32 + 8.0 * R,
                 "act_bwd": 2.0 * R * I + 4.0 * R * 2 * I + R * 2 * I * 33.0 / 32}
    ntok = R + 128.0 * E
    # each of the two token-layout stages: both operands read once, written padded with scales
    min_bytes["quant_t"] = 0.5 * (2.0 * R * (I + d) + (I + d) * ntok * 33.0 / 32
                                  + 2.0 * R * (d + 2 * I) + (d + 2 * I) * ntok * 33.0 / 32)
    mfma_peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    # The weight gradients write an output the size of the expert weights (E*2I*d BF16 for
    # W13), which can outweigh their products: algorithmic bytes = the gradient written
    # once (and read once when accumulated) + both operands read once (BF16, or E4M3 codes
    # with one E8M0 scale per 32).
    eb = (1.0 + 1.0 / 32) if mx else 2.0
    acc_rw = 2.0 if args.wgrad_accumulate else 1.0
    gemm_bytes = {"wgrad_w2": acc_rw * 2.0 * E * d * I + eb * R * (d + I),
                  "wgrad_w13": acc_rw * 2.0 * E * 2 * I * d + eb * R * (2 * I + d)}
    if dom in gemm_flop:
        achieved = gemm_flop[dom] / (stage_us[dom] * 1e-6) / 1e12
        nb = gemm_bytes.get(dom)
        t_mfma = gemm_flop[dom] / (mfma_peak * 1e12)
        if nb is not None and nb / (PEAK_HBM_GBS * 1e9) > t_mfma:
            # bytes bind: the HBM roofline, with the MFMA fraction beside it
            bach = nb / (stage_us[dom] * 1e-6) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": bach, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": bach / PEAK_HBM_GBS,
                    "algorithmic_per_launch": nb, "avg_launch_us": stage_us[dom],
                    "traffic": traffic_for(dom, workload),
                    "mfma": {"achieved": achieved, "peak": mfma_peak, "unit": "TFLOP/s",
                             "frac": achieved / mfma_peak}}
        else:
            roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": achieved / mfma_peak,
                    "algorithmic_per_launch": gemm_flop[dom], "avg_launch_us": stage_us[dom],
                    "traffic": traffic_for(dom, workload)}
    else:
        nbytes = min_bytes.get(dom, float("nan"))
        achieved = nbytes / (stage_us[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "algorithmic_per_launch": nbytes, "avg_launch_us": stage_us[dom],
                "traffic": traffic_for(dom, workload)}
    gemm_us = sum(stage_us.get(s, 0.0) for s in gemm_flop)
    gemm_tflops = (sum(gemm_flop[s] for s in gemm_flop if s in stage_us) / (gemm_us * 1e-6) / 1e12
                   if gemm_us > 0 else None)
    layer_bytes = n_active_mean * 3 * I * d * 2.0 + 4.0 * T * d + 8.0 * R

    out = {
        "metric": METRIC,
        "value": layer_bytes / (ms_step * 1e-3) / 1e9 if decode else tflops,
        "unit": "GB/s" if decode else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3" if mx else "bf16",
        "weight_prepare_us": prep_us,
        "data": "synthetic: seeded numpy draws, x ~ N(0,1), W ~ N(0,1/fan_in) in BF16, "
                + ("Zipf(1.2) top-k routing with 8 forced-empty experts, dY ~ N(0,1)"
                   if cfg_name == "train" else "uniform distinct top-k routing")
                + ", softmax-of-normal scores"
                + ("; 16 routings over disjoint expert groups, cycled" if cfg_name == "decode1" else "")
                + ("; 4 copies of the weights, rotated" if cfg_name == "decode32" else ""),
        "config": {"workload": "%s: T=%d d=%d I=%d E=%d k=%d %s %s%s" % (
            cfg_name, T, d, I, E, k, "MXFP8-E4M3" if mx else "BF16",
            ("forward+backward" + (", weight gradients accumulated" if args.wgrad_accumulate else "")
             + (", h recomputed in the backward" if args.recompute_h else ""))
            if training else
            ("forward of pre-dispatched rows (moe_forward_routed: W13 + SwiGLU, W2)" if args.routed
             else "forward, fused (mega) decode" if args.mega else "forward"),
            "" if args.activation == "swiglu" else ", %s" % {"geglu": "GeGLU", "reglu": "ReGLU"}[args.activation]),
            "T": T, "d": d, "I": I, "E": E, "k": k, "routed_rows": R,
            "flop_per_step": flop},
        "tokens_per_s": T / (ms_step * 1e-3),
        "tflops": tflops,
        "mfma_frac_layer": tflops / mfma_peak,
        "gemm_tflops": gemm_tflops,
        "gemm_mfma_frac": gemm_tflops / mfma_peak if gemm_tflops else None,
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "wall_ms_per_step": 1e3 * wall / args.steps,
        "ms_per_step_with_kernel_events": ms_step_profiled,
        "roofline": roof,
        "_inp": inp,
    }
    if decode:
        out["decode"] = {"active_experts_per_call": n_active_mean,
                         "weight_bytes_per_call": n_active_mean * 3 * I * d * 2.0,
                         "layer_hbm_gbs": layer_bytes / (ms_step * 1e-3) / 1e9,
                         "layer_hbm_frac": layer_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS}
    layer.close()
    return out


if __name__ == "__main__":
    main()

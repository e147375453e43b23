"""Benchmark of the SVDQuant linear (fused W4A4 + low-rank) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--fmt mxfp4|int4|int8] [--workload fc1|...]

A step is one forward of the layer -- activation kernel (smoothing, 4-bit
group quantization, low-rank down-projection) then the 4-bit GEMM with the
up-projection, bias and rounding in its epilogue -- over one batch of
synthetic tokens already resident in HBM.  The pack (smoothing factors, SVD,
residual quantization) is offline and not timed.

Default workload: the FLUX.1-shaped MLP fc1 linear at 1024^2 (4608 tokens x
3072 -> 12288), bf16 activations, MXFP4 group 32 with e8m0 scales, rank 32.
Metric: effective TOPS = 2 M K N / t (the low-rank FLOPs are not counted).

Prints one JSON line.  The CPU baseline is the CPU oracle's own float64
forward timed on a bounded sample of the same layer, on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TOPS of fused W4A4+low-rank linear (FLUX fc1 shape), % of MFMA peak"
PEAK_TFLOPS = {"mxfp4_g32": 10100.0, "int4_g64": 5000.0, "int8_w8a8": 5000.0}   # MI355X dense MFMA: fp4, int8, int8
FMT_NAMES = {"mxfp4": "mxfp4_g32", "int4": "int4_g64", "int8": "int8_w8a8"}
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: (M, K, N, dtype)
    "fc1": (4608, 3072, 12288, "bf16"),
    "fc2": (4608, 12288, 3072, "bf16"),
    "qkv": (4608, 3072, 9216, "bf16"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 200 untimed forwards (about 25 ms of work at fc1) bring the power-limited
    # clock to its steady state; after 10 the timed region still catches the
    # settling transient (125 against 115.7 us per forward on one box)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--fmt", default="mxfp4", choices=["mxfp4", "int4", "int8"],
                    help="int8: the 8-bit setting (per-token / per-channel INT8; use --rank 16)")
    ap.add_argument("--workload", default="fc1", choices=sorted(WORKLOADS))
    ap.add_argument("--rank", type=int, default=32)
    ap.add_argument("--rotate", type=int, default=4, help="distinct X/Y/weight buffer sets cycled per step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--kernel-iters", type=int, default=50)
    ap.add_argument("--lowrank-study", action="store_true",
                    help="instead of the headline line, time the forward three ways -- W4A4 only (rank 0), "
                         "fused low-rank branch, low-rank branch as separate passes -- and print their overheads")
    ap.add_argument("--chain-study", action="store_true",
                    help="instead of the headline line, time the FLUX MLP pair (fc1 + GELU -> fc2; --fmt mxfp4 or int4) with "
                         "fc2's activation pass as its own kernel and chained into fc1's GEMM epilogue")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line, print one JSON record per (config, shape, format) over "
                         "every shape of the five workload configs: forward, activation-kernel and GEMM times "
                         "and their rooflines")
    ap.add_argument("--sweep-configs", default="1,2,3,4,5", help="configs the sweep covers")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the layer, time a plain device copy of MIB MiB (the reference kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k2_gemm_flux_fc1_mxfp4_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "diffusion_smooth_group_amd", "csrc", "svdq_kernels.hip")


def measured_traffic(workload, fmt_name):
    """HBM-side bytes per GEMM launch from the committed counter summary, or
    None if there is none for this workload or the kernel source changed since."""
    import hashlib
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != sha or kv.get("workload") != workload or kv.get("format") != fmt_name:
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for counter scaling."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 3}}), flush=True)


def _codes_scales(rows, K, fmt):
    """Bytes of one operand's codes and scales."""
    if fmt == "int8_w8a8":
        return rows * K + 4 * rows
    G = 64 if fmt == "int4_g64" else 32
    sb = 2 if fmt == "int4_g64" else 1
    return rows * K // 2 + (rows * K // G) * sb


def k1_bytes(M, K, r, fmt):
    return 2 * M * K + _codes_scales(M, K, fmt) + 2 * M * r + 2 * K * r + 4 * K


def k2_bytes(M, K, N, r, fmt):
    return _codes_scales(M, K, fmt) + _codes_scales(N, K, fmt) + 2 * M * r + 2 * r * N + 4 * N + 2 * M * N


def cpu_baseline(spec, d, lin_export, fmt_name, rank):
    """The oracle's forward (float64, as the parity tests use it) on a bounded
    sample of the layer."""
    import threadpoolctl  # noqa: F401  (reports the BLAS threads)
    from threadpoolctl import threadpool_info
    import oracle as o
    rows, cols = 512, 2048
    W = np.ascontiguousarray(d["W"][:, :cols])
    L2q = np.ascontiguousarray(lin_export["L2q"][:, :cols])
    pf = o.pack_from_factors(W, spec.dtype, lin_export["lam"], lin_export["L1x"][:, :rank], L2q[:rank], fmt_name)
    layer = {"dtype": spec.dtype, "fmt": fmt_name, "lam": lin_export["lam"], "invlam": lin_export["invlam"],
             "L1x": lin_export["L1x"], "L2q": L2q, "qw": pf["qw"], "sw": pf["sw"],
             "bias": None if d["bias"] is None else d["bias"][:cols]}
    Xs = np.ascontiguousarray(d["X"][:rows])
    o.forward(layer, Xs)                     # warm
    reps, t0 = 0, time.perf_counter()
    while True:
        o.forward(layer, Xs)
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 20:
            break
    t = el / reps
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": 2.0 * rows * spec.K * cols / t / 1e12, "unit": "TOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {spec.M} tokens x {cols} of {spec.N} output columns, the oracle's float64 "
                      f"forward (activation quantization, exact 4-bit product, down- and up-projection, bias, "
                      f"one rounding), {reps} reps, {t * 1e3:.1f} ms each; host os.cpu_count()={os.cpu_count()}"}


def lowrank_study(args):
    """Cost of the low-rank branch on top of the 4-bit path: the layer with
    its branch switched off (W4A4 only, same 4-bit codes), the fused forward,
    and the branch run as separate passes (a second read of X, Y read back
    and rewritten)."""
    import ctypes as C
    import torch
    from diffusion_smooth_group_amd import svdq as S
    from diffusion_smooth_group_amd import workloads as wl
    fmt_name = FMT_NAMES[args.fmt]
    fmt = {"mxfp4": S.FMT_MXFP4_G32, "int4": S.FMT_INT4_G64, "int8": S.FMT_INT8_W8A8}[args.fmt]
    M, K, N, dts = WORKLOADS[args.workload]
    dt = S.BF16 if dts == "bf16" else S.F16
    spec = {"fc1": wl.config_shapes(3)[0], "fc2": wl.config_shapes(3)[1]}.get(args.workload, wl.config_shapes(2)[0])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.generate(spec)
    Xd0 = S.bits_to_device(d["X"], dt, dev)
    absmax = S.activation_absmax(Xd0, dt)
    torch.cuda.synchronize()
    am = absmax.cpu().numpy()
    lin = S.SVDQLinear.pack(d["W"], dt, am, args.rank, fmt, d["bias"], rank_capacity=args.rank)
    nrot = max(1, args.rotate)
    lib = S.lib_handle()
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)
    Xs = [Xd0] + [Xd0.clone() for _ in range(nrot - 1)]
    Ys = [torch.empty((M, N), dtype=Xd0.dtype, device=dev) for _ in range(nrot)]
    layers, blobs = [lin.layer], [lin.blob]
    for _ in range(nrot - 1):
        b = torch.empty_like(lin.blob)
        layers.append(S.layer_copy(lin.layer, S._t_ptr(b), b.numel(), True))
        blobs.append(b)
    # W4A4 only: the same blobs (same 4-bit codes) with the low-rank branch
    # switched off in the descriptor
    plain = []
    for L in layers:
        L0 = S.svdq_layer.from_buffer_copy(L)
        L0.rank = 0
        L0.rank_active = 0
        plain.append(L0)
    wsb = S.workspace_size(lin.layer, M)
    wss = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(nrot)]

    def time_fwd(descs, flags):
        def fwd(i):
            j = i % nrot
            rc = lib.svdq_linear_forward(C.byref(descs[j]), S._t_ptr(Xs[j]), M, K, S._t_ptr(Ys[j]), N,
                                         S._t_ptr(wss[j]), wsb, flags, sh)
            if rc != 0:
                raise S.SvdqError("svdq_linear_forward", rc)
        for i in range(args.warmup):
            fwd(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fwd(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    runs = {"w4a4": [], "fused": [], "unfused": []}
    for _ in range(3):              # interleaved rounds, medians reported
        runs["w4a4"].append(time_fwd(plain, 0))
        runs["fused"].append(time_fwd(layers, 0))
        runs["unfused"].append(time_fwd(layers, S.FLAG_UNFUSED_LOWRANK))
    t0, tf, tu = (float(np.median(runs[k])) for k in ("w4a4", "fused", "unfused"))
    print(json.dumps({
        "study": "low-rank branch cost over the W4A4 forward: fused vs separate passes",
        "workload": f"flux_{args.workload}_{M}x{K}x{N}", "format": fmt_name, "rank": args.rank,
        "activation_dtype": dts, "rotating_buffer_sets": nrot, "steps": args.steps, "rounds": 3,
        "t_w4a4_us": round(t0, 2), "t_fused_us": round(tf, 2), "t_unfused_us": round(tu, 2),
        "overhead_fused_pct": round(100.0 * (tf - t0) / t0, 1),
        "overhead_unfused_pct": round(100.0 * (tu - t0) / t0, 1),
        "runs_us": {k: [round(x, 2) for x in v] for k, v in runs.items()}}), flush=True)


def chain_study(args):
    """The MLP pair fc1 (+GELU) -> fc2 (--fmt mxfp4 or int4) two ways: unchained (fc1 writes Y1,
    fc2's activation kernel reads it back) and chained (fc2's codes, scales
    and down-projection come out of fc1's GEMM epilogue; Y1 is not stored)."""
    import ctypes as C
    import torch
    from diffusion_smooth_group_amd import svdq as S
    from diffusion_smooth_group_amd import workloads as wl
    fc1, fc2 = wl.config_shapes(3)
    M, K, H = fc1.M, fc1.K, fc1.N
    dt = S.BF16
    fmt = {"mxfp4": S.FMT_MXFP4_G32, "int4": S.FMT_INT4_G64}[args.fmt]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d1 = wl.generate(fc1)
    d2 = wl.generate(fc2, fc1_inputs=d1)
    lins = []
    for d in (d1, d2):
        am = S.activation_absmax(S.bits_to_device(d["X"], dt, dev), dt)
        torch.cuda.synchronize()
        lins.append(S.SVDQLinear.pack(d["W"], dt, am.cpu().numpy(), args.rank, fmt, d["bias"],
                                      rank_capacity=args.rank))
    lib = S.lib_handle()
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)
    nrot = max(1, args.rotate)
    X0 = S.bits_to_device(d1["X"], dt, dev)
    sets = []
    for r in range(nrot):
        L = []
        blobs = []
        for lin in lins:
            if r == 0:
                L.append(lin.layer)
                continue
            b = torch.empty_like(lin.blob)
            L.append(S.layer_copy(lin.layer, S._t_ptr(b), b.numel(), True))
            blobs.append(b)
        cw = C.c_size_t()
        lib.svdq_chain_workspace_size(C.byref(L[0]), C.byref(L[1]), M, C.byref(cw))
        sets.append({"L": L, "blobs": blobs, "X": X0 if r == 0 else X0.clone(),
                     "Y1": torch.empty((M, H), dtype=X0.dtype, device=dev),
                     "Y2": torch.empty((M, K), dtype=X0.dtype, device=dev),
                     "ws1": torch.empty(cw.value, dtype=torch.uint8, device=dev), "ws1b": cw.value,
                     "ws2": torch.empty(S.workspace_size(L[1], M), dtype=torch.uint8, device=dev),
                     "ws2b": S.workspace_size(L[1], M)})

    def check(rc, fn):
        if rc != 0:
            raise S.SvdqError(fn, rc)

    def unchained(i):
        z = sets[i % nrot]
        check(lib.svdq_linear_forward(C.byref(z["L"][0]), S._t_ptr(z["X"]), M, K, S._t_ptr(z["Y1"]), H,
                                      S._t_ptr(z["ws1"]), z["ws1b"], S.FLAG_GELU, sh), "svdq_linear_forward")
        check(lib.svdq_linear_forward(C.byref(z["L"][1]), S._t_ptr(z["Y1"]), M, H, S._t_ptr(z["Y2"]), K,
                                      S._t_ptr(z["ws2"]), z["ws2b"], 0, sh), "svdq_linear_forward")

    def chained(i):
        z = sets[i % nrot]
        check(lib.svdq_linear_forward_chain(C.byref(z["L"][0]), C.byref(z["L"][1]), S._t_ptr(z["X"]), M, K, None, 0,
                                            S._t_ptr(z["ws1"]), z["ws1b"], S._t_ptr(z["ws2"]), z["ws2b"],
                                            S.FLAG_GELU, sh), "svdq_linear_forward_chain")
        check(lib.svdq_gemm_forward(C.byref(z["L"][1]), M, S._t_ptr(z["Y2"]), K, S._t_ptr(z["ws2"]), z["ws2b"], 0,
                                    sh), "svdq_gemm_forward")

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    runs = {"unchained": [], "chained": []}
    for _ in range(3):              # interleaved rounds, medians reported
        runs["unchained"].append(timed(unchained))
        runs["chained"].append(timed(chained))
    tu, tc = (float(np.median(runs[k])) for k in ("unchained", "chained"))
    flops = 2.0 * M * K * H * 2
    print(json.dumps({
        "study": "MLP pair fc1 (+GELU) -> fc2: fc2's activation pass as its own kernel vs chained into fc1's epilogue",
        "workload": f"flux_mlp_{M}x{K}x{H}x{K}", "format": FMT_NAMES[args.fmt], "rank": args.rank,
        "activation_dtype": "bf16",
        "rotating_buffer_sets": nrot, "steps": args.steps, "rounds": 3,
        "t_unchained_us": round(tu, 2), "t_chained_us": round(tc, 2),
        "saving_pct": round(100.0 * (tu - tc) / tu, 1),
        "pair_tops_unchained": round(flops / tu * 1e-6, 1), "pair_tops_chained": round(flops / tc * 1e-6, 1),
        "runs_us": {k: [round(x, 2) for x in v] for k, v in runs.items()}}), flush=True)


def sweep(args):
    """Every shape of the five workload configs, each format it names: the
    forward (activation kernel + GEMM, HIP events around each kernel, 20
    steps over 2 rotating buffer sets after 5 warm-up steps), as TOPS and
    against its roofline max(ops / MFMA peak, bytes / HBM peak)."""
    import ctypes as C
    import torch
    from diffusion_smooth_group_amd import svdq as S
    from diffusion_smooth_group_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = S.lib_handle()
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)
    fmt_codes = {wl.MXFP4: S.FMT_MXFP4_G32, wl.INT4: S.FMT_INT4_G64}
    steps, warm, nrot = 20, 5, 2
    cfgs = [int(c) for c in args.sweep_configs.split(",")]
    fc1_cache = {}     # the MLP pair's first layer, whose output feeds the second
    n_rec = 0
    for cfg in cfgs:
        for spec in wl.config_shapes(cfg):
            dt = S.BF16 if spec.dtype == wl.BF16 else S.F16
            t_gen = time.time()
            if spec.x_dist == "gelu_of_fc1":
                key = (spec.seed[0], spec.seed[1] - 1)
                d = wl.generate(spec, fc1_inputs=fc1_cache.get(key))
            else:
                d = wl.generate(spec)
                if cfg == 3 and "fc1" in spec.name:
                    fc1_cache[tuple(spec.seed)] = d
            t_gen = time.time() - t_gen
            # MLP fc1 layers carry the block's GELU in their epilogue
            gelu = "fc1" in spec.name
            M, K, N = spec.M, spec.K, spec.N
            Xd = S.bits_to_device(d["X"], dt, dev)
            am = S.activation_absmax(Xd, dt)
            torch.cuda.synchronize()
            for fmt in spec.formats:
                fmt_name = fmt
                rank, rl = spec.rank, spec.lora_rank
                t_pack = time.time()
                lin = S.SVDQLinear.pack(d["W"], dt, am.cpu().numpy(), rank, fmt_codes[fmt], d["bias"],
                                        rank_capacity=rank + rl)
                if rl:
                    lin.attach_lora(d["lora_A"], d["lora_B"], 1.0)
                t_pack = time.time() - t_pack
                ra = rank + rl
                layers, blobs = [lin.layer], [lin.blob]
                for _ in range(nrot - 1):
                    b = torch.empty_like(lin.blob)
                    layers.append(S.layer_copy(lin.layer, S._t_ptr(b), b.numel(), True))
                    blobs.append(b)
                Xs = [Xd] + [Xd.clone() for _ in range(nrot - 1)]
                Ys = [torch.empty((M, N), dtype=Xd.dtype, device=dev) for _ in range(nrot)]
                wsb = S.workspace_size(lin.layer, M)
                wss = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(nrot)]
                flags = S.FLAG_GELU if gelu else 0

                def step(i):
                    j = i % nrot
                    rc = lib.svdq_quantize_activations(C.byref(layers[j]), S._t_ptr(Xs[j]), M, K, S._t_ptr(wss[j]),
                                                       wsb, sh)
                    if rc != 0:
                        raise S.SvdqError("svdq_quantize_activations", rc)
                    rc = lib.svdq_gemm_forward(C.byref(layers[j]), M, S._t_ptr(Ys[j]), N, S._t_ptr(wss[j]), wsb,
                                               flags, sh)
                    if rc != 0:
                        raise S.SvdqError("svdq_gemm_forward", rc)
                for i in range(warm):
                    step(i)
                torch.cuda.synchronize()
                # each kernel timed from its own dispatch timestamps
                S.timing_start(2 * steps)
                for i in range(steps):
                    step(i)
                torch.cuda.synchronize()
                kinds, kus = S.timing_stop(4 * steps)
                k1u, k2u = kus[kinds == S.KERNEL_ACT], kus[kinds == S.KERNEL_GEMM]
                t1 = float(np.median(k1u))
                t2 = float(np.median(k2u))
                tf = float(np.median(k1u + k2u))
                ops = 2.0 * M * K * N
                peak = PEAK_TFLOPS[fmt_name]
                b2 = k2_bytes(M, K, N, ra, fmt_name)
                b1 = k1_bytes(M, K, ra, fmt_name)
                t_mfma = ops / (peak * 1e12) * 1e6
                t_hbm = b2 / (HBM_PEAK_GBS * 1e9) * 1e6
                floor = max(t_mfma, t_hbm)
                rec = {"sweep": True, "config": cfg, "shape": spec.name, "M": M, "K": K, "N": N,
                       "format": fmt_name, "dtype": spec.dtype, "rank_active": ra, "gelu": gelu,
                       "t_fwd_us": round(tf, 2), "t_k1_us": round(t1, 2), "t_gemm_us": round(t2, 2),
                       "tops_fwd": round(ops / (tf * 1e-6) / 1e12, 1), "tops_gemm": round(ops / (t2 * 1e-6) / 1e12, 1),
                       "gemm_roofline": {"bound": "mfma" if t_mfma >= t_hbm else "hbm", "peak_tflops": peak,
                                         "t_mfma_us": round(t_mfma, 2), "t_hbm_us": round(t_hbm, 2),
                                         "algorithmic_bytes": b2, "frac": round(floor / t2, 4)},
                       "k1_roofline": {"bound": "hbm", "algorithmic_bytes": b1,
                                       "frac": round(b1 / (HBM_PEAK_GBS * 1e9) * 1e6 / t1, 4)},
                       "pack_s": round(t_pack, 2), "gen_s": round(t_gen, 2)}
                if fmt_name == "int4_g64":
                    rec["gemm_roofline"]["frac_vs_fp4_peak"] = round(ops / (PEAK_TFLOPS["mxfp4_g32"] * 1e12) * 1e6 / t2, 4)
                print(json.dumps(rec), flush=True)
                n_rec += 1
                del layers, blobs, Xs, Ys, wss, lin
                torch.cuda.empty_cache()
            del Xd, d
    print(json.dumps({"sweep_done": True, "records": n_rec, "configs": cfgs}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU sharding "
              f"is a design note, not a run.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.lowrank_study:
        lowrank_study(args)
        return
    if args.chain_study:
        chain_study(args)
        return
    if args.sweep:
        sweep(args)
        return
    import torch
    from diffusion_smooth_group_amd import svdq as S
    from diffusion_smooth_group_amd import workloads as wl

    fmt_name = FMT_NAMES[args.fmt]
    fmt = {"mxfp4": S.FMT_MXFP4_G32, "int4": S.FMT_INT4_G64, "int8": S.FMT_INT8_W8A8}[args.fmt]
    M, K, N, dts = WORKLOADS[args.workload]
    dt = S.BF16 if dts == "bf16" else S.F16
    if args.workload == "fc1":
        spec = wl.config_shapes(3)[0]
    elif args.workload == "fc2":
        spec = wl.config_shapes(3)[1]
    else:
        spec = wl.config_shapes(2)[0]
    assert (spec.M, spec.K, spec.N) == (M, K, N)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    d = wl.generate(spec)
    Xd0 = S.bits_to_device(d["X"], dt, dev)
    absmax = S.activation_absmax(Xd0, dt)
    torch.cuda.synchronize()
    lin = S.SVDQLinear.pack(d["W"], dt, absmax.cpu().numpy(), args.rank, fmt, d["bias"], rank_capacity=args.rank)
    t_pack = time.time() - t0
    torch.cuda.synchronize()

    # rotating buffer sets so the 256 MB last-level cache cannot hold a step's working set
    nrot = max(1, args.rotate)
    Xs = [Xd0] + [Xd0.clone() for _ in range(nrot - 1)]
    Ys = [torch.empty((M, N), dtype=Xd0.dtype, device=dev) for _ in range(nrot)]
    layers = [lin.layer]
    blobs = [lin.blob]
    for _ in range(nrot - 1):
        b = torch.empty_like(lin.blob)
        layers.append(S.layer_copy(lin.layer, S._t_ptr(b), b.numel(), True))
        blobs.append(b)
    ws_bytes = S.workspace_size(lin.layer, M)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(nrot)]
    lib = S.lib_handle()
    import ctypes as C
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)

    def fwd(i):
        j = i % nrot
        rc = lib.svdq_linear_forward(C.byref(layers[j]), S._t_ptr(Xs[j]), M, K, S._t_ptr(Ys[j]), N,
                                     S._t_ptr(wss[j]), ws_bytes, 0, sh)
        if rc != 0:
            raise S.SvdqError("svdq_linear_forward", rc)

    def k1(i):
        j = i % nrot
        rc = lib.svdq_quantize_activations(C.byref(layers[j]), S._t_ptr(Xs[j]), M, K, S._t_ptr(wss[j]), ws_bytes, sh)
        if rc != 0:
            raise S.SvdqError("svdq_quantize_activations", rc)

    def k2(i):
        j = i % nrot
        rc = lib.svdq_gemm_forward(C.byref(layers[j]), M, S._t_ptr(Ys[j]), N, S._t_ptr(wss[j]), ws_bytes, 0, sh)
        if rc != 0:
            raise S.SvdqError("svdq_gemm_forward", rc)

    sclk_idle = S.probe_clock(stream)
    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` forwards
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        fwd(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # ---- the same forward loop again, each kernel launched with an event
    # pair that takes that kernel's own dispatch begin / end timestamps
    # (svdq_timing_start: hipExtLaunchKernel, nothing added to the stream
    # between kernels), so K1 + K2 <= the forward by construction
    n_inst = max(args.steps, args.kernel_iters)
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    S.timing_start(2 * n_inst)
    ev2.record(stream)
    for i in range(n_inst):
        fwd(i)
    ev3.record(stream)
    torch.cuda.synchronize()
    kinds, kus = S.timing_stop(4 * n_inst)
    ms_step_kt = ev2.elapsed_time(ev3) / n_inst
    t_k1 = kus[kinds == S.KERNEL_ACT]
    t_k2 = kus[kinds == S.KERNEL_GEMM]
    if len(t_k1) != n_inst or len(t_k2) != n_inst:
        raise RuntimeError(f"kernel timing recorded {len(t_k1)} / {len(t_k2)} launches, expected {n_inst}")
    # per-forward times: an event pair around each forward on the stream the
    # kernels run on (distribution of the step the headline averages)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (ea, eb) in enumerate(evs):
        ea.record(stream)
        fwd(i)
        eb.record(stream)
    torch.cuda.synchronize()
    t_step = np.array([ea.elapsed_time(eb) * 1e3 for ea, eb in evs])
    sclk_after = S.probe_clock(stream)      # a light kernel right after the loop
    # three more forwards with the GEMM traced (per-workgroup wall and
    # shader-clock counters): the clock the GEMM itself ran at
    traces = []
    for i in range(3):
        # the traced launch sits inside a run of forwards (no idle gap before it)
        for q in range(10):
            fwd(q)
        j = (n_inst + i) % nrot
        k1(n_inst + i)
        rc = lib.svdq_gemm_forward(C.byref(layers[j]), M, S._t_ptr(Ys[j]), N, S._t_ptr(wss[j]), ws_bytes,
                                   S.FLAG_TRACE, sh)
        if rc != 0:
            raise S.SvdqError("svdq_gemm_forward", rc)
        for q in range(3):
            fwd(q)
        rec, hz = S.trace_read()
        r = rec.astype(np.float64)
        # a staggered launch has workgroups past their XCD's tile count, which
        # only record their start and end (well under a microsecond): the
        # per-workgroup statistics cover the workgroups that ran a tile
        r = r[(r[:, 2] - r[:, 0]) > 1e-6 * hz]
        wg_ticks = r[:, 2] - r[:, 0]
        traces.append({"sclk_mhz": float((r[:, 3] - r[:, 1]).sum() / wg_ticks.sum() * hz * 1e-6),
                       "span_us": float((r[:, 2].max() - r[:, 0].min()) / hz * 1e6),
                       "wg_us": np.percentile(wg_ticks / hz * 1e6, [10, 50, 90]).tolist(),
                       "workgroups": int(len(r))})
    tr = sorted(traces, key=lambda t: t["span_us"])[1]          # the median of the three by span
    t_fw = t_k1 + t_k2

    def stats(t):
        return {"mean": round(float(np.mean(t)), 2), "median": round(float(np.median(t)), 2),
                "p10": round(float(np.percentile(t, 10)), 2), "p90": round(float(np.percentile(t, 90)), 2)}

    # the matrix core's sustained FP4 rate with no memory traffic, on random
    # and on zero operands (second of two runs each)
    ceil = {}
    for rnd, key in ((True, "random"), (False, "zero")):
        S.probe_mfma_rate(rnd, 2000, stream)
        tf, mhz = S.probe_mfma_rate(rnd, 2000, stream)
        ceil[key + "_tflops"] = round(tf, 1)
        ceil[key + "_mhz"] = round(mhz, 1)

    flops = 2.0 * M * K * N
    tops = flops / (ms_step * 1e-3) / 1e12
    k2_mean = float(np.mean(t_k2))
    k1_mean = float(np.mean(t_k1))
    k2_tflops = flops / (k2_mean * 1e-6) / 1e12
    k1_gbs = k1_bytes(M, K, args.rank, fmt_name) / (k1_mean * 1e-6) / 1e9
    peak = PEAK_TFLOPS[fmt_name]
    out = {
        "metric": METRIC if args.fmt != "int8" else METRIC.replace("W4A4", "W8A8"),
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.fmt,
        "data": "synthetic",
        "config": {"workload": f"flux_{args.workload}_{M}x{K}x{N}", "M": M, "K": K, "N": N, "rank": args.rank,
                   "format": fmt_name, "activation_dtype": dts, "parallelism": "single GPU",
                   "rotating_buffer_sets": nrot},
        "pct_of_peak": round(100.0 * tops / peak, 2),
        "roofline": {"bound": "mfma", "kernel": "k2_gemm", "achieved": round(k2_tflops, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(k2_tflops / peak, 4),
                     "traffic": measured_traffic(f"flux_{args.workload}_{M}x{K}x{N}", fmt_name),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": k2_bytes(M, K, N, args.rank, fmt_name),
                     "time_source": "mean K2 duration over a forward loop, each launch timed by events bound to the "
                                    "kernel's own dispatch timestamps (hipExtLaunchKernel)",
                     "frac_of_sustained_fp4_rate": round(k2_tflops / ceil["random_tflops"], 4)
                     if fmt_name == "mxfp4_g32" else None,
                     "frac_at_traced_clock": round(k2_tflops / (peak * tr["sclk_mhz"] / 2400.0), 4)},
        "k1_roofline": {"bound": "hbm", "kernel": "k1_act", "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": k1_bytes(M, K, args.rank, fmt_name)},
        "kernel_us": {"k1_act": stats(t_k1), "k2_gemm": stats(t_k2), "k1_plus_k2": stats(t_fw),
                      "launches": n_inst, "forward_loop_us_per_step": round(ms_step_kt * 1e3, 2)},
        "forward_us": dict(stats(t_step), note="one event pair around each of `steps` forwards (distribution "
                                               "of the step the headline averages; the pairs add a little)"),
        "sclk_mhz": {"idle_probe": round(sclk_idle, 1), "probe_after_forward_loop": round(sclk_after, 1),
                     "gemm_traced": round(tr["sclk_mhz"], 1)},
        "k2_trace": {"workgroups": tr["workgroups"], "span_us": round(tr["span_us"], 2),
                     "workgroup_us_p10_p50_p90": [round(x, 2) for x in tr["wg_us"]],
                     "note": "median (by span) of three traced GEMM launches, each inside a run of forwards; "
                             "sclk = shader cycles / wall time summed over workgroups"},
        "mfma_fp4_sustained": ceil,
        "gemm_only_tops": round(k2_tflops, 2),
        "timed_wall_s": round(wall, 4),
        "pack_s": round(t_pack, 2),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(spec, d, lin.export(), fmt_name, args.rank)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the W4A4 RPBH rotate-then-quantize linear layer on one MI355X.

Workload: the image-DiT projection -- 4096 bf16 tokens, d_in = d_out = 3072,
RPBH block h = 128, 16-level Lloyd-Max codebooks for weights and activations,
bf16 output (synthetic inputs of that shape and distribution, see synth).

One step = the whole run-time path on one batch: the fused rotate + quantize
of the activations (orbit_quant_act) and the codebook-decode GEMM with its
r s / K epilogue (orbit_qlinear).  The weights are packed once beforehand: in
the method the rotation is absorbed into the weights offline.

Reported: effective TFLOP/s of the layer, 2 M N K / (t_quant + t_gemm); the
GEMM's TFLOP/s against the fp16 dense MFMA peak; the rotate/quant stage's
GB/s against the HBM peak.  Per-kernel times come from HIP events recorded on
the stream the kernels run on.  Activations rotate through a pool of buffers
larger than the 256 MB Infinity Cache, so the quant stage reads from HBM.
The oracle (fp64, host cores) is timed on the same workload as a baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_MFMA_F16 = 2516.6   # TFLOP/s, MI355X dense fp16/bf16
PEAK_HBM = 8000.0        # GB/s, MI355X HBM3E
POOL_BYTES = 600 << 20   # > 2x the 256 MB Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(HERE, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters")
    ap.add_argument("--only", choices=["quant", "gemm", "copy"], default=None,
                    help="launch only one kernel --steps times (for counter runs): the "
                         "activation rotate+quantize, the decode GEMM, or a plain device "
                         "copy of COPY_BYTES that calibrates FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


COPY_BYTES = 256 << 20   # calibration copy: 256 MiB read + 256 MiB written per launch


def cpu_baseline(inp, rounds_target_s=10.0):
    """The oracle as it stands, on this host's cores: rotate + quantize the
    activations and the fp64 product from codes, for a bounded token sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    X64 = oracle.bf16_bits_to_f64(inp["X"])
    W64 = oracle.bf16_bits_to_f64(inp["W"])
    cb = oracle.codebook(4)
    w = oracle.pack_weights(W64, inp["perm"], inp["signs"], inp["h"], cb, 4)  # offline, untimed
    K, N = inp["K"], inp["N"]

    def run(rows):
        a = oracle.quant_act(X64[:rows], inp["perm"], inp["signs"], inp["h"], cb, 4, inp["eps"])
        oracle.qlinear_codes(a["idx"], a["s"], cb["centroids"], w["idx"], w["r_bf16"],
                             cb["centroids"], K)

    run(64)  # warm-up
    rows, elapsed, total_rows = 512, 0.0, 0
    t0 = time.perf_counter()
    while elapsed < rounds_target_s and total_rows < 16 * inp["M"]:
        run(rows)
        total_rows += rows
        elapsed = time.perf_counter() - t0
    flops = 2.0 * total_rows * N * K
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{total_rows} tokens of the 4096-token workload in blocks of {rows} "
                      f"(rotate + quantize + fp64 product from codes), {elapsed:.1f} s"}


def rotation_ablation(rbp, torch, dev, stream, M=16384, d=4096, h=128, n=20):
    """The rotation variants of OrbitQuant's ablation (page, Experiments) on
    the 16384 x 4096 bf16 activations of the int8 workload (d a power of two,
    so the full RHT applies): orbit_rotate (bf16 in, fp16 out) with RPBH
    (h = 128), Block-RHT (identity permutation) and the full RHT (h = d),
    against a dense Haar rotation done as one bf16 GEMM by torch (timing
    only; it is not part of the library).  Microseconds per launch."""
    import synth
    perm, signs = synth.rotation_params(d, 4096)
    g = torch.Generator(device=dev).manual_seed(3)
    X = torch.randn((M, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((M, d), dtype=torch.float16, device=dev)
    Q = torch.linalg.qr(torch.randn((d, d), generator=g, device=dev))[0].to(torch.bfloat16)
    rots = {"rpbh_h128": rbp.Rotation(perm, signs, h),
            "block_rht_h128": rbp.Rotation(np.arange(d, dtype=np.int32), signs, h),
            "full_rht_h4096": rbp.Rotation(perm, signs, d)}

    def timed(fn):
        for _ in range(3):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    res = {k: round(timed(lambda r=r: rbp.rotate(r, X, out_dtype=torch.float16, out=out)), 2)
           for k, r in rots.items()}
    res["haar_dense_bf16_gemm"] = round(timed(lambda: torch.matmul(X, Q)), 2)
    res["bytes_per_launch"] = M * d * 4
    res["unit"] = "us"
    return res


def mlp_pair(rbp, torch, dev, stream, n=3):
    """The DiT MLP pair at its real shape: 16384 tokens, up 3072 -> 12288
    (W2A4, h = 256), GELU, down 12288 -> 3072 (W2A4, h = 256, 48 blocks).
    Fused: GELU in the up GEMM's epilogue and the down layer's permutation
    folded into the up layer's weight rows, so the down quantizer runs with
    the identity permutation on the up output as written.  Unfused: the up
    GEMM, a separate GELU pass (torch, bf16 in and out), the down quantizer
    with its permutation.  Microseconds per pair and effective TFLOP/s."""
    import synth
    inp = synth.make(4)
    M, K, N = inp["M"], inp["K"], inp["N"]
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    X, W_up, W_dn = to(inp["X"]), to(inp["W"]), to(inp["W2"])
    perm2 = inp["perm2"]
    rot_up = rbp.Rotation(inp["perm"], inp["signs"], 256)
    rot_dn = rbp.Rotation(perm2, inp["signs2"], 256)
    rot_dn_f = rbp.Rotation(np.arange(N, dtype=np.int32), inp["signs2"], 256)
    ca_up, cw_up = rbp.Codebook(K, 4), rbp.Codebook(K, 2)
    ca_dn, cw_dn = rbp.Codebook(N, 4), rbp.Codebook(N, 2)
    iw_up, r_up = rbp.pack_weights(rot_up, cw_up, W_up)
    iw_upf, r_upf = rbp.pack_weights(rot_up, cw_up,
                                     W_up[torch.from_numpy(perm2).long().to(dev)].contiguous())
    iw_dn, r_dn = rbp.pack_weights(rot_dn, cw_dn, W_dn)
    H = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def fused():
        ia, s = rbp.quant_act(rot_up, ca_up, X)
        rbp.qlinear(ia, s, ca_up, iw_upf, r_upf, cw_up, K, out=H, act="gelu")
        ib, s2 = rbp.quant_act(rot_dn_f, ca_dn, H)
        rbp.qlinear(ib, s2, ca_dn, iw_dn, r_dn, cw_dn, N, out=out)

    def unfused():
        ia, s = rbp.quant_act(rot_up, ca_up, X)
        rbp.qlinear(ia, s, ca_up, iw_up, r_up, cw_up, K, out=H)
        G = torch.nn.functional.gelu(H)
        ib, s2 = rbp.quant_act(rot_dn, ca_dn, G)
        rbp.qlinear(ib, s2, ca_dn, iw_dn, r_dn, cw_dn, N, out=out)

    def timed(fn):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    tf, tu = timed(fused), timed(unfused)
    flops = 2.0 * 2 * M * K * N
    return {"workload": "MLP pair W2A4: 16384 tokens, 3072 -> 12288 -> 3072, h = 256, GELU",
            "fused_us": round(tf, 1), "unfused_us": round(tu, 1),
            "fused_tflops": round(flops / tf / 1e6, 1), "unfused_tflops": round(flops / tu / 1e6, 1)}


def weight_only(rbp, torch, dev, stream, n=10):
    """The per-group rotated weight-only paths, int8 and its int4 sibling,
    on two shapes: the int8 workload (16384 tokens, 4096 -> 4096, h = 128;
    compute-bound) and an AdaLN-style projection (16 conditioning vectors,
    3072 -> 18432; bound by the weight stream).  Per shape: the rotation of
    the activations (bf16 -> fp16) and each GEMM in microseconds per launch,
    with TFLOP/s and the weight bytes streamed per microsecond (GB/s)."""
    import synth

    def timed(fn):
        for _ in range(2):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    res = {}
    for name, (M, K, N) in (("int8_workload_16384x4096x4096", (16384, 4096, 4096)),
                            ("adaln_16x3072x18432", (16, 3072, 18432))):
        perm, signs = synth.rotation_params(K, 7)
        g = torch.Generator(device=dev).manual_seed(5)
        X = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        W = (torch.randn((N, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
        rot = rbp.Rotation(perm, signs, 128)
        q8, s8 = rbp.int8_pack_weights(rot, W, 128)
        q4, s4 = rbp.int4_pack_weights(rot, W, 128)
        xr = rbp.rotate(rot, X, out_dtype=torch.float16)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_rot = timed(lambda: rbp.rotate(rot, X, out_dtype=torch.float16, out=xr))
        t8 = timed(lambda: rbp.int8_linear(xr, q8, s8, 128, out=out))
        t4 = timed(lambda: rbp.int4_linear(xr, q4, s4, 128, out=out))
        flops = 2.0 * M * K * N
        res[name] = {"rotate_us": round(t_rot, 2),
                     "w8a16_us": round(t8, 2), "w4a16_us": round(t4, 2),
                     "w8a16_tflops": round(flops / t8 / 1e6, 1),
                     "w4a16_tflops": round(flops / t4 / 1e6, 1),
                     "w8_weight_gbps": round(N * K / t8 / 1e3, 1),
                     "w4_weight_gbps": round(N * K / 2 / t4 / 1e3, 1)}
    return res


def video_layer(rbp, torch, dev, stream, n=10):
    """The video-DiT projection (32768 tokens, 2048 -> 8192, h = 128, 64-level
    activation and 16-level weight codebooks, W4A6): the fused rotate +
    quantize and the decode GEMM, microseconds per launch with HBM GB/s and
    TFLOP/s."""
    import synth
    inp = synth.make(5)
    M, K, N = inp["M"], inp["K"], inp["N"]
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    X, W = to(inp["X"]), to(inp["W"])
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    ca, cw = rbp.Codebook(K, inp["bits_a"]), rbp.Codebook(K, inp["bits_w"])
    iw, r = rbp.pack_weights(rot, cw, W)
    ia, s = rbp.quant_act(rot, ca, X)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    tq = timed(lambda: rbp.quant_act(rot, ca, X))
    tg = timed(lambda: rbp.qlinear(ia, s, ca, iw, r, cw, K, out=out))
    qbytes = M * K * 2 + M * K * inp["bits_a"] // 8 + M * 4
    return {"workload": "video-DiT projection W4A6: 32768 tokens, 2048 -> 8192, h = 128",
            "quant_us": round(tq, 2), "quant_gbps": round(qbytes / tq / 1e3, 1),
            "gemm_us": round(tg, 2), "gemm_tflops": round(2.0 * M * N * K / tg / 1e6, 1)}


def source_digest(files):
    """sha256 over the kernel sources a traffic measurement was taken with."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(entry):
    """HBM bytes per launch from the counter passes (FETCH_SIZE and WRITE_SIZE,
    each scaled by what it reads for a copy of known size), or None when the
    kernel sources changed since the counters were taken."""
    if not entry or source_digest(entry["sources"]) != entry["source_digest"]:
        return None
    return int(round(entry["fetch_kib"] * 1024 * entry["fetch_scale"] +
                     entry["write_kib"] * 1024 * entry["write_scale"]))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path is not "
              "sharded across GPUs in this build", file=sys.stderr)
        sys.exit(2)
    import torch
    import rotation_bit_ptq_amd as rbp
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make(2)
    M, K, N, h = inp["M"], inp["K"], inp["N"], inp["h"]

    rot = rbp.Rotation(inp["perm"], inp["signs"], h, dev)
    cb = rbp.Codebook(K, 4)
    x_bytes = M * K * 2
    pool_n = max(2, POOL_BYTES // x_bytes)
    X0 = torch.from_numpy(inp["X"].view(np.int16)).view(torch.bfloat16).to(dev)
    pool = [X0] + [X0.clone() for _ in range(pool_n - 1)]
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    iw, r = rbp.pack_weights(rot, cb, W)           # offline

    idx_a = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    import ctypes
    lib = rbp.lib
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def quant(X):
        st = lib.orbit_quant_act(ctypes.byref(rot.struct), ctypes.byref(cb.struct),
                                 ctypes.c_void_p(X.data_ptr()), 1, M, K, inp["eps"],
                                 ctypes.c_void_p(idx_a.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                 None, sp)
        assert st == 0, st

    def gemm():
        st = lib.orbit_qlinear(ctypes.c_void_p(idx_a.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                               ctypes.byref(cb.struct), ctypes.c_void_p(iw.data_ptr()),
                               ctypes.c_void_p(r.data_ptr()), ctypes.byref(cb.struct), None, 0,
                               M, N, K, ctypes.c_void_p(out.data_ptr()), 1, sp)
        assert st == 0, st

    if args.only is not None:
        # one kernel alone, for rocprofv3 counter passes (no timing line)
        if args.only == "copy":
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            step = lambda i: dst.copy_(src)  # noqa: E731
        elif args.only == "quant":
            step = lambda i: quant(pool[i % pool_n])  # noqa: E731
        else:
            quant(pool[0])
            step = lambda i: gemm()  # noqa: E731
        for i in range(args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "launches": args.warmup + args.steps,
                          "copy_bytes": COPY_BYTES if args.only == "copy" else None}), flush=True)
        return

    for i in range(args.warmup):
        quant(pool[i % pool_n])
        gemm()
    torch.cuda.synchronize()

    # the timed steps: nothing but the two launches per step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        quant(pool[i % pool_n])
        gemm()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same steps again with events between the kernels, for the split
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        quant(pool[i % pool_n])
        e[1].record(stream)
        gemm()
        e[2].record(stream)
    torch.cuda.synchronize()
    tq_step = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    tg_step = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    ms_per_step = wall / args.steps * 1e3
    flops = 2.0 * M * N * K
    quant_bytes = M * K * 2 + M * K // 2 + M * 4      # bf16 in, 4-bit codes + fp32 s out
    value = flops / (wall / args.steps) / 1e12

    # Per-kernel launch duration for the rooflines: the same kernels launched
    # back to back on the same stream, events around the whole run, so the
    # figure is the kernel's own duration (what a kernel trace reports)
    # rather than the kernel plus the event overhead of the step loop.  Back
    # to back, the GEMM finds its codes in L2 from its previous launch; in the
    # steps the quantizer's stream has evicted them and a kernel trace shows
    # it ~4 % slower there (the step_*_us fields carry the event-split step
    # figures, which include the events' own overhead).
    def per_launch(fn, n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    n_kern = max(args.steps, 20)
    tq = per_launch(lambda i: quant(pool[i % pool_n]), n_kern)
    tg = per_launch(lambda i: gemm(), n_kern)
    gemm_tflops = flops / tg / 1e12
    quant_gbps = quant_bytes / tq / 1e9

    traffic_gemm = traffic_quant = None
    if os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic))
            traffic_gemm = measured_traffic(tr.get("qlinear_gemm"))
            traffic_quant = measured_traffic(tr.get("quant_act"))
        except Exception:  # noqa: BLE001
            traffic_gemm = traffic_quant = None

    line = {
        "metric": "W4A4 RPBH qlinear effective TFLOP/s + rotate/quant stage HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "image-DiT projection W4A4: 4096 bf16 tokens x d_in 3072 -> "
                               "d_out 3072, RPBH h=128, 16-level act/weight codebooks, bf16 out",
                   "tokens": M, "d_in": K, "d_out": N, "h": h, "bits_a": 4, "bits_w": 4},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_MFMA_F16,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_MFMA_F16, 4),
                     "traffic": traffic_gemm, "kernel": "orbit_qlinear (codebook-decode GEMM)"},
        "roofline_quant": {"bound": "hbm", "achieved": round(quant_gbps, 1), "peak": PEAK_HBM,
                           "unit": "GB/s", "frac": round(quant_gbps / PEAK_HBM, 4),
                           "traffic": traffic_quant,
                           "kernel": "orbit_quant_act (fused rotate + quantize)",
                           "bytes_per_launch": quant_bytes},
        "gemm_us": round(tg * 1e6, 2),
        "quant_us": round(tq * 1e6, 2),
        "step_gemm_us": round(tg_step.mean() * 1e6, 2),
        "step_quant_us": round(tq_step.mean() * 1e6, 2),
        "quant_gbps": round(quant_gbps, 1),
        "gemm_tflops": round(gemm_tflops, 2),
    }
    line["rotation_ablation"] = rotation_ablation(rbp, torch, dev, stream)
    line["mlp_pair"] = mlp_pair(rbp, torch, dev, stream)
    line["weight_only"] = weight_only(rbp, torch, dev, stream)
    line["video_layer"] = video_layer(rbp, torch, dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="run the step loop untimed for this much device time before the "
                         "warm-up steps, so that the timed steps see the clock the matrix "
                         "cores hold under sustained load (0: no settling)")
    ap.add_argument("--traffic", default=os.path.join(HERE, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters")
    ap.add_argument("--only", choices=["quant", "gemm", "copy", "mfma", "video_quant",
                                       "video_gemm", "full_rht", "w8a16", "w4a16",
                                       "w8a16_narrow", "w4a16_narrow", "mlp_up_gemm"], default=None,
                    help="launch only one kernel --steps times (for counter runs): the "
                         "activation rotate+quantize, the decode GEMM, a plain device "
                         "copy of COPY_BYTES that calibrates FETCH_SIZE / WRITE_SIZE, "
                         "the matrix-core loop of the measured MFMA ceiling, the video "
                         "projection's quantizer or GEMM, the full RHT (h = d = 4096) "
                         "of the rotation ablation, a weight-only GEMM (int8 workload, "
                         "or the AdaLN-style shape with _narrow), or the MLP pair's up GEMM")
    return ap.parse_args()


COPY_BYTES = 256 << 20   # calibration copy: 256 MiB read + 256 MiB written per launch


def cpu_baseline(inp, gpu_idx, gpu_s, rounds_target_s=10.0, block=512):
    """The oracle as it stands, on this host's cores: rotate + quantize the
    activations and the fp64 product from codes, over the workload's tokens
    in blocks of `block`, in order, for whole passes over all the tokens
    until about `rounds_target_s` seconds have passed (at most 30 passes;
    the weights are packed once beforehand, untimed).

    The same leg compares the GPU's activation codes and norms for every
    token the oracle quantized with the oracle's own (the parity rule of the
    method's codes: mismatches only inside the 1e-6 decision band), which is
    where code_mismatch_frac and band_frac come from."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = int(os.environ.get("OMP_NUM_THREADS", cores))
    X64 = oracle.bf16_bits_to_f64(inp["X"])
    W64 = oracle.bf16_bits_to_f64(inp["W"])
    cb = oracle.codebook(4)
    w = oracle.pack_weights(W64, inp["perm"], inp["signs"], inp["h"], cb, 4)  # offline, untimed
    M, K, N = inp["M"], inp["K"], inp["N"]
    mism = {"f64": 0, "f32": 0}
    outside = band = n_codes = 0
    s_err = 0.0

    def run(lo, hi):
        a = oracle.quant_act(X64[lo:hi], inp["perm"], inp["signs"], inp["h"], cb, 4, inp["eps"])
        oracle.qlinear_codes(a["idx"], a["s"], cb["centroids"], w["idx"], w["r_bf16"],
                             cb["centroids"], K)
        return a

    run(0, 64)  # warm-up
    blocks, elapsed, nb, passes = M // block, 0.0, 0, 0
    t0 = time.perf_counter()
    checks = []
    while passes < 30 and (passes == 0 or elapsed < rounds_target_s):
        for b in range(blocks):
            lo, hi = b * block, (b + 1) * block
            a = run(lo, hi)
            if passes == 0:
                checks.append((lo, hi, a))
            nb += 1
        passes += 1
        elapsed = time.perf_counter() - t0
    # the parity check, outside the timed oracle work
    for lo, hi, a in checks:
        got = oracle.unpack_indices(gpu_idx[lo:hi], 4, K)
        near = oracle.boundary_band(a["u"], cb["thresholds"], 1e-6)
        for dec in mism:
            bad = got != oracle.quantize_codes(a["u"], cb["thresholds"], dec)
            mism[dec] += int(bad.sum())
            outside += int((bad & ~near).sum())
        band += int(near.sum())
        n_codes += got.size
        s_err = max(s_err, float(np.max(np.abs(gpu_s[lo:hi] - a["s"]) / a["s"])))
    tokens = nb * block
    flops = 2.0 * tokens * N * K
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": f"{passes} whole passes over all {blocks * block} tokens of the workload "
                      f"in blocks of {block} ({tokens} tokens: rotate + quantize + fp64 "
                      f"product from codes against all {N} packed weight rows), "
                      f"{elapsed:.1f} s"}, {
        "tokens_checked": blocks * block, "codes_checked": n_codes,
        "code_mismatch_frac": mism["f64"] / max(n_codes, 1),
        "code_mismatch_frac_f32_decision": mism["f32"] / max(n_codes, 1),
        "mismatches_outside_band": outside,
        "band_frac": band / max(n_codes, 1),
        "s_max_rel_err": s_err}


def settled_launch_us(torch, stream, fn, n, warmup=5, runs=3):
    """Microseconds per launch of fn on the launching stream: the median of
    `runs` runs of n back-to-back launches (events around each run) after
    `warmup` launches, over which the clock settles."""
    for _ in range(warmup):
        fn()
    per = []
    for _ in range(runs):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / n)
    return sorted(per)[len(per) // 2]


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
        return settled_launch_us(torch, stream, fn, n)

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
        return settled_launch_us(torch, stream, fn, n)

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
    the activations (bf16 -> fp16) and each GEMM in microseconds per launch
    (the same weights every launch), with TFLOP/s and the weight bytes
    streamed per microsecond (GB/s)."""
    import synth

    def timed(fn):
        return settled_launch_us(torch, stream, fn, n)

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
        return settled_launch_us(torch, stream, fn, n)

    tq = timed(lambda: rbp.quant_act(rot, ca, X))
    tg = timed(lambda: rbp.qlinear(ia, s, ca, iw, r, cw, K, out=out))
    qbytes = M * K * 2 + M * K * inp["bits_a"] // 8 + M * 4
    return {"workload": "video-DiT projection W4A6: 32768 tokens, 2048 -> 8192, h = 128",
            "quant_us": round(tq, 2), "quant_gbps": round(qbytes / tq / 1e3, 1),
            "gemm_us": round(tg, 2), "gemm_tflops": round(2.0 * M * N * K / tg / 1e6, 1)}


def other_kernel(rbp, torch, dev, which):
    """One launch of the video projection's quantizer or GEMM, of the full
    RHT of the rotation ablation, of a weight-only GEMM (the int8
    workload's 16384 x 4096 -> 4096, or the AdaLN-style 16 x 3072 -> 18432
    with _narrow), or of the MLP pair's up GEMM (16384 x 3072 -> 12288,
    W2A4, GELU), as a function of the step, for the counter passes of
    --only."""
    import synth
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    if which == "mlp_up_gemm":
        inp = synth.make(4)
        M, K, N = inp["M"], inp["K"], inp["N"]
        rot = rbp.Rotation(inp["perm"], inp["signs"], 256)
        ca, cw = rbp.Codebook(K, 4), rbp.Codebook(K, 2)
        iw, r = rbp.pack_weights(rot, cw, to(inp["W"]))
        ia, s = rbp.quant_act(rot, ca, to(inp["X"]))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        return lambda i: rbp.qlinear(ia, s, ca, iw, r, cw, K, out=out, act="gelu")
    if which.startswith(("w8a16", "w4a16")):
        M, K, N = (16, 3072, 18432) if which.endswith("_narrow") else (16384, 4096, 4096)
        perm, signs = synth.rotation_params(K, 7)
        g = torch.Generator(device=dev).manual_seed(5)
        X = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        W = (torch.randn((N, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
        rot = rbp.Rotation(perm, signs, 128)
        pack, linear = ((rbp.int8_pack_weights, rbp.int8_linear) if which.startswith("w8")
                        else (rbp.int4_pack_weights, rbp.int4_linear))
        q, sc = pack(rot, W, 128)
        xr = rbp.rotate(rot, X, out_dtype=torch.float16)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        return lambda i: linear(xr, q, sc, 128, out=out)
    if which == "full_rht":
        M, d = 16384, 4096
        perm, signs = synth.rotation_params(d, 4096)
        g = torch.Generator(device=dev).manual_seed(3)
        X = torch.randn((M, d), generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty((M, d), dtype=torch.float16, device=dev)
        rot = rbp.Rotation(perm, signs, d)
        return lambda i: rbp.rotate(rot, X, out_dtype=torch.float16, out=out)
    inp = synth.make(5)
    K = inp["K"]
    X, W = to(inp["X"]), to(inp["W"])
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    ca, cw = rbp.Codebook(K, inp["bits_a"]), rbp.Codebook(K, inp["bits_w"])
    if which == "video_quant":
        return lambda i: rbp.quant_act(rot, ca, X)
    iw, r = rbp.pack_weights(rot, cw, W)
    ia, s = rbp.quant_act(rot, ca, X)
    out = torch.empty((inp["M"], inp["N"]), dtype=torch.bfloat16, device=dev)
    return lambda i: rbp.qlinear(ia, s, ca, iw, r, cw, K, out=out)


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


def launch_stats(torch, stream, fn, n):
    """Kernel time on the launching stream: the mean over n back-to-back
    launches (events around the whole run, as a kernel trace averages), and
    the median / p10 / p90 of n launches each bracketed by its own events
    (those include the events' own overhead)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    b.synchronize()
    mean = a.elapsed_time(b) * 1e3 / n
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    return {"mean_us": round(mean, 3), "median_us": round(float(np.median(t)), 3),
            "p10_us": round(float(np.percentile(t, 10)), 3),
            "p90_us": round(float(np.percentile(t, 90)), 3)}


def quant_neighbours(torch, dev, stream, quant, gemm, pool, n=40):
    """The quantizer's launch time (median of launches each bracketed by its
    own events) alone and right after three different kernels: the GEMM as in
    the step, a loop of random-operand MFMAs of about the GEMM's length (the
    matrix cores' load without the GEMM's memory traffic), and a 25 MiB device
    copy (memory traffic without matrix work).  Microseconds."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(HERE, "rotation_bit_ptq_amd", "libpeaks.so"))
    lib.peaks_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(11)
    seed = torch.randn(4096 * 8, generator=g, device=dev).to(torch.float16)
    sink = torch.empty(n_cu * 2 * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def mfma(trips):
        assert lib.peaks_mfma_loop(ctypes.c_void_p(seed.data_ptr()), trips, 1,
                                   ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(clocks.data_ptr()), sp) == 0
    src = torch.empty(25 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gemm()
    a.record(stream)
    gemm()
    b.record(stream)
    b.synchronize()
    t_gemm = a.elapsed_time(b) * 1e3
    a.record(stream)
    mfma(1000)
    b.record(stream)
    b.synchronize()
    trips = max(50, int(1000 * t_gemm / (a.elapsed_time(b) * 1e3)))

    def timed(pre):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (e0, e1) in enumerate(ev):
            if pre is not None:
                pre()
            e0.record(stream)
            quant(pool[i % len(pool)])
            e1.record(stream)
        torch.cuda.synchronize()
        return round(float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])), 2)
    return {"alone": timed(None), "after_gemm": timed(gemm), "after_mfma_loop": timed(lambda: mfma(trips)),
            "after_copy_25MiB": timed(lambda: dst.copy_(src)), "unit": "us (median, events per launch)"}


def measured_peaks(torch, dev, stream, trips=20000, chains_sweep=False):
    """Ceilings measured on this device: a plain device copy (HBM read +
    write) and a loop of fp16 matrix-core products from registers (random
    normal operands, which set the clock the matrix cores run at under
    load, and constant ones), with the shader clock over the loop.  With
    chains_sweep, also the random-operand loop with 4, 8, 12 and 16
    independent accumulators per wave, at one and two waves per SIMD."""
    import ctypes
    res = {}
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    st = launch_stats(torch, stream, lambda i: dst.copy_(src), 10)
    res["copy_gbps"] = round(2 * COPY_BYTES / st["mean_us"] / 1e3, 1)
    del src, dst
    lib = ctypes.CDLL(os.path.join(HERE, "rotation_bit_ptq_amd", "libpeaks.so"))
    lib.peaks_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    chains = lib.peaks_mfma_chains()
    wall_ghz = lib.peaks_wall_clock_khz() * 1e-6
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(11)
    seeds = {"random": torch.randn(4096 * 8, generator=g, device=dev).to(torch.float16),
             "constant": torch.full((4096 * 8,), 0.5, device=dev, dtype=torch.float16)}
    sink = torch.empty(n_cu * 2 * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    # warm-up: the first loops after other work run before the shader clock
    # has settled (measured 1.46 against 1.71 PFLOP/s for the same loop run
    # first and second), so ~40 ms of the random-operand loop go first
    for _ in range(6):
        assert lib.peaks_mfma_loop(ctypes.c_void_p(seeds["random"].data_ptr()), trips, 1,
                                   ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(clocks.data_ptr()), sp) == 0
    for kind, seed in seeds.items():
        for wps in (1, 2):
            run = lambda i: lib.peaks_mfma_loop(ctypes.c_void_p(seed.data_ptr()), trips, wps,  # noqa: E731
                                                ctypes.c_void_p(sink.data_ptr()),
                                                ctypes.c_void_p(clocks.data_ptr()), sp)
            assert run(0) == 0
            st = launch_stats(torch, stream, run, 5)
            flops = 2.0 * 32 * 32 * 16 * chains * trips * n_cu * 4 * wps
            ck = clocks.cpu().numpy()
            res[f"mfma_{kind}_{wps}w_tflops"] = round(flops / st["mean_us"] / 1e6, 1)
            res[f"mfma_{kind}_{wps}w_sclk_ghz"] = round(float(ck[0]) / float(ck[1]) * wall_ghz, 3)
    if chains_sweep:
        lib.peaks_mfma_loop_chains.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        sweep = {}
        for ch in (4, 8, 12, 16):
            for wps in (1, 2):
                tr = trips * 4 // ch  # the same products per wave
                run = lambda i: lib.peaks_mfma_loop_chains(  # noqa: E731
                    ctypes.c_void_p(seeds["random"].data_ptr()), tr, wps, ch,
                    ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), sp)
                assert run(0) == 0
                st = launch_stats(torch, stream, run, 5)
                flops = 2.0 * 32 * 32 * 16 * ch * tr * n_cu * 4 * wps
                ck = clocks.cpu().numpy()
                sweep[f"{ch}_chains_{wps}w"] = {
                    "tflops": round(flops / st["mean_us"] / 1e6, 1),
                    "sclk_ghz": round(float(ck[0]) / float(ck[1]) * wall_ghz, 3)}
        res["mfma_random_chains"] = sweep
    # LDS reads per compute unit and shader clock (eight waves, independent
    # reads, no bank conflicts): 4-byte lanes as a decode lookup, 16-byte
    # lanes as an MFMA operand
    lib.peaks_lds_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lsink = torch.empty(n_cu * 512, dtype=torch.int32, device=dev)
    cyc = torch.zeros(n_cu, dtype=torch.int64, device=dev)
    for kind, lane_bytes in ((0, 4), (1, 16)):
        for _ in range(2):
            assert lib.peaks_lds_read(kind, 2048, ctypes.c_void_p(lsink.data_ptr()),
                                      ctypes.c_void_p(cyc.data_ptr()), sp) == 0
        torch.cuda.synchronize()
        mean_cycles = float(cyc.double().mean().item())
        res[f"lds_read_b{8 * lane_bytes}_bytes_per_clk_cu"] = round(8 * 2048 * 8 * 64 * lane_bytes / mean_cycles, 1)
    return res


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
        if args.only == "mfma":
            print(json.dumps({"only": "mfma", **measured_peaks(torch, dev, stream, chains_sweep=True)}),
                  flush=True)
            return
        if args.only == "copy":
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            step = lambda i: dst.copy_(src)  # noqa: E731
        elif args.only == "quant":
            step = lambda i: quant(pool[i % pool_n])  # noqa: E731
        elif args.only in ("video_quant", "video_gemm", "full_rht", "w8a16", "w4a16",
                           "w8a16_narrow", "w4a16_narrow", "mlp_up_gemm"):
            step = other_kernel(rbp, torch, dev, args.only)
        else:
            quant(pool[0])
            step = lambda i: gemm()  # noqa: E731
        for i in range(args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "launches": args.warmup + args.steps,
                          "copy_bytes": COPY_BYTES if args.only == "copy" else None}), flush=True)
        return

    # Settling.  From a lightly loaded device the first milliseconds of the
    # step loop run at a boosted clock, the power controller then pulls the
    # clock below its sustained level for several milliseconds (the GEMM
    # goes from ~70 us to ~86 us and back), and the step time settles after
    # ~50 ms.  A serving loop runs at the settled rate, so the step loop runs
    # untimed for settle_ms of device time first, in chunks of ten steps with
    # an event after each; the first and last chunks are reported.
    settle = None
    if args.settle_ms > 0:
        per, i = 10, 0
        chunks = []

        def enqueue_chunk():
            nonlocal i
            for _ in range(per):
                quant(pool[i % pool_n])
                gemm()
                i += 1
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e

        ev = [torch.cuda.Event(enable_timing=True)]
        ev[0].record(stream)
        ev.append(enqueue_chunk())
        done_ms = 0.0
        while done_ms < args.settle_ms and len(chunks) < 100000:
            ev.append(enqueue_chunk())   # the device stays busy while the host waits
            ev[-2].synchronize()
            ms = ev[-3].elapsed_time(ev[-2])
            chunks.append(ms * 1e3 / per)
            done_ms += ms
        # the first chunk also holds the kernels' first launches in the
        # process; the next ones show the clock's transient
        settle = {"device_ms": round(done_ms, 2), "steps": i, "chunk_steps": per,
                  "us_per_step_chunks_2_to_9": [round(c, 1) for c in chunks[1:9]],
                  "us_per_step_last_chunk": round(chunks[-1], 2)}

    for i in range(args.warmup):
        quant(pool[i % pool_n])
        gemm()
    torch.cuda.synchronize()

    # the timed steps: nothing but the two launches per step (and an event
    # on the stream at each end, which shows how much of the wall time the
    # device spent on them and how long the host took to enqueue them)
    e_first = torch.cuda.Event(enable_timing=True)
    e_last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_first.record(stream)
    for i in range(args.steps):
        quant(pool[i % pool_n])
        gemm()
    e_last.record(stream)
    enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    device_ms_per_step = e_first.elapsed_time(e_last) / args.steps

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
    n_kern = max(args.steps, 20)
    cold = launch_stats(torch, stream, lambda i: quant(pool[i % pool_n]), n_kern)
    warm = launch_stats(torch, stream, lambda i: quant(pool[0]), n_kern)
    gst = launch_stats(torch, stream, lambda i: gemm(), n_kern)
    tq, tg = cold["mean_us"] * 1e-6, gst["mean_us"] * 1e-6
    gemm_tflops = flops / tg / 1e12
    quant_gbps = quant_bytes / tq / 1e9
    peaks = measured_peaks(torch, dev, stream)
    mfma_ceiling = peaks["mfma_random_1w_tflops"]

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
                     "traffic": traffic_gemm, "kernel": "orbit_qlinear (codebook-decode GEMM)",
                     "flops_per_launch": flops,
                     "peak_measured": mfma_ceiling,
                     "frac_of_measured": round(gemm_tflops / mfma_ceiling, 4)},
        "roofline_quant": {"bound": "hbm", "achieved": round(quant_gbps, 1), "peak": PEAK_HBM,
                           "unit": "GB/s", "frac": round(quant_gbps / PEAK_HBM, 4),
                           "traffic": traffic_quant,
                           "kernel": "orbit_quant_act (fused rotate + quantize)",
                           "bytes_per_launch": quant_bytes,
                           "peak_measured": peaks["copy_gbps"],
                           "frac_of_measured": round(quant_gbps / peaks["copy_gbps"], 4)},
        "gemm_us": round(tg * 1e6, 2),
        "quant_us": round(tq * 1e6, 2),
        "quant_cold": cold,
        "quant_warm": warm,
        "quant_warm_gbps": round(quant_bytes / warm["mean_us"] / 1e3, 1),
        "gemm_launch": gst,
        "measured_peaks": peaks,
        "settle": settle,
        "step_device_ms": round(device_ms_per_step, 5),
        "step_host_enqueue_ms": round(enqueue / args.steps * 1e3, 5),
        "step_gemm_us": round(tg_step.mean() * 1e6, 2),
        "step_quant_us": round(tq_step.mean() * 1e6, 2),
        "quant_gbps": round(quant_gbps, 1),
        "gemm_tflops": round(gemm_tflops, 2),
    }
    line["quant_after"] = quant_neighbours(torch, dev, stream, quant, gemm, pool)
    line["rotation_ablation"] = rotation_ablation(rbp, torch, dev, stream)
    line["mlp_pair"] = mlp_pair(rbp, torch, dev, stream)
    line["weight_only"] = weight_only(rbp, torch, dev, stream)
    line["video_layer"] = video_layer(rbp, torch, dev, stream)
    if not args.no_cpu_baseline:
        quant(pool[0])
        torch.cuda.synchronize()
        line["cpu_baseline"], line["code_parity"] = cpu_baseline(
            inp, idx_a.cpu().numpy(), s.cpu().numpy().astype(np.float64))
        cp = line["code_parity"]
        # the method's bar for the codes: mismatches only inside the 1e-6
        # decision band, and both fractions below 1e-5
        cp["within_bar"] = bool(cp["mismatches_outside_band"] == 0 and
                                cp["code_mismatch_frac"] < 1e-5 and cp["band_frac"] < 1e-5)
    print(json.dumps(line), flush=True)
    if "code_parity" in line and not line["code_parity"]["within_bar"]:
        sys.exit("activation codes outside the parity bar: " + json.dumps(line["code_parity"]))


if __name__ == "__main__":
    main()

"""Benchmark: chunkwise gated delta rule forward on one MI355X.

One step = one gdn_chunk_fwd call over the "gdn" workload (B=2, H=16,
T=4096, Dk=Dv=128, chunk 64, bf16 q/k/v, fp32 gates, fp32 state, bf16
output o as the workload specifies; hT in fp32):
chunk-local cumsum, the intra-chunk beta*K*K^T with decay mask, the (I+A)^-1
solve, the WY form, the sequential inter-chunk state pass and the output
product - the whole hot path, in two kernel launches (the parallel per-chunk
solve, then the state pass with the output).  Inputs are generated once,
copied to HBM, and stay resident; only the launches are timed.

Prints ONE JSON line (rank 0) with the metric, a roofline object for one
gdn_chunk_fwd call (both kernels, timed live with HIP events on the launch
stream), and the fp64 CPU oracle timed on the host as a reported baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
KERNEL_SOURCES = ("chunkwise_gated_delta_gdn_amd/csrc/chunk_kernels.h",
                  "chunkwise_gated_delta_gdn_amd/csrc/chunk_prep2.h",
                  "chunkwise_gated_delta_gdn_amd/csrc/chunk_chain1.h",
                  "chunkwise_gated_delta_gdn_amd/csrc/chunk_dispatch.h",
                  "chunkwise_gated_delta_gdn_amd/csrc/gdn_common.h")
CAMERA_SOURCES = ("chunkwise_gated_delta_gdn_amd/csrc/prep.hip",
                  "chunkwise_gated_delta_gdn_amd/csrc/frame_scan.hip",
                  "chunkwise_gated_delta_gdn_amd/csrc/gdn_common.h")
BWD_SOURCES = ("chunkwise_gated_delta_gdn_amd/csrc/gdn_bwd.hip",
               "chunkwise_gated_delta_gdn_amd/csrc/chunk_bwd.h",
               "chunkwise_gated_delta_gdn_amd/csrc/chunk_bwd.hip",
               "chunkwise_gated_delta_gdn_amd/csrc/chunk_chain1.h",
               "chunkwise_gated_delta_gdn_amd/csrc/chunk_prep2.h",
               "chunkwise_gated_delta_gdn_amd/csrc/gdn_common.h")
# workload -> (rocprofv3 HBM counter record, kernel sources it was taken on)
TRAFFIC = {
    "gdn": (os.path.join(ROOT, "profiles", "chunk_fwd_kernel_gdn_traffic.json"), KERNEL_SOURCES),
    "camera": (os.path.join(ROOT, "profiles", "camera_prep_scan_traffic.json"), CAMERA_SOURCES),
    "camera_den": (os.path.join(ROOT, "profiles", "camera_prep_scan_den_traffic.json"), CAMERA_SOURCES),
    "gdn_bwd": (os.path.join(ROOT, "profiles", "gdn_bwd_traffic.json"), BWD_SOURCES),
    "deltaproduct": (os.path.join(ROOT, "profiles", "deltaproduct_traffic.json"), KERNEL_SOURCES),
    "deltaproduct_bwd": (os.path.join(ROOT, "profiles", "deltaproduct_bwd_traffic.json"), BWD_SOURCES),
    "camera_bwd": (os.path.join(ROOT, "profiles", "camera_bwd_traffic.json"), CAMERA_SOURCES),
}


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(B, T, H, Dk, Dv, C, in_bytes=2, out_bytes=4, with_h0=False):
    """Bytes: every input read once, every output written once.  FLOPs per
    (token, head): 10*C*d + 6*d^2 + 2*C^2/3 (five C x C x d tile products,
    three d x d state products, the triangular solve), d = Dk = Dv."""
    d = Dk
    nbytes = B * T * H * (2 * Dk + Dv) * in_bytes          # q, k, v
    nbytes += B * T * H * 2 * 4                             # beta, log_decay
    nbytes += B * T * H * Dv * out_bytes                    # o
    nbytes += B * H * Dk * Dv * 4 * (2 if with_h0 else 1)   # hT (and h0)
    flops = B * T * H * (10 * C * d + 6 * d * d + 2 * C * C / 3)
    return nbytes, flops


def measured_traffic(workload):
    """HBM bytes per step of a workload from the committed rocprofv3
    FETCH_SIZE and WRITE_SIZE counters, or None if there is no record or it
    was taken on other kernel source."""
    if workload not in TRAFFIC:
        return None
    path, sources = TRAFFIC[workload]
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(d, B, T, H, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on host cores over a bounded
    sample of heads of the same workload; scale to tokens/s of the whole."""
    import numpy as np
    import oracle
    threads = min(os.cpu_count() or 1, 16)
    # estimate: ~7*d^2 fp64 FLOP per token-head at ~1 GFLOP/s per thread
    per_head = 7 * d["q"].shape[-1] ** 2 * B * T / 1e9
    nheads = int(max(1, min(H, budget_s * threads / max(per_head, 1e-9))))
    hs = list(range(nheads))
    sub = {n: np.ascontiguousarray(d[n][:, :, hs]) for n in ("q", "k", "v", "beta", "g")}
    used = min(threads, B * nheads)
    # repeat the sample until it has held the cores for about budget_s of
    # CPU time in all (a whole fast sample alone is too short to time well)
    reps, dt = 0, 0.0
    while reps < 50 and (reps == 0 or dt * used < budget_s):
        t0 = time.perf_counter()
        oracle.gdn_recurrent(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"], 1.0, None,
                             nthreads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    # tokens/s of the whole workload: B*T tokens need H heads of work
    value = reps * B * T * (nheads / H) / dt
    return {"value": value, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cpu": host_cpu_model(), "nproc": os.cpu_count(),
            "sample": f"fp64 token recurrence on heads 0..{nheads - 1} of {H} (all B={B}, T={T}), "
                      f"{reps} run(s), {dt:.2f} s wall on {used} threads, scaled by {nheads}/{H}"}


def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def measured_peaks(dev, reps=10):
    """Achievable peaks on this device, measured next to the spec figures:
    HBM bandwidth of a plain 1 GiB device-to-device copy (read + write
    bytes over the time) and the bf16 rate of a large square matrix product
    (the vendor GEMM), each the best of `reps` runs timed with HIP events."""
    import torch
    n = 256 * 1024 * 1024                           # 1 GiB of fp32 each way
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    b = torch.randn((m, m), dtype=torch.bfloat16, device=dev)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)
    t_copy = best(lambda: dst.copy_(src))
    t_mm = best(lambda: torch.mm(a, b))
    out = {"hbm_copy_gbs": 2 * n * 4 / t_copy / 1e9, "bf16_gemm_tflops": 2 * m ** 3 / t_mm / 1e12,
           "how": "1 GiB device copy (read+write bytes / time); 8192^3 bf16 torch.mm; best of "
                  f"{reps}, HIP events"}
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


# workloads that time another operation on a named workload's inputs
BASE = {"camera_reverse": "camera", "camera_den": "camera", "camera_bwd": "camera", "gdn_bwd": "gdn",
        "deltaproduct_bwd": "deltaproduct"}


def _prepare(name, dev):
    """Inputs of a workload on the GPU and a step() closure that runs the
    workload's hot path once through the C ABI."""
    import torch
    from chunkwise_gated_delta_gdn_amd import gdn, inputs
    base = BASE.get(name, name)  # same inputs
    wl = inputs.WORKLOADS[base]
    d = inputs.workload_inputs(base)
    bf = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(x).to(dev)
    if name == "gdn_bwd":
        # gradients of the gdn workload's forward under seeded upstream gradients
        B, T, H, Dk, Dv = wl["B"], wl["T"], wl["H"], wl["Dk"], wl["Dv"]
        up = inputs.gdn_upstream(B, T, H, Dk, Dv, 20265, "bf16")
        q, k, v, dout = bf(d["q"]), bf(d["k"]), bf(d["v"]), bf(up["dout"])
        beta, g = f32(d["beta"]), f32(d["g"])

        def step():
            return gdn.gdn_bwd(q, k, v, beta, g, dout, Dk ** -0.5)
        # read q, k, v, dout (bf16), beta, g; write dq, dk, dv (fp32), dbeta, dg, dh0
        nbytes = B * T * H * ((2 * Dk + 2 * Dv) * 2 + 8 + (2 * Dk + Dv) * 4 + 8) + B * H * Dk * Dv * 4
        # per token and head: two forward recomputations (4 Dk Dv each) and the
        # backward step (12 Dk Dv), FLOPs
        flops = B * T * H * 20 * Dk * Dv
        return d, step, B * T, nbytes, flops
    if name == "deltaproduct_bwd":
        # gradients of the DeltaProduct workload's forward under seeded dout
        B, T, H, r, dk, Dv = wl["B"], wl["T"], wl["H"], wl["r"], wl["dk"], wl["Dv"]
        K = r * dk
        up = inputs.gdn_upstream(B, T, H, K, Dv, 20266, "bf16")
        q, k, v, dout = bf(d["q"]), bf(d["k"]), bf(d["v"]), bf(up["dout"])
        beta, g = f32(d["beta"]), f32(d["g"])

        def step():
            return gdn.deltaproduct_bwd(q, k, v, beta, g, d["mask"], dout, K ** -0.5)
        # read q, k (K), v, dout (Dv), bf16, beta (r), g; write dq, dk, dv (fp32),
        # dbeta (r), dg, dh0
        nbytes = (B * T * H * ((2 * K + 2 * Dv) * 2 + (r + 1) * 4 + (2 * K + Dv) * 4 + (r + 1) * 4)
                  + B * H * K * Dv * 4)
        # per token and head, per sub-key: two forward recomputations (4 dk Dv
        # each) and the backward step (12 dk Dv)
        flops = B * T * H * 20 * K * Dv
        return d, step, B * T, nbytes, flops
    if wl["kind"] == "gdn":
        q, k, v = bf(d["q"]), bf(d["k"]), bf(d["v"])
        beta, g = f32(d["beta"]), f32(d["g"])
        h0 = None if d["h0"] is None else f32(d["h0"])

        def step():
            return gdn.gdn_chunk_fwd(q, k, v, beta, g, 1.0, h0, chunk=wl["chunk"], out_dtype=torch.bfloat16)
        B, T, H = wl["B"], wl["T"], wl["H"]
        nbytes, flops = algorithmic_work(B, T, H, wl["Dk"], wl["Dv"], wl["chunk"], out_bytes=2,
                                         with_h0=h0 is not None)
        return d, step, B * T, nbytes, flops
    if wl["kind"] == "deltaproduct":
        q, k, v = bf(d["q"]), bf(d["k"]), bf(d["v"])
        beta, g = f32(d["beta"]), f32(d["g"])
        K = wl["r"] * wl["dk"]

        def step():
            return gdn.deltaproduct_chunk_fwd(q, k, v, beta, g, d["mask"], K ** -0.5, chunk=wl["chunk"],
                                              out_dtype=torch.bfloat16)
        B, T, H, r, Dv = wl["B"], wl["T"], wl["H"], wl["r"], wl["Dv"]
        nbytes = B * T * H * (2 * K + Dv) * 2 + B * T * H * (r + 1) * 4 + B * T * H * Dv * 2 + B * H * K * Dv * 4
        C, dk = wl["chunk"], wl["dk"]
        NR = C * r
        # per chunk: Gram r*C^2*dk, W/U NR^2*(K+Dv), state 2*NR*K*Dv, output 2*C*K*Dv + r*C^2*dk, all x2 FLOP
        per_chunk = 2 * (r * C * C * dk * 2 + NR * NR * (K + Dv) + 2 * NR * K * Dv + C * K * Dv) + 2 * NR ** 3 / 3
        flops = B * H * (T // C) * per_chunk
        return d, step, B * T, nbytes, flops
    if name == "camera_bwd":
        # gradients of the camera scan (forward direction) on the GPU prep's
        # outputs (formed once, outside the timed steps) under seeded dout
        import numpy as np
        t = {n: f32(d[n]) for n in ("q_norm_w", "k_norm_w", "proj_q", "proj_kv", "rope_cos", "rope_sin",
                                    "beta", "g")}
        pr = gdn.gdn_prep(bf(d["qkv"]), t["q_norm_w"], t["k_norm_w"], t["proj_q"], t["proj_kv"], t["rope_cos"],
                          t["rope_sin"], d["k_scale"], d["eps"])
        rng = np.random.default_rng(20263 + 7)
        dout = bf(inputs.cast(rng.standard_normal(tuple(pr["q"].shape)), "bf16"))

        qkv = bf(d["qkv"])

        def step():
            # the scan's backward, then the prep's backward on its gradients
            sg = gdn.gdn_recurrent_bwd(pr["q"], pr["k"], pr["v"], t["beta"], t["g"], dout, wl["F"], 1.0)
            return gdn.gdn_prep_bwd(qkv, t["q_norm_w"], t["k_norm_w"], t["proj_q"], t["proj_kv"], t["rope_cos"],
                                    t["rope_sin"], d["k_scale"], d["eps"], sg[0], sg[1], sg[2])
        B, F, S, H, D = wl["B"], wl["F"], wl["S"], wl["H"], wl["D"]
        N = F * S
        # scan backward: read q, k, v, dout (bf16), beta, g; write dq, dk, dv
        # (fp32), dbeta, dg, dh0.  Prep backward: read qkv (bf16), the three
        # fp32 gradients, projections, tables; write dqkv (fp32), projection
        # and weight gradients
        scan_bytes = B * H * N * (4 * D * 2 + 4 + 3 * D * 4 + 4) + B * H * F * 8 + B * H * D * D * 4
        prep_bytes = B * N * 3 * H * D * (2 + 4 + 4) + B * N * 32 * 4 * 2 + N * D * 4 + 2 * H * D * 4
        # per token: the forward's G and H (4 D^2), A (2 D^2), u and r (4 D^2),
        # dk (4 D^2), dq (2 D^2)
        flops = B * H * N * 16 * D * D
        return d, step, B * N, scan_bytes + prep_bytes, flops
    # camera: prep, then the frame-synchronous scan on its outputs (the
    # anti-causal direction for camera_reverse)
    reverse = name == "camera_reverse"
    qkv = bf(d["qkv"])
    t = {n: f32(d[n]) for n in ("q_norm_w", "k_norm_w", "proj_q", "proj_kv", "rope_cos", "rope_sin", "beta", "g")}

    with_den = name == "camera_den"

    def step():
        pr = gdn.gdn_prep(qkv, t["q_norm_w"], t["k_norm_w"], t["proj_q"], t["proj_kv"], t["rope_cos"],
                          t["rope_sin"], d["k_scale"], d["eps"])
        num = gdn.gdn_recurrent_fwd(pr["q"], pr["k"], pr["v"], t["beta"], t["g"], 1.0, reverse=reverse)
        if with_den:        # normaliser stream on the prep's q and k (stand-ins for its own rows)
            return num, gdn.gdn_recurrent_den_fwd(pr["q"], pr["k"], t["beta"], t["g"], 1.0)
        return num
    B, F, S, H, D = wl["B"], wl["F"], wl["S"], wl["H"], wl["D"]
    N = F * S
    prep_bytes = B * N * 3 * H * D * 2 * 2 + B * N * 32 * 4 + N * D * 4 + B * H * N * 3 * 4
    scan_bytes = B * H * N * D * 2 * 3 + B * H * N * 4 + B * H * N * D * 4 + (0 if reverse else B * H * D * D * 4)
    if with_den:            # q, k, beta read, den and zT written
        scan_bytes += B * H * N * D * 2 * 2 + B * H * N * 4 + B * H * N * 4 + B * H * D * 4
    flops = B * H * N * 4 * D * D * 2
    return d, step, B * N, prep_bytes + scan_bytes, flops


def copy_probe(dev, mib=512, reps=5):
    """A plain device-to-device copy of known size, for scaling the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="gdn", choices=("gdn", "gdn_long", "deltaproduct", "camera", "camera_reverse", "camera_den",
                             "gdn_bwd", "camera_bwd", "deltaproduct_bwd"),
                    help="gdn is the headline workload; the others time the other operations")
    ap.add_argument("--copy-probe", action="store_true", help="run only the copy calibration kernel")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 "
                                   "(every kernel here works on one device's share; nothing "
                                   "crosses GPUs)"}))
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(dev)
        return
    d, step, tokens, nbytes, flops = _prepare(args.workload, dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = float(np.mean(kern_ms))
    achieved_gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    from chunkwise_gated_delta_gdn_amd import inputs
    wl = inputs.WORKLOADS[BASE.get(args.workload, args.workload)]
    if args.workload == "gdn_bwd":
        metric = "tokens/sec of gated-delta backward (B*T/s) at H=16, D=128"
        desc = (f"gdn_bwd: gradients of the gdn workload (B={wl['B']} H={wl['H']} T={wl['T']} "
                f"Dk=Dv={wl['Dk']}), bf16 q/k/v/dout, fp32 gradients, no dhT")
        kernel = ("gdn_bwd = chunk_prep2_kernel<128, 64, bwd> + chunk_chain1_kernel<128, 64, 3> (forward states) "
                  "+ chunk_bchain_kernel<128> (reverse state pass) + chunk_bgrad_kernel<128> (per-chunk gradients)")
        traffic = measured_traffic(args.workload)
    elif args.workload == "deltaproduct_bwd":
        metric = "tokens/sec of gated DeltaProduct backward (B*T/s)"
        desc = ("deltaproduct_bwd: gradients of the deltaproduct workload (B=2 H=8 T=2048 K=2x128 Dv=128 r=2, "
                "lower-triangular step mask), bf16 q/k/v/dout, fp32 gradients, no dhT")
        kernel = ("deltaproduct_bwd = chunk_prep2_kernel<128, 64, bwd> (both sub-keys) + chunk_chain1_kernel<128, 64, 5> "
                  "and <128, 64, 4> (forward states, v') + chunk_bchain_kernel<128> and chunk_bgrad_kernel<128> "
                  "(sub-key 1), then their error-gradient forms <128, true> (sub-key 0)")
        traffic = measured_traffic(args.workload)
    elif args.workload == "camera_bwd":
        metric = "tokens/sec of camera scan + prep backward (B*N/s)"
        desc = ("camera_bwd: gradients of the camera workload (B=1 F=8 S=30x52 H=16 D=64): the scan's on the "
                "GPU prep's bf16 outputs under bf16 dout, then the prep's on those fp32 gradients (qkv, norm "
                "weights, projections)")
        kernel = ("gdn_recurrent_bwd (frame_gram_bf16_kernel for G, H and A, frame_reduce_kernel, frame_state_kernel, "
                  "frame_bstate_kernel, frame_bgrad_kernel) + gdn_prep_bwd (prep_bwd_kernel, prep_bwd_reduce_kernel)")
        traffic = measured_traffic(args.workload)
    elif args.workload in ("gdn", "gdn_long"):
        metric = "tokens/sec of chunkwise gated-delta fwd (B*T/s) at H=16, D=128"
        desc = (f"{args.workload}: B={wl['B']} H={wl['H']} T={wl['T']} Dk=Dv={wl['Dk']} chunk={wl['chunk']}, "
                f"bf16 q/k/v and output, fp32 gates and state, " + ("h0~N(0,0.02^2)" if wl["h0_std"] else "h0=0"))
        kernel = "gdn_chunk_fwd = chunk_prep2_kernel + chunk_chain1_kernel <KD=128, C=64>"
        traffic = measured_traffic(args.workload)
    elif args.workload == "deltaproduct":
        metric = "tokens/sec of chunkwise gated DeltaProduct fwd (B*T/s)"
        desc = "deltaproduct: B=2 H=8 T=2048 K=2x128 Dv=128 chunk=32 r=2, bf16 q/k/v and output, lower-triangular step mask"
        kernel = ("deltaproduct_chunk_fwd = chunk_prep2_kernel (both sub-keys) + chunk_chain1_kernel<128, 64, 1> "
                  "+ chunk_chain1_kernel<128, 64, 2> (two passes, lower unitriangular step mask)")
        traffic = measured_traffic(args.workload)
    else:
        rev = args.workload == "camera_reverse"
        metric = "tokens/sec of camera prep + frame-synchronous scan (B*N/s)"
        desc = ("camera: B=1 F=8 S=30x52 H=16 D=64, bf16 prep output, fp32 scan output"
                + (", reverse (anti-causal) scan" if rev else "")
                + (", plus the normaliser stream on the prep's q and k" if args.workload == "camera_den" else ""))
        kernel = "gdn_prep + gdn_recurrent_fwd (prep_kernel, frame_gram/state/out kernels)"
        traffic = measured_traffic(args.workload)
    rec = {
        "metric": metric,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generators of chunkwise_gated_delta_gdn_amd.inputs)",
        "config": {"workload": desc, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel, "kernel_ms": kernel_ms, "algorithmic_bytes": nbytes,
                     "algorithmic_flops": flops,
                     "mfma_tflops": flops / (kernel_ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }
    if args.workload in ("gdn", "gdn_long"):
        rec["config"].update({"global_batch": wl["B"], "seq_len": wl["T"], "heads": wl["H"],
                              "head_dim": wl["Dk"], "chunk": wl["chunk"]})
    mp = measured_peaks(dev)
    r = rec["roofline"]
    r["measured_peak"] = mp
    r["frac_of_measured_hbm"] = achieved_gbs / mp["hbm_copy_gbs"]
    r["mfma_frac_of_measured_gemm"] = r["mfma_tflops"] / mp["bf16_gemm_tflops"]
    if not args.no_cpu_baseline and args.workload == "gdn":
        rec["cpu_baseline"] = cpu_baseline(d, wl["B"], wl["T"], wl["H"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

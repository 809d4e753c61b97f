"""Benchmark of the HiF4 W4A4 hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
Wan2.2 FFN-up activations (57,600 video tokens x 5120 channels) and the
FFN-up weight (13,824 x 5120), each stage one C-ABI call:
  1. hif4_percentile_mask: per-channel type-7 99.9th percentile of |X| and
     the top-1% (52-channel) protection mask;
  2. hif4_quantize(W, mask): weight codes + meta, protected channels kept bf16;
  3. hif4_quantize(X, mask): the 4-bit activation stream, protected channels
     kept bf16;
  4. hif4_dequantize(W codes -> bf16): the weight operand, decoded once;
  5. hif4_linear_xcodes_wbf16(X codes, W, kept): the W4A4 contraction plus the
     bf16 residual over the 52 protected channels, Y fp32 [57600][13824]
     (two small packing kernels and one gemm_w4a4_u64_kernel launch, which
     decodes X per tile and adds the residual before its epilogue).
Inputs are resident in HBM before the timed region. `value` is whole-step
throughput counted as the linear layer's 2*M*N*K flops per step time.
`roofline` is the contraction kernel's, timed with HIP events on its stream;
its `traffic` comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
profiles/ and is reported only while the kernel source still hashes to the
value recorded there.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 HiF4 linear TFLOP/s + quantize GB/s, % of MI355X roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(x, w, mask_np, rows_sample):
    """The oracle, as it stands, on a bounded sample of the same step."""
    import numpy as np

    import oracle
    import workloads

    idx = np.linspace(0, x.shape[0] - 1, rows_sample).astype(np.int64)
    xs = workloads.bits(x[torch_index(idx)])
    wb = workloads.bits(w)
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    wc, wm, wk = oracle.quantize(wb, mask_np)
    xc, xm, xk = oracle.quantize(xs, mask_np)
    oracle.linear_protected(xc, xm, xk, wc, wm, wk, with_mag=False)
    dt = time.perf_counter() - t0
    n, k = w.shape
    flops = 2.0 * rows_sample * n * k
    omp = os.environ.get("OMP_NUM_THREADS")
    cores = min(threads, int(omp)) if omp and omp.isdigit() else threads
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{rows_sample} of {x.shape[0]} rows of X quantized (masked) + full W quantized "
                  f"(masked) + fp64 linear with the protected-channel residual on those rows; "
                  f"{dt:.1f} s",
    }


GEMM_SRC = os.path.join(ROOT, "bit_block_float_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a4_u64_kernel_ffn_up_traffic.txt")


def measured_traffic():
    """HBM bytes per launch of gemm_w4a4_u64_kernel from the committed counter
    summary, or None if it is missing or the kernel source has changed."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE, encoding="utf-8"):
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
        src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if fields.get("gemm.hip sha256") != src:
            return None
        return float(fields["traffic bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def torch_index(idx):
    import torch
    return torch.from_numpy(idx).to(torch.long)


def time_higptq(torch, workloads, hif4, dev, w_bf16, stream, reps=2):
    """HiGPTQ over the whole weight (80 groups of 64 columns), each of the
    three schemes: one untimed pass, then `reps` timed passes from the same
    start. Reported apart from the hot-path step (it is a calibration pass,
    run once per layer)."""
    spec = workloads.WORKLOADS["higptq"]
    n, k = w_bf16.shape
    u = workloads.higptq_factor(k, device="cuda", seed=spec["index"])
    w0 = w_bf16.float()
    w = torch.empty_like(w0)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    meta = torch.empty((n, k // 64), dtype=torch.int32, device=dev)
    ws = torch.empty((hif4.higptq_workspace_bytes(n),), dtype=torch.uint8, device=dev)
    units = k // 64
    # compensation per group: 2 n 64 flops and 8 bytes of W (read + write)
    # per element after the group, 64 (u + 1) .. k
    flops = sum(2.0 * n * 64 * (k - 64 * (g + 1)) for g in range(units))
    wbytes = sum(8.0 * n * (k - 64 * (g + 1)) for g in range(units))
    out = {"workload": f"W {n}x{k} (the FFN-up weight), random inverse-Hessian factor U {k}x{k}",
           "groups": units}
    for scheme in (1, 2, 3):
        times = []
        for rep in range(reps + 1):
            w.copy_(w0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for unit in range(units):
                hif4.higptq_unit(w, u, unit, codes, meta, workspace=ws, stream=stream,
                                 scheme=scheme)
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                times.append(e0.elapsed_time(e1))
        ms = sum(times) / len(times)
        log(f"HiGPTQ scheme {scheme} over W {n}x{k}: {ms:.2f} ms")
        # rates over the whole pass (group kernels included): the compensation
        # streams W, so its bound is HBM
        out[f"scheme{scheme}"] = {"ms": ms, "update_TFLOP/s": flops / (ms * 1e-3) / 1e12,
                                  "W_GB/s": wbytes / ms / 1e6,
                                  "frac_hbm": wbytes / ms / 1e6 / HBM_PEAK_GBS}
    return out


def time_autoround(torch, hif4, dev, w_bf16, stream, reps=10):
    """The quantize step of HiAutoRound (given offsets K per level-3 group, M
    per element) over the whole weight, as each iteration of its training loop
    runs it. Algorithmic bytes: read 2 (x) + 4 (M) + 1 (K) B per element,
    write 0.5 + 1/16 B (codes, meta)."""
    n, k = w_bf16.shape
    g = torch.Generator(device="cuda").manual_seed(5)
    koff = torch.rand((n, k // 4), generator=g, device=dev) * 5.0 - 2.5
    moff = torch.rand((n, k), generator=g, device=dev) * 2.0 - 1.0
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    meta = torch.empty((n, k // 64), dtype=torch.int32, device=dev)
    hif4.quantize_offsets(w_bf16, koff, moff, codes=codes, meta=meta, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        hif4.quantize_offsets(w_bf16, koff, moff, codes=codes, meta=meta, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = n * k * (2 + 4 + 1 + 0.5 + 1 / 16)
    log(f"HiAutoRound quantize step over W {n}x{k}: {ms:.3f} ms")
    return {"workload": f"W {n}x{k} bf16 (the FFN-up weight), K uniform in [-2.5, 2.5), "
                        "M uniform in [-1, 1)",
            "ms": ms, "GB/s": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / HBM_PEAK_GBS}


def time_calibration(torch, workloads, hif4, dev, stream, reps=3):
    """The calibration pass: percentile + top-n mask over 16 calibration
    batches (921,600 x 5120 bf16 = 9.4 GB), then the masked quantize of the
    13,824 x 5120 weight. Reported apart from the hot-path step."""
    spec = workloads.WORKLOADS["calib"]
    rows, c, n = spec["batches"] * spec["rows_per_batch"], spec["C"], spec["N"]
    x = workloads.calib_x(spec["batches"], spec["rows_per_batch"], c, device="cuda",
                          seed=spec["index"])
    w = workloads.normal_bf16(n, c, 0.02, device="cuda", seed=spec["index"] + 1000)
    stats = torch.empty((c,), dtype=torch.float32, device=dev)
    mask = torch.empty((c,), dtype=torch.uint8, device=dev)
    pws = torch.empty((hif4.percentile_workspace_bytes(rows, c),), dtype=torch.uint8, device=dev)
    codes = torch.empty((n, c // 2), dtype=torch.uint8, device=dev)
    meta = torch.empty((n, c // 64), dtype=torch.int32, device=dev)
    kept = torch.empty((n, spec["n_protect"]), dtype=torch.bfloat16, device=dev)
    tp, tq = [], []
    for rep in range(reps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        hif4.percentile_mask(x, spec["q"], spec["n_protect"], stats=stats, mask=mask,
                             workspace=pws, stream=stream)
        e[1].record(stream)
        st = hif4.lib().hif4_quantize(hif4._ptr(w), n, c, c, hif4._ptr(mask), spec["n_protect"],
                                      hif4._ptr(kept), hif4._ptr(codes), hif4._ptr(meta),
                                      hif4._stream(stream))
        hif4._ok(st, "hif4_quantize(W)")
        e[2].record(stream)
        torch.cuda.synchronize()
        if rep:
            tp.append(e[0].elapsed_time(e[1]))
            tq.append(e[1].elapsed_time(e[2]))
    t_p, t_q = sum(tp) / len(tp), sum(tq) / len(tq)
    pbytes = rows * c * 2
    log(f"calibration pass: percentile over {rows}x{c} {t_p:.2f} ms, masked W quantize {t_q:.3f} ms")
    del x
    return {"workload": f"{spec['batches']} batches x {spec['rows_per_batch']} x {c} bf16 "
                        f"(Student-t(2.5) x per-channel and per-batch LogNormal scales), q = "
                        f"{spec['q']}, {spec['n_protect']} protected; W {n}x{c}",
            "percentile_mask_ms": t_p, "percentile_GB/s": pbytes / t_p / 1e6,
            "percentile_frac_hbm": pbytes / t_p / 1e6 / HBM_PEAK_GBS,
            "percentile_exact_pass_channels": hif4.percentile_exact_channels(pws, rows, c),
            "quantize_w_masked_ms": t_q}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6144)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the HiGPTQ timing that follows the hot-path steps")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the kernels shard by rows; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from bit_block_float_amd import hif4

    hif4.require_gpu()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones((n,), dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: 3 copies of {args.copy_probe} MiB done")
        return
    spec = workloads.WORKLOADS["ffn_up"]
    M, N, K = spec["M"], spec["N"], spec["K"]
    q, n_protect = spec["q"], spec["n_protect"]

    log(f"generating inputs X {M}x{K}, W {N}x{K} on {torch.cuda.get_device_name(dev)}")
    x = workloads.heavy_tailed_x(M, K, device="cuda", seed=spec["index"])
    w = workloads.normal_bf16(N, K, 0.02, device="cuda", seed=spec["index"] + 1000)

    # outputs and workspaces allocated once, outside the timed region
    stats = torch.empty((K,), dtype=torch.float32, device=dev)
    mask = torch.empty((K,), dtype=torch.uint8, device=dev)
    pws = torch.empty((hif4.percentile_workspace_bytes(M, K),), dtype=torch.uint8, device=dev)
    wcodes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wmeta = torch.empty((N, K // 64), dtype=torch.int32, device=dev)
    kept = torch.empty((N, n_protect), dtype=torch.bfloat16, device=dev)
    xcodes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xmeta = torch.empty((M, K // 64), dtype=torch.int32, device=dev)
    xkept = torch.empty((M, n_protect), dtype=torch.bfloat16, device=dev)
    wdeq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    lws = torch.empty((hif4.linear_workspace_bytes(M, N, 0, n_protect),), dtype=torch.uint8,
                      device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev: ev[0].record(stream)
        hif4.percentile_mask(x, q, n_protect, stats=stats, mask=mask, workspace=pws, stream=stream)
        if ev: ev[1].record(stream)
        # the mask count is fixed by construction (n_protect); no host sync needed
        st = hif4.lib().hif4_quantize(hif4._ptr(w), N, K, K, hif4._ptr(mask), n_protect,
                                      hif4._ptr(kept), hif4._ptr(wcodes), hif4._ptr(wmeta),
                                      hif4._stream(stream))
        hif4._ok(st, "hif4_quantize(W)")
        if ev: ev[2].record(stream)
        st = hif4.lib().hif4_quantize(hif4._ptr(x), M, K, K, hif4._ptr(mask), n_protect,
                                      hif4._ptr(xkept), hif4._ptr(xcodes), hif4._ptr(xmeta),
                                      hif4._stream(stream))
        hif4._ok(st, "hif4_quantize(X)")
        if ev: ev[3].record(stream)
        hif4.dequantize(wcodes, wmeta, out_dtype=torch.bfloat16, out=wdeq, stream=stream)
        if ev: ev[4].record(stream)
        hif4.linear_xcodes_wbf16(xcodes, xmeta, wdeq, x_kept=xkept, w_kept=kept, y=y,
                                 workspace=lws, stream=stream)
        if ev: ev[5].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    def avg_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs)

    t_pct, t_wq, t_xq, t_wd, t_lin = (avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3), avg_ms(3, 4),
                                      avg_ms(4, 5))
    ms_step = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    q_bytes = M * K * (2 + 0.5 + 4 / 64) + M * n_protect * 2 + K  # + kept values, mask
    wq_bytes = N * K * (2 + 0.5 + 4 / 64) + N * n_protect * 2 + K
    wd_bytes = N * K * (0.5 + 4 / 64 + 2)           # read codes + meta, write bf16
    pct_bytes = M * K * 2                           # one read of X (algorithmic minimum)
    gemm_tflops = flops / (t_lin * 1e-3) / 1e12
    parts = {
        "percentile_mask": {"ms": t_pct, "GB/s": pct_bytes / t_pct / 1e6,
                            "frac_hbm": pct_bytes / t_pct / 1e6 / HBM_PEAK_GBS,
                            "exact_pass_channels": hif4.percentile_exact_channels(pws, M, K)},
        "quantize_w_masked": {"ms": t_wq, "GB/s": wq_bytes / t_wq / 1e6,
                              "note": "W (141.6 MB bf16) fits the 256 MB MALL"},
        "quantize_x_masked": {"ms": t_xq, "GB/s": q_bytes / t_xq / 1e6,
                       "frac_hbm": q_bytes / t_xq / 1e6 / HBM_PEAK_GBS},
        "dequantize_w": {"ms": t_wd, "GB/s": wd_bytes / t_wd / 1e6},
        "gemm_w4a4": {"ms": t_lin, "TFLOP/s": gemm_tflops,
                      "frac_bf16_mfma": gemm_tflops / BF16_MFMA_PEAK_TFLOPS},
    }
    out = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "ffn_up: X 57600x5120 bf16 (Student-t(3) x LogNormal(0,1) per channel, "
                        "5 outlier channels x50), W 13824x5120 bf16 ~0.02 N(0,1); "
                        "percentile q=0.999, 52 protected channels; Y fp32",
            "M": M, "N": N, "K": K,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_w4a4_u64_kernel (hif4_linear_xcodes_wbf16, one launch per step), "
                      "2*M*N*K flops per launch over its HIP-event time",
            "achieved": gemm_tflops,
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / BF16_MFMA_PEAK_TFLOPS,
            "traffic": measured_traffic(),
        },
        "quantize": parts["quantize_x_masked"],
        "parts": parts,
    }
    if not args.no_extras:
        out["extensions"] = {"higptq": time_higptq(torch, workloads, hif4, dev, w, stream)}
        out["extensions"]["calibration"] = time_calibration(torch, workloads, hif4, dev, stream)
        out["extensions"]["hiautoround_quantize"] = time_autoround(torch, hif4, dev, w, stream)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(x.cpu(), w.cpu(), mask.cpu().numpy(), args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

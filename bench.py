"""Benchmark of the FP8 W8A8 linear hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|mlp_down|mlp_down_tensor|large|tiny]

A step is one pass of the whole hot path over one batch of synthetic input:
dynamic activation quantization followed by the block-scaled GEMM (weights
are quantized once, offline, before timing).  The default workload is the
decode shape: N = 11008, K = 4096, and one step runs the three decode batch
sizes M = 1, 4 and 16 back to back.  Each GEMM of a decode step reads a
different copy of the weight codes (8 copies, 360 MB, more than the 256 MB
Infinity Cache) so the weight really comes from HBM.

Timing: W warm-up steps, then exactly K steps replayed from HIP graphs (one
graph per step pattern), bracketed by torch.cuda.synchronize() on both sides
(one process, one GPU: no barrier needed).  The dominant kernel's average
launch duration is measured with one HIP event pair on the launch stream
around a run of back-to-back launches of that kernel, queued behind a
bounded GPU-side delay so that no host gap falls inside the timed span.

Prints ONE JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
N_WCOPIES = 8
CALIB_COPY_BYTES = 256 << 20   # plain device copy whose counters calibrate FETCH/WRITE_SIZE
KERNEL_SOURCES = ("fp8_w8a8_block_amd/csrc/gemm_kernels.hip",
                  "fp8_w8a8_block_amd/csrc/prefill_asm.inc",
                  "fp8_w8a8_block_amd/csrc/device_common.h")
TRAFFIC_FILE = os.path.join("profiles", "traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dominant_kernel(workload, decode):
    # the prefill-shaped workloads all have K % 512 == 0 and M > 64: the
    # hand-scheduled kernel
    return "gemm_decode_kernel" if decode or workload == "tiny" else "gemm_prefill_asm_kernel"


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def quant_bytes(M, K):
    """Algorithmic bytes of the activation quantizer: bf16 in, codes + scales out."""
    return 2 * M * K + M * K + 4 * M * (K // 128)


def gemm_bytes(M, N, K, per_tensor=False):
    """Each operand once: A codes + scales, W codes + scales, bf16 out."""
    sa = 4 if per_tensor else 4 * M * (K // 128)
    sw = 4 if per_tensor else 4 * (N // 128) * (K // 128)
    return M * K + sa + N * K + sw + 2 * M * N


def gemm_flops(M, N, K):
    return 2 * M * N * K


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "prefill", "mlp_down", "mlp_down_tensor", "large", "tiny"])
    p.add_argument("--cpu-baseline-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the secondary prefill measurement of the decode run")
    return p.parse_args()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class Workload:
    """Device buffers and the launch list of one step."""

    def __init__(self, name):
        import torch
        import fp8_w8a8_block_amd as fp8
        from workloads import synth
        self.fp8 = fp8
        self.name = name
        base = "mlp_down" if name == "mlp_down_tensor" else name
        self.mode = "tensor" if name == "mlp_down_tensor" else "block"
        c = synth.CONFIGS[base]
        self.cfg = c
        self.N, self.K = c["N"], c["K"]
        self.Ms = list(c["decode_m"]) if base == "decode" else [c["M"]]
        ch = synth.outlier_channels(c["cfg"], self.K, c["n_outliers"])
        self.A_bits = [synth.make_activation(c["cfg"], M, self.K, c["a_kind"], c["a_std"], ch,
                                             c["outlier_mult"]) for M in self.Ms]
        W_bits = synth.make_weight(c["cfg"], self.N, self.K, c["w_std"])
        self.W_bits = W_bits
        wd = dev_bf16(W_bits)
        wq, ws = fp8.quant_weight_block(wd, self.mode)
        torch.cuda.synchronize()
        del wd
        ncopy = N_WCOPIES if base == "decode" else 1
        self.wq = [wq] + [wq.clone() for _ in range(ncopy - 1)]
        self.ws = ws
        self.x = [dev_bf16(b) for b in self.A_bits]
        self.aq = [torch.empty((M, self.K), dtype=torch.uint8, device="cuda") for M in self.Ms]
        if self.mode == "block":
            self.as_ = [torch.empty((M, self.K // 128), dtype=torch.float32, device="cuda")
                        for M in self.Ms]
        else:
            self.as_ = [torch.empty((1,), dtype=torch.float32, device="cuda") for _ in self.Ms]
        nws = fp8.workspace_bytes(0, max(self.Ms), 0, self.K, self.mode)
        self.ws_buf = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda") if nws else None
        self.out = [torch.empty((M, self.N), dtype=torch.bfloat16, device="cuda") for M in self.Ms]
        self.ncopy = ncopy
        self.launches_per_step = len(self.Ms)
        # fp8_linear workspace per batch size (None where the call is fused)
        self.lin_ws = []
        for M in self.Ms:
            n = fp8.workspace_bytes(3, M, self.N, self.K, self.mode)
            self.lin_ws.append(torch.empty(n, dtype=torch.uint8, device="cuda") if n else None)
        # A codes and scales for timing the GEMM kernel alone
        for j in range(len(self.Ms)):
            fp8.quant_act(self.x[j], self.mode, workspace=self.ws_buf, q=self.aq[j],
                          scales=self.as_[j])
        torch.cuda.synchronize()

    def copy_index(self, step, j):
        return (step * self.launches_per_step + j) % self.ncopy

    def n_patterns(self):
        # step patterns repeat when the weight-copy rotation does
        from math import gcd
        return self.ncopy // gcd(self.ncopy, self.launches_per_step)

    def step(self, s):
        """One pass of the hot path: for each batch size, one W8A8 linear call
        (dynamic activation quantization + block GEMM).  The library fuses the
        two for small M and runs them back to back otherwise."""
        fp8 = self.fp8
        for j, M in enumerate(self.Ms):
            fp8.linear(self.x[j], self.wq[self.copy_index(s, j)], self.ws, self.mode,
                       out=self.out[j], workspace=self.lin_ws[j])

    def bytes_per_step(self):
        """Algorithmic bytes of one step: for a fused call the bf16 input, the
        weight codes and scales and the output; for a two-kernel call the
        quantizer's bytes plus the GEMM's (GEMM bytes returned separately)."""
        pt = self.mode == "tensor"
        total, g_total = 0, 0
        for j, M in enumerate(self.Ms):
            g = gemm_bytes(M, self.N, self.K, pt)
            g_total += g
            if self.lin_ws[j] is None:          # fused: codes never leave the chip
                total += g - M * self.K - 4 * M * (self.K // 128) + 2 * M * self.K
            else:
                total += quant_bytes(M, self.K) + (2 * M * self.K if pt else 0) + g
        return total, total - g_total, g_total

    def flops_per_step(self):
        return sum(gemm_flops(M, self.N, self.K) for M in self.Ms)


def time_gemm_launches(wl, n_launches):
    """Average duration of the GEMM kernel: one HIP event pair on the launch
    stream around n back-to-back GEMM launches (cycling through the batch
    sizes and weight copies of the step), all queued behind a bounded
    GPU-side delay so that no host gap falls inside the timed span."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e7))          # a bounded GPU-side delay while the host queues work
    e0.record()
    for i in range(n_launches):
        j = i % len(wl.Ms)
        wl.fp8.block_gemm(wl.aq[j], wl.as_[j], wl.wq[i % wl.ncopy], wl.ws, wl.mode,
                          out=wl.out[j])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_launches
    return float(ms), n_launches


def calibration_copy():
    """One plain device-to-device copy of known size; under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE give the scale factor for the kernels' counters."""
    import torch
    src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def secondary_prefill(steps=20):
    """GEMM-only TFLOP/s of the 4096^3 prefill shape, as context in the decode line."""
    import torch
    wl = Workload("prefill")
    for s in range(3):
        wl.step(s)
    torch.cuda.synchronize()
    ms, n = time_gemm_launches(wl, steps)
    tf = wl.flops_per_step() / (ms * 1e-3) / 1e12
    del wl
    torch.cuda.empty_cache()
    return {"workload": "prefill M=N=K=4096", "kernel": "gemm_prefill_asm_kernel",
            "gemm_us": ms * 1e3, "TFLOP/s": tf, "frac_of_5000": tf / FP8_PEAK_TFLOPS}


def cpu_baseline(wl, target_s):
    """Oracle timed on the host on a bounded sample of the same step."""
    from oracle import gemm, quant
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count() or 1
    if wl.mode == "block":
        # weight quantization is offline: done once, outside the timed sample
        if len(wl.Ms) > 1:
            rows = wl.N
        else:
            rows = 128 * max(1, min(wl.N // 128, 4))
        rwq, rws = quant.quant_weight_block_ref(wl.W_bits[:rows])
    else:
        rows = 128 * max(1, min(wl.N // 128, 4))
        amax_w = quant.tensor_amax_ref(wl.W_bits)
        rwq, rws = quant.quant_tensor_with_amax_ref(wl.W_bits[:rows], amax_w)
    a_rows = [min(M, 256) for M in wl.Ms]
    nbytes = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for j, M in enumerate(wl.Ms):
            ab = wl.A_bits[j][:a_rows[j]]
            if wl.mode == "block":
                aq, as_ = quant.quant_act_ref(ab)
                gemm.gemm_block_ref(aq, as_, rwq, rws)
                nbytes += quant_bytes(a_rows[j], wl.K) + gemm_bytes(a_rows[j], rows, wl.K)
            else:
                aq, as_ = quant.quant_tensor_ref(ab)
                gemm.gemm_tensor_ref(aq, as_, rwq, rws)
                nbytes += quant_bytes(a_rows[j], wl.K) + gemm_bytes(a_rows[j], rows, wl.K, True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    flops = sum(gemm_flops(r, rows, wl.K) for r in a_rows) * reps
    sample = (f"oracle quant_act + fp64 GEMM, rows M={a_rows} of A against {rows} of {wl.N} "
              f"weight rows, K={wl.K}, repeated {reps}x; weight quantized beforehand")
    if len(wl.Ms) > 1:
        return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": round(el, 2)}
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(el, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    calibration_copy()
    wl = Workload(args.workload)
    decode = len(wl.Ms) > 1

    # warm-up (eager), then capture one HIP graph per step pattern
    for s in range(args.warmup):
        wl.step(s)
    torch.cuda.synchronize()
    graphs = []
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for p in range(wl.n_patterns()):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                wl.step(p)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    for p in range(len(graphs)):       # graph warm-up replays
        graphs[p].replay()
    torch.cuda.synchronize()

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    ms_per_step = sec / K * 1e3

    total_b, q_b, g_b = wl.bytes_per_step()
    flops = wl.flops_per_step()
    Ms, N_, K_, mode, ncopy = wl.Ms, wl.N, wl.K, wl.mode, wl.ncopy

    n_l = 96 if decode else 24
    g_ms_mean, n_l = time_gemm_launches(wl, n_l)
    gemm_bytes_per_launch = g_b / wl.launches_per_step
    flops_per_launch = flops / wl.launches_per_step

    if decode:
        metric_value = total_b / (sec / K) / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": gemm_bytes_per_launch / (g_ms_mean * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        metric_value = flops / (sec / K) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": flops_per_launch / (g_ms_mean * 1e-3) / 1e12,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(args.workload)
    roof["kernel"] = dominant_kernel(args.workload, decode)
    roof["avg_launch_us"] = g_ms_mean * 1e3
    roof["launches_timed"] = n_l
    roof["algorithmic_bytes_per_launch" if decode else "flop_per_launch"] = (
        gemm_bytes_per_launch if decode else flops_per_launch)
    roof["kernel_source_hash"] = kernel_source_hash()

    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(wl, args.cpu_baseline_seconds)
    secondary = None
    if decode and not args.no_secondary:
        del wl
        torch.cuda.empty_cache()
        secondary = secondary_prefill()

    config = {"workload": args.workload, "M": Ms if decode else Ms[0], "N": N_, "K": K_,
              "scales": "per-tensor" if mode == "tensor" else "A 1x128, W 128x128",
              "step": "fp8_linear (dynamic activation quantization + block GEMM)" +
                      (" for each M" if decode else ""),
              "weight_copies": ncopy}
    line = {
        "metric": ("FP8 block-scaled GEMM TFLOPS (prefill) & GB/s (decode) as % of MI355X "
                   "roofline"),
        "value": metric_value,
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded numpy, shapes and distributions of the workload)",
        "config": config,
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_bytes": {"total": total_b, "gemm_kernels": g_b},
        "step_flop": flops,
        "tflops_per_step": flops / (sec / K) / 1e12,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

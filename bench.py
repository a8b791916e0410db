"""Benchmark of the FP8 W8A8 linear hot path on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode|prefill|mlp_down|mlp_down_tensor|large|tiny|kv_cache|
                                moe_decode|moe_prefill]

A step is one pass of the whole hot path over one batch of synthetic input:
dynamic activation quantization followed by the block-scaled GEMM (weights
are quantized once, offline, before timing).  The default workload is the
decode shape: N = 11008, K = 4096, and one step runs the three decode batch
sizes M = 1, 4 and 16 back to back.  Each GEMM of a decode step reads a
different copy of the weight codes (8 copies, 360 MB, more than the 256 MB
Infinity Cache) so the weight really comes from HBM.

Timing: W warm-up steps, then exactly K steps replayed from HIP graphs (a
graph of 8 consecutive steps replayed K // 8 times, single-step graphs for
the rest), bracketed by torch.cuda.synchronize() on both sides (one process,
one GPU: no barrier needed).  The dominant kernel's average
launch duration is measured with one HIP event pair on the launch stream
around a run of back-to-back launches of that kernel, queued behind a
bounded GPU-side delay so that no host gap falls inside the timed span.

The kv_cache workload times the FP8 KV-cache codec instead: a step stores
the keys and values of 65536 tokens (8 heads of 128) as E4M3 codes into two
paged 1 GiB caches and restores to bf16 the tokens the previous step stored
(two input batches alternate, so the codes read back have been pushed out of
the Infinity Cache by a step's worth of other traffic).

The moe_decode and moe_prefill workloads time one GPU's expert shard of an
FP8 MoE layer (32 of 256 experts, hidden 7168, fused gate and up projection
N = 4096, top-8 routing): a step quantizes the routed rows of a 256-token
decode batch or an 8192-token prefill chunk and runs the grouped GEMM.

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
KV_SOURCES = ("fp8_w8a8_block_amd/csrc/kv_kernels.hip",
              "fp8_w8a8_block_amd/csrc/device_common.h")
TRAFFIC_FILE = os.path.join("profiles", "traffic.json")


def kernel_source_hash(workload=None):
    """Hash of the dominant kernel's sources with comments and blank lines
    removed, so that counters stay attached to the code they measured."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in (KV_SOURCES if workload == "kv_cache" else KERNEL_SOURCES):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def dominant_kernel(workload, decode):
    if workload == "kv_cache":
        return "kv_write_kernel"
    if workload == "moe_decode":
        return "gemm_grouped_decode_kernel"
    if workload == "moe_prefill":
        return "gemm_prefill_asm_kernel"
    if workload == "tiny":
        return "linear_decode_kernel"     # 16 x 256 x 512: one fused launch
    # the prefill-shaped workloads all have K % 512 == 0 and M > 64: the
    # hand-scheduled kernel
    return "gemm_decode_kernel" if decode else "gemm_prefill_asm_kernel"


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(workload):
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
                   choices=["decode", "prefill", "mlp_down", "mlp_down_tensor", "large", "tiny",
                            "kv_cache", "moe_decode", "moe_prefill"])
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


def gemm_kernel_name(M, K):
    """The kernel fp8_block_gemm dispatches for an M x K activation (the
    library's dispatch rule: the decode tile up to 64 rows and K <= 16384,
    the hand-scheduled prefill kernel above 64 rows when K % 512 == 0)."""
    if M <= 64 and K // 128 <= 128:
        return "gemm_decode_kernel"
    return "gemm_prefill_asm_kernel" if (K // 128) % 4 == 0 else "gemm_prefill_kernel"


def fused_bytes(M, N, K):
    """Algorithmic bytes of one fused linear launch: bf16 input, weight codes
    and scales, bf16 output (the activation codes never leave the chip)."""
    return 2 * M * K + N * K + 4 * (N // 128) * (K // 128) + 2 * M * N


def time_step_kernels(wl, n_per):
    """For each batch size of the step, the launch that carries its GEMM:
    the fused linear kernel where the step's fp8_linear call is one launch,
    otherwise the GEMM kernel alone (on codes quantized beforehand).  Each is
    timed as n_per back-to-back launches (rotating over the weight copies)
    with one HIP event pair on the launch stream, behind a bounded GPU-side
    delay so that no host gap falls inside the timed span."""
    pt = wl.mode == "tensor"
    res = []
    for j, M in enumerate(wl.Ms):
        fused = wl.lin_ws[j] is None
        if fused:
            def fn(i, j=j):
                wl.fp8.linear(wl.x[j], wl.wq[i % wl.ncopy], wl.ws, wl.mode, out=wl.out[j])
            b, kernel = fused_bytes(M, wl.N, wl.K), "linear_decode_kernel"
        else:
            def fn(i, j=j):
                wl.fp8.block_gemm(wl.aq[j], wl.as_[j], wl.wq[i % wl.ncopy], wl.ws, wl.mode,
                                  out=wl.out[j])
            b, kernel = gemm_bytes(M, wl.N, wl.K, pt), gemm_kernel_name(M, wl.K)
        ms = time_launches(fn, n_per)
        f = gemm_flops(M, wl.N, wl.K)
        res.append({"M": M, "kernel": kernel, "avg_launch_us": ms * 1e3, "launches_timed": n_per,
                    "algorithmic_bytes": b, "GB/s": b / (ms * 1e-3) / 1e9,
                    "frac_of_8000": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "flop": f, "TFLOP/s": f / (ms * 1e-3) / 1e12,
                    "frac_of_5000": f / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS})
    return res


def time_quantizer(wl):
    """The dynamic activation quantizer on its own: average duration of
    back-to-back launches on the workload's largest activation (the kernel
    the two-launch path runs), against its algorithmic bytes.  The launches
    rotate over enough copies of the input and outputs (more than 600 MB in
    all, up to 16) that they come from HBM, not from the 256 MB Infinity
    Cache."""
    import torch
    j = max(range(len(wl.Ms)), key=lambda i: wl.Ms[i])
    M, K = wl.Ms[j], wl.K
    # block: bf16 in, codes and 1x128 scales out; tensor: the bf16 read twice
    # (global amax, then encode), codes and one scale out
    b = quant_bytes(M, K) if wl.mode == "block" else 5 * M * K + 4
    n_c = int(min(16, max(1, -(-600_000_000 // quant_bytes(M, K)))))
    xs = [wl.x[j]] + [wl.x[j].clone() for _ in range(n_c - 1)]
    qs = [wl.aq[j]] + [torch.empty_like(wl.aq[j]) for _ in range(n_c - 1)]
    ss = [wl.as_[j]] + [torch.empty_like(wl.as_[j]) for _ in range(n_c - 1)]
    n_l = 96 if M <= 64 else 24
    ms = time_launches(lambda i: wl.fp8.quant_act(xs[i % n_c], wl.mode, workspace=wl.ws_buf,
                                                  q=qs[i % n_c], scales=ss[i % n_c]), n_l)
    del xs, qs, ss
    name = "quant_act_block_kernel" if wl.mode == "block" else "absmax_partial_kernel + quant_tensor_kernel"
    return {"kernel": name, "M": M, "K": K, "avg_launch_us": ms * 1e3, "launches_timed": n_l,
            "input_copies": n_c,
            "algorithmic_bytes_per_launch": b, "GB/s": b / (ms * 1e-3) / 1e9,
            "frac_of_8000": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


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


SECONDARY = ("prefill", "mlp_down", "mlp_down_tensor", "large")


def secondary_gemm(name, n_launches=None):
    """GEMM-only TFLOP/s of a prefill-shaped workload (codes quantized
    beforehand), as context in the decode line."""
    import torch
    wl = Workload(name)
    for s in range(2):
        wl.step(s)
    torch.cuda.synchronize()
    n = n_launches or (8 if wl.Ms[0] * wl.N * wl.K > 1e12 else 24)
    r = dict(time_step_kernels(wl, n)[0])
    r.update({"workload": name, "N": wl.N, "K": wl.K,
              "scales": "per-tensor" if wl.mode == "tensor" else "A 1x128, W 128x128"})
    del wl
    torch.cuda.empty_cache()
    return r


def mfma_reference(n=5, grid=256, iters=2048):
    """Timed matrix-unit reference for the prefill lines: the FP8
    MFMA alone (hbm_probe.hip's mfma_chain_kernel: 8 waves per CU, 16
    independent accumulators, operands in registers), n back-to-back launches
    timed like the kernels, on random E4M3 codes (NaN codes replaced) and on
    zero codes.  What it reaches is the rate the chip sustains for FP8 MFMAs
    at the clock it holds under that load."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "fp8_w8a8_block_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp8_w8a8_block_amd.build`")
    probe = ctypes.CDLL(path)
    probe.mfma_chain_probe.restype = ctypes.c_int
    probe.mfma_chain_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    rnd = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, device="cuda", generator=g)
    rnd[(rnd & 0x7F) == 0x7F] -= 1                 # E4M3 NaN codes -> the largest finite
    zero = torch.zeros_like(rnd)
    sink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    flop = grid * 8 * iters * 16 * 2 * 16 * 16 * 128
    res = {}
    for name, codes in (("random_codes", rnd), ("zero_codes", zero)):
        def run(i, codes=codes):
            st = torch.cuda.current_stream().cuda_stream
            rc = probe.mfma_chain_probe(codes.data_ptr(), iters, sink.data_ptr(), grid, st)
            if rc != 0:
                raise RuntimeError(f"mfma_chain_probe failed: {rc}")
        run(0)
        ms = time_launches(run, n)
        tf = flop / (ms * 1e-3) / 1e12
        res[name] = {"avg_launch_us": ms * 1e3, "TFLOP/s": tf, "frac_of_5000": tf / FP8_PEAK_TFLOPS}
    res["flop_per_launch"] = flop
    res["note"] = ("mfma_chain_kernel (fp8_w8a8_block_amd/csrc/hbm_probe.hip): "
                   "v_mfma_f32_16x16x128_f8f6f4 only, 8 waves per CU, operands in registers")
    del rnd, zero, sink
    torch.cuda.empty_cache()
    return res


def hbm_reference(nbytes=1 << 30, n=10):
    """Timed HBM references beside the kernels, each n back-to-back
    launches timed like the kernels: torch's device copy of a 1 GiB buffer
    (2 GiB moved per launch), and a plain streaming read (hbm_probe.hip, its
    own library) of the same 1 GiB and of 45.1 MB -- the decode weight's
    bytes, rotating over eight such buffers so the Infinity Cache holds none
    of them."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "fp8_w8a8_block_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp8_w8a8_block_amd.build`")
    probe = ctypes.CDLL(path)
    probe.hbm_read_probe.restype = ctypes.c_int
    probe.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    grid = 2048
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    c_ms = time_launches(lambda i: dst.copy_(src), n)

    def read(buf):
        st = torch.cuda.current_stream().cuda_stream
        rc = probe.hbm_read_probe(buf.data_ptr(), buf.numel(), sink.data_ptr(), grid, st)
        if rc != 0:
            raise RuntimeError(f"hbm_read_probe failed: {rc}")
    r_ms = time_launches(lambda i: read(src), n)
    del dst
    small = 11008 * 4096
    bufs = [src[i * small:(i + 1) * small] for i in range(8)]
    s_ms = time_launches(lambda i: read(bufs[i % 8]), 4 * n)
    del src, bufs
    torch.cuda.empty_cache()
    return {"copy": {"bytes_moved": 2 * nbytes, "avg_launch_us": c_ms * 1e3,
                     "GB/s": 2 * nbytes / (c_ms * 1e-3) / 1e9},
            "read_stream": {"bytes_read": nbytes, "avg_launch_us": r_ms * 1e3,
                            "GB/s": nbytes / (r_ms * 1e-3) / 1e9},
            "read_stream_decode_bytes": {"bytes_read": small, "avg_launch_us": s_ms * 1e3,
                                         "GB/s": small / (s_ms * 1e-3) / 1e9},
            "note": ("torch.Tensor.copy_ over a 1 GiB device buffer; hbm_read_kernel "
                     "(fp8_w8a8_block_amd/csrc/hbm_probe.hip) reading 1 GiB, and 45.1 MB "
                     "(one decode weight) rotating over 8 buffers")}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def blas_threads():
    try:
        import threadpoolctl
        return max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        return os.cpu_count() or 1


def oracle_linear_sample(A_bits, W_bits, a_rows, w_rows, mode, target_s, max_reps=1000):
    """Repeat the oracle's quantization of a_rows rows of A and its GEMM
    against w_rows rows of W (quantized once beforehand, as offline weight
    quantization is) for about target_s seconds.  Returns (reps, seconds,
    bytes moved per the algorithmic count, flop)."""
    from oracle import gemm, quant
    K = A_bits.shape[1]
    if mode == "block":
        rwq, rws = quant.quant_weight_block_ref(W_bits[:w_rows])
    else:
        rwq, rws = quant.quant_tensor_with_amax_ref(W_bits[:w_rows], quant.tensor_amax_ref(W_bits))
    ab = A_bits[:a_rows]
    reps, t0 = 0, time.perf_counter()
    while True:
        if mode == "block":
            aq, as_ = quant.quant_act_ref(ab)
            gemm.gemm_block_ref(aq, as_, rwq, rws)
        else:
            aq, as_ = quant.quant_tensor_ref(ab)
            gemm.gemm_tensor_ref(aq, as_, rwq, rws)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= max_reps:
            break
    nbytes = quant_bytes(a_rows, K) + gemm_bytes(a_rows, w_rows, K, mode != "block")
    return reps, el, reps * nbytes, reps * gemm_flops(a_rows, w_rows, K)


def single_thread_baselines(target_s):
    """The oracle on one BLAS thread, on bounded samples of the tiny, decode
    (M = 16) and prefill workloads: quantize the activation rows and multiply
    them against weight rows quantized beforehand."""
    from workloads import synth
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(1)
    except Exception:
        limit = None
    out = []
    try:
        for name, M, a_rows, w_rows in (("tiny", None, 16, 256), ("decode", 16, 16, 1024),
                                        ("prefill", None, 64, 512)):
            d = synth.make_config(name, M=M)
            reps, el, nb, fl = oracle_linear_sample(d["A"], d["W"], a_rows, w_rows, "block",
                                                    target_s)
            out.append({"workload": name, "threads": 1, "GB/s": nb / el / 1e9,
                        "GFLOP/s": fl / el / 1e9, "seconds": round(el, 2),
                        "sample": f"quant_act of {a_rows} rows of A (K={d['K']}) + fp64 GEMM "
                                  f"against {w_rows} of {d['N']} weight rows, repeated {reps}x"})
    finally:
        if limit is not None:
            limit.unregister()
    return out


def cpu_baseline(wl, target_s):
    """Oracle timed on the host on a bounded sample of the same step, with
    all BLAS threads, then on one thread for the tiny, decode and prefill
    workloads."""
    threads = blas_threads()
    if len(wl.Ms) > 1 or wl.mode != "block":
        rows = wl.N if len(wl.Ms) > 1 else 128 * max(1, min(wl.N // 128, 4))
    else:
        rows = 128 * max(1, min(wl.N // 128, 4))
    a_rows = [min(M, 256) for M in wl.Ms]
    nbytes, flops, el_all, reps_all = 0, 0, 0.0, []
    per = target_s / len(wl.Ms)
    for j, M in enumerate(wl.Ms):
        reps, el, nb, fl = oracle_linear_sample(wl.A_bits[j], wl.W_bits, a_rows[j], rows,
                                                wl.mode, per)
        nbytes += nb
        flops += fl
        el_all += el
        reps_all.append(reps)
    sample = (f"oracle quant_act + fp64 GEMM, rows M={a_rows} of A against {rows} of {wl.N} "
              f"weight rows, K={wl.K}, repeated {reps_all}x; weight quantized beforehand")
    res = {"cores": threads, "kind": "oracle", "sample": sample, "seconds": round(el_all, 2),
           "cpu_model": cpu_model(), "logical_cpus": os.cpu_count()}
    if len(wl.Ms) > 1:
        res.update({"value": nbytes / el_all / 1e9, "unit": "GB/s"})
    else:
        res.update({"value": flops / el_all / 1e12, "unit": "TFLOP/s"})
    res["single_thread"] = single_thread_baselines(min(3.0, target_s / 3))
    return res


def kv_write_bytes(T, HD):
    """Algorithmic bytes of one cache write: bf16 keys and values in, E4M3
    codes of both out, the slot of each token, the two scales."""
    return T * (2 * 2 * HD + 2 * HD + 8) + 8


def kv_read_bytes(T, HD):
    """One restore: codes and slot of each token in, bf16 out, the scale."""
    return T * (HD + 2 * HD + 8) + 4


class KVWorkload:
    """Two alternating batches of paged-cache traffic: step s stores batch
    s % 2 and restores the keys and values of batch (s + 1) % 2."""

    def __init__(self):
        import torch
        import fp8_w8a8_block_amd as fp8
        from workloads import synth
        self.fp8 = fp8
        c = synth.KV_CONFIG
        self.c = c
        self.T, self.H, self.D = c["T"], c["H"], c["D"]
        self.bs, self.nb = c["block_size"], c["num_blocks"]
        self.batches = []
        for b in range(2):
            d = synth.make_kv(c["cfg"] + 100 * b, self.T, self.H, self.D, self.bs, self.nb,
                              c["n_seqs"], c["key_outlier_dims"], c["key_outlier_mult"],
                              c["pad_frac"])
            self.batches.append({"key_bits": d["key"], "value_bits": d["value"],
                                 "slots_host": d["slots"],
                                 "key": dev_bf16(d["key"]), "value": dev_bf16(d["value"]),
                                 "slots": torch.from_numpy(d["slots"]).cuda()})
        f = synth.bf16_bits_to_f32_input(self.batches[0]["key_bits"][:4096])
        self.k_scale = torch.tensor([float(np.abs(f).max()) / 448.0], dtype=torch.float32,
                                    device="cuda")
        self.v_scale = torch.ones(1, dtype=torch.float32, device="cuda")
        shape = (self.nb, self.bs, self.H, self.D)
        self.kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        self.vc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        self.kout = torch.empty((self.T, self.H, self.D), dtype=torch.bfloat16, device="cuda")
        self.vout = torch.empty_like(self.kout)
        for b in range(2):
            self.write(b)
        torch.cuda.synchronize()

    def write(self, b):
        B = self.batches[b]
        self.fp8.kv_cache_write(B["key"], B["value"], B["slots"], self.kc, self.vc,
                                self.k_scale, self.v_scale)

    def step(self, s):
        self.write(s % 2)
        r = self.batches[(s + 1) % 2]["slots"]
        self.fp8.kv_cache_read(self.kc, r, self.k_scale, out=self.kout)
        self.fp8.kv_cache_read(self.vc, r, self.v_scale, out=self.vout)

    def bytes_per_step(self):
        HD = self.H * self.D
        return kv_write_bytes(self.T, HD) + 2 * kv_read_bytes(self.T, HD)


def timed_steps(step, n_patterns, K):
    """Wall time of exactly K steps replayed from HIP graphs: one graph of
    S >= 8 consecutive steps (S a multiple of the number of step patterns)
    replayed K // S times, then single-step graphs for the K % S left, so the
    host's per-replay cost is paid once per S steps.  Step s runs pattern
    s % n_patterns.  Returns seconds between two device synchronizations."""
    import torch
    S = n_patterns * -(-8 // n_patterns)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    singles = []
    with torch.cuda.stream(stream):
        for p in range(n_patterns):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(p)
            singles.append(g)
        block = torch.cuda.CUDAGraph()
        with torch.cuda.graph(block, stream=stream):
            for s in range(S):
                step(s % n_patterns)
    torch.cuda.current_stream().wait_stream(stream)
    block.replay()                     # warm-up replays
    for g in singles:
        g.replay()
    torch.cuda.synchronize()
    full, rem = divmod(K, S)
    t0 = time.perf_counter()
    for _ in range(full):
        block.replay()
    for r in range(rem):
        singles[(full * S + r) % n_patterns].replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_launches(fn, n_launches):
    """Average duration of one kernel: an event pair on the launch stream
    around n back-to-back launches queued behind a bounded GPU-side delay."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e7))
    e0.record()
    for i in range(n_launches):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_launches


def kv_cpu_baseline(wl, target_s):
    """The KV-cache oracle timed on the host: store + restore of a token
    sample of batch 0 into a cache sized for that sample."""
    from oracle import kv_cache
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count() or 1
    n = 1024
    B = wl.batches[0]
    ks = np.float32(wl.k_scale.item())
    HD = wl.H * wl.D
    cache = np.zeros((n // wl.bs, wl.bs, wl.H, wl.D), dtype=np.uint8)
    slots = np.arange(n, dtype=np.int64)
    reps, t0 = 0, time.perf_counter()
    while True:
        lo = (reps * n) % wl.T
        kc = kv_cache.kv_write_ref(B["key_bits"][lo:lo + n], slots, cache, ks)
        vc = kv_cache.kv_write_ref(B["value_bits"][lo:lo + n], slots, cache, np.float32(1.0))
        kv_cache.kv_read_ref(kc, slots, ks)
        kv_cache.kv_read_ref(vc, slots, np.float32(1.0))
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 64:
            break
    nbytes = reps * (kv_write_bytes(n, HD) + 2 * kv_read_bytes(n, HD))
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle store + restore of {n}-token slices of the same keys and values "
                      f"(H={wl.H}, D={wl.D}) into a {n}-slot cache, repeated {reps}x",
            "seconds": round(el, 2)}


def main_kv(args):
    import torch
    calibration_copy()
    wl = KVWorkload()
    for s in range(args.warmup):
        wl.step(s)
    torch.cuda.synchronize()
    K = args.steps
    sec = timed_steps(wl.step, 2, K)

    HD = wl.H * wl.D
    n_l = 40
    w_ms = time_launches(lambda i: wl.write(i % 2), n_l)
    r_ms = time_launches(lambda i: wl.fp8.kv_cache_read(
        wl.kc, wl.batches[i % 2]["slots"], wl.k_scale, out=wl.kout), n_l)
    wb = kv_write_bytes(wl.T, HD)
    rb = kv_read_bytes(wl.T, HD)
    roof = {"bound": "hbm", "achieved": wb / (w_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic("kv_cache")
    roof["kernel"] = "kv_write_kernel"
    roof["avg_launch_us"] = w_ms * 1e3
    roof["launches_timed"] = n_l
    roof["algorithmic_bytes_per_launch"] = wb
    roof["kernel_source_hash"] = kernel_source_hash("kv_cache")
    read = {"kernel": "kv_read_kernel", "avg_launch_us": r_ms * 1e3,
            "algorithmic_bytes_per_launch": rb, "GB/s": rb / (r_ms * 1e-3) / 1e9,
            "frac_of_8000": rb / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    cpu = kv_cpu_baseline(wl, args.cpu_baseline_seconds) if args.cpu_baseline_seconds > 0 else None
    total = wl.bytes_per_step()
    line = {
        "metric": "FP8 KV-cache codec GB/s (store + restore) as % of MI355X HBM roofline",
        "value": total / (sec / K) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": sec / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 <-> fp8e4m3 (fp32 scale arithmetic)",
        "data": "synthetic (seeded numpy, paged slot mapping)",
        "config": {"workload": "kv_cache", "tokens": wl.T, "kv_heads": wl.H, "head_dim": wl.D,
                   "block_size": wl.bs, "num_blocks": wl.nb,
                   "cache_bytes_each": wl.nb * wl.bs * HD,
                   "step": "store K and V of one batch, restore K and V of the other"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": read,
        "step_bytes": {"total": total},
    }
    print(json.dumps(line), flush=True)


class MoEWorkload:
    """One GPU's expert shard of an FP8 MoE layer: the routed rows of one
    batch, grouped by expert, through dynamic 1x128 quantization and the
    grouped block GEMM against 32 experts' 128x128-block FP8 weights."""

    def __init__(self, name):
        import torch
        import fp8_w8a8_block_amd as fp8
        from workloads import synth
        self.fp8 = fp8
        self.name = name
        c = synth.MOE_CONFIGS[name]
        self.c = c
        self.E, self.N, self.K = c["experts_local"], c["N"], c["K"]
        rows, offsets = synth.make_moe_routing(c["cfg"], c["tokens"], c["top_k"],
                                               c["experts_total"], self.E)
        self.offsets_host = offsets
        self.M = len(rows)
        tok = synth.make_moe_tokens(c["cfg"], c["tokens"], self.K, c["n_outliers"],
                                    c["outlier_mult"])
        self.a_bits = tok[rows]
        self.x = dev_bf16(self.a_bits)
        self.wq = torch.empty((self.E, self.N, self.K), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty((self.E, self.N // 128, self.K // 128), dtype=torch.float32,
                              device="cuda")
        for e in range(self.E):
            q, sc = fp8.quant_weight_block(dev_bf16(synth.make_moe_weight(c["cfg"], e, self.N,
                                                                          self.K, c["w_std"])))
            self.wq[e].copy_(q)
            self.ws[e].copy_(sc)
        self.offsets = torch.from_numpy(offsets).cuda()
        self.aq = torch.empty((self.M, self.K), dtype=torch.uint8, device="cuda")
        self.as_ = torch.empty((self.M, self.K // 128), dtype=torch.float32, device="cuda")
        self.out = torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")
        fp8.quant_act(self.x, "block", q=self.aq, scales=self.as_)
        torch.cuda.synchronize()
        self.active = int((np.diff(offsets) > 0).sum())

    def step(self, s):
        self.fp8.quant_act(self.x, "block", q=self.aq, scales=self.as_)
        self.gemm()

    def gemm(self):
        self.fp8.grouped_gemm(self.aq, self.as_, self.wq, self.ws, self.offsets, out=self.out)

    def gemm_bytes(self):
        """Each operand once: A codes and scales, the weights and weight
        scales of the experts that have rows, the bf16 output."""
        M, N, K = self.M, self.N, self.K
        return (M * K + 4 * M * (K // 128) + self.active * (N * K + 4 * (N // 128) * (K // 128)) +
                2 * M * N)

    def flops(self):
        return 2 * self.M * self.N * self.K


def moe_cpu_baseline(wl, target_s):
    """The oracle on the host: quantize and multiply up to 64 rows of each of
    two experts against those experts' full weights (quantized beforehand)."""
    from oracle import moe, quant
    from workloads import synth
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count() or 1
    counts = np.diff(wl.offsets_host)
    experts = [int(e) for e in np.argsort(-counts)[:2]]
    wq, ws = zip(*[quant.quant_weight_block_ref(synth.make_moe_weight(wl.c["cfg"], e, wl.N, wl.K,
                                                                      wl.c["w_std"]))
                   for e in experts])
    wq, ws = np.stack(wq), np.stack(ws)
    rows = [np.arange(wl.offsets_host[e], wl.offsets_host[e] + min(64, counts[e])) for e in experts]
    sub_off = np.array([0, len(rows[0]), len(rows[0]) + len(rows[1])])
    a_bits = wl.a_bits[np.concatenate(rows)]
    reps, t0 = 0, time.perf_counter()
    while True:
        aq, as_ = quant.quant_act_ref(a_bits)
        moe.grouped_gemm_ref(aq, as_, wq, ws, sub_off)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    m = int(sub_off[-1])
    sample = (f"oracle quant_act + grouped GEMM of {m} rows (up to 64 of each of the two busiest "
              f"experts) against their full {wl.N}x{wl.K} weights, repeated {reps}x; weights "
              "quantized beforehand")
    if wl.name == "moe_decode":
        nbytes = reps * (3 * m * wl.K + 2 * (wl.N * wl.K + 4 * (wl.N // 128) * (wl.K // 128)) +
                         2 * m * wl.N)
        return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": round(el, 2)}
    return {"value": reps * 2 * m * wl.N * wl.K / el / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(el, 2)}


def main_moe(args):
    import torch
    calibration_copy()
    wl = MoEWorkload(args.workload)
    for s in range(args.warmup):
        wl.step(s)
    torch.cuda.synchronize()
    K = args.steps
    sec = timed_steps(wl.step, 1, K)
    n_l = 20
    g_ms = time_launches(lambda i: wl.gemm(), n_l)
    decode = wl.name == "moe_decode"
    if decode:
        step_bytes = quant_bytes(wl.M, wl.K) + wl.gemm_bytes()
        value, unit = step_bytes / (sec / K) / 1e9, "GB/s"
    else:
        value, unit = wl.flops() / (sec / K) / 1e12, "TFLOP/s"
    # the roof that binds: every expert's weight must come from HBM, so at
    # these row counts (2 * rows / experts FLOP per weight byte, below the
    # chip's 625 FLOP/B) the grouped GEMM is bound by HBM, not by the MFMA
    if wl.gemm_bytes() / HBM_PEAK_GBS / 1e9 >= wl.flops() / FP8_PEAK_TFLOPS / 1e12:
        roof = {"bound": "hbm", "achieved": wl.gemm_bytes() / (g_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "algorithmic_bytes_per_launch": wl.gemm_bytes(),
                "tflops": wl.flops() / (g_ms * 1e-3) / 1e12}
    else:
        roof = {"bound": "mfma", "achieved": wl.flops() / (g_ms * 1e-3) / 1e12,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "flop_per_launch": wl.flops()}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(args.workload)
    roof["kernel"] = dominant_kernel(args.workload, decode)
    roof["avg_launch_us"] = g_ms * 1e3
    roof["launches_timed"] = n_l
    roof["kernel_source_hash"] = kernel_source_hash(args.workload)
    cpu = moe_cpu_baseline(wl, args.cpu_baseline_seconds) if args.cpu_baseline_seconds > 0 else None
    counts = np.diff(wl.offsets_host)
    line = {
        "metric": ("FP8 block-scaled MoE grouped GEMM " +
                   ("GB/s (decode)" if decode else "TFLOPS (prefill)") +
                   " as % of MI355X roofline"),
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": sec / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded numpy, skewed top-k routing)",
        "config": {"workload": args.workload, "tokens": wl.c["tokens"], "top_k": wl.c["top_k"],
                   "experts_total": wl.c["experts_total"], "experts_local": wl.E,
                   "rows": wl.M, "rows_per_expert_min_mean_max": [int(counts.min()),
                                                                  float(counts.mean()),
                                                                  int(counts.max())],
                   "N": wl.N, "K": wl.K, "scales": "A 1x128, W 128x128 per expert",
                   "step": "quant_act of the routed rows + grouped GEMM"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_flop": wl.flops(),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "kv_cache":
        return main_kv(args)
    if args.workload.startswith("moe_"):
        return main_moe(args)
    calibration_copy()
    wl = Workload(args.workload)
    decode = len(wl.Ms) > 1

    # warm-up (eager), then the timed steps from HIP graphs
    for s in range(args.warmup):
        wl.step(s)
    torch.cuda.synchronize()
    K = args.steps
    sec = timed_steps(wl.step, wl.n_patterns(), K)
    ms_per_step = sec / K * 1e3

    total_b, q_b, g_b = wl.bytes_per_step()
    flops = wl.flops_per_step()
    Ms, N_, K_, mode, ncopy = wl.Ms, wl.N, wl.K, wl.mode, wl.ncopy

    n_l = 32 if decode else 24
    launches = time_step_kernels(wl, n_l)
    tot_us = sum(r["avg_launch_us"] for r in launches)
    tot_b = sum(r["algorithmic_bytes"] for r in launches)
    tot_f = sum(r["flop"] for r in launches)
    kernels = sorted({r["kernel"] for r in launches})

    if decode:
        metric_value = total_b / (sec / K) / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": tot_b / (tot_us * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        metric_value = flops / (sec / K) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": tot_f / (tot_us * 1e-6) / 1e12,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(args.workload)
    roof["kernel"] = " + ".join(kernels)
    roof["avg_launch_us"] = tot_us / len(launches)
    roof["launches_timed"] = n_l * len(launches)
    roof["algorithmic_bytes_per_launch" if decode else "flop_per_launch"] = (
        tot_b / len(launches) if decode else tot_f / len(launches))
    roof["per_launch"] = launches
    roof["kernel_source_hash"] = kernel_source_hash()

    quantizer = time_quantizer(wl)
    cpu = None
    if args.cpu_baseline_seconds > 0:
        cpu = cpu_baseline(wl, args.cpu_baseline_seconds)
    secondary = None
    hbm_ref = hbm_reference()
    mfma_ref = None if decode else mfma_reference()
    if decode and not args.no_secondary:
        del wl
        torch.cuda.empty_cache()
        secondary = [secondary_gemm(n) for n in SECONDARY]

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
        "quantizer": quantizer,
        "hbm_reference": hbm_ref,
    }
    if mfma_ref is not None:
        line["mfma_reference"] = mfma_ref
        # the dominant kernel against what the matrix units alone sustain on
        # random codes, beside its fraction of the 5.0 PFLOP/s figure
        roof["frac_of_mfma_reference"] = roof["achieved"] / mfma_ref["random_codes"]["TFLOP/s"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

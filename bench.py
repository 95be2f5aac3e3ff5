"""Benchmark of the causal Based forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--workload NAME|INDEX]
                [--no-cpu-baseline] [--all] [--page-shapes] [--decode B,H,K,V[;...]] [--with-state]

A step is one full forward (every kernel of the path) over one batch of synthetic bf16 inputs that are
resident in device memory before timing starts. Before the W warm-up steps, untimed steps run back to back
for at least MS milliseconds (default 300) so that the GPU clocks have settled; then exactly K steps are
timed. The default workload is B=4, T=8192, H=16, K=16, V=64 with bf16 output. Prints one JSON line on
stdout; diagnostics go to stderr.

Work model: canonical FLOPs B*H*T*(4*P*V + 2*64*(K+V)), P = 1+K+K*K (field flops_src of the page "Write a
fast Based (Taylor linear attention) forward kernel"); algorithmic bytes = q, k, v read once + o written
once = B*T*H*(4K + 2V) + B*T*H*V*(2 or 4).
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

METRIC = "Based fwd tokens/s and TFLOP/s (% of MFMA/HBM roofline), B=4 T=8192 H=16 K=16"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def canonical_flops(B, T, H, K, V, C=64):
    P = 1 + K + K * K
    return B * H * T * (4 * P * V + 2 * C * (K + V))


def algorithmic_bytes(B, T, H, K, V, out_bytes):
    return B * T * H * (4 * K + 2 * V) + B * T * H * V * out_bytes


LIB_FILE = os.path.join(ROOT, "taylor_feature_map_amd", "libbased.so")


def traffic_file(workload_name):
    return os.path.join(ROOT, "profiles", f"based_chunk_readout_traffic_{workload_name}.md")


def device_code_digest(lib=LIB_FILE):
    """SHA-256 of the instruction bytes of the gfx950 code object inside the built library, or None
    without one. It changes whenever the device code does (kernel source, compiler flags) and not for
    comments, host code or the directory the library was built in."""
    from taylor_feature_map_amd.codeobj import text_digest
    return text_digest(lib)


def measured_traffic(workload_name):
    """HBM bytes per read-out launch from the committed rocprofv3 summary of this workload, or None when
    there is none or it was taken on different device code."""
    path = traffic_file(workload_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            key, val = line.strip().split(":", 1)
            fields[key.strip()] = val.strip()
    digest = device_code_digest()
    if digest is None or fields.get("device_code_sha256") != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def pick_workload(sel):
    from taylor_feature_map_amd.inputs import HEADLINE, WORKLOADS
    if sel is None:
        return HEADLINE
    if sel.isdigit():
        return WORKLOADS[int(sel)]
    for w in WORKLOADS:
        if w.name == sel:
            return w
    raise SystemExit(f"unknown workload {sel}; choose from {[w.name for w in WORKLOADS]}")


def cpu_baseline(w, qb, kb, vb, budget_s=10.0):
    """The oracle's chunked feature-map form (float64 numpy, chunk 256) on whole (b, h) sequences of the
    same workload, taken in order (and again from the first pair when all are done) until about
    `budget_s` seconds of oracle time have passed; scaled to tokens/s of the whole workload."""
    from oracle import based_ref_chunked, bf16_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_total = 0, 0.0
    while t_total < budget_s:
        b, h = pairs[done % len(pairs)]
        q = bf16_to_f64(qb[b:b + 1, :, h:h + 1])
        k = bf16_to_f64(kb[b:b + 1, :, h:h + 1])
        v = bf16_to_f64(vb[b:b + 1, :, h:h + 1])
        t0 = time.perf_counter()
        based_ref_chunked(q, k, v, w.scale, 256)
        t_total += time.perf_counter() - t0
        done += 1
    tokens_equiv = w.B * w.T * done / len(pairs)
    return {
        "value": tokens_equiv / t_total,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} (b,h) sequences of T={w.T} (the workload's {len(pairs)} pairs in order, "
                  f"{done / len(pairs):.2f} passes) through the float64 chunked oracle (chunk 256) in "
                  f"{t_total:.2f} s; tokens/s scaled to the whole B*T workload",
        "seconds": round(t_total, 3),
        "canonical_gflops": canonical_flops(1, w.T, done, w.K, w.V) / t_total / 1e9,
        "cpu_model": _cpu_model(),
        "blas": _blas_name(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_name():
    try:
        deps = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{deps.get('name')} {deps.get('version')}"
    except Exception:
        return None


SWEEP_BYTES = 1 << 30  # read before every cold step: 4x the 256 MB Infinity Cache, 256x the L2


def counter_summary(workload_name):
    """MFMA-busy figures of the read-out kernel from the committed rocprofv3 counter summary of this
    workload, or None when there is none or it was taken on different device code."""
    path = os.path.join(ROOT, "profiles", f"based_kernels_{workload_name}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            key, val = line.strip().split(":", 1)
            fields[key.strip()] = val.strip()
    digest = device_code_digest()
    if digest is None or fields.get("device_code_sha256") != digest or "readout_mfma_busy_frac" not in fields:
        return None
    return {"readout_mfma_busy_frac": float(fields["readout_mfma_busy_frac"]),
            "readout_valu_insts_per_token_head": float(fields.get("readout_valu_insts_per_token_head", "nan"))}


def run_bench(w, steps, warmup, with_cpu=True, device_inputs=False, settle_s=0.3, cpu_budget_s=10.0, cold_steps=10):
    """Times the whole forward on workload w.

    Warm: `steps` back-to-back steps after the clocks have settled (the throughput), the same again with
    HIP events around every kernel (their average durations), and single steps between events. Cold:
    before each of `cold_steps` steps a read of a 1 GiB buffer (a sum) evicts L2 and the Infinity Cache, so
    the step reads its inputs from HBM; the read leaves no dirty lines behind to drain inside the step.
    Cold steps are timed once between events and once with events around every kernel."""
    import torch

    from taylor_feature_map_amd import Timer, based_forward, plan
    from taylor_feature_map_amd.inputs import make_qkv_device, make_workload

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if device_inputs:
        q, k, v = make_qkv_device(w.B, w.T, w.H, w.K, w.V, w.seed, dev)
        with_cpu = False
    else:
        qb, kb, vb = make_workload(w)
        to = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = to(qb), to(kb), to(vb)
    out_dtype = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
    out = torch.empty((w.B, w.T, w.H, w.V), dtype=out_dtype, device=dev)
    segments, seg_len, ws_bytes = plan(w.B, w.T, w.H, w.K, w.V)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    timer = Timer(max_launches=3 * max(steps, cold_steps) + 16)  # events around every kernel of a step

    def step(t=None):
        based_forward(q, k, v, w.scale, out=out, workspace=ws, timer=t)

    def kernel_times(t):
        res = {}
        for kid in Timer.KERNELS:
            n, ms = t.read(kid)
            if n:
                res[Timer.kernel_name(kid)] = {"launches": n, "avg_us": ms * 1e3 / n}
        return res

    # Settle: untimed back-to-back steps for at least settle_s seconds before the warm-up steps. The GPU
    # needs tens of milliseconds of continuous work to reach its loaded clocks (the first ~30 ms of a
    # burst run ~15% slower), far more than a few warm-up steps of this size take.
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n_settle += 20
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps, bracketed by device synchronisation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps

    # The same K steps again with HIP events recorded on the launch stream around every kernel (events at
    # kernel boundaries cost a few microseconds each, so the throughput above is taken without them).
    timer.reset()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    ms_instrumented = (time.perf_counter() - t1) * 1e3 / steps
    warm_kernels = kernel_times(timer)

    # Single warm steps, each bracketed by HIP events on the launch stream: median and minimum.
    def bracketed(before=None):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if before is not None:
            before()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    single = [bracketed() for _ in range(steps)]

    # Cold steps: a read-only sweep of 1 GiB before each one.
    sweep = torch.ones(SWEEP_BYTES // 4, dtype=torch.float32, device=dev)
    evict = lambda: sweep.sum()  # noqa: E731
    cold = [bracketed(evict) for _ in range(cold_steps)]
    timer.reset()
    for _ in range(cold_steps):
        evict()
        step(timer)
        torch.cuda.synchronize()
    cold_kernels = kernel_times(timer)
    del sweep

    out_bytes = 4 if w.out_dtype == "f32" else 2
    flops = canonical_flops(w.B, w.T, w.H, w.K, w.V)
    nbytes = algorithmic_bytes(w.B, w.T, w.H, w.K, w.V, out_bytes)
    tokens = w.B * w.T
    dom = "based_chunk_readout_kernel"
    cold_us = cold_kernels[dom]["avg_us"]
    warm_us = warm_kernels[dom]["avg_us"]
    cold_med = float(np.median(cold))

    def roof(us):
        achieved = nbytes / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.name), "kernel": dom,
                "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": us}

    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "scale": w.scale, "out_dtype": w.out_dtype, "seed": w.seed,
                   "segments": segments, "segment_len": seg_len},
        "roofline": dict(roof(cold_us), cache="cold"),
        "roofline_warm": dict(roof(warm_us), cache="warm"),
        "tflops_canonical": flops / (ms_per_step * 1e-3) / 1e12,
        "path_hbm_frac": nbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "path_hbm_frac_cold": nbytes / (cold_med * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "path_mfma_frac": flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "ms_per_step_with_kernel_events": ms_instrumented,
        "ms_per_step_single_median": float(np.median(single)),
        "ms_per_step_single_min": float(np.min(single)),
        "ms_per_step_cold_median": cold_med,
        "ms_per_step_cold_min": float(np.min(cold)),
        "kernels": warm_kernels,
        "kernels_cold": cold_kernels,
        "counters": counter_summary(w.name),
        "device": device_info(props),
    }
    if with_cpu:
        result["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, cpu_budget_s)
    return result


def config_summary(r):
    """The per-configuration figures carried in the main JSON line."""
    c = r["config"]
    return {"workload": c["workload"], "segments": c["segments"], "ms_per_step": r["ms_per_step"],
            "ms_per_step_cold": r["ms_per_step_cold_median"], "tokens_per_s": r["value"],
            "tflops_canonical": r["tflops_canonical"], "path_hbm_frac": r["path_hbm_frac"],
            "path_hbm_frac_cold": r["path_hbm_frac_cold"], "readout_us_cold": r["roofline"]["avg_launch_us"],
            "readout_hbm_frac_cold": r["roofline"]["frac"], "readout_us_warm": r["roofline_warm"]["avg_launch_us"],
            "readout_hbm_frac_warm": r["roofline_warm"]["frac"], "traffic": r["roofline"]["traffic"],
            "counters": r["counters"],
            "kernels_cold_us": {k: round(v["avg_us"], 3) for k, v in r["kernels_cold"].items()}}


def device_info(props):
    """Name, compute units, peak shader clock and L2 size of cuda:0 as HIP reports them."""
    import ctypes

    from taylor_feature_map_amd import _lib
    cus, khz, l2 = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _lib.check(_lib.lib().based_device_info(0, ctypes.byref(cus), ctypes.byref(khz), ctypes.byref(l2)),
               "based_device_info")
    return {"name": props.name, "cus": cus.value, "peak_clock_mhz": khz.value / 1e3, "l2_bytes": l2.value,
            "arch": getattr(props, "gcnArchName", "")}


def _settle(fn, settle_s):
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def decode_bench(B, H, K, V, steps, settle_s):
    """The one-token recurrent step (based_decode_step) on B sequences x H heads: the state is read and
    written once per token, so its roofline is HBM. Algorithmic bytes per step = the fp32 state and
    normaliser read and written (8 (P V + P) per (b, h)) + q, k, v read + o written (bf16)."""
    import torch

    from taylor_feature_map_amd import _lib
    from taylor_feature_map_amd.based import feature_dim
    dev = torch.device("cuda:0")
    P = feature_dim(K)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn((B, H, K), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, H, K), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, H, V), generator=g, device=dev).to(torch.bfloat16)
    S = torch.zeros((B, H, P, V), dtype=torch.float32, device=dev)
    z = torch.zeros((B, H, P), dtype=torch.float32, device=dev)
    o = torch.empty((B, H, V), dtype=torch.bfloat16, device=dev)
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, K, V, float("nan"), S.data_ptr(), z.data_ptr(),
            o.data_ptr(), _lib.BASED_BF16, stream)

    def step():
        _lib.check(L.based_decode_step(*args), "based_decode_step")

    _settle(step, settle_s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = B * H * (8 * (P * V + P) + 4 * K + 2 * V + 2 * V)
    return {"workload": f"decode_b{B}_h{H}_k{K}_v{V}", "us_per_step": us, "tokens_per_s": B / (us * 1e-6),
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def state_forward_bench(w, steps, settle_s):
    """The forward with a state carried in and the state after the last token written out
    (based_forward_state), against the plain forward on the same inputs."""
    import torch

    from taylor_feature_map_amd import _lib, plan
    from taylor_feature_map_amd.based import feature_dim
    from taylor_feature_map_amd.inputs import make_qkv_device
    dev = torch.device("cuda:0")
    q, k, v = make_qkv_device(w.B, w.T, w.H, w.K, w.V, w.seed, dev)
    P = feature_dim(w.K)
    s_in = torch.randn((w.B, w.H, P, w.V), device=dev) * 0.1
    z_in = torch.rand((w.B, w.H, P), device=dev) + float(w.T)
    s_out, z_out = torch.empty_like(s_in), torch.empty_like(z_in)
    out = torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device=dev)
    _, _, need = plan(w.B, w.T, w.H, w.K, w.V)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    scale = float("nan") if w.scale is None else w.scale
    base = (q.data_ptr(), k.data_ptr(), v.data_ptr(), w.B, w.T, w.H, w.K, w.V, scale, out.data_ptr(),
            _lib.BASED_BF16)

    def plain():
        _lib.check(L.based_forward_ws(*base, ws.data_ptr(), ws.numel(), stream), "based_forward_ws")

    def with_state():
        _lib.check(L.based_forward_state(*base, s_in.data_ptr(), z_in.data_ptr(), s_out.data_ptr(),
                                         z_out.data_ptr(), ws.data_ptr(), ws.numel(), stream),
                   "based_forward_state")

    res = {"workload": f"state_{w.name}"}
    for name, fn in (("plain", plain), ("with_state", with_state)):
        _settle(fn, settle_s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_ms"] = e0.elapsed_time(e1) / steps
    res["state_bytes_in_out"] = 2 * w.B * w.H * (P * w.V + P) * 4
    return res


def copy_probe(mib, reps):
    """A plain copy of known size: reads and writes mib MiB per launch. Profiler counters taken on it give
    the factor between counter readings and bytes moved."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * 1024 * 1024 // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": reps}))


def row_probe(B, T, H, reps):
    """Reads a (B, T, H, 16) bf16 tensor as the read-out kernel reads q and k: one workgroup per (b, h),
    32-byte rows at a stride of H * 32 bytes, 16-byte loads, heads that share a 128-byte line on one XCD.
    Every byte is read once per launch, so profiler counters taken on it give the factor between counter
    readings and bytes read for this access pattern."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "taylor_feature_map_amd", "libbased_probe.so")
    lib = ctypes.CDLL(path)
    lib.based_probe_read_rows.restype = ctypes.c_int
    lib.based_probe_read_rows.argtypes = [ctypes.c_void_p] + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 2
    dev = torch.device("cuda:0")
    x = torch.ones((B, T, H, 16), dtype=torch.bfloat16, device=dev)
    sink = torch.empty(B * H * 64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    for _ in range(reps):
        rc = lib.based_probe_read_rows(x.data_ptr(), B, T, H, sink.data_ptr(), stream)
        if rc != 0:
            raise SystemExit(f"based_probe_read_rows failed: {rc}")
    torch.cuda.synchronize()
    print(json.dumps({"row_probe_bytes_read": B * T * H * 32, "launches": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back steps for at least this long before the warm-up steps")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="measure the selected workload only (the JSON line then has no other configurations)")
    ap.add_argument("--all", action="store_true", help="also print a line per workload to stderr")
    ap.add_argument("--oracle-all", action="store_true",
                    help="with --all, also time the oracle (3 s sample) on every workload")
    ap.add_argument("--page-shapes", action="store_true",
                    help="also print a line per measure and grader shape of the page to stderr")
    ap.add_argument("--decode", default=None, metavar="B,H,K,V[;B,H,K,V...]",
                    help="also print a line per one-token decode-step shape (stderr)")
    ap.add_argument("--with-state", action="store_true",
                    help="also print the forward with state in and out against the plain forward (stderr)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--row-probe", default=None, metavar="B,T,H",
                    help="only run the 32-byte-row read probe over a (B,T,H,16) bf16 tensor (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this implementation has no multi-GPU path "
              "(every (batch, head) pair is independent; see the sharding notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_probe_mib > 0:
        copy_probe(a.copy_probe_mib, a.steps)
        return
    if a.row_probe:
        row_probe(*(int(x) for x in a.row_probe.split(",")), a.steps)
        return
    if a.steps < 1 or a.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    from taylor_feature_map_amd.inputs import WORKLOADS
    w_main = pick_workload(a.workload)
    # Every benchmark configuration is measured (warm and cold) and summarised in the JSON line; the main
    # workload's figures are the line's own. --all adds the headline shape with fp32 output on stderr.
    summaries, main_res = [], None
    for w in ([w_main] if a.only else WORKLOADS):
        r = run_bench(w, a.steps, a.warmup, with_cpu=(w == w_main and not a.no_cpu_baseline) or a.oracle_all,
                      settle_s=a.settle_ms / 1e3, cpu_budget_s=10.0 if w == w_main else 3.0)
        summaries.append(config_summary(r))
        if "cpu_baseline" in r and w != w_main:
            summaries[-1]["oracle_tokens_per_s"] = r["cpu_baseline"]["value"]
        if a.all:
            log(json.dumps(summaries[-1]))
        if w == w_main:
            main_res = r
    if main_res is None:
        main_res = run_bench(w_main, a.steps, a.warmup, with_cpu=not a.no_cpu_baseline, settle_s=a.settle_ms / 1e3)
    if a.all:
        import dataclasses
        head = pick_workload(None)
        extra = dataclasses.replace(head, name=head.name + "_f32out", out_dtype="f32")
        log(json.dumps(config_summary(run_bench(extra, a.steps, a.warmup, with_cpu=False,
                                                settle_s=a.settle_ms / 1e3))))
    if a.page_shapes:
        from taylor_feature_map_amd.inputs import PAGE_SHAPES
        for w in PAGE_SHAPES:
            if "_measure_" not in w.name and "_grader_" not in w.name:
                continue
            r = run_bench(w, max(5, a.steps // 5), max(2, a.warmup // 5), device_inputs=True,
                          settle_s=a.settle_ms / 1e3)
            log(json.dumps({"workload": w.name, "ms_per_step": r["ms_per_step"], "tokens_per_s": r["value"],
                            "tflops": r["tflops_canonical"], "path_hbm_frac": r["path_hbm_frac"],
                            "path_mfma_frac": r["path_mfma_frac"], "segments": r["config"]["segments"],
                            "kernels": r["kernels"]}))
            import torch
            torch.cuda.empty_cache()
    if a.decode:
        for spec in a.decode.split(";"):
            B, H, K, V = (int(x) for x in spec.split(","))
            log(json.dumps(decode_bench(B, H, K, V, max(a.steps, 100), a.settle_ms / 1e3)))
    if a.with_state:
        log(json.dumps(state_forward_bench(pick_workload(a.workload), a.steps, a.settle_ms / 1e3)))
    main_res["configs"] = summaries
    print(json.dumps(main_res), flush=True)


if __name__ == "__main__":
    main()

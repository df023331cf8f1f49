"""Forward throughput of the MI355X attention path on synthetic inputs.

One step is one ffpa_fwd launch over the whole workload (every query row of every head), with the
inputs already resident in HBM.  The default workload is large-head-dim self-attention
B=1, H=8, N=4096, D=512 in bf16; the JSON line also carries the D=1024 workloads as secondary
measurements.  FLOPs per step = 4*B*Hq*Nq*Nkv*D (halved when causal).  Peak = MI355X dense bf16/fp16
MFMA, 2516.6 TFLOP/s.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA (twice the 16-bit rate)
PEAK_SCLK_MHZ = 2400.0  # the shader clock the published peaks assume
METRIC = "forward TFLOPS + % of MI355X bf16 MFMA peak at D=512 and D=1024"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def timed(fn, steps: int, warmup: int, clock: bool = False):
    """Runs fn `warmup` times untimed, then `steps` times, each launch between its own pair of HIP
    events on torch's current stream (the stream the library's calls enqueue on), with a device
    synchronisation on both sides of the timed region.  Returns per-launch statistics in ms and, with
    clock=True, the shader clock of the timed launches: each launch's first wave of workgroup 0
    stamps the shader-clock and 100 MHz counters at its start and end (ffpa_clock_stamps), and the
    median over the launches of cycles / time is reported in MHz."""
    import torch

    import exact_attention_head_amd as ffpa

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    stamps = torch.zeros((steps, 4), dtype=torch.int64, device="cuda") if clock else None
    for i, (e0, e1) in enumerate(ev):
        if clock:
            ffpa.library().ffpa_clock_stamps(stamps[i].data_ptr())
        e0.record(stream)
        fn()
        e1.record(stream)
    if clock:
        ffpa.library().ffpa_clock_stamps(None)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    total = ev[0][0].elapsed_time(ev[-1][1])
    sclk = None
    if clock:
        st = stamps.cpu().tolist()
        mhz = [(c1 - c0) * 100.0 / (r1 - r0) for c0, r0, c1, r1 in st if r1 > r0 and c1 > c0]
        sclk = round(_median(mhz), 1) if mhz else None
    return dict(median_ms=_median(per), min_ms=per[0], max_ms=per[-1], mean_ms=total / steps, sclk_mhz=sclk)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def time_workload(w, steps: int, warmup: int, clock: bool = False):
    """Times `steps` launches after `warmup` untimed ones; returns (launch statistics, inputs, outputs)."""
    import torch

    import exact_attention_head_amd as ffpa
    import workloads as W

    q, k, v, mask = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = mask.to(dev) if mask is not None else None
    gqa = w.Hq != w.Hkv
    o = torch.empty_like(qd)

    def step():
        return ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=w.causal, enable_gqa=gqa, return_lse=True, out=o)

    res = {}

    def step_keep():
        res["lse"] = step()[1]

    st = timed(step_keep, steps, warmup, clock=clock)
    return st, (q, k, v, mask), (o.cpu(), res["lse"].cpu())


def time_dropout(w, p: float, steps: int, warmup: int):
    """Times the forward with attention dropout (ffpa_fwd_dropout, keep words drawn once beforehand) and,
    separately, the keep-word generator (ffpa_dropout_keep); returns the two launch statistics."""
    import torch

    import exact_attention_head_amd as ffpa
    import workloads as W

    q, k, v, mask = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = mask.to(dev) if mask is not None else None
    o = torch.empty_like(qd)
    keep = ffpa.dropout_keep(w.B, w.Hq, w.Nq, w.Nkv, p, seed=w.seed, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        return ffpa.attn(qd, kd, vd, attn_mask=md, dropout_p=p, dropout_keep=keep, is_causal=w.causal,
                         enable_gqa=w.Hq != w.Hkv, return_lse=True, out=o)

    def gen():
        st = ffpa.ffpa_dropout_keep(keep.data_ptr(), w.B, w.Hq, w.Nq, w.Nkv, p, w.seed, 0, stream.cuda_stream)
        if st != ffpa.OK:
            raise RuntimeError(f"ffpa_dropout_keep returned {st}")

    return timed(fwd, steps, warmup), timed(gen, steps, warmup)


def fp8_quantize(x):
    """Per-head e4m3 codes of a host float tensor [B, H, N, D] and the factors that undo the scaling
    (head max |x| / 448): input preparation, outside the timed region."""
    import torch

    s = (x.float().abs().amax(dim=(2, 3)) / 448.0).clamp_min(1e-12)
    return (x.float() / s[:, :, None, None]).to(torch.float8_e4m3fn), s.float()


def time_fp8(w, steps: int, warmup: int, clock: bool = False):
    """Times ffpa_fwd_fp8 on the workload's q, k, v quantised per head to e4m3 (bf16 output)."""
    import torch

    import exact_attention_head_amd as ffpa
    import workloads as W

    q, k, v, mask = W.make_inputs(w)
    dev = torch.device("cuda:0")
    (q8, dq), (k8, dk), (v8, dv) = (fp8_quantize(t) for t in (q, k, v))
    qd, kd, vd, dqd, dkd, dvd = (t.to(dev) for t in (q8, k8, v8, dq, dk, dv))
    md = mask.to(dev) if mask is not None else None
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

    def step():
        ffpa.attn_fp8(qd, kd, vd, dqd, dkd, dvd, attn_mask=md, is_causal=w.causal, enable_gqa=w.Hq != w.Hkv, out=o)

    return timed(step, steps, warmup, clock=clock)


def time_varlen(w, steps: int, warmup: int, clock: bool = False):
    """As time_workload, for a packed variable-length batch (one ffpa_fwd_varlen launch per step)."""
    import torch

    import exact_attention_head_amd as ffpa
    import workloads as W

    q, k, v, cu_q, cu_k = W.make_varlen_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, cqd, ckd = (t.to(dev) for t in (q, k, v, cu_q, cu_k))
    Tq, Tk = q.shape[0], k.shape[0]
    o = torch.empty_like(qd)
    lse = torch.empty((w.Hq, Tq), dtype=torch.float32, device=dev)
    dtype = ffpa.FFPA_BF16 if w.dtype == torch.bfloat16 else ffpa.FFPA_FP16
    # the offsets are checked once on the host, as attn_varlen does before every launch
    for c, T, mx in ((cu_q, Tq, max(w.lens_q)), (cu_k, Tk, max(w.lens_k))):
        assert ffpa.ffpa_check_cu_seqlens(c.tolist(), T, mx) == ffpa.OK
    stream = torch.cuda.current_stream()

    def step():
        st = ffpa.ffpa_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), cqd.data_ptr(), ckd.data_ptr(),
                                  o.data_ptr(), lse.data_ptr(), len(w.lens_q), w.Hq, w.Hkv, Tq, Tk, max(w.lens_q),
                                  max(w.lens_k), w.D, float("nan"), w.causal, dtype, stream.cuda_stream)
        if st != ffpa.OK:
            raise RuntimeError(f"ffpa_fwd_varlen returned {st}")

    return timed(step, steps, warmup, clock=clock)


def time_backward(w, steps: int, warmup: int):
    """Times ffpa_bwd (dQ, dK, dV) of a dense workload after one forward for its O and LSE; returns the
    statistics of the whole ffpa_bwd call."""
    import torch

    import exact_attention_head_amd as ffpa
    import workloads as W

    q, k, v, mask = W.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = mask.to(dev) if mask is not None else None
    gqa = w.Hq != w.Hkv
    o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=w.causal, enable_gqa=gqa, return_lse=True)
    do = torch.randn(qd.shape, generator=torch.Generator(device=dev).manual_seed(w.seed + 5), device=dev,
                     dtype=torch.float32).to(w.dtype)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    nbytes = ffpa.ffpa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    desc, keep = (None, None) if md is None else ffpa._mask_desc(md, w.B, w.Hq, w.Nq, w.Nkv)
    dtype = ffpa.FFPA_BF16 if w.dtype == torch.bfloat16 else ffpa.FFPA_FP16
    stream = torch.cuda.current_stream()

    def step():
        st = ffpa.ffpa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           desc, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                           float("nan"), w.causal, dtype, ws.data_ptr(), nbytes, stream.cuda_stream)
        if st != ffpa.OK:
            raise RuntimeError(f"ffpa_bwd returned {st}")

    st = timed(step, steps, warmup)
    del keep
    return st


def cpu_baseline(w, inputs, outputs, seconds: float):
    """Times the fp64 oracle on a bounded sample of rows of the same workload (all host threads it
    uses), scales to TFLOPS by the metric's FLOP count, and compares those rows with the GPU output."""
    import numpy as np

    import oracle
    import workloads as W

    q, k, v, mask = inputs
    o_gpu, lse_gpu = outputs
    rng = np.random.default_rng(w.seed + 99)
    rows_all = rng.permutation(w.B * w.Hq * w.Nq)  # seeded random rows, drawn until the time budget is spent

    def row_flops(rows):
        if not w.causal:
            return 4.0 * w.Nkv * w.D * len(rows)
        vis = [min(w.Nkv, (r % w.Nq) + w.Nkv - w.Nq + 1) for r in rows]
        return 4.0 * w.D * float(sum(vis))

    n = 8
    t_total, f_total, done = 0.0, 0.0, []
    O_ref, L_ref = [], []
    while True:
        batch = rows_all[len(done):len(done) + n]
        if len(batch) == 0:
            break
        t0 = time.perf_counter()
        o_r, l_r = oracle.attention_rows(q, k, v, batch, mask=mask, is_causal=w.causal)
        dt = time.perf_counter() - t0
        t_total += dt
        f_total += row_flops(batch)
        done.extend(batch)
        O_ref.append(o_r)
        L_ref.append(l_r)
        if t_total >= seconds:
            break
        n = max(1, min(len(rows_all), int(len(batch) * min(4.0, max(1.5, seconds / max(t_total, 1e-3) / 2)))))
    rows = np.asarray(done, dtype=np.int64)
    o_ref, l_ref = np.concatenate(O_ref), np.concatenate(L_ref)
    og = o_gpu.float().numpy().reshape(-1, w.D)[rows].astype(np.float64)
    lg = lse_gpu.numpy().reshape(-1)[rows].astype(np.float64)
    fin = np.isfinite(l_ref)
    parity = dict(rows=int(rows.size), o_max_abs=float(np.abs(og - o_ref).max()),
                  o_rel_l2=float(np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)),
                  lse_max_abs=float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0)
    sample = (f"{rows.size} seeded random query rows of {w.B * w.Hq * w.Nq} (all heads), each against all of "
              f"its {w.Nkv if not w.causal else 'visible'} keys; fp64 oracle, ~{seconds:.0f} s budget")
    return dict(value=f_total / t_total / 1e12, unit="TFLOPS", cores=oracle.max_threads(), kind="oracle",
                sample=sample, seconds=round(t_total, 2)), parity


# the forward kernels and their launcher (the C-ABI checks and the backward do not change what a
# forward launch moves)
KERNEL_SOURCES = ("ffpa_kernel.hpp", "ffpa_row_kernel.hpp", "ffpa_launch.hpp", "ffpa_inst.hip", "ffpa_fp8_kernel.hpp",
                  "ffpa_fp8.hip")


def kernel_fingerprint() -> str:
    """First 16 hex digits of the SHA-256 over the kernel sources (ties measured traffic to a kernel)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str, workload: str):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs (already scaled by the copy
    calibration), or None when none were taken for this workload or the kernel changed since."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tj = json.load(f)
    if tj.get("kernel_sources_sha256_16") != kernel_fingerprint():
        log("traffic counters were taken on other kernel sources: traffic = null")
        return None
    ent = tj.get(workload)
    return None if ent is None else ent["hbm_bytes_per_launch"]


def copy_calibration() -> None:
    """A plain device copy of known size (for scaling the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch

    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_direction": n, "launches": 3}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_d_self",
                    help="tiny | large_d_self | gqa_causal | cross_mask | sweep:<D>[:fp16] | varlen_causal | "
                         "fp8:<one of those> (the fp8 forward on the workload quantised per head) | "
                         "bwd:<a dense one> (the backward alone)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 --pmc), if present")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="secondary lines for the whole head-dim sweep (every D, bf16 and fp16) instead of the default set")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch

    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    def pick(name):
        if name.startswith("sweep:"):
            parts = name.split(":")
            return W.sweep(int(parts[1]), torch.float16 if len(parts) > 2 and parts[2] == "fp16" else torch.bfloat16)
        return getattr(W, name)()

    fp8_main = args.workload.startswith("fp8:")
    bwd_main = args.workload.startswith("bwd:")
    w = pick(args.workload[4:] if fp8_main or bwd_main else args.workload)
    log(f"workload {'fp8 ' if fp8_main else ''}{w.name}: warmup {args.warmup}, steps {args.steps}")
    packed = isinstance(w, W.VarlenWorkload)
    if bwd_main:
        # the backward alone (profiling runs): one JSON line, five products' FLOPs against the peak
        st = time_backward(w, args.steps, args.warmup)
        tf = 2.5 * w.flops / (st["median_ms"] * 1e-3) / 1e12
        log(f"backward {w.name}: median {st['median_ms']:.4f} ms/call, {tf:.1f} TFLOPS "
            f"({100 * tf / PEAK_TFLOPS:.1f}% of peak)")
        print(json.dumps({"metric": "backward TFLOPS", "value": round(tf, 2), "unit": "TFLOPS", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(st["median_ms"], 5),
                          "higher_is_better": True, "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp16",
                          "data": "synthetic", "config": w.describe(),
                          "roofline": dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_TFLOPS, unit="TFLOP/s",
                                           frac=round(tf / PEAK_TFLOPS, 4),
                                           kernel="ffpa_bwd_kernel (dK/dV pass + dQ pass)")}), flush=True)
        return 0
    if fp8_main:
        # the fp8 forward alone (profiling runs): one JSON line against the fp8 peak, no CPU leg
        st = time_fp8(w, args.steps, args.warmup, clock=True)
        tf = w.flops / (st["median_ms"] * 1e-3) / 1e12
        log(f"fp8 {w.name}: median {st['median_ms']:.4f} ms/launch, {tf:.1f} TFLOPS "
            f"({100 * tf / PEAK_FP8_TFLOPS:.1f}% of the fp8 peak), shader clock {st['sclk_mhz']} MHz")
        print(json.dumps({"metric": "fp8 forward TFLOPS", "value": round(tf, 2), "unit": "TFLOPS", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(st["median_ms"], 5),
                          "higher_is_better": True, "dtype": "e4m3", "data": "synthetic", "sclk_mhz": st["sclk_mhz"],
                          "config": dict(w.describe(), inputs="e4m3 per-head factors"),
                          "roofline": dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_FP8_TFLOPS,
                                           unit="TFLOP/s", frac=round(tf / PEAK_FP8_TFLOPS, 4),
                                           traffic=measured_traffic(args.traffic_json, "fp8:" + w.name),
                                           traffic_unit="HBM bytes per launch",
                                           kernel="ffpa_fwd_fp8_kernel")}), flush=True)
        return 0
    if packed:
        st, inputs, outputs = time_varlen(w, args.steps, args.warmup, clock=True), None, None
    else:
        st, inputs, outputs = time_workload(w, args.steps, args.warmup, clock=True)
    # the headline figure is the median launch; mean, min and max sit beside it
    ms = st["median_ms"]
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"{w.name}: median {ms:.4f} ms/launch (min {st['min_ms']:.4f}, mean {st['mean_ms']:.4f}), "
        f"{tflops:.1f} TFLOPS ({100 * tflops / PEAK_TFLOPS:.1f}% of peak), shader clock {st['sclk_mhz']} MHz")

    traffic = measured_traffic(args.traffic_json, w.name)
    import exact_attention_head_amd as ffpa

    kernel = ffpa.kernel_name(w.D)
    roofline = dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tflops / PEAK_TFLOPS, 4), traffic=traffic, traffic_unit="HBM bytes per launch",
                    kernel=kernel, flops_per_launch=w.flops, avg_launch_ms=round(st["mean_ms"], 5),
                    median_launch_ms=round(ms, 5))

    secondary = []
    if args.sweep:
        names = [f"sweep:{d}" for d in W.SWEEP_D] + [f"sweep:{d}:fp16" for d in W.SWEEP_D]
    else:
        names = ["cross_mask", "sweep:1024", "gqa_causal", "sweep:512", "varlen_causal", "fp8:large_d_self",
                 "fp8:sweep:512", "fp8:sweep:1024", "drop:large_d_self", "drop:sweep:1024", "bwd:large_d_self", "bwd:sweep:1024"]
    if not args.no_secondary and args.workload == "large_d_self":
        for name in names:
            backward = name.startswith("bwd:")
            dropout = name.startswith("drop:")
            fp8 = name.startswith("fp8:")
            w2 = pick(name[5:] if dropout else (name[4:] if backward or fp8 else name))
            peak = PEAK_FP8_TFLOPS if fp8 else PEAK_TFLOPS
            if fp8:
                # e4m3 inputs with per-head factors, both products on the fp8 matrix core: against its peak
                st2, flops2 = time_fp8(w2, max(5, args.steps // 2), 2), w2.flops
            elif dropout:
                # forward with attention dropout at p = 0.1: same FLOP count; the keep-word generator apart
                st2, gst = time_dropout(w2, 0.1, max(5, args.steps // 2), 2)
                gen_ms = gst["median_ms"]
                flops2 = w2.flops
                log(f"dropout keep words {w2.name}: {gen_ms:.4f} ms/launch")
            elif backward:
                # the backward's five products: 10*B*Hq*Nq*Nkv*D FLOPs (2.5x the forward), halved for causal
                st2 = time_backward(w2, max(3, args.steps // 5), 1)
                flops2 = 2.5 * w2.flops
            elif isinstance(w2, W.VarlenWorkload):
                st2, flops2 = time_varlen(w2, max(5, args.steps // 2), 2), w2.flops
            else:
                (st2, _, _), flops2 = time_workload(w2, max(5, args.steps // 2), 2), w2.flops
            ms2 = st2["median_ms"]
            tf2 = flops2 / (ms2 * 1e-3) / 1e12
            tag = ("backward " if backward else ("dropout p=0.1 " if dropout else ("fp8 " if fp8 else ""))) + w2.name
            log(f"{tag}: {ms2:.4f} ms/launch, {tf2:.1f} TFLOPS ({100 * tf2 / peak:.1f}% of the "
                f"{'fp8' if fp8 else 'bf16'} peak)")
            kname = ("ffpa_bwd_kernel (dK/dV pass + dQ pass)" if backward else
                     ("ffpa_fwd_fp8_kernel" if fp8 else ffpa.kernel_name(w2.D)))
            secondary.append(dict(workload=tag, D=w2.D,
                                  dtype="e4m3" if fp8 else ("bf16" if w2.dtype == torch.bfloat16 else "fp16"),
                                  kernel=kname, peak_tflops=peak,
                                  **({"keep_words_ms": round(gen_ms, 4)} if dropout else {}),
                                  ms_per_step=round(ms2, 4), min_ms=round(st2["min_ms"], 4),
                                  mean_ms=round(st2["mean_ms"], 4), tflops=round(tf2, 2),
                                  frac_of_peak=round(tf2 / peak, 4)))

    cpu, parity = None, None
    if packed and not args.no_cpu_baseline:
        log("cpu baseline: measured on the dense workloads only")
    elif not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on sampled rows (~{args.cpu_seconds:.0f} s)")
        cpu, parity = cpu_baseline(w, inputs, outputs, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.4g} TFLOPS on {cpu['cores']} threads; parity {parity}")

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp16", "data": "synthetic",
        "median_ms": round(ms, 5), "min_ms": round(st["min_ms"], 5), "mean_ms": round(st["mean_ms"], 5),
        "max_ms": round(st["max_ms"], 5), "sclk_mhz": st["sclk_mhz"], "cpu_model": cpu_model(),
        "config": w.describe(), "frac_of_peak": round(tflops / PEAK_TFLOPS, 4),
        # the same fraction against the peak at the shader clock the launches ran at (the published peak
        # assumes the 2400 MHz maximum)
        "frac_of_peak_at_sclk": (round(tflops / (PEAK_TFLOPS * st["sclk_mhz"] / PEAK_SCLK_MHZ), 4)
                                 if st["sclk_mhz"] else None),
        "roofline": roofline,
        "cpu_baseline": cpu, "parity_sample": parity, "secondary": secondary,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

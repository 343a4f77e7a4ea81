"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
fa_fwd on the largest prefill workload (causal GQA, B=1, Hq=32, Hkv=8,
N=16384, d=128, bf16) followed by fa_fwd_kvcache (split-KV decode +
combine) on the GQA decode workload (B=64, Hq=32, Hkv=8, d=128, cache
capacity 8192, lengths uniform in [1024, 8192]). Inputs are generated on
the device before the timed region.

Clocks. The GPU's clocks take about a second of sustained work to settle,
so after the --warmup steps the step keeps running until --settle seconds
of wall time have passed since the first warm-up step; only then are the
--steps timed steps run. The JSON reports how long that phase lasted
(`settle_s`) and how many steps it took.

Each launch is bracketed by HIP events on the stream it runs on; `value` is
the prefill's algorithmic TFLOP/s (4*B*H*Nq*Nk*d, halved for causal) over
its mean event time, and the decode's algorithmic GB/s is reported beside
it. After the step loop, and outside its clock, the other prefill workloads
(the causal training shape B=8 H=16 N=2048 d=128, and the non-causal
variance-4 shapes at d=64 and d=256) are timed one after another, each
after its own short settle, and reported with their own rooflines under
`configs`; then the backward, the FP8 forward (with its quantisation timed
apart), the paged-cache decode and decode steps that append 1 or 4 new
tokens per sequence. The CPU float64 oracle is timed last, on a bounded
sample of each workload, and the outputs of the timed launches are compared
with it on the same rows (`parity`: max-abs error of O and LSE against the
bars 2e-2 and 1e-3). Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle SECONDS]
                    [--prefill NAME] [--configs all|none|NAME,...]
                    [--no-cpu-baseline] [--splits S] [--bwd-steps N]
                    [--fp8-steps N] [--fp8-workload NAME] [--paged-steps N] [--append-steps N]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak; split-KV decode HBM GB/s & % peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 8192 flop/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0
TOL_O, TOL_LSE = 2e-2, 1e-3  # max-abs bars of O (bf16) and LSE against the float64 oracle
DEFAULT_PREFILL = "gqa_bf16_causal_h32kv8_n16384_d128"
DEFAULT_DECODE = "gqa_bf16_decode_b64_h32kv8_cap8192_d128"
# the other bf16 prefill workloads, timed after the step loop
OTHER_PREFILL = ["mha_bf16_causal_b8_h16_n2048_d128", "mha_bf16_b4_h16_n4096_d64_qkvar4",
                 "mha_bf16_b2_h8_n4096_d256_qkvar4"]
_CSRC = os.path.join(ROOT, "exact_io_aware_online_amd", "csrc")
# the files a kernel's machine code depends on
PREFILL_KERNEL_SOURCE = [os.path.join(_CSRC, f) for f in ("fa_fwd_bf16.hip", "fa_device.h", "fa_launch.h")]
DECODE_KERNEL_SOURCE = [os.path.join(_CSRC, f) for f in ("fa_decode.hip", "fa_device.h", "fa_launch.h")]


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_flops(w):
    f = 4.0 * w["B"] * w["Hq"] * w["Nq"] * w["Nk"] * w["d"]
    return f / 2 if w["causal"] else f


def decode_bytes(w, lens_sum, nq=1):
    """Algorithmic bytes of one decode call: the visible K and V rows, q, o,
    lse and the lengths."""
    return (lens_sum * w["Hkv"] * w["d"] * 2 * 2 + 2 * w["B"] * nq * w["Hq"] * w["d"] * 2
            + w["B"] * w["Hq"] * nq * 4 + w["B"] * 4)


def stored_traffic(kernel_key, src):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha256_16") != source_hash(src):
        return None
    return rec.get("bytes_per_launch")


def _host_info():
    blas = "unknown"
    cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        cores = max([p.get("num_threads", 1) for p in pools] or [cores])
        if pools:
            blas = f"{pools[0].get('internal_api', '?')} {pools[0].get('version', '')}".strip()
    except Exception:
        pass
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return int(cores), cpu, blas


def cpu_baseline(name, w, budget_s=12.0, tensors=None, block_rows=1024, outputs=None):
    """The CPU float64 oracle, as is, on blocks of query rows of whole
    (batch, head) slices of the same prefill workload until about
    `budget_s` seconds have passed. The oracle materialises every row's
    full score row (all Nk keys, then the mask), so its rate per row does
    not depend on which rows are taken; the rate is reported in the
    metric's accounting (the workload's algorithmic flops per query row).
    `tensors` are the workload's (q, k, v), else they are drawn on the CPU.
    With `outputs` (the GPU's O and LSE of the timed launches, on the CPU)
    the same oracle rows are compared with them; the comparison is not
    counted in the oracle's time. Returns (baseline, parity or None)."""
    import numpy as np
    import torch

    import seeded_inputs as SI
    from oracle import sdpa as O

    q, k, v = tensors if tensors is not None else SI.prefill_inputs(device="cpu", **w)
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    G = w["Hq"] // w["Hkv"]
    rows_done = 0
    slices = 0
    err_o = err_l = 0.0
    cmp_s = 0.0
    t0 = time.perf_counter()
    done = False
    for b in range(w["B"]):
        for h in range(w["Hq"]):
            kv = h // G
            kk, vv = f64(k[b:b + 1, :, kv:kv + 1]), f64(v[b:b + 1, :, kv:kv + 1])
            for r0 in range(0, w["Nq"], block_rows):
                r1 = min(r0 + block_rows, w["Nq"])
                if w["causal"]:  # absolute row indices: the mask compares them with key positions
                    o_ref, l_ref = O.attention_rows(f64(q[b:b + 1, :r1, h:h + 1]), kk, vv, True, scale, 0, 0,
                                                    rows=np.arange(r0, r1))
                else:
                    o_ref, l_ref = O.attention_rows(f64(q[b:b + 1, r0:r1, h:h + 1]), kk, vv, False, scale, 0, 0)
                if outputs is not None:
                    c0 = time.perf_counter()
                    err_o = max(err_o, float(np.max(np.abs(f64(outputs[0][b, r0:r1, h]) - o_ref))))
                    err_l = max(err_l, float(np.max(np.abs(f64(outputs[1][b, h, r0:r1]) - l_ref))))
                    cmp_s += time.perf_counter() - c0
                rows_done += r1 - r0
                if time.perf_counter() - t0 >= budget_s:
                    done = True
                    break
            slices += 1
            if done:
                break
        if done:
            break
    el = time.perf_counter() - t0 - cmp_s
    per_row = prefill_flops(w) / (w["B"] * w["Hq"] * w["Nq"])
    cores, cpu, blas = _host_info()
    base = {"value": per_row * rows_done / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_done} query rows ({rows_done / w['Nq']:.2f} (batch, head) slices) of {name}, "
                      f"full fp64 score row each, {el:.1f} s",
            "cpu": cpu, "blas": blas}
    parity = None
    if outputs is not None:
        parity = {"rows": rows_done, "max_abs_o": err_o, "max_abs_lse": err_l, "bar_o": TOL_O, "bar_lse": TOL_LSE,
                  "within": err_o <= TOL_O and err_l <= TOL_LSE}
    return base, parity


def cpu_baseline_decode(name, w, q, kc, vc, lens, budget_s=4.0, outputs=None):
    """The CPU float64 oracle's decode on whole sequences (all query heads)
    of the decode workload until about `budget_s` seconds have passed;
    GB/s over the same algorithmic bytes as the GPU figure. With `outputs`
    (the GPU's O and LSE) the same sequences are compared with them, outside
    the oracle's time. Returns (baseline, parity or None)."""
    import numpy as np
    import torch

    from oracle import sdpa as O

    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    lens_h = lens.cpu().numpy()
    nbytes = 0
    seqs = 0
    err_o = err_l = 0.0
    cmp_s = 0.0
    t0 = time.perf_counter()
    for b in range(w["B"]):
        n = int(lens_h[b])
        o_ref, l_ref = O.decode(f64(q[b:b + 1]), f64(kc[b:b + 1, :n]), f64(vc[b:b + 1, :n]), [n], scale)
        if outputs is not None:
            c0 = time.perf_counter()
            err_o = max(err_o, float(np.max(np.abs(f64(outputs[0][b, 0]) - o_ref[0]))))
            err_l = max(err_l, float(np.max(np.abs(f64(outputs[1][b]) - l_ref[0]))))
            cmp_s += time.perf_counter() - c0
        nbytes += n * w["Hkv"] * w["d"] * 2 * 2 + 2 * w["Hq"] * w["d"] * 2 + w["Hq"] * 4 + 4
        seqs += 1
        if time.perf_counter() - t0 - cmp_s >= budget_s:
            break
    el = time.perf_counter() - t0 - cmp_s
    cores, cpu, blas = _host_info()
    base = {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{seqs} of {w['B']} sequences of {name} (all query heads), fp64, {el:.1f} s",
            "cpu": cpu, "blas": blas}
    parity = None
    if outputs is not None:
        parity = {"sequences": seqs, "max_abs_o": err_o, "max_abs_lse": err_l, "bar_o": TOL_O, "bar_lse": TOL_LSE,
                  "within": err_o <= TOL_O and err_l <= TOL_LSE}
    return base, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=2.0,
                    help="keep running warm-up steps until this many seconds have passed (clock settle)")
    ap.add_argument("--prefill", default=DEFAULT_PREFILL)
    ap.add_argument("--decode", default=DEFAULT_DECODE)
    ap.add_argument("--configs", default="all",
                    help="other prefill workloads timed after the step loop: all, none, or names joined by ','")
    ap.add_argument("--config-launches", type=int, default=30)
    ap.add_argument("--config-settle", type=float, default=0.4)
    ap.add_argument("--splits", type=int, default=0, help="decode num_splits (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time for the headline")
    ap.add_argument("--cpu-budget-other", type=float, default=3.0, help="seconds of oracle time per other config")
    ap.add_argument("--bwd-steps", type=int, default=20,
                    help="timed fa_bwd calls on the causal training-shape workload (0 = skip)")
    ap.add_argument("--fp8-steps", type=int, default=20,
                    help="timed FP8 forward calls (fa_fwd_fp8, Q and K quantised with the rotation) after the step "
                         "loop (0 = skip)")
    ap.add_argument("--fp8-workload", default="mha_bf16_causal_b8_h16_n2048_d128",
                    help="bf16 prefill workload the FP8 forward runs on (default: the causal training shape)")
    ap.add_argument("--append-steps", type=int, default=20,
                    help="timed decode-with-append calls (1 and 4 new tokens per sequence) (0 = skip)")
    ap.add_argument("--paged-steps", type=int, default=20,
                    help="timed paged-cache decode calls after the step loop (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (outside the timed "
                         "region) as the known-size reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single GPU's share; no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_online_amd as fa
    import seeded_inputs as SI

    fa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    Ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        """Mean event time (ms) of n calls of fn, each bracketed by events."""
        evs = [(Ev(), Ev()) for _ in range(n)]
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) / n

    def settle(fn, seconds, min_calls=1):
        t0 = time.perf_counter()
        n = 0
        while n < min_calls or time.perf_counter() - t0 < seconds:
            fn()
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return n, time.perf_counter() - t0

    wp = SI.PREFILL_WORKLOADS[args.prefill]
    wd = SI.DECODE_WORKLOADS[args.decode]
    q, k, v = SI.prefill_inputs(device=dev, **wp)
    scale_p = 1.0 / math.sqrt(wp["d"])
    o = torch.empty_like(q)
    lse = torch.empty((wp["B"], wp["Hq"], wp["Nq"]), dtype=torch.float32, device=dev)

    qd, kc, vc, lens = SI.decode_inputs(device=dev, **wd)
    S = args.splits or fa.fa_kvcache_default_splits(wd["B"], wd["Hkv"], wd["capacity"], wd["d"])
    od = torch.empty_like(qd)
    lsed = torch.empty((wd["B"], wd["Hq"]), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_fwd_kvcache_workspace_size(wd["B"], wd["Hq"], wd["d"], S)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    scale_d = 1.0 / math.sqrt(wd["d"])
    lens_sum = int(lens.to(torch.int64).sum().item())
    dec_bytes = decode_bytes(wd, lens_sum)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, o=o, lse=lse, causal=wp["causal"], scale=scale_p)
        if ev is not None:
            ev[1].record()
        fa.fa_fwd_kvcache(qd, kc, vc, lens, o=od, lse=lsed, num_splits=S, scale=scale_d, workspace=ws)
        if ev is not None:
            ev[2].record()

    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    settle_steps, settle_s = settle(step, args.settle, min_calls=args.warmup)

    events = [[Ev() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pf_ms = [e[0].elapsed_time(e[1]) for e in events]
    dc_ms = [e[1].elapsed_time(e[2]) for e in events]
    pf_mean = sum(pf_ms) / len(pf_ms)
    dc_mean = sum(dc_ms) / len(dc_ms)
    flops = prefill_flops(wp)
    tflops = flops / (pf_mean * 1e-3) / 1e12
    gbs = dec_bytes / (dc_mean * 1e-3) / 1e9

    def prefill_entry(name, w, ms, launches):
        tf = prefill_flops(w) / (ms * 1e-3) / 1e12
        return {"workload": name, "kernel": f"fwd_bf16_kernel<{w['d']}>", "bound": "mfma",
                "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic("prefill:" + name, PREFILL_KERNEL_SOURCE),
                "algorithmic_flops_per_launch": prefill_flops(w), "mean_launch_ms": round(ms, 5),
                "launches": launches}

    configs = {args.prefill: prefill_entry(args.prefill, wp, pf_mean, args.steps)}
    other = OTHER_PREFILL if args.configs == "all" else ([] if args.configs == "none" else args.configs.split(","))
    cpu_tensors = {}
    for name in other:
        if name == args.prefill:
            continue
        w = SI.PREFILL_WORKLOADS[name]
        qx, kx, vx = SI.prefill_inputs(device=dev, **w)
        ox = torch.empty_like(qx)
        lx = torch.empty((w["B"], w["Hq"], w["Nq"]), dtype=torch.float32, device=dev)
        sc = 1.0 / math.sqrt(w["d"])
        fn = lambda: fa.fa_fwd(qx, kx, vx, o=ox, lse=lx, causal=w["causal"], scale=sc)
        settle(fn, args.config_settle, min_calls=3)
        ms = timed(fn, args.config_launches)
        configs[name] = prefill_entry(name, w, ms, args.config_launches)
        if not args.no_cpu_baseline:
            cpu_tensors[name] = ((qx.cpu(), kx.cpu(), vx.cpu()), (ox.cpu(), lx.cpu()))
        del qx, kx, vx, ox, lx

    # The backward of the causal training-shape workload (fa_bwd: dQ, dK,
    # dV from the forward's O and LSE). Algorithmic work: the five
    # N x N x d products of the gradient formulas, 2.5x the forward's.
    wt_name = "mha_bf16_causal_b8_h16_n2048_d128"
    wt = SI.PREFILL_WORKLOADS[wt_name]
    bwd = fp8 = None
    if args.bwd_steps > 0 or args.fp8_steps > 0:
        qt, kt, vt = SI.prefill_inputs(device=dev, **wt)
        ot = torch.empty_like(qt)
        lt = torch.empty((wt["B"], wt["Hq"], wt["Nq"]), dtype=torch.float32, device=dev)
        scale_t = 1.0 / math.sqrt(wt["d"])
        fa.fa_fwd(qt, kt, vt, o=ot, lse=lt, causal=True, scale=scale_t)
    if args.bwd_steps > 0:
        g = torch.Generator(device=dev)
        g.manual_seed(wt["seed"] + 1000)
        dout = torch.randn(qt.shape, generator=g, device=dev).to(qt.dtype)
        dq, dk, dv = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
        bws = torch.empty(max(fa.fa_bwd_workspace_size(wt["B"], wt["Hq"], wt["Nq"]), 1), dtype=torch.uint8,
                          device=dev)

        def bstep():
            fa.fa_bwd(qt, kt, vt, ot, lt, dout, causal=True, scale=scale_t, dq=dq, dk=dk, dv=dv, workspace=bws)
        settle(bstep, 0.2, min_calls=3)
        b_ms = timed(bstep, args.bwd_steps)
        b_tf = 2.5 * prefill_flops(wt) / (b_ms * 1e-3) / 1e12
        bwd = {"workload": wt_name, "value": round(b_tf, 2), "unit": "TFLOP/s", "mean_launch_ms": round(b_ms, 5),
               "frac": round(b_tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops_per_launch": 2.5 * prefill_flops(wt),
               "kernels": "bwd_prep_kernel + bwd_dq_kernel + bwd_dkdv_kernel", "steps": args.bwd_steps}
        del dout, dq, dk, dv, bws

    # The same workload in FP8: Q and K rotated and block-quantised, V
    # block-quantised (timed on its own, outside the attention's clock),
    # then fa_fwd_fp8, priced against the dense FP8 peak.
    if args.fp8_steps > 0:
        wf_name = args.fp8_workload
        wf = SI.PREFILL_WORKLOADS.get(wf_name)
        if wf is None or wf["dtype"] != "bf16":
            raise SystemExit(f"--fp8-workload: not a bf16 prefill workload: {wf_name}")
        if wf_name == wt_name:
            qf, kf, vf = qt, kt, vt
        else:
            qf, kf, vf = SI.prefill_inputs(device=dev, **wf)
        scale_f = 1.0 / math.sqrt(wf["d"])
        signs = SI.random_signs(wf["d"], seed=wf["seed"] + 4000).to(dev)
        q8, qs8 = fa.fa_quantize_fp8(qf, signs=signs)
        k8, ks8 = fa.fa_quantize_fp8(kf, signs=signs)
        vt8, vs8 = fa.fa_quantize_fp8(vf, transpose=True)
        o8 = torch.empty_like(qf)
        l8 = torch.empty((wf["B"], wf["Hq"], wf["Nq"]), dtype=torch.float32, device=dev)

        def fstep():
            fa.fa_fwd_fp8(q8, qs8, k8, ks8, vt8, vs8, wf["Nq"], wf["Nk"], causal=wf["causal"], scale=scale_f, o=o8,
                          lse=l8)

        def qstep():
            fa.fa_quantize_fp8(qf, signs=signs, codes=q8, scales=qs8)
            fa.fa_quantize_fp8(kf, signs=signs, codes=k8, scales=ks8)
            fa.fa_quantize_fp8(vf, transpose=True, codes=vt8, scales=vs8)
        settle(fstep, 0.2, min_calls=3)
        f_ms = timed(fstep, args.fp8_steps)
        q_ms = timed(qstep, 10)
        f_tf = prefill_flops(wf) / (f_ms * 1e-3) / 1e12
        fp8 = {"workload": wf_name, "value": round(f_tf, 2), "unit": "TFLOP/s",
               "kernel": f"fwd_fp8_kernel<{wf['d']}>", "dtype": "e4m3", "peak": PEAK_FP8_TFLOPS,
               "frac": round(f_tf / PEAK_FP8_TFLOPS, 4), "mean_launch_ms": round(f_ms, 5),
               "quantize_ms": round(q_ms, 5), "steps": args.fp8_steps}
        del q8, k8, vt8, o8, qf, kf, vf

    # The decode workload again over a paged cache (256-row pages in a
    # shuffled pool, the same keys).
    paged = None
    if args.paged_steps > 0:
        P = 256
        pps = wd["capacity"] // P
        g = torch.Generator(device="cpu")
        g.manual_seed(wd["seed"] + 2000)
        perm = torch.randperm(wd["B"] * pps, generator=g).to(dev)
        bt = perm.reshape(wd["B"], pps).to(torch.int32).contiguous()
        inv = torch.argsort(perm)
        kp = kc.reshape(wd["B"] * pps, P, wd["Hkv"], wd["d"])[inv].contiguous()
        vp = vc.reshape(wd["B"] * pps, P, wd["Hkv"], wd["d"])[inv].contiguous()

        def pstep():
            fa.fa_fwd_kvcache_paged(qd, kp, vp, bt, lens, o=od, lse=lsed, num_splits=S, scale=scale_d, workspace=ws)
        settle(pstep, 0.2, min_calls=3)
        p_ms = timed(pstep, args.paged_steps)
        paged = {"value": round(dec_bytes / (p_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "page_size": P,
                 "mean_launch_ms": round(p_ms, 5), "frac": round(dec_bytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "steps": args.paged_steps}
        del kp, vp

    # Decode steps that append 1 or 4 new tokens per sequence to the same
    # cache (the write happens inside the split kernel), queries bottom-right
    # causal; lengths are capped so the new rows fit. Bytes: the visible
    # cache rows read, the new rows read and written, q, o, lse, lengths.
    append = None
    if args.append_steps > 0:
        append = {}
        for nq in (1, 4):
            lens_a = torch.clamp(lens, max=wd["capacity"] - nq).contiguous()
            g = torch.Generator(device=dev)
            g.manual_seed(wd["seed"] + 3000 + nq)
            qa = torch.randn((wd["B"], nq, wd["Hq"], wd["d"]), generator=g, device=dev).to(torch.bfloat16)
            kn = torch.randn((wd["B"], nq, wd["Hkv"], wd["d"]), generator=g, device=dev).to(torch.bfloat16)
            vn = torch.randn((wd["B"], nq, wd["Hkv"], wd["d"]), generator=g, device=dev).to(torch.bfloat16)
            oa = torch.empty_like(qa)
            la = torch.empty((wd["B"], wd["Hq"], nq), dtype=torch.float32, device=dev)
            Sa = fa.fa_kvcache_append_default_splits(wd["B"], nq, wd["Hkv"], wd["Hq"], wd["capacity"], wd["d"])
            wsa = torch.empty(max(fa.fa_fwd_kvcache_workspace_size(wd["B"] * nq, wd["Hq"], wd["d"], Sa), 1),
                              dtype=torch.uint8, device=dev)
            rows = int(lens_a.to(torch.int64).sum().item()) + wd["B"] * nq
            a_bytes = (rows * wd["Hkv"] * wd["d"] * 2 * 2 + 2 * kn.numel() * 2 * 2
                       + qa.numel() * 2 + oa.numel() * 2 + la.numel() * 4 + lens.numel() * 4)

            def astep():
                fa.fa_fwd_kvcache_append(qa, kc, vc, lens_a, kn, vn, causal=True, o=oa, lse=la, num_splits=Sa,
                                         scale=scale_d, workspace=wsa)
            settle(astep, 0.1, min_calls=3)
            a_ms = timed(astep, args.append_steps)
            a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
            append[f"q{nq}"] = {"value": round(a_gbs, 1), "unit": "GB/s", "queries_per_seq": nq, "num_splits": Sa,
                                "mean_launch_ms": round(a_ms, 5), "frac": round(a_gbs / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes_per_launch": a_bytes, "steps": args.append_steps}

    dec_traffic = stored_traffic("decode:" + args.decode, DECODE_KERNEL_SOURCE)
    head = configs[args.prefill]
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": round(settle_s, 3),
        "settle_steps": settle_steps,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.prefill,
            "batch": wp["B"], "q_heads": wp["Hq"], "kv_heads": wp["Hkv"], "seq_len": wp["Nq"],
            "head_dim": wp["d"], "causal": wp["causal"],
            "decode_workload": args.decode, "decode_num_splits": S,
        },
        "roofline": {k2: head[k2] for k2 in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic",
                                             "algorithmic_flops_per_launch", "mean_launch_ms")},
        "configs": configs,
        "decode": {
            "workload": args.decode,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": dec_traffic,
                         "algorithmic_bytes_per_launch": dec_bytes, "mean_launch_ms": round(dc_mean, 5)},
            "num_splits": S,
            "paged": paged,
            "append": append,
        },
        "backward": bwd,
        "fp8": fp8,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
    }
    if not args.no_cpu_baseline:
        # the oracle, timed on a sample; the timed launches' outputs are
        # compared with it on the same rows (the "parity" entries)
        out["cpu_baseline"], configs[args.prefill]["parity"] = cpu_baseline(
            args.prefill, wp, args.cpu_budget, tensors=(q.cpu(), k.cpu(), v.cpu()), outputs=(o.cpu(), lse.cpu()))
        for name, (tens, outs) in cpu_tensors.items():
            configs[name]["cpu_baseline"], configs[name]["parity"] = cpu_baseline(
                name, SI.PREFILL_WORKLOADS[name], args.cpu_budget_other, tensors=tens, outputs=outs)
        out["decode"]["cpu_baseline"], out["decode"]["parity"] = cpu_baseline_decode(
            args.decode, wd, qd, kc, vc, lens, args.cpu_budget_other, outputs=(od.cpu(), lsed.cpu()))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

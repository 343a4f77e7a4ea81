"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
fa_fwd on the training-shape causal workload (B=8, H=16, N=2048, d=128,
bf16) followed by fa_fwd_kvcache (split-KV decode + combine) on the GQA
decode workload (B=64, Hq=32, Hkv=8, d=128, cache capacity 8192, lengths
uniform in [1024, 8192]). Inputs are generated on the device before the
timed region. Each launch is bracketed by HIP events on the stream it runs
on; `value` is the prefill's algorithmic TFLOP/s (4*B*H*Nq*Nk*d, halved for
causal) over its mean event time, and the decode's algorithmic GB/s is
reported beside it. After the step loop, and outside its clock, the
backward, the FP8 forward (with its quantisation timed apart), the
paged-cache decode and decode steps that append 1 or 4 new tokens per
sequence are timed on the same workloads. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prefill NAME]
                    [--no-cpu-baseline] [--splits S] [--bwd-steps N]
                    [--fp8-steps N] [--paged-steps N] [--append-steps N]
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
DEFAULT_PREFILL = "mha_bf16_causal_b8_h16_n2048_d128"
DEFAULT_DECODE = "gqa_bf16_decode_b64_h32kv8_cap8192_d128"
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


def cpu_baseline(name, w, budget_s=12.0):
    """The CPU float64 oracle, as is, on whole (batch, head) slices of the
    same prefill workload until about `budget_s` seconds have passed."""
    import numpy as np
    import torch

    import seeded_inputs as SI
    from oracle import sdpa as O

    q, k, v = SI.prefill_inputs(device="cpu", **w)
    f64 = lambda t: t.to(torch.float64).numpy()
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    G = w["Hq"] // w["Hkv"]
    done = 0
    t0 = time.perf_counter()
    for b in range(w["B"]):
        for h in range(w["Hq"]):
            kv = h // G
            O.attention_rows(f64(q[b:b + 1, :, h:h + 1]), f64(k[b:b + 1, :, kv:kv + 1]),
                             f64(v[b:b + 1, :, kv:kv + 1]), w["causal"], scale, 0, 0)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    per_head = prefill_flops(dict(w, B=1, Hq=1))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        cores = max([p.get("num_threads", 1) for p in pools] or [1])
        if pools:
            blas = f"{pools[0].get('internal_api', '?')} {pools[0].get('version', '')}".strip()
    except Exception:
        cores = os.cpu_count()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": per_head * done / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w['B'] * w['Hq']} (batch, head) slices of {name}, "
                      f"full fp64 score matrix each, {el:.1f} s",
            "cpu": cpu, "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks take on the order of a second of sustained work to
    # settle; the default warmup (~1 s of steps) lets them before timing.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--prefill", default=DEFAULT_PREFILL)
    ap.add_argument("--decode", default=DEFAULT_DECODE)
    ap.add_argument("--splits", type=int, default=0, help="decode num_splits (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--bwd-steps", type=int, default=50,
                    help="timed fa_bwd calls on the prefill workload after the step loop (0 = skip)")
    ap.add_argument("--fp8-steps", type=int, default=50,
                    help="timed FP8 forward calls (fa_fwd_fp8 on the prefill workload, quantised with the "
                         "rotation) after the step loop (0 = skip)")
    ap.add_argument("--append-steps", type=int, default=50,
                    help="timed decode-with-append calls (1 and 4 new tokens per sequence) after the step loop "
                         "(0 = skip)")
    ap.add_argument("--paged-steps", type=int, default=50,
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

    wp = SI.PREFILL_WORKLOADS[args.prefill]
    wd = SI.DECODE_WORKLOADS[args.decode]
    q, k, v = SI.prefill_inputs(device=dev, **wp)
    scale_p = 1.0 / math.sqrt(wp["d"])
    o = torch.empty_like(q)
    lse = torch.empty((wp["B"], wp["Hq"], wp["Nq"]), dtype=torch.float32, device=dev)

    qd, kc, vc, lens = SI.decode_inputs(device=dev, **wd)
    S = args.splits or fa.fa_kvcache_default_splits(wd["B"], wd["Hkv"], wd["capacity"])
    od = torch.empty_like(qd)
    lsed = torch.empty((wd["B"], wd["Hq"]), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_fwd_kvcache_workspace_size(wd["B"], wd["Hq"], wd["d"], S)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    scale_d = 1.0 / math.sqrt(wd["d"])
    lens_sum = int(lens.to(torch.int64).sum().item())
    dec_bytes = (lens_sum * wd["Hkv"] * wd["d"] * 2 * 2            # K and V rows actually visible
                 + qd.numel() * 2 + od.numel() * 2 + lsed.numel() * 4 + lens.numel() * 4)

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
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

    # The backward of the same prefill workload (fa_bwd: dQ, dK, dV from the
    # forward's O and LSE), timed after the step loop. Algorithmic work: the
    # five N x N x d products of the gradient formulas, 2.5x the forward's.
    bwd = None
    if args.bwd_steps > 0 and wp["dtype"] == "bf16" and wp["d"] in (64, 128):
        g = torch.Generator(device=dev)
        g.manual_seed(wp["seed"] + 1000)
        dout = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(max(fa.fa_bwd_workspace_size(wp["B"], wp["Hq"], wp["Nq"]), 1), dtype=torch.uint8,
                          device=dev)
        fa.fa_fwd(q, k, v, o=o, lse=lse, causal=wp["causal"], scale=scale_p)

        def bstep():
            fa.fa_bwd(q, k, v, o, lse, dout, causal=wp["causal"], scale=scale_p, dq=dq, dk=dk, dv=dv,
                      workspace=bws)
        for _ in range(max(3, args.bwd_steps // 5)):
            bstep()
        torch.cuda.synchronize()
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.bwd_steps)]
        for e0, e1 in bev:
            e0.record()
            bstep()
            e1.record()
        torch.cuda.synchronize()
        b_ms = sum(e0.elapsed_time(e1) for e0, e1 in bev) / len(bev)
        b_tf = 2.5 * prefill_flops(wp) / (b_ms * 1e-3) / 1e12
        bwd = {"value": round(b_tf, 2), "unit": "TFLOP/s", "mean_launch_ms": round(b_ms, 5),
               "frac": round(b_tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops_per_launch": 2.5 * prefill_flops(wp),
               "kernels": "bwd_prep_kernel + bwd_dq_kernel + bwd_dkdv_kernel", "steps": args.bwd_steps}

    # The decode workload again over a paged cache (256-row pages in a
    # shuffled pool, the same keys), timed after the step loop.
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
        for _ in range(max(3, args.paged_steps // 5)):
            pstep()
        torch.cuda.synchronize()
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.paged_steps)]
        for e0, e1 in pev:
            e0.record()
            pstep()
            e1.record()
        torch.cuda.synchronize()
        p_ms = sum(e0.elapsed_time(e1) for e0, e1 in pev) / len(pev)
        paged = {"value": round(dec_bytes / (p_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "page_size": P,
                 "mean_launch_ms": round(p_ms, 5), "frac": round(dec_bytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "steps": args.paged_steps}
        del kp, vp

    # Decode steps that append 1 or 4 new tokens per sequence to the same
    # cache (the write happens inside the split kernel), queries bottom-right
    # causal; lengths are capped so the new rows fit. Bytes: the visible
    # cache rows read, the new rows read and written, q, o, lse, lengths.
    # The prefill workload in FP8: Q and K rotated and block-quantised, V
    # block-quantised (outside the attention's clock, timed on its own),
    # then fa_fwd_fp8; its TFLOP/s is priced against the dense FP8 peak.
    fp8 = None
    if args.fp8_steps > 0 and wp["dtype"] == "bf16" and wp["d"] in (64, 128, 256) and wp["Nk"] <= 65536:
        signs = SI.random_signs(wp["d"], seed=wp["seed"] + 4000).to(dev)
        q8, qs8 = fa.fa_quantize_fp8(q, signs=signs)
        k8, ks8 = fa.fa_quantize_fp8(k, signs=signs)
        vt8, vs8 = fa.fa_quantize_fp8(v, transpose=True)
        o8 = torch.empty_like(q)
        l8 = torch.empty_like(lse)

        def fstep():
            fa.fa_fwd_fp8(q8, qs8, k8, ks8, vt8, vs8, wp["Nq"], wp["Nk"], causal=wp["causal"], scale=scale_p,
                          o=o8, lse=l8)

        def qstep():
            fa.fa_quantize_fp8(q, signs=signs, codes=q8, scales=qs8)
            fa.fa_quantize_fp8(k, signs=signs, codes=k8, scales=ks8)
            fa.fa_quantize_fp8(v, transpose=True, codes=vt8, scales=vs8)
        for _ in range(max(3, args.fp8_steps // 5)):
            fstep()
        torch.cuda.synchronize()
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.fp8_steps)]
        for e0, e1 in fev:
            e0.record()
            fstep()
            e1.record()
        torch.cuda.synchronize()
        f_ms = sum(e0.elapsed_time(e1) for e0, e1 in fev) / len(fev)
        qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for e0, e1 in qev:
            e0.record()
            qstep()
            e1.record()
        torch.cuda.synchronize()
        q_ms = sum(e0.elapsed_time(e1) for e0, e1 in qev) / len(qev)
        f_tf = prefill_flops(wp) / (f_ms * 1e-3) / 1e12
        fp8 = {"value": round(f_tf, 2), "unit": "TFLOP/s", "kernel": f"fwd_fp8_kernel<{wp['d']}>", "dtype": "e4m3",
               "peak": PEAK_FP8_TFLOPS, "frac": round(f_tf / PEAK_FP8_TFLOPS, 4), "mean_launch_ms": round(f_ms, 5),
               "quantize_ms": round(q_ms, 5), "steps": args.fp8_steps}
        del q8, k8, vt8, o8

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
            wsa = torch.empty(max(fa.fa_fwd_kvcache_workspace_size(wd["B"] * nq, wd["Hq"], wd["d"], S), 1),
                              dtype=torch.uint8, device=dev)
            rows = int(lens_a.to(torch.int64).sum().item()) + wd["B"] * nq
            a_bytes = (rows * wd["Hkv"] * wd["d"] * 2 * 2 + 2 * kn.numel() * 2 * 2
                       + qa.numel() * 2 + oa.numel() * 2 + la.numel() * 4 + lens.numel() * 4)

            def astep():
                fa.fa_fwd_kvcache_append(qa, kc, vc, lens_a, kn, vn, causal=True, o=oa, lse=la, num_splits=S,
                                         scale=scale_d, workspace=wsa)
            for _ in range(max(3, args.append_steps // 5)):
                astep()
            torch.cuda.synchronize()
            aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.append_steps)]
            for e0, e1 in aev:
                e0.record()
                astep()
                e1.record()
            torch.cuda.synchronize()
            a_ms = sum(e0.elapsed_time(e1) for e0, e1 in aev) / len(aev)
            a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
            append[f"q{nq}"] = {"value": round(a_gbs, 1), "unit": "GB/s", "queries_per_seq": nq,
                                "mean_launch_ms": round(a_ms, 5), "frac": round(a_gbs / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes_per_launch": a_bytes, "steps": args.append_steps}

    traffic = stored_traffic("prefill:" + args.prefill, PREFILL_KERNEL_SOURCE)
    dec_traffic = stored_traffic("decode:" + args.decode, DECODE_KERNEL_SOURCE)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        "roofline": {
            "kernel": f"fwd_bf16_kernel<{wp['d']}>",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "mean_launch_ms": round(pf_mean, 5),
        },
        "decode": {
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
        out["cpu_baseline"] = cpu_baseline(args.prefill, wp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

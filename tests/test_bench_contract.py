"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal,
the algorithmic FLOP accounting of the metric, and that stored HBM traffic
is reported only for the kernel source it was measured on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_prefill_flops_accounting():
    # 4 B H Nq Nk d, halved for causal, as the metric states
    w = dict(B=8, Hq=16, Nq=2048, Nk=2048, d=128, causal=True)
    assert bench.prefill_flops(w) == 4 * 8 * 16 * 2048 * 2048 * 128 / 2
    assert bench.prefill_flops(dict(w, causal=False)) == 4 * 8 * 16 * 2048 * 2048 * 128
    # the headline workload: 137.44 GFLOP per launch
    assert abs(bench.prefill_flops(w) / 1e9 - 137.44) < 0.01


def test_stored_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"k": {"source_sha256_16": bench.source_hash([str(src)]), "bytes_per_launch": 123}}
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("k", [str(src)]) == 123
    assert bench.stored_traffic("missing", [str(src)]) is None
    src.write_text("kernel v2")  # the kernel changed since the counters were taken
    assert bench.stored_traffic("k", [str(src)]) is None


def test_committed_traffic_records_are_well_formed():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        recs = json.load(f)
    for key, rec in recs.items():
        if key.startswith("_"):
            continue
        for field in ("kernel", "source_sha256_16", "fetch_kib", "write_kib", "fetch_factor", "write_factor",
                      "bytes_per_launch"):
            assert field in rec, (key, field)
        expect = (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]) * 1024
        assert abs(rec["bytes_per_launch"] - expect) <= 1e-3 * expect + 1024, key


def test_cpu_baseline_fields_on_a_tiny_workload():
    w = dict(B=1, Hq=2, Hkv=1, Nq=64, Nk=64, d=64, causal=True, dtype="bf16", seed=1)
    r, parity = bench.cpu_baseline("tiny", w, budget_s=0.5)
    assert parity is None
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "of tiny" in r["sample"]
    assert isinstance(r["cpu"], str) and isinstance(r["blas"], str)


def test_cpu_baseline_compares_the_given_outputs():
    # the parity entry: the oracle's rows against the outputs handed in (here
    # the oracle's own result rounded to bf16, then one element moved)
    import math

    import numpy as np
    import torch

    import seeded_inputs as SI
    from oracle import sdpa as O
    w = dict(B=1, Hq=2, Hkv=1, Nq=64, Nk=64, d=64, causal=True, dtype="bf16", seed=1)
    q, k, v = SI.prefill_inputs(device="cpu", **w)
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    o_ref, l_ref = O.attention(*(t.double().numpy() for t in (q, k, v)), True, scale)
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(l_ref).float()
    _, par = bench.cpu_baseline("tiny", w, budget_s=5.0, tensors=(q, k, v), outputs=(o, lse))
    assert par["rows"] == 128 and par["within"] and par["max_abs_o"] <= 1e-2 and par["max_abs_lse"] <= 1e-6
    o2 = o.clone()
    o2[0, 63, 1, 5] += 0.5
    _, par2 = bench.cpu_baseline("tiny", w, budget_s=5.0, tensors=(q, k, v), outputs=(o2, lse))
    assert not par2["within"] and par2["max_abs_o"] >= 0.4

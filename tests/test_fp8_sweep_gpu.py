"""GPU parity of the FP8 forward on a seeded sweep of random shapes.

Random batch, GQA group, head dimension, query and key counts (around the
64-row quantisation block and the 32/64-key tiles, Nq != Nk included) and
mask, on e4m3 codes drawn at the workloads' scale; each case is compared
with the FP8 oracle under the same rule as the hand-picked FP8 cases: O
within 2e-2 and LSE within 1e-3, a row over the O bar only where the oracle
shows probabilities within float32 rounding of an e4m3 midpoint.
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from test_fp8_gpu import assert_fp8_matches

pytestmark = pytest.mark.gpu

EDGE = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257]


def _cases(n=14, seed=2031):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4]))
        nq = int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 400))
        nk = int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 400))
        out.append((int(rng.choice([1, 2])), hkv * g, hkv, nq, nk, bool(rng.random() < 0.5), d, 1400 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=["B{}H{}kv{}q{}k{}c{}d{}s{}".format(*c) for c in CASES])
def test_fp8_sweep(case):
    import exact_io_aware_online_amd as fa
    B, Hq, Hkv, Nq, Nk, causal, d, seed = case
    print(f"fp8 sweep B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} d={d} seed={seed}", flush=True)
    dev = torch.device("cuda")
    ins = SI.fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fa_fwd_fp8(*(t.to(dev) for t in ins), Nq, Nk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    excused = assert_fp8_matches(o, lse, ins, Nq, Nk, causal, scale)
    assert excused <= max(2, Nq * B * Hq // 1000)

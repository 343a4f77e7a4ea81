"""Host-side check (no GPU) of the balanced decode's work partition, restated
from the kernel's arithmetic: the tiles of every (sequence, key/value head)
pair laid end to end, cut into U = (S - 1) B Hkv runs
[floor(u A / U), floor((u+1) A / U)); a run writes one partial per pair it
touches at slot u + Hkv NZ(b) + h; the combine reads, for a pair, the slots
of the units from the owner of its first tile to the owner of its last,
skipping units whose run is empty. For random lengths (empty sequences,
one-tile caches, more units than tiles) every tile belongs to exactly one
run, no two partials share a slot, every slot fits the workspace
(S B Hq (d + 1) floats), and the combine reads exactly the partials written
for its pair."""

import random

import pytest


def plan(lens, Hkv, S, cap, T):
    B = len(lens)
    n = [(min(max(x, 0), cap) + T - 1) // T for x in lens]
    A = Hkv * sum(n)
    U = (S - 1) * B * Hkv
    start = lambda u: (A // U) * u + ((A % U) * u) // U
    # flat tile -> (b, h, i)
    flat = []
    for b in range(B):
        for h in range(Hkv):
            for i in range(n[b]):
                flat.append((b, h, i))
    assert len(flat) == A
    nz_before = [sum(1 for x in n[:b] if x > 0) for b in range(B)]
    written = {}
    covered = [0] * A
    for u in range(U):
        t0, t1 = start(u), start(u + 1)
        pairs = []
        for t in range(t0, t1):
            covered[t] += 1
            b, h, _ = flat[t]
            if not pairs or pairs[-1] != (b, h):
                pairs.append((b, h))
        for b, h in pairs:
            slot = u + Hkv * nz_before[b] + h
            assert slot not in written, "two partials share a slot"
            assert 0 <= slot < S * B * Hkv, "slot beyond the workspace"
            written[slot] = (u, b, h)
    assert all(c == 1 for c in covered)
    # the combine's view of every pair
    unit_of = lambda t: ((t + 1) * U - 1) // A
    pre = 0
    read = set()
    for b in range(B):
        for h in range(Hkv):
            if n[b] == 0:
                continue
            s0 = Hkv * pre + h * n[b]
            u0, u1 = unit_of(s0), unit_of(s0 + n[b] - 1)
            slot0 = u0 + Hkv * nz_before[b] + h
            for s in range(u1 - u0 + 1):
                u = u0 + s
                if A >= U or start(u) < start(u + 1):
                    assert written.get(slot0 + s) == (u, b, h), "combine reads a partial of another pair"
                    read.add(slot0 + s)
        pre += n[b]
    assert read == set(written), "a written partial is never read"


@pytest.mark.parametrize("seed", range(40))
def test_balanced_decode_partition(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 3, 5, 17, 64, 70])
    Hkv = rng.choice([1, 2, 8])
    T = rng.choice([32, 64])
    cap = rng.choice([64, 100, 300, 1024, 4000])
    S = rng.choice([2, 3, 5, 9, 40])
    lens = [rng.choice([0, 1, rng.randrange(0, cap + 1), cap, cap + 5]) for _ in range(B)]
    if sum(lens) == 0:
        lens[0] = 1
    plan(lens, Hkv, S, cap, T)


def test_balanced_decode_partition_more_units_than_tiles():
    plan([1, 0, 3, 0, 2], Hkv=2, S=40, cap=64, T=64)
    plan([65], Hkv=1, S=9, cap=128, T=64)

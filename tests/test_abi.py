"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the device (CPU only: no call here
reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import exact_io_aware_online_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# a non-null address that is never dereferenced: every call below fails
# validation before any pointer is used
FAKE = ctypes.c_void_p(0x1000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_size", "fa_kvcache_default_splits",
            "fa_status_string", "fa_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libfa.so does not export {n}"


def test_status_strings_and_version():
    assert fa.fa_abi_version() == 2
    for s in range(5):
        assert fa.fa_status_string(s).startswith("FA_")
    assert fa.fa_status_string(99) == "FA_ERR_UNKNOWN"


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=128,
             causal=0, scale=0.1, dtype=fa.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                           a["Nk"], a["d"], a["causal"], ctypes.c_float(a["scale"]), a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-3), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=fa.FA_DTYPE_F32, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(B=2, Nq=2**30 + 64), fa.FA_ERR_UNSUPPORTED),   # 2^31 + 128 query rows
    (dict(B=2, Nk=2**30 + 64), fa.FA_ERR_UNSUPPORTED),   # 2^31 + 128 key rows
    (dict(B=0), fa.FA_OK),          # no-op, nothing launched
    (dict(Nq=0), fa.FA_OK),         # no-op, nothing launched
])
def test_fwd_host_validation(kw, status):
    assert _fwd(**kw) == status


def _kv(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, o=FAKE, lse=None, S=4, B=2, Hq=8, Hkv=2, cap=256, d=128,
             scale=0.1, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd_kvcache(a["q"], a["kc"], a["vc"], a["lens"], a["o"], a["lse"], a["S"], a["B"], a["Hq"],
                                   a["Hkv"], a["cap"], a["d"], ctypes.c_float(a["scale"]), a["ws"], a["ws_bytes"],
                                   a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(S=0), fa.FA_ERR_INVALID_ARG),
    (dict(cap=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(lens=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(kc=None), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=64, Hkv=2), fa.FA_ERR_UNSUPPORTED),   # 32 query heads per KV head
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(B=0), fa.FA_OK),
])
def test_kvcache_host_validation(kw, status):
    assert _kv(**kw) == status


def test_workspace_size_formula():
    assert fa.fa_fwd_kvcache_workspace_size(64, 32, 128, 1) == 0
    assert fa.fa_fwd_kvcache_workspace_size(64, 32, 128, 8) == 64 * 32 * 8 * 129 * 4
    assert fa.fa_fwd_kvcache_workspace_size(0, 32, 128, 8) == 0
    # the exact boundary: one byte short is rejected before launch
    need = fa.fa_fwd_kvcache_workspace_size(2, 8, 128, 4)
    assert _kv(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE


def test_default_splits():
    # single-query decode: the fewest runs per pair whose waves of resident
    # workgroups leave at most 1/8 of the slot-time idle (else the least
    # idle), runs of at least ~8 tiles, no split with plenty of pairs
    assert fa.fa_kvcache_default_splits(64, 8, 8192, 128, 256, 2) == 2      # 512 pairs, 512 slots: one wave
    assert fa.fa_kvcache_default_splits(64, 8, 8192, 128, 256, 4) == 3      # 1024 slots: 2 runs per pair
    assert fa.fa_kvcache_default_splits(64, 8, 8192, 128, 256, 3) == 4      # 768 slots: 1536 runs, 2 full waves
    assert fa.fa_kvcache_default_splits(48, 8, 8192, 128, 256, 2) == 5      # 384 pairs: 1536 runs, 3 full waves
    assert fa.fa_kvcache_default_splits(48, 8, 8192, 128, 256, 4) == 6      # 1920 runs on 1024 slots, 1/16 idle
    assert fa.fa_kvcache_default_splits(75, 8, 8192, 128, 256, 4) == 4      # 600 pairs: 1800 runs, 2 waves
    assert fa.fa_kvcache_default_splits(6, 8, 8192, 128, 256, 2) == 11      # 48 pairs: 480 runs, not 528
    assert fa.fa_kvcache_default_splits(128, 8, 8192, 128, 256, 2) == 2     # 1024 pairs, 2 full waves
    assert fa.fa_kvcache_default_splits(136, 8, 8192, 128, 256, 4) == 6     # 1088 pairs: 5440 runs, 6 waves
    assert fa.fa_kvcache_default_splits(160, 8, 8192, 128, 256, 4) == 4     # 1280 pairs: 3840 runs, 4 waves
    assert fa.fa_kvcache_default_splits(240, 8, 4096, 128, 256, 4) == 2     # 1920 pairs: 2 waves, 1/16 idle
    assert fa.fa_kvcache_default_splits(136, 8, 2048, 128, 256, 4) == 5     # runs of 8 tiles: at most 4 a pair
    assert fa.fa_kvcache_default_splits(1, 8, 8192, 128, 256, 3) == 17      # capped by run length: 128 / 8 + 1
    assert fa.fa_kvcache_default_splits(2, 1, 1000000, 128, 256, 3) == 337  # 672 of 768 slots: 1/8 idle
    assert fa.fa_kvcache_default_splits(1, 1, 64, 128, 256, 3) == 1         # one tile: nothing to balance
    assert fa.fa_kvcache_default_splits(4096, 8, 8192, 128, 256, 3) == 1    # 4+ pairs per slot
    assert fa.fa_kvcache_default_splits(0, 8, 8192, 128, 256, 3) == 1


def test_append_default_splits():
    # at most 16 (query, query head) columns per key/value head and at least
    # 64 (sequence, key/value head) pairs: the balanced decode, whose rule is
    # fa_kvcache_default_splits
    for B, Nq, Hkv, Hq, cap, d in [(64, 1, 8, 32, 8192, 128), (64, 4, 8, 32, 8192, 128), (8, 1, 8, 32, 8192, 64),
                                   (4096, 2, 8, 32, 8192, 128), (32, 2, 2, 16, 4096, 256), (64, 16, 1, 1, 64, 128)]:
        assert (fa.fa_kvcache_append_default_splits(B, Nq, Hkv, Hq, cap, d, 256, 3)
                == fa.fa_kvcache_default_splits(B, Hkv, cap, d, 256, 3)), (B, Nq, Hkv, Hq, cap, d)
    assert fa.fa_kvcache_append_default_splits(64, 4, 8, 32, 8192, 128, 256, 4) == 3    # 512 pairs, 1024 slots
    assert fa.fa_kvcache_append_default_splits(0, 1, 8, 32, 8192, 128, 256, 3) == 1
    # more columns, or fewer pairs: splits of the keys by position
    assert fa.fa_kvcache_append_default_splits(64, 8, 8, 32, 8192, 128, 256, 3) == 3    # 1024 items: 4 waves at most
    assert fa.fa_kvcache_append_default_splits(16, 8, 8, 32, 8192, 128, 256, 3) == 8    # ~1024-key splits
    assert fa.fa_kvcache_append_default_splits(1, 8, 8, 32, 8192, 128, 256, 3) == 48    # fill 768 slots, 2 groups
    assert fa.fa_kvcache_append_default_splits(1, 1, 8, 32, 8192, 128, 256, 3) == 96    # 8 pairs: fill 768 slots
    assert fa.fa_kvcache_append_default_splits(1, 1, 1, 1, 64, 128, 256, 3) == 1        # one block: cannot split
    assert fa.fa_kvcache_append_default_splits(1, 5, 1, 4, 64, 128, 256, 3) == 1
    assert fa.fa_kvcache_append_default_splits(4096, 8, 8, 32, 8192, 128, 256, 3) == 1  # capped by the slot budget


def test_paged_decode_host_validation():
    L = fa.lib()
    null = None
    # page size not a multiple of 64, missing block table: rejected before any HIP call
    assert L.fa_fwd_kvcache_paged(null, null, null, null, null, null, null, 1, 2, 4, 2, 96, 4, 8, 128, 0.1,
                                  null, 0, null) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_kvcache_paged(null, null, null, null, null, null, null, 1, 2, 4, 2, 128, 4, 8, 128, 0.1,
                                  null, 0, null) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_kvcache_paged(null, null, null, null, null, null, null, 1, 2, 4, 2, 0, 4, 8, 128, 0.1,
                                  null, 0, null) == fa.FA_ERR_INVALID_ARG
    # B = 0 is a no-op even without buffers
    assert L.fa_fwd_kvcache_paged(null, null, null, null, null, null, null, 1, 0, 4, 2, 128, 4, 8, 128, 0.1,
                                  null, 0, null) == fa.FA_OK


def test_backward_host_validation():
    L = fa.lib()
    null = None
    args = lambda **kw: dict(dict(B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, causal=0, scale=0.1), **kw)
    def call(**kw):
        a = args(**kw)
        return L.fa_bwd(null, null, null, null, null, null, null, null, null, a["B"], a["Hq"], a["Hkv"], a["Nq"],
                        a["Nk"], a["d"], a["causal"], a["scale"], null, 0, null)
    assert call(Hq=3) == fa.FA_ERR_INVALID_ARG       # Hq % Hkv
    assert call(d=256) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == fa.FA_ERR_INVALID_ARG
    assert call(causal=2) == fa.FA_ERR_INVALID_ARG
    assert call() == fa.FA_ERR_INVALID_ARG           # null tensors
    assert call(B=2, Nk=2**30 + 64) == fa.FA_ERR_UNSUPPORTED  # 2^31 + 128 key rows
    assert call(B=0) == fa.FA_OK
    assert fa.fa_bwd_workspace_size(2, 3, 33) == 2 * 2 * 3 * 64 * 4
    assert fa.fa_bwd_workspace_size(2, 3, 0) == 0


def test_append_host_validation():
    import ctypes
    L = fa.lib()
    null = None
    fake = ctypes.c_void_p(64)  # never dereferenced: every case fails or ends before a launch
    def call(q=fake, kn=null, vn=null, o=fake, lens=fake, causal=1, S=1, B=2, Nq=3, Hq=8, Hkv=2, cap=256, d=128,
             ws=null, ws_bytes=0):
        return L.fa_fwd_kvcache_append(q, kn, vn, fake, fake, lens, o, null, causal, S, B, Nq, Hq, Hkv, cap, d, 0.1,
                                       ws, ws_bytes, null)
    assert call(Nq=0) == fa.FA_ERR_INVALID_ARG
    assert call(kn=fake) == fa.FA_ERR_INVALID_ARG          # k_new without v_new
    assert call(vn=fake) == fa.FA_ERR_INVALID_ARG
    assert call(Hq=6, Hkv=4) == fa.FA_ERR_INVALID_ARG      # Hq % Hkv
    assert call(Hq=64, Hkv=2) == fa.FA_ERR_UNSUPPORTED     # more than 16 query heads per key/value head
    assert call(B=40000, Nq=40000) == fa.FA_ERR_UNSUPPORTED
    assert call(q=null) == fa.FA_ERR_INVALID_ARG
    assert call(S=2) == fa.FA_ERR_WORKSPACE                 # splits need the (B * Nq)-row workspace
    need = fa.fa_fwd_kvcache_workspace_size(2 * 3, 8, 128, 2)
    assert need == 2 * 3 * 8 * 2 * 129 * 4
    assert call(S=2, ws=fake, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert call(B=0, q=null, o=null, lens=null) == fa.FA_OK
    # paged: page size not a multiple of 64, missing block table
    def paged(page=128, bt=fake):
        return L.fa_fwd_kvcache_paged_append(fake, null, null, fake, fake, bt, fake, fake, null, 1, 1, 2, 3, 8, 2,
                                             page, 4, 16, 128, 0.1, null, 0, null)
    assert paged(page=96) == fa.FA_ERR_INVALID_ARG
    assert paged(bt=null) == fa.FA_ERR_INVALID_ARG


def test_fp8_host_validation():
    import ctypes
    L = fa.lib()
    null = None
    fake = ctypes.c_void_p(64)  # never dereferenced: every case fails or ends before a launch
    assert fa.fa_fp8_padded_rows(1) == 64 and fa.fa_fp8_padded_rows(64) == 64 and fa.fa_fp8_padded_rows(65) == 128
    assert fa.fa_fp8_padded_rows(0) == 0
    def quant(x=fake, codes=fake, scales=fake, transpose=0, B=1, N=10, H=2, d=128):
        return L.fa_quantize_fp8(x, null, codes, scales, transpose, B, N, H, d, null)
    assert quant(d=96) == fa.FA_ERR_UNSUPPORTED
    assert quant(transpose=2) == fa.FA_ERR_INVALID_ARG
    assert quant(x=null) == fa.FA_ERR_INVALID_ARG
    assert quant(scales=null) == fa.FA_ERR_INVALID_ARG
    assert quant(N=-1) == fa.FA_ERR_INVALID_ARG
    assert quant(N=0, x=null) == fa.FA_OK
    def fwd(q=fake, k=fake, o=fake, B=1, Hq=4, Hkv=2, Nq=100, Nk=100, d=128, causal=0, scale=0.1):
        return L.fa_fwd_fp8(q, fake, k, fake, fake, fake, o, null, B, Hq, Hkv, Nq, Nk, d, causal, scale, null)
    assert fwd(d=96) == fa.FA_ERR_UNSUPPORTED
    assert fwd(Hq=3) == fa.FA_ERR_INVALID_ARG
    assert fwd(causal=2) == fa.FA_ERR_INVALID_ARG
    assert fwd(scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fwd(Nk=65537) == fa.FA_ERR_UNSUPPORTED
    assert fwd(q=null) == fa.FA_ERR_INVALID_ARG
    assert fwd(k=null) == fa.FA_ERR_INVALID_ARG
    assert fwd(k=null, Nk=0, q=null, Nq=0) == fa.FA_OK


def test_backward_window_varlen_host_validation():
    import ctypes
    L = fa.lib()
    null = None
    fake = ctypes.c_void_p(64)  # never dereferenced: every case fails or ends before a launch
    def win(d=128, Hq=4, B=1, q=fake, ws=null, ws_bytes=0):
        return L.fa_bwd_window(q, fake, fake, fake, fake, fake, fake, fake, fake, B, Hq, 2, 64, 80, d, 10, 0, 0.1, ws,
                               ws_bytes, null)
    assert win(d=256) == fa.FA_ERR_UNSUPPORTED
    assert win(Hq=3) == fa.FA_ERR_INVALID_ARG
    assert win(q=null) == fa.FA_ERR_INVALID_ARG
    assert win() == fa.FA_ERR_WORKSPACE
    assert win(B=0) == fa.FA_OK
    def var(cu=fake, total_q=100, B=2):
        return L.fa_bwd_varlen(fake, fake, fake, fake, fake, fake, fake, fake, fake, cu, cu, B, 4, 2, 64, 64, total_q,
                               90, 128, -1, 0, 0.1, null, 0, null)
    assert var(cu=null) == fa.FA_ERR_INVALID_ARG
    assert var() == fa.FA_ERR_WORKSPACE
    assert var(B=0, cu=null) == fa.FA_OK


def test_noalloc_decode_host_validation():
    L = fa.lib()
    null = None
    f = ctypes.c_float(0.1)
    # the Python constant is the header's
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20
    # beyond the static scratch: rejected before anything else
    assert L.fa_fwd_kvcache_noalloc(null, null, null, null, null, null, 8, 4096, 32, 8, 8192, 128, f,
                                    null) == fa.FA_ERR_WORKSPACE
    # within it, but bad arguments: rejected on the host, no device lookup
    assert L.fa_fwd_kvcache_noalloc(null, null, null, null, null, null, 4, 8, 8, 2, 256, 128, f,
                                    null) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, null, 0, 8, 8, 2, 256, 128, f,
                                    null) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, null, 4, 8, 6, 4, 256, 128, f,
                                    null) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, null, 4, 8, 8, 2, 256, 96, f,
                                    null) == fa.FA_ERR_UNSUPPORTED
    # B = 0 is a no-op
    assert L.fa_fwd_kvcache_noalloc(null, null, null, null, null, null, 4, 0, 8, 2, 256, 128, f,
                                    null) == fa.FA_OK

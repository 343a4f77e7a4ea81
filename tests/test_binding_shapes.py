"""Host-side checks of the Python binding (no GPU): every tensor a kernel
writes through a raw pointer must have the shape the call implies, and a
wrong one raises ValueError before anything reaches the library.

The device test of ``_check`` is relaxed here (CPU tensors stand in for
device tensors) and the library is replaced by a stand-in whose only
working functions are the pure size queries; any other call fails the
test, so a passing case proves the error came first.
"""

import pytest
import torch

import exact_io_aware_online_amd as fa


class _NoLaunch:
    def fa_fwd_kvcache_workspace_size(self, B, Hq, d, S):
        return 0 if S <= 1 else B * Hq * S * (d + 1) * 4

    def fa_bwd_workspace_size(self, B, Hq, Nq):
        return 0

    def fa_fp8_padded_rows(self, n):
        return (n + 63) // 64 * 64

    def fa_kvcache_default_splits(self, *a):
        return 1

    def __getattr__(self, name):
        raise AssertionError(f"{name} was called: a launch was attempted before the shape check")


@pytest.fixture(autouse=True)
def no_device(monkeypatch):
    def check(t, name, dtype=None, device=None):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    monkeypatch.setattr(fa, "_check", check)
    monkeypatch.setattr(fa, "lib", lambda: _NoLaunch())


bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_fa_fwd_output_shapes():
    q, k = z(2, 10, 4, 64), z(2, 12, 2, 64)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, k.clone(), o=z(2, 10, 4, 32))
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, k.clone(), lse=z(2, 10, 4, dtype=f32))


def test_fa_fwd_window_output_shapes():
    q, k = z(2, 10, 4, 64), z(2, 12, 2, 64)
    with pytest.raises(ValueError):
        fa.fa_fwd_window(q, k, k.clone(), 3, 0, o=z(2, 9, 4, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_window(q, k, k.clone(), 3, 0, lse=z(2, 4, 9, dtype=f32))


def test_fa_fwd_varlen_output_shapes():
    q, k = z(30, 4, 64), z(40, 2, 64)
    cu = torch.tensor([0, 10, 30], dtype=i32)
    cuk = torch.tensor([0, 15, 40], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(q, k, k.clone(), cu, cuk, 20, o=z(29, 4, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(q, k, k.clone(), cu, cuk, 20, lse=z(30, 4, dtype=f32))
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(q, k, k.clone(), cu, cuk[:2].contiguous(), 20)


def test_fa_fwd_kvcache_output_shapes():
    q, kc = z(3, 1, 8, 128), z(3, 256, 2, 128)
    lens = torch.tensor([1, 2, 3], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache(q, kc, kc.clone(), lens, num_splits=1, o=z(3, 1, 8, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache(q, kc, kc.clone(), lens, num_splits=1, lse=z(3, 4, dtype=f32))


def test_fa_fwd_kvcache_paged_output_shapes():
    q, kp = z(3, 1, 8, 128), z(6, 64, 2, 128)
    bt = torch.zeros((3, 2), dtype=i32)
    lens = torch.tensor([1, 2, 3], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_paged(q, kp, kp.clone(), bt, lens, num_splits=1, o=z(2, 1, 8, 128))
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_paged(q, kp, kp.clone(), bt, lens, num_splits=1, lse=z(3, 8, 1, dtype=f32))


def test_fa_fwd_kvcache_append_output_shapes():
    q, kc = z(2, 3, 8, 64), z(2, 128, 2, 64)
    kn = z(2, 3, 2, 64)
    lens = torch.tensor([5, 6], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_append(q, kc, kc.clone(), lens, kn, kn.clone(), num_splits=1, o=z(2, 1, 8, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_append(q, kc, kc.clone(), lens, kn, kn.clone(), num_splits=1, lse=z(2, 8, dtype=f32))
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_append(q, kc, kc.clone(), lens, z(2, 3, 2, 32), kn.clone(), num_splits=1)


def test_fa_fwd_kvcache_paged_append_output_shapes():
    q, kp = z(2, 2, 8, 64), z(4, 64, 2, 64)
    bt = torch.zeros((2, 2), dtype=i32)
    lens = torch.tensor([5, 6], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_paged_append(q, kp, kp.clone(), bt, lens, num_splits=1, o=z(2, 1, 8, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache_paged_append(q, kp, kp.clone(), bt, lens, num_splits=1, lse=z(2, 8, 1, dtype=f32))


def test_fa_fwd_fp8_output_shapes():
    u8 = torch.uint8
    q8, k8, vt8 = z(1, 2, 128, 64, dtype=u8), z(1, 1, 64, 64, dtype=u8), z(1, 1, 64, 64, dtype=u8)
    qs, ks, vs = z(1, 2, 2, dtype=u8), z(1, 1, 1, dtype=u8), z(1, 1, 1, dtype=u8)
    with pytest.raises(ValueError):
        fa.fa_fwd_fp8(q8, qs, k8, ks, vt8, vs, 100, 60, o=z(1, 100, 2, 32))
    with pytest.raises(ValueError):
        fa.fa_fwd_fp8(q8, qs, k8, ks, vt8, vs, 100, 60, lse=z(1, 100, 2, dtype=f32))
    with pytest.raises(ValueError):
        fa.fa_fwd_fp8(q8, z(1, 2, 1, dtype=u8), k8, ks, vt8, vs, 100, 60)


def test_fa_bwd_gradient_shapes():
    q, k = z(1, 10, 4, 64), z(1, 12, 2, 64)
    lse = z(1, 4, 10, dtype=f32)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, k.clone(), q.clone(), lse, q.clone(), dk=z(1, 12, 4, 64))
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, k.clone(), q.clone(), z(1, 4, 9, dtype=f32), q.clone())


def test_fa_bwd_window_shapes():
    q, k = z(1, 10, 4, 64), z(1, 12, 2, 64)
    lse = z(1, 4, 10, dtype=f32)
    for kw in (dict(dq=z(1, 9, 4, 64)), dict(dk=z(1, 12, 4, 64)), dict(dv=z(1, 11, 2, 64))):
        with pytest.raises(ValueError):
            fa.fa_bwd_window(q, k, k.clone(), q.clone(), lse, q.clone(), 2, 0, **kw)
    with pytest.raises(ValueError):
        fa.fa_bwd_window(q, k, k.clone(), z(1, 9, 4, 64), lse, q.clone(), 2, 0)
    with pytest.raises(ValueError):
        fa.fa_bwd_window(q, k, k.clone(), q.clone(), z(1, 4, 11, dtype=f32), q.clone(), 2, 0)
    with pytest.raises(ValueError):
        fa.fa_bwd_window(q, k, z(1, 11, 2, 64), q.clone(), lse, q.clone(), 2, 0)


def test_fa_bwd_varlen_shapes():
    q, k = z(30, 4, 64), z(40, 2, 64)
    lse = z(4, 30, dtype=f32)
    cu = torch.tensor([0, 10, 30], dtype=i32)
    cuk = torch.tensor([0, 15, 40], dtype=i32)
    for kw in (dict(dq=z(29, 4, 64)), dict(dk=z(40, 4, 64)), dict(dv=z(39, 2, 64))):
        with pytest.raises(ValueError):
            fa.fa_bwd_varlen(q, k, k.clone(), q.clone(), lse, q.clone(), cu, cuk, 20, 25, **kw)
    with pytest.raises(ValueError):
        fa.fa_bwd_varlen(q, k, k.clone(), q.clone(), z(30, 4, dtype=f32), q.clone(), cu, cuk, 20, 25)
    with pytest.raises(ValueError):
        fa.fa_bwd_varlen(q, k, k.clone(), q.clone(), lse, q.clone(), cu, cuk[:2].contiguous(), 20, 25)

"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments on the host
before anything is enqueued (no HIP call is reached on these paths)."""

import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_strided_amd as X
from block_sparse_attention_strided_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    with open(os.path.join(ROOT, "include", "xattn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(xattn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def _shape(lq=(256,), lk=(512,), hq=4, hkv=2, d=128, dtype=torch.bfloat16, table=None, phys=0):
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(lq, lk):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    return X.Shape(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, cu_q=cu_q, cu_k=cu_k,
                   device="cpu", block_table=table, num_phys_blocks=phys)


def test_workspace_size_is_positive_and_grows():
    p = X.make_params()
    small = X.xattn_workspace_size(_shape(), p)
    big = X.xattn_workspace_size(_shape(lq=(1024,), lk=(8192,)), p)
    assert 0 < small < big


@pytest.mark.parametrize("kw,pk,code", [
    (dict(hq=3, hkv=2), {}, _lib.XATTN_ERR_INVALID),           # Hq % Hkv
    (dict(d=96), {}, _lib.XATTN_ERR_UNSUPPORTED),               # head_dim
    (dict(lq=(200,), lk=(512,)), {}, _lib.XATTN_ERR_UNSUPPORTED),  # not a multiple of 128
    (dict(lq=(512,), lk=(256,)), {}, _lib.XATTN_ERR_INVALID),  # Lk < Lq
    ({}, dict(block_size=64), _lib.XATTN_ERR_UNSUPPORTED),
    ({}, dict(stride=3), _lib.XATTN_ERR_UNSUPPORTED),
    ({}, dict(threshold=float("nan")), _lib.XATTN_ERR_INVALID),
    ({}, dict(kv_chunk_tokens=100), _lib.XATTN_ERR_INVALID),
    ({}, dict(select_mode=7), _lib.XATTN_ERR_INVALID),
    ({}, dict(num_to_choose=-1), _lib.XATTN_ERR_INVALID),
    ({}, dict(reuse_selection=2), _lib.XATTN_ERR_INVALID),
    (dict(lq=(128,), lk=(128 * 4097,)), {}, _lib.XATTN_ERR_UNSUPPORTED),  # too long
])
def test_invalid_arguments_are_rejected_before_any_work(kw, pk, code):
    s = _shape(**kw)
    p = X.make_params(**pk)
    lib = _lib.load()
    assert lib.xattn_workspace_size(ctypes.byref(s.c), ctypes.byref(p)) == 0
    fake = ctypes.c_void_p(0x1000)
    rc = lib.xattn_estimate(ctypes.byref(s.c), ctypes.byref(p), fake, fake, fake, fake, 1 << 40, None)
    assert rc == code, _lib.last_error()
    assert _lib.last_error()


def test_workspace_and_pointer_checks():
    s = _shape()
    p = X.make_params()
    lib = _lib.load()
    need = lib.xattn_workspace_size(ctypes.byref(s.c), ctypes.byref(p))
    fake = ctypes.c_void_p(0x1000)
    rc = lib.xattn_estimate(ctypes.byref(s.c), ctypes.byref(p), fake, fake, fake, None, need, None)
    assert rc == _lib.XATTN_ERR_WORKSPACE
    rc = lib.xattn_estimate(ctypes.byref(s.c), ctypes.byref(p), fake, fake, fake, fake, need - 1, None)
    assert rc == _lib.XATTN_ERR_WORKSPACE
    rc = lib.xattn_estimate(ctypes.byref(s.c), ctypes.byref(p), fake, None, fake, fake, need, None)
    assert rc == _lib.XATTN_ERR_INVALID
    rc = lib.xattn_select(ctypes.byref(s.c), ctypes.byref(p), None, fake, None, None, fake, need, None)
    assert rc == _lib.XATTN_ERR_INVALID
    rc = lib.xattn_sparse_attn(ctypes.byref(s.c), ctypes.byref(p), fake, fake, fake, None, fake, None,
                               fake, need, None)
    assert rc == _lib.XATTN_ERR_INVALID
    rc = lib.xattn_merge_attn(4, 2, 6, fake, fake, fake, fake, fake, fake, None)
    assert rc == _lib.XATTN_ERR_INVALID
    assert lib.xattn_merge_attn(0, 2, 8, None, None, None, None, None, None, None) == 0


def test_block_table_too_short_is_rejected():
    t = torch.zeros((1, 2), dtype=torch.int32)
    s = _shape(lq=(128,), lk=(512,), table=t, phys=4)
    p = X.make_params()
    assert _lib.load().xattn_workspace_size(ctypes.byref(s.c), ctypes.byref(p)) == 0
    assert "max_blocks_per_seq" in _lib.last_error()


def test_vt_pages_reserved_only_for_the_single_phase_kernel():
    """The V^T pages (read only by the single-phase bf16 attention: odd GQA
    groups, or K/V spans beyond 31-bit offsets) are reserved only when some
    launch can run that kernel: with an even group the workspace does not
    grow with the paged cache; with an odd group it grows by one V page per
    cache page; fp32 never reserves them."""
    p = X.make_params()
    t = torch.zeros((1, 4), dtype=torch.int32)
    page = 128 * 2 * 128 * 2  # one bf16 page of V at 2 kv heads, d = 128
    lib = _lib.load()

    def size(hq, phys, dtype=torch.bfloat16):
        s = _shape(lq=(128,), lk=(512,), hq=hq, hkv=2, table=t, phys=phys, dtype=dtype)
        return lib.xattn_workspace_size(ctypes.byref(s.c), ctypes.byref(p))

    assert size(4, 16) == size(4, 4096)                      # group 2
    assert size(6, 4096) - size(6, 16) == (4096 - 16) * page  # group 3
    assert size(6, 4096, torch.float32) == size(6, 16, torch.float32)
    # an even group whose cache spans 2 GiB or more reserves them too
    big = (1 << 31) // page
    assert size(4, big) - size(4, big - 1) == big * page


def test_kernel_timing_hook_host_side():
    """The measurement hook checks its outputs and, with nothing recorded,
    reads zero launches without touching a device."""
    lib = _lib.load()
    assert lib.xattn_kernel_timing_read(None, None) == -1
    assert lib.xattn_kernel_timing(1) == 0
    assert X.xattn_kernel_timing_read() == (0.0, 0)
    assert lib.xattn_kernel_timing(0) == 0
    assert X.xattn_kernel_timing_read() == (0.0, 0)

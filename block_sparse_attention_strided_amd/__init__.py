"""MI355X (gfx950) XAttention block-sparse prefill: Python binding of libxattn.

The functions here carry the names of the C entry points (include/xattn.h)
and only marshal arguments: PyTorch provides device memory and streams,
every computation runs in the library's HIP kernels.  Nothing falls back to
a CPU or PyTorch implementation; a missing library raises at first use.
"""

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    GQA_ANY,
    GQA_MAJORITY,
    SELECT_CHUNK_VOTE,
    SELECT_CHUNK_VOTE_SPARSE,
    SELECT_PER_KVHEAD,
    XattnAux,
    XattnParams,
    XattnShape,
)

_MODES = {"per_kvhead": SELECT_PER_KVHEAD, "chunk_vote": SELECT_CHUNK_VOTE,
          "chunk_vote_sparse": SELECT_CHUNK_VOTE_SPARSE}
_AGGS = {"any": GQA_ANY, "majority": GQA_MAJORITY}


class XattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("xattn error %d: %s" % (code, msg))
        self.code = code


def _check(rc):
    if rc != 0:
        raise XattnError(rc, _lib.last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Shape:
    """XattnShape plus the host/device arrays it points to (kept alive here).

    q: [total_q, Hq, d] tensor (its dtype picks bf16 or fp32); cu_q / cu_k:
    host int sequences of length batch+1; block_table: optional int32 device
    tensor [batch, max_blocks] (-1 = unallocated page).
    """

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, dtype, cu_q, cu_k, device,
                 block_table=None, num_phys_blocks=0):
        self.cu_q_list = [int(x) for x in cu_q]
        self.cu_k_list = [int(x) for x in cu_k]
        n = len(self.cu_q_list)
        self._cu_q_host = (ctypes.c_int32 * n)(*self.cu_q_list)
        self._cu_k_host = (ctypes.c_int32 * n)(*self.cu_k_list)
        self.cu_q_dev = torch.tensor(self.cu_q_list, dtype=torch.int32, device=device)
        self.cu_k_dev = torch.tensor(self.cu_k_list, dtype=torch.int32, device=device)
        self.block_table = block_table
        s = XattnShape()
        s.batch = n - 1
        s.num_q_heads = num_q_heads
        s.num_kv_heads = num_kv_heads
        s.head_dim = head_dim
        s.dtype = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(dtype, 99)
        s.cu_q_host = ctypes.cast(self._cu_q_host, ctypes.POINTER(ctypes.c_int32))
        s.cu_k_host = ctypes.cast(self._cu_k_host, ctypes.POINTER(ctypes.c_int32))
        s.cu_q = self.cu_q_dev.data_ptr()
        s.cu_k = self.cu_k_dev.data_ptr()
        if block_table is not None:
            assert block_table.dtype == torch.int32 and block_table.is_contiguous()
            s.block_table = block_table.data_ptr()
            s.max_blocks_per_seq = block_table.shape[1]
            s.num_phys_blocks = int(num_phys_blocks)
        else:
            s.block_table = None
            s.max_blocks_per_seq = 0
            s.num_phys_blocks = 0
        self.c = s
        self.batch = n - 1
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        lq = [self.cu_q_list[b + 1] - self.cu_q_list[b] for b in range(self.batch)]
        lk = [self.cu_k_list[b + 1] - self.cu_k_list[b] for b in range(self.batch)]
        self.max_qb = max(lq) // 128 if lq else 0
        self.max_kb = max(lk) // 128 if lk else 0
        self.total_q = self.cu_q_list[-1]


def make_params(*, stride=8, threshold=0.9, est_scale=0.0, softmax_scale=0.0, kv_chunk_tokens=4096,
                select_mode="chunk_vote", group_agg="any", block_size=128, num_to_choose=0,
                reuse_selection=0):
    p = XattnParams()
    p.stride = stride
    p.block_size = block_size
    p.threshold = threshold
    p.est_scale = est_scale
    p.softmax_scale = softmax_scale
    p.kv_chunk_tokens = kv_chunk_tokens
    p.select_mode = _MODES.get(select_mode, select_mode) if isinstance(select_mode, str) else select_mode
    p.group_agg = _AGGS.get(group_agg, group_agg) if isinstance(group_agg, str) else group_agg
    p.num_to_choose = num_to_choose
    p.reuse_selection = int(reuse_selection)
    return p


def xattn_workspace_size(shape, params):
    n = _lib.load().xattn_workspace_size(ctypes.byref(shape.c), ctypes.byref(params))
    if n == 0:
        raise XattnError(-1, _lib.last_error())
    return n


def alloc_workspace(shape, params, device="cuda"):
    n = xattn_workspace_size(shape, params)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def xattn_estimate(shape, params, q, k, block_sums, ws, stream=None):
    _check(_lib.load().xattn_estimate(ctypes.byref(shape.c), ctypes.byref(params), _ptr(q), _ptr(k),
                                      _ptr(block_sums), _ptr(ws), ws.numel(), _stream(stream)))


def xattn_select(shape, params, block_sums, mask_kv, hist_sel, counts, ws, stream=None):
    _check(_lib.load().xattn_select(ctypes.byref(shape.c), ctypes.byref(params), _ptr(block_sums),
                                    _ptr(mask_kv), _ptr(hist_sel), _ptr(counts), _ptr(ws), ws.numel(),
                                    _stream(stream)))


def xattn_sparse_attn(shape, params, q, k, v, mask_kv, out, lse, ws, stream=None):
    _check(_lib.load().xattn_sparse_attn(ctypes.byref(shape.c), ctypes.byref(params), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(mask_kv), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream(stream)))


def xattn_attn_plan(shape, params, v, mask_kv, ws, stream=None):
    _check(_lib.load().xattn_attn_plan(ctypes.byref(shape.c), ctypes.byref(params), _ptr(v), _ptr(mask_kv),
                                       _ptr(ws), ws.numel(), _stream(stream)))


def xattn_attn_run(shape, params, q, k, v, mask_kv, out, lse, ws, stream=None):
    _check(_lib.load().xattn_attn_run(ctypes.byref(shape.c), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(mask_kv), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def xattn_kernel_timing(on):
    """Enable (True) or disable the library's event pairs around every
    attention kernel launch (the measurement hook of include/xattn.h)."""
    _check(_lib.load().xattn_kernel_timing(1 if on else 0))


def xattn_kernel_timing_read():
    """(total ms, launches) of the attention kernels recorded since the last
    read or switch; forgets them."""
    total = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check(_lib.load().xattn_kernel_timing_read(ctypes.byref(total), ctypes.byref(n)))
    return total.value, n.value


def xattn_merge_attn(o_a, lse_a, o_b, lse_b, o, lse, stream=None):
    rows, heads, hd = o_a.shape
    _check(_lib.load().xattn_merge_attn(rows, heads, hd, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                        _ptr(o), _ptr(lse), _stream(stream)))


class Ring:
    """Device ring of slots for streaming pinned host K/V history."""

    def __init__(self, num_slots, slot_blocks, num_kv_heads, head_dim, dtype, *, staged=False):
        """staged=True: xattn_ring_create_staged with slot_blocks = max_blocks
        (num_slots is ignored)."""
        self.handle = ctypes.c_void_p()
        code = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(dtype, 99)
        if staged:
            _check(_lib.load().xattn_ring_create_staged(slot_blocks, num_kv_heads, head_dim, code,
                                                        ctypes.byref(self.handle)))
        else:
            _check(_lib.load().xattn_ring_create(num_slots, slot_blocks, num_kv_heads, head_dim, code,
                                                 ctypes.byref(self.handle)))

    def set_copy_delay_us(self, usec):
        _check(_lib.load().xattn_ring_set_copy_delay_us(self.handle, usec))

    def offload_chunk(self, k, v, k_host_dst, v_host_dst, num_blocks, stream=None):
        """Write a prefilled chunk's K/V back to pinned host history."""
        _check(_lib.load().xattn_ring_offload_chunk(self.handle, _ptr(k), _ptr(v), _ptr(k_host_dst),
                                                    _ptr(v_host_dst), int(num_blocks), _stream(stream)))

    def offload_wait(self, stream=None):
        _check(_lib.load().xattn_ring_offload_wait(self.handle, _stream(stream)))

    def close(self):
        if self.handle:
            _lib.load().xattn_ring_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _aux(aux):
    if aux is None:
        return None
    a = XattnAux()
    a.block_sums = aux.get("block_sums").data_ptr() if aux.get("block_sums") is not None else None
    a.mask_kv = aux.get("mask_kv").data_ptr() if aux.get("mask_kv") is not None else None
    a.hist_sel = aux.get("hist_sel").data_ptr() if aux.get("hist_sel") is not None else None
    return a


def xattn_prefill_chunk_static(shape, params, q, k, v, out, lse, counts, *, aux=None, stream=None):
    """Resident-K/V prefill on the library's static per-device scratch (no
    workspace, no device allocation)."""
    a = _aux(aux)
    _check(_lib.load().xattn_prefill_chunk_static(
        ctypes.byref(shape.c), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
        _ptr(counts), ctypes.byref(a) if a is not None else None, _stream(stream)))


def xattn_prefill_chunk(shape, params, q, k, v, out, lse, counts, ws, *, aux=None, ring=None,
                        k_hist=None, v_hist=None, hist_blocks=0, stream=None):
    a = _aux(aux)
    _check(_lib.load().xattn_prefill_chunk(
        ring.handle if ring is not None else None, ctypes.byref(shape.c), ctypes.byref(params),
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_hist), _ptr(v_hist), int(hist_blocks), _ptr(out), _ptr(lse),
        _ptr(counts), ctypes.byref(a) if a is not None else None, _ptr(ws), ws.numel(), _stream(stream)))

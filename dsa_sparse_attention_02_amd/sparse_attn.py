"""Thin Python binding of libsparse_attn.so (include/sparse_attn.h).

Argument marshalling only: torch supplies device memory and the current stream,
every step of the computation runs in the library's HIP kernels.  Functions
carry the C entry points' names.  There is no fallback: if the library is not
built, or a call returns an error status, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(6)
SA_OUT_F32, SA_OUT_BF16 = 0, 1

EXPORTS = (
    "sa_abi_version", "sa_status_string",
    "sa_decode_workspace_size", "sparse_attn_decode", "sparse_attn_select_decode", "sparse_attn_attend_decode",
    "sa_prefill_workspace_size", "sparse_attn_prefill", "sparse_attn_select_prefill", "sparse_attn_attend_prefill",
    "sparse_attn_decode_profiled", "sparse_attn_prefill_profiled", "sparse_attn_decode_append",
    "sa_prefill_varlen_workspace_size", "sparse_attn_prefill_varlen", "sparse_attn_prefill_varlen_profiled",
    "sa_decode_blocks_workspace_size", "sparse_attn_decode_blocks", "sa_prefill_blocks_workspace_size",
    "sparse_attn_prefill_blocks", "sa_decode_workspace_size_cfg", "sparse_attn_decode_cfg",
    "sa_decode_tune_workspace_size", "sa_decode_tune", "sparse_attn_decode_noalloc",
    "sparse_attn_prefill_varlen_cfg",
)


class sa_decode_config(ctypes.Structure):
    _fields_ = [("attn_splits", ctypes.c_int32), ("topk_path", ctypes.c_int32), ("attn_partners", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 1)]


SA_TOPK_DEFAULT, SA_TOPK_THRESHOLD, SA_TOPK_ONEPASS_U2, SA_TOPK_ONEPASS_U4 = 0, 1, 2, 3


class sa_prefill_config(ctypes.Structure):
    _fields_ = [("pipeline", ctypes.c_int32), ("attn_partners", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


SA_PREFILL_SERIAL, SA_PREFILL_PIPELINED = 0, 1
SA_ATTN_PARTNERS_DEFAULT, SA_ATTN_PARTNERS_2, SA_ATTN_PARTNERS_4 = 0, 2, 4


class sa_params(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("idx_relu", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class sa_paged_cache(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("idx_k", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
                ("context_lens", ctypes.c_void_p)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libsparse_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with dsa_sparse_attention_02_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, sz = ctypes.c_int32, ctypes.c_size_t
        pp, pc = ctypes.POINTER(sa_params), ctypes.POINTER(sa_paged_cache)
        sig = {
            "sa_abi_version": (i32, []),
            "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "sa_decode_workspace_size": (ctypes.c_int, [pp, i32, i32, ctypes.POINTER(sz)]),
            "sa_prefill_workspace_size": (ctypes.c_int, [pp, i32, i32, ctypes.POINTER(sz)]),
            "sparse_attn_decode": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P]),
            "sparse_attn_select_decode": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, sz, P]),
            "sparse_attn_attend_decode": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, sz, P]),
            "sparse_attn_prefill": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P]),
            "sparse_attn_select_prefill": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, sz, P]),
            "sparse_attn_attend_prefill": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, sz, P]),
            "sparse_attn_decode_profiled": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P, P, i32,
                                                           ctypes.POINTER(i32)]),
            "sparse_attn_prefill_profiled": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P, P, i32,
                                                            ctypes.POINTER(i32)]),
            "sparse_attn_decode_append": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, P, P, sz, P]),
            "sa_prefill_varlen_workspace_size": (ctypes.c_int, [pp, i32, P, P, ctypes.POINTER(sz)]),
            "sparse_attn_prefill_varlen": (ctypes.c_int, [pp, pc, i32, P, P, P, P, P, P, P, P, P, sz, P]),
            "sparse_attn_prefill_varlen_profiled": (ctypes.c_int, [pp, pc, i32, P, P, P, P, P, P, P, P, P, sz, P,
                                                                   P, i32, ctypes.POINTER(i32)]),
            "sparse_attn_prefill_varlen_cfg": (ctypes.c_int, [pp, pc, i32, P, P, P, P, P, P, P, P, P, P, sz, P]),
            "sa_decode_blocks_workspace_size": (ctypes.c_int, [pp, i32, i32, ctypes.POINTER(sz)]),
            "sparse_attn_decode_blocks": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P]),
            "sa_prefill_blocks_workspace_size": (ctypes.c_int, [pp, i32, i32, i32, ctypes.POINTER(sz)]),
            "sparse_attn_prefill_blocks": (ctypes.c_int, [pp, pc, i32, i32, i32, P, P, P, P, P, P, P, sz, P]),
            "sa_decode_workspace_size_cfg": (ctypes.c_int, [pp, i32, i32, P, ctypes.POINTER(sz)]),
            "sparse_attn_decode_cfg": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, P, sz, P]),
            "sa_decode_tune_workspace_size": (ctypes.c_int, [pp, i32, i32, ctypes.POINTER(sz)]),
            "sa_decode_tune": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P, sz, P, i32, P,
                                              ctypes.POINTER(ctypes.c_float)]),
            "sparse_attn_decode_noalloc": (ctypes.c_int, [pp, pc, i32, i32, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sa_status_string(status).decode()


def _check(status: int, where: str):
    if status != SA_OK:
        raise SparseAttnError(status, where)


@dataclass(frozen=True)
class Params:
    num_heads: int
    qk_dim: int
    v_dim: int
    idx_heads: int
    idx_dim: int
    block_size: int
    topk: int
    softmax_scale: float
    idx_relu: int = 1
    out_bf16: bool = False

    @staticmethod
    def from_shape(shape, out_bf16: bool = False) -> "Params":
        return Params(shape.num_heads, shape.qk_dim, shape.v_dim, shape.idx_heads, shape.idx_dim,
                      shape.block_size, shape.topk, float(shape.softmax_scale), shape.idx_relu, out_bf16)

    def c(self) -> sa_params:
        return sa_params(self.num_heads, self.qk_dim, self.v_dim, self.idx_heads, self.idx_dim, self.block_size,
                         self.topk, self.softmax_scale, self.idx_relu, SA_OUT_BF16 if self.out_bf16 else SA_OUT_F32)


# ------------------------------------------------------------ torch layer --
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t, name, dtypes, shape=None):
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


@dataclass
class PagedCache:
    """Device tensors of a paged cache: kv [num_blocks][bs][qk_dim] bf16,
    idx_k [num_blocks][bs][idx_dim] bf16, block_table [seqs][max_blocks] int32,
    context_lens [seqs] int32 (decode)."""
    kv: object
    idx_k: object
    block_table: object
    context_lens: object = None

    def c(self) -> sa_paged_cache:
        torch = _torch()
        bt = _dev(self.block_table, "block_table", (torch.int32,))
        kv = self.kv if self.kv is not None else self.idx_k
        cl = None
        if self.context_lens is not None:
            cl = _dev(self.context_lens, "context_lens", (torch.int32,))
        return sa_paged_cache(_ptr(self.kv), _ptr(self.idx_k), int(kv.shape[0]), bt.data_ptr(), int(bt.shape[1]),
                              _ptr(cl))


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context of a call: the caller's stream when one is given, so
    that the caching allocator ties the call's temporaries (workspace and
    default outputs) to the stream the kernels run on."""
    import contextlib
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(nbytes: int, device, stream=None):
    torch = _torch()
    with _on(stream):
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def decode_workspace_size(p: Params, batch: int, max_ctx: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_decode_workspace_size(ctypes.byref(p.c()), batch, max_ctx, ctypes.byref(n)),
           "sa_decode_workspace_size")
    return n.value


def prefill_workspace_size(p: Params, num_rows: int, q_start: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_prefill_workspace_size(ctypes.byref(p.c()), num_rows, q_start, ctypes.byref(n)),
           "sa_prefill_workspace_size")
    return n.value


def _index_out(rows: int, k: int, device, stream=None):
    torch = _torch()
    with _on(stream):
        return torch.empty((rows, k), dtype=torch.int32, device=device)


def _outputs(p: Params, rows: int, device, want_lse: bool, stream=None):
    torch = _torch()
    with _on(stream):
        topk_idx = torch.empty((rows, p.topk), dtype=torch.int32, device=device)
        out = torch.empty((rows, p.num_heads, p.v_dim), dtype=torch.bfloat16 if p.out_bf16 else torch.float32,
                          device=device)
        lse = torch.empty((rows, p.num_heads), dtype=torch.float32, device=device) if want_lse else None
    return topk_idx, out, lse


def sparse_attn_decode(p: Params, cache: PagedCache, max_ctx: int, q, idx_q, idx_w, *, want_lse=True,
                       workspace=None, outputs=None, stream=None):
    """Indexer -> top-k -> sparse attention for one query row per sequence.
    Returns (topk_idx [B][k] int32, out [B][H][D_v], lse [B][H] or None)."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(decode_workspace_size(p, B, max_ctx), q.device, stream)
    _check(lib().sparse_attn_decode(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx, q.data_ptr(),
                                    idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(),
                                    _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)), "sparse_attn_decode")
    return topk_idx, out, lse


def sparse_attn_decode_noalloc(p: Params, cache: PagedCache, max_ctx: int, q, idx_q, idx_w, *, want_lse=True,
                               outputs=None, stream=None):
    """sparse_attn_decode with the library's static scratch array instead of a
    workspace (the C call allocates nothing; only default outputs are
    allocated here).  Calls that overlap on one GPU race."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    _check(lib().sparse_attn_decode_noalloc(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx, q.data_ptr(),
                                            idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(),
                                            out.data_ptr(), _ptr(lse), _stream(stream)),
           "sparse_attn_decode_noalloc")
    return topk_idx, out, lse


def sparse_attn_decode_append(p: Params, cache: PagedCache, max_ctx: int, new_kv, new_idx_k, q, idx_q, idx_w, *,
                              want_lse=True, workspace=None, outputs=None, stream=None):
    """sparse_attn_decode after writing each sequence's current token (position
    context_lens[b] - 1) into the cache: new_kv [B][qk_dim] and new_idx_k
    [B][idx_dim] (bf16) overwrite that position's slot in cache.kv / cache.idx_k.
    Returns (topk_idx, out, lse) as sparse_attn_decode."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    _dev(new_kv, "new_kv", _bf16_types(), (B, p.qk_dim))
    _dev(new_idx_k, "new_idx_k", _bf16_types(), (B, p.idx_dim))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(decode_workspace_size(p, B, max_ctx), q.device, stream)
    _check(lib().sparse_attn_decode_append(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx,
                                           new_kv.data_ptr(), new_idx_k.data_ptr(), q.data_ptr(), idx_q.data_ptr(),
                                           idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(), _ptr(lse),
                                           ws.data_ptr(), ws.numel(), _stream(stream)), "sparse_attn_decode_append")
    return topk_idx, out, lse


def sparse_attn_decode_profiled(p: Params, cache: PagedCache, max_ctx: int, q, idx_q, idx_w, events, *,
                                want_lse=True, workspace=None, outputs=None, stream=None):
    """sparse_attn_decode that also records `events` (HipEvents) around its kernels.
    Returns (topk_idx, out, lse, number of marks the call takes)."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(decode_workspace_size(p, B, max_ctx), q.device, stream)
    ev = (ctypes.c_void_p * max(1, len(events)))(*[e.handle for e in events])
    n = ctypes.c_int32()
    _check(lib().sparse_attn_decode_profiled(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx,
                                             q.data_ptr(), idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(),
                                             out.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream),
                                             ev, len(events), ctypes.byref(n)), "sparse_attn_decode_profiled")
    return topk_idx, out, lse, n.value


def sparse_attn_prefill_profiled(p: Params, cache: PagedCache, q_start: int, q, idx_q, idx_w, events, *,
                                 want_lse=True, workspace=None, outputs=None, stream=None):
    """sparse_attn_prefill that also records `events` around its kernels."""
    torch = _torch()
    L = q.shape[0]
    _dev(q, "q", _bf16_types(), (L, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (L, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (L, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, L, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(prefill_workspace_size(p, L, q_start), q.device, stream)
    ev = (ctypes.c_void_p * max(1, len(events)))(*[e.handle for e in events])
    n = ctypes.c_int32()
    _check(lib().sparse_attn_prefill_profiled(ctypes.byref(p.c()), ctypes.byref(cache.c()), L, q_start,
                                              q.data_ptr(), idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(),
                                              out.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream),
                                              ev, len(events), ctypes.byref(n)), "sparse_attn_prefill_profiled")
    return topk_idx, out, lse, n.value


def _host_i32(a, name, n):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if a.shape != (n,):
        raise SparseAttnError(SA_ERR_SHAPE, f"{name}: expected {n} int32 entries, got shape {a.shape}")
    return a


def prefill_varlen_workspace_size(p: Params, cu_seqlens, q_starts) -> int:
    q_starts = np.asarray(q_starts)
    cu = _host_i32(cu_seqlens, "cu_seqlens", len(q_starts) + 1)
    qs = _host_i32(q_starts, "q_starts", len(q_starts))
    n = ctypes.c_size_t()
    _check(lib().sa_prefill_varlen_workspace_size(ctypes.byref(p.c()), len(qs), cu.ctypes.data, qs.ctypes.data,
                                                  ctypes.byref(n)), "sa_prefill_varlen_workspace_size")
    return n.value


def sparse_attn_prefill_varlen(p: Params, cache: PagedCache, cu_seqlens, q_starts, q, idx_q, idx_w, *,
                               want_lse=True, workspace=None, outputs=None, stream=None, events=None,
                               pipeline=None, attn_partners=None):
    """Prefill of several sequences in one call: sequence s owns packed rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1 (host int32 arrays), its row i at
    position q_starts[s] + i, block-table row s.  With `events`, the profiling
    entry point records them around the kernels and the mark count is returned
    as a fourth value.  With `pipeline` (SA_PREFILL_*) or `attn_partners`
    (SA_ATTN_PARTNERS_*), the configured entry point runs that schedule and
    attention kernel."""
    torch = _torch()
    q_starts = np.asarray(q_starts)
    cu = _host_i32(cu_seqlens, "cu_seqlens", len(q_starts) + 1)
    qs = _host_i32(q_starts, "q_starts", len(q_starts))
    L = q.shape[0]
    if int(cu[-1]) != L:
        raise SparseAttnError(SA_ERR_SHAPE, f"cu_seqlens ends at {int(cu[-1])}, but q has {L} rows")
    _dev(q, "q", _bf16_types(), (L, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (L, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (L, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, L, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(prefill_varlen_workspace_size(p, cu, qs), q.device, stream)
    args = (ctypes.byref(p.c()), ctypes.byref(cache.c()), len(qs), cu.ctypes.data, qs.ctypes.data, q.data_ptr(),
            idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(), _ptr(lse), ws.data_ptr(),
            ws.numel(), _stream(stream))
    if pipeline is not None or attn_partners is not None:
        if events is not None:
            raise SparseAttnError(SA_ERR_SHAPE, "a configuration and events are exclusive")
        cfg = sa_prefill_config(pipeline=pipeline or SA_PREFILL_SERIAL,
                                attn_partners=attn_partners or SA_ATTN_PARTNERS_DEFAULT)
        _check(lib().sparse_attn_prefill_varlen_cfg(*args[:5], ctypes.byref(cfg), *args[5:]),
               "sparse_attn_prefill_varlen_cfg")
        return topk_idx, out, lse
    if events is None:
        _check(lib().sparse_attn_prefill_varlen(*args), "sparse_attn_prefill_varlen")
        return topk_idx, out, lse
    ev = (ctypes.c_void_p * max(1, len(events)))(*[e.handle for e in events])
    n = ctypes.c_int32()
    _check(lib().sparse_attn_prefill_varlen_profiled(*args, ev, len(events), ctypes.byref(n)),
           "sparse_attn_prefill_varlen_profiled")
    return topk_idx, out, lse, n.value


def decode_blocks_workspace_size(p: Params, batch: int, max_ctx: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_decode_blocks_workspace_size(ctypes.byref(p.c()), batch, max_ctx, ctypes.byref(n)),
           "sa_decode_blocks_workspace_size")
    return n.value


def prefill_blocks_workspace_size(p: Params, num_rows: int, q_start: int, q_block: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_prefill_blocks_workspace_size(ctypes.byref(p.c()), num_rows, q_start, q_block, ctypes.byref(n)),
           "sa_prefill_blocks_workspace_size")
    return n.value


def sparse_attn_decode_blocks(p: Params, cache: PagedCache, max_ctx: int, q, idx_q, idx_w, *, want_lse=True,
                              workspace=None, outputs=None, stream=None):
    """Block-granular decode: p.topk counts kept KV blocks (cache blocks) per
    row.  Returns (block_idx [B][k] int32, out [B][H][D_v], lse [B][H] or None)."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    blk, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(decode_blocks_workspace_size(p, B, max_ctx), q.device, stream)
    _check(lib().sparse_attn_decode_blocks(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx, q.data_ptr(),
                                           idx_q.data_ptr(), idx_w.data_ptr(), blk.data_ptr(), out.data_ptr(),
                                           _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)),
           "sparse_attn_decode_blocks")
    return blk, out, lse


def sparse_attn_prefill_blocks(p: Params, cache: PagedCache, q_start: int, q_block: int, q, idx_q, idx_w, *,
                               want_lse=True, workspace=None, stream=None):
    """Block-granular prefill of sequence 0: query blocks of q_block rows, p.topk
    kept KV blocks each.  Returns (block_idx [ceil(L/q_block)][k] int32, out, lse)."""
    torch = _torch()
    L = q.shape[0]
    _dev(q, "q", _bf16_types(), (L, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (L, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (L, p.idx_heads))
    groups = (L + max(1, q_block) - 1) // max(1, q_block)
    blk = _index_out(groups, p.topk, q.device, stream)
    _, out, lse = _outputs(p, L, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(prefill_blocks_workspace_size(p, L, q_start, q_block),
                                                            q.device)
    _check(lib().sparse_attn_prefill_blocks(ctypes.byref(p.c()), ctypes.byref(cache.c()), L, q_start, q_block,
                                            q.data_ptr(), idx_q.data_ptr(), idx_w.data_ptr(), blk.data_ptr(),
                                            out.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)),
           "sparse_attn_prefill_blocks")
    return blk, out, lse


def _cfg(attn_splits: int, topk_path: int = SA_TOPK_DEFAULT, attn_partners: int = SA_ATTN_PARTNERS_DEFAULT):
    return sa_decode_config(attn_splits=attn_splits, topk_path=topk_path, attn_partners=attn_partners)


def decode_workspace_size_cfg(p: Params, batch: int, max_ctx: int, attn_splits: int = 0,
                              topk_path: int = SA_TOPK_DEFAULT) -> int:
    n = ctypes.c_size_t()
    _check(lib().sa_decode_workspace_size_cfg(ctypes.byref(p.c()), batch, max_ctx,
                                              ctypes.byref(_cfg(attn_splits, topk_path)), ctypes.byref(n)),
           "sa_decode_workspace_size_cfg")
    return n.value


def sparse_attn_decode_cfg(p: Params, cache: PagedCache, max_ctx: int, attn_splits: int, q, idx_q, idx_w, *,
                           topk_path=SA_TOPK_DEFAULT, attn_partners=SA_ATTN_PARTNERS_DEFAULT, want_lse=True,
                           workspace=None, outputs=None, stream=None):
    """sparse_attn_decode with attn_splits attention splits per row (0 = default),
    a top-k path (SA_TOPK_*) and an attention kernel (SA_ATTN_PARTNERS_*)."""
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(
        decode_workspace_size_cfg(p, B, max_ctx, attn_splits, topk_path), q.device)
    _check(lib().sparse_attn_decode_cfg(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx,
                                        ctypes.byref(_cfg(attn_splits, topk_path, attn_partners)), q.data_ptr(),
                                        idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(), _ptr(lse),
                                        ws.data_ptr(), ws.numel(), _stream(stream)), "sparse_attn_decode_cfg")
    return topk_idx, out, lse


def decode_tune(p: Params, cache: PagedCache, max_ctx: int, q, idx_q, idx_w, *, reps=10, stream=None):
    """Run-time tuning of the decode split count, top-k path and attention
    kernel on these inputs (waits for the stream).  Returns (attn_splits,
    topk_path, attn_partners, microseconds per call)."""
    torch = _torch()
    B = q.shape[0]
    n = ctypes.c_size_t()
    _check(lib().sa_decode_tune_workspace_size(ctypes.byref(p.c()), B, max_ctx, ctypes.byref(n)),
           "sa_decode_tune_workspace_size")
    ws = _workspace(n.value, q.device, stream)
    topk_idx, out, lse = _outputs(p, B, q.device, True, stream)
    best = sa_decode_config()
    us = ctypes.c_float()
    _check(lib().sa_decode_tune(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx, q.data_ptr(),
                                idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(), _ptr(lse),
                                ws.data_ptr(), ws.numel(), _stream(stream), reps, ctypes.byref(best),
                                ctypes.byref(us)), "sa_decode_tune")
    return best.attn_splits, best.topk_path, best.attn_partners, us.value


class HipEvent:
    """A raw hipEvent_t (created with the HIP runtime) for the profiling entry points."""
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            # use the HIP runtime already mapped into the process (torch's), never a second copy
            lib()
            path = "libamdhip64.so.7"
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            h = ctypes.CDLL(path)
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        h = ctypes.c_void_p()
        if self.hip().hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.handle = h.value

    def elapsed_ms(self, later: "HipEvent") -> float:
        t = ctypes.c_float()
        if self.hip().hipEventSynchronize(later.handle) != 0 or \
                self.hip().hipEventElapsedTime(ctypes.byref(t), self.handle, later.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def __del__(self):
        if getattr(self, "handle", None) and self._hip is not None:
            self._hip.hipEventDestroy(self.handle)


def sparse_attn_select_decode(p: Params, cache: PagedCache, max_ctx: int, idx_q, idx_w, *, workspace=None,
                              topk_idx=None, stream=None):
    torch = _torch()
    B = idx_q.shape[0]
    _dev(idx_q, "idx_q", _bf16_types(), (B, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (B, p.idx_heads))
    if topk_idx is None:
        topk_idx = _index_out(B, p.topk, idx_q.device, stream)
    ws = workspace if workspace is not None else _workspace(decode_workspace_size(p, B, max_ctx), idx_q.device, stream)
    _check(lib().sparse_attn_select_decode(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx,
                                           idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), ws.data_ptr(),
                                           ws.numel(), _stream(stream)), "sparse_attn_select_decode")
    return topk_idx


def sparse_attn_attend_decode(p: Params, cache: PagedCache, max_ctx: int, q, topk_idx, *, want_lse=True,
                              workspace=None, stream=None):
    torch = _torch()
    B = q.shape[0]
    _dev(q, "q", _bf16_types(), (B, p.num_heads, p.qk_dim))
    _dev(topk_idx, "topk_idx", (torch.int32,), (B, p.topk))
    _, out, lse = _outputs(p, B, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(decode_workspace_size(p, B, max_ctx), q.device, stream)
    _check(lib().sparse_attn_attend_decode(ctypes.byref(p.c()), ctypes.byref(cache.c()), B, max_ctx, q.data_ptr(),
                                           topk_idx.data_ptr(), out.data_ptr(), _ptr(lse), ws.data_ptr(),
                                           ws.numel(), _stream(stream)), "sparse_attn_attend_decode")
    return out, lse


def sparse_attn_prefill(p: Params, cache: PagedCache, q_start: int, q, idx_q, idx_w, *, want_lse=True,
                        workspace=None, outputs=None, stream=None):
    """Indexer -> top-k -> sparse attention for rows q_start .. q_start+L-1 of sequence 0."""
    torch = _torch()
    L = q.shape[0]
    _dev(q, "q", _bf16_types(), (L, p.num_heads, p.qk_dim))
    _dev(idx_q, "idx_q", _bf16_types(), (L, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (L, p.idx_heads))
    topk_idx, out, lse = outputs if outputs is not None else _outputs(p, L, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(prefill_workspace_size(p, L, q_start), q.device, stream)
    _check(lib().sparse_attn_prefill(ctypes.byref(p.c()), ctypes.byref(cache.c()), L, q_start, q.data_ptr(),
                                     idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), out.data_ptr(),
                                     _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)), "sparse_attn_prefill")
    return topk_idx, out, lse


def sparse_attn_select_prefill(p: Params, cache: PagedCache, q_start: int, idx_q, idx_w, *, workspace=None,
                               stream=None):
    torch = _torch()
    L = idx_q.shape[0]
    _dev(idx_q, "idx_q", _bf16_types(), (L, p.idx_heads, p.idx_dim))
    _dev(idx_w, "idx_w", (torch.float32,), (L, p.idx_heads))
    topk_idx = _index_out(L, p.topk, idx_q.device, stream)
    ws = workspace if workspace is not None else _workspace(prefill_workspace_size(p, L, q_start), idx_q.device, stream)
    _check(lib().sparse_attn_select_prefill(ctypes.byref(p.c()), ctypes.byref(cache.c()), L, q_start,
                                            idx_q.data_ptr(), idx_w.data_ptr(), topk_idx.data_ptr(), ws.data_ptr(),
                                            ws.numel(), _stream(stream)), "sparse_attn_select_prefill")
    return topk_idx


def sparse_attn_attend_prefill(p: Params, cache: PagedCache, q_start: int, q, topk_idx, *, want_lse=True,
                               workspace=None, stream=None):
    torch = _torch()
    L = q.shape[0]
    _dev(q, "q", _bf16_types(), (L, p.num_heads, p.qk_dim))
    _dev(topk_idx, "topk_idx", (torch.int32,), (L, p.topk))
    _, out, lse = _outputs(p, L, q.device, want_lse, stream)
    ws = workspace if workspace is not None else _workspace(prefill_workspace_size(p, L, q_start), q.device, stream)
    _check(lib().sparse_attn_attend_prefill(ctypes.byref(p.c()), ctypes.byref(cache.c()), L, q_start, q.data_ptr(),
                                            topk_idx.data_ptr(), out.data_ptr(), _ptr(lse), ws.data_ptr(),
                                            ws.numel(), _stream(stream)), "sparse_attn_attend_prefill")
    return out, lse


def to_device(w: dict, device="cuda"):
    """Copy a synth workload's arrays to `device` (bf16 data keeps its bit patterns)."""
    torch = _torch()

    def t(a, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dt is not None:
            x = x.view(dt)
        return x.to(device)

    return dict(q=t(w["q"], torch.bfloat16), idx_q=t(w["idx_q"], torch.bfloat16), idx_w=t(w["idx_w"]),
                cache=PagedCache(kv=t(w["kv"], torch.bfloat16), idx_k=t(w["idx_k"], torch.bfloat16),
                                 block_table=t(w["block_table"]), context_lens=t(w["context_lens"])))

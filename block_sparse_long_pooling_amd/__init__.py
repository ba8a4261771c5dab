"""Block-sparse causal prefill attention for MI355X (gfx950).

Thin ctypes binding over libflashprefill.so: argument marshalling only.
Every step of the method (pooling, scoring, thresholding, attention, mean
correction) runs in the library's HIP kernels; torch provides device memory
and the current stream.  Function names follow the C entry points
(include/flashprefill.h).  If the library is missing the functions raise;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FLASHPREFILL_LIB selects another build of the same library (the host-side
# address-sanitizer build the CPU tests use); by default, the in-tree one.
LIB_PATH = os.environ.get("FLASHPREFILL_LIB") or os.path.join(_HERE, "libflashprefill.so")

FP_OK, FP_INVALID_ARGUMENT, FP_UNSUPPORTED, FP_WORKSPACE_TOO_SMALL, FP_DEVICE_ERROR = range(5)
FP_DTYPE_BF16, FP_DTYPE_FP8_E4M3FN = 0, 1
FP_MAX_BATCH = 128
FP_NOALLOC_SCRATCH_BYTES = 64 << 20


class fp_params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("mean_correction", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("shared_selection", ctypes.c_int32), ("query_probes", ctypes.c_int32)]


class FlashPrefillError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"flashprefill status {status}: {detail}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)

EXPORTS = {
    "fp_select_blocks": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P, ctypes.c_int32,
                                        _P, _P, _P, _P, _P, _P, _P]),
    "fp_select_blocks_fp8": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P, ctypes.c_int32,
                                            _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "fp_sparse_prefill_fwd": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P, _P, _P, _P,
                                             ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "fp_sparse_prefill_varlen_paged": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P,
                                                      ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                      _I32P, ctypes.c_int32, _P, _P, _P,
                                                      ctypes.c_size_t, _P, _P, _P]),
    "fp_sparse_prefill_varlen_paged_noalloc": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P,
                                                              ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                              _I32P, ctypes.c_int32, _P, _P, _P, _P, _P]),
    "fp_sparse_prefill_varlen_paged_fp8": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P,
                                                          ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                          _I32P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                                          ctypes.c_size_t, _P, _P, _P]),
    "fp_sparse_prefill_chunked_paged": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P,
                                                       ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                       _I32P, _I32P, ctypes.c_int32, _P, ctypes.c_int32,
                                                       _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "fp_sparse_prefill_chunked_paged_fp8": (ctypes.c_int, [ctypes.POINTER(fp_params), _P, _P, _P,
                                                           ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                                           _I32P, _I32P, ctypes.c_int32, _P, ctypes.c_int32,
                                                           _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                                           _P]),
    "fp_chunked_sizes": (ctypes.c_int, [ctypes.POINTER(fp_params), _I32P, _I32P, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_size_t)]),
    "fp_index_capacity": (ctypes.c_int64, [ctypes.POINTER(fp_params), _I32P, ctypes.c_int32]),
    "fp_count_entries": (ctypes.c_int64, [ctypes.POINTER(fp_params), _I32P, ctypes.c_int32]),
    "fp_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fp_params), _I32P, ctypes.c_int32]),
    "fp_attention_workgroups": (ctypes.c_int64, [ctypes.POINTER(fp_params), _I32P, ctypes.c_int32,
                                                 ctypes.c_int32]),
    "fp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp_last_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load libflashprefill.so (built by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int):
    if status != FP_OK:
        raise FlashPrefillError(status, lib().fp_last_error().decode())


def _shared_code(shared) -> int:
    """shared_selection: False (per head), True or 'union' (1), 'pooled' (2)."""
    if shared is False or shared is None or shared == 0:
        return 0
    if shared is True or shared == "union" or shared == 1:
        return 1
    if shared == "pooled" or shared == 2:
        return 2
    raise ValueError(f"shared_selection must be False, True/'union' or 'pooled', not {shared!r}")


def make_params(num_q_heads, num_kv_heads, head_dim, block_size, alpha, mean_correction=True,
                softmax_scale=0.0, dtype=FP_DTYPE_BF16, shared_selection=False,
                query_probes=0) -> fp_params:
    return fp_params(int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
                     float(alpha), float(softmax_scale), int(bool(mean_correction)), int(dtype),
                     _shared_code(shared_selection), int(query_probes))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _cu_host(cu_seqlens) -> ctypes.Array:
    vals = [int(x) for x in (cu_seqlens.tolist() if torch.is_tensor(cu_seqlens) else cu_seqlens)]
    return (ctypes.c_int32 * len(vals))(*vals)


def fp_index_capacity(params: fp_params, cu_seqlens: Sequence[int]) -> int:
    cu = _cu_host(cu_seqlens)
    return int(lib().fp_index_capacity(ctypes.byref(params), cu, len(cu) - 1))


def fp_count_entries(params: fp_params, cu_seqlens: Sequence[int]) -> int:
    cu = _cu_host(cu_seqlens)
    return int(lib().fp_count_entries(ctypes.byref(params), cu, len(cu) - 1))


def fp_varlen_workspace_bytes(params: fp_params, cu_seqlens: Sequence[int]) -> int:
    cu = _cu_host(cu_seqlens)
    return int(lib().fp_varlen_workspace_bytes(ctypes.byref(params), cu, len(cu) - 1))


def fp_attention_workgroups(params: fp_params, cu_seqlens: Sequence[int], paged: bool = False) -> int:
    """Workgroups the attention launch uses for these lengths: one per query
    block and query head (bf16 and fp8, contiguous or paged); -1 for invalid
    arguments."""
    cu = _cu_host(cu_seqlens)
    return int(lib().fp_attention_workgroups(ctypes.byref(params), cu, len(cu) - 1, int(bool(paged))))


@dataclass
class Selection:
    """Outputs of fp_select_blocks (device tensors)."""
    pooled_q: torch.Tensor      # fp32 [Hq, nB, d]
    pooled_k: torch.Tensor      # fp32 [Hkv, nB, d]
    pooled_v: Optional[torch.Tensor]    # fp32 [Hkv, nB, d]
    pooled_kv: Optional[torch.Tensor]   # bf16 [2, Hkv, nB, d]: K_bar, V_bar (mean correction)
    kv_idx: torch.Tensor        # int32, triangular-packed lists
    kv_cnt: torch.Tensor        # int32 [Hq, nB]
    block_size: int


def alloc_selection(params: fp_params, seqlen: int, device, pool_v: Optional[bool] = None) -> Selection:
    """Output buffers for fp_select_blocks on one sequence."""
    B, d, Hq = params.block_size, params.head_dim, params.num_q_heads
    nB = (seqlen + B - 1) // B
    if pool_v is None:
        pool_v = bool(params.mean_correction)
    pq = torch.empty((Hq, nB, d), dtype=torch.float32, device=device)
    pk = torch.empty((params.num_kv_heads, nB, d), dtype=torch.float32, device=device)
    pv = torch.empty_like(pk) if pool_v else None
    pkv = torch.empty((2, params.num_kv_heads, nB, d), dtype=torch.bfloat16, device=device) if pool_v else None
    cap = fp_index_capacity(params, [0, seqlen])
    kv_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    kv_cnt = torch.empty((Hq, nB), dtype=torch.int32, device=device)
    return Selection(pq, pk, pv, pkv, kv_idx, kv_cnt, B)


def fp_select_blocks(params: fp_params, q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                     pool_v: Optional[bool] = None, sel: Optional[Selection] = None) -> Selection:
    """Pooling + block scores + threshold + lists for one sequence (bf16 q/k/v).

    ``sel`` supplies preallocated output buffers (see alloc_selection)."""
    S = q.shape[0]
    dev = q.device
    if sel is None:
        sel = alloc_selection(params, S, dev, pool_v)
    pool_v = sel.pooled_v is not None or sel.pooled_kv is not None
    _check(lib().fp_select_blocks(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v) if pool_v else None,
                                  S, _ptr(sel.pooled_q), _ptr(sel.pooled_k), _ptr(sel.pooled_v),
                                  _ptr(sel.pooled_kv), _ptr(sel.kv_idx), _ptr(sel.kv_cnt), _stream(dev)))
    return sel


@dataclass
class Fp8Inputs:
    """Outputs of fp_select_blocks_fp8: e4m3 codes (uint8) and fp32 scales per
    (head, block), ready for fp_sparse_prefill_fwd in fp8 mode."""
    q8: torch.Tensor
    k8: torch.Tensor
    v8: torch.Tensor
    q_scale: torch.Tensor       # [Hq, nB]
    k_scale: torch.Tensor       # [Hkv, nB]
    v_scale: torch.Tensor


def fp_select_blocks_fp8(params: fp_params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         sel: Optional[Selection] = None, f8: Optional[Fp8Inputs] = None):
    """One pass over bf16 q/k/v: fp8 codes and scales, pooled means, then block
    scores + threshold + lists.  params.dtype must be fp8.  Returns (Selection, Fp8Inputs)."""
    S = q.shape[0]
    dev = q.device
    if sel is None:
        sel = alloc_selection(params, S, dev, pool_v=bool(params.mean_correction))
        sel.pooled_v = None
    if f8 is None:
        B = params.block_size
        nB = (S + B - 1) // B
        f8 = Fp8Inputs(torch.empty(q.shape, dtype=torch.uint8, device=dev),
                       torch.empty(k.shape, dtype=torch.uint8, device=dev),
                       torch.empty(v.shape, dtype=torch.uint8, device=dev),
                       torch.empty((q.shape[1], nB), dtype=torch.float32, device=dev),
                       torch.empty((k.shape[1], nB), dtype=torch.float32, device=dev),
                       torch.empty((v.shape[1], nB), dtype=torch.float32, device=dev))
    _check(lib().fp_select_blocks_fp8(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), S,
                                      _ptr(f8.q8), _ptr(f8.k8), _ptr(f8.v8), _ptr(f8.q_scale), _ptr(f8.k_scale),
                                      _ptr(f8.v_scale), _ptr(sel.pooled_q), _ptr(sel.pooled_k), _ptr(sel.pooled_kv),
                                      _ptr(sel.kv_idx), _ptr(sel.kv_cnt), _stream(dev)))
    return sel, f8


def fp_sparse_prefill_fwd(params: fp_params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          sel: Selection, q_scale=None, k_scale=None, v_scale=None,
                          out: Optional[torch.Tensor] = None, return_lse: bool = False,
                          lse: Optional[torch.Tensor] = None):
    """Attention over the kept blocks (+ mean correction) for one sequence.

    q/k/v are bf16, or uint8 e4m3fn codes with fp32 scales [H, nB] when
    params.dtype is FP_DTYPE_FP8_E4M3FN.  Returns out (bf16 [S, Hq, d]) and,
    with return_lse, lse (fp32 [Hq, S]).
    """
    S, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, S), dtype=torch.float32, device=dev)
    _check(lib().fp_sparse_prefill_fwd(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), S,
                                       _ptr(sel.kv_idx), _ptr(sel.kv_cnt), _ptr(sel.pooled_kv),
                                       _ptr(out), _ptr(lse), _stream(dev)))
    return (out, lse) if return_lse else out


@dataclass
class VarlenResult:
    out: torch.Tensor
    lse: Optional[torch.Tensor]
    kv_idx: torch.Tensor
    kv_cnt: torch.Tensor
    workspace: torch.Tensor


def fp_sparse_prefill_varlen_paged(params: fp_params, q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_table: torch.Tensor, cu_seqlens,
                                   return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None) -> VarlenResult:
    """Continuous batch over a paged KV cache (bf16): selection + attention."""
    T, Hq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    dev = q.device
    cu = _cu_host(cu_seqlens)
    batch = len(cu) - 1
    cap = fp_index_capacity(params, list(cu))
    ncnt = fp_count_entries(params, list(cu))
    wsb = fp_varlen_workspace_bytes(params, list(cu))
    kv_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty(max(ncnt, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().fp_sparse_prefill_varlen_paged(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), page_size, num_pages,
        _ptr(block_table), block_table.shape[1], cu, batch, _ptr(kv_idx), _ptr(kv_cnt),
        _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return VarlenResult(out, lse, kv_idx, kv_cnt, workspace)


def fp_sparse_prefill_varlen_paged_noalloc(params: fp_params, q: torch.Tensor, k_cache: torch.Tensor,
                                           v_cache: torch.Tensor, block_table: torch.Tensor, cu_seqlens,
                                           out: torch.Tensor, kv_idx: torch.Tensor, kv_cnt: torch.Tensor,
                                           lse: Optional[torch.Tensor] = None) -> None:
    """fp_sparse_prefill_varlen_paged with the library's own scratch: the
    caller passes every output buffer, and the call allocates nothing."""
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    cu = _cu_host(cu_seqlens)
    _check(lib().fp_sparse_prefill_varlen_paged_noalloc(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), page_size, num_pages,
        _ptr(block_table), block_table.shape[1], cu, len(cu) - 1, _ptr(kv_idx), _ptr(kv_cnt),
        _ptr(out), _ptr(lse), _stream(q.device)))


@dataclass
class Fp8Cache:
    """The fp8 paged cache: e4m3 pages shaped like the bf16 ones and fp32
    scales [num_pages, Hkv], one per (page holding a block's first token, head)."""
    k8: torch.Tensor
    v8: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor


def alloc_fp8_cache(k_cache: torch.Tensor) -> Fp8Cache:
    num_pages, _, Hkv, _ = k_cache.shape
    dev = k_cache.device
    return Fp8Cache(torch.empty(k_cache.shape, dtype=torch.uint8, device=dev),
                    torch.empty(k_cache.shape, dtype=torch.uint8, device=dev),
                    torch.empty((num_pages, Hkv), dtype=torch.float32, device=dev),
                    torch.empty((num_pages, Hkv), dtype=torch.float32, device=dev))


def fp_sparse_prefill_varlen_paged_fp8(params: fp_params, q: torch.Tensor, k_cache: torch.Tensor,
                                       v_cache: torch.Tensor, block_table: torch.Tensor, cu_seqlens,
                                       return_lse: bool = False, cache: Optional[Fp8Cache] = None,
                                       workspace: Optional[torch.Tensor] = None,
                                       out: Optional[torch.Tensor] = None):
    """fp8 inference over a paged batch (bf16 inputs): quantize + pool in one
    pass (codes into the fp8 paged cache), selection, fp8 attention reading the
    e4m3 pages.  Returns (VarlenResult, Fp8Cache)."""
    T, Hq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    dev = q.device
    cu = _cu_host(cu_seqlens)
    batch = len(cu) - 1
    cap = fp_index_capacity(params, list(cu))
    ncnt = fp_count_entries(params, list(cu))
    wsb = fp_varlen_workspace_bytes(params, list(cu))
    kv_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty(max(ncnt, 1), dtype=torch.int32, device=dev)
    if cache is None:
        cache = alloc_fp8_cache(k_cache)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().fp_sparse_prefill_varlen_paged_fp8(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), page_size, num_pages,
        _ptr(block_table), block_table.shape[1], cu, batch, _ptr(cache.k8), _ptr(cache.v8),
        _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(kv_idx), _ptr(kv_cnt),
        _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return VarlenResult(out, lse, kv_idx, kv_cnt, workspace), cache


def fp_chunked_sizes(params: fp_params, cu_seqlens_q: Sequence[int], kv_lens: Sequence[int]):
    """(kv_idx entries, kv_cnt entries, workspace bytes) for fp_sparse_prefill_chunked_paged."""
    cu = _cu_host(cu_seqlens_q)
    kl = _cu_host(kv_lens)
    cap, cnt, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib().fp_chunked_sizes(ctypes.byref(params), cu, kl, len(cu) - 1, ctypes.byref(cap),
                                  ctypes.byref(cnt), ctypes.byref(ws)))
    return int(cap.value), int(cnt.value), int(ws.value)


def alloc_pooled_cache(params: fp_params, num_pages: int, device) -> torch.Tensor:
    """fp32 [2, num_pages, Hkv, d]: the pooled-means cache kept between chunked calls."""
    return torch.zeros((2, num_pages, params.num_kv_heads, params.head_dim), dtype=torch.float32,
                       device=device)


def fp_sparse_prefill_chunked_paged(params: fp_params, q: torch.Tensor, k_cache: torch.Tensor,
                                    v_cache: torch.Tensor, block_table: torch.Tensor, cu_seqlens_q,
                                    kv_lens, pooled_cache: Optional[torch.Tensor] = None,
                                    prefix_pooled: bool = False, return_lse: bool = False,
                                    workspace: Optional[torch.Tensor] = None,
                                    out: Optional[torch.Tensor] = None) -> VarlenResult:
    """Chunked prefill over a paged KV cache (bf16): request b's q rows are the
    last q_len of its kv_lens[b]-token context; selection + attention."""
    T, Hq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    dev = q.device
    cu = _cu_host(cu_seqlens_q)
    kl = _cu_host(kv_lens)
    batch = len(cu) - 1
    cap, ncnt, wsb = fp_chunked_sizes(params, list(cu), list(kl))
    kv_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty(max(ncnt, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().fp_sparse_prefill_chunked_paged(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), page_size, num_pages,
        _ptr(block_table), block_table.shape[1], cu, kl, batch, _ptr(pooled_cache), int(bool(prefix_pooled)),
        _ptr(kv_idx), _ptr(kv_cnt), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return VarlenResult(out, lse, kv_idx, kv_cnt, workspace)


def fp_sparse_prefill_chunked_paged_fp8(params: fp_params, q: torch.Tensor, k_cache: torch.Tensor,
                                        v_cache: torch.Tensor, block_table: torch.Tensor, cu_seqlens_q,
                                        kv_lens, cache: Fp8Cache, pooled_cache: Optional[torch.Tensor] = None,
                                        prefix_pooled: bool = False, return_lse: bool = False,
                                        workspace: Optional[torch.Tensor] = None,
                                        out: Optional[torch.Tensor] = None) -> VarlenResult:
    """Chunked prefill with fp8 attention: selection on the bf16 pages as in
    fp_sparse_prefill_chunked_paged; the chunks' query blocks are encoded into
    the e4m3 pages of `cache` (earlier blocks must hold the codes of earlier
    calls), and attention reads the e4m3 pages."""
    T, Hq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    dev = q.device
    cu = _cu_host(cu_seqlens_q)
    kl = _cu_host(kv_lens)
    batch = len(cu) - 1
    cap, ncnt, wsb = fp_chunked_sizes(params, list(cu), list(kl))
    kv_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty(max(ncnt, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().fp_sparse_prefill_chunked_paged_fp8(
        ctypes.byref(params), _ptr(q), _ptr(k_cache), _ptr(v_cache), page_size, num_pages,
        _ptr(block_table), block_table.shape[1], cu, kl, batch, _ptr(pooled_cache), int(bool(prefix_pooled)),
        _ptr(cache.k8), _ptr(cache.v8), _ptr(cache.k_scale), _ptr(cache.v_scale),
        _ptr(kv_idx), _ptr(kv_cnt), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return VarlenResult(out, lse, kv_idx, kv_cnt, workspace)


def lists_to_mask(kv_idx: torch.Tensor, kv_cnt: torch.Tensor, num_heads: int, nB: int,
                  offset: int = 0, cnt_offset: int = 0) -> "numpy.ndarray":
    """Host helper: triangular-packed lists -> boolean mask [Hq, nB, nB] (numpy)."""
    import numpy as np
    idx = kv_idx.cpu().numpy()
    cnt = kv_cnt.reshape(-1).cpu().numpy()
    mask = np.zeros((num_heads, nB, nB), dtype=bool)
    tri = nB * (nB + 1) // 2
    for h in range(num_heads):
        for I in range(nB):
            c = int(cnt[cnt_offset + h * nB + I])
            base = offset + h * tri + I * (I + 1) // 2
            mask[h, I, idx[base:base + c]] = True
    return mask

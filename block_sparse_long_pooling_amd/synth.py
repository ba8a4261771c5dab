"""Seeded synthetic inputs for block-sparse causal prefill attention.

This module only draws and lays out inputs: it holds none of the method's
arithmetic (no pooling, scoring, thresholding or attention).  Both the HIP
path and the CPU oracle consume what it produces.

The recipe stands in for the activations of one attention layer of a
Llama-3-8B-shaped model (32 query heads, 8 KV heads, head_dim 128), the model
the FlashPrefill page (gist.science technical summary, section 4) evaluates
on; no real activations are available, so the structure that block-sparse
selection reacts to is planted by hand:

* Q, K, V: iid N(0, 1), drawn with ``numpy.random.default_rng(seed)`` (PCG64)
  as float32, in the order Q ``(S, Hq, d)``, K ``(S, Hkv, d)``,
  V ``(S, Hkv, d)``, then the sink direction u and the vertical direction w,
  each ``standard_normal(d)`` rescaled to norm 3.
* A sinusoidal positional term of amplitude 1 is added to every head of Q and
  K (not V): P[t, 2f] = sin(t * w_f), P[t, 2f+1] = cos(t * w_f),
  w_f = 10000 ** (-2f / d).  Nearby tokens then score higher, so the diagonal
  ("slash") pattern appears.
* Sinks: u is added to K at tokens 0..3 on every KV head (vertical pattern at
  the start of the sequence).
* Verticals (optional): w is added to K at tokens 4096*k, k >= 1.
* Everything is rounded to bfloat16 (round to nearest even).

fp8 inputs are quantized from the bf16 tensors with one fp32 scale per
(head, 128-token block): scale = amax / 448 (1 when the block is all zero),
codes = OCP e4m3fn(clamp(x / scale, +-448)), rounded to nearest even.

The paged batch lays each request's K/V into a page pool sized 1.25x the
total tokens; pages are handed out in the order of a seeded permutation of
the pool.  Page slots that hold no token are filled with bf16 NaN so that any
read of them shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

SINK_TOKENS = 4
VERTICAL_PERIOD = 4096
DIRECTION_NORM = 3.0
FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic prefill workload (a single attention layer)."""
    name: str
    seqlens: tuple          # one entry per request
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    alphas: tuple           # threshold ratios to run
    seed: int               # single sequence: the seed; batch: base seed (request b uses seed + b)
    verticals: bool
    dtype: str = "bf16"     # "bf16" | "fp8"
    paged: bool = False
    page_size: int = 64
    pool_factor: float = 1.25
    perm_seed: int = 5

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


WORKLOADS: Dict[str, Workload] = {
    # 1 sequence of 1024 tokens, 4 query heads on 1 KV head, d 64, block 64.
    "tiny_s1k_gqa4_d64": Workload("tiny_s1k_gqa4_d64", (1024,), 4, 1, 64, 64,
                                  (0.1,), 1, verticals=False),
    # Llama-3-8B-shaped layer at 32K.
    "llama8b_s32k": Workload("llama8b_s32k", (32768,), 32, 8, 128, 128,
                             (0.1,), 2, verticals=True),
    # Same layer at 128K, threshold ratio swept.
    "llama8b_s128k": Workload("llama8b_s128k", (131072,), 32, 8, 128, 128,
                              (0.05, 0.1, 0.2), 3, verticals=True),
    # The 128K layer quantized to fp8 e4m3 with per-(head, 128-token) scales.
    "llama8b_s128k_fp8": Workload("llama8b_s128k_fp8", (131072,), 32, 8, 128, 128,
                                  (0.1,), 3, verticals=True, dtype="fp8"),
    # Continuous batch of 8 requests over a paged KV cache (page 64 tokens).
    "paged_batch8": Workload("paged_batch8",
                             (4096, 8192, 16384, 16384, 32768, 32768, 65536, 131072),
                             32, 8, 128, 128, (0.1,), 500, verticals=True, paged=True),
}


def positional(seqlen: int, head_dim: int) -> np.ndarray:
    """Sinusoidal term [seqlen, head_dim] (float32), interleaved sin/cos."""
    return _pos_slice(0, seqlen, head_dim)


def _unit_direction(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d, dtype=np.float32).astype(np.float64)
    return (u * (DIRECTION_NORM / np.linalg.norm(u))).astype(np.float32)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> torch.bfloat16 (CPU), round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def make_sequence(seqlen: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  seed: int, verticals: bool, chunk: int = 8192):
    """Q [S,Hq,d], K [S,Hkv,d], V [S,Hkv,d] as CPU bf16 tensors.

    Draws are made in chunks of ``chunk`` tokens; PCG64 normals are consumed
    sequentially, so the result equals one draw of the whole array.
    """
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, d = seqlen, num_q_heads, num_kv_heads, head_dim
    q = torch.empty((S, Hq, d), dtype=torch.bfloat16)
    k32 = np.empty((S, Hkv, d), dtype=np.float32)
    v = torch.empty((S, Hkv, d), dtype=torch.bfloat16)
    for t0 in range(0, S, chunk):
        t1 = min(S, t0 + chunk)
        blk = rng.standard_normal((t1 - t0, Hq, d), dtype=np.float32)
        blk += _pos_slice(t0, t1, d)[:, None, :]
        q[t0:t1] = to_bf16(blk)
    for t0 in range(0, S, chunk):
        t1 = min(S, t0 + chunk)
        k32[t0:t1] = rng.standard_normal((t1 - t0, Hkv, d), dtype=np.float32)
    for t0 in range(0, S, chunk):
        t1 = min(S, t0 + chunk)
        v[t0:t1] = to_bf16(rng.standard_normal((t1 - t0, Hkv, d), dtype=np.float32))
    u = _unit_direction(rng, d)
    w = _unit_direction(rng, d)
    for t0 in range(0, S, chunk):
        t1 = min(S, t0 + chunk)
        k32[t0:t1] += _pos_slice(t0, t1, d)[:, None, :]
    k32[:min(SINK_TOKENS, S)] += u[None, None, :]
    if verticals:
        for t in range(VERTICAL_PERIOD, S, VERTICAL_PERIOD):
            k32[t] += w[None, :]
    k = to_bf16(k32)
    return q, k, v


def _pos_slice(t0: int, t1: int, d: int) -> np.ndarray:
    t = np.arange(t0, t1, dtype=np.float64)[:, None]
    f = np.arange(d // 2, dtype=np.float64)[None, :]
    omega = 10000.0 ** (-2.0 * f / d)
    p = np.empty((t1 - t0, d), dtype=np.float64)
    p[:, 0::2] = np.sin(t * omega)
    p[:, 1::2] = np.cos(t * omega)
    return p.astype(np.float32)


def quantize_fp8_blockwise(x: torch.Tensor, block: int):
    """bf16 [S,H,d] -> (e4m3fn codes as uint8 [S,H,d], fp32 scales [H, nB]).

    One scale per (head, ``block``-token block): amax / 448, or 1 for an
    all-zero block.  Codes are the OCP e4m3fn encoding of clamp(x / scale).
    """
    S, H, d = x.shape
    nB = (S + block - 1) // block
    codes = torch.empty((S, H, d), dtype=torch.uint8)
    scales = torch.empty((H, nB), dtype=torch.float32)
    for J in range(nB):
        t0, t1 = J * block, min(S, (J + 1) * block)
        seg = x[t0:t1].float()                                  # [n, H, d]
        amax = seg.abs().amax(dim=(0, 2))                       # [H]
        sc = torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax))
        scales[:, J] = sc
        y = (seg / sc[None, :, None]).clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX)
        codes[t0:t1] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scales


def fp8_codes_to_float(codes: torch.Tensor) -> torch.Tensor:
    """Decode e4m3fn codes (uint8) to float32 values (exact)."""
    return codes.view(torch.float8_e4m3fn).float()


@dataclasses.dataclass
class PagedBatch:
    seqlens: List[int]
    cu_seqlens: torch.Tensor        # int32 [batch+1]
    q: torch.Tensor                 # bf16 [sum S, Hq, d]
    k_cache: torch.Tensor           # bf16 [num_pages, page, Hkv, d]
    v_cache: torch.Tensor
    block_table: torch.Tensor       # int32 [batch, max_pages_per_seq], -1 where unused
    page_size: int
    requests: list                  # per request (q, k, v) contiguous, for checking


def make_paged_batch(seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                     head_dim: int, seed_base: int, verticals: bool, page_size: int = 64,
                     pool_factor: float = 1.25, perm_seed: int = 5,
                     keep_requests: bool = True) -> PagedBatch:
    """Continuous batch: packed Q and a paged K/V pool with a block table."""
    seqlens = [int(s) for s in seqlens]
    total = sum(seqlens)
    pages_per = [(s + page_size - 1) // page_size for s in seqlens]
    num_pages = max(int(math.ceil(pool_factor * total / page_size)), sum(pages_per))
    perm = np.random.default_rng(perm_seed).permutation(num_pages)
    max_pages = max(pages_per) if pages_per else 1
    block_table = torch.full((len(seqlens), max_pages), -1, dtype=torch.int32)
    k_cache = torch.full((num_pages, page_size, num_kv_heads, head_dim), float("nan"),
                         dtype=torch.bfloat16)
    v_cache = torch.full_like(k_cache, float("nan"))
    q = torch.empty((total, num_q_heads, head_dim), dtype=torch.bfloat16)
    cu = [0]
    requests = []
    nxt = 0
    for b, S in enumerate(seqlens):
        qb, kb, vb = make_sequence(S, num_q_heads, num_kv_heads, head_dim,
                                   seed_base + b, verticals)
        q[cu[-1]:cu[-1] + S] = qb
        pages = perm[nxt:nxt + pages_per[b]]
        nxt += pages_per[b]
        block_table[b, :pages_per[b]] = torch.from_numpy(pages.astype(np.int32))
        for p_i, page in enumerate(pages):
            t0, t1 = p_i * page_size, min(S, (p_i + 1) * page_size)
            k_cache[page, :t1 - t0] = kb[t0:t1]
            v_cache[page, :t1 - t0] = vb[t0:t1]
        cu.append(cu[-1] + S)
        if keep_requests:
            requests.append((qb, kb, vb))
    return PagedBatch(seqlens, torch.tensor(cu, dtype=torch.int32), q, k_cache, v_cache,
                      block_table, page_size, requests)


def workload_inputs(w: Workload, keep_requests: bool = True):
    """Inputs for a named workload: a dict for a single sequence, or a PagedBatch."""
    if w.paged:
        return make_paged_batch(w.seqlens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                w.seed, w.verticals, w.page_size, w.pool_factor,
                                w.perm_seed, keep_requests)
    q, k, v = make_sequence(w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim,
                            w.seed, w.verticals)
    out = {"q": q, "k": k, "v": v}
    if w.dtype == "fp8":
        for name in ("q", "k", "v"):
            c, s = quantize_fp8_blockwise(out[name], w.block_size)
            out[name + "8"] = c
            out[name + "_scale"] = s
    return out

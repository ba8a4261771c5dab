"""Plain CPU oracle for block-sparse causal prefill attention (fp64, NumPy).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The library never calls it, and it
shares no code, table or helper with the HIP path.

What it computes, step by step, in the order the pages give:

1. Block approximation (FlashPrefill, gist.science technical summary,
   section 2.A "Approximation par Blocs"): keys are replaced by their per-block
   mean k_bar; queries are pooled the same way (q_bar), and V is pooled for
   the correction term (step 5).
2. Pooled block logits s[h, I, J] = sigma * q_bar[h, I] . k_bar[h // g, J] for
   J <= I (causal blocks only).
3. Block scores Score[h, I, J] = softmax over J <= I of s[h, I, :].
4. Max-based dynamic threshold (same page, section 2.B, the threshold
   equation): thresh_I = alpha * max_{J <= I} Score[I, J]; block J is kept iff
   Score[I, J] >= thresh_I.  The result is one ascending list of kept KV
   blocks per (query head, query block) (section 2.C, index-based skipping).
5. Attention over the kept blocks with the mean-correction term
   (FlashPrefill V2 abstract, which names the term but prints no formula):
   row i of query block I attends to every token j <= i of the kept blocks,
   and, when the correction is on, to one pooled entry per skipped block
   J < I with logit sigma * q_i . k_bar_J + ln n_J and value v_bar_J (the
   skipped block stands in as n_J copies of its mean key and mean value).
   Output o_i = sum w v / sum w, lse_i = max z + ln sum exp(z - max z).

Readings taken where the pages are silent (listed with reasons in the design
notes): Score is softmax-normalised (3); sigma = 1/sqrt(d) (2); the compare
is inclusive (4); selection is per query head with KV head h // g (2, 4);
partial last blocks average their valid tokens; the correction form (5); a
skipped diagonal block gets no correction entry (its mean mixes future
tokens).  fp8 inputs are judged on their dequantized values.

Chunked prefill (FlashPrefill V2 abstract and the authors' post: the
operator serves continuous batching over a paged KV cache): a call brings q_len new queries at the end of a context of kv_len
tokens whose keys and values are all present.  Blocks are counted from the
start of the context and row i of the chunk sits at position P0 + i, P0 =
kv_len - q_len (bottom-right causal alignment).  Query block I >= first =
floor(P0 / block) holds the chunk's queries in [I block, (I + 1) block) and
sees blocks J <= I; its q_bar is the mean of the queries it holds, so a block
the chunk enters part way pools only the chunk's queries (the earlier queries
of that block belong to an earlier call).  Keys are pooled over whole context
blocks.  When the chunk starts on a block boundary its result equals the last
q_len rows of the full prefill; otherwise every row past the first query
block still does.  Skeleton queries need a chunk that starts on a boundary.

Group-shared selection (an option, not in the pages; it serves the
PackGQA-style head packing the V2 abstract names): the g query heads of a KV
head share one list, so every head of a packed group computes on every tile
fetched for it.  Two ways to form it: the union of the heads' own lists, or
one list scored from the group-pooled query (the mean of the g heads' block
means, i.e. the mean over the group's heads and the block's tokens) against
the KV head's k_bar, thresholded as in steps 2-4.

Skeleton-query scoring (FlashPrefill, gist.science technical summary,
section 2.A: attention patterns can be found from a skeleton set of
uniformly spaced queries): optionally each query block is represented by its
queries at offsets 0, st, 2 st, ... (st = block / P, P the probe count), whose
mean replaces q_bar in step 2; P = block is the plain block mean.

Pins (tests/test_oracle.py): alpha = 0 reduces to dense causal attention
computed by an independent routine; masks equal brute-force per-block scoring
on tiny inputs; every probability row sums to 1; the correction equals dense
attention in closed form when K and V are constant within blocks; constant V
gives constant output; the argmax block is always kept and masks nest in
alpha; GQA equals MHA with repeated K/V; a varlen batch equals its requests;
a chunk equals per-token brute force written from positions, and the last
rows of the full prefill; the chunk's fp8 query codes equal the blockwise
quantizer when the chunk starts on a block boundary, and each query block's
codes and scale come from exactly the chunk rows whose positions fall in it.  The correction's definition itself is a reading, not a formula from the pages;
only its implementation under that reading is pinned.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

BAND_REL = 1e-3   # blocks whose score lies within this relative distance of the threshold


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def num_blocks(seqlen: int, block: int) -> int:
    return (seqlen + block - 1) // block


def block_lengths(seqlen: int, block: int) -> np.ndarray:
    """n_J: tokens in block J (block, except for a partial last block)."""
    nB = num_blocks(seqlen, block)
    return np.array([min(block, seqlen - J * block) for J in range(nB)], dtype=np.int64)


def block_means(x, block: int, stride: int = 1) -> np.ndarray:
    """Per-block mean over the valid tokens.  x [S, H, d] -> [H, nB, d] (fp64).

    stride > 1 averages only the block's tokens at offsets 0, stride,
    2 stride, ... (the skeleton queries; a partial block keeps those it has).
    """
    S, H, d = x.shape
    nB = num_blocks(S, block)
    out = np.empty((H, nB, d), dtype=np.float64)
    for J in range(nB):
        seg = _f64(x[J * block:min(S, (J + 1) * block):stride])   # [n_J / stride, H, d]
        out[:, J, :] = seg.mean(axis=0)
    return out


def causal_blocks(nq: int, nB: int, first: int = 0) -> np.ndarray:
    """[nq, nB]: query block first + i may see KV blocks J <= first + i."""
    return np.arange(nB)[None, :] <= (first + np.arange(nq))[:, None]


def chunk_block_means(q, block: int, P0: int, stride: int = 1) -> np.ndarray:
    """Query block means of a chunk whose row r is position P0 + r.

    q [q_len, H, d] -> [H, n, d] for query blocks first .. first + n - 1,
    first = P0 // block: block I averages the chunk's rows at positions
    [max(I block, P0), min((I + 1) block, P0 + q_len)).  stride > 1 (skeleton
    queries) requires P0 to be a multiple of the block.
    """
    q_len, H, d = q.shape
    if stride > 1 and P0 % block:
        raise ValueError("skeleton queries need a chunk that starts on a block boundary")
    if q_len == 0:
        return np.empty((H, 0, d), dtype=np.float64)
    first, last = P0 // block, (P0 + q_len - 1) // block
    out = np.empty((H, last - first + 1, d), dtype=np.float64)
    for i, I in enumerate(range(first, last + 1)):
        r0 = max(I * block, P0) - P0
        r1 = min((I + 1) * block, P0 + q_len) - P0
        out[:, i, :] = _f64(q[r0:r1:stride]).mean(axis=0)
    return out


def block_logits(q_bar: np.ndarray, k_bar: np.ndarray, sigma: float, first: int = 0) -> np.ndarray:
    """s[h, i, J] = sigma * q_bar[h, i] . k_bar[h // g, J] for J <= first + i; -inf above.

    Row i is query block first + i (first = 0 for a whole sequence).
    """
    Hq, nq, _ = q_bar.shape
    Hkv, nB, _ = k_bar.shape
    g = Hq // Hkv
    causal = causal_blocks(nq, nB, first)
    s = np.full((Hq, nq, nB), -np.inf)
    for h in range(Hq):
        full = sigma * (q_bar[h] @ k_bar[h // g].T)
        s[h] = np.where(causal, full, -np.inf)
    return s


def block_scores(s: np.ndarray) -> np.ndarray:
    """Score[h, I, J] = softmax over the causal blocks J <= I of s[h, I, :]."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)                      # exp(-inf) = 0 above the diagonal
    return e / e.sum(axis=-1, keepdims=True)


def threshold(score: np.ndarray, alpha: float, first: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """keep = Score >= alpha * max_{J<=I} Score over causal blocks.

    Also returns the band flags: causal blocks whose score lies within
    BAND_REL relative of the threshold (only meaningful for alpha > 0).
    Row i is query block first + i.
    """
    nq, nB = score.shape[-2:]
    causal = causal_blocks(nq, nB, first)[None]
    thresh = alpha * score.max(axis=-1, keepdims=True)
    keep = causal & (score >= thresh)
    if alpha > 0:
        band = causal & (np.abs(score - thresh) <= BAND_REL * thresh)
    else:
        band = np.zeros_like(keep)
    return keep, band


class Selection:
    """Everything the selection step produces for one sequence."""

    def __init__(self, q_bar, k_bar, v_bar, s, score, keep, band, block, first=0):
        self.q_bar, self.k_bar, self.v_bar = q_bar, k_bar, v_bar
        self.s, self.score, self.keep, self.band = s, score, keep, band
        self.block = block
        self.first = first     # query block of row 0 (chunked prefill), else 0

    def lists(self) -> List[List[np.ndarray]]:
        """Kept KV blocks per (query head, query block row), ascending."""
        Hq, nq, _ = self.keep.shape
        return [[np.flatnonzero(self.keep[h, i, :self.first + i + 1]) for i in range(nq)]
                for h in range(Hq)]


def share_across_group(keep: np.ndarray, band: np.ndarray, g: int) -> Tuple[np.ndarray, np.ndarray]:
    """Group-shared selection: the g query heads of a KV head share one mask,
    the union of their own masks (a block any of them keeps is kept for all).
    A union entry is flagged near-threshold when any head's entry is."""
    Hq = keep.shape[0]
    shp = (Hq // g, g) + keep.shape[1:]
    ku = keep.reshape(shp).any(axis=1)
    bu = band.reshape(shp).any(axis=1)
    return np.repeat(ku, g, axis=0), np.repeat(bu, g, axis=0)


def group_pooled_queries(q_bar: np.ndarray, g: int) -> np.ndarray:
    """[Hq, nq, d] block means -> [Hq / g, nq, d]: each KV head's row is the
    mean of its g query heads' rows (heads hk*g .. hk*g + g - 1)."""
    Hq, nq, d = q_bar.shape
    return q_bar.reshape(Hq // g, g, nq, d).mean(axis=1)


def _shared_mode(shared) -> str:
    """shared: False / None (per head), True or 'union', or 'pooled'."""
    if shared is False or shared is None:
        return "none"
    if shared is True or shared == "union":
        return "union"
    if shared == "pooled":
        return "pooled"
    raise ValueError(f"unknown group-shared selection {shared!r}")


def _select(q_bar, k_bar, sigma, alpha, first, mode):
    """Steps 2-4 on given means: logits, scores, keep and band per query head."""
    Hq, Hkv = q_bar.shape[0], k_bar.shape[0]
    g = Hq // Hkv
    if mode == "pooled":
        s = np.repeat(block_logits(group_pooled_queries(q_bar, g), k_bar, sigma, first), g, axis=0)
    else:
        s = block_logits(q_bar, k_bar, sigma, first)
    score = block_scores(s)
    keep, band = threshold(score, alpha, first)
    if mode == "union":
        keep, band = share_across_group(keep, band, g)
    return s, score, keep, band


def probe_stride(block: int, probes: int) -> int:
    """Token stride of the skeleton queries: block / probes (1 when probes is 0)."""
    if probes == 0:
        return 1
    if probes < 0 or block % probes:
        raise ValueError("probes must divide the block size")
    return block // probes


def select_blocks(q, k, v, block: int, alpha: float, sigma: Optional[float] = None,
                  pool_v: bool = True, shared=False, probes: int = 0) -> Selection:
    """Pooling, block scores and thresholding for one sequence.

    q [S, Hq, d], k and v [S, Hkv, d] (any float dtype; upcast to fp64).
    shared: False, per query head; True or 'union', one mask per KV head, the
    union over its query heads; 'pooled', one mask per KV head scored from
    the group-pooled query (s, score and band are then per KV head, repeated
    over its query heads).
    probes: 0, or P dividing the block: q_bar averages the skeleton queries
    at every (block / P)-th token of the block instead of all its tokens.
    """
    d = q.shape[-1]
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    q_bar = block_means(q, block, probe_stride(block, probes))
    k_bar = block_means(k, block)
    v_bar = block_means(v, block) if pool_v else None
    s, score, keep, band = _select(q_bar, k_bar, sigma, alpha, 0, _shared_mode(shared))
    return Selection(q_bar, k_bar, v_bar, s, score, keep, band, block)


def block_entries(q, k, v, keep_row: np.ndarray, h: int, I: int, block: int, sigma: float,
                  g: int, correction: bool, k_bar=None, v_bar=None, q_offset: int = 0):
    """Logits z [n_I, n_entries] and values [n_entries, d] for query block I of head h.

    Entries: the tokens of every kept block J <= I (token j masked to -inf for
    rows i < j), then, with the correction, one pooled entry per skipped J < I.
    Positions count from the start of the keys; q row r holds position
    r + q_offset (q_offset > 0 for a chunk at the end of a longer context).
    """
    S = k.shape[0]
    hk = h // g
    r0, r1 = max(I * block, q_offset), min(S, (I + 1) * block)
    rows = np.arange(r0, r1)
    q_i = _f64(q[r0 - q_offset:r1 - q_offset, h])              # [n_I, d]
    kept = [J for J in range(I + 1) if keep_row[J]]
    if kept:
        tok = np.concatenate([np.arange(J * block, min(S, (J + 1) * block)) for J in kept])
    else:
        tok = np.zeros(0, dtype=np.int64)
    z = sigma * (q_i @ _f64(k[tok, hk]).T)                      # [n_I, n_tok]
    z[tok[None, :] > rows[:, None]] = -np.inf                  # causal inside block I
    vals = _f64(v[tok, hk])
    if correction:
        skipped = [J for J in range(I) if not keep_row[J]]
        if skipped:
            n = block_lengths(S, block)[skipped].astype(np.float64)
            zc = sigma * (q_i @ k_bar[hk, skipped].T) + np.log(n)[None, :]
            z = np.concatenate([z, zc], axis=1)
            vals = np.concatenate([vals, v_bar[hk, skipped]], axis=0)
    return z, vals


def softmax_rows(z: np.ndarray):
    """Row softmax pieces: (max M, weights exp(z - M), row sums l)."""
    M = z.max(axis=1, keepdims=True)
    w = np.exp(z - M)
    return M[:, 0], w, w.sum(axis=1)


def sparse_attention(q, k, v, sel: Selection, correction: bool, sigma: Optional[float] = None,
                     pairs: Optional[Iterable[Tuple[int, int]]] = None,
                     keep: Optional[np.ndarray] = None):
    """Attention over the kept blocks (plus the correction entries).

    Returns o [S, Hq, d] and lse [Hq, S] (fp64); rows of (head, query block)
    pairs not listed in ``pairs`` stay NaN.  ``keep`` overrides the selection's
    mask (used to evaluate under a mask produced elsewhere).
    """
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    block = sel.block
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    keep = sel.keep if keep is None else keep
    nB = num_blocks(S, block)
    if pairs is None:
        pairs = [(h, I) for h in range(Hq) for I in range(nB)]
    o = np.full((S, Hq, d), np.nan)
    lse = np.full((Hq, S), np.nan)
    for h, I in pairs:
        z, vals = block_entries(q, k, v, keep[h, I], h, I, block, sigma, g, correction,
                                sel.k_bar, sel.v_bar)
        M, w, l = softmax_rows(z)
        r0, r1 = I * block, min(S, (I + 1) * block)
        o[r0:r1, h] = (w @ vals) / l[:, None]
        lse[h, r0:r1] = M + np.log(l)
    return o, lse


def select_blocks_chunked(q, k, v, block: int, alpha: float, sigma: Optional[float] = None,
                          pool_v: bool = True, shared=False, probes: int = 0) -> Selection:
    """Pooling, block scores and thresholding for a chunk of new queries.

    q [q_len, Hq, d] are the last q_len tokens of a context whose keys and
    values are k, v [kv_len, Hkv, d]; the chunk may start inside a block
    (not with skeleton queries).  Row i of the result is query block first + i,
    first = (kv_len - q_len) // block (no rows for an empty chunk); keys are
    pooled over the whole context.
    """
    q_len, kv_len = q.shape[0], k.shape[0]
    if not 0 <= q_len <= kv_len:
        raise ValueError(f"chunk of {q_len} queries for a context of {kv_len} tokens")
    d = q.shape[-1]
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    P0 = kv_len - q_len
    first = P0 // block if q_len else num_blocks(kv_len, block)
    q_bar = chunk_block_means(q, block, P0, probe_stride(block, probes))
    k_bar = block_means(k, block)
    v_bar = block_means(v, block) if pool_v else None
    s, score, keep, band = _select(q_bar, k_bar, sigma, alpha, first, _shared_mode(shared))
    return Selection(q_bar, k_bar, v_bar, s, score, keep, band, block, first)


def sparse_attention_chunked(q, k, v, sel: Selection, correction: bool, sigma: Optional[float] = None,
                             keep: Optional[np.ndarray] = None,
                             pairs: Optional[Iterable[Tuple[int, int]]] = None):
    """Attention of a chunk (see select_blocks_chunked): o [q_len, Hq, d], lse [Hq, q_len].

    Row r of the chunk is position kv_len - q_len + r and sees every key at or
    before it in the kept blocks, plus the correction entries.  ``pairs``
    (head, i) limits the work to query blocks first + i of those heads; other
    rows stay NaN.
    """
    q_len, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    block = sel.block
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    keep = sel.keep if keep is None else keep
    P0 = k.shape[0] - q_len
    o = np.full((q_len, Hq, d), np.nan)
    lse = np.full((Hq, q_len), np.nan)
    if pairs is None:
        pairs = [(h, i) for h in range(Hq) for i in range(keep.shape[1])]
    for h, i in pairs:
        I = sel.first + i
        z, vals = block_entries(q, k, v, keep[h, i], h, I, block, sigma, g, correction,
                                sel.k_bar, sel.v_bar, q_offset=P0)
        M, w, l = softmax_rows(z)
        r0, r1 = max(I * block, P0) - P0, min(k.shape[0], (I + 1) * block) - P0
        o[r0:r1, h] = (w @ vals) / l[:, None]
        lse[h, r0:r1] = M + np.log(l)
    return o, lse


def attention_probabilities(q, k, v, sel: Selection, correction: bool, h: int, I: int,
                            sigma: Optional[float] = None) -> np.ndarray:
    """Normalised weights of every entry for the rows of query block I of head h."""
    d = q.shape[-1]
    g = q.shape[1] // k.shape[1]
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    z, _ = block_entries(q, k, v, sel.keep[h, I], h, I, sel.block, sigma, g, correction,
                         sel.k_bar, sel.v_bar)
    _, w, l = softmax_rows(z)
    return w / l[:, None]


E4M3_MAX = 448.0


def e4m3_encode(y) -> np.ndarray:
    """OCP FP8 E4M3 ("fn") codes of fp32 values within [-448, 448].

    Written from the format: sign bit, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the
    largest finite value is 1.75 * 2^8 = 448 (code 0x7e; 0x7f is NaN).  The
    magnitude is rounded to the nearest representable value, ties to the
    even mantissa.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)     # exact
    if np.any(np.abs(y) > E4M3_MAX) or np.any(~np.isfinite(y)):
        raise ValueError("e4m3_encode takes finite values within [-448, 448]")
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    _, E = np.frexp(a)                                       # a = m 2^E, m in [0.5, 1)
    e = np.maximum(E - 1, -6)                                # below 2^-6 the spacing stays 2^-9
    step = np.ldexp(1.0, e - 3)                              # spacing of representable values
    v = np.round(a / step) * step                            # exact quotient; round half to even
    _, E2 = np.frexp(v)
    normal = v >= 2.0 ** -6
    ef = np.where(normal, E2 - 1 + 7, 0)
    mant = np.where(normal, v / np.ldexp(1.0, E2 - 1) - 1.0, v / 2.0 ** -9)
    mant = np.where(normal, mant * 8.0, mant)
    return (sign | (ef.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Values of finite E4M3 codes (fp64)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef, m = (c >> 3) & 15, c & 7
    return s * np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))


def quantize_fp8_blockwise(x, block: int):
    """Codes and scales for fp8 inputs (reading R10): per (head, block) the
    scale is amax / 448 in fp32 (1 for an all-zero block); the codes are the
    E4M3 rounding of clamp(x / scale, -448, 448), the division in fp32, so
    every integer decision is taken in the same precision as on the GPU.
    x [S, H, d] -> (codes uint8 [S, H, d], scales fp32 [H, nB])."""
    x32 = np.asarray(x, dtype=np.float32)
    S, H, d = x32.shape
    nB = num_blocks(S, block)
    codes = np.empty((S, H, d), dtype=np.uint8)
    scales = np.empty((H, nB), dtype=np.float32)
    for J in range(nB):
        seg = x32[J * block:min(S, (J + 1) * block)]
        amax = np.abs(seg).max(axis=(0, 2))
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, J] = sc
        y = np.clip(seg / sc[None, :, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
        codes[J * block:min(S, (J + 1) * block)] = e4m3_encode(y)
    return codes, scales


def quantize_fp8_chunk(q, block: int, P0: int):
    """Codes and scales of a chunk's queries for fp8 chunked prefill (reading
    R10 applied to the chunk's query blocks): row r is position P0 + r, and
    query block I holds the chunk's rows at positions
    [max(I block, P0), min((I + 1) block, P0 + q_len)); each (head, query
    block) gets scale amax / 448 over those rows (1 if all zero) and codes
    E4M3(clamp(x / scale)), the division in fp32.
    q [q_len, H, d] -> (codes uint8 [q_len, H, d], scales fp32 [H, n]) for
    query blocks first .. first + n - 1, first = P0 // block."""
    x32 = np.asarray(q, dtype=np.float32)
    q_len, H, d = x32.shape
    codes = np.empty((q_len, H, d), dtype=np.uint8)
    if q_len == 0:
        return codes, np.empty((H, 0), dtype=np.float32)
    first, last = P0 // block, (P0 + q_len - 1) // block
    scales = np.empty((H, last - first + 1), dtype=np.float32)
    for i, I in enumerate(range(first, last + 1)):
        r0 = max(I * block, P0) - P0
        r1 = min((I + 1) * block, P0 + q_len) - P0
        seg = x32[r0:r1]
        amax = np.abs(seg).max(axis=(0, 2))
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, i] = sc
        y = np.clip(seg / sc[None, :, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
        codes[r0:r1] = e4m3_encode(y)
    return codes, scales


def dequantize_chunk(codes_value, scales, block: int, P0: int) -> np.ndarray:
    """x = x8 * scale[h, I - first] for a chunk's fp8 values (row r at position P0 + r)."""
    x8 = _f64(codes_value)
    I = (P0 + np.arange(x8.shape[0])) // block - P0 // block
    return x8 * _f64(scales)[:, I].T[:, :, None]


def dequantize_blockwise(codes_value, scales, block: int) -> np.ndarray:
    """x = x8 * scale[h, t // block] for fp8 values decoded to float ([S, H, d])."""
    x8 = _f64(codes_value)
    S = x8.shape[0]
    sc = _f64(scales)                                           # [H, nB]
    idx = np.arange(S) // block
    return x8 * sc[:, idx].T[:, :, None]


def flops_executed(sel: Selection, seqlen: int, head_dim: int, correction: bool,
                   keep: Optional[np.ndarray] = None) -> Tuple[float, float]:
    """Algorithmic work: (F_kept, F_corr).

    F_kept = 4 d sum over kept (h, I, J) of n_I n_J (diagonal tile counted in
    full); F_corr = 4 d sum over (h, I) of n_I * |skipped J < I|.
    """
    keep = sel.keep if keep is None else keep
    n = block_lengths(seqlen, sel.block).astype(np.float64)
    f_kept = 4.0 * head_dim * float(np.einsum("hij,i,j->", keep.astype(np.float64), n, n))
    f_corr = 0.0
    if correction:
        nB = len(n)
        strict = np.tril(np.ones((nB, nB), dtype=bool), -1)[None]
        skipped = (strict & ~keep).sum(axis=2).astype(np.float64)   # [Hq, nB]
        f_corr = 4.0 * head_dim * float((skipped * n[None, :]).sum())
    return f_kept, f_corr

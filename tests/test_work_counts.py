"""Pins for the work counts the measurement rests on (no GPU).

The effective TFLOP/s of every bench figure divides an algorithmic FLOP count
by a time.  Three implementations produce that count: the oracle's
flops_executed (from a keep mask), the benchmark's work_counts (from the
device lists of one sequence) and its list_work (kept and skipped block counts
from the lists of a paged or chunked batch).  Each is checked here against a
count written per query token with plain loops:

  a query token i of block I executes, for every kept block J <= I, the n_J
  keys of that block (the diagonal tile is executed in full, so J = I counts
  n_I keys, not only those at or before i), and, with the correction on, one
  pooled entry for every skipped block J < I (a skipped diagonal has none:
  its mean mixes future tokens).  Each key or entry costs 2 d FLOP for q.k and
  2 d for p.v (FlashPrefill, gist.science technical summary, section 2.B:
  the threshold fixes what is kept and so what is skipped; 2.C: skipped
  blocks are never touched).

The masks include partial last blocks and skipped diagonal blocks, so
counting the skipped diagonal, using n_J for n_I, or counting the diagonal
tile only up to the token, each fails a test below.
"""
import math

import numpy as np
import pytest
import torch

import bench
import oracle as O


def _loop_flops(keep, S, B, d, correction, P0=0, q_len=None):
    """(F_kept, F_corr) by a per-token loop.  keep [Hq, nq, nB] for query
    blocks first .. first + nq - 1 of a context of S tokens whose last q_len
    tokens (from position P0) are the queries."""
    Hq, nq, nB = keep.shape
    q_len = S - P0 if q_len is None else q_len
    first = P0 // B
    n = [min(B, S - J * B) for J in range(nB)]
    fk = fc = 0
    for h in range(Hq):
        for pos in range(P0, P0 + q_len):
            I = pos // B
            row = keep[h, I - first]
            for J in range(I + 1):
                if row[J]:
                    fk += n[J]
                elif J < I and correction:
                    fc += 1
    return 4.0 * d * fk, 4.0 * d * fc


def _random_mask(Hq, nB, seed, p_keep, first=0, force_skip_diag=True):
    """Random causal mask, every row non-empty; with force_skip_diag some
    rows keep an earlier block but not their diagonal."""
    r = np.random.default_rng(seed)
    nq = nB - first
    keep = np.zeros((Hq, nq, nB), dtype=bool)
    for h in range(Hq):
        for i in range(nq):
            I = first + i
            row = r.random(I + 1) < p_keep
            if not row.any():
                row[r.integers(0, I + 1)] = True
            keep[h, i, :I + 1] = row
    if force_skip_diag:
        for h in range(Hq):
            for i in range(nq):
                I = first + i
                if I > 0 and (h + i) % 3 == 0:
                    keep[h, i, I] = False
                    keep[h, i, r.integers(0, I)] = True
    return keep


def _sink_dominated(S, Hq, Hkv, d, seed):
    """Queries and the sink keys share one strong direction, so block 0
    outscores the diagonal block and thresholds skip diagonals."""
    r = np.random.default_rng(seed)
    u = r.standard_normal(d)
    u *= 4.0 / np.linalg.norm(u)
    q = r.standard_normal((S, Hq, d)) * 0.5 + u
    k = r.standard_normal((S, Hkv, d)) * 0.5
    k[:4] += 8 * u
    v = r.standard_normal((S, Hkv, d))
    return q, k, v


def _layout(keeps, lens, starts, B):
    """Device list layout of per-request masks: request regions follow each
    other; row (h, I) of a request starts at h (tri(nb) - tri(first)) +
    tri(I) - tri(first), capacity I + 1; counts [Hq, nb - first] per
    request.  Unused capacity holds -1."""
    tri = lambda n: n * (n + 1) // 2
    idx, cnt = [], []
    for keep, L, P0 in zip(keeps, lens, starts):
        Hq, nq, nb = keep.shape
        first = P0 // B
        assert nq == nb - first
        reg = np.full(Hq * (tri(nb) - tri(first)), -1, dtype=np.int32)
        c = np.zeros((Hq, nq), dtype=np.int32)
        for h in range(Hq):
            for i in range(nq):
                I = first + i
                js = [J for J in range(I + 1) if keep[h, i, J]]
                o = h * (tri(nb) - tri(first)) + tri(I) - tri(first)
                reg[o:o + len(js)] = js
                c[h, i] = len(js)
        idx.append(reg)
        cnt.append(c.reshape(-1))
    return torch.from_numpy(np.concatenate(idx)), torch.from_numpy(np.concatenate(cnt))


class _Sel:
    def __init__(self, kv_idx, kv_cnt, Hq, nB):
        self.kv_idx = kv_idx
        self.kv_cnt = kv_cnt.view(Hq, nB)


# ------------------------------------------------------- oracle flops_executed

@pytest.mark.parametrize("alpha", [0.1, 0.5, 1.0])
@pytest.mark.parametrize("S,B", [(200, 32), (256, 64), (97, 16)])
def test_flops_executed_matches_token_loop(alpha, S, B):
    d, Hq, Hkv = 8, 4, 2
    q, k, v = _sink_dominated(S, Hq, Hkv, d, seed=S + B)
    sel = O.select_blocks(q, k, v, B, alpha)
    nB = O.num_blocks(S, B)
    if alpha >= 0.5:
        diag = sel.keep[:, np.arange(1, nB), np.arange(1, nB)]
        assert not diag.all(), "the inputs must skip some diagonal blocks"
    for corr in (False, True):
        fk, fc = O.flops_executed(sel, S, d, corr)
        ek, ec = _loop_flops(sel.keep, S, B, d, corr)
        assert fk == ek and fc == ec, (fk, ek, fc, ec)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flops_executed_random_masks(seed):
    S, B, d, Hq = 150, 32, 16, 3
    nB = O.num_blocks(S, B)
    keep = _random_mask(Hq, nB, seed, p_keep=0.4)
    q, k, v = _sink_dominated(S, Hq, 1, d, seed)
    sel = O.select_blocks(q, k, v, B, 0.3)
    fk, fc = O.flops_executed(sel, S, d, True, keep=keep)
    assert (fk, fc) == _loop_flops(keep, S, B, d, True)


# ----------------------------------------------------------- Selection.lists

@pytest.mark.parametrize("P0", [0, 32, 45])
def test_selection_lists_from_mask_loop(P0):
    S, B = 160, 16
    q, k, v = _sink_dominated(S, 4, 2, 8, seed=P0)
    sel = O.select_blocks_chunked(q[P0:], k, v, B, 0.4) if P0 else O.select_blocks(q, k, v, B, 0.4)
    lists = sel.lists()
    Hq, nq, nB = sel.keep.shape
    assert len(lists) == Hq and all(len(l) == nq for l in lists)
    for h in range(Hq):
        for i in range(nq):
            I = sel.first + i
            expect = []
            for J in range(nB):
                if J <= I and sel.keep[h, i, J]:
                    expect.append(J)
            assert list(lists[h][i]) == expect


# ------------------------------------------------------------ bench counters

@pytest.mark.parametrize("S,B", [(200, 32), (256, 64), (1000, 128)])
@pytest.mark.parametrize("source", ["oracle", "random"])
def test_bench_work_counts(S, B, source):
    d, Hq, Hkv = 16, 4, 2
    nB = O.num_blocks(S, B)
    if source == "oracle":
        q, k, v = _sink_dominated(S, Hq, Hkv, d, seed=S)
        keep = O.select_blocks(q, k, v, B, 0.5).keep
    else:
        keep = _random_mask(Hq, nB, S, p_keep=0.3)
    kv_idx, kv_cnt = _layout([keep], [S], [0], B)
    for corr in (False, True):
        fk, fc, kept = bench.work_counts(None, _Sel(kv_idx, kv_cnt, Hq, nB), S, Hq, d, B, corr)
        ek, ec = _loop_flops(keep, S, B, d, corr)
        assert kept == int(keep.sum())
        assert (fk, fc) == (ek, ec)


@pytest.mark.parametrize("chunk", [None, 64, 200])
def test_bench_list_work(chunk):
    """list_work's kept / skipped counts on a batch of requests (whole
    prompts, or the last `chunk` tokens of each context new, chunk a multiple
    of the block or not), and the bench's FLOP formula for full blocks."""
    B, d, Hq, Hkv = 32, 8, 4, 2
    lens = [256, 96, 320, 32]
    keeps, starts = [], []
    for b, L in enumerate(lens):
        q, k, v = _sink_dominated(L, Hq, Hkv, d, seed=10 + b)
        P0 = 0 if chunk is None else max(0, L - chunk)
        sel = (O.select_blocks_chunked(q[P0:], k, v, B, 0.3) if P0 else O.select_blocks(q, k, v, B, 0.3))
        keeps.append(sel.keep)
        starts.append(P0)
    kv_idx, kv_cnt = _layout(keeps, lens, starts, B)
    kept, skipped = bench.list_work(kv_idx, kv_cnt, lens, starts, Hq, B, torch.device("cpu"))
    e_kept = sum(int(kp.sum()) for kp in keeps)
    e_skip = 0
    for kp, L, P0 in zip(keeps, lens, starts):
        first = P0 // B
        for h in range(kp.shape[0]):
            for i in range(kp.shape[1]):
                I = first + i
                e_skip += sum(1 for J in range(I) if not kp[h, i, J])
    assert (kept, skipped) == (e_kept, e_skip)
    if chunk is None or chunk % B == 0:
        # every length is a multiple of B and every chunk starts on a block
        # boundary: the bench's 4 d B (B kept + skipped) is the token loop's count
        f = 4.0 * d * B * (B * kept + skipped)
        loop = [sum(_loop_flops(kp, L, B, d, True, P0=P0)) for kp, L, P0 in zip(keeps, lens, starts)]
        assert f == sum(loop)
        if chunk is None:
            fo = sum(sum(O.flops_executed(O.Selection(None, None, None, None, None, kp, None, B), L, d, True))
                     for kp, L in zip(keeps, lens))
            assert f == fo

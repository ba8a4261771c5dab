"""Parity of the chunked-prefill entry (new queries at the end of a context
whose K/V are in a paged cache) with the CPU oracle, bit-identity with the
last rows of the whole-prompt entry, and the pooled-means cache across calls.
Unused page slots hold NaN, so a read outside a context shows."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import BF16_TOL, LSE_TOL, compare_mask, dev

pytestmark = pytest.mark.gpu

CASES = [
    # context lengths, chunk starts (multiples of B), Hq, Hkv, d, B, page
    ([300, 1024, 77, 2048], [128, 0, 0, 1536], 8, 2, 128, 128, 64),
    ([640, 129, 255, 64], [256, 64, 192, 64], 4, 1, 64, 64, 16),     # last request: empty chunk
    ([4096, 1000, 2000], [3968, 512, 1024], 32, 8, 128, 128, 64),
]
# Chunks that start inside a block: the first query block holds only the
# chunk's tail of it (one row, for starts at B - 1 or at the last token).
UNALIGNED = [
    ([300, 1024, 777, 2048], [131, 5, 700, 1677], 8, 2, 128, 128, 64),
    ([640, 129, 255, 100], [250, 63, 1, 100], 4, 1, 64, 64, 16),   # last: empty chunk ending mid-block
    ([4096, 1000, 2000], [4095, 999, 1030], 32, 8, 128, 128, 64),  # single-token chunks
]


def _case_id(c):
    aligned = all(P0 % c[5] == 0 for P0 in c[1])
    return "b%d_d%d_B%d_p%d%s" % (len(c[0]), c[4], c[5], c[6], "" if aligned else "_unaligned")


def _tri(n):
    return n * (n + 1) // 2


def _chunks(pb, starts):
    """The chunks' queries packed back to back, cu_seqlens_q, context lengths."""
    parts, cu = [], [0]
    for b, P0 in enumerate(starts):
        qb = pb.requests[b][0][P0:]
        parts.append(qb)
        cu.append(cu[-1] + qb.shape[0])
    return torch.cat(parts), cu, [int(x) for x in pb.seqlens]


def _run(pb, q, cu, kv_lens, Hq, Hkv, d, B, alpha, corr, cache=None, reuse=False):
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    res = fp.fp_sparse_prefill_chunked_paged(p, q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                             pb.block_table.to(dev()), cu, kv_lens, pooled_cache=cache,
                                             prefix_pooled=reuse, return_lse=True)
    torch.cuda.synchronize()
    return res


def _masks(res, Hq, kv_lens, starts, B):
    """Per request the [Hq, nq, nb] mask read from the chunk-layout lists, which
    must be ascending, causal and non-empty."""
    idx = res.kv_idx.cpu().numpy()
    cnt = res.kv_cnt.cpu().numpy()
    io = co = 0
    masks = []
    for L, P0 in zip(kv_lens, starts):
        nb = (L + B - 1) // B
        first = P0 // B if P0 < L else nb
        nq, rowsz = nb - first, _tri(nb) - _tri(first)
        m = np.zeros((Hq, nq, nb), dtype=bool)
        for h in range(Hq):
            for i in range(nq):
                I = first + i
                c = int(cnt[co + h * nq + i])
                assert 1 <= c <= I + 1, (h, I, c)
                s0 = io + h * rowsz + _tri(I) - _tri(first)
                lst = idx[s0:s0 + c]
                assert np.all(np.diff(lst) > 0) and lst[0] >= 0 and lst[-1] <= I, (h, I, lst)
                m[h, i, lst] = True
        masks.append(m)
        io += Hq * rowsz
        co += Hq * nq
    assert io == res.kv_idx.numel() or io == 0
    return masks


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.4])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("case", CASES + UNALIGNED, ids=_case_id)
def test_chunked_matches_oracle(case, alpha, corr):
    lengths, starts, Hq, Hkv, d, B, page = case
    print(f"chunked {case} alpha={alpha} corr={corr}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=300 + len(lengths), verticals=True,
                                page_size=page)
    q, cu, kv_lens = _chunks(pb, starts)
    res = _run(pb, q, cu, kv_lens, Hq, Hkv, d, B, alpha, corr)
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    masks = _masks(res, Hq, kv_lens, starts, B)
    for b, (L, P0) in enumerate(zip(kv_lens, starts)):
        if L == P0:
            continue
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        ref = O.select_blocks_chunked(qb[P0:], kb, vb, B, alpha)
        outside, inside, band = compare_mask(masks[b], ref)
        assert outside == 0, (b, outside, inside, band)
        o_ref, lse_ref = O.sparse_attention_chunked(qb[P0:], kb, vb, ref, corr, keep=masks[b])
        err = np.abs(out[cu[b]:cu[b + 1]] - o_ref).max()
        lerr = np.abs(lse[:, cu[b]:cu[b + 1]] - lse_ref).max()
        print(f"  request {b} kv={L} chunk={L - P0}: kept {int(masks[b].sum())} err {err:.3e} lse {lerr:.3e}",
              flush=True)
        assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("case", CASES[:2] + UNALIGNED, ids=_case_id)
def test_chunked_equals_last_rows_of_whole_prompt(case):
    """Chunks give bit-identical rows to the whole-prompt entry: same pooled
    sums, same lists, same tiles in order.  A chunk that starts inside a
    block pools fewer queries there, so that block's rows are left out."""
    lengths, starts, Hq, Hkv, d, B, page = case
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=41, verticals=True, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True)
    full = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                             pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    q, cu, kv_lens = _chunks(pb, starts)
    res = _run(pb, q, cu, kv_lens, Hq, Hkv, d, B, 0.2, True)
    for b, P0 in enumerate(starts):
        skip = min(-P0 % B, cu[b + 1] - cu[b])             # rows of a block the chunk enters part way
        f0 = int(pb.cu_seqlens[b]) + P0 + skip
        f1 = int(pb.cu_seqlens[b + 1])
        assert torch.equal(res.out[cu[b] + skip:cu[b + 1]], full.out[f0:f1]), b
        assert torch.equal(res.lse[:, cu[b] + skip:cu[b + 1]], full.lse[:, f0:f1]), b


@pytest.mark.parametrize("cut", [[1024, 384], [1000, 333]], ids=["aligned", "unaligned"])
def test_pooled_cache_carries_the_prefix_between_calls(cut):
    """Two calls over the same contexts: the first pools its chunks into the
    cache, the second reads those prefix means from it.  The second equals a
    call that pools the prefix itself, and the cache is really read.  With
    an unaligned cut the block holding the cut is pooled again, whole, by
    the second call."""
    lengths, Hq, Hkv, d, B, page = [1500, 700], 8, 2, 128, 128, 32
    # first chunk: tokens [0, cut)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=77, verticals=True, page_size=page)
    num_pages = pb.k_cache.shape[0]
    p = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True)
    cache = fp.alloc_pooled_cache(p, num_pages, dev())
    # call 1: the contexts end at cut
    q1 = torch.cat([pb.requests[b][0][:cut[b]] for b in range(2)])
    cu1 = [0, cut[0], cut[0] + cut[1]]
    _run(pb, q1, cu1, cut, Hq, Hkv, d, B, 0.15, True, cache=cache, reuse=False)
    # call 2: the rest, prefix means from the cache
    q2, cu2, kv_lens = _chunks(pb, cut)
    r_reuse = _run(pb, q2, cu2, kv_lens, Hq, Hkv, d, B, 0.15, True, cache=cache, reuse=True)
    r_fresh = _run(pb, q2, cu2, kv_lens, Hq, Hkv, d, B, 0.15, True)
    assert torch.equal(r_reuse.out, r_fresh.out) and torch.equal(r_reuse.lse, r_fresh.lse)
    assert torch.equal(r_reuse.kv_cnt, r_fresh.kv_cnt)       # list slots past a row's count are unwritten
    for ma, mb in zip(_masks(r_reuse, Hq, kv_lens, cut, B), _masks(r_fresh, Hq, kv_lens, cut, B)):
        assert np.array_equal(ma, mb)
    # the cache entries of the first blocks hold their means: wipe them and the result moves
    wiped = cache.clone()
    for b in range(2):
        for J in range(cut[b] // B):
            wiped[:, int(pb.block_table[b, J * B // page])] = 0
    r_wiped = _run(pb, q2, cu2, kv_lens, Hq, Hkv, d, B, 0.15, True, cache=wiped, reuse=True)
    assert not torch.equal(r_wiped.out, r_fresh.out)
    # and the cache matches the pooled means the oracle computes (fp32 sums of bf16 inputs)
    for b in range(2):
        kb, vb = (t.float().numpy() for t in pb.requests[b][1:])
        kbar = O.block_means(kb, B)
        vbar = O.block_means(vb, B)
        for J in range((lengths[b] + B - 1) // B):
            pg = int(pb.block_table[b, J * B // page])
            np.testing.assert_allclose(cache[0, pg].cpu().numpy(), kbar[:, J], atol=1e-5, rtol=0)
            np.testing.assert_allclose(cache[1, pg].cpu().numpy(), vbar[:, J], atol=1e-5, rtol=0)


def test_chunked_with_skeleton_queries_and_shared_lists():
    """The selection options apply to chunks as to whole prompts: chunk rows
    stay bit-identical to the whole-prompt entry with the same options."""
    lengths, starts, Hq, Hkv, d, B, page = CASES[0]
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=61, verticals=True, page_size=page)
    for shared, probes in ((False, 16), (True, 0), (True, 4), ("pooled", 0), ("pooled", 8)):
        p = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True, shared_selection=shared,
                           query_probes=probes)
        full = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                 pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
        q, cu, kv_lens = _chunks(pb, starts)
        res = fp.fp_sparse_prefill_chunked_paged(p, q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                 pb.block_table.to(dev()), cu, kv_lens, return_lse=True)
        torch.cuda.synchronize()
        for b, P0 in enumerate(starts):
            f0, f1 = int(pb.cu_seqlens[b]) + P0, int(pb.cu_seqlens[b + 1])
            assert torch.equal(res.out[cu[b]:cu[b + 1]], full.out[f0:f1]), (shared, probes, b)
        # and the chunk's lists are the oracle's with the same options
        masks = _masks(res, Hq, kv_lens, starts, B)
        for b, (L, P0) in enumerate(zip(kv_lens, starts)):
            if L == P0:
                continue
            qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
            ref = O.select_blocks_chunked(qb[P0:], kb, vb, B, 0.2, shared=shared, probes=probes)
            outside, inside, band = compare_mask(masks[b], ref)
            assert outside == 0, (shared, probes, b, outside)

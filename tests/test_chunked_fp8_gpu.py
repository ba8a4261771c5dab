"""Chunked prefill with fp8 attention (the fp8 chunked entry).

A request's context is prefilled in two calls: the first covers its tokens
[0, P0), the second the chunk [P0, L).  After the second call:

- the e4m3 pages hold, for every block of every context, the oracle's
  blockwise codes of the whole context, bit for bit (a block the first call
  left partial is encoded again, whole), and the page-keyed scales equal the
  oracle's;
- the chunk's lists equal the bf16 chunked entry's bit for bit (selection
  reads the bf16 pages), and the oracle's selection outside the threshold
  band;
- the chunk's outputs match the oracle's attention on the dequantized codes
  (Q encoded over the chunk's queries of each block) under the GPU's lists.

Unused page slots of the bf16 cache hold NaN, so a read outside a context
shows.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import FP8_TOL, chunk_masks, compare_mask, dev

pytestmark = pytest.mark.gpu

FP8 = fp.FP_DTYPE_FP8_E4M3FN
FP8_LSE_TOL = 5e-2

CASES = [
    # context lengths, chunk starts, Hq, Hkv, d, B, page
    ([300, 1024, 77, 2048], [128, 0, 0, 1536], 8, 2, 128, 128, 64),
    ([640, 129, 255, 64], [256, 64, 192, 64], 4, 1, 64, 64, 16),      # last request: empty chunk
    ([300, 1024, 777, 2048], [131, 5, 700, 1677], 8, 2, 128, 128, 64),  # chunks that start inside a block
    ([4096, 1000, 2000], [4095, 999, 1030], 32, 8, 128, 128, 64),       # single-token chunks
]


def _case_id(c):
    aligned = all(P0 % c[5] == 0 for P0 in c[1])
    return "b%d_d%d_B%d_p%d%s" % (len(c[0]), c[4], c[5], c[6], "" if aligned else "_unaligned")


def _queries(pb, lo, hi):
    """Queries [lo[b], hi[b]) of each request packed back to back, and cu_seqlens_q."""
    parts, cu = [], [0]
    for b in range(len(lo)):
        parts.append(pb.requests[b][0][lo[b]:hi[b]])
        cu.append(cu[-1] + hi[b] - lo[b])
    return torch.cat(parts), cu


def _masks(res, Hq, kv_lens, starts, B):
    return chunk_masks(res.kv_idx, res.kv_cnt, Hq, kv_lens, starts, B)


def _two_calls(pb, starts, p, cache, pooled=None, reuse_second=False):
    """Call 1 prefills [0, P0) of each context, call 2 the chunk [P0, L).
    Returns call 2's result, its cu_seqlens_q and the context lengths."""
    lengths = [int(x) for x in pb.seqlens]
    bt = pb.block_table.to(dev())
    kd, vd = pb.k_cache.to(dev()), pb.v_cache.to(dev())
    q1, cu1 = _queries(pb, [0] * len(starts), starts)
    fp.fp_sparse_prefill_chunked_paged_fp8(p, q1.to(dev()), kd, vd, bt, cu1, starts, cache, pooled_cache=pooled)
    q2, cu2 = _queries(pb, starts, lengths)
    res = fp.fp_sparse_prefill_chunked_paged_fp8(p, q2.to(dev()), kd, vd, bt, cu2, lengths, cache,
                                                 pooled_cache=pooled, prefix_pooled=reuse_second,
                                                 return_lse=True)
    torch.cuda.synchronize()
    return res, q2, cu2, lengths


@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_chunked_fp8_matches_oracle(case, corr):
    lengths, starts, Hq, Hkv, d, B, page = case
    print(f"chunked fp8 {case} corr={corr}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=900 + len(lengths), verticals=True, page_size=page)
    alpha = 0.15
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr, dtype=FP8)
    cache = fp.alloc_fp8_cache(pb.k_cache.to(dev()))
    res, q2, cu2, kv_lens = _two_calls(pb, starts, p, cache)
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    # the lists are the bf16 chunked entry's, bit for bit
    pb16 = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    r16 = fp.fp_sparse_prefill_chunked_paged(pb16, q2.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                             pb.block_table.to(dev()), cu2, kv_lens)
    torch.cuda.synchronize()
    assert torch.equal(res.kv_cnt, r16.kv_cnt)
    masks = _masks(res, Hq, kv_lens, starts, B)
    for ma, mb in zip(masks, _masks(r16, Hq, kv_lens, starts, B)):
        assert np.array_equal(ma, mb)
    k8, v8 = cache.k8.cpu(), cache.v8.cpu()
    ks, vs = cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()
    for b, (L, P0) in enumerate(zip(kv_lens, starts)):
        nb = (L + B - 1) // B
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        pages = pb.block_table[b, :(L + page - 1) // page].tolist()
        # the e4m3 pages: the oracle's codes of the whole context, bit for bit
        deq = {}
        for name, pool, sc_pool, x in (("k", k8, ks, kb), ("v", v8, vs, vb)):
            c_ref, s_ref = O.quantize_fp8_blockwise(x, B)
            c_gpu = pool[pages].reshape(-1, Hkv, d)[:L].numpy()
            assert np.array_equal(c_gpu, c_ref), (b, name)
            s_gpu = np.stack([sc_pool[pages[J * B // page]] for J in range(nb)], axis=1)
            assert np.array_equal(s_gpu, s_ref), (b, name)
            deq[name] = O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c_ref)).numpy(), s_ref, B)
        if L == P0:
            continue
        ref = O.select_blocks_chunked(qb[P0:], kb, vb, B, alpha)
        outside, inside, band = compare_mask(masks[b], ref)
        assert outside == 0, (b, outside, inside, band)
        qc, qs = O.quantize_fp8_chunk(qb[P0:], B, P0)
        q_deq = O.dequantize_chunk(synth.fp8_codes_to_float(torch.from_numpy(qc)).numpy(), qs, B, P0)
        # attention on the dequantized codes under the GPU's lists (means of the bf16 data)
        o_ref, lse_ref = O.sparse_attention_chunked(q_deq, deq["k"], deq["v"], ref, corr, keep=masks[b])
        err = np.abs(out[cu2[b]:cu2[b + 1]] - o_ref).max()
        lerr = np.abs(lse[:, cu2[b]:cu2[b + 1]] - lse_ref).max()
        print(f"  request {b} kv={L} chunk={L - P0}: kept {int(masks[b].sum())} err {err:.3e} lse {lerr:.3e}",
              flush=True)
        assert err <= FP8_TOL and lerr <= FP8_LSE_TOL


@pytest.mark.parametrize("cut", [[1024, 384], [1000, 333]], ids=["aligned", "unaligned"])
def test_chunked_fp8_pooled_cache_between_calls(cut):
    """With the pooled cache kept between the calls, the second call reads the
    prefix means from it: it equals a second call that pools the prefix
    itself, bit for bit, and the cache holds the same bits as after the same
    two calls through the bf16 chunked entry (the encoding pass forms the
    chunk blocks' means in the pooling kernel's summation order)."""
    lengths, Hq, Hkv, d, B, page = [1500, 700], 8, 2, 128, 128, 32
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=97, verticals=True, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True, dtype=FP8)
    pooled = fp.alloc_pooled_cache(p, pb.k_cache.shape[0], dev())
    cache = fp.alloc_fp8_cache(pb.k_cache.to(dev()))
    r_reuse, q2, cu2, kv_lens = _two_calls(pb, cut, p, cache, pooled=pooled, reuse_second=True)
    r_fresh = fp.fp_sparse_prefill_chunked_paged_fp8(p, q2.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                     pb.block_table.to(dev()), cu2, kv_lens, cache,
                                                     return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(r_reuse.out, r_fresh.out) and torch.equal(r_reuse.lse, r_fresh.lse)
    assert torch.equal(r_reuse.kv_cnt, r_fresh.kv_cnt)
    p16 = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True)
    pooled16 = fp.alloc_pooled_cache(p16, pb.k_cache.shape[0], dev())
    bt, kd, vd = pb.block_table.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev())
    q1, cu1 = _queries(pb, [0, 0], cut)
    fp.fp_sparse_prefill_chunked_paged(p16, q1.to(dev()), kd, vd, bt, cu1, cut, pooled_cache=pooled16)
    r16 = fp.fp_sparse_prefill_chunked_paged(p16, q2.to(dev()), kd, vd, bt, cu2, kv_lens, pooled_cache=pooled16,
                                             prefix_pooled=True)
    torch.cuda.synchronize()
    used = torch.zeros(pb.k_cache.shape[0], dtype=torch.bool)
    for b, L in enumerate(lengths):
        for J in range((L + B - 1) // B):
            used[int(pb.block_table[b, J * B // page])] = True
    assert torch.equal(pooled[:, used.to(dev())], pooled16[:, used.to(dev())])
    assert torch.equal(r_reuse.kv_cnt, r16.kv_cnt)


def test_chunked_fp8_rejects_bf16_params():
    lengths, starts, Hq, Hkv, d, B, page = CASES[1]
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=912, verticals=False, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.2)
    cache = fp.alloc_fp8_cache(pb.k_cache.to(dev()))
    q2, cu2 = _queries(pb, starts, lengths)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_sparse_prefill_chunked_paged_fp8(p, q2.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                               pb.block_table.to(dev()), cu2, lengths, cache)
    assert e.value.status == fp.FP_INVALID_ARGUMENT

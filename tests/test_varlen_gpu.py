"""Parity of the paged, variable-length entry (continuous batching) with the
CPU oracle run request by request, at small sizes with ragged lengths.
Unused page slots hold NaN, so a read outside a request's tokens shows."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import BF16_TOL, LSE_TOL, check_lists, compare_mask, dev, run_single

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, Hq, Hkv, d, B, page
    ([300, 1024, 77, 2048], 8, 2, 128, 128, 64),
    ([1, 129, 640, 255], 4, 1, 64, 64, 16),
    ([513, 0, 1000], 6, 3, 128, 64, 32),
    ([4096, 100, 2000, 64, 1500], 32, 8, 128, 128, 64),
]


def _run_paged(pb, Hq, Hkv, d, B, alpha, corr):
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    res = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                            pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    return res


def _region_offsets(lengths, Hq, B):
    idx, cnt = [0], [0]
    for L in lengths:
        nb = (L + B - 1) // B
        idx.append(idx[-1] + Hq * nb * (nb + 1) // 2)
        cnt.append(cnt[-1] + Hq * nb)
    return idx, cnt


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.4])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_d%d_B%d_p%d" % (len(c[0]), c[3], c[4], c[5]))
def test_paged_matches_oracle_per_request(case, alpha, corr):
    lengths, Hq, Hkv, d, B, page = case
    print(f"paged {case} alpha={alpha} corr={corr}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=700 + len(lengths), verticals=True,
                                page_size=page)
    res = _run_paged(pb, Hq, Hkv, d, B, alpha, corr)
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    assert np.isfinite(out).all()
    idx_off, cnt_off = _region_offsets(lengths, Hq, B)
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        nb = (L + B - 1) // B
        mask = check_lists(res.kv_idx, res.kv_cnt, Hq, nb, offset=idx_off[b], cnt_offset=cnt_off[b])
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        ref = O.select_blocks(qb, kb, vb, B, alpha)
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside, inside, band)
        o_ref, lse_ref = O.sparse_attention(qb, kb, vb, ref, corr, keep=mask)
        t0, t1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        err = np.abs(out[t0:t1] - o_ref).max()
        lerr = np.abs(lse[:, t0:t1] - lse_ref).max()
        print(f"  request {b} L={L}: kept {int(mask.sum())} err {err:.3e} lse {lerr:.3e}", flush=True)
        assert err <= BF16_TOL and lerr <= LSE_TOL


def test_paged_equals_single_sequence_calls():
    """The batch gives bit-identical results to one call per request on
    contiguous K/V (same kernels, same order of arithmetic)."""
    lengths, Hq, Hkv, d, B, page = [700, 1300, 64], 8, 2, 128, 128, 32
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=900, verticals=True, page_size=page)
    res = _run_paged(pb, Hq, Hkv, d, B, 0.2, True)
    for b, L in enumerate(lengths):
        q, k, v = pb.requests[b]
        sel, (o, l) = run_single(q, k, v, B, 0.2, correction=True)
        t0, t1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        assert torch.equal(res.out[t0:t1], o), b
        assert torch.equal(res.lse[:, t0:t1], l), b


def test_page_permutation_invariance():
    lengths, Hq, Hkv, d, B = [900, 333], 4, 2, 64, 64
    a = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=11, verticals=False, page_size=16, perm_seed=1)
    b = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=11, verticals=False, page_size=16, perm_seed=2)
    assert not torch.equal(a.block_table, b.block_table)
    ra = _run_paged(a, Hq, Hkv, d, B, 0.3, True)
    rb = _run_paged(b, Hq, Hkv, d, B, 0.3, True)
    assert torch.equal(ra.out, rb.out) and torch.equal(ra.lse, rb.lse)


def test_out_of_range_page_reads_zero():
    """A block-table entry outside the pool reads as zeros instead of faulting:
    the result equals a cache whose page holds zeros."""
    lengths, Hq, Hkv, d, B, page = [256], 2, 1, 64, 64, 64
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=5, verticals=False, page_size=page)
    bad = pb.block_table.clone()
    victim = int(bad[0, 1])
    bad[0, 1] = 10 ** 6
    zeroed_k, zeroed_v = pb.k_cache.clone(), pb.v_cache.clone()
    zeroed_k[victim] = 0
    zeroed_v[victim] = 0
    p = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True)
    r1 = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                           bad.to(dev()), pb.cu_seqlens, return_lse=True)
    r2 = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), zeroed_k.to(dev()), zeroed_v.to(dev()),
                                           pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(r1.out, r2.out)

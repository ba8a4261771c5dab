"""fp8 inference over a paged batch (the fp8 paged cache).

- The e4m3 pages hold, token by token, the codes of each request's blockwise
  quantization, bit for bit against the oracle's quantizer; the page-keyed
  scales equal the oracle's.
- The lists match the oracle's selection on the bf16 data outside the
  threshold band.
- Outputs match the oracle's attention on the dequantized codes under the
  GPU's lists.
- Each request's rows and LSE equal the single-sequence fp8 entries' bit for
  bit (same codes, same lists, same tiles in the same order).
Unused page slots of the bf16 cache hold NaN, so a read outside a request's
tokens shows.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import FP8_TOL, check_lists, compare_mask, dev

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, Hq, Hkv, d, B, page
    ([3000, 700, 129, 1500], 8, 2, 128, 128, 64),
    ([640, 65, 255, 1], 4, 1, 64, 64, 16),
]
FP8 = fp.FP_DTYPE_FP8_E4M3FN


def _offsets(lengths, Hq, B):
    idx, cnt = [0], [0]
    for L in lengths:
        nb = (L + B - 1) // B
        idx.append(idx[-1] + Hq * nb * (nb + 1) // 2)
        cnt.append(cnt[-1] + Hq * nb)
    return idx, cnt


@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_d%d_B%d_p%d" % (len(c[0]), c[3], c[4], c[5]))
def test_fp8_paged_matches_oracle(case, corr):
    lengths, Hq, Hkv, d, B, page = case
    print(f"fp8 paged {case} corr={corr}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=800 + len(lengths), verticals=True, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=corr, dtype=FP8)
    bt = pb.block_table.to(dev())
    res, cache = fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                       bt, pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    out = res.out.float().cpu().numpy()
    assert np.isfinite(out).all() and torch.isfinite(res.lse).all()
    k8, v8 = cache.k8.cpu(), cache.v8.cpu()
    ks, vs = cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()
    idx_off, cnt_off = _offsets(lengths, Hq, B)
    for b, L in enumerate(lengths):
        nb = (L + B - 1) // B
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        pages = pb.block_table[b, :(L + page - 1) // page].tolist()
        # the fp8 pages and scales: the oracle's codes of this request, bit for bit
        codes = {}
        for name, pool, sc_pool, x in (("k", k8, ks, kb), ("v", v8, vs, vb)):
            c_ref, s_ref = O.quantize_fp8_blockwise(x, B)
            c_gpu = pool[pages].reshape(-1, Hkv, d)[:L].numpy()
            assert np.array_equal(c_gpu, c_ref), (b, name)
            s_gpu = np.stack([sc_pool[pages[J * B // page]] for J in range(nb)], axis=1)
            assert np.array_equal(s_gpu, s_ref), (b, name)
            codes[name] = O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c_ref)).numpy(), s_ref, B)
        qc, qs = O.quantize_fp8_blockwise(qb, B)
        q_deq = O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(qc)).numpy(), qs, B)
        # lists: selection on the bf16 data
        mask = check_lists(res.kv_idx, res.kv_cnt, Hq, nb, offset=idx_off[b], cnt_offset=cnt_off[b])
        ref = O.select_blocks(qb, kb, vb, B, 0.15)
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside, inside, band)
        # attention on the dequantized codes under the GPU's lists (means of the bf16 data)
        o_ref, _ = O.sparse_attention(q_deq, codes["k"], codes["v"], ref, corr, keep=mask)
        t0, t1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        err = np.abs(out[t0:t1] - o_ref).max()
        print(f"  request {b} L={L}: kept {int(mask.sum())} err {err:.3e}", flush=True)
        assert err <= FP8_TOL


@pytest.mark.parametrize("case", CASES[:1], ids=["B128"])
def test_fp8_paged_equals_single_sequence_calls(case):
    lengths, Hq, Hkv, d, B, page = case
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=811, verticals=True, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True, dtype=FP8)
    res, _ = fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                   pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    for b, L in enumerate(lengths):
        qd, kd, vd = (t.to(dev()) for t in pb.requests[b])
        sel, f8 = fp.fp_select_blocks_fp8(p, qd, kd, vd)
        o, lse = fp.fp_sparse_prefill_fwd(p, f8.q8, f8.k8, f8.v8, sel, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                          v_scale=f8.v_scale, return_lse=True)
        torch.cuda.synchronize()
        t0, t1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        assert torch.equal(res.out[t0:t1], o), b
        assert torch.equal(res.lse[:, t0:t1], lse), b


def test_fp8_paged_rejects_bf16_params():
    lengths, Hq, Hkv, d, B, page = CASES[1]
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=812, verticals=False, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.2)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                              pb.block_table.to(dev()), pb.cu_seqlens)
    assert e.value.status == fp.FP_INVALID_ARGUMENT


def test_fp8_out_of_range_page_reads_zero():
    """A block-table entry outside the pool reads as zeros (codes 0, scale 1)
    instead of faulting or giving NaN rows: the result equals a cache whose
    page holds zeros.  With page = block, the bad page is the first page of
    its block, so its scale lookup is the one that falls outside the pool."""
    lengths, Hq, Hkv, d, B, page = [320], 4, 1, 64, 64, 64
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=6, verticals=False, page_size=page)
    bad = pb.block_table.clone()
    victim = int(bad[0, 2])
    bad[0, 2] = 10 ** 6
    zeroed_k, zeroed_v = pb.k_cache.clone(), pb.v_cache.clone()
    zeroed_k[victim] = 0
    zeroed_v[victim] = 0
    p = fp.make_params(Hq, Hkv, d, B, 0.0, mean_correction=True, dtype=FP8)
    r1, _ = fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                  bad.to(dev()), pb.cu_seqlens, return_lse=True)
    r2, _ = fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), zeroed_k.to(dev()), zeroed_v.to(dev()),
                                                  pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(r1.out.float()).all() and torch.isfinite(r1.lse).all()
    assert torch.equal(r1.out, r2.out) and torch.equal(r1.lse, r2.lse)

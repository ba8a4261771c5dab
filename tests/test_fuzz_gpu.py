"""Randomised parity of the HIP path against the CPU oracle (hypothesis, a
fixed and bounded set of examples, derandomised so every run draws the same
cases).

Each example draws a shape -- lengths 1 .. 2048 including partial blocks,
head pairs (Hq, Hkv) from {(1,1), (4,1), (8,2), (32,8)}, d in {64, 128},
block in {64, 128}, a threshold ratio, the correction on or off -- and runs
it through the single-sequence entries (bf16, or fp8 on the codes of the
blockwise recipe), the paged entry with a random split into requests and a
random page permutation, or the chunked entries (bf16, or fp8 after a first
call over each prefix) with chunks that start at any token.  The oracle
decides: masks equal outside the 1e-3 band, outputs within 2e-2 (bf16) or
6e-2 (fp8, against the oracle on the dequantized codes), LSE within 1e-2
(bf16)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import BF16_TOL, FP8_TOL, LSE_TOL, check_lists, chunk_masks, compare_mask, dev

pytestmark = pytest.mark.gpu

HEADS = [(1, 1), (4, 1), (8, 2), (32, 8)]
FUZZ = settings(max_examples=25, deadline=None, derandomize=True, print_blob=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _lengths(total_cap):
    return st.lists(st.integers(1, 2048), min_size=1, max_size=3).filter(lambda l: sum(l) <= total_cap)


@FUZZ
@given(S=st.integers(1, 2048), heads=st.sampled_from(HEADS), d=st.sampled_from([64, 128]),
       B=st.sampled_from([64, 128]), alpha=st.sampled_from([0.0, 0.03, 0.1, 0.3, 0.7, 1.0]),
       corr=st.booleans(), fp8=st.booleans(), seed=st.integers(0, 10 ** 6))
def test_fuzz_single_sequence(S, heads, d, B, alpha, corr, fp8, seed):
    Hq, Hkv = heads
    print(f"fuzz single S={S} Hq={Hq} Hkv={Hkv} d={d} B={B} alpha={alpha} corr={corr} fp8={fp8} seed={seed}",
          flush=True)
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed, verticals=S > 4096)
    nB = (S + B - 1) // B
    pb = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    sel = fp.fp_select_blocks(pb, qd, kd, vd)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    if fp8:
        q8, sq = synth.quantize_fp8_blockwise(q, B)
        k8, sk = synth.quantize_fp8_blockwise(k, B)
        v8, sv = synth.quantize_fp8_blockwise(v, B)
        p8 = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
        out = fp.fp_sparse_prefill_fwd(p8, q8.to(dev()), k8.to(dev()), v8.to(dev()), sel, q_scale=sq.to(dev()),
                                       k_scale=sk.to(dev()), v_scale=sv.to(dev()))
        lse = None
        deq = []
        for x in (qn, kn, vn):
            c, s = O.quantize_fp8_blockwise(x, B)
            deq.append(O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c)).numpy(), s, B))
    else:
        out, lse = fp.fp_sparse_prefill_fwd(pb, qd, kd, vd, sel, return_lse=True)
    torch.cuda.synchronize()
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    ref = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0, (outside, inside, band)
    if fp8:
        o_ref, _ = O.sparse_attention(deq[0], deq[1], deq[2], ref, corr, keep=mask)
        err = float(np.abs(out.float().cpu().numpy() - o_ref).max())
        print(f"  kept {int(mask.sum())} band {band} err {err:.3e}", flush=True)
        assert err <= FP8_TOL
    else:
        o_ref, lse_ref = O.sparse_attention(qn, kn, vn, ref, corr, keep=mask)
        err = float(np.abs(out.float().cpu().numpy() - o_ref).max())
        lerr = float(np.abs(lse.cpu().numpy() - lse_ref).max())
        print(f"  kept {int(mask.sum())} band {band} err {err:.3e} lse {lerr:.3e}", flush=True)
        assert err <= BF16_TOL and lerr <= LSE_TOL


@FUZZ
@given(lengths=_lengths(4096), heads=st.sampled_from(HEADS), d=st.sampled_from([64, 128]),
       B=st.sampled_from([64, 128]), page=st.sampled_from([16, 32, 64]),
       alpha=st.sampled_from([0.0, 0.1, 0.4]), corr=st.booleans(), seed=st.integers(0, 10 ** 6))
def test_fuzz_paged_batch(lengths, heads, d, B, page, alpha, corr, seed):
    Hq, Hkv = heads
    print(f"fuzz paged lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} B={B} page={page} alpha={alpha} corr={corr} "
          f"seed={seed}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=seed, verticals=False, page_size=page,
                                perm_seed=seed + 1)
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    res = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                            pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    io = co = 0
    for b, L in enumerate(lengths):
        nb = (L + B - 1) // B
        mask = check_lists(res.kv_idx, res.kv_cnt, Hq, nb, offset=io, cnt_offset=co)
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        ref = O.select_blocks(qb, kb, vb, B, alpha)
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside, inside, band)
        o_ref, lse_ref = O.sparse_attention(qb, kb, vb, ref, corr, keep=mask)
        t0, t1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        err = float(np.abs(out[t0:t1] - o_ref).max())
        lerr = float(np.abs(lse[:, t0:t1] - lse_ref).max())
        print(f"  request {b} L={L}: kept {int(mask.sum())} err {err:.3e} lse {lerr:.3e}", flush=True)
        assert err <= BF16_TOL and lerr <= LSE_TOL
        io += Hq * nb * (nb + 1) // 2
        co += Hq * nb


@FUZZ
@given(lengths=_lengths(4096), heads=st.sampled_from(HEADS), d=st.sampled_from([64, 128]),
       B=st.sampled_from([64, 128]), page=st.sampled_from([16, 32, 64]),
       alpha=st.sampled_from([0.0, 0.1, 0.4]), corr=st.booleans(), fp8=st.booleans(),
       fracs=st.lists(st.floats(0.0, 1.0), min_size=3, max_size=3), seed=st.integers(0, 10 ** 6))
def test_fuzz_chunked(lengths, heads, d, B, page, alpha, corr, fp8, fracs, seed):
    Hq, Hkv = heads
    starts = [int(f * L) for f, L in zip(fracs, lengths)]          # chunk [P0, L), any token, maybe empty
    print(f"fuzz chunked lengths={lengths} starts={starts} Hq={Hq} Hkv={Hkv} d={d} B={B} page={page} "
          f"alpha={alpha} corr={corr} fp8={fp8} seed={seed}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=seed, verticals=False, page_size=page,
                                perm_seed=seed + 1)
    kc, vc, bt = pb.k_cache.to(dev()), pb.v_cache.to(dev()), pb.block_table.to(dev())

    def packed(lo, hi):
        return (torch.cat([pb.requests[b][0][lo[b]:hi[b]] for b in range(len(lengths))]).to(dev()),
                np.concatenate([[0], np.cumsum([hi[b] - lo[b] for b in range(len(lengths))])]).tolist())

    q2, cu2 = packed(starts, lengths)
    if fp8:
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
        cache = fp.alloc_fp8_cache(kc)
        q1, cu1 = packed([0] * len(lengths), starts)
        fp.fp_sparse_prefill_chunked_paged_fp8(p, q1, kc, vc, bt, cu1, starts, cache)     # the prefixes
        res = fp.fp_sparse_prefill_chunked_paged_fp8(p, q2, kc, vc, bt, cu2, lengths, cache, return_lse=True)
    else:
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
        res = fp.fp_sparse_prefill_chunked_paged(p, q2, kc, vc, bt, cu2, lengths, return_lse=True)
    torch.cuda.synchronize()
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    masks = chunk_masks(res.kv_idx, res.kv_cnt, Hq, lengths, starts, B)
    for b, (L, P0) in enumerate(zip(lengths, starts)):
        if P0 == L:
            continue
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        ref = O.select_blocks_chunked(qb[P0:], kb, vb, B, alpha)
        outside, inside, band = compare_mask(masks[b], ref)
        assert outside == 0, (b, outside, inside, band)
        r0, r1 = cu2[b], cu2[b + 1]
        if fp8:
            deq = [O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c)).numpy(), s_, B)
                   for c, s_ in (O.quantize_fp8_blockwise(x, B) for x in (kb, vb))]
            qc, qs = O.quantize_fp8_chunk(qb[P0:], B, P0)
            q_deq = O.dequantize_chunk(synth.fp8_codes_to_float(torch.from_numpy(qc)).numpy(), qs, B, P0)
            o_ref, _ = O.sparse_attention_chunked(q_deq, deq[0], deq[1], ref, corr, keep=masks[b])
            err = float(np.abs(out[r0:r1] - o_ref).max())
            print(f"  request {b} L={L} P0={P0}: kept {int(masks[b].sum())} err {err:.3e}", flush=True)
            assert err <= FP8_TOL
        else:
            o_ref, lse_ref = O.sparse_attention_chunked(qb[P0:], kb, vb, ref, corr, keep=masks[b])
            err = float(np.abs(out[r0:r1] - o_ref).max())
            lerr = float(np.abs(lse[:, r0:r1] - lse_ref).max())
            print(f"  request {b} L={L} P0={P0}: kept {int(masks[b].sum())} err {err:.3e} lse {lerr:.3e}",
                  flush=True)
            assert err <= BF16_TOL and lerr <= LSE_TOL

"""Randomised parity of the HIP path against the CPU oracle (hypothesis, a
fixed and bounded set of examples, derandomised so every run draws the same
cases).

Each example draws a shape -- lengths 1 .. 2048 including partial blocks,
head pairs (Hq, Hkv) from {(1,1), (4,1), (8,2), (32,8)}, d in {64, 128},
block in {64, 128}, a threshold ratio, the correction on or off -- and runs
it through the single-sequence entries (bf16, or fp8 on the codes of the
blockwise recipe) or the paged entry with a random split into requests and a
random page permutation.  The oracle decides: masks equal outside the 1e-3
band, outputs within 2e-2 (bf16) or 6e-2 (fp8, against the oracle on the
dequantized codes), LSE within 1e-2 (bf16)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import BF16_TOL, FP8_TOL, LSE_TOL, check_lists, compare_mask, dev

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

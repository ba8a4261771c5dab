"""The entries hold no state between or across calls (the allocation-free
entry's scratch aside), so calls enqueued on two streams at once -- a bf16
layer on one, a paged fp8 batch or a chunked call on the other -- give the
same bits as the same calls run one after the other."""
import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import synth

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _layer(q, k, v, p):
    sel = fp.fp_select_blocks(p, q, k, v)
    out, lse = fp.fp_sparse_prefill_fwd(p, q, k, v, sel, return_lse=True)
    return [sel.kv_cnt, sel.pooled_k, out, lse]


def _paged8(pb, p8, kc, vc, bt):
    r, c = fp.fp_sparse_prefill_varlen_paged_fp8(p8, pb.q.to(dev()), kc, vc, bt, pb.cu_seqlens, return_lse=True)
    return [r.kv_cnt, r.out, r.lse]


def _chunked(pb, p, kc, vc, bt, starts):
    lengths = [int(x) for x in pb.seqlens]
    q = torch.cat([pb.requests[b][0][P0:] for b, P0 in enumerate(starts)]).to(dev())
    cu = [0]
    for b, P0 in enumerate(starts):
        cu.append(cu[-1] + lengths[b] - P0)
    r = fp.fp_sparse_prefill_chunked_paged(p, q, kc, vc, bt, cu, lengths, return_lse=True)
    return [r.kv_cnt, r.out, r.lse]


def test_two_streams_equal_one_after_the_other():
    S, Hq, Hkv, d, B = 16384, 8, 2, 128, 128
    q, k, v = (t.to(dev()) for t in synth.make_sequence(S, Hq, Hkv, d, seed=41, verticals=True))
    p = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True)
    lengths = [3000, 700, 9000]
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=42, verticals=True, page_size=64)
    kc, vc, bt = pb.k_cache.to(dev()), pb.v_cache.to(dev()), pb.block_table.to(dev())
    p8 = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    starts = [2500, 640, 7000]
    torch.cuda.synchronize()

    seq = [_layer(q, k, v, p), _paged8(pb, p8, kc, vc, bt), _chunked(pb, p, kc, vc, bt, starts)]
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()      # default priority
    for pair in ((0, 1), (0, 2), (1, 2)):
        res = {}
        runs = {0: lambda: _layer(q, k, v, p), 1: lambda: _paged8(pb, p8, kc, vc, bt),
                2: lambda: _chunked(pb, p, kc, vc, bt, starts)}
        for stream, which in zip((s1, s2), pair):
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                res[which] = runs[which]()
        torch.cuda.synchronize()
        for which in pair:
            for a, b in zip(res[which], seq[which]):
                assert torch.equal(a, b), (pair, which)

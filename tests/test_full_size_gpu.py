"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: every block list against the oracle's selection (bit-exact
outside the threshold band), and outputs of a sample of (head, query block)
pairs -- always including the first and last query blocks, at 32K and 128K
64 workgroups spread over the attention launch and every XCD slot, and 16
pairs per request of the paged batch -- against the oracle evaluated
under the GPU's mask."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import BF16_TOL, FP8_TOL, LSE_TOL, check_lists, compare_mask, dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sample_pairs(Hq, nB, n, seed):
    r = np.random.default_rng(seed)
    pairs = {(0, 0), (Hq - 1, nB - 1), (Hq // 2, nB - 1), (1 % Hq, nB // 2)}
    while len(pairs) < n:
        pairs.add((int(r.integers(Hq)), int(r.integers(nB))))
    return sorted(pairs)


def _launch_pairs(Hq, nB, grid):
    """(head, query block) pairs of 64 workgroups evenly spaced over the
    attention launch (one workgroup per pair: query blocks longest first, the
    heads of one KV head on one XCD), every head and XCD slot among them."""
    assert grid == nB * Hq

    def xcd_head(slot):
        return (slot % 8) * (Hq // 8) + slot // 8 if Hq % 8 == 0 else slot

    pairs = set()
    for k in range(64):
        idx = min(grid - 1, k * grid // 64 + (5 * k) % Hq)
        rank, slot = divmod(idx, Hq)
        pairs.add((xcd_head(slot), nB - 1 - rank))
    return pairs


class _Seq:
    def __init__(self, name):
        w = synth.WORKLOADS[name]
        self.w = w
        self.S, self.Hq, self.Hkv, self.d, self.B = (w.seqlens[0], w.num_q_heads, w.num_kv_heads,
                                                     w.head_dim, w.block_size)
        print(f"generating {name}", flush=True)
        q, k, v = synth.make_sequence(self.S, self.Hq, self.Hkv, self.d, w.seed, w.verticals)
        self.cpu = (q, k, v)
        self.gpu = tuple(t.to(dev()) for t in (q, k, v))
        self.np = tuple(t.float().numpy() for t in (q, k, v))


@pytest.fixture(scope="module")
def s32k():
    return _Seq("llama8b_s32k")


@pytest.fixture(scope="module")
def s128k():
    return _Seq("llama8b_s128k")


def _check_full(seq, alpha, n_pairs, seed):
    S, Hq, Hkv, d, B = seq.S, seq.Hq, seq.Hkv, seq.d, seq.B
    nB = (S + B - 1) // B
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True)
    qd, kd, vd = seq.gpu
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    out, lse = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, return_lse=True)
    torch.cuda.synchronize()
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = seq.np
    ref = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    density = mask.sum() / (Hq * nB * (nB + 1) / 2)
    print(f"  alpha={alpha}: density {density:.4f}, band {band}, mismatches in band {inside}, "
          f"outside {outside}", flush=True)
    assert outside == 0
    # pooled means against the oracle's
    np.testing.assert_allclose(sel.pooled_k.cpu().numpy(), ref.k_bar, rtol=0, atol=1e-5)
    grid = fp.fp_attention_workgroups(p, [0, S])
    spread = _launch_pairs(Hq, nB, grid)
    pairs = sorted(set(_sample_pairs(Hq, nB, n_pairs, seed)) | spread)
    print(f"  grid {grid}: {len(spread)} pairs spread over the launch", flush=True)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, ref, True, pairs=pairs, keep=mask)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    worst, lworst = 0.0, 0.0
    for h, I in pairs:
        r0, r1 = I * B, min(S, (I + 1) * B)
        worst = max(worst, float(np.abs(o[r0:r1, h] - o_ref[r0:r1, h]).max()))
        lworst = max(lworst, float(np.abs(l[h, r0:r1] - lse_ref[h, r0:r1]).max()))
    print(f"  {len(pairs)} sampled pairs: max|o-ref| {worst:.3e}, max|lse-ref| {lworst:.3e}", flush=True)
    assert worst <= BF16_TOL and lworst <= LSE_TOL
    assert np.isfinite(o).all()


def test_32k_full_size(s32k):
    _check_full(s32k, 0.1, 96, seed=2)


@pytest.mark.parametrize("alpha", [0.05, 0.1, 0.2])
def test_128k_full_size(s128k, alpha):
    _check_full(s128k, alpha, 48, seed=int(alpha * 100))


def test_paged_batch8_full_size():
    w = synth.WORKLOADS["paged_batch8"]
    Hq, Hkv, d, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating paged_batch8", flush=True)
    pb = synth.workload_inputs(w)
    p = fp.make_params(Hq, Hkv, d, B, w.alphas[0], mean_correction=True)
    res = fp.fp_sparse_prefill_varlen_paged(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                            pb.block_table.to(dev()), pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    assert np.isfinite(out).all()
    idx_off, cnt_off = 0, 0
    kept_total, causal_total = 0, 0
    for b, L in enumerate(pb.seqlens):
        nb = (L + B - 1) // B
        mask = check_lists(res.kv_idx, res.kv_cnt, Hq, nb, offset=idx_off, cnt_offset=cnt_off)
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        ref = O.select_blocks(qb, kb, vb, B, w.alphas[0])
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside)
        pairs = _sample_pairs(Hq, nb, 16, seed=b)
        o_ref, lse_ref = O.sparse_attention(qb, kb, vb, ref, True, pairs=pairs, keep=mask)
        t0 = int(pb.cu_seqlens[b])
        for h, I in pairs:
            r0, r1 = I * B, min(L, (I + 1) * B)
            err = np.abs(out[t0 + r0:t0 + r1, h] - o_ref[r0:r1, h]).max()
            lerr = np.abs(lse[h, t0 + r0:t0 + r1] - lse_ref[h, r0:r1]).max()
            assert err <= BF16_TOL and lerr <= LSE_TOL, (b, h, I, err, lerr)
        kept_total += int(mask.sum())
        causal_total += Hq * nb * (nb + 1) // 2
        print(f"  request {b} L={L}: density {mask.sum() / (Hq * nb * (nb + 1) / 2):.4f}, band {band}, "
              f"in-band mismatches {inside}", flush=True)
        idx_off += Hq * nb * (nb + 1) // 2
        cnt_off += Hq * nb
    print(f"  overall density {kept_total / causal_total:.4f}", flush=True)


def test_paged_batch8_fp8_full_size():
    """The fp8 paged entry in the configuration the benchmark times (8
    requests, 307,200 tokens): the e4m3 pages and their page-keyed scales
    equal the oracle's quantizer per request bit for bit, the lists match the
    oracle outside the band, and sampled outputs match the oracle's attention
    on the dequantized codes under the GPU's lists."""
    w = synth.WORKLOADS["paged_batch8"]
    Hq, Hkv, d, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating paged_batch8 (fp8)", flush=True)
    pb = synth.workload_inputs(w)
    page = pb.k_cache.shape[1]
    p = fp.make_params(Hq, Hkv, d, B, w.alphas[0], mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    res, cache = fp.fp_sparse_prefill_varlen_paged_fp8(p, pb.q.to(dev()), pb.k_cache.to(dev()), pb.v_cache.to(dev()),
                                                       pb.block_table.to(dev()), pb.cu_seqlens)
    torch.cuda.synchronize()
    out = res.out.float().cpu().numpy()
    assert np.isfinite(out).all()
    k8, v8 = cache.k8.cpu(), cache.v8.cpu()
    ks, vs = cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()
    idx_off, cnt_off = 0, 0
    for b, L in enumerate(pb.seqlens):
        nb = (L + B - 1) // B
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        pages = pb.block_table[b, :(L + page - 1) // page].tolist()
        deq = []
        for x, pool, sc in ((qb, None, None), (kb, k8, ks), (vb, v8, vs)):
            c_ref, s_ref = O.quantize_fp8_blockwise(x, B)
            if pool is not None:
                assert np.array_equal(pool[pages].reshape(-1, Hkv, d)[:L].numpy(), c_ref), b
                assert np.array_equal(np.stack([sc[pages[J * B // page]] for J in range(nb)], axis=1), s_ref), b
            deq.append(O.dequantize_blockwise(synth.fp8_codes_to_float(torch.from_numpy(c_ref)).numpy(), s_ref, B))
        mask = check_lists(res.kv_idx, res.kv_cnt, Hq, nb, offset=idx_off, cnt_offset=cnt_off)
        ref = O.select_blocks(qb, kb, vb, B, w.alphas[0])
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside)
        pairs = _sample_pairs(Hq, nb, 16, seed=50 + b)
        o_ref, _ = O.sparse_attention(deq[0], deq[1], deq[2], ref, True, pairs=pairs, keep=mask)
        t0 = int(pb.cu_seqlens[b])
        worst = max(float(np.abs(out[t0 + I * B:t0 + min(L, (I + 1) * B), h] - o_ref[I * B:min(L, (I + 1) * B), h]).max())
                    for h, I in pairs)
        print(f"  request {b} L={L}: kept {int(mask.sum())}, sampled max|o-ref| {worst:.3e}", flush=True)
        assert worst <= FP8_TOL, (b, worst)
        idx_off += Hq * nb * (nb + 1) // 2
        cnt_off += Hq * nb


def test_paged_batch8_chunked_last4096_full_size():
    """The chunked entry in the configuration the benchmark times: the 8
    requests' last 4096 tokens are new, their prefix means come from the
    pooled cache written by an earlier call over the prefixes.  Every output
    row and LSE equals the whole-prompt call's (a property of the reading of
    chunked prefill that holds at any size), and the prefix call's rows equal
    the whole prompt's first rows."""
    w = synth.WORKLOADS["paged_batch8"]
    Hq, Hkv, d, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating paged_batch8", flush=True)
    pb = synth.workload_inputs(w)
    p = fp.make_params(Hq, Hkv, d, B, w.alphas[0], mean_correction=True)
    qd, kc, vc, bt = (x.to(dev()) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    full = fp.fp_sparse_prefill_varlen_paged(p, qd, kc, vc, bt, pb.cu_seqlens, return_lse=True)
    cu = [int(x) for x in pb.cu_seqlens]
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    cut = [max(0, L - 4096) for L in lens]
    cache = fp.alloc_pooled_cache(p, kc.shape[0], dev())
    q_pre = torch.cat([qd[cu[b]:cu[b] + cut[b]] for b in range(len(lens))])
    cu_pre = [0]
    for c_ in cut:
        cu_pre.append(cu_pre[-1] + c_)
    pre = fp.fp_sparse_prefill_chunked_paged(p, q_pre, kc, vc, bt, cu_pre, cut, pooled_cache=cache,
                                             return_lse=True)
    q_new = torch.cat([qd[cu[b] + cut[b]:cu[b + 1]] for b in range(len(lens))])
    cu_new = [0]
    for b in range(len(lens)):
        cu_new.append(cu_new[-1] + lens[b] - cut[b])
    res = fp.fp_sparse_prefill_chunked_paged(p, q_new, kc, vc, bt, cu_new, lens, pooled_cache=cache,
                                             prefix_pooled=True, return_lse=True)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        assert torch.equal(res.out[cu_new[b]:cu_new[b + 1]], full.out[cu[b] + cut[b]:cu[b + 1]]), b
        assert torch.equal(res.lse[:, cu_new[b]:cu_new[b + 1]], full.lse[:, cu[b] + cut[b]:cu[b + 1]]), b
        assert torch.equal(pre.out[cu_pre[b]:cu_pre[b + 1]], full.out[cu[b]:cu[b] + cut[b]]), b
    print(f"  {cu_new[-1]} new rows and {cu_pre[-1]} prefix rows equal the whole-prompt rows", flush=True)


def test_paged_batch8_chunked_fp8_last4096_full_size():
    """The fp8 chunked entry in the configuration the benchmark times: the
    e4m3 pages of the whole prompts come from the fp8 paged entry, the
    prefix means from the pooled cache of a bf16 prefix call, and the timed
    call encodes the last 4096 tokens of each context.  The chunks' e4m3
    blocks equal the oracle's codes bit for bit, the lists equal the bf16
    chunked entry's, and sampled (head, query block) outputs and LSE match
    the oracle's attention on the dequantized codes under those lists."""
    w = synth.WORKLOADS["paged_batch8"]
    Hq, Hkv, d, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating paged_batch8 (fp8 chunked)", flush=True)
    pb = synth.workload_inputs(w)
    page = pb.k_cache.shape[1]
    alpha = w.alphas[0]
    p16 = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True)
    p8 = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    qd, kc, vc, bt = (x.to(dev()) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    _, c8 = fp.fp_sparse_prefill_varlen_paged_fp8(p8, qd, kc, vc, bt, pb.cu_seqlens)
    cu = [int(x) for x in pb.cu_seqlens]
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    cut = [max(0, L - 4096) for L in lens]
    cache = fp.alloc_pooled_cache(p16, kc.shape[0], dev())
    q_pre = torch.cat([qd[cu[b]:cu[b] + cut[b]] for b in range(len(lens))])
    cu_pre = [0]
    for c_ in cut:
        cu_pre.append(cu_pre[-1] + c_)
    fp.fp_sparse_prefill_chunked_paged(p16, q_pre, kc, vc, bt, cu_pre, cut, pooled_cache=cache)
    q_new = torch.cat([qd[cu[b] + cut[b]:cu[b + 1]] for b in range(len(lens))])
    cu_new = [0]
    for b in range(len(lens)):
        cu_new.append(cu_new[-1] + lens[b] - cut[b])
    res = fp.fp_sparse_prefill_chunked_paged_fp8(p8, q_new, kc, vc, bt, cu_new, lens, c8, pooled_cache=cache,
                                                 prefix_pooled=True, return_lse=True)
    r16 = fp.fp_sparse_prefill_chunked_paged(p16, q_new, kc, vc, bt, cu_new, lens, pooled_cache=cache,
                                             prefix_pooled=True)
    torch.cuda.synchronize()
    assert torch.equal(res.kv_cnt, r16.kv_cnt)
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    idx8, idx16, cnt = res.kv_idx.cpu().numpy(), r16.kv_idx.cpu().numpy(), res.kv_cnt.cpu().numpy()
    k8, v8 = c8.k8.cpu(), c8.v8.cpu()
    ks, vs = c8.k_scale.cpu().numpy(), c8.v_scale.cpu().numpy()
    tri = lambda n: n * (n + 1) // 2
    io = co = 0
    for b, (L, P0) in enumerate(zip(lens, cut)):
        nb, first = (L + B - 1) // B, P0 // B
        nq, rowsz = nb - first, tri(nb) - tri(first)
        qb, kb, vb = (t.float().numpy() for t in pb.requests[b])
        pages = pb.block_table[b, :(L + page - 1) // page].tolist()
        # lists: equal to the bf16 chunked entry's, read into a mask
        mask = np.zeros((Hq, nq, nb), dtype=bool)
        for h in range(Hq):
            for i in range(nq):
                c = int(cnt[co + h * nq + i])
                s0 = io + h * rowsz + tri(first + i) - tri(first)
                assert np.array_equal(idx8[s0:s0 + c], idx16[s0:s0 + c]), (b, h, i)
                mask[h, i, idx8[s0:s0 + c]] = True
        ref = O.select_blocks_chunked(qb[P0:], kb, vb, B, alpha)
        outside, inside, band = compare_mask(mask, ref)
        assert outside == 0, (b, outside)
        # the chunk's blocks in the e4m3 pages, against the oracle's codes
        deq = {}
        pairs = _sample_pairs(Hq, nq, 8, seed=70 + b)
        need = sorted({J for h, i in pairs for J in np.nonzero(mask[h, i])[0]} | set(range(first, nb)))
        for name, pool, sc, x in (("k", k8, ks, kb), ("v", v8, vs, vb)):
            full = np.full(x.shape, np.nan)
            for J in need:                                # blockwise codes: each block on its own
                c_ref, s_ref = O.quantize_fp8_blockwise(x[J * B:(J + 1) * B], B)
                if J >= first:
                    r0 = J * B
                    got = pool[pages[r0 // page:(r0 + B + page - 1) // page]].reshape(-1, Hkv, d)
                    assert np.array_equal(got[:min(B, L - r0)].numpy(), c_ref), (b, name, J)
                    assert np.array_equal(sc[pages[r0 // page]], s_ref[:, 0]), (b, name, J)
                full[J * B:(J + 1) * B] = O.dequantize_blockwise(
                    synth.fp8_codes_to_float(torch.from_numpy(c_ref)).numpy(), s_ref, B)
            deq[name] = full
        qc, qs = O.quantize_fp8_chunk(qb[P0:], B, P0)
        q_deq = O.dequantize_chunk(synth.fp8_codes_to_float(torch.from_numpy(qc)).numpy(), qs, B, P0)
        o_ref, lse_ref = O.sparse_attention_chunked(q_deq, deq["k"], deq["v"], ref, True, keep=mask, pairs=pairs)
        worst = lworst = 0.0
        for h, i in pairs:
            r0, r1 = i * B, min(L - P0, (i + 1) * B)
            worst = max(worst, float(np.abs(out[cu_new[b] + r0:cu_new[b] + r1, h] - o_ref[r0:r1, h]).max()))
            lworst = max(lworst, float(np.abs(lse[h, cu_new[b] + r0:cu_new[b] + r1] - lse_ref[h, r0:r1]).max()))
        print(f"  request {b} L={L}: kept {int(mask.sum())}, sampled max|o-ref| {worst:.3e} "
              f"max|lse-ref| {lworst:.3e}", flush=True)
        assert worst <= FP8_TOL and lworst <= 5e-2, (b, worst, lworst)
        io += Hq * rowsz
        co += Hq * nq


@pytest.mark.parametrize("shared,probes", [(True, 0), ("pooled", 0), (False, 16)],
                         ids=["shared_lists", "pooled_lists", "skeleton16"])
def test_128k_selection_options_full_size(s128k, shared, probes):
    """The selection options, at the 128K layer's full size: group-shared
    lists (the union of a KV head's query heads' masks, or the list of the
    group-pooled query) and skeleton-query scoring (q_bar from 16 probes per
    block).  Lists match the oracle's outside the threshold band; sampled
    outputs match the oracle under the GPU's lists."""
    seq = s128k
    S, Hq, Hkv, d, B = seq.S, seq.Hq, seq.Hkv, seq.d, seq.B
    nB = S // B
    p = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, shared_selection=shared, query_probes=probes)
    qd, kd, vd = seq.gpu
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    out = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel)
    torch.cuda.synchronize()
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = seq.np
    ref = O.select_blocks(qn, kn, vn, B, 0.1, shared=shared, probes=probes)
    outside, inside, band = compare_mask(mask, ref)
    print(f"  shared={shared} probes={probes}: density {mask.sum() / (Hq * nB * (nB + 1) / 2):.4f}, "
          f"band {band}, in-band mismatches {inside}", flush=True)
    assert outside == 0
    pairs = _sample_pairs(Hq, nB, 12, seed=7 + probes)
    o_ref, _ = O.sparse_attention(qn, kn, vn, ref, True, pairs=pairs, keep=mask)
    o = out.float().cpu().numpy()
    worst = max(float(np.abs(o[I * B:(I + 1) * B, h] - o_ref[I * B:(I + 1) * B, h]).max()) for h, I in pairs)
    print(f"  {len(pairs)} sampled pairs: max|o-ref| {worst:.3e}", flush=True)
    assert worst <= BF16_TOL

"""The one-pass fp8 preparation (fp_select_blocks_fp8): its e4m3 codes and
scales equal the oracle's quantizer bit for bit, its block means equal the
oracle's to fp32 rounding and the bf16 selection's (fp_select_blocks) bit for
bit -- both kernels sum a block in the same token tree -- so its lists are the
bf16 selection's, which match the oracle's outside the threshold band; and
attention on its outputs matches the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import FP8_TOL, check_lists, compare_mask, dev

pytestmark = pytest.mark.gpu

SHAPES = [
    # S, Hq, Hkv, d, B: ragged tails, head counts that leave a workgroup's head group part-empty
    (1000, 4, 2, 128, 128),
    (1024, 3, 1, 64, 64),
    (129, 5, 5, 128, 64),
    (2048, 32, 8, 128, 128),
    (77, 6, 2, 64, 128),
]


def _prep(q, k, v, B, alpha, corr):
    S, Hq, d = q.shape
    p8 = fp.make_params(Hq, k.shape[1], d, B, alpha, mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    sel, f8 = fp.fp_select_blocks_fp8(p8, q.to(dev()), k.to(dev()), v.to(dev()))
    torch.cuda.synchronize()
    return p8, sel, f8


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s)
def test_codes_scales_and_means(shape):
    S, Hq, Hkv, d, B = shape
    print(f"fp8 prep {shape}", flush=True)
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=S + Hq, verticals=True)
    v[: min(S, B), 0] = 0                     # an all-zero (head, block): scale 1, codes 0
    _, sel, f8 = _prep(q, k, v, B, 0.1, True)
    nB = (S + B - 1) // B
    for x, c, s in ((q, f8.q8, f8.q_scale), (k, f8.k8, f8.k_scale), (v, f8.v8, f8.v_scale)):
        c_ref, s_ref = O.quantize_fp8_blockwise(x.float().numpy(), B)
        assert np.array_equal(s.cpu().numpy(), s_ref)
        got = c.cpu().numpy()
        assert np.array_equal(got, c_ref), int((got != c_ref).sum())
    assert f8.v_scale[0, 0].item() == 1.0 and not f8.v8[: min(S, B), 0].any()
    for x, m in ((q, sel.pooled_q), (k, sel.pooled_k)):
        np.testing.assert_allclose(m.cpu().numpy(), O.block_means(x.float().numpy(), B), rtol=0, atol=2e-6)
    pkv = sel.pooled_kv.float().cpu().numpy()
    for i, x in enumerate((k, v)):
        ref = O.block_means(x.float().numpy(), B)
        assert np.abs(pkv[i] - ref).max() <= np.abs(ref).max() * 2.0 ** -8 + 1e-6   # bf16 rounding of the means


@pytest.mark.parametrize("probes", [0, 16])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s)
def test_means_and_lists_equal_the_bf16_selection(shape, probes):
    """The fused pass and the pooling kernel add a block's tokens in the same
    order, so the means (fp32 and their bf16 copies), counts and lists agree
    bit for bit."""
    S, Hq, Hkv, d, B = shape
    q, k, v = (t.to(dev()) for t in synth.make_sequence(S, Hq, Hkv, d, seed=3 * S + Hq, verticals=True))
    p16 = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, query_probes=probes)
    p8 = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN, query_probes=probes)
    s16 = fp.fp_select_blocks(p16, q, k, v)
    s8, _ = fp.fp_select_blocks_fp8(p8, q, k, v)
    torch.cuda.synchronize()
    for name in ("pooled_q", "pooled_k", "pooled_kv", "kv_cnt"):
        assert torch.equal(getattr(s8, name), getattr(s16, name)), name
    nB = (S + B - 1) // B
    assert np.array_equal(fp.lists_to_mask(s8.kv_idx, s8.kv_cnt, Hq, nB), fp.lists_to_mask(s16.kv_idx, s16.kv_cnt, Hq, nB))


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.5])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("shape", SHAPES[:4], ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s)
def test_attention_on_prepared_inputs(shape, alpha, corr):
    S, Hq, Hkv, d, B = shape
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=2 * S + Hq, verticals=True)
    p8, sel, f8 = _prep(q, k, v, B, alpha, corr)
    res = fp.fp_sparse_prefill_fwd(p8, f8.q8, f8.k8, f8.v8, sel, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                   v_scale=f8.v_scale, return_lse=True)
    torch.cuda.synchronize()
    nB = (S + B - 1) // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    ref = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0, (outside, inside, band)
    deq = [O.dequantize_blockwise(O.e4m3_decode(c.cpu().numpy()), s.cpu().numpy(), B)
           for c, s in ((f8.q8, f8.q_scale), (f8.k8, f8.k_scale), (f8.v8, f8.v_scale))]
    o_ref, lse_ref = O.sparse_attention(deq[0], deq[1], deq[2], ref, corr, keep=mask)
    out, lse = res
    err = np.abs(out.float().cpu().numpy() - o_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"  {shape} alpha={alpha} corr={corr}: max|o-ref| {err:.3e} max|lse-ref| {lerr:.3e}", flush=True)
    assert err <= FP8_TOL and lerr <= 5e-2


def test_prep_with_skeleton_queries():
    S, Hq, Hkv, d, B = 1000, 4, 2, 128, 128
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=31, verticals=True)
    p8 = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN, query_probes=16)
    sel, f8 = fp.fp_select_blocks_fp8(p8, q.to(dev()), k.to(dev()), v.to(dev()))
    torch.cuda.synchronize()
    ref = O.select_blocks(q.float().numpy(), k.float().numpy(), v.float().numpy(), B, 0.2, probes=16)
    np.testing.assert_allclose(sel.pooled_q.cpu().numpy(), ref.q_bar, rtol=0, atol=2e-6)
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, (S + B - 1) // B)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0
    c_ref, s_ref = O.quantize_fp8_blockwise(q.float().numpy(), B)       # codes do not depend on the probes
    assert np.array_equal(f8.q8.cpu().numpy(), c_ref) and np.array_equal(f8.q_scale.cpu().numpy(), s_ref)


@pytest.mark.slow
def test_prep_128k_full_size_sampled():
    """The one-pass preparation at the 128K layer's full size, in the launch
    configuration the benchmark times: sampled (tensor, head, block) slices of
    the codes and scales equal the oracle's quantizer bit for bit, and the
    sampled block means equal the oracle's to fp32 rounding."""
    w = synth.WORKLOADS["llama8b_s128k"]
    S, Hq, Hkv, d, B = w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating llama8b_s128k", flush=True)
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, w.seed, w.verticals)
    _, sel, f8 = _prep(q, k, v, B, 0.1, True)
    nB = S // B
    r = np.random.default_rng(11)
    got = {"q": (f8.q8.cpu().numpy(), f8.q_scale.cpu().numpy(), sel.pooled_q.cpu().numpy()),
           "k": (f8.k8.cpu().numpy(), f8.k_scale.cpu().numpy(), sel.pooled_k.cpu().numpy()),
           "v": (f8.v8.cpu().numpy(), f8.v_scale.cpu().numpy(), None)}
    src = {"q": q, "k": k, "v": v}
    n = 0
    for name, x in src.items():
        H = x.shape[1]
        picks = {(0, 0), (H - 1, nB - 1)} | {(int(r.integers(H)), int(r.integers(nB))) for _ in range(10)}
        for h, J in sorted(picks):
            seg = x[J * B:(J + 1) * B, h:h + 1].float().numpy()          # [B, 1, d]
            c_ref, s_ref = O.quantize_fp8_blockwise(seg, B)
            codes, scales, means = got[name]
            assert scales[h, J] == s_ref[0, 0], (name, h, J)
            assert np.array_equal(codes[J * B:(J + 1) * B, h], c_ref[:, 0]), (name, h, J)
            if means is not None:
                np.testing.assert_allclose(means[h, J], O.block_means(seg, B)[0, 0], rtol=0, atol=2e-6)
            n += 1
    print(f"  {n} sampled (tensor, head, block) slices bit-exact", flush=True)

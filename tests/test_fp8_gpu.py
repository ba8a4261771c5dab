"""Parity of the fp8 (e4m3fn) attention path with the CPU oracle.

Selection runs on the bf16 data (its pooled means also feed the mean
correction); attention reads e4m3 codes with per-(head, block) fp32 scales.
The oracle evaluates attention on the dequantized codes (code * scale) under
the GPU's mask, so what is judged is the kernel's own arithmetic (fp8 P,
fp32 accumulation), to max-abs 6e-2."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import FP8_TOL, check_lists, compare_mask, dev

pytestmark = pytest.mark.gpu

SHAPES = [
    (1024, 4, 1, 64, 64),
    (1000, 4, 2, 128, 128),
    (2048, 32, 8, 128, 128),
    (300, 8, 2, 64, 128),
    (129, 2, 1, 128, 64),
]


def _run(q, k, v, B, alpha, corr, lse=True):
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    q8, sq = synth.quantize_fp8_blockwise(q, B)
    k8, sk = synth.quantize_fp8_blockwise(k, B)
    v8, sv = synth.quantize_fp8_blockwise(v, B)
    pb = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    p8 = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    sel = fp.fp_select_blocks(pb, qd, kd, vd)
    res = fp.fp_sparse_prefill_fwd(p8, q8.to(dev()), k8.to(dev()), v8.to(dev()), sel,
                                   q_scale=sq.to(dev()), k_scale=sk.to(dev()), v_scale=sv.to(dev()),
                                   return_lse=lse)
    torch.cuda.synchronize()
    deq = tuple(O.dequantize_blockwise(synth.fp8_codes_to_float(c).numpy(), s.numpy(), B)
                for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    return sel, res, deq


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.5])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s)
def test_fp8_matches_oracle(shape, alpha, corr):
    S, Hq, Hkv, d, B = shape
    print(f"fp8 {shape} alpha={alpha} corr={corr}", flush=True)
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=S + 3 * Hq, verticals=True)
    sel, (out, lse), (qd8, kd8, vd8) = _run(q, k, v, B, alpha, corr)
    nB = (S + B - 1) // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    ref = O.select_blocks(qn, kn, vn, B, alpha)             # selection on the bf16 data
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0
    o_ref, lse_ref = O.sparse_attention(qd8, kd8, vd8, ref, corr, keep=mask)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    err = np.abs(o - o_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"  max|o-ref| {err:.3e}  max|lse-ref| {lerr:.3e}", flush=True)
    assert err <= FP8_TOL
    assert lerr <= 5e-2


def test_fp8_constant_v():
    """Constant V gives that constant for every row.  The entries +-3 * 2^-k
    are exact in bf16 and (up to the fp32 rounding of the scale 3/448) in
    e4m3, so the correction's pooled means equal the dequantized values too."""
    S, Hq, Hkv, d, B = 1100, 8, 2, 128, 128
    q, k, _ = synth.make_sequence(S, Hq, Hkv, d, seed=4, verticals=True)
    j = torch.arange(d)
    c = (3.0 * torch.where(j % 2 == 0, 1.0, -1.0) * 2.0 ** (-(j % 8).float())).to(torch.bfloat16)
    v = c.expand(S, Hkv, d).contiguous()
    for alpha in (0.0, 0.3):
        for corr in (True, False):
            _, out, (_, _, vd8) = _run(q, k, v, B, alpha, corr, lse=False)
            np.testing.assert_allclose(vd8[0, 0], c.float().numpy(), rtol=1e-6)
            np.testing.assert_allclose(out.float().cpu().numpy(),
                                       np.broadcast_to(c.float().numpy(), (S, Hq, d)), atol=2e-2)


@pytest.mark.slow
def test_fp8_128k_full_size():
    w = synth.WORKLOADS["llama8b_s128k_fp8"]
    S, Hq, Hkv, d, B = w.seqlens[0], w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print("generating llama8b_s128k_fp8", flush=True)
    inp = synth.workload_inputs(w)
    pb = fp.make_params(Hq, Hkv, d, B, w.alphas[0], mean_correction=True)
    p8 = fp.make_params(Hq, Hkv, d, B, w.alphas[0], mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    qd, kd, vd = (inp[n].to(dev()) for n in ("q", "k", "v"))
    sel = fp.fp_select_blocks(pb, qd, kd, vd)
    out, lse = fp.fp_sparse_prefill_fwd(p8, inp["q8"].to(dev()), inp["k8"].to(dev()), inp["v8"].to(dev()),
                                        sel, q_scale=inp["q_scale"].to(dev()), k_scale=inp["k_scale"].to(dev()),
                                        v_scale=inp["v_scale"].to(dev()), return_lse=True)
    torch.cuda.synchronize()
    nB = S // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
    ref = O.select_blocks(qn, kn, vn, B, w.alphas[0])
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0
    deq = [O.dequantize_blockwise(synth.fp8_codes_to_float(inp[n + "8"]).numpy(), inp[n + "_scale"].numpy(), B)
           for n in ("q", "k", "v")]
    # every query head (each XCD's heads) and query blocks across the whole
    # sequence: 64 pairs, plus the first and last blocks
    r = np.random.default_rng(4)
    pairs = sorted({(0, 0), (Hq - 1, nB - 1), (5, nB // 2)} |
                   {(k % Hq, int(r.integers(k * nB // 64, (k + 1) * nB // 64))) for k in range(64)})
    o_ref, lse_ref = O.sparse_attention(deq[0], deq[1], deq[2], ref, True, pairs=pairs, keep=mask)
    o = out.float().cpu().numpy()
    worst = max(float(np.abs(o[I * B:(I + 1) * B, h] - o_ref[I * B:(I + 1) * B, h]).max()) for h, I in pairs)
    print(f"  fp8 128K: {len(pairs)} sampled pairs, max|o-ref| {worst:.3e}", flush=True)
    assert worst <= FP8_TOL

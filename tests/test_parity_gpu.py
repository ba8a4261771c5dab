"""Parity of the HIP path (through the C-ABI) with the CPU oracle on seeded
inputs at small sizes: pooled means, masks (bit-exact outside the 1e-3
threshold band), outputs (max-abs 2e-2 for bf16) and log-sum-exp."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O
from block_sparse_long_pooling_amd import synth

from gpu_util import (BF16_TOL, LSE_TOL, check_lists, compare_mask, dev, oracle_inputs,
                      run_single)

pytestmark = pytest.mark.gpu

SHAPES = [
    # S, Hq, Hkv, d, B, verticals
    (1024, 4, 1, 64, 64, False),       # the tiny workload's shape
    (1000, 4, 2, 128, 128, True),      # ragged tail
    (300, 8, 2, 64, 64, False),
    (77, 2, 1, 128, 64, False),
    (129, 4, 4, 128, 128, False),      # one full block + 1 token
    (1, 1, 1, 64, 64, False),          # single token
    (2048, 32, 8, 128, 128, True),     # Llama-3-8B head shape, 16 blocks
    (640, 6, 3, 64, 128, True),
]


def _case(S, Hq, Hkv, d, B, verticals, seed=0):
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=S * 7 + Hq + seed, verticals=verticals)
    return q, k, v


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s[:5])
def test_pooled_means(shape):
    S, Hq, Hkv, d, B, vert = shape
    print(f"pooled means {shape}", flush=True)
    q, k, v = _case(*shape)
    sel, _ = run_single(q, k, v, B, 0.1, correction=True, lse=False)
    qn, kn, vn = oracle_inputs(q, k, v)
    for got, x in ((sel.pooled_q, qn), (sel.pooled_k, kn), (sel.pooled_v, vn)):
        ref = O.block_means(x, B)
        np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=0, atol=2e-6 * max(1.0, np.abs(ref).max()))
    # The bf16 copies are the fp32 means rounded to nearest even, bit for bit.
    for i, got32 in enumerate((sel.pooled_k, sel.pooled_v)):
        assert torch.equal(sel.pooled_kv[i].cpu(), got32.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.3, 0.5, 0.9, 1.0])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s[:5])
def test_mask_and_output(shape, alpha, corr):
    S, Hq, Hkv, d, B, vert = shape
    print(f"parity {shape} alpha={alpha} corr={corr}", flush=True)
    q, k, v = _case(*shape)
    sel, (out, lse) = run_single(q, k, v, B, alpha, correction=corr)
    nB = (S + B - 1) // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    qn, kn, vn = oracle_inputs(q, k, v)
    ref = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0, f"{outside} mask mismatches outside the band (inside {inside}/{band})"
    if alpha == 0.0:
        assert mask.sum() == Hq * nB * (nB + 1) // 2
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, ref, corr, keep=mask)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    err = np.abs(o - o_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"  kept {int(mask.sum())} max|o-ref|={err:.3e} max|lse-ref|={lerr:.3e}", flush=True)
    assert err <= BF16_TOL
    assert lerr <= LSE_TOL


def test_deterministic():
    q, k, v = _case(2048, 32, 8, 128, 128, True)
    a_sel, (a_o, a_l) = run_single(q, k, v, 128, 0.2)
    b_sel, (b_o, b_l) = run_single(q, k, v, 128, 0.2)
    assert torch.equal(a_sel.kv_cnt, b_sel.kv_cnt)
    assert np.array_equal(check_lists(a_sel.kv_idx, a_sel.kv_cnt, 32, 16),
                          check_lists(b_sel.kv_idx, b_sel.kv_cnt, 32, 16))
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


def test_constant_v_gives_constant_output():
    S, Hq, Hkv, d, B = 1500, 8, 2, 128, 128
    q, k, _ = _case(S, Hq, Hkv, d, B, True)
    c = torch.linspace(-2, 2, d).to(torch.bfloat16)
    v = c.expand(S, Hkv, d).contiguous()
    for alpha in (0.0, 0.3, 1.0):
        _, (out, _) = run_single(q, k, v, B, alpha)
        np.testing.assert_allclose(out.float().cpu().numpy(),
                                   np.broadcast_to(c.float().numpy(), (S, Hq, d)), atol=2e-2)


def test_dense_alpha0_matches_torch_sdpa():
    """alpha = 0 keeps every causal block: compare with torch's own causal
    attention (fp32 on the GPU, K/V expanded to the query heads)."""
    S, Hq, Hkv, d, B = 1200, 8, 2, 128, 128
    q, k, v = _case(S, Hq, Hkv, d, B, True)
    _, out = run_single(q, k, v, B, 0.0, correction=True, lse=False)
    g = Hq // Hkv
    Q = q.to(dev()).float().permute(1, 0, 2)[None]
    K = k.to(dev()).float().repeat_interleave(g, dim=1).permute(1, 0, 2)[None].contiguous()
    V = v.to(dev()).float().repeat_interleave(g, dim=1).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].permute(1, 0, 2)
    assert (out.float() - ref).abs().max().item() <= BF16_TOL


def test_errors_leave_outputs_untouched():
    """Invalid arguments return a status and launch nothing."""
    q, k, v = _case(256, 4, 2, 64, 64, False)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    p = fp.make_params(4, 2, 64, 64, 1.5)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_select_blocks(p, qd, kd, vd)
    assert e.value.status == fp.FP_INVALID_ARGUMENT
    p = fp.make_params(4, 2, 96, 64, 0.5)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_select_blocks(p, qd, kd, vd)
    assert e.value.status == fp.FP_UNSUPPORTED


@pytest.mark.parametrize("mode", ["union", "pooled"])
@pytest.mark.parametrize("alpha", [0.1, 0.4, 0.9])
@pytest.mark.parametrize("shape", [SHAPES[1], SHAPES[2], SHAPES[6], SHAPES[7]],
                         ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s[:5])
def test_shared_selection(shape, alpha, mode):
    """Group-shared selection: one list per KV head (the union of its query
    heads' lists, or the list of the group-pooled query), identical for the
    g heads, equal to the oracle's outside the threshold band, and attention
    on it matches the oracle."""
    S, Hq, Hkv, d, B, vert = shape
    print(f"shared selection {shape} alpha={alpha} mode={mode}", flush=True)
    q, k, v = _case(*shape, seed=5)
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True, shared_selection=mode)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    out, lse = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, return_lse=True)
    torch.cuda.synchronize()
    nB = (S + B - 1) // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    g = Hq // Hkv
    for hk in range(Hkv):
        assert (mask[hk * g:(hk + 1) * g] == mask[hk * g]).all()
    qn, kn, vn = oracle_inputs(q, k, v)
    ref = O.select_blocks(qn, kn, vn, B, alpha, shared=mode)
    own = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0, (outside, inside, band)
    if mode == "union":
        assert (mask | ~own.keep | own.band).all()          # covers every head's own mask
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, ref, True, keep=mask)
    err = np.abs(out.float().cpu().numpy() - o_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"  kept {int(mask.sum())} (own {int(own.keep.sum())}) err {err:.3e} lse {lerr:.3e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("probes", [1, 8, 0])
@pytest.mark.parametrize("shape", [SHAPES[1], SHAPES[3], SHAPES[6]], ids=lambda s: "S%d_h%d-%d_d%d_B%d" % s[:5])
def test_skeleton_queries(shape, probes):
    """q_bar from the skeleton queries (every (B/P)-th query of a block):
    pooled means, masks and outputs match the oracle with the same probes."""
    S, Hq, Hkv, d, B, vert = shape
    print(f"skeleton queries {shape} probes={probes}", flush=True)
    q, k, v = _case(*shape, seed=9)
    p = fp.make_params(Hq, Hkv, d, B, 0.2, mean_correction=True, query_probes=probes)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    out, lse = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = oracle_inputs(q, k, v)
    ref = O.select_blocks(qn, kn, vn, B, 0.2, probes=probes)
    np.testing.assert_allclose(sel.pooled_q.cpu().numpy(), ref.q_bar, rtol=0, atol=2e-6 * max(1.0, np.abs(ref.q_bar).max()))
    nB = (S + B - 1) // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    outside, inside, band = compare_mask(mask, ref)
    assert outside == 0, (outside, inside, band)
    o_ref, lse_ref = O.sparse_attention(qn, kn, vn, ref, True, keep=mask)
    err = np.abs(out.float().cpu().numpy() - o_ref).max()
    lerr = np.abs(lse.cpu().numpy() - lse_ref).max()
    print(f"  kept {int(mask.sum())} err {err:.3e} lse {lerr:.3e}", flush=True)
    assert err <= BF16_TOL and lerr <= LSE_TOL

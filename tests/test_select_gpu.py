"""Selection at many column tiles: lists against the oracle's masks.

The selection kernel streams the pooled keys in tiles of 32 blocks, two per
step, from the last tile to the first, thresholds every tile against the
row's running max, and scores a tile again only where a row's bits were set
before its max last grew.
These cases span several steps, head-group sizes that do not divide 32
(unused score rows), one and many query heads per KV head, both head
dimensions and both block sizes, a ragged last block and the dense and
max-only thresholds, per-head lists and both group-shared forms (union and
group-pooled query).  Every (h, I, J) entry must match the oracle outside
the near-threshold band (FlashPrefill, gist.science technical summary,
sections 2.A-2.C).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import synth
from oracle import flashprefill_oracle as O

from gpu_util import BF16_TOL, FP8_TOL, check_lists, compare_mask, dev, oracle_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # S, Hq, Hkv, d, B
    (9600, 6, 2, 64, 64),        # g = 3: 30 of 32 score rows used, 150 blocks
    (12000, 8, 1, 128, 128),     # g = 8, ragged last block
    (8229, 2, 2, 64, 64),        # g = 1: 32 query blocks per row wave, ragged
    (6000, 12, 2, 128, 64),      # g = 6: 30 rows used
    (20000, 32, 1, 64, 128),     # g = 32: one query block per row wave
    (16384, 4, 1, 128, 64),      # 256 blocks: eight column tiles
]


def _ids(c):
    return "S%d_h%d-%d_d%d_B%d" % c


@pytest.fixture(scope="module", params=CASES, ids=_ids)
def case(request):
    S, Hq, Hkv, d, B = request.param
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=S + 13 * Hq + d, verticals=True)
    print(f"case {_ids(request.param)}", flush=True)
    return request.param, (q, k, v), tuple(t.to(dev()) for t in (q, k, v)), oracle_inputs(q, k, v)


@pytest.mark.parametrize("shared", [False, True, "pooled"], ids=["own", "union", "pooled"])
@pytest.mark.parametrize("alpha", [0.0, 0.05, 0.3, 1.0])
def test_lists_match_oracle(case, alpha, shared):
    (S, Hq, Hkv, d, B), _, (qd, kd, vd), (qn, kn, vn) = case
    nB = (S + B - 1) // B
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=False, shared_selection=shared)
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    torch.cuda.synchronize()
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    ref = O.select_blocks(qn, kn, vn, B, alpha, pool_v=False, shared=shared)
    outside, inside, band = compare_mask(mask, ref)
    print(f"  alpha={alpha} shared={shared}: density {mask.sum() / (Hq * nB * (nB + 1) / 2):.4f}, "
          f"band {band}, in-band mismatches {inside}", flush=True)
    assert outside == 0
    if alpha == 0.0:
        assert mask.sum() == Hq * nB * (nB + 1) // 2          # every causal block
    if shared:
        g = Hq // Hkv
        grouped = mask.reshape(Hkv, g, nB, nB)
        assert (grouped == grouped[:, :1]).all()               # one list per KV head


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_maximum_blocks_per_request(fp8):
    """A request at the largest supported block count (4096 blocks of 64
    tokens, 262,144 tokens): 128 column tiles per row in the selection
    kernel, full-length kept-block bitmaps in attention; bf16, and fp8 with
    the fused preparation.  Lists match the oracle outside the band (fp8
    selection is on the bf16 data); sampled outputs match the oracle under
    the GPU's lists (for fp8, on the dequantized codes)."""
    S, Hq, Hkv, d, B, alpha = 4096 * 64, 2, 1, 64, 64, 0.1
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=77, verticals=True)
    print(f"case S={S} Hq={Hq} Hkv={Hkv} d={d} B={B} fp8={fp8}", flush=True)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    qn, kn, vn = oracle_inputs(q, k, v)
    if fp8:
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True, dtype=fp.FP_DTYPE_FP8_E4M3FN)
        sel, f8 = fp.fp_select_blocks_fp8(p, qd, kd, vd)
        out = fp.fp_sparse_prefill_fwd(p, f8.q8, f8.k8, f8.v8, sel, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                       v_scale=f8.v_scale)
        att = [O.dequantize_blockwise(synth.fp8_codes_to_float(c.cpu()).numpy(), sc.cpu().numpy(), B)
               for c, sc in ((f8.q8, f8.q_scale), (f8.k8, f8.k_scale), (f8.v8, f8.v_scale))]
        tol = FP8_TOL
    else:
        p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True)
        sel = fp.fp_select_blocks(p, qd, kd, vd)
        out = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel)
        att = [qn, kn, vn]
        tol = BF16_TOL
    torch.cuda.synchronize()
    nB = S // B
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    ref = O.select_blocks(qn, kn, vn, B, alpha)
    outside, inside, band = compare_mask(mask, ref)
    print(f"  density {mask.sum() / (Hq * nB * (nB + 1) / 2):.4f}, band {band}, in-band mismatches {inside}",
          flush=True)
    assert outside == 0
    pairs = [(0, 0), (1, nB - 1), (0, nB - 1), (1, 2048), (0, 4000), (1, 63)]
    o_ref, _ = O.sparse_attention(att[0], att[1], att[2], ref, True, pairs=pairs, keep=mask)
    o = out.float().cpu().numpy()
    worst = max(float(np.abs(o[I * B:(I + 1) * B, h] - o_ref[I * B:(I + 1) * B, h]).max()) for h, I in pairs)
    print(f"  {len(pairs)} sampled pairs: max|o-ref| {worst:.3e}", flush=True)
    assert worst <= tol


@pytest.mark.parametrize("alpha", [0.05, 0.3, 1.0])
@pytest.mark.parametrize("layout", ["scattered", "first", "mixed"])
def test_row_max_away_from_diagonal(layout, alpha):
    """Rows whose largest block score lies away from their diagonal tile, so
    the selection kernel meets it late in its last-to-first walk and must
    score earlier tiles again.  Query head j shares a direction u_j with the
    keys, which carry a_jJ u_j in block J: a_jJ random per block
    ("scattered"), falling from block 0 ("first": the max is always the
    first block, met last), or per head ("mixed": rising for head 0, whose
    max is on the diagonal, falling for head 1, random for heads 2 and 3, so
    rows of one row wave differ in whether they are scored again).  The u_j
    are orthogonal.  256 blocks of 64 tokens = 8 column tiles."""
    S, Hq, Hkv, d, B = 16384, 4, 1, 128, 64
    nB = S // B
    gen = torch.Generator().manual_seed({"scattered": 41, "first": 42, "mixed": 43}[layout])
    U = torch.zeros(Hq, d)
    for j in range(Hq):
        U[j, 32 * j:32 * (j + 1)] = 2.0                      # orthogonal, |u_j|^2 = 128
    if layout == "scattered":
        A = torch.rand(nB, generator=gen).repeat(Hq, 1)
    elif layout == "first":
        A = torch.linspace(1.0, 0.0, nB).repeat(Hq, 1)
    else:
        A = torch.stack([torch.linspace(0.0, 1.0, nB), torch.linspace(1.0, 0.0, nB),
                         torch.rand(nB, generator=gen), torch.rand(nB, generator=gen)])
    A = 4.0 * A          # head 0's max lies in its diagonal tile in 99% of rows (mixed), head 1's in tile 0
    q = (U[None] + torch.randn(S, Hq, d, generator=gen)).to(torch.bfloat16)
    kdir = (A.t()[:, :, None] * U[None]).sum(1)              # [nB, d]
    k = (kdir.repeat_interleave(B, 0)[:, None, :] + torch.randn(S, Hkv, d, generator=gen)).to(torch.bfloat16)
    v = torch.randn(S, Hkv, d, generator=gen).to(torch.bfloat16)
    print(f"case {layout} alpha={alpha}", flush=True)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    qn, kn, vn = oracle_inputs(q, k, v)
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=False)
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    torch.cuda.synchronize()
    mask = check_lists(sel.kv_idx, sel.kv_cnt, Hq, nB)
    ref = O.select_blocks(qn, kn, vn, B, alpha, pool_v=False)
    outside, inside, band = compare_mask(mask, ref)
    print(f"  density {mask.sum() / (Hq * nB * (nB + 1) / 2):.4f}, band {band}, in-band mismatches {inside}",
          flush=True)
    assert outside == 0
    assert 0 < mask.sum() < Hq * nB * (nB + 1) // 2

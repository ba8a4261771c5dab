"""Selection at many column tiles: lists against the oracle's masks.

The selection kernel streams the pooled keys in tiles of 32 blocks, two per
step, and scores a tile again only where some row can keep a block in it.
These cases span several steps, head-group sizes that do not divide 32
(unused score rows), one and many query heads per KV head, both head
dimensions and both block sizes, a ragged last block and the dense and
max-only thresholds.  Every (h, I, J) entry must match the oracle outside
the near-threshold band (FlashPrefill, gist.science technical summary,
sections 2.A-2.C).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import synth
from oracle import flashprefill_oracle as O

from gpu_util import check_lists, compare_mask, dev, oracle_inputs

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


@pytest.mark.parametrize("shared", [False, True])
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

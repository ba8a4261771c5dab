"""Launch configuration of the persistent attention kernel (GPU): every
kernel variant gets the grid its own occupancy allows, whichever variant a
process launches first."""
import pytest
import torch

import block_sparse_long_pooling_amd as fp


@pytest.mark.gpu
def test_persistent_grid_per_variant():
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    cu = [0, 1 << 17]
    small = fp.make_params(4, 1, 64, 64, 0.1)        # d 64, block 64: small LDS tiles
    big = fp.make_params(32, 8, 128, 128, 0.1)       # d 128, block 128: 128 KiB of LDS tiles
    a1 = fp.fp_attention_workgroups(small, cu)
    b1 = fp.fp_attention_workgroups(big, cu)
    a2 = fp.fp_attention_workgroups(small, cu)
    b2 = fp.fp_attention_workgroups(big, cu)
    bp = fp.fp_attention_workgroups(big, cu, paged=True)
    print(f"grids: d64/B64 {a1}, d128/B128 {b1} (paged {bp}), {ncu} CUs", flush=True)
    assert (a1, b1) == (a2, b2)
    for n in (a1, b1, bp):
        assert n > 0 and n % 8 == 0 and n <= 8 * ncu
    # the d128/B128 kernel holds one workgroup per CU (four 32 KiB tiles)
    assert b1 == ncu // 8 * 8 and bp == b1
    # the d64/B64 variant fits several per CU, so it must not inherit that grid
    assert a1 > b1
    # fp8 launches one workgroup per (query block, head)
    p8 = fp.make_params(32, 8, 128, 128, 0.1, dtype=fp.FP_DTYPE_FP8_E4M3FN)
    assert fp.fp_attention_workgroups(p8, cu) == 32 * (cu[1] // 128)

"""The entries only enqueue kernels on the caller's stream (no allocation,
no memset, no host synchronisation), so a serving loop can capture a whole
layer's selection and attention in a HIP graph and replay it.  Each replay
must equal the eager result bit for bit, with eager work and
synchronisations between replays, and a replay after the inputs change in
place must follow them."""
import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import synth

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _capture(step):
    """Warm up on a side stream, then capture one call of step()."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = step()
    torch.cuda.synchronize()
    return g, res


def _replays_match(g, outputs, reference, clobber, n=3):
    for rep in range(n):
        clobber()                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, ref in zip(("out", "lse", "kv_cnt", "kv_idx"), outputs, reference):
            assert torch.equal(x, ref), (rep, name)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_single_sequence_step_replays(fp8):
    S, Hq, Hkv, d, B = 4096 + 77, 8, 2, 128, 128
    print(f"graph single sequence fp8={fp8}", flush=True)
    q, k, v = synth.make_sequence(S, Hq, Hkv, d, seed=91, verticals=True)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    dtype = fp.FP_DTYPE_FP8_E4M3FN if fp8 else fp.FP_DTYPE_BF16
    p = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, dtype=dtype)
    if fp8:
        sel, f8 = fp.fp_select_blocks_fp8(p, qd, kd, vd)
    else:
        sel, f8 = fp.alloc_selection(p, S, dev()), None
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((Hq, S), dtype=torch.float32, device=dev())

    def step():
        if fp8:
            fp.fp_select_blocks_fp8(p, qd, kd, vd, sel=sel, f8=f8)
            fp.fp_sparse_prefill_fwd(p, f8.q8, f8.k8, f8.v8, sel, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                     v_scale=f8.v_scale, out=out, lse=lse)
        else:
            fp.fp_select_blocks(p, qd, kd, vd, sel=sel)
            fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    outputs = (out, lse, sel.kv_cnt, sel.kv_idx)
    reference = tuple(x.clone() for x in outputs)
    g, _ = _capture(step)

    def clobber():
        out.zero_()
        lse.fill_(-1.0)
        sel.kv_cnt.zero_()

    _replays_match(g, outputs, reference, clobber)
    # new inputs in place: the replay computes on them, as an eager call does
    q2, k2, v2 = synth.make_sequence(S, Hq, Hkv, d, seed=92, verticals=True)
    qd.copy_(q2.to(dev()))
    kd.copy_(k2.to(dev()))
    vd.copy_(v2.to(dev()))
    g.replay()
    torch.cuda.synchronize()
    replayed = tuple(x.clone() for x in outputs)
    assert not torch.equal(replayed[0], reference[0])
    step()
    torch.cuda.synchronize()
    for name, x, ref in zip(("out", "lse", "kv_cnt", "kv_idx"), outputs, replayed):
        assert torch.equal(x, ref), name


def test_paged_batch_step_replays():
    lengths, Hq, Hkv, d, B, page = [3000, 700, 128, 1500], 8, 2, 128, 128, 64
    print(f"graph paged batch {lengths}", flush=True)
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=93, verticals=True, page_size=page)
    p = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True)
    qd, kc, vc, bt = (x.to(dev()) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    ref = fp.fp_sparse_prefill_varlen_paged(p, qd, kc, vc, bt, pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    reference = (ref.out.clone(), ref.lse.clone(), ref.kv_cnt.clone())

    def step():
        return fp.fp_sparse_prefill_varlen_paged(p, qd, kc, vc, bt, pb.cu_seqlens, return_lse=True)

    g, res = _capture(step)

    def clobber():
        res.out.zero_()
        res.lse.fill_(-1.0)
        res.kv_cnt.zero_()

    _replays_match(g, (res.out, res.lse, res.kv_cnt), reference, clobber)

"""The allocation-free paged entry (fp_sparse_prefill_varlen_paged_noalloc)
against the entry that takes a caller's workspace: same lists, outputs and
LSE, bit for bit, on calls in a row whose inputs shrink (the library's
scratch keeps the previous call's contents, which must not leak into the
next).  The workspace entry itself is checked against the oracle by the
paged parity tests; equality with it carries that bar over."""
import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import synth

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _both(pb, Hq, Hkv, d, B, alpha, corr):
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=corr)
    q, kc, vc, bt = (x.to(_dev()) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    T = q.shape[0]
    cap = fp.fp_index_capacity(p, pb.cu_seqlens)
    ncnt = fp.fp_count_entries(p, pb.cu_seqlens)
    out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=_dev())
    lse = torch.empty((Hq, T), dtype=torch.float32, device=_dev())
    kv_idx = torch.full((cap,), -1, dtype=torch.int32, device=_dev())
    kv_cnt = torch.full((ncnt,), -1, dtype=torch.int32, device=_dev())
    fp.fp_sparse_prefill_varlen_paged_noalloc(p, q, kc, vc, bt, pb.cu_seqlens, out, kv_idx, kv_cnt, lse)
    ref = fp.fp_sparse_prefill_varlen_paged(p, q, kc, vc, bt, pb.cu_seqlens, return_lse=True)
    torch.cuda.synchronize()
    # lists: the workspace entry's counts and, per row, its first count entries
    assert torch.equal(kv_cnt, ref.kv_cnt[:ncnt])
    return out, lse, kv_idx, kv_cnt, ref


def _lists_equal(kv_idx, ref_idx, kv_cnt, lengths, Hq, B):
    idx, ridx, cnt = kv_idx.cpu(), ref_idx.cpu(), kv_cnt.cpu()
    io = co = 0
    for L in lengths:
        nb = (L + B - 1) // B
        for h in range(Hq):
            for I in range(nb):
                c = int(cnt[co + h * nb + I])
                o = io + h * nb * (nb + 1) // 2 + I * (I + 1) // 2
                if not torch.equal(idx[o:o + c], ridx[o:o + c]):
                    return False
        io += Hq * nb * (nb + 1) // 2
        co += Hq * nb
    return True


CALLS = [
    # lengths, Hq, Hkv, d, B, page, alpha, correction
    ([3000, 700, 129, 4096, 1500], 8, 2, 128, 128, 64, 0.15, True),
    ([513, 64], 8, 2, 128, 128, 32, 0.3, True),
    ([200], 4, 1, 64, 64, 16, 0.2, False),
]


def test_noalloc_equals_workspace_entry_on_shrinking_calls():
    for lengths, Hq, Hkv, d, B, page, alpha, corr in CALLS:
        print(f"noalloc: lengths {lengths} Hq {Hq} Hkv {Hkv} d {d} B {B} page {page} alpha {alpha} corr {corr}",
              flush=True)
        pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=1300 + len(lengths), verticals=True,
                                    page_size=page)
        out, lse, kv_idx, kv_cnt, ref = _both(pb, Hq, Hkv, d, B, alpha, corr)
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref.out)
        assert torch.equal(lse, ref.lse)
        assert _lists_equal(kv_idx, ref.kv_idx, kv_cnt, lengths, Hq, B)


def test_noalloc_full_size_paged_batch_then_smaller():
    """The 8-request batch at full size (307,200 tokens, 59 MB of pooled
    means, within the 64 MiB scratch), then a smaller batch."""
    w = synth.WORKLOADS["paged_batch8"]
    print("noalloc: paged_batch8 full size", flush=True)
    pb = synth.workload_inputs(w, keep_requests=False)
    p = fp.make_params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, 0.1)
    assert fp.fp_varlen_workspace_bytes(p, pb.cu_seqlens) <= fp.FP_NOALLOC_SCRATCH_BYTES
    out, lse, kv_idx, kv_cnt, ref = _both(pb, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, 0.1, True)
    assert torch.equal(out, ref.out) and torch.equal(lse, ref.lse)
    del pb, out, lse, kv_idx, kv_cnt, ref
    lengths = [4096, 1000]
    print(f"noalloc: then {lengths}", flush=True)
    pb = synth.make_paged_batch(lengths, 32, 8, 128, seed_base=1400, verticals=True, page_size=64)
    out, lse, kv_idx, kv_cnt, ref = _both(pb, 32, 8, 128, 128, 0.1, True)
    assert torch.equal(out, ref.out) and torch.equal(lse, ref.lse)
    assert _lists_equal(kv_idx, ref.kv_idx, kv_cnt, lengths, 32, 128)

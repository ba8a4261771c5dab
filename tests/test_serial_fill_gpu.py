"""LDS race check: the library against its debug variant whose kernels fill a
tile buffer (by DMA or from registers) only after every wave has finished
reading the tile before it (built with FP_SERIAL_DMA=1).  Both run the same
arithmetic in the same order, so every output -- lists, counts, pooled
means, O, LSE, fp8 codes -- must be bit-identical; a fill that raced with a
read in the pipelined kernels would show as a difference.  The cases span
the bf16 kernel at block sizes 128 and 64 (thousands of workgroups, kept
and correction tiles, a last block of at most 64 tokens, the 32-key tiles
of d = 128 at block size 64), the paged and
chunked walks, and the fp8 kept and correction pipelines."""
import contextlib
import ctypes
import os

import pytest
import torch

import block_sparse_long_pooling_amd as fp
from block_sparse_long_pooling_amd import build, synth

from gpu_util import dev

pytestmark = pytest.mark.gpu

FP8 = fp.FP_DTYPE_FP8_E4M3FN


@contextlib.contextmanager
def serial_library():
    """Route the binding through libflashprefill_serial.so for the block."""
    if not os.path.exists(build.SERIAL_LIB):
        raise RuntimeError(f"{build.SERIAL_LIB} is missing: build it with __graft_entry__.build()")
    with open(build.SERIAL_LIB, "rb") as f1, open(fp.LIB_PATH, "rb") as f2:
        assert f1.read() != f2.read(), "the serial variant is the same build as the library"
    main = fp.lib()
    ser = ctypes.CDLL(build.SERIAL_LIB)
    for name, (res, args) in fp.EXPORTS.items():
        fn = getattr(ser, name)
        fn.restype = res
        fn.argtypes = args
    fp._lib = ser
    try:
        yield
    finally:
        torch.cuda.synchronize()
        fp._lib = main


def _both(run):
    """run() under the pipelined library, then under the serial one."""
    a = run()
    torch.cuda.synchronize()
    with serial_library():
        b = run()
        torch.cuda.synchronize()
    return a, b


def _equal(a, b, what):
    for name in a:
        if a[name] is None:
            continue
        assert torch.equal(a[name], b[name]), (what, name)


@pytest.mark.parametrize("S,Hq,Hkv,d,B,alpha", [
    (16384, 32, 8, 128, 128, 0.1),     # 4096 workgroups
    (16384, 32, 8, 128, 128, 0.0),     # every block kept
    (16420, 8, 2, 128, 128, 0.2),      # last block of 36 tokens: one 64-key tile
    (5000, 4, 1, 64, 64, 0.3),         # ragged last block, block size 64
    (3000, 8, 2, 128, 64, 0.2),        # d 128 at block size 64: 32-key tiles
])
def test_bf16_single_sequence_serial_equals_pipelined(S, Hq, Hkv, d, B, alpha):
    print(f"serial fill bf16 S={S} Hq={Hq} d={d} B={B} alpha={alpha}", flush=True)
    q, k, v = (t.to(dev()) for t in synth.make_sequence(S, Hq, Hkv, d, seed=21, verticals=True))
    p = fp.make_params(Hq, Hkv, d, B, alpha, mean_correction=True)

    def run():
        sel = fp.fp_select_blocks(p, q, k, v)
        out, lse = fp.fp_sparse_prefill_fwd(p, q, k, v, sel, return_lse=True)
        mask = fp.lists_to_mask(sel.kv_idx, sel.kv_cnt, Hq, (S + B - 1) // B)   # slots past a count are unwritten
        return {"mask": torch.as_tensor(mask), "cnt": sel.kv_cnt, "pk": sel.pooled_k, "out": out, "lse": lse}

    a, b = _both(run)
    _equal(a, b, "bf16")


def test_fp8_single_sequence_serial_equals_pipelined():
    S, Hq, Hkv, d, B = 16384, 32, 8, 128, 128
    q, k, v = (t.to(dev()) for t in synth.make_sequence(S, Hq, Hkv, d, seed=22, verticals=True))
    p = fp.make_params(Hq, Hkv, d, B, 0.1, mean_correction=True, dtype=FP8)

    def run():
        sel, f8 = fp.fp_select_blocks_fp8(p, q, k, v)
        out, lse = fp.fp_sparse_prefill_fwd(p, f8.q8, f8.k8, f8.v8, sel, q_scale=f8.q_scale, k_scale=f8.k_scale,
                                            v_scale=f8.v_scale, return_lse=True)
        mask = fp.lists_to_mask(sel.kv_idx, sel.kv_cnt, Hq, S // B)
        return {"mask": torch.as_tensor(mask), "cnt": sel.kv_cnt, "k8": f8.k8, "ks": f8.k_scale, "out": out,
                "lse": lse}

    a, b = _both(run)
    _equal(a, b, "fp8")


def test_paged_and_chunked_serial_equal_pipelined():
    lengths, Hq, Hkv, d, B, page = [3000, 700, 129, 9000], 8, 2, 128, 128, 64
    pb = synth.make_paged_batch(lengths, Hq, Hkv, d, seed_base=23, verticals=True, page_size=page)
    qd, kc, vc, bt = (x.to(dev()) for x in (pb.q, pb.k_cache, pb.v_cache, pb.block_table))
    p16 = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True)
    p8 = fp.make_params(Hq, Hkv, d, B, 0.15, mean_correction=True, dtype=FP8)
    starts = [1001, 640, 0, 8100]                      # chunk starts, aligned or not
    q2 = torch.cat([pb.requests[b][0][P0:] for b, P0 in enumerate(starts)]).to(dev())
    cu2 = [0]
    for b, P0 in enumerate(starts):
        cu2.append(cu2[-1] + lengths[b] - P0)

    def run():
        r = fp.fp_sparse_prefill_varlen_paged(p16, qd, kc, vc, bt, pb.cu_seqlens, return_lse=True)
        r8, c8 = fp.fp_sparse_prefill_varlen_paged_fp8(p8, qd, kc, vc, bt, pb.cu_seqlens, return_lse=True)
        rc = fp.fp_sparse_prefill_chunked_paged(p16, q2, kc, vc, bt, cu2, lengths, return_lse=True)
        rc8 = fp.fp_sparse_prefill_chunked_paged_fp8(p8, q2, kc, vc, bt, cu2, lengths, c8, return_lse=True)
        # (unused slots of the e4m3 pages are never written, so the pages are
        # compared through the outputs that read them)
        return {"out": r.out, "lse": r.lse, "cnt": r.kv_cnt, "out8": r8.out, "lse8": r8.lse,
                "outc": rc.out, "lsec": rc.lse, "cntc": rc.kv_cnt, "outc8": rc8.out, "lsec8": rc8.lse}

    a, b = _both(run)
    _equal(a, b, "paged/chunked")

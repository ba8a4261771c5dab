"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every entry point the header declares, sizes its buffers as documented, and
rejects bad arguments with the documented status before touching a device."""
import ctypes
import os
import re

import pytest

import block_sparse_long_pooling_amd as fp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashprefill.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"fp_select_blocks", "fp_sparse_prefill_fwd", "fp_sparse_prefill_varlen_paged"} <= set(names)
    l = fp.lib()
    for n in names:
        assert hasattr(l, n), n
    assert set(names) == set(fp.EXPORTS)


def test_status_strings():
    l = fp.lib()
    assert l.fp_status_string(0) == b"ok"
    assert l.fp_status_string(3) == b"workspace too small"
    assert l.fp_status_string(99) == b"unknown status"


def _p(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=128, alpha=0.1)
    base.update(kw)
    return fp.make_params(**base)


def test_sizes():
    p = _p()
    S = 1000
    nB = 8
    assert fp.fp_index_capacity(p, [0, S]) == 32 * nB * (nB + 1) // 2
    assert fp.fp_count_entries(p, [0, S]) == 32 * nB
    cu = [0, 100, 300, 300, 1000]
    nbs = [1, 2, 0, 6]
    assert fp.fp_index_capacity(p, cu) == sum(32 * n * (n + 1) // 2 for n in nbs)
    assert fp.fp_count_entries(p, cu) == 32 * sum(nbs)
    ws = fp.fp_varlen_workspace_bytes(p, cu)
    per = sum(nbs) * 128 * 4
    assert ws >= per * (32 + 8 + 8)
    p0 = _p(mean_correction=False)
    assert fp.fp_varlen_workspace_bytes(p0, cu) < ws
    assert fp.fp_index_capacity(_p(head_dim=96), [0, S]) == -1
    assert fp.fp_index_capacity(p, [1, S]) == -1


def test_attention_workgroups_host():
    """Attention launches one workgroup per (query block, head), bf16 and fp8,
    contiguous or paged; bad arguments give -1."""
    p8 = _p(dtype=fp.FP_DTYPE_FP8_E4M3FN)
    for p in (_p(), p8):
        for paged in (False, True):
            assert fp.fp_attention_workgroups(p, [0, 1000], paged=paged) == 32 * 8
            assert fp.fp_attention_workgroups(p, [0, 100, 300, 300, 1000], paged=paged) == 32 * (1 + 2 + 0 + 6)
    p64 = _p(block_size=64)
    assert fp.fp_attention_workgroups(p64, [0, 1000]) == 32 * 16
    assert fp.fp_attention_workgroups(_p(), [0, 0]) == 0
    assert fp.fp_attention_workgroups(_p(head_dim=96), [0, 1000]) == -1
    assert fp.fp_attention_workgroups(_p(), [1, 1000]) == -1
    cu = (ctypes.c_int32 * 2)(0, 1000)
    assert fp.lib().fp_attention_workgroups(ctypes.byref(_p()), cu, 1, 2) == -1


BAD_PARAMS = [
    (dict(num_q_heads=30, num_kv_heads=8), fp.FP_INVALID_ARGUMENT),
    (dict(num_kv_heads=0), fp.FP_INVALID_ARGUMENT),
    (dict(head_dim=96), fp.FP_UNSUPPORTED),
    (dict(block_size=32), fp.FP_UNSUPPORTED),
    (dict(alpha=-0.1), fp.FP_INVALID_ARGUMENT),
    (dict(alpha=1.5), fp.FP_INVALID_ARGUMENT),
    (dict(alpha=float("nan")), fp.FP_INVALID_ARGUMENT),
    (dict(num_q_heads=64, num_kv_heads=1), fp.FP_UNSUPPORTED),
]

FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


@pytest.mark.parametrize("kw,status", BAD_PARAMS)
def test_bad_params_rejected(kw, status):
    l = fp.lib()
    p = _p(**kw)
    rc = l.fp_select_blocks(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == status
    assert l.fp_last_error().decode()
    rc = l.fp_sparse_prefill_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, 1024, FAKE, FAKE,
                                 FAKE, FAKE, None, None)
    assert rc == status


def test_bad_pointers_rejected():
    l = fp.lib()
    p = _p()
    assert l.fp_select_blocks(ctypes.byref(p), None, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              None) == fp.FP_INVALID_ARGUMENT
    assert l.fp_select_blocks(ctypes.byref(p), MISALIGNED, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, None) == fp.FP_INVALID_ARGUMENT
    assert l.fp_select_blocks(ctypes.byref(p), FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              None) == fp.FP_INVALID_ARGUMENT
    assert l.fp_select_blocks(None, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              None) == fp.FP_INVALID_ARGUMENT
    # bf16 pooled means need V
    assert l.fp_select_blocks(ctypes.byref(p), FAKE, FAKE, None, 1024, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                              None) == fp.FP_INVALID_ARGUMENT
    assert l.fp_select_blocks(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, FAKE, None, MISALIGNED, FAKE,
                              FAKE, None) == fp.FP_INVALID_ARGUMENT
    # empty sequence: nothing to do, nothing launched
    assert l.fp_select_blocks(ctypes.byref(p), None, None, None, 0, None, None, None, None, None, None,
                              None) == fp.FP_OK
    # correction without pooled inputs
    assert l.fp_sparse_prefill_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, 1024, FAKE, FAKE,
                                   None, FAKE, None, None) == fp.FP_INVALID_ARGUMENT
    assert l.fp_sparse_prefill_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, 1024, FAKE, FAKE,
                                   MISALIGNED, FAKE, None, None) == fp.FP_INVALID_ARGUMENT
    # fp8 without scales
    p8 = _p(dtype=fp.FP_DTYPE_FP8_E4M3FN)
    assert l.fp_sparse_prefill_fwd(ctypes.byref(p8), FAKE, FAKE, FAKE, None, None, None, 1024, FAKE, FAKE,
                                   FAKE, FAKE, None, None) == fp.FP_INVALID_ARGUMENT
    assert "scale" in l.fp_last_error().decode()


def _varlen(p, cu, page_size=64, num_pages=100, max_pages=64, ws=1 << 30):
    l = fp.lib()
    c = (ctypes.c_int32 * len(cu))(*cu)
    return l.fp_sparse_prefill_varlen_paged(ctypes.byref(p), FAKE, FAKE, FAKE, page_size, num_pages, FAKE,
                                            max_pages, c, len(cu) - 1, FAKE, FAKE, ctypes.c_void_p(1 << 24),
                                            ws, FAKE, None, None)


def test_varlen_validation():
    p = _p()
    assert _varlen(p, [0, 100, 50]) == fp.FP_INVALID_ARGUMENT           # non-monotone
    assert _varlen(p, [5, 100]) == fp.FP_INVALID_ARGUMENT               # cu[0] != 0
    assert _varlen(p, [0, 100], page_size=48) == fp.FP_INVALID_ARGUMENT  # 128 % 48 != 0
    assert _varlen(p, [0, 4096], max_pages=10) == fp.FP_INVALID_ARGUMENT
    assert _varlen(p, [0, 100], num_pages=0) == fp.FP_INVALID_ARGUMENT
    assert _varlen(p, [0, 1000], ws=16) == fp.FP_WORKSPACE_TOO_SMALL
    assert _varlen(_p(dtype=fp.FP_DTYPE_FP8_E4M3FN), [0, 100]) == fp.FP_UNSUPPORTED
    assert _varlen(p, [0] * 130) == fp.FP_UNSUPPORTED                  # batch > 128
    assert _varlen(p, [0, 0, 0]) == fp.FP_OK                            # nothing to do
    assert fp.lib().fp_last_error() == b""


def _chunked(p, cu, kv, page_size=64, num_pages=100, max_pages=64, ws=1 << 30, cache=None, reuse=0,
             kv_lens_null=False):
    l = fp.lib()
    c = (ctypes.c_int32 * len(cu))(*cu)
    k = None if kv_lens_null else (ctypes.c_int32 * len(kv))(*kv)
    return l.fp_sparse_prefill_chunked_paged(ctypes.byref(p), FAKE, FAKE, FAKE, page_size, num_pages, FAKE,
                                             max_pages, c, k, len(cu) - 1, cache, reuse, FAKE, FAKE,
                                             ctypes.c_void_p(1 << 24), ws, FAKE, None, None)


def test_chunked_validation():
    p = _p()
    # a chunk that starts at 900, inside block 7, is accepted, but not with skeleton queries
    assert _chunked(_p(query_probes=16), [0, 100], [1000]) == fp.FP_UNSUPPORTED
    assert "block boundary" in fp.lib().fp_last_error().decode()
    assert _chunked(p, [0, 300], [200]) == fp.FP_INVALID_ARGUMENT      # more queries than context
    assert _chunked(p, [0, 128], [256], kv_lens_null=True) == fp.FP_INVALID_ARGUMENT
    assert _chunked(p, [0, 128], [256], reuse=1) == fp.FP_INVALID_ARGUMENT           # reuse without a cache
    assert _chunked(p, [0, 128], [256], cache=FAKE, reuse=2) == fp.FP_INVALID_ARGUMENT
    assert _chunked(p, [0, 128], [4096], max_pages=10) == fp.FP_INVALID_ARGUMENT     # pages cover the context
    assert _chunked(p, [0, 128], [256], cache=MISALIGNED) == fp.FP_INVALID_ARGUMENT
    assert _chunked(p, [0, 128], [256], ws=16) == fp.FP_WORKSPACE_TOO_SMALL
    assert _chunked(_p(dtype=fp.FP_DTYPE_FP8_E4M3FN), [0, 128], [256]) == fp.FP_UNSUPPORTED
    assert _chunked(p, [0, 0, 0], [256, 512]) == fp.FP_OK                # no queries: nothing to do
    assert fp.lib().fp_last_error() == b""


def test_chunked_sizes():
    p = _p()                                   # 32/8 heads, d 128, block 128, correction on
    cap, cnt, ws = fp.fp_chunked_sizes(p, [0, 256], [1024])      # query blocks 6, 7 of 8
    tri = lambda n: n * (n + 1) // 2
    assert cap == 32 * (tri(8) - tri(6))
    assert cnt == 32 * 2
    a256 = lambda x: (x + 255) // 256 * 256
    assert ws == a256(2 * 128 * 32 * 4) + a256(8 * 128 * 8 * 4) + a256(2 * 8 * 128 * 8 * 2)
    # whole prompts: the same sizes as the varlen entry
    cu = [0, 1000, 1300, 5000]
    lens = [cu[i + 1] - cu[i] for i in range(3)]
    assert fp.fp_chunked_sizes(p, cu, lens) == (fp.fp_index_capacity(p, cu), fp.fp_count_entries(p, cu),
                                                fp.fp_varlen_workspace_bytes(p, cu))
    # a chunk entering block 7 of 8 part way: query blocks 7 and ... 7
    cap, cnt, _ = fp.fp_chunked_sizes(p, [0, 100], [1000])
    assert (cap, cnt) == (32 * (tri(8) - tri(7)), 32)
    cap, cnt, _ = fp.fp_chunked_sizes(p, [0, 200], [1000])        # from 800, inside block 6
    assert (cap, cnt) == (32 * (tri(8) - tri(6)), 64)
    cap, cnt, _ = fp.fp_chunked_sizes(p, [0, 0], [1000])          # empty: no query blocks
    assert (cap, cnt) == (0, 0)
    with pytest.raises(fp.FlashPrefillError):
        fp.fp_chunked_sizes(_p(query_probes=16), [0, 100], [1000])


def test_select_blocks_fp8_validation():
    l = fp.lib()
    p8 = _p(dtype=fp.FP_DTYPE_FP8_E4M3FN)

    def call(p, seqlen=1024, q8=FAKE, pkv=FAKE, scale=FAKE):
        return l.fp_select_blocks_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, seqlen, q8, FAKE, FAKE, scale, FAKE, FAKE,
                                      FAKE, FAKE, pkv, FAKE, FAKE, None)

    assert call(_p()) == fp.FP_INVALID_ARGUMENT                     # params must describe fp8 attention
    assert "fp8" in l.fp_last_error().decode()
    assert call(p8, q8=ctypes.c_void_p((1 << 20) + 4)) == fp.FP_INVALID_ARGUMENT   # codes 8-byte aligned
    assert call(p8, pkv=None) == fp.FP_INVALID_ARGUMENT             # correction needs pooled_kv_bf16
    assert call(p8, scale=None) == fp.FP_INVALID_ARGUMENT
    assert call(p8, seqlen=-1) == fp.FP_INVALID_ARGUMENT
    assert call(p8, seqlen=0) == fp.FP_OK


def test_shared_selection_flag_validated():
    p = _p()
    c = (ctypes.c_int32 * 2)(0, 1024)
    assert fp.lib().fp_index_capacity(ctypes.byref(p), c, 1) > 0
    p.shared_selection = 2
    assert fp.lib().fp_index_capacity(ctypes.byref(p), c, 1) > 0
    p.shared_selection = 3
    assert fp.lib().fp_index_capacity(ctypes.byref(p), c, 1) == -1
    assert "shared_selection" in fp.lib().fp_last_error().decode()


def test_query_probes_validated():
    c = (ctypes.c_int32 * 2)(0, 1024)
    for probes, ok in ((0, True), (1, True), (16, True), (128, True), (3, False), (-1, False), (256, False)):
        p = _p(query_probes=probes)
        assert (fp.lib().fp_index_capacity(ctypes.byref(p), c, 1) > 0) == ok, probes


def test_shared_selection_names():
    assert [fp.make_params(4, 1, 64, 64, 0.1, shared_selection=x).shared_selection
            for x in (False, True, "union", "pooled")] == [0, 1, 1, 2]
    with pytest.raises(ValueError):
        fp.make_params(4, 1, 64, 64, 0.1, shared_selection="mean")


def test_fp8_paged_validation_and_workspace():
    l = fp.lib()
    cu = (ctypes.c_int32 * 3)(0, 1000, 1300)
    p16, p8 = _p(), _p(dtype=fp.FP_DTYPE_FP8_E4M3FN)
    ws16 = l.fp_varlen_workspace_bytes(ctypes.byref(p16), cu, 2)
    ws8 = l.fp_varlen_workspace_bytes(ctypes.byref(p8), cu, 2)
    a256 = lambda x: (x + 255) // 256 * 256
    assert ws8 == ws16 + a256(1300 * 32 * 128) + a256(11 * 32 * 4)     # Q codes + Q scales (11 blocks)

    def call(p, k8=FAKE, ks=FAKE, ws=1 << 30):
        return l.fp_sparse_prefill_varlen_paged_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, 64, 100, FAKE, 64, cu, 2,
                                                    k8, FAKE, ks, FAKE, FAKE, FAKE, ctypes.c_void_p(1 << 24), ws,
                                                    FAKE, None, None)
    assert call(p16) == fp.FP_INVALID_ARGUMENT                          # bf16 params
    assert "fp8" in l.fp_last_error().decode()
    assert call(p8, k8=None) == fp.FP_INVALID_ARGUMENT                  # no fp8 pages
    assert call(p8, k8=MISALIGNED) == fp.FP_INVALID_ARGUMENT
    assert call(p8, ks=None) == fp.FP_INVALID_ARGUMENT                  # no scale cache
    assert call(p8, ws=ws16) == fp.FP_WORKSPACE_TOO_SMALL               # the bf16 size is not enough


def test_chunked_fp8_validation_and_workspace():
    l = fp.lib()
    p16, p8 = _p(), _p(dtype=fp.FP_DTYPE_FP8_E4M3FN)
    a256 = lambda x: (x + 255) // 256 * 256
    # chunk of 200 queries from 800 (query blocks 6, 7): Q codes of 200 rows, Q scales of 2 blocks
    _, _, ws16 = fp.fp_chunked_sizes(p16, [0, 200], [1000])
    _, _, ws8 = fp.fp_chunked_sizes(p8, [0, 200], [1000])
    assert ws8 == ws16 + a256(200 * 32 * 128) + a256(2 * 32 * 4)

    def call(p, cu=(0, 200), kv=(1000,), k8=FAKE, ks=FAKE, ws=1 << 30, pooled=None, reuse=0, kv_null=False):
        c = (ctypes.c_int32 * len(cu))(*cu)
        k = None if kv_null else (ctypes.c_int32 * len(kv))(*kv)
        return l.fp_sparse_prefill_chunked_paged_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, 64, 100, FAKE, 64, c, k,
                                                     len(cu) - 1, pooled, reuse, k8, FAKE, ks, FAKE, FAKE, FAKE,
                                                     ctypes.c_void_p(1 << 24), ws, FAKE, None, None)
    assert call(p16) == fp.FP_INVALID_ARGUMENT                          # bf16 params
    assert "fp8" in l.fp_last_error().decode()
    assert call(p8, kv_null=True) == fp.FP_INVALID_ARGUMENT
    assert call(p8, reuse=1) == fp.FP_INVALID_ARGUMENT                  # reuse without a pooled cache
    assert call(p8, cu=(0, 1200)) == fp.FP_INVALID_ARGUMENT             # more queries than context
    assert call(p8, k8=None) == fp.FP_INVALID_ARGUMENT                  # no fp8 pages
    assert call(p8, k8=MISALIGNED) == fp.FP_INVALID_ARGUMENT
    assert call(p8, ks=None) == fp.FP_INVALID_ARGUMENT                  # no scale cache
    assert call(p8, ws=ws16) == fp.FP_WORKSPACE_TOO_SMALL               # the bf16 size is not enough
    assert call(_p(dtype=fp.FP_DTYPE_FP8_E4M3FN, query_probes=16)) == fp.FP_UNSUPPORTED   # probes, unaligned
    assert call(p8, cu=(0, 0, 0), kv=(256, 512)) == fp.FP_OK            # no queries: nothing to do
    assert l.fp_last_error() == b""


def test_noalloc_entry_rejects_batches_beyond_its_scratch():
    """The allocation-free entry checks the pooled-mean scratch it needs
    against its fixed array on the host, before any device work."""
    l = fp.lib()
    p = _p()
    cu = (ctypes.c_int32 * 3)(0, 1 << 19, 1 << 20)     # 2 x 512K tokens: about 200 MB of means
    need = l.fp_varlen_workspace_bytes(ctypes.byref(p), cu, 2)
    assert need > fp.FP_NOALLOC_SCRATCH_BYTES
    d = ctypes.c_void_p(256)
    rc = l.fp_sparse_prefill_varlen_paged_noalloc(ctypes.byref(p), d, d, d, 64, 100000, d, 8192, cu, 2,
                                                  d, d, d, None, None)
    assert rc == fp.FP_WORKSPACE_TOO_SMALL
    assert b"scratch" in l.fp_last_error()

"""Helpers shared by the GPU parity tests: run the HIP path through the
C-ABI binding and compare against the CPU oracle."""
import numpy as np
import torch

import block_sparse_long_pooling_amd as fp
import oracle as O

BF16_TOL = 2e-2
FP8_TOL = 6e-2
# Correction logits use bf16-rounded pooled keys: |dz| <= sigma*|q|*|k_bar|*2^-9,
# about 6e-3 at these shapes; the lse bound is set above that.
LSE_TOL = 1e-2


def dev():
    return torch.device("cuda:0")


def check_lists(kv_idx, kv_cnt, Hq, nB, offset=0, cnt_offset=0):
    """Lists are strictly ascending, causal and non-empty; returns the mask."""
    idx = kv_idx.cpu().numpy()
    cnt = kv_cnt.reshape(-1).cpu().numpy()
    tri = nB * (nB + 1) // 2
    mask = np.zeros((Hq, nB, nB), dtype=bool)
    for h in range(Hq):
        for I in range(nB):
            c = int(cnt[cnt_offset + h * nB + I])
            assert 1 <= c <= I + 1, (h, I, c)
            lst = idx[offset + h * tri + I * (I + 1) // 2: offset + h * tri + I * (I + 1) // 2 + c]
            assert np.all(np.diff(lst) > 0) and lst[0] >= 0 and lst[-1] <= I, (h, I, lst)
            mask[h, I, lst] = True
    return mask


def compare_mask(mask, sel: "O.Selection"):
    """Return (mismatches outside the band, mismatches inside, band size)."""
    diff = mask != sel.keep
    return int((diff & ~sel.band).sum()), int((diff & sel.band).sum()), int(sel.band.sum())


def run_single(q, k, v, B, alpha, correction=True, lse=True):
    """Selection + attention on the GPU for one bf16 sequence (CPU tensors in)."""
    S, Hq, d = q.shape
    p = fp.make_params(Hq, k.shape[1], d, B, alpha, mean_correction=correction)
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    sel = fp.fp_select_blocks(p, qd, kd, vd)
    res = fp.fp_sparse_prefill_fwd(p, qd, kd, vd, sel, return_lse=lse)
    torch.cuda.synchronize()
    return sel, res


def oracle_inputs(q, k, v):
    return q.float().numpy(), k.float().numpy(), v.float().numpy()


def chunk_masks(kv_idx, kv_cnt, Hq, kv_lens, starts, B):
    """Per request the [Hq, nq, nb] mask of lists in the chunked layout (query
    blocks first .. nb-1, first = start // B, none for an empty chunk); the
    lists must be ascending, causal and non-empty."""
    tri = lambda n: n * (n + 1) // 2
    idx = kv_idx.cpu().numpy()
    cnt = kv_cnt.reshape(-1).cpu().numpy()
    io = co = 0
    masks = []
    for L, P0 in zip(kv_lens, starts):
        nb = (L + B - 1) // B
        first = P0 // B if P0 < L else nb
        nq, rowsz = nb - first, tri(nb) - tri(first)
        m = np.zeros((Hq, nq, nb), dtype=bool)
        for h in range(Hq):
            for i in range(nq):
                I = first + i
                c = int(cnt[co + h * nq + i])
                assert 1 <= c <= I + 1, (h, I, c)
                s0 = io + h * rowsz + tri(I) - tri(first)
                lst = idx[s0:s0 + c]
                assert np.all(np.diff(lst) > 0) and lst[0] >= 0 and lst[-1] <= I, (h, I, lst)
                m[h, i, lst] = True
        masks.append(m)
        io += Hq * rowsz
        co += Hq * nq
    return masks

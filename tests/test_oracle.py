"""Pins for the CPU oracle: each check comes from something other than the
oracle itself (a textbook routine, brute force, a closed form, an invariant
the threshold equation implies), so that a dropped term, a wrong sign, index
or operand fails at least one of them."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_pooling_amd import synth


def _rand_qkv(S, Hq, Hkv, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((S, Hq, d)) * scale
    k = r.standard_normal((S, Hkv, d)) * scale
    v = r.standard_normal((S, Hkv, d))
    return q, k, v


def _dense_causal_torch(q, k, v):
    """Full causal softmax attention by torch's own routine (fp64, CPU)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)[None].contiguous()
    V = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)[None].contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def _dense_causal_matrix(q, k, v):
    """Textbook dense causal attention with the full S x S matrix; also lse."""
    S, Hq, d = q.shape
    g = Hq // k.shape[1]
    o = np.empty_like(q)
    lse = np.empty((Hq, S))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    for h in range(Hq):
        a = q[:, h] @ k[:, h // g].T / math.sqrt(d)
        a[mask] = -np.inf
        m = a.max(axis=1, keepdims=True)
        e = np.exp(a - m)
        o[:, h] = (e @ v[:, h // g]) / e.sum(1, keepdims=True)
        lse[h] = m[:, 0] + np.log(e.sum(1))
    return o, lse


# ---------------------------------------------------------------- alpha = 0

@pytest.mark.parametrize("S,B,Hq,Hkv,d", [(200, 64, 4, 2, 16), (128, 32, 2, 2, 8), (64, 64, 3, 1, 8),
                                          (33, 16, 1, 1, 4)])
@pytest.mark.parametrize("corr", [False, True])
def test_alpha0_is_dense_causal(S, B, Hq, Hkv, d, corr):
    q, k, v = _rand_qkv(S, Hq, Hkv, d, seed=S + d)
    sel = O.select_blocks(q, k, v, B, alpha=0.0)
    assert sel.keep.sum() == Hq * O.num_blocks(S, B) * (O.num_blocks(S, B) + 1) // 2
    o, lse = O.sparse_attention(q, k, v, sel, correction=corr)
    o_t = _dense_causal_torch(q, k, v)
    o_m, lse_m = _dense_causal_matrix(q, k, v)
    np.testing.assert_allclose(o, o_t, atol=1e-12, rtol=0)
    np.testing.assert_allclose(o, o_m, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_m, atol=1e-12, rtol=0)


# ---------------------------------------------------------- brute-force mask

def _brute_force_keep(q, k, B, alpha):
    """Per-block scoring written with Python loops and math.fsum."""
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    nB = (S + B - 1) // B
    sig = 1.0 / math.sqrt(d)

    def mean(x, J, h):
        toks = range(J * B, min(S, (J + 1) * B))
        return [math.fsum(float(x[t, h, c]) for t in toks) / len(toks) for c in range(d)]

    keep = np.zeros((Hq, nB, nB), dtype=bool)
    band = np.zeros((Hq, nB, nB), dtype=bool)
    for h in range(Hq):
        kb = [mean(k, J, h // g) for J in range(nB)]
        for I in range(nB):
            qb = mean(q, I, h)
            s = [sig * math.fsum(a * b for a, b in zip(qb, kb[J])) for J in range(I + 1)]
            m = max(s)
            den = math.fsum(math.exp(x - m) for x in s)
            score = [math.exp(x - m) / den for x in s]
            thr = alpha * max(score)
            for J in range(I + 1):
                keep[h, I, J] = score[J] >= thr
                band[h, I, J] = alpha > 0 and abs(score[J] - thr) <= 1e-3 * thr
    return keep, band


@pytest.mark.parametrize("alpha", [0.05, 0.1, 0.3, 0.5, 0.9, 1.0])
def test_mask_matches_brute_force(alpha):
    q, k, v = synth.make_sequence(320, 4, 2, 16, seed=7, verticals=False)
    q, k = q.float().numpy(), k.float().numpy()
    sel = O.select_blocks(q, k, None, 32, alpha, pool_v=False)
    keep_bf, band_bf = _brute_force_keep(q, k, 32, alpha)
    outside = ~(sel.band | band_bf)
    assert np.array_equal(sel.keep[outside], keep_bf[outside])
    # A non-trivial mask: something is skipped for alpha >= 0.3 on this input.
    if alpha >= 0.3:
        causal = np.tril(np.ones(sel.keep.shape[1:], bool))
        assert sel.keep.sum() < sel.keep.shape[0] * causal.sum()


def test_mask_brute_force_partial_block_and_gqa():
    q, k, _ = _rand_qkv(77, 6, 2, 8, seed=3, scale=2.0)
    for alpha in (0.2, 0.6):
        sel = O.select_blocks(q, k, None, 16, alpha, pool_v=False)
        keep_bf, band_bf = _brute_force_keep(q, k, 16, alpha)
        outside = ~(sel.band | band_bf)
        assert np.array_equal(sel.keep[outside], keep_bf[outside])


def test_block_means_brute_force():
    x = np.random.default_rng(1).standard_normal((45, 3, 5))
    m = O.block_means(x, 16)
    for h in range(3):
        for J in range(3):
            toks = range(16 * J, min(45, 16 * J + 16))
            for c in range(5):
                ref = math.fsum(x[t, h, c] for t in toks) / len(toks)
                assert abs(m[h, J, c] - ref) < 1e-15
    assert list(O.block_lengths(45, 16)) == [16, 16, 13]


# ----------------------------------------------------------- normalisation

@pytest.mark.parametrize("corr", [False, True])
def test_probability_rows_sum_to_one(corr):
    q, k, v = synth.make_sequence(256, 2, 1, 16, seed=5, verticals=False)
    q, k, v = (t.float().numpy() for t in (q, k, v))
    sel = O.select_blocks(q, k, v, 32, alpha=0.5)
    for h in range(2):
        for I in range(8):
            p = O.attention_probabilities(q, k, v, sel, corr, h, I)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)
            assert (p >= 0).all()


# ----------------------------------------------------- correction (closed form)

def _block_constant_inputs(S, B, Hq, Hkv, d, seed):
    """K and V constant inside every block; queries near their block's key
    direction, so the diagonal block is the strict argmax of every row."""
    r = np.random.default_rng(seed)
    nB = (S + B - 1) // B
    g = Hq // Hkv
    c = r.standard_normal((Hkv, nB, d))
    c *= (2.5 + r.random((Hkv, nB, 1))) / np.linalg.norm(c, axis=-1, keepdims=True) * math.sqrt(math.sqrt(d))
    vb = r.standard_normal((Hkv, nB, d))
    blk = np.arange(S) // B
    k = c[:, blk].transpose(1, 0, 2).copy()
    v = vb[:, blk].transpose(1, 0, 2).copy()
    q = np.repeat(c, g, axis=0)[:, blk].transpose(1, 0, 2) + 0.3 * r.standard_normal((S, Hq, d))
    return q, k, v


@pytest.mark.parametrize("alpha", [0.01, 0.1, 0.3, 0.7, 1.0])
def test_correction_closed_form_equals_dense(alpha):
    S, B = 256, 16
    q, k, v = _block_constant_inputs(S, B, 4, 2, 16, seed=11)
    sel = O.select_blocks(q, k, v, B, alpha)
    nB = S // B
    # precondition of the closed form: the diagonal is always kept
    assert all(sel.keep[h, I, I] for h in range(4) for I in range(nB))
    o, lse = O.sparse_attention(q, k, v, sel, correction=True)
    o_d, lse_d = _dense_causal_matrix(q, k, v)
    np.testing.assert_allclose(o, o_d, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_d, atol=1e-12, rtol=0)
    if alpha >= 0.3:
        # something really was skipped, and without the correction the result differs
        assert (~sel.keep & np.tril(np.ones((nB, nB), bool), -1)[None]).any()
        o_nc, _ = O.sparse_attention(q, k, v, sel, correction=False)
        assert np.abs(o_nc - o_d).max() > 1e-3


def test_hand_worked_example():
    """S=4, B=2, d=4 (sigma = 1/2), one head, worked by hand.

    Keys: k0 = k1 = 0, k2 = k3 = (2,0,0,0).  Queries q2 = q3 = (3,0,0,0).
    Pooled logits of query block 1: s10 = 0, s11 = 3, so block 0 scores
    e^-3 = 0.0498 of the row max: skipped at alpha = 0.1, kept at 0.04.
    Values v0..v3 = unit vectors e0..e3, so v_bar0 = (1/2, 1/2, 0, 0).
    Row 2: token 2 with logit 3, correction entry ln 2 + 0 with value v_bar0:
      o2 = (1, 1, e^3, 0) / (e^3 + 2),  lse2 = ln(e^3 + 2).
    Row 3: tokens 2, 3 (logit 3 each) and the same correction entry:
      o3 = (1, 1, e^3, e^3) / (2 e^3 + 2),  lse3 = ln(2 e^3 + 2).
    Rows 0, 1 see only block 0 with zero keys: o0 = e0, o1 = (e0 + e1) / 2.
    Without the correction rows 2, 3 see block 1 only: o2 = e2, o3 = (e2+e3)/2.
    """
    q = np.zeros((4, 1, 4)); k = np.zeros((4, 1, 4)); v = np.zeros((4, 1, 4))
    q[0, 0] = [1, 2, 3, 4]
    q[2, 0, 0] = q[3, 0, 0] = 3.0
    k[2, 0, 0] = k[3, 0, 0] = 2.0
    for t in range(4):
        v[t, 0, t] = 1.0
    e3 = math.exp(3.0)
    sel = O.select_blocks(q, k, v, 2, alpha=0.1)
    assert sel.keep[0].tolist() == [[True, False], [False, True]]
    o, lse = O.sparse_attention(q, k, v, sel, correction=True)
    np.testing.assert_allclose(o[0, 0], [1, 0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(o[1, 0], [0.5, 0.5, 0, 0], atol=1e-15)
    np.testing.assert_allclose(o[2, 0], np.array([1, 1, e3, 0]) / (e3 + 2), atol=1e-15)
    np.testing.assert_allclose(o[3, 0], np.array([1, 1, e3, e3]) / (2 * e3 + 2), atol=1e-15)
    np.testing.assert_allclose(lse[0], [0, math.log(2), math.log(e3 + 2), math.log(2 * e3 + 2)],
                               atol=1e-14)
    o_nc, _ = O.sparse_attention(q, k, v, sel, correction=False)
    np.testing.assert_allclose(o_nc[2, 0], [0, 0, 1, 0], atol=1e-15)
    np.testing.assert_allclose(o_nc[3, 0], [0, 0, 0.5, 0.5], atol=1e-15)
    sel2 = O.select_blocks(q, k, v, 2, alpha=0.04)
    assert sel2.keep[0].tolist() == [[True, False], [True, True]]


def test_skipped_diagonal_gets_no_correction():
    """A strong sink in block 0 makes the diagonal of later rows fall below
    the threshold; the rows then see the kept past blocks and the correction
    entries of skipped strictly-past blocks only."""
    S, B, d = 96, 16, 8
    r = np.random.default_rng(4)
    q = 0.1 * r.standard_normal((S, 1, d))
    k = 0.1 * r.standard_normal((S, 1, d))
    v = r.standard_normal((S, 1, d))
    q[:, 0, 0] += 3.0
    k[:16, 0, 0] += 6.0
    sel = O.select_blocks(q, k, v, B, alpha=0.5)
    assert not sel.keep[0, 5, 5] and sel.keep[0, 5, 0]
    p = O.attention_probabilities(q, k, v, sel, True, 0, 5)
    kept = int(sel.keep[0, 5, :6].sum())
    skipped_past = 5 - int(sel.keep[0, 5, :5].sum())
    assert p.shape[1] == kept * B + skipped_past


# --------------------------------------------------------------- invariants

def test_constant_v_gives_constant_output():
    q, k, _ = _rand_qkv(150, 4, 2, 8, seed=9, scale=1.5)
    v = np.broadcast_to(np.array([0.25, -1, 2, 0, 3, 1, -2, 0.5]), (150, 2, 8)).copy()
    for alpha in (0.0, 0.2, 0.9):
        for corr in (False, True):
            sel = O.select_blocks(q, k, v, 32, alpha)
            o, _ = O.sparse_attention(q, k, v, sel, corr)
            np.testing.assert_allclose(o, np.broadcast_to(v[0, 0], o.shape), atol=1e-13)


def test_threshold_invariants():
    q, k, _ = synth.make_sequence(1024, 4, 1, 64, seed=1, verticals=False)
    q, k = q.float().numpy(), k.float().numpy()
    nB = 16
    causal = np.tril(np.ones((nB, nB), bool))
    prev = None
    for alpha in (0.0, 0.05, 0.1, 0.3, 0.5, 0.9, 1.0):
        sel = O.select_blocks(q, k, None, 64, alpha, pool_v=False)
        am = sel.s.argmax(axis=2)
        for h in range(4):
            for I in range(nB):
                assert sel.keep[h, I, am[h, I]]                 # argmax always kept
        assert not (sel.keep & ~causal).any()                   # never a future block
        if prev is not None:
            assert not (sel.keep & ~prev).any()                 # masks nest as alpha grows
        prev = sel.keep
    # alpha = 1: only blocks tied with the max survive
    sel = O.select_blocks(q, k, None, 64, 1.0, pool_v=False)
    assert np.array_equal(sel.keep.sum(axis=2), np.ones((4, nB), int))


def test_single_block_is_dense_for_every_alpha():
    q, k, v = _rand_qkv(40, 2, 1, 8, seed=2)
    o_d, _ = _dense_causal_matrix(q, k, v)
    for alpha in (0.0, 0.5, 1.0):
        sel = O.select_blocks(q, k, v, 64, alpha)
        o, _ = O.sparse_attention(q, k, v, sel, True)
        np.testing.assert_allclose(o, o_d, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _rand_qkv(128, 8, 2, 16, seed=21, scale=1.3)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    for alpha in (0.2, 0.7):
        a = O.select_blocks(q, k, v, 16, alpha)
        b = O.select_blocks(q, kr, vr, 16, alpha)
        assert np.array_equal(a.keep, b.keep)
        oa, la = O.sparse_attention(q, k, v, a, True)
        ob, lb = O.sparse_attention(q, kr, vr, b, True)
        np.testing.assert_allclose(oa, ob, atol=1e-13)
        np.testing.assert_allclose(la, lb, atol=1e-13)


def test_pairs_subset_matches_full():
    q, k, v = _rand_qkv(100, 4, 2, 8, seed=8)
    sel = O.select_blocks(q, k, v, 16, 0.4)
    o, lse = O.sparse_attention(q, k, v, sel, True)
    pairs = [(0, 0), (3, 6), (1, 4)]
    o2, lse2 = O.sparse_attention(q, k, v, sel, True, pairs=pairs)
    for h, I in pairs:
        r0, r1 = 16 * I, min(100, 16 * I + 16)
        np.testing.assert_array_equal(o2[r0:r1, h], o[r0:r1, h])
        np.testing.assert_array_equal(lse2[h, r0:r1], lse[h, r0:r1])
    assert np.isnan(o2[16:32, 0]).all()


def test_chunked_pairs_subset_matches_full():
    q, k, v = _rand_qkv(100, 4, 2, 8, seed=18)
    P0 = 37                                                   # the chunk enters block 2 at row 5
    sel = O.select_blocks_chunked(q[P0:], k, v, 16, 0.4)
    o, lse = O.sparse_attention_chunked(q[P0:], k, v, sel, True)
    pairs = [(0, 0), (3, 4), (1, 2)]
    o2, lse2 = O.sparse_attention_chunked(q[P0:], k, v, sel, True, pairs=pairs)
    for h, i in pairs:
        r0, r1 = max(16 * (2 + i), P0) - P0, min(100, 16 * (3 + i)) - P0
        np.testing.assert_array_equal(o2[r0:r1, h], o[r0:r1, h])
        np.testing.assert_array_equal(lse2[h, r0:r1], lse[h, r0:r1])
    assert np.isnan(o2[:11, 1]).all() and np.isfinite(o2[:11, 0]).all()


def test_flop_count_dense_closed_form():
    S, B, d, Hq = 256, 64, 16, 2
    q, k, v = _rand_qkv(S, Hq, 1, d, seed=1)
    sel = O.select_blocks(q, k, v, B, 0.0)
    fk, fc = O.flops_executed(sel, S, d, True)
    nB = S // B
    assert fk == 4 * d * Hq * B * B * nB * (nB + 1) // 2
    assert fc == 0.0


# ------------------------------------------------------------------- fp8

def test_dequantize_blockwise_elementwise():
    r = np.random.default_rng(0)
    x8 = r.standard_normal((70, 3, 4))
    sc = r.random((3, 3)) + 0.5
    x = O.dequantize_blockwise(x8, sc, 32)
    for t in range(70):
        for h in range(3):
            assert np.allclose(x[t, h], x8[t, h] * sc[h, t // 32], rtol=0, atol=0)


# ----------------------------------------------------------- chunked prefill

def _brute_force_chunk(qc, k, v, B, alpha, corr):
    """A chunk of new queries at the end of a context, written from token
    positions with Python loops: query row r is position P0 + r and sees the
    keys at or before it in the kept blocks, plus one pooled entry per skipped
    past block (n_J copies of its mean key and value).  A query block the
    chunk enters part way pools the chunk's queries it holds."""
    q_len, Hq, d = qc.shape
    S, Hkv, _ = k.shape
    g = Hq // Hkv
    P0 = S - q_len
    sig = 1.0 / math.sqrt(d)
    nB = (S + B - 1) // B

    def mean(x, rows, h):
        return [math.fsum(float(x[t, h, c]) for t in rows) / len(rows) for c in range(d)]

    def dot(a, b):
        return math.fsum(x * y for x, y in zip(a, b))

    o = np.zeros((q_len, Hq, d))
    lse = np.zeros((Hq, q_len))
    keep_rows = {}
    for h in range(Hq):
        hk = h // g
        kb = [mean(k, range(J * B, min(S, J * B + B)), hk) for J in range(nB)]
        vb = [mean(v, range(J * B, min(S, J * B + B)), hk) for J in range(nB)]
        for I in range(P0 // B, nB):
            qb = mean(qc, range(max(I * B, P0) - P0, min(S, I * B + B) - P0), h)
            s = [sig * dot(qb, kb[J]) for J in range(I + 1)]
            m = max(s)
            den = math.fsum(math.exp(x - m) for x in s)
            score = [math.exp(x - m) / den for x in s]
            keep = [score[J] >= alpha * max(score) for J in range(I + 1)]
            keep_rows[h, I] = keep
            for p in range(max(I * B, P0), min(S, I * B + B)):
                qr = [float(x) for x in qc[p - P0, h]]
                z, vals = [], []
                for J in range(I + 1):
                    if keep[J]:
                        for t in range(J * B, min(S, J * B + B)):
                            if t <= p:
                                z.append(sig * dot(qr, k[t, hk]))
                                vals.append([float(x) for x in v[t, hk]])
                    elif corr and J < I:
                        n = min(S, J * B + B) - J * B
                        z.append(sig * dot(qr, kb[J]) + math.log(n))
                        vals.append(vb[J])
                M = max(z)
                w = [math.exp(x - M) for x in z]
                l = math.fsum(w)
                for c in range(d):
                    o[p - P0, h, c] = math.fsum(wi * vi[c] for wi, vi in zip(w, vals)) / l
                lse[h, p - P0] = M + math.log(l)
    return o, lse, keep_rows


@pytest.mark.parametrize("P0", [0, 8, 24, 3, 13, 39])
@pytest.mark.parametrize("corr", [False, True])
def test_chunk_matches_brute_force(P0, corr):
    q, k, v = _rand_qkv(45, 2, 1, 4, seed=11 + P0, scale=3.0)
    qc = q[P0:]
    alpha = 0.5
    sel = O.select_blocks_chunked(qc, k, v, 8, alpha)
    assert sel.first == P0 // 8 and sel.keep.shape == (2, 6 - P0 // 8, 6)
    o, lse = O.sparse_attention_chunked(qc, k, v, sel, corr)
    o_bf, lse_bf, keep_bf = _brute_force_chunk(qc, k, v, 8, alpha, corr)
    for (h, I), keep in keep_bf.items():
        i = I - sel.first
        row = sel.keep[h, i, :I + 1]
        outside = ~sel.band[h, i, :I + 1]
        assert np.array_equal(row[outside], np.array(keep)[outside])
        assert not sel.keep[h, i, I + 1:].any()
    if not sel.band.any():
        np.testing.assert_allclose(o, o_bf, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_bf, atol=1e-12, rtol=0)
    # something is skipped, so the correction entries are exercised
    assert (~sel.keep & O.causal_blocks(sel.keep.shape[1], 6, sel.first)[None]).any()


@pytest.mark.parametrize("P0", [0, 32, 64, 96])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 3)])
def test_chunk_equals_last_rows_of_full_prefill(P0, Hq, Hkv):
    S, B = 133, 32
    q, k, v = _rand_qkv(S, Hq, Hkv, 8, seed=P0 + Hq, scale=1.3)
    full = O.select_blocks(q, k, v, B, 0.2)
    o_f, lse_f = O.sparse_attention(q, k, v, full, correction=True)
    sel = O.select_blocks_chunked(q[P0:], k, v, B, 0.2)
    o_c, lse_c = O.sparse_attention_chunked(q[P0:], k, v, sel, correction=True)
    assert np.array_equal(sel.keep, full.keep[:, P0 // B:, :])
    np.testing.assert_allclose(o_c, o_f[P0:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse_c, lse_f[:, P0:], atol=1e-12, rtol=0)
    lists = sel.lists()
    assert all(list(lists[h][i]) == list(full.lists()[h][i + P0 // B]) for h in range(Hq)
               for i in range(len(lists[h])))


def test_chunk_rejects_unaligned_probes_or_too_long():
    q, k, v = _rand_qkv(40, 2, 1, 4, seed=5)
    O.select_blocks_chunked(q[3:], k, v, 8, 0.1)                  # a chunk may start inside a block ...
    with pytest.raises(ValueError):
        O.select_blocks_chunked(q[3:], k, v, 8, 0.1, probes=2)    # ... but not with skeleton queries
    with pytest.raises(ValueError):
        O.select_blocks_chunked(np.concatenate([q, q[:8]]), k, v, 8, 0.1)


@pytest.mark.parametrize("P0", [5, 31, 33, 100])
def test_unaligned_chunk_dense_is_bottom_right_causal_attention(P0):
    """alpha = 0 keeps every causal block, so a chunk starting anywhere is
    plain causal attention of its queries over the context with bottom-right
    alignment (torch's routine with an explicit mask)."""
    S, Hq, Hkv, d, B = 133, 4, 2, 8, 32
    q, k, v = _rand_qkv(S, Hq, Hkv, d, seed=40 + P0, scale=1.5)
    sel = O.select_blocks_chunked(q[P0:], k, v, B, 0.0)
    assert sel.first == P0 // B and sel.keep.shape[1] == (S + B - 1) // B - P0 // B
    o, lse = O.sparse_attention_chunked(q[P0:], k, v, sel, correction=True)
    g = Hq // Hkv
    Q = torch.from_numpy(q[P0:]).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)[None].contiguous()
    V = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)[None].contiguous()
    allowed = torch.arange(S)[None, :] <= (P0 + torch.arange(S - P0))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=allowed)[0].permute(1, 0, 2)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    z = torch.einsum("hqd,hkd->hqk", Q[0], K[0]) / math.sqrt(d)
    lse_ref = torch.logsumexp(z.masked_fill(~allowed[None], -math.inf), dim=-1)
    np.testing.assert_allclose(lse, lse_ref.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("P0", [1, 40, 70])
def test_unaligned_chunk_later_blocks_equal_full_prefill(P0):
    """Past the block it enters part way, a chunk's query blocks hold the same
    queries as in the full prefill, so their masks and rows are the full
    prefill's; the entered block pools fewer queries."""
    S, Hq, Hkv, B = 133, 4, 2, 32
    q, k, v = _rand_qkv(S, Hq, Hkv, 8, seed=50 + P0, scale=2.0)
    full = O.select_blocks(q, k, v, B, 0.2)
    o_f, lse_f = O.sparse_attention(q, k, v, full, correction=True)
    sel = O.select_blocks_chunked(q[P0:], k, v, B, 0.2)
    o_c, lse_c = O.sparse_attention_chunked(q[P0:], k, v, sel, correction=True)
    f, r = P0 // B, (P0 // B + 1) * B - P0                        # first query block, its rows in the chunk
    assert np.array_equal(sel.keep[:, 1:], full.keep[:, f + 1:])
    np.testing.assert_allclose(o_c[r:], o_f[P0 + r:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse_c[:, r:], lse_f[:, P0 + r:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(sel.q_bar[:, 0], q[P0:P0 + r].mean(axis=0), atol=1e-15, rtol=0)
    assert not np.allclose(sel.q_bar[:, 0], full.q_bar[:, f])


def test_empty_chunk():
    q, k, v = _rand_qkv(40, 2, 1, 4, seed=6)
    sel = O.select_blocks_chunked(q[40:], k, v, 8, 0.1)
    assert sel.keep.shape == (2, 0, 5)
    o, lse = O.sparse_attention_chunked(q[40:], k, v, sel, True)
    assert o.shape == (0, 2, 4) and lse.shape == (2, 0)
    sel = O.select_blocks_chunked(q[37:37], k[:37], v[:37], 8, 0.1)      # ends inside a block: no rows
    assert sel.keep.shape == (2, 0, 5)


# ------------------------------------------------------ e4m3 encoder (fp8)

def _e4m3_table():
    """Codes 0..126 and their values, from the format definition (bias 7,
    3 mantissa bits, exponent field 0 = subnormals m/8 * 2^-6)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = np.array([(c & 7) / 8 * 2.0 ** -6 if c >> 3 == 0 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7)
                     for c in range(0x7F)])
    return codes, vals


def test_e4m3_encode_every_finite_value():
    codes, vals = _e4m3_table()
    assert vals[-1] == 448.0
    assert np.array_equal(O.e4m3_encode(vals.astype(np.float32)), codes)
    assert np.array_equal(O.e4m3_encode(-vals[1:].astype(np.float32)), codes[1:] | 0x80)
    assert np.array_equal(O.e4m3_decode(codes), vals)


def test_e4m3_ties_go_to_even_mantissa():
    codes, vals = _e4m3_table()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)   # exact in fp32
    got = O.e4m3_encode(mids)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(got, want)
    # just off the midpoint the nearer value wins
    above = np.nextafter(mids, np.float32(np.inf))
    assert np.array_equal(O.e4m3_encode(above), codes[1:])


def test_e4m3_encode_matches_torch_cast():
    r = np.random.default_rng(3)
    y = (r.choice([-1, 1], 20000) * np.exp(r.uniform(np.log(1e-5), np.log(448.0), 20000))).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(y), ref)


def test_quantize_blockwise_scale_rule():
    r = np.random.default_rng(4)
    x = r.standard_normal((300, 3, 16)).astype(np.float32) * 2
    x[128:256, 1] = 0.0                                      # an all-zero (head, block)
    codes, scales = O.quantize_fp8_blockwise(x, 128)
    assert scales.dtype == np.float32 and scales.shape == (3, 3)
    assert scales[1, 1] == 1.0 and not codes[128:256, 1].any()
    for h in range(3):
        for J in range(3):
            seg = x[J * 128:(J + 1) * 128, h]
            if J == 1 and h == 1:
                continue
            assert scales[h, J] == np.float32(np.abs(seg).max()) / np.float32(448)
            i = np.unravel_index(np.abs(seg).argmax(), seg.shape)
            assert codes[J * 128 + i[0], h, i[1]] & 0x7F == 0x7E         # the amax element maps to 448
    deq = O.dequantize_blockwise(O.e4m3_decode(codes), scales, 128)
    big = np.abs(deq) >= 2.0 ** -6 * scales[:, np.arange(300) // 128].T[:, :, None]
    rel = np.abs(deq - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4


def test_quantize_blockwise_matches_generator_quantizer():
    q, k, v = synth.make_sequence(700, 4, 2, 32, seed=9, verticals=True)
    for x in (q, k, v):
        c_t, s_t = synth.quantize_fp8_blockwise(x, 128)
        c_o, s_o = O.quantize_fp8_blockwise(x.float().numpy(), 128)
        assert np.array_equal(c_o, c_t.numpy()) and np.array_equal(s_o, s_t.numpy())


def test_quantize_chunk_aligned_equals_blockwise():
    """A chunk that starts on a block boundary has the blockwise codes and
    scales of its own rows."""
    r = np.random.default_rng(5)
    q = (r.standard_normal((300, 3, 16)) * 3).astype(np.float32)
    c, s = O.quantize_fp8_chunk(q, 128, 2 * 128)
    c_ref, s_ref = O.quantize_fp8_blockwise(q, 128)
    assert np.array_equal(c, c_ref) and np.array_equal(s, s_ref)


@pytest.mark.parametrize("P0", [37, 127, 128 + 1])
def test_quantize_chunk_windows_from_positions(P0):
    """Each query block's scale and codes come from exactly the chunk's rows
    whose positions fall in it: the first window holds the rows up to the
    next block boundary, the last one stops at the chunk's end."""
    B, q_len = 128, 400
    r = np.random.default_rng(P0)
    q = (r.standard_normal((q_len, 2, 8)) * r.uniform(0.5, 4, (q_len, 1, 1))).astype(np.float32)
    c, s = O.quantize_fp8_chunk(q, B, P0)
    pos = P0 + np.arange(q_len)
    blocks = np.unique(pos // B)
    assert s.shape == (2, len(blocks))
    for i, I in enumerate(blocks):
        rows = np.nonzero(pos // B == I)[0]                      # the chunk's rows in block I
        if i == 0:
            assert len(rows) == B - P0 % B
        seg = q[rows]
        for h in range(2):
            assert s[h, i] == np.float32(np.abs(seg[:, h]).max()) / np.float32(448)
        cs, ss = O.quantize_fp8_blockwise(seg, len(rows))          # the window as a one-block sequence
        assert np.array_equal(c[rows], cs) and np.array_equal(s[:, i], ss[:, 0])
    # dequantized values sit within E4M3's half-ulp (2^-4 relative) of the input in its normal range
    deq = O.dequantize_chunk(O.e4m3_decode(c), s, B, P0)
    big = np.abs(q) >= 2.0 ** -6 * s[:, pos // B - P0 // B].T[:, :, None]
    assert big.mean() > 0.9
    assert (np.abs(deq - q)[big] / np.abs(q)[big]).max() <= 2.0 ** -4


# ------------------------------------------------- group-shared selection

def _brute_force_union(q, k, B, alpha):
    keep, band = _brute_force_keep(q, k, B, alpha)
    g = q.shape[1] // k.shape[1]
    Hkv = k.shape[1]
    ku = np.zeros_like(keep)
    for hk in range(Hkv):
        ku[hk * g:(hk + 1) * g] = keep[hk * g:(hk + 1) * g].any(axis=0)
    bu = np.zeros_like(band)
    for hk in range(Hkv):
        bu[hk * g:(hk + 1) * g] = band[hk * g:(hk + 1) * g].any(axis=0)
    return ku, bu


@pytest.mark.parametrize("alpha", [0.1, 0.5, 1.0])
def test_shared_selection_is_the_group_union(alpha):
    q, k, v = synth.make_sequence(320, 8, 2, 16, seed=12, verticals=False)
    q, k, v = q.float().numpy(), k.float().numpy(), v.float().numpy()
    own = O.select_blocks(q, k, v, 32, alpha)
    sh = O.select_blocks(q, k, v, 32, alpha, shared=True)
    ku, bu = _brute_force_union(q, k, 32, alpha)
    outside = ~(sh.band | bu)
    assert np.array_equal(sh.keep[outside], ku[outside])
    assert (sh.keep | ~own.keep).all()                     # a superset of each head's own mask
    for hk in range(2):
        assert (sh.keep[hk * 4:(hk + 1) * 4] == sh.keep[hk * 4]).all()
    if alpha >= 0.5:
        assert sh.keep.sum() > own.keep.sum()              # the heads disagree somewhere


def test_shared_selection_without_groups_is_per_head():
    q, k, v = _rand_qkv(200, 3, 3, 8, seed=21, scale=2.0)
    own = O.select_blocks(q, k, v, 16, 0.4)
    sh = O.select_blocks(q, k, v, 16, 0.4, shared=True)
    assert np.array_equal(own.keep, sh.keep) and np.array_equal(own.band, sh.band)


def test_shared_selection_chunked_equals_full_rows():
    q, k, v = _rand_qkv(133, 4, 2, 8, seed=22, scale=1.3)
    full = O.select_blocks(q, k, v, 32, 0.3, shared=True)
    ch = O.select_blocks_chunked(q[64:], k, v, 32, 0.3, shared=True)
    assert np.array_equal(ch.keep, full.keep[:, 2:, :])


def _brute_force_group_pooled(q, k, B, alpha):
    """One mask per KV head from the mean over its g query heads and the
    block's tokens, written with Python loops and math.fsum, repeated over
    the group's query heads."""
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    nB = (S + B - 1) // B
    sig = 1.0 / math.sqrt(d)
    keep = np.zeros((Hq, nB, nB), dtype=bool)
    band = np.zeros((Hq, nB, nB), dtype=bool)
    for hk in range(Hkv):
        heads = range(hk * g, (hk + 1) * g)

        def kmean(J):
            toks = range(J * B, min(S, (J + 1) * B))
            return [math.fsum(float(k[t, hk, c]) for t in toks) / len(toks) for c in range(d)]

        def qmean(I):
            toks = range(I * B, min(S, (I + 1) * B))
            n = len(toks) * g
            return [math.fsum(float(q[t, h, c]) for t in toks for h in heads) / n for c in range(d)]

        kb = [kmean(J) for J in range(nB)]
        for I in range(nB):
            qb = qmean(I)
            s_ = [sig * math.fsum(a * b for a, b in zip(qb, kb[J])) for J in range(I + 1)]
            m = max(s_)
            den = math.fsum(math.exp(x - m) for x in s_)
            score = [math.exp(x - m) / den for x in s_]
            thr = alpha * max(score)
            for J in range(I + 1):
                for h in heads:
                    keep[h, I, J] = score[J] >= thr
                    band[h, I, J] = alpha > 0 and abs(score[J] - thr) <= 1e-3 * thr
    return keep, band


@pytest.mark.parametrize("alpha", [0.1, 0.3, 0.6])
def test_group_pooled_selection_matches_brute_force(alpha):
    q, k, v = _rand_qkv(300, 6, 2, 8, seed=31, scale=3.0)     # g = 3, 19 blocks, ragged last block
    sel = O.select_blocks(q, k, v, 16, alpha, shared="pooled")
    keep, band = _brute_force_group_pooled(q, k, 16, alpha)
    outside = ~(sel.band | band)
    assert np.array_equal(sel.keep[outside], keep[outside])
    for hk in range(2):
        assert (sel.keep[hk * 3:(hk + 1) * 3] == sel.keep[hk * 3]).all()


def test_group_pooled_logits_are_the_head_mean():
    """Block logits are linear in q_bar, so the group-pooled logit of a block
    pair is the mean of the group's per-head logits."""
    q, k, v = _rand_qkv(256, 8, 2, 16, seed=32)
    own = O.select_blocks(q, k, v, 32, 0.2)
    pooled = O.select_blocks(q, k, v, 32, 0.2, shared="pooled")
    fin = np.isfinite(own.s)
    mean = own.s.reshape(2, 4, 8, 8).mean(axis=1)
    ref = np.repeat(mean, 4, axis=0)
    assert np.allclose(pooled.s[fin], ref[fin], rtol=0, atol=1e-12)
    assert np.array_equal(np.isfinite(pooled.s), fin)


def test_group_pooled_equals_per_head_when_heads_agree():
    q, k, v = _rand_qkv(200, 3, 3, 8, seed=33, scale=2.0)      # g = 1
    own = O.select_blocks(q, k, v, 16, 0.4)
    pooled = O.select_blocks(q, k, v, 16, 0.4, shared="pooled")
    assert np.array_equal(own.keep, pooled.keep) and np.array_equal(own.band, pooled.band)
    q1 = np.repeat(q[:, :1], 4, axis=1)                          # g = 4, four equal heads
    own = O.select_blocks(q1, k[:, :1], v[:, :1], 16, 0.4)
    pooled = O.select_blocks(q1, k[:, :1], v[:, :1], 16, 0.4, shared="pooled")
    assert np.array_equal(own.keep, pooled.keep)


def test_group_pooled_chunked_equals_full_rows():
    q, k, v = _rand_qkv(133, 4, 2, 8, seed=34, scale=1.3)
    full = O.select_blocks(q, k, v, 32, 0.3, shared="pooled")
    ch = O.select_blocks_chunked(q[64:], k, v, 32, 0.3, shared="pooled")
    assert np.array_equal(ch.keep, full.keep[:, 2:, :])


def test_unknown_group_sharing_rejected():
    q, k, v = _rand_qkv(64, 2, 1, 8, seed=35)
    with pytest.raises(ValueError):
        O.select_blocks(q, k, v, 32, 0.3, shared="mean")


# ------------------------------------------------- skeleton-query scoring

def test_skeleton_query_means_brute_force():
    x = np.random.default_rng(8).standard_normal((45, 3, 5))
    for P, st in ((16, 1), (4, 4), (2, 8), (1, 16)):
        m = O.block_means(x, 16, O.probe_stride(16, P))
        for h in range(3):
            for J in range(3):
                toks = range(16 * J, min(45, 16 * J + 16), st)
                for c in range(5):
                    assert abs(m[h, J, c] - math.fsum(x[t, h, c] for t in toks) / len(toks)) < 1e-15
    assert np.array_equal(O.block_means(x, 16, 1), O.block_means(x, 16))
    with pytest.raises(ValueError):
        O.probe_stride(16, 3)


def test_skeleton_selection_uses_only_the_probes():
    """Changing non-probe queries leaves the mask alone; with one probe per
    block the mask equals brute-force scoring of each block's first query."""
    q, k, v = synth.make_sequence(320, 4, 2, 16, seed=13, verticals=False)
    q, k, v = q.float().numpy(), k.float().numpy(), v.float().numpy()
    a = O.select_blocks(q, k, v, 32, 0.3, probes=4)
    q2 = q.copy()
    q2[np.arange(320) % 8 != 0] += 5.0
    b = O.select_blocks(q2, k, v, 32, 0.3, probes=4)
    assert np.array_equal(a.keep, b.keep) and np.array_equal(a.q_bar, b.q_bar)
    assert not np.array_equal(O.select_blocks(q2, k, v, 32, 0.3).q_bar, a.q_bar)
    one = O.select_blocks(q, k, v, 32, 0.3, probes=1)
    keep_bf, band_bf = _brute_force_keep(q[::32].repeat(32, axis=0)[:320], k, 32, 0.3)
    outside = ~(one.band | band_bf)
    assert np.array_equal(one.keep[outside], keep_bf[outside])
    full = O.select_blocks(q, k, v, 32, 0.3, probes=32)
    assert np.array_equal(full.keep, O.select_blocks(q, k, v, 32, 0.3).keep)

"""Checks of the seeded input generator and the bf16 / fp8 encoders it uses."""
import hashlib
import math

import numpy as np
import torch

from block_sparse_long_pooling_amd import synth


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Independent float32 -> bf16 round-to-nearest-even on the bit pattern."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _e4m3fn_value_table():
    """All finite OCP e4m3fn values (codes 0..126 positive), from the format."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_generator_is_deterministic_and_chunk_free():
    a = synth.make_sequence(300, 4, 2, 16, seed=3, verticals=True)
    b = synth.make_sequence(300, 4, 2, 16, seed=3, verticals=True, chunk=37)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = synth.make_sequence(300, 4, 2, 16, seed=4, verticals=True)
    assert not torch.equal(a[0], c[0])


def test_generator_structure():
    S, d = 8200, 16
    q, k, v = synth.make_sequence(S, 2, 1, d, seed=2, verticals=True)
    r = np.random.default_rng(2)
    q0 = r.standard_normal((S, 2, d), dtype=np.float32)
    k0 = r.standard_normal((S, 1, d), dtype=np.float32)
    v0 = r.standard_normal((S, 1, d), dtype=np.float32)
    u = r.standard_normal(d, dtype=np.float32).astype(np.float64)
    w = r.standard_normal(d, dtype=np.float32).astype(np.float64)
    u *= 3 / np.linalg.norm(u)
    w *= 3 / np.linalg.norm(w)
    t = np.arange(S)[:, None]
    omega = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    pos = np.zeros((S, d))
    pos[:, 0::2] = np.sin(t * omega)
    pos[:, 1::2] = np.cos(t * omega)
    kk = k0[:, 0].astype(np.float64) + pos
    kk[:4] += u
    kk[4096] += w
    kk[8192] += w
    assert np.abs(k[:, 0].float().numpy() - kk).max() < 0.05            # bf16 rounding
    assert np.abs(q.float().numpy() - (q0 + pos[:, None].astype(np.float32))).max() < 0.05
    assert np.abs(v.float().numpy() - v0).max() < 0.02
    # v carries no positional term
    assert abs(float(v.float().mean())) < 0.02


def test_bf16_cast_is_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    # include exact ties
    x[:4] = np.array([1.00390625, 1.01171875, -3.0078125, 0.0], dtype=np.float32)
    got = synth.to_bf16(x).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _bf16_rne_bits(x))


def test_fp8_quantizer_matches_format_and_bounds():
    q, _, _ = synth.make_sequence(300, 3, 1, 32, seed=9, verticals=False)
    codes, scales = synth.quantize_fp8_blockwise(q, 128)
    assert scales.shape == (3, 3)
    table = _e4m3fn_value_table()
    dec = synth.fp8_codes_to_float(codes).numpy().astype(np.float64)
    # decode through the format table
    c = codes.numpy()
    mag = table[c & 0x7F]
    sign = np.where(c & 0x80, -1.0, 1.0)
    assert np.array_equal(dec, sign * mag)
    xs = q.float().numpy().astype(np.float64)
    for h in range(3):
        for J in range(3):
            seg = xs[J * 128:(J + 1) * 128, h]
            amax = np.abs(seg).max()
            assert abs(scales[h, J].item() - np.float32(amax) / np.float32(448)) <= 1e-7 * amax
            y = seg / scales[h, J].item()
            d = dec[J * 128:(J + 1) * 128, h]
            assert np.abs(d).max() <= 448
            # nearest representable value: error at most half a step
            normal = np.abs(y) >= 2.0 ** -6
            rel = np.abs(d[normal] - y[normal]) / np.abs(y[normal])
            assert rel.max() <= 2.0 ** -4 + 1e-12
            sub = ~normal
            if sub.any():
                assert np.abs(d[sub] - y[sub]).max() <= 2.0 ** -10 + 1e-15


def test_fp8_zero_block_scale_is_one():
    x = torch.zeros((128, 1, 8), dtype=torch.bfloat16)
    codes, scales = synth.quantize_fp8_blockwise(x, 128)
    assert scales.item() == 1.0 and int(codes.sum()) == 0


def test_paged_batch_layout():
    pb = synth.make_paged_batch([100, 64, 200], 4, 2, 16, seed_base=500, verticals=True,
                                page_size=16)
    assert pb.cu_seqlens.tolist() == [0, 100, 164, 364]
    assert pb.k_cache.shape[0] == math.ceil(1.25 * 364 / 16)
    used = set()
    for b, S in enumerate(pb.seqlens):
        qb, kb, vb = pb.requests[b]
        assert torch.equal(pb.q[pb.cu_seqlens[b]:pb.cu_seqlens[b + 1]], qb)
        for t in range(S):
            page = int(pb.block_table[b, t // 16])
            used.add(page)
            assert torch.equal(pb.k_cache[page, t % 16], kb[t])
            assert torch.equal(pb.v_cache[page, t % 16], vb[t])
        # the tail of the last page holds NaN
        last = int(pb.block_table[b, (S - 1) // 16])
        if S % 16:
            assert torch.isnan(pb.k_cache[last, S % 16:].float()).all()
    assert len(used) == sum((s + 15) // 16 for s in pb.seqlens)
    # each request regenerates from seed_base + b with positions from 0
    q1, _, _ = synth.make_sequence(64, 4, 2, 16, seed=501, verticals=True)
    assert torch.equal(pb.requests[1][0], q1)


def test_workload_table():
    w = synth.WORKLOADS["paged_batch8"]
    assert w.total_tokens == 307200
    assert math.ceil(w.pool_factor * w.total_tokens / w.page_size) == 6000
    assert synth.WORKLOADS["llama8b_s128k"].alphas == (0.05, 0.1, 0.2)

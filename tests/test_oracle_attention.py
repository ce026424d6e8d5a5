"""Pins for the oracle attention: an independent library routine (torch SDPA in
float64 on the CPU), exact permutation invariance, closed forms and brute
force with scalar loops."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import cache as C
from oracle import fp8
from oracle.allocator import OracleAllocator


def _paged_f32(rng, lens, H, D, bs, N, order=None):
    """Write random float32 K/V for sequences of the given lengths through an
    oracle allocator; return the pools, tables and the logical K/V."""
    a = OracleAllocator(N, bs, order)
    kp = np.full((N, H, bs, D), 0x7FC00000, dtype=np.uint32)   # NaN sentinel
    vp = kp.copy()
    logical = []
    for s, n in enumerate(lens):
        slots = a.alloc_prompt(s, n)
        k = rng.standard_normal((n, H, D), dtype=np.float32)
        v = rng.standard_normal((n, H, D), dtype=np.float32)
        C.write_rows(kp, k.view(np.uint32), slots, bs)
        C.write_rows(vp, v.view(np.uint32), slots, bs)
        logical.append((k.astype(np.float64), v.astype(np.float64)))
    tables = [a.block_table(s) for s in range(len(lens))]
    return kp, vp, tables, logical


def _sdpa(q, k, v, mask, scale):
    """torch reference: q [S, D], k/v [L, D], boolean mask [S, L] (True = keep)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    out = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=t(mask), scale=scale)
    return out[0, 0].numpy()


def test_decode_equals_unpaged_sdpa():
    rng = np.random.default_rng(0)
    lens, H, D, bs = [1, 5, 16, 17, 40], 3, 32, 4
    kp, vp, tables, logical = _paged_f32(rng, lens, H, D, bs, 40, rng.permutation(40))
    q = rng.standard_normal((len(lens), H, D))
    scale = 1 / math.sqrt(D)
    out = A.decode(q, kp, vp, C.F32, tables, lens, bs, scale)
    for i, (k, v) in enumerate(logical):
        for h in range(H):
            mask = np.ones((1, lens[i]), dtype=bool)
            ref = _sdpa(q[i, h][None], k[:, h], v[:, h], mask, scale)[0]
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-12)


def test_chunk_equals_unpaged_sdpa_bottom_right_mask():
    """Chunk rows sit at the end of the sequence: row r sees keys 0..L-S+r."""
    rng = np.random.default_rng(1)
    H, D, bs = 2, 16, 8
    ctx, S = [0, 3, 20], [5, 8, 13]
    lens = [c + s for c, s in zip(ctx, S)]
    kp, vp, tables, logical = _paged_f32(rng, lens, H, D, bs, 30, rng.permutation(30))
    qsl = np.concatenate([[0], np.cumsum(S)])
    q = rng.standard_normal((qsl[-1], H, D))
    scale = 0.3
    out = A.prefill_chunk(q, qsl, kp, vp, C.F32, tables, lens, bs, scale)
    for i, (k, v) in enumerate(logical):
        L = lens[i]
        mask = np.zeros((S[i], L), dtype=bool)
        for r in range(S[i]):
            mask[r, : ctx[i] + r + 1] = True
        for h in range(H):
            ref = _sdpa(q[qsl[i]:qsl[i + 1], h], k[:, h], v[:, h], mask, scale)
            np.testing.assert_allclose(out[qsl[i]:qsl[i + 1], h], ref, rtol=0, atol=1e-12)


def test_chunk_without_context_equals_sdpa_is_causal():
    rng = np.random.default_rng(2)
    H, D, bs, S = 2, 16, 4, 11
    kp, vp, tables, logical = _paged_f32(rng, [S], H, D, bs, 10, rng.permutation(10))
    q = rng.standard_normal((S, H, D))
    out = A.prefill_chunk(q, [0, S], kp, vp, C.F32, tables, [S], bs, 0.25)
    k, v = logical[0]
    for h in range(H):
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
        ref = F.scaled_dot_product_attention(t(q[:, h]), t(k[:, h]), t(v[:, h]), is_causal=True,
                                             scale=0.25)[0, 0].numpy()
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def test_chunk_row_equals_decode_of_truncated_sequence():
    rng = np.random.default_rng(3)
    H, D, bs, ctx, S = 2, 16, 4, 6, 7
    L = ctx + S
    kp, vp, tables, _ = _paged_f32(rng, [L], H, D, bs, 10, rng.permutation(10))
    q = rng.standard_normal((S, H, D))
    out = A.prefill_chunk(q, [0, S], kp, vp, C.F32, tables, [L], bs, 0.2)
    for r in range(S):
        d = A.decode(q[r][None], kp, vp, C.F32, tables, [ctx + r + 1], bs, 0.2)
        assert np.array_equal(out[r], d[0])


def test_output_exactly_invariant_under_physical_permutation():
    rng = np.random.default_rng(4)
    lens, H, D, bs, N = [9, 4, 13], 2, 8, 4, 16
    x = [(rng.standard_normal((n, H, D), dtype=np.float32),
          rng.standard_normal((n, H, D), dtype=np.float32)) for n in lens]
    q = rng.standard_normal((3, H, D))
    outs = []
    for order in [None, rng.permutation(N), rng.permutation(N)[::-1]]:
        a = OracleAllocator(N, bs, order)
        kp = np.zeros((N, H, bs, D), dtype=np.uint32)
        vp = kp.copy()
        for s, (k, v) in enumerate(x):
            slots = a.alloc_prompt(s, lens[s])
            C.write_rows(kp, k.view(np.uint32), slots, bs)
            C.write_rows(vp, v.view(np.uint32), slots, bs)
        tables = [a.block_table(s) for s in range(3)]
        outs.append(A.decode(q, kp, vp, C.F32, tables, lens, bs, 0.35))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 8
    V = rng.standard_normal((6, D))
    K = rng.standard_normal((6, D))
    # one key: the output is that value row
    assert np.array_equal(A.attend(rng.standard_normal((1, D)), K[:1], V[:1], 0.7, [1])[0], V[0])
    # zero query or identical keys: the mean of V
    np.testing.assert_allclose(A.attend(np.zeros((1, D)), K, V, 0.7, [6])[0], V.mean(0), atol=1e-15)
    Keq = np.repeat(K[:1], 6, axis=0)
    np.testing.assert_allclose(A.attend(rng.standard_normal((1, D)), Keq, V, 0.7, [6])[0],
                               V.mean(0), atol=1e-15)
    # no visible key: zeros
    assert np.all(A.attend(rng.standard_normal((1, D)), K[:0], V[:0], 0.7, [0]) == 0)
    # one dominant key: the output approaches that key's value row
    q = 40.0 * K[2] / np.linalg.norm(K[2])
    Kd = K.copy()
    Kd[2] = q
    out = A.attend(q[None], Kd, V, 1.0, [6])[0]
    np.testing.assert_allclose(out, V[2], atol=1e-12)


def _brute_decode(q, K, V, scale):
    """Scalar loops with math.exp and math.fsum."""
    L, D = len(K), len(q)
    s = [scale * math.fsum(q[d] * K[j][d] for d in range(D)) for j in range(L)]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    z = math.fsum(p)
    return [math.fsum(p[j] * V[j][d] for j in range(L)) / z for d in range(D)]


def test_brute_force_tiny_decode_shape():
    """The tiny decode shape: 3 sequences of 6, 9, 5 tokens, 4 heads x 64,
    block 4, a shuffled pool of 10 blocks."""
    rng = np.random.default_rng(6)
    lens, H, D, bs = [6, 9, 5], 4, 64, 4
    kp, vp, tables, logical = _paged_f32(rng, lens, H, D, bs, 10, rng.permutation(10))
    q = rng.standard_normal((3, H, D))
    out = A.decode(q, kp, vp, C.F32, tables, lens, bs, 1 / 8)
    for i, (k, v) in enumerate(logical):
        for h in range(H):
            ref = _brute_decode(q[i, h].tolist(), k[:, h].tolist(), v[:, h].tolist(), 1 / 8)
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-13)


def test_fp8_pool_equals_dequantised_float_pool():
    """fp8 storage: code value times the (block, head) scale, per block."""
    rng = np.random.default_rng(7)
    H, D, bs, N = 2, 16, 4, 8
    lens = [7, 3]
    a = OracleAllocator(N, bs, rng.permutation(N))
    kc = np.zeros((N, H, bs, D), dtype=np.uint8)
    vc = kc.copy()
    ks = rng.uniform(0.01, 0.1, (N, H)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, (N, H)).astype(np.float32)
    for s, n in enumerate(lens):
        slots = a.alloc_prompt(s, n)
        C.write_rows_fp8(kc, rng.standard_normal((n, H, D), dtype=np.float32), slots, ks, bs)
        C.write_rows_fp8(vc, rng.standard_normal((n, H, D), dtype=np.float32), slots, vs, bs)
    # dequantise position by position (code value * scale of the block holding it)
    tables = [a.block_table(s) for s in range(2)]
    q = rng.standard_normal((2, H, D))
    out = A.decode(q, kc, vc, C.FP8, tables, lens, bs, 0.25, ks, vs)
    for i in range(2):
        Kd = np.stack([fp8.decode(kc[tables[i][p // bs], :, p % bs, :]) *
                       ks[tables[i][p // bs]][:, None].astype(np.float64) for p in range(lens[i])])
        Vd = np.stack([fp8.decode(vc[tables[i][p // bs], :, p % bs, :]) *
                       vs[tables[i][p // bs]][:, None].astype(np.float64) for p in range(lens[i])])
        for h in range(H):
            ref = _brute_decode(q[i, h].tolist(), Kd[:, h].tolist(), Vd[:, h].tolist(), 0.25)
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-13)


def test_fp8_write_quantises_with_block_scale():
    rng = np.random.default_rng(8)
    N, H, bs, D = 4, 2, 4, 8
    codes = np.zeros((N, H, bs, D), dtype=np.uint8)
    scales = np.array([[0.5, 2.0]] * N, dtype=np.float32)
    x = rng.standard_normal((3, H, D), dtype=np.float32) * 4
    C.write_rows_fp8(codes, x, [5, -1, 14], scales, bs)
    assert np.array_equal(codes[1, 0, 1], fp8.encode((x[0, 0] / np.float32(0.5)).astype(np.float64)))
    assert np.array_equal(codes[1, 1, 1], fp8.encode((x[0, 1] / np.float32(2.0)).astype(np.float64)))
    assert np.array_equal(codes[3, 1, 2], fp8.encode((x[2, 1] / np.float32(2.0)).astype(np.float64)))
    assert codes.sum() == codes[1, :, 1].sum() + codes[3, :, 2].sum()      # slot -1 skipped


def test_storage_decoders():
    x = np.array([1.5, -2.25, 3.0e-5, 65504.0], dtype=np.float32)
    assert np.array_equal(C.to_float64(x.view(np.uint32), C.F32), x.astype(np.float64))
    h = x.astype(np.float16)
    assert np.array_equal(C.to_float64(h.view(np.uint16), C.F16), h.astype(np.float64))
    b = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(C.to_float64(b.view(torch.int16).numpy().view(np.uint16), C.BF16),
                          b.to(torch.float64).numpy())

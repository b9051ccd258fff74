"""Pins for the fp64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something fixed outside it: a library
routine (torch's float8/bfloat16 casts, numpy complex rotation, scipy
softmax), exact rational brute force, a closed form, an invariant the pages
state, or a brute-force sort.  A dropped term, wrong sign, wrong index or
transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# codecs
# --------------------------------------------------------------------------
def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # OCP E4M3FN landmarks: max finite, smallest subnormal, smallest normal, one
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0


def test_e4m3_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(1)
    mags = np.concatenate([rng.uniform(0, 460, 3000), np.exp(rng.uniform(-14, 6, 3000)),
                           rng.uniform(0, 0.02, 1000)]).astype(np.float32)
    x = np.concatenate([mags, -mags]).astype(np.float32)
    # exact midpoints between neighbours exercise the even tie rule
    tab = orc.e4m3_table()
    pos = np.sort(tab[(~np.isnan(tab)) & (tab >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.f64_to_e4m3(float(v)) for v in x], dtype=np.uint8)
    ref = np.where(ref == 0x80, 0, ref)  # the oracle emits +0 for a rounded-away negative
    assert np.array_equal(got, ref)
    # saturation at +-448 (torch gives NaN there, the FP8 cache saturates)
    assert orc.f64_to_e4m3(1000.0) == 0x7E and orc.f64_to_e4m3(-1e6) == 0xFE


def test_bf16_encode_matches_torch(orc):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(4000), np.exp(rng.uniform(-100, 80, 2000))]).astype(np.float32)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f64_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = orc.bf16_array_to_f64(got)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_e2m1_and_e8m0_tables(orc):
    # OCP Microscaling Formats v1.0, FP4 E2M1 magnitudes (codes 0..7)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [orc.e2m1_to_f64(c) for c in range(8)] == grid
    assert [orc.e2m1_to_f64(c | 8) for c in range(1, 8)] == [-g for g in grid[1:]]
    assert orc.e8m0_to_f64(127) == 1.0 and orc.e8m0_to_f64(130) == 8.0 and orc.e8m0_to_f64(120) == 2.0 ** -7
    assert math.isnan(orc.e8m0_to_f64(255))


def test_fp4_to_fp8_lossless(orc):
    """[zcldvi]: E4M3 has two more exponent bits than E2M1, so FP4 -> FP8 dequantisation is lossless."""
    for c in range(16):
        v = orc.e2m1_to_f64(c)
        for e in range(-8, 7):  # block scales that keep the value inside the E4M3 range
            x = v * 2.0 ** e
            if x != 0 and abs(x) < 2.0 ** -9:
                continue
            assert orc.e4m3_to_f64(orc.f64_to_e4m3(x)) == x


# --------------------------------------------------------------------------
# RoPE on the last 64 dims
# --------------------------------------------------------------------------
def test_rope_against_complex_rotation(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64)
    for pos in [0, 1, 7, 4095, 1048575]:
        z = x[0::2] + 1j * x[1::2]
        theta = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)
        zr = z * np.exp(1j * pos * theta)
        ref = np.empty(64)
        ref[0::2], ref[1::2] = zr.real, zr.imag
        # fp64 angles: theta may differ by an ulp between libms, scaled by pos
        assert np.allclose(orc.rope64(x, pos), ref, rtol=0, atol=1e-12 + 1e-14 * pos)


def test_rope_invariants(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal(64)
    assert np.array_equal(orc.rope64(x, 0), x)
    for a, b in [(3, 5), (1000, 24), (1 << 19, 1 << 19)]:
        r = orc.rope64(x, a)
        assert abs(np.linalg.norm(r) - np.linalg.norm(x)) < 1e-12
        assert np.allclose(orc.rope64(r, b), orc.rope64(x, a + b), atol=1e-9)
        assert np.allclose(orc.rope64(r, a, inverse=True), x, atol=1e-9)


# --------------------------------------------------------------------------
# compression
# --------------------------------------------------------------------------
def _dq(orc, ent):
    return orc.dequant_entries(*ent)


def _e4m3_quantum(v):
    """spacing of the E4M3 grid around |v| (scaled values)."""
    a = np.maximum(np.abs(v), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(a)) - 3)


def test_compress_m1_is_quantised_roped_token(orc, gen):
    d = 128
    kv = gen.normal_bf16(11, 1, (16, d))
    logits = gen.normal_f32(11, 2, (16,))
    nope, rope, scale = orc.compress(kv, logits, 0, 1)
    x = orc.bf16_array_to_f64(kv)
    for p in range(16):
        s = float(scale[p])
        assert s == np.float32(np.max(np.abs(x[p, :64])) / 448.0)
        deq = orc.e4m3_table()[nope[p]] * s
        assert np.all(np.abs(deq - x[p, :64]) <= 0.5 * _e4m3_quantum(x[p, :64] / s) * s + 1e-15)
        r = orc.rope64(x[p, 64:], p)
        rb = orc.bf16_array_to_f64(rope[p])
        assert np.all(np.abs(rb - r) <= np.abs(r) * 2.0 ** -8 + 1e-30)


def test_compress_weights_are_block_softmax(orc, gen):
    """One-hot tokens read the weights back: entry dim i = weight of token i (scipy softmax)."""
    from scipy.special import softmax

    m, d = 4, 128
    nblk = 6
    x = np.zeros((nblk * m, d))
    for t in range(nblk * m):
        x[t, t % m] = 1.0
    kv = np.array([orc.f64_to_bf16(v) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)
    logits = gen.normal_f32(12, 2, (nblk * m,))
    ent = orc.compress(kv, logits, 0, m)
    deq = _dq(orc, ent)
    for b in range(nblk):
        w = softmax(logits[b * m:(b + 1) * m].astype(np.float64))
        s = float(ent[2][b])
        assert np.all(np.abs(deq[b, :m] - w) <= 0.5 * _e4m3_quantum(w / s) * s + 1e-15)
        assert np.all(deq[b, m:64] == 0)


def test_compress_uniform_logits_is_mean(orc, gen):
    m, d = 4, 512
    kv = gen.normal_bf16(13, 1, (64, d))
    logits = np.zeros(64, np.float32)
    ent = orc.compress(kv, logits, 0, m)
    x = orc.bf16_array_to_f64(kv)
    deq = _dq(orc, ent)
    for b in range(16):
        mean = x[b * m:(b + 1) * m].mean(axis=0)
        s = float(ent[2][b])
        assert np.all(np.abs(deq[b, :448] - mean[:448]) <= 0.5 * _e4m3_quantum(mean[:448] / s) * s + 1e-15)
        r = orc.rope64(mean[448:], (b + 1) * m - 1)
        assert np.all(np.abs(deq[b, 448:] - r) <= np.abs(r) * 2.0 ** -8 + 1e-30)


def test_compress_constant_block_and_permutation(orc, gen):
    m, d = 4, 128
    base = gen.normal_bf16(14, 1, (8, d))
    kv = np.repeat(base, m, axis=0)  # 8 constant blocks
    logits = gen.normal_f32(14, 2, (8 * m,))
    ent = orc.compress(kv, logits, 0, m)
    # a constant block equals the m=1 entry of its last token (same position)
    one = orc.compress(kv, logits, 0, 1)
    last = np.arange(8) * m + m - 1
    assert np.allclose(_dq(orc, ent), _dq(orc, tuple(a[last] for a in one)), rtol=0, atol=1e-12)
    # permuting tokens together with their logits inside a block changes nothing
    kv2 = gen.normal_bf16(14, 3, (32, d))
    lg2 = gen.normal_f32(14, 4, (32,))
    perm = np.concatenate([b * m + np.random.default_rng(b).permutation(m) for b in range(8)])
    a = _dq(orc, orc.compress(kv2, lg2, 0, m))
    b = _dq(orc, orc.compress(kv2[perm], lg2[perm], 0, m))
    # fp64 summation order may move a value across an FP8/bf16 rounding boundary, nothing more
    assert np.mean(a == b) > 0.999
    diff = np.abs(a - b)
    assert np.all(diff <= np.abs(a) * 2.0 ** -3 + 1e-12)


def test_compress_chunked_equals_whole(orc, gen):
    m, d = 4, 128
    kv = gen.normal_bf16(15, 1, (96, d))
    logits = gen.normal_f32(15, 2, (96,))
    whole = orc.compress(kv, logits, 0, m)
    tail = orc.compress(kv[40:], logits[40:], 40, m)
    for a, b in zip(whole, tail):
        assert np.array_equal(a[10:], b)
    with pytest.raises(AssertionError):
        orc.compress(kv[2:], logits[2:], 2, m)


# --------------------------------------------------------------------------
# index scores
# --------------------------------------------------------------------------
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _mx_frac(data, scale, row, d_i):
    out = []
    for c in range(d_i):
        byte = int(data[row, c // 2])
        nib = (byte >> 4) if c & 1 else (byte & 15)
        v = E2M1[nib & 7] * (-1 if nib & 8 else 1)
        out.append(v * Fraction(2) ** (int(scale[row, c // 32]) - 127))
    return out


def test_index_scores_exact_bruteforce(orc, gen):
    T, h_i, d_i, N, m = 3, 4, 64, 10, 4
    kd, ks, _ = gen.mxfp4(21, 1, N, d_i)
    qd, qs, _ = gen.mxfp4(21, 2, T * h_i, d_i)
    w = gen.pow2_weights(21, 3, (T, h_i))
    pos = np.array([39, 17, 2], np.int64)
    seq = np.zeros(T, np.int32)
    got = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, N)
    for t in range(T):
        qv = [_mx_frac(qd, qs, t * h_i + h, d_i) for h in range(h_i)]
        for j in range(N):
            if j >= (pos[t] + 1) // m:
                assert got[t, j] == -np.inf
                continue
            kv = _mx_frac(kd, ks, j, d_i)
            exact = sum(Fraction(float(w[t, h])) * max(Fraction(0), sum(a * b for a, b in zip(qv[h], kv)))
                        for h in range(h_i))
            assert Fraction(got[t, j]) == exact


def test_index_scores_closed_form_and_scale(orc, gen):
    T, h_i, d_i, N = 2, 8, 128, 5
    ones = np.full((N, d_i // 2), 0x22, np.uint8)  # every element E2M1 1.0
    unit = np.full((N, d_i // 32), 127, np.uint8)
    qd = np.full((T * h_i, d_i // 2), 0x22, np.uint8)
    qs = np.full((T * h_i, d_i // 32), 127, np.uint8)
    w = gen.pow2_weights(22, 1, (T, h_i))
    pos = np.full(T, 4 * N - 1, np.int64)
    seq = np.zeros(T, np.int32)
    got = orc.index_scores(qd, qs, w, seq, pos, ones, unit, N, 4, N)
    assert np.array_equal(got, np.repeat((w.sum(axis=1).astype(np.float64) * d_i)[:, None], N, axis=1))
    # doubling every key block scale doubles every score and keeps the order
    kd, ks, _ = gen.mxfp4(22, 2, 64, d_i)
    qd, qs, _ = gen.mxfp4(22, 3, T * h_i, d_i)
    pos = np.full(T, 255, np.int64)
    s1 = orc.index_scores(qd, qs, w, seq, pos, kd, ks, 64, 4, 64)
    s2 = orc.index_scores(qd, qs, w, seq, pos, kd, ks + 1, 64, 4, 64)
    assert np.array_equal(s2, 2 * s1)
    assert np.array_equal(orc.topk(s1.astype(np.float32), pos, 4, 16), orc.topk(s2.astype(np.float32), pos, 4, 16))


def test_index_negated_query_zeroes_relu(orc, gen):
    """ReLU per head: a query and its negation cannot both score above zero on one head."""
    T, h_i, d_i, N = 1, 1, 64, 32
    kd, ks, _ = gen.mxfp4(23, 1, N, d_i)
    qd, qs, _ = gen.mxfp4(23, 2, 1, d_i)
    neg = qd ^ np.uint8(0x88)
    w = np.ones((1, 1), np.float32)
    pos = np.full(1, 4 * N - 1, np.int64)
    seq = np.zeros(1, np.int32)
    a = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, 4, N)
    b = orc.index_scores(neg, qs, w, seq, pos, kd, ks, N, 4, N)
    assert np.all((a == 0) | (b == 0))
    assert np.any(a > 0) and np.any(b > 0)


def test_index_exact_witness_closed_forms(orc, gen):
    """The fp32-exactness witness: log2 of (sum of |product terms|) over the finest
    quantum a term can carry (1/4 x q scale x key scale x head weight), worst visible
    (row, column); +inf for a head weight that is not a power of two."""
    d_i, N, m = 128, 4, 4
    ones = np.full((N, d_i // 2), 0x22, np.uint8)  # every element E2M1 1.0
    unit = np.full((N, d_i // 32), 127, np.uint8)
    q1 = np.full((1, d_i // 2), 0x22, np.uint8)
    qs1 = np.full((1, d_i // 32), 127, np.uint8)
    seq, pos = np.zeros(1, np.int32), np.full(1, 4 * N - 1, np.int64)
    # one head, unit weight: 128 terms of 1 against a quantum of 1/4 -> log2(512) = 9
    w = np.ones((1, 1), np.float32)
    assert orc.index_exact_witness(q1, qs1, w, seq, pos, ones, unit, N, m, N) == 9.0
    # two heads, weights 1 and 1/2: (128 + 64) / (1/4 * 1/2) = 1536
    q2 = np.repeat(q1, 2, axis=0)
    qs2 = np.repeat(qs1, 2, axis=0)
    w2 = np.array([[1.0, 0.5]], np.float32)
    assert orc.index_exact_witness(q2, qs2, w2, seq, pos, ones, unit, N, m, N) == math.log2(1536.0)
    # a key block scale 2^-30 beside unit blocks: the quantum falls by 2^30, the sum barely moves
    ks = unit.copy()
    ks[:, 1] = 127 - 30
    got = orc.index_exact_witness(q1, qs1, w, seq, pos, ones, ks, N, m, N)
    assert got >= 24 and got == math.log2((96 + 32 * 2.0 ** -30) / (0.25 * 2.0 ** -30))
    # a head weight that is not a power of two
    w3 = np.array([[0.75]], np.float32)
    assert orc.index_exact_witness(q1, qs1, w3, seq, pos, ones, unit, N, m, N) == math.inf
    # no visible column: nothing to check
    assert orc.index_exact_witness(q1, qs1, w, seq, np.full(1, 2, np.int64), ones, unit, N, m, N) == -math.inf
    # only visible columns count: a wide-span key beyond the row's position is ignored
    ks2 = unit.copy()
    ks2[N - 1, 1] = 127 - 30
    pos2 = np.full(1, 4 * (N - 1) - 1, np.int64)  # entries 0 .. N-2 visible
    assert orc.index_exact_witness(q1, qs1, w, seq, pos2, ones, ks2, N, m, N) == 9.0
    # the generator's N(0,1) data keeps a wide margin below 24 bits
    kd, kss, _ = gen.mxfp4(24, 1, 64, d_i)
    qd, qss, _ = gen.mxfp4(24, 2, 8, d_i)
    wg = gen.pow2_weights(24, 3, (1, 8))
    wit = orc.index_exact_witness(qd, qss, wg, seq, np.full(1, 255, np.int64), kd, kss, 64, m, 64)
    assert 9.0 < wit < 20.0


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------
def _brute_topk(scores, nv, k):
    cand = sorted(range(nv), key=lambda j: (-float(scores[j]), j))[:k]
    return sorted(cand) + [-1] * (k - min(k, nv))


def test_topk_bruteforce_with_ties(orc):
    rng = np.random.default_rng(5)
    T, n, m = 40, 300, 4
    scores = rng.integers(0, 12, size=(T, n)).astype(np.float32)  # many ties
    scores[::3] = rng.standard_normal((len(range(0, T, 3)), n)).astype(np.float32)
    pos = rng.integers(0, 4 * n + 8, size=T).astype(np.int64)
    for k in (1, 7, 64, 400):
        got = orc.topk(scores, pos, m, k)
        for t in range(T):
            nv = min(n, (int(pos[t]) + 1) // m)
            assert list(got[t]) == _brute_topk(scores[t], nv, k)


def test_topk_all_equal_takes_lowest(orc):
    scores = np.zeros((2, 100), np.float32)
    pos = np.array([399, 39], np.int64)
    got = orc.topk(scores, pos, 4, 16)
    assert list(got[0]) == list(range(16))
    assert list(got[1]) == list(range(10)) + [-1] * 6


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _cache(gen, seed, rows, dn):
    return gen.entries(seed, 40, rows, dn)


def test_sparse_with_all_selected_equals_dense(orc, gen):
    m, H, d, W, N = 4, 4, 128, 8, 64
    comp = _cache(gen, 31, N, d - 64)
    win = gen.entries(31, 41, 16, d - 64)
    q = gen.normal_bf16(31, 42, (3, H, d))
    pos = np.array([255, 130, 9], np.int64)
    seq = np.zeros(3, np.int32)
    nv = (pos + 1) // m
    idx = np.full((3, N), -1, np.int32)
    for t in range(3):
        idx[t, :nv[t]] = np.arange(nv[t])
    a = orc.attend(q, seq, pos, comp, N, win, 16, W, m, 1 / math.sqrt(d), idx=idx)
    b = orc.attend(q, seq, pos, comp, N, win, 16, W, m, 1 / math.sqrt(d))
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_m1_all_selected_no_window_is_causal_attention(orc, gen):
    """m=1, k=all, W=0: textbook causal softmax(Q K^T s) V with K=V and partial RoPE (numpy)."""
    T, H, d = 12, 3, 128
    kv = gen.normal_bf16(32, 1, (T, d))
    logits = gen.normal_f32(32, 2, (T,))
    comp = orc.compress(kv, logits, 0, 1)
    q = gen.normal_bf16(32, 3, (T, H, d))
    pos = np.arange(T, dtype=np.int64)
    seq = np.zeros(T, np.int32)
    idx = np.tile(np.arange(T, dtype=np.int32), (T, 1))
    dummy = gen.entries(32, 4, 1, d - 64)
    sm = 1 / math.sqrt(d)
    out, lse = orc.attend(q, seq, pos, comp, T, dummy, 1, 0, 1, sm, idx=idx)
    K = orc.dequant_entries(*comp)
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)

    def rot(v, p):
        z = (v[..., 0::2] + 1j * v[..., 1::2]) * np.exp(1j * p * theta)
        r = np.empty_like(v)
        r[..., 0::2], r[..., 1::2] = z.real, z.imag
        return r

    Q = orc.bf16_array_to_f64(q)
    for t in range(T):
        qr = Q[t].copy()
        qr[:, 64:] = rot(qr[:, 64:], t)
        s = qr @ K[:t + 1].T * sm
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ K[:t + 1]
        o[:, 64:] = rot(o[:, 64:], -t)
        assert np.allclose(out[t], o, rtol=1e-10, atol=1e-12)
        l = np.log(np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1)) + s.max(axis=1)
        assert np.allclose(lse[t], l, rtol=1e-12)


def test_single_key_closed_form_and_identical_keys(orc, gen):
    H, d, N, t = 2, 512, 8, 31
    comp = _cache(gen, 33, N, d - 64)
    win = gen.entries(33, 41, 1, d - 64)
    q = gen.normal_bf16(33, 42, (1, H, d))
    pos = np.array([t], np.int64)
    seq = np.zeros(1, np.int32)
    idx = np.array([[5, -1, -1]], np.int32)
    out, lse = orc.attend(q, seq, pos, comp, N, win, 1, 0, 4, 0.05, idx=idx)
    e = orc.dequant_entries(*comp)[5]
    ref = e.copy()
    ref[448:] = orc.rope64(e[448:], t, inverse=True)
    assert np.allclose(out[0], ref[None], rtol=0, atol=1e-12)
    qr = orc.bf16_array_to_f64(q[0])
    qr[:, 448:] = np.stack([orc.rope64(qr[h, 448:], t) for h in range(H)])
    assert np.allclose(lse[0], 0.05 * qr @ e, rtol=1e-12)
    # the same entry selected three times: softmax weights sum to one, output is that entry
    idx3 = np.array([[5, 5, 5]], np.int32)
    out3, lse3 = orc.attend(q, seq, pos, comp, N, win, 1, 0, 4, 0.05, idx=idx3)
    assert np.allclose(out3, out, rtol=0, atol=1e-12) and np.allclose(lse3, lse + math.log(3), atol=1e-12)


def test_lse_merge_of_branches(orc, gen):
    """The union softmax equals the log-sum-exp merge of the selected-only and window-only branches."""
    H, d, N, W, t = 4, 512, 256, 128, 1023
    comp = _cache(gen, 34, N, d - 64)
    win = gen.entries(34, 41, W, d - 64)
    q = gen.normal_bf16(34, 42, (1, H, d))
    pos = np.array([t], np.int64)
    seq = np.zeros(1, np.int32)
    idx = gen.random_idx(34, 43, np.array([N]), 64)
    sm = 1 / math.sqrt(d)
    full = orc.attend(q, seq, pos, comp, N, win, W, W, 4, sm, idx=idx)
    sel = orc.attend(q, seq, pos, comp, N, win, W, 0, 4, sm, idx=idx)
    wnd = orc.attend(q, seq, pos, comp, N, win, W, W, 4, sm, idx=np.full_like(idx, -1))
    l = np.logaddexp(sel[1], wnd[1])
    o = np.exp(sel[1] - l)[..., None] * sel[0] + np.exp(wnd[1] - l)[..., None] * wnd[0]
    assert np.allclose(full[1], l, rtol=1e-12) and np.allclose(full[0], o, rtol=1e-9, atol=1e-12)


def test_empty_key_set(orc, gen):
    d = 128
    comp = _cache(gen, 35, 4, d - 64)
    q = gen.normal_bf16(35, 42, (1, 2, d))
    out, lse = orc.attend(q, np.zeros(1, np.int32), np.array([2], np.int64), comp, 4, comp, 4, 0, 4, 0.1,
                          idx=np.array([[0, 1]], np.int32))  # pos 2 < m-1: nothing visible, no window
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# facts the pages state about the storage format
# --------------------------------------------------------------------------
def test_page_facts_fixture():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    f = {x["name"]: x for x in facts["facts"]}
    assert f["m"]["value"] == 4 and f["k"]["value"] == 1024 and f["window"]["value"] == 128
    assert f["m_hca"]["value"] == 128 and f["rope_dims"]["value"] == 64
    d = 512
    entry_bytes = (d - f["rope_dims"]["value"]) * 1 + f["rope_dims"]["value"] * 2 + 4
    ratio = entry_bytes / (d * 2)
    lo, hi = f["mixed_kv_vs_bf16"]["value"]
    assert lo <= ratio <= hi  # "close to half" of pure bf16


def test_window_branch_is_last_W_tokens(orc, gen):
    """Window only (nothing selected): textbook softmax over raw tokens max(0,t-W+1)..t from the ring."""
    H, d, W, cap = 2, 128, 5, 8
    ring = gen.entries(36, 41, cap, d - 64)
    q = gen.normal_bf16(36, 42, (4, H, d))
    pos = np.array([0, 3, 9, 21], np.int64)
    seq = np.zeros(4, np.int32)
    none = np.full((4, 2), -1, np.int32)
    sm = 1 / math.sqrt(d)
    out, lse = orc.attend(q, seq, pos, ring, cap, ring, cap, W, 4, sm, idx=none)
    E = orc.dequant_entries(*ring)
    Q = orc.bf16_array_to_f64(q)
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)

    def rot(v, p):
        z = (v[..., 0::2] + 1j * v[..., 1::2]) * np.exp(1j * p * theta)
        r = np.empty_like(v)
        r[..., 0::2], r[..., 1::2] = z.real, z.imag
        return r

    for i, t in enumerate(pos):
        toks = list(range(max(0, t - W + 1), t + 1))
        K = E[[p % cap for p in toks]]
        qr = Q[i].copy()
        qr[:, 64:] = rot(qr[:, 64:], t)
        s = qr @ K.T * sm
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ K
        o[:, 64:] = rot(o[:, 64:], -t)
        assert np.allclose(out[i], o, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# compression variants: per-channel weights, index-key compression to MXFP4
# ---------------------------------------------------------------------------
def test_compress_channel_equal_logits_is_scalar(orc, gen):
    """Per-channel logits that repeat the token's logit on every channel give the
    scalar-weight routine's bytes exactly."""
    m, d = 4, 256
    kv = gen.normal_bf16(31, 1, (32, d))
    logits = gen.normal_f32(31, 2, (32,))
    a = orc.compress(kv, logits, 8, m)
    b = orc.compress_channel(kv, np.repeat(logits[:, None], d, axis=1), 8, m)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_compress_channel_selects_per_channel(orc, gen):
    """Channel e with one logit 0 and the others -1000 (weights exactly 1 and 0)
    takes that token's value: the entry equals the m=1 entry of the token built
    channel by channel, at the block's RoPE position."""
    m, d = 4, 128
    nblk = 3
    kv = gen.normal_bf16(32, 1, (nblk * m, d))
    rng = np.random.default_rng(7)
    pick = rng.integers(0, m, size=(nblk, d))
    logits = np.full((nblk * m, d), -1000.0, np.float32)
    sel = np.zeros((nblk, d), np.uint16)
    for b in range(nblk):
        for e in range(d):
            logits[b * m + pick[b, e], e] = 0.0
            sel[b, e] = kv[b * m + pick[b, e], e]
    got = orc.compress_channel(kv, logits, 0, m)
    for b in range(nblk):
        p = (b + 1) * m - 1  # the block's entry is roped at its last token
        want = orc.compress(sel[b:b + 1], np.zeros(1, np.float32), p, 1)
        for x, y in zip(got, want):
            assert np.array_equal(x[b:b + 1], y)


def test_compress_channel_uniform_logits_is_mean(orc, gen):
    m, d = 2, 128
    kv = gen.normal_bf16(33, 1, (8, d))
    x = orc.bf16_array_to_f64(kv)
    rng = np.random.default_rng(3)
    logits = np.repeat(rng.standard_normal((4, 1, d)).astype(np.float32), m, axis=1).reshape(8, d)
    ent = orc.compress_channel(kv, logits, 0, m)
    deq = _dq(orc, ent)
    for b in range(4):
        mean = x[b * m:(b + 1) * m].mean(axis=0)
        s = float(ent[2][b])
        assert np.all(np.abs(deq[b, :64] - mean[:64]) <= 0.5 * _e4m3_quantum(mean[:64] / s) * s + 1e-15)


def _e2m1_brute(orc, v):
    """Nearest E2M1 code by search over all 16 codes (ties: even mantissa bit; +0 for zero)."""
    best, bd = 0, None
    for c in range(16):
        dc = abs(orc.e2m1_to_f64(c) - v)
        if bd is None or dc < bd or (dc == bd and (c & 1) == 0 and (best & 1) == 1):
            best, bd = c, dc
    mag = best & 7
    return (8 if (v < 0 and mag != 0) else 0) | mag


def test_e2m1_encoder_brute_force(orc):
    grid = [i / 8.0 for i in range(-64, 65)] + [0.24, 0.26, 0.749, 0.751, 4.99, 5.01, 5.5, 6.5, 7.0, 1e3, -1e3, -0.0]
    for v in grid:
        assert orc.f64_to_e2m1(v) == _e2m1_brute(orc, v), v


def test_mxfp4_scale_rule_and_zero_block(orc):
    rng = np.random.default_rng(11)
    for _ in range(200):
        c = rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)
        codes, sb = orc.mxfp4_block(c)
        amax = np.max(np.abs(c))
        assert 4.0 <= amax / 2.0 ** (sb - 127) < 8.0
        s = 2.0 ** (sb - 127)
        for x, k in zip(c, codes):
            assert k == _e2m1_brute(orc, x / s)
    codes, sb = orc.mxfp4_block(np.zeros(32))
    assert sb == 127 and not codes.any()


def test_compress_index_keys_m1_and_representable(orc, gen):
    """m=1: each token quantised alone (brute-force check); tokens made of E2M1 values
    times a power of two, block maximum 4 or 6, come back exactly."""
    d_i = 128
    k = gen.normal_bf16(34, 1, (6, d_i))
    data, scale = orc.compress_index_keys(k, np.zeros(6, np.float32), 0, 1)
    x = orc.bf16_array_to_f64(k)
    for t in range(6):
        for blk in range(d_i // 32):
            codes, sb = orc.mxfp4_block(x[t, 32 * blk:32 * blk + 32])
            assert scale[t, blk] == sb
            packed = data[t, 16 * blk:16 * blk + 16]
            assert np.array_equal(packed & 15, codes[0::2]) and np.array_equal(packed >> 4, codes[1::2])
    rng = np.random.default_rng(5)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for e in (-3, 0, 7):
        v = rng.choice(vals, size=(2, d_i)) * rng.choice([-1, 1], size=(2, d_i))
        v[:, ::32] = 6.0  # every block's maximum is 6: scale exactly 2^e
        tok = np.array([orc.f64_to_bf16(a) for a in (v * 2.0 ** e).ravel()], np.uint16).reshape(2, d_i)
        data, scale = orc.compress_index_keys(tok, np.zeros(2, np.float32), 0, 1)
        assert np.all(scale == 127 + e)
        dec = np.array([[orc.e2m1_to_f64(int(b) & 15), orc.e2m1_to_f64(int(b) >> 4)] for b in data.ravel()]).reshape(2, d_i)
        assert np.array_equal(dec * 2.0 ** e, v * 2.0 ** e)


def test_compress_index_keys_uniform_logits_mean(orc):
    """Two tokens, equal logits: the entry is their mean (chosen exactly representable)."""
    d_i = 64
    a = np.full(d_i, 4.0)
    b = np.full(d_i, 2.0)
    a[1::2], b[1::2] = -3.0, -1.0  # means 3 and -2
    tok = np.array([orc.f64_to_bf16(x) for x in np.concatenate([a, b])], np.uint16).reshape(2, d_i)
    data, scale = orc.compress_index_keys(tok, np.zeros(2, np.float32), 0, 2)
    dec = np.array([[orc.e2m1_to_f64(int(x) & 15), orc.e2m1_to_f64(int(x) >> 4)] for x in data[0]]).reshape(-1)
    # block maximum 3: scale 2^(floor(log2 3) - 2) = 1/2 (byte 126); 3 and -2 are 6 and -4 in E2M1
    assert np.all(scale[0] == 126)
    want = np.where(np.arange(d_i) % 2 == 0, 3.0, -2.0)
    assert np.array_equal(dec * 0.5, want)


# --------------------------------------------------------------------------
# attention gradient (oracle/backward.py)
# --------------------------------------------------------------------------
def _bw():
    from oracle import backward
    return backward


def _rotated(g, tp, d):
    gr = np.array(g, dtype=np.float64)
    gr[..., d - 64:] = _bw().rope_rows(gr[..., d - 64:], tp)
    return gr


def test_bwd_forward_core_matches_oracle_attend(orc, gen):
    """The fp64 forward the gradient is taken of is the oracle's attention step."""
    bw = _bw()
    m, H, d, W, N = 4, 4, 128, 8, 64
    comp = _cache(gen, 51, N, d - 64)
    win = gen.entries(51, 41, 16, d - 64)
    q = gen.normal_bf16(51, 42, (3, H, d))
    pos = np.array([255, 130, 9], np.int64)
    seq = np.zeros(3, np.int32)
    rng = np.random.default_rng(51)
    idx = rng.integers(-3, 70, size=(3, 12)).astype(np.int32)  # masked, out-of-range and valid picks
    sm = 1 / math.sqrt(d)
    out, lse = orc.attend(q, seq, pos, comp, N, win, 16, W, m, sm, idx=idx)
    qf = orc.bf16_array_to_f64(q)
    ce, we = orc.dequant_entries(*comp), orc.dequant_entries(*win)
    for t in range(3):
        rows = bw.key_rows(t, seq, pos, m, N, 16, W, idx)
        keys = np.stack([(ce if kd == "c" else we)[r] for kd, r in rows])
        o, l = bw.attend_core(qf[t], keys, int(pos[t]), sm)
        assert np.allclose(o, out[t], rtol=0, atol=1e-12) and np.allclose(l, lse[t], rtol=0, atol=1e-12)


def test_bwd_matches_central_differences():
    """Every element of dq and de against a central difference of the fp64 forward."""
    bw = _bw()
    rng = np.random.default_rng(52)
    H, d, n, tp, sm = 3, 128, 7, 1234, 0.09
    qh = rng.standard_normal((H, d))
    keys = rng.standard_normal((n, d)) * 1.5
    g = rng.standard_normal((H, d))
    dq, dk = bw.attend_core_bwd(qh, keys, tp, sm, g)

    def loss(qq, kk):
        return float((g * bw.attend_core(qq, kk, tp, sm)[0]).sum())

    h = 1e-6
    num_q = np.zeros_like(qh)
    for i in range(H):
        for e in range(d):
            a, b = qh.copy(), qh.copy()
            a[i, e] += h
            b[i, e] -= h
            num_q[i, e] = (loss(a, keys) - loss(b, keys)) / (2 * h)
    num_k = np.zeros_like(keys)
    for u in range(n):
        for e in range(d):
            a, b = keys.copy(), keys.copy()
            a[u, e] += h
            b[u, e] -= h
            num_k[u, e] = (loss(qh, a) - loss(qh, b)) / (2 * h)
    assert np.allclose(dq, num_q, rtol=1e-6, atol=1e-7)
    assert np.allclose(dk, num_k, rtol=1e-6, atol=1e-7)


def test_bwd_shift_of_all_entries_closed_form():
    """Shifting every entry by c leaves the softmax unchanged and moves each output by R(-tp) c,
    so the entry gradients sum to the rotated output gradients summed over heads."""
    bw = _bw()
    rng = np.random.default_rng(53)
    H, d, n, tp = 5, 128, 11, 777
    qh, keys, g = rng.standard_normal((H, d)), rng.standard_normal((n, d)), rng.standard_normal((H, d))
    _, dk = bw.attend_core_bwd(qh, keys, tp, 0.1, g)
    assert np.allclose(dk.sum(axis=0), _rotated(g, tp, d).sum(axis=0), rtol=1e-12, atol=1e-12)


def test_bwd_single_key():
    """One key: the softmax is constant (dq = 0) and the output is the key (de = sum_h g~_h)."""
    bw = _bw()
    rng = np.random.default_rng(54)
    H, d, tp = 4, 128, 41
    qh, key, g = rng.standard_normal((H, d)), rng.standard_normal((1, d)), rng.standard_normal((H, d))
    dq, dk = bw.attend_core_bwd(qh, key, tp, 0.2, g)
    assert np.abs(dq).max() < 1e-13
    assert np.allclose(dk[0], _rotated(g, tp, d).sum(axis=0), rtol=0, atol=1e-12)


def test_bwd_batch_accumulates_every_row(orc, gen):
    """Rows sharing entries: the accumulated entry gradients of the whole batch sum to the rotated
    output gradients of every row with keys; a row without keys has dq = 0."""
    bw = _bw()
    m, H, d, W, N = 4, 3, 128, 6, 48
    comp = _cache(gen, 55, 2 * N, d - 64)
    win = gen.entries(55, 41, 2 * 8, d - 64)
    T = 5
    q = gen.normal_bf16(55, 42, (T, H, d))
    pos = np.array([150, 151, 150, 2, 40], np.int64)
    seq = np.array([0, 0, 1, 1, 0], np.int32)
    rng = np.random.default_rng(55)
    idx = rng.integers(0, 30, size=(T, 10)).astype(np.int32)
    idx[3] = -1  # row 3 (position 2): no visible entry is selected; window 0 leaves it empty
    g = rng.standard_normal((T, H, d))
    W0 = np.array([W, W, W, 0, W])
    dq = np.zeros((T, H, d))
    tot = np.zeros(d)
    for t in range(T):  # rows with their own window sizes, one call each, summed
        dqt, dc, dw = bw.attend_bwd(q[t:t + 1], seq[t:t + 1], pos[t:t + 1], comp, N, win, 8, int(W0[t]), m,
                                    0.1, g[t:t + 1], idx=idx[t:t + 1])
        dq[t] = dqt[0]
        tot += dc.sum(axis=0) + dw.sum(axis=0)
    want = sum(_rotated(g[t], pos[t], d).sum(axis=0) for t in range(T) if t != 3)
    assert np.allclose(tot, want, rtol=1e-11, atol=1e-11)
    assert np.abs(dq[3]).max() == 0.0
    # the batch call accumulates the same entry gradients as the per-row calls
    keep = [0, 1, 2, 4]
    dqb, dcb, dwb = bw.attend_bwd(q[keep], seq[keep], pos[keep], comp, N, win, 8, W, m, 0.1, g[keep], idx=idx[keep])
    acc_c, acc_w = np.zeros_like(dcb), np.zeros_like(dwb)
    for t in keep:
        _, dc, dw = bw.attend_bwd(q[t:t + 1], seq[t:t + 1], pos[t:t + 1], comp, N, win, 8, W, m, 0.1, g[t:t + 1],
                                  idx=idx[t:t + 1])
        acc_c += dc
        acc_w += dw
    assert np.allclose(dcb, acc_c, rtol=1e-12, atol=1e-12) and np.allclose(dwb, acc_w, rtol=1e-12, atol=1e-12)
    assert np.array_equal(dqb, dq[keep])


# --------------------------------------------------------------------------
# indexer backward (oracle/index_backward.py)
# --------------------------------------------------------------------------
def _ibw():
    from oracle import index_backward

    return index_backward


def test_index_bwd_forward_core_matches_oracle(orc, gen):
    """The fp64 forward on dequantised values equals oracle.index_scores on the MXFP4 inputs."""
    ib = _ibw()
    T, h_i, d_i, N, B, m = 5, 8, 128, 300, 2, 4
    kd, ks, _ = gen.mxfp4(41, 1, B * N, d_i)
    qd, qs, _ = gen.mxfp4(41, 2, T * h_i, d_i)
    w = gen.pow2_weights(41, 3, (T, h_i))
    seq = np.array([0, 1, 0, 1, 1], np.int32)
    pos = np.array([1199, 700, 4, 1000, 3], np.int64)
    ref = orc.index_scores(qd.reshape(T, h_i, -1), qs.reshape(T, h_i, -1), w, seq, pos, kd, ks, N, m, N)
    qv = ib.dequant_mxfp4(qd, qs).reshape(T, h_i, d_i)
    got = ib.index_scores_f64(qv, w, ib.dequant_mxfp4(kd, ks), seq, pos, N, m, N)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.max(np.abs(got[fin] - ref[fin])) <= 1e-12 * np.max(np.abs(ref[fin]))


def test_index_bwd_matches_central_differences():
    """Every gradient element against central differences of L = sum G * score[idx] (continuous
    fp64 inputs; entries whose dot products sit within 1e-3 of the ReLU kink are excluded)."""
    ib = _ibw()
    rng = np.random.default_rng(42)
    T, h, d, N, B, m, k = 3, 4, 32, 12, 2, 1, 5
    qv = rng.standard_normal((T, h, d))
    kv = rng.standard_normal((B * N, d))
    w = rng.uniform(0.5, 2.0, (T, h))
    seq = np.array([0, 1, 0], np.int32)
    pos = np.array([N - 1, N - 1, 6], np.int64)
    idx = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[2, 0] = 9          # not visible at pos 6: ignored
    idx[1, 3] = -1         # padding: ignored
    G = rng.standard_normal((T, k))

    def loss(qv_, w_, kv_):
        s = ib.index_scores_f64(qv_, w_, kv_, seq, pos, N, m, N)
        tot = 0.0
        for t in range(T):
            for a in range(k):
                j = idx[t, a]
                if 0 <= j < (pos[t] + 1) // m:
                    tot += G[t, a] * s[t, j]
        return tot

    for t in range(T):  # keep every used dot product away from the kink
        for a in range(k):
            j = idx[t, a]
            if 0 <= j < (pos[t] + 1) // m:
                dots = qv[t] @ kv[seq[t] * N + j]
                assert np.all(np.abs(dots) > 1e-3)
    dq, dw, dk = ib.index_bwd_f64(qv, w, kv, seq, pos, N, m, idx, G)
    eps = 1e-6
    for arr, grad in ((qv, dq), (w, dw), (kv, dk)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = arr[i]
            arr[i] = old + eps
            lp = loss(qv, w, kv)
            arr[i] = old - eps
            lm = loss(qv, w, kv)
            arr[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd)), f"{i}: {fd} vs {grad[i]}"


def test_index_bwd_closed_forms():
    """One head, unit weight, one selected key: with <q, k> > 0, dq = G k, dk = G q and
    dw = G <q, k>; with <q, k> < 0 every gradient is zero; scaling w scales dq and dk."""
    ib = _ibw()
    q = np.array([[[1.0, 2.0, -0.5, 0.25]]])
    kv = np.array([[0.5, 1.0, 1.0, -2.0]])  # <q, k> = 0.5 + 2 - 0.5 - 0.5 = 1.5
    seq, pos = np.zeros(1, np.int32), np.zeros(1, np.int64)
    idx, G = np.zeros((1, 1), np.int32), np.array([[3.0]])
    dq, dw, dk = ib.index_bwd_f64(q, np.ones((1, 1)), kv, seq, pos, 1, 1, idx, G)
    assert np.array_equal(dq[0, 0], 3.0 * kv[0]) and np.array_equal(dk[0], 3.0 * q[0, 0]) and dw[0, 0] == 4.5
    dq2, dw2, dk2 = ib.index_bwd_f64(q, np.full((1, 1), 0.25), kv, seq, pos, 1, 1, idx, G)
    assert np.array_equal(dq2, 0.25 * dq) and np.array_equal(dk2, 0.25 * dk) and dw2[0, 0] == dw[0, 0]
    dq3, dw3, dk3 = ib.index_bwd_f64(-q, np.ones((1, 1)), kv, seq, pos, 1, 1, idx, G)
    assert not dq3.any() and not dw3.any() and not dk3.any()


def test_index_bwd_rows_accumulate(gen):
    """Rows selecting the same key: its gradient is the sum of each row's alone."""
    ib = _ibw()
    rng = np.random.default_rng(43)
    T, h, d, N = 4, 8, 64, 20
    qv = rng.standard_normal((T, h, d))
    kv = rng.standard_normal((N, d))
    w = rng.uniform(0.1, 1.0, (T, h))
    seq, pos = np.zeros(T, np.int32), np.full(T, N - 1, np.int64)
    idx = np.tile(np.array([[3, 7, 11]], np.int32), (T, 1))
    G = rng.standard_normal((T, 3))
    _, _, dk = ib.index_bwd_f64(qv, w, kv, seq, pos, N, 1, idx, G)
    want = sum(ib.index_bwd_f64(qv[t:t + 1], w[t:t + 1], kv, seq[:1], pos[:1], N, 1, idx[:1], G[t:t + 1])[2]
               for t in range(T))
    assert np.allclose(dk, want, rtol=1e-13, atol=1e-13)
    assert not dk[[0, 1, 2, 4, 19]].any()

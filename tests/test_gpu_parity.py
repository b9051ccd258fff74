"""GPU parity: every libcsa call (through its C ABI) against the fp64 oracle.

Bars: index scores and top-k indices bit-exact; attention outputs and lse
within 2e-3 relative RMS and 1e-2 max-abs; compressed entries within one
FP8 quantum / one bf16 ulp of the oracle (both round the same fp32/fp64
value, so only values within rounding of a boundary may differ).
"""
import math
import sys

import numpy as np
import pytest

from gen import configs

pytestmark = pytest.mark.gpu

REL_RMS = 2e-3
MAX_ABS = 1e-2


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_long_compress_amd as csa

    return csa


@pytest.fixture(scope="module")
def dev(lib):
    from gen import device

    return device


def rel_rms(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_attn_close(out, lse, ref_out, ref_lse, what):
    out = np.asarray(out, np.float64)
    r = rel_rms(out, ref_out)
    ma = float(np.max(np.abs(out - ref_out)))
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    rl = rel_rms(np.asarray(lse)[fin], ref_lse[fin]) if fin.any() else 0.0
    ml = float(np.max(np.abs(np.asarray(lse)[fin] - ref_lse[fin]))) if fin.any() else 0.0
    print(f"{what}: out rel-rms {r:.2e} max-abs {ma:.2e}; lse rel-rms {rl:.2e} max-abs {ml:.2e}", flush=True)
    assert r <= REL_RMS and ma <= MAX_ABS, f"{what}: out rel-rms {r:.3e} max-abs {ma:.3e}"
    assert rl <= REL_RMS and ml <= MAX_ABS, f"{what}: lse rel-rms {rl:.3e} max-abs {ml:.3e}"


def compare_entries(orc, got, ref, what):
    """got/ref: (nope u8, rope u16, scale f32) for the same entries."""
    gn, gr, gs = got
    rn, rr, rs = ref
    # scale: both sides round the fp64 amax/448 to fp32 once; only a last-bit difference of libm's
    # exp / cos inside the merge or RoPE can move it, by at most one fp32 ulp
    ulp = np.spacing(np.abs(rs).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(gs.astype(np.float64) - rs) <= ulp), f"{what}: scale beyond one fp32 ulp"
    tab = orc.e4m3_table()
    gv = tab[gn] * gs[:, None].astype(np.float64)
    rv = tab[rn] * rs[:, None].astype(np.float64)
    diff_codes = gn != rn
    frac = diff_codes.mean()
    # a differing code may move at most one FP8 step
    q = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rv) / rs[:, None], 2.0 ** -6))) - 3) * rs[:, None]
    assert np.all(np.abs(gv - rv) <= 1.01 * q + 1e-30), f"{what}: nope value moved more than one FP8 step"
    # both sides round the same fp64 value; only libm last-bit differences may flip a code
    assert frac <= 1e-5, f"{what}: {frac:.2e} of FP8 codes differ"
    g = orc.bf16_array_to_f64(gr)
    r = orc.bf16_array_to_f64(rr)
    assert np.all(np.abs(g - r) <= np.abs(r) * 2.0 ** -7 + 1e-30), f"{what}: rope beyond one bf16 ulp"
    assert (gr != rr).mean() <= 1e-4, f"{what}: {(gr != rr).mean():.2e} of bf16 values differ"
    print(f"{what}: {frac:.2e} FP8 codes differ, {(gr != rr).mean():.2e} bf16 differ", flush=True)


# ---------------------------------------------------------------------------
# csa_compress
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,m,tok0,n_tok,cap", [
    (128, 4, 0, 2048, 512),
    (512, 4, 1024, 4096, 4096),
    (512, 128, 0, 8192, 64),
    (512, 1, 130944, 256, 8320),
    (128, 1, 0, 300, 300),
    (512, 4, 131072, 64, 40),    # slots wrap: entry J at J % cap
    (128, 31, 0, 310, 16),       # the longest block of the short-block kernel (31 <= 32 weights)
    (512, 33, 66, 330, 16),      # long-block kernel: a group of 32 rows, then a ragged one
    (512, 200, 0, 1000, 8),      # more logits than lanes: the second logit pass
])
def test_compress(lib, dev, gen, orc, d, m, tok0, n_tok, cap):
    import torch

    _say(f"compress d={d} m={m} tok0={tok0} n_tok={n_tok} cap={cap}")
    kv = gen.normal_bf16(201, 1, (n_tok, d))
    logits = gen.normal_f32(201, 2, (n_tok,))
    cache = lib.KvCache.empty(2, cap, d)
    lib.csa_compress(dev.bf16(kv), dev.t(logits), tok0, m, 1, cache)
    torch.cuda.synchronize()
    got = dev.host_entries(cache)
    ref = orc.compress(kv, logits, tok0, m)
    n = n_tok // m
    slots = cap + (tok0 // m + np.arange(n)) % cap  # sequence 1
    compare_entries(orc, tuple(a[slots] for a in got), ref, f"compress d={d} m={m}")
    # sequence 0 untouched
    assert not got[0][:cap].any() and not got[2][:cap].any()


@pytest.mark.parametrize("d,m,tok0,n_tok,cap", [
    (512, 4, 8, 64, 40),
    (128, 128, 0, 256, 4),      # HCA ratio
    (512, 1, 3, 17, 32),        # window ring, wrap-around
])
def test_compress_channel(lib, dev, gen, orc, d, m, tok0, n_tok, cap):
    """Per-channel compression weights against the oracle (same bar as csa_compress)."""
    import torch

    _say(f"compress_channel d={d} m={m} tok0={tok0} n_tok={n_tok} cap={cap}")
    kv = gen.normal_bf16(211, 1, (n_tok, d))
    logits = gen.normal_f32(211, 2, (n_tok, d))
    cache = lib.KvCache.empty(2, cap, d)
    lib.csa_compress_channel(dev.bf16(kv), dev.t(logits), tok0, m, 1, cache)
    torch.cuda.synchronize()
    got = dev.host_entries(cache)
    ref = orc.compress_channel(kv, logits, tok0, m)
    n = n_tok // m
    slots = cap + (tok0 // m + np.arange(n)) % cap
    compare_entries(orc, tuple(a[slots] for a in got), ref, f"compress_channel d={d} m={m}")
    assert not got[0][:cap].any() and not got[2][:cap].any()


@pytest.mark.parametrize("d_i,m,tok0,n_tok,cap", [
    (128, 4, 0, 4096, 1024),
    (64, 4, 12, 400, 200),
    (128, 1, 5, 77, 100),
    (128, 128, 0, 1024, 8),
    (64, 100, 0, 500, 8),        # more logits than lanes
])
def test_compress_index_keys(lib, dev, gen, orc, d_i, m, tok0, n_tok, cap):
    """Raw key tokens -> MXFP4 index keys: codes and scales equal the oracle's bit for bit
    (an all-zero block and a wide-magnitude block included)."""
    import torch

    _say(f"compress_index_keys d_i={d_i} m={m} tok0={tok0} n_tok={n_tok} cap={cap}")
    k = gen.normal_bf16(221, 1, (n_tok, d_i))
    k[:m] = 0  # first entry: all-zero blocks (scale byte 127)
    if n_tok >= 2 * m:
        big = np.array([orc.f64_to_bf16(v) for v in np.geomspace(1e-6, 1e6, d_i)], np.uint16)
        k[m:2 * m] = big  # second entry: saturation and underflow to zero inside a block
    logits = gen.normal_f32(221, 2, (n_tok,))
    out = lib.IndexKeys(torch.zeros(2 * cap, d_i // 2, dtype=torch.uint8, device="cuda"),
                        torch.zeros(2 * cap, d_i // 32, dtype=torch.uint8, device="cuda"), cap)
    lib.csa_compress_index_keys(dev.bf16(k), dev.t(logits), tok0, m, 1, out)
    torch.cuda.synchronize()
    data, scale = out.data.cpu().numpy(), out.scale.cpu().numpy()
    ref_d, ref_s = orc.compress_index_keys(k, logits, tok0, m)
    n = n_tok // m
    slots = cap + (tok0 // m + np.arange(n)) % cap
    assert np.array_equal(scale[slots], ref_s), "E8M0 scales differ"
    bad = data[slots] != ref_d
    assert not bad.any(), f"{bad.sum()} packed code bytes differ; first at {np.argwhere(bad)[:3].tolist()}"
    assert not data[:cap].any() and not scale[:cap].any()  # sequence 0 untouched


def test_compress_rejects_partial_block(lib, dev, gen):
    cache = lib.KvCache.empty(1, 16, 128)
    kv = gen.normal_bf16(202, 1, (6, 128))
    with pytest.raises(lib.CsaError) as e:
        lib.csa_compress(dev.bf16(kv), dev.t(gen.normal_f32(202, 2, (6,))), 0, 4, 0, cache)
    assert e.value.code == lib.CSA_EINVAL


# ---------------------------------------------------------------------------
# csa_index_scores
# ---------------------------------------------------------------------------
def _index_case(gen, seed, T, h_i, d_i, N, B, pos, seq, plant=0.0):
    kd, ks, _ = gen.mxfp4(seed, 1, B * N, d_i, plant_frac=plant)
    qd, qs, _ = gen.mxfp4(seed, 2, T * h_i, d_i)
    w = gen.pow2_weights(seed, 3, (T, h_i))
    return (qd.reshape(T, h_i, d_i // 2), qs.reshape(T, h_i, d_i // 32), w, np.asarray(seq, np.int32),
            np.asarray(pos, np.int64), kd, ks)


@pytest.mark.parametrize("T,h_i,d_i,N,B,m,n_cols,mode", [
    (4, 8, 128, 5000, 4, 4, 5000, "decode"),        # ragged key chunk
    (32, 8, 128, 16384, 32, 4, 16384, "decode"),
    (3, 4, 64, 700, 2, 4, 650, "decode"),
    (2048, 4, 64, 512, 1, 4, 512, "prefill"),       # small prefill
    (200, 8, 128, 3000, 1, 4, 3000, "prefill"),     # ragged rows and columns
    (300, 8, 64, 2000, 1, 4, 1999, "prefill"),      # d_i = 64 with 8 heads
    (150, 4, 128, 1500, 1, 4, 1500, "prefill"),     # d_i = 128 with 4 heads
    (130, 8, 128, 900, 3, 4, 900, "mixed"),          # several sequences inside one tile
    (96, 4, 128, 400, 2, 2, 400, "mixed"),
])
def test_index_scores_bit_exact(lib, dev, gen, orc, T, h_i, d_i, N, B, m, n_cols, mode):
    import torch

    _say(f"index T={T} h_i={h_i} d_i={d_i} N={N} B={B} m={m} n_cols={n_cols} {mode}")
    rng = np.random.default_rng(T + N)
    if mode == "decode":
        seq = np.arange(T) % B
        pos = rng.integers(m * N // 2, m * N + 5, size=T)
    elif mode == "prefill":
        seq = np.zeros(T, np.int64)
        pos = np.sort(rng.integers(0, m * N, size=T))
    else:
        seq = rng.integers(0, B, size=T)
        pos = rng.integers(0, m * N, size=T)
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 300 + T, T, h_i, d_i, N, B, pos, seq)
    wit = orc.index_exact_witness(qd, qs, w, seq, pos, kd, ks, N, m, n_cols)
    assert wit < 24, f"inputs break the fp32 exactness precondition ({wit:.1f} bits)"
    ref = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, n_cols).astype(np.float32)
    keys = dev.index_keys((kd, ks), N)
    got = lib.csa_index_scores(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, m, n_cols)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), f"{bad.sum()} scores differ; first at {np.argwhere(bad)[:3].tolist()}"


@pytest.mark.parametrize("G,group,h_i,d_i,N,B,m,n_cols,layout", [
    (4, 2, 8, 128, 5000, 4, 4, 5000, "mtp"),       # 4 sequences x 2 tokens at consecutive positions
    (3, 4, 8, 128, 9000, 3, 4, 8990, "mtp"),       # 4 tokens: two matrix tiles per key tile; ragged columns
    (5, 2, 4, 64, 700, 2, 4, 650, "mtp"),
    (2, 4, 4, 128, 3000, 2, 2, 3000, "mtp"),       # h_i = 4: four rows in one tile
    (6, 2, 8, 128, 4000, 3, 4, 4000, "mixed"),     # rows of a group on different sequences
    (3, 4, 8, 64, 2500, 4, 4, 2500, "mixed"),
])
def test_index_scores_grouped_bit_exact(lib, dev, gen, orc, G, group, h_i, d_i, N, B, m, n_cols, layout):
    """Multi-token decode: rows in groups of one sequence stream its keys once;
    the scores equal the oracle's and the plain kernel's bit for bit, also when
    a group's rows belong to different sequences."""
    import torch

    T = G * group
    _say(f"grouped index G={G} group={group} h_i={h_i} d_i={d_i} N={N} n_cols={n_cols} {layout}")
    rng = np.random.default_rng(T + N + group)
    if layout == "mtp":
        seq = np.repeat(np.arange(G) % B, group)
        p0 = rng.integers(m * N // 2, m * N - group, size=G)
        p0[0] = m * 37 - 1 - group // 2  # a group whose rows straddle a block boundary
        pos = (p0[:, None] + np.arange(group)[None, :]).reshape(-1)
    else:
        seq = rng.integers(0, B, size=T)
        pos = rng.integers(0, m * N, size=T)
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 500 + T, T, h_i, d_i, N, B, pos, seq)
    wit = orc.index_exact_witness(qd, qs, w, seq, pos, kd, ks, N, m, n_cols)
    assert wit < 24, f"inputs break the fp32 exactness precondition ({wit:.1f} bits)"
    ref = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, n_cols).astype(np.float32)
    keys = dev.index_keys((kd, ks), N)
    args = (dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, m, n_cols)
    got = lib.csa_index_scores_grouped(*args, group)
    plain = lib.csa_index_scores(*args)
    torch.cuda.synchronize()
    got, plain = got.cpu().numpy(), plain.cpu().numpy()
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), f"{bad.sum()} scores differ; first at {np.argwhere(bad)[:3].tolist()}"
    assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))


def test_index_scores_grouped_summary_topk(lib, dev, gen, orc):
    """Grouped indexer writing the row summary of long rows + csa_topk(prepared)
    equals the oracle's selection."""
    import torch

    for (G, group, N, k, plant) in [(2, 2, 70000, 1024, 0.05), (2, 4, 100000, 2048, 0.02)]:
        T = G * group
        _say(f"grouped index + summary top-k G={G} group={group} N={N} k={k}")
        seq = np.repeat(np.arange(G), group)
        pos = np.repeat(np.full(G, 4 * N - group), group) + np.tile(np.arange(group), G)
        pos = np.minimum(pos, 4 * N - 1)
        qd, qs, w, seq, pos, kd, ks = _index_case(gen, 900 + T + N, T, 8, 128, N, G, pos, seq, plant=plant)
        ref = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, 4, N).astype(np.float32)
        ref_i = orc.topk(ref, pos, 4, k)
        keys = dev.index_keys((kd, ks), N)
        ws = torch.full((lib.csa_topk_workspace(T, N, k) + 256,), 0x5A, dtype=torch.uint8, device="cuda")
        ws = ws[: lib.csa_topk_workspace(T, N, k)]
        sc = lib.csa_index_scores_grouped(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, 4, N, group,
                                          topk_ws=ws)
        idx = lib.csa_topk(sc, dev.t(pos), 4, k, ws=ws, prepared=True)
        torch.cuda.synchronize()
        got = sc.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        assert np.array_equal(idx.cpu().numpy(), ref_i)


# ---------------------------------------------------------------------------
# csa_topk
# ---------------------------------------------------------------------------
def _cluster_scores(rng, T, n, k):
    """Rows whose k-th largest score lies in a dense cluster: a set of equal scores (X = 10.0,
    often more of them than a histogram descent stops at or ranks directly) and distinct
    scores 8 .. 3005 ulps above X, over a background below 7; some rows also hold a few
    scores in [20, 40), which widen the key span so the descent takes several levels.  Odd
    rows put the k-th largest among the equal scores, even rows among the distinct ones."""
    s = np.abs(rng.standard_normal((T, n))).astype(np.float32)
    x = np.float32(10.0).view(np.uint32)
    for t in range(T):
        n_hi = 0 if t % 3 == 0 else int(rng.integers(1, k // 4 + 1))
        c1 = int(rng.integers(65, 600))
        if t % 2:
            c2 = int(rng.integers(max(1, k - n_hi - c1), k - n_hi))
        else:
            c2 = int(rng.integers(k - n_hi, k - n_hi + min(2000, n // 4)))
        cols = rng.choice(n, size=min(n, n_hi + c1 + c2), replace=False)
        a, b = n_hi, n_hi + c1
        s[t, cols[:a]] = rng.uniform(20, 40, a).astype(np.float32)
        s[t, cols[a:b]] = x.view(np.float32)
        s[t, cols[b:]] = (x + rng.integers(8, 3006, len(cols) - b).astype(np.uint32)).view(np.float32)
    return s


@pytest.mark.parametrize("T,n_cols,k,m,kind", [
    (64, 512, 64, 4, "normal"),
    (16, 40000, 1024, 4, "normal"),     # longer than the LDS cache
    (32, 16384, 1024, 4, "ties"),
    (8, 3000, 1024, 4, "short"),        # some rows see fewer than k columns
    (5, 2048, 2048, 1, "normal"),
    (4, 70000, 1024, 4, "allequal"),
    # many rows of up to 36,864 columns (one workgroup per row, the row held in registers)
    (160, 16384, 512, 4, "ties"),       # equal keys beyond the direct-ranking limit
    (128, 8192, 1024, 4, "allequal"),   # one key value: the lowest columns by column passes
    (200, 20000, 1024, 4, "short"),
    (144, 36864, 2048, 4, "normal"),    # widest rows of this path; 4th largest key per thread
    (130, 36863, 1500, 4, "signed"),    # odd length: unaligned rows load by element; 3rd largest
    (129, 4097, 1024, 4, "ties"),
    (150, 18433, 513, 4, "short"),
    (140, 3000, 1, 1, "normal"),
    # many rows, longer (one workgroup per row, row streamed from global memory)
    (136, 65536, 2048, 4, "normal"),    # longest rows of this path
    (128, 40000, 1024, 4, "ties"),
    # few long rows (selection from the row summary)
    (4, 262144, 1024, 4, "normal"),
    (8, 100000, 2048, 4, "ties"),       # candidates overflow LDS: whole-row selection
    (6, 300000, 1024, 4, "short"),
    (3, 70000, 1, 4, "normal"),
    (2, 1048576, 2048, 4, "normal"),    # summary longer than one pass of registers
    # many rows longer than 65,536 columns (one workgroup per row, radix select; rows of at most
    # 36,608 visible columns are cached in LDS)
    (160, 70000, 1024, 4, "normal"),
    (160, 70000, 1024, 4, "ties"),
    (160, 70000, 1024, 4, "short"),
    (128, 70001, 2048, 4, "signed"),
    # dense clusters of near-equal keys (a tie cluster larger than the descents' stop counts, and
    # distinct keys a few thousand order-key units above it) on every selection path
    (130, 20000, 1050, 4, "cluster"),   # registers
    (130, 36864, 2048, 4, "cluster"),
    (130, 3000, 700, 4, "cluster"),
    (130, 50000, 1050, 4, "cluster"),   # streamed
    (160, 70000, 1050, 4, "cluster"),   # radix select
    (4, 200000, 1050, 4, "cluster"),    # row summary
    (8, 100000, 1024, 4, "cluster"),
    (3, 70000, 2048, 4, "cluster"),
    (64, 262144, 1024, 4, "cluster"),
])
def test_topk_bit_exact(lib, dev, orc, T, n_cols, k, m, kind):
    import torch

    _say(f"topk T={T} n_cols={n_cols} k={k} m={m} {kind}")
    rng = np.random.default_rng(n_cols + k)
    if kind == "cluster":
        scores = _cluster_scores(rng, T, n_cols, k)
    elif kind == "ties":
        scores = rng.integers(0, 50, size=(T, n_cols)).astype(np.float32)
    elif kind == "allequal":
        scores = np.zeros((T, n_cols), np.float32)
        scores[:, ::7] = -0.0
    elif kind == "signed":
        scores = rng.standard_normal((T, n_cols)).astype(np.float32) * 10
    else:
        scores = np.abs(rng.standard_normal((T, n_cols))).astype(np.float32) * 10
    if kind == "short":
        pos = rng.integers(0, m * n_cols, size=T).astype(np.int64)
        pos[0] = 5
    else:
        pos = np.full(T, m * n_cols - 1, np.int64)
    ref = orc.topk(scores, pos, m, k)
    got = lib.csa_topk(dev.t(scores), dev.t(pos), m, k)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.array_equal(got, ref), f"rows differ: {np.where((got != ref).any(axis=1))[0][:5].tolist()}"


def test_indexer_summary_and_workspace_reuse(lib, dev, gen, orc):
    """Indexer-written row summary + csa_topk(prepared) equals the oracle, and so
    does the plain path; one workspace serves calls of different shapes.  Few
    rows longer than 65,536 columns select from the summary (the largest
    order-preserving key of every 32-column group); other shapes ignore it."""
    import torch

    _say("indexer row summary, workspace reuse")
    ws = torch.full((64 << 20,), 0x5A, dtype=torch.uint8, device="cuda")  # contents need no initialisation
    for (T, N, k, plant) in [(4, 70000, 1024, 0.05), (3, 9000, 512, 0.0), (8, 100000, 2048, 0.02),
                             (4, 70000, 1024, 0.0), (2, 262144, 1024, 0.05)]:
        qd, qs, w, seq, pos, kd, ks = _index_case(gen, 700 + T + N, T, 8, 128, N, T, np.full(T, 4 * N - 1),
                                                  np.arange(T), plant=plant)
        ref = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, 4, N).astype(np.float32)
        ref_i = orc.topk(ref, pos, 4, k)
        keys = dev.index_keys((kd, ks), N)
        summary = N > 65536
        ng = -(-N // 32)
        b = ref.view(np.uint32).astype(np.uint64)
        b[b == 0x80000000] = 0
        okey = np.where(b & 0x80000000, b ^ 0xFFFFFFFF, b | 0x80000000).astype(np.uint64)
        pad = np.zeros((T, ng * 32), np.uint64)
        pad[:, :N] = okey
        want_g = pad.reshape(T, ng, 32).max(axis=2).astype(np.uint32)
        gsum = lambda: ws[: T * ng * 4].view(torch.int32).cpu().numpy().view(np.uint32).reshape(T, ng)  # noqa: E731

        sc = lib.csa_index_scores(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, 4, N, topk_ws=ws)
        torch.cuda.synchronize()
        if summary:
            assert np.array_equal(gsum(), want_g), "row summary written by the indexer"
            ws[: T * ng * 4].fill_(0xA5)
        ix2 = lib.csa_topk(sc, dev.t(pos), 4, k, ws=ws)
        torch.cuda.synchronize()
        if summary:
            assert np.array_equal(gsum(), want_g), "row summary written by the selection"
        sc2 = lib.csa_index_scores(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, 4, N, topk_ws=ws)
        ix = lib.csa_topk(sc2, dev.t(pos), 4, k, ws=ws, prepared=True)
        torch.cuda.synchronize()
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        assert np.array_equal(ix.cpu().numpy(), ref_i)
        assert np.array_equal(ix2.cpu().numpy(), ref_i)


# ---------------------------------------------------------------------------
# csa_sparse_mqa / hca_dense_mqa
# ---------------------------------------------------------------------------
def _attn_inputs(gen, seed, B, N, W, H, d, T, L, win_cap):
    comp = gen.entries(seed, 20, B * N, d - 64)
    win = gen.entries(seed, 21, B * win_cap, d - 64)
    q = gen.normal_bf16(seed, 23, (T, H, d))
    return comp, win, q


@pytest.mark.parametrize("T,B,L,H,d,k,W,m,win_cap", [
    (4, 4, 8192, 64, 512, 1024, 128, 4, 128),      # decode, split-KV
    (32, 32, 4096, 64, 512, 1024, 128, 4, 128),
    (3, 2, 600, 32, 512, 256, 128, 4, 128),        # fewer visible than k (-1 padding)
    (6, 3, 2048, 16, 128, 64, 128, 4, 200),
    (2, 2, 64, 64, 512, 64, 0, 4, 1),              # no window branch
    (64, 4, 8192, 64, 512, 1024, 128, 4, 128),     # 4 splits of 288 keys
    (128, 4, 8192, 64, 512, 1024, 128, 4, 128),    # 2 splits of 576 keys: the two-role 64-head kernel
    (4, 4, 8192, 64, 128, 1024, 128, 4, 128),      # 64 heads with d = 128, split-KV
    (40, 2, 4096, 64, 128, 512, 128, 4, 130),      # 64 heads with d = 128, longer splits
    (2, 2, 4096, 32, 128, 2048, 64, 4, 64),        # k = 2048, 32 heads
])
def test_sparse_mqa_decode(lib, dev, gen, orc, T, B, L, H, d, k, W, m, win_cap):
    import torch

    _say(f"sparse_mqa T={T} B={B} L={L} H={H} d={d} k={k} W={W} m={m}")
    N = L // m
    comp, win, q = _attn_inputs(gen, 400 + T, B, N, W, H, d, T, L, win_cap)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.full(T, L - 1, np.int64)
    pos[-1] = L - 3  # a row whose last block is incomplete
    nv = (pos + 1) // m
    idx = gen.random_idx(401 + T, 1, nv, k)
    sm = 1.0 / math.sqrt(d)
    ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, win_cap, W, m, sm, idx=idx)
    out, lse = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(idx), m, dev.kv_cache(comp, N),
                                  dev.kv_cache(win, win_cap) if W > 0 else None, W, sm)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "sparse_mqa")


@pytest.mark.parametrize("path", ["sparse", "dense"])
@pytest.mark.parametrize("T", [4, 8, 16])
def test_attention_short_rows_in_a_split_batch(lib, dev, gen, orc, path, T):
    """Rows whose key lists are far shorter than the split partition (set by T and the key
    bound) next to full rows.  T=4: 18 splits, two workgroups of 32 heads per split; T=8: 9
    splits, shared the same way; T=16: 16 splits of one workgroup.  Sparse: a row at
    position 5 has 1 valid selected entry and 1,023 masked ones, so whole splits see no
    visible key.  Dense: its key list is 6 window tokens, so most splits are empty.  Every
    row against the oracle."""
    import torch

    _say(f"short rows in a split batch path={path} T={T}")
    H, d, W = 64, 512, 128
    if path == "sparse":
        m, B, L, k = 4, 4, 8192, 1024
    else:
        m, B, L, k = 128, 4, 131072, 0
    N = L // m
    comp, win, q = _attn_inputs(gen, 480 + T, B, N, W, H, d, T, L, W)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.array([L - 1, 5, 300, 2000, L - 1, 130, 7, 4000] * 2, np.int64)[:T]
    sm = 1.0 / math.sqrt(d)
    kvc, kvw = dev.kv_cache(comp, N), dev.kv_cache(win, W)
    if path == "sparse":
        idx = gen.random_idx(481 + T, 1, (pos + 1) // m, k)
        out, lse = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(idx), m, kvc, kvw, W, sm)
    else:
        idx = None
        out, lse = lib.hca_dense_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), m, N, kvc, kvw, W, sm)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, W, W, m, sm, idx=idx)
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"short rows {path} T={T}")


def test_sparse_mqa_ignores_invalid_idx(lib, dev, gen, orc):
    import torch

    _say("sparse_mqa invalid idx entries")
    B, N, H, d, k, W, m = 2, 256, 64, 512, 128, 128, 4
    comp, win, q = _attn_inputs(gen, 450, B, N, W, H, d, 2, 1024, 128)
    seq = np.array([0, 1], np.int32)
    pos = np.array([1023, 500], np.int64)
    idx = gen.random_idx(451, 1, np.array([256, 125]), k)
    idx[1, 5] = 200  # not yet visible at t=500 (visible: j < 125)
    idx[0, 7] = -1
    sm = 1.0 / math.sqrt(d)
    ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, 128, W, m, sm, idx=idx)
    out, lse = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(idx), m, dev.kv_cache(comp, N),
                                  dev.kv_cache(win, 128), W, sm)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "sparse_mqa invalid idx")


@pytest.mark.parametrize("T,B,L,H,d,W,m", [
    (8, 8, 131072, 64, 512, 128, 128),   # decode, 1024 entries
    (3, 3, 20000, 32, 512, 128, 128),
    (5, 1, 640, 16, 128, 64, 128),
    (128, 8, 131072, 64, 512, 128, 128),  # 4 splits of 288 keys: the two-role 64-head kernel
])
def test_dense_mqa_decode(lib, dev, gen, orc, T, B, L, H, d, W, m):
    import torch

    _say(f"dense_mqa T={T} B={B} L={L} H={H} d={d} W={W} m={m}")
    N = L // m
    comp, win, q = _attn_inputs(gen, 500 + T, B, N, W, H, d, T, L, W)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.full(T, L - 1, np.int64)
    pos[0] = L - 200
    sm = 1.0 / math.sqrt(d)
    ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, W, W, m, sm)
    out, lse = lib.hca_dense_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), m, N, dev.kv_cache(comp, N),
                                 dev.kv_cache(win, W), W, sm)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "dense_mqa")


def _f64_to_bf16_bits(x):
    """Round-to-nearest-even fp64 -> fp32 -> bf16 bits (test-side input shaping only)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _plant(orc, q, comp, cap, seq, rows, key_of_row, d, boost):
    """Add to every head of each row's query a multiple of one entry's FP8 part,
    so that entry's score rises by about ``boost`` (its value vector is unchanged)."""
    dn = d - 64
    tab = orc.e4m3_table()
    qf = orc.bf16_array_to_f64(q).reshape(q.shape)
    sm = 1.0 / math.sqrt(d)
    for t in rows:
        e = int(seq[t]) * cap + int(key_of_row[t])
        kv = tab[comp[0][e]] * float(comp[2][e])
        alpha = boost / (sm * float(kv @ kv))
        qf[t, :, :dn] += alpha * kv[None, :]
    return _f64_to_bf16_bits(qf)


@pytest.mark.parametrize("kind,path,T", [
    ("jump", "sparse", 512), ("jump", "sparse", 4), ("jump", "dense", 4),
    ("scale", "sparse", 512), ("scale", "sparse", 4), ("scale", "dense", 4),
])
def test_attention_reference_restarts(lib, dev, gen, orc, kind, path, T):
    """Inputs that break the per-split softmax references after the first tile:
    'jump' plants, in a later tile of every row's key list, an entry whose score
    is ~40 above the rest (reference max + 8 exceeded); 'scale' gives 1% of the
    entries a 32x larger FP8 scale with tiny codes (scale reference x16
    exceeded) while their values stay small.  T=512 runs one split per row
    (many tiles), T=4 the split-KV path; rows are compared with the oracle."""
    import torch

    _say(f"attention restarts kind={kind} path={path} T={T}")
    H, d, W = 64, 512, 128
    dn = d - 64
    if path == "sparse":
        m, B, L, k = 4, 2, 16384, 1024
    else:
        m, B, L, k = 128, 2, 131072, 0
    N = L // m
    comp, win, q = _attn_inputs(gen, 700 + T, B, N, W, H, d, T, L, W)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.full(T, L - 1, np.int64)
    if path == "sparse":
        idx = gen.random_idx(701 + T, 1, (pos + 1) // m, k)
    else:
        idx = None
    if kind == "scale":
        sel = np.random.default_rng(702).random(B * N) < 0.01
        nope, rope, scale = comp
        nope, scale = nope.copy(), scale.copy()
        nope[sel] = 1  # smallest FP8 subnormal
        scale[sel] *= 32.0
        comp = (nope, rope, scale)
    else:
        # key-list position 64 * (2 + t % 9) + 37: a later tile of the row, and the
        # second tile of its split when the key list is cut into splits of 64
        u_star = 64 * (2 + np.arange(T) % 9) + 37
        j_star = idx[np.arange(T), u_star] if idx is not None else u_star
        q = _plant(orc, q, comp, N, seq, range(T), j_star, d, 40.0)
    sm = 1.0 / math.sqrt(d)
    qd = dev.bf16(q)
    if path == "sparse":
        out, lse = lib.csa_sparse_mqa(qd, dev.t(seq), dev.t(pos), dev.t(idx), m, dev.kv_cache(comp, N),
                                      dev.kv_cache(win, W), W, sm)
    else:
        out, lse = lib.hca_dense_mqa(qd, dev.t(seq), dev.t(pos), m, N, dev.kv_cache(comp, N), dev.kv_cache(win, W),
                                     W, sm)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 8 else np.array([0, 1, 2, 77, 200, 301, 444, T - 1])
    sub = lambda a: np.ascontiguousarray(a[rows])  # noqa: E731
    ref_o, ref_l = orc.attend(sub(q), sub(seq), sub(pos), comp, N, win, W, W, m, sm,
                              idx=sub(idx) if idx is not None else None)
    if kind == "jump":
        # the planted entry carries almost all the weight: the output is close to its value vector
        assert np.all(ref_l[:, 0] > 20.0)
    assert_attn_close(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ref_o, ref_l, f"restarts {kind} {path}")


def test_sparse_all_selected_equals_dense(lib, dev, gen):
    """k >= visible entries: CSA equals HCA at the same m (GPU against GPU, both checked against the oracle above)."""
    import torch

    _say("sparse(all) == dense")
    B, N, H, d, W, m = 2, 300, 64, 512, 128, 4
    comp, win, q = _attn_inputs(gen, 600, B, N, W, H, d, 2, 1200, 128)
    seq = np.array([0, 1], np.int32)
    pos = np.array([1199, 777], np.int64)
    idx = np.full((2, 512), -1, np.int32)
    for i in range(2):
        nv = (pos[i] + 1) // m
        idx[i, :nv] = np.arange(nv)
    sm = 1.0 / math.sqrt(d)
    a = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(idx), m, dev.kv_cache(comp, N),
                           dev.kv_cache(win, 128), W, sm)
    b = lib.hca_dense_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), m, N, dev.kv_cache(comp, N), dev.kv_cache(win, 128), W,
                          sm)
    torch.cuda.synchronize()
    # same key set, different split-KV partitioning: equal within the attention bar
    assert rel_rms(a[0].cpu().numpy(), b[0].cpu().numpy()) < REL_RMS


# ---------------------------------------------------------------------------
# end to end: the small prefill workload through every call
# ---------------------------------------------------------------------------
def test_end_to_end_prefill_small(lib, dev, gen, orc):
    import torch

    _say("end-to-end prefill_small")
    wl = configs.named("prefill_small")
    T, d, m, k, W, H = wl["T"], wl["d"], wl["m"], wl["k"], wl["W"], wl["H"]
    # GPU
    comp = lib.KvCache.empty(1, wl["comp_cap"], d)
    win = lib.KvCache.empty(1, wl["win_cap"], d)
    hca = lib.KvCache.empty(1, wl["hca_cap"], d)
    kv = dev.bf16(wl["kv"])
    lg = dev.t(wl["logits"])
    lib.csa_compress(kv, lg, 0, m, 0, comp)
    lib.csa_compress(kv, lg, 0, 1, 0, win)
    lib.csa_compress(kv, lg, 0, wl["m_hca"], 0, hca)
    seq, pos = dev.t(wl["seq"]), dev.t(wl["pos"])
    scores = lib.csa_index_scores(dev.t(wl["iq"][0]), dev.t(wl["iq"][1]), dev.t(wl["w"]), seq, pos,
                                  dev.index_keys(wl["keys"], wl["N"]), m, wl["n_cols"])
    idx = lib.csa_topk(scores, pos, m, k)
    out, lse = lib.csa_sparse_mqa(dev.bf16(wl["q"]), seq, pos, idx, m, comp, win, W, wl["sm_scale"])
    hout, hlse = lib.hca_dense_mqa(dev.bf16(wl["q"]), seq, pos, wl["m_hca"], wl["hca_cap"], hca, win, W,
                                   wl["sm_scale"])
    torch.cuda.synchronize()
    # oracle, step by step from the same raw inputs
    o_comp = orc.compress(wl["kv"], wl["logits"], 0, m)
    o_win = orc.compress(wl["kv"], wl["logits"], 0, 1)
    o_hca = orc.compress(wl["kv"], wl["logits"], 0, wl["m_hca"])
    compare_entries(orc, dev.host_entries(comp), o_comp, "e2e compress m=4")
    o_scores = orc.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0],
                                wl["keys"][1], wl["N"], m, wl["n_cols"]).astype(np.float32)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), o_scores.view(np.uint32))
    o_idx = orc.topk(o_scores, wl["pos"], m, k)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    # attention from the oracle's own caches (entries may differ in rare FP8 roundings)
    ref_o, ref_l = orc.attend(wl["q"], wl["seq"], wl["pos"], o_comp, wl["comp_cap"], o_win, wl["T"], W, m,
                              wl["sm_scale"], idx=o_idx)
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "e2e sparse")
    ref_o, ref_l = orc.attend(wl["q"], wl["seq"], wl["pos"], o_hca, wl["hca_cap"], o_win, wl["T"], W, wl["m_hca"],
                              wl["sm_scale"])
    assert_attn_close(hout.cpu().numpy(), hlse.cpu().numpy(), ref_o, ref_l, "e2e dense")


# ---------------------------------------------------------------------------
# paged compressed cache (and window ring): same results as the contiguous layout
# ---------------------------------------------------------------------------
def _paged_like(lib, torch, n_seq, cap, d, page, perm, extra):
    """An empty paged cache: n_seq sequences of cap slots, physical pages perm[s * npp + i] (+ extra spare pages)."""
    npp = cap // page
    rows = (n_seq * npp + extra) * page
    pages = torch.tensor(np.asarray(perm, np.int32).reshape(n_seq, npp), device="cuda")
    return lib.KvCache(torch.zeros(rows, d - 64, dtype=torch.uint8, device="cuda"),
                       torch.zeros(rows, 64, dtype=torch.bfloat16, device="cuda"),
                       torch.zeros(rows, dtype=torch.float32, device="cuda"), cap, pages=pages, page=page)


def _slot_rows(cache, s, cap):
    if cache.pages is None:
        return s * cap + np.arange(cap)
    pg = cache.pages.cpu().numpy()[s]
    i = np.arange(cap)
    return pg[i // cache.page] * cache.page + i % cache.page


@pytest.mark.parametrize("share,page,wpage", [(False, 16, 32), (True, 16, 32), (False, 128, 128), (True, 1, 1)])
def test_paged_cache_matches_contiguous(lib, dev, gen, share, page, wpage):
    """Compression into a paged cache (pages in a shuffled order, a spare page unused), then
    CSA and HCA attention with paged entries and a paged window ring, equal the contiguous
    layout bit for bit.  share: sequence 1 reuses sequence 0's first four physical pages (a
    common prefix compressed once), against a contiguous cache holding copies."""
    import torch

    _say(f"paged cache, shared prefix {share}, page {page}, window page {wpage}")
    B, m, d, cap, W = 3, 4, 512, 128, 128
    L = m * cap
    npp = cap // page
    kv = [gen.normal_bf16(700 + b, 1, (L, d)) for b in range(B)]
    lg = [gen.normal_f32(700 + b, 2, (L,)) for b in range(B)]
    P = max(1, 64 // page) if page < cap else 0  # shared pages (P * page entries = P * page * m tokens)
    if share:
        kv[1][: P * page * m] = kv[0][: P * page * m]
        lg[1][: P * page * m] = lg[0][: P * page * m]
    rng = np.random.default_rng(11)
    perm = rng.permutation(B * npp + 1)[: B * npp]
    if share:
        perm = perm.reshape(B, npp)
        perm[1, :P] = perm[0, :P]
        perm = perm.reshape(-1)
    contig = lib.KvCache.empty(B, cap, d)
    paged = _paged_like(lib, torch, B, cap, d, page, perm, 1)
    wperm = rng.permutation(B * (W // wpage))
    wc = lib.KvCache.empty(B, W, d)
    wp = _paged_like(lib, torch, B, W, d, wpage, wperm, 0)
    for b in range(B):
        for cache in (contig, paged):
            if share and b == 1 and cache is paged:
                # the shared prefix is already in place: compress only this sequence's own blocks
                lib.csa_compress(dev.bf16(kv[b][P * page * m:]), dev.t(lg[b][P * page * m:]), P * page * m, m, b, cache)
            else:
                lib.csa_compress(dev.bf16(kv[b]), dev.t(lg[b]), 0, m, b, cache)
        for cache in (wc, wp):
            lib.csa_compress(dev.bf16(kv[b][L - W:]), dev.t(lg[b][L - W:]), L - W, 1, b, cache)
    torch.cuda.synchronize()
    for b in range(B):
        for (a, c) in ((contig, paged), (wc, wp)):
            ra, rc = _slot_rows(a, b, a.cap), _slot_rows(c, b, c.cap)
            for x, y in ((a.nope, c.nope), (a.rope, c.rope), (a.scale, c.scale)):
                assert torch.equal(x[torch.tensor(ra, device="cuda")], y[torch.tensor(rc, device="cuda")])
    # attention over both layouts
    T, H, k = 2 * B, 64, 96
    seq = np.repeat(np.arange(B), 2).astype(np.int32)
    pos = np.tile(np.array([L - 1, L - 37]), B).astype(np.int64)
    q = gen.normal_bf16(799, 3, (T, H, d))
    idx = np.stack([np.sort(rng.choice((int(p) + 1) // m, size=k, replace=False)) for p in pos]).astype(np.int32)
    args = dict(seq=dev.t(seq), pos=dev.t(pos), m=m, window=W, sm_scale=1.0 / np.sqrt(d))
    o1, l1 = lib.csa_sparse_mqa(dev.bf16(q), idx=dev.t(idx), comp=contig, win=wc, **args)
    o2, l2 = lib.csa_sparse_mqa(dev.bf16(q), idx=dev.t(idx), comp=paged, win=wp, **args)
    h1, hl1 = lib.hca_dense_mqa(dev.bf16(q), max_vis=cap, comp=contig, win=wc, **args)
    h2, hl2 = lib.hca_dense_mqa(dev.bf16(q), max_vis=cap, comp=paged, win=wp, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(h1, h2) and torch.equal(hl1, hl2)
    # the gradient through both layouts: dq identical; entry gradients land in the physical rows
    # (a shared page sums its sequences' gradients in one fixed-point sum, the contiguous layout
    # keeps them apart and they are added here in fp32)
    dout = dev.t(gen.normal_f32(798, 4, (T, H, d), sigma=0.01))
    for sel in (True, False):
        if sel:
            fa = (o1, l1, contig, wc, dev.t(idx))
            fb = (o2, l2, paged, wp, dev.t(idx))
        else:
            fa = (h1, hl1, contig, wc, None)
            fb = (h2, hl2, paged, wp, None)
        g1 = lib.csa_mqa_bwd(dev.bf16(q), args["seq"], args["pos"], fa[4], m, fa[2], fa[3], W, args["sm_scale"],
                             fa[0], fa[1], dout)
        g2 = lib.csa_mqa_bwd(dev.bf16(q), args["seq"], args["pos"], fb[4], m, fb[2], fb[3], W, args["sm_scale"],
                             fb[0], fb[1], dout)
        torch.cuda.synchronize()
        assert torch.equal(g1[0], g2[0]), "dq differs between layouts"
        for got, ref, ca, cb in ((g2[1], g1[1], contig, paged), (g2[2], g1[2], wc, wp)):
            want = torch.zeros_like(got)
            for b in range(B):
                want.index_add_(0, torch.tensor(_slot_rows(cb, b, cb.cap), device="cuda", dtype=torch.int64),
                                ref[torch.tensor(_slot_rows(ca, b, ca.cap), device="cuda")])
            r = rel_rms(got.cpu().numpy(), want.cpu().numpy())
            assert r <= 1e-5, f"paged entry gradients differ (rel-rms {r:.2e}, selection {sel})"


def _paged_from_host(lib, torch, dev, ent, n_seq, cap, page, rng, extra=1):
    """Host entries indexed seq*cap + slot, placed on the device in pages of `page` slots at
    seeded shuffled physical pages (plus `extra` unused pages)."""
    npp = cap // page
    perm = rng.permutation(n_seq * npp + extra)[: n_seq * npp].astype(np.int32)
    rows = (perm.reshape(n_seq, npp)[:, :, None] * page + np.arange(page)[None, None, :]).reshape(-1)
    n_rows = (n_seq * npp + extra) * page
    arrs = []
    for a in ent:
        b = np.zeros((n_rows,) + a.shape[1:], a.dtype)
        b[rows] = a
        arrs.append(b)
    return lib.KvCache(dev.t(arrs[0]), dev.bf16(arrs[1]), dev.t(arrs[2]), cap,
                       pages=torch.tensor(perm.reshape(n_seq, npp), device="cuda"), page=page)


@pytest.mark.parametrize("path,T,B,L,H,d,k,W,m,page,wpage", [
    ("sparse", 128, 4, 8192, 64, 512, 1024, 128, 4, 64, 32),    # two-role kernel, paged
    ("sparse", 4, 4, 8192, 64, 512, 1024, 128, 4, 16, 128),     # split-KV 64-head kernel, paged
    ("sparse", 4, 2, 8192, 64, 128, 1024, 128, 4, 256, 8),      # 64 heads, d = 128, paged
    ("sparse", 6, 3, 2048, 16, 128, 64, 128, 4, 32, 1),         # 16 heads, paged
    ("dense", 128, 8, 131072, 64, 512, 0, 128, 128, 128, 64),   # HCA, two-role kernel, paged
    ("dense", 8, 8, 131072, 64, 512, 0, 128, 128, 1024, 128),   # HCA decode, paged
])
def test_paged_attention_against_oracle(lib, dev, gen, orc, path, T, B, L, H, d, k, W, m, page, wpage):
    """Attention reading a paged compressed cache and a paged window ring (pages in a shuffled
    physical order) against the oracle on the logical entries (seq * cap + slot)."""
    import torch

    _say(f"paged attention {path} T={T} B={B} L={L} H={H} d={d} k={k} page={page} wpage={wpage}")
    N = L // m
    comp, win, q = _attn_inputs(gen, 800 + T + d, B, N, W, H, d, T, L, W)
    rng = np.random.default_rng(T + page)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.full(T, L - 1, np.int64)
    pos[0] = L - 7
    pos[-1] = L // 2 + 1
    sm = 1.0 / math.sqrt(d)
    pc = _paged_from_host(lib, torch, dev, comp, B, N, page, rng)
    pw = _paged_from_host(lib, torch, dev, win, B, W, wpage, rng, extra=0)
    if path == "sparse":
        idx = gen.random_idx(801 + T, 1, (pos + 1) // m, k)
        ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, W, W, m, sm, idx=idx)
        out, lse = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(idx), m, pc, pw, W, sm)
    else:
        ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, W, W, m, sm)
        out, lse = lib.hca_dense_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), m, N, pc, pw, W, sm)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"paged {path}")


# --------------------------------------------------------------------------
# attention backward (csa_mqa_bwd) against the fp64 gradient of the oracle
# --------------------------------------------------------------------------
def assert_grad_close(got, ref, what):
    got = np.asarray(got, np.float64)
    r = rel_rms(got, ref)
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    ma = float(np.max(np.abs(got - ref))) / scale
    print(f"{what}: rel-rms {r:.2e} max-abs/max {ma:.2e}", flush=True)
    assert r <= REL_RMS and ma <= MAX_ABS, f"{what}: rel-rms {r:.3e} max-abs/max {ma:.3e}"


@pytest.mark.parametrize("T,B,L,H,k,W,m,win_cap,sel,same_seq", [
    (6, 3, 4096, 64, 200, 128, 4, 128, True, False),    # 5 tiles + a ragged one; -1 padding in one row
    (16, 1, 2048, 32, 96, 64, 4, 96, True, True),       # 16 rows of one sequence: shared entries and window
    (5, 2, 512, 16, 0, 16, 4, 16, False, False),        # every visible entry (no selection), small window
    (3, 3, 256, 64, 64, 0, 4, 1, True, False),          # no window branch
])
def test_mqa_bwd(lib, dev, gen, orc, T, B, L, H, k, W, m, win_cap, sel, same_seq):
    import torch

    from oracle import backward as obw

    d = 512
    _say(f"mqa_bwd T={T} B={B} L={L} H={H} k={k} W={W} m={m} sel={sel}")
    N = L // m
    comp, win, q = _attn_inputs(gen, 700 + T, B, N, W, H, d, T, L, win_cap)
    seq = (np.zeros(T) if same_seq else np.arange(T) % B).astype(np.int32)
    pos = (L - 1 - np.arange(T) * (3 if same_seq else 37)).astype(np.int64)
    pos[-1] = min(pos[-1], 70)  # a short row: partial window, fewer visible entries than k
    nv = (pos + 1) // m
    idx = gen.random_idx(701 + T, 1, nv, k) if sel else None
    dout = gen.normal_f32(702 + T, 1, (T, H, d)) * 0.01
    sm = 1.0 / math.sqrt(d)
    kvc = dev.kv_cache(comp, N)
    kvw = dev.kv_cache(win, win_cap) if W > 0 else None
    tq, tseq, tpos = dev.bf16(q), dev.t(seq), dev.t(pos)
    tidx = dev.t(idx) if sel else None
    if sel:
        out, lse = lib.csa_sparse_mqa(tq, tseq, tpos, tidx, m, kvc, kvw, W, sm)
    else:
        out, lse = lib.hca_dense_mqa(tq, tseq, tpos, m, int(nv.max()), kvc, kvw, W, sm)
    dq, dcomp, dwin = lib.csa_mqa_bwd(tq, tseq, tpos, tidx, m, kvc, kvw, W, sm, out, lse, dev.t(dout))
    dq2, dcomp2, dwin2 = lib.csa_mqa_bwd(tq, tseq, tpos, tidx, m, kvc, kvw, W, sm, out, lse, dev.t(dout))
    torch.cuda.synchronize()
    # entry gradients are summed in fixed point: two runs give the same bits
    assert torch.equal(dq, dq2) and torch.equal(dcomp, dcomp2), "backward differs between two runs"
    assert dwin is None or torch.equal(dwin, dwin2)
    rq, rc, rw = obw.attend_bwd(q, seq, pos, comp, N, win, win_cap, W, m, sm, dout, idx=idx)
    assert_grad_close(dq.cpu().numpy(), rq, "dq")
    got_c = dcomp.cpu().numpy()
    assert np.array_equal(got_c != 0, rc != 0) or np.all(got_c[rc == 0] == 0), "dcomp rows outside the key sets"
    assert_grad_close(got_c, rc, "dcomp")
    if W > 0:
        got_w = dwin.cpu().numpy()
        assert np.all(got_w[rw == 0] == 0), "dwin rows outside the windows"
        assert_grad_close(got_w, rw, "dwin")


# --------------------------------------------------------------------------
# determinism and batch invariance (the rule stated at the top of csa.h)
# --------------------------------------------------------------------------
def test_batch_invariance_and_determinism(lib, dev, gen, orc):
    """Row 0 of a decode batch, run alone and inside batches of 4, 7, 8, 14, 15, 32 and 200
    rows: its index scores and top-k indices are the same bits in every batch; its attention
    output is the same bits whenever the split-KV partition and the head split are the same
    (at k = 1024, window = 128: T <= 7 takes 18 splits shared by two workgroups, 8 <= T <= 14
    takes 9 shared splits, T = 15 takes 18 splits of one workgroup), agrees within the
    attention bar otherwise, does not change when the other rows' inputs change, and repeats
    bit for bit run to run.  HCA with max_vis at 1x and 8x the visible count: within the
    attention bar (the bound sets the partition)."""
    import torch

    _say("batch invariance")
    B, N, m, H, d, k, W, h_i, d_i = 4, 4096, 4, 64, 512, 1024, 128, 8, 128
    L = N * m
    Tmax = 200
    rng = np.random.default_rng(77)
    seq = (np.arange(Tmax) % B).astype(np.int32)
    pos = rng.integers(L // 2, L, size=Tmax).astype(np.int64)
    pos[0] = L - 1
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 9100, Tmax, h_i, d_i, N, B, pos, seq)
    keys = dev.index_keys((kd, ks), N)
    comp, win, q = _attn_inputs(gen, 9101, B, N, W, H, d, Tmax, L, W)
    kvc, kvw = dev.kv_cache(comp, N), dev.kv_cache(win, W)
    sm = 1.0 / math.sqrt(d)
    res = {}
    for T in (1, 4, 7, 8, 14, 15, 32, Tmax):
        sl = slice(0, T)
        sc = lib.csa_index_scores(dev.t(qd[sl]), dev.t(qs[sl]), dev.t(w[sl]), dev.t(seq[sl]), dev.t(pos[sl]), keys, m, N)
        ix = lib.csa_topk(sc, dev.t(pos[sl]), m, k)
        o, l = lib.csa_sparse_mqa(dev.bf16(q[sl]), dev.t(seq[sl]), dev.t(pos[sl]), ix, m, kvc, kvw, W, sm)
        o2, l2 = lib.csa_sparse_mqa(dev.bf16(q[sl]), dev.t(seq[sl]), dev.t(pos[sl]), ix, m, kvc, kvw, W, sm)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(l, l2), f"T={T}: attention differs run to run"
        res[T] = (sc[0].cpu().numpy(), ix[0].cpu().numpy(), o[0].cpu().numpy(), l[0].cpu().numpy())
    wit = orc.index_exact_witness(qd[:1], qs[:1], w[:1], seq[:1], pos[:1], kd, ks, N, m, N)
    assert wit < 24
    s0, i0, o0, l0 = res[1]
    same = {4: 1, 7: 1, 14: 8}  # T -> a batch size with the same partition and head split
    for T in (4, 7, 8, 14, 15, 32, Tmax):
        s, i, o, l = res[T]
        assert np.array_equal(s.view(np.uint32), s0.view(np.uint32)), f"T={T}: index scores of row 0 differ"
        assert np.array_equal(i, i0), f"T={T}: top-k of row 0 differs"
        if T in same:
            _, _, oe, le = res[same[T]]
            assert np.array_equal(o.view(np.uint32), oe.view(np.uint32)) and np.array_equal(l, le), \
                f"T={T}: attention of row 0 differs from T={same[T]} with the same partition"
        else:
            # another partition: fp16 partials and P round differently; both sides meet the oracle bar
            r, ma = rel_rms(o, o0), float(np.max(np.abs(o - o0)))
            print(f"T={T}: row 0 against T=1: rel-rms {r:.2e} max-abs {ma:.2e}", flush=True)
            assert r <= REL_RMS and ma <= MAX_ABS and np.max(np.abs(l - l0)) <= MAX_ABS, f"T={T}: row 0 differs"
    # other rows' inputs changed: row 0 unchanged (same T, same partition)
    T = 32
    q2 = q[:T].copy()
    q2[1:] = gen.normal_bf16(9102, 1, q2[1:].shape)
    ix = lib.csa_topk(lib.csa_index_scores(dev.t(qd[:T]), dev.t(qs[:T]), dev.t(w[:T]), dev.t(seq[:T]),
                                           dev.t(pos[:T]), keys, m, N), dev.t(pos[:T]), m, k)
    o, l = lib.csa_sparse_mqa(dev.bf16(q2), dev.t(seq[:T]), dev.t(pos[:T]), ix, m, kvc, kvw, W, sm)
    torch.cuda.synchronize()
    assert np.array_equal(o[0].cpu().numpy().view(np.uint32), res[32][2].view(np.uint32))
    # HCA: the bound max_vis sets the partition; 1x and 8x agree within rounding, each repeats exactly
    mh = 128
    Nh = L // mh
    hcomp = gen.entries(9103, 1, B * Nh, d - 64)
    kvh = dev.kv_cache(hcomp, Nh)
    outs = []
    for mv in (Nh, 8 * Nh):
        a = lib.hca_dense_mqa(dev.bf16(q[:4]), dev.t(seq[:4]), dev.t(pos[:4]), mh, mv, kvh, kvw, W, sm)
        b = lib.hca_dense_mqa(dev.bf16(q[:4]), dev.t(seq[:4]), dev.t(pos[:4]), mh, mv, kvh, kvw, W, sm)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        outs.append(a[0].cpu().numpy())
    r = rel_rms(outs[1], outs[0])
    print(f"HCA max_vis 1x vs 8x: rel-rms {r:.2e}", flush=True)
    assert r <= REL_RMS


def test_debug_check_rejects_rope_beyond_fp16(lib, dev, gen, orc, monkeypatch):
    """CSA_DEBUG_CHECKS=1: an entry whose bf16 RoPE dim exceeds the fp16 range is rejected
    before the attention runs (only when a row reads it); without the variable the call runs."""
    import torch

    _say("debug range check of RoPE dims")
    B, N, H, d, k, W, m = 2, 256, 64, 512, 64, 16, 4
    comp, win, q = _attn_inputs(gen, 460, B, N, W, H, d, 2, N * m, W)
    rope = comp[1].copy()
    rope[5, 3] = _f64_to_bf16_bits(np.array([70000.0]))[0]  # entry 5 of sequence 0
    comp = (comp[0], rope, comp[2])
    seq = np.array([0, 1], np.int32)
    pos = np.array([N * m - 1, N * m - 1], np.int64)
    sm = 1.0 / math.sqrt(d)
    kvc, kvw = dev.kv_cache(comp, N), dev.kv_cache(win, W)
    with_5 = np.tile(np.arange(k, dtype=np.int32), (2, 1))           # row 0 reads entry 5 of sequence 0
    without = np.tile(np.arange(100, 100 + k, dtype=np.int32), (2, 1))
    monkeypatch.setenv("CSA_DEBUG_CHECKS", "1")
    with pytest.raises(lib.CsaError) as e:
        lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(with_5), m, kvc, kvw, W, sm)
    assert e.value.code == lib.CSA_EINVAL and "65504" in str(e.value)
    with pytest.raises(lib.CsaError):
        lib.hca_dense_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), m, N, kvc, kvw, W, sm)
    out, lse = lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(without), m, kvc, kvw, W, sm)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.attend(q, seq, pos, comp, N, win, W, W, m, sm, idx=without)
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "debug check, entry not read")
    monkeypatch.setenv("CSA_DEBUG_CHECKS", "0")
    lib.csa_sparse_mqa(dev.bf16(q), dev.t(seq), dev.t(pos), dev.t(with_5), m, kvc, kvw, W, sm)  # not checked
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# csa_index_topk: indexer + top-k fused, no score rows written
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,h_i,d_i,N,B,m,n_cols,k,mode,plant", [
    (4, 8, 128, 70000, 4, 4, 70000, 1024, "decode", 0.05),     # rows kernel, long rows
    (4, 8, 128, 262144, 4, 4, 262144, 1024, "decode", 0.05),   # the 1M-context decode shape
    (3, 8, 128, 5000, 3, 4, 4990, 512, "decode", 0.0),
    (8, 8, 128, 100000, 8, 4, 100000, 2048, "decode", 0.02),
    (5, 4, 64, 3000, 2, 4, 3000, 1, "decode", 0.0),
    (6, 8, 128, 20000, 3, 4, 20000, 64, "short", 0.0),        # some rows see fewer than k columns
    (2048, 4, 64, 512, 1, 4, 512, 64, "prefill", 0.0),        # the small prefill shape (matrix-core GEMM)
    (300, 8, 128, 3000, 1, 4, 3000, 1024, "prefill", 0.0),
    (200, 8, 128, 9000, 3, 4, 9000, 256, "mixed", 0.0),       # several sequences in a tile
    (130, 8, 128, 40000, 1, 4, 40000, 1024, "prefill", 0.05),
    (100, 8, 64, 5000, 1, 4, 5000, 2048, "prefill", 0.0),    # 8,192 candidates in LDS
    (130, 8, 128, 12000, 1, 4, 12000, 1100, "prefill", 0.02), # 4,096 (k = 1024 and below: 3,072)
])
def test_index_topk_bit_exact(lib, dev, gen, orc, T, h_i, d_i, N, B, m, n_cols, k, mode, plant):
    import torch

    _say(f"index_topk T={T} h_i={h_i} d_i={d_i} N={N} k={k} {mode}")
    rng = np.random.default_rng(T + N + k)
    if mode == "decode":
        seq = np.arange(T) % B
        pos = np.full(T, m * N - 1, np.int64)
        pos[-1] = m * N - 5
    elif mode == "short":
        seq = np.arange(T) % B
        pos = rng.integers(0, m * N, size=T)
        pos[0] = m * 100 + 3
    elif mode == "prefill":
        seq = np.zeros(T, np.int64)
        pos = np.sort(rng.integers(0, m * N, size=T))
        pos[-1] = m * N - 1
    else:
        seq = rng.integers(0, B, size=T)
        pos = rng.integers(0, m * N, size=T)
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 950 + T + k, T, h_i, d_i, N, B, pos, seq, plant=plant)
    wit = orc.index_exact_witness(qd, qs, w, seq, pos, kd, ks, N, m, n_cols)
    assert wit < 24, f"inputs break the fp32 exactness precondition ({wit:.1f} bits)"
    ref = orc.topk(orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, n_cols).astype(np.float32), pos, m, k)
    keys = dev.index_keys((kd, ks), N)
    args = (dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, m, n_cols)
    ws = torch.full((lib.csa_index_topk_workspace(T, n_cols, k, h_i),), 0x5A, dtype=torch.uint8, device="cuda")
    got = lib.csa_index_topk(*args, k, ws=ws)
    again = lib.csa_index_topk(*args, k, ws=ws)  # the workspace needs no initialisation between calls
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.where((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5].tolist()}"
    assert np.array_equal(again.cpu().numpy(), ref)


@pytest.mark.parametrize("T,N,B,k,layout", [
    (3, 20000, 3, 1024, "decode"),
    (100, 6000, 1, 512, "prefill"),
])
def test_index_topk_fallback_equal_scores(lib, dev, gen, orc, T, N, B, k, layout):
    """Every key identical: each row's scores are all equal, so every visible column reaches
    the threshold, the candidate space overflows and each row is scored again and selected
    over the whole row: the k lowest visible columns."""
    import torch

    _say(f"index_topk fallback, equal scores T={T} N={N} k={k} {layout}")
    m, h_i, d_i = 4, 8, 128
    rng = np.random.default_rng(31)
    seq = (np.arange(T) % B).astype(np.int32)
    pos = rng.integers(m * 2000, m * N, size=T).astype(np.int64) if layout == "prefill" else \
        np.full(T, m * N - 1, np.int64)
    qd, qs, w, seq, pos, _, _ = _index_case(gen, 960, T, h_i, d_i, N, B, pos, seq)
    kd = np.full((B * N, d_i // 2), 0x22, np.uint8)
    ks = np.full((B * N, d_i // 32), 127, np.uint8)
    ref = orc.topk(orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, N).astype(np.float32), pos, m, k)
    got = lib.csa_index_topk(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), dev.index_keys((kd, ks), N), m,
                             N, k)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_index_topk_fallback_too_few(lib, dev, gen, orc):
    """High scores planted only in sampled column groups after the sampled prefix (the prefix
    is 2,048 columns at k <= 1024, then one 32-column group in 16): the sample predicts far more
    high columns than there are, fewer than k columns reach the threshold, and the rows are
    scored again and selected over the whole row."""
    import torch

    _say("index_topk fallback, too few candidates")
    T, B, N, m, k, h_i, d_i = 2, 2, 70000, 4, 1024, 8, 128
    seq = np.arange(T, dtype=np.int32)
    pos = np.full(T, m * N - 1, np.int64)
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 970, T, h_i, d_i, N, B, pos, seq)
    kd, ks = kd.copy(), ks.copy()
    cols = np.concatenate([2048 + 512 * g + np.arange(32) for g in range(8)])  # 8 sampled groups
    for b in range(B):
        kd[b * N + cols] = qd[b, 0]   # aligned with head 0 of the row's query: large scores
        ks[b * N + cols] = qs[b, 0]
    sc = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, N)
    assert np.all(np.sort(sc, axis=1)[:, -256] > np.sort(sc, axis=1)[:, -257])  # the planted 256 lead each row
    ref = orc.topk(sc.astype(np.float32), pos, m, k)
    got = lib.csa_index_topk(dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), dev.index_keys((kd, ks), N), m,
                             N, k)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


# --------------------------------------------------------------------------
# csa_index_bwd: gradient of the indexer scores against the fp64 oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,h_i,d_i,N,B,m,n_sel,layout", [
    (6, 8, 128, 3000, 2, 4, 1024, "decode"),     # selected by the library's own top-k
    (64, 4, 64, 500, 1, 4, 64, "prefill"),       # causal rows of one sequence: keys shared by many rows
    (3, 8, 128, 5000, 3, 4, 2500, "random"),     # more selected columns than one chunk; -1 and invisible entries
    (40, 8, 64, 800, 2, 2, 300, "random"),
])
def test_index_bwd(lib, dev, gen, orc, T, h_i, d_i, N, B, m, n_sel, layout):
    import torch

    from oracle import index_backward as ib

    _say(f"index_bwd T={T} h_i={h_i} d_i={d_i} N={N} n_sel={n_sel} {layout}")
    rng = np.random.default_rng(T + N + n_sel)
    if layout == "prefill":
        seq = np.zeros(T, np.int64)
        pos = np.sort(rng.integers(m * 4, m * N, size=T))
    else:
        seq = np.arange(T) % B
        pos = rng.integers(m * N // 2, m * N, size=T)
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 980 + T, T, h_i, d_i, N, B, pos, seq)
    keys = dev.index_keys((kd, ks), N)
    tq, tqs, tw, tseq, tpos = dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos)
    if layout in ("decode", "prefill"):
        idx = lib.csa_topk(lib.csa_index_scores(tq, tqs, tw, tseq, tpos, keys, m, N), tpos, m, n_sel).cpu().numpy()
    else:
        idx = rng.integers(-1, N, size=(T, n_sel)).astype(np.int32)
    G = gen.normal_f32(981 + T, 1, (T, n_sel))
    rq, rw, rk = ib.index_bwd(qd, qs, w, seq, pos, kd, ks, N, m, idx, G)
    dq, dw, dk = lib.csa_index_bwd(tq, tqs, tw, tseq, tpos, keys, m, dev.t(idx), dev.t(G))
    dk2 = lib.csa_index_bwd(tq, tqs, tw, tseq, tpos, keys, m, dev.t(idx), dev.t(G))[2]
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2), "key gradients differ between two runs"
    for got, ref, name in ((dq, rq, "dq"), (dw, rw, "dw"), (dk, rk, "dkeys")):
        got = got.cpu().numpy().astype(np.float64).reshape(ref.shape)
        r = rel_rms(got, ref)
        ma = float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30)
        print(f"index_bwd {name}: rel-rms {r:.2e} max-abs/max {ma:.2e}", flush=True)
        assert r <= 1e-5 and ma <= 1e-5, f"{name}: rel-rms {r:.3e} max-abs/max {ma:.3e}"
    # key rows no row selected (validly) get no gradient
    nv = (pos + 1) // m
    used = np.zeros(B * N, bool)
    for t in range(T):
        v = idx[t][(idx[t] >= 0) & (idx[t] < nv[t])]
        used[seq[t] * N + v] = True
    assert not dk.cpu().numpy()[~used].any(), "gradient on key rows no row selected"


# --------------------------------------------------------------------------
# paged index keys, and compressed pages stored on the host / on disk and loaded back
# --------------------------------------------------------------------------
@pytest.mark.parametrize("page", [64, 1024])
def test_paged_index_keys_all_paths(lib, dev, gen, orc, page):
    """Index keys in a paged layout (pages in a shuffled order, spare pages unused) read by
    every indexer path.  The prefill matrix-core kernel writes score rows, and the fused
    selection runs its sample and emit passes, over two sequences in one batch.  The grouped
    multi-token kernel also reads them.  Scores and indices equal the oracle's on the logical
    keys bit for bit.  The indexer backward equals the contiguous layout's bit for bit, its key
    gradients landing on the physical rows."""
    import torch

    _say(f"paged index keys, every indexer path, page {page}")
    B, m, d_i, h_i, N, k = 2, 4, 128, 8, 4096, 256
    npp = N // page
    rng = np.random.default_rng(page)
    perm = rng.permutation(B * npp + 2)[: B * npp].astype(np.int32)
    n_phys = (B * npp + 2) * page
    phys = (perm.reshape(B, npp)[:, :, None] * page + np.arange(page)[None, None, :]).reshape(-1)  # logical -> physical
    # the prefill rows: sequence 0, then sequence 1 (both inside one 64-query tile at the seam)
    T = 130
    seq = (np.arange(T) >= 65).astype(np.int32)
    pos = np.concatenate([np.sort(rng.integers(m * 8, m * N, size=65)), np.sort(rng.integers(m * 8, m * N, size=T - 65))])
    qd, qs, w, seq, pos, kd, ks = _index_case(gen, 870 + page, T, h_i, d_i, N, B, pos, seq, plant=0.02)
    assert orc.index_exact_witness(qd, qs, w, seq, pos, kd, ks, N, m, N) < 24
    pd = np.zeros((n_phys, d_i // 2), np.uint8)
    ps = np.full((n_phys, d_i // 32), 127, np.uint8)
    pd[phys], ps[phys] = kd, ks
    keys_p = lib.IndexKeys(dev.t(pd), dev.t(ps), N, pages=torch.tensor(perm.reshape(B, npp), device="cuda"), page=page)
    keys_c = dev.index_keys((kd, ks), N)
    ref = orc.index_scores(qd, qs, w, seq, pos, kd, ks, N, m, N).astype(np.float32)
    ref_i = orc.topk(ref, pos, m, k)
    tq, tqs, tw, tseq, tpos = dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos)
    sc = lib.csa_index_scores(tq, tqs, tw, tseq, tpos, keys_p, m, N)
    ix = lib.csa_index_topk(tq, tqs, tw, tseq, tpos, keys_p, m, N, k)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref.view(np.uint32)), "paged prefill scores"
    assert np.array_equal(ix.cpu().numpy(), ref_i), "paged prefill fused selection"
    # grouped multi-token rows: two rows per sequence share each key stream
    rows = np.array([64, 63, 129, 128])  # near the ends of the two sequences
    g_args = [dev.t(np.ascontiguousarray(a[rows])) for a in (qd, qs, w, seq, pos)]
    gsc = lib.csa_index_scores_grouped(*g_args, keys_p, m, N, 2)
    torch.cuda.synchronize()
    assert np.array_equal(gsc.cpu().numpy().view(np.uint32), ref[rows].view(np.uint32)), "paged grouped scores"
    # backward: paged against contiguous, key gradients compared through the page table
    G = gen.normal_f32(872 + page, 1, (T, k))
    dq_p, dw_p, dk_p = lib.csa_index_bwd(tq, tqs, tw, tseq, tpos, keys_p, m, ix, dev.t(G), key_rows=n_phys)
    dq_c, dw_c, dk_c = lib.csa_index_bwd(tq, tqs, tw, tseq, tpos, keys_c, m, ix, dev.t(G))
    torch.cuda.synchronize()
    assert torch.equal(dq_p, dq_c) and torch.equal(dw_p, dw_c), "paged backward: dq / dw"
    dk_p = dk_p.cpu().numpy()
    assert np.array_equal(dk_p[phys], dk_c.cpu().numpy()), "paged backward: key gradients"
    spare = np.setdiff1d(np.arange(n_phys), phys)
    assert not dk_p[spare].any(), "gradient on a spare page"


def test_paged_index_keys_and_page_files(lib, dev, gen, orc, tmp_path):
    """Index keys compressed into a paged layout (pages in a shuffled order, shared page table with
    the compressed entries) equal the oracle's keys; the indexer and the fused selection read them
    bit-exactly against the oracle.  Sequence 0's pages (entries and keys) go to a file and come back
    into a fresh cache at other physical pages byte for byte, and a sequence reading the reloaded
    prefix gets the same scores, selection and attention as the original."""
    import torch

    _say("paged index keys, page files")
    B, m, d, d_i, h_i, cap, page, k, W, H = 2, 4, 512, 128, 8, 1024, 128, 256, 128, 64
    L, npp = cap * m, cap // page
    rng = np.random.default_rng(12)
    perm = rng.permutation(B * npp + 3)[: B * npp].astype(np.int32)
    pages = torch.tensor(perm.reshape(B, npp), device="cuda")
    n_phys = (B * npp + 3) * page
    kv = lib.KvCache(torch.zeros(n_phys, d - 64, dtype=torch.uint8, device="cuda"),
                     torch.zeros(n_phys, 64, dtype=torch.bfloat16, device="cuda"),
                     torch.zeros(n_phys, dtype=torch.float32, device="cuda"), cap, pages=pages, page=page)
    keys = lib.IndexKeys(torch.zeros(n_phys, d_i // 2, dtype=torch.uint8, device="cuda"),
                         torch.zeros(n_phys, d_i // 32, dtype=torch.uint8, device="cuda"), cap, pages=pages, page=page)
    toks = [gen.normal_bf16(830 + b, 1, (L, d)) for b in range(B)]
    ikt = [gen.normal_bf16(830 + b, 2, (L, d_i)) for b in range(B)]
    lgs = [gen.normal_f32(830 + b, 3, (L,)) for b in range(B)]
    for b in range(B):
        lib.csa_compress(dev.bf16(toks[b]), dev.t(lgs[b]), 0, m, b, kv)
        lib.csa_compress_index_keys(dev.bf16(ikt[b]), dev.t(lgs[b]), 0, m, b, keys)
    torch.cuda.synchronize()
    # logical key rows (seq * cap + j) against the oracle's compression
    ref_d = np.zeros((B * cap, d_i // 2), np.uint8)
    ref_s = np.zeros((B * cap, d_i // 32), np.uint8)
    for b in range(B):
        ref_d[b * cap:(b + 1) * cap], ref_s[b * cap:(b + 1) * cap] = orc.compress_index_keys(ikt[b], lgs[b], 0, m)
    phys = (perm.reshape(B, npp)[:, :, None] * page + np.arange(page)[None, None, :]).reshape(-1)
    assert np.array_equal(keys.data.cpu().numpy()[phys], ref_d) and np.array_equal(keys.scale.cpu().numpy()[phys], ref_s)
    # indexer and fused selection through the page table, against the oracle on the logical keys
    T = 6
    seq = (np.arange(T) % B).astype(np.int32)
    pos = np.array([L - 1, L - 1, L - 9, 1500, 700, L // 2], np.int64)
    qd, qs, _ = gen.mxfp4(831, 1, T * h_i, d_i)
    qd, qs = qd.reshape(T, h_i, -1), qs.reshape(T, h_i, -1)
    w = gen.pow2_weights(831, 2, (T, h_i))
    ref = orc.index_scores(qd, qs, w, seq, pos, ref_d, ref_s, cap, m, cap).astype(np.float32)
    ref_i = orc.topk(ref, pos, m, k)
    args = (dev.t(qd), dev.t(qs), dev.t(w), dev.t(seq), dev.t(pos), keys, m, cap)
    sc = lib.csa_index_scores(*args)
    fused = lib.csa_index_topk(*args, k)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref.view(np.uint32)), "paged index scores"
    assert np.array_equal(fused.cpu().numpy(), ref_i), "fused selection over paged keys"
    # sequence 0's pages to a file, back into a fresh cache at other physical pages
    path = str(tmp_path / "prefix.pages")
    lib.save_pages(path, kv, keys, perm[:npp].tolist())
    perm2 = rng.permutation(npp + 2)[:npp].astype(np.int32)
    n2 = (npp + 2) * page
    kv2 = lib.KvCache(torch.zeros(n2, d - 64, dtype=torch.uint8, device="cuda"),
                      torch.zeros(n2, 64, dtype=torch.bfloat16, device="cuda"),
                      torch.zeros(n2, dtype=torch.float32, device="cuda"), cap,
                      pages=torch.tensor(perm2[None, :], device="cuda"), page=page)
    keys2 = lib.IndexKeys(torch.zeros(n2, d_i // 2, dtype=torch.uint8, device="cuda"),
                          torch.zeros(n2, d_i // 32, dtype=torch.uint8, device="cuda"), cap,
                          pages=torch.tensor(perm2[None, :], device="cuda"), page=page)
    lib.load_pages(path, kv2, keys2, perm2.tolist())
    for i in range(npp):
        a = torch.arange(page, device="cuda")
        r1, r2 = int(perm[i]) * page + a, int(perm2[i]) * page + a
        for x, y in ((kv.nope, kv2.nope), (kv.rope, kv2.rope), (kv.scale, kv2.scale), (keys.data, keys2.data),
                     (keys.scale, keys2.scale)):
            assert torch.equal(x[r1], y[r2]), f"page {i} differs after the round trip"
    # the reloaded prefix as sequence 0 of its own cache: same scores, selection and attention
    rows = np.where(seq == 0)[0]
    sub = lambda a: np.ascontiguousarray(a[rows])  # noqa: E731
    a2 = (dev.t(sub(qd)), dev.t(sub(qs)), dev.t(sub(w)), dev.t(np.zeros(len(rows), np.int32)), dev.t(sub(pos)), keys2,
          m, cap)
    sc2 = lib.csa_index_scores(*a2)
    ix2 = lib.csa_index_topk(*a2, k)
    win = dev.kv_cache(gen.entries(832, 1, B * W, d - 64), W)
    q = gen.normal_bf16(833, 1, (len(rows), H, d))
    sm = 1.0 / math.sqrt(d)
    o1, l1 = lib.csa_sparse_mqa(dev.bf16(q), dev.t(np.zeros(len(rows), np.int32)), dev.t(sub(pos)),
                                fused[torch.tensor(rows, device="cuda")].contiguous(), m, kv, win, W, sm)
    o2, l2 = lib.csa_sparse_mqa(dev.bf16(q), dev.t(np.zeros(len(rows), np.int32)), dev.t(sub(pos)), ix2, m, kv2, win,
                                W, sm)
    torch.cuda.synchronize()
    assert np.array_equal(sc2.cpu().numpy().view(np.uint32), ref[rows].view(np.uint32))
    assert np.array_equal(ix2.cpu().numpy(), ref_i[rows])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.gpu
def test_mfma_probe_runs():
    """The matrix-core probe the benchmark uses for context: one small launch of each kind
    completes, reports its flop count and writes a finite value per thread."""
    import torch

    import compressed_sparse_long_compress_amd as csa

    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    assert csa.mfma_probe(0, 8, 16, sink) == 16 * 16 * 32 * 2 * 4 * 16 * 8 * 4
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    sink.fill_(float("nan"))
    assert csa.mfma_probe(1, 8, 16, sink) == 32 * 32 * 64 * 2 * 4 * 16 * 8 * 4
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()

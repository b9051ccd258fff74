"""GPU parity at the full sizes of the named workloads, in the launch
configuration bench.py times.  Indices and scores are compared in full; the
oracle computes attention for every row of the decode batches and for a seeded
sample of rows of the prefill chunk, whose top-k is checked on every row."""
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


def _close(out, lse, ref_o, ref_l, what):
    out = np.asarray(out, np.float64)
    r = float(np.linalg.norm(out - ref_o) / np.linalg.norm(ref_o))
    ma = float(np.max(np.abs(out - ref_o)))
    lr = float(np.max(np.abs(np.asarray(lse, np.float64) - ref_l)))
    print(f"{what}: rel-rms {r:.2e} max-abs {ma:.2e} lse max-abs {lr:.2e}", flush=True)
    assert r <= REL_RMS and ma <= MAX_ABS and lr <= MAX_ABS


@pytest.mark.parametrize("name", ["csa_decode_1m", "csa_decode_64k"])
def test_csa_decode_full(lib, orc, name):
    import torch

    from bench import DecodeSet

    _say(f"full-size {name}")
    wl = configs.named(name)
    ds = DecodeSet(wl, replicas=1)
    ds.step(0)
    torch.cuda.synchronize()
    wit = orc.index_exact_witness(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0],
                                  wl["keys"][1], wl["N"], wl["m"], wl["n_cols"])
    assert wit < 24
    ref_s = orc.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0], wl["keys"][1],
                             wl["N"], wl["m"], wl["n_cols"]).astype(np.float32)
    got_s = ds.scores.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32)), "scores differ"
    ref_i = orc.topk(ref_s, wl["pos"], wl["m"], wl["k"])
    got_i = ds.idx.cpu().numpy()
    assert np.array_equal(got_i, ref_i), "top-k differs"
    # the fused indexer + top-k (no score rows) on the same batch
    fused = lib.csa_index_topk(ds.iq, ds.iqs, ds.w, ds.seq, ds.pos, ds.keys[0], wl["m"], wl["n_cols"], wl["k"])
    torch.cuda.synchronize()
    assert np.array_equal(fused.cpu().numpy(), ref_i), "fused index + top-k differs"
    if name == "csa_decode_1m":
        # the planted 5% dominate the selection (the structure makes top-k non-uniform)
        planted = wl["planted"].reshape(wl["B"], wl["N"])
        frac = np.mean([planted[b, ref_i[b][ref_i[b] >= 0]].mean() for b in range(wl["B"])])
        print(f"planted share of the top-k: {frac:.3f}", flush=True)
        assert frac > 0.5
    ref_o, ref_l = orc.attend(wl["q"], wl["seq"], wl["pos"], wl["comp"], wl["N"], wl["win"], wl["W"], wl["W"],
                              wl["m"], wl["sm_scale"], wl["rope_base"], idx=ref_i)
    _close(ds.out.cpu().numpy(), ds.lse.cpu().numpy(), ref_o, ref_l, name)


def test_hca_decode_1m_full(lib, orc):
    import torch

    from gen import device as dev

    _say("full-size hca_decode_1m")
    wl = configs.named("hca_decode_1m")
    out, lse = lib.hca_dense_mqa(dev.bf16(wl["q"]), dev.t(wl["seq"]), dev.t(wl["pos"]), wl["m"], wl["N"],
                                 dev.kv_cache(wl["comp"], wl["N"]), dev.kv_cache(wl["win"], wl["W"]), wl["W"],
                                 wl["sm_scale"], wl["rope_base"])
    torch.cuda.synchronize()
    ref_o, ref_l = orc.attend(wl["q"], wl["seq"], wl["pos"], wl["comp"], wl["N"], wl["win"], wl["W"], wl["W"],
                              wl["m"], wl["sm_scale"], wl["rope_base"])
    _close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "hca_decode_1m")


def test_prefill_chunk_sampled(lib, orc):
    """8,192 new tokens after a 131,072-token context: compress (CSA m=4, window
    m=1, HCA m'=128 on its own layer), index, top-k and both attentions on the
    GPU; the oracle recomputes the caches from the raw tokens and checks 48
    seeded rows of every later stage."""
    import torch

    from gen import device as dev

    _say("prefill_chunk sampled")
    wl = configs.named("prefill_chunk")
    T, L0, m, mh, d, W, k = wl["T"], wl["L0"], wl["m"], wl["m_hca"], wl["d"], wl["W"], wl["k"]
    total = wl["total"]
    comp = lib.KvCache.empty(1, wl["comp_cap"], d)
    hca = lib.KvCache.empty(1, wl["hca_cap"], d)
    win = lib.KvCache.empty(1, wl["win_cap"], d)
    win_h = lib.KvCache.empty(1, wl["win_cap"], d)
    kv, lg = dev.bf16(wl["kv"]), dev.t(wl["logits"])
    kvh, lgh = dev.bf16(wl["kv_hca"]), dev.t(wl["logits_hca"])
    # older context (set-up) then the new chunk
    lib.csa_compress(kv[:L0], lg[:L0], 0, m, 0, comp)
    lib.csa_compress(kvh[:L0], lgh[:L0], 0, mh, 0, hca)
    lib.csa_compress(kv[L0 - W:L0], lg[L0 - W:L0], L0 - W, 1, 0, win)
    lib.csa_compress(kvh[L0 - W:L0], lgh[L0 - W:L0], L0 - W, 1, 0, win_h)
    lib.csa_compress(kv[L0:], lg[L0:], L0, m, 0, comp)
    lib.csa_compress(kv[L0:], lg[L0:], L0, 1, 0, win)
    lib.csa_compress(kvh[L0:], lgh[L0:], L0, mh, 0, hca)
    lib.csa_compress(kvh[L0:], lgh[L0:], L0, 1, 0, win_h)
    seq, pos = dev.t(wl["seq"]), dev.t(wl["pos"])
    scores = lib.csa_index_scores(dev.t(wl["iq"][0]), dev.t(wl["iq"][1]), dev.t(wl["w"]), seq, pos,
                                  dev.index_keys(wl["keys"], wl["N"]), m, wl["n_cols"])
    idx = lib.csa_topk(scores, pos, m, k)
    out, lse = lib.csa_sparse_mqa(dev.bf16(wl["q"]), seq, pos, idx, m, comp, win, W, wl["sm_scale"])
    hout, hlse = lib.hca_dense_mqa(dev.bf16(wl["q_hca"]), seq, pos, mh, wl["hca_cap"], hca, win_h, W, wl["sm_scale"])
    torch.cuda.synchronize()

    # oracle caches from the raw tokens
    o_comp = orc.compress(wl["kv"], wl["logits"], 0, m)
    o_hca = orc.compress(wl["kv_hca"], wl["logits_hca"], 0, mh)
    g_comp = dev.host_entries(comp)
    assert np.mean(g_comp[0] != o_comp[0]) <= 1e-5 and np.mean(g_comp[1] != o_comp[1]) <= 1e-4
    g_hca = dev.host_entries(hca)
    assert np.mean(g_hca[0] != o_hca[0]) <= 1e-5 and np.mean(g_hca[1] != o_hca[1]) <= 1e-4
    wcap = wl["win_cap"]
    o_win = tuple(np.zeros((wcap,) + a.shape[1:], a.dtype) for a in o_comp)
    o_winh = tuple(np.zeros((wcap,) + a.shape[1:], a.dtype) for a in o_comp)
    orc.compress_into(wl["kv"][L0 - W:], wl["logits"][L0 - W:], L0 - W, 1, wl["rope_base"], *o_win)
    orc.compress_into(wl["kv_hca"][L0 - W:], wl["logits_hca"][L0 - W:], L0 - W, 1, wl["rope_base"], *o_winh)

    rows = np.sort(np.random.default_rng(105).choice(T, size=48, replace=False))
    rows[0], rows[-1] = 0, T - 1
    sub = lambda a: np.ascontiguousarray(a[rows])  # noqa: E731
    ref_s = orc.index_scores(sub(wl["iq"][0]), sub(wl["iq"][1]), sub(wl["w"]), sub(wl["seq"]), sub(wl["pos"]),
                             wl["keys"][0], wl["keys"][1], wl["N"], m, wl["n_cols"]).astype(np.float32)
    got_s = scores.cpu().numpy()[rows]
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32)), "scores differ"
    ref_i = orc.topk(ref_s, sub(wl["pos"]), m, k)
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx[rows], ref_i), "top-k differs"
    # every row's selection: the oracle's sort of the GPU's score matrix (bit-exact on the rows
    # checked above) against the GPU's indices, on all 8,192 rows
    all_i = orc.topk(scores.cpu().numpy(), wl["pos"], m, k)
    bad = np.where((all_i != got_idx).any(axis=1))[0]
    assert bad.size == 0, f"top-k differs on {bad.size} rows, first {bad[:5].tolist()}"
    del all_i
    # the fused indexer + top-k (no score rows): the same indices on every row
    fused = lib.csa_index_topk(dev.t(wl["iq"][0]), dev.t(wl["iq"][1]), dev.t(wl["w"]), seq, pos,
                               dev.index_keys(wl["keys"], wl["N"]), m, wl["n_cols"], k)
    torch.cuda.synchronize()
    bad = np.where((fused.cpu().numpy() != got_idx).any(axis=1))[0]
    assert bad.size == 0, f"fused index + top-k differs on {bad.size} rows, first {bad[:5].tolist()}"
    ref_o, ref_l = orc.attend(sub(wl["q"]), sub(wl["seq"]), sub(wl["pos"]), o_comp, wl["comp_cap"], o_win, wcap, W, m,
                              wl["sm_scale"], wl["rope_base"], idx=ref_i)
    _close(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ref_o, ref_l, "prefill sparse")
    ref_o, ref_l = orc.attend(sub(wl["q_hca"]), sub(wl["seq"]), sub(wl["pos"]), o_hca, wl["hca_cap"], o_winh, wcap, W,
                              mh, wl["sm_scale"], wl["rope_base"])
    _close(hout.cpu().numpy()[rows], hlse.cpu().numpy()[rows], ref_o, ref_l, "prefill dense")

    # ---- gradient of the sparse layer at full size: dq on the sampled rows against the oracle;
    #      the entry gradients through properties that hold at any size ----
    import gen as gen_mod
    from oracle import backward as obw

    _say("prefill_chunk backward")
    H = wl["H"]
    dout = gen_mod.normal_f32(108, 1, (T, H, d), sigma=0.01)
    dq, dcomp, dwin = lib.csa_mqa_bwd(dev.bf16(wl["q"]), seq, pos, idx, m, comp, win, W, wl["sm_scale"], out, lse,
                                      dev.t(dout))
    torch.cuda.synchronize()
    rq, _, _ = obw.attend_bwd(sub(wl["q"]), sub(wl["seq"]), sub(wl["pos"]), o_comp, wl["comp_cap"], o_win, wcap, W,
                              m, wl["sm_scale"], sub(dout), rope_base=wl["rope_base"], idx=ref_i)
    r = float(np.linalg.norm(dq.cpu().numpy()[rows] - rq) / np.linalg.norm(rq))
    print(f"prefill backward dq (48 rows): rel-rms {r:.2e}", flush=True)
    assert r <= 2e-3
    # entries no row selected get no gradient
    picked = np.zeros(wl["comp_cap"], bool)
    iv = idx.cpu().numpy()
    picked[iv[iv >= 0]] = True
    dc = dcomp.cpu().numpy()
    assert np.all(dc[~picked] == 0), "gradient on entries no row selected"
    # shifting every key by c moves every output by R(-t) c: the entry gradients of the whole
    # batch sum to the output gradients rotated by RoPE at each row's position
    want = np.zeros(d)
    p64 = np.asarray(wl["pos"], np.int64)
    for t in range(T):
        g = dout[t].astype(np.float64).sum(axis=0)
        g[d - 64:] = obw.rope_rows(g[d - 64:], int(p64[t]), wl["rope_base"])
        want += g
    got = dcomp.double().sum(dim=0).cpu().numpy() + dwin.double().sum(dim=0).cpu().numpy()
    r = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    print(f"prefill backward: sum of entry gradients rel-rms {r:.2e}", flush=True)
    assert r <= 2e-3

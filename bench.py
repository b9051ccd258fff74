"""Benchmark: CSA decode at 1M context on one MI355X (libcsa HIP kernels).

One step = the CSA decode hot path for a batch of 4 sequences, each with a
1,048,576-token context (262,144 compressed entries at m=4):
    csa_index_scores (MXFP4 indexer over every entry; it also writes the
                      selection's row summary: the largest score of every
                      32-column group)
 -> csa_topk (k = 1024)
 -> csa_sparse_mqa (64 query heads over the 1024 selected entries + a
    128-token window, d = 512).
Inputs are seeded synthetic tensors resident in HBM before timing starts;
8 replica sets of the keys and the compressed cache (~5.5 GB) rotate step by
step so the 256 MB Infinity Cache cannot serve a step from the previous one.
The timed steps are captured as one HIP graph (replica sets rotating as in
the eager loop) and replayed once; its outputs are checked against the eager
step.

Prints ONE JSON line: queries/s for the batch, a roofline object for the
dominant kernel (the indexer, bound by HBM), the chunked prefill (8,192 new
tokens after 131,072: tokens/s and its MFMA-bound kernels against their
peaks), and the fp64 CPU oracle timed on the same decode batch as a reported
baseline.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--all]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth

# HBM bytes per launch of the indexer kernel on the csa_decode_1m workload, from
# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (scaled by a 256 MiB copy: fetch x2.0,
# write x1.0; see profiles/csa_decode_1m_hbm_counters.md), valid for the kernel
# source with this SHA-256 only.
INDEX_TRAFFIC = {"sha256": "b18be7603c59c00594d3057c40396d74df1b4e5c589746bd8420d3e41bffbdee", "bytes": 75746141}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def index_traffic():
    """Counter-measured bytes per indexer launch, or None once the kernel source changed."""
    import hashlib

    src = os.path.join(ROOT, "compressed_sparse_long_compress_amd", "csrc", "index_scores.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return INDEX_TRAFFIC["bytes"] if sha == INDEX_TRAFFIC["sha256"] else None


def index_bytes_per_query(N, h_i, d_i):
    """Algorithmic HBM bytes of csa_index_scores per query row: every MXFP4 key
    (d_i/2 data + d_i/32 scale bytes) and the query (h_i MXFP4 vectors and their
    fp32 head weights).  17,826,368 B per row at 1M context."""
    key = d_i // 2 + d_i // 32
    return N * key + h_i * key + h_i * 4


def index_excess_bytes_per_query(N):
    """Bytes the indexer writes beyond the algorithmic ones: the fp32 score row and
    the selection's row summary (one 4-byte key per 32 columns)."""
    return N * 4 + (N + 31) // 32 * 4


def step_bytes_per_query(N, h_i, d_i, k, W, H, d):
    """Algorithmic HBM bytes of the whole decode step per query: the indexer's
    keys and query, the gathered entries (k + W) x (d-64 + 128 + 4) B, the bf16
    query and the fp32 output (18,691,136 B per query at 1M context)."""
    entry = (d - 64) + 64 * 2 + 4
    return index_bytes_per_query(N, h_i, d_i) + (k + W) * entry + H * d * 2 + H * d * 4


class DecodeSet:
    """Device tensors of one CSA decode workload, with replica rotation."""

    def __init__(self, wl, replicas):
        import torch

        import compressed_sparse_long_compress_amd as csa
        from gen import device as dev

        self.wl = wl
        B, N, W = wl["B"], wl["N"], wl["W"]
        keys0 = dev.index_keys(wl["keys"], N)
        comp0 = dev.kv_cache(wl["comp"], N)
        if wl.get("page"):
            # paged layout: the same entries in pages placed in a seeded shuffled order
            import numpy as np

            pg = wl["page"]
            npp = N // pg
            perm = np.random.default_rng(wl["seed"]).permutation(B * npp).astype(np.int32)
            src = torch.arange(B * N, device="cuda")
            dst = (torch.tensor(perm, device="cuda").view(B, npp).repeat_interleave(pg, dim=1) * pg
                   + torch.arange(N, device="cuda").remainder(pg)).view(-1)
            nope, rope, scale = (torch.empty_like(a) for a in (comp0.nope, comp0.rope, comp0.scale))
            nope[dst], rope[dst], scale[dst] = comp0.nope[src], comp0.rope[src], comp0.scale[src]
            comp0 = csa.KvCache(nope, rope, scale, N, pages=torch.tensor(perm, device="cuda").view(B, npp), page=pg)
        self.keys = [keys0] + [csa.IndexKeys(keys0.data.clone(), keys0.scale.clone(), N) for _ in range(replicas - 1)]
        self.comp = [comp0] + [csa.KvCache(comp0.nope.clone(), comp0.rope.clone(), comp0.scale.clone(), N,
                                           pages=comp0.pages, page=comp0.page) for _ in range(replicas - 1)]
        self.win = dev.kv_cache(wl["win"], W)
        self.q = dev.bf16(wl["q"])
        self.iq = dev.t(wl["iq"][0])
        self.iqs = dev.t(wl["iq"][1])
        self.w = dev.t(wl["w"])
        self.seq = dev.t(wl["seq"])
        self.pos = dev.t(wl["pos"])
        T = wl["T"]
        self.scores = torch.empty(T, wl["n_cols"], dtype=torch.float32, device="cuda")
        self.idx = torch.empty(T, wl["k"], dtype=torch.int32, device="cuda")
        self.out = torch.empty(T, wl["H"], wl["d"], dtype=torch.float32, device="cuda")
        self.lse = torch.empty(T, wl["H"], dtype=torch.float32, device="cuda")
        self.tws = csa.topk_workspace(T, wl["n_cols"], wl["k"])
        mws = csa.csa_mqa_workspace(T, wl["H"], wl["d"], wl["k"] + W)
        self.mws = torch.empty(max(mws, 1), dtype=torch.uint8, device="cuda")
        self.replicas = replicas

    def index(self, r):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        if wl.get("tokens", 1) > 1:
            # rows of a sequence adjacent: each sequence's keys streamed once for all its rows
            csa.csa_index_scores_grouped(self.iq, self.iqs, self.w, self.seq, self.pos, self.keys[r], wl["m"],
                                         wl["n_cols"], wl["tokens"], out=self.scores, topk_ws=self.tws)
        else:
            csa.csa_index_scores(self.iq, self.iqs, self.w, self.seq, self.pos, self.keys[r], wl["m"], wl["n_cols"],
                                 out=self.scores, topk_ws=self.tws)

    def topk(self, r):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        csa.csa_topk(self.scores, self.pos, wl["m"], wl["k"], out=self.idx, ws=self.tws, prepared=True)

    def attend(self, r):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        csa.csa_sparse_mqa(self.q, self.seq, self.pos, self.idx, wl["m"], self.comp[r], self.win, wl["W"],
                           wl["sm_scale"], wl["rope_base"], out=self.out, lse=self.lse, ws=self.mws)

    def step(self, i):
        r = i % self.replicas
        self.index(r)
        self.topk(r)
        self.attend(r)

    def capture(self, n_steps):
        """One HIP graph holding n_steps whole steps, replica sets rotating as in the eager
        loop (the library issues kernels only: no memset, no allocation).  Returns the
        eager step's (indices, out, lse), which every replay must reproduce."""
        import torch

        self.step(0)
        torch.cuda.synchronize()
        want = (self.idx.clone(), self.out.clone(), self.lse.clone())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(self.replicas):
                self.step(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(n_steps):
                self.step(i)
        torch.cuda.synchronize()
        return want

    def step_median(self, n):
        """Median duration of one step: one HIP graph per replica set, each holding a single
        step, replayed n times in rotation with an event pair around every replay."""
        import torch

        graphs = []
        for r in range(self.replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            graphs[i % self.replicas].replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
        del graphs
        return t[n // 2]

    def check(self, want, what):
        import torch

        torch.cuda.synchronize()
        assert torch.equal(self.idx, want[0]) and torch.equal(self.out, want[1]) and torch.equal(self.lse, want[2]), \
            f"{what}: differs from the eager step"


class PrefillSet:
    """Device tensors of the chunked-prefill workload (8,192 new tokens after a
    131,072-token context, one sequence, paired HCA layer).  One step compresses
    the new chunk (CSA m=4, HCA m'=128, both window rings), selects the top-1024
    entries per query with the fused indexer + top-k (every (query, entry) pair
    scored, no score rows written) and runs both attentions for all 8,192
    queries.  The older context is compressed in set-up."""

    def __init__(self, wl):
        import torch

        import compressed_sparse_long_compress_amd as csa
        from gen import device as dev

        self.wl = wl
        T, L0, m, mh, d, W, k = (wl[x] for x in ("T", "L0", "m", "m_hca", "d", "W", "k"))
        self.comp = csa.KvCache.empty(1, wl["comp_cap"], d)
        self.hca = csa.KvCache.empty(1, wl["hca_cap"], d)
        self.win = csa.KvCache.empty(1, wl["win_cap"], d)
        self.win_h = csa.KvCache.empty(1, wl["win_cap"], d)
        self.kv, self.lg = dev.bf16(wl["kv"]), dev.t(wl["logits"])
        self.kvh, self.lgh = dev.bf16(wl["kv_hca"]), dev.t(wl["logits_hca"])
        if L0 > 0:  # the older context (none for the small prefill case)
            csa.csa_compress(self.kv[:L0], self.lg[:L0], 0, m, 0, self.comp)
            csa.csa_compress(self.kvh[:L0], self.lgh[:L0], 0, mh, 0, self.hca)
            csa.csa_compress(self.kv[L0 - W:L0], self.lg[L0 - W:L0], L0 - W, 1, 0, self.win)
            csa.csa_compress(self.kvh[L0 - W:L0], self.lgh[L0 - W:L0], L0 - W, 1, 0, self.win_h)
        self.seq, self.pos = dev.t(wl["seq"]), dev.t(wl["pos"])
        self.iq, self.iqs, self.w = dev.t(wl["iq"][0]), dev.t(wl["iq"][1]), dev.t(wl["w"])
        self.keys = dev.index_keys(wl["keys"], wl["N"])
        self.q, self.qh = dev.bf16(wl["q"]), dev.bf16(wl["q_hca"])
        self.scores = torch.empty(T, wl["n_cols"], dtype=torch.float32, device="cuda")
        self.idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        self.out = torch.empty(T, wl["H"], d, dtype=torch.float32, device="cuda")
        self.lse = torch.empty(T, wl["H"], dtype=torch.float32, device="cuda")
        self.hout, self.hlse = torch.empty_like(self.out), torch.empty_like(self.lse)
        self.tws = csa.topk_workspace(T, wl["n_cols"], k)
        self.itk_ws = torch.empty(csa.csa_index_topk_workspace(T, wl["n_cols"], k, wl["h_i"]), dtype=torch.uint8,
                                  device="cuda")
        self.replicas = 1

    def step(self, i):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        L0, m, mh, W, k = wl["L0"], wl["m"], wl["m_hca"], wl["W"], wl["k"]
        csa.csa_compress(self.kv[L0:], self.lg[L0:], L0, m, 0, self.comp)
        csa.csa_compress(self.kv[L0:], self.lg[L0:], L0, 1, 0, self.win)
        csa.csa_compress(self.kvh[L0:], self.lgh[L0:], L0, mh, 0, self.hca)
        csa.csa_compress(self.kvh[L0:], self.lgh[L0:], L0, 1, 0, self.win_h)
        # indexer and top-k fused: no score rows are written
        csa.csa_index_topk(self.iq, self.iqs, self.w, self.seq, self.pos, self.keys, m, wl["n_cols"], k, out=self.idx,
                           ws=self.itk_ws)
        csa.csa_sparse_mqa(self.q, self.seq, self.pos, self.idx, m, self.comp, self.win, W, wl["sm_scale"],
                           out=self.out, lse=self.lse)
        csa.hca_dense_mqa(self.qh, self.seq, self.pos, mh, wl["hca_cap"], self.hca, self.win_h, W, wl["sm_scale"],
                          out=self.hout, lse=self.hlse)


class PrefillBwdSet(PrefillSet):
    """Gradient of both attention layers of the chunked-prefill step (training side): the
    forward runs once in set-up (its indices, out and lse are the backward's inputs), the
    output gradient is seeded N(0, 0.01^2).  One step clears the entry-gradient buffers and
    runs csa_mqa_bwd for the CSA layer (selected entries + window) and the HCA layer (every
    visible entry + window)."""

    def __init__(self, wl):
        import torch

        super().__init__(wl)
        self.step_fwd = super().step
        self.step_fwd(0)
        T, H, d = wl["T"], wl["H"], wl["d"]
        g = torch.Generator(device="cuda")
        g.manual_seed(107)
        self.dout = torch.randn(T, H, d, generator=g, device="cuda") * 0.01
        self.douth = torch.randn(T, H, d, generator=g, device="cuda") * 0.01
        self.dq = torch.empty(T, H, d, dtype=torch.float32, device="cuda")
        self.dqh = torch.empty_like(self.dq)
        self.dc = torch.zeros(self.comp.nope.shape[0], d, dtype=torch.float32, device="cuda")
        self.dw = torch.zeros(self.win.nope.shape[0], d, dtype=torch.float32, device="cuda")
        self.dch = torch.zeros(self.hca.nope.shape[0], d, dtype=torch.float32, device="cuda")
        self.dwh = torch.zeros(self.win_h.nope.shape[0], d, dtype=torch.float32, device="cuda")
        rows = max(self.dc.shape[0], self.dch.shape[0]) + max(self.dw.shape[0], self.dwh.shape[0])
        self.bws = torch.empty(rows * d * 8, dtype=torch.uint8, device="cuda")  # fixed-point entry gradients
        torch.cuda.synchronize()

    def bwd(self, layer):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        if layer == "csa":
            self.dc.zero_()
            self.dw.zero_()
            csa.csa_mqa_bwd(self.q, self.seq, self.pos, self.idx, wl["m"], self.comp, self.win, wl["W"],
                            wl["sm_scale"], self.out, self.lse, self.dout, dq=self.dq, dcomp=self.dc, dwin=self.dw,
                            ws=self.bws)
        else:
            self.dch.zero_()
            self.dwh.zero_()
            csa.csa_mqa_bwd(self.qh, self.seq, self.pos, None, wl["m_hca"], self.hca, self.win_h, wl["W"],
                            wl["sm_scale"], self.hout, self.hlse, self.douth, dq=self.dqh, dcomp=self.dch,
                            dwin=self.dwh, ws=self.bws)

    def step(self, i):
        self.bwd("csa")
        self.bwd("hca")

    def flops(self):
        """MFMA work of each layer: per (row, head, key) 2d each for S, dP, dq and 4d for the
        entry gradient (two products), 10 d in all."""
        import numpy as np

        wl = self.wl
        pos = np.asarray(wl["pos"], np.int64)
        win = np.minimum(pos + 1, wl["W"])
        keys_c = np.minimum(wl["k"], (pos + 1) // wl["m"]) + win
        keys_h = (pos + 1) // wl["m_hca"] + win
        per = wl["H"] * 10 * wl["d"]
        return {"csa": float(keys_c.sum()) * per, "hca": float(keys_h.sum()) * per}


class HcaSet:
    """HCA decode at 1M context: 8 sequences, 8,192 entries each (m'=128)."""

    def __init__(self, wl, replicas):
        import torch

        import compressed_sparse_long_compress_amd as csa
        from gen import device as dev

        self.wl = wl
        comp0 = dev.kv_cache(wl["comp"], wl["N"])
        self.comp = [comp0] + [csa.KvCache(comp0.nope.clone(), comp0.rope.clone(), comp0.scale.clone(), wl["N"])
                               for _ in range(replicas - 1)]
        self.win = dev.kv_cache(wl["win"], wl["W"])
        self.q, self.seq, self.pos = dev.bf16(wl["q"]), dev.t(wl["seq"]), dev.t(wl["pos"])
        self.out = torch.empty(wl["T"], wl["H"], wl["d"], dtype=torch.float32, device="cuda")
        self.lse = torch.empty(wl["T"], wl["H"], dtype=torch.float32, device="cuda")
        n = csa.csa_mqa_workspace(wl["T"], wl["H"], wl["d"], wl["N"] + wl["W"])
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        self.replicas = replicas

    def step(self, i):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        csa.hca_dense_mqa(self.q, self.seq, self.pos, wl["m"], wl["N"], self.comp[i % self.replicas], self.win,
                          wl["W"], wl["sm_scale"], wl["rope_base"], out=self.out, lse=self.lse, ws=self.ws)


class CompressSet:
    """One chunk's compression: entries with per-token weights, with per-channel weights,
    and MXFP4 index keys, each from 8,192 raw tokens (m=4)."""

    CALLS = ("compress", "compress_channel", "compress_index_keys")

    def __init__(self, wl):
        import torch

        import compressed_sparse_long_compress_amd as csa
        from gen import device as dev

        self.wl = wl
        T, d, d_i, m = wl["T"], wl["d"], wl["d_i"], wl["m"]
        self.kv, self.lg, self.lgc, self.ik = (dev.bf16(wl["kv"]), dev.t(wl["logits"]), dev.t(wl["logits_ch"]),
                                               dev.bf16(wl["ik"]))
        self.c1 = csa.KvCache.empty(1, T // m, d)
        self.c2 = csa.KvCache.empty(1, T // m, d)
        self.keys = csa.IndexKeys(torch.zeros(T // m, d_i // 2, dtype=torch.uint8, device="cuda"),
                                  torch.zeros(T // m, d_i // 32, dtype=torch.uint8, device="cuda"), T // m)
        self.replicas = 1

    def call(self, name):
        import compressed_sparse_long_compress_amd as csa

        m = self.wl["m"]
        if name == "compress":
            csa.csa_compress(self.kv, self.lg, 0, m, 0, self.c1)
        elif name == "compress_channel":
            csa.csa_compress_channel(self.kv, self.lgc, 0, m, 0, self.c2)
        else:
            csa.csa_compress_index_keys(self.ik, self.lg, 0, m, 0, self.keys)

    def step(self, i):
        for name in self.CALLS:
            self.call(name)

    def bytes_per_call(self):
        """Algorithmic HBM bytes of each call: inputs read once, outputs written once."""
        T, d, d_i, m = (self.wl[x] for x in ("T", "d", "d_i", "m"))
        n = T // m
        entry = (d - 64) + 64 * 2 + 4
        return {"compress": T * (2 * d + 4) + n * entry,
                "compress_channel": T * (2 * d + 4 * d) + n * entry,
                "compress_index_keys": T * (2 * d_i + 4) + n * (d_i // 2 + d_i // 32)}


def time_calls(ds, n):
    """Average duration of each call of a CompressSet: n back-to-back launches between one pair of events."""
    import torch

    res = {}
    for name in ds.CALLS:
        for _ in range(3):
            ds.call(name)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            ds.call(name)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n / 1e3
    return res


def time_steps(ds, steps, warmup, fn=None):
    import torch

    fn = fn or ds.step
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def time_kernels(ds, steps):
    """Per-call durations with events around each call, over a second timed region."""
    import torch

    names = ["index", "topk", "attend"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        r = i % ds.replicas
        ev[i][0].record()
        ds.index(r)
        ev[i][1].record()
        ds.topk(r)
        ev[i][2].record()
        ds.attend(r)
        ev[i][3].record()
    torch.cuda.synchronize()
    out = {}
    for j, n in enumerate(names):
        out[n] = sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps / 1e3
    return out


def time_index_launches(ds, n):
    """Average duration of the indexer kernel: n back-to-back launches (replicas
    rotating, so each reads keys that are not in the caches) between one pair
    of events on the launch stream, divided by n.  Launches queued back to back
    start as the previous one ends, so this tracks the kernel's own duration
    (what rocprofv3 --kernel-trace reports) rather than one dispatch latency
    per call."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for i in range(ds.replicas):
        ds.index(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        ds.index(i % ds.replicas)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n / 1e3


def measure_copy_gbs(n=20):
    """Bandwidth of a plain device-to-device copy on this GPU (1 GiB read + 1 GiB written per
    copy, torch's copy kernel), as context for the HBM roofline: what a streaming kernel
    reaches here, against the 8 TB/s published peak."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / n
    del a, b
    return 2.0 * (1 << 30) / sec / 1e9


def measure_mfma_tflops(n=5):
    """The matrix-core rate this GPU sustains for the path's MFMA shapes (the library's probe:
    MFMAs back to back, no memory traffic), best of n launches: context for the MFMA
    fractions, which stay against the published peaks."""
    import torch

    import compressed_sparse_long_compress_amd as csa

    blocks = 1024  # four workgroups of four waves per CU
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    res = {}
    for name, kind, iters in (("fp16", 0, 10000), ("mxfp4", 1, 5000)):
        csa.mfma_probe(kind, blocks, 100, sink)
        best = None
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fl = csa.mfma_probe(kind, blocks, iters, sink)
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 1e3
            best = sec if best is None or sec < best else best
        res[name] = fl / best / 1e12
    del sink
    return res


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


ORACLE_SMALL_ONE_THREAD = r"""
import sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle
from gen import configs
wl = configs.named("prefill_small")
m, k, W = wl["m"], wl["k"], wl["W"]
t0 = time.perf_counter()
comp = oracle.compress(wl["kv"], wl["logits"], 0, m)
win = oracle.compress(wl["kv"], wl["logits"], 0, 1)
hca = oracle.compress(wl["kv"], wl["logits"], 0, wl["m_hca"])
sc = oracle.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0], wl["keys"][1],
                         wl["N"], m, wl["n_cols"]).astype(np.float32)
idx = oracle.topk(sc, wl["pos"], m, k)
oracle.attend(wl["q"], wl["seq"], wl["pos"], comp, wl["comp_cap"], win, wl["T"], W, m, wl["sm_scale"], idx=idx)
oracle.attend(wl["q"], wl["seq"], wl["pos"], hca, wl["hca_cap"], win, wl["T"], W, wl["m_hca"], wl["sm_scale"])
print(time.perf_counter() - t0)
"""


def oracle_small_one_thread():
    """Seconds the fp64 oracle takes, on one thread (a child process with OMP_NUM_THREADS=1),
    for the whole small prefill case: compress (m=4, m=1, m'=128), index scores, top-k and
    both attentions over 2,048 query rows."""
    import subprocess

    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", ORACLE_SMALL_ONE_THREAD, ROOT], env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:
        raise RuntimeError("single-thread oracle run failed: " + r.stderr[-500:])
    return float(r.stdout.strip().splitlines()[-1])


def cpu_baseline(wl):
    """The fp64 oracle (as written, untuned) on the same batch: index scores,
    top-k and sparse attention for every query row of the workload, repeated
    for about 10 s.  The oracle's OpenMP loops run over (row, column chunk) for
    the scores and over rows elsewhere, with every host core."""
    import numpy as np

    import oracle

    T = wl["T"]
    reps = 0
    t0 = time.perf_counter()
    while reps < 200 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        sc = oracle.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0],
                                 wl["keys"][1], wl["N"], wl["m"], wl["n_cols"]).astype(np.float32)
        idx = oracle.topk(sc, wl["pos"], wl["m"], wl["k"])
        oracle.attend(wl["q"], wl["seq"], wl["pos"], wl["comp"], wl["N"], wl["win"], wl["W"], wl["W"], wl["m"],
                      wl["sm_scale"], wl["rope_base"], idx=idx)
        reps += 1
    dt = time.perf_counter() - t0
    ncpu = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", ncpu))
    return {"value": T * reps / dt, "unit": "queries/s", "cores": min(threads, ncpu), "host_cpus": ncpu,
            "cpu_model": cpu_model(), "kind": "oracle",
            "small_prefill_one_thread_s": oracle_small_one_thread(),
            "sample": f"all {T} query rows of the batch (full 1M-context rows), {reps} passes, {dt:.1f} s wall; "
                      f"OpenMP threads {min(threads, ncpu)} of {ncpu} host CPUs"}


def time_back_to_back(fn, n):
    """Average duration of n launches of fn queued back to back between one pair of events."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n / 1e3


MXFP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 (fp4) MFMA
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA


def prefill_flops(wl):
    """Algorithmic work of the chunked prefill: indexer 2 h_i d_i flop per visible
    (query, entry) pair; attention 4 d flop per (row, head, key) (QK and PV) over
    each row's key set (selected entries + window; HCA: every visible entry + window)."""
    import numpy as np

    pos = np.asarray(wl["pos"], np.int64)
    nv = np.minimum((pos + 1) // wl["m"], wl["n_cols"])
    win = np.minimum(pos + 1, wl["W"])
    per_key = wl["H"] * 4 * wl["d"]
    return {"index": float(nv.sum()) * 2 * wl["h_i"] * wl["d_i"],
            "sparse_mqa": float((np.minimum(wl["k"], nv) + win).sum()) * per_key,
            "hca_mqa": float(((pos + 1) // wl["m_hca"] + win).sum()) * per_key}


def prefill_measure(steps):
    """The chunked-prefill workload: whole steps (compress the chunk, fused index + top-k, both
    attentions) and back-to-back launches of each call: the fused selection, the indexer alone
    (score rows written, against the MXFP4 peak), the top-k on those rows, both attentions
    (against the fp16 peak)."""
    import torch

    import compressed_sparse_long_compress_amd as csa
    from gen import configs

    wl = configs.named("prefill_chunk")
    ds = PrefillSet(wl)
    n = max(steps, 3)
    sec, _ = time_steps(ds, n, 2)
    m, k, W = wl["m"], wl["k"], wl["W"]
    t_index = time_back_to_back(lambda: csa.csa_index_scores(ds.iq, ds.iqs, ds.w, ds.seq, ds.pos, ds.keys, m,
                                                              wl["n_cols"], out=ds.scores), n)
    t_topk = time_back_to_back(lambda: csa.csa_topk(ds.scores, ds.pos, m, k, out=ds.idx, ws=ds.tws), n)
    t_fused = time_back_to_back(lambda: csa.csa_index_topk(ds.iq, ds.iqs, ds.w, ds.seq, ds.pos, ds.keys, m,
                                                           wl["n_cols"], k, out=ds.idx, ws=ds.itk_ws), n)
    t_sparse = time_back_to_back(lambda: csa.csa_sparse_mqa(ds.q, ds.seq, ds.pos, ds.idx, m, ds.comp, ds.win, W,
                                                            wl["sm_scale"], out=ds.out, lse=ds.lse), n)
    t_hca = time_back_to_back(lambda: csa.hca_dense_mqa(ds.qh, ds.seq, ds.pos, wl["m_hca"], wl["hca_cap"], ds.hca,
                                                        ds.win_h, W, wl["sm_scale"], out=ds.hout, lse=ds.hlse), n)
    fl = prefill_flops(wl)
    mm = measure_mfma_tflops()
    res = {"workload": "prefill_chunk", "tokens": wl["T"], "context": wl["total"],
           "tokens_per_s": wl["T"] * n / sec, "ms_per_step": sec / n * 1e3, "steps": n,
           "per_call_ms": {"index_topk_fused": t_fused * 1e3, "index": t_index * 1e3, "topk": t_topk * 1e3,
                           "sparse_mqa": t_sparse * 1e3, "hca_mqa": t_hca * 1e3},
           "index_topk_fused": {"calls": "csa_index_topk (sample, threshold, emit, pick)",
                                "ms": t_fused * 1e3, "split_ms": (t_index + t_topk) * 1e3,
                                "mxfp4_tflops": fl["index"] / t_fused / 1e12},
           "index": {"kernel": "k_index_gemm<128, 8>", "bound": "mfma", "flops": fl["index"],
                     "achieved": fl["index"] / t_index / 1e12, "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": fl["index"] / t_index / 1e12 / MXFP4_PEAK_TFLOPS},
           "sparse_mqa": {"kernel": "k_mqa64ws<512, false>", "bound": "mfma", "flops": fl["sparse_mqa"],
                          "achieved": fl["sparse_mqa"] / t_sparse / 1e12, "peak": FP16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": fl["sparse_mqa"] / t_sparse / 1e12 / FP16_PEAK_TFLOPS},
           "hca_mqa": {"kernel": "k_mqa64ws<512, false>", "bound": "mfma", "flops": fl["hca_mqa"],
                       "achieved": fl["hca_mqa"] / t_hca / 1e12, "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": fl["hca_mqa"] / t_hca / 1e12 / FP16_PEAK_TFLOPS},
           "mfma_measured_tflops": mm}
    res["index"]["frac_of_measured"] = res["index"]["achieved"] / mm["mxfp4"]
    for key in ("sparse_mqa", "hca_mqa"):
        res[key]["frac_of_measured"] = res[key]["achieved"] / mm["fp16"]
    del ds
    return res


def run_workload(name, steps, warmup):
    """Time one named workload; returns (wl, dataset, seconds for `steps` steps)."""
    from gen import configs

    wl = configs.named("prefill_chunk" if name == "prefill_chunk_bwd" else name)
    if name.startswith("csa_decode"):
        ds = DecodeSet(wl, replicas=8)
    elif name == "compress_chunk":
        ds = CompressSet(wl)
    elif name == "hca_decode_1m":
        ds = HcaSet(wl, replicas=8)
    elif name == "prefill_chunk_bwd":
        ds = PrefillBwdSet(wl)
    else:
        ds = PrefillSet(wl)
    sec, _ = time_steps(ds, steps, warmup)
    return wl, ds, sec


def secondary(steps, warmup):
    """The other decode workloads (opt-in): 1M CSA decode with two query rows per sequence,
    64K CSA decode, 1M HCA decode."""
    res = {}
    for name in ("csa_decode_1m_mtp2", "csa_decode_64k", "hca_decode_1m"):
        wl, ds, sec = run_workload(name, steps, warmup)
        T, N, W, H, d = (wl[x] for x in ("T", "N", "W", "H", "d"))
        entry = (d - 64) + 64 * 2 + 4
        if wl["kind"] == "hca_decode":
            # every visible entry and the window per query, the bf16 query and fp32 output; 4 d flop
            # per (query, head, key)
            step_bytes = T * ((N + W) * entry + H * d * 2 + H * d * 4)
            flops = T * H * (N + W) * 4 * d
        else:
            # the keys once per sequence (rows of a sequence share them), each row's query, gathered
            # entries, query and output
            B, h_i, d_i, k = wl["B"], wl["h_i"], wl["d_i"], wl["k"]
            key = d_i // 2 + d_i // 32
            step_bytes = B * N * key + T * (h_i * (key + 4) + (k + W) * entry + H * d * 2 + H * d * 4)
            flops = None
        gbs = step_bytes * steps / sec / 1e9
        res[name] = {"queries_per_s": T * steps / sec, "ms_per_step": sec / steps * 1e3, "step_bytes": step_bytes,
                     "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        if flops is not None:
            tf = flops * steps / sec / 1e12
            res[name].update({"mfma_tflops": tf, "mfma_frac": tf / FP16_PEAK_TFLOPS})
        del ds
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also time the other workloads (secondary object)")
    ap.add_argument("--workload", default="csa_decode_1m",
                    choices=["csa_decode_1m", "csa_decode_1m_mtp2", "csa_decode_1m_paged", "csa_decode_64k",
                             "prefill_chunk_bwd",
                             "hca_decode_1m", "prefill_chunk", "prefill_small", "compress_chunk"],
                    help="time only this workload and print its line (profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill object")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 device copies of 256 MiB (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the CSA/HCA path here is built and timed on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_long_compress_amd as csa  # noqa: F401  (fails loudly without libcsa.so)
    from gen import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": a.numel(), "copies": 5}))
        return
    if args.workload == "compress_chunk":
        wl, ds, sec = run_workload(args.workload, args.steps, args.warmup)
        calls = time_calls(ds, args.steps)
        by = ds.bytes_per_call()
        print(json.dumps({"workload": args.workload, "value": wl["T"] * args.steps / sec, "unit": "tokens/s",
                          "ms_per_step": sec / args.steps * 1e3, "steps": args.steps,
                          "per_call_us": {k: v * 1e6 for k, v in calls.items()},
                          "hbm_gbs": {k: by[k] / calls[k] / 1e9 for k in calls}}))
        return
    if args.workload == "prefill_chunk_bwd":
        wl, ds, sec = run_workload(args.workload, args.steps, args.warmup)
        fl = ds.flops()
        per = {}
        for layer in ("csa", "hca"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                ds.bwd(layer)
            e1.record()
            torch.cuda.synchronize()
            per[layer] = e0.elapsed_time(e1) / args.steps / 1e3
        tot = sum(fl.values())
        print(json.dumps({"workload": args.workload, "value": wl["T"] * args.steps / sec, "unit": "tokens/s",
                          "ms_per_step": sec / args.steps * 1e3, "steps": args.steps, "dtype": "f16 mfma, 64-bit fixed-point entry gradients",
                          "per_layer_ms": {k: v * 1e3 for k, v in per.items()},
                          "tflops": {k: fl[k] / per[k] / 1e12 for k in per},
                          "mfma": {"achieved": tot / (sec / args.steps) / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                                   "frac": tot / (sec / args.steps) / 1e12 / 2500.0}}))
        return
    if args.workload == "prefill_chunk":
        print(json.dumps(prefill_measure(args.steps)), flush=True)
        return
    if args.workload != "csa_decode_1m":
        wl, ds, sec = run_workload(args.workload, args.steps, args.warmup)
        unit = "tokens/s" if args.workload.startswith("prefill") else "queries/s"
        print(json.dumps({"workload": args.workload, "value": wl["T"] * args.steps / sec, "unit": unit,
                          "ms_per_step": sec / args.steps * 1e3, "steps": args.steps}))
        return
    t0 = time.perf_counter()
    wl = configs.named("csa_decode_1m")
    log(f"generated csa_decode_1m inputs in {time.perf_counter() - t0:.1f} s")
    ds = DecodeSet(wl, replicas=8)
    log("uploaded 8 replica sets")
    want = ds.capture(args.steps)
    log(f"captured the {args.steps} timed steps as one HIP graph")
    eager_sec, _ = time_steps(ds, args.steps, args.warmup)
    ds.check(want, "eager steps")
    for i in range(args.warmup):
        ds.step(i)
    ds.idx.fill_(-3)
    ds.out.zero_()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    ds.graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sec = e0.elapsed_time(e1) / 1e3
    ds.check(want, "graph replay")
    log(f"timed {args.steps} steps as one graph replay: {sec * 1e3 / args.steps:.4f} ms/step "
        f"(eager {eager_sec * 1e3 / args.steps:.4f}, host wall {wall:.4f} s); the replay's outputs equal the eager step")
    kern = time_kernels(ds, args.steps)
    log("per-call ms: " + ", ".join(f"{k} {v * 1e3:.4f}" for k, v in kern.items()))
    idx_sec = time_index_launches(ds, args.steps)
    log(f"indexer kernel, back-to-back launches: {idx_sec * 1e6:.2f} us")
    med_sec = ds.step_median(max(args.steps, 100))
    log(f"one-step graphs, median of {max(args.steps, 100)} replays: {med_sec * 1e3:.4f} ms/step")

    B, N, h_i, d_i, k, W, H, d = (wl[x] for x in ("B", "N", "h_i", "d_i", "k", "W", "H", "d"))
    qps = B * args.steps / sec
    idx_bytes = B * index_bytes_per_query(N, h_i, d_i)
    achieved = idx_bytes / idx_sec / 1e9
    step_bytes = B * step_bytes_per_query(N, h_i, d_i, k, W, H, d)
    result = {
        "metric": "CSA decode queries/s + HBM GB/s % at 1M ctx; prefill tokens/s; top-k exact",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+fp16",
        "data": "synthetic (seeded N(0,1) before quantisation, 5% planted index keys)",
        "config": {"workload": "csa_decode_1m", "batch": B, "context": wl["L"], "entries_per_seq": N, "m": wl["m"],
                   "k": k, "window": W, "heads": H, "head_dim": d, "indexer": f"{h_i}x{d_i} mxfp4",
                   "replicas": ds.replicas, "timing": "the timed steps replayed as one HIP graph (replica sets rotated)"},
        "eager_ms_per_step": eager_sec / args.steps * 1e3,
        "median_ms_per_step": med_sec * 1e3,  # one step per graph, events around each replay
        "step_bytes": step_bytes,
        "step_hbm_gbs": step_bytes * args.steps / sec / 1e9,
        "step_hbm_frac": step_bytes * args.steps / sec / 1e9 / HBM_PEAK_GBS,
        "per_call_us": {kk: v * 1e6 for kk, v in kern.items()},
        "roofline": {"kernel": "k_index_rows<128, 8>", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": index_traffic(),
                     "bytes_per_launch": idx_bytes, "excess_bytes_per_launch": B * index_excess_bytes_per_query(N),
                     "kernel_us": idx_sec * 1e6},
    }
    del ds
    copy_gbs = measure_copy_gbs()
    result["roofline"]["copy_gbs_measured"] = copy_gbs
    result["roofline"]["frac_of_copy"] = achieved / copy_gbs
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write); the indexer reaches {achieved / copy_gbs:.2f} of it")
    if not args.no_prefill:
        log("timing the chunked prefill (8,192 tokens after 131,072)")
        result["prefill"] = prefill_measure(max(args.steps // 4, 3))
        log(f"prefill: {result['prefill']['tokens_per_s']:.4g} tokens/s")
    if args.all:
        result["secondary"] = secondary(max(args.steps // 2, 20), args.warmup)
    if not args.no_cpu:
        log("timing the CPU oracle on the same batch")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: CSA decode at 1M context on one MI355X (libcsa HIP kernels).

One step = the CSA decode hot path for a batch of 4 sequences, each with a
1,048,576-token context (262,144 compressed entries at m=4):
    csa_index_scores (MXFP4 indexer over every entry; it also builds the
                      first radix histogram of the selection)
 -> csa_topk (k = 1024)
 -> csa_sparse_mqa (64 query heads over the 1024 selected entries + a
    128-token window, d = 512).
Inputs are seeded synthetic tensors resident in HBM before timing starts;
8 replica sets of the keys and the compressed cache (~5.5 GB) rotate step by
step so the 256 MB Infinity Cache cannot serve a step from the previous one.

Prints ONE JSON line: queries/s for the batch, a roofline object for the
dominant kernel (the indexer, bound by HBM), and the fp64 CPU oracle timed
on the same batch as a reported baseline.

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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def index_bytes_per_query(N, h_i, d_i):
    """Algorithmic HBM bytes of csa_index_scores per query row: every MXFP4 key
    (d_i/2 data + d_i/32 scale bytes), the query (h_i keys' worth + fp32
    weights), and the fp32 score row written."""
    key = d_i // 2 + d_i // 32
    return N * key + h_i * key + h_i * 4 + N * 4


def step_bytes_per_query(N, h_i, d_i, k, W, H, d):
    """Algorithmic HBM bytes of the whole decode step per query: indexer bytes,
    the score row read back by top-k, k indices, the gathered entries
    (k + W) x (d-64 + 128 + 4) B, the bf16 query and fp32 output + lse."""
    entry = (d - 64) + 64 * 2 + 4
    return (index_bytes_per_query(N, h_i, d_i) + N * 4 + k * 4 * 2 + (k + W) * entry + H * d * 2 + H * d * 4
            + H * 4)


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
        self.keys = [keys0] + [csa.IndexKeys(keys0.data.clone(), keys0.scale.clone(), N) for _ in range(replicas - 1)]
        self.comp = [comp0] + [csa.KvCache(comp0.nope.clone(), comp0.rope.clone(), comp0.scale.clone(), N)
                               for _ in range(replicas - 1)]
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
        csa.csa_index_scores(self.iq, self.iqs, self.w, self.seq, self.pos, self.keys[r], wl["m"], wl["n_cols"],
                             out=self.scores, topk_ws=self.tws)

    def topk(self, r):
        import compressed_sparse_long_compress_amd as csa

        wl = self.wl
        csa.csa_topk(self.scores, self.pos, wl["m"], wl["k"], out=self.idx, ws=self.tws, hist_ready=True)

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


def time_steps(ds, steps, warmup):
    import torch

    for i in range(warmup):
        ds.step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    t0 = time.perf_counter()
    for i in range(steps):
        ds.step(i)
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


def cpu_baseline(wl):
    """The fp64 oracle (as written, untuned) on the same batch: index scores,
    top-k and sparse attention for every query row of the workload."""
    import numpy as np

    import oracle

    T = wl["T"]
    t0 = time.perf_counter()
    sc = oracle.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0], wl["keys"][1],
                             wl["N"], wl["m"], wl["n_cols"]).astype(np.float32)
    idx = oracle.topk(sc, wl["pos"], wl["m"], wl["k"])
    oracle.attend(wl["q"], wl["seq"], wl["pos"], wl["comp"], wl["N"], wl["win"], wl["W"], wl["W"], wl["m"],
                  wl["sm_scale"], wl["rope_base"], idx=idx)
    dt = time.perf_counter() - t0
    cores = min(T, os.cpu_count() or 1)  # the oracle parallelises over query rows
    return {"value": T / dt, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"all {T} query rows of the batch (full 1M-context rows), {dt:.1f} s wall"}


def secondary(steps, warmup):
    """Other workloads (opt-in): 64K CSA decode, 1M HCA decode, chunked prefill."""
    import torch

    import compressed_sparse_long_compress_amd as csa
    from gen import configs
    from gen import device as dev

    res = {}
    wl = configs.named("csa_decode_64k")
    ds = DecodeSet(wl, replicas=8)
    sec, _ = time_steps(ds, steps, warmup)
    res["csa_decode_64k"] = {"queries_per_s": wl["B"] * steps / sec, "ms_per_step": sec / steps * 1e3}
    del ds
    wl = configs.named("hca_decode_1m")
    comp = [dev.kv_cache(wl["comp"], wl["N"]) for _ in range(8)]
    win, q, seq, pos = dev.kv_cache(wl["win"], wl["W"]), dev.bf16(wl["q"]), dev.t(wl["seq"]), dev.t(wl["pos"])
    ws = torch.empty(max(csa.csa_mqa_workspace(wl["T"], wl["H"], wl["d"], wl["N"] + wl["W"]), 1), dtype=torch.uint8,
                     device="cuda")

    def hstep(i):
        csa.hca_dense_mqa(q, seq, pos, wl["m"], wl["N"], comp[i % 8], win, wl["W"], wl["sm_scale"], ws=ws)

    for i in range(warmup):
        hstep(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        hstep(i)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    res["hca_decode_1m"] = {"queries_per_s": wl["B"] * steps / sec, "ms_per_step": sec / steps * 1e3}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also time the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the CSA/HCA path here is built and timed on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_long_compress_amd as csa  # noqa: F401  (fails loudly without libcsa.so)
    from gen import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    t0 = time.perf_counter()
    wl = configs.named("csa_decode_1m")
    log(f"generated csa_decode_1m inputs in {time.perf_counter() - t0:.1f} s")
    ds = DecodeSet(wl, replicas=8)
    log("uploaded 8 replica sets")
    sec, wall = time_steps(ds, args.steps, args.warmup)
    log(f"timed {args.steps} steps: {sec * 1e3 / args.steps:.3f} ms/step (wall {wall:.3f} s)")
    kern = time_kernels(ds, args.steps)
    log("per-call ms: " + ", ".join(f"{k} {v * 1e3:.4f}" for k, v in kern.items()))

    B, N, h_i, d_i, k, W, H, d = (wl[x] for x in ("B", "N", "h_i", "d_i", "k", "W", "H", "d"))
    qps = B * args.steps / sec
    idx_bytes = B * index_bytes_per_query(N, h_i, d_i)
    achieved = idx_bytes / kern["index"] / 1e9
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
        "dtype": "mxfp4+bf16",
        "data": "synthetic (seeded N(0,1) before quantisation, 5% planted index keys)",
        "config": {"workload": "csa_decode_1m", "batch": B, "context": wl["L"], "entries_per_seq": N, "m": wl["m"],
                   "k": k, "window": W, "heads": H, "head_dim": d, "indexer": f"{h_i}x{d_i} mxfp4",
                   "replicas": ds.replicas},
        "step_hbm_gbs": step_bytes * args.steps / sec / 1e9,
        "step_hbm_frac": step_bytes * args.steps / sec / 1e9 / HBM_PEAK_GBS,
        "per_call_us": {kk: v * 1e6 for kk, v in kern.items()},
        "roofline": {"kernel": "k_index_rows<128>", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": idx_bytes},
    }
    if args.all:
        result["secondary"] = secondary(max(args.steps // 2, 20), args.warmup)
    if not args.no_cpu:
        log("timing the CPU oracle on the same batch")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Workload builders: seeded synthetic inputs with the shapes of the CSA / HCA
settings the pages describe (m=4, top-k 1024, window 128, m'=128, RoPE on the
last 64 dims, bf16 RoPE dims + FP8 E4M3 rest, FP4 indexer), at context
lengths up to one million tokens.

Every builder returns a plain ``dict`` of numpy arrays and integers.  Values
are N(0,1) before encoding; indexer head weights are 2^-u, u in {0,1,2};
RoPE base 10000; softmax scale 1/sqrt(d).  One RNG stream per tensor, so the
same seed always yields the same bytes whatever else is built.

Named workloads (seeds 101..105):
  prefill_small  T=2048 prefill, B=1, d=128, 16 heads, indexer 4x64, k=64
  csa_decode_64k B=32, L=65,536 (16,384 entries), 64 heads, d=512, k=1024
  hca_decode_1m  B=8,  L=1,048,576 at m'=128 (8,192 entries)
  csa_decode_1m  B=4,  L=1,048,576 (262,144 entries), 5% planted index keys
  csa_decode_1m_mtp2  the same cache, two query rows per sequence (positions L-2, L-1)
  csa_decode_1m_paged the same workload with the compressed cache in shuffled 1,024-entry pages
  prefill_chunk  8,192 new tokens after a 131,072-token context (CSA + HCA)
  compress_chunk 8,192 raw tokens (d=512) and index-key tokens (d_i=128), seed 106
"""
import math

import numpy as np

from . import entries, mxfp4, normal_bf16, normal_f32, pow2_weights

ROPE_BASE = 10000.0


def csa_decode(B, L, m=4, H=64, d=512, h_i=8, d_i=128, k=1024, W=128, plant_frac=0.0, seed=102, n_cols=None,
               tokens=1):
    """Decode over a pre-built cache: `tokens` query rows per sequence at the
    positions L-tokens .. L-1 (tokens > 1: a multi-token step, e.g. the target
    pass over draft tokens, rows of a sequence adjacent), T = B * tokens."""
    N = L // m
    dn = d - 64
    T = B * tokens
    wl = dict(kind="csa_decode", B=B, L=L, m=m, H=H, d=d, h_i=h_i, d_i=d_i, k=k, W=W, N=N, seed=seed,
              rope_base=ROPE_BASE, sm_scale=1.0 / math.sqrt(d), T=T, n_cols=N if n_cols is None else n_cols,
              comp_cap=N, win_cap=W, tokens=tokens)
    wl["pos"] = np.tile(np.arange(L - tokens, L, dtype=np.int64), B)
    wl["seq"] = np.repeat(np.arange(B, dtype=np.int32), tokens)
    wl["comp"] = entries(seed, 20, B * N, dn)
    wl["win"] = entries(seed, 21, B * W, dn)
    kd, ks, planted = mxfp4(seed, 22, B * N, d_i, plant_frac=plant_frac)
    wl["keys"] = (kd, ks)
    wl["planted"] = planted
    wl["q"] = normal_bf16(seed, 23, (T, H, d))
    qd, qs, _ = mxfp4(seed, 24, T * h_i, d_i)
    wl["iq"] = (qd.reshape(T, h_i, d_i // 2), qs.reshape(T, h_i, d_i // 32))
    wl["w"] = pow2_weights(seed, 25, (T, h_i))
    return wl


def hca_decode(B, L, m=128, H=64, d=512, W=128, seed=103):
    """One decode query per sequence over all L/m compressed entries + window."""
    N = L // m
    dn = d - 64
    wl = dict(kind="hca_decode", B=B, L=L, m=m, H=H, d=d, W=W, N=N, seed=seed, rope_base=ROPE_BASE,
              sm_scale=1.0 / math.sqrt(d), T=B, comp_cap=N, win_cap=W)
    wl["pos"] = np.full(B, L - 1, dtype=np.int64)
    wl["seq"] = np.arange(B, dtype=np.int32)
    wl["comp"] = entries(seed, 30, B * N, dn)
    wl["win"] = entries(seed, 31, B * W, dn)
    wl["q"] = normal_bf16(seed, 33, (B, H, d))
    return wl


def prefill(T, L0=0, m=4, m_hca=128, H=64, d=512, h_i=8, d_i=128, k=1024, W=128, seed=105, hca=True):
    """Causal prefill of T new tokens after L0 context tokens (batch 1).

    Raw bf16 tokens and per-token compression logits for the whole context
    (CSA layer, and an independent HCA layer when ``hca``), queries for the
    new tokens, MXFP4 indexer queries, head weights, and MXFP4 index keys for
    every compressed entry.  The window ring holds raw tokens at slot p % cap
    with cap = T + W (every query of the chunk sees its whole window).
    """
    total = L0 + T
    assert L0 % m == 0 and T % m == 0 and L0 % m_hca == 0 and T % m_hca == 0
    N = total // m
    wl = dict(kind="prefill", T=T, L0=L0, total=total, m=m, m_hca=m_hca, H=H, d=d, h_i=h_i, d_i=d_i, k=k, W=W,
              N=N, N_hca=total // m_hca, seed=seed, rope_base=ROPE_BASE, sm_scale=1.0 / math.sqrt(d),
              n_cols=N, comp_cap=N, hca_cap=total // m_hca, win_cap=T + W)
    wl["pos"] = (L0 + np.arange(T)).astype(np.int64)
    wl["seq"] = np.zeros(T, dtype=np.int32)
    wl["kv"] = normal_bf16(seed, 1, (total, d))
    wl["logits"] = normal_f32(seed, 2, (total,))
    wl["q"] = normal_bf16(seed, 5, (T, H, d))
    qd, qs, _ = mxfp4(seed, 7, T * h_i, d_i)
    wl["iq"] = (qd.reshape(T, h_i, d_i // 2), qs.reshape(T, h_i, d_i // 32))
    wl["w"] = pow2_weights(seed, 8, (T, h_i))
    kd, ks, _ = mxfp4(seed, 9, N, d_i)
    wl["keys"] = (kd, ks)
    if hca:
        wl["kv_hca"] = normal_bf16(seed, 3, (total, d))
        wl["logits_hca"] = normal_f32(seed, 4, (total,))
        wl["q_hca"] = normal_bf16(seed, 6, (T, H, d))
    return wl


def compress_chunk(T=8192, d=512, d_i=128, m=4, seed=106):
    """Raw inputs of one chunk's compression: bf16 tokens, one logit per token and one
    per (token, channel), and raw bf16 index-key tokens."""
    wl = dict(kind="compress", T=T, d=d, d_i=d_i, m=m, seed=seed, rope_base=ROPE_BASE)
    wl["kv"] = normal_bf16(seed, 1, (T, d))
    wl["logits"] = normal_f32(seed, 2, (T,))
    wl["logits_ch"] = normal_f32(seed, 3, (T, d))
    wl["ik"] = normal_bf16(seed, 4, (T, d_i))
    return wl


def named(name, **over):
    """The five named workloads at full size (keyword overrides allowed)."""
    if name == "prefill_small":
        kw = dict(T=2048, L0=0, m=4, m_hca=128, H=16, d=128, h_i=4, d_i=64, k=64, W=128, seed=101)
        kw.update(over)
        return prefill(**kw)
    if name == "csa_decode_64k":
        kw = dict(B=32, L=65536, seed=102)
        kw.update(over)
        return csa_decode(**kw)
    if name == "hca_decode_1m":
        kw = dict(B=8, L=1 << 20, seed=103)
        kw.update(over)
        return hca_decode(**kw)
    if name == "csa_decode_1m":
        kw = dict(B=4, L=1 << 20, plant_frac=0.05, seed=104)
        kw.update(over)
        return csa_decode(**kw)
    if name == "compress_chunk":
        return compress_chunk(**over)
    if name == "csa_decode_1m_paged":
        kw = dict(B=4, L=1 << 20, plant_frac=0.05, seed=104)
        kw.update(over)
        wl = csa_decode(**kw)
        wl["page"] = 1024  # compressed entries per page; pages in a seeded shuffled order
        return wl
    if name == "csa_decode_1m_mtp2":
        kw = dict(B=4, L=1 << 20, plant_frac=0.05, seed=104, tokens=2)
        kw.update(over)
        return csa_decode(**kw)
    if name == "prefill_chunk":
        kw = dict(T=8192, L0=131072, seed=105)
        kw.update(over)
        return prefill(**kw)
    raise KeyError(name)

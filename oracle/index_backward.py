"""ORACLE — fp64 gradient of the lightning-indexer scores (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the library never does.

The pages warm the lightning indexer up before sparse training and train its
QK path in FP4 with quantisation awareness ([xmsumi] § 预训练：32T Token 炼就基座;
[hortopato] training section); both need the gradient of the indexer scores.
The pages give no formula, so this module writes out the plain derivative of
the forward that ``oracle.c`` computes ([xmsumi] § CSA: the indexer scores
every compressed entry per query token; reading: score = sum_h w_h ReLU(<q_h, k_j>)
over MXFP4-dequantised vectors).

Forward, per query row t and visible column j:
    dot_h = <q_h, k_j>,  score = sum_h w_h max(0, dot_h)
Given G = dL/dscore at the selected columns (idx[t][a], G[t][a]; entries with
idx < 0 or j >= (pos+1)/m are ignored), with the ReLU's derivative taken as 0
at 0 (a subgradient):
    dq_h   += G w_h [dot_h > 0] k_j
    dw_h   += G max(0, dot_h)
    dk_j   += G sum_h w_h [dot_h > 0] q_h      (summed over every row selecting j)
Gradients are with respect to the dequantised values (quantisation passes the
gradient straight through; the caller maps it further).

Pins (tests/test_oracle_pins.py): ``index_scores_f64`` reproduces
oracle.index_scores; central differences of it match every gradient away from
the kink; closed forms for one head and one key; scaling laws.
"""
import numpy as np

from . import e2m1_to_f64, e8m0_to_f64

_E2M1 = None


def dequant_mxfp4(data, scale):
    """MXFP4 rows -> fp64 [rows, d]: element 2i in the low nibble, one E8M0 scale per 32."""
    global _E2M1
    if _E2M1 is None:
        _E2M1 = np.array([e2m1_to_f64(n) for n in range(16)], np.float64)
    data = np.asarray(data, np.uint8)
    scale = np.asarray(scale, np.uint8)
    lead = data.shape[:-1]
    d = data.shape[-1] * 2
    nib = np.empty(lead + (d,), np.uint8)
    nib[..., 0::2] = data & 15
    nib[..., 1::2] = data >> 4
    e8 = np.array([e8m0_to_f64(b) for b in range(256)], np.float64)
    return _E2M1[nib] * np.repeat(e8[scale], 32, axis=-1)


def index_scores_f64(qv, w, kv, seq, pos, cap, m, n_cols):
    """Scores from dequantised inputs: qv [T, h, d], w [T, h], kv [rows, d] -> [T, n_cols] (-inf not visible)."""
    T = qv.shape[0]
    out = np.full((T, n_cols), -np.inf)
    for t in range(T):
        nv = min((int(pos[t]) + 1) // m, n_cols)
        keys = kv[int(seq[t]) * cap: int(seq[t]) * cap + nv]
        dots = keys @ qv[t].T                       # [nv, h]
        out[t, :nv] = np.maximum(dots, 0.0) @ np.asarray(w[t], np.float64)
    return out


def index_bwd_f64(qv, w, kv, seq, pos, cap, m, idx, G):
    """Gradient of sum_t,a G[t][a] score[t][idx[t][a]] -> (dq [T, h, d], dw [T, h], dk [rows, d])."""
    T, h, d = qv.shape
    w = np.asarray(w, np.float64)
    dq = np.zeros((T, h, d))
    dw = np.zeros((T, h))
    dk = np.zeros(kv.shape)
    for t in range(T):
        nv = (int(pos[t]) + 1) // m
        for a in range(idx.shape[1]):
            j = int(idx[t, a])
            if j < 0 or j >= nv:
                continue
            r = int(seq[t]) * cap + j
            g = float(G[t, a])
            dots = qv[t] @ kv[r]                     # [h]
            act = (dots > 0.0).astype(np.float64)
            dw[t] += g * np.maximum(dots, 0.0)
            coef = g * w[t] * act                    # [h]
            dq[t] += coef[:, None] * kv[r][None, :]
            dk[r] += coef @ qv[t]
    return dq, dw, dk


def index_bwd(iq, iq_scale, w, seq, pos, keys, key_scale, cap, m, idx, G):
    """index_bwd_f64 on MXFP4 inputs (dequantised exactly)."""
    return index_bwd_f64(dequant_mxfp4(iq, iq_scale), w, dequant_mxfp4(keys, key_scale), seq, pos, cap, m,
                         np.asarray(idx), np.asarray(G, np.float64))

"""ORACLE — fp64 gradient of the attention step (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the library never does.

The pages train the model with the sparse attention in place: [xmsumi]
§ 预训练 brings the sparse attention in during the 64K stage, after a warm-up
of the lightning indexer, and [hortopato] (training section) quantises the
indexer QK path for quantisation-aware training.  Training needs the gradient
of the attention step; the pages give no formula for it, so this module writes
out the plain definition: the exact derivative of the forward that ``oracle.c``
computes ([xmsumi] § CSA / § HCA / § 关键技术细节: attention over the selected
compressed entries plus the window, RoPE on the last 64 dims of queries and
entries, reverse RoPE on the output).

Forward, per query row t (position tp) and head h, over its key set U(t):
    q~   = R(tp) q               (RoPE on the last 64 dims)
    s_u  = c <q~, e_u>,  p_u = exp(s_u - lse),  o~ = sum_u p_u e_u
    out  = R(-tp) o~             (reverse RoPE on the last 64 dims)
Given g = dL/d out:
    g~   = R(tp) g               (the adjoint of R(-tp))
    D    = <g~, o~>              (= <g, out>)
    ds_u = p_u (<g~, e_u> - D)
    dq   = R(-tp) (c sum_u ds_u e_u)
    de_u += c ds_u q~ + p_u g~   (K and V are the same entry)
Gradients are taken with respect to the dequantised entries (fp64 values of the
stored FP8 * scale / BF16 dims) and the pre-RoPE query.  Entries selected by
several rows or heads accumulate.

Pins (tests/test_oracle_pins.py): the forward core reproduces oracle.attend;
central differences of the fp64 forward match every gradient; the closed forms
sum_u de_u = sum_h g~_h (a shift of every entry moves every output by the same
rotated shift) and, for a single key, dq = 0 and de = sum_h g~_h.
"""
import numpy as np

from . import bf16_array_to_f64, dequant_entries


def rope_rows(x, pos, base=10000.0, inverse=False):
    """RoPE of the last axis (64 dims, pairs (2i, 2i+1), theta_i = base^(-2i/64)) at pos."""
    x = np.asarray(x, dtype=np.float64)
    i = np.arange(32, dtype=np.float64)
    a = float(pos) * np.power(float(base), -2.0 * i / 64.0)
    if inverse:
        a = -a
    c, s = np.cos(a), np.sin(a)
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return y


def attend_core(qh, keys, tp, sm_scale, base=10000.0):
    """One query row: qh [H, d] pre-RoPE fp64, keys [n, d] fp64 -> (out [H, d], lse [H])."""
    H, d = qh.shape
    dn = d - 64
    out = np.zeros((H, d))
    if keys.shape[0] == 0:
        return out, np.full(H, -np.inf)
    qr = qh.copy()
    qr[:, dn:] = rope_rows(qh[:, dn:], tp, base)
    s = sm_scale * (qr @ keys.T)
    mx = s.max(axis=1)
    lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    out = p @ keys
    out[:, dn:] = rope_rows(out[:, dn:], tp, base, inverse=True)
    return out, lse


def attend_core_bwd(qh, keys, tp, sm_scale, g, base=10000.0):
    """Gradients of sum(g * out) for one row: (dq [H, d], dkeys [n, d])."""
    H, d = qh.shape
    dn = d - 64
    n = keys.shape[0]
    if n == 0:
        return np.zeros((H, d)), np.zeros((0, d))
    qr = qh.copy()
    qr[:, dn:] = rope_rows(qh[:, dn:], tp, base)
    s = sm_scale * (qr @ keys.T)
    mx = s.max(axis=1)
    lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])  # [H, n]
    o = p @ keys  # before the reverse RoPE
    gr = np.asarray(g, dtype=np.float64).copy()
    gr[:, dn:] = rope_rows(gr[:, dn:], tp, base)
    D = (gr * o).sum(axis=1)
    ds = p * (gr @ keys.T - D[:, None])
    dqr = sm_scale * (ds @ keys)
    dq = dqr.copy()
    dq[:, dn:] = rope_rows(dqr[:, dn:], tp, base, inverse=True)
    dkeys = sm_scale * (ds.T @ qr) + p.T @ gr
    return dq, dkeys


def key_rows(t, seq, pos, m, comp_cap, win_cap, W, idx=None):
    """Key set of row t, in the forward's order: [('c', row) ...] selected (or all visible)
    compressed entries, then [('w', row) ...] window tokens lo .. tp."""
    tp = int(pos[t])
    nv = (tp + 1) // m
    cb, wb = int(seq[t]) * comp_cap, int(seq[t]) * win_cap
    rows = []
    if idx is not None:
        for j in np.asarray(idx[t]):
            if 0 <= int(j) < nv:
                rows.append(("c", cb + int(j)))
    else:
        rows += [("c", cb + j) for j in range(nv)]
    lo = max(0, tp - W + 1)
    n_win = tp - lo + 1 if W > 0 else 0
    rows += [("w", wb + p % win_cap) for p in range(lo, lo + n_win)]
    return rows


def attend_bwd(q, seq, pos, comp, comp_cap, win, win_cap, W, m, sm_scale, dout, rope_base=10000.0, idx=None):
    """Gradient of sum(dout * out) for the whole batch.

    q [T, H, d] bf16 bits (pre-RoPE); comp / win = (nope, rope, scale) stored entries indexed
    by seq*cap + slot; dout [T, H, d].  Returns (dq [T, H, d], dcomp [rows_c, d],
    dwin [rows_w, d]) in fp64; dcomp / dwin are indexed like the stored entries."""
    q = bf16_array_to_f64(q)
    T, H, d = q.shape
    ce = dequant_entries(*comp)
    we = dequant_entries(*win)
    dq = np.zeros((T, H, d))
    dcomp = np.zeros_like(ce)
    dwin = np.zeros_like(we)
    for t in range(T):
        rows = key_rows(t, seq, pos, m, comp_cap, win_cap, W, idx)
        keys = np.stack([(ce if kind == "c" else we)[r] for kind, r in rows]) if rows else np.zeros((0, d))
        dq[t], dk = attend_core_bwd(q[t], keys, int(pos[t]), sm_scale, np.asarray(dout[t], np.float64), rope_base)
        for (kind, r), v in zip(rows, dk):
            (dcomp if kind == "c" else dwin)[r] += v
    return dq, dcomp, dwin

"""Pure-Python brute force and an element-level mask expansion, written
independently of the oracle, for tiny inputs only."""
import math

import numpy as np

import workloads as wl


def tok_of_logical(T, HW):
    """tok[j] = frame-major token at temporal-major logical position j."""
    return np.arange(T * HW).reshape(T, HW).T.reshape(-1)


def element_mask(w, b, h):
    """bool [L][L] over frame-major tokens (query, key) for head (b, h)."""
    L = w.L
    if w.kind == wl.VIDEO:
        HW = w.Hg * w.Wg
        i = np.arange(L)
        t, y, x = i // HW, (i % HW) // w.Wg, i % w.Wg
        pat = int(w.head_pattern[h])
        if pat == wl.DENSE:
            return np.ones((L, L), bool)
        if pat == wl.SPATIAL:
            return (t[None, :] == t[:, None]) | (t[None, :] == w.anchor)
        return (np.abs(y[None, :] - y[:, None]) <= w.radius) & (np.abs(x[None, :] - x[:, None]) <= w.radius)
    if w.kind == wl.BLOCK:
        blk = w.block[b, h].astype(bool)
        ml = np.kron(blk, np.ones((w.bq, w.bk), bool))[:L, :L]
    elif w.kind == wl.SLICE:
        ml = np.zeros((L, L), bool)
        nqb = w.nqb
        for i in range(nqb):
            e = (b * w.H + h) * nqb + i
            keys = w.col_idx[w.row_ptr[e]:w.row_ptr[e + 1]]
            ml[i * w.bq:(i + 1) * w.bq, keys] = True
    else:
        raise ValueError(w.kind)
    lay = w.layout()[h]
    if lay == wl.TEMPORAL_MAJOR:
        lot = np.argsort(tok_of_logical(w.T, w.Hg * w.Wg))  # logical position of each token
        return ml[np.ix_(lot, lot)]
    return ml


def brute_attend(q, K, V, keep):
    """Masked softmax attention of one query with math.fsum (tiny sizes)."""
    d = len(q)
    idx = [k for k in range(len(K)) if keep[k]]
    if not idx:
        return [0.0] * d
    s = [math.fsum(float(q[c]) * float(K[k][c]) for c in range(d)) / math.sqrt(d) for k in idx]
    m = max(s)
    wts = [math.exp(v - m) for v in s]
    den = math.fsum(wts)
    return [math.fsum(wts[e] * float(V[k][c]) for e, k in enumerate(idx)) / den for c in range(d)]

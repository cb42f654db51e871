"""Float64 brute force used to pin the oracle on tiny inputs.

It is written in a different formulation from the oracle on purpose:
  * GDN: for every node, walk its root path explicitly and apply the published
    matrix form S <- a (I - b k k^T) S + b k v^T step by step on a d_k x d_v
    matrix, then o = S^T (s q).  (The oracle walks the tree once, column by
    column, in the expanded A / r / u form.)
  * Attention: append all tree rows after the resident rows in tree-index
    order, build the explicit (n x (L + n)) visibility matrix from ancestor
    sets found by walking parent links, and take a dense softmax.  (The oracle
    orders each row's keys by position and never builds a mask.)
"""
import numpy as np


def widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ancestors_or_self(parent, i):
    s = set()
    while i >= 0:
        s.add(i)
        i = parent[i]
    return s


def gdn_tree(parent, S_base, q, k, v, alpha, beta, scale):
    """S_base [hv][dv][dk] (S[a][c] at [h][c][a]); returns o [n][hv][dv] in float64."""
    q, k, v, alpha, beta = map(widen, (q, k, v, alpha, beta))
    S_base = np.asarray(S_base, np.float64)
    n, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    o = np.zeros((n, hv, dv))
    states = np.zeros((n, hv, dv, dk))
    for i in range(n):
        path = []
        x = i
        while x >= 0:
            path.append(x)
            x = parent[x]
        path.reverse()
        for h in range(hv):
            g = h // (hv // hk)
            S = S_base[h].T.copy()              # d_k x d_v
            for j in path:
                kj = k[j, g][:, None]
                S = alpha[j, h] * (np.eye(dk) - beta[j, h] * (kj @ kj.T)) @ S \
                    + beta[j, h] * (kj @ v[j, h][None, :])
            o[i, h] = S.T @ (scale * q[i, g])
            states[i, h] = S.T
    return o, states


def attn_tree(parent, L, Kc, Vc, q, kt, vt, scale):
    """Dense masked softmax.  Kc, Vc [hkv][cap][D]; q [n][hq][D]; kt, vt [n][hkv][D]."""
    Kc, Vc, q, kt, vt = map(widen, (Kc, Vc, q, kt, vt))
    n, hq, D = q.shape
    hkv = Kc.shape[0]
    vis = np.zeros((n, L + n), bool)
    vis[:, :L] = True
    for i in range(n):
        for j in ancestors_or_self(parent, i):
            vis[i, L + j] = True
    o = np.zeros((n, hq, D))
    for j in range(hq):
        m = j // (hq // hkv)
        keys = np.concatenate([Kc[m, :L], kt[:, m]], 0)
        vals = np.concatenate([Vc[m, :L], vt[:, m]], 0)
        z = scale * (q[:, j] @ keys.T)
        z = np.where(vis, z, -np.inf)
        z = z - z.max(1, keepdims=True)
        w = np.exp(z)
        w = w / w.sum(1, keepdims=True)
        o[:, j] = w @ vals
    return o


def rel_err(a, b):
    """max |a - b| / max |b| over a tensor (NaN or Inf anywhere counts as infinite)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        return np.inf
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))

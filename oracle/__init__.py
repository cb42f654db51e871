"""CPU oracle for the tree-verify path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library neither imports nor
links it, and it shares no code with the GPU library: the arithmetic lives in
``oracle.c`` (plain float32 C, ascending-order sums, no contraction), this file
only marshals arrays and states the round's bookkeeping (commit and rollback)
as plain array operations.

Every function follows the passages cited in ``oracle.c``: the hot verbs and
the verified-row rule of "Adding a model" (step 4 of "The adapter path in ten
steps"), the state sections and K/V views of "Adding a model" ("The model
layer: architecture registry and per-model state"), and the round of "One
request, end to end" (section 2.6, "The decode loop").  The Gated DeltaNet
step is the published recurrence (Yang, Kautz, Hatamizadeh, ICLR 2025).

The short causal convolution in front of a GDN layer (``gdn_conv``, the gdn.conv
state section of "Adding a model", "The model layer: architecture registry and
per-model state") is the published Gated DeltaNet block's depthwise conv + SiLU +
q/k L2 norm, taken along each node's root path with the slot's committed tail
before the root; ``conv_tail_commit`` is its commit.

Pins (tests that tie this oracle to something other than itself) live in
``tests/test_oracle_pins.py``: hand-worked examples in ``tests/golden/``,
closed forms, a float64 brute force written in a different formulation
(matrix form of the recurrence per root path; dense softmax over an explicit
mask), library softmax attention, library depthwise conv1d (chains, and every
root path of a tree), and torch's bfloat16 conversion for ``to_storage``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# HDT_ORACLE_LIBRARY names another build of oracle.c (the sanitizer build of the tests)
_LOAD_PATH = os.environ.get("HDT_ORACLE_LIBRARY") or _LIB_PATH
MAX_NODES = 64


def build() -> str:
    """Compile liboracle.so with gcc: float32, no fast-math, no contraction."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-o", tmp, src, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    lib.orc_tree_meta.restype = _I
    lib.orc_tree_meta.argtypes = [_I, _P, _I64, _P, _P, _P, _P]
    lib.orc_gdn_tree.restype = None
    lib.orc_gdn_tree.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _F, _P,
                                 _P]
    lib.orc_gdn_commit.restype = None
    lib.orc_gdn_commit.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P]
    lib.orc_attn_row.restype = None
    lib.orc_attn_row.argtypes = [_I, _I, _I, _I, _P, _I64, _I64, _P, _P, _P, _P, _P, _I, _F,
                                 _I, _I, _P]
    lib.orc_attn_tree.restype = None
    lib.orc_attn_tree.argtypes = [_I, _I, _I, _I, _P, _I64, _I64, _P, _P, _P, _P, _P, _I,
                                  _F, _P]
    lib.orc_gdn_conv.restype = None
    lib.orc_gdn_conv.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _F, _P,
                                 _P, _P]
    return lib


def _load():
    global _lib
    if _lib is None:
        if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        _lib = configure(ctypes.CDLL(_LOAD_PATH))
    return _lib


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _dtype_code(*arrays) -> int:
    kinds = {a.dtype for a in arrays if a is not None}
    if kinds == {np.dtype(np.float32)}:
        return 0
    if kinds == {np.dtype(np.uint16)}:
        return 1
    raise TypeError(f"inputs must be all float32 or all bfloat16 bits (uint16), got {kinds}")


def tree_meta(parent, L: int = 0):
    """depth [n] int32, mask [n] uint64 (ancestor-or-self bits), anc [n][64] int32 (ancestor
    at each depth, -1 beyond), pos [n] int64.  Raises ValueError on an invalid tree."""
    par = np.asarray(parent, dtype=np.int32)
    n = len(par)
    depth = np.zeros(max(n, 1), np.int32)
    mask = np.zeros(max(n, 1), np.uint64)
    anc = np.zeros((max(n, 1), MAX_NODES), np.int32)
    pos = np.zeros(max(n, 1), np.int64)
    rc = _load().orc_tree_meta(n, par.ctypes.data, L, depth.ctypes.data, mask.ctypes.data,
                               anc.ctypes.data, pos.ctypes.data)
    if rc != 0:
        raise ValueError("invalid parent array")
    return depth[:n], mask[:n], anc[:n], pos[:n]


def gdn_tree(parent, S_base, q, k, v, alpha, beta, scale=None, want_states=False):
    """One GDN layer over a tree.  Shapes: S_base [hv][dv][dk] f32; q,k [n][hk][dk];
    v [n][hv][dv]; alpha,beta [n][hv] (float32 or bf16 bits).  Returns o [n][hv][dv] f32
    (and the per-node states [n][hv][dv][dk] when want_states)."""
    par = np.asarray(parent, dtype=np.int32)
    n, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(dk)))
    dt = _dtype_code(q, k, v, alpha, beta)
    S_base = _c(S_base.astype(np.float32, copy=False))
    q, k, v, alpha, beta = map(_c, (q, k, v, alpha, beta))
    o = np.zeros((n, hv, dv), np.float32)
    states = np.zeros((n, hv, dv, dk), np.float32) if want_states else None
    _load().orc_gdn_tree(dk, dv, hk, hv, n, par.ctypes.data, S_base.ctypes.data, q.ctypes.data,
                         k.ctypes.data, v.ctypes.data, alpha.ctypes.data, beta.ctypes.data, dt,
                         scale, o.ctypes.data, states.ctypes.data if want_states else None)
    return (o, states) if want_states else o


def gdn_commit(path, S_base, k, v, alpha, beta):
    """Recurrent state after accepting `path`: sequential recurrence from S_base."""
    p = np.asarray(path, dtype=np.int32)
    n, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    dt = _dtype_code(k, v, alpha, beta)
    S_base = _c(S_base.astype(np.float32, copy=False))
    k, v, alpha, beta = map(_c, (k, v, alpha, beta))
    out = np.zeros((hv, dv, dk), np.float32)
    _load().orc_gdn_commit(dk, dv, hk, hv, len(p), p.ctypes.data, S_base.ctypes.data,
                           k.ctypes.data, v.ctypes.data, alpha.ctypes.data, beta.ctypes.data, dt,
                           out.ctypes.data)
    return out


def attn_row(parent, L, Kc, Vc, q, kt, vt, node, j, scale=None):
    """One output row (node, q head j) of an attention layer.  Kc, Vc [hkv][cap][D] hold at
    least L resident rows per head; q [n][hq][D]; kt, vt [n][hkv][D]."""
    par = np.asarray(parent, dtype=np.int32)
    n, hq, D = q.shape
    hkv, cap = Kc.shape[0], Kc.shape[1]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(D)))
    dt = _dtype_code(Kc, Vc, q, kt, vt)
    Kc, Vc, q, kt, vt = map(_c, (Kc, Vc, q, kt, vt))
    o = np.zeros(D, np.float32)
    _load().orc_attn_row(hq, hkv, D, n, par.ctypes.data, L, cap, Kc.ctypes.data, Vc.ctypes.data,
                         q.ctypes.data, kt.ctypes.data, vt.ctypes.data, dt, scale, node, j,
                         o.ctypes.data)
    return o


def attn_tree(parent, L, Kc, Vc, q, kt, vt, scale=None):
    """All rows of an attention layer: o [n][hq][D] float32."""
    par = np.asarray(parent, dtype=np.int32)
    n, hq, D = q.shape
    hkv, cap = Kc.shape[0], Kc.shape[1]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(D)))
    dt = _dtype_code(Kc, Vc, q, kt, vt)
    Kc, Vc, q, kt, vt = map(_c, (Kc, Vc, q, kt, vt))
    o = np.zeros((n, hq, D), np.float32)
    _load().orc_attn_tree(hq, hkv, D, n, par.ctypes.data, L, cap, Kc.ctypes.data,
                          Vc.ctypes.data, q.ctypes.data, kt.ctypes.data, vt.ctypes.data, dt,
                          scale, o.ctypes.data)
    return o


def commit_kv_rows(tree_rows: np.ndarray, path) -> np.ndarray:
    """Rows appended to a K or V view by commit_tree: row L+d is the tree row of path[d].
    tree_rows [n][hkv][D] -> [hkv][m][D]."""
    return np.ascontiguousarray(np.transpose(tree_rows[np.asarray(path, dtype=np.int64)], (1, 0, 2)))


def valid_path(parent, path) -> bool:
    """A path a round may commit: starts at the root and follows parent links."""
    if len(path) < 1 or path[0] != 0:
        return False
    return all(0 <= path[d] < len(parent) and parent[path[d]] == path[d - 1]
               for d in range(1, len(path)))


def leading_chain(parent) -> int:
    """Length c of the tree's leading chain: nodes 0..c-1 with parent[i] = i-1."""
    c = 1
    while c < len(parent) and parent[c] == c - 1:
        c += 1
    return c


def rollback_plan(parent, L: int, n: int):
    """rollback_to(n) with a pending tree of committed length L: keep exactly n tokens.
    Returns the chain prefix to commit ([] to drop the round), or None when n is outside
    [L, L + leading chain] (not supported without state anchors)."""
    c = leading_chain(parent)
    if n == L:
        return []
    if L < n <= L + c:
        return list(range(n - L))
    return None


CONV_EPS = 1e-6  # L2-norm epsilon of the published Gated DeltaNet q/k normalisation


def gdn_conv(parent, tail, q, k, v, W, eps=CONV_EPS):
    """Short causal conv + SiLU (+ per-head L2 norm of q and k) of one GDN layer over a
    tree.  tail [w-1][C] committed pre-conv inputs (row w-2 newest); q,k [n][hk][dk],
    v [n][hv][dv] pre-conv inputs; W [C][w] float32, C = 2 hk dk + hv dv (q, k, v
    channels in that order).  Returns float32 (q', k', v') of the input shapes."""
    par = np.asarray(parent, dtype=np.int32)
    n, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    W = _c(np.asarray(W, dtype=np.float32))
    w = W.shape[1]
    C = 2 * hk * dk + hv * dv
    assert W.shape == (C, w) and 1 <= w <= 8
    if tail is None or w == 1:
        tail = np.zeros((max(w - 1, 1), C), q.dtype)
    assert tail.shape[1] == C
    dt = _dtype_code(tail, q, k, v)
    tail, q, k, v = map(_c, (tail, q, k, v))
    qo = np.zeros((n, hk, dk), np.float32)
    ko = np.zeros((n, hk, dk), np.float32)
    vo = np.zeros((n, hv, dv), np.float32)
    _load().orc_gdn_conv(hk, dk, hv, dv, w, n, par.ctypes.data, tail.ctypes.data, q.ctypes.data,
                         k.ctypes.data, v.ctypes.data, W.ctypes.data, dt, eps, qo.ctypes.data,
                         ko.ctypes.data, vo.ctypes.data)
    return qo, ko, vo


def conv_rows(q, k, v) -> np.ndarray:
    """Pre-conv inputs of each node as one channel row: [n][C] = q | k | v."""
    n = q.shape[0]
    return np.concatenate([q.reshape(n, -1), k.reshape(n, -1), v.reshape(n, -1)], axis=1)


def conv_tail_commit(tail: np.ndarray, q, k, v, path) -> np.ndarray:
    """Conv tail after commit_tree(path): the last w-1 rows of the committed tail followed
    by the path's pre-conv input rows (bit copies).  tail [w-1][C] -> [w-1][C]."""
    rows = conv_rows(q, k, v)[np.asarray(path, dtype=np.int64)]
    seq = np.concatenate([tail, rows.astype(tail.dtype, copy=False)], axis=0)
    return np.ascontiguousarray(seq[len(seq) - tail.shape[0]:])


def to_storage(x: np.ndarray, like: np.ndarray) -> np.ndarray:
    """float32 values in the storage dtype of `like`: unchanged for float32, else bfloat16
    bit patterns rounded to nearest even (NaN is not expected here)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if like.dtype == np.float32:
        return x
    b = x.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def gdn_conv_layer(parent, S_base, tail, q, k, v, alpha, beta, W, scale=None, want_states=False):
    """A GDN layer whose q, k, v arrive before the short conv: gdn_conv, its outputs stored
    in the input dtype (as the layer's activations are), then gdn_tree.  Returns what
    gdn_tree returns, plus the stored post-conv (q', k', v')."""
    qc, kc, vc = (to_storage(x, q) for x in gdn_conv(parent, tail, q, k, v, W))
    out = gdn_tree(parent, S_base, qc, kc, vc, alpha, beta, scale=scale, want_states=want_states)
    return out, (qc, kc, vc)


def greedy_walk(parent, draft, target):
    """The round's accept rule ("One request, end to end", 2.6: walk the verified tree with
    the model's own tokens, keep the longest agreeing path plus one token of the model's
    own).  draft[i] is node i's token (the root's is the model's own token from the last
    round and is not compared); target[i] is the model's own next token after node i.
    The root agrees; node i > 0 agrees when its parent agrees and draft[i] equals
    target[parent[i]].  The accepted node is the deepest agreeing node, the lowest index
    among equals; returns (its root path, target of that node = the bonus token)."""
    n = len(parent)
    depth = [0] * n
    agree = [False] * n
    agree[0] = True
    for i in range(1, n):
        p = parent[i]
        depth[i] = depth[p] + 1
        agree[i] = agree[p] and int(draft[i]) == int(target[p])
    best = 0
    for i in range(n):
        if agree[i] and depth[i] > depth[best]:
            best = i
    path = []
    x = best
    while x >= 0:
        path.append(x)
        x = parent[x]
    return path[::-1], int(target[best])

"""Seeded, counter-based synthetic inputs for the tree-verify path.

The generator lives in ``synth.c`` (SplitMix64 as a counter-based generator,
Box-Muller normals).  This package builds it, wraps it, and defines the
workloads: shapes, value recipes, draft trees and accepted paths.  It holds
none of the method's arithmetic; the CPU oracle and the GPU path both read
the exact bits it produces.

Value recipes (from the workload descriptions that accompany the pages):
  q, k (tree and resident keys): N(0,1) per element, then each (row, head)
  vector divided by its L2 norm; v: N(0,1); beta = sigmoid(N(0,1));
  alpha = exp(-softplus(N(0,1))); the resident recurrent state S: N(0, 1/d_k).
  Storage is float32 for the tiny workload and bfloat16 (round to nearest
  even) otherwise; the recurrent state is always float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
# HDT_SYNTH_LIBRARY names another build of synth.c (the sanitizer build of the tests)
_LOAD_PATH = os.environ.get("HDT_SYNTH_LIBRARY") or _LIB_PATH

NORMAL, NORMAL_L2, SIGMOID, EXP_NEG_SOFTPLUS = 0, 1, 2, 3
DEFAULT_SEED = 20261202


def build() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LOAD_PATH)
        lib.synth_u64.restype = ctypes.c_uint64
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        lib.synth_fill.restype = None
        lib.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def key(seed: int, name: str) -> int:
    return _load().synth_key(seed, name.encode())


def u64(k: int, counter: int) -> int:
    return _load().synth_u64(k, counter)


def normal(k: int, i: int) -> float:
    return _load().synth_normal(k, i)


def fill(seed: int, name: str, kind: int, shape, *, dtype: str, row0: int = 0, rows=None,
         scale: float = 1.0) -> np.ndarray:
    """Rows [row0, row0+rows) of the tensor `name`, flattened to [rows, shape[-1]].

    dtype "f32" returns float32 values; "bf16" returns the bfloat16 bit
    patterns as uint16 (round to nearest even from the float32 value).
    """
    cols = int(shape[-1])
    total_rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    if rows is None:
        rows = total_rows - row0
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    p = out.ctypes.data
    _load().synth_fill(key(seed, name), kind, row0, rows, cols, scale,
                       p if dtype == "f32" else None, p if dtype == "bf16" else None)
    if rows == total_rows and row0 == 0:
        return out.reshape(shape)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (test helper)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------
# Draft trees and accepted paths (parent-index arrays, parent[i] < i, node 0 is the root)
# --------------------------------------------------------------------------------------------

class _Stream:
    """Sequential draws from one counter-based stream."""

    def __init__(self, seed: int, name: str):
        self.k = key(seed, name)
        self.c = 0

    def uint(self, lo: int, hi: int) -> int:
        """Uniform integer in [lo, hi] (inclusive)."""
        x = u64(self.k, self.c)
        self.c += 1
        return lo + int(((x >> 11) * (hi - lo + 1)) >> 53)


def depths(parent) -> list:
    d = []
    for i, p in enumerate(parent):
        d.append(0 if p < 0 else d[p] + 1)
    return d


def chain_tree(n: int) -> list:
    return [-1] + list(range(n - 1))


def random_tree(seed: int, name: str, n: int, max_depth: int) -> list:
    """parent[i] uniform over earlier nodes j with depth[j] < max_depth."""
    s = _Stream(seed, name)
    parent, dep = [-1], [0]
    for i in range(1, n):
        cands = [j for j in range(i) if dep[j] < max_depth]
        p = cands[s.uint(0, len(cands) - 1)]
        parent.append(p)
        dep.append(dep[p] + 1)
    return parent


def draft_tree(seed: int, name: str, n: int = 16, max_depth: int = 15) -> list:
    """A block-draft chain below the root plus lookup continuations.

    n = 16: chain of c = 15 - b nodes (b ~ U{2..6}) under the root, then the b
    remaining nodes as lookup runs of length U{1..3}, each run hanging off a
    uniform chain node.  n = 32: a chain of 15 plus 16 lookup-run nodes, every
    node at depth <= max_depth.
    """
    s = _Stream(seed, name)
    if n <= 16:
        b = s.uint(2, 6) if n == 16 else max(0, (n - 1) // 3)
        c = min(n - 1 - b, max_depth)
    else:
        c = min(15, max_depth, n - 1)
    parent = [-1] + list(range(c))
    dep = list(range(c + 1))
    remaining = n - 1 - c
    while remaining > 0:
        length = min(s.uint(1, 3), remaining)
        at = s.uint(0, c)
        length = min(length, max_depth - dep[at])
        if length <= 0:
            continue
        prev = at
        for _ in range(length):
            parent.append(prev)
            dep.append(dep[prev] + 1)
            prev = len(parent) - 1
        remaining -= length
    return parent


def root_path(parent, node: int) -> list:
    p = []
    while node >= 0:
        p.append(node)
        node = parent[node]
    return p[::-1]


def accepted_path(seed: int, name: str, parent) -> list:
    """m ~ U{1 .. 1 + max depth}, then a uniform node at depth m-1, then its root path."""
    s = _Stream(seed, name)
    dep = depths(parent)
    m = s.uint(1, 1 + max(dep))
    at = [i for i, d in enumerate(dep) if d == m - 1]
    return root_path(parent, at[s.uint(0, len(at) - 1)])


# --------------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    layer_kind: list                # 0 = Gated DeltaNet, 1 = attention
    gdn_hk: int
    gdn_hv: int
    gdn_dk: int
    gdn_dv: int
    attn_hq: int
    attn_hkv: int
    attn_d: int
    dtype: str                      # storage dtype of q/k/v/gates/KV: "f32" or "bf16"
    lengths: list                   # resident context per slot
    n_nodes: int
    tree_kind: str                  # "random4" | "draft"
    max_depth: int = 15
    extra: dict = field(default_factory=dict)

    @property
    def n_slots(self):
        return len(self.lengths)

    @property
    def n_gdn(self):
        return sum(1 for k in self.layer_kind if k == 0)

    @property
    def n_attn(self):
        return sum(1 for k in self.layer_kind if k == 1)

    def tree(self, seed: int, slot: int = 0) -> list:
        if self.tree_kind == "random4":
            return random_tree(seed, f"{self.name}/tree/{slot}", self.n_nodes, 4)
        return draft_tree(seed, f"{self.name}/tree/{slot}", self.n_nodes, self.max_depth)


def stack_kinds(n_layers: int = 64) -> list:
    """Three Gated DeltaNet layers then one attention layer, repeated."""
    return [1 if l % 4 == 3 else 0 for l in range(n_layers)]


WORKLOADS = {
    # 1 GDN layer (1 head, 64x64) + 1 attention layer (2 q heads, 1 kv head, dim 64), fp32,
    # 256 resident tokens, 8-node random tree of depth <= 4.
    "tiny": Workload("tiny", [0, 1], 1, 1, 64, 64, 2, 1, 64, "f32", [256], 8, "random4", 4),
    # One GDN + attention layer pair at 27B-like shapes, 8,192 resident tokens, 16-node tree.
    "pair_8k": Workload("pair_8k", [0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [8192], 16,
                        "draft"),
    # Full 64-layer stack (48 GDN + 16 attention), 65,536 resident tokens, 16-node tree.
    "stack_65k": Workload("stack_65k", stack_kinds(), 16, 32, 128, 128, 24, 4, 256, "bf16",
                          [65536], 16, "draft"),
    # Long context: 262,144 resident tokens, 32-node tree of depth <= 15.
    "stack_262k": Workload("stack_262k", stack_kinds(), 16, 32, 128, 128, 24, 4, 256, "bf16",
                           [262144], 32, "draft"),
    # stack_65k with the width-4 short causal conv in front of every GDN layer (pre-conv
    # q, k, v in; the conv tails are part of the committed state).
    "stack_65k_conv": Workload("stack_65k_conv", stack_kinds(), 16, 32, 128, 128, 24, 4, 256,
                               "bf16", [65536], 16, "draft", extra={"conv": 4}),
    # Four slots in one pass: 131,072 + 3 x 8,192 resident tokens, 16-node tree each.
    "joint4": Workload("joint4", stack_kinds(), 16, 32, 128, 128, 24, 4, 256, "bf16",
                       [131072, 8192, 8192, 8192], 16, "draft"),
}


# Tensor names: every tensor of a workload has its own stream, so any slice of it can be
# regenerated alone.  Row counters of the resident cache are per (slot, layer, kv head), so a
# shorter or longer context is a prefix/extension of the same rows.

def gdn_inputs(w: Workload, seed: int, slot: int, layer: int, n: int, tag: str = "verify"):
    """q, k [n][hk][dk]; v [n][hv][dv]; alpha, beta [n][hv] in the storage dtype."""
    base = f"{w.name}/s{slot}/l{layer}/{tag}/gdn"
    dt = w.dtype
    q = fill(seed, base + "/q", NORMAL_L2, (n, w.gdn_hk, w.gdn_dk), dtype=dt)
    k = fill(seed, base + "/k", NORMAL_L2, (n, w.gdn_hk, w.gdn_dk), dtype=dt)
    v = fill(seed, base + "/v", NORMAL, (n, w.gdn_hv, w.gdn_dv), dtype=dt)
    a = fill(seed, base + "/alpha", EXP_NEG_SOFTPLUS, (n, w.gdn_hv), dtype=dt)
    b = fill(seed, base + "/beta", SIGMOID, (n, w.gdn_hv), dtype=dt)
    return q, k, v, a, b


def gdn_state(w: Workload, seed: int, slot: int, layer: int) -> np.ndarray:
    """Resident recurrent state, float32 [hv][dv][dk]: element S[a][c] of head h sits at
    [h][c][a] (value-major: one value column of the key-by-value state is contiguous)."""
    return fill(seed, f"{w.name}/s{slot}/l{layer}/S", NORMAL, (w.gdn_hv, w.gdn_dv, w.gdn_dk),
                dtype="f32", scale=float(np.sqrt(1.0 / w.gdn_dk)))


def attn_inputs(w: Workload, seed: int, slot: int, layer: int, n: int, tag: str = "verify",
                sharp: bool = False, q_scale: float = 1.0, v_scale: float = 1.0):
    """q [n][hq][D]; tree k, v [n][hkv][D].  sharp=True draws q, k without normalisation
    (a parity-only variant whose softmax is far from flat), q as q_scale N(0,1).  v_scale
    multiplies the tree's value rows (parity-only: a power of two makes every tree row's
    share of an output visible even under a flat softmax over a long context)."""
    base = f"{w.name}/s{slot}/l{layer}/{tag}/attn"
    dt = w.dtype
    kq = NORMAL if sharp else NORMAL_L2
    q = fill(seed, base + "/q", kq, (n, w.attn_hq, w.attn_d), dtype=dt, scale=q_scale)
    k = fill(seed, base + "/k", kq, (n, w.attn_hkv, w.attn_d), dtype=dt)
    v = fill(seed, base + "/v", NORMAL, (n, w.attn_hkv, w.attn_d), dtype=dt, scale=v_scale)
    return q, k, v


def kv_rows(w: Workload, seed: int, slot: int, layer: int, head: int, row0: int, rows: int,
            sharp: bool = False, v_scale: float = 1.0):
    """Resident cache rows [row0, row0+rows) of one kv head: K (unit rows), V (normal, times
    v_scale: a parity-only variant whose values pass the fp16 range)."""
    base = f"{w.name}/s{slot}/l{layer}/h{head}"
    K = fill(seed, base + "/K", NORMAL if sharp else NORMAL_L2, (row0 + rows, w.attn_d),
             dtype=w.dtype, row0=row0, rows=rows)
    V = fill(seed, base + "/V", NORMAL, (row0 + rows, w.attn_d), dtype=w.dtype, row0=row0,
             rows=rows, scale=v_scale)
    return K, V


# --------------------------------------------------------------------------------------------
# Short causal convolution of the GDN layers (pre-conv inputs, taps, committed tails)
# --------------------------------------------------------------------------------------------

def conv_channels(w: Workload) -> int:
    """Channels of one token through the conv: q (hk dk), k (hk dk), v (hv dv)."""
    return 2 * w.gdn_hk * w.gdn_dk + w.gdn_hv * w.gdn_dv


def conv_width(w: Workload) -> int:
    return int(w.extra.get("conv", 0))


def conv_inputs(w: Workload, seed: int, slot: int, layer: int, n: int, tag: str = "verify"):
    """Pre-conv q, k [n][hk][dk], v [n][hv][dv] (projection outputs, N(0,1)) and the gates
    alpha, beta [n][hv], in the storage dtype."""
    base = f"{w.name}/s{slot}/l{layer}/{tag}/conv"
    dt = w.dtype
    q = fill(seed, base + "/q", NORMAL, (n, w.gdn_hk, w.gdn_dk), dtype=dt)
    k = fill(seed, base + "/k", NORMAL, (n, w.gdn_hk, w.gdn_dk), dtype=dt)
    v = fill(seed, base + "/v", NORMAL, (n, w.gdn_hv, w.gdn_dv), dtype=dt)
    a = fill(seed, base + "/alpha", EXP_NEG_SOFTPLUS, (n, w.gdn_hv), dtype=dt)
    b = fill(seed, base + "/beta", SIGMOID, (n, w.gdn_hv), dtype=dt)
    return q, k, v, a, b


def conv_weight(w: Workload, seed: int, layer: int) -> np.ndarray:
    """Depthwise taps of one GDN layer, float32 [C][width], N(0, 1/width): a conv output
    over N(0,1) inputs has unit variance."""
    width = conv_width(w)
    return fill(seed, f"{w.name}/l{layer}/conv_w", NORMAL, (conv_channels(w), width),
                dtype="f32", scale=float(np.sqrt(1.0 / width)))


def conv_tail(w: Workload, seed: int, slot: int, layer: int) -> np.ndarray:
    """Committed pre-conv inputs of the last width-1 tokens, [width-1][C] (row width-2 is
    the newest), in the storage dtype."""
    width = conv_width(w)
    return fill(seed, f"{w.name}/s{slot}/l{layer}/conv_tail", NORMAL,
                (max(width - 1, 1), conv_channels(w)), dtype=w.dtype)[:width - 1]


# --------------------------------------------------------------------------------------------
# Tokens of a round: each node's draft token and the model's own next token after it
# --------------------------------------------------------------------------------------------

def round_tokens(seed: int, name: str, parent, vocab: int = 151_936, agree: float = 0.7,
                 distinct: bool = True):
    """(draft[n], target[n]) int32.  Draft tokens are uniform over the vocabulary (distinct
    among siblings unless distinct=False); the model's own token after node x is, with
    probability `agree`, the draft token of one of x's children (uniform among them), else
    a uniform token."""
    s = _Stream(seed, name)
    n = len(parent)
    if distinct and n > vocab:
        raise ValueError("distinct sibling tokens need a vocabulary of at least n tokens")
    draft = np.zeros(n, np.int32)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    draft[0] = s.uint(0, vocab - 1)
    for x in range(n):
        used = set()
        for c in children[x]:
            t = s.uint(0, vocab - 1)
            while distinct and t in used:
                t = s.uint(0, vocab - 1)
            used.add(t)
            draft[c] = t
    target = np.zeros(n, np.int32)
    thresh = int(agree * 1_000_000)
    for x in range(n):
        if children[x] and s.uint(0, 999_999) < thresh:
            target[x] = draft[children[x][s.uint(0, len(children[x]) - 1)]]
        else:
            target[x] = s.uint(0, vocab - 1)
    return draft, target


def tokens_for_path(seed: int, name: str, parent, path, vocab: int = 151_936):
    """(draft, target) whose accept walk keeps exactly `path`: round_tokens, then the
    model's token after each path node but the last set to the next path node's draft
    token, and after the last to a token none of its children carries."""
    draft, target = round_tokens(seed, name, parent, vocab=vocab)
    for a, b in zip(path, path[1:]):
        target[a] = draft[b]
    last = path[-1]
    kids = {int(draft[c]) for c in range(len(parent)) if parent[c] == last}
    t = int(target[last])
    while t in kids:
        t = (t + 1) % vocab
    target[last] = t
    return draft, target

"""The recorded-bytes sequence on the tiny configuration (the analogue of the refactor gate of
"Adding a model", "The tests a new model must pass": the exact bytes after a prefill, a
decode, a block verify, a rollback, a tree verify and a commit).

One sequence over a slot of the tiny workload (1 Gated DeltaNet layer of one 64 x 64 head
+ 1 attention layer of 2 q heads on 1 kv head, dim 64, float32, 256 resident tokens):

  prefill   a 24-token span, committed whole;
  decode    one token, committed;
  block     a 6-token chain, then rollback to keep its first 3 tokens;
  tree      an 8-node random tree (depth <= 4), then commit of a seeded path.

`inputs` draws every input from the seeded generator; `run_oracle` runs the sequence
through the oracle and returns every output, the recurrent state after each step and the
cache rows appended by each step.  The stored digests of those bytes live in
tests/golden/c0_sequence.json, written by tests/golden/record_c0.py.
"""
from __future__ import annotations

import hashlib

import numpy as np

import oracle
import synth

SEED = 20261202
W = synth.WORKLOADS["tiny"]
L0 = W.lengths[0]
STEPS = ("prefill", "decode", "block", "tree")


def trees():
    """(parent array, path kept) of each step, in order."""
    t = synth.random_tree(SEED, "gate/tree", 8, 4)
    return {"prefill": (synth.chain_tree(24), list(range(24))),
            "decode": ([-1], [0]),
            "block": (synth.chain_tree(6), [0, 1, 2]),
            "tree": (t, synth.accepted_path(SEED, "gate/path", t))}


def inputs(step: str, n: int):
    """Host arrays of one step: GDN q, k, v, alpha, beta and attention q, k, v (float32)."""
    g = synth.gdn_inputs(W, SEED, 0, 0, n, f"gate/{step}")
    a = synth.attn_inputs(W, SEED, 0, 1, n, f"gate/{step}")
    return (dict(q=g[0], k=g[1], v=g[2], alpha=g[3], beta=g[4]), dict(q=a[0], k=a[1], v=a[2]))


def capacity() -> int:
    return L0 + sum(len(p) for _, p in trees().values()) + 64


def run_oracle():
    """{step: {"gdn_o", "attn_o", "state", "k_rows", "v_rows"}} as float32 arrays."""
    S = synth.gdn_state(W, SEED, 0, 0)
    cap = capacity()
    Kc = np.zeros((W.attn_hkv, cap, W.attn_d), np.float32)
    Vc = np.zeros_like(Kc)
    for h in range(W.attn_hkv):
        Kc[h, :L0], Vc[h, :L0] = synth.kv_rows(W, SEED, 0, 1, h, 0, L0)
    L = L0
    out = {}
    for step in STEPS:
        parent, path = trees()[step]
        g, a = inputs(step, len(parent))
        o_g = oracle.gdn_tree(parent, S, g["q"], g["k"], g["v"], g["alpha"], g["beta"])
        o_a = oracle.attn_tree(parent, L, Kc, Vc, a["q"], a["k"], a["v"])
        S = oracle.gdn_commit(path, S, g["k"], g["v"], g["alpha"], g["beta"])
        kr = oracle.commit_kv_rows(a["k"], path)
        vr = oracle.commit_kv_rows(a["v"], path)
        Kc[:, L:L + len(path)] = kr
        Vc[:, L:L + len(path)] = vr
        L += len(path)
        out[step] = {"gdn_o": o_g, "attn_o": o_a, "state": S.copy(), "k_rows": kr, "v_rows": vr}
    return out


def digest(a: np.ndarray) -> str:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return hashlib.sha256(a.tobytes()).hexdigest()


def digests(result) -> dict:
    return {step: {name: digest(arr) for name, arr in sorted(r.items())} for step, r in result.items()}

"""Pins for the CPU oracle: each check ties it to something other than itself.

  * hand-worked examples (tests/golden/*.json) with exact expected values;
  * closed forms of the Gated DeltaNet step and of masked softmax attention;
  * a float64 brute force in a different formulation (tests/brute.py);
  * library softmax attention (torch scaled_dot_product_attention, float64, CPU);
  * the pages' invariant that a verified row equals the sequential decode row
    ("Adding a model", step 4 of "The adapter path in ten steps"), bit for bit.

PINS maps a name to a check that raises AssertionError on failure;
tests/test_oracle_mutants.py reruns them against deliberately broken copies
of the oracle to show each plausible mistake is caught.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SEED = 1234


def _f32(x):
    return np.asarray(x, np.float32)


def _gdn_case(seed, n=9, hk=2, hv=4, dk=8, dv=6, dtype="f32", tree="random"):
    w = synth.Workload("pin", [0], hk, hv, dk, dv, 2, 1, 8, dtype, [0], n, "random4")
    parent = synth.random_tree(seed, f"pin/gdn/{seed}", n, 5) if tree == "random" \
        else synth.chain_tree(n)
    q, k, v, a, b = synth.gdn_inputs(w, seed, 0, 0, n)
    S = synth.gdn_state(w, seed, 0, 0)
    return parent, S, q, k, v, a, b


def _attn_case(seed, n=8, hq=6, hkv=2, D=16, L=23, dtype="f32", sharp=False, tree="random"):
    w = synth.Workload("pin", [1], 1, 1, 8, 8, hq, hkv, D, dtype, [L], n, "random4")
    parent = synth.random_tree(seed, f"pin/attn/{seed}", n, 5) if tree == "random" \
        else synth.chain_tree(n)
    q, kt, vt = synth.attn_inputs(w, seed, 0, 0, n, sharp=sharp)
    cap = L + n + 3
    Kc = np.zeros((hkv, cap, D), q.dtype)
    Vc = np.zeros((hkv, cap, D), q.dtype)
    for h in range(hkv):
        K, V = synth.kv_rows(w, seed, 0, 0, h, 0, L, sharp=sharp)
        Kc[h, :L], Vc[h, :L] = K, V
    return parent, L, Kc, Vc, q, kt, vt


# ---------------------------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------------------------

def pin_gdn_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "gdn_hand_example.json")))
    S = np.transpose(_f32(g["S_base_rows_a_cols_c"]))[None]          # [hv][dv][dk]
    n = len(g["parent"])
    q = _f32(g["q"]).reshape(n, 1, 2)
    k = _f32(g["k"]).reshape(n, 1, 2)
    v = _f32(g["v"]).reshape(n, 1, 2)
    a = _f32(g["alpha"]).reshape(n, 1)
    b = _f32(g["beta"]).reshape(n, 1)
    o, states = oracle.gdn_tree(g["parent"], S, q, k, v, a, b, scale=g["scale"],
                                want_states=True)
    assert np.array_equal(o[:, 0], _f32(g["o"]))
    assert np.array_equal(states[:, 0], np.transpose(_f32(g["S_nodes_rows_a_cols_c"]), (0, 2, 1)))
    Sc = oracle.gdn_commit(g["commit_path"], S, k, v, a, b)
    assert np.array_equal(Sc[0], np.transpose(_f32(g["S_after_commit_rows_a_cols_c"])))


def pin_attn_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "attn_hand_example.json")))
    n, D = len(g["parent"]), g["D"]
    Kc = _f32(g["K_resident"]).reshape(1, g["L"], D)
    Vc = _f32(g["V_resident"]).reshape(1, g["L"], D)
    o = oracle.attn_tree(g["parent"], g["L"], Kc, Vc, _f32(g["q"]).reshape(n, 1, D),
                         _f32(g["k_tree"]).reshape(n, 1, D), _f32(g["v_tree"]).reshape(n, 1, D),
                         scale=g["scale"])
    np.testing.assert_allclose(o[:, 0], _f32(g["o"]), rtol=0, atol=g["tolerance"] * 10)


def pin_tree_meta_brute():
    for seed in range(6):
        parent = synth.random_tree(seed, "pin/meta", 40, 9)
        depth, mask, anc, pos = oracle.tree_meta(parent, L=100)
        for i in range(len(parent)):
            chain = []
            x = i
            while x >= 0:
                chain.append(x)
                x = parent[x]
            assert depth[i] == len(chain) - 1
            assert pos[i] == 100 + len(chain) - 1
            assert int(mask[i]) == sum(1 << j for j in chain)
            assert list(anc[i, :len(chain)]) == chain[::-1]
            assert (anc[i, len(chain):] == -1).all()
    for bad in ([0], [-1, 1], [-1, 0, 3], [-1, -1], []):
        with pytest.raises(ValueError):
            oracle.tree_meta(bad)


def pin_gdn_brute():
    for seed, dtype in ((1, "f32"), (2, "bf16"), (3, "f32")):
        parent, S, q, k, v, a, b = _gdn_case(seed, dtype=dtype)
        s = float(np.float32(1 / np.sqrt(8)))
        o, states = oracle.gdn_tree(parent, S, q, k, v, a, b, want_states=True)
        ob, sb = brute.gdn_tree(parent, S, q, k, v, a, b, s)
        assert brute.rel_err(o, ob) < 1e-5, brute.rel_err(o, ob)
        assert brute.rel_err(states, sb) < 1e-5


def pin_gdn_closed_forms():
    parent, S, q, k, v, a, b = _gdn_case(7, n=7)
    s = float(np.float32(1 / np.sqrt(8)))
    ones, zeros = np.ones_like(a), np.zeros_like(b)
    # alpha = 1, beta = 0: the state never moves and o = s S_base^T q.
    o, st = oracle.gdn_tree(parent, S, q, k, v, ones, zeros, want_states=True)
    for i in range(len(parent)):
        for h in range(S.shape[0]):
            assert np.array_equal(st[i, h], S[h])
            exp = S[h].astype(np.float64) @ (s * q[i, h // 2].astype(np.float64))
            np.testing.assert_allclose(o[i, h], exp, rtol=1e-5, atol=1e-6)
    # beta = 0: S_i = (product of alpha along the root path) S_base.
    o, st = oracle.gdn_tree(parent, S, q, k, v, a, zeros, want_states=True)
    for i in range(len(parent)):
        prod = np.ones(S.shape[0])
        for j in synth.root_path(parent, i):
            prod = prod * a[j].astype(np.float64)
        np.testing.assert_allclose(st[i], prod[:, None, None] * S, rtol=1e-5, atol=1e-7)
    # S_base = 0 at the root: o_0 = s b_0 (k_0 . q_0) v_0.
    o = oracle.gdn_tree(parent, np.zeros_like(S), q, k, v, a, b)
    for h in range(S.shape[0]):
        g = h // 2
        exp = s * b[0, h] * float(k[0, g].astype(np.float64) @ q[0, g]) * v[0, h]
        np.testing.assert_allclose(o[0, h], exp, rtol=1e-5, atol=1e-7)
    # beta = 1 with unit k: the delta rule writes v at key k, k^T S_i = v_i.
    o, st = oracle.gdn_tree(parent, S, q, k, v, a, ones, want_states=True)
    for i in range(len(parent)):
        for h in range(S.shape[0]):
            kk = k[i, h // 2].astype(np.float64)
            np.testing.assert_allclose(st[i, h].astype(np.float64) @ kk, v[i, h],
                                       rtol=0, atol=1e-5)


def pin_gdn_chain_is_sequential():
    # A chain verify equals step-by-step decode with a commit after each step, bit for bit.
    parent, S, q, k, v, a, b = _gdn_case(11, n=6, tree="chain")
    o_tree, st_tree = oracle.gdn_tree(parent, S, q, k, v, a, b, want_states=True)
    cur = S.copy()
    for i in range(6):
        sl = slice(i, i + 1)
        o1 = oracle.gdn_tree([-1], cur, q[sl], k[sl], v[sl], a[sl], b[sl])
        assert np.array_equal(o1[0], o_tree[i])
        cur = oracle.gdn_commit([0], cur, k[sl], v[sl], a[sl], b[sl])
        assert np.array_equal(cur, st_tree[i])
    # and a commit of the whole path equals the tree state at the path's end
    assert np.array_equal(oracle.gdn_commit(list(range(6)), S, k, v, a, b), st_tree[5])


def pin_attn_brute():
    for seed, dtype, sharp in ((1, "f32", False), (2, "bf16", False), (3, "f32", True),
                               (4, "bf16", True)):
        parent, L, Kc, Vc, q, kt, vt = _attn_case(seed, dtype=dtype, sharp=sharp)
        s = float(np.float32(1 / np.sqrt(16)))
        o = oracle.attn_tree(parent, L, Kc, Vc, q, kt, vt)
        ob = brute.attn_tree(parent, L, Kc, Vc, q, kt, vt, s)
        assert brute.rel_err(o, ob) < 1e-5, brute.rel_err(o, ob)


def pin_attn_library():
    torch = pytest.importorskip("torch")
    parent, L, Kc, Vc, q, kt, vt = _attn_case(5, sharp=True)
    n, hq, D = q.shape
    hkv = Kc.shape[0]
    o = oracle.attn_tree(parent, L, Kc, Vc, q, kt, vt)
    vis = np.zeros((n, L + n), bool)
    vis[:, :L] = True
    _, mask, _, _ = oracle.tree_meta(parent)
    for i in range(n):
        for j in range(n):
            vis[i, L + j] = bool((int(mask[i]) >> j) & 1)
    for j in range(hq):
        m = j // (hq // hkv)
        K = np.concatenate([Kc[m, :L], kt[:, m]], 0).astype(np.float64)
        V = np.concatenate([Vc[m, :L], vt[:, m]], 0).astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, j].astype(np.float64))[None], torch.from_numpy(K)[None],
            torch.from_numpy(V)[None], attn_mask=torch.from_numpy(vis)[None],
            scale=1 / np.sqrt(D))[0].numpy()
        assert brute.rel_err(o[:, j], ref) < 1e-5


def pin_attn_closed_forms():
    # Empty context, the root alone: one key of weight 1, o = v_root exactly.
    parent, L, Kc, Vc, q, kt, vt = _attn_case(8, L=0)
    o = oracle.attn_tree(parent, 0, Kc, Vc, q, kt, vt)
    for j in range(q.shape[1]):
        assert np.array_equal(o[0, j], vt[0, j // 3])
    # All keys equal: uniform weights, o = mean of the visible values.
    parent, L, Kc, Vc, q, kt, vt = _attn_case(9, sharp=True)
    Kc[:] = Kc[:, :1]
    kt[:] = Kc[:, 0][None]
    o = oracle.attn_tree(parent, L, Kc, Vc, q, kt, vt)
    for i in range(len(parent)):
        for j in range(q.shape[1]):
            m = j // 3
            rows = [Vc[m, t] for t in range(L)] + [vt[x, m] for x in synth.root_path(parent, i)]
            np.testing.assert_allclose(o[i, j], np.mean(np.asarray(rows, np.float64), 0),
                                       rtol=1e-5, atol=1e-6)


def pin_attn_verify_equals_decode():
    # Row of node i at context L == row of the decode step at L + depth(i) once the
    # ancestors' rows are committed, bit for bit.
    parent, L, Kc, Vc, q, kt, vt = _attn_case(10, dtype="bf16", sharp=True)
    o = oracle.attn_tree(parent, L, Kc, Vc, q, kt, vt)
    for i in range(len(parent)):
        path = synth.root_path(parent, i)
        Kd, Vd = Kc.copy(), Vc.copy()
        Kd[:, L:L + len(path) - 1] = oracle.commit_kv_rows(kt, path[:-1])
        Vd[:, L:L + len(path) - 1] = oracle.commit_kv_rows(vt, path[:-1])
        sl = slice(i, i + 1)
        od = oracle.attn_tree([-1], L + len(path) - 1, Kd, Vd, q[sl], kt[sl], vt[sl])
        assert np.array_equal(od[0], o[i])


def pin_identical_siblings():
    # Two identical subtrees under the root give identical rows, bit for bit.
    parent = [-1, 0, 1, 0, 3]
    gp, S, q, k, v, a, b = _gdn_case(12, n=5)
    for arr in (q, k, v, a, b):
        arr[3:5] = arr[1:3]
    o = oracle.gdn_tree(parent, S, q, k, v, a, b)
    assert np.array_equal(o[1:3], o[3:5])
    _, L, Kc, Vc, q, kt, vt = _attn_case(12, n=5)
    for arr in (q, kt, vt):
        arr[3:5] = arr[1:3]
    o = oracle.attn_tree(parent, L, Kc, Vc, q, kt, vt)
    assert np.array_equal(o[1:3], o[3:5])


def pin_commit_and_rollback_rules():
    parent = [-1, 0, 1, 2, 1, 4]
    assert oracle.leading_chain(parent) == 4
    assert oracle.rollback_plan(parent, 50, 50) == []
    assert oracle.rollback_plan(parent, 50, 53) == [0, 1, 2]
    assert oracle.rollback_plan(parent, 50, 54) == [0, 1, 2, 3]
    assert oracle.rollback_plan(parent, 50, 55) is None
    assert oracle.rollback_plan(parent, 50, 49) is None
    assert oracle.valid_path(parent, [0, 1, 4, 5])
    assert not oracle.valid_path(parent, [0, 4])
    assert not oracle.valid_path(parent, [1, 2])
    kt = np.arange(6 * 2 * 3).reshape(6, 2, 3)
    rows = oracle.commit_kv_rows(kt, [0, 1, 4])
    assert rows.shape == (2, 3, 3) and np.array_equal(rows[1, 2], kt[4, 1])


# ---------------------------------------------------------------------------------------------
# Short causal convolution of the GDN layers
# ---------------------------------------------------------------------------------------------

def _conv_case(seed, n=7, width=4, dtype="f32", tree="random"):
    w = synth.Workload("pin", [0], 2, 4, 8, 6, 2, 1, 8, dtype, [0], n, "random4",
                       extra={"conv": width})
    parent = synth.random_tree(seed, f"pin/conv/{seed}", n, 5) if tree == "random" \
        else synth.chain_tree(n)
    q, k, v, _, _ = synth.conv_inputs(w, seed, 0, 0, n)
    return parent, synth.conv_tail(w, seed, 0, 0), q, k, v, synth.conv_weight(w, seed, 0)


def _wide(x):
    return synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def _library_conv_chain(tail, rows, W, hk=2, dk=8):
    """torch (float64) depthwise conv1d over [tail; rows], then SiLU, then F.normalize of
    every q and k head: [len(rows)][C]."""
    import torch
    import torch.nn.functional as F
    seq = np.concatenate([_wide(tail), _wide(rows)], axis=0).astype(np.float64)
    C, w = W.shape
    x = torch.from_numpy(seq.T.copy())[None]                        # [1][C][T]
    y = F.conv1d(x, torch.from_numpy(W.astype(np.float64))[:, None, :], groups=C)[0].T
    y = F.silu(y)
    cq = hk * dk
    for lo in range(0, 2 * cq, dk):
        y[:, lo:lo + dk] = F.normalize(y[:, lo:lo + dk], dim=1)
    return y.numpy()


def pin_conv_library_chain():
    # A chain over the committed tail is the textbook causal depthwise conv1d.
    for seed, dtype, width in ((21, "f32", 4), (22, "bf16", 4), (23, "f32", 3), (24, "f32", 1)):
        parent, tail, q, k, v, W = _conv_case(seed, n=6, width=width, dtype=dtype, tree="chain")
        got = oracle.conv_rows(*oracle.gdn_conv(parent, tail, q, k, v, W))
        want = _library_conv_chain(tail, oracle.conv_rows(q, k, v), W)
        assert brute.rel_err(got, want) < 1e-5, (seed, brute.rel_err(got, want))


def pin_conv_tree_brute():
    # Every node of a tree equals the library chain conv over its own root path.
    for seed, dtype in ((25, "f32"), (26, "bf16")):
        parent, tail, q, k, v, W = _conv_case(seed, n=9, dtype=dtype)
        got = oracle.conv_rows(*oracle.gdn_conv(parent, tail, q, k, v, W))
        rows = oracle.conv_rows(q, k, v)
        for i in range(len(parent)):
            want = _library_conv_chain(tail, rows[synth.root_path(parent, i)], W)[-1]
            assert brute.rel_err(got[i], want) < 1e-5, (seed, i)


def pin_conv_single_taps():
    # One nonzero tap reads one input: the node itself, or r steps up the path / the tail.
    parent, tail, q, k, v, W = _conv_case(27, n=9)
    d = synth.depths(parent)
    rows, tl = oracle.conv_rows(q, k, v), _wide(tail)
    cq = 2 * 8
    for j in range(4):
        Wj = np.zeros_like(W)
        Wj[:, j] = 1.0
        got = oracle.conv_rows(*oracle.gdn_conv(parent, tail, q, k, v, Wj))
        r = 3 - j
        for i in range(len(parent)):
            path = synth.root_path(parent, i)
            x = rows[path[d[i] - r]] if r <= d[i] else tl[3 - (r - d[i])]
            y = x.astype(np.float64) / (1.0 + np.exp(-x.astype(np.float64)))
            for lo in range(0, 2 * cq, 8):
                y[lo:lo + 8] /= np.sqrt((y[lo:lo + 8] ** 2).sum() + oracle.CONV_EPS)
            np.testing.assert_allclose(got[i], y, rtol=2e-6, atol=1e-7)


def pin_conv_commit_then_decode():
    # Verifying a chain equals decoding it token by token, committing each token's
    # pre-conv row into the tail in between: bit for bit.
    parent, tail, q, k, v, W = _conv_case(28, n=6, dtype="bf16", tree="chain")
    whole = oracle.gdn_conv(parent, tail, q, k, v, W)
    cur = tail.copy()
    for i in range(6):
        sl = slice(i, i + 1)
        one = oracle.gdn_conv([-1], cur, q[sl], k[sl], v[sl], W)
        for a, b in zip(one, whole):
            assert np.array_equal(a[0], b[i])
        cur = oracle.conv_tail_commit(cur, q[sl], k[sl], v[sl], [0])
    # one commit of the whole chain lands on the same tail
    assert np.array_equal(oracle.conv_tail_commit(tail, q, k, v, list(range(6))), cur)
    # hand-checked tail bookkeeping: 3 rows, paths of 1 and of 4 nodes
    t = np.array([[1], [2], [3]], np.float32)
    x = np.array([[10], [11], [12], [13], [14]], np.float32)
    one_col = (x[:, None, :1], x[:, None, :0], x[:, None, :0])  # q only, C = 1
    assert oracle.conv_tail_commit(t, *one_col, [0]).ravel().tolist() == [2, 3, 10]
    assert oracle.conv_tail_commit(t, *one_col, [0, 2, 3, 4]).ravel().tolist() == [12, 13, 14]


def pin_storage_rounding():
    # float32 -> bfloat16 storage rounding equals torch's conversion (nearest even), ties
    # included.
    import torch
    rng = np.random.default_rng(29)
    x = rng.standard_normal(4096).astype(np.float32) * 10
    ties = (rng.integers(0, 0x7F00, 512).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, 3.4e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_storage(x, np.zeros(1, np.uint16)), want)
    assert oracle.to_storage(x, x) is not None and np.array_equal(oracle.to_storage(x, x), x)


# ---------------------------------------------------------------------------------------------
# The accept walk
# ---------------------------------------------------------------------------------------------

def pin_walk_hand_examples():
    g = json.load(open(os.path.join(GOLDEN, "walk_hand_example.json")))
    for c in g["cases"]:
        path, bonus = oracle.greedy_walk(c["parent"], c["draft"], c["target"])
        assert path == c["path"] and bonus == c["bonus"], c["name"]


def _walk_brute(parent, draft, target):
    """Every root path, kept when each of its edges agrees; the longest wins, then the
    lowest last node."""
    best = None
    for x in range(len(parent)):
        path = synth.root_path(parent, x)
        if all(int(draft[c]) == int(target[p]) for p, c in zip(path, path[1:])):
            if best is None or len(path) > len(best):
                best = path
    return best, int(target[best[-1]])


def pin_walk_brute_and_greedy_descent():
    for seed in range(40):
        n = 1 + seed % 33
        parent = synth.random_tree(seed, "pin/walk", n, 1 + seed % 9)
        draft, target = synth.round_tokens(seed, "pin/walk/tokens", parent, vocab=4 + seed % 5,
                                           agree=0.8, distinct=False)
        got = oracle.greedy_walk(parent, draft, target)
        assert got == _walk_brute(parent, draft, target), seed
    # distinct sibling tokens: the walk is the plain greedy descent
    for seed in range(20):
        parent = synth.draft_tree(seed, "pin/walk/draft", 16)
        draft, target = synth.round_tokens(seed, "pin/walk/draft/tokens", parent)
        x = 0
        while True:
            nxt = [c for c in range(len(parent)) if parent[c] == x and draft[c] == target[x]]
            assert len(nxt) <= 1
            if not nxt:
                break
            x = nxt[0]
        assert oracle.greedy_walk(parent, draft, target) == (synth.root_path(parent, x),
                                                             int(target[x]))
        path = synth.accepted_path(seed, "pin/walk/path", parent)
        draft, target = synth.tokens_for_path(seed, "pin/walk/path/tokens", parent, path)
        assert oracle.greedy_walk(parent, draft, target)[0] == path


PINS = {name[4:]: fn for name, fn in list(globals().items()) if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()

"""Parity at the benchmark's full per-layer sizes, on sampled outputs.

Each case runs a slice of the 64-layer stack (three Gated DeltaNet layers and one
attention layer, the stack's own first four layers with their own data) at the full
shapes and resident length of a benchmark workload, with the same tree, the same slot
capacity and therefore the same kernel shapes as bench.py.  Every GDN output is checked
against the oracle; attention rows are checked on a sample of (node, q head) rows that
the oracle computes one by one over the full resident context.  After the pass a
seeded path is committed and the committed state and cache rows are checked.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_host
from tests import gpu_util as gu
from tests.brute import rel_err

pytestmark = pytest.mark.gpu

SEED = 20261202
FIRST4 = [0, 0, 0, 1]


def _slice(w):
    return synth.Workload(w.name, FIRST4, w.gdn_hk, w.gdn_hv, w.gdn_dk, w.gdn_dv, w.attn_hq,
                          w.attn_hkv, w.attn_d, w.dtype, w.lengths, w.n_nodes, w.tree_kind,
                          w.max_depth, extra=dict(w.extra))


def _say(msg):
    print(msg, flush=True)


def _check_gdn(inst, s, l):
    got = gu.outputs(inst, s)[l]
    err = gu.check_layer(inst, s, l, got)
    _say(f"  slot {s} layer {l} (GDN): max relative error {err:.2e}")


def _check_attn_sampled(inst, s, l, nodes, heads):
    """Rows (node, j) of attention layer l of slot s against the oracle's row routine."""
    w, h = inst.w, inst.host[s][l]
    ai = sum(1 for x in w.layer_kind[:l] if x == 1)
    got = gu.outputs(inst, s)[l]
    assert np.isfinite(got).all()
    worst = ew = 0.0
    for j in heads:
        ref = np.stack([oracle.attn_row(inst.trees[s], inst.lengths[s], inst.h_kc[s][ai],
                                        inst.h_vc[s][ai], h["q"], h["k"], h["v"], i, j)
                        for i in nodes])
        err = rel_err(got[nodes, j], ref)
        worst = max(worst, err)
        ew = max(ew, gu.elementwise_worst(got[nodes, j][:, None], ref[:, None]))
        assert err <= gu.TOL_BF16_OUT, f"slot {s} layer {l} q head {j}: {err:.3e}"
    _say(f"  slot {s} layer {l} (attention, {len(nodes)} nodes x {len(heads)} heads): "
         f"max relative error {worst:.2e}, elementwise worst {ew:.2e}")


def _check_commit(inst, eng, s, path):
    """commit_tree(path): GDN state against the oracle's sequential recurrence; the new
    cache rows bit for bit."""
    w = inst.w
    L = inst.lengths[s]
    eng.commit_tree(s, path, gu.stream())
    gu.sync()
    gi = ai = 0
    for l, kind in enumerate(w.layer_kind):
        h = inst.host[s][l]
        if kind == 0:
            k, v = h["k"], h["v"]
            if inst.conv > 0:  # the recurrence ran on the stored post-conv activations
                _, (_, k, v) = oracle.gdn_conv_layer(inst.trees[s], inst.h_state[s][gi],
                                                     inst.h_tail[s][gi], h["q"], h["k"], h["v"],
                                                     h["alpha"], h["beta"], inst.h_conv_w[gi])
                want = oracle.conv_tail_commit(inst.h_tail[s][gi], h["q"], h["k"], h["v"], path)
                assert np.array_equal(to_host(inst.tail[s][gi], w.dtype), want), \
                    f"slot {s} layer {l}: committed conv tail"
            ref = oracle.gdn_commit(path, inst.h_state[s][gi], k, v, h["alpha"], h["beta"])
            got = inst.state[s][gi].cpu().numpy()
            for hh in range(w.gdn_hv):  # per head (P17)
                err = rel_err(got[hh], ref[hh])
                assert err <= gu.TOL_F32, f"slot {s} layer {l} head {hh}: committed state {err:.3e}"
            gi += 1
        else:
            m = len(path)
            for name, cache in (("k", inst.kc[s]), ("v", inst.vc[s])):
                got = to_host(cache[ai, :, L:L + m], w.dtype)
                want = oracle.commit_kv_rows(h[name], path)
                assert np.array_equal(got, want), f"slot {s} layer {l}: committed {name} rows"
            ai += 1
    assert eng.kv_length(s) == L + len(path)
    _say(f"  slot {s}: commit of a {len(path)}-node path matches")


def _bench_capacity(w, parent):
    """The slot capacity bench.py allocates for the default run (it sets the split size)."""
    path = synth.accepted_path(SEED, f"{w.name}/bench-path", parent)
    return w.lengths[0] + (10 + 2 * 50) * len(path) + 64


def _nodes_sample(parent):
    d = synth.depths(parent)
    leaves = [i for i in range(len(parent)) if i not in parent]
    deepest = max(range(len(parent)), key=lambda i: d[i])
    return sorted(set([0, 1, len(parent) // 2, deepest] + leaves[:2]))


def test_stack65k_slice_at_full_size():
    """The 65,536-token, 16-node workload of the benchmark: 96 query rows per kv head
    (the 6-computing-wave split shape), 1,056-key splits."""
    w = _slice(synth.WORKLOADS["stack_65k"])
    parent = synth.WORKLOADS["stack_65k"].tree(SEED, 0)
    cap = _bench_capacity(synth.WORKLOADS["stack_65k"], parent)
    _say(f"stack_65k slice: L={w.lengths[0]} nodes={len(parent)} capacity={cap}")
    inst = Instance(w, SEED, trees=[parent], capacity=[cap])
    eng = inst.engine(max_nodes=len(parent))
    assert eng.split_size(0, w.lengths[0]) == 1056
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    for l in range(3):
        _check_gdn(inst, 0, l)
    heads = [0, 5, 6, 11, 12, 17, 18, 23]  # first and last q head of every kv head
    _check_attn_sampled(inst, 0, 3, list(range(len(parent))), heads)
    _check_commit(inst, eng, 0, synth.accepted_path(SEED, "full/c2-path", parent))
    eng.close()


def test_stack65k_conv_slice_at_full_size():
    """The 65,536-token, 16-node workload with the width-4 conv in front of every GDN
    layer: pre-conv inputs, committed tails, tails rolled by commit."""
    base = synth.WORKLOADS["stack_65k_conv"]
    w = _slice(base)
    parent = base.tree(SEED, 0)
    cap = _bench_capacity(base, parent)
    _say(f"stack_65k_conv slice: L={w.lengths[0]} nodes={len(parent)} capacity={cap}")
    inst = Instance(w, SEED, trees=[parent], capacity=[cap])
    eng = inst.engine(max_nodes=len(parent))
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    for l in range(3):
        _check_gdn(inst, 0, l)
    _check_attn_sampled(inst, 0, 3, _nodes_sample(parent), [0, 11, 23])
    _check_commit(inst, eng, 0, synth.accepted_path(SEED, "full/conv-path", parent))
    eng.close()


def test_stack262k_slice_at_full_size():
    """262,144 resident tokens and a 32-node tree: 192 query rows per kv head (the
    four-wave, three-block split shape)."""
    base = synth.WORKLOADS["stack_262k"]
    w = _slice(base)
    parent = base.tree(SEED, 0)
    _say(f"stack_262k slice: L={w.lengths[0]} nodes={len(parent)}")
    inst = Instance(w, SEED, trees=[parent], capacity=[_bench_capacity(base, parent)])
    eng = inst.engine(max_nodes=len(parent))
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    for l in range(3):
        _check_gdn(inst, 0, l)
    _check_attn_sampled(inst, 0, 3, _nodes_sample(parent), [0, 7, 14, 23])
    _check_commit(inst, eng, 0, synth.accepted_path(SEED, "full/c3-path", parent))
    eng.close()


def test_joint4_slice_at_full_size():
    """Four slots in one pass (131,072 + 3 x 8,192 resident tokens, 16 nodes each): every
    slot's rows against the oracle, then a commit on one slot and a rollback on another."""
    base = synth.WORKLOADS["joint4"]
    w = _slice(base)
    _say(f"joint4 slice: L={w.lengths}")
    inst = Instance(w, SEED)
    eng = inst.engine()
    eng.forward_tree([inst.tree_arg(s) for s in range(w.n_slots)], gu.stream())
    gu.sync()
    for s in range(w.n_slots):
        for l in range(3):
            _check_gdn(inst, s, l)
        _check_attn_sampled(inst, s, 3, _nodes_sample(inst.trees[s]), [0, 11, 23])
    _check_commit(inst, eng, 0, synth.accepted_path(SEED, "full/c4-path", inst.trees[0]))
    L1 = inst.lengths[1]
    eng.rollback_to(1, L1, gu.stream())
    gu.sync()
    assert eng.kv_length(1) == L1
    eng.close()


# ------------------------------------------------------------------------------ peaked and loud

def _base2_scores(inst, s, l, node, j):
    """Base-2 scores c2 q.k of row (node, q head j) over the committed keys (float64)."""
    w, h = inst.w, inst.host[s][l]
    ai = sum(1 for x in w.layer_kind[:l] if x == 1)
    m = j // (w.attn_hq // w.attn_hkv)
    L = inst.lengths[s]
    q = synth.bf16_bits_to_f32(h["q"][node, j]).astype(np.float64)
    K = synth.bf16_bits_to_f32(inst.h_kc[s][ai][m, :L]).astype(np.float64)
    return (K @ q) * (1.0 / np.sqrt(w.attn_d)) / np.log(2.0)


def _rescales(scores, split, tile=32, lazy=8.0):
    """How often, within a split, a tile's max exceeds the running max by more than `lazy`
    (the rule under which the running max moves after a split's first tile)."""
    count = 0
    for s0 in range(0, len(scores), split):
        run = -np.inf
        for t0 in range(s0, min(s0 + split, len(scores)), tile):
            mt = scores[t0:t0 + tile].max()
            if run > -np.inf and mt > run + lazy:
                count += 1
            if mt > run + lazy or run == -np.inf:
                run = mt
    return count


@pytest.mark.parametrize("wname", ["stack_65k", "stack_262k"])
def test_peaked_softmax_slice_at_full_size(wname):
    """Unnormalised keys and queries drawn as 6 N(0,1): scores spread over tens of units, so
    within the 1,056-key (65,536) and 8,384-key (262,144) splits the running max moves after
    the first tile, and the split maxima differ widely in the fold.  Sampled rows against
    the oracle's row routine."""
    base = synth.WORKLOADS[wname]
    w = _slice(base)
    parent = base.tree(SEED, 0)
    cap = _bench_capacity(base, parent)
    _say(f"{wname} slice, peaked softmax: L={w.lengths[0]} nodes={len(parent)}")
    inst = Instance(w, SEED, trees=[parent], capacity=[cap], sharp=True, q_scale=6.0)
    eng = inst.engine(max_nodes=len(parent))
    split = eng.split_size(0, w.lengths[0])
    assert split == (1056 if wname == "stack_65k" else 8384)  # 8,384: two row groups at 32 nodes
    moves = sum(_rescales(_base2_scores(inst, 0, 3, i, j), split) for i in (0, len(parent) - 1) for j in (0, 23))
    assert moves > 0, "the inputs never move the running max inside a split"
    _say(f"  running-max moves inside splits (4 sampled rows, from the inputs): {moves}")
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    _check_attn_sampled(inst, 0, 3, _nodes_sample(parent), [0, 7, 14, 23])
    eng.close()


@pytest.mark.parametrize("wname", ["stack_65k", "stack_262k"])
def test_loud_tree_rows_slice_at_full_size(wname):
    """Tree value rows scaled by 4,096 (a power of two, so the bf16 rows stay exact): under
    the flat softmax of unit keys each tree row then carries a visible share of its
    descendants' outputs, so a missing, extra or misplaced ancestor row moves a sampled row
    far past 2e-2.  Every node's rows are checked on four q heads."""
    base = synth.WORKLOADS[wname]
    w = _slice(base)
    parent = base.tree(SEED, 0)
    cap = _bench_capacity(base, parent)
    _say(f"{wname} slice, loud tree rows: L={w.lengths[0]} nodes={len(parent)}")
    inst = Instance(w, SEED, trees=[parent], capacity=[cap], v_scale=4096.0)
    eng = inst.engine(max_nodes=len(parent))
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    # the tree rows dominate: without them an output row is a flat average of unit-variance
    # values over the whole context, about 1 / sqrt(L) in size
    got = gu.outputs(inst, 0)[3]
    assert np.abs(got).max() > 25.0 / np.sqrt(w.lengths[0])
    _check_attn_sampled(inst, 0, 3, list(range(len(parent))), [0, 7, 14, 23])
    eng.close()


def test_verify_equals_decode_at_65536():
    """verified row == decode row bit for bit at the benchmark's length: the shortest leaf
    path of the draft tree, decoded token by token through the four-layer slice (1,056-key
    splits, the fold over 62 committed splits)."""
    base = synth.WORKLOADS["stack_65k"]
    w = _slice(base)
    parent = base.tree(SEED, 0)
    L = w.lengths[0]
    inst = Instance(w, SEED, trees=[parent], capacity=[_bench_capacity(base, parent)])
    eng = inst.engine(max_nodes=len(parent))
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    verified = gu.raw_outputs(inst, 0)
    eng.rollback_to(0, L, gu.stream())
    d = synth.depths(parent)
    leaves = [i for i in range(len(parent)) if i not in parent]
    leaf = min(leaves, key=lambda i: (d[i], i))
    path = synth.root_path(parent, leaf)
    _say(f"stack_65k slice: decode of leaf {leaf}'s root path {path} at L={L}")
    for j in path:
        step_io = gu.row_io(inst, 0, j)
        eng.forward_tree([(0, [-1], step_io)], gu.stream())
        eng.commit_tree(0, [0], gu.stream())
        gu.sync()
        for l in range(4):
            row = to_host(step_io[l]["o"], w.dtype)[0]
            assert np.array_equal(row, verified[l][j]), f"node {j} layer {l}: verify row != decode row"
    eng.close()

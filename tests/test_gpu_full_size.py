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
    worst = 0.0
    for j in heads:
        ref = np.stack([oracle.attn_row(inst.trees[s], inst.lengths[s], inst.h_kc[s][ai],
                                        inst.h_vc[s][ai], h["q"], h["k"], h["v"], i, j)
                        for i in nodes])
        err = rel_err(got[nodes, j], ref)
        worst = max(worst, err)
        assert err <= gu.TOL_BF16_OUT, f"slot {s} layer {l} q head {j}: {err:.3e}"
    _say(f"  slot {s} layer {l} (attention, {len(nodes)} nodes x {len(heads)} heads): "
         f"max relative error {worst:.2e}")


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
            err = rel_err(got, ref)
            assert err <= gu.TOL_F32, f"slot {s} layer {l}: committed state {err:.3e}"
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
    return w.lengths[0] + (5 + 2 * 20) * len(path) + 64


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

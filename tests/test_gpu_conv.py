"""GPU parity of the short causal conv in front of the GDN layers (the gdn.conv state
section), through the C ABI:

  * every layer's output vs the oracle's conv -> stored activations -> recurrence
    (2e-2 for bf16 outputs, 2e-3 for float32);
  * commit_tree: recurrent state vs the oracle (2e-3), conv tails bit for bit;
  * verified row == sequential decode row, bit for bit, and the state and tails after a
    commit equal those after decoding the same path;
  * rollback_to a chain prefix rolls the tails like commit_tree of that prefix;
  * joint verify of two conv slots == each alone, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_host
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SEED = 20261203
CONV_MINI = synth.Workload("conv_mini", [0, 1, 0, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16",
                           [1000], 16, "draft", extra={"conv": 4})
CONV_TINY = synth.Workload("conv_tiny", [0, 1, 0], 1, 2, 64, 64, 2, 1, 64, "f32", [256], 8,
                           "random4", 4, extra={"conv": 3})
CONV_W1 = synth.Workload("conv_w1", [0, 0, 1], 4, 8, 128, 128, 12, 2, 256, "bf16", [700], 12,
                         "draft", extra={"conv": 1})
CONV_W2 = synth.Workload("conv_w2", [0, 1], 4, 8, 64, 64, 12, 2, 256, "bf16", [513], 24,
                         "draft", extra={"conv": 2})
WL = {w.name: w for w in (CONV_MINI, CONV_TINY, CONV_W1, CONV_W2)}


def run_verify(inst, eng, slots=None):
    slots = range(len(inst.lengths)) if slots is None else slots
    eng.forward_tree([inst.tree_arg(s) for s in slots], gu.stream())
    gu.sync()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("wname", sorted(WL))
def test_conv_forward_matches_oracle(wname):
    w = WL[wname]
    _say(f"conv forward {wname}: width {w.extra['conv']}, {w.n_nodes} nodes, L={w.lengths[0]}")
    inst = Instance(w, SEED)
    eng = inst.engine()
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(len(w.layer_kind)):
        err = gu.check_layer(inst, 0, l, got[l])
        _say(f"  layer {l}: max relative error {err:.2e}")
    eng.close()


def _oracle_commit(inst, eng, path, s=0):
    """Commit `path` and check every GDN layer's state and tail and every attention
    layer's rows against the oracle."""
    w, L = inst.w, inst.lengths[s]
    eng.commit_tree(s, path, gu.stream())
    gu.sync()
    gi = ai = 0
    for l, kind in enumerate(w.layer_kind):
        h = inst.host[s][l]
        if kind == 0:
            _, (qc, kc, vc) = oracle.gdn_conv_layer(inst.trees[s], inst.h_state[s][gi],
                                                    inst.h_tail[s][gi], h["q"], h["k"], h["v"],
                                                    h["alpha"], h["beta"], inst.h_conv_w[gi])
            ref = oracle.gdn_commit(path, inst.h_state[s][gi], kc, vc, h["alpha"], h["beta"])
            got = inst.state[s][gi].cpu().numpy()
            for hh in range(w.gdn_hv):
                assert gu.rel_err(got[hh], ref[hh]) <= gu.TOL_F32, f"layer {l} head {hh}"
            if inst.conv > 1:
                want = oracle.conv_tail_commit(inst.h_tail[s][gi], h["q"], h["k"], h["v"], path)
                assert np.array_equal(to_host(inst.tail[s][gi], w.dtype), want), f"layer {l} tail"
            gi += 1
        else:
            m = len(path)
            for name, cache in (("k", inst.kc[s]), ("v", inst.vc[s])):
                rows = to_host(cache[ai, :, L:L + m], w.dtype)
                assert np.array_equal(rows, oracle.commit_kv_rows(h[name], path))
            ai += 1
    assert eng.kv_length(s) == L + len(path)


@pytest.mark.parametrize("wname", ["conv_mini", "conv_tiny", "conv_w2"])
def test_conv_commit_matches_oracle(wname):
    w = WL[wname]
    inst = Instance(w, SEED)
    eng = inst.engine()
    run_verify(inst, eng)
    path = synth.accepted_path(SEED, f"{wname}/path", inst.trees[0])
    _say(f"conv commit {wname}: path of {len(path)}")
    _oracle_commit(inst, eng, path)
    eng.close()


def decode_rows_along(inst, eng, node, s=0):
    outs = []
    for j in synth.root_path(inst.trees[s], node):
        step_io = gu.row_io(inst, s, j)
        eng.forward_tree([(s, [-1], step_io)], gu.stream())
        eng.commit_tree(s, [0], gu.stream())
        gu.sync()
        outs.append([to_host(io["o"], inst.w.dtype).copy() for io in step_io])
    return outs


@pytest.mark.parametrize("wname", ["conv_mini", "conv_tiny", "conv_w2"])
def test_conv_verify_row_equals_decode_row(wname):
    w = WL[wname]
    inst = Instance(w, SEED)
    parent, L = inst.trees[0], inst.lengths[0]
    eng = inst.engine()
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    verified = gu.raw_outputs(inst, 0)
    eng.rollback_to(0, L)
    leaves = [i for i in range(len(parent)) if i not in parent]
    _say(f"conv verify == decode {wname}: {len(leaves)} leaves")
    for leaf in leaves[:4]:
        gu.restore(inst, snap)
        eng.reset(0, L)
        outs = decode_rows_along(inst, eng, leaf)
        for step, j in enumerate(synth.root_path(parent, leaf)):
            for l in range(len(w.layer_kind)):
                assert np.array_equal(outs[step][l][0], verified[l][j]), \
                    f"leaf {leaf} node {j} layer {l}: verify row != decode row"
    eng.close()


def test_conv_committed_equals_decoded():
    inst = Instance(CONV_MINI, SEED)
    eng = inst.engine()
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    path = synth.accepted_path(SEED, "conv_mini/path2", inst.trees[0])
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    committed = (inst.state[0].clone(), inst.tail[0].clone())
    gu.restore(inst, snap)
    eng.reset(0, 1000)
    decode_rows_along(inst, eng, path[-1])
    assert torch.equal(inst.state[0], committed[0])
    assert torch.equal(inst.tail[0], committed[1])
    eng.close()


def test_conv_rollback_keeps_chain_prefix_like_commit():
    inst = Instance(CONV_MINI, SEED)
    parent = inst.trees[0]
    c = oracle.leading_chain(parent)
    keep = max(1, c - 1)
    eng = inst.engine()
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    eng.rollback_to(0, 1000 + keep, gu.stream())
    gu.sync()
    rolled = (inst.state[0].clone(), inst.tail[0].clone())
    gu.restore(inst, snap)
    eng.reset(0, 1000)
    run_verify(inst, eng)
    _oracle_commit(inst, eng, list(range(keep)))
    assert torch.equal(inst.state[0], rolled[0])
    assert torch.equal(inst.tail[0], rolled[1])
    eng.close()


def test_conv_joint_equals_lone():
    w = synth.Workload("conv_joint", [0, 1, 0], 16, 32, 128, 128, 24, 4, 256, "bf16",
                       [1000, 300], 16, "draft", extra={"conv": 4})
    inst = Instance(w, SEED)
    eng = inst.engine()
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    joint = [gu.raw_outputs(inst, s) for s in range(2)]
    for s in range(2):
        eng.rollback_to(s, inst.lengths[s])
    for s in range(2):
        gu.restore(inst, snap)
        run_verify(inst, eng, slots=[s])
        lone = gu.raw_outputs(inst, s)
        eng.rollback_to(s, inst.lengths[s])
        for l in range(len(w.layer_kind)):
            assert np.array_equal(lone[l], joint[s][l]), f"slot {s} layer {l}"
    eng.close()

"""GPU parity: the HIP path through the C ABI against the CPU oracle, and the pages'
bit-exact invariants on the GPU.

  * outputs of every layer vs the oracle (max relative error per (layer, head) tensor:
    2e-2 for bf16 outputs, 2e-3 for float32 outputs and state);
  * commit_tree: state vs the oracle's sequential recurrence (2e-3), K/V rows bit-exact;
  * verified row == sequential decode row, bit for bit ("Adding a model", step 4 of
    "The adapter path in ten steps");
  * joint verify == lone verify, bit for bit ("Parallel requests", "On Flash-Next");
  * edge cases: empty context, one node, 64 nodes, trees across split boundaries,
    rows past the committed length holding NaN.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_host
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # the gpu marker selects these; collection still works on CPU
    pytest.skip("no GPU", allow_module_level=True)

import hybrid_deltanet_tree_amd as hdt  # noqa: E402

SEED = 20261202
W = synth.WORKLOADS

# Small bf16 workload with the 27B-like head shapes: 2 GDN + 2 attention layers.
MINI = synth.Workload("mini", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000], 16,
                      "draft")
# 20-node trees at 6 q heads per kv head: 120 query rows, two row groups per split
RG2 = synth.Workload("rg2", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1300], 20,
                     "draft")


def run_verify(inst, eng, slots=None):
    slots = range(len(inst.lengths)) if slots is None else slots
    eng.forward_tree([inst.tree_arg(s) for s in slots], gu.stream())
    gu.sync()


# ------------------------------------------------------------------------------ oracle parity

@pytest.mark.parametrize("wname,L", [("tiny", 256), ("tiny", 0), ("tiny", 301), ("pair_8k", 8192)])
def test_forward_matches_oracle(wname, L):
    inst = Instance(W[wname], SEED, lengths=[L])
    eng = inst.engine()
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(len(inst.w.layer_kind)):
        gu.check_layer(inst, 0, l, got[l])


@pytest.mark.parametrize("L", [1300, 2017])
def test_two_row_groups_match_oracle(L):
    """More than 96 query rows per kv head: the split pass runs two row groups per split
    (on one XCD), with the split size scaled to keep one wave of workgroups."""
    inst = Instance(RG2, SEED, lengths=[L])
    eng = inst.engine(max_nodes=20)
    assert eng.split_size(0, L) % 32 == 0
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(len(RG2.layer_kind)):
        gu.check_layer(inst, 0, l, got[l])


def test_bf16_small_heads():
    # bf16 storage with d_k = d_v = 64 and D = 64: the narrow-slice code paths
    w = synth.Workload("bf16_64", [0, 1, 0, 1], 2, 4, 64, 64, 4, 2, 64, "bf16", [700], 12, "draft")
    inst = Instance(w, SEED)
    eng = inst.engine()
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(4):
        gu.check_layer(inst, 0, l, got[l])
    path = synth.accepted_path(SEED, "bf16_64/path", inst.trees[0])
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    for gi, l in enumerate((0, 2)):
        h = inst.host[0][l]
        ref = oracle.gdn_commit(path, inst.h_state[0][gi], h["k"], h["v"], h["alpha"], h["beta"])
        assert gu.rel_err(inst.state[0][gi].cpu().numpy(), ref) <= gu.TOL_F32


def test_forward_matches_oracle_sharp_softmax():
    # unnormalised q, k: a peaked softmax exercises the running max and rescaling
    inst = Instance(MINI, SEED, lengths=[777], sharp=True)
    eng = inst.engine()
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(4):
        gu.check_layer(inst, 0, l, got[l])


def test_resident_values_past_the_fp16_range():
    # resident V of magnitude ~2^20 (split averages past 65,504) over many splits: the partials keep
    # the float32 range, so every output is finite and matches the oracle
    inst = Instance(MINI, SEED, lengths=[6000], kv_v_scale=1048576.0)
    eng = inst.engine()
    assert eng.split_size(0, 6000) < 6000  # several committed splits per row
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(4):
        assert np.isfinite(got[l]).all(), f"layer {l}"
        gu.check_layer(inst, 0, l, got[l])


@pytest.mark.parametrize("wname,L", [("tiny", 256), ("mini", 1000)])
def test_commit_matches_oracle(wname, L):
    w = MINI if wname == "mini" else W[wname]
    inst = Instance(w, SEED, lengths=[L])
    kc0, vc0 = inst.kc[0].clone(), inst.vc[0].clone()
    eng = inst.engine()
    run_verify(inst, eng)
    path = synth.accepted_path(SEED, f"{wname}/path", inst.trees[0])
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + len(path)
    gi = ai = 0
    for l, kind in enumerate(w.layer_kind):
        h = inst.host[0][l]
        if kind == 0:
            ref = oracle.gdn_commit(path, inst.h_state[0][gi], h["k"], h["v"], h["alpha"], h["beta"])
            got = inst.state[0][gi].cpu().numpy()
            for hh in range(w.gdn_hv):
                assert gu.rel_err(got[hh], ref[hh]) <= gu.TOL_F32
            gi += 1
        else:
            m = len(path)
            for name, cache, c0 in (("k", inst.kc[0], kc0), ("v", inst.vc[0], vc0)):
                rows = to_host(cache[ai, :, L:L + m], w.dtype)
                assert np.array_equal(rows, oracle.commit_kv_rows(h[name], path))
                assert torch.equal(cache[ai, :, :L], c0[ai, :, :L])
            ai += 1


# ------------------------------------------------------------------------------ invariants

def decode_rows_along(inst, eng, node, s=0):
    """Decode the root path of `node` one token at a time (1-node tree + commit) from the
    slot's current state; return each step's raw outputs."""
    outs = []
    for j in synth.root_path(inst.trees[s], node):
        step_io = gu.row_io(inst, s, j)
        eng.forward_tree([(s, [-1], step_io)], gu.stream())
        eng.commit_tree(s, [0], gu.stream())
        gu.sync()
        outs.append([to_host(io["o"], inst.w.dtype).copy() for io in step_io])
    return outs


@pytest.mark.parametrize("wname,L,tree", [("tiny", 256, "chain"), ("tiny", 250, "random"),
                                          ("mini", 1000, "draft"), ("mini", 1275, "draft"),
                                          ("rg2", 1300, "draft"), ("mini", 8185, "draft")])
def test_verify_row_equals_decode_row(wname, L, tree):
    w = {"mini": MINI, "rg2": RG2}.get(wname) or W[wname]
    parent = synth.chain_tree(8) if tree == "chain" else w.tree(SEED + L)
    inst = Instance(w, SEED, lengths=[L], trees=[parent])
    eng = inst.engine(max_nodes=len(parent))
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    verified = gu.raw_outputs(inst, 0)
    eng.rollback_to(0, L)
    leaves = [i for i in range(len(parent)) if i not in parent]
    for leaf in leaves:
        gu.restore(inst, snap)
        eng.reset(0, L)
        outs = decode_rows_along(inst, eng, leaf)
        for step, j in enumerate(synth.root_path(parent, leaf)):
            for l in range(len(w.layer_kind)):
                assert np.array_equal(outs[step][l][0], verified[l][j]), \
                    f"leaf {leaf} node {j} layer {l}: verify row != decode row"


def test_committed_state_equals_decoded_state():
    inst = Instance(MINI, SEED, lengths=[1000])
    eng = inst.engine()
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    path = synth.accepted_path(SEED, "mini/path2", inst.trees[0])
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    committed = [t.clone() for t in (inst.state[0], inst.kc[0], inst.vc[0])]
    gu.restore(inst, snap)
    eng.reset(0, 1000)
    decode_rows_along(inst, eng, path[-1])
    assert torch.equal(inst.state[0], committed[0])
    assert torch.equal(inst.kc[0][:, :, :1000 + len(path)], committed[1][:, :, :1000 + len(path)])
    assert torch.equal(inst.vc[0][:, :, :1000 + len(path)], committed[2][:, :, :1000 + len(path)])


@pytest.mark.parametrize("L", [8185, 8190])
def test_rows_straddling_a_split_rung(L):
    """A tree whose rows straddle a rung of the split ladder: at 64 splits per kv head,
    rows that see up to 8,192 keys take 128-key splits and deeper rows 160-key splits, so
    the layer runs two launch pairs, one per node group.  Both groups match the oracle."""
    inst = Instance(MINI, SEED, lengths=[L])
    eng = inst.engine()
    d = synth.depths(inst.trees[0])
    assert {eng.split_size(0, L + x) for x in d} == {128, 160}
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(len(MINI.layer_kind)):
        gu.check_layer(inst, 0, l, got[l])
    eng.close()


def test_capacity_does_not_change_bits():
    """The same tree at the same length in slots of very different capacity: the split
    size follows each row's position, so every output bit is the same."""
    outs = []
    for cap in (1000 + 64, 1 << 17):
        inst = Instance(MINI, SEED, lengths=[1000], capacity=[cap])
        eng = inst.engine()
        run_verify(inst, eng)
        outs.append(gu.raw_outputs(inst, 0))
        eng.close()
    for l in range(len(MINI.layer_kind)):
        assert np.array_equal(outs[0][l], outs[1][l]), f"layer {l}"


def test_joint_with_a_straddling_tree_equals_lone():
    w = synth.Workload("joint_straddle", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16",
                       [8185, 1000], 16, "draft")
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


def test_joint_equals_lone():
    w = synth.Workload("joint_mini", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16",
                       [1000, 300, 1300], 16, "draft")
    inst = Instance(w, SEED)
    snap = gu.snapshot(inst)
    eng = inst.engine()
    run_verify(inst, eng, [0, 1, 2])
    joint = [gu.raw_outputs(inst, s) for s in range(3)]
    paths = [synth.accepted_path(SEED, f"joint/{s}", inst.trees[s]) for s in range(3)]
    for s in range(3):
        eng.commit_tree(s, paths[s], gu.stream())
    gu.sync()
    joint_state = [(inst.state[s].clone(), inst.kc[s].clone(), inst.vc[s].clone()) for s in range(3)]
    gu.restore(inst, snap)
    for s in range(3):
        for io in inst.io[s]:
            io["o"].zero_()
        eng.reset(s, w.lengths[s])
    for s in (2, 0, 1):
        run_verify(inst, eng, [s])
        lone = gu.raw_outputs(inst, s)
        for l in range(4):
            assert np.array_equal(lone[l], joint[s][l]), f"slot {s} layer {l}"
        eng.commit_tree(s, paths[s], gu.stream())
        gu.sync()
        for a, b in zip((inst.state[s], inst.kc[s], inst.vc[s]), joint_state[s]):
            assert torch.equal(a, b)


def test_joint_of_eight_trees_mixed_sizes():
    """The most trees one call takes (8): lengths 0 .. 2,100 with one slot filled to its
    capacity exactly, trees of 1 to 64 nodes (so the split pass mixes row groups); every
    slot's rows equal its lone verify bit for bit, and two slots match the oracle."""
    lengths = [0, 1, 31, 257, 1000, 1300, 2047, 2100]
    trees = [[-1], synth.chain_tree(2), synth.draft_tree(SEED, "j8/16", 16),
             synth.random_tree(SEED, "j8/64", 64, 6), synth.chain_tree(5),
             synth.draft_tree(SEED, "j8/20", 20), synth.random_tree(SEED, "j8/9", 9, 3),
             synth.draft_tree(SEED, "j8/16b", 16)]
    w = synth.Workload("joint8", [0, 1, 0, 1], 4, 8, 128, 128, 12, 2, 256, "bf16", lengths, 64,
                       "draft")
    caps = [L + len(t) + 64 for L, t in zip(lengths, trees)]
    caps[6] = lengths[6] + len(trees[6])  # filled exactly
    inst = Instance(w, SEED, trees=trees, capacity=caps)
    eng = inst.engine(max_nodes=64)
    snap = gu.snapshot(inst)
    run_verify(inst, eng, list(range(8)))
    joint = [gu.raw_outputs(inst, s) for s in range(8)]
    for s in (3, 6):
        got = gu.outputs(inst, s)
        for l in range(4):
            gu.check_layer(inst, s, l, got[l])
    for s in range(8):
        eng.rollback_to(s, lengths[s])
    for s in range(8):
        gu.restore(inst, snap)
        for io in inst.io[s]:
            io["o"].zero_()
        run_verify(inst, eng, [s])
        lone = gu.raw_outputs(inst, s)
        eng.rollback_to(s, lengths[s])
        for l in range(4):
            assert np.array_equal(lone[l], joint[s][l]), f"slot {s} layer {l}"
    eng.close()


# ------------------------------------------------------------------------------ edge cases

def test_empty_context_root_returns_its_value():
    inst = Instance(W["tiny"], SEED, lengths=[0])
    eng = inst.engine()
    run_verify(inst, eng)
    o = gu.outputs(inst, 0)[1]
    v = inst.host[0][1]["v"]
    for j in range(2):
        assert np.array_equal(o[0, j], v[0, 0])


@pytest.mark.parametrize("L", [255, 256, 200])
def test_deep_chain_of_64_across_splits(L):
    w = synth.Workload("tiny64", [0, 1], 1, 1, 64, 64, 2, 1, 64, "f32", [L], 64, "random4")
    inst = Instance(w, SEED, trees=[synth.chain_tree(64)])
    eng = inst.engine(max_nodes=64)
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(2):
        gu.check_layer(inst, 0, l, got[l])


def test_many_branch_points_replay_from_committed_state():
    """A bushy 64-node tree: more branch points than the walk keeps in LDS, so some parents
    are restored by replaying their root path from the committed state (the ancestor
    table is built).  Outputs against the oracle; verified rows equal decoded rows."""
    w = synth.Workload("bushy", [0, 1], 4, 8, 128, 128, 12, 2, 256, "bf16", [700], 64, "random4")
    parent = synth.random_tree(SEED, "bushy", 64, 5)
    branch = {parent[c] for c in range(1, 64) if parent[c] != c - 1}
    assert len(branch) > 8  # beyond the 8 kept states
    inst = Instance(w, SEED, trees=[parent])
    eng = inst.engine(max_nodes=64)
    snap = gu.snapshot(inst)
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(2):
        gu.check_layer(inst, 0, l, got[l])
    verified = gu.raw_outputs(inst, 0)
    eng.rollback_to(0, 700)
    leaves = [i for i in range(64) if i not in parent]
    for leaf in leaves[-3:]:
        gu.restore(inst, snap)
        eng.reset(0, 700)
        outs = decode_rows_along(inst, eng, leaf)
        for step, j in enumerate(synth.root_path(parent, leaf)):
            for l in range(2):
                assert np.array_equal(outs[step][l][0], verified[l][j]), f"leaf {leaf} node {j} layer {l}"
    eng.close()


def test_single_node_and_nan_past_length():
    inst = Instance(MINI, SEED, lengths=[1000], trees=[[-1]], poison=True)
    eng = inst.engine()
    run_verify(inst, eng)
    got = gu.outputs(inst, 0)
    for l in range(4):
        gu.check_layer(inst, 0, l, got[l])
    inst2 = Instance(MINI, SEED, lengths=[1000], poison=True)
    eng2 = inst2.engine()
    run_verify(inst2, eng2)
    got = gu.outputs(inst2, 0)
    for l in range(4):
        gu.check_layer(inst2, 0, l, got[l])


def test_rollback_keeps_chain_prefix_like_commit():
    parent = [-1, 0, 1, 2, 3, 1, 5, 2]   # leading chain of 5
    a = Instance(MINI, SEED, lengths=[1000], trees=[parent])
    b = Instance(MINI, SEED, lengths=[1000], trees=[parent])
    ea, eb = a.engine(), b.engine()
    run_verify(a, ea)
    run_verify(b, eb)
    ea.rollback_to(0, 1003)
    eb.commit_tree(0, [0, 1, 2])
    gu.sync()
    assert ea.kv_length(0) == eb.kv_length(0) == 1003
    assert torch.equal(a.state[0], b.state[0])
    assert torch.equal(a.kc[0][:, :, :1003], b.kc[0][:, :, :1003])
    with pytest.raises(hdt.HdtError):
        ea.rollback_to(0, 1000)   # below the committed length
    run_verify(a, ea)
    with pytest.raises(hdt.HdtError) as e:
        ea.rollback_to(0, 1003 + 6)   # past the leading chain
    assert e.value.status == -1
    ea.rollback_to(0, 1003)
    assert ea.kv_length(0) == 1003

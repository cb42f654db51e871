"""The headline configuration end to end: 48 Gated DeltaNet + 16 attention layers (3:1) at
65,536 resident tokens with a 16-node draft tree, in the slot capacity and launch shapes
that bench.py times.

  * deep and mid-stack layers against the oracle: every output of GDN layers 28-30 and
    60-62 (all heads, all nodes), sampled rows of attention layers 31 and 63 over the
    full resident context;
  * every verified row of all 64 layers equals the decode step's row, bit for bit, along
    the accepted path ("Adding a model", step 4 of "The adapter path in ten steps");
  * after the decode of that path, all 48 committed states against the oracle's
    sequential recurrence per head (2e-3) and the K/V rows of all 16 attention layers bit
    for bit; then the same round verified again equals the first pass bit for bit, and
    commit_tree of the path equals the decoded state and rows bit for bit.

Layer l is attention iff l % 4 == 3 (three GDN layers, then one attention layer).
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_host
from tests import gpu_util as gu
from tests.brute import rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SEED = 20261202
CHECK_GDN = [28, 29, 30, 60, 61, 62]
CHECK_ATTN = [31, 63]


def _say(msg):
    print(msg, flush=True)


def _bench_capacity(w, parent):
    """The slot capacity bench.py allocates for its default run (10 warm-up and 2 x 50 timed
    rounds of the seeded path)."""
    path = synth.accepted_path(SEED, f"{w.name}/bench-path", parent)
    return w.lengths[0] + (10 + 2 * 50) * len(path) + 64


def _attn_rows(inst, s, l, nodes, heads):
    w, h = inst.w, inst.host[s][l]
    ai = sum(1 for x in w.layer_kind[:l] if x == 1)
    got = gu.outputs(inst, s)[l]
    assert np.isfinite(got).all(), f"layer {l}: non-finite output"
    worst = 0.0
    for j in heads:
        ref = np.stack([oracle.attn_row(inst.trees[s], inst.lengths[s], inst.h_kc[s][ai],
                                        inst.h_vc[s][ai], h["q"], h["k"], h["v"], i, j)
                        for i in nodes])
        err = rel_err(got[nodes, j], ref)
        worst = max(worst, err)
        assert err <= gu.TOL_BF16_OUT, f"layer {l} q head {j}: {err:.3e}"
    return worst


def test_stack65k_all_64_layers():
    w = synth.WORKLOADS["stack_65k"]
    parent = w.tree(SEED, 0)
    n = len(parent)
    L = w.lengths[0]
    cap = _bench_capacity(w, parent)
    d = synth.depths(parent)
    path = synth.root_path(parent, max(range(n), key=lambda i: (d[i], -i)))  # the deepest path
    _say(f"stack_65k, 64 layers: L={L} nodes={n} capacity={cap} path={path}")
    inst = Instance(w, SEED, trees=[parent], capacity=[cap], keep_host=False,
                    host_layers=CHECK_GDN + CHECK_ATTN)
    eng = inst.engine(max_nodes=n)
    assert eng.split_size(0, L) == 1056
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    verified = gu.raw_outputs(inst, 0)
    got = gu.outputs(inst, 0)
    for l in range(64):
        assert np.isfinite(got[l]).all(), f"layer {l}: non-finite output"
        assert np.abs(got[l]).max() > 0, f"layer {l}: all-zero output"
    for l in CHECK_GDN:
        err = gu.check_layer(inst, 0, l, got[l])
        _say(f"  layer {l} (GDN, all rows): max relative error {err:.2e}")
    nodes = sorted(set([0, 1, n // 2, n - 1] + [i for i in range(n) if i not in parent][:2]))
    for l in CHECK_ATTN:
        err = _attn_rows(inst, 0, l, nodes, [0, 5, 6, 11, 12, 17, 18, 23])
        _say(f"  layer {l} (attention, {len(nodes)} nodes x 8 heads): max relative error {err:.2e}")

    # verified rows == decode rows along the path, every layer, bit for bit
    state0 = inst.state[0].clone()
    eng.rollback_to(0, L, gu.stream())
    for step, j in enumerate(path):
        step_io = gu.row_io(inst, 0, j)
        eng.forward_tree([(0, [-1], step_io)], gu.stream())
        eng.commit_tree(0, [0], gu.stream())
        gu.sync()
        for l in range(64):
            row = to_host(step_io[l]["o"], w.dtype)[0]
            assert np.array_equal(row, verified[l][j]), f"node {j} layer {l}: verify row != decode row"
    _say(f"  decode of the {len(path)}-node path: every row of 64 layers equals the verified row")
    assert eng.kv_length(0) == L + len(path)
    decoded_state = inst.state[0].clone()
    m = len(path)
    decoded_rows = [c[:, :, L:L + m].clone() for c in (inst.kc[0], inst.vc[0])]

    # the decoded state of all 48 GDN layers against the oracle, per head; all 16 layers' rows
    gi = ai = 0
    worst = 0.0
    st = decoded_state.cpu().numpy()
    for l, kind in enumerate(w.layer_kind):
        h = inst.host[0][l]
        if kind == 0:
            base = synth.gdn_state(w, SEED, 0, l)
            ref = oracle.gdn_commit(path, base, h["k"], h["v"], h["alpha"], h["beta"])
            for hh in range(w.gdn_hv):
                err = rel_err(st[gi, hh], ref[hh])
                worst = max(worst, err)
                assert err <= gu.TOL_F32, f"layer {l} head {hh}: committed state {err:.3e}"
            gi += 1
        else:
            for name, rows in (("k", decoded_rows[0]), ("v", decoded_rows[1])):
                assert np.array_equal(to_host(rows[ai], w.dtype), oracle.commit_kv_rows(h[name], path)), \
                    f"layer {l}: committed {name} rows"
            ai += 1
    _say(f"  48 committed states: worst per-head relative error {worst:.2e}; 16 layers' rows bit-exact")

    # the same round again from the saved state: same bits; commit_tree == decoded
    inst.state[0].copy_(state0)
    eng.reset(0, L)
    for io in inst.io[0]:
        io["o"].zero_()
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    again = gu.raw_outputs(inst, 0)
    for l in range(64):
        assert np.array_equal(again[l], verified[l]), f"layer {l}: second pass differs"
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    assert torch.equal(inst.state[0], decoded_state), "commit_tree state != decoded state"
    assert torch.equal(inst.kc[0][:, :, L:L + m], decoded_rows[0])
    assert torch.equal(inst.vc[0][:, :, L:L + m], decoded_rows[1])
    assert eng.kv_length(0) == L + m
    _say("  second pass equals the first; commit_tree equals the decode bit for bit")
    eng.close()

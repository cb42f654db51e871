"""forward_tree captured into a HIP graph: every replay writes the eager pass's bits; the
reusable graph (hdt_graph_forward) equals an eager twin round after round.

The pass enqueues kernels only (no allocation, copy or fill), so a captured round
can be replayed; each replay is checked against the eager outputs, with eager work
and synchronisations between the replays.
"""
import numpy as np
import pytest

import synth
from synth.device import Instance
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED = 20261202
MINI = synth.Workload("mini", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000], 16,
                      "draft")


def test_graph_replays_match_eager():
    import torch
    import hybrid_deltanet_tree_amd as hdt
    inst = Instance(MINI, SEED, lengths=[1000])
    eng = inst.engine()
    stream = torch.cuda.Stream()
    tree = [inst.tree_arg(0)]
    # the first forward allocates the engine's scratch: it may not be captured
    g0 = torch.cuda.CUDAGraph()
    with pytest.raises(hdt.HdtError) as err:
        with torch.cuda.graph(g0, stream=stream):
            eng.forward_tree(tree, torch.cuda.current_stream().cuda_stream)
    assert err.value.status == -5  # HDT_E_ORDER
    del g0
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        eng.forward_tree(tree, stream.cuda_stream)
    torch.cuda.synchronize()
    eager = gu.raw_outputs(inst, 0)
    rows = [c[:, :, 1000:1016].clone() for c in (inst.kc[0], inst.vc[0])]
    eng.rollback_to(0, 1000)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        eng.forward_tree(tree, torch.cuda.current_stream().cuda_stream)
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for io in inst.io[0]:
            io["o"].zero_()
        inst.kc[0][:, :, 1000:1016].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gu.raw_outputs(inst, 0)
        for l in range(len(MINI.layer_kind)):
            assert np.array_equal(got[l], eager[l]), f"replay {rep} layer {l} differs from eager"
        assert torch.equal(inst.kc[0][:, :, 1000:1016], rows[0])
        scratch.mul_(1.0001).add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
    eng.rollback_to(0, 1000)
    assert eng.kv_length(0) == 1000
    del g
    eng.close()


CONV = synth.Workload("graph_conv", [0, 1, 0, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000], 16,
                      "draft", extra={"conv": 4})


@pytest.mark.parametrize("wname,lengths", [("mini", [1000]), ("mini", [1000, 3000]), ("conv", [1000])])
def test_reusable_graph_across_rounds(wname, lengths):
    """hdt_graph_forward over rounds that each verify a different 16-node tree and commit a
    path, so the lengths and the split plan move from round to round: every round's outputs,
    and the states, conv tails and cache rows at the end, equal an eager twin's bit for bit,
    and after its two first instantiations the graph is updated in place rather than rebuilt."""
    import torch
    w = {"mini": MINI, "conv": CONV}[wname]
    rounds = 8
    cap = [L + 16 * rounds + 64 for L in lengths]
    a = Instance(w, SEED, lengths=lengths, capacity=cap)
    b = Instance(w, SEED, lengths=lengths, capacity=cap)
    ea, eb = a.engine(), b.engine()
    graph = eb.graph()
    stream = torch.cuda.current_stream().cuda_stream
    slots = range(len(lengths))
    for r in range(rounds):
        trees = [synth.draft_tree(SEED + r, f"graph/round{r}/slot{s}", 16, 15) for s in slots]
        paths = [synth.accepted_path(SEED + r, f"graph/path{r}/slot{s}", t) for s, t in zip(slots, trees)]
        for inst in (a, b):
            for s in slots:
                for io in inst.io[s]:
                    io["o"].zero_()
        ea.forward_tree([(s, trees[s], a.io[s]) for s in slots], stream)
        graph.forward([(s, trees[s], b.io[s]) for s in slots], stream)
        torch.cuda.synchronize()
        for s in slots:
            got, want = gu.raw_outputs(b, s), gu.raw_outputs(a, s)
            for l in range(len(w.layer_kind)):
                assert np.array_equal(got[l], want[l]), f"round {r} slot {s} layer {l}"
        for s in slots:
            ea.commit_tree(s, paths[s], stream)
            eb.commit_tree(s, paths[s], stream)
        assert [eb.kv_length(s) for s in slots] == [ea.kv_length(s) for s in slots]
    torch.cuda.synchronize()
    for s in slots:
        assert torch.equal(a.state[s], b.state[s]) and torch.equal(a.kc[s], b.kc[s]) and torch.equal(a.vc[s], b.vc[s])
        if a.conv > 1:
            assert torch.equal(a.tail[s], b.tail[s])
    inst_n, upd = graph.stats()
    print(f"graph: {inst_n} instantiations, {upd} updates over {rounds} rounds", flush=True)
    assert inst_n + upd == rounds and inst_n >= 2 and upd >= rounds - 4
    graph.close()
    ea.close()
    eb.close()

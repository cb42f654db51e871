"""forward_tree captured into a HIP graph: every replay writes the eager pass's bits.

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

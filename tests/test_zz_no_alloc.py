"""hdt_forward_tree_noalloc: the forward_tree variant that allocates nothing (its scratch is a
static array of the library, one per device), for callers that cannot allocate.

  * the very first call of a fresh engine (nothing allocated yet) gives hdt_forward_tree's
    outputs bit for bit, and commit_tree after it gives the same state and cache rows;
  * two calls in a row, the second with a smaller tree, each equal hdt_forward_tree;
  * a round whose static scratch a later call on the device reused is refused by commit
    (HDT_E_ORDER) and can still be dropped.
"""
import numpy as np
import pytest

import synth
from synth.device import Instance
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hybrid_deltanet_tree_amd as hdt  # noqa: E402

SEED = 20261202
MINI = synth.Workload("mini", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000], 16,
                      "draft")


def _run(inst, eng, noalloc, tree=None):
    for io in inst.io[0]:
        io["o"].zero_()
    arg = inst.tree_arg(0) if tree is None else (0, tree[0], tree[1])
    if noalloc:
        eng.forward_tree_noalloc([arg], gu.stream())
    else:
        eng.forward_tree([arg], gu.stream())
    gu.sync()
    return gu.raw_outputs(inst, 0)


def test_first_call_and_commit_equal_forward_tree():
    a = Instance(MINI, SEED)
    b = Instance(MINI, SEED)
    ea, eb = a.engine(), b.engine()
    got = _run(a, ea, noalloc=True)      # the engine has allocated nothing yet
    want = _run(b, eb, noalloc=False)
    for l in range(4):
        assert np.array_equal(got[l], want[l]), f"layer {l}"
    path = synth.accepted_path(SEED, "noalloc/path", a.trees[0])
    ea.commit_tree(0, path, gu.stream())
    eb.commit_tree(0, path, gu.stream())
    gu.sync()
    assert torch.equal(a.state[0], b.state[0])
    L, m = MINI.lengths[0], len(path)
    assert torch.equal(a.kc[0][:, :, :L + m], b.kc[0][:, :, :L + m])
    assert torch.equal(a.vc[0][:, :, :L + m], b.vc[0][:, :, :L + m])
    assert ea.kv_length(0) == eb.kv_length(0) == L + m
    ea.close()
    eb.close()


def test_two_calls_second_smaller():
    inst = Instance(MINI, SEED)
    eng = inst.engine()
    for tree in (inst.trees[0], [-1, 0, 1, 1, 3]):
        inst.set_inputs(0, "noalloc", parent=tree)
        got = _run(inst, eng, noalloc=True)
        eng.rollback_to(0, MINI.lengths[0], gu.stream())
        want = _run(inst, eng, noalloc=False)
        eng.rollback_to(0, MINI.lengths[0], gu.stream())
        for l in range(4):
            assert np.array_equal(got[l], want[l]), f"{len(tree)} nodes, layer {l}"
    eng.close()


def test_reused_scratch_refuses_the_older_round():
    a = Instance(MINI, SEED)
    b = Instance(MINI, SEED + 1)
    ea, eb = a.engine(), b.engine()
    _run(a, ea, noalloc=True)
    _run(b, eb, noalloc=True)           # takes the device's static scratch
    with pytest.raises(hdt.HdtError) as e:
        ea.commit_tree(0, [0], gu.stream())
    assert e.value.status == -5 and "reused" in ea.last_error()
    ea.rollback_to(0, MINI.lengths[0], gu.stream())   # dropping it is still allowed
    eb.commit_tree(0, [0, 1], gu.stream())            # the latest round commits
    gu.sync()
    assert ea.kv_length(0) == MINI.lengths[0] and eb.kv_length(0) == MINI.lengths[0] + 2
    ea.close()
    eb.close()

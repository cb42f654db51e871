"""State snapshots on the device (hdt_state_bytes / hdt_state_copy): the cache state of
"Adding a model", "The model layer: architecture registry and per-model state" (sections
copied whole, views sliced by length; clone, restore, and a signature that refuses a
restore across shapes).

  * clone, then a committed round, then restore: the recurrent state and conv tails are
    back bit for bit, the length is the snapshot's, and the same round verified again
    gives the first pass's bits;
  * refused without any change: a snapshot of an engine of another shape, a snapshot that
    holds more committed rows than the slot now has, and a buffer that holds no snapshot.
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
MINI_CONV = synth.Workload("mini_conv", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000],
                           16, "draft", extra={"conv": 4})
OTHER = synth.Workload("other", [0, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000], 16,
                       "draft", extra={"conv": 4})


def _buf(nbytes):
    b = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-b.data_ptr()) % 256
    return b[off:off + nbytes]


def test_clone_restore_round_trip():
    inst = Instance(MINI_CONV, SEED)
    eng = inst.engine()
    L = inst.lengths[0]
    n = eng.state_bytes()
    buf = _buf(n)
    eng.state_copy(0, buf, restore=False, stream=gu.stream())
    gu.sync()
    state0, tail0 = inst.state[0].clone(), inst.tail[0].clone()
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    first = gu.raw_outputs(inst, 0)
    path = synth.accepted_path(SEED, "snap/path", inst.trees[0])
    eng.commit_tree(0, path, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + len(path)
    assert not torch.equal(inst.state[0], state0)
    eng.state_copy(0, buf, restore=True, stream=gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L
    assert torch.equal(inst.state[0], state0)
    assert torch.equal(inst.tail[0], tail0)
    for io in inst.io[0]:
        io["o"].zero_()
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    gu.sync()
    again = gu.raw_outputs(inst, 0)
    for l in range(4):
        assert np.array_equal(again[l], first[l]), f"layer {l}"
    eng.close()


def test_restore_refusals_change_nothing():
    inst = Instance(MINI_CONV, SEED)
    eng = inst.engine()
    L = inst.lengths[0]
    other = Instance(OTHER, SEED)
    eo = other.engine()
    # the same number of GDN layers, so snapshots of the same size: only the signature
    # (layer order) tells them apart
    assert eo.state_bytes() == eng.state_bytes()
    big = _buf(max(eo.state_bytes(), eng.state_bytes()))
    # a snapshot of another model shape
    eo.state_copy(0, big, restore=False, stream=gu.stream())
    gu.sync()
    state0 = inst.state[0].clone()
    with pytest.raises(hdt.HdtError) as e:
        eng.state_copy(0, big, restore=True, stream=gu.stream())
    assert e.value.status == -1 and "another shape" in eng.last_error()
    # a buffer that holds no snapshot
    big.zero_()
    with pytest.raises(hdt.HdtError) as e:
        eng.state_copy(0, big, restore=True, stream=gu.stream())
    assert e.value.status == -1 and "no state snapshot" in eng.last_error()
    # a snapshot with more committed rows than the slot now holds
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    eng.commit_tree(0, [0, 1], gu.stream())
    eng.state_copy(0, big, restore=False, stream=gu.stream())
    gu.sync()
    after = inst.state[0].clone()
    eng.reset(0, L)
    with pytest.raises(hdt.HdtError) as e:
        eng.state_copy(0, big, restore=True, stream=gu.stream())
    assert e.value.status == -1
    assert eng.kv_length(0) == L and torch.equal(inst.state[0], after)
    assert not torch.equal(after, state0)
    eng.close()
    eo.close()

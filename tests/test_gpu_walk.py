"""The accept walk on the device (walk_commit): the walk's output against the oracle's
accept rule, bit for bit, and the commit it feeds against commit_tree of that path, bit
for bit (state, K/V rows, conv tails), with no host wait between walk and commit."""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SEED = 20261204
MINI = synth.Workload("walk_mini", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16", [1000],
                      16, "draft")
TINY = synth.Workload("walk_tiny", [0, 1], 1, 2, 64, 64, 2, 1, 64, "f32", [256], 8, "random4", 4)
CONV = synth.Workload("walk_conv", [0, 1, 0], 16, 32, 128, 128, 24, 4, 256, "bf16", [700], 16,
                      "draft", extra={"conv": 4})
BIG = synth.Workload("walk_64", [0, 1], 4, 8, 128, 128, 12, 2, 256, "bf16", [513], 64, "draft",
                     max_depth=40)
WL = {w.name: w for w in (MINI, TINY, CONV, BIG)}


def _tokens(parent, tag, agree=0.7):
    d, t = synth.round_tokens(SEED, tag, parent, agree=agree)
    return d, t


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _state(inst, s=0):
    out = [inst.state[s].clone(), inst.kc[s].clone(), inst.vc[s].clone()]
    if inst.conv > 0:
        out.append(inst.tail[s].clone())
    return out


def _walk_vs_commit(inst, eng, draft, target, s=0):
    """walk_commit, then the same round with commit_tree of the oracle's path: the walk's
    output equals the oracle's, and both commits leave the same bits."""
    L = inst.lengths[s]
    n = len(inst.trees[s])
    path, bonus = oracle.greedy_walk(inst.trees[s], draft, target)
    snap = gu.snapshot(inst)
    eng.forward_tree([inst.tree_arg(s)], gu.stream())
    out = torch.full((2 + n,), -7, dtype=torch.int32, device="cuda")
    eng.walk_commit(s, _dev(draft), _dev(target), out, gu.stream())
    assert eng.kv_length(s) == L + len(path)  # waits for the walk
    got = out.cpu().numpy()
    assert got[0] == len(path) and got[1] == bonus
    assert list(got[2:2 + len(path)]) == path
    walked = _state(inst, s)
    gu.restore(inst, snap)
    eng.reset(s, L)
    eng.forward_tree([inst.tree_arg(s)], gu.stream())
    eng.commit_tree(s, path, gu.stream())
    gu.sync()
    for a, b in zip(walked, _state(inst, s)):
        assert torch.equal(a, b)
    return path


@pytest.mark.parametrize("wname", sorted(WL))
def test_walk_matches_oracle_and_commit_tree(wname):
    w = WL[wname]
    inst = Instance(w, SEED)
    eng = inst.engine()
    lens = []
    for k, agree in enumerate((0.7, 0.95, 0.3)):
        draft, target = _tokens(inst.trees[0], f"{wname}/{k}", agree)
        path = _walk_vs_commit(inst, eng, draft, target)
        lens.append(len(path))
        inst.lengths[0] = eng.kv_length(0)
        gu.restore(inst, gu.snapshot(inst))
    print(f"{wname}: accepted path lengths {lens}", flush=True)
    eng.close()


def test_walk_edges():
    inst = Instance(MINI, SEED)
    eng = inst.engine()
    parent = inst.trees[0]
    n = len(parent)
    # nothing agrees: the root alone
    draft = np.arange(n, dtype=np.int32) + 1000
    target = np.zeros(n, dtype=np.int32)
    assert _walk_vs_commit(inst, eng, draft, target) == [0]
    inst.lengths[0] = eng.kv_length(0)
    # the leading chain agrees throughout, no branch does
    c = oracle.leading_chain(parent)
    target = np.full(n, -1, dtype=np.int32)
    for i in range(c - 1):
        target[i] = draft[i + 1]
    assert _walk_vs_commit(inst, eng, draft, target) == list(range(c))
    eng.close()


def test_walk_then_next_round_without_sync():
    """Round after round, the next forward_tree follows walk_commit with no host wait of
    the caller's own; the library waits for the walk's length itself."""
    inst = Instance(MINI, SEED)
    eng = inst.engine()
    parent = inst.trees[0]
    n = len(parent)
    out = torch.zeros(2 + n, dtype=torch.int32, device="cuda")
    L = inst.lengths[0]
    for r in range(4):
        draft, target = _tokens(parent, f"rounds/{r}")
        path, _ = oracle.greedy_walk(parent, draft, target)
        eng.forward_tree([inst.tree_arg(0)], gu.stream())
        eng.walk_commit(0, _dev(draft), _dev(target), out, gu.stream())
        L += len(path)
    assert eng.kv_length(0) == L
    eng.close()


def test_joint_slots_walk_separately():
    w = synth.Workload("walk_joint", [0, 1, 0, 1], 16, 32, 128, 128, 24, 4, 256, "bf16",
                       [1000, 333], 16, "draft")
    inst = Instance(w, SEED)
    eng = inst.engine()
    eng.forward_tree([inst.tree_arg(s) for s in range(2)], gu.stream())
    outs, want = [], []
    for s in range(2):
        draft, target = _tokens(inst.trees[s], f"joint/{s}")
        want.append(oracle.greedy_walk(inst.trees[s], draft, target))
        outs.append(torch.zeros(2 + len(inst.trees[s]), dtype=torch.int32, device="cuda"))
        eng.walk_commit(s, _dev(draft), _dev(target), outs[s], gu.stream())
    for s in range(2):
        path, bonus = want[s]
        got = outs[s].cpu().numpy()
        assert got[0] == len(path) and got[1] == bonus and list(got[2:2 + len(path)]) == path
        assert eng.kv_length(s) == w.lengths[s] + len(path)
    eng.close()

"""The recorded-bytes gate on the tiny configuration (the refactor gate of "Adding a model",
"The tests a new model must pass": a prefill, a decode, a block verify, a rollback, a tree
verify and a commit, and every byte they produce).

  * CPU: the oracle's bytes over the sequence (tests/c0_gate.py) must equal the recorded
    digests (tests/golden/c0_sequence.json, written by tests/golden/record_c0.py from the
    oracle alone): any byte that moves fails.
  * GPU: the same sequence through the C ABI (forward_span, forward_tree + commit_tree,
    forward_block + rollback_to, forward_tree + commit_tree) matches those oracle values
    per (layer, head) within 2e-3 with the appended cache rows bit for bit, and a second
    run in a fresh engine gives the same bytes as the first.
"""
import json
import os

import numpy as np
import pytest

from tests import c0_gate
from tests.brute import rel_err

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c0_sequence.json")


def test_oracle_bytes_equal_the_recording():
    rec = json.load(open(GOLDEN))
    assert rec["seed"] == c0_gate.SEED and rec["steps"] == list(c0_gate.STEPS)
    now = c0_gate.digests(c0_gate.run_oracle())
    for step in c0_gate.STEPS:
        for name, d in rec["digests"][step].items():
            assert now[step][name] == d, f"{step}/{name}: the oracle's bytes moved"


def _gpu_sequence():
    """Run the sequence on the device; returns the same structure as run_oracle (outputs and
    state as float32, rows as float32)."""
    import torch
    from synth.device import Instance, to_device
    from tests import gpu_util as gu
    w = c0_gate.W
    inst = Instance(w, c0_gate.SEED, lengths=[c0_gate.L0], trees=[[-1]],
                    capacity=[c0_gate.capacity()])
    eng = inst.engine(max_nodes=8)
    st = gu.stream()
    out = {}
    L = c0_gate.L0
    for step in c0_gate.STEPS:
        parent, path = c0_gate.trees()[step]
        n = len(parent)
        g, a = c0_gate.inputs(step, n)
        io = [{k: to_device(v, "f32", "cuda") for k, v in g.items()},
              {k: to_device(v, "f32", "cuda") for k, v in a.items()}]
        io[0]["o"] = torch.zeros((n, w.gdn_hv, w.gdn_dv), device="cuda")
        io[1]["o"] = torch.zeros((n, w.attn_hq, w.attn_d), device="cuda")
        if step == "prefill":
            eng.forward_span(0, n, io, st)
        elif step == "block":
            eng.forward_block(0, n, io, st)
            eng.rollback_to(0, L + len(path), st)
        else:
            eng.forward_tree([(0, parent, io)], st)
            eng.commit_tree(0, path, st)
        gu.sync()
        m = len(path)
        assert eng.kv_length(0) == L + m
        out[step] = {"gdn_o": io[0]["o"].cpu().numpy(), "attn_o": io[1]["o"].cpu().numpy(),
                     "state": inst.state[0][0].cpu().numpy().copy(),
                     "k_rows": inst.kc[0][0, :, L:L + m].cpu().numpy().copy(),
                     "v_rows": inst.vc[0][0, :, L:L + m].cpu().numpy().copy()}
        L += m
    eng.close()
    return out


@pytest.mark.gpu
def test_gpu_sequence_matches_the_gated_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ref = c0_gate.run_oracle()
    rec = json.load(open(GOLDEN))
    assert c0_gate.digests(ref) == rec["digests"]
    first = _gpu_sequence()
    for step in c0_gate.STEPS:
        r, g = ref[step], first[step]
        for name in ("gdn_o", "attn_o"):
            assert np.isfinite(g[name]).all()
            for hh in range(r[name].shape[1]):
                err = rel_err(g[name][:, hh], r[name][:, hh])
                assert err <= 2e-3, f"{step} {name} head {hh}: {err:.3e}"
        for hh in range(r["state"].shape[0]):
            assert rel_err(g["state"][hh], r["state"][hh]) <= 2e-3, f"{step} state"
        for name in ("k_rows", "v_rows"):
            assert np.array_equal(g[name], r[name]), f"{step} {name}"
    second = _gpu_sequence()
    for step in c0_gate.STEPS:
        for name, arr in first[step].items():
            assert np.array_equal(arr.view(np.uint32), second[step][name].view(np.uint32)), \
                f"{step}/{name}: a second run gave other bytes"

"""Helpers for the GPU tests: run the library on an Instance, read results back, and
compare with the oracle under the stated tolerances."""
import numpy as np

import oracle
import synth
from synth.device import to_host
from tests.brute import rel_err

TOL_BF16_OUT = 2e-2   # max relative error per (layer, head) tensor, bf16 outputs
TOL_F32 = 2e-3        # max relative error on float32 state and float32 outputs


def stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def sync():
    import torch
    torch.cuda.synchronize()


def outputs(inst, s):
    """Per-layer outputs of slot s as host arrays (float32 values)."""
    res = []
    for l, io in enumerate(inst.io[s]):
        o = to_host(io["o"], inst.w.dtype)
        res.append(synth.bf16_bits_to_f32(o) if inst.w.dtype == "bf16" else o)
    return res


def raw_outputs(inst, s):
    """Per-layer outputs of slot s as raw storage bits (for bit-exact comparisons)."""
    return [to_host(io["o"], inst.w.dtype).copy() for io in inst.io[s]]


def oracle_layer(inst, s, l, L=None):
    """Oracle output of layer l of slot s (all rows), float32."""
    w, h = inst.w, inst.host[s][l]
    parent = inst.trees[s]
    L = inst.lengths[s] if L is None else L
    if w.layer_kind[l] == 0:
        gi = sum(1 for x in w.layer_kind[:l] if x == 0)
        if inst.conv > 0:
            return oracle.gdn_conv_layer(parent, inst.h_state[s][gi], inst.h_tail[s][gi], h["q"],
                                         h["k"], h["v"], h["alpha"], h["beta"],
                                         inst.h_conv_w[gi])[0]
        return oracle.gdn_tree(parent, inst.h_state[s][gi], h["q"], h["k"], h["v"], h["alpha"],
                               h["beta"])
    ai = sum(1 for x in w.layer_kind[:l] if x == 1)
    return oracle.attn_tree(parent, L, inst.h_kc[s][ai], inst.h_vc[s][ai], h["q"], h["k"], h["v"])


def max_rel_per_head(got, ref):
    """P17: per (layer, head) tensor max|a-b| / max|b|; returns the worst head."""
    worst = 0.0
    for hh in range(ref.shape[1]):
        worst = max(worst, rel_err(got[:, hh], ref[:, hh]))
    return worst


def elementwise_worst(got, ref, floor=1e-2):
    """P17's elementwise worst case, reported beside the per-head figure: the largest
    |a - b| / |b| over elements whose reference is at least `floor` times the largest
    reference magnitude of its head (smaller elements have no stable relative error)."""
    worst = 0.0
    for hh in range(ref.shape[1]):
        r = ref[:, hh].astype(np.float64)
        g = got[:, hh].astype(np.float64)
        big = np.abs(r) >= floor * np.abs(r).max()
        if big.any():
            worst = max(worst, float((np.abs(g - r)[big] / np.abs(r)[big]).max()))
    return worst


def check_layer(inst, s, l, got, tol=None):
    ref = oracle_layer(inst, s, l)
    tol = tol if tol is not None else (TOL_BF16_OUT if inst.w.dtype == "bf16" else TOL_F32)
    err = max_rel_per_head(got, ref)
    assert np.isfinite(got).all(), f"layer {l}: non-finite output"
    print(f"    slot {s} layer {l}: per-head {err:.2e}, elementwise worst "
          f"{elementwise_worst(got, ref):.2e}", flush=True)
    assert err <= tol, f"slot {s} layer {l}: max relative error {err:.3e} > {tol}"
    return err


def snapshot(inst):
    return [(inst.state[s].clone(), inst.kc[s].clone(), inst.vc[s].clone(),
             inst.tail[s].clone() if inst.conv > 0 else None)
            for s in range(len(inst.lengths))]


def restore(inst, snap):
    for s, (st, kc, vc, tl) in enumerate(snap):
        inst.state[s].copy_(st)
        inst.kc[s].copy_(kc)
        inst.vc[s].copy_(vc)
        if tl is not None:
            inst.tail[s].copy_(tl)


def row_io(inst, s, node):
    """Per-layer io dicts that view row `node` of slot s's tree inputs (a 1-node tree)."""
    res = []
    for io in inst.io[s]:
        res.append({k: t[node:node + 1] for k, t in io.items()})
    return res

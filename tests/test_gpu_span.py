"""Prefill spans (forward_span) and state anchors on the device:

  * every output row of a span against the oracle (the sequential recurrence over the
    span; attention of each token over every earlier position), and the committed state
    and K/V rows after it;
  * a span equals decoding its tokens one by one, bit for bit (outputs, state, rows);
  * anchors hold the state at their positions bit for bit; rollback_to an anchor
    restores it, and forwarding the rest of the span again gives the same bits.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_device, to_host
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SEED = 20261205
SPAN = synth.Workload("span", [0, 1, 0, 1], 2, 4, 128, 128, 12, 2, 256, "bf16", [300], 16, "draft")
SPAN_CONV = synth.Workload("span_conv", [0, 0, 1], 2, 4, 128, 128, 12, 2, 256, "bf16", [300], 16,
                           "draft", extra={"conv": 4})
SPAN_F32 = synth.Workload("span_f32", [0, 1], 1, 2, 64, 64, 2, 1, 64, "f32", [100], 8, "random4", 4)


def _say(msg):
    print(msg, flush=True)


def span_inputs(inst, T, tag="span", sharp=False, q_scale=1.0):
    """Per-layer host arrays and device tensors holding T rows (attention q and k drawn as
    for Instance(sharp=..., q_scale=...))."""
    w = inst.w
    host, dev = [], []
    for l, kind in enumerate(w.layer_kind):
        if kind == 0:
            gen = synth.conv_inputs if inst.conv > 0 else synth.gdn_inputs
            q, k, v, a, b = gen(w, SEED, 0, l, T, tag)
            h = dict(q=q, k=k, v=v, alpha=a, beta=b)
            oshape = (T, w.gdn_hv, w.gdn_dv)
        else:
            q, k, v = synth.attn_inputs(w, SEED, 0, l, T, tag, sharp=sharp, q_scale=q_scale)
            h = dict(q=q, k=k, v=v)
            oshape = (T, w.attn_hq, w.attn_d)
        d = {name: to_device(a, w.dtype, "cuda") for name, a in h.items()}
        d["o"] = torch.zeros(oshape, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                             device="cuda")
        host.append(h)
        dev.append(d)
    return host, dev


def _f32(a, dtype):
    return synth.bf16_bits_to_f32(a) if dtype == "bf16" else a


def check_span_against_oracle(inst, host, dev, L, T):
    w = inst.w
    gi = ai = 0
    for l, kind in enumerate(w.layer_kind):
        h = host[l]
        got = _f32(to_host(dev[l]["o"], w.dtype), w.dtype)
        if kind == 0:
            chain = synth.chain_tree(T)
            if inst.conv > 0:
                ref, (_, kc, vc) = oracle.gdn_conv_layer(chain, inst.h_state[0][gi], inst.h_tail[0][gi],
                                                         h["q"], h["k"], h["v"], h["alpha"], h["beta"],
                                                         inst.h_conv_w[gi])
            else:
                ref = oracle.gdn_tree(chain, inst.h_state[0][gi], h["q"], h["k"], h["v"], h["alpha"],
                                      h["beta"])
                kc, vc = h["k"], h["v"]
            err = gu.max_rel_per_head(got, ref)
            tol = gu.TOL_BF16_OUT if w.dtype == "bf16" else gu.TOL_F32
            assert err <= tol, f"layer {l}: {err:.3e}"
            state = oracle.gdn_commit(list(range(T)), inst.h_state[0][gi], kc, vc, h["alpha"], h["beta"])
            assert gu.rel_err(inst.state[0][gi].cpu().numpy(), state) <= gu.TOL_F32
            gi += 1
        else:
            # token t attends to positions 0 .. L + t: the resident rows, then the span's
            Kf = inst.h_kc[0][ai].copy()
            Vf = inst.h_vc[0][ai].copy()
            Kf[:, L:L + T] = np.transpose(h["k"], (1, 0, 2))
            Vf[:, L:L + T] = np.transpose(h["v"], (1, 0, 2))
            worst = 0.0
            for t in range(T):
                for j in range(w.attn_hq):
                    ref = oracle.attn_row([-1], L + t, Kf, Vf, h["q"][t:t + 1], h["k"][t:t + 1],
                                          h["v"][t:t + 1], 0, j)
                    worst = max(worst, gu.rel_err(got[t, j], ref))
            tol = gu.TOL_BF16_OUT if w.dtype == "bf16" else gu.TOL_F32
            assert worst <= tol, f"layer {l}: {worst:.3e}"
            for name, cache in (("k", inst.kc[0]), ("v", inst.vc[0])):
                rows = to_host(cache[ai, :, L:L + T], w.dtype)
                assert np.array_equal(rows, np.transpose(h[name], (1, 0, 2)))
            ai += 1
        _say(f"  layer {l} matches the oracle")


@pytest.mark.parametrize("wname,T,mn", [("span", 200, 64), ("span_conv", 150, 64),
                                        ("span_f32", 70, 16), ("span", 37, 16)])
def test_span_matches_oracle(wname, T, mn):
    w = {"span": SPAN, "span_conv": SPAN_CONV, "span_f32": SPAN_F32}[wname]
    L = w.lengths[0]
    _say(f"span {wname}: {T} tokens at {L}, chains of {mn}")
    inst = Instance(w, SEED, capacity=[L + T + 64])
    eng = inst.engine(max_nodes=mn)
    host, dev = span_inputs(inst, T)
    eng.forward_span(0, T, dev, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    check_span_against_oracle(inst, host, dev, L, T)
    eng.close()


def _decode_span(inst, eng, dev, T, snaps_at=()):
    """Decode the span token by token (1-node tree + commit); returns the raw outputs and
    state snapshots at the requested lengths."""
    outs = [torch.zeros_like(d["o"]) for d in dev]
    snaps = {}
    L0 = eng.kv_length(0)
    for t in range(T):
        step = [{k: x[t:t + 1] for k, x in d.items()} for d in dev]
        eng.forward_tree([(0, [-1], step)], gu.stream())
        eng.commit_tree(0, [0], gu.stream())
        for o, d in zip(outs, step):
            o[t:t + 1].copy_(d["o"])
        if L0 + t + 1 in snaps_at:
            gu.sync()
            snaps[L0 + t + 1] = [inst.state[0].clone()] + ([inst.tail[0].clone()] if inst.conv else [])
    gu.sync()
    return outs, snaps


@pytest.mark.parametrize("wname", ["span", "span_conv"])
def test_span_equals_decode_and_anchors(wname):
    w = {"span": SPAN, "span_conv": SPAN_CONV}[wname]
    L, T, every = w.lengths[0], 130, 48
    inst = Instance(w, SEED, capacity=[L + T + 64])
    eng = inst.engine(max_nodes=64)
    host, dev = span_inputs(inst, T)
    snap = gu.snapshot(inst)
    positions = [p for p in range(L + 1, L + T + 1) if p % every == 0]  # 336, 384, 432
    _say(f"{wname}: anchors every {every} at {positions}")
    dec_outs, snaps = _decode_span(inst, eng, dev, T, snaps_at=set(positions))
    decoded = [inst.state[0].clone(), inst.kc[0].clone(), inst.vc[0].clone()]
    # the same span in one call, with anchors
    gu.restore(inst, snap)
    eng.reset(0, L)
    n_max = (L + T) // every + 1
    a_state = torch.zeros((n_max,) + tuple(inst.state[0].shape), dtype=torch.float32, device="cuda")
    a_conv = (torch.zeros((n_max,) + tuple(inst.tail[0].shape), dtype=inst.tail[0].dtype, device="cuda")
              if inst.conv > 1 else None)
    eng.set_anchors(0, every, n_max, a_state, a_conv)
    for d in dev:
        d["o"].zero_()
    eng.forward_span(0, T, dev, gu.stream())
    gu.sync()
    for l in range(len(w.layer_kind)):
        assert torch.equal(dev[l]["o"], dec_outs[l]), f"layer {l}: span row != decode row"
    for a, b in zip([inst.state[0], inst.kc[0], inst.vc[0]], decoded):
        assert torch.equal(a, b)
    for p in positions:
        k = p // every - 1
        assert torch.equal(a_state[k], snaps[p][0]), f"anchor at {p}"
        if a_conv is not None:
            assert torch.equal(a_conv[k], snaps[p][1]), f"conv anchor at {p}"
    assert eng.anchor_below(0, L + T) == positions[-1]
    assert eng.anchor_below(0, positions[0] - 1) == -1
    # roll back to the middle anchor, forward the rest again: the same bits
    mid = positions[1]
    final = [x.clone() for x in (inst.state[0], inst.kc[0], inst.vc[0])]
    outs_full = [d["o"].clone() for d in dev]
    eng.rollback_to(0, mid, gu.stream())
    assert eng.kv_length(0) == mid and eng.anchor_below(0, L + T) == mid
    gu.sync()
    assert torch.equal(inst.state[0], snaps[mid][0])
    rest = [{k: x[mid - L:] for k, x in d.items()} for d in dev]
    for d in rest:
        d["o"].zero_()
    eng.forward_span(0, L + T - mid, rest, gu.stream())
    gu.sync()
    for a, b in zip((inst.state[0], inst.kc[0], inst.vc[0]), final):
        assert torch.equal(a, b)
    for l in range(len(w.layer_kind)):
        assert torch.equal(dev[l]["o"][mid - L:], outs_full[l][mid - L:])
    eng.close()

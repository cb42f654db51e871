"""The chunked prefill (forward_chunked): the WY form of the delta rule and causal attention
on the matrix cores, against the oracle.

  * every output row of a span, the committed state and the K/V rows it writes, against
    the oracle's sequential recurrence and attention of each token over every earlier
    position: spans whose chunks start and end off the 64-token grid, a one-token span, a
    span that fills exactly one chunk, and a span of two pieces (longer than 2,048 tokens)
    with sampled attention rows;
  * anchors hold the oracle's state at their positions; rollback to an anchor and forwarding
    the rest again gives the same bits (the pass is deterministic);
  * full size: the stack's head shapes at 65,536 resident tokens and a 2,048-token span,
    four sampled GDN heads and sampled attention rows over the whole context.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.device import Instance, to_device, to_host
from tests import gpu_util as gu
from tests.brute import rel_err
from tests.test_gpu_span import SEED, SPAN, SPAN_CONV, check_span_against_oracle, span_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hybrid_deltanet_tree_amd as hdt  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _f32(a):
    return synth.bf16_bits_to_f32(a)


@pytest.mark.parametrize("L,T", [(300, 200), (300, 37), (300, 1), (256, 64), (0, 100)])
def test_chunked_matches_oracle(L, T):
    _say(f"chunked prefill: {T} tokens at {L}")
    inst = Instance(SPAN, SEED, lengths=[L], capacity=[L + T + 64])
    eng = inst.engine()
    host, dev = span_inputs(inst, T)
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    check_span_against_oracle(inst, host, dev, L, T)
    eng.close()


def _span_conv(width):
    if width == 4:
        return SPAN_CONV
    return synth.Workload(f"span_conv{width}", [0, 0, 1], 2, 4, 128, 128, 12, 2, 256, "bf16", [300], 16,
                          "draft", extra={"conv": width})


@pytest.mark.parametrize("width,L,T", [(4, 300, 150), (4, 300, 2), (4, 256, 64), (2, 300, 70), (1, 300, 70)])
def test_chunked_conv_matches_oracle(width, L, T):
    """The short conv in front of each GDN layer: outputs and state against the oracle's conv
    and recurrence, and the tail afterwards holds the last width - 1 pre-conv rows of (old
    tail, span) bit for bit (with T = 2 and width 4, one of them from the old tail; width 1
    has no tail)."""
    w = _span_conv(width)
    _say(f"chunked prefill with the width-{width} conv: {T} tokens at {L}")
    inst = Instance(w, SEED, lengths=[L], capacity=[L + T + 64])
    eng = inst.engine()
    host, dev = span_inputs(inst, T)
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    check_span_against_oracle(inst, host, dev, L, T)
    gi = 0
    for l, kind in enumerate(w.layer_kind):
        if kind != 0 or width == 1:
            continue
        h = host[l]
        want = oracle.conv_tail_commit(inst.h_tail[0][gi], h["q"], h["k"], h["v"], list(range(T)))
        assert np.array_equal(to_host(inst.tail[0][gi], w.dtype), want), f"layer {l} tail"
        gi += 1
    eng.close()


def test_chunked_conv_anchors_and_rollback():
    """Anchors of a conv model hold the oracle's state and the tail at their positions;
    rollback to an anchor and forwarding the rest again gives the same bits."""
    w = SPAN_CONV
    L, T, every = 300, 300, 128  # anchors at 384 and 512
    inst = Instance(w, SEED, lengths=[L], capacity=[L + T + 64])
    eng = inst.engine()
    n_max = 8
    astate = torch.zeros((n_max,) + tuple(inst.state[0].shape), dtype=torch.float32, device="cuda")
    aconv = torch.zeros((n_max,) + tuple(inst.tail[0].shape), dtype=inst.tail[0].dtype, device="cuda")
    eng.set_anchors(0, every, n_max, astate, aconv)
    host, dev = span_inputs(inst, T)
    S0 = [x.copy() for x in inst.h_state[0]]
    tail0 = [x.copy() for x in inst.h_tail[0]]
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    first = [to_host(d["o"], w.dtype).copy() for d in dev]
    final = (inst.state[0].clone(), inst.tail[0].clone())
    gdn = [l for l, kind in enumerate(w.layer_kind) if kind == 0]
    for pos in (384, 512):
        assert eng.anchor_below(0, pos) == pos
        k, n = pos // every - 1, pos - L
        for gi, l in enumerate(gdn):
            h = host[l]
            _, (_, kc, vc) = oracle.gdn_conv_layer(synth.chain_tree(T), S0[gi], tail0[gi], h["q"], h["k"],
                                                   h["v"], h["alpha"], h["beta"], inst.h_conv_w[gi])
            ref = oracle.gdn_commit(list(range(n)), S0[gi], kc, vc, h["alpha"], h["beta"])
            err = rel_err(astate[k, gi].cpu().numpy(), ref)
            assert err <= gu.TOL_F32, f"anchor {pos} layer {l}: {err:.3e}"
            want = oracle.conv_tail_commit(tail0[gi], h["q"], h["k"], h["v"], list(range(n)))
            assert np.array_equal(to_host(aconv[k, gi], w.dtype), want), f"anchor {pos} layer {l} tail"
    eng.rollback_to(0, 384, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == 384
    rest = [{name: x[384 - L:] for name, x in d.items()} for d in dev]
    for d in rest:
        d["o"].zero_()
    eng.forward_chunked(0, T - (384 - L), rest, gu.stream())
    gu.sync()
    for l, d in enumerate(dev):
        assert np.array_equal(to_host(d["o"], w.dtype)[384 - L:], first[l][384 - L:]), f"layer {l}"
    assert torch.equal(inst.state[0], final[0]) and torch.equal(inst.tail[0], final[1])
    eng.close()


def oracle_chain(S0, q, k, v, a, b, piece=256):
    """Outputs and final state of the sequential recurrence over a long chain, in pieces
    of `piece` tokens (each piece starts from the state the previous one ended in)."""
    T = q.shape[0]
    outs, S = [], S0
    for t0 in range(0, T, piece):
        t1 = min(T, t0 + piece)
        o, states = oracle.gdn_tree(synth.chain_tree(t1 - t0), S, q[t0:t1], k[t0:t1], v[t0:t1],
                                    a[t0:t1], b[t0:t1], want_states=True)
        outs.append(o)
        S = states[-1]
    return np.concatenate(outs), S


def _check_attn_rows(got, h, Kc, Vc, L, tokens, heads):
    """Rows (t, j) against the oracle: token t sees positions 0 .. L + t (the span's own
    rows already in Kc, Vc)."""
    worst = 0.0
    for t in tokens:
        for j in heads:
            ref = oracle.attn_row([-1], L + t, Kc, Vc, h["q"][t:t + 1], h["k"][t:t + 1], h["v"][t:t + 1], 0, j)
            err = rel_err(got[t, j], ref)
            worst = max(worst, err)
            assert err <= gu.TOL_BF16_OUT, f"token {t} head {j}: {err:.3e}"
    return worst


def test_chunked_two_pieces():
    L, T = 300, 2100  # pieces of 2,048 and 52 tokens
    _say(f"chunked prefill: {T} tokens at {L} (two pieces)")
    inst = Instance(SPAN, SEED, lengths=[L], capacity=[L + T + 64])
    eng = inst.engine()
    host, dev = span_inputs(inst, T)
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    w = inst.w
    gi = ai = 0
    tokens = sorted(set(list(range(0, T, 97)) + [2046, 2047, 2048, 2049, T - 1]))
    for l, kind in enumerate(w.layer_kind):
        h = host[l]
        got = _f32(to_host(dev[l]["o"], w.dtype))
        if kind == 0:
            ref, S = oracle_chain(inst.h_state[0][gi], h["q"], h["k"], h["v"], h["alpha"], h["beta"])
            err = gu.max_rel_per_head(got, ref)
            assert err <= gu.TOL_BF16_OUT, f"layer {l}: {err:.3e}"
            serr = rel_err(inst.state[0][gi].cpu().numpy(), S)
            assert serr <= gu.TOL_F32, f"layer {l} state: {serr:.3e}"
            _say(f"  layer {l} (GDN): outputs {err:.2e}, state {serr:.2e}")
            gi += 1
        else:
            Kf = inst.h_kc[0][ai].copy()
            Vf = inst.h_vc[0][ai].copy()
            Kf[:, L:L + T] = np.transpose(h["k"], (1, 0, 2))
            Vf[:, L:L + T] = np.transpose(h["v"], (1, 0, 2))
            worst = _check_attn_rows(got, h, Kf, Vf, L, tokens, range(w.attn_hq))
            for name, cache in (("k", inst.kc[0]), ("v", inst.vc[0])):
                rows = to_host(cache[ai, :, L:L + T], w.dtype)
                assert np.array_equal(rows, np.transpose(h[name], (1, 0, 2)))
            _say(f"  layer {l} (attention, {len(tokens)} tokens): {worst:.2e}")
            ai += 1
    eng.close()


def _moves(scores, keys, tile=32, lazy=8.0):
    """How often a tile's max exceeds the running max by more than `lazy` within the first
    `keys` keys (the rule under which the running max moves after the first tile)."""
    count, run = 0, -np.inf
    for t0 in range(0, keys, tile):
        mt = scores[t0:t0 + tile].max()
        if run > -np.inf and mt > run + lazy:
            count += 1
        if mt > run + lazy or run == -np.inf:
            run = mt
    return count


def test_chunked_peaked_softmax():
    """Unnormalised keys and queries drawn as 12 N(0,1): scores spread over tens of units, so
    the running max of a row moves after its first tile and the accumulators are rescaled in
    the tile loop.  With at most four key splits and L + T >= 1,024 every split holds at least
    256 keys, so moves within the first 256 keys happen inside the first split."""
    L, T = 2000, 200
    _say(f"chunked prefill, peaked softmax: {T} tokens at {L}")
    inst = Instance(SPAN, SEED, lengths=[L], capacity=[L + T + 64], sharp=True, q_scale=12.0)
    eng = inst.engine()
    host, dev = span_inputs(inst, T, sharp=True, q_scale=12.0)
    w = inst.w
    l = 1  # the first attention layer
    h = host[l]
    G = w.attn_hq // w.attn_hkv
    moves = 0
    for t in (0, T - 1):
        for j in (0, w.attn_hq - 1):
            q = _f32(h["q"][t, j]).astype(np.float64)
            K = _f32(inst.h_kc[0][0][j // G, :L]).astype(np.float64)
            moves += _moves((K @ q) * (1.0 / np.sqrt(w.attn_d)) / np.log(2.0), 256)
    assert moves > 0, "the inputs never move the running max after the first tile"
    _say(f"  running-max moves in the first 256 keys (4 sampled rows, from the inputs): {moves}")
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    got = _f32(to_host(dev[l]["o"], w.dtype))
    Kf = inst.h_kc[0][0].copy()
    Vf = inst.h_vc[0][0].copy()
    Kf[:, L:L + T] = np.transpose(h["k"], (1, 0, 2))
    Vf[:, L:L + T] = np.transpose(h["v"], (1, 0, 2))
    worst = _check_attn_rows(got, h, Kf, Vf, L, [0, 1, 63, 64, 127, 150, T - 1], range(w.attn_hq))
    _say(f"  attention (7 tokens x {w.attn_hq} heads): {worst:.2e}")
    eng.close()


def test_chunked_anchors_and_rollback():
    L, T, every = 300, 300, 128  # anchors at 384 and 512
    inst = Instance(SPAN, SEED, lengths=[L], capacity=[L + T + 64])
    eng = inst.engine()
    w = inst.w
    n_max = 8
    astate = torch.zeros((n_max, w.n_gdn, w.gdn_hv, w.gdn_dv, w.gdn_dk), dtype=torch.float32, device="cuda")
    eng.set_anchors(0, every, n_max, astate)
    host, dev = span_inputs(inst, T)
    S0 = [s.copy() for s in inst.h_state[0]]
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    first = [to_host(d["o"], w.dtype).copy() for d in dev]
    final = inst.state[0].clone()
    gdn = [l for l, kind in enumerate(w.layer_kind) if kind == 0]
    for pos in (384, 512):
        assert eng.anchor_below(0, pos) == pos
        k = pos // every - 1
        for gi, l in enumerate(gdn):
            h = host[l]
            ref = oracle.gdn_commit(list(range(pos - L)), S0[gi], h["k"], h["v"], h["alpha"], h["beta"])
            err = rel_err(astate[k, gi].cpu().numpy(), ref)
            assert err <= gu.TOL_F32, f"anchor {pos} layer {l}: {err:.3e}"
    # back to 384, then the rest of the span again
    eng.rollback_to(0, 384, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == 384
    rest = [{name: x[384 - L:] for name, x in d.items()} for d in dev]
    for d in rest:
        d["o"].zero_()
    eng.forward_chunked(0, T - (384 - L), rest, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    for l, d in enumerate(dev):
        assert np.array_equal(to_host(d["o"], w.dtype)[384 - L:], first[l][384 - L:]), f"layer {l}"
    assert torch.equal(inst.state[0], final)
    eng.close()


def test_chunked_full_size_sampled():
    """The stack's head shapes (16 q/k and 32 v GDN heads of 128 x 128; 24 q / 4 kv heads of
    256) at 65,536 resident tokens, one GDN and one attention layer, a 2,048-token span."""
    base = synth.WORKLOADS["stack_65k"]
    w = synth.Workload("stack_65k_prefill", [0, 1], base.gdn_hk, base.gdn_hv, base.gdn_dk, base.gdn_dv,
                       base.attn_hq, base.attn_hkv, base.attn_d, base.dtype, [65536], 16, "draft")
    L, T = 65536, 2048
    _say(f"chunked prefill, full size: {T} tokens at {L}")
    inst = Instance(w, SEED, capacity=[L + T + 64])
    eng = inst.engine()
    host, dev = span_inputs(inst, T, tag="prefill")
    eng.forward_chunked(0, T, dev, gu.stream())
    gu.sync()
    assert eng.kv_length(0) == L + T
    # GDN: v heads 0, 1 (q/k head 0) and 30, 31 (q/k head 15)
    h = host[0]
    vh, kh = [0, 1, 30, 31], [0, 15]
    ref, S = oracle_chain(inst.h_state[0][0][vh], h["q"][:, kh], h["k"][:, kh], h["v"][:, vh],
                          h["alpha"][:, vh], h["beta"][:, vh], piece=512)
    got = _f32(to_host(dev[0]["o"], w.dtype))[:, vh]
    err = gu.max_rel_per_head(got, ref)
    assert err <= gu.TOL_BF16_OUT, f"GDN outputs: {err:.3e}"
    serr = rel_err(inst.state[0][0][vh].cpu().numpy(), S)
    assert serr <= gu.TOL_F32, f"GDN state: {serr:.3e}"
    _say(f"  GDN (4 heads): outputs {err:.2e}, state {serr:.2e}")
    # attention: sampled tokens, every q head, over all 65,536 + t keys
    h = host[1]
    Kf = inst.h_kc[0][0].copy()
    Vf = inst.h_vc[0][0].copy()
    Kf[:, L:L + T] = np.transpose(h["k"], (1, 0, 2))
    Vf[:, L:L + T] = np.transpose(h["v"], (1, 0, 2))
    got = _f32(to_host(dev[1]["o"], w.dtype))
    worst = _check_attn_rows(got, h, Kf, Vf, L, [0, 1, 21, 22, 127, 1000, 2047], range(w.attn_hq))
    _say(f"  attention (7 tokens x 24 heads): {worst:.2e}")
    eng.close()


def test_chunked_refusals_change_nothing():
    inst = Instance(SPAN, SEED, lengths=[300], capacity=[400])
    eng = inst.engine()
    host, dev = span_inputs(inst, 64)
    before = inst.state[0].clone()
    with pytest.raises(hdt.HdtError) as e:
        eng.forward_chunked(0, 101, dev, gu.stream())  # past capacity
    assert e.value.status == -4
    eng.forward_tree([inst.tree_arg(0)], gu.stream())
    with pytest.raises(hdt.HdtError) as e:
        eng.forward_chunked(0, 64, dev, gu.stream())  # a round is pending
    assert e.value.status == -5
    gu.sync()
    assert torch.equal(inst.state[0], before) and eng.kv_length(0) == 300
    eng.close()

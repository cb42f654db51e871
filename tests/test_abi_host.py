"""The C ABI on the host (no GPU): the library loads, exports what include/hdt.h declares,
computes tree metadata bit for bit like the oracle, and refuses bad calls with the right
status while changing nothing.  No call here reaches a HIP runtime function."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

hdt = pytest.importorskip("hybrid_deltanet_tree_amd")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "hdt.h")
FAKE = 1 << 20  # a 16-byte-aligned address that is never dereferenced on the host


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hdt_status|void|const char \*)\s*(hdt_\w+)\(", src,
                                 re.M)))


def test_header_is_plain_c():
    # include/hdt.h compiles as C11 in a C program that uses every part of it it needs
    import subprocess
    src = os.path.join(os.path.dirname(__file__), "c_abi", "verify_round.c")
    subprocess.check_call(["gcc", "-fsyntax-only", "-std=c11", "-Wall", "-Werror",
                           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I" + os.path.dirname(HEADER), src])


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(hdt.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(hdt.EXPORTED)


@pytest.mark.parametrize("seed", range(8))
def test_tree_meta_matches_oracle(seed):
    parent = synth.random_tree(seed, "abi/meta", 64 if seed % 2 else 17, 20)
    d0, m0, a0, p0 = oracle.tree_meta(parent, L=12345)
    d1, m1, a1, p1 = hdt.tree_meta(parent, L=12345)
    assert list(d0) == d1
    assert [int(x) for x in m0] == m1
    assert [list(r) for r in a0] == a1
    assert list(p0) == p1


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 3], [-1, -1], [-1, 0, -2]])
def test_tree_meta_rejects(bad):
    with pytest.raises(hdt.HdtError) as e:
        hdt.tree_meta(bad)
    assert e.value.status == -2


def make_engine(**kw):
    args = dict(gdn_hk=2, gdn_hv=4, gdn_dk=64, gdn_dv=64, attn_hq=4, attn_hkv=2, attn_d=64,
                io_dtype=hdt.HDT_BF16, max_nodes=8,
                slots=[dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=1000, length=100),
                       dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=300, length=295)])
    kinds = kw.pop("layer_kind", [0, 0, 0, 1])
    args.update(kw)
    return hdt.Engine(kinds, **args)


@pytest.mark.parametrize("kw,status", [
    (dict(layer_kind=[0, 2]), -1),
    (dict(gdn_dk=96, gdn_dv=96), -7),
    (dict(gdn_hv=3), -1),
    (dict(max_nodes=0), -1),
    (dict(max_nodes=65), -1),
    (dict(attn_d=128), -7),
    (dict(attn_hq=5), -1),
    (dict(attn_hq=34, attn_hkv=2), -7),
    (dict(attn_hq=14, attn_hkv=2, attn_d=256), -7),
    (dict(io_dtype=hdt.HDT_F32, attn_d=256), -7),
    (dict(io_dtype=7), -1),
    (dict(slots=[dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=10, length=11)]), -1),
    (dict(slots=[dict(gdn_state=0, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1)]), -1),
    (dict(slots=[dict(gdn_state=FAKE + 4, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1)]), -1),
    (dict(slots=[]), -1),
    (dict(gdn_conv=-1, gdn_conv_weight=FAKE), -1),
    (dict(gdn_conv=5, gdn_conv_weight=FAKE), -7),
    (dict(gdn_conv=4), -1),                                   # no taps
    (dict(gdn_conv=4, gdn_conv_weight=FAKE + 8), -1),         # misaligned taps
    (dict(gdn_conv=4, gdn_conv_weight=FAKE), -1),             # slots without conv tails
    (dict(gdn_conv=4, gdn_conv_weight=FAKE,
          slots=[dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1,
                      conv_state=FAKE + 4)]), -1),
])
def test_create_rejects(kw, status):
    with pytest.raises(hdt.HdtError) as e:
        make_engine(**kw)
    assert e.value.status == status


def test_create_accepts_conv():
    conv_slot = dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1,
                     conv_state=FAKE)
    make_engine(gdn_conv=4, gdn_conv_weight=FAKE, slots=[conv_slot]).close()
    # width 1 keeps no tail; no GDN layer needs no taps
    make_engine(gdn_conv=1, gdn_conv_weight=FAKE).close()
    make_engine(gdn_conv=4, layer_kind=[1]).close()


def test_forward_rejects_misaligned_conv_inputs():
    conv_slot = dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1,
                     conv_state=FAKE)
    eng = make_engine(gdn_conv=4, gdn_conv_weight=FAKE, slots=[conv_slot])
    layers = fake_layers()
    layers[1] = dict(layers[1], k=FAKE + 2)
    with pytest.raises(hdt.HdtError) as e:
        eng.forward_tree([(0, [-1, 0], layers)])
    assert e.value.status == -1 and "conv inputs" in eng.last_error()
    assert eng.kv_length(0) == 1
    eng.close()


def test_walk_commit_rejects_without_touching_the_device():
    e = make_engine()
    with pytest.raises(hdt.HdtError) as err:
        e.walk_commit(0, FAKE, FAKE, FAKE)
    assert err.value.status == -5  # no pending round
    for args, status in (((5, FAKE, FAKE, FAKE), -1), ((0, 0, FAKE, FAKE), -1),
                         ((0, FAKE, FAKE, None), -1), ((0, FAKE + 2, FAKE, FAKE), -1)):
        with pytest.raises(hdt.HdtError) as err:
            e.walk_commit(*args)
        assert err.value.status == status
    assert e.kv_length(0) == 100
    e.close()


def test_span_and_anchor_rejections_on_the_host():
    e = make_engine()
    layers = [dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, o=FAKE) for _ in range(4)]
    for args, status in (((0, 0, layers), -1), ((7, 4, layers), -1), ((1, 6, layers), -4)):
        with pytest.raises(hdt.HdtError) as err:
            e.forward_span(*args)
        assert err.value.status == status
    bad = [dict(l) for l in layers]
    bad[3]["q"] = FAKE + 8  # attention buffers must be 16-byte aligned
    with pytest.raises(hdt.HdtError) as err:
        e.forward_span(0, 4, bad)
    assert err.value.status == -1
    assert e.kv_length(0) == 100 and e.kv_length(1) == 295
    assert e.anchor_below(0, 10 ** 6) == -1
    for args in ((0, -1, 4, FAKE), (0, 64, 0, FAKE), (0, 64, 4, None), (0, 64, 4, FAKE + 4)):
        with pytest.raises(hdt.HdtError):
            e.set_anchors(*args)
    e.set_anchors(0, 64, 4, FAKE)
    assert e.anchor_below(0, 10 ** 6) == -1  # nothing filled yet
    with pytest.raises(hdt.HdtError) as err:
        e.rollback_to(0, 64)  # below the length, no filled anchor there
    assert err.value.status == -7
    e.set_anchors(0, 0)
    e.close()


def test_chunked_prefill_rejections_on_the_host():
    """forward_chunked refuses bad arguments and the shapes it does not run before anything
    touches the device, and a refused call changes nothing."""
    ok = dict(gdn_dk=128, gdn_dv=128, attn_hq=12, attn_hkv=2, attn_d=256)
    e = make_engine(**ok)
    layers = fake_layers()
    for args, status in (((0, 0, layers), -1), ((7, 4, layers), -1), ((1, 6, layers), -4)):
        with pytest.raises(hdt.HdtError) as err:
            e.forward_chunked(*args)
        assert err.value.status == status
    bad = [dict(l) for l in layers]
    bad[0]["v"] = FAKE + 8  # 16-byte alignment
    with pytest.raises(hdt.HdtError) as err:
        e.forward_chunked(0, 4, bad)
    assert err.value.status == -1
    no_gates = [dict(l) for l in layers]
    no_gates[1]["alpha"] = None
    with pytest.raises(hdt.HdtError) as err:
        e.forward_chunked(0, 4, no_gates)
    assert err.value.status == -1
    assert e.kv_length(0) == 100 and e.kv_length(1) == 295
    e.close()
    for kw in (dict(ok, gdn_dk=64, gdn_dv=64), dict(ok, attn_hq=4, attn_d=64),
               dict(ok, io_dtype=hdt.HDT_F32, attn_hq=4, attn_d=64)):
        e = make_engine(**kw)
        with pytest.raises(hdt.HdtError) as err:
            e.forward_chunked(0, 4, layers)
        assert err.value.status == -7, kw
        assert e.kv_length(0) == 100
        e.close()


def fake_layers(n_layers=4):
    return [dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, o=FAKE) for _ in range(n_layers)]


@pytest.mark.parametrize("trees,status", [
    ([], -1),
    ([(0, [-1, 0], fake_layers())] * 9, -1),
    ([(2, [-1, 0], fake_layers())], -1),
    ([(0, [-1, 0], fake_layers()), (0, [-1], fake_layers())], -1),
    ([(0, list(range(-1, 8)), fake_layers())], -1),
    ([(0, [-1, 1], fake_layers())], -2),
    ([(0, [0, 0], fake_layers())], -2),
    ([(1, [-1, 0, 1, 2, 3, 4], fake_layers())], -4),
    ([(0, [-1], [dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE)] * 4)], -1),
    ([(0, [-1], fake_layers()[:3] + [dict(q=FAKE + 2, k=FAKE, v=FAKE, o=FAKE)])], -1),
])
def test_forward_tree_rejects_and_changes_nothing(trees, status):
    e = make_engine()
    with pytest.raises(hdt.HdtError) as err:
        e.forward_tree(trees)
    assert err.value.status == status
    assert e.last_error()
    assert e.kv_length(0) == 100 and e.kv_length(1) == 295
    # nothing pending: commit is out of order, rollback to the length is a no-op
    with pytest.raises(hdt.HdtError) as err:
        e.commit_tree(0, [0])
    assert err.value.status == -5
    e.rollback_to(0, 100)
    assert e.kv_length(0) == 100


def test_sequencing_rules_without_pending_round():
    e = make_engine()
    with pytest.raises(hdt.HdtError) as err:
        e.rollback_to(0, 99)
    assert err.value.status == -7
    with pytest.raises(hdt.HdtError) as err:
        e.rollback_to(0, 101)
    assert err.value.status == -5
    with pytest.raises(hdt.HdtError) as err:
        e.reset(0, 1001)
    assert err.value.status == -1
    e.reset(0, 7)
    assert e.kv_length(0) == 7
    with pytest.raises(hdt.HdtError):
        e.kv_length(5)


def _ladder_next(s):
    return (s + max(32, s // 32) + 31) // 32 * 32


def test_split_size_depends_on_position_only():
    # bf16 storage: a row at position p (p + 1 keys) takes the smallest rung of the
    # ladder 128, s + max(32, s/32) rounded up to 32, ... that cuts its keys into at most
    # 256 / (H_kv row_groups) splits, a row group being 96 query rows of the engine's
    # largest tree.  The slot's capacity and committed length never enter.
    e = make_engine()
    assert e.split_size(0, 0) == 128 and e.split_size(1, 299) == 128
    big = [dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=65536 + 1024, length=65536),
           dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=262144 + 1024, length=0)]
    e2 = make_engine(attn_hkv=4, attn_hq=24, attn_d=256, slots=big)
    assert e2.split_size(0, 65536) == 1056 and e2.split_size(1, 65536) == 1056
    assert e2.split_size(0, 65535) == 1024 and e2.split_size(1, 262144) == 4160
    assert e2.split_size(1, 8192) == 160 and e2.split_size(1, 0) == 128
    e2.reset(0, 5)
    assert e2.split_size(0, 65536) == 1056
    with pytest.raises(hdt.HdtError):
        e2.split_size(0, 65536 + 1024)
    with pytest.raises(hdt.HdtError):
        e2.split_size(0, -1)
    # invariants over positions and shapes: a rung of the ladder, at most per_head
    # splits, the rung below would need more, nondecreasing in the position
    for hkv, mn in ((1, 8), (2, 8), (4, 16), (4, 17), (4, 33), (8, 64), (4, 64)):
        rg = -(-(mn * 2) // 96) if hkv != 4 else -(-(mn * 6) // 96)
        hq = hkv * (6 if hkv == 4 else 2)
        slot = [dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=1 << 20, length=0)]
        eng = make_engine(attn_hkv=hkv, attn_hq=hq, attn_d=256 if hkv == 4 else 64, max_nodes=mn,
                          slots=slot)
        per_head = max(1, 256 // (hkv * rg))
        rungs, x = set(), 128
        while x < (1 << 21):
            rungs.add(x)
            x = _ladder_next(x)
        prev = 0
        for pos in (0, 1, 127, 128, 4095, 8191, 65535, 65536, 65537, 131071, 262143, 262144,
                    (1 << 20) - 1):
            sz = eng.split_size(0, pos)
            k = pos + 1
            assert sz in rungs and sz >= prev
            assert -(-k // sz) <= per_head
            assert sz == 128 or -(-k // max(r for r in rungs if r < sz)) > per_head
            prev = sz
    # 32-node trees at 6 q heads per kv head: 192 rows, two row groups per split
    e3 = make_engine(attn_hkv=4, attn_hq=24, attn_d=256, max_nodes=32, slots=big)
    assert e3.split_size(1, 262144) == 8384 and e3.split_size(0, 65536) == 2080
    # float32 storage: per slot, from the capacity alone (a power of two)
    f32 = make_engine(io_dtype=hdt.HDT_F32, slots=big[:1])
    assert f32.split_size(0, 0) == 512 and f32.split_size(0, 65000) == 512
    f32b = make_engine(io_dtype=hdt.HDT_F32, attn_hkv=4, attn_hq=8, slots=big)
    assert f32b.split_size(0, 7) == 1024 and f32b.split_size(1, 7) == 4096


def test_one_hip_runtime_in_process():
    # libhdt and PyTorch must share one HIP runtime: two mapped copies of
    # libamdhip64 mean device pointers and streams cross runtime instances.
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_io_list_must_have_one_entry_per_layer():
    """The binding refuses a per-layer io list of the wrong length before the library could
    read past the end of the array it builds."""
    e = make_engine()
    for layers in (fake_layers()[:3], fake_layers() + fake_layers()[:1], []):
        with pytest.raises(ValueError):
            e.forward_tree([(0, [-1, 0], layers)])
        with pytest.raises(ValueError):
            e.forward_block(0, 2, layers)
        with pytest.raises(ValueError):
            e.forward_span(0, 2, layers)
        with pytest.raises(ValueError):
            e.forward_chunked(0, 2, layers)
    assert e.kv_length(0) == 100
    e.close()


class _FakeBuf:
    """A device-buffer stand-in: an address and a size, never dereferenced on the host."""

    def __init__(self, ptr, nbytes):
        self.ptr, self.nbytes = ptr, nbytes

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def test_state_snapshot_size_and_host_refusals():
    e = make_engine()
    n = e.state_bytes()
    # header, the GDN state (3 layers x 4 heads x 64 x 64 float32), no conv tails
    assert n == 256 + 3 * 4 * 64 * 64 * 4
    conv_slot = dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=10, length=1,
                     conv_state=FAKE)
    ec = make_engine(gdn_conv=4, gdn_conv_weight=FAKE, slots=[conv_slot])
    C = 2 * 2 * 64 + 4 * 64
    assert ec.state_bytes() == 256 + 3 * 4 * 64 * 64 * 4 + 3 * 3 * C * 2
    ec.close()
    for slot, buf, status in ((5, _FakeBuf(FAKE, n), -1), (0, _FakeBuf(0, n), -1),
                              (0, _FakeBuf(FAKE + 16, n), -1), (0, _FakeBuf(FAKE, n - 1), -1)):
        for restore in (False, True):
            with pytest.raises(hdt.HdtError) as err:
                e.state_copy(slot, buf, restore=restore)
            assert err.value.status == status
    assert e.kv_length(0) == 100
    e.close()


def test_noalloc_forward_refuses_more_than_its_static_scratch():
    """hdt_forward_tree_noalloc checks its scratch against the 48 MiB static array on the host,
    before it touches the device: a 64-layer model at the 27B-like shapes with 64-node trees
    needs more (50 MB of pending corrections alone)."""
    kinds = [1 if l % 4 == 3 else 0 for l in range(64)]
    slot = [dict(gdn_state=FAKE, k_cache=FAKE, v_cache=FAKE, capacity=70000, length=65536)]
    e = make_engine(layer_kind=kinds, gdn_hk=16, gdn_hv=32, gdn_dk=128, gdn_dv=128, attn_hq=24,
                    attn_hkv=4, attn_d=256, max_nodes=64, slots=slot)
    with pytest.raises(hdt.HdtError) as err:
        e.forward_tree_noalloc([(0, [-1, 0], fake_layers(64))])
    assert err.value.status == -4 and "static scratch" in e.last_error()
    assert e.kv_length(0) == 65536
    with pytest.raises(hdt.HdtError) as err:   # ... and is still subject to the pending rules
        e.commit_tree(0, [0])
    assert err.value.status == -5
    e.close()


def test_graph_entry_points_refuse_null_on_the_host():
    """The reusable-graph verbs refuse a missing graph or output pointer before any HIP call."""
    import ctypes
    e = make_engine()
    assert hdt.hdt_graph_create(e.h, None) == -1
    assert hdt.hdt_graph_forward(None, 1, None, None) == -1
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert hdt.hdt_graph_stats(None, ctypes.byref(a), ctypes.byref(b)) == -1
    hdt.hdt_graph_destroy(None)  # a no-op
    e.close()

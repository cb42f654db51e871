"""The seeded input generator: reproducible, sliceable, shaped as the workloads ask."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 1234567: the first outputs of the published generator
    # (Steele, Lea, Flood 2014; the same sequence as Java's SplittableRandom and the
    # reference C code by S. Vigna).
    expected = [6457827717110365317, 3203168211198807973, 9817491932198370423]
    assert [synth.u64(1234567, c) for c in range(3)] == expected


def test_normals_reproducible_and_sliceable():
    full = synth.fill(7, "x", synth.NORMAL, (50, 33), dtype="f32")
    part = synth.fill(7, "x", synth.NORMAL, (50, 33), dtype="f32", row0=20, rows=10)
    assert np.array_equal(full[20:30], part)
    assert np.array_equal(full, synth.fill(7, "x", synth.NORMAL, (50, 33), dtype="f32"))
    assert not np.array_equal(full, synth.fill(8, "x", synth.NORMAL, (50, 33), dtype="f32"))


def test_distributions():
    x = synth.fill(3, "n", synth.NORMAL, (2000, 100), dtype="f32").astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = synth.fill(3, "u", synth.NORMAL_L2, (100, 128), dtype="f32").astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, rtol=1e-6)
    b = synth.fill(3, "b", synth.SIGMOID, (1000, 32), dtype="f32")
    a = synth.fill(3, "a", synth.EXP_NEG_SOFTPLUS, (1000, 32), dtype="f32")
    assert (b > 0).all() and (b < 1).all() and abs(np.median(b) - 0.5) < 0.02
    assert (a > 0).all() and (a < 1).all() and abs(np.median(a) - 0.5) < 0.02


def test_bf16_is_round_to_nearest_even_of_f32():
    f = synth.fill(5, "r", synth.NORMAL, (64, 64), dtype="f32")
    h = synth.fill(5, "r", synth.NORMAL, (64, 64), dtype="bf16")
    w = synth.bf16_bits_to_f32(h)
    # the widened bf16 value is the nearest bf16 to the float32 value
    assert (np.abs(w - f) <= np.abs(f) * 2.0 ** -8).all()
    bits = f.view(np.uint32)
    exp_bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(h, exp_bits)


def test_trees():
    for seed in range(20):
        for n in (16, 32):
            p = synth.draft_tree(seed, "t", n, 15)
            assert len(p) == n and p[0] == -1
            assert all(0 <= p[i] < i for i in range(1, n))
            assert max(synth.depths(p)) <= 15
        r = synth.random_tree(seed, "r", 8, 4)
        assert max(synth.depths(r)) <= 4 and all(0 <= r[i] < i for i in range(1, 8))
        path = synth.accepted_path(seed, "a", p)
        assert path[0] == 0 and all(p[path[d]] == path[d - 1] for d in range(1, len(path)))
    # a 16-node draft tree: a long block chain plus a few lookup branches
    p = synth.draft_tree(1, "t", 16, 15)
    assert synth.depths(p).count(1) >= 1 and 9 <= max(synth.depths(p)) <= 15
    assert synth.chain_tree(4) == [-1, 0, 1, 2]


def test_workloads():
    w = synth.WORKLOADS["stack_65k"]
    assert w.n_gdn == 48 and w.n_attn == 16 and w.layer_kind[3] == 1 and w.layer_kind[4] == 0
    assert synth.WORKLOADS["joint4"].lengths == [131072, 8192, 8192, 8192]
    S = synth.gdn_state(synth.WORKLOADS["tiny"], 1, 0, 0)
    assert S.shape == (1, 64, 64) and S.dtype == np.float32
    assert abs(S.std() - 1 / 8) < 0.01

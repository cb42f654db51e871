"""The price-table sweep runs on the device: one small entry with two joint slots."""
import pytest

pytestmark = pytest.mark.gpu


def test_price_entry_small():
    import torch
    from hybrid_deltanet_tree_amd import price_table as pt
    print("price entry: 4 nodes, 2048 tokens, 2 slots", flush=True)
    mem = pt.make_slots(2, 4096, 20261202)
    r = pt.measure(4, 2048, 2, mem, reps=3, warmup=1)
    assert r["n_nodes"] == 4 and r["context"] == 2048 and r["slots"] == 2
    assert r["commit_path"] == 4
    assert 0 < r["verify_p10_ms"] <= r["verify_ms"] <= r["verify_p90_ms"] < 1000
    assert 0 < r["commit_ms"] < 1000
    torch.cuda.synchronize()

"""Verify-cost price table: the measured time of one verify round of the 64-layer stack on
this GPU, against tree size, resident context and the number of slots verified jointly.

StairCut, the tree cutter of "One request, end to end" (2.6, "The decode loop"), trims the
merged draft tree by comparing expected accepted tokens with what the verify pass costs on
the device; "Adding a model" ("The adapter path in ten steps", the data-files step) keeps
one such price file per model profile and device.  This module measures those prices and
writes them as JSON, one entry per (n_nodes, context, slots):

  python -m hybrid_deltanet_tree_amd.price_table --out hybrid_deltanet_tree_amd/prices/hybrid64_bf16.mi355x.json

Timing only: resident K/V rows are unit-norm random vectors, the state random; every slot
holds the same context, and each tree is a chain of up to 12 nodes with runs of two hung
off chain nodes, the shape of a block draft merged with lookup continuations.  verify_ms
is the median of the joint forward_tree captured as one HIP graph and replayed;
commit_ms is the median eager commit_tree of the tree's deepest root path on slot 0.
"""
import argparse
import json
import os
import statistics
import time

import torch

from . import HDT_BF16, Engine

KINDS = [1 if l % 4 == 3 else 0 for l in range(64)]          # 48 GDN + 16 attention
GDN = dict(gdn_hk=16, gdn_hv=32, gdn_dk=128, gdn_dv=128)
ATTN = dict(attn_hq=24, attn_hkv=4, attn_d=256)


def tree_of(n: int) -> list:
    """A chain of min(n, 12) nodes; the other nodes as runs of two hung off chain nodes
    1, 4, 7, 10, 1, ... (parent order: every parent index is below its child's)."""
    c = min(n, 12)
    parent = [-1] + list(range(c - 1))
    anchor = min(1, c - 1)
    while len(parent) < n:
        parent.append(anchor)
        if len(parent) < n:
            parent.append(len(parent) - 1)
        anchor = anchor + 3 if anchor + 3 < c else min(1, c - 1)
    return parent


def deepest_path(parent: list) -> list:
    """Root-to-node path of the deepest node (the lowest index among equals)."""
    depth = []
    for p in parent:
        depth.append(0 if p < 0 else depth[p] + 1)
    i = max(range(len(parent)), key=lambda j: (depth[j], -j))
    path = []
    while i >= 0:
        path.append(i)
        i = parent[i]
    return path[::-1]


def layer_io(n: int, dev):
    io = []
    for kind in KINDS:
        if kind == 0:
            d = dict(q=torch.randn(n, 16, 128, device=dev), k=torch.randn(n, 16, 128, device=dev),
                     v=torch.randn(n, 32, 128, device=dev), alpha=torch.rand(n, 32, device=dev),
                     beta=torch.rand(n, 32, device=dev))
            d["q"] = torch.nn.functional.normalize(d["q"], dim=-1)
            d["k"] = torch.nn.functional.normalize(d["k"], dim=-1)
            d = {k: v.to(torch.bfloat16) for k, v in d.items()}
            d["o"] = torch.empty(n, 32, 128, dtype=torch.bfloat16, device=dev)
        else:
            d = dict(q=torch.nn.functional.normalize(torch.randn(n, 24, 256, device=dev), dim=-1),
                     k=torch.nn.functional.normalize(torch.randn(n, 4, 256, device=dev), dim=-1),
                     v=torch.randn(n, 4, 256, device=dev))
            d = {k: v.to(torch.bfloat16) for k, v in d.items()}
            d["o"] = torch.empty(n, 24, 256, dtype=torch.bfloat16, device=dev)
        io.append(d)
    return io


def measure(n_nodes, context, n_slots, slots_mem, reps, warmup):
    """Median / p10 / p90 ms of one joint forward_tree over n_slots trees of n_nodes, and
    the median ms of committing the deepest path on slot 0."""
    dev = "cuda"
    descs = [dict(gdn_state=m["state"], k_cache=m["kc"], v_cache=m["vc"], capacity=m["cap"],
                  length=context) for m in slots_mem[:n_slots]]
    eng = Engine(KINDS, **GDN, **ATTN, io_dtype=HDT_BF16, max_nodes=n_nodes, slots=descs)
    parent = tree_of(n_nodes)
    path = deepest_path(parent)
    ios = [layer_io(n_nodes, dev) for _ in range(n_slots)]
    trees = [(s, parent, ios[s]) for s in range(n_slots)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def drop():
        for s in range(n_slots):
            eng.rollback_to(s, context, sp)

    for _ in range(warmup):  # eager: the first call allocates the engine's scratch
        eng.forward_tree(trees, sp)
        drop()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        eng.forward_tree(trees, torch.cuda.current_stream().cuda_stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    g.replay()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    verify = sorted(a.elapsed_time(b) for a, b in ev)
    del g
    drop()
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in cev:
        eng.forward_tree(trees, sp)
        a.record(stream)
        eng.commit_tree(0, path, sp)
        b.record(stream)
        for s in range(1, n_slots):
            eng.rollback_to(s, context, sp)
        eng.reset(0, context)  # timing only: slot 0's contents are not kept consistent
    torch.cuda.synchronize()
    commit = sorted(a.elapsed_time(b) for a, b in cev)
    eng.close()
    return {"n_nodes": n_nodes, "context": context, "slots": n_slots,
            "verify_ms": round(statistics.median(verify), 4),
            "verify_p10_ms": round(verify[len(verify) // 10], 4),
            "verify_p90_ms": round(verify[(9 * len(verify)) // 10], 4),
            "commit_path": len(path), "commit_ms": round(statistics.median(commit), 4)}


def make_slots(n_slots, cap, seed):
    """Per-slot K/V caches [16][4][cap][256] bf16 (unit-norm K rows) and GDN state
    [48][32][128][128] f32, filled layer by layer to bound the temporaries."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    mem = []
    for _ in range(n_slots):
        kc = torch.empty(16, 4, cap, 256, dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        for l in range(16):
            x = torch.randn(4, cap, 256, device="cuda", generator=gen)
            kc[l] = torch.nn.functional.normalize(x, dim=-1).to(torch.bfloat16)
            vc[l] = torch.randn(4, cap, 256, device="cuda", generator=gen).to(torch.bfloat16)
            del x
        state = torch.randn(48, 32, 128, 128, device="cuda", generator=gen) * (1.0 / 128) ** 0.5
        mem.append(dict(kc=kc, vc=vc, state=state, cap=cap))
    torch.cuda.synchronize()
    return mem


PRICE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "prices")


def load(path: str = None) -> dict:
    """A price file; by default the one measured on MI355X for the 64-layer bf16 stack."""
    with open(path or os.path.join(PRICE_DIR, "hybrid64_bf16.mi355x.json")) as f:
        return json.load(f)


def lookup(table: dict, n_nodes: int, context: int, slots: int = 1) -> float:
    """Verify ms for a tree of n_nodes over `context` resident tokens in a joint pass of
    `slots` slots: the smallest measured tree size >= n_nodes and slot count >= slots,
    linear in context between the two nearest measured contexts (clamped at the ends,
    extrapolated linearly beyond the largest)."""
    rows = table["entries"]
    ns = sorted({r["n_nodes"] for r in rows if r["n_nodes"] >= n_nodes})
    ss = sorted({r["slots"] for r in rows if r["slots"] >= slots})
    if not ns or not ss:
        raise KeyError(f"no price for {n_nodes} nodes over {slots} slots")
    pts = sorted((r["context"], r["verify_ms"]) for r in rows
                 if r["n_nodes"] == ns[0] and r["slots"] == ss[0])
    if context <= pts[0][0]:
        return pts[0][1]
    lo, hi = pts[-2:] if context >= pts[-1][0] else next(
        (a, b) for a, b in zip(pts, pts[1:]) if a[0] <= context <= b[0])
    if lo[0] == hi[0]:
        return hi[1]
    return lo[1] + (hi[1] - lo[1]) * (context - lo[0]) / (hi[0] - lo[0])


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default="verify_price_table.json")
    ap.add_argument("--nodes", default="1,2,4,8,12,16,24,32")
    ap.add_argument("--contexts", default="8192,32768,65536,131072,262144")
    ap.add_argument("--slots", default="1,2,4")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    args = ap.parse_args()
    nodes = [int(x) for x in args.nodes.split(",")]
    contexts = [int(x) for x in args.contexts.split(",")]
    slot_counts = [int(x) for x in args.slots.split(",")]
    torch.manual_seed(20261202)
    mem = make_slots(max(slot_counts), max(contexts) + max(nodes) + 64, 20261202)
    t0 = time.perf_counter()
    rows = []
    for ns in slot_counts:
        for L in contexts:
            for n in nodes:
                r = measure(n, L, ns, mem, args.reps, args.warmup)
                rows.append(r)
                print(json.dumps(r), flush=True)
    props = torch.cuda.get_device_properties(0)
    out = {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
           "compute_units": props.multi_processor_count,
           "model": "64 layers, 3:1 (48 Gated DeltaNet: 16 qk / 32 v heads, dk = dv = 128, fp32 state; "
                    "16 attention: 24 q / 4 kv heads, D = 256); bf16 activations and K/V",
           "timing": f"verify_ms: median of {args.reps} HIP graph replays of one joint "
                     "forward_tree; commit_ms: median eager commit_tree of the deepest path",
           "entries": rows, "elapsed_s": round(time.perf_counter() - t0, 1)}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {args.out} ({len(rows)} entries)")


if __name__ == "__main__":
    main()

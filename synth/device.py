"""Instantiate a synthetic workload in device memory for the GPU library.

Allocation and copying only: every value comes from ``synth`` and reaches the
device bit for bit.  Tests and the bench use this; the oracle reads the same
host arrays (small workloads) or regenerates the rows it needs (large ones).
"""
from __future__ import annotations

import numpy as np

import synth


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, dtype: str, device):
    """float32 array or bf16 bit patterns (uint16) -> torch tensor on `device`."""
    torch = _torch()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host(t, dtype: str) -> np.ndarray:
    """Inverse of to_device: bf16 -> uint16 bits, f32 -> float32."""
    torch = _torch()
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().astype(np.float32, copy=False)


def _tdtype(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class Instance:
    """A workload on the device.

    Per slot s: state[s] float32 [n_gdn][hv][dv][dk]; kc[s], vc[s] [n_attn][hkv][cap][D];
    io[s][l] dict of device tensors (q, k, v, alpha, beta for GDN layers; q, k, v for
    attention layers; o for both).  host[s][l] holds the host arrays of each layer's
    tree inputs; h_state / h_kc / h_vc hold the resident data when keep_host.
    With a conv width (w.extra["conv"]): conv_w float32 [n_gdn][C][width] taps (host:
    h_conv_w), tail[s] [n_gdn][width-1][C] committed pre-conv rows (host: h_tail[s]),
    and the GDN layers' q, k, v are pre-conv inputs.
    """

    def __init__(self, w: synth.Workload, seed: int, *, device="cuda", lengths=None,
                 trees=None, n_nodes=None, capacity=None, sharp=False, poison=False,
                 keep_host=True, tag="verify", q_scale=1.0, v_scale=1.0, host_layers=None,
                 kv_v_scale=1.0):
        torch = _torch()
        self.w, self.seed, self.device, self.sharp = w, seed, device, sharp
        self.q_scale, self.v_scale = q_scale, v_scale
        # layers whose resident data stays on the host (keep_host=False: none unless listed)
        self.host_layers = set(range(len(w.layer_kind))) if keep_host else set(host_layers or ())
        self.lengths = list(lengths if lengths is not None else w.lengths)
        ns = len(self.lengths)
        if trees is None:
            trees = [w.tree(seed, s) for s in range(ns)]
        self.trees = [list(t) for t in trees]
        nmax = max(len(t) for t in self.trees) if n_nodes is None else n_nodes
        if capacity is None:
            capacity = [L + max(64, 4 * nmax) for L in self.lengths]
        elif isinstance(capacity, int):
            capacity = [capacity] * ns
        self.capacity = list(capacity)
        dt, tdt = w.dtype, _tdtype(w.dtype)
        self.state, self.kc, self.vc, self.io, self.host = [], [], [], [], []
        self.h_state, self.h_kc, self.h_vc = [], [], []
        self.conv = synth.conv_width(w)
        self.tail, self.h_tail, self.conv_w, self.h_conv_w = [], [], None, []
        if self.conv > 0:
            C = synth.conv_channels(w)
            self.h_conv_w = [synth.conv_weight(w, seed, l)
                             for l, kind in enumerate(w.layer_kind) if kind == 0]
            self.conv_w = torch.from_numpy(np.stack(self.h_conv_w)).to(device)
            for s in range(ns):
                ht = [synth.conv_tail(w, seed, s, l) for l, kind in enumerate(w.layer_kind)
                      if kind == 0]
                self.h_tail.append(ht)
                t = torch.zeros((w.n_gdn, self.conv - 1, C), dtype=tdt, device=device)
                for gi, a in enumerate(ht):
                    if self.conv > 1:
                        t[gi] = to_device(a, dt, device)
                self.tail.append(t)
        for s in range(ns):
            L, cap = self.lengths[s], self.capacity[s]
            st = torch.empty((w.n_gdn, w.gdn_hv, w.gdn_dv, w.gdn_dk), dtype=torch.float32,
                             device=device)
            hs = []
            gi = 0
            for l, kind in enumerate(w.layer_kind):
                if kind == 0:
                    a = synth.gdn_state(w, seed, s, l)
                    st[gi] = torch.from_numpy(a).to(device)
                    hs.append(a if l in self.host_layers else None)
                    gi += 1
            self.state.append(st)
            self.h_state.append(hs)
            fill = float("nan") if poison else 0.0
            kc = torch.full((w.n_attn, w.attn_hkv, cap, w.attn_d), fill, dtype=tdt, device=device)
            vc = torch.full((w.n_attn, w.attn_hkv, cap, w.attn_d), fill, dtype=tdt, device=device)
            hk, hv = [], []
            ai = 0
            for l, kind in enumerate(w.layer_kind):
                if kind != 1:
                    continue
                keep = l in self.host_layers
                if keep:
                    hK = np.zeros((w.attn_hkv, cap, w.attn_d), np.uint16 if dt == "bf16" else np.float32)
                    hV = np.zeros_like(hK)
                for h in range(w.attn_hkv):
                    K, V = synth.kv_rows(w, seed, s, l, h, 0, L, sharp=sharp, v_scale=kv_v_scale)
                    if L > 0:
                        kc[ai, h, :L] = to_device(K, dt, device)
                        vc[ai, h, :L] = to_device(V, dt, device)
                    if keep:
                        hK[h, :L], hV[h, :L] = K, V
                hk.append(hK if keep else None)
                hv.append(hV if keep else None)
                ai += 1
            self.kc.append(kc)
            self.vc.append(vc)
            self.h_kc.append(hk)
            self.h_vc.append(hv)
            self.io.append([])
            self.host.append([])
            self.set_inputs(s, tag)

    def set_inputs(self, s: int, tag: str = "verify", parent=None):
        """(Re)generate slot s's per-layer tree inputs under `tag` for tree `parent`."""
        torch = _torch()
        w, dt, dev = self.w, self.w.dtype, self.device
        if parent is not None:
            self.trees[s] = list(parent)
        n = len(self.trees[s])
        ios, hosts = [], []
        for l, kind in enumerate(w.layer_kind):
            if kind == 0:
                gen = synth.conv_inputs if self.conv > 0 else synth.gdn_inputs
                q, k, v, a, b = gen(w, self.seed, s, l, n, tag)
                host = dict(q=q, k=k, v=v, alpha=a, beta=b)
                io = {name: to_device(arr, dt, dev) for name, arr in host.items()}
                io["o"] = torch.zeros((n, w.gdn_hv, w.gdn_dv), dtype=_tdtype(dt), device=dev)
            else:
                q, k, v = synth.attn_inputs(w, self.seed, s, l, n, tag, sharp=self.sharp,
                                            q_scale=self.q_scale, v_scale=self.v_scale)
                host = dict(q=q, k=k, v=v)
                io = {name: to_device(arr, dt, dev) for name, arr in host.items()}
                io["o"] = torch.zeros((n, w.attn_hq, w.attn_d), dtype=_tdtype(dt), device=dev)
            ios.append(io)
            hosts.append(host)
        self.io[s] = ios
        self.host[s] = hosts

    def slot_descs(self):
        return [dict(gdn_state=self.state[s], k_cache=self.kc[s], v_cache=self.vc[s],
                     capacity=self.capacity[s], length=self.lengths[s],
                     conv_state=self.tail[s] if self.conv > 1 else None)
                for s in range(len(self.lengths))]

    def engine(self, max_nodes=None):
        import hybrid_deltanet_tree_amd as hdt
        w = self.w
        mn = max_nodes or max(len(t) for t in self.trees)
        return hdt.Engine(w.layer_kind, gdn_hk=w.gdn_hk, gdn_hv=w.gdn_hv, gdn_dk=w.gdn_dk,
                          gdn_dv=w.gdn_dv, attn_hq=w.attn_hq, attn_hkv=w.attn_hkv,
                          attn_d=w.attn_d, io_dtype=hdt.HDT_BF16 if w.dtype == "bf16" else hdt.HDT_F32,
                          max_nodes=mn, slots=self.slot_descs(), gdn_conv=self.conv,
                          gdn_conv_weight=self.conv_w)

    def tree_arg(self, s: int):
        return (s, self.trees[s], self.io[s])

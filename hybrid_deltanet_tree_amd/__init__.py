"""Python binding of libhdt, the tree-verify library for AMD MI355X (gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  The raw C entry points keep their C names (``hdt_create``,
``hdt_forward_tree``, ...); ``Engine`` is a thin wrapper that fills the C
structs from tensors (anything with ``data_ptr()``) and raises ``HdtError`` on
a non-zero status.  Importing this package fails loudly when libhdt.so has not
been built: there is no fallback path.

The verbs follow "Adding a model" (step 4 of "The adapter path in ten steps":
forward_tree, forward_block, commit_tree, rollback_to, kv.length, reset).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# HDT_LIBRARY names another build of the same sources (the sanitizer build of the tests)
LIB_PATH = os.environ.get("HDT_LIBRARY") or os.path.join(_HERE, "libhdt.so")

HDT_MAX_NODES = 64
HDT_MAX_TREES = 8
HDT_F32, HDT_BF16 = 0, 1
STATUS = {0: "HDT_OK", -1: "HDT_E_INVALID", -2: "HDT_E_TREE", -3: "HDT_E_PATH",
          -4: "HDT_E_CAPACITY", -5: "HDT_E_ORDER", -6: "HDT_E_HIP", -7: "HDT_E_UNSUPPORTED"}
KIND_GDN, KIND_ATTN_SPLIT, KIND_ATTN_FOLD, KIND_COMMIT, KIND_CONV, KIND_WALK = 0, 1, 2, 3, 4, 5
KIND_WY_PREP, KIND_WY_SCAN, KIND_PF_ATTN, KIND_PF_FOLD = 6, 7, 8, 9

# PyTorch owns the device memory and the streams, so libhdt must run on the same
# HIP runtime instance.  PyTorch ships its own libamdhip64 under the same soname;
# importing it first makes the loader resolve libhdt's dependency to that copy
# instead of mapping a second runtime (which then fails to open the device).
import torch  # noqa: E402,F401  (load order only)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() (or "
                      "python hybrid_deltanet_tree_amd/build.py) first")

_lib = ctypes.CDLL(LIB_PATH)


class hdt_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("layer_kind", ctypes.POINTER(ctypes.c_uint8)),
                ("gdn_hk", ctypes.c_int32), ("gdn_hv", ctypes.c_int32),
                ("gdn_dk", ctypes.c_int32), ("gdn_dv", ctypes.c_int32),
                ("attn_hq", ctypes.c_int32), ("attn_hkv", ctypes.c_int32),
                ("attn_d", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("gdn_scale", ctypes.c_float), ("attn_scale", ctypes.c_float),
                ("max_nodes", ctypes.c_int32), ("gdn_conv", ctypes.c_int32),
                ("gdn_conv_weight", ctypes.c_void_p)]


class hdt_slot_desc(ctypes.Structure):
    _fields_ = [("gdn_state", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("length", ctypes.c_int64), ("gdn_conv_state", ctypes.c_void_p)]


class hdt_layer_io(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("o", ctypes.c_void_p)]


class hdt_tree(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("n_nodes", ctypes.c_int32),
                ("parent", ctypes.POINTER(ctypes.c_int32)),
                ("io", ctypes.POINTER(hdt_layer_io))]


_E = ctypes.c_void_p
_S = ctypes.c_int
_sigs = {
    "hdt_create": (_S, [ctypes.POINTER(hdt_model_desc), ctypes.c_int32,
                        ctypes.POINTER(hdt_slot_desc), ctypes.POINTER(_E)]),
    "hdt_destroy": (None, [_E]),
    "hdt_forward_tree": (_S, [_E, ctypes.c_int32, ctypes.POINTER(hdt_tree), ctypes.c_void_p]),
    "hdt_forward_tree_noalloc": (_S, [_E, ctypes.c_int32, ctypes.POINTER(hdt_tree), ctypes.c_void_p]),
    "hdt_graph_create": (_S, [_E, ctypes.POINTER(ctypes.c_void_p)]),
    "hdt_graph_forward": (_S, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(hdt_tree), ctypes.c_void_p]),
    "hdt_graph_stats": (_S, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "hdt_graph_destroy": (None, [ctypes.c_void_p]),
    "hdt_forward_block": (_S, [_E, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(hdt_layer_io),
                               ctypes.c_void_p]),
    "hdt_commit_tree": (_S, [_E, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                             ctypes.c_void_p]),
    "hdt_rollback_to": (_S, [_E, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]),
    "hdt_walk_commit": (_S, [_E, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p]),
    "hdt_forward_span": (_S, [_E, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(hdt_layer_io),
                              ctypes.c_void_p]),
    "hdt_forward_chunked": (_S, [_E, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(hdt_layer_io),
                                 ctypes.c_void_p]),
    "hdt_set_anchors": (_S, [_E, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                             ctypes.c_void_p]),
    "hdt_anchor_below": (_S, [_E, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "hdt_kv_length": (_S, [_E, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "hdt_reset": (_S, [_E, ctypes.c_int32, ctypes.c_int64]),
    "hdt_tree_meta": (_S, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "hdt_split_size": (_S, [_E, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "hdt_profile": (_S, [_E, ctypes.c_int32]),
    "hdt_profile_read": (_S, [_E, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_int64)]),
    "hdt_state_bytes": (_S, [_E, ctypes.POINTER(ctypes.c_int64)]),
    "hdt_state_copy": (_S, [_E, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                            ctypes.c_void_p]),
    "hdt_last_error": (ctypes.c_char_p, [_E]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args
    globals()[_name] = _f

EXPORTED = tuple(_sigs)


class Graph:
    """hdt_graph of an Engine (see Engine.graph)."""

    def __init__(self, engine):
        self.engine = engine
        h = ctypes.c_void_p()
        engine._check(hdt_graph_create(engine.h, ctypes.byref(h)))
        self.h = h

    def forward(self, trees, stream=0):
        arr, keep = self.engine._trees(trees)
        self.engine._check(hdt_graph_forward(self.h, len(trees), arr, stream))

    def stats(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        self.engine._check(hdt_graph_stats(self.h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def close(self):
        if getattr(self, "h", None):
            hdt_graph_destroy(self.h)
            self.h = None


class HdtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _i32(values):
    return (ctypes.c_int32 * max(1, len(values)))(*values)


def tree_meta(parent, L: int = 0):
    """Host tree metadata: (depth, mask, anc [n][64], pos) as Python lists."""
    n = len(parent)
    depth = (ctypes.c_int32 * max(1, n))()
    mask = (ctypes.c_uint64 * max(1, n))()
    anc = (ctypes.c_int32 * (max(1, n) * HDT_MAX_NODES))()
    pos = (ctypes.c_int64 * max(1, n))()
    st = hdt_tree_meta(n, _i32(parent), L, ctypes.addressof(depth), ctypes.addressof(mask),
                       ctypes.addressof(anc), ctypes.addressof(pos))
    if st != 0:
        raise HdtError(st, "invalid parent array")
    return (list(depth[:n]), list(mask[:n]),
            [list(anc[i * HDT_MAX_NODES:(i + 1) * HDT_MAX_NODES]) for i in range(n)],
            list(pos[:n]))


class Engine:
    """One engine over caller-owned slots.

    layer_kind: list of 0 (GDN) / 1 (attention).  slots: list of dicts with
    'gdn_state', 'k_cache', 'v_cache' (tensors or device pointers), 'capacity'
    and 'length', and 'conv_state' when gdn_conv > 1.  gdn_conv_weight: the
    [n_gdn][C][gdn_conv] float32 taps when gdn_conv > 0.
    """

    def __init__(self, layer_kind, *, gdn_hk=0, gdn_hv=0, gdn_dk=0, gdn_dv=0, attn_hq=0,
                 attn_hkv=0, attn_d=0, io_dtype=HDT_BF16, gdn_scale=0.0, attn_scale=0.0,
                 max_nodes=16, slots=(), gdn_conv=0, gdn_conv_weight=None):
        self._kinds = (ctypes.c_uint8 * len(layer_kind))(*layer_kind)
        self.layer_kind = list(layer_kind)
        self.desc = hdt_model_desc(len(layer_kind), self._kinds, gdn_hk, gdn_hv, gdn_dk, gdn_dv,
                                   attn_hq, attn_hkv, attn_d, io_dtype, gdn_scale, attn_scale,
                                   max_nodes, gdn_conv, _ptr(gdn_conv_weight))
        arr = (hdt_slot_desc * max(1, len(slots)))()
        for i, s in enumerate(slots):
            arr[i] = hdt_slot_desc(_ptr(s.get("gdn_state")), _ptr(s.get("k_cache")),
                                   _ptr(s.get("v_cache")), int(s["capacity"]), int(s["length"]),
                                   _ptr(s.get("conv_state")))
        self._keep = [slots, gdn_conv_weight]
        h = _E()
        st = hdt_create(ctypes.byref(self.desc), len(slots), arr, ctypes.byref(h))
        if st != 0:
            raise HdtError(st, "hdt_create rejected the descriptor")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            hdt_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def _check(self, st: int):
        if st != 0:
            raise HdtError(st, hdt_last_error(self.h).decode())

    def _io_array(self, layers):
        if len(layers) != len(self.layer_kind):
            raise ValueError(f"{len(layers)} per-layer io entries for a model of "
                             f"{len(self.layer_kind)} layers")
        arr = (hdt_layer_io * len(layers))()
        for l, io in enumerate(layers):
            arr[l] = hdt_layer_io(_ptr(io.get("q")), _ptr(io.get("k")), _ptr(io.get("v")),
                                  _ptr(io.get("alpha")), _ptr(io.get("beta")), _ptr(io.get("o")))
        return arr

    def _trees(self, trees):
        arr = (hdt_tree * len(trees))()
        keep = []
        for i, (slot, parent, layers) in enumerate(trees):
            par = _i32(parent)
            io = self._io_array(layers)
            keep += [par, io]
            arr[i] = hdt_tree(slot, len(parent), par, io)
        return arr, keep

    def forward_tree(self, trees, stream=0):
        """trees: list of (slot, parent list, per-layer list of dicts q/k/v/alpha/beta/o)."""
        arr, keep = self._trees(trees)
        self._check(hdt_forward_tree(self.h, len(trees), arr, stream))

    def forward_tree_noalloc(self, trees, stream=0):
        """forward_tree with the library's static scratch: allocates nothing."""
        arr, keep = self._trees(trees)
        self._check(hdt_forward_tree_noalloc(self.h, len(trees), arr, stream))

    def graph(self):
        """A reusable graph of the verify pass (hdt_graph_create): .forward(trees, stream) is
        forward_tree as one graph launch, .stats() the (instantiations, updates) counts,
        .close() destroys it (before the engine)."""
        return Graph(self)

    def forward_block(self, slot, n, layers, stream=0):
        self._check(hdt_forward_block(self.h, slot, n, self._io_array(layers), stream))

    def commit_tree(self, slot, path, stream=0):
        self._check(hdt_commit_tree(self.h, slot, _i32(path), len(path), stream))

    def rollback_to(self, slot, n, stream=0):
        self._check(hdt_rollback_to(self.h, slot, n, stream))

    def forward_span(self, slot, T, layers, stream=0):
        """Prefill of T tokens: layers as for forward_tree, each array holding T rows."""
        self._check(hdt_forward_span(self.h, slot, T, self._io_array(layers), stream))

    def forward_chunked(self, slot, T, layers, stream=0):
        """The same prefill computed a chunk at a time on the matrix cores (equal to
        forward_span up to rounding)."""
        self._check(hdt_forward_chunked(self.h, slot, T, self._io_array(layers), stream))

    def set_anchors(self, slot, every, n_max=0, state=None, conv=None):
        self._check(hdt_set_anchors(self.h, slot, every, n_max, _ptr(state), _ptr(conv)))

    def anchor_below(self, slot, n) -> int:
        out = ctypes.c_int64()
        self._check(hdt_anchor_below(self.h, slot, n, ctypes.byref(out)))
        return out.value

    def walk_commit(self, slot, draft, target, out, stream=0):
        """Accept walk + commit on the device: draft, target int32 [n], out int32 [2 + n]
        (m, bonus token, path)."""
        self._check(hdt_walk_commit(self.h, slot, _ptr(draft), _ptr(target), _ptr(out), stream))

    def kv_length(self, slot) -> int:
        out = ctypes.c_int64()
        self._check(hdt_kv_length(self.h, slot, ctypes.byref(out)))
        return out.value

    def reset(self, slot, length):
        self._check(hdt_reset(self.h, slot, length))

    def split_size(self, slot, position) -> int:
        """Split size of the row at `position` of `slot` (it sees keys 0..position)."""
        out = ctypes.c_int64()
        self._check(hdt_split_size(self.h, slot, position, ctypes.byref(out)))
        return out.value

    def profile(self, enable: bool):
        self._check(hdt_profile(self.h, 1 if enable else 0))

    def profile_read(self, kind: int):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        self._check(hdt_profile_read(self.h, kind, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def state_bytes(self) -> int:
        """Size of a state snapshot of this engine's shape."""
        out = ctypes.c_int64()
        self._check(hdt_state_bytes(self.h, ctypes.byref(out)))
        return out.value

    def state_copy(self, slot, buf, restore=False, stream=0):
        """Save (restore=False) or restore slot's state sections and length through `buf`
        (a device tensor of at least state_bytes() bytes, 256-byte aligned)."""
        nbytes = buf.numel() * buf.element_size() if hasattr(buf, "numel") else 0
        self._check(hdt_state_copy(self.h, slot, _ptr(buf), nbytes, 1 if restore else 0, stream))

    def last_error(self) -> str:
        return hdt_last_error(self.h).decode()

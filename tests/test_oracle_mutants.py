"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check the pins catch them.

Each mutant is oracle.c with one edit: a dropped term, a wrong sign, a wrong index, a
transposed operand or a wrong head map.  The pins of tests/test_oracle_pins.py run against
the mutant library; at least one must fail, or the pins would not be pinning that part.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "decay_dropped": ("A[a] = alpha * Pc[a];", "A[a] = Pc[a];"),
    "delta_sign": ("const float u = beta * (v[c] - r);", "const float u = beta * (v[c] + r);"),
    "beta_dropped": ("const float u = beta * (v[c] - r);", "const float u = (v[c] - r);"),
    "write_from_parent": ("Sc[a] = A[a] + k[a] * u;", "Sc[a] = Pc[a] + k[a] * u;"),
    "readout_parent_state": ("acc = acc + Sc[a] * (scale * q[a]);",
                             "acc = acc + Pc[a] * (scale * q[a]);"),
    "readout_unscaled": ("acc = acc + Sc[a] * (scale * q[a]);", "acc = acc + Sc[a] * q[a];"),
    "state_transposed": ("for (int a = 0; a < dk; ++a) A[a] = alpha * Pc[a];",
                         "for (int a = 0; a < dk; ++a) A[a] = alpha * P[(size_t)a * dv + c];"),
    "qk_head_map": ("      const int g = h / ratio;\n      for (int a = 0; a < dk; ++a) {",
                    "      const int g = h % hk;\n      for (int a = 0; a < dk; ++a) {"),
    "root_not_from_base": ("const float *P = (parent[i] < 0) ? S_base + (size_t)h * hs",
                           "const float *P = (parent[i] < 0) ? S_base"),
    "ancestor_order_reversed": (
        "kv = ld(kt, dtype, ((int64_t)path[depth - 1 - (t - L)] * hkv + m_head) * D + d);",
        "kv = ld(kt, dtype, ((int64_t)path[t - L] * hkv + m_head) * D + d);"),
    "kv_head_map": ("const int m_head = j / (hq / hkv);", "const int m_head = j % hkv;"),
    "attn_unscaled": ("z[t] = scale * dot;", "z[t] = dot;"),
    "self_not_visible": ("const int64_t nkeys = L + depth;", "const int64_t nkeys = L + depth - 1;"),
    "mask_without_self": ("mask[i] = ((p < 0) ? 0 : mask[p]) | (1ULL << i);",
                          "mask[i] = ((p < 0) ? 0 : mask[p]);"),
    "softmax_unnormalised": ("for (int d = 0; d < D; ++d) o[d] = o[d] / l;",
                             "for (int d = 0; d < D; ++d) o[d] = o[d];"),
    "conv_taps_reversed": ("acc = acc + W[c * w + j] * xin;",
                           "acc = acc + W[c * w + (w - 1 - j)] * xin;"),
    "conv_tail_rows_reversed": ("xin = ld(tail, dtype, (int64_t)((w - 1) - (r - d)) * C + c);",
                                "xin = ld(tail, dtype, (int64_t)((r - d) - 1) * C + c);"),
    "conv_ancestor_off_by_one": ("const int node = up[r];", "const int node = up[r > 0 ? r - 1 : 0];"),
    "conv_silu_sign": ("const float y = acc / (1.0f + expf(-acc));",
                       "const float y = acc / (1.0f + expf(acc));"),
    "conv_no_activation": ("const float y = acc / (1.0f + expf(-acc));",
                           "const float y = acc;"),
    "conv_norm_dropped": ("const float inv = 1.0f / sqrtf(ss + eps);", "const float inv = 1.0f;"),
    "conv_k_channels_shifted": ("xin = ld(k, dtype, (int64_t)node * CQ + (c - CQ));",
                                "xin = ld(q, dtype, (int64_t)node * CQ + (c - CQ));"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(lib), str(path), "-lm"])
    return oracle.configure(ctypes.CDLL(str(lib)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    lib = _build_mutant(tmp_path, name, *MUTANTS[name])
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for pin, fn in pins.PINS.items():
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(pin)
    assert failed, f"no pin catches the mutant {name}"


# The accept walk lives in oracle/__init__.py (plain Python): its mutants are the function's
# source with one edit, executed in the oracle module's namespace.
WALK_MUTANTS = {
    "walk_tie_to_highest_index": ("if agree[i] and depth[i] > depth[best]:",
                                  "if agree[i] and depth[i] >= depth[best]:"),
    "walk_compares_own_target": ("int(draft[i]) == int(target[p])", "int(draft[i]) == int(target[i])"),
    "walk_ignores_parent": ("agree[i] = agree[p] and int(draft[i])", "agree[i] = int(draft[i])"),
    "walk_bonus_is_draft": ("return path[::-1], int(target[best])", "return path[::-1], int(draft[best])"),
    "walk_path_unreversed": ("return path[::-1], int(target[best])", "return path, int(target[best])"),
}


@pytest.mark.parametrize("name", sorted(WALK_MUTANTS))
def test_walk_mutant_is_caught(name, monkeypatch):
    import inspect
    import textwrap
    old, new = WALK_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.greedy_walk))
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "greedy_walk", ns["greedy_walk"])
    failed = []
    for pin in ("walk_hand_examples", "walk_brute_and_greedy_descent"):
        try:
            pins.PINS[pin]()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    assert failed, f"no pin catches the mutant {name}"

"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, for the CPU tests.

Three libraries are rebuilt from their sources with clang's sanitizers on the host side:
the oracle (oracle/oracle.c), the input generator (synth/synth.c) and libhdt (every
source; `-Xarch_host` puts the sanitizers on the host pass only, the gfx950 code objects
are built as usual).  They go to _build/sanitize/ and are rebuilt when a source is newer.
The tests load them through HDT_LIBRARY, HDT_ORACLE_LIBRARY and HDT_SYNTH_LIBRARY in a
child Python that has clang's ASan runtime preloaded (Python itself is not instrumented,
so the runtime must come first).
"""
from __future__ import annotations

import glob
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def runtime() -> str | None:
    """clang's shared ASan runtime (UBSan's handlers are part of it), or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _stale(out: str, sources: list[str]) -> bool:
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    return any(os.path.getmtime(s) > t for s in sources)


def _build(out: str, sources: list[str], cmd: list[str]) -> str:
    if _stale(out, sources):
        tmp = out + ".tmp"
        res = subprocess.run(cmd + ["-o", tmp], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitizer build of {os.path.basename(out)} failed:\n"
                               + res.stdout[-4000:] + res.stderr[-4000:])
        os.replace(tmp, out)
    return out


def build() -> dict:
    """Build (or reuse) the three sanitized libraries; returns the environment that selects them."""
    os.makedirs(OUT, exist_ok=True)
    orc_src = [os.path.join(ROOT, "oracle", "oracle.c")]
    syn_src = [os.path.join(ROOT, "synth", "synth.c")]
    csrc = os.path.join(ROOT, "hybrid_deltanet_tree_amd", "csrc")
    hdt_src = [os.path.join(csrc, n) for n in ("kernels.hip", "kv_attention.hip", "conv.hip", "prefill.hip", "engine.cpp")]
    hdt_dep = hdt_src + glob.glob(os.path.join(csrc, "*.h")) + [os.path.join(ROOT, "include", "hdt.h")]
    orc = _build(os.path.join(OUT, "liboracle.so"), orc_src,
                 [LLVM, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", *SAN,
                  *orc_src, "-lm"])
    syn = _build(os.path.join(OUT, "libsynth.so"), syn_src,
                 [LLVM, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN, *syn_src, "-lm"])
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    hdt = _build(os.path.join(OUT, "libhdt.so"), hdt_dep,
                 [HIPCC, "-O1", "-g", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
                  "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                  "-Wno-unused-command-line-argument", *host_san,
                  "-I", os.path.join(ROOT, "include"), *hdt_src])
    return {"HDT_LIBRARY": hdt, "HDT_ORACLE_LIBRARY": orc, "HDT_SYNTH_LIBRARY": syn}

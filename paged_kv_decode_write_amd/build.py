"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_write_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection
turned off (-Xclang -target-feature -Xclang -packed-fp32-ops), and linked with the C-ABI
host layer into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpagedkv.so")
CHECKED_OUT = os.path.join(HERE, "libpagedkv_checked.so")  # PAGEDKV_CHECKED: device-side checks
PROBE_OUT = os.path.join(HERE, "libpagedkv_probe.so")
PROBE_SOURCES = ["read_probe.hip"]  # measurement utility, a library of its own
# A native C++ caller of the C ABI (eager step, HIP stream capture of several steps, replay),
# built against each library; tests/test_native_abi.py runs it.
NATIVE_SRC = os.path.join(ROOT, "tests", "native", "decode_step_graph.cpp")
NATIVE_OUT = {"libpagedkv.so": os.path.join(HERE, "decode_step_graph"),
              "libpagedkv_checked.so": os.path.join(HERE, "decode_step_graph_checked")}

SOURCES = ["api.cpp", "kv_write.hip", "decode_valu.hip", "decode_mfma.hip", "decode_sk.hip",
           "decode_reduce.hip", "prefill_mfma.hip", "kv_write_rope.hip", "block_table.hip",
           "check.hip"]
ARCH = os.environ.get("PAGEDKV_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (set HIPCC)")


def common_flags(extra=()):
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra]


def compile_one(src: str, obj: str, extra=()) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *common_flags(extra), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"compiling {src} failed")
    noise = "packed-fp32-ops"
    warn = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l and l.strip())
    if warn.strip():
        sys.stderr.write(warn + "\n")


def link(sources, out: str, jobs: int = 8, extra=()) -> str:
    with tempfile.TemporaryDirectory(prefix="pagedkv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in sources]
        with ThreadPoolExecutor(max_workers=min(jobs, len(sources))) as ex:
            list(ex.map(lambda so: compile_one(so[0], so[1], extra), zip(sources, objs)))
        tmp_out = out + ".tmp"
        cmd = [hipcc(), *common_flags(extra), "-shared", *objs, "-o", tmp_out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
            raise RuntimeError(f"linking {os.path.basename(out)} failed")
        os.replace(tmp_out, out)
    return out


def build(out: str = OUT, jobs: int = 8, extra=()) -> str:
    """Build libpagedkv.so (the path) at `out`."""
    return link(SOURCES, out, jobs, extra)


def build_checked(out: str = CHECKED_OUT, jobs: int = 8) -> str:
    """Build libpagedkv_checked.so: the same library with PAGEDKV_CHECKED, which validates
    each call's slot ids, block ids, lengths and query spans on the device first."""
    return link(SOURCES, out, jobs, extra=("-DPAGEDKV_CHECKED",))


def build_probe(out: str = PROBE_OUT) -> str:
    """Build libpagedkv_probe.so (the streaming-read measurement utility)."""
    return link(PROBE_SOURCES, out)


def build_native(lib_name: str = "libpagedkv.so") -> str:
    """Build the native C-ABI test program against `lib_name` (already built next to this
    file); the program finds the library through an $ORIGIN run path."""
    out = NATIVE_OUT[lib_name]
    # -l (not a path) so the program records the bare file name and the run path finds it
    lib_flag = "-l" + lib_name[len("lib"):-len(".so")]
    cmd = [hipcc(), *common_flags(), "-x", "hip", NATIVE_SRC, f"-L{HERE}", lib_flag,
           "-Wl,-rpath,$ORIGIN", "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"building {os.path.basename(out)} failed")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
    print(build_checked())
    print(build_probe())
    for name in NATIVE_OUT:
        print(build_native(name))

"""A native C++ program calls the C ABI directly (tests/native/decode_step_graph.cpp).

It is built next to the library against each build (default and PAGEDKV_CHECKED). On the GPU it
runs the fused decode step eagerly, checks it bit for bit against paged_kv_write followed by
paged_decode_attention_ex and a one-token context against its new value row, then records
eight steps into a HIP graph with the runtime's own stream capture and checks three replays
bit for bit against the eager step (output and both pools). The CPU tests check that the
programs resolve the in-tree libraries and call only functions the header declares.
"""
import os
import re
import subprocess
import sys

import pytest

from paged_kv_decode_write_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv.h")


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"\b(paged_\w+)\s*\(", text))


def test_native_program_calls_only_declared_functions():
    src = open(b.NATIVE_SRC).read()
    called = set(re.findall(r"\b(paged_\w+)\s*\(", src))
    assert {"paged_decode_step", "paged_kv_write", "paged_decode_attention_ex",
            "paged_kv_check_status"} <= called
    assert called <= _declared()


@pytest.mark.parametrize("lib_name", sorted(b.NATIVE_OUT))
def test_native_program_resolves_the_in_tree_library(lib_name):
    exe = b.NATIVE_OUT[lib_name]
    if not os.path.exists(exe) or not os.path.exists(os.path.join(b.HERE, lib_name)):
        pytest.skip("native test program not built")
    out = subprocess.run(["ldd", exe], capture_output=True, text=True, check=True).stdout
    line = next(l for l in out.splitlines() if lib_name in l)
    assert os.path.realpath(line.split("=>")[1].split("(")[0].strip()) == \
        os.path.realpath(os.path.join(b.HERE, lib_name))


@pytest.mark.gpu
@pytest.mark.parametrize("lib_name", sorted(b.NATIVE_OUT))
def test_native_step_and_graph_capture(gpu, lib_name):
    exe = b.NATIVE_OUT[lib_name]
    if not os.path.exists(exe):
        raise FileNotFoundError(f"{exe} is missing: build it first")
    print(f"running {os.path.basename(exe)}", flush=True)
    sys.stdout.flush()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout + res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    assert "native ABI ok" in res.stdout
    want = "checked" if lib_name == "libpagedkv_checked.so" else "default"
    assert f"({want} build" in res.stdout

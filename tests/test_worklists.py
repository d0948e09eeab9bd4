"""The scheduler's work lists cover every tile exactly once (host only, no GPU).

tests/worklist_check.cpp includes libdkv's host source and checks, for seeded random
shapes (prompt groups with empty prompts and groups, ragged and empty responses,
windows, GQA ratios, head dims 64 / 128 / 512, atomic and split modes): every
(kv head, sequence, query tile) of the forward and dQ lists exactly once; every own
key tile exactly once; every (prompt key tile, sequence whose rows see it) exactly once
in atomic mode and every (prompt key tile, slice) exactly once in split mode; every
own key tile split into row chunks (a call that accumulates them) covered chunk by chunk
on the chunk grid, within the workspace plan's bound; every layout output row exactly
once, all source rows in bounds; and, run on the host, the kernels' own walks
(dkv_walks.h): every query item's key tiles (64 and 32 keys) cover the keys its rows
see and none wholly outside them, and the dK/dV row walk (with and without the
windowed rotation) over every key item visits exactly the rows the scheduler counts as
visible, once each, in whole aligned steps.  It is built with hipcc
(host code only) and linked against the built libdkv.so for the launch symbols.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "shared_prompt_exact_dkv_amd"))


def test_worklists_cover_every_tile_once(tmp_path):
    import build as B   # the package's build script: hipcc path
    lib = os.path.join(ROOT, "shared_prompt_exact_dkv_amd")
    if not os.path.exists(os.path.join(lib, "libdkv.so")):
        pytest.fail("libdkv.so is not built; run __graft_entry__.build()")
    exe = str(tmp_path / "worklist_check")
    cmd = [B.HIPCC, "-std=c++17", "-O1", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "worklist_check.cpp"), "-L" + lib, "-ldkv",
           "-Wl,-rpath," + lib, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

"""The C ABI as a C program sees it: tests/abi_consumer.c includes include/dkv.h, links
libdkv.so and the HIP runtime (no Python, no torch), runs one DualKV step (Call 1 and
Call 2, forward and backward, the prompt keys' gradient accumulated in fp32 by both calls
and cast once; §2.2, §3.2) and checks every output against the C oracle.

On the CPU the program is compiled with gcc as C11 under -Wall -Werror and linked, which
checks that the header is plain C and that every entry point it calls is exported.  On
the GPU it runs, as a child process, for global and windowed causal masks, bf16 and
fp32, with the contiguous and a permuted GQA head map."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "shared_prompt_exact_dkv_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(out_dir):
    import oracle
    oracle.build(force=False)   # oracle/liboracle.so, compiled only when missing
    for lib in (os.path.join(PKG, "libdkv.so"), os.path.join(ORACLE, "liboracle.so")):
        if not os.path.exists(lib):
            pytest.fail("%s is not built (run __graft_entry__.build())" % lib)
    exe = os.path.join(str(out_dir), "abi_consumer")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "abi_consumer.c"), "-L" + PKG, "-ldkv",
           "-L" + ORACLE, "-loracle", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + ":".join((PKG, ORACLE, os.path.join(ROCM, "lib"))), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, "gcc failed:\n" + r.stdout + r.stderr
    return exe


def test_c_consumer_compiles_and_links(tmp_path):
    exe = _compile(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr   # no arguments: usage, nothing run


@pytest.mark.gpu
@pytest.mark.parametrize("window_left,dtype,headmap", [
    (-1, 0, 0),    # bf16, global causal, contiguous heads
    (40, 0, 1),    # bf16, window 40, permuted head map
    (-1, 1, 1),    # fp32, global causal, permuted head map
    (20, 1, 0),    # fp32, window 20
])
def test_c_consumer_step_matches_oracle(tmp_path, window_left, dtype, headmap):
    exe = _compile(tmp_path)
    print("abi_consumer window_left=%d dtype=%d headmap=%d" % (window_left, dtype, headmap),
          flush=True)
    r = subprocess.run([exe, str(window_left), str(dtype), str(headmap)], capture_output=True,
                       text=True, timeout=300)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, "abi_consumer exited %d" % r.returncode
    assert "all tensors within bound" in r.stdout

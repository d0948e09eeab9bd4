"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/dkv_oracle.c (a dropped term, a
wrong sign, an off-by-one window edge, a wrong operand, a missing factor), builds
it on the CPU, and checks that the independent pins (torch float64 SDPA with
autograd, and finite differences) reject it.  The shipped oracle is untouched.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "dkv_oracle.c")

MUTATIONS = {
    "drop_softmax_jacobian_term": ("double ds = p[i] * (dp[i] - D);", "double ds = p[i] * dp[i];"),
    "wrong_sign_delta": ("double ds = p * (dot(dot_, vj, d) - delta",
                         "double ds = p * (dot(dot_, vj, d) + delta"),
    "window_off_by_one": ("lo = t - window_left;", "lo = t - window_left + 1;"),
    "dv_wrong_operand": ("dvj[c] += p * dot_[c];", "dvj[c] += p * qt[c];"),
    "dk_missing_scale": ("dkj[c] += scale * ds * qt[c];\n                        dvj[c] += p * dot_[c];",
                         "dkj[c] += ds * qt[c];\n                        dvj[c] += p * dot_[c];"),
    # the selected-row forms used at full workload sizes
    "scatter_drop_delta": ("const double ds = s[i] * (dp[i] - delta);\n                double *dkj",
                           "const double ds = s[i] * dp[i];\n                double *dkj"),
    "scatter_dv_wrong_weight": ("dvj[c] += s[i] * dot_[c];", "dvj[c] += dot_[c];"),
    "fwd_sel_missing_norm": ("const double w = exp(p[i] - m) / l;", "const double w = exp(p[i] - m);"),
    "lse_missing_max": ("return m + log(l);", "return log(l);"),
    "gqa_wrong_head": ("int g = kvh[h];\n    double m", "int g = kvh[h] * 0;\n    double m"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / (name + ".c")
    mutated.write_text(src.replace(old, new))
    so = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                           str(mutated), "-lm"])
    return str(so)


def _pins_pass():
    """The library-routine pin of tests/test_oracle.py on one windowed GQA case."""
    from tests.test_oracle import _sdpa_ref, _rand
    S, Hq, Hkv, d, wl = 11, 4, 2, 6, 4
    q, k, v, do = _rand((S, Hq, d), 1), _rand((S, Hkv, d), 2), _rand((S, Hkv, d), 3), \
        _rand((S, Hq, d), 4)
    kvh = [h // 2 for h in range(Hq)]
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    o_ref, lse_ref = _sdpa_ref(qt, kt, vt, 1.0 / math.sqrt(d), wl, kvh)
    (o_ref * do).sum().backward()
    o, lse = oracle.seq_fwd(q, k, v, window_left=wl)
    g = oracle.seq_bwd(q, k, v, do, window_left=wl)
    ok = np.allclose(o, o_ref.detach().numpy(), atol=1e-10, rtol=0)
    ok &= np.allclose(lse, lse_ref.detach().numpy(), atol=1e-10, rtol=0)
    for a, b in ((g["dq"], qt.grad), (g["dk"], kt.grad), (g["dv"], vt.grad)):
        ok &= np.allclose(a, b.numpy(), atol=1e-9, rtol=0)
    # selected-row forms: every row selected, so they must reproduce the same values
    rows = list(range(S))
    o2, lse2 = oracle.rows_fwd(k, v, rows, q, window_left=wl)
    ok &= np.allclose(o2, o_ref.detach().numpy(), atol=1e-10, rtol=0)
    dk2, dv2 = np.zeros((S, Hkv, d)), np.zeros((S, Hkv, d))
    dq2 = oracle.rows_bwd_scatter(k, v, rows, q, do, dk2, dv2, window_left=wl)
    for a, b in ((dq2, qt.grad), (dk2, kt.grad), (dv2, vt.grad)):
        ok &= np.allclose(a, b.numpy(), atol=1e-9, rtol=0)
    return bool(ok)


@pytest.fixture(autouse=True)
def _float64_default():
    """The pins build tensors in float64; the default is restored after each test."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def test_unmutated_oracle_passes_pins():
    oracle.use_library(None)
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(tmp_path, name):
    old, new = MUTATIONS[name]
    so = _build(tmp_path, name, old, new)
    try:
        oracle.use_library(so)
        assert not _pins_pass(), "pins failed to catch mutation " + name
    finally:
        oracle.use_library(None)

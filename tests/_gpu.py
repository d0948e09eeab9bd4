"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run the
library's calls, and compare against the oracle with the stated tolerances.

Tolerances: fp32 inputs -> max|err| <= 1e-5; bf16 inputs -> max|err| <= 2e-2 *
max|ref| per tensor; fp16 inputs -> 5e-3 * max|ref| + 2^-24, one fp16 subnormal spacing
(1e-4 absolute where the reference tensor is exactly zero).  The oracle sees exactly the values the GPU sees (16-bit inputs
are drawn in fp32, rounded to the 16-bit type, and the same rounded values feed both
sides).
"""
import numpy as np
import torch

import shared_prompt_exact_dkv_amd as dkv

DEV = "cuda:0"


def tdt(dtype: str):
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dtype]


def to_dev(x: dict, dtype: str) -> dict:
    out = {}
    for k, v in x.items():
        if k == "cu":
            out["cu"] = v.to(DEV)
            out["cu_host"] = [int(c) for c in v]
        elif isinstance(v, torch.Tensor) and v.is_floating_point():
            out[k] = v.to(tdt(dtype)).to(DEV).contiguous()
    return out


def tol(dtype: str, ref: np.ndarray) -> float:
    if dtype == "fp32":
        return 1e-5
    m = float(np.abs(ref).max()) if ref.size else 0.0
    # fp16 rounds P, dS and the outputs with a unit 8 times finer than bf16's (11 vs 8
    # significand bits); its bound is a quarter of bf16's, twice the ratio as headroom,
    # plus one fp16 spacing below 2^-14 (2^-24): there fp16 is subnormal, and storing a
    # result of that size alone costs up to half of it.
    if dtype == "bf16":
        rel, floor = 2e-2, 0.0
    else:
        rel, floor = 5e-3, 2.0 ** -24
    # A reference that is exactly zero (e.g. dQ under a zero-width window) leaves a
    # relative bound of zero; fp32 accumulation noise is then held to 1e-4 absolute.
    return rel * m + floor if m > 0 else 1e-4


def check(name: str, got, ref: np.ndarray, dtype: str, bound=None):
    g = got.detach().float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.isfinite(g).all(), name + ": non-finite values"
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    b = tol(dtype, ref) if bound is None else bound
    assert err <= b, "%s: max|err| = %.3e > %.3e" % (name, err, b)
    return err


def dualkv_forward(d: dict, window_left=-1, scale=0.0):
    """Call 1 over the prompt then Call 2 over the responses."""
    P = d["q_p"].shape[0]
    cu_p = torch.tensor([0, P], dtype=torch.int32, device=DEV)
    o_p, lse_p = dkv.dkv_ctx_fwd(d["q_p"], d["k_p"], d["v_p"], cu_p, cu_host=[0, P],
                                 window_left=window_left, softmax_scale=scale)
    o_r, lse_r = dkv.dkv_fwd(d["q_r"], d["k_p"], d["v_p"], d["k_r"], d["v_r"], d["cu"],
                             cu_host=d["cu_host"], window_left=window_left,
                             softmax_scale=scale)
    return o_p, lse_p, o_r, lse_r

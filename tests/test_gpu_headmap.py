"""GPU parity with an explicit grouped-query head map, and the standalone single cast.

Head map (dkv_params::kv_head_of_q): q-head h reads kv head map[h], every kv head named
by Hq / Hkv q-heads (GQA, the paper's §3.1 and §4.1).  The oracle takes the same map
(its kvh argument), so every output and gradient is compared element by element; a
permuted map must differ from the contiguous one, so a kernel that ignored the map
would fail.  The cast (§3.2 Stage 2: the fp32 accumulator cast once) is compared bit
for bit with the host's round-to-nearest-even conversion.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import DEV, check, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")


def _perm_map(Hq, Hkv, seed):
    """A seeded map that gives every kv head Hq / Hkv q-heads, in shuffled order."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    m = np.repeat(np.arange(Hkv), G)
    while True:
        rng.shuffle(m)
        if Hkv == 1 or any(int(m[h]) != h // G for h in range(Hq)):
            return [int(v) for v in m]


CASES = [
    # P, lens, Hq, Hkv, d, window_left, dtype, split
    (70, [40, 95], 8, 2, 64, -1, "fp32", False),
    (90, [60, 33], 6, 2, 128, 50, "fp32", False),
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16", False),
    (61, [70, 131, 5], 6, 2, 128, -1, "bf16", True),
    (45, [90, 17], 10, 2, 64, 30, "fp16", False),
    (100, [40, 70], 12, 4, 64, -1, "bf16", False),
    (37, [40, 3], 128, 2, 64, -1, "bf16", False),      # 64 q-heads per kv head
    (20, [33], 192, 2, 128, 15, "bf16", False),          # 96: members past lane 63
    (70, [45, 100], 8, 2, 512, -1, "bf16", False),
    (37, [61, 130], 6, 2, 512, 50, "bf16", True),
    (40, [70, 9], 16, 4, 512, -1, "fp16", False),
]


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,dtype,split", CASES)
def test_permuted_head_map_matches_oracle(P, lens, Hq, Hkv, d, wl, dtype, split):
    seed = 3 * P + Hq + d
    kvh = _perm_map(Hq, Hkv, seed)
    print("[headmap] P=%d lens=%s Hq=%d Hkv=%d d=%d wl=%d %s map=%s"
          % (P, lens, Hq, Hkv, d, wl, dtype, kvh), flush=True)
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, dtype, seed=seed)
    N = len(lens)
    do_copies = workloads.split_prompt_grad(x["do_p"], N, seed=seed)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, window_left=wl, kvh=kvh)
    t = to_dev(x, dtype)
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], t["cu"],
                                                cu_host=t["cu_host"], window_left=wl,
                                                kv_head_of_q=kvh)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl, split=split,
                            kv_head_of_q=kvh)
    torch.cuda.synchronize()
    check("o_p", o_p, ref["o_p"], dtype)
    check("o_r", o_r, ref["o_r"], dtype)
    lb = 1e-5 if dtype == "fp32" else 2e-3
    check("lse_p", lse_p.t(), ref["lse_p"], dtype, bound=lb)
    check("lse_r", lse_r.t(), ref["lse_r"], dtype, bound=lb)
    for k in GRADS:
        check(k, g[k], ref[k], dtype)
    # the map matters: the contiguous map's reference differs from this one
    ref0 = oracle.ncopy_reference(x, window_left=wl, backward=False)
    assert np.abs(ref0["o_r"] - ref["o_r"]).max() > 10 * (2e-2 * np.abs(ref["o_r"]).max())


def test_contiguous_map_given_explicitly_is_bitwise_the_default():
    P, lens, Hq, Hkv, d = 96, [50, 70], 8, 2, 128
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=9)
    t = to_dev(x, "bf16")
    kvh = [h // (Hq // Hkv) for h in range(Hq)]
    outs = []
    for m in (None, kvh):
        f = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                               t["cu"], cu_host=t["cu_host"], kv_head_of_q=m)
        g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                *f, t["do_p"], t["do_r"], t["cu"], cu_host=t["cu_host"],
                                split=True, kv_head_of_q=m)
        outs.append(list(f) + [g[k] for k in GRADS])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_standalone_cast_is_round_to_nearest_even(dtype):
    # fp32 values over many binades, with exact ties of the 16-bit types' rounding
    # (halfway between two representable values), subnormals of the target type and
    # signed zeros: the device cast must equal the host's nearest-even conversion.
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    g = torch.Generator().manual_seed(31)
    rows, Hkv, d = 77, 3, 64
    n = rows * Hkv * d
    mant = torch.randint(0, 1 << 23, (n,), generator=g, dtype=torch.int64)
    expo = torch.randint(90, 150, (n,), generator=g, dtype=torch.int64)
    sign = torch.randint(0, 2, (n,), generator=g, dtype=torch.int64)
    bits = (sign << 31) | (expo << 23) | mant
    # every fourth value an exact tie: the bits below the target mantissa are 100...0
    keep = 7 if dtype == "bf16" else 10
    tie = (bits >> (23 - keep) << (23 - keep)) | (1 << (22 - keep))
    bits = torch.where(torch.arange(n) % 4 == 0, tie, bits)
    acc = bits.to(torch.int32).view(torch.float32).view(rows, Hkv, d).clone()
    acc[0, 0, :4] = torch.tensor([0.0, -0.0, 1e-7, -3e-8])
    acc_dv = -acc.flip(0).contiguous()
    want_k, want_v = acc.to(tdt), acc_dv.to(tdt)
    dk = torch.empty(rows, Hkv, d, dtype=tdt, device=DEV)
    dv = torch.empty_like(dk)
    dkv.dkv_cast_acc(acc.to(DEV), acc_dv.to(DEV), dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(dk.cpu().view(torch.int16 if dtype != "fp32" else torch.int32),
                       want_k.view(torch.int16 if dtype != "fp32" else torch.int32))
    assert torch.equal(dv.cpu().view(torch.int16 if dtype != "fp32" else torch.int32),
                       want_v.view(torch.int16 if dtype != "fp32" else torch.int32))

"""GPU parity in fp16, the precision of the paper's kernel benchmark (§4.1, Table 1):
the same 16-bit MFMA kernels as bf16, with the fp16 MFMA and fp16 rounding of P, dS
and the outputs.  Forward and backward of both calls against the oracle on the same
fp16-rounded inputs, max|err| <= 5e-3 * max|ref| + 2^-24 per tensor (LSE 1e-3 absolute)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import check, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")

CASES = [
    # P, lens, Hq, Hkv, d, window_left, scaled
    (130, [77, 64, 129], 8, 2, 128, -1, True),
    (130, [77, 64, 129], 8, 2, 128, -1, False),
    (191, [45, 150, 7], 16, 2, 64, 40, False),
    (0, [50, 90], 4, 4, 64, -1, False),
    (61, [70, 131, 5], 6, 2, 128, 30, False),
    (70, [45, 100], 8, 2, 512, -1, False),
    (129, [33, 64, 1], 4, 1, 512, 40, False),
    (37, [61, 130], 6, 2, 512, 50, True),
]


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,scaled", CASES)
@pytest.mark.parametrize("split", [False, True])
def test_fp16_matches_oracle(P, lens, Hq, Hkv, d, wl, scaled, split):
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "fp16", seed=50 + P, scaled=scaled)
    do_copies = workloads.split_prompt_grad(x["do_p"], len(lens), seed=50 + P)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, window_left=wl)
    t = to_dev(x, "fp16")
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                                t["v_r"], t["cu"], cu_host=t["cu_host"],
                                                window_left=wl)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl, split=split)
    torch.cuda.synchronize()
    assert o_r.dtype == torch.float16 and g["dk_p"].dtype == torch.float16
    check("o_p", o_p, ref["o_p"], "fp16")
    check("o_r", o_r, ref["o_r"], "fp16")
    check("lse_p", lse_p.t(), ref["lse_p"], "fp16", bound=1e-3)
    check("lse_r", lse_r.t(), ref["lse_r"], "fp16", bound=1e-3)
    for k in GRADS:
        if g[k] is None:
            assert ref[k].size == 0, k
            continue
        check(k, g[k], ref[k], "fp16")


def test_fp16_prompt_groups():
    groups = [(64, [32, 20]), (100, [50]), (0, [40, 7])]
    xs, pk = workloads.make_group_inputs(groups, 8, 2, 128, "fp16", seed=9)
    ref = oracle.grouped_reference(xs)
    t = to_dev(pk, "fp16")
    kw = dict(cu_host=t["cu_host"], ctx_cu_host=[int(c) for c in pk["ctx_cu"]],
              group_seq_cu_host=[int(c) for c in pk["seq_cu"]])
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                                t["v_r"], t["cu"], **kw)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"], **kw)
    torch.cuda.synchronize()
    check("o_r", o_r, ref["o_r"], "fp16")
    for k in GRADS:
        check(k, g[k], ref[k], "fp16")


@pytest.mark.parametrize("op", [dkv.DKV_UNPACK, dkv.DKV_UNPACK_BWD, dkv.DKV_FIRST_TOKEN_SCATTER])
def test_fp16_layout(op):
    groups = [(37, [20, 0, 65]), (5, [3])]
    cu, ccu, scu = [0, 20, 20, 85, 88], [0, 37, 42], [0, 3, 4]
    rows_in, rows_out = dkv.layout_rows(op, cu, 42, ccu, scu)
    x = torch.randn((rows_in, 64), generator=torch.Generator().manual_seed(op)).to(torch.float16)
    out = dkv.dkv_layout(op, x.to("cuda:0"), cu, 42, ctx_cu_host=ccu, group_seq_cu_host=scu)
    torch.cuda.synchronize()
    fn = {dkv.DKV_UNPACK: oracle.layout_unpack, dkv.DKV_UNPACK_BWD: oracle.layout_unpack_bwd,
          dkv.DKV_FIRST_TOKEN_SCATTER: oracle.first_token_scatter}[op]
    ref = fn(x.float().numpy().astype(np.float64), groups)
    got = out.float().cpu().numpy().astype(np.float64)
    # one fp16 rounding of an fp32 sum (copies exactly)
    assert (np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-30).all()

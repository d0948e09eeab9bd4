"""dkv_bwd_noalloc (the backward without a workspace, for callers that cannot allocate)
against dkv_bwd on the same inputs, through the C ABI: two calls in a row, the second
with a smaller input, so the second runs over the scratch the first left behind.

Both entry points run the same kernels; dQ_R, dK_R, dV_R have one writer per element
and must agree bit for bit, and so must dK_P, dV_P in split mode.  With atomic adds the
shared-prompt gradient is summed in a scheduling-dependent order, so there it is held
to the bf16 bound (2e-2 * max|ref|) against dkv_bwd's result and against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import DEV, check, to_dev

pytestmark = pytest.mark.gpu


def _both(P, lens, Hq, Hkv, d, wl, split, seed):
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=seed)
    t = to_dev(x, "bf16")
    f = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], t["cu"],
                           cu_host=t["cu_host"], window_left=wl)
    o_p, lse_p, o_r, lse_r = f
    cu_p = torch.tensor([0, P], dtype=torch.int32, device=DEV)
    flags = dkv.DKV_ACC_FINALIZE | (dkv.DKV_ACC_SPLIT if split else 0)
    out = {}
    for name, fn in (("ws", dkv.dkv_bwd), ("noalloc", dkv.dkv_bwd_noalloc)):
        acc = torch.empty((2, P, Hkv, d), dtype=torch.float32, device=DEV)
        dkv.dkv_ctx_bwd(t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], cu_p,
                        cu_host=[0, P], window_left=wl, acc_dk=acc[0], acc_dv=acc[1],
                        acc_flags=dkv.DKV_ACC_ZERO)
        g = fn(t["q_r"], t["k_p"], t["v_p"], t["k_r"], t["v_r"], o_r, lse_r, t["do_r"], t["cu"],
               acc_dk_p=acc[0], acc_dv_p=acc[1], acc_flags=flags, cu_host=t["cu_host"],
               window_left=wl)
        out[name] = dict(zip(("dq_r", "dk_r", "dv_r", "dk_p", "dv_p"), g))
    torch.cuda.synchronize()
    return x, out


@pytest.mark.parametrize("split", [False, True])
def test_noalloc_matches_workspace_entry_on_two_calls(split):
    cases = [(300, [400, 250, 90], 8, 2, 128, -1), (64, [50, 20], 4, 2, 64, 30)]
    for P, lens, Hq, Hkv, d, wl in cases:
        print("[noalloc] split=%s P=%d lens=%s Hq=%d Hkv=%d d=%d wl=%d"
              % (split, P, lens, Hq, Hkv, d, wl), flush=True)
        seed = P + len(lens)
        x, out = _both(P, lens, Hq, Hkv, d, wl, split, seed)
        a, b = out["ws"], out["noalloc"]
        exact = ("dq_r", "dk_r", "dv_r") + (("dk_p", "dv_p") if split else ())
        for k in exact:
            assert torch.equal(a[k], b[k]), k
        ref = oracle.ncopy_reference(x, window_left=wl)
        for k in ("dk_p", "dv_p"):
            check(k + " vs dkv_bwd", b[k], a[k].float().cpu().numpy().astype(np.float64), "bf16")
            check(k + " vs oracle", b[k], ref[k], "bf16")
        for k in ("dq_r", "dk_r", "dv_r"):
            check(k + " vs oracle", b[k], ref[k], "bf16")

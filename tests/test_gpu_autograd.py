"""torch autograd over the two calls (`dualkv_attention`, `DualKVAttention`): for a
loss over (o_p, o_r) autograd returns exactly what `dualkv_backward` gives when fed that
loss's upstream gradients (split mode, so the shared prompt's K/V gradient is bitwise
reproducible), and those match the oracle's N-copy gradients (eq. (6): the prompt keys'
gradient summed over Call 1 and every response).  A loss that uses only o_r gives the
prompt rows a zero upstream gradient."""
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import check, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r")
GRADS = ("dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")

CASES = [
    # P, lens, Hq, Hkv, d, window_left
    (100, [70, 0, 131], 8, 2, 128, -1),
    (61, [70, 5], 6, 2, 64, 30),
    (90, [77, 40], 8, 2, 512, 50),
    (150, [160, 90], 6, 2, 256, -1),
]


def _autograd(t, wl, use_prompt_output=True):
    leaves = {k: t[k].clone().requires_grad_(True) for k in NAMES}
    o_p, o_r = dkv.dualkv_attention(*[leaves[k] for k in NAMES], t["cu"], cu_host=t["cu_host"],
                                    window_left=wl, split=True)
    # d loss / d o = the seeded upstream gradients exactly (bf16 values times fp32 ones)
    loss = (o_r.float() * t["do_r"].float()).sum()
    if use_prompt_output:
        loss = loss + (o_p.float() * t["do_p"].float()).sum()
    loss.backward()
    return o_p.detach(), o_r.detach(), {g: leaves[k].grad for g, k in zip(GRADS, NAMES)}


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl", CASES)
def test_autograd_equals_explicit_calls_and_oracle(P, lens, Hq, Hkv, d, wl):
    print("autograd case P=%d lens=%s Hq=%d Hkv=%d d=%d wl=%d" % (P, lens, Hq, Hkv, d, wl),
          flush=True)
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=950 + d, dout=True)
    t = to_dev(x, "bf16")
    o_p, o_r, ga = _autograd(t, wl)
    fo = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl)
    ge = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], *fo,
                             t["do_p"], t["do_r"], t["cu"], cu_host=t["cu_host"], window_left=wl,
                             split=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, fo[0]) and torch.equal(o_r, fo[2])
    for k in GRADS:
        assert torch.equal(ga[k], ge[k]), k
    do_copies = workloads.split_prompt_grad(x["do_p"], len(lens), seed=7)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, window_left=wl)
    for k in GRADS:
        check(k, ga[k], ref[k], "bf16")


def test_autograd_with_unused_prompt_output():
    P, lens, Hq, Hkv, d, wl = 100, [70, 0, 131], 8, 2, 128, -1
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=977, dout=True)
    t = to_dev(x, "bf16")
    _, _, ga = _autograd(t, wl, use_prompt_output=False)
    fo = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl)
    ge = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], *fo,
                             torch.zeros_like(t["do_p"]), t["do_r"], t["cu"],
                             cu_host=t["cu_host"], window_left=wl, split=True)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(ga[k], ge[k]), k

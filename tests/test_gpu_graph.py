"""HIP graph capture of the whole DualKV step through the C ABI: Call 1 and Call 2,
forward and backward, with the shared prompt gradient accumulated across both calls and
cast once (§2.2 two-call decomposition, §3.2).  Every replay must give what the eager
calls give on the same inputs; between replays the inputs change in place and eager
calls of another shape run, so the captured work lists must not depend on staging
buffers that later calls reuse."""
import numpy as np
import pytest
import torch

import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import DEV, check, to_dev

pytestmark = pytest.mark.gpu

INPUTS = ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r")

CASES = [
    # P, lens, Hq, Hkv, d, window_left, split
    (100, [70, 0, 131], 8, 2, 128, -1, True),
    (100, [70, 0, 131], 8, 2, 128, -1, False),
    (90, [77, 40], 8, 2, 512, -1, True),
    (150, [160, 90], 6, 2, 256, 60, True),
    (61, [70, 5], 6, 2, 64, 30, True),
    (1500, [40, 70], 8, 2, 128, -1, False),   # Call 1 with row chunks in the graph
]


def _step(t, wl, split, **kw):
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], t["cu"],
                                                cu_host=t["cu_host"], window_left=wl, **kw)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl, split=split, **kw)
    return dict(o_p=o_p, lse_p=lse_p, o_r=o_r, lse_r=lse_r, **g)


def _other_shape_work(d, seed):
    # Eager calls of another shape: their work lists go through the staging pool that
    # the captured calls' lists would occupy if they were not reserved for the graph.
    x = workloads.make_inputs(37, [150, 3, 64], 4, 2, d, "bf16", seed=seed, dout=True)
    u = to_dev(x, "bf16")
    _step(u, -1, False)


def _capture_and_replay(t, step, new_inputs, d, split):
    """Capture step(t) into a graph; then three times: load new inputs into t, run eager
    calls of another shape, run step(t) eagerly, replay the graph, and compare."""
    step(t)                        # eager first: the library and its kernels are loaded
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        out = step(t)
    torch.cuda.synchronize()
    for r in range(3):
        x = new_inputs(r)
        for k in INPUTS:
            t[k].copy_(x[k].to(torch.bfloat16).to(DEV))
        _other_shape_work(d, seed=700 + r)
        ref = step(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            if split or k not in ("dk_p", "dv_p"):
                assert torch.equal(out[k], v), "replay %d: %s differs from the eager call" % (r, k)
            else:
                # fp32 atomics add the responses' prompt terms in another order
                check("replay %d: %s" % (r, k), out[k],
                      v.float().cpu().numpy().astype(np.float64), "bf16")
    del graph
    torch.cuda.synchronize()


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,split", CASES)
def test_graph_replays_match_eager_calls(P, lens, Hq, Hkv, d, wl, split):
    print("graph case P=%d lens=%s Hq=%d Hkv=%d d=%d wl=%d split=%s" %
          (P, lens, Hq, Hkv, d, wl, split), flush=True)
    t = to_dev(workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=500 + d, dout=True),
               "bf16")
    _capture_and_replay(
        t, lambda u: _step(u, wl, split),
        lambda r: workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=600 + 10 * d + r,
                                        dout=True), d, split)


def test_graph_with_prompt_groups_and_head_map():
    # Several prompts in the micro-batch (each shared by its own responses, one of them
    # empty, one group without responses) and a shuffled GQA head map: the group and
    # head tables travel in the captured copy with the work lists.
    groups = [(64, [32, 20]), (100, [50]), (0, [40, 7]), (30, [])]
    Hq, Hkv, d, wl = 8, 2, 128, 50
    kvh = [1, 0, 1, 0, 0, 1, 1, 0]
    print("graph case: prompt groups %s, head map %s, window %d" % (groups, kvh, wl), flush=True)
    pk = workloads.make_group_inputs(groups, Hq, Hkv, d, "bf16", seed=801)[1]
    t = to_dev(pk, "bf16")
    kw = dict(ctx_cu_host=[int(c) for c in pk["ctx_cu"]],
              group_seq_cu_host=[int(c) for c in pk["seq_cu"]], kv_head_of_q=kvh)
    _capture_and_replay(
        t, lambda u: _step(u, wl, True, **kw),
        lambda r: workloads.make_group_inputs(groups, Hq, Hkv, d, "bf16", seed=810 + r)[1],
        d, True)


def test_noalloc_refuses_a_capturing_stream():
    # dkv_bwd_noalloc copies its work lists from pageable host memory, which a graph
    # cannot capture: on a capturing stream it returns DKV_ERR_UNSUPPORTED and enqueues
    # nothing.  The same call outside capture runs.
    P, lens, Hq, Hkv, d = 40, [30, 20], 4, 2, 64
    t = to_dev(workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=3, dout=True), "bf16")
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], t["cu"],
                                                cu_host=t["cu_host"])
    acc = torch.zeros((2, P, Hkv, d), dtype=torch.float32, device=DEV)

    def call():
        return dkv.dkv_bwd_noalloc(t["q_r"], t["k_p"], t["v_p"], t["k_r"], t["v_r"], o_r,
                                   lse_r, t["do_r"], t["cu"], acc_dk_p=acc[0],
                                   acc_dv_p=acc[1], cu_host=t["cu_host"])

    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.stream(s):
        graph.capture_begin()
        try:
            call()
        except dkv.DkvError as e:
            err = e
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    assert err is not None and err.status == 2 and "capturing" in str(err)
    call()
    torch.cuda.synchronize()

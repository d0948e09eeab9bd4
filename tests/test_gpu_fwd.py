"""GPU parity of the forward (Call 1 + Call 2, and the N-copy packing through the
same causal kernel) against the CPU oracle of eq. (2)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import DEV, check, dualkv_forward, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # P, lens, Hq, Hkv, d, window_left, dtype, scaled
    (64, [32, 32, 32, 32], 2, 2, 64, -1, "fp32", False),        # the tiny workload
    (100, [37, 0, 1, 130], 4, 1, 64, -1, "fp32", False),
    (70, [65, 3], 8, 2, 128, -1, "fp32", False),
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16", True),
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16", False),
    (0, [50, 90], 4, 4, 64, -1, "bf16", False),
    (33, [200], 32, 8, 128, -1, "bf16", False),
    (191, [45, 150, 7], 16, 2, 64, 40, "bf16", False),
    (97, [120, 33], 4, 2, 128, 0, "bf16", False),
    (150, [100, 60], 8, 1, 128, 127, "fp32", False),
    (5, [3, 2, 1], 1, 1, 64, -1, "bf16", False),
    # query heads per kv head that do not divide the 32-row steps / 128-row tiles
    (61, [70, 131, 5], 6, 2, 128, -1, "bf16", False),
    (45, [90, 17], 10, 2, 64, 30, "bf16", False),
    # head dim 512 (the hybrid-layer workload's GQA 4:1 included)
    (70, [45, 100], 8, 2, 512, -1, "bf16", False),
    (40, [70, 9], 16, 4, 512, -1, "bf16", True),
    (129, [33, 64, 1], 4, 1, 512, 40, "bf16", False),
    (100, [150, 20], 16, 4, 512, 63, "bf16", False),
    (0, [80], 4, 4, 512, -1, "bf16", False),
    # head dim 512 with 3 and 2 query heads per kv head (rows of a step or tile split
    # tokens unevenly), over several 128-row / 64-key tiles and ragged tails
    (37, [61, 130], 6, 2, 512, 50, "bf16", False),
    (90, [77], 8, 4, 512, -1, "bf16", True),
    (200, [300, 45], 8, 2, 512, -1, "bf16", False),
    (0, [3, 1], 2, 1, 512, -1, "bf16", False),   # one key tile: the shortest pipelines
    # the largest grouped-query ratios (128 at head dims 64 / 128, 32 at 512), and a
    # window far past every position (run as the global mask)
    (37, [40, 3], 128, 1, 64, -1, "bf16", False),
    (20, [33], 128, 1, 128, 15, "bf16", False),
    (24, [40, 9], 32, 1, 512, -1, "bf16", False),
    (50, [40, 90], 8, 2, 128, 2147483647, "bf16", False),
]


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,dtype,scaled", CASES)
def test_dualkv_forward_matches_oracle(P, lens, Hq, Hkv, d, wl, dtype, scaled):
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, dtype, seed=P + len(lens), scaled=scaled,
                              dout=False)
    ref = oracle.ncopy_reference(x, window_left=wl, backward=False)
    dd = to_dev(x, dtype)
    o_p, lse_p, o_r, lse_r = dualkv_forward(dd, window_left=wl)
    torch.cuda.synchronize()
    check("o_p", o_p, ref["o_p"], dtype)
    check("o_r", o_r, ref["o_r"], dtype)
    check("lse_p", lse_p.t(), ref["lse_p"], dtype, bound=1e-5 if dtype == "fp32" else 2e-3)
    check("lse_r", lse_r.t(), ref["lse_r"], dtype, bound=1e-5 if dtype == "fp32" else 2e-3)


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128)])
def test_ncopy_packing_through_causal_kernel(dtype, d):
    P, lens, Hq, Hkv = 70, [40, 0, 95], 8, 2
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, dtype, seed=5, dout=False)
    ref = oracle.ncopy_reference(x, backward=False)
    # eq. (1): N sequences [P, R_i], each its own causal sequence.
    qs, ks, vs, cu = [], [], [], [0]
    for i in range(len(lens)):
        q, k, v = oracle.copy_of(x, i)
        qs.append(q), ks.append(k), vs.append(v)
        cu.append(cu[-1] + q.shape[0])
    t = lambda a: torch.from_numpy(np.concatenate(a)).to(torch.float32)
    dd = to_dev({"q": t(qs), "k": t(ks), "v": t(vs), "cu": torch.tensor(cu, dtype=torch.int32)},
                dtype)
    o, lse = dkv.dkv_ctx_fwd(dd["q"], dd["k"], dd["v"], dd["cu"], cu_host=dd["cu_host"])
    torch.cuda.synchronize()
    for i in range(len(lens)):
        a = cu[i]
        check("o prompt copy %d" % i, o[a:a + P], ref["o_p"], dtype)
        check("o resp copy %d" % i, o[a + P:cu[i + 1]],
              ref["o_r"][x["cu"][i]:x["cu"][i + 1]], dtype)


def test_explicit_softmax_scale():
    P, lens, Hq, Hkv, d = 40, [30, 20], 4, 2, 64
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "fp32", seed=11, dout=False)
    ref = oracle.ncopy_reference(x, scale=0.05, backward=False)
    dd = to_dev(x, "fp32")
    o_p, lse_p, o_r, lse_r = dualkv_forward(dd, scale=0.05)
    torch.cuda.synchronize()
    check("o_p", o_p, ref["o_p"], "fp32")
    check("o_r", o_r, ref["o_r"], "fp32")
    check("lse_r", lse_r.t(), ref["lse_r"], "fp32")


def test_prompt_rows_identical_across_copies_P1():
    # P1 on the GPU: in the N-copy packing every copy's prompt rows come out bitwise
    # identical, and equal to Call 1 over the single prompt copy.
    P, lens, Hq, Hkv, d = 96, [10, 20, 30, 40], 8, 2, 128
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=3, dout=False)
    dd = to_dev(x, "bf16")
    N = len(lens)
    q = torch.cat([dd["q_p"]] * N)
    k = torch.cat([dd["k_p"]] * N)
    v = torch.cat([dd["v_p"]] * N)
    cu = torch.arange(N + 1, dtype=torch.int32) * P
    o, lse = dkv.dkv_ctx_fwd(q, k, v, cu.to(DEV), cu_host=cu.tolist())
    o1, lse1 = dkv.dkv_ctx_fwd(dd["q_p"], dd["k_p"], dd["v_p"],
                               torch.tensor([0, P], dtype=torch.int32, device=DEV),
                               cu_host=[0, P])
    torch.cuda.synchronize()
    for i in range(N):
        assert torch.equal(o[i * P:(i + 1) * P], o1)
        assert torch.equal(lse[:, i * P:(i + 1) * P], lse1)

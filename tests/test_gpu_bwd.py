"""GPU parity of the backward against the CPU oracle.

The oracle runs the N-copy packing (eq. (2)) where each copy's prompt rows get their
own upstream gradient dO_P^(i); the GPU sees the single prompt copy with their sum
(Appendix A.5), and sums the shared prompt's K/V gradient over both calls and all N
responses in one fp32 accumulator (eq. (6)), cast once.
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

CASES = [
    # P, lens, Hq, Hkv, d, window_left, dtype, scaled
    (64, [32, 32, 32, 32], 2, 2, 64, -1, "fp32", False),        # the tiny workload
    (100, [37, 0, 1, 130], 4, 1, 64, -1, "fp32", False),
    (70, [65, 3], 8, 2, 128, -1, "fp32", False),
    (150, [100, 60], 8, 1, 128, 127, "fp32", False),
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16", True),
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16", False),
    (0, [50, 90], 4, 4, 64, -1, "bf16", False),
    (33, [200], 32, 8, 128, -1, "bf16", False),
    (191, [45, 150, 7], 16, 2, 64, 40, "bf16", False),
    (97, [120, 33], 4, 2, 128, 0, "bf16", False),
    (300, [140, 260, 1], 8, 2, 128, 200, "bf16", False),
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


def _run(P, lens, Hq, Hkv, d, wl, dtype, scaled, seed, split=False):
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, dtype, seed=seed, scaled=scaled)
    N = len(lens)
    do_copies = workloads.split_prompt_grad(x["do_p"], N, seed=seed)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, window_left=wl)
    t = to_dev(x, dtype)
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], t["cu"],
                                                cu_host=t["cu_host"], window_left=wl)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                            cu_host=t["cu_host"], window_left=wl, split=split)
    torch.cuda.synchronize()
    return x, t, ref, g, (o_p, lse_p, o_r, lse_r)


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,dtype,scaled", CASES)
def test_dualkv_backward_matches_oracle(P, lens, Hq, Hkv, d, wl, dtype, scaled):
    x, t, ref, g, fwd = _run(P, lens, Hq, Hkv, d, wl, dtype, scaled, seed=P + 3 * len(lens))
    for k in GRADS:
        if g[k] is None:
            assert ref[k].size == 0, k
            continue
        check(k, g[k], ref[k], dtype)


def _random_cases(n, seed):
    """Seeded random shapes over the supported space: prompt length (0 allowed),
    response lengths (0 and 1 allowed), grouped-query ratio, head dim, window."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([64, 96, 128, 192, 256, 512]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8] if d <= 128 else [1, 2, 3, 4]))
        P = int(rng.choice([0, int(rng.integers(1, 200))]))
        N = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, 160, size=N)]
        if sum(lens) == 0:
            lens[0] = int(rng.integers(1, 160))
        wl = int(rng.choice([-1, -1, int(rng.integers(0, 150))]))
        cases.append((P, lens, hkv * g, hkv, d, wl))
    return cases


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl", _random_cases(12, 2026))
def test_random_shapes_match_oracle(P, lens, Hq, Hkv, d, wl):
    x, t, ref, g, fwd = _run(P, lens, Hq, Hkv, d, wl, "bf16", False, seed=7 + P)
    o_p, lse_p, o_r, lse_r = fwd
    check("o_r", o_r, ref["o_r"], "bf16")
    for k in GRADS:
        if g[k] is None:
            assert ref[k].size == 0, k
            continue
        check(k, g[k], ref[k], "bf16")


def test_accumulator_order_is_free():
    # Call 2 first (clearing) then Call 1 (finalizing) gives the same dK_P / dV_P.
    P, lens, Hq, Hkv, d, dtype = 96, [50, 70, 20], 8, 2, 128, "bf16"
    x, t, ref, g, (o_p, lse_p, o_r, lse_r) = _run(P, lens, Hq, Hkv, d, -1, dtype, False, 4)
    acc = torch.empty((2, P, Hkv, d), dtype=torch.float32, device=DEV)
    dkv.dkv_bwd(t["q_r"], t["k_p"], t["v_p"], t["k_r"], t["v_r"], o_r, lse_r, t["do_r"],
                t["cu"], acc_dk_p=acc[0], acc_dv_p=acc[1], acc_flags=dkv.DKV_ACC_ZERO,
                cu_host=t["cu_host"])
    cu_p = torch.tensor([0, P], dtype=torch.int32, device=DEV)
    _, dk_p, dv_p = dkv.dkv_ctx_bwd(t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], cu_p,
                                    cu_host=[0, P], acc_dk=acc[0], acc_dv=acc[1],
                                    acc_flags=dkv.DKV_ACC_FINALIZE)
    torch.cuda.synchronize()
    check("dk_p", dk_p, ref["dk_p"], dtype)
    check("dv_p", dv_p, ref["dv_p"], dtype)
    # both orders agree to fp32 reassociation before the single bf16 cast
    assert (dk_p.float() - g["dk_p"].float()).abs().max().item() <= \
        2e-2 * g["dk_p"].float().abs().max().item()


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128)])
def test_ncopy_backward_through_causal_kernel(dtype, d):
    # The N-copy packing of eq. (1) through dkv_ctx_bwd with direct dK/dV writes: each
    # copy's gradients must match that copy's oracle gradients.
    P, lens, Hq, Hkv = 70, [40, 0, 95], 8, 2
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, dtype, seed=9)
    N = len(lens)
    do_copies = workloads.split_prompt_grad(x["do_p"], N, seed=9)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, keep_copies=True)
    qs, ks, vs, dos, cu = [], [], [], [], [0]
    for i in range(N):
        q, k, v = oracle.copy_of(x, i)
        a, b = int(x["cu"][i]), int(x["cu"][i + 1])
        qs.append(q), ks.append(k), vs.append(v)
        dos.append(np.concatenate([do_copies[i].numpy(), x["do_r"][a:b].numpy()]))
        cu.append(cu[-1] + q.shape[0])
    f = lambda z: torch.from_numpy(np.concatenate(z)).to(torch.float32)
    dd = to_dev({"q": f(qs), "k": f(ks), "v": f(vs), "do": f(dos),
                 "cu": torch.tensor(cu, dtype=torch.int32)}, dtype)
    o, lse = dkv.dkv_ctx_fwd(dd["q"], dd["k"], dd["v"], dd["cu"], cu_host=dd["cu_host"])
    dq, dk, dv = dkv.dkv_ctx_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], dd["cu"],
                                 cu_host=dd["cu_host"])
    torch.cuda.synchronize()
    for i in range(N):
        c = ref["copies"][i]
        a, b = cu[i], cu[i + 1]
        bound = None
        if dtype == "bf16":
            # per-copy do_p^(i) is not bf16-representable; its bf16 rounding is an input
            # perturbation of ~2^-9 relative, well inside the tolerance used here
            bound = None
        check("dq copy %d" % i, dq[a:b], c["dq"], dtype, bound)
        check("dk copy %d" % i, dk[a:b], c["dk"], dtype, bound)
        check("dv copy %d" % i, dv[a:b], c["dv"], dtype, bound)


def test_repeated_backward_consistent():
    # fp32 atomics may reorder the shared-prompt sums; every run must stay within the
    # tolerance of the oracle and of each other.
    P, lens, Hq, Hkv, d = 200, [64] * 8, 8, 2, 64
    x, t, ref, g, fwd = _run(P, lens, Hq, Hkv, d, -1, "fp32", False, 21)
    o_p, lse_p, o_r, lse_r = fwd
    for _ in range(3):
        g2 = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                 o_p, lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                                 cu_host=t["cu_host"])
        torch.cuda.synchronize()
        for k in GRADS:
            check(k, g2[k], ref[k], "fp32")


# Split mode (DKV_ACC_SPLIT): chunks of ceil(N / 8) responses store their prompt-key
# sums into slices, added in slice order.  N > 8 gives chunks of several sequences;
# the windowed cases have prompt tiles that no row of a chunk sees (zero slices).
SPLIT_CASES = [
    # P, lens, Hq, Hkv, d, window_left, dtype
    (130, [77, 64, 129], 8, 2, 128, -1, "bf16"),
    (96, [40, 0, 33, 70, 1, 20, 55, 64, 12, 90, 8, 31], 8, 2, 128, -1, "bf16"),
    (300, [140, 260, 1, 90, 17, 3, 200, 45, 9, 60], 8, 2, 64, 100, "bf16"),
    (70, [65, 3, 40], 8, 2, 128, -1, "fp32"),
    (100, [150, 20], 16, 4, 512, 63, "bf16"),
]


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,dtype", SPLIT_CASES)
def test_split_mode_matches_oracle_and_repeats_bitwise(P, lens, Hq, Hkv, d, wl, dtype):
    x, t, ref, g, (o_p, lse_p, o_r, lse_r) = _run(P, lens, Hq, Hkv, d, wl, dtype, False,
                                                  seed=11 + P, split=True)
    for k in GRADS:
        check(k, g[k], ref[k], dtype)
    # a second run gives the same bits for every gradient
    g2 = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                             lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                             cu_host=t["cu_host"], window_left=wl, split=True)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g[k], g2[k]), k
    # the atomic mode sums the same fp32 terms in another order
    ga = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                             lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                             cu_host=t["cu_host"], window_left=wl)
    torch.cuda.synchronize()
    for k in ("dq_p", "dq_r", "dk_r", "dv_r"):
        assert torch.equal(g[k], ga[k]), k
    for k in ("dk_p", "dv_p"):
        check(k + " (atomic vs split)", ga[k], g[k].detach().float().cpu().numpy().astype(np.float64),
              dtype)


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl,dtype", [
    (1500, [40, 70], 8, 2, 128, -1, "bf16"),    # 6000 flattened prompt rows: two chunks
    (1100, [30], 16, 2, 64, 700, "bf16"),       # G = 8 with a window: chunks of windowed rows
    (1500, [20], 8, 2, 128, -1, "fp32"),        # the fp32 dK/dV kernel
    (700, [50], 16, 2, 512, -1, "bf16"),        # the head-dim-split dK/dV kernel
    (1200, [40], 16, 2, 512, 600, "bf16"),      # its windowed row walk, rotated, in chunks
    (900, [60, 10], 12, 2, 256, -1, "bf16"),    # the pair dK/dV kernel
])
def test_call1_row_chunks(P, lens, Hq, Hkv, d, wl, dtype):
    # Call 1 over a prompt whose first key tiles see more than 4096 flattened query rows:
    # without DKV_ACC_SPLIT those tiles' rows are split over several work items that each
    # add into the accumulator; with it each element keeps one writer.  Both match the
    # oracle, and agree with each other up to the order of the fp32 additions.
    print("call1 chunks: P=%d lens=%s Hq=%d Hkv=%d d=%d wl=%d %s" % (P, lens, Hq, Hkv, d, wl, dtype),
          flush=True)
    assert P * (Hq // Hkv) > 4096
    x, t, ref, g, (o_p, lse_p, o_r, lse_r) = _run(P, lens, Hq, Hkv, d, wl, dtype, False,
                                                  seed=P + d, split=False)
    for k in GRADS:
        check(k + " (row chunks)", g[k], ref[k], dtype)
    g1 = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                             lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                             cu_host=t["cu_host"], window_left=wl, split=True)
    torch.cuda.synchronize()
    for k in GRADS:
        check(k + " (one writer)", g1[k], ref[k], dtype)
    for k in ("dq_p", "dq_r", "dk_r", "dv_r"):
        assert torch.equal(g[k], g1[k]), k
    for k in ("dk_p", "dv_p"):
        check(k + " (row chunks vs one writer)", g[k],
              g1[k].detach().float().cpu().numpy().astype(np.float64), dtype)

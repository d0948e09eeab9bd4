"""GPU parity of micro-batches that hold several prompt groups.

Each group has its own prompt (its own shared K_P, V_P) and its own responses; the
groups are independent instances of the method, run in one launch per kernel
(§2.2 "Data pipeline": several groups per micro-batch, each with its own context KV
and cu_seqlens).  The oracle is the N-copy definition applied group by group
(oracle.grouped_reference); the GPU sees the groups packed one after another: all
prompts in one prompt tensor, all responses in one response tensor.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prompt_exact_dkv_amd as dkv
from tests._gpu import check, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r")

MIXED = [(64, [32, 20]), (100, [50]), (0, [40, 7]), (30, [])]

CASES = [
    # groups [(P_j, response lengths)], Hq, Hkv, d, window_left, dtype
    (MIXED, 8, 2, 128, -1, "bf16"),
    (MIXED, 8, 2, 128, 50, "bf16"),
    ([(40, [30, 1]), (70, [0, 65])], 4, 2, 64, -1, "fp32"),
    ([(150, [100]), (33, [60, 61])], 8, 1, 128, 70, "fp32"),
    ([(70, [45]), (129, [33, 64, 1]), (0, [20])], 8, 2, 512, 40, "bf16"),
    ([(90, [77, 5]), (40, [130])], 16, 4, 512, -1, "bf16"),
    ([(200, [150]), (3, [60, 60])], 32, 8, 128, -1, "bf16"),
    ([(57, [10, 80, 3]), (190, [70, 0, 44])], 6, 2, 64, 60, "bf16"),
]


def _run(groups, Hq, Hkv, d, wl, dtype, seed, split=False):
    xs, pk = workloads.make_group_inputs(groups, Hq, Hkv, d, dtype, seed=seed)
    do_copies = [workloads.split_prompt_grad(x["do_p"], len(lens), seed=seed + j)
                 if len(lens) else None for j, (x, (_, lens)) in enumerate(zip(xs, groups))]
    ref = oracle.grouped_reference(xs, do_copies=do_copies, window_left=wl)
    t = to_dev(pk, dtype)
    ctx_cu = [int(c) for c in pk["ctx_cu"]]
    seq_cu = [int(c) for c in pk["seq_cu"]]
    kw = dict(cu_host=t["cu_host"], window_left=wl, ctx_cu_host=ctx_cu,
              group_seq_cu_host=seq_cu)
    fwd = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                             t["cu"], **kw)
    o_p, lse_p, o_r, lse_r = fwd
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"], split=split, **kw)
    torch.cuda.synchronize()
    return t, ref, fwd, g, kw


@pytest.mark.parametrize("groups,Hq,Hkv,d,wl,dtype", CASES)
def test_prompt_groups_match_oracle(groups, Hq, Hkv, d, wl, dtype):
    t, ref, (o_p, lse_p, o_r, lse_r), g, _ = _run(groups, Hq, Hkv, d, wl, dtype,
                                                  seed=100 + Hq + d)
    check("o_p", o_p, ref["o_p"], dtype)
    check("o_r", o_r, ref["o_r"], dtype)
    lb = 1e-5 if dtype == "fp32" else 2e-3
    check("lse_p", lse_p.t(), ref["lse_p"], dtype, bound=lb)
    check("lse_r", lse_r.t(), ref["lse_r"], dtype, bound=lb)
    for k in GRADS:
        check(k, g[k], ref[k], dtype)


SPLIT_CASES = [
    # 12 responses in 3 groups: the chunks of ceil(12 / 8) = 2 responses straddle groups
    ([(96, [40, 0, 33, 70, 1]), (50, [20, 55, 64]), (130, [12, 90, 8, 31])], 8, 2, 128, -1,
     "bf16"),
    ([(70, [65, 3]), (0, [40]), (45, [20, 9, 33])], 8, 2, 64, 30, "fp32"),
    ([(100, [150]), (60, [20, 70])], 16, 4, 512, 63, "bf16"),
]


@pytest.mark.parametrize("groups,Hq,Hkv,d,wl,dtype", SPLIT_CASES)
def test_prompt_groups_split_mode(groups, Hq, Hkv, d, wl, dtype):
    t, ref, (o_p, lse_p, o_r, lse_r), g, kw = _run(groups, Hq, Hkv, d, wl, dtype, seed=7,
                                                   split=True)
    for k in GRADS:
        check(k, g[k], ref[k], dtype)
    args = (t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p, lse_p, o_r, lse_r,
            t["do_p"], t["do_r"], t["cu"])
    g2 = dkv.dualkv_backward(*args, split=True, **kw)
    ga = dkv.dualkv_backward(*args, **kw)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g[k], g2[k]), k
    for k in ("dk_p", "dv_p"):
        check(k + " (atomic vs split)", ga[k],
              g[k].detach().float().cpu().numpy().astype(np.float64), dtype)


def test_prompt_groups_call1_row_chunks():
    # Two prompts long enough (over 4096 flattened rows) that Call 1 splits their first
    # key tiles' rows into chunks added into the accumulator, an empty prompt, and a group
    # without responses: the chunked result and the one-writer (split mode) result both
    # match the oracle, the latter bitwise on a second run, and they agree with each other
    # up to the order of the fp32 additions.
    groups = [(1500, [40]), (0, [30]), (1100, [30, 20]), (60, [])]
    Hq, Hkv, d, wl, dtype = 8, 2, 128, -1, "bf16"
    print("groups with call-1 row chunks: %s" % groups, flush=True)
    t, ref, (o_p, lse_p, o_r, lse_r), g, kw = _run(groups, Hq, Hkv, d, wl, dtype, seed=21)
    for k in GRADS:
        check(k + " (row chunks)", g[k], ref[k], dtype)
    args = (t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p, lse_p, o_r, lse_r,
            t["do_p"], t["do_r"], t["cu"])
    g1 = dkv.dualkv_backward(*args, split=True, **kw)
    g2 = dkv.dualkv_backward(*args, split=True, **kw)
    torch.cuda.synchronize()
    for k in GRADS:
        check(k + " (one writer)", g1[k], ref[k], dtype)
        assert torch.equal(g1[k], g2[k]), k
    for k in ("dk_p", "dv_p"):
        check(k + " (row chunks vs one writer)", g[k],
              g1[k].detach().float().cpu().numpy().astype(np.float64), dtype)


def test_one_group_equals_no_groups():
    # One group spanning every response gives the bits of the call without groups.
    P, lens, Hq, Hkv, d = 130, [77, 64, 129], 8, 2, 128
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "bf16", seed=3)
    t = to_dev(x, "bf16")
    base = dict(cu_host=t["cu_host"])
    grp = dict(base, ctx_cu_host=[0, P], group_seq_cu_host=[0, len(lens)])
    outs = []
    for kw in (base, grp):
        o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                    t["k_r"], t["v_r"], t["cu"], **kw)
        g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                o_p, lse_p, o_r, lse_r, t["do_p"], t["do_r"], t["cu"],
                                split=True, **kw)
        outs.append([o_r, lse_r] + [g[k] for k in GRADS])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_full_size_groups_sparse_gradient():
    # The multi-group micro-batch that bench.py times (4 prompts of U{2048..8192}
    # tokens, 8 responses each), through the same calls.  As in the full-size
    # single-prompt test, dO is zero except on a few prompt rows of every group and a
    # few rows of the first and last response of every group, so every key / value
    # gradient is a sum the oracle computes exactly; O, LSE and dQ on those rows.
    w = workloads.WORKLOADS["multi_group"]
    shapes = w.group_shapes()
    Hq, Hkv, d, wl = w.Hq, w.Hkv, w.d, w.window_left
    xs, pk = workloads.make_group_inputs(shapes, Hq, Hkv, d, "bf16", seed=w.seed,
                                         scaled=w.scaled, dout=False)
    cu = [int(c) for c in pk["cu"]]
    ccu = [int(c) for c in pk["ctx_cu"]]
    scu = [int(c) for c in pk["seq_cu"]]
    P, T = ccu[-1], cu[-1]
    print("[groups] P=%s T=%d" % ([p for p, _ in shapes], T), flush=True)
    rows_of = lambda n: sorted({r for r in (0, 1, n // 2, n - 2, n - 1) if 0 <= r < n})
    g = torch.Generator().manual_seed(4242)
    f32 = torch.float32
    do_p = torch.zeros((P, Hq, d), dtype=f32)
    do_r = torch.zeros((T, Hq, d), dtype=f32)
    p_rows, seqs = {}, {}
    for j in range(len(shapes)):
        p_rows[j] = rows_of(shapes[j][0])
        idx = [ccu[j] + r for r in p_rows[j]]
        do_p[idx] = torch.randn((len(idx), Hq, d), generator=g, dtype=f32).to(torch.bfloat16).float()
        for i in sorted({scu[j], scu[j + 1] - 1}):
            seqs[i] = (j, rows_of(cu[i + 1] - cu[i]))
            idx = [cu[i] + r for r in seqs[i][1]]
            do_r[idx] = torch.randn((len(idx), Hq, d), generator=g, dtype=f32).to(torch.bfloat16).float()

    t = {k: pk[k].to(torch.bfloat16).to("cuda:0") for k in ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r")}
    cu_d = pk["cu"].to("cuda:0")
    kw = dict(cu_host=cu, window_left=wl, ctx_cu_host=ccu, group_seq_cu_host=scu)
    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], cu_d, **kw)
    gr = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                             lse_p, o_r, lse_r, do_p.to(torch.bfloat16).to("cuda:0"),
                             do_r.to(torch.bfloat16).to("cuda:0"), cu_d, **kw)
    torch.cuda.synchronize()

    f64 = lambda a: np.ascontiguousarray(a.numpy(), dtype=np.float64)
    dk_p_ref = np.zeros((P, Hkv, d))
    dv_p_ref = np.zeros((P, Hkv, d))
    dk_r_ref = np.zeros((T, Hkv, d))
    dv_r_ref = np.zeros((T, Hkv, d))
    for j, (Pj, lens) in enumerate(shapes):
        x = xs[j]
        k_p, v_p = f64(x["k_p"]), f64(x["v_p"])
        rows = p_rows[j]
        idx = [ccu[j] + r for r in rows]
        o_ref, lse_ref = oracle.rows_fwd(k_p, v_p, rows, x["q_p"][rows], window_left=wl)
        check("o_p[group %d]" % j, o_p[idx], o_ref, "bf16")
        check("lse_p[group %d]" % j, lse_p[:, idx].t(), lse_ref, "bf16", bound=2e-3)
        dq_ref = np.zeros((len(rows), Hq, d))
        dk_j = dk_p_ref[ccu[j]:ccu[j + 1]]
        dv_j = dv_p_ref[ccu[j]:ccu[j + 1]]
        for _ in range(len(lens)):   # each copy's prompt rows get dO_P / N_j
            dq_ref += oracle.rows_bwd_scatter(k_p, v_p, rows, x["q_p"][rows],
                                              f64(do_p[idx]) / len(lens), dk_j, dv_j,
                                              window_left=wl)
        check("dq_p[group %d]" % j, gr["dq_p"][idx], dq_ref, "bf16")
    for i, (j, rows) in seqs.items():
        a, b = cu[i], cu[i + 1]
        Pj = shapes[j][0]
        k_i = np.concatenate([f64(xs[j]["k_p"]), f64(pk["k_r"][a:b])])
        v_i = np.concatenate([f64(xs[j]["v_p"]), f64(pk["v_r"][a:b])])
        idx = [a + r for r in rows]
        o_ref, lse_ref = oracle.rows_fwd(k_i, v_i, [Pj + r for r in rows], pk["q_r"][idx],
                                         window_left=wl)
        check("o_r[seq %d]" % i, o_r[idx], o_ref, "bf16")
        check("lse_r[seq %d]" % i, lse_r[:, idx].t(), lse_ref, "bf16", bound=2e-3)
        dk_i = np.zeros_like(k_i)
        dv_i = np.zeros_like(v_i)
        dq_i = oracle.rows_bwd_scatter(k_i, v_i, [Pj + r for r in rows], pk["q_r"][idx],
                                       f64(do_r[idx]), dk_i, dv_i, window_left=wl)
        check("dq_r[seq %d]" % i, gr["dq_r"][idx], dq_i, "bf16")
        dk_p_ref[ccu[j]:ccu[j + 1]] += dk_i[:Pj]
        dv_p_ref[ccu[j]:ccu[j + 1]] += dv_i[:Pj]
        dk_r_ref[a:b] = dk_i[Pj:]
        dv_r_ref[a:b] = dv_i[Pj:]
    check("dk_p", gr["dk_p"], dk_p_ref, "bf16")
    check("dv_p", gr["dv_p"], dv_p_ref, "bf16")
    check("dk_r", gr["dk_r"], dk_r_ref, "bf16")
    check("dv_r", gr["dv_r"], dv_r_ref, "bf16")


def _random_group_cases(n, seed):
    """Seeded random micro-batches of prompt groups: group count, prompt lengths (0
    allowed), response counts (0 allowed) and lengths (0 and 1 allowed), GQA ratio,
    head dim, window and 16-bit type."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([64, 128, 512]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 6] if d < 512 else [1, 2, 4]))
        groups = []
        for _ in range(int(rng.integers(1, 5))):
            P = int(rng.choice([0, int(rng.integers(1, 160))]))
            lens = [int(x) for x in rng.integers(0, 120, size=int(rng.integers(0, 4)))]
            groups.append((P, lens))
        if sum(sum(ls) for _, ls in groups) == 0:
            groups.append((int(rng.integers(1, 100)), [int(rng.integers(1, 100))]))
        wl = int(rng.choice([-1, -1, int(rng.integers(0, 120))]))
        cases.append((groups, hkv * g, hkv, d, wl, str(rng.choice(["bf16", "fp16"]))))
    return cases


@pytest.mark.parametrize("groups,Hq,Hkv,d,wl,dtype", _random_group_cases(10, 77))
def test_random_prompt_groups(groups, Hq, Hkv, d, wl, dtype):
    t, ref, (o_p, lse_p, o_r, lse_r), g, _ = _run(groups, Hq, Hkv, d, wl, dtype,
                                                  seed=300 + d + Hq)
    check("o_p", o_p, ref["o_p"], dtype)
    check("o_r", o_r, ref["o_r"], dtype)
    for k in GRADS:
        check(k, g[k], ref[k], dtype)

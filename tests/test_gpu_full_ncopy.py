"""At full workload sizes, every output of the two-call path on ALL rows, against the
same library's causal path run on the N-copy packing (eq. (1)-(2)): the equivalence the
method rests on (§2.2; App. A.2 every copy's prompt rows equal; App. A.5 the prompt's
gradient is the sum over the copies).  The oracle checks the full-size runs on sampled
rows (tests/test_gpu_full.py) and the causal path at small sizes; this checks the rest of
every row at the sizes bench.py times.

Each copy's prompt rows get the upstream gradient dO_P / N (N a power of two, so the
division is exact and the copies' sum is dO_P).  With the prompt length a multiple of the
key tiles, Call 2 visits the N-copy sequence's key tiles in the same order, so the
response rows' O, LSE and dQ, the prompt rows' O and LSE (Call 1 against each copy's
prefix), and the response keys' dK, dV agree bit for bit, except on the windowed d = 512
layer: there the dK/dV row walk is rotated onto a clock counted from the sequence's first
row, which differs between the packings, so those agree within the bf16 bound.  The prompt's dQ and
the shared dK_P, dV_P are compared with the fp32 sum over the copies, within the bf16
bound (max|err| <= 2e-2 max|ref|)."""
import pytest
import torch

import workloads
import shared_prompt_exact_dkv_amd as dkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _close(name, got, ref):
    got, ref = got.float(), ref.float()
    err = (got - ref).abs().max().item()
    bound = 2e-2 * ref.abs().max().item()
    print("    %-8s max|err| %.3e  bound %.3e" % (name, err, bound), flush=True)
    assert torch.isfinite(got).all(), name
    assert err <= bound, "%s: max|err| = %.3e > %.3e" % (name, err, bound)


@pytest.mark.parametrize("name,keys_bitwise", [
    ("qwen3_8b", True), ("dapo_varlen", True), ("large_rollout", True),
    ("d512_global", True), ("d512_swa", False), ("d256_swa", True), ("hd96", True),
    ("hd192", True)])
def test_two_calls_equal_ncopy_causal_path_on_every_row(name, keys_bitwise):
    w = workloads.WORKLOADS[name]
    lens = w.resp_lens()
    N, P, Hq, Hkv, d, wl = w.N, w.P, w.Hq, w.Hkv, w.d, w.window_left
    assert N & (N - 1) == 0 and P % 128 == 0
    print("[ncopy] %s: P=%d N=%d Hq=%d Hkv=%d d=%d wl=%d" % (name, P, N, Hq, Hkv, d, wl),
          flush=True)
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, w.dtype, seed=w.seed + 50, scaled=w.scaled,
                              dout=True)
    cu = [int(c) for c in x["cu"]]
    dt = torch.bfloat16
    t = {k: x[k].to(dt).to(DEV) for k in ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r")}
    del x
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)

    o_p, lse_p, o_r, lse_r = dkv.dualkv_forward(t["q_p"], t["k_p"], t["v_p"], t["q_r"],
                                                t["k_r"], t["v_r"], cu_d, cu_host=cu,
                                                window_left=wl)
    g = dkv.dualkv_backward(t["q_p"], t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_p,
                            lse_p, o_r, lse_r, t["do_p"], t["do_r"], cu_d, cu_host=cu,
                            window_left=wl)

    # N-copy packing: copy i is [prompt; response i]
    pieces = lambda a, b: torch.cat([z for i in range(N) for z in (a, b[cu[i]:cu[i + 1]])])
    qn, kn, vn = (pieces(t[n + "_p"], t[n + "_r"]) for n in ("q", "k", "v"))
    don = pieces(t["do_p"] / N, t["do_r"])
    cun = [0]
    for r in lens:
        cun.append(cun[-1] + P + r)
    on, lsen = dkv.dkv_ctx_fwd(qn, kn, vn, None, cu_host=cun, window_left=wl)
    dqn, dkn, dvn = dkv.dkv_ctx_bwd(qn, kn, vn, on, lsen, don, None, cu_host=cun,
                                    window_left=wl)
    torch.cuda.synchronize()
    print("[ncopy] %s: both paths done" % name, flush=True)

    prompt_idx = torch.cat([torch.arange(cun[i], cun[i] + P) for i in range(N)]).to(DEV)
    resp_idx = torch.cat([torch.arange(cun[i] + P, cun[i + 1]) for i in range(N)]).to(DEV)
    assert torch.equal(on[resp_idx], o_r), "o_r"
    assert torch.equal(lsen[:, resp_idx], lse_r), "lse_r"
    assert torch.equal(dqn[resp_idx], g["dq_r"]), "dq_r"
    for i in range(N):   # every copy's prompt rows equal Call 1 (App. A.2)
        assert torch.equal(on[cun[i]:cun[i] + P], o_p), "o_p, copy %d" % i
        assert torch.equal(lsen[:, cun[i]:cun[i] + P], lse_p), "lse_p, copy %d" % i
    if keys_bitwise:
        assert torch.equal(dkn[resp_idx], g["dk_r"]), "dk_r"
        assert torch.equal(dvn[resp_idx], g["dv_r"]), "dv_r"
    else:
        _close("dk_r", g["dk_r"], dkn[resp_idx])
        _close("dv_r", g["dv_r"], dvn[resp_idx])
    # the prompt: sums over the copies (App. A.5, eq. (6))
    sum_copies = lambda a: a[prompt_idx].float().view(N, P, *a.shape[1:]).sum(0)
    _close("dq_p", g["dq_p"], sum_copies(dqn))
    _close("dk_p", g["dk_p"], sum_copies(dkn))
    _close("dv_p", g["dv_p"], sum_copies(dvn))

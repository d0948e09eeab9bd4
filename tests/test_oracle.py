"""Pins for the CPU oracle (runs without a GPU).

The oracle (oracle/dkv_oracle.c) is eq. (2) of the DualKV paper (arXiv 2605.15422,
§2.1) for one causal sequence, with its gradients.  These tests tie it to things
other than itself:

* an independent library routine: torch's scaled_dot_product_attention in float64
  with an explicit boolean mask, and torch autograd through it;
* central finite differences of L = sum(dO * O) (brute force, tiny inputs);
* closed forms (equal keys, zero scale, zero-width window);
* the paper's own properties of the two-call decomposition (§2.2, eqs. (3)-(6),
  Appendix A.2 and A.5): prompt rows agree across copies (P1); response rows equal
  eq. (4) (P2); the copies' prompt K/V gradients sum to the shared-prompt gradient
  of eq. (6) (P3), checked against a separate two-call formulation differentiated
  by torch autograd.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads



@pytest.fixture(autouse=True)
def _float64_default():
    """The pins build tensors in float64; the default is restored after each test so
    that no other test module sees it."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _sdpa_ref(q, k, v, scale, window_left, kvh):
    """torch fp64 SDPA with an explicit boolean mask; returns O, LSE and a closure."""
    S, Hq, d = q.shape
    idx = torch.as_tensor(kvh, dtype=torch.long)
    kk = k[:, idx, :]              # [S, Hq, d]
    vv = v[:, idx, :]
    t = torch.arange(S).view(-1, 1)
    j = torch.arange(S).view(1, -1)
    vis = j <= t
    if window_left >= 0:
        vis = vis & (j >= t - window_left)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2), kk.permute(1, 0, 2), vv.permute(1, 0, 2),
        attn_mask=vis, scale=scale).permute(1, 0, 2)
    s = torch.einsum("thc,jhc->htj", q, kk) * scale
    s = s.masked_fill(~vis.unsqueeze(0), float("-inf"))
    lse = torch.logsumexp(s, dim=-1).transpose(0, 1)   # [S, Hq]
    return o, lse


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


CASES = [
    # S, Hq, Hkv, d, window_left, scale
    (1, 1, 1, 4, -1, None),
    (7, 2, 1, 8, -1, None),
    (13, 4, 2, 16, -1, 0.3),
    (16, 4, 1, 8, 3, None),
    (21, 2, 2, 5, 0, None),
    (19, 6, 3, 8, 100, None),
]


@pytest.mark.parametrize("S,Hq,Hkv,d,wl,scale", CASES)
def test_fwd_bwd_match_torch_sdpa_fp64(S, Hq, Hkv, d, wl, scale):
    q = _rand((S, Hq, d), 1)
    k = _rand((S, Hkv, d), 2)
    v = _rand((S, Hkv, d), 3)
    do = _rand((S, Hq, d), 4)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    kvh = [h // (Hq // Hkv) for h in range(Hq)]
    o, lse = oracle.seq_fwd(q, k, v, scale=scale, window_left=wl)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    o_ref, lse_ref = _sdpa_ref(qt, kt, vt, sc, wl, kvh)
    np.testing.assert_allclose(o, o_ref.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.detach().numpy(), rtol=0, atol=1e-12)
    (o_ref * do).sum().backward()
    g = oracle.seq_bwd(q, k, v, do, scale=scale, window_left=wl)
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"], kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"], vt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["lse"], lse_ref.detach().numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("wl", [-1, 2])
def test_bwd_matches_central_finite_differences(wl):
    S, Hq, Hkv, d = 6, 2, 1, 3
    q, k, v, do = _rand((S, Hq, d), 11), _rand((S, Hkv, d), 12), _rand((S, Hkv, d), 13), \
        _rand((S, Hq, d), 14)

    def loss(q_, k_, v_):
        o, _ = oracle.seq_fwd(q_, k_, v_, window_left=wl)
        return float((o * do.numpy()).sum())

    g = oracle.seq_bwd(q, k, v, do, window_left=wl)
    eps = 1e-6
    for name, x, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        fd = np.zeros(x.shape)
        for idx in np.ndindex(*x.shape):
            xp = x.clone(); xp[idx] += eps
            xm = x.clone(); xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            fd[idx] = (loss(**{n + "_": a for n, a in args_p.items()})
                       - loss(**{n + "_": a for n, a in args_m.items()})) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=2e-8, err_msg=name)


def test_closed_form_equal_keys_uniform_weights():
    S, Hq, Hkv, d, wl = 9, 2, 1, 4, 3
    q = _rand((S, Hq, d), 21)
    krow = _rand((1, 1, d), 22)
    k = krow.expand(S, Hkv, d).clone()
    v = _rand((S, Hkv, d), 23)
    sc = 0.7
    o, lse = oracle.seq_fwd(q, k, v, scale=sc, window_left=wl)
    for t in range(S):
        j0 = max(0, t - wl)
        n = t - j0 + 1
        mean_v = v[j0:t + 1, 0].mean(0).numpy()
        for h in range(Hq):
            np.testing.assert_allclose(o[t, h], mean_v, atol=1e-13)
            s = sc * float(q[t, h] @ krow[0, 0])
            assert abs(lse[t, h] - (s + math.log(n))) < 1e-12


def test_closed_form_zero_scale():
    S, Hq, Hkv, d = 8, 4, 2, 3
    q, k, v, do = _rand((S, Hq, d), 31), _rand((S, Hkv, d), 32), _rand((S, Hkv, d), 33), \
        _rand((S, Hq, d), 34)
    o, lse = oracle.seq_fwd(q, k, v, scale=0.0)
    g = oracle.seq_bwd(q, k, v, do, scale=0.0)
    kvh = [h // 2 for h in range(Hq)]
    dv = np.zeros((S, Hkv, d))
    for t in range(S):
        for h in range(Hq):
            np.testing.assert_allclose(o[t, h], v[:t + 1, kvh[h]].mean(0).numpy(), atol=1e-13)
            assert abs(lse[t, h] - math.log(t + 1)) < 1e-13
            dv[:t + 1, kvh[h]] += do[t, h].numpy() / (t + 1)
    assert np.abs(g["dq"]).max() == 0.0
    assert np.abs(g["dk"]).max() == 0.0
    np.testing.assert_allclose(g["dv"], dv, atol=1e-13)


def test_closed_form_zero_width_window():
    S, Hq, Hkv, d = 7, 4, 2, 5
    q, k, v, do = _rand((S, Hq, d), 41), _rand((S, Hkv, d), 42), _rand((S, Hkv, d), 43), \
        _rand((S, Hq, d), 44)
    o, lse = oracle.seq_fwd(q, k, v, window_left=0)
    g = oracle.seq_bwd(q, k, v, do, window_left=0)
    sc = 1.0 / math.sqrt(d)
    for t in range(S):
        for h in range(Hq):
            np.testing.assert_allclose(o[t, h], v[t, h // 2].numpy(), atol=1e-14)
            assert abs(lse[t, h] - sc * float(q[t, h] @ k[t, h // 2])) < 1e-13
    assert np.abs(g["dq"]).max() < 1e-15 and np.abs(g["dk"]).max() < 1e-15
    dv = do.view(S, Hkv, 2, d).sum(2).numpy()
    np.testing.assert_allclose(g["dv"], dv, atol=1e-13)


def test_selected_rows_and_keys_match_full():
    S, Hq, Hkv, d, wl = 23, 4, 2, 8, 6
    q, k, v, do = _rand((S, Hq, d), 51), _rand((S, Hkv, d), 52), _rand((S, Hkv, d), 53), \
        _rand((S, Hq, d), 54)
    full = oracle.seq_bwd(q, k, v, do, window_left=wl)
    o_full, lse_full = oracle.seq_fwd(q, k, v, window_left=wl)
    rows = [0, 5, 22, 11]
    keys = [22, 0, 7]
    part = oracle.seq_bwd(q, k, v, do, window_left=wl, rows=rows, keys=keys)
    o_part, lse_part = oracle.seq_fwd(q, k, v, window_left=wl, rows=rows)
    np.testing.assert_array_equal(part["dq"], full["dq"][rows])
    np.testing.assert_array_equal(part["dk"], full["dk"][keys])
    np.testing.assert_array_equal(o_part, o_full[rows])
    np.testing.assert_array_equal(lse_part, lse_full[rows])
    rows_only = oracle.seq_bwd(q, k, v, do, window_left=wl, rows=rows, need_keys=False)
    np.testing.assert_array_equal(rows_only["dq"], full["dq"][rows])


# --- the paper's two-call decomposition, written independently with torch autograd ---

def _attend(qr, kk, vv, qpos, kpos, scale, wl, kvh):
    """softmax(scale * q k^T + mask) v with explicit logical positions (eqs. (3)/(4))."""
    idx = torch.as_tensor(kvh, dtype=torch.long)
    kk = kk[:, idx, :]
    vv = vv[:, idx, :]
    s = torch.einsum("thc,jhc->htj", qr, kk) * scale
    vis = kpos.view(1, -1) <= qpos.view(-1, 1)
    if wl >= 0:
        vis = vis & (kpos.view(1, -1) >= qpos.view(-1, 1) - wl)
    s = s.masked_fill(~vis.unsqueeze(0), float("-inf"))
    a = torch.softmax(s, dim=-1)
    lse = torch.logsumexp(s, dim=-1).transpose(0, 1)
    return torch.einsum("htj,jhc->thc", a, vv), lse


def _two_call(x, wl, scale):
    """Call 1 (eq. 3) over the single prompt, Call 2 (eq. 4) per response.  K_P/V_P
    are single leaf tensors, so autograd sums both calls' gradients (eq. 6)."""
    t = {n: torch.as_tensor(np.asarray(x[n]), dtype=torch.float64).clone().requires_grad_(True)
         for n in ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r")}
    cu = [int(c) for c in x["cu"]]
    P, Hq, d = t["q_p"].shape
    Hkv = t["k_p"].shape[1]
    kvh = [h // (Hq // Hkv) for h in range(Hq)]
    ppos = torch.arange(P)
    o_p, lse_p = _attend(t["q_p"], t["k_p"], t["v_p"], ppos, ppos, scale, wl, kvh)
    o_r, lse_r = [], []
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        kk = torch.cat([t["k_p"], t["k_r"][a:b]], 0)
        vv = torch.cat([t["v_p"], t["v_r"][a:b]], 0)
        qpos = P + torch.arange(b - a)          # context_seqlen = P shifts the mask
        kpos = torch.arange(P + b - a)
        o, l = _attend(t["q_r"][a:b], kk, vv, qpos, kpos, scale, wl, kvh)
        o_r.append(o)
        lse_r.append(l)
    o_r = torch.cat(o_r, 0)
    lse_r = torch.cat(lse_r, 0)
    loss = (o_p * torch.as_tensor(np.asarray(x["do_p"]))).sum() + \
        (o_r * torch.as_tensor(np.asarray(x["do_r"]))).sum()
    loss.backward()
    return {"o_p": o_p.detach().numpy(), "lse_p": lse_p.detach().numpy(),
            "o_r": o_r.detach().numpy(), "lse_r": lse_r.detach().numpy(),
            "dq_p": t["q_p"].grad.numpy(), "dk_p": t["k_p"].grad.numpy(),
            "dv_p": t["v_p"].grad.numpy(), "dq_r": t["q_r"].grad.numpy(),
            "dk_r": t["k_r"].grad.numpy(), "dv_r": t["v_r"].grad.numpy()}


TWO_CALL_CASES = [
    # P, lens, Hq, Hkv, d, wl
    (5, [3, 4, 1], 2, 1, 4, -1),
    (8, [6, 0, 2, 5], 4, 2, 8, -1),
    (7, [9, 3], 2, 2, 4, 4),
    (0, [5, 3], 2, 1, 4, -1),
    (6, [4], 3, 1, 4, -1),
    (9, [2, 7, 5], 4, 1, 8, 0),
    (4, [8, 8], 2, 1, 4, 20),
]


@pytest.mark.parametrize("P,lens,Hq,Hkv,d,wl", TWO_CALL_CASES)
def test_ncopy_equals_two_call_properties_P1_P2_P3(P, lens, Hq, Hkv, d, wl):
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "fp32", seed=7 + P, scaled=False)
    N = len(lens)
    do_copies = workloads.split_prompt_grad(x["do_p"], N, seed=3)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, window_left=wl, keep_copies=True)
    two = _two_call(x, wl, 1.0 / math.sqrt(d))
    # P1: prompt rows of every copy are identical (bitwise) in the forward.
    for c in ref["copies"][1:]:
        np.testing.assert_array_equal(c["o"][:P], ref["copies"][0]["o"][:P])
        np.testing.assert_array_equal(c["lse"][:P], ref["copies"][0]["lse"][:P])
    # P1 does not extend to the backward: the copies' prompt-row grads differ.
    if N > 1 and P > 0:
        assert np.abs(ref["copies"][0]["dv"][:P] - ref["copies"][1]["dv"][:P]).max() > 0
    # P2: response rows of eq. (2) equal eq. (4); prompt rows equal eq. (3).
    for key in ("o_p", "lse_p", "o_r", "lse_r"):
        np.testing.assert_allclose(ref[key], two[key], rtol=0, atol=1e-12, err_msg=key)
    # P3: per-copy prompt K/V grads, summed over copies, equal eq. (6) (Call 1 fed the
    # summed prompt-row gradient plus every response's Call-2 term); likewise dQ_P.
    for key in ("dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r"):
        np.testing.assert_allclose(ref[key], two[key], rtol=0, atol=1e-11, err_msg=key)


def test_ncopy_single_sequence_is_plain_causal():
    # N = 1 reduces to ordinary causal attention over P + R tokens.
    x = workloads.make_inputs(6, [5], 2, 1, 4, "fp32", seed=99)
    ref = oracle.ncopy_reference(x)
    q, k, v = oracle.copy_of(x, 0)
    o, lse = oracle.seq_fwd(q, k, v)
    np.testing.assert_array_equal(np.concatenate([ref["o_p"], ref["o_r"]]), o)
    np.testing.assert_array_equal(np.concatenate([ref["lse_p"], ref["lse_r"]]), lse)


def test_split_prompt_grad_sums_to_prompt_grad():
    do_p = workloads.make_inputs(16, [3], 4, 2, 8, "bf16", seed=5)["do_p"]
    parts = workloads.split_prompt_grad(do_p, 8, seed=1)
    np.testing.assert_allclose(parts.sum(0).numpy(), do_p.double().numpy(), rtol=0, atol=1e-15)
    assert (parts[0] - parts[1]).abs().max() > 0


def test_oracle_rejects_bad_arguments():
    q = torch.zeros(3, 2, 4)
    k = torch.zeros(3, 1, 4)
    with pytest.raises(ValueError):
        oracle.seq_fwd(q, k, k, kvh=[0, 1])      # kv-head index out of range
    with pytest.raises(ValueError):
        oracle.seq_fwd(q, k, k, rows=[3])        # row out of range


@pytest.mark.parametrize("S,Hq,Hkv,d,wl,scale", CASES)
def test_selected_rows_match_torch_sdpa_fp64(S, Hq, Hkv, d, wl, scale):
    # The selected-row forms used at full workload sizes (queries of the selected
    # rows only; upstream gradient zero on every other row) against torch fp64 SDPA
    # and autograd with dO zero outside the selected rows.
    q = _rand((S, Hq, d), 11)
    k = _rand((S, Hkv, d), 12)
    v = _rand((S, Hkv, d), 13)
    rows = sorted({0, S // 2, S - 1})
    do = torch.zeros((S, Hq, d))
    do[rows] = _rand((len(rows), Hq, d), 14)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    kvh = [h // (Hq // Hkv) for h in range(Hq)]
    o, lse = oracle.rows_fwd(k, v, rows, q[rows], scale=scale, window_left=wl)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    o_ref, lse_ref = _sdpa_ref(qt, kt, vt, sc, wl, kvh)
    np.testing.assert_allclose(o, o_ref.detach().numpy()[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.detach().numpy()[rows], rtol=0, atol=1e-12)
    (o_ref * do).sum().backward()
    dk = np.zeros((S, Hkv, d))
    dv = np.zeros((S, Hkv, d))
    dq = oracle.rows_bwd_scatter(k, v, rows, q[rows], do[rows], dk, dv, scale=scale,
                                 window_left=wl)
    np.testing.assert_allclose(dq, qt.grad.numpy()[rows], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-11)
    # the rows with a zero upstream gradient have a zero query gradient
    others = [t for t in range(S) if t not in rows]
    assert np.abs(qt.grad.numpy()[others]).max(initial=0.0) == 0.0


def test_scatter_accumulates_across_calls():
    # Two calls with disjoint rows add into the same dk / dv: the sum equals one call
    # with both row sets (what the full-size tests do over the copies of eq. (1)).
    S, Hq, Hkv, d = 30, 4, 2, 8
    q, k, v = _rand((S, Hq, d), 21), _rand((S, Hkv, d), 22), _rand((S, Hkv, d), 23)
    do = _rand((S, Hq, d), 24)
    a, b = [3, 17], [9, 29]
    dk1, dv1 = np.zeros((S, Hkv, d)), np.zeros((S, Hkv, d))
    oracle.rows_bwd_scatter(k, v, a, q[a], do[a], dk1, dv1)
    oracle.rows_bwd_scatter(k, v, b, q[b], do[b], dk1, dv1)
    dk2, dv2 = np.zeros((S, Hkv, d)), np.zeros((S, Hkv, d))
    ab = a + b
    oracle.rows_bwd_scatter(k, v, ab, q[ab], do[ab], dk2, dv2)
    np.testing.assert_allclose(dk1, dk2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv1, dv2, rtol=0, atol=1e-12)


def _two_call_grouped(packed, wl, scale):
    """Several prompt groups in one packed micro-batch, as one autograd graph: each
    prompt's Call 1 (eq. 3) over its own rows, and each response's Call 2 (eq. 4)
    over its own group's prompt rows then its own rows.  Prompt K/V rows are slices
    of one leaf tensor, so autograd sums every call's gradient into the right rows."""
    t = {n: torch.as_tensor(np.asarray(packed[n]), dtype=torch.float64).clone().requires_grad_(True)
         for n in ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r")}
    cu = [int(c) for c in packed["cu"]]
    ccu = [int(c) for c in packed["ctx_cu"]]
    scu = [int(c) for c in packed["seq_cu"]]
    Hq, Hkv = t["q_p"].shape[1], t["k_p"].shape[1]
    kvh = [h // (Hq // Hkv) for h in range(Hq)]
    o_p, lse_p, o_r, lse_r = [], [], [], []
    for j in range(len(ccu) - 1):
        c0, c1 = ccu[j], ccu[j + 1]
        P = c1 - c0
        ppos = torch.arange(P)
        o, l = _attend(t["q_p"][c0:c1], t["k_p"][c0:c1], t["v_p"][c0:c1], ppos, ppos, scale,
                       wl, kvh)
        o_p.append(o)
        lse_p.append(l)
        for i in range(scu[j], scu[j + 1]):
            a, b = cu[i], cu[i + 1]
            kk = torch.cat([t["k_p"][c0:c1], t["k_r"][a:b]], 0)
            vv = torch.cat([t["v_p"][c0:c1], t["v_r"][a:b]], 0)
            o, l = _attend(t["q_r"][a:b], kk, vv, P + torch.arange(b - a),
                           torch.arange(P + b - a), scale, wl, kvh)
            o_r.append(o)
            lse_r.append(l)
    o_p, lse_p, o_r, lse_r = (torch.cat(z, 0) for z in (o_p, lse_p, o_r, lse_r))
    loss = (o_p * torch.as_tensor(np.asarray(packed["do_p"]))).sum() + \
        (o_r * torch.as_tensor(np.asarray(packed["do_r"]))).sum()
    loss.backward()
    out = {"o_p": o_p, "lse_p": lse_p, "o_r": o_r, "lse_r": lse_r}
    out = {k: v.detach().numpy() for k, v in out.items()}
    for n in ("q_p", "k_p", "v_p", "q_r", "k_r", "v_r"):
        out["d" + n] = t[n].grad.numpy()
    return out


@pytest.mark.parametrize("wl", [-1, 3])
def test_grouped_reference_matches_packed_two_call_autograd(wl):
    # Three prompt groups, one of them without a prompt and one without responses:
    # every response must see only its own group's prompt, and each prompt's K/V
    # gradient must collect only its own group's terms.
    groups = [(5, [3, 4]), (0, [6]), (7, [2, 0, 5]), (4, [])]
    Hq, Hkv, d = 4, 2, 4
    xs, packed = workloads.make_group_inputs(groups, Hq, Hkv, d, "fp32", seed=31)
    ref = oracle.grouped_reference(xs, window_left=wl)
    two = _two_call_grouped(packed, wl, 1.0 / math.sqrt(d))
    for key in ("o_p", "lse_p", "o_r", "lse_r", "dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r"):
        np.testing.assert_allclose(ref[key], two[key], rtol=0, atol=1e-11, err_msg=key)
    # Sharing one prompt across all groups would change the answer.
    assert np.abs(ref["o_r"][:7] - oracle.ncopy_reference(
        dict(xs[0], q_r=packed["q_r"][:7], k_r=packed["k_r"][:7], v_r=packed["v_r"][:7],
             do_r=packed["do_r"][:7], cu=packed["cu"][:3]), window_left=wl, backward=False)["o_r"]).max() == 0
    assert np.abs(ref["o_r"][7:13] - oracle.ncopy_reference(
        dict(xs[0], q_r=packed["q_r"][7:13], k_r=packed["k_r"][7:13], v_r=packed["v_r"][7:13],
             do_r=packed["do_r"][7:13], cu=workloads.cu_seqlens([6])), window_left=wl, backward=False)["o_r"]).max() > 1e-3

"""Pins of the oracle's layout conversions (N-copy packing <-> single-prompt packing,
first-token predictor rows), on the CPU.

* closed forms written out by hand for a small micro-batch (rows hold their own index);
* adjoint identities: <unpack(x), y> == <x, unpack_bwd(y)> and
  <gather(h), g> == <h, scatter(g)> for random x, y, h, g -- the gradient maps are
  pinned to the forward maps, so a wrong index or a missing term fails;
* round trip pack(unpack(x)) == x;
* the attention oracle's own N-copy copies (eq. (1)) are unpack() of the packed Q/K/V,
  and unpack_bwd() of the copies' gradients gives the shared-prompt gradient sum of
  eq. (6) / App. A.5.
"""
import numpy as np
import pytest

import oracle
import workloads

GROUPS = [
    [(3, [2, 1])],
    [(4, [3, 0, 2]), (0, [2]), (2, []), (5, [1, 4])],
    [(0, [1, 1])],
]


def test_closed_forms_small_batch():
    groups = [(3, [2, 1]), (2, [2])]
    # packed rows: prompt A = 0,1,2; prompt B = 3,4; resp A0 = 5,6; A1 = 7; B0 = 8,9
    x = np.arange(10, dtype=np.float64).reshape(10, 1)
    nc = oracle.layout_unpack(x, groups)
    np.testing.assert_array_equal(nc[:, 0], [0, 1, 2, 5, 6, 0, 1, 2, 7, 3, 4, 8, 9])
    np.testing.assert_array_equal(oracle.layout_pack(nc, groups), x)
    pred = oracle.first_token_gather(x, groups)
    np.testing.assert_array_equal(pred[:, 0], [2, 5, 2, 4, 8])
    # scatter of ones: the last prompt row of A collects two first tokens, of B one;
    # every response row but the last of its response collects one.
    sc = oracle.first_token_scatter(np.ones((5, 1)), groups)
    np.testing.assert_array_equal(sc[:, 0], [0, 0, 2, 0, 1, 1, 0, 0, 1, 0])
    # unpack_bwd of ones: a prompt row counts its group's copies
    ub = oracle.layout_unpack_bwd(np.ones((13, 1)), groups)
    np.testing.assert_array_equal(ub[:, 0], [2, 2, 2, 1, 1, 1, 1, 1, 1, 1])


def _rows(groups):
    P = sum(p for p, _ in groups)
    T = sum(sum(ls) for _, ls in groups)
    nc = sum(p * len(ls) + sum(ls) for p, ls in groups)
    return P + T, nc, T


@pytest.mark.parametrize("groups", GROUPS)
def test_adjoint_identities(groups):
    packed, nc, T = _rows(groups)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((packed, 3, 2))
    y = rng.standard_normal((nc, 3, 2))
    lhs = float((oracle.layout_unpack(x, groups) * y).sum())
    rhs = float((x * oracle.layout_unpack_bwd(y, groups)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    h = rng.standard_normal((packed, 5))
    g = rng.standard_normal((T, 5))
    lhs = float((oracle.first_token_gather(h, groups) * g).sum())
    rhs = float((h * oracle.first_token_scatter(g, groups)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("groups", GROUPS)
def test_pack_inverts_unpack(groups):
    packed, nc, T = _rows(groups)
    x = np.random.default_rng(6).standard_normal((packed, 4))
    back = oracle.layout_pack(oracle.layout_unpack(x, groups), groups)
    # prompts of groups without responses are absent from the N-copy packing
    at = 0
    for P, lens in groups:
        if not lens:
            x[at:at + P] = 0.0
        at += P
    np.testing.assert_array_equal(back, x)


def test_unpack_matches_attention_copies_and_grad_sum():
    P, lens, Hq, Hkv, d = 6, [4, 0, 3], 2, 1, 4
    groups = [(P, lens)]
    x = workloads.make_inputs(P, lens, Hq, Hkv, d, "fp32", seed=12)
    for n in ("q", "k", "v"):
        packed = np.concatenate([x[n + "_p"].numpy(), x[n + "_r"].numpy()])
        nc = oracle.layout_unpack(packed, groups)
        expect = np.concatenate([oracle.copy_of(x, i)[("q", "k", "v").index(n)]
                                 for i in range(len(lens))])
        np.testing.assert_array_equal(nc, expect)
    do_copies = workloads.split_prompt_grad(x["do_p"], len(lens), seed=2)
    ref = oracle.ncopy_reference(x, do_copies=do_copies, keep_copies=True)
    for key in ("dk", "dv", "dq"):
        per_copy = np.concatenate([c[key] for c in ref["copies"]])
        summed = oracle.layout_unpack_bwd(per_copy, groups)
        np.testing.assert_allclose(summed[:P], ref[key + "_p"], rtol=0, atol=1e-12)
        np.testing.assert_array_equal(summed[P:], ref[key + "_r"])

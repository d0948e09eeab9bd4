"""GPU parity of the layout conversions (dkv_layout) against the oracle's
definitions: pure row moves (pack, unpack, first-token gather, and the zero rows) bit
for bit; the summing gradient maps (unpack_bwd, first-token scatter) within one
rounding of the float64 sum (fp32: 1e-5 absolute at unit-scale inputs; bf16: 2^-8 of
each element's magnitude, one bf16 rounding of an fp32 sum)."""
import numpy as np
import pytest
import torch

import oracle
import shared_prompt_exact_dkv_amd as dkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

GROUPS = [
    [(37, [20, 0, 65, 1])],
    [(4, [3, 0, 2]), (0, [2]), (2, []), (50, [1, 40, 17]), (1, [3])],
    [(0, [18, 1])],
]

OPS = {
    dkv.DKV_PACK: oracle.layout_pack,
    dkv.DKV_UNPACK: oracle.layout_unpack,
    dkv.DKV_UNPACK_BWD: oracle.layout_unpack_bwd,
    dkv.DKV_FIRST_TOKEN_GATHER: oracle.first_token_gather,
    dkv.DKV_FIRST_TOKEN_SCATTER: oracle.first_token_scatter,
}
SUMS = (dkv.DKV_UNPACK_BWD, dkv.DKV_FIRST_TOKEN_SCATTER)


def _arrays(groups):
    cu, ccu, scu = [0], [0], [0]
    for P, lens in groups:
        ccu.append(ccu[-1] + P)
        scu.append(scu[-1] + len(lens))
        for r in lens:
            cu.append(cu[-1] + r)
    return cu, ccu, scu


@pytest.mark.parametrize("gi", range(len(GROUPS)))
@pytest.mark.parametrize("op", sorted(OPS))
@pytest.mark.parametrize("dtype,tail", [("bf16", (4, 64)), ("fp32", (33, 4)), ("bf16", (8,))])
def test_layout_matches_oracle(gi, op, dtype, tail):
    groups = GROUPS[gi]
    cu, ccu, scu = _arrays(groups)
    rows_in, rows_out = dkv.layout_rows(op, cu, ccu[-1], ccu, scu)
    g = torch.Generator().manual_seed(100 * gi + op)
    x = torch.randn((rows_in,) + tail, generator=g, dtype=torch.float32)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    x = x.to(tdt)
    xd = x.to(DEV)
    out = torch.full((rows_out,) + tail, float("nan"), dtype=tdt, device=DEV)
    dkv.dkv_layout(op, xd, cu, ccu[-1], ctx_cu_host=ccu, group_seq_cu_host=scu, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = OPS[op](x.float().numpy().astype(np.float64), groups)
    assert got.shape == ref.shape
    if op in SUMS:
        bound = 1e-5 if dtype == "fp32" else 2.0 ** -8 * np.abs(ref) + 1e-30
        assert (np.abs(got - ref) <= bound).all(), float(np.abs(got - ref).max())
    else:
        np.testing.assert_array_equal(got, ref)


def test_one_prompt_without_groups_matches_groups():
    # The single-prompt call (no group arrays) equals one group spanning every response.
    cu, P = [0, 30, 30, 77], 45
    x = torch.randn((P * 3 + 77, 128), dtype=torch.float32).to(torch.bfloat16).to(DEV)
    a = dkv.dkv_layout(dkv.DKV_UNPACK_BWD, x, cu, P)
    b = dkv.dkv_layout(dkv.DKV_UNPACK_BWD, x, cu, P, ctx_cu_host=[0, P], group_seq_cu_host=[0, 3])
    torch.cuda.synchronize()
    assert torch.equal(a, b)

"""The C ABI library loads, exports every function include/dkv.h declares, and
rejects invalid arguments on the host (no GPU needed: validation runs before any
HIP call)."""
import ctypes

import pytest

from shared_prompt_exact_dkv_amd import _lib as L


def test_exports_every_header_function():
    names = L.header_functions()
    assert {"dkv_ctx_fwd", "dkv_fwd", "dkv_ctx_bwd", "dkv_bwd", "dkv_cast_acc",
            "dkv_workspace_size", "dkv_last_error"} <= set(names)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.dkv_version()


def _params(**kw):
    base = dict(num_seqs=2, ctx_len=16, num_heads_q=8, num_heads_kv=2, head_dim=128,
                window_left=-1, softmax_scale=0.0, dtype=L.DKV_BF16, cu_host=[0, 5, 9],
                cu_dev=0x1000)
    base.update(kw)
    return L.make_params(**base)


FAKE = 0x10000   # 16-byte aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status,frag", [
    (dict(num_heads_q=6, num_heads_kv=4), L.DKV_ERR_INVALID_ARG, "multiple"),
    (dict(head_dim=80), L.DKV_ERR_INVALID_ARG, "head_dim"),
    (dict(head_dim=320), L.DKV_ERR_INVALID_ARG, "head_dim"),
    (dict(head_dim=256, dtype=L.DKV_FP32), L.DKV_ERR_UNSUPPORTED, "fp16 only"),
    (dict(head_dim=192, dtype=L.DKV_FP32), L.DKV_ERR_UNSUPPORTED, "fp16 only"),
    (dict(window_left=-2), L.DKV_ERR_INVALID_ARG, "window_left"),
    (dict(cu_host=[1, 5, 9]), L.DKV_ERR_INVALID_ARG, "cu_seqlens[0]"),
    (dict(cu_host=[0, 5, 4]), L.DKV_ERR_INVALID_ARG, "decreases"),
    (dict(dtype=7), L.DKV_ERR_INVALID_ARG, "dtype"),
    (dict(ctx_len=-1), L.DKV_ERR_INVALID_ARG, "ctx_len"),
    (dict(kv_head_of_q=[0, 0, 0, 1, 1, 1, 1, 1]), L.DKV_ERR_INVALID_ARG, "kv head 0"),
    (dict(kv_head_of_q=[0, 0, 0, 0, 1, 1, 1, 2]), L.DKV_ERR_INVALID_ARG, "outside"),
    (dict(kv_head_of_q=[0, 0, 0, 0, 1, 1, 1, -1]), L.DKV_ERR_INVALID_ARG, "outside"),
    (dict(softmax_scale=float("nan")), L.DKV_ERR_INVALID_ARG, "scale"),
    (dict(head_dim=512, dtype=L.DKV_FP32), L.DKV_ERR_UNSUPPORTED, "fp16 only"),
    (dict(dtype=3), L.DKV_ERR_INVALID_ARG, "dtype"),
    (dict(head_dim=512, num_heads_q=64, num_heads_kv=1), L.DKV_ERR_UNSUPPORTED, "head_dim 512"),
])
def test_fwd_rejects_invalid_params(kw, status, frag):
    p, keep = _params(**kw)
    lib = L.lib()
    st = lib.dkv_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == status
    assert frag in L.last_error()


def test_cu_seqlens_dev_is_optional():
    # The kernels read sequence bounds staged from the host copy, so the device copy may
    # be absent; validation and sizing do not depend on it.
    lib = L.lib()
    p0, k0 = _params(cu_dev=0)
    p1, k1 = _params()
    for call in (L.DKV_CALL_FWD, L.DKV_CALL_BWD):
        assert lib.dkv_workspace_size(p0, call) == lib.dkv_workspace_size(p1, call)
    st = lib.dkv_fwd(p0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None)
    assert st == L.DKV_ERR_WORKSPACE


def test_head_map_validation_and_workspace():
    # A permuted GQA map (every kv head named by Hq / Hkv q-heads) is accepted and adds
    # its head table to the staged workspace; the contiguous map given explicitly is run
    # as no map.
    lib = L.lib()
    none, k0 = _params()
    contig, k1 = _params(kv_head_of_q=[h // 4 for h in range(8)])
    perm, k2 = _params(kv_head_of_q=[1, 0, 1, 0, 0, 1, 1, 0])
    for call in (L.DKV_CALL_CTX_FWD, L.DKV_CALL_FWD, L.DKV_CALL_BWD):
        p_ctx = call in (L.DKV_CALL_CTX_FWD,)
        if p_ctx:
            none, k0 = _params(ctx_len=0)
            contig, k1 = _params(ctx_len=0, kv_head_of_q=[h // 4 for h in range(8)])
            perm, k2 = _params(ctx_len=0, kv_head_of_q=[1, 0, 1, 0, 0, 1, 1, 0])
        a, b, c = (lib.dkv_workspace_size(p, call) for p in (none, contig, perm))
        assert a == b and c > a, (call, a, b, c)


def test_noalloc_backward_refuses_on_the_host():
    # The entry point without a workspace validates like dkv_bwd and refuses calls whose
    # scratch exceeds its 64 MiB array, before any device work (and before it looks up
    # the array's device address).
    lib = L.lib()
    args = [FAKE] * 13 + [0, FAKE, FAKE, None]
    bad, k0 = _params(head_dim=3)
    assert lib.dkv_bwd_noalloc(bad, *args) == L.DKV_ERR_INVALID_ARG
    assert "head_dim" in L.last_error()
    T = 200_000   # 64 q-heads: the -D and -LSE / scale rows alone need 102 MB
    big, k1 = _params(num_seqs=2, cu_host=[0, T // 2, T], num_heads_q=64, num_heads_kv=8)
    assert lib.dkv_workspace_size(big, L.DKV_CALL_BWD) > (64 << 20)
    assert lib.dkv_bwd_noalloc(big, *args) == L.DKV_ERR_UNSUPPORTED
    assert "64" in L.last_error() or str(64 << 20) in L.last_error()


def test_ctx_calls_require_zero_ctx_len():
    p, keep = _params(ctx_len=4)
    st = L.lib().dkv_ctx_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "ctx_len" in L.last_error()


def test_null_and_misaligned_pointers():
    p, keep = _params()
    lib = L.lib()
    st = lib.dkv_fwd(p, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "q_resp" in L.last_error()
    st = lib.dkv_fwd(p, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "aligned" in L.last_error()


def test_workspace_checks():
    p, keep = _params()
    lib = L.lib()
    need = lib.dkv_workspace_size(p, L.DKV_CALL_FWD)
    assert 0 < need < (1 << 20)
    st = lib.dkv_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == L.DKV_ERR_WORKSPACE
    st = lib.dkv_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, None)
    assert st == L.DKV_ERR_WORKSPACE and "aligned" in L.last_error()
    st = lib.dkv_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == L.DKV_ERR_WORKSPACE
    bad, keep2 = _params(head_dim=3)
    assert lib.dkv_workspace_size(bad, L.DKV_CALL_FWD) == ctypes.c_size_t(-1).value
    assert lib.dkv_workspace_size(p, 99) == ctypes.c_size_t(-1).value


def test_head_dim_512_workspace():
    # The d = 512 forward takes 128 query rows per workgroup, as at d = 128, so its
    # work list has the same length; its backward uses smaller tiles (32 dQ rows, 32
    # keys per workgroup), so those lists are longer than at d = 128.
    p128, k1 = _params(cu_host=[0, 300, 700], num_heads_q=16, num_heads_kv=4)
    p512, k2 = _params(cu_host=[0, 300, 700], num_heads_q=16, num_heads_kv=4, head_dim=512)
    lib = L.lib()
    a, b = lib.dkv_workspace_size(p128, L.DKV_CALL_FWD), lib.dkv_workspace_size(p512, L.DKV_CALL_FWD)
    assert 0 < a == b < (1 << 24)
    a, b = lib.dkv_workspace_size(p128, L.DKV_CALL_BWD), lib.dkv_workspace_size(p512, L.DKV_CALL_BWD)
    assert 0 < a < b < (1 << 24)


def test_empty_batch_is_a_no_op():
    p, keep = _params(cu_host=[0, 0, 0], cu_dev=0)
    lib = L.lib()
    assert lib.dkv_workspace_size(p, L.DKV_CALL_FWD) == 0
    assert lib.dkv_fwd(p, None, None, None, None, None, None, None, None, 0, None) == L.DKV_OK


def test_split_workspace_adds_the_slices():
    # N = 2 responses: one sequence per chunk in both modes, so the split workspace is
    # the plain one plus the dK and dV slices, 2 * S * P * Hkv * d fp32 with S = N.
    p, keep = _params()   # N = 2, P = 16, Hkv = 2, d = 128
    lib = L.lib()
    plain = lib.dkv_workspace_size(p, L.DKV_CALL_BWD)
    split = lib.dkv_workspace_size(p, L.DKV_CALL_BWD_SPLIT)
    assert split - plain == 2 * (2 * 16 * 2 * 128 * 4)
    # many responses: at most 8 slices
    cu = [0] + [5 * (i + 1) for i in range(20)]
    p20, k20 = _params(num_seqs=20, cu_host=cu)
    extra = lib.dkv_workspace_size(p20, L.DKV_CALL_BWD_SPLIT) - lib.dkv_workspace_size(
        p20, L.DKV_CALL_BWD)
    assert 0 < extra <= 2 * (8 * 16 * 2 * 128 * 4)


def test_split_flag_validation():
    p, keep = _params()
    lib = L.lib()
    plain = lib.dkv_workspace_size(p, L.DKV_CALL_BWD)
    F = FAKE
    # Call 1 takes DKV_ACC_SPLIT (one writer per element: no row chunks), so validation
    # passes it (here the call then fails at its first HIP call, without a GPU); an
    # unknown flag is refused before anything is enqueued
    pc, keepc = _params(ctx_len=0)
    st = lib.dkv_ctx_bwd(pc, F, F, F, F, F, F, F, F, F, F, F, L.DKV_ACC_SPLIT, F, 1 << 20, None)
    assert st != L.DKV_ERR_INVALID_ARG
    st = lib.dkv_ctx_bwd(pc, F, F, F, F, F, F, F, F, F, F, F, 8, F, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "DKV_ACC_SPLIT" in L.last_error()
    # a workspace sized for the atomic mode is too small for the slices
    st = lib.dkv_bwd(p, F, F, F, F, F, F, F, F, F, F, F, F, F, L.DKV_ACC_SPLIT, F, F, F, plain,
                     None)
    assert st == L.DKV_ERR_WORKSPACE
    st = lib.dkv_bwd(p, F, F, F, F, F, F, F, F, F, F, F, F, F, 8, F, F, F, plain, None)
    assert st == L.DKV_ERR_INVALID_ARG and "flags" in L.last_error()


def test_offset_range_limits():
    # The bf16 kernels address a sequence's rows with 32-bit byte offsets: a sequence
    # whose query rows pass 2^31 bytes is refused up front, and the largest that fits
    # is accepted.
    lib = L.lib()
    row = 32 * 128 * 2                        # Hq = 32, d = 128, bf16
    longest = (1 << 31) // row - 64 - 1
    ok, k1 = _params(num_seqs=1, ctx_len=16, num_heads_q=32, num_heads_kv=8,
                     cu_host=[0, longest])
    assert lib.dkv_workspace_size(ok, L.DKV_CALL_FWD) != ctypes.c_size_t(-1).value
    bad, k2 = _params(num_seqs=1, ctx_len=16, num_heads_q=32, num_heads_kv=8,
                      cu_host=[0, longest + 2])
    st = lib.dkv_fwd(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_UNSUPPORTED and "2^31" in L.last_error()
    # fp32 kernels use 64-bit row offsets: no such limit
    f32, k3 = _params(num_seqs=1, ctx_len=16, num_heads_q=32, num_heads_kv=8,
                      cu_host=[0, longest + 2], dtype=L.DKV_FP32)
    assert lib.dkv_workspace_size(f32, L.DKV_CALL_FWD) != ctypes.c_size_t(-1).value


@pytest.mark.parametrize("groups,frag", [
    (([0, 10, 17], [0, 1, 2]), "ctx_cu_host[num_groups]"),     # prompts sum to 17, P = 16
    (([0, 10, 16], [0, 1, 3]), "group_seq_cu_host[num_groups]"),
    (([0, 10, 8, 16], [0, 1, 1, 2]), "ctx_cu_host decreases"),
    (([0, 8, 16], [0, 2, 1, 2][:3]), "group_seq_cu_host decreases"),
    (([1, 8, 16], [0, 1, 2]), "must be 0"),
])
def test_prompt_groups_are_validated(groups, frag):
    p, keep = _params(ctx_cu_host=groups[0], group_seq_cu_host=groups[1])
    st = L.lib().dkv_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG
    assert frag in L.last_error()


def test_prompt_groups_only_for_the_response_call():
    p, keep = _params(ctx_len=0, ctx_cu_host=[0, 0], group_seq_cu_host=[0, 2])
    st = L.lib().dkv_ctx_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "num_groups" in L.last_error()


def test_prompt_groups_workspace_matches_one_group():
    # Groups that span every sequence with one prompt plan the same work as no groups;
    # splitting the prompt in two adds at most the second group's prompt-key tiles.
    lib = L.lib()
    p0, k0 = _params(num_seqs=3, cu_host=[0, 100, 300, 301], ctx_len=300)
    p1, k1 = _params(num_seqs=3, cu_host=[0, 100, 300, 301], ctx_len=300,
                     ctx_cu_host=[0, 300], group_seq_cu_host=[0, 3])
    p2, k2 = _params(num_seqs=3, cu_host=[0, 100, 300, 301], ctx_len=300,
                     ctx_cu_host=[0, 200, 300], group_seq_cu_host=[0, 2, 3])
    for call in (L.DKV_CALL_FWD, L.DKV_CALL_BWD, L.DKV_CALL_BWD_SPLIT):
        a, b, c = (lib.dkv_workspace_size(p, call) for p in (p0, p1, p2))
        assert a == b, call
        assert c != (1 << 64) - 1 and c > 0, call


def test_layout_validation():
    lib = L.lib()
    p, keep = _params()
    st = lib.dkv_layout(p, 7, 64, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "op" in L.last_error()
    st = lib.dkv_layout(p, L.DKV_PACK, 12, FAKE, FAKE, FAKE, 1 << 20, None)   # not 16-byte rows
    assert st == L.DKV_ERR_INVALID_ARG and "row_elems" in L.last_error()
    st = lib.dkv_layout(p, L.DKV_UNPACK, 64, FAKE, FAKE, FAKE, 0, None)
    assert st == L.DKV_ERR_WORKSPACE
    st = lib.dkv_layout(p, L.DKV_UNPACK, 64, None, FAKE, FAKE, 1 << 20, None)
    assert st == L.DKV_ERR_INVALID_ARG and "in" in L.last_error()
    # work lists: unpack of N = 2 copies of a 16-row prompt plus 9 response rows
    n = lib.dkv_layout_workspace_size(p, L.DKV_UNPACK)
    assert 0 < n < 4096


def test_binding_rejects_host_tensors():
    # The kernels dereference every pointer on the GPU: a host tensor's pointer would be
    # read as a device address.
    import torch
    import shared_prompt_exact_dkv_amd as dkv
    q = torch.zeros(12, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(12, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 5, 12], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        dkv.dkv_fwd(q, k[:8], k[:8], k, k, cu)
    with pytest.raises(ValueError, match="GPU tensor"):
        dkv.dkv_ctx_fwd(q, k, k, cu)
    with pytest.raises(ValueError, match="GPU tensor"):
        dkv.dkv_cast_acc(torch.zeros(8, 2, 64), torch.zeros(8, 2, 64), k[:8], k[:8])
    with pytest.raises(ValueError, match="GPU tensor"):
        dkv.dkv_layout(dkv.DKV_PACK, torch.zeros(12, 64, dtype=torch.bfloat16), [0, 4], 8)


def test_binding_checks_tensor_shapes(monkeypatch):
    # The C ABI takes plain pointers, so the binding checks shapes, dtypes, layout and
    # devices before any call: a short query tensor, a wrong output shape, a transposed
    # view or a tensor on another device would otherwise be read or written out of
    # bounds.  Without a GPU the checks run on CPU tensors (the call's device is taken to
    # be the CPU), and a meta tensor stands for a tensor on another device.
    import torch
    import shared_prompt_exact_dkv_amd as dkv
    monkeypatch.setattr(dkv, "_gpu", lambda t, name: t.device)
    P, T, Hq, Hkv, d = 8, 12, 4, 2, 64
    bf = torch.bfloat16
    q = torch.zeros(T, Hq, d, dtype=bf)
    k = torch.zeros(T, Hkv, d, dtype=bf)
    kp = torch.zeros(P, Hkv, d, dtype=bf)
    cu = torch.tensor([0, 5, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="q_r"):
        dkv.dkv_fwd(q[:10], kp, kp, k[:10], k[:10], cu)            # cu says 12 rows
    with pytest.raises(ValueError, match="out"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu, out=torch.zeros(T - 1, Hq, d, dtype=bf))
    with pytest.raises(ValueError, match="lse"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu, lse=torch.zeros(T, Hq))   # transposed layout
    with pytest.raises(ValueError, match="v_p"):
        dkv.dkv_fwd(q, kp, kp[:4], k, k, cu)
    with pytest.raises(ValueError, match="acc_dk_p"):
        dkv.dkv_bwd(q, kp, kp, k, k, q, torch.zeros(Hq, T), q, cu,
                    acc_dk_p=torch.zeros(P, Hkv, d, dtype=bf), acc_dv_p=None)
    with pytest.raises(ValueError, match="not contiguous"):
        dkv.dkv_ctx_fwd(q.transpose(0, 1).contiguous().transpose(0, 1), k, k, cu)
    # every tensor on the call's device
    with pytest.raises(ValueError, match="k_p is on meta"):
        dkv.dkv_fwd(q, kp.to("meta"), kp, k, k, cu)
    with pytest.raises(ValueError, match="dout_r is on meta"):
        dkv.dkv_bwd(q, kp, kp, k, k, q, torch.zeros(Hq, T), q.to("meta"), cu,
                    acc_dk_p=torch.zeros(P, Hkv, d), acc_dv_p=torch.zeros(P, Hkv, d))
    # cu_seqlens: int32 prefix sums, consistent with cu_host
    with pytest.raises(ValueError, match="int32"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu.long())
    with pytest.raises(ValueError, match="entries"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu, cu_host=[0, T])
    with pytest.raises(ValueError, match="disagree"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu, cu_host=[0, 6, T])
    with pytest.raises(ValueError, match="kv_head_of_q"):
        dkv.dkv_fwd(q, kp, kp, k, k, cu, kv_head_of_q=[0, 1, 0])
    # the standalone cast: outputs of the accumulator's shape and of one dtype
    acc = torch.zeros(P, Hkv, d)
    with pytest.raises(ValueError, match="dk"):
        dkv.dkv_cast_acc(acc, acc, kp[:4], kp)
    with pytest.raises(ValueError, match="dv"):
        dkv.dkv_cast_acc(acc, acc, kp, kp.half())
    with pytest.raises(ValueError, match="acc_dv"):
        dkv.dkv_cast_acc(acc, acc[:4], kp, kp)

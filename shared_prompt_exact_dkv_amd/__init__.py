"""DualKV shared-prompt attention for AMD MI355X (gfx950).

Thin torch binding of libdkv's C ABI (include/dkv.h).  The functions below only
marshal arguments: torch tensors supply device memory and the current stream, and
every step of the attention runs in libdkv's HIP kernels.

Method: "DualKV: Shared-Prompt Flash Attention for Efficient RL Training with Large
Rollouts and Long Contexts" (arXiv 2605.15422).  Call 1 (``dkv_ctx_fwd`` /
``dkv_ctx_bwd``) is causal self-attention over the single prompt copy, eq. (3);
Call 2 (``dkv_fwd`` / ``dkv_bwd``) is the shared-prompt attention of the responses,
eq. (4); the shared prompt K/V gradient is the sum of eq. (6).
"""
from __future__ import annotations

import math

import torch

from . import _lib as L
from ._lib import DKV_ACC_FINALIZE, DKV_ACC_SPLIT, DKV_ACC_ZERO, DkvError  # noqa: F401
from ._lib import (DKV_FIRST_TOKEN_GATHER, DKV_FIRST_TOKEN_SCATTER, DKV_PACK,  # noqa: F401
                   DKV_UNPACK, DKV_UNPACK_BWD)

__all__ = ["dkv_workspace_size", "dkv_ctx_fwd", "dkv_fwd", "dkv_ctx_bwd", "dkv_bwd",
           "dkv_bwd_noalloc",
           "dkv_cast_acc", "dkv_layout", "layout_rows", "dualkv_forward", "dualkv_backward",
           "DualKVAttention", "dualkv_attention",
           "DkvError", "DKV_ACC_ZERO", "DKV_ACC_FINALIZE", "DKV_ACC_SPLIT", "DKV_PACK",
           "DKV_UNPACK", "DKV_UNPACK_BWD", "DKV_FIRST_TOKEN_GATHER", "DKV_FIRST_TOKEN_SCATTER"]

_DT = {torch.bfloat16: L.DKV_BF16, torch.float32: L.DKV_FP32, torch.float16: L.DKV_FP16}


def _p(t):
    return None if t is None else t.data_ptr()


def _host_cu(cu_seqlens, cu_host):
    """The host copy of cu_seqlens, which the library validates and schedules from (the
    kernels read the bounds staged from it, never a device copy).  cu_seqlens must be an
    int32 tensor of N + 1 prefix sums; given alone it is read back (on a GPU tensor that
    waits for the device).  Given with cu_host it must agree in length, and, when it is
    on the CPU, in every value (a GPU tensor's values are not read back: the call would
    otherwise wait for the device)."""
    if cu_seqlens is None:
        if cu_host is None:
            raise ValueError("cu_seqlens or cu_host is required")
        return [int(c) for c in cu_host]
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D torch.int32 tensor")
    if cu_host is None:
        return [int(c) for c in cu_seqlens.cpu().tolist()]
    cu = [int(c) for c in cu_host]
    if cu_seqlens.numel() != len(cu):
        raise ValueError("cu_seqlens has %d entries, cu_host %d" % (cu_seqlens.numel(), len(cu)))
    if cu_seqlens.device.type == "cpu" and cu_seqlens.tolist() != cu:
        raise ValueError("cu_seqlens and cu_host disagree")
    return cu


def _params(q, k, cu_seqlens, cu_host, ctx_len, window_left, softmax_scale, groups=None,
            kv_head_of_q=None):
    if q.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % q.dtype)
    cu = _host_cu(cu_seqlens, cu_host)
    ctx_cu, seq_cu = groups if groups is not None else (None, None)
    if kv_head_of_q is not None:
        kv_head_of_q = [int(h) for h in kv_head_of_q]
        if len(kv_head_of_q) != q.shape[1]:
            raise ValueError("kv_head_of_q has %d entries for %d q-heads"
                             % (len(kv_head_of_q), q.shape[1]))
    return L.make_params(num_seqs=len(cu) - 1, ctx_len=ctx_len, num_heads_q=q.shape[1],
                         num_heads_kv=k.shape[1], head_dim=q.shape[2],
                         window_left=window_left, softmax_scale=softmax_scale,
                         dtype=_DT[q.dtype], cu_host=cu, ctx_cu_host=ctx_cu,
                         group_seq_cu_host=seq_cu, kv_head_of_q=kv_head_of_q)


def _groups(ctx_cu_host, group_seq_cu_host):
    """Prompt groups of a micro-batch: (ctx_cu_host, group_seq_cu_host) or None."""
    if ctx_cu_host is None and group_seq_cu_host is None:
        return None
    return [int(c) for c in ctx_cu_host], [int(c) for c in group_seq_cu_host]


def _need(t, shape, dtype, name, device=None):
    """The C ABI takes plain pointers: check here that a tensor has the shape, dtype,
    layout and device the call reads or writes through it (device: the first tensor's,
    which must be a GPU)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous %s tensor of shape %s, got %s %s%s"
                         % (name, dtype, tuple(shape), t.dtype, tuple(t.shape),
                            "" if t.is_contiguous() else " (not contiguous)"))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s; every tensor of the call must be on %s"
                         % (name, t.device, device))


def _gpu(t, name):
    """The device of a call: its first tensor's, which must be a GPU tensor."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (the kernels read device memory)" % name)
    return t.device


def _need_qkv(q, k, v, T, name):
    Hq, d = q.shape[1], q.shape[2]
    dev = _gpu(q, "q" + name)
    _need(q, (T, Hq, d), q.dtype, "q" + name, dev)
    _need(k, (T, k.shape[1], d), q.dtype, "k" + name, dev)
    _need(v, (T, k.shape[1], d), q.dtype, "v" + name, dev)
    return dev


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _ws(params, call, device, workspace):
    n = L.lib().dkv_workspace_size(params, call)
    if n == (1 << 64) - 1:
        L.check(L.DKV_ERR_INVALID_ARG)
    if n == 0:
        return None, 0
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on %s" % device)
        if workspace.numel() * workspace.element_size() >= n:
            return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(n, dtype=torch.uint8, device=device), n


def dkv_workspace_size(call: int, q, k, cu_seqlens, *, cu_host=None, ctx_len=0,
                       window_left=-1, softmax_scale=0.0, ctx_cu_host=None,
                       group_seq_cu_host=None, kv_head_of_q=None) -> int:
    p, keep = _params(q, k, cu_seqlens, cu_host, ctx_len, window_left, softmax_scale,
                      _groups(ctx_cu_host, group_seq_cu_host), kv_head_of_q)
    return int(L.lib().dkv_workspace_size(p, call))


def dkv_ctx_fwd(q, k, v, cu_seqlens, *, cu_host=None, window_left=-1, softmax_scale=0.0,
                out=None, lse=None, workspace=None, kv_head_of_q=None):
    """Causal self-attention of each sequence of ``cu_seqlens`` (Call 1, eq. (3)).
    q [T,Hq,d], k/v [T,Hkv,d] -> (o [T,Hq,d], lse [Hq,T] fp32).  kv_head_of_q: optional
    GQA map (q-head h reads kv head kv_head_of_q[h]; default h // (Hq / Hkv))."""
    p, keep = _params(q, k, cu_seqlens, cu_host, 0, window_left, softmax_scale,
                      kv_head_of_q=kv_head_of_q)
    T, Hq, _ = q.shape
    dev = _need_qkv(q, k, v, p.cu_seqlens_host[p.num_seqs], "")
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, q.shape, q.dtype, "out", dev)
    _need(lse, (Hq, T), torch.float32, "lse", dev)
    ws, nws = _ws(p, L.DKV_CALL_CTX_FWD, q.device, workspace)
    L.check(L.lib().dkv_ctx_fwd(p, _p(q), _p(k), _p(v), _p(o), _p(lse), _p(ws), nws,
                                _stream(q.device)))
    return o, lse


def dkv_fwd(q_resp, k_p, v_p, k_r, v_r, cu_seqlens, *, cu_host=None, window_left=-1,
            softmax_scale=0.0, out=None, lse=None, workspace=None, ctx_cu_host=None,
            group_seq_cu_host=None, kv_head_of_q=None):
    """Shared-prompt attention of the responses (Call 2, eq. (4)); P = k_p.shape[0].
    With prompt groups, group j's prompt is rows ctx_cu_host[j]..ctx_cu_host[j+1] of
    k_p/v_p, shared by sequences group_seq_cu_host[j]..group_seq_cu_host[j+1].
    kv_head_of_q as in dkv_ctx_fwd.  -> (o_r [T_R,Hq,d], lse_r [Hq,T_R] fp32)."""
    p, keep = _params(q_resp, k_r, cu_seqlens, cu_host, k_p.shape[0], window_left,
                      softmax_scale, _groups(ctx_cu_host, group_seq_cu_host), kv_head_of_q)
    T, Hq, _ = q_resp.shape
    dev = _need_qkv(q_resp, k_r, v_r, p.cu_seqlens_host[p.num_seqs], "_r")
    _need(k_p, (k_p.shape[0],) + tuple(k_r.shape[1:]), q_resp.dtype, "k_p", dev)
    _need(v_p, k_p.shape, q_resp.dtype, "v_p", dev)
    o = torch.empty_like(q_resp) if out is None else out
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q_resp.device) if lse is None else lse
    _need(o, q_resp.shape, q_resp.dtype, "out", dev)
    _need(lse, (Hq, T), torch.float32, "lse", dev)
    ws, nws = _ws(p, L.DKV_CALL_FWD, q_resp.device, workspace)
    L.check(L.lib().dkv_fwd(p, _p(q_resp), _p(k_p), _p(v_p), _p(k_r), _p(v_r), _p(o), _p(lse),
                            _p(ws), nws, _stream(q_resp.device)))
    return o, lse


def dkv_ctx_bwd(q, k, v, o, lse, dout, cu_seqlens, *, cu_host=None, window_left=-1,
                softmax_scale=0.0, dq=None, dk=None, dv=None, acc_dk=None, acc_dv=None,
                acc_flags=0, workspace=None, kv_head_of_q=None):
    """Backward of Call 1 (eq. (3)).  Without accumulators dk/dv are written directly;
    with acc_dk/acc_dv (fp32 [T,Hkv,d]) the key/value gradients are added into them
    (cleared first with DKV_ACC_ZERO, cast into dk/dv with DKV_ACC_FINALIZE).
    kv_head_of_q as in dkv_ctx_fwd.  -> (dq, dk, dv)."""
    p, keep = _params(q, k, cu_seqlens, cu_host, 0, window_left, softmax_scale,
                      kv_head_of_q=kv_head_of_q)
    dev = _need_qkv(q, k, v, p.cu_seqlens_host[p.num_seqs], "")
    _need(o, q.shape, q.dtype, "o", dev)
    _need(dout, q.shape, q.dtype, "dout", dev)
    _need(lse, (q.shape[1], q.shape[0]), torch.float32, "lse", dev)
    if (acc_dk is None) != (acc_dv is None):
        raise ValueError("acc_dk and acc_dv go together")
    dq = torch.empty_like(q) if dq is None else dq
    if acc_dk is None or (acc_flags & L.DKV_ACC_FINALIZE):
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
    _need(dq, q.shape, q.dtype, "dq", dev)
    _need(dk, k.shape, k.dtype, "dk", dev)
    _need(dv, k.shape, k.dtype, "dv", dev)
    _need(acc_dk, k.shape, torch.float32, "acc_dk", dev)
    _need(acc_dv, k.shape, torch.float32, "acc_dv", dev)
    ws, nws = _ws(p, L.DKV_CALL_CTX_BWD, q.device, workspace)
    L.check(L.lib().dkv_ctx_bwd(p, _p(q), _p(k), _p(v), _p(o), _p(lse), _p(dout), _p(dq),
                                _p(dk), _p(dv), _p(acc_dk), _p(acc_dv), int(acc_flags), _p(ws),
                                nws, _stream(q.device)))
    return dq, dk, dv


def dkv_bwd(q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, cu_seqlens, *, acc_dk_p, acc_dv_p,
            acc_flags=0, cu_host=None, window_left=-1, softmax_scale=0.0, dq_r=None, dk_r=None,
            dv_r=None, dk_p=None, dv_p=None, workspace=None, ctx_cu_host=None,
            group_seq_cu_host=None, kv_head_of_q=None, _noalloc=False):
    """Backward of Call 2 (eq. (4), §3.2).  Adds the responses' prompt-key gradients
    into acc_dk_p/acc_dv_p (fp32 [P,Hkv,d]); with DKV_ACC_FINALIZE also casts the
    accumulator into dk_p/dv_p; with DKV_ACC_SPLIT the terms reach the accumulator
    through per-chunk slices and a fixed-order sum instead of atomic adds.
    Prompt groups and kv_head_of_q as in dkv_fwd.  -> (dq_r, dk_r, dv_r, dk_p, dv_p)."""
    p, keep = _params(q_resp, k_r, cu_seqlens, cu_host, k_p.shape[0], window_left,
                      softmax_scale, _groups(ctx_cu_host, group_seq_cu_host), kv_head_of_q)
    dev = _need_qkv(q_resp, k_r, v_r, p.cu_seqlens_host[p.num_seqs], "_r")
    _need(k_p, (k_p.shape[0],) + tuple(k_r.shape[1:]), q_resp.dtype, "k_p", dev)
    _need(v_p, k_p.shape, q_resp.dtype, "v_p", dev)
    _need(o_r, q_resp.shape, q_resp.dtype, "o_r", dev)
    _need(dout_r, q_resp.shape, q_resp.dtype, "dout_r", dev)
    _need(lse_r, (q_resp.shape[1], q_resp.shape[0]), torch.float32, "lse_r", dev)
    _need(acc_dk_p, k_p.shape, torch.float32, "acc_dk_p", dev)
    _need(acc_dv_p, k_p.shape, torch.float32, "acc_dv_p", dev)
    dq_r = torch.empty_like(q_resp) if dq_r is None else dq_r
    dk_r = torch.empty_like(k_r) if dk_r is None else dk_r
    dv_r = torch.empty_like(v_r) if dv_r is None else dv_r
    if acc_flags & L.DKV_ACC_FINALIZE:
        dk_p = torch.empty_like(k_p) if dk_p is None else dk_p
        dv_p = torch.empty_like(v_p) if dv_p is None else dv_p
    _need(dq_r, q_resp.shape, q_resp.dtype, "dq_r", dev)
    _need(dk_r, k_r.shape, k_r.dtype, "dk_r", dev)
    _need(dv_r, k_r.shape, k_r.dtype, "dv_r", dev)
    _need(dk_p, k_p.shape, k_p.dtype, "dk_p", dev)
    _need(dv_p, k_p.shape, k_p.dtype, "dv_p", dev)
    if _noalloc:
        L.check(L.lib().dkv_bwd_noalloc(p, _p(q_resp), _p(k_p), _p(v_p), _p(k_r), _p(v_r),
                                        _p(o_r), _p(lse_r), _p(dout_r), _p(dq_r), _p(dk_r),
                                        _p(dv_r), _p(acc_dk_p), _p(acc_dv_p), int(acc_flags),
                                        _p(dk_p), _p(dv_p), _stream(q_resp.device)))
        return dq_r, dk_r, dv_r, dk_p, dv_p
    call = L.DKV_CALL_BWD_SPLIT if acc_flags & L.DKV_ACC_SPLIT else L.DKV_CALL_BWD
    ws, nws = _ws(p, call, q_resp.device, workspace)
    L.check(L.lib().dkv_bwd(p, _p(q_resp), _p(k_p), _p(v_p), _p(k_r), _p(v_r), _p(o_r),
                            _p(lse_r), _p(dout_r), _p(dq_r), _p(dk_r), _p(dv_r), _p(acc_dk_p),
                            _p(acc_dv_p), int(acc_flags), _p(dk_p), _p(dv_p), _p(ws), nws,
                            _stream(q_resp.device)))
    return dq_r, dk_r, dv_r, dk_p, dv_p


def dkv_bwd_noalloc(q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, cu_seqlens, *, acc_dk_p,
                    acc_dv_p, acc_flags=0, cu_host=None, window_left=-1, softmax_scale=0.0,
                    dq_r=None, dk_r=None, dv_r=None, dk_p=None, dv_p=None, ctx_cu_host=None,
                    group_seq_cu_host=None, kv_head_of_q=None):
    """dkv_bwd without a workspace (the library's own 64 MiB scratch array per GPU; see
    dkv_bwd_noalloc in include/dkv.h).  Pass every output tensor to avoid torch
    allocations here too.  Calls that overlap on one GPU race."""
    return dkv_bwd(q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, cu_seqlens,
                   acc_dk_p=acc_dk_p, acc_dv_p=acc_dv_p, acc_flags=acc_flags, cu_host=cu_host,
                   window_left=window_left, softmax_scale=softmax_scale, dq_r=dq_r, dk_r=dk_r,
                   dv_r=dv_r, dk_p=dk_p, dv_p=dv_p, ctx_cu_host=ctx_cu_host,
                   group_seq_cu_host=group_seq_cu_host, kv_head_of_q=kv_head_of_q,
                   _noalloc=True)




def dkv_cast_acc(acc_dk, acc_dv, dk, dv):
    """Cast the fp32 accumulators acc_dk/acc_dv [rows, Hkv, d] into dk/dv (same shape,
    bf16 / fp16 / fp32), once."""
    dev = _gpu(acc_dk, "acc_dk")
    if acc_dk.dim() != 3:
        raise ValueError("acc_dk must be [rows, Hkv, d]")
    if dk is None or dv is None or dk.dtype not in _DT:
        raise ValueError("dk and dv must be bf16, fp16 or fp32 tensors")
    _need(acc_dk, acc_dk.shape, torch.float32, "acc_dk", dev)
    _need(acc_dv, acc_dk.shape, torch.float32, "acc_dv", dev)
    _need(dk, acc_dk.shape, dk.dtype, "dk", dev)
    _need(dv, acc_dk.shape, dk.dtype, "dv", dev)
    rows, Hkv, d = acc_dk.shape
    p, keep = L.make_params(num_seqs=0, ctx_len=0, num_heads_q=Hkv, num_heads_kv=Hkv,
                            head_dim=d, dtype=_DT[dk.dtype], cu_host=[0])
    L.check(L.lib().dkv_cast_acc(p, rows, _p(acc_dk), _p(acc_dv), _p(dk), _p(dv),
                                 _stream(dk.device)))
    return dk, dv


def layout_rows(op: int, cu_host, ctx_len: int, ctx_cu_host=None, group_seq_cu_host=None):
    """(input rows, output rows) of a layout op for these sequences and groups."""
    cu = [int(c) for c in cu_host]
    N, T = len(cu) - 1, cu[-1]
    if ctx_cu_host is None:
        plen = [ctx_len] * N
    else:
        plen = [0] * N
        for j in range(len(ctx_cu_host) - 1):
            for i in range(group_seq_cu_host[j], group_seq_cu_host[j + 1]):
                plen[i] = ctx_cu_host[j + 1] - ctx_cu_host[j]
    ncopy = sum(plen) + T
    packed = ctx_len + T
    return {L.DKV_PACK: (ncopy, packed), L.DKV_UNPACK: (packed, ncopy),
            L.DKV_UNPACK_BWD: (ncopy, packed), L.DKV_FIRST_TOKEN_GATHER: (packed, T),
            L.DKV_FIRST_TOKEN_SCATTER: (T, packed)}[op]


def dkv_layout(op: int, x, cu_host, ctx_len: int, *, ctx_cu_host=None, group_seq_cu_host=None,
               out=None, workspace=None):
    """Move per-token rows between the N-copy and the single-prompt packing, or form /
    scatter the first-token predictor rows (see dkv_layout_op in include/dkv.h).
    x [rows_in, ...] (bf16 or fp32, contiguous); returns out [rows_out, ...]."""
    if x.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % x.dtype)
    rows_in, rows_out = layout_rows(op, cu_host, ctx_len, ctx_cu_host, group_seq_cu_host)
    if x.shape[0] != rows_in:
        raise ValueError("layout op %d expects %d input rows, got %d" % (op, rows_in, x.shape[0]))
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    dev = _gpu(x, "x")
    if out is not None and out.device != dev:
        raise ValueError("out is on %s; x is on %s" % (out.device, dev))
    row_elems = math.prod(x.shape[1:])
    if out is not None and (tuple(out.shape) != (rows_out,) + tuple(x.shape[1:])
                            or out.dtype != x.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous %s tensor of shape %s"
                         % (x.dtype, (rows_out,) + tuple(x.shape[1:])))
    cu = [int(c) for c in cu_host]
    p, keep = L.make_params(num_seqs=len(cu) - 1, ctx_len=ctx_len, num_heads_q=1,
                            num_heads_kv=1, head_dim=64, dtype=_DT[x.dtype], cu_host=cu,
                            ctx_cu_host=ctx_cu_host, group_seq_cu_host=group_seq_cu_host)
    out = torch.empty((rows_out,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device) \
        if out is None else out
    n = L.lib().dkv_layout_workspace_size(p, op)
    if n == (1 << 64) - 1:
        L.check(L.DKV_ERR_INVALID_ARG)
    ws, nws = (None, 0) if n == 0 else (
        (workspace, workspace.numel()) if workspace is not None and workspace.numel() >= n
        else (torch.empty(n, dtype=torch.uint8, device=x.device), n))
    L.check(L.lib().dkv_layout(p, op, row_elems, _p(x), _p(out), _p(ws), nws,
                               _stream(x.device)))
    return out


def _prompt_cu(P, ctx_cu_host):
    """Sequence bounds of Call 1 over the prompt(s), as a host list only: the library
    schedules from the host copy, so no device tensor (and no copy to the device, which
    a stream capturing a graph would refuse) is made."""
    return [0, P] if ctx_cu_host is None else [int(c) for c in ctx_cu_host]


def dualkv_forward(q_p, k_p, v_p, q_r, k_r, v_r, cu_seqlens, *, cu_host=None, window_left=-1,
                   softmax_scale=0.0, ctx_cu_host=None, group_seq_cu_host=None,
                   kv_head_of_q=None):
    """The two calls of the forward: Call 1 over the prompt(s), Call 2 over the
    responses.  With prompt groups (see dkv_fwd), Call 1 is varlen causal attention
    over the prompts.  -> (o_p, lse_p, o_r, lse_r)."""
    cu_p_host = _prompt_cu(q_p.shape[0], ctx_cu_host)
    o_p, lse_p = dkv_ctx_fwd(q_p, k_p, v_p, None, cu_host=cu_p_host, window_left=window_left,
                             softmax_scale=softmax_scale, kv_head_of_q=kv_head_of_q)
    o_r, lse_r = dkv_fwd(q_r, k_p, v_p, k_r, v_r, cu_seqlens, cu_host=cu_host,
                         window_left=window_left, softmax_scale=softmax_scale,
                         ctx_cu_host=ctx_cu_host, group_seq_cu_host=group_seq_cu_host,
                         kv_head_of_q=kv_head_of_q)
    return o_p, lse_p, o_r, lse_r


def dualkv_backward(q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r, do_p, do_r,
                    cu_seqlens, *, cu_host=None, window_left=-1, softmax_scale=0.0,
                    acc=None, split=False, ctx_cu_host=None, group_seq_cu_host=None,
                    kv_head_of_q=None):
    """The two calls of the backward sharing one fp32 accumulator for dK_P/dV_P
    (eq. (6)): Call 1 clears it and adds the prompt self-attention term, Call 2 adds
    the N responses' terms and casts once (split=True: Call 1 with one writer per
    element, Call 2 through per-chunk slices and a fixed-order sum, bitwise
    reproducible).  -> dict of dq_p, dk_p, dv_p, dq_r, dk_r, dv_r."""
    if acc is None:
        acc = torch.empty((2,) + tuple(k_p.shape), dtype=torch.float32, device=k_p.device)
    cu_p_host = _prompt_cu(q_p.shape[0], ctx_cu_host)
    dq_p, _, _ = dkv_ctx_bwd(q_p, k_p, v_p, o_p, lse_p, do_p, None, cu_host=cu_p_host,
                             window_left=window_left, softmax_scale=softmax_scale,
                             acc_dk=acc[0], acc_dv=acc[1],
                             acc_flags=DKV_ACC_ZERO | (DKV_ACC_SPLIT if split else 0),
                             kv_head_of_q=kv_head_of_q)
    dq_r, dk_r, dv_r, dk_p, dv_p = dkv_bwd(q_r, k_p, v_p, k_r, v_r, o_r, lse_r, do_r,
                                           cu_seqlens, acc_dk_p=acc[0], acc_dv_p=acc[1],
                                           acc_flags=DKV_ACC_FINALIZE | (DKV_ACC_SPLIT if split else 0),
                                           cu_host=cu_host,
                                           window_left=window_left,
                                           softmax_scale=softmax_scale,
                                           ctx_cu_host=ctx_cu_host,
                                           group_seq_cu_host=group_seq_cu_host,
                                           kv_head_of_q=kv_head_of_q)
    return {"dq_p": dq_p, "dk_p": dk_p, "dv_p": dv_p, "dq_r": dq_r, "dk_r": dk_r, "dv_r": dv_r}


class DualKVAttention(torch.autograd.Function):
    """torch autograd over the two calls: the forward is dualkv_forward, the backward
    dualkv_backward, so the prompt keys' gradient of eq. (6) (the Call-1 term plus every
    response's Call-2 term) is summed in the library's fp32 accumulator and cast once.
    Differentiable inputs: q_p, k_p, v_p, q_r, k_r, v_r; outputs (o_p, o_r).  The LSEs
    are kept for the backward; an output the loss does not use gets a zero gradient."""

    @staticmethod
    def forward(ctx, q_p, k_p, v_p, q_r, k_r, v_r, cu_seqlens, opts):
        o_p, lse_p, o_r, lse_r = dualkv_forward(
            q_p, k_p, v_p, q_r, k_r, v_r, cu_seqlens, cu_host=opts["cu_host"],
            window_left=opts["window_left"], softmax_scale=opts["softmax_scale"],
            ctx_cu_host=opts["ctx_cu_host"], group_seq_cu_host=opts["group_seq_cu_host"],
            kv_head_of_q=opts["kv_head_of_q"])
        ctx.save_for_backward(q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r)
        ctx.cu_seqlens = cu_seqlens
        ctx.opts = opts
        return o_p, o_r

    @staticmethod
    def backward(ctx, do_p, do_r):
        q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r = ctx.saved_tensors
        do_p = torch.zeros_like(o_p) if do_p is None else do_p.contiguous()
        do_r = torch.zeros_like(o_r) if do_r is None else do_r.contiguous()
        o = ctx.opts
        g = dualkv_backward(q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r, do_p, do_r,
                            ctx.cu_seqlens, cu_host=o["cu_host"], window_left=o["window_left"],
                            softmax_scale=o["softmax_scale"], split=o["split"],
                            ctx_cu_host=o["ctx_cu_host"],
                            group_seq_cu_host=o["group_seq_cu_host"],
                            kv_head_of_q=o["kv_head_of_q"])
        return (g["dq_p"], g["dk_p"], g["dv_p"], g["dq_r"], g["dk_r"], g["dv_r"], None, None)


def dualkv_attention(q_p, k_p, v_p, q_r, k_r, v_r, cu_seqlens, *, cu_host=None, window_left=-1,
                     softmax_scale=0.0, split=False, ctx_cu_host=None, group_seq_cu_host=None,
                     kv_head_of_q=None):
    """DualKV attention as one differentiable op (DualKVAttention): -> (o_p, o_r).
    split=True makes the backward's prompt-key gradient bitwise reproducible."""
    opts = {"cu_host": cu_host, "window_left": window_left, "softmax_scale": softmax_scale,
            "split": split, "ctx_cu_host": ctx_cu_host, "group_seq_cu_host": group_seq_cu_host,
            "kv_head_of_q": kv_head_of_q}
    return DualKVAttention.apply(q_p, k_p, v_p, q_r, k_r, v_r, cu_seqlens, opts)

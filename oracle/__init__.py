"""CPU oracle for DualKV shared-prompt attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP path (``shared_prompt_exact_dkv_amd``) and never imports it.

The oracle is the plain definition the method must reproduce exactly: causal
attention of every sequence of the N-copy packing, "DualKV: Shared-Prompt Flash
Attention ..." (arXiv 2605.15422) §2.1, eqs. (1)-(2).  Sequence i of that packing is
the prompt followed by response i, ``[P, R_i]``, so its Q/K/V are the prompt rows
concatenated with response i's rows.  ``dkv_oracle.c`` computes one such sequence
in double precision; this module builds the copies, runs them, and maps the results
onto the single-prompt layout of §2.2 (eq. 5):

* O_P, LSE_P   -> copy 1's prompt rows (all copies agree, Appendix A.2)
* O_R, LSE_R   -> each copy's response rows
* dQ_R, dK_R, dV_R -> each copy's response rows
* dQ_P, dK_P, dV_P -> the sum over copies of the prompt rows' gradients (eq. (6) and
  Appendix A.5: the shared prompt receives every copy's contribution)

Each copy's prompt rows get their own upstream gradient dO_P^(i); the single
prompt copy of the DualKV packing receives their sum (Appendix A.5).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dkv_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile the C oracle into oracle/liboracle.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        common = [ctypes.c_int] * 4 + [_ip, ctypes.c_int, ctypes.c_double]
        lib.oracle_fwd_rows.argtypes = common + [_dp, _dp, _dp, ctypes.c_int, _ip, _dp, _dp]
        lib.oracle_bwd_rows.argtypes = common + [_dp, _dp, _dp, _dp, ctypes.c_int, _ip,
                                                 _dp, _dp, _dp]
        lib.oracle_bwd_keys.argtypes = common + [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                                 _ip, _dp, _dp]
        lib.oracle_bwd_scatter.argtypes = common + [_dp, _dp, ctypes.c_int, _ip, _dp, _dp,
                                                    _dp, _dp, _dp]
        lib.oracle_fwd_sel.argtypes = common + [_dp, _dp, ctypes.c_int, _ip, _dp, _dp, _dp]
        for f in (lib.oracle_fwd_rows, lib.oracle_bwd_rows, lib.oracle_bwd_keys,
                  lib.oracle_bwd_scatter, lib.oracle_fwd_sel):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def use_library(path=None):
    """Load the oracle from ``path`` (default: oracle/liboracle.so).  Tests use this
    to run the pins against deliberately broken builds of dkv_oracle.c."""
    global _lib, _SO
    _lib = None
    _SO = os.path.join(_HERE, "liboracle.so") if path is None else path
    return _load()


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu().to(dtype=torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _kvh(Hq: int, Hkv: int, kvh=None) -> np.ndarray:
    if kvh is None:
        G = Hq // Hkv
        kvh = [h // G for h in range(Hq)]
    return _i32(kvh)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def seq_fwd(q, k, v, *, scale=None, window_left=-1, kvh=None, rows=None):
    """Eq. (2) for one sequence. q [S,Hq,d], k/v [S,Hkv,d] -> (o [n,Hq,d], lse [n,Hq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    kv = _kvh(Hq, Hkv, kvh)
    sel = _i32(np.arange(S) if rows is None else rows)
    o = np.zeros((len(sel), Hq, d))
    lse = np.zeros((len(sel), Hq))
    if S == 0 or len(sel) == 0:
        return o, lse
    rc = _load().oracle_fwd_rows(S, Hq, Hkv, d, _ptr(kv, _ip), int(window_left), scale,
                                 _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), len(sel),
                                 _ptr(sel, _ip), _ptr(o, _dp), _ptr(lse, _dp))
    if rc != 0:
        raise ValueError("oracle_fwd_rows failed (%d)" % rc)
    return o, lse


def seq_bwd(q, k, v, dout, *, scale=None, window_left=-1, kvh=None, rows=None,
            keys=None, need_keys=True):
    """Gradients of eq. (2) for one sequence with upstream gradient ``dout``.

    Returns dict with dq [len(rows),Hq,d], lse/delta [len(rows),Hq] for the
    selected query positions, and dk/dv [len(keys),Hkv,d] for the selected key
    positions.  Key gradients need every row's lse and delta, so the row pass
    covers all positions whenever keys are requested.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    kv = _kvh(Hq, Hkv, kvh)
    lib = _load()
    all_rows = _i32(np.arange(S))
    rsel = all_rows if (rows is None or need_keys) else _i32(rows)
    dq = np.zeros((len(rsel), Hq, d))
    lse = np.zeros((len(rsel), Hq))
    delta = np.zeros((len(rsel), Hq))
    if S > 0 and len(rsel) > 0:
        rc = lib.oracle_bwd_rows(S, Hq, Hkv, d, _ptr(kv, _ip), int(window_left), scale,
                                 _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(dout, _dp),
                                 len(rsel), _ptr(rsel, _ip), _ptr(dq, _dp), _ptr(lse, _dp),
                                 _ptr(delta, _dp))
        if rc != 0:
            raise ValueError("oracle_bwd_rows failed (%d)" % rc)
    out = {}
    if rows is not None and need_keys:
        r = np.asarray(rows, dtype=np.int64)
        out.update(dq=dq[r], lse=lse[r], delta=delta[r])
    else:
        out.update(dq=dq, lse=lse, delta=delta)
    if need_keys:
        ksel = all_rows if keys is None else _i32(keys)
        dk = np.zeros((len(ksel), Hkv, d))
        dv = np.zeros((len(ksel), Hkv, d))
        if S > 0 and len(ksel) > 0:
            rc = lib.oracle_bwd_keys(S, Hq, Hkv, d, _ptr(kv, _ip), int(window_left), scale,
                                     _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp),
                                     _ptr(dout, _dp), _ptr(lse, _dp), _ptr(delta, _dp),
                                     len(ksel), _ptr(ksel, _ip), _ptr(dk, _dp),
                                     _ptr(dv, _dp))
            if rc != 0:
                raise ValueError("oracle_bwd_keys failed (%d)" % rc)
        out.update(dk=dk, dv=dv)
    return out


def copy_of(x: dict, i: int):
    """Sequence i of the N-copy packing (eq. 1): prompt rows then response i's rows."""
    cu = [int(c) for c in x["cu"]]
    a, b = cu[i], cu[i + 1]
    cat = lambda p, r: np.concatenate([_f64(p), _f64(r)[a:b]], 0)
    return cat(x["q_p"], x["q_r"]), cat(x["k_p"], x["k_r"]), cat(x["v_p"], x["v_r"])


def ncopy_reference(x: dict, *, do_copies=None, scale=None, window_left=-1, kvh=None,
                    backward=True, keep_copies=False) -> dict:
    """Expected single-prompt-layout outputs from the N-copy definition.

    ``x`` holds q_p,k_p,v_p,q_r,k_r,v_r,cu (and do_r when ``backward``).
    ``do_copies`` is [N,P,Hq,d]: copy i's prompt-row upstream gradient; when absent
    every copy receives do_p / N (so that the single prompt copy sees do_p).
    Returns o_p [P,Hq,d], lse_p [P,Hq], o_r [T,Hq,d], lse_r [T,Hq] and, with
    ``backward``, dq_p, dk_p, dv_p, dq_r, dk_r, dv_r.
    """
    cu = [int(c) for c in x["cu"]]
    N = len(cu) - 1
    q_p = _f64(x["q_p"])
    P, Hq, d = q_p.shape
    Hkv = _f64(x["k_p"]).shape[1]
    T = cu[-1]
    res = {
        "o_p": np.zeros((P, Hq, d)), "lse_p": np.zeros((P, Hq)),
        "o_r": np.zeros((T, Hq, d)), "lse_r": np.zeros((T, Hq)),
    }
    if backward:
        if do_copies is None:
            do_copies = np.broadcast_to(_f64(x["do_p"]) / N, (N, P, Hq, d))
        do_copies = _f64(do_copies)
        do_r = _f64(x["do_r"])
        for key, shape in (("dq_p", (P, Hq, d)), ("dk_p", (P, Hkv, d)), ("dv_p", (P, Hkv, d)),
                           ("dq_r", (T, Hq, d)), ("dk_r", (T, Hkv, d)), ("dv_r", (T, Hkv, d))):
            res[key] = np.zeros(shape)
    copies = []
    for i in range(N):
        a, b = cu[i], cu[i + 1]
        qi, ki, vi = copy_of(x, i)
        o, lse = seq_fwd(qi, ki, vi, scale=scale, window_left=window_left, kvh=kvh)
        if i == 0:
            res["o_p"][:] = o[:P]
            res["lse_p"][:] = lse[:P]
        res["o_r"][a:b] = o[P:]
        res["lse_r"][a:b] = lse[P:]
        rec = {"o": o, "lse": lse}
        if backward:
            doi = np.concatenate([do_copies[i], do_r[a:b]], 0)
            g = seq_bwd(qi, ki, vi, doi, scale=scale, window_left=window_left, kvh=kvh)
            res["dq_p"] += g["dq"][:P]
            res["dk_p"] += g["dk"][:P]
            res["dv_p"] += g["dv"][:P]
            res["dq_r"][a:b] = g["dq"][P:]
            res["dk_r"][a:b] = g["dk"][P:]
            res["dv_r"][a:b] = g["dv"][P:]
            rec.update(g)
        if keep_copies:
            copies.append(rec)
    if keep_copies:
        res["copies"] = copies
    return res


def grouped_reference(xs, *, do_copies=None, scale=None, window_left=-1, kvh=None,
                      backward=True) -> dict:
    """Expected outputs for a micro-batch of several prompt groups, packed group after
    group (prompt rows of group 1, 2, ...; response rows of group 1, 2, ...).

    Each group is its own instance of the method -- its own prompt, shared by its own
    responses only ("Data pipeline" of §2.2: groups are processed independently, each
    with its own context KV and cu_seqlens) -- so each is ncopy_reference() of that
    group's inputs ``xs[j]`` (``do_copies[j]`` its per-copy prompt gradients), and the
    results are concatenated in the packed order.  A group without responses still
    has its prompt rows: they are the one sequence [P, 0] (eq. (3) alone).
    """
    parts = []
    for j, x in enumerate(xs):
        if len(x["cu"]) == 1:
            x = dict(x, cu=np.zeros(2, dtype=np.int32))
        parts.append(ncopy_reference(x, do_copies=None if do_copies is None else do_copies[j],
                                     scale=scale, window_left=window_left, kvh=kvh,
                                     backward=backward))
    return {key: np.concatenate([r[key] for r in parts], 0) for key in parts[0]}


def rows_fwd(k, v, rows, q_rows, *, scale=None, window_left=-1, kvh=None):
    """Eq. (2) at selected positions ``rows`` of one sequence whose keys / values are
    ``k`` / ``v`` [S, Hkv, d]; ``q_rows`` [n, Hq, d] are those rows' queries.
    -> (o [n, Hq, d], lse [n, Hq])."""
    k, v, qs = _f64(k), _f64(v), _f64(q_rows)
    S, Hkv, d = k.shape
    Hq = qs.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    kv = _kvh(Hq, Hkv, kvh)
    sel = _i32(rows)
    o = np.zeros((len(sel), Hq, d))
    lse = np.zeros((len(sel), Hq))
    if len(sel):
        rc = _load().oracle_fwd_sel(S, Hq, Hkv, d, _ptr(kv, _ip), int(window_left), scale,
                                    _ptr(k, _dp), _ptr(v, _dp), len(sel), _ptr(sel, _ip),
                                    _ptr(qs, _dp), _ptr(o, _dp), _ptr(lse, _dp))
        if rc != 0:
            raise ValueError("oracle_fwd_sel failed (%d)" % rc)
    return o, lse


def rows_bwd_scatter(k, v, rows, q_rows, dout_rows, dk, dv, *, scale=None, window_left=-1,
                     kvh=None):
    """Gradients of eq. (2) for one sequence whose upstream gradient is zero except at
    positions ``rows`` (queries ``q_rows``, gradients ``dout_rows``, [n, Hq, d]).
    Adds the key / value gradients into ``dk`` / ``dv`` (float64 [S, Hkv, d], modified
    in place) and returns dq [n, Hq, d] for those rows (every other row's dq is 0)."""
    k, v = _f64(k), _f64(v)
    qs, ds = _f64(q_rows), _f64(dout_rows)
    S, Hkv, d = k.shape
    Hq = qs.shape[1]
    assert dk.dtype == np.float64 and dk.flags.c_contiguous and dk.shape == k.shape
    assert dv.dtype == np.float64 and dv.flags.c_contiguous and dv.shape == k.shape
    scale = default_scale(d) if scale is None else float(scale)
    kv = _kvh(Hq, Hkv, kvh)
    sel = _i32(rows)
    dq = np.zeros((len(sel), Hq, d))
    if len(sel):
        rc = _load().oracle_bwd_scatter(S, Hq, Hkv, d, _ptr(kv, _ip), int(window_left), scale,
                                        _ptr(k, _dp), _ptr(v, _dp), len(sel), _ptr(sel, _ip),
                                        _ptr(qs, _dp), _ptr(ds, _dp), _ptr(dq, _dp),
                                        _ptr(dk, _dp), _ptr(dv, _dp))
        if rc != 0:
            raise ValueError("oracle_bwd_scatter failed (%d)" % rc)
    return dq



# ---------------------------------------------------------------------------
# Layout conversions between the two packings (§2.1 eq. (1), §2.2 eq. (5), §2.3,
# App. A.2 / A.3 / A.5).  ``groups`` is [(P_j, [R_i of group j])]; tensors are
# [rows, ...] with any trailing shape.  The N-copy packing holds, sequence after
# sequence, the sequence's prompt then its response; the single-prompt packing holds
# every prompt once, in group order, then every response.


def _split_packed(x, groups):
    x = np.asarray(x)
    prompts, resps, at = [], [], 0
    for P, _ in groups:
        prompts.append(x[at:at + P])
        at += P
    for _, lens in groups:
        rs = []
        for R in lens:
            rs.append(x[at:at + R])
            at += R
        resps.append(rs)
    assert at == x.shape[0]
    return prompts, resps


def _split_ncopy(x, groups):
    x = np.asarray(x)
    copies, at = [], 0
    for P, lens in groups:
        cs = []
        for R in lens:
            cs.append((x[at:at + P], x[at + P:at + P + R]))
            at += P + R
        copies.append(cs)
    assert at == x.shape[0]
    return copies


def layout_pack(x_ncopy, groups):
    """N-copy -> single-prompt packing: each prompt from its group's first copy (every
    copy holds the same prompt rows, App. A.2); zeros for a prompt without copies."""
    copies = _split_ncopy(x_ncopy, groups)
    x = np.asarray(x_ncopy)
    prompts = [cs[0][0] if cs else np.zeros((P,) + x.shape[1:], x.dtype)
               for (P, _), cs in zip(groups, copies)]
    resps = [r for cs in copies for _, r in cs]
    return np.concatenate(prompts + resps, 0)


def layout_unpack(x_packed, groups):
    """Single-prompt -> N-copy packing: every sequence gets its group's prompt rows
    followed by its own rows (eq. (1))."""
    prompts, resps = _split_packed(x_packed, groups)
    x = np.asarray(x_packed)
    parts = [z for p, rs in zip(prompts, resps) for r in rs for z in (p, r)]
    return np.concatenate(parts, 0) if parts else np.zeros((0,) + x.shape[1:], x.dtype)


def layout_unpack_bwd(g_ncopy, groups):
    """Gradient of layout_unpack: a prompt row collects the sum of its group's copies'
    gradients (App. A.5), in float64; response rows are passed through."""
    copies = _split_ncopy(g_ncopy, groups)
    g = _f64(g_ncopy)
    prompts = []
    for (P, _), cs in zip(groups, copies):
        acc = np.zeros((P,) + g.shape[1:])
        for p, _ in cs:
            acc += _f64(p)
        prompts.append(acc)
    resps = [_f64(r) for cs in copies for _, r in cs]
    return np.concatenate(prompts + resps, 0)


def first_token_gather(h_packed, groups):
    """The hidden state that predicts each response token: for token r > 0 of a
    response its row r - 1, for r = 0 the last row of its group's prompt (§2.3);
    zeros when the prompt is empty.  [T_R, ...]."""
    prompts, resps = _split_packed(h_packed, groups)
    h = np.asarray(h_packed)
    out = []
    for p, rs in zip(prompts, resps):
        for r in rs:
            if r.shape[0] == 0:
                continue
            first = p[-1:] if p.shape[0] else np.zeros((1,) + h.shape[1:], h.dtype)
            out += [first, r[:-1]]
    return np.concatenate(out, 0) if out else np.zeros((0,) + h.shape[1:], h.dtype)


def first_token_scatter(g_pred, groups):
    """Gradient of first_token_gather, in float64: the last prompt row of a group gets
    the sum of its responses' first-token gradients, response row r the gradient of
    token r + 1, every other row zero.  [sum P_j + T_R, ...]."""
    g = _f64(g_pred)
    tail = g.shape[1:]
    prompts, resps, at = [], [], 0
    for P, lens in groups:
        pg = np.zeros((P,) + tail)
        for R in lens:
            seg = g[at:at + R]
            at += R
            if R == 0:
                resps.append(seg)
                continue
            if P > 0:
                pg[P - 1] += seg[0]
            resps.append(np.concatenate([seg[1:], np.zeros((1,) + tail)], 0))
        prompts.append(pg)
    assert at == g.shape[0]
    return np.concatenate(prompts + resps, 0)

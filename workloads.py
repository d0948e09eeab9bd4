"""Seeded synthetic workloads for DualKV shared-prompt attention.

This module only draws inputs.  It holds none of the attention arithmetic, so both
the CPU oracle (``oracle/``) and the HIP path may use it without sharing method code.

Shapes follow the workloads in "DualKV: Shared-Prompt Flash Attention for Efficient
RL Training with Large Rollouts and Long Contexts" (arXiv 2605.15422): Qwen3-8B
attention dimensions (H=32 query heads, 8 KV heads, d=128, §4.1 / Table 1),
GRPO/DAPO rollout sizes (§4.2), and the Gemma-4 head-dim-512 global and head-dim-256
sliding-window layers (§3 "Head dimensions and sliding-window support").  No
dataset is read: every tensor is drawn from a seeded CPU generator.

Single-prompt packing (§2.2, eq. 5): the prompt is stored once as rows [0, P) and
response i occupies rows P + cu[i] ... P + cu[i+1] - 1.  Tensors are token-major
``[tokens, heads, d]``.  The HIP path receives the prompt and response parts as
separate tensors (q_p/k_p/v_p and q_r/k_r/v_r).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    P: int                      # shared prompt tokens
    N: int                      # responses
    R: Optional[int]            # fixed response length (None -> drawn)
    R_range: Optional[tuple]    # (lo, hi) inclusive when drawn uniformly
    Hq: int
    Hkv: int
    d: int
    dtype: str                  # "fp32", "bf16" or "fp16"
    window_left: int = -1       # -1 = global causal
    seed: int = 0
    scaled: bool = True         # values ~ N(0,1)/sqrt(d) (else N(0,1))
    groups: int = 1             # prompt groups in the micro-batch, N responses each
    P_range: Optional[tuple] = None   # (lo, hi) inclusive: per-group prompt lengths drawn

    def resp_lens(self) -> list:
        if self.R is not None:
            return [self.R] * self.N
        g = torch.Generator().manual_seed(10_000 + self.seed)
        lo, hi = self.R_range
        return torch.randint(lo, hi + 1, (self.N,), generator=g).tolist()

    def group_shapes(self) -> list:
        """[(P_j, response lengths of group j)] of the micro-batch's prompt groups."""
        if self.groups == 1 and self.P_range is None:
            return [(self.P, self.resp_lens())]
        g = torch.Generator().manual_seed(30_000 + self.seed)
        out = []
        for _ in range(self.groups):
            P = self.P if self.P_range is None else \
                int(torch.randint(self.P_range[0], self.P_range[1] + 1, (1,), generator=g))
            if self.R is not None:
                lens = [self.R] * self.N
            else:
                lens = torch.randint(self.R_range[0], self.R_range[1] + 1, (self.N,),
                                     generator=g).tolist()
            out.append((P, lens))
        return out


# The five workloads (the d=512 "layer pair" is two layers: global and windowed).
# Sliding window (1024) is read as 1024 visible keys including the query itself,
# i.e. window_left = 1023.
WORKLOADS = {
    "tiny": Workload("tiny", P=64, N=4, R=32, R_range=None, Hq=2, Hkv=2, d=64,
                     dtype="fp32", seed=1, scaled=False),
    "qwen3_8b": Workload("qwen3_8b", P=4096, N=32, R=4096, R_range=None, Hq=32, Hkv=8,
                         d=128, dtype="bf16", seed=2),
    "dapo_varlen": Workload("dapo_varlen", P=8192, N=16, R=None, R_range=(512, 4096),
                            Hq=32, Hkv=8, d=128, dtype="bf16", seed=3),
    "large_rollout": Workload("large_rollout", P=16384, N=64, R=1024, R_range=None,
                              Hq=32, Hkv=8, d=128, dtype="bf16", seed=4),
    "d512_global": Workload("d512_global", P=57344, N=8, R=8192, R_range=None, Hq=16,
                            Hkv=4, d=512, dtype="bf16", seed=5),
    "d512_swa": Workload("d512_swa", P=57344, N=8, R=8192, R_range=None, Hq=16, Hkv=4,
                         d=512, dtype="bf16", window_left=1023, seed=6),
    # The sliding-window layers of the same hybrid model run at head dim 256 (§3 "Head
    # dimensions and sliding-window support"): the d = 512 pair's shape and window at
    # d = 256.
    "d256_swa": Workload("d256_swa", P=57344, N=8, R=8192, R_range=None, Hq=16, Hkv=4,
                         d=256, dtype="bf16", window_left=1023, seed=15),
    # Head dims 96 and 192 (App. E.1 "Numerical correctness" checks d in {64, 96, 128, 192,
    # 256}; the pages time neither): the Qwen3-8B-shaped micro-batch at those head dims,
    # timing the d = 96 path (rows staged 128 wide) and the d = 192 pair kernels (rows
    # staged 256 wide).
    "hd96": Workload("hd96", P=4096, N=32, R=4096, R_range=None, Hq=32, Hkv=8, d=96,
                     dtype="bf16", seed=16),
    "hd192": Workload("hd192", P=4096, N=32, R=4096, R_range=None, Hq=32, Hkv=8, d=192,
                      dtype="bf16", seed=17),
    # The shapes of the paper's kernel benchmark (§4.1, Table 1): Qwen3-8B attention
    # dimensions, R = 2048 per response, fp16, global causal.
    "table1_p4k": Workload("table1_p4k", P=4096, N=28, R=2048, R_range=None, Hq=32, Hkv=8,
                           d=128, dtype="fp16", seed=11),
    "table1_p16k": Workload("table1_p16k", P=16384, N=28, R=2048, R_range=None, Hq=32,
                            Hkv=8, d=128, dtype="fp16", seed=12),
    "table1_p32k": Workload("table1_p32k", P=32768, N=16, R=2048, R_range=None, Hq=32,
                            Hkv=8, d=128, dtype="fp16", seed=13),
    "table1_p64k": Workload("table1_p64k", P=65536, N=16, R=2048, R_range=None, Hq=32,
                            Hkv=8, d=128, dtype="fp16", seed=14),
    # A GRPO micro-batch holding several prompts (§2.2 "Data pipeline"): 4 prompt
    # groups of 8 responses, prompts U{2048..8192} and responses U{512..2048} tokens
    # (the LongReason setting of §4.2 caps prompts at 8192 and responses at 2048).
    "multi_group": Workload("multi_group", P=0, N=8, R=None, R_range=(512, 2048), Hq=32,
                            Hkv=8, d=128, dtype="bf16", seed=7, groups=4,
                            P_range=(2048, 8192)),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[name]


def cu_seqlens(lens) -> torch.Tensor:
    cu = [0]
    for r in lens:
        cu.append(cu[-1] + int(r))
    return torch.tensor(cu, dtype=torch.int32)


def _draw(g: torch.Generator, shape, dtype: str, scale: float, keep: bool = False) -> torch.Tensor:
    """Values exactly representable in ``dtype``: fp32 tensors, or (``keep``) tensors
    already in ``dtype``."""
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=g.device) * scale
    if dtype in ("bf16", "fp16"):
        x = x.to(torch_dtype(dtype))
        if not keep:
            x = x.to(torch.float32)
    return x


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch_dtype(dtype)).to(torch.float32) if dtype in ("bf16", "fp16") else x


def add_key_ramp(x: dict, P: int, lens, d: int, dtype: str, rise: float, seed: int,
                 key_span: float = 3.0) -> dict:
    """Logits that climb along the key axis (for inputs of make_inputs on the CPU).

    A seeded unit vector u is added to every key at logical position pos (prompt row j:
    j; row r of a response: P + r) as key_span * pos / L * u, L the longest logical
    position, and to every query row as a * u, with a chosen so that a query's logit
    climbs by ``rise`` log2 units from key position 0 to L: a * key_span / sqrt(d) *
    log2(e) = rise.  The queries carry the large component and the keys only a small,
    slowly growing one, so the softmax weight spreads over a row's latest keys (about
    L / rise positions per halving) instead of one key, and keys share no large common
    component: the backward stays well conditioned.  Values are rounded to ``dtype``
    again, so both sides of a comparison see the same numbers.
    """
    g = torch.Generator().manual_seed(90_000 + seed)
    u = torch.randn(d, generator=g, dtype=torch.float64)
    u = (u / u.norm()).to(torch.float32)
    L = max(1, P + max([int(r) for r in lens] + [0]) - 1)
    a = rise * math.sqrt(d) / (key_span * math.log2(math.e))
    c = key_span / L
    out = dict(x)
    for name in ("q_p", "q_r"):
        out[name] = _round(x[name] + a * u, dtype)
    out["k_p"] = _round(x["k_p"] + (c * torch.arange(P, dtype=torch.float32)).view(-1, 1, 1) * u,
                        dtype)
    pos = torch.cat([torch.arange(int(r), dtype=torch.float32) + P for r in lens]) \
        if len(lens) else torch.zeros(0)
    out["k_r"] = _round(x["k_r"] + (c * pos).view(-1, 1, 1) * u, dtype)
    return out


def make_inputs(P: int, lens, Hq: int, Hkv: int, d: int, dtype: str = "fp32",
                seed: int = 0, scaled: bool = False, dout: bool = True,
                device: str = "cpu") -> dict:
    """Single-prompt packed inputs (fp32 tensors holding ``dtype``-exact values; on a
    non-CPU ``device`` the tensors are drawn there and kept in ``dtype``).

    Returns q_p [P,Hq,d], k_p/v_p [P,Hkv,d], q_r [T,Hq,d], k_r/v_r [T,Hkv,d],
    do_p [P,Hq,d] (the prompt-row upstream gradient seen by the single prompt
    copy), do_r [T,Hq,d] and cu (int32 [N+1]).
    """
    g = torch.Generator(device=device).manual_seed(seed)
    keep = device != "cpu"
    T = int(sum(lens))
    s = 1.0 / math.sqrt(d) if scaled else 1.0
    out = {
        "q_p": _draw(g, (P, Hq, d), dtype, s, keep),
        "k_p": _draw(g, (P, Hkv, d), dtype, s, keep),
        "v_p": _draw(g, (P, Hkv, d), dtype, s, keep),
        "q_r": _draw(g, (T, Hq, d), dtype, s, keep),
        "k_r": _draw(g, (T, Hkv, d), dtype, s, keep),
        "v_r": _draw(g, (T, Hkv, d), dtype, s, keep),
        "cu": cu_seqlens(lens),
    }
    if dout:
        out["do_p"] = _draw(g, (P, Hq, d), dtype, 1.0, keep)
        out["do_r"] = _draw(g, (T, Hq, d), dtype, 1.0, keep)
    return out


def make_group_inputs(groups, Hq: int, Hkv: int, d: int, dtype: str = "fp32", seed: int = 0,
                      scaled: bool = False, dout: bool = True, device: str = "cpu") -> tuple:
    """A micro-batch of several prompt groups: ``groups`` is a list of (P_j, lens_j).

    Group j's tensors are drawn by make_inputs with seed ``seed + j``.  Returns
    (per-group input dicts, packed dict): the packed dict concatenates the groups'
    prompt rows (q_p, k_p, v_p, do_p) and response rows (q_r, k_r, v_r, do_r) in group
    order, with cu (int32 [N+1] over all responses), ctx_cu (prefix sums of the P_j)
    and seq_cu (prefix sums of the groups' response counts).
    """
    xs = [make_inputs(P, lens, Hq, Hkv, d, dtype, seed=seed + j, scaled=scaled, dout=dout,
                      device=device)
          for j, (P, lens) in enumerate(groups)]
    names = ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r"] + (["do_p", "do_r"] if dout else [])
    packed = {n: torch.cat([x[n] for x in xs], 0) for n in names}
    all_lens = [int(r) for _, lens in groups for r in lens]
    packed["cu"] = cu_seqlens(all_lens)
    packed["ctx_cu"] = cu_seqlens([P for P, _ in groups])
    packed["seq_cu"] = cu_seqlens([len(lens) for _, lens in groups])
    return xs, packed


def split_prompt_grad(do_p: torch.Tensor, N: int, seed: int) -> torch.Tensor:
    """Per-copy prompt-row upstream gradients dO_P^(i), i = 1..N, in float64.

    In the N-copy packing each copy's prompt rows receive their own upstream
    gradient; in the single-prompt packing the one prompt copy receives their sum
    (the paper's Appendix A.5: the residual stream aggregates the N branches).
    dO_P^(i) = do_p / N + e_i, where the e_i are multiples of 1/256 that sum to
    exactly zero, so sum_i dO_P^(i) equals do_p to within float64 rounding.
    """
    g = torch.Generator().manual_seed(20_000 + seed)
    base = do_p.to(torch.float64) / N
    if N == 1:
        return base.unsqueeze(0).clone()
    e = torch.randint(-64, 65, (N - 1,) + tuple(do_p.shape), generator=g).to(torch.float64) / 256.0
    last = -e.sum(0)
    parts = torch.cat([e, last.unsqueeze(0)], 0) + base.unsqueeze(0)
    return parts


def workload_inputs(w: Workload, dout: bool = True, device: str = "cpu") -> dict:
    lens = w.resp_lens()
    x = make_inputs(w.P, lens, w.Hq, w.Hkv, w.d, w.dtype, seed=w.seed, scaled=w.scaled,
                    dout=dout, device=device)
    x["lens"] = lens
    return x

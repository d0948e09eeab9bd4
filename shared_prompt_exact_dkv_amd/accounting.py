"""Work accounting for DualKV attention: visible (query, key) pairs and useful FLOPs.

A "pair" is one visible (query row, key) pair of one query head.  Causal attention
over L tokens with a left window w (key j visible from t iff t - w <= j <= t) has
C(L) = sum_{t<L} (min(t, w) + 1) pairs per head; C(L) = L(L+1)/2 when global.

* N-copy packing (paper §2.1, eq. (2)): sum_i C(P + R_i).
* DualKV (§2.2): Call 1 over the prompt, C(P), plus Call 2, whose response rows sit
  at logical positions P .. P+R_i-1, i.e. sum_i (C(P + R_i) - C(P)).

Their ratio is the ideal attention speedup of Appendix C.2 (arXiv Eq. 34) up to the
paper's continuous approximation.  Useful FLOPs count only visible pairs: 4*d per
pair for the forward (Q K^T and P V) and 10*d for the backward (five products).
"""
from __future__ import annotations


def causal_pairs(L: int, window_left: int = -1) -> int:
    if L <= 0:
        return 0
    if window_left < 0 or L <= window_left + 1:
        return L * (L + 1) // 2
    w = window_left
    return (w + 1) * (w + 2) // 2 + (L - w - 1) * (w + 1)


def pairs_call1(P: int, window_left: int = -1) -> int:
    return causal_pairs(P, window_left)


def pairs_call2(P: int, lens, window_left: int = -1) -> int:
    c = causal_pairs(P, window_left)
    return sum(causal_pairs(P + int(r), window_left) - c for r in lens)


def pairs_dualkv(P: int, lens, window_left: int = -1) -> int:
    return pairs_call1(P, window_left) + pairs_call2(P, lens, window_left)


def pairs_ncopy(P: int, lens, window_left: int = -1) -> int:
    return sum(causal_pairs(P + int(r), window_left) for r in lens)


def ideal_speedup(P: int, lens, window_left: int = -1) -> float:
    return pairs_ncopy(P, lens, window_left) / pairs_dualkv(P, lens, window_left)


FWD_FLOPS_PER_PAIR_PER_DIM = 4
BWD_FLOPS_PER_PAIR_PER_DIM = 10


def useful_flops(pairs: int, Hq: int, d: int, fwd: bool = True, bwd: bool = True) -> int:
    per = (FWD_FLOPS_PER_PAIR_PER_DIM if fwd else 0) + (BWD_FLOPS_PER_PAIR_PER_DIM if bwd else 0)
    return per * d * Hq * pairs


def token_reduction(P: int, N: int, R: int) -> float:
    """rho = N(P+R) / (P+NR), paper §2.2 and Appendix C.3."""
    return N * (P + R) / (P + N * R)


def prompt_bytes_saved(N: int, P: int, H: int, Hk: int, d: int, elem: int = 2) -> dict:
    """Appendix C.1 Table 6: tensors an N-copy call holds N-1 extra copies of."""
    kv = 2 * (N - 1) * P * Hk * d * elem
    q = (N - 1) * P * H * d * elem
    lse = (N - 1) * P * H * 4
    return {"kv_shared": kv, "q_prompt": q, "lse_prompt": lse, "total": kv + q + lse}

"""Host-side accounting for one MoE layer call: FLOPs, bytes, padding, skew.

These are the quantities the AI-infra book (ch. 9) uses to reason about the
expert layer, written as functions so the benchmark can report them and the
tests can pin them to the book's worked numbers:

* expert size P_e = 3*h*I parameters (section 9.3.2: 3 x 4096 x 1536);
* useful expert FLOPs F_e(m) = 2*m*P_e (section 9.3.2 equations);
* expected number of distinct active experts E[U] = E*(1-(1-K/E)^M)
  (section 9.3.3; the second "E" of the printed formula is the expert count);
* rows a grouped GEMM executes when every expert is padded to a tile
  (section 9.4.3, local counts [32,16,8,4,2,1,1,0]);
* expert skew s = max_j m_j / (n*k/R) (section 9.4.2 equations);
* rows on the card that holds a hot expert (section 9.4.1);
* replica-aware load: rows per card when hot experts have replicas that
  share their assignments, and when a replica's copy cost is paid back
  (section 9.4.2, Example 9.6: N_min = floor(T_copy / dt) + 1).
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np


def expert_params(H: int, I: int) -> int:
    """Parameters of one SwiGLU expert: gate [I,H], up [I,H], down [H,I]."""
    return 3 * H * I


def expert_bytes(H: int, I: int, bytes_per_weight: float, with_channel_scales: bool = False) -> int:
    """Weight bytes of one expert; fp8 experts add one fp32 scale per output channel (2I + H)."""
    b = int(expert_params(H, I) * bytes_per_weight)
    if with_channel_scales:
        b += 4 * (2 * I + H)
    return b


def useful_flops(assignments: int, H: int, I: int) -> int:
    """2 * m * P_e summed over assignments (no padding)."""
    return 2 * assignments * expert_params(H, I)


def router_flops(T: int, H: int, E: int) -> int:
    return 2 * T * H * E


def expected_active_experts(E: int, K: int, M: int) -> float:
    """E[U] = E * (1 - (1 - K/E)^M) for M tokens each picking K of E experts uniformly."""
    return E * (1.0 - (1.0 - K / E) ** M)


def padded_rows(counts: Sequence[int], tile: int) -> int:
    """Rows executed when each non-empty expert is padded up to a multiple of ``tile``."""
    return int(sum(-(-int(c) // tile) * tile for c in counts if c > 0))


def split_padded_rows(counts: Sequence[int], max_tile: int, align: int) -> int:
    """Rows executed when an expert's c rows are cut into ceil(c/max_tile) equal tiles, each rounded
    up to a multiple of ``align`` (the large-batch bf16 grouped GEMM: max_tile 256, align 64)."""
    total = 0
    for c in counts:
        c = int(c)
        if c <= 0:
            continue
        m = -(-c // max_tile)
        per = -(-c // m)
        total += m * min(max_tile, -(-per // align) * align)
    return total


def padded_rows_to_max(counts: Sequence[int]) -> int:
    """Rows executed when every expert (empty ones included) is padded to the largest count."""
    return int(len(counts) * max(int(c) for c in counts))


def skew(counts: Sequence[int], n: int, k: int, groups: int) -> float:
    """s_expert = max_j m_j / (n*k/R) for R groups (cards) with loads m_j."""
    return max(counts) / (n * k / groups)


def group_loads(expert_loads: Sequence[float], groups: int) -> np.ndarray:
    """Loads of ``groups`` cards when experts are split into equal contiguous id ranges."""
    a = np.asarray(expert_loads, dtype=np.float64)
    return a.reshape(groups, -1).sum(axis=1)


def hot_expert_card_rows(n: int, k: int, E: int, hot_rows: float, groups: int) -> float:
    """Rows on the card holding one hot expert with ``hot_rows`` rows when the other
    n*k - hot_rows rows spread evenly over the remaining E - 1 experts."""
    rest = (n * k - hot_rows) / (E - 1)
    per_card = E // groups
    return hot_rows + (per_card - 1) * rest


def replica_card_rows(counts: Sequence[int], placement: Sequence[Sequence[int]]) -> np.ndarray:
    """Rows each card multiplies when the assignments of an expert are split evenly over its
    replicas.  ``placement[c]`` lists the experts card c holds (an expert on several cards has
    that many replicas); an expert's m rows go m // r to each of its r replicas, the remainder
    one row each to its first replicas in card order.  Every expert with rows must be placed."""
    counts = [int(c) for c in counts]
    holders = {}
    for c, experts in enumerate(placement):
        for e in experts:
            holders.setdefault(int(e), []).append(c)
    rows = np.zeros(len(placement), dtype=np.int64)
    for e, m in enumerate(counts):
        if m == 0:
            continue
        cards = holders.get(e)
        if not cards:
            raise ValueError(f"expert {e} has {m} rows but no card holds it")
        q, rem = divmod(m, len(cards))
        for i, c in enumerate(cards):
            rows[c] += q + (1 if i < rem else 0)
    return rows


def replica_break_even(t_copy: float, dt: float) -> int:
    """Smallest number of batches N with N * dt > t_copy: floor(t_copy / dt) + 1."""
    return int(math.floor(t_copy / dt)) + 1


def replica_net_saving(batches: int, t_copy: float, dt: float) -> float:
    """Time saved by a replica over ``batches`` batches after paying its copy once."""
    return batches * dt - t_copy


def replica_memory_bytes(expert_bytes_: int, layers: int, replicas_per_layer: int = 1) -> int:
    """HBM one card gives up for ``replicas_per_layer`` extra experts in each of ``layers`` layers."""
    return expert_bytes_ * layers * replicas_per_layer


def layer_hbm_bytes(counts: Iterable[int], T: int, H: int, I: int, E: int, act_bytes: int,
                    w_bytes_per_expert: int, router_w_bytes: int, y_bytes: int = 4) -> int:
    """Algorithmic HBM bytes of one layer call: the weights of every active expert
    once, the router weight, x read once, y written once (index arrays are ignored)."""
    active = sum(1 for c in counts if c > 0)
    return active * w_bytes_per_expert + router_w_bytes + T * H * act_bytes + T * H * y_bytes


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def gib(nbytes: float) -> float:
    return nbytes / float(1 << 30)


def mib(nbytes: float) -> float:
    return nbytes / float(1 << 20)


def isclose(a: float, b: float, rel: float) -> bool:
    return math.isclose(a, b, rel_tol=rel)

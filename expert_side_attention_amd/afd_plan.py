"""Attention:FFN pool planning from measured stage times (host side, not on
the kernel path).

Rules restated from the pages:
* Rate matching: the two pools should finish a step at the same rate, so
  that neither waits for the other; a higher attention cost needs more
  attention GPUs, a higher FFN cost more expert GPUs (AFD Disagg MoE notes
  page, case 2 on capacity alignment).  Here that principle is applied
  directly: with per-step costs t_a and t_f spread evenly over a pool, the
  step period is the slower pool's, max(t_a / n_a, t_f / n_f), and n_a is the
  integer in [1, N - 1] that minimises it (both pools must exist for the
  layer to run).  Among splits with the same period the one nearest the
  proportional share N t_a / (t_a + t_f) is taken, then the smaller n_a.
* Micro-pipeline: with attention and FFN on separate pools the steady period
  is the longer stage plus the hand-over, max(t_a, t_f) + t_comm, against
  t_a + t_f when both run on the same GPUs (A/F 分离 page, 深入推导, 微流水).
* Rank layout: FFN ranks come first; the attention rank count must be at
  least the FFN rank count and a whole multiple of it (vLLM AFD plugin page
  in Spanish, "Con qué te vas a tropezar": 64A16F is legal, 16A64F and 64A24F
  are not).
* Traffic: dispatch plus combine move factor * h * k * bytes_per_elem * 2
  bytes per token per layer, factor = 2 as the A/F page prints it (深入推导,
  通信账).
"""
from __future__ import annotations

import json


def step_period(attn_cost: float, ffn_cost: float, n_attn: int, n_ffn: int) -> float:
    """Per-step period of two pools that each spread their stage evenly."""
    return max(attn_cost / n_attn, ffn_cost / n_ffn)


def split_gpus(attn_cost: float, ffn_cost: float, total_gpus: int):
    """(attention GPUs, FFN GPUs) for stage costs measured in the same unit:
    the split with the shortest step period (see the module notes)."""
    if total_gpus < 2:
        raise ValueError("need at least one GPU per pool")
    if attn_cost < 0 or ffn_cost < 0 or attn_cost + ffn_cost <= 0:
        raise ValueError("costs must be non-negative and not both zero")
    share = total_gpus * attn_cost / (attn_cost + ffn_cost)

    def rank(n):
        return (step_period(attn_cost, ffn_cost, n, total_gpus - n), abs(n - share), n)

    n_attn = min(range(1, total_gpus), key=rank)
    return n_attn, total_gpus - n_attn


def check_rank_counts(num_attention_ranks: int, num_ffn_ranks: int) -> None:
    """Raise ValueError unless the plugin's rank rule holds."""
    a, f = num_attention_ranks, num_ffn_ranks
    if f < 1 or a < 1:
        raise ValueError("each role needs at least one rank")
    if a < f:
        raise ValueError(f"{a}A{f}F: attention ranks must not be fewer than FFN ranks")
    if a % f:
        raise ValueError(f"{a}A{f}F: attention ranks must be a multiple of FFN ranks")


def rank_roles(num_attention_ranks: int, num_ffn_ranks: int):
    """Role of each global rank: FFN ranks first, then attention ranks."""
    check_rank_counts(num_attention_ranks, num_ffn_ranks)
    return ["ffn"] * num_ffn_ranks + ["attention"] * num_attention_ranks


def pipeline_period(t_a: float, t_f: float, t_comm: float = 0.0):
    """Steady per-step period co-located vs disaggregated, same time unit."""
    colocated = t_a + t_f
    disaggregated = max(t_a, t_f) + t_comm
    return {"colocated": colocated, "disaggregated": disaggregated,
            "gain": colocated / disaggregated if disaggregated > 0 else float("inf")}


def comm_bytes_per_token_layer(h: int, k: int, bytes_per_elem: int = 1, factor: int = 2) -> int:
    """Dispatch + combine bytes per token per layer as the A/F page counts them."""
    return factor * h * k * bytes_per_elem * 2


def ffn_step_ms(bench_json_path: str) -> float:
    """Measured FFN layer time per step (ms) from a bench.py JSON line file."""
    with open(bench_json_path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                return float(json.loads(line)["ms_per_step"])
    raise ValueError(f"no bench line in {bench_json_path}")

"""Attention:FFN planning helpers against the rules and examples the pages
state (CPU)."""
import os

import pytest

from expert_side_attention_amd import afd_plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rank_rule_examples_from_plugin_page():
    P.check_rank_counts(64, 16)          # 64A16F: legal
    with pytest.raises(ValueError):
        P.check_rank_counts(16, 64)      # fewer attention than FFN ranks
    with pytest.raises(ValueError):
        P.check_rank_counts(64, 24)      # not a multiple
    P.check_rank_counts(1, 1)            # the one-host example: 1 + 1
    assert P.rank_roles(4, 2) == ["ffn", "ffn", "attention", "attention", "attention",
                                  "attention"]


def test_split_follows_cost_share():
    assert P.split_gpus(1.0, 1.0, 16) == (8, 8)
    assert P.split_gpus(3.0, 1.0, 16) == (12, 4)
    # attention is at least one GPU and FFN keeps at least one
    assert P.split_gpus(0.0, 5.0, 8) == (1, 7)
    assert P.split_gpus(5.0, 0.0, 8) == (7, 1)
    # a cost ratio of 1:63 over 128 GPUs gives the 2A+126F shape the notes
    # page mentions for DeepSeek-V3.2
    assert P.split_gpus(1.0, 63.0, 128) == (2, 126)
    # ties go to the even count: share 0.5 of 5 GPUs -> 2.5 -> 2
    assert P.split_gpus(1.0, 1.0, 5) == (2, 3)
    for a, f, n in [(0.3, 0.7, 10), (2.0, 5.0, 64), (9.0, 1.0, 7)]:
        na, nf = P.split_gpus(a, f, n)
        assert na + nf == n and na >= 1 and nf >= 1
        assert abs(na - n * a / (a + f)) <= 0.5 + 1e-12


def test_split_rejects_bad_input():
    with pytest.raises(ValueError):
        P.split_gpus(1.0, 1.0, 1)
    with pytest.raises(ValueError):
        P.split_gpus(0.0, 0.0, 8)


def test_pipeline_period_is_the_longer_stage_plus_handover():
    r = P.pipeline_period(3.0, 2.0, 0.5)
    assert r["colocated"] == 5.0 and r["disaggregated"] == 3.5
    r = P.pipeline_period(2.0, 2.0, 0.0)
    assert r["gain"] == 2.0  # balanced stages, free hand-over: twice the rate


def test_comm_bytes_match_the_pages_figure():
    assert P.comm_bytes_per_token_layer(4096, 8, 1) == 131072


def test_ffn_time_from_a_measured_bench_line():
    t_f = P.ffn_step_ms(os.path.join(ROOT, "profiles", "bench_decode_h4096_e64.json"))
    assert 0.0 < t_f < 100.0
    # with attention costing the same per step, the pools split evenly
    assert P.split_gpus(t_f, t_f, 32) == (16, 16)

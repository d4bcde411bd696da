"""Attention:FFN planning helpers against the rules and examples the pages
state (CPU)."""
import pytest

from expert_side_attention_amd import afd_plan as P


def test_rank_rule_examples_from_plugin_page():
    P.check_rank_counts(64, 16)          # 64A16F: legal
    with pytest.raises(ValueError):
        P.check_rank_counts(16, 64)      # fewer attention than FFN ranks
    with pytest.raises(ValueError):
        P.check_rank_counts(64, 24)      # not a multiple
    P.check_rank_counts(1, 1)            # the one-host example: 1 + 1
    assert P.rank_roles(4, 2) == ["ffn", "ffn", "attention", "attention", "attention",
                                  "attention"]


def _page_choose_split(attn_cost, ffn_cost, total_gpus):
    """The notes page's proportional-share example (case 2), as it prints it."""
    share = attn_cost / (attn_cost + ffn_cost)
    a = max(1, round(total_gpus * share))
    return a, total_gpus - a


def test_split_balances_the_two_pools():
    assert P.split_gpus(1.0, 1.0, 16) == (8, 8)
    assert P.split_gpus(3.0, 1.0, 16) == (12, 4)
    # the notes page's example: a 1:63 cost ratio over 128 GPUs is 2A + 126F
    assert P.split_gpus(1.0, 63.0, 128) == (2, 126) == _page_choose_split(1.0, 63.0, 128)
    # both pools exist: attention keeps one GPU at zero cost, FFN keeps one
    # where the page's rounding would leave it none
    assert P.split_gpus(0.0, 5.0, 8) == (1, 7)
    assert P.split_gpus(5.0, 0.0, 8) == (7, 1)
    assert _page_choose_split(5.0, 0.0, 8) == (8, 0)
    # equal periods (2/5 GPUs give 0.5 either way): nearest the share 2.5,
    # then the smaller attention pool
    assert P.split_gpus(1.0, 1.0, 5) == (2, 3)


def test_split_is_never_slower_than_any_other_split():
    import random
    rng = random.Random(0)
    agree = 0
    for _ in range(2000):
        a, f, n = rng.uniform(0.01, 10), rng.uniform(0.01, 10), rng.randint(2, 200)
        na, nf = P.split_gpus(a, f, n)
        assert na + nf == n and na >= 1 and nf >= 1
        best = min(P.step_period(a, f, i, n - i) for i in range(1, n))
        assert P.step_period(a, f, na, nf) == best
        pa, pf = _page_choose_split(a, f, n)
        if pf >= 1:
            # the page's rounding of the share never gives a faster step,
            # and it is off by at most one GPU
            assert P.step_period(a, f, na, nf) <= P.step_period(a, f, pa, pf)
            assert abs(pa - na) <= 1
            agree += (pa, pf) == (na, nf)
    assert agree > 1500


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


def test_ffn_time_from_a_bench_line(tmp_path):
    line = ('{"metric": "m", "value": 1.0, "unit": "tokens/s", "ms_per_step": 0.5,'
            ' "config": {"workload": "decode_h4096_e64"}}')
    p = tmp_path / "bench.json"
    p.write_text("[bench] building\n" + line + "\n")
    t_f = P.ffn_step_ms(str(p))
    assert t_f == 0.5
    # with attention costing the same per step, the pools split evenly
    assert P.split_gpus(t_f, t_f, 32) == (16, 16)

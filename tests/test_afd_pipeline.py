"""Attention/FFN micro-pipeline harness: schedule order and CU-mask layout
(CPU)."""
import pytest

from expert_side_attention_amd import afd_pipeline as AP


def test_schedule_edges_and_order():
    ops = AP.ping_pong_schedule(3, 2)
    assert len(ops) == 12
    index = {(o.kind, o.layer, o.mb): i for i, o in enumerate(ops)}
    for i, o in enumerate(ops):
        assert all(w < i for w in o.waits)            # waits only on earlier ops
        if o.kind == "ffn":
            assert o.stream == 1 and o.waits == (index[("attn", o.layer, o.mb)],)
        else:
            assert o.stream == 0
            want = () if o.layer == 0 else (index[("ffn", o.layer - 1, o.mb)],)
            assert o.waits == want
    # micro-batches never wait on each other: that freedom is the overlap
    for o in ops:
        assert all(ops[w].mb == o.mb for w in o.waits)


def test_schedule_simulated_period():
    """Run the schedule through a two-server simulation: with separate
    attention and FFN servers the steady period per layer approaches
    M * max(t_a, t_f) for M = 2 micro-batches, and a single server gives
    M * (t_a + t_f)."""
    t = {"attn": 3.0, "ffn": 2.0}
    L, M = 50, 2
    ops = AP.ping_pong_schedule(L, M)

    def simulate(shared):
        free = [0.0, 0.0]
        end = []
        for o in ops:
            srv = 0 if shared else o.stream
            start = max([free[srv]] + [end[w] for w in o.waits])
            end.append(start + t[o.kind])
            free[srv] = end[-1]
        return max(end)

    assert simulate(True) == pytest.approx(L * M * (3.0 + 2.0))
    per_layer = simulate(False) / L
    assert per_layer == pytest.approx(M * 3.0, rel=0.05)


def test_cu_mask_words():
    assert AP.cu_mask_words([0], 256) == [0xFF, 0, 0, 0, 0, 0, 0, 0]
    assert AP.cu_mask_words([3, 4], 256) == [0xFF000000, 0xFF, 0, 0, 0, 0, 0, 0]
    w = AP.cu_mask_words(range(32), 256)
    assert w == [0xFFFFFFFF] * 8
    with pytest.raises(ValueError):
        AP.cu_mask_words([32], 256)
    with pytest.raises(ValueError):
        AP.cu_mask_words([], 256)
    with pytest.raises(ValueError):
        AP.cu_mask_words([0], 252)


def test_split_blocks_follow_cost_share():
    a, f = AP.split_blocks(1.0, 1.0, 256)
    assert (len(a), len(f)) == (16, 16)
    assert a == list(range(16)) and f == list(range(16, 32))
    a, f = AP.split_blocks(1.0, 3.0, 256)
    assert (len(a), len(f)) == (8, 24)
    # disjoint and covering the chip
    assert sorted(a + f) == list(range(32))

"""bench.py's algorithmic work model, the numerator of every roofline figure
(CPU): bytes and flops per forward and per dominant launch, written out by
hand for known shapes, and the compute-bound tile rule on chosen counts."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from afd_inputs import CONFIGS, LayerShape  # noqa: E402


def test_decode_layer_bytes_and_flops():
    s = CONFIGS["decode_h4096_e64"]  # T 256, h 4096, E 64, k 8, I 1536, one shared 1536, bf16
    counts = [32] * 64  # every expert touched
    m = bench.work_model(s, counts)
    gate_up = 64 * (2 * 1536 * 4096 * 2) + (2 * 1536 * 4096 * 2) + 256 * 4096 * 2
    down = 64 * (4096 * 1536 * 2) + (4096 * 1536 * 2)
    assert m["touched_experts"] == 64
    assert m["gate_up_bytes"] == gate_up == 1_637_875_712
    assert m["ffn_bytes"] == gate_up + down
    # forward: both GEMMs, router weights, input and output
    assert m["forward_bytes"] == (64 * 3 * 1536 * 4096 * 2 + 3 * 1536 * 4096 * 2
                                  + 64 * 4096 * 2 + 2 * 256 * 4096 * 2)
    assert m["forward_flops"] == (2 * 256 * 8 * 3 * 4096 * 1536 + 2 * 256 * 1 * 3 * 4096 * 1536
                                  + 2 * 256 * 4096 * 64)
    assert m["gate_up_flops"] == 2 * 256 * 8 * 2 * 4096 * 1536 + 2 * 256 * 2 * 4096 * 1536


def test_untouched_experts_cost_nothing_and_w8a8_adds_block_scales():
    s = LayerShape("t", T=4, h=256, E=8, k=2, I=128, mode="w8a8")
    counts = [3, 0, 0, 5, 0, 0, 0, 0]  # two experts touched
    m = bench.work_model(s, counts)
    per_weight = 1 + 4 / (128 * 128)  # E4M3 byte plus its share of a 128x128 block scale
    assert m["touched_experts"] == 2
    assert abs(m["gate_up_bytes"] - (2 * 2 * 128 * 256 * per_weight + 4 * 256 * 2)) < 1e-6
    assert abs(m["ffn_bytes"] - (2 * 3 * 128 * 256 * per_weight + 4 * 256 * 2)) < 1e-6


def test_compute_bound_tile_rule():
    # average rows per expert above 112 (bf16): groups of at least 129 rows get
    # whole 256-row tiles, plus one for a remainder of more than 128 rows
    s = LayerShape("t", T=1000, h=256, E=4, k=2, I=128, S=1, Is=128, mode="bf16")
    rows, tiles = bench.big_tile_rows(s, [700, 129, 128, 1043], 1000)
    # 700 = 2 x 256 + 188 (a third tile); 129 -> one tile; 128 stays streaming;
    # 1043 = 4 x 256 + 19 (19 rows stream); shared 1000 = 3 x 256 + 232 (a fourth)
    assert rows == [700, 129, 0, 1024, 1000]
    assert tiles == 3 + 1 + 0 + 4 + 4
    # the decode regime has no compute-bound tiles
    d = CONFIGS["decode_h4096_e64"]
    assert bench.big_tile_rows(d, [32] * 64, 256) == ([0] * 65, 0)

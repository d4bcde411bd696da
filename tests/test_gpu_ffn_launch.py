"""The single launch of both weight-streaming GEMMs (bf16 decode regime)
against one launch per GEMM (config split_gemms = 1): bitwise the same
outputs, since every item keeps its per-row arithmetic; repeatable across
forwards and independent of how a batch is split.  The oracle comparisons
of these layers are in test_gpu_parity.py, which runs the single launch
wherever a layer allows it.  GPU only."""
import pytest
import torch

from afd_inputs import LayerShape, SyntheticLayer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SHAPES = [
    # decode regime (at most 48 routed rows per expert on average), hidden a
    # multiple of 256: shared experts of another width, two shared experts,
    # an odd expert count, down stages of 256 bytes (I_s = 128 * odd), a
    # wide intermediate, several row tiles per expert
    LayerShape("ffn_many", T=77, h=512, E=64, k=8, I=256, S=2, Is=128, mode="bf16"),
    LayerShape("ffn_odd_e", T=150, h=256, E=37, k=5, I=256, S=1, Is=384, mode="bf16"),
    LayerShape("ffn_wide", T=512, h=256, E=256, k=8, I=1024, S=1, Is=1024, mode="bf16"),
    LayerShape("ffn_h1024", T=256, h=1024, E=64, k=8, I=512, S=1, Is=512, mode="bf16"),
    LayerShape("ffn_rows", T=600, h=512, E=128, k=8, I=256, S=1, Is=256, mode="bf16"),
    LayerShape("ffn_t1", T=1, h=256, E=8, k=2, I=128, S=1, Is=128, mode="bf16"),
    # enough down items per resident workgroup (657 tiles at most x 16
    # column blocks, over 32 per CU of 256) for 128-column down items; the
    # layers above take 256-column ones
    LayerShape("ffn_narrow", T=1024, h=2048, E=512, k=8, I=128, S=1, Is=256, mode="bf16"),
    # over 1024 tokens: the dispatch runs in blocks and its scan kernel zeroes
    # the tile counters
    LayerShape("ffn_blocks", T=2100, h=256, E=512, k=8, I=128, S=1, Is=128, mode="bf16"),
]


def _layers(shape, seed):
    from expert_side_attention_amd.workload import build_layer
    syn = SyntheticLayer(shape, seed=seed)
    one = build_layer(syn, DEV)
    k = one._keep
    split = type(one)(mode="bf16", hidden=shape.h, num_experts=shape.E, top_k=shape.k,
                      inter=shape.I, max_tokens=shape.T, router_w=k[0], router_b=k[1],
                      gate_w=k[2], up_w=k[3], down_w=k[4], num_shared=shape.S,
                      shared_inter=shape.Is, sh_gate_w=k[8], sh_up_w=k[9], sh_down_w=k[10],
                      split_gemms=True)
    return syn, one, split


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_single_launch_equals_split_launches(shape):
    from expert_side_attention_amd.workload import to_device
    syn, one, split = _layers(shape, seed=31)
    print(f"[ffn] {shape}", flush=True)
    x = to_device(syn.hidden(), DEV, True)
    _, tr = one.forward(x, trace=True)
    torch.cuda.synchronize()
    assert int(tr["sync_timeouts"][0]) == 0  # every down item found its tile complete
    one.profile_enable(["gate_up", "down", "ffn"])
    split.profile_enable(["gate_up", "down", "ffn"])
    a = one.forward(x).clone()
    b = split.forward(x).clone()
    torch.cuda.synchronize()
    pa, pb = one.profile_read(), split.profile_read()
    one.profile_enable([])
    split.profile_enable([])
    # the layer ran the single launch, the split layer the two launches
    assert pa["ffn"][1] == 1 and pa["gate_up"][1] == 0 and pa["down"][1] == 0, pa
    assert pb["ffn"][1] == 0 and pb["gate_up"][1] == 1 and pb["down"][1] == 1, pb
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # repeatable: the order in which workgroups take items and wait for
    # tiles never reaches the results
    out = torch.empty_like(a)
    for i in range(12):
        one.forward(x, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), a.view(torch.int16)), f"forward {i}"
    one.close()
    split.close()


def test_single_launch_batch_split_and_two_streams():
    """Per-token results do not depend on the batch (halves give the same
    bits), and two handles running the single launch on two streams at once
    give the serial results."""
    from expert_side_attention_amd.workload import to_device
    shape = LayerShape("ffn_split", T=384, h=512, E=64, k=8, I=256, S=1, Is=256, mode="bf16")
    syn, one, split = _layers(shape, seed=17)
    x = to_device(syn.hidden(), DEV, True)
    full = one.forward(x).clone()
    p1 = one.forward(x[:150].contiguous()).clone()
    p2 = one.forward(x[150:].contiguous()).clone()
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([p1, p2]).view(torch.int16), full.view(torch.int16))
    sib = one.sibling()
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    x0, x1 = x[:192].contiguous(), x[192:].contiguous()
    o0, o1 = torch.empty_like(x0), torch.empty_like(x1)
    torch.cuda.synchronize()
    for _ in range(4):
        one.forward(x0, out=o0, stream=s0)
        sib.forward(x1, out=o1, stream=s1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o0, o1]).view(torch.int16), full.view(torch.int16))
    for layer in (one, split, sib):
        layer.close()


@pytest.mark.parametrize("name", ["decode_h4096_e64", "dsv3_decode_t512"])
def test_single_launch_full_size_alternating_inputs(name):
    """At the benchmark sizes (every CU, all XCDs): one handle alternating
    three different batches gives, every time, the bits of the separate
    launches on the same batch.  A z row read before its gate/up items had
    written it through, or a line of an earlier forward's z served from a
    cache, would show up here as a difference."""
    from afd_inputs import CONFIGS
    from expert_side_attention_amd.workload import to_device
    shape = CONFIGS[name]
    syn, one, split = _layers(shape, seed=0)
    print(f"[ffn] full size {name}", flush=True)
    base = to_device(syn.hidden(), DEV, True)
    xs = [base, base.flip(0).contiguous(), torch.roll(base, 7, dims=1).contiguous()]
    refs = [split.forward(x).clone() for x in xs]
    out = torch.empty_like(base)
    for i in range(24):
        j = i % 3
        _, tr = one.forward(xs[j], out=out, trace=True)
        torch.cuda.synchronize()
        assert int(tr["sync_timeouts"][0]) == 0
        assert torch.equal(out.view(torch.int16), refs[j].view(torch.int16)), (i, j)
    one.close()
    split.close()

"""A forward captured in a HIP graph and replayed equals the eager forward.

The FFN service of the AFD plugin runs decode as a captured graph (vLLM AFD
Plugin page, connector table: the synchronous connectors use full-decode
graph mode), so `afd_ffn_forward` must be capturable: it enqueues kernels
only, never allocates, synchronises or reads device memory on the host.

Every replay is checked bitwise against the eager result for the same input,
with eager forwards and synchronisations of the program in between, over
several replays and inputs that route differently; the first replay of each
input is also checked against the fp64 oracle (routing within the fp32
slack, outputs within the bf16 / W8A8 tolerances).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from afd_inputs import LayerShape, SyntheticLayer  # noqa: E402
from oracle import afd_oracle as O  # noqa: E402

from parity import check_outputs, check_routing, decode_store, routing_slack  # noqa: E402

pytestmark = pytest.mark.gpu


def _layer(shape, seed):
    from expert_side_attention_amd.workload import build_layer, hidden_tensor
    syn = SyntheticLayer(shape, seed=seed)
    return syn, build_layer(syn, "cuda:0"), hidden_tensor(syn, "cuda:0")


def _host(t):
    return O.bf16_to_f64(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))


def _check_vs_oracle(orc, shape, x_store, out, ids):
    ref = orc.forward(x_store)
    beta = routing_slack(decode_store(x_store, shape.mode), orc._wr, orc._b, shape.h)
    differ = check_routing(ref["logits"], beta, ids, shape.k)
    assert differ.mean() <= 0.01
    return check_outputs(_host(out), ref["out"], shape.mode, keep=~differ)


@pytest.mark.parametrize("shape", [
    LayerShape("graph_bf16", T=128, h=256, E=16, k=4, I=256, S=1, Is=256, mode="bf16"),
    LayerShape("graph_w8a8", T=96, h=256, E=8, k=2, I=256, S=1, Is=128, mode="w8a8"),
    LayerShape("graph_prefill", T=1200, h=256, E=4, k=2, I=256, S=1, Is=128, mode="bf16"),
    # the tiled router (two K splits) under capture
    LayerShape("graph_router_tiled", T=4200, h=1024, E=64, k=2, I=128, mode="bf16"),
], ids=lambda s: s.name)
def test_graph_replay_matches_eager(shape):
    syn, layer, x = _layer(shape, seed=11)
    # three inputs with different routing: the batch, its rows rolled, and
    # rows negated (exact in bf16; flips the sign of every logit)
    inputs = [x, torch.roll(x, shifts=37, dims=0).contiguous(), (-x).contiguous()]
    xs = syn.hidden()
    stores = [xs, np.roll(xs, 37, axis=0), xs ^ np.uint16(0x8000)]
    eager, ids = [], []
    for xi in inputs:
        o, tr = layer.forward(xi, trace=True)
        eager.append(o.clone())
        ids.append(tr["topk_ids"].cpu().numpy())
    torch.cuda.synchronize()
    orc = O.OracleFFN(syn, threads=8)

    s = torch.cuda.Stream()
    x_static = torch.empty_like(x)
    out_static = torch.empty_like(x)
    with torch.cuda.stream(s):
        x_static.copy_(inputs[0])
        layer.forward(x_static, out=out_static, stream=s)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(x_static, out=out_static, stream=s)
    torch.cuda.synchronize()

    scratch = torch.empty_like(x)
    for rep in range(3):
        for i, xi in enumerate(inputs):
            x_static.copy_(xi)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_static, eager[i]), f"replay {rep} input {i}"
            if rep == 0:
                rel, mabs = _check_vs_oracle(orc, shape, stores[i], out_static, ids[i])
                print(f"[graph] {shape.name} input {i}: replay vs oracle rel-L2 {rel:.3e} "
                      f"max-abs/max {mabs:.3e}", flush=True)
            # eager work of the program between replays
            layer.forward(inputs[(i + 1) % 3], out=scratch)
            torch.cuda.synchronize()
            assert torch.equal(scratch, eager[(i + 1) % 3])
    layer.close()

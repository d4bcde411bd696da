"""The attention/FFN micro-pipeline harness: every placement of the
ping-pong schedule (co-located on one stream, overlapped on two streams,
split over CU-masked streams) yields the hidden states of the plain loop
over layers and micro-batches, bit for bit; and in that loop the FFN
service's output of every layer and micro-batch matches the fp64 oracle on
the input that layer received."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from afd_inputs import LayerShape, SyntheticLayer  # noqa: E402
from oracle import afd_oracle as O  # noqa: E402

from parity import check_outputs, check_routing, decode_store, routing_slack  # noqa: E402

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def test_pipeline_placements_agree():
    from expert_side_attention_amd import afd_pipeline as AP
    from expert_side_attention_amd.workload import build_layer, hidden_tensor
    T, M, layers = 64, 2, 4
    shape = LayerShape("pipe_bf16", T=M * T, h=512, E=16, k=4, I=256, S=1, Is=256,
                       mode="bf16")
    syn = SyntheticLayer(shape, seed=5)
    f0 = build_layer(syn, "cuda:0", max_tokens=T)
    ffns = [f0, f0.sibling()]
    x = hidden_tensor(syn, "cuda:0")
    xs = [x[m * T:(m + 1) * T].contiguous() for m in range(M)]
    attn = [AP.AttentionStub(T, shape.h, 256, heads=4, d=128, device="cuda:0", seed=m + 1)
            for m in range(M)]
    res = AP.measure(ffns, xs, attn, layers=layers, reps=3)
    assert res["outputs_identical"]

    hb = [xi.clone() for xi in xs]
    ab = [torch.empty_like(xi) for xi in xs]
    orc = O.OracleFFN(syn, threads=8)
    for layer in range(layers):
        for m in range(M):
            attn[m].forward(hb[m], ab[m])
            _, tr = ffns[m].forward(ab[m], out=hb[m], trace=True)
            torch.cuda.synchronize()
            # the FFN service's step of this layer vs the oracle on its input
            a = _bits(ab[m])
            ref = orc.forward(a)
            beta = routing_slack(decode_store(a, "bf16"), orc._wr, orc._b, shape.h)
            differ = check_routing(ref["logits"], beta, tr["topk_ids"].cpu().numpy(), shape.k)
            assert differ.mean() <= 0.01
            rel, mabs = check_outputs(O.bf16_to_f64(_bits(hb[m])), ref["out"], "bf16",
                                      keep=~differ)
            print(f"[pipeline] layer {layer} micro-batch {m}: FFN vs oracle rel-L2 {rel:.3e}",
                  flush=True)
    torch.cuda.synchronize()
    for m in range(M):
        assert torch.isfinite(hb[m].float()).all()
        assert torch.equal(hb[m], res["finals"]["serial"][m])
    assert set(res["period_ms"]) == {"serial", "overlap", "split"}
    assert all(v > 0 for v in res["period_ms"].values())
    assert res["split"]["attn_cus"] + res["split"]["ffn_cus"] == res["num_cus"]

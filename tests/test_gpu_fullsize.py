"""Full-size layers (the benchmark workloads) vs the fp64 oracle.

The GPU runs the whole batch in the benchmark's launch configuration; the
oracle checks routing for every token (selection rule within the fp32
slack), the dispatch of every micro-batch bit for bit, W8A8 input bytes and
weight quantisation bit for bit, and the outputs of sampled tokens, which it
computes one by one.  GPU only; each test holds a few tens of GB of device
memory and needs tens of seconds of host time."""
import numpy as np
import pytest
import torch

from afd_inputs import CONFIGS, SyntheticLayer
from oracle import afd_oracle as O

from parity import (check_dispatch, check_gpu_logits, check_outputs, check_routing,
                    check_selection_on_gpu_logits, check_w8a8_z, check_weights,
                    check_weights_on_gpu_logits, decode_store, logit_abs_sums)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy()


def _sample(T, n=12):
    return sorted(set(np.linspace(0, T - 1, n).astype(int).tolist()))


def check_full(name, microbatches=1, n_sample=12):
    from expert_side_attention_amd.workload import build_layer, to_device
    syn = SyntheticLayer(CONFIGS[name], seed=0)
    s = syn.shape
    print(f"[fullsize] {name}: building weights", flush=True)
    T = s.T
    mbT = T // microbatches
    layer = build_layer(syn, DEV, max_tokens=mbT)
    layers = [layer]
    if microbatches > 1:
        k = layer._keep
        for _ in range(microbatches - 1):
            layers.append(type(layer)(
                mode=s.mode, hidden=s.h, num_experts=s.E, top_k=s.k, inter=s.I,
                max_tokens=mbT, router_w=k[0], router_b=k[1], gate_w=k[2], up_w=k[3],
                down_w=k[4], gate_s=k[5], up_s=k[6], down_s=k[7], num_shared=s.S,
                shared_inter=s.Is, sh_gate_w=k[8], sh_up_w=k[9], sh_down_w=k[10],
                sh_gate_s=k[11], sh_up_s=k[12], sh_down_s=k[13]))
    x = syn.hidden()
    xt = to_device(x, DEV, s.mode != "f32")
    streams = [torch.cuda.Stream() for _ in range(microbatches)]
    torch.cuda.synchronize()
    outs, trs = [], []
    for i in range(microbatches):
        o, tr = layers[i].forward(xt[i * mbT:(i + 1) * mbT], stream=streams[i], trace=True)
        outs.append(o)
        trs.append(tr)
    torch.cuda.synchronize()
    out = np.concatenate([_np(o) for o in outs])
    trs = [{kk: v.cpu().numpy() for kk, v in tr.items()} for tr in trs]
    # no down item of a single GEMM launch gave up waiting for its row tile
    assert all(int(tr["sync_timeouts"][0]) == 0 for tr in trs)
    print(f"[fullsize] {name}: GPU done; oracle routing", flush=True)

    orc = O.OracleFFN(syn, threads=16)
    logits, ids, w = orc.route(x)
    sums = logit_abs_sums(decode_store(x, s.mode), orc._wr, orc._b)
    beta = (s.h + 2) * 2.0 ** -24 * sums
    gpu_ids = np.concatenate([tr["topk_ids"] for tr in trs])
    gpu_logits = np.concatenate([tr["logits"] for tr in trs])
    lr, lq = check_gpu_logits(gpu_logits, logits, sums, s.h)
    check_selection_on_gpu_logits(gpu_logits, gpu_ids, s.k)
    wrel = check_weights_on_gpu_logits(np.concatenate([tr["topk_w"] for tr in trs]),
                                       gpu_logits, gpu_ids)
    print(f"[fullsize] {name}: logits within {lr:.2e} of the worst-case bound, {lq:.2e} of "
          f"the realistic one; weights {wrel:.2e} relative to the GPU logits' softmax",
          flush=True)
    differ = check_routing(logits, beta, gpu_ids, s.k)
    print(f"[fullsize] {name}: {int(differ.sum())} near-tie tokens of {T}", flush=True)
    assert differ.mean() <= 0.01
    same = ~differ
    gpu_w = np.concatenate([tr["topk_w"] for tr in trs])
    ratio = check_weights(gpu_w, w, beta, gpu_ids, same)
    print(f"[fullsize] {name}: routing weights within {ratio:.2e} of their worst-case bound",
          flush=True)
    for tr in trs:
        check_dispatch(tr, s.E)
    if s.mode == "w8a8":
        q, sc = O.quantize_1x128(O.bf16_to_f64(x).astype(np.float32))
        assert np.array_equal(np.concatenate([tr["x_q"] for tr in trs]), q)
        assert np.array_equal(np.concatenate([tr["x_s"] for tr in trs]), sc)
        # weight bytes of a few experts: the library's block quantiser vs the oracle's
        k = layer._keep
        for e in (0, s.E // 2, s.E - 1):
            mats = syn.expert(e)
            for (wq, ws), m in zip(((k[2], k[5]), (k[3], k[6]), (k[4], k[7])), mats):
                rq, rs = O.quantize_128x128(O.bf16_to_f64(m).astype(np.float32))
                assert np.array_equal(wq[e].cpu().numpy(), rq)
                assert np.array_equal(ws[e].cpu().numpy(), rs)
        # E4M3 z of every row of three experts and of the shared expert
        for i, tr in enumerate(trs):
            xm = x[i * mbT:(i + 1) * mbT]
            busy = np.argsort(-tr["counts"], kind="stable")[:3]
            rows, frac, worst = check_w8a8_z(orc, xm, tr, groups=[int(e) for e in busy])
            print(f"[fullsize] {name}: W8A8 z of {rows} rows, {frac:.5f} of the codes equal "
                  f"the oracle's, scales within {worst:.2f} of their bound", flush=True)
    tokens = [t for t in _sample(T, n_sample) if same[t]]
    print(f"[fullsize] {name}: oracle outputs of tokens {tokens}", flush=True)
    ref = orc.forward(x, tokens=tokens)
    rel, mabs = check_outputs(out[tokens], ref["out"], s.mode)
    print(f"[fullsize] {name}: rel-L2 {rel:.3e} max-abs/max {mabs:.3e}", flush=True)
    for l in layers:
        l.close()


def test_decode_h4096_e64_full_batch():
    check_full("decode_h4096_e64", n_sample=16)


def test_dsv3_decode_t512():
    check_full("dsv3_decode_t512")


def test_dsv3_w8a8_t2048():
    check_full("dsv3_w8a8_t2048")


def test_prefill_skew_two_microbatches():
    check_full("prefill_skew_t16384", microbatches=2, n_sample=16)


def test_dsv3_ep8_shard():
    check_full("dsv3_ep8_shard_t512")


def test_dsv3_w8a8_ep8_shard():
    check_full("dsv3_w8a8_ep8_shard_t2048")

"""The allocation-free forward (afd_ffn_forward_static, through the C ABI)
against the handle forward (afd_ffn_forward) on the same inputs: the same
kernels, so the same bits, on two calls in a row, the second with a smaller
batch, for each precision and both weight-streaming tile shapes; and the
capacity error when a batch's workspace exceeds the fixed scratch.  GPU."""
import ctypes

import pytest
import torch

from afd_inputs import LayerShape, SyntheticLayer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("shape,T2", [
    (LayerShape("na_bf16_stream", T=256, h=1024, E=32, k=8, I=512, S=1, Is=512, mode="bf16"), 77),
    (LayerShape("na_bf16_prefill", T=600, h=512, E=16, k=4, I=256, S=1, Is=256, mode="bf16"), 33),
    (LayerShape("na_w8a8", T=256, h=512, E=16, k=4, I=256, S=1, Is=384, mode="w8a8"), 50),
    (LayerShape("na_f32", T=64, h=256, E=8, k=2, I=256, S=1, Is=128, mode="f32"), 5),
    # one cooperative launch per forward (single_launch = 1)
    (LayerShape("na_single_f32", T=16, h=256, E=8, k=2, I=512, mode="f32"), 5),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_static_forward_matches_handle_forward(shape, T2):
    from expert_side_attention_amd.workload import build_layer, hidden_tensor
    print(f"[no-alloc] {shape.name} T={shape.T} then T={T2}", flush=True)
    syn = SyntheticLayer(shape, seed=17)
    layer = build_layer(syn, DEV, single_launch=shape.name.startswith("na_single"))
    x = hidden_tensor(syn, DEV)
    iv = torch.int32 if shape.mode == "f32" else torch.int16
    for T in (shape.T, T2):
        xi = x[:T].contiguous()
        ref = layer.forward(xi).clone()
        got = layer.forward_static(xi)
        torch.cuda.synchronize()
        assert torch.equal(got.view(iv), ref.view(iv)), f"T = {T}"
    layer.close()


def test_static_forward_refuses_batches_beyond_the_scratch():
    from expert_side_attention_amd import AfdError
    from expert_side_attention_amd import _ffi as F
    # 4096 tokens of a 4096-wide, 64-expert, top-8 layer: ~390 MB of workspace
    cfg = F.afd_ffn_config(abi_version=F.AFD_FFN_ABI_VERSION, mode=F.AFD_MODE_BF16,
                           hidden=4096, num_experts=64, top_k=8, inter=1536, num_shared=1,
                           shared_inter=1536, max_tokens=4096, has_router_bias=0)
    fake = 0x1000  # never dereferenced: the size check comes first
    w = F.afd_ffn_weights(router_w=fake, gate_w=fake, up_w=fake, down_w=fake,
                          sh_gate_w=fake, sh_up_w=fake, sh_down_w=fake)
    with pytest.raises(AfdError) as ei:
        F.afd_ffn_forward_static(cfg, w, fake, fake + (1 << 30), 4096, 0)
    assert ei.value.status == F.AFD_ERR_CAPACITY
    assert "scratch" in F.afd_ffn_last_error()

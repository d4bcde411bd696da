"""HIP path vs fp64 oracle on small layers that still span several row and
column tiles, ragged tails, empty experts, several shared experts, every
router variant and all three precisions.  Calls go through the C ABI
(ctypes binding).  GPU only."""
import numpy as np
import pytest
import torch

from afd_inputs import CONFIGS, LayerShape, SyntheticLayer, f32_to_bf16_bits, tie_case
from oracle import afd_oracle as O

from parity import (TOL, check_dispatch, check_gpu_logits, check_outputs, check_routing,
                    check_selection_on_gpu_logits, check_w8a8_z, check_weights,
                    check_weights_on_gpu_logits, decode_store, logit_abs_sums)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy()


def run_gpu(syn, x_store=None, max_tokens=None, layer=None, single_launch=False):
    from expert_side_attention_amd.workload import build_layer, to_device
    s = syn.shape
    layer = layer or build_layer(syn, DEV, max_tokens=max_tokens, single_launch=single_launch)
    x = syn.hidden() if x_store is None else x_store
    xt = to_device(x, DEV, s.mode != "f32")
    out, tr = layer.forward(xt, trace=True)
    torch.cuda.synchronize()
    return layer, _np(out), {k: v.cpu().numpy() for k, v in tr.items()}


def check_layer(syn, x_store=None, threads=8, expect_exact_routing=False, single_launch=False):
    s = syn.shape
    x = syn.hidden() if x_store is None else x_store
    print(f"[parity] {s} single_launch={single_launch}", flush=True)
    _, out, tr = run_gpu(syn, x, single_launch=single_launch)
    # no down item of a single GEMM launch gave up waiting for its row tile
    assert int(tr["sync_timeouts"][0]) == 0
    orc = O.OracleFFN(syn, threads=threads)
    ref = orc.forward(x)
    x64 = decode_store(x, s.mode)
    sums = logit_abs_sums(x64, orc._wr, orc._b)
    beta = (s.h + 2) * 2.0 ** -24 * sums
    lr, lq = check_gpu_logits(tr["logits"], ref["logits"], sums, s.h)
    check_selection_on_gpu_logits(tr["logits"], tr["topk_ids"], s.k)
    wrel = check_weights_on_gpu_logits(tr["topk_w"], tr["logits"], tr["topk_ids"])
    differ = check_routing(ref["logits"], beta, tr["topk_ids"], s.k)
    if expect_exact_routing:
        assert not differ.any()
    assert differ.mean() <= 0.01, f"{differ.sum()} tokens route differently"
    check_dispatch(tr, s.E)
    same = ~differ
    check_weights(tr["topk_w"], ref["w"], beta, tr["topk_ids"], same)
    print(f"[parity] logits: max error {lr:.2e} of the worst-case bound, {lq:.2e} of the "
          f"realistic one; weights {wrel:.2e} relative to the GPU logits' softmax", flush=True)
    if s.mode == "w8a8":
        assert np.array_equal(tr["x_q"], ref["x_q"])
        assert np.array_equal(tr["x_s"], ref["x_s"])
        rows, frac, worst = check_w8a8_z(orc, x, tr)
        print(f"[parity] W8A8 z of {rows} rows: {frac:.5f} of the codes equal the oracle's, "
              f"scales within {worst:.2f} of their bound", flush=True)
    rel, mabs = check_outputs(out, ref["out"], s.mode, keep=same)
    print(f"[parity] rel-L2 {rel:.3e} max-abs/max {mabs:.3e} "
          f"near-tie tokens {int(differ.sum())}", flush=True)
    return out, tr, ref


SMALL = [
    # name, shape
    CONFIGS["tiny_fp32"],
    LayerShape("bf16_ragged", T=300, h=256, E=8, k=3, I=384, S=1, Is=256, mode="bf16"),
    LayerShape("bf16_many_experts", T=77, h=512, E=64, k=8, I=256, S=2, Is=128, mode="bf16"),
    LayerShape("bf16_e256", T=40, h=128, E=256, k=8, I=128, mode="bf16"),
    LayerShape("bf16_e512", T=20, h=128, E=512, k=4, I=128, S=1, Is=128, mode="bf16"),
    # an expert count that fills no 16-expert router slice, odd k
    LayerShape("bf16_odd_e", T=150, h=256, E=37, k=5, I=256, S=1, Is=128, mode="bf16"),
    # more slots than one combine pass gathers (eight at a time)
    LayerShape("bf16_k16", T=40, h=128, E=64, k=16, I=128, S=1, Is=128, mode="bf16"),
    # the most shared experts the library takes
    LayerShape("bf16_s8", T=64, h=128, E=8, k=2, I=128, S=8, Is=128, mode="bf16"),
    # enough 64-row work items for the 8-wave gate/up shape, 512-byte down stages
    LayerShape("bf16_e256_wide", T=512, h=256, E=256, k=8, I=1024, S=1, Is=1024, mode="bf16"),
    LayerShape("bf16_zipf", T=500, h=256, E=32, k=4, I=128, S=1, Is=128, mode="bf16",
               router="zipf"),
    LayerShape("bf16_big_t", T=2100, h=128, E=64, k=2, I=128, mode="bf16"),
    # the register router with its K range in four partial planes (at most 64
    # experts, h a multiple of 1024), the bias added by the top-k after them
    LayerShape("bf16_kparts_zipf", T=300, h=1024, E=48, k=6, I=128, S=1, Is=128, mode="bf16",
               router="zipf"),
    LayerShape("bf16_e512_blocks", T=2049, h=128, E=512, k=8, I=128, S=1, Is=128,
               mode="bf16"),
    # the same regime with hidden a multiple of 256: gate/up and down in one
    # launch over several dispatch blocks
    LayerShape("bf16_ffn_blocks", T=2100, h=256, E=512, k=8, I=128, S=1, Is=256,
               mode="bf16"),
    LayerShape("f32_k_eq_e", T=70, h=128, E=4, k=4, I=128, S=1, Is=256, mode="f32"),
    LayerShape("w8a8_small", T=200, h=512, E=8, k=2, I=256, S=1, Is=384, mode="w8a8"),
    LayerShape("w8a8_many", T=96, h=256, E=32, k=8, I=384, mode="w8a8"),
    LayerShape("w8a8_dense", T=600, h=256, E=8, k=2, I=256, S=1, Is=128, mode="w8a8"),
    LayerShape("w8a8_h384", T=200, h=384, E=8, k=2, I=256, S=1, Is=384, mode="w8a8"),
    LayerShape("bf16_dense", T=700, h=256, E=4, k=1, I=128, S=1, Is=384, mode="bf16"),
    LayerShape("bf16_prefill_h384", T=520, h=384, E=4, k=2, I=256, S=1, Is=128, mode="bf16"),
    LayerShape("bf16_prefill_skew", T=1500, h=256, E=16, k=2, I=256, S=1, Is=256,
               mode="bf16", router="zipf"),
    # compute-bound tiles whose column tiles split unevenly into the XCD tile
    # windows: gate/up 9 column tiles (groups of 5 and 4; the shared expert's
    # narrower I_s leaves 5), down 3
    LayerShape("bf16_prefill_windows", T=1000, h=768, E=4, k=2, I=1152, S=1, Is=640,
               mode="bf16"),
    # tiny layers, at most 16 tokens, also run as one launch (FUSED below)
    LayerShape("fused_bf16_shared", T=13, h=512, E=32, k=6, I=256, S=2, Is=128, mode="bf16"),
    LayerShape("fused_bf16_e512_k16", T=7, h=128, E=512, k=16, I=128, S=1, Is=256,
               mode="bf16", router="zipf"),
    LayerShape("fused_f32_t1", T=1, h=128, E=4, k=4, I=128, S=1, Is=128, mode="f32"),
    LayerShape("fused_f32_h384", T=16, h=384, E=16, k=3, I=384, S=1, Is=128, mode="f32"),
]

# shapes also checked with single_launch = 1 (tile lists then stay empty)
FUSED = {"tiny_fp32", "fused_bf16_shared", "fused_bf16_e512_k16", "fused_f32_t1",
         "fused_f32_h384"}


# long batches at small width: 64 dispatch blocks, large tile lists and grids,
# the compute-bound bf16 kernel and the fp8 tiled kernel
LONG = [
    LayerShape("bf16_t65536", T=65536, h=128, E=64, k=8, I=128, S=1, Is=128, mode="bf16"),
    LayerShape("w8a8_t32768", T=32768, h=256, E=32, k=2, I=128, S=1, Is=128, mode="w8a8"),
    # the tiled router: K split in two, a partial second column tile of experts
    LayerShape("bf16_router_tiled", T=4500, h=1024, E=320, k=4, I=128, S=1, Is=128,
               mode="bf16"),
]


@pytest.mark.parametrize("shape", LONG, ids=[s.name for s in LONG])
def test_long_batch_parity(shape):
    check_layer(SyntheticLayer(shape, seed=21), threads=16)


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_small_layer_parity(shape):
    _, tr, _ = check_layer(SyntheticLayer(shape, seed=3))
    # the kernel sequence has at least one weight-streaming or tiled row tile
    assert tr["num_tiles"][0] > 0 or tr["num_tiles"][1] > 0


@pytest.mark.parametrize("shape", [s for s in SMALL if s.name in FUSED],
                         ids=lambda s: s.name)
def test_single_launch_parity(shape):
    """The same tiny layers run as one cooperative launch: the same parity
    rules, and no GEMM tile lists (the single-launch path builds none)."""
    _, tr, _ = check_layer(SyntheticLayer(shape, seed=3), single_launch=True,
                           expect_exact_routing=shape.name == "tiny_fp32")
    assert tr["num_tiles"].tolist() == [0, 0]


@pytest.mark.parametrize("shape", [
    LayerShape("rep_fused_bf16", T=16, h=256, E=16, k=4, I=256, S=1, Is=256, mode="bf16"),
    LayerShape("rep_fused_f32", T=9, h=256, E=8, k=2, I=512, mode="f32"),
], ids=lambda s: s.name)
def test_single_launch_path_repeats_and_splits(shape):
    """The single-launch forward: bitwise repeatable, and a token's result
    does not depend on the other tokens of the batch (any batch of at most
    16 tokens takes the same path)."""
    syn = SyntheticLayer(shape, seed=23)
    from expert_side_attention_amd.workload import build_layer, to_device
    layer = build_layer(syn, DEV, single_launch=True)
    x = to_device(syn.hidden(), DEV, shape.mode != "f32")
    iv = torch.int32 if shape.mode == "f32" else torch.int16
    ref, tr = layer.forward(x, trace=True)
    ref = ref.clone()
    assert tr["num_tiles"].tolist() == [0, 0]
    out = torch.empty_like(ref)
    for i in range(12):
        layer.forward(x, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(iv), ref.view(iv)), f"forward {i}"
    a = layer.forward(x[:5].contiguous()).clone()
    b = layer.forward(x[5:].contiguous()).clone()
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a, b]).view(iv), ref.view(iv))
    layer.close()


def test_tiny_fp32_is_fp32_accurate():
    out, tr, ref = check_layer(SyntheticLayer(CONFIGS["tiny_fp32"], seed=0),
                               expect_exact_routing=True)
    rel = np.linalg.norm(out - ref["out"]) / np.linalg.norm(ref["out"])
    assert rel < 1e-5, rel


def test_exact_ties_pick_lowest_index():
    shape = LayerShape("ties", T=64, h=256, E=16, k=4, I=128, mode="bf16")
    syn = SyntheticLayer(shape, seed=4)
    x, wr = tie_case(T=64, h=256, E=16, seed=4)

    class Src:
        pass
    src = Src()
    src.shape = shape
    src.router_weight = lambda: wr
    src.router_bias = lambda: None
    src.expert = syn.expert
    src.shared = syn.shared
    src.hidden = lambda: x
    from expert_side_attention_amd.workload import build_layer, to_device
    layer = build_layer(syn, DEV)
    # replace the router weight with the integer-valued one
    layer2 = type(layer)(mode="bf16", hidden=256, num_experts=16, top_k=4, inter=128,
                         max_tokens=64, router_w=to_device(wr, DEV, True),
                         gate_w=layer._keep[2], up_w=layer._keep[3], down_w=layer._keep[4])
    xt = to_device(x, DEV, True)
    out, tr = layer2.forward(xt, trace=True)
    torch.cuda.synchronize()
    ref = O.OracleFFN(src).forward(x)
    assert np.array_equal(tr["topk_ids"].cpu().numpy(), ref["ids"])
    l = ref["logits"]
    assert np.any(l[:, 0] == l[:, 1])  # ties really occur


def test_uniform_router_selects_all_in_index_order():
    shape = LayerShape("uniform", T=33, h=128, E=8, k=8, I=128, mode="bf16")
    syn = SyntheticLayer(shape, seed=5)
    from expert_side_attention_amd.workload import build_layer, to_device
    base = build_layer(syn, DEV)
    zero = torch.zeros((8, 128), dtype=torch.bfloat16, device=DEV)
    layer = type(base)(mode="bf16", hidden=128, num_experts=8, top_k=8, inter=128,
                       max_tokens=33, router_w=zero, gate_w=base._keep[2],
                       up_w=base._keep[3], down_w=base._keep[4])
    out, tr = layer.forward(to_device(syn.hidden(), DEV, True), trace=True)
    torch.cuda.synchronize()
    assert np.array_equal(tr["topk_ids"].cpu().numpy(), np.tile(np.arange(8), (33, 1)))
    assert np.allclose(tr["topk_w"].cpu().numpy(), 0.125, atol=1e-7)


def test_determinism_and_microbatch_split():
    shape = LayerShape("split", T=257, h=256, E=16, k=4, I=256, S=1, Is=128, mode="bf16")
    syn = SyntheticLayer(shape, seed=6)
    from expert_side_attention_amd.workload import build_layer, to_device
    layer = build_layer(syn, DEV)
    xt = to_device(syn.hidden(), DEV, True)
    a = layer.forward(xt).clone()
    b = layer.forward(xt).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # rows of a token never mix with other tokens' rows, so a split batch
    # gives the same bits per token (both halves stay on the register router
    # and the streaming GEMMs, whose per-row summation order is fixed)
    p1 = layer.forward(xt[:100].contiguous()).clone()
    p2 = layer.forward(xt[100:].contiguous()).clone()
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([p1, p2]).view(torch.int16), a.view(torch.int16))


@pytest.mark.parametrize("shape", [
    LayerShape("rep_bf16_bm64", T=256, h=1024, E=64, k=8, I=512, S=1, Is=512, mode="bf16"),
    LayerShape("rep_bf16_bm128", T=512, h=1024, E=64, k=8, I=512, S=1, Is=512, mode="bf16"),
    LayerShape("rep_bf16_prefill", T=2048, h=1024, E=8, k=2, I=512, S=1, Is=512, mode="bf16"),
    LayerShape("rep_w8a8_stream", T=512, h=1024, E=64, k=8, I=512, S=1, Is=512, mode="w8a8"),
    LayerShape("rep_w8a8_tiled", T=2048, h=1024, E=8, k=2, I=512, S=1, Is=512, mode="w8a8"),
    LayerShape("rep_f32", T=128, h=256, E=8, k=2, I=256, S=1, Is=256, mode="f32"),
], ids=lambda s: s.name)
def test_repeated_forwards_are_bitwise_identical(shape):
    """Many forwards of one input give the same bits every time, for every
    kernel family: a pipeline that read a buffer before all of its loads
    had landed would show up here as run-to-run differences."""
    syn = SyntheticLayer(shape, seed=21)
    from expert_side_attention_amd.workload import build_layer, to_device
    layer = build_layer(syn, DEV)
    x = to_device(syn.hidden(), DEV, shape.mode != "f32")
    ref = layer.forward(x).clone()
    out = torch.empty_like(ref)
    iv = torch.int32 if shape.mode == "f32" else torch.int16
    for i in range(24):
        layer.forward(x, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(iv), ref.view(iv)), f"forward {i}"
    layer.close()


@pytest.mark.parametrize("shape", [
    # decode-regime plans: every expert's rows sit in one tile of one kernel,
    # whose per-row arithmetic does not depend on the row's position
    LayerShape("perm_bf16_bm128", T=300, h=256, E=16, k=4, I=256, S=1, Is=128, mode="bf16"),
    LayerShape("perm_bf16_bm64", T=100, h=256, E=32, k=4, I=256, mode="bf16"),
    LayerShape("perm_w8a8_bm128", T=200, h=256, E=8, k=2, I=256, S=1, Is=128, mode="w8a8"),
    LayerShape("perm_w8a8_bm64", T=96, h=256, E=32, k=8, I=128, mode="w8a8"),
    LayerShape("perm_f32", T=64, h=128, E=8, k=2, I=128, S=1, Is=128, mode="f32"),
], ids=lambda s: s.name)
def test_token_permutation_equivariance(shape):
    """Permuting the tokens permutes the output rows, bit for bit: routing,
    dispatch order and tiles change, the arithmetic of each token does not."""
    syn = SyntheticLayer(shape, seed=13)
    from expert_side_attention_amd.workload import build_layer, to_device
    layer = build_layer(syn, DEV)
    x = to_device(syn.hidden(), DEV, shape.mode != "f32")
    perm = torch.randperm(shape.T, generator=torch.Generator().manual_seed(5)).to(DEV)
    a = layer.forward(x).clone()
    b = layer.forward(x[perm].contiguous()).clone()
    torch.cuda.synchronize()
    iv = torch.int32 if shape.mode == "f32" else torch.int16
    assert torch.equal(b.view(iv), a[perm].view(iv))
    layer.close()


def test_two_streams_two_handles_match_serial():
    shape = LayerShape("streams", T=512, h=256, E=16, k=4, I=256, S=1, Is=256, mode="bf16")
    syn = SyntheticLayer(shape, seed=7)
    from expert_side_attention_amd.workload import build_layer, to_device
    l0 = build_layer(syn, DEV, max_tokens=256)
    k = l0._keep
    l1 = type(l0)(mode="bf16", hidden=256, num_experts=16, top_k=4, inter=256,
                  max_tokens=256, router_w=k[0], gate_w=k[2], up_w=k[3], down_w=k[4],
                  num_shared=1, shared_inter=256, sh_gate_w=k[8], sh_up_w=k[9],
                  sh_down_w=k[10])
    xt = to_device(syn.hidden(), DEV, True)
    serial = torch.cat([l0.forward(xt[:256].contiguous()), l0.forward(xt[256:].contiguous())])
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    x0, x1 = xt[:256].contiguous(), xt[256:].contiguous()
    o0, o1 = torch.empty_like(x0), torch.empty_like(x1)
    torch.cuda.synchronize()
    for _ in range(3):
        l0.forward(x0, out=o0, stream=s0)
        l1.forward(x1, out=o1, stream=s1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o0, o1]).view(torch.int16), serial.view(torch.int16))


def test_edge_token_counts_and_errors():
    from expert_side_attention_amd import AfdError
    from expert_side_attention_amd.workload import build_layer, to_device
    shape = LayerShape("edges", T=64, h=128, E=8, k=2, I=128, S=1, Is=128, mode="bf16")
    syn = SyntheticLayer(shape, seed=8)
    layer = build_layer(syn, DEV, max_tokens=64)
    xt = to_device(syn.hidden(), DEV, True)
    full = layer.forward(xt).clone()
    one = layer.forward(xt[:1].contiguous()).clone()
    empty = layer.forward(xt[:0].contiguous())
    torch.cuda.synchronize()
    assert empty.shape == (0, 128)
    assert torch.equal(one.view(torch.int16), full[:1].view(torch.int16))
    big = torch.zeros((65, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(AfdError) as ei:
        layer.forward(big)
    assert ei.value.status == 3  # AFD_ERR_CAPACITY
    with pytest.raises(AfdError) as ei:
        layer.forward(xt, out=xt)
    assert ei.value.status == 1  # aliasing
    # a hidden pointer off the 16-byte grid is refused before any launch
    from expert_side_attention_amd import _ffi as F
    res = torch.empty_like(full)
    with pytest.raises(AfdError) as ei:
        F.afd_ffn_forward(layer._h, xt.data_ptr() + 2, res.data_ptr(), 1,
                          torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == 1 and "aligned" in F.afd_ffn_last_error()


def test_quantiser_all_bf16_values():
    """Every finite bf16 value through the 1x128 quantiser, in rows whose
    group maxima span the whole range (so results land on every E4M3
    binade, subnormals and zero included): codes and scales bit-exact."""
    from expert_side_attention_amd import quantize_fp8_1x128
    from expert_side_attention_amd.workload import to_device
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (allv >> 7) & 0xFF
    vals = allv[exp != 0xFF]                        # drop Inf/NaN
    g = np.random.default_rng(0)
    rows = []
    for rep in range(2):
        p = g.permutation(vals)
        rows.append(p[: (len(p) // 128) * 128].reshape(-1, 128))
    x = np.concatenate(rows)
    x[::7, 5] = 0x0000          # zeros
    x[::11, :] = 0x8000         # all negative-zero rows -> scale 1
    xt = to_device(x, DEV, True)
    q, s = quantize_fp8_1x128(xt)
    torch.cuda.synchronize()
    rq, rs = O.quantize_1x128(O.bf16_to_f64(x).astype(np.float32))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_block_quantiser_matches_oracle():
    from expert_side_attention_amd import quantize_fp8_128x128
    from expert_side_attention_amd.workload import to_device
    g = np.random.default_rng(1)
    w = (g.standard_normal((3, 256, 384)) * 0.02).astype(np.float32)
    w[1, :128, 128:256] *= 1e-30                    # tiny block
    w[2, 128:, :128] = 0                            # zero block
    wb = f32_to_bf16_bits(w)
    q, s = quantize_fp8_128x128(to_device(wb, DEV, True))
    torch.cuda.synchronize()
    for e in range(3):
        rq, rs = O.quantize_128x128(O.bf16_to_f64(wb[e]).astype(np.float32))
        assert np.array_equal(q[e].cpu().numpy(), rq)
        assert np.array_equal(s[e].cpu().numpy(), rs)


def test_fp32_encoder_every_value_in_range():
    """The fp32 1x128 quantiser (the one W8A8 applies to z) on every fp32
    value from 2^-10 (below it everything rounds to zero) to 448, both signs,
    plus a sample of smaller ones: each group of 128 holds 448 and 127 test
    values, so its scale is exactly 1 and every code is the encoding of the
    value itself.  Codes and scales bit-exact against the oracle."""
    from expert_side_attention_amd import quantize_fp8_1x128
    lo_field, hi_field = 117, 135            # fp32 exponent fields of 2^-10 .. 2^8
    m448 = 0x600000                          # 448 = 1.75 * 2^8
    chunks = []
    for f in range(lo_field, hi_field + 1):
        m = np.arange((m448 + 1) if f == hi_field else (1 << 23), dtype=np.uint32)
        chunks.append((np.uint32(f) << np.uint32(23)) | m)
    small = np.random.default_rng(3).integers(0, lo_field << 23, 1 << 20, dtype=np.uint32)
    chunks.append(small)
    checked = 0
    for c in chunks:
        for sign in (0, 1):
            bits = c | np.uint32(sign << 31)
            n = -(-bits.size // 127)
            vals = np.zeros(n * 127, np.uint32)
            vals[: bits.size] = bits
            x = np.empty((n, 128), np.float32)
            x[:, 0] = 448.0
            x[:, 1:] = vals.view(np.float32).reshape(n, 127)
            q, s = quantize_fp8_1x128(torch.from_numpy(x).to(DEV))
            torch.cuda.synchronize()
            rq, rs = O.quantize_1x128(x)
            assert np.all(rs == 1.0)
            assert np.array_equal(s.cpu().numpy(), rs)
            assert np.array_equal(q.cpu().numpy(), rq), f"chunk starting {bits[0]:#x}"
            checked += bits.size
    assert checked > 300_000_000

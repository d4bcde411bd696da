"""The GPU parity rules (tests/parity.py) on the CPU: an fp32 emulation of
the layer's routing and W8A8 z step, built from torch float32 arithmetic
rather than the oracle, must pass every rule, and the same emulation with a
planted mistake must fail it.  This checks that the rules are neither too
tight for a correct fp32 implementation nor too loose to notice a wrong one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from afd_inputs import LayerShape, SyntheticLayer
from oracle import afd_oracle as O

from parity import (check_gpu_logits, check_selection_on_gpu_logits, check_w8a8_z,
                    check_weights_on_gpu_logits, decode_store, logit_abs_sums)


def _routing_fp32(syn):
    """Logits as an fp32 GEMM of the bf16 operands, then the top-k and the
    renormalised softmax in fp32."""
    s = syn.shape
    x = torch.from_numpy(decode_store(syn.hidden(), s.mode)).float()
    wr = torch.from_numpy(decode_store(syn.router_weight(), s.mode)).float()
    l = x @ wr.T
    b = syn.router_bias()
    if b is not None:
        l = l + torch.from_numpy(b)
    l = l.numpy()
    ids = O.select_topk(l.astype(np.float64), s.k)
    sel = np.take_along_axis(l, ids.astype(np.int64), 1)
    e = np.exp(sel - l.max(axis=1, keepdims=True), dtype=np.float32)
    w = (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return l, ids, w


@pytest.mark.parametrize("shape", [
    LayerShape("r_bf16", T=64, h=512, E=16, k=4, I=128, mode="bf16"),
    LayerShape("r_zipf", T=64, h=1024, E=32, k=8, I=128, mode="bf16", router="zipf"),
], ids=lambda s: s.name)
def test_routing_rules_accept_fp32_and_reject_mistakes(shape):
    syn = SyntheticLayer(shape, seed=2)
    orc = O.OracleFFN(syn)
    ref_l, _, _ = orc.route(syn.hidden())
    sums = logit_abs_sums(decode_store(syn.hidden(), shape.mode), orc._wr, orc._b)
    l, ids, w = _routing_fp32(syn)
    check_gpu_logits(l, ref_l, sums, shape.h)
    check_selection_on_gpu_logits(l, ids, shape.k)
    check_weights_on_gpu_logits(w, l, ids)
    # planted mistakes
    with pytest.raises(AssertionError):           # a logit off by 1e-4 relative
        bad = l.copy()
        bad[3, 5] *= 1 + 1e-4
        check_gpu_logits(bad, ref_l, sums, shape.h)
    with pytest.raises(AssertionError):           # two slots swapped
        bad = ids.copy()
        bad[0, [0, 1]] = bad[0, [1, 0]]
        check_selection_on_gpu_logits(l, bad, shape.k)
    with pytest.raises(AssertionError):           # weights off by 1e-5 relative
        check_weights_on_gpu_logits(w * np.float32(1 + 1e-5), l, ids)
    with pytest.raises(AssertionError):           # softmax without renormalisation
        full = np.exp(l - l.max(axis=1, keepdims=True))
        full /= full.sum(axis=1, keepdims=True)
        check_weights_on_gpu_logits(np.take_along_axis(full, ids.astype(np.int64), 1), l, ids)


def _z_trace_fp32(syn, orc, quant=None):
    """Dispatched-row z of a W8A8 layer computed in fp32 (torch float32
    products of the dequantised operands), quantised per row and 128
    channels; `quant` replaces the quantiser to plant a mistake."""
    s = syn.shape
    x = syn.hidden()
    ref = orc.forward(x)
    xin = torch.from_numpy(orc.expert_input(x)[0]).float()
    T, k = s.T, s.k
    R, Z = T * k + s.S * T, max(s.I, s.Is if s.S else 0)
    zq = np.zeros((R, Z), np.uint8)
    zs = np.ones((R, Z // 128), np.float32)
    quant = quant or O.quantize_1x128
    groups = []
    for e in range(s.E):
        rows = np.arange(ref["offsets"][e], ref["offsets"][e + 1])
        groups.append((syn.expert(e), rows, ref["perm"][rows], s.I))
    for j in range(s.S):
        groups.append((syn.shared(j), T * k + j * T + np.arange(T), np.arange(T), s.Is))
    for mats, rows, toks, N in groups:
        if not len(rows):
            continue
        G, U, _ = (torch.from_numpy(m).float() for m in orc._weights(mats))
        xr = xin[torch.from_numpy(np.asarray(toks, np.int64))]
        z = (F.silu(xr @ G.T) * (xr @ U.T)).numpy()
        q, sc = quant(z)
        zq[rows, :N], zs[rows, :N // 128] = q, sc
    return x, {"offsets": ref["offsets"], "perm": ref["perm"], "z_q": zq, "z_s": zs}


def test_w8a8_z_rule_accepts_fp32_and_rejects_mistakes():
    shape = LayerShape("z_w8a8", T=48, h=512, E=8, k=2, I=256, S=1, Is=384, mode="w8a8")
    syn = SyntheticLayer(shape, seed=4)
    orc = O.OracleFFN(syn)
    x, tr = _z_trace_fp32(syn, orc)
    rows, frac, _ = check_w8a8_z(orc, x, tr)
    assert rows == 48 * 2 + 48 and frac > 0.999

    def wrong_axis(z):                            # groups of 128 consecutive rows
        n = -(-z.shape[0] // 128) * 128
        zp = np.zeros((n, z.shape[1]), np.float32)
        zp[:z.shape[0]] = z
        q, s = O.quantize_1x128(zp.T)
        qq = q.T[:z.shape[0]]
        ss = np.repeat(s.T, 128, axis=0)[:z.shape[0], ::1]
        return qq, np.ascontiguousarray(ss[:, :z.shape[1] // 128])

    def half_scale(z):                            # scale of z / 2 stored with z's codes
        q, _ = O.quantize_1x128(z)
        _, s = O.quantize_1x128(z / 2)
        return q, s

    def no_quant(z):                              # z truncated to E4M3 without a scale
        return O.e4m3_encode(z), np.ones((z.shape[0], z.shape[1] // 128), np.float32)

    for planted in (wrong_axis, half_scale, no_quant):
        _, bad = _z_trace_fp32(syn, orc, quant=planted)
        with pytest.raises(AssertionError):
            check_w8a8_z(orc, x, bad)

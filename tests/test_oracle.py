"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes one part of the layer by something other than the oracle's
own formula: published facts of the OCP E4M3FN format, brute-force
enumeration, closed forms, special cases that reduce to a torch library
routine, and invariants of the dispatch permutation.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from afd_inputs import (CONFIGS, LayerShape, SyntheticLayer, f32_to_bf16_bits,
                        tie_case)
from oracle import afd_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_bf16(bits):
    """Decode bf16 bit patterns through torch's own bfloat16 type."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double()


class ArraySource:
    """Weight source built from explicit arrays (storage form)."""

    def __init__(self, shape, wr, b, experts, shared=()):
        self.shape, self._wr, self._b = shape, wr, b
        self._experts, self._shared = experts, shared

    def router_weight(self):
        return self._wr

    def router_bias(self):
        return self._b

    def expert(self, e):
        return self._experts[e]

    def shared(self, j):
        return self._shared[j]


# ---------------------------------------------------------------- E4M3 codec
def test_e4m3_table_matches_ocp_facts():
    v = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    # published E4M3FN facts: max normal 448, min normal 2^-6, min subnormal
    # 2^-9, max subnormal 7 * 2^-9, 1.0 = 0x38, NaN only at S.1111.111,
    # no infinities, 254 finite values
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x38] == 1.0
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254 and not np.isinf(v).any()
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # monotone codes
    assert np.array_equal(v[0x80:0xFF], -pos)           # sign symmetry
    # constant spacing inside each binade: 2^(e-3) for [2^e, 2^(e+1))
    for e in range(-6, 9):
        inb = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(inb) == (7 if e == 8 else 8)     # 480 would be NaN
        assert np.all(np.diff(inb) == 2.0 ** (e - 3))


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def _brute_encode(x):
    """Nearest finite E4M3 value by exhaustive distance, ties to even code,
    saturating beyond 448; sign of the input kept."""
    grid = [(c, float(O.e4m3_decode(np.uint8(c)))) for c in range(0x7F)]
    out = []
    for v in np.asarray(x, np.float32).astype(np.float64):
        a = min(abs(v), 448.0)
        best = min(grid, key=lambda cg: (abs(cg[1] - a), cg[0] & 1))
        c = best[0]
        out.append(c | 0x80 if math.copysign(1.0, v) < 0 else c)
    return np.array(out, np.uint8)


def test_e4m3_encode_vs_brute_force():
    g = np.random.default_rng(1)
    grid = O.e4m3_positive_grid()
    mids = (grid[:-1] + grid[1:]) / 2               # exact ties
    xs = np.concatenate([
        g.standard_normal(3000) * 50, g.standard_normal(1000) * 1e-2,
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30, 2.0 ** -10,
         -2.0 ** -11, 3 * 2.0 ** -10, 1e-40]]).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(xs), _brute_encode(xs))


# ---------------------------------------------------------------- quantisers
def test_quantize_1x128_scale_and_bounds():
    g = np.random.default_rng(2)
    x = (g.standard_normal((5, 512)) * 3).astype(np.float32)
    x[2] = 0.0                                         # all-zero row -> s = 1
    x[3, 128:256] *= 1000                               # distinct group amax
    q, s = O.quantize_1x128(x)
    assert q.shape == (5, 512) and s.shape == (5, 4)
    amax = np.abs(x.reshape(5, 4, 128)).max(axis=2)
    ref_s = np.float32(amax / np.float32(448))          # fp32 division
    ref_s = np.where(amax == 0, np.float32(1), ref_s)
    assert np.array_equal(s, ref_s)
    # group maxima encode to +-448
    for r in (0, 1, 3, 4):
        for gi in range(4):
            grp = x[r, gi * 128:(gi + 1) * 128]
            i = np.argmax(np.abs(grp))
            assert q[r, gi * 128 + i] in (0x7E, 0xFE)
    assert np.all(q[2] == 0)
    # error within half a grid spacing: 2^-4 relative for normals,
    # 2^-10 * s absolute for subnormals
    deq = O.e4m3_decode(q).reshape(5, 4, 128) * s[..., None]
    err = np.abs(deq - x.reshape(5, 4, 128))
    bound = np.maximum(np.abs(x.reshape(5, 4, 128)) * 2.0 ** -4,
                       s[..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantize_128x128_block_layout():
    # block (i, j) gets amax 448 * 2^(i + 3j): any transposed or shifted block
    # index shows up in the scales.
    R, C = 3 * 128, 2 * 128
    w = np.zeros((R, C), np.float32)
    for i in range(3):
        for j in range(2):
            blk = np.full((128, 128), 0.5, np.float32)
            blk[7 + i, 11 + j] = 448.0
            w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = blk * 2.0 ** (i + 3 * j)
    q, s = O.quantize_128x128(w)
    assert s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            assert s[i, j] == 2.0 ** (i + 3 * j)
            assert q[i * 128 + 7 + i, j * 128 + 11 + j] == 0x7E
            assert q[i * 128, j * 128] == 0x30          # 0.5 = 2^-1 -> e=6
    assert np.array_equal(O.dequantize_128x128(q, s), w.astype(np.float64))


# ---------------------------------------------------------------- routing
def test_router_logits_vs_loops():
    g = np.random.default_rng(3)
    x = g.standard_normal((4, 16))
    w = g.standard_normal((5, 16))
    b = g.standard_normal(5)
    l = O.router_logits(x, w, b)
    for t in range(4):
        for e in range(5):
            ref = math.fsum(x[t, i] * w[e, i] for i in range(16)) + b[e]
            assert abs(l[t, e] - ref) < 1e-12


def _brute_topk_set(l, k):
    """The unique k-subset whose members all beat all non-members under the
    key (larger logit, then smaller index)."""
    E = len(l)
    beats = lambda a, c: l[a] > l[c] or (l[a] == l[c] and a < c)
    found = [S for S in itertools.combinations(range(E), k)
             if all(beats(a, c) for a in S for c in range(E) if c not in S)]
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_brute_force(k):
    g = np.random.default_rng(4 + k)
    l = g.standard_normal((40, 8))
    l[:, 5] = l[:, 2]                                   # exact ties
    l[::3, 7] = l[::3, 0]
    ids = O.select_topk(l, k)
    for t in range(40):
        S = _brute_topk_set(l[t], k)
        assert sorted(ids[t].tolist()) == list(S)
        # slots in order: logit descending, index ascending
        key = [(-l[t, e], e) for e in ids[t]]
        assert key == sorted(key)


def test_topk_exact_ties_integer_inputs():
    x, w = tie_case(T=32, h=256, E=16, seed=5)
    l = O.router_logits(O.bf16_to_f64(x), O.bf16_to_f64(w))
    assert np.all(l == np.round(l))                    # integer logits
    ids = O.select_topk(l, 4)
    for t in range(32):
        assert sorted(ids[t].tolist()) == list(_brute_topk_set(l[t], 4))
    # duplicated router rows give equal logits: the lower index must win
    assert np.any(l[:, 0] == l[:, 1])


def test_weights_closed_forms():
    g = np.random.default_rng(6)
    l = g.standard_normal((50, 8)) * 3
    ids = O.select_topk(l, 2)
    w = O.topk_weights(l, ids)
    a = np.take_along_axis(l, ids.astype(np.int64), 1)
    # k = 2: w0 = sigmoid(l0 - l1)
    assert np.allclose(w[:, 0], 1 / (1 + np.exp(a[:, 1] - a[:, 0])), atol=1e-15)
    # general k: full softmax, then renormalised over the selected experts
    ids5 = O.select_topk(l, 5)
    p = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    ps = np.take_along_axis(p, ids5.astype(np.int64), 1)
    assert np.allclose(O.topk_weights(l, ids5), ps / ps.sum(1, keepdims=True),
                       atol=1e-15)
    assert np.allclose(O.topk_weights(l, ids5).sum(1), 1.0, atol=1e-15)


# ---------------------------------------------------------------- dispatch
def _naive_dispatch(ids, E):
    T, k = len(ids), len(ids[0])
    perm, counts, slot_row = [], [], {}
    for e in range(E):
        c = 0
        for t in range(T):
            for j in range(k):
                if ids[t][j] == e:
                    slot_row[(t, j)] = len(perm)
                    perm.append(t)
                    c += 1
        counts.append(c)
    return counts, perm, slot_row


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (37, 8, 3), (64, 16, 8), (1, 4, 4)])
def test_dispatch_invariants_and_naive(T, E, k):
    g = np.random.default_rng(T * 31 + E)
    l = g.standard_normal((T, E))
    ids = O.select_topk(l, k)
    counts, offsets, perm, slot_row = O.dispatch(ids, E)
    nc, nperm, nslot = _naive_dispatch(ids.tolist(), E)
    assert counts.tolist() == nc and perm.tolist() == nperm
    for (t, j), r in nslot.items():
        assert slot_row[t, j] == r
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.bincount(perm, minlength=T), np.full(T, k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                # ascending tokens
    # slot_row is the inverse: the row of (t, j) holds token t of expert ids[t,j]
    for t in range(T):
        for j in range(k):
            r = slot_row[t, j]
            assert perm[r] == t
            assert offsets[ids[t, j]] <= r < offsets[ids[t, j] + 1]


# ---------------------------------------------------------------- experts
def _small_shape(**kw):
    base = dict(name="t", T=12, h=128, E=1, k=1, I=256, S=0, Is=0, mode="bf16")
    base.update(kw)
    return LayerShape(**base)


def test_dense_swiglu_special_case():
    """E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN."""
    shp = _small_shape()
    L = SyntheticLayer(shp, seed=7)
    out = O.OracleFFN(L).forward(L.hidden())["out"]
    G, U, D = (torch_bf16(m) for m in L.expert(0))
    x = torch_bf16(L.hidden())
    ref = (F.silu(x @ G.T) * (x @ U.T)) @ D.T
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_uniform_logits_mean_of_experts():
    """W_r = 0 and k = E: every expert is selected in index order with weight
    1/E, so the layer is the mean of all experts."""
    shp = _small_shape(E=4, k=4)
    L = SyntheticLayer(shp, seed=8)
    zero_wr = np.zeros((4, 128), np.uint16)
    src = ArraySource(shp, zero_wr, None, [L.expert(e) for e in range(4)])
    res = O.OracleFFN(src).forward(L.hidden())
    assert np.array_equal(res["ids"], np.tile(np.arange(4), (12, 1)))
    assert np.allclose(res["w"], 0.25, atol=1e-15)
    x = torch_bf16(L.hidden())
    ref = sum((F.silu(x @ torch_bf16(L.expert(e)[0]).T)
               * (x @ torch_bf16(L.expert(e)[1]).T)) @ torch_bf16(L.expert(e)[2]).T
              for e in range(4)) / 4
    assert np.allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_combine_pairs_weights_with_experts():
    """Experts that differ only by a scalar factor c_e on the down matrix:
    out[t] = (sum_j w[t,j] c_{ids[t,j]}) y[t].  A weight applied to the wrong
    expert's output breaks the ratio."""
    shp = _small_shape(E=6, k=3, T=20)
    L = SyntheticLayer(shp, seed=9)
    G, U, D = L.expert(0)
    Df = O.bf16_to_f64(D).astype(np.float32)
    experts = [(G, U, f32_to_bf16_bits(Df * np.float32(2.0 ** e))) for e in range(6)]
    src = ArraySource(shp, L.router_weight(), None, experts)
    res = O.OracleFFN(src).forward(L.hidden())
    x = torch_bf16(L.hidden())
    y = ((F.silu(x @ torch_bf16(G).T) * (x @ torch_bf16(U).T))
         @ torch_bf16(D).T).numpy()
    factor = (res["w"] * 2.0 ** res["ids"]).sum(1)
    assert np.allclose(res["out"], factor[:, None] * y, rtol=1e-12, atol=1e-14)


def test_shared_expert_is_added_with_weight_one():
    shp1 = _small_shape(E=4, k=2, S=1, Is=128)
    shp0 = _small_shape(E=4, k=2)
    L = SyntheticLayer(shp1, seed=10)
    experts = [L.expert(e) for e in range(4)]
    with_s = ArraySource(shp1, L.router_weight(), None, experts, [L.shared(0)])
    without = ArraySource(shp0, L.router_weight(), None, experts)
    x = L.hidden()
    diff = (O.OracleFFN(with_s).forward(x)["out"]
            - O.OracleFFN(without).forward(x)["out"])
    xt = torch_bf16(x)
    G, U, D = (torch_bf16(m) for m in L.shared(0))
    ref = (F.silu(xt @ G.T) * (xt @ U.T)) @ D.T
    assert np.allclose(diff, ref.numpy(), rtol=1e-10, atol=1e-13)


def test_token_subset_and_permutation_equivariance():
    shp = _small_shape(E=8, k=2, T=24, S=1, Is=128)
    L = SyntheticLayer(shp, seed=11)
    orc = O.OracleFFN(L)
    x = L.hidden()
    full = orc.forward(x)
    sub = orc.forward(x, tokens=[3, 17, 5])
    assert np.array_equal(sub["ids"], full["ids"][[3, 17, 5]])
    assert np.allclose(sub["out"], full["out"][[3, 17, 5]], rtol=0, atol=1e-15)
    p = np.random.default_rng(0).permutation(24)
    perm_res = orc.forward(x[p])
    assert np.allclose(perm_res["out"], full["out"][p], rtol=0, atol=1e-15)
    assert np.array_equal(perm_res["counts"], full["counts"])


def test_w8a8_error_band():
    """W8A8 against the same layer with the same (quantised) weights but exact
    activations: the only differences are the two activation quantisations,
    whose element error is at most 2^-4 relative (about 2-3% rms), so the
    output error must be clearly non-zero and well below 6%."""
    shp = _small_shape(E=4, k=2, T=32, h=256, I=256, S=1, Is=256, mode="w8a8")
    L = SyntheticLayer(shp, seed=12)
    res = O.OracleFFN(L).forward(L.hidden())
    x = torch_bf16(L.hidden())
    w = torch.from_numpy(res["w"])

    def deq(m):
        q, s = O.quantize_128x128(O.bf16_to_f64(m).astype(np.float32))
        return torch.from_numpy(O.dequantize_128x128(q, s))

    def ffn(mats, rows):
        G, U, D = (deq(m) for m in mats)
        return (F.silu(rows @ G.T) * (rows @ U.T)) @ D.T

    ref = ffn(L.shared(0), x)
    for t in range(32):
        for j in range(2):
            ref[t] += w[t, j] * ffn(L.expert(int(res["ids"][t, j])), x[t:t + 1])[0]
    ref = ref.numpy()
    rel = np.linalg.norm(res["out"] - ref) / np.linalg.norm(ref)
    assert 2e-3 < rel < 6e-2, rel
    # the layer input bytes are the 1x128 quantiser's output
    q, s = O.quantize_1x128(O.bf16_to_f64(L.hidden()).astype(np.float32))
    assert np.array_equal(res["x_q"], q) and np.array_equal(res["x_s"], s)


def _e4m3_grid_from_definition():
    """Finite non-negative E4M3FN values built from the format's definition
    (4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent
    field 0, exponent 15 with mantissa 7 reserved for NaN); index == code."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def _requantised_z_brute(z64):
    """What the W8A8 layer feeds its down product, rebuilt step by step
    without the oracle's quantiser: z rounded to fp32; per row, groups of 128
    consecutive channels; s = fp32 quotient amax / 448 (1 if that is 0);
    each element divided by s in fp32 and replaced by the nearest E4M3 value
    (ties to the even code, saturating at 448); value = code value * s."""
    grid = _e4m3_grid_from_definition()
    z32 = np.asarray(z64, np.float64).astype(np.float32)
    out = np.empty(z32.shape, np.float64)
    for r in range(z32.shape[0]):
        for g0 in range(0, z32.shape[1], 128):
            grp = z32[r, g0:g0 + 128]
            amax = np.float32(np.max(np.abs(grp)))
            s = np.float32(amax / np.float32(448.0))
            if amax == 0 or s == 0:
                s = np.float32(1.0)
            v = (grp / s).astype(np.float32).astype(np.float64)
            a = np.minimum(np.abs(v), 448.0)
            d = np.abs(a[:, None] - grid[None, :])
            best = d.min(axis=1, keepdims=True)
            cand = d == best
            # among equally near grid values take the even code
            code = np.where(cand & (np.arange(len(grid)) % 2 == 0)[None, :],
                            np.arange(len(grid))[None, :], 10 ** 6).min(axis=1)
            code = np.where(cand.sum(axis=1) == 1, d.argmin(axis=1), code)
            out[r, g0:g0 + 128] = np.copysign(grid[code], v) * np.float64(s)
    return out


def _z_pin_holds(swiglu_fn):
    """D = identity, so swiglu(quant_z=True) must return the re-quantised z
    itself, bit for bit.  Rows and groups span several orders of magnitude so
    that a scale taken over the wrong set of elements changes the result."""
    g = np.random.default_rng(31)
    n, h = 256, 256
    x = O.bf16_to_f64(f32_to_bf16_bits(g.standard_normal((n, h)).astype(np.float32)))
    x *= (2.0 ** g.integers(-6, 4, size=(n, 1)))
    G = O.bf16_to_f64(f32_to_bf16_bits((g.standard_normal((h, h)) * 0.05).astype(np.float32)))
    U = O.bf16_to_f64(f32_to_bf16_bits((g.standard_normal((h, h)) * 0.05).astype(np.float32)))
    U[128:] *= 64.0                                   # second channel group much larger
    D = np.eye(h)
    got = swiglu_fn(x, G, U, D, quant_z=True)
    xt = torch.from_numpy(x)
    z = (F.silu(xt @ torch.from_numpy(G).T) * (xt @ torch.from_numpy(U).T)).numpy()
    return np.array_equal(got, _requantised_z_brute(z))


def test_w8a8_z_requantisation_step():
    """The W8A8 re-quantisation of z between the two expert products (W8A8
    precision: vLLM AFD plugin page, "效能基準測試"), pinned bit for bit
    against a brute-force rebuild from the E4M3 definition."""
    assert _z_pin_holds(O.swiglu)


def _mutant_no_requant(xr, G, U, D, quant_z=False):
    return (O.silu(xr @ G.T) * (xr @ U.T)) @ D.T


def _mutant_wrong_axis(xr, G, U, D, quant_z=False):
    z = O.silu(xr @ G.T) * (xr @ U.T)
    q, s = O.quantize_1x128(z.astype(np.float32).T)   # groups of 128 tokens
    return O.dequantize_1x128(q, s).T @ D.T


def _mutant_no_fp32_rounding(xr, G, U, D, quant_z=False):
    z = O.silu(xr @ G.T) * (xr @ U.T)                 # scale from the fp64 z
    R, C = z.shape
    grp = z.reshape(R, C // 128, 128)
    s = (np.abs(grp).max(axis=2) / 448.0).astype(np.float32)
    v = (grp / s[..., None].astype(np.float64)).astype(np.float32)
    q = O.e4m3_encode(v).reshape(R, C)
    return O.dequantize_1x128(q, s) @ D.T


def _mutant_fp64_scale(xr, G, U, D, quant_z=False):
    z = (O.silu(xr @ G.T) * (xr @ U.T)).astype(np.float32).astype(np.float64)
    R, C = z.shape
    grp = z.reshape(R, C // 128, 128)
    s = np.abs(grp).max(axis=2) / 448.0               # scale never rounded to fp32
    v = (grp / s[..., None]).astype(np.float32)
    q = O.e4m3_encode(v).reshape(R, C)
    return (O._decode_fast(q).reshape(R, C // 128, 128) * s[..., None]).reshape(R, C) @ D.T


@pytest.mark.parametrize("mutant", [_mutant_no_requant, _mutant_wrong_axis,
                                    _mutant_no_fp32_rounding, _mutant_fp64_scale],
                         ids=["no_requant", "wrong_axis", "no_fp32_rounding", "fp64_scale"])
def test_w8a8_z_pin_rejects_planted_mistakes(mutant):
    """Each plausible mistake in the z step, planted in a copy of the
    oracle's function, fails the pin above."""
    assert not _z_pin_holds(mutant)


def test_w8a8_layer_applies_z_step():
    """E = 1, k = 1, W8A8 with D = (7/16) I: a block scale of exactly 2^-10
    and codes of exactly 448 make the quantised D equal D, so the layer
    output is 7/16 times the re-quantised z of the quantised input and gate /
    up weights (those quantisers are pinned above).  Fails if the layer
    skips, misplaces or changes the z step."""
    shp = _small_shape(T=16, h=256, I=256, mode="w8a8")
    L = SyntheticLayer(shp, seed=13)
    G, U, _ = L.expert(0)
    D = f32_to_bf16_bits(np.eye(256, dtype=np.float32) * np.float32(0.4375))
    src = ArraySource(shp, L.router_weight(), None, [(G, U, D)])
    x = L.hidden()
    out = O.OracleFFN(src).forward(x)["out"]
    q, s = O.quantize_1x128(O.bf16_to_f64(x).astype(np.float32))
    xq = torch.from_numpy(O.dequantize_1x128(q, s))

    def deq(m):
        qq, ss = O.quantize_128x128(O.bf16_to_f64(m).astype(np.float32))
        return torch.from_numpy(O.dequantize_128x128(qq, ss))

    assert torch.equal(deq(D), torch.from_numpy(O.bf16_to_f64(D)))
    z = (F.silu(xq @ deq(G).T) * (xq @ deq(U).T)).numpy()
    assert np.array_equal(out, 0.4375 * _requantised_z_brute(z))


# ---------------------------------------------------------------- pages' figure
def test_comm_volume_figure_from_pages():
    """The A/F page's traffic example (h = 4096, k = 8, FP8) prints about
    131 KB per token per layer for dispatch + combine; its product is
    2 * h * k * 1 B * 2 = 131072 B.  The oracle's dispatch sends each token to
    exactly k expert rows of h elements, which is the h * k factor."""
    with open(os.path.join(GOLDEN, "comm_volume_af_page.json")) as f:
        gold = json.load(f)
    h, k = gold["h"], gold["k"]
    ids = O.select_topk(np.random.default_rng(0).standard_normal((64, 64)), k)
    counts, _, perm, _ = O.dispatch(ids, 64)
    rows_per_token = len(perm) / 64
    bytes_per_token = gold["factor"] * h * rows_per_token * gold["bytes_per_elem"] * 2
    assert bytes_per_token == gold["bytes_per_token_layer"]
    assert abs(bytes_per_token / 1000 - gold["printed_kb"]) < 0.1

"""Plain fp64 reference of one MoE FFN-service layer (CPU, NumPy).

TEST INFRASTRUCTURE ONLY: used by the tests, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product path.  It shares no code,
table or constant generator with the HIP library.

What the layer computes.  On the FFN side of Attention-FFN Disaggregation the
service takes the hidden states the attention side sends, runs the MoE
feed-forward on them and sends the result back (vLLM AFD plugin page,
"系統架構 / 2. FFN Service").  The expert path consists of routing and of
experts that are large matrix products, sparsely activated, with a dispatch
of hidden states to the chosen experts and a combine of their outputs (A/F
分离 page, "为什么要拆" and the "机制" flowchart; vLLM AFD plugin page,
"Attention-FFN 解耦的原理").  The pages leave the exact form open; the
readings taken here are:

  router   logits l = X W_r^T (+ b), fp64;
  top-k    the k experts with the largest logit, ties to the lower index,
           slots ordered by (logit descending, index ascending);
  weights  softmax over all E restricted to the selected k and renormalised,
           i.e. w_j = exp(l_j - m) / sum_j' exp(l_j' - m), m = max_e l_e;
  dispatch stable counting sort of (token, slot) pairs by expert: within an
           expert, tokens ascend; no capacity limit, no dropping;
  experts  SwiGLU: y = D (silu(G x) * (U x)), silu(a) = a / (1 + e^-a);
  shared   always-on shared experts added with weight 1 after the routed sum;
  combine  out[t] = sum_j w[t,j] y[row(t,j)] + sum_s y_s[t].

W8A8 (the plugin page's benchmark precision, "效能基準測試"; FP8 also in the
A/F 分离 page's traffic example, "深入推导"): weights are OCP E4M3FN codes
with one fp32 scale per 128x128 block; activations are quantised per token
per 128 channels before the gate/up product and again (after rounding z to
fp32) before the down product.  The router stays on the unquantised input.
Quantiser: s = fl32(amax / 448), s = 1 when amax = 0 or s underflows to 0;
q = e4m3(fl32(x / s)), round to nearest even on the finite E4M3 grid,
saturating at +-448, keeping the sign of zero.

Everything is computed in fp64 from exactly decoded inputs (bf16, fp32 and
e4m3 x scale are all exact in fp64).  Intermediate rounding of the HIP path
(bf16 z and y) is deliberately not modelled: the comparison tolerance covers
it.

Parity pins (tests/test_oracle.py): dense SwiGLU special case vs a torch
library routine; uniform-logit mean-of-experts case; sum of weights; brute
force subset enumeration for top-k; exact ties; naive dispatch enumeration
and dispatch invariants; the full E4M3 code table against the OCP formula
and the codec's rounding/saturation rules; quantiser scale and block-index
checks; the W8A8 re-quantisation of z bit for bit against a brute-force
rebuild from the E4M3 definition (with identity down weights, also through
the whole layer), with planted mistakes in that step shown to fail; W8A8
error band against the unquantised layer.  No function here is left
unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "e4m3_decode", "e4m3_encode", "e4m3_positive_grid",
    "quantize_1x128", "quantize_128x128", "router_logits", "select_topk",
    "topk_weights", "dispatch", "swiglu", "OracleFFN",
]

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3FN codes: sign s, exponent field e (bias 7), mantissa m.

    e = 0: (-1)^s 2^-6 (m/8); otherwise (-1)^s 2^(e-7) (1 + m/8); the code
    S.1111.111 is NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = s * val
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def e4m3_positive_grid() -> np.ndarray:
    """All finite non-negative E4M3FN values, ascending; index == code."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode fp32 values to E4M3FN codes.

    |v| > 448 saturates to 448; otherwise the nearest grid value, ties to the
    value with an even mantissa.  In the binade [2^e, 2^(e+1)), e >= -6, the
    grid spacing is 2^(e-3); below 2^-6 it is 2^-9 (subnormals).  Dividing by
    the spacing (a power of two, exact) and rounding half-to-even gives the
    grid point; an even multiple of the spacing is an even mantissa.  The
    sign bit of the input is kept, also for results of zero."""
    x = np.asarray(v, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, p = np.frexp(a)                       # a = f 2^p, f in [0.5, 1)
    e = (p - 1).astype(np.int64)             # a in [2^e, 2^(e+1))
    normal = a >= 2.0 ** -6
    spacing = np.where(normal, np.ldexp(1.0, e - 3), 2.0 ** -9)
    n = np.rint(a / spacing)                 # exact division, ties to even
    # normal: value n * 2^(e-3), n in [8, 16] -> exponent field e + 7 and
    # mantissa n - 8 (n = 16 is mantissa 0 of the next binade, i.e. the
    # next code); subnormal: the code is n itself (n = 8 is 2^-6, code 8).
    code = np.where(normal, (e + 7) * 8 + (n.astype(np.int64) - 8),
                    n.astype(np.int64)).astype(np.uint8)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def _scale_of(amax: np.ndarray) -> np.ndarray:
    """s = fl32(amax / 448), replaced by 1 where amax = 0 or s = 0.

    amax is an fp32 value; the fp64 quotient rounded once to fp32 equals the
    correctly rounded fp32 quotient (double rounding is harmless for a
    division with these precisions)."""
    s = (np.asarray(amax, np.float64) / E4M3_MAX).astype(np.float32)
    return np.where((amax == 0) | (s == 0), np.float32(1.0), s).astype(np.float32)


def quantize_1x128(x: np.ndarray):
    """Per-row, per-128-column quantiser.  x: fp32 [R, C], C % 128 == 0.

    Returns (codes uint8 [R, C], scales fp32 [R, C/128])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % 128 == 0
    g = x.reshape(R, C // 128, 128).astype(np.float64)
    s = _scale_of(np.abs(g).max(axis=2))
    v = (g / s[..., None].astype(np.float64)).astype(np.float32)
    return e4m3_encode(v).reshape(R, C), s


def quantize_128x128(w: np.ndarray):
    """Per-128x128-block quantiser.  w: fp32 [R, C], R, C multiples of 128.

    Returns (codes uint8 [R, C], scales fp32 [R/128, C/128]); block (i, j)
    covers rows 128i..128i+127 and columns 128j..128j+127."""
    w = np.asarray(w, dtype=np.float32)
    R, C = w.shape
    assert R % 128 == 0 and C % 128 == 0
    b = w.reshape(R // 128, 128, C // 128, 128).astype(np.float64)
    s = _scale_of(np.abs(b).max(axis=(1, 3)))
    v = (b / s[:, None, :, None].astype(np.float64)).astype(np.float32)
    return e4m3_encode(v).reshape(R, C), s


_DECODE_TABLE = None


def _decode_fast(q: np.ndarray) -> np.ndarray:
    """e4m3_decode through a 256-entry table of its own results."""
    global _DECODE_TABLE
    if _DECODE_TABLE is None:
        _DECODE_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))
    return _DECODE_TABLE[np.asarray(q, np.uint8)]


def dequantize_1x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    R, C = q.shape
    return (_decode_fast(q).reshape(R, C // 128, 128)
            * s.astype(np.float64)[..., None]).reshape(R, C)


def dequantize_128x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    R, C = q.shape
    return (_decode_fast(q).reshape(R // 128, 128, C // 128, 128)
            * s.astype(np.float64)[:, None, :, None]).reshape(R, C)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, wr: np.ndarray, b=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] W_r[e, i] (+ b[e]), fp64.  x [T,h], wr [E,h]."""
    l = np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T
    if b is not None:
        l = l + np.asarray(b, np.float64)[None, :]
    return l


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32: experts ordered by (logit desc, index asc), first k."""
    T, E = logits.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -logits), axis=-1)
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w [T, k]: exp(l_sel - m) / sum exp(l_sel - m), m = max over all E."""
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(np.take_along_axis(logits, ids.astype(np.int64), axis=1) - m)
    return ex / ex.sum(axis=1, keepdims=True)


def dispatch(ids: np.ndarray, E: int):
    """Stable counting sort of (token, slot) pairs by expert.

    Returns counts [E], offsets [E+1] (exclusive scan), perm [T*k] (token of
    each dispatched row; rows of expert e are offsets[e]..offsets[e+1]-1 with
    ascending tokens) and slot_row [T, k] (dispatched row of each pair)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    counts = np.zeros(E, np.int64)
    members = []
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0]
        members.append(toks)
        counts[e] = toks.size
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = (np.concatenate(members) if T * k else np.zeros(0, np.int64))
    slot_row = np.zeros((T, k), np.int64)
    for j in range(k):
        for t in range(T):
            e = ids[t, j]
            slot_row[t, j] = offsets[e] + np.searchsorted(members[e], t)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), slot_row.astype(np.int32))


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu(xr: np.ndarray, G: np.ndarray, U: np.ndarray, D: np.ndarray,
           quant_z: bool = False) -> np.ndarray:
    """y = D (silu(G x) * (U x)) for each row x of xr (all fp64).

    quant_z: W8A8 -- round z to fp32 and pass it through the 1x128 quantiser
    before the down product."""
    z = silu(xr @ G.T) * (xr @ U.T)
    if quant_z:
        q, s = quantize_1x128(z.astype(np.float32))
        z = dequantize_1x128(q, s)
    return z @ D.T


class OracleFFN:
    """The layer on one set of weights, in fp64.

    ``src`` provides the weights in storage form (bf16 bit patterns or fp32):
    ``router_weight()``, ``router_bias()``, ``expert(e)`` -> (gate, up, down)
    and ``shared(j)``; ``shape`` has the sizes (h, E, k, I, S, Is, mode)."""

    def __init__(self, src, shape=None, threads: int = 1):
        self.src = src
        self.threads = max(1, int(threads))
        self.shape = shape if shape is not None else src.shape
        s = self.shape
        assert 1 <= s.k <= s.E
        self._wr = self._decode(src.router_weight())
        b = src.router_bias()
        self._b = None if b is None else np.asarray(b, np.float64)

    # storage -> fp64
    def _decode(self, a):
        if self.shape.mode == "f32":
            return np.asarray(a, np.float32).astype(np.float64)
        return bf16_to_f64(a)

    def _weights(self, mats):
        """Decode one expert's (gate, up, down); W8A8 quantises them first."""
        if self.shape.mode != "w8a8":
            return tuple(self._decode(m) for m in mats)
        out = []
        for m in mats:
            q, s = quantize_128x128(self._decode(m).astype(np.float32))
            out.append(dequantize_128x128(q, s))
        return tuple(out)

    def quantized_weights(self, mats):
        """W8A8 codes and scales of one expert's matrices (for byte parity)."""
        return [quantize_128x128(self._decode(m).astype(np.float32)) for m in mats]

    def route(self, x_store: np.ndarray):
        """Router, top-k and weights for the given tokens' hidden states."""
        x = self._decode(x_store)
        logits = router_logits(x, self._wr, self._b)
        ids = select_topk(logits, self.shape.k)
        return logits, ids, topk_weights(logits, ids)

    def expert_input(self, x_store: np.ndarray):
        """fp64 rows fed to the expert GEMMs (W8A8: quantised and decoded)."""
        x = self._decode(x_store)
        if self.shape.mode != "w8a8":
            return x, None
        q, s = quantize_1x128(x.astype(np.float32))
        return dequantize_1x128(q, s), (q, s)

    def forward(self, x_store: np.ndarray, tokens=None):
        """Run the layer.

        tokens=None: the whole batch; the result also holds the dispatch
        (counts, offsets, perm, slot_row).  Otherwise only the listed tokens
        are computed (routing and outputs of a token do not depend on the
        other tokens of the batch)."""
        s = self.shape
        x_all = x_store
        if tokens is not None:
            tokens = np.asarray(tokens, np.int64)
            x_all = x_store[tokens]
        logits, ids, w = self.route(x_all)
        xin, xq = self.expert_input(x_all)
        n = x_all.shape[0]
        quant_z = s.mode == "w8a8"
        routed = np.zeros((n, s.h), np.float64)
        # y of every (token, slot); experts are independent, so they may be
        # evaluated by several threads (each writes its own (t, j) slots)
        y_slot = np.zeros((n, s.k, s.h), np.float64)

        def run_expert(e):
            hit = np.nonzero(ids == e)
            if hit[0].size == 0:
                return
            G, U, D = self._weights(self.src.expert(e))
            y_slot[hit[0], hit[1]] = swiglu(xin[hit[0]], G, U, D, quant_z)

        if self.threads == 1:
            for e in range(s.E):
                run_expert(e)
        else:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(run_expert, range(s.E)))
        routed = np.einsum("tj,tjh->th", w, y_slot)
        out = routed.copy()
        for j in range(s.S):
            G, U, D = self._weights(self.src.shared(j))
            out += swiglu(xin, G, U, D, quant_z)
        res = {"logits": logits, "ids": ids, "w": w, "out": out}
        if xq is not None:
            res["x_q"], res["x_s"] = xq
        if tokens is None:
            (res["counts"], res["offsets"], res["perm"],
             res["slot_row"]) = dispatch(ids, s.E)
        return res

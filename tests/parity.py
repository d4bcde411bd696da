"""Comparison rules shared by the GPU parity tests (HIP path vs fp64 oracle).

Routing: the oracle's logits are fp64, the GPU's fp32 (bf16 products are
exact in fp32, so only the summation order differs).  A GPU selection is
accepted when it is a valid top-k of the oracle logits perturbed by at most
beta[t, e] = (h + 2) 2^-24 (sum_i |x_i w_ei| + |b_e|) per logit -- the
worst-case error bound of an fp32 sum of h exact products plus the bias add.
Where no two candidates are that close, this forces the exact oracle set and
slot order.  Exact ties are tested separately with integer inputs, where the
fp32 sums are exact and the lowest-index rule must hold bit for bit.

Dispatch: given the GPU's ids, counts/offsets/perm/slot_row must equal the
oracle's dispatch of those ids bit for bit.

Router logits (traced): the GPU's fp32 logits must lie within the rigorous
bound beta of the oracle's, and within a realistic one: rounding errors of a
sum of h terms grow like a random walk, so 4 sqrt(h + 2) 2^-24 (sum_i |x_i
w_ei| + |b_e|) leaves a wide margin.  Given its own logits, the GPU's
selection must be bit-exact (the top-k by (logit desc, index asc)) and its
weights must be the renormalised softmax of those logits up to the fp32
rounding of exp, sum and divide.

W8A8 z (traced): the E4M3 codes and 1x128 scales the gate/up step feeds to
the down product, against the oracle's z of the same rows (see check_w8a8_z).

Outputs: rel-L2 <= 5e-3 and max-abs <= 1e-2 max|ref| (fp32, bf16); rel-L2 <=
2e-2 for W8A8.  Tokens whose selected experts differ from the oracle's
(near ties) are excluded from the output comparison and counted.
"""
from __future__ import annotations

import numpy as np

from oracle import afd_oracle as O

TOL = {"f32": (5e-3, 1e-2), "bf16": (5e-3, 1e-2), "w8a8": (2e-2, None)}


def decode_store(a, mode):
    return np.asarray(a, np.float32).astype(np.float64) if mode == "f32" else O.bf16_to_f64(a)


U32 = 2.0 ** -24


def logit_abs_sums(x64, wr64, b):
    """sum_i |x_i w_ei| (+ |b_e|) for every (token, expert)."""
    s = np.abs(x64) @ np.abs(wr64).T
    if b is not None:
        s = s + np.abs(np.asarray(b, np.float64))[None, :]
    return s


def routing_slack(x64, wr64, b, h):
    return (h + 2) * U32 * logit_abs_sums(x64, wr64, b)


def check_gpu_logits(gpu_logits, ref_logits, sums, h):
    """GPU fp32 logits vs the oracle's fp64 logits; returns the largest error
    as a fraction of the rigorous and of the realistic bound."""
    g = np.asarray(gpu_logits, np.float64)
    err = np.abs(g - ref_logits)
    rigorous = (h + 2) * U32 * sums
    realistic = 4.0 * np.sqrt(h + 2) * U32 * sums
    assert np.all(err <= rigorous), f"logit error {err.max():.3e} beyond the worst-case bound"
    worst = np.unravel_index(np.argmax(err / realistic), err.shape)
    assert np.all(err <= realistic), (f"logit error {err[worst]:.3e} at {worst} beyond "
                                      f"{realistic[worst]:.3e}")
    return float(np.max(err / rigorous)), float(np.max(err / realistic))


def check_selection_on_gpu_logits(gpu_logits, gpu_ids, k):
    """Bit-exact: the ids are the top-k of the GPU's own logits, slots by
    (logit descending, index ascending)."""
    want = O.select_topk(np.asarray(gpu_logits, np.float64), k)
    bad = np.nonzero(np.any(np.asarray(gpu_ids) != want, axis=1))[0]
    assert bad.size == 0, f"tokens {bad[:10]} do not take the top-k of their own logits"


def check_weights_on_gpu_logits(gpu_w, gpu_logits, gpu_ids):
    """w_j = exp(l_j - m) / sum_j' exp(l_j' - m) of the GPU's own logits (m =
    max over all experts), computed in fp64.  fp32 error budget per weight:
    l_j - m rounds with relative error u, i.e. |l_j - m| u in the exponent;
    expf within 2 ulp; the sum of k terms; the divide: |dw_j| <= w_j 2 u
    (|l_j - m| + max_j' |l_j' - m| + k + 6), u = 2^-24.  Returns the largest
    relative error."""
    l = np.asarray(gpu_logits, np.float64)
    ids = np.asarray(gpu_ids, np.int64)
    k = ids.shape[1]
    m = l.max(axis=1, keepdims=True)
    d = m - np.take_along_axis(l, ids, 1)
    ex = np.exp(-d)
    ref = ex / ex.sum(axis=1, keepdims=True)
    bound = ref * 2 * U32 * (d + d.max(axis=1, keepdims=True) + k + 6)
    err = np.abs(np.asarray(gpu_w, np.float64) - ref)
    assert np.all(err <= bound), f"weights off by {np.max(err / ref):.3e} relative"
    return float(np.max(err / ref))


def _e4m3_half_spacing(v):
    """Half the E4M3 grid spacing at |v| (v already divided by the scale)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


def check_w8a8_z(orc, x_store, tr, groups=None):
    """The E4M3 z and 1x128 scales of dispatched rows (traced z_q / z_s) vs
    the oracle's z of the same (token, expert) pairs, in fp64 from the same
    quantised input and weights.  Per element, the GPU's accumulation may
    differ from fp64 by dz <= 1.1 |u| dg + |silu(g)| du + 4 u |z| with dg, du
    <= c sum_i |x_i w_i|.  The gfx950 fp8 MFMAs do not sum their 32 products
    in IEEE fp32: product bits more than about 13 below the largest product
    of one instruction are dropped (measured with a small in-bounds probe of
    the 16x16x32 fp8 instruction: 448 + 127 * 2^-9 sums to 448.234375).
    Those truncations add like a random walk over the h / 32 instructions of
    a dot product whose largest products are a few times the mean, so c =
    2^-13 sqrt(32) / sqrt(h / 32) = 2^-8 / sqrt(h), or the fp32 random-walk
    bound 4 sqrt(h) 2^-24 where that is larger.
    Checks: each group's scale within (max dz) / 448 + 2 u s of fl32(amax /
    448); each group's largest code decodes to +-448; every dequantised
    element within the E4M3 rounding of the GPU's z (half a grid step at
    z / s) of the oracle's z, plus dz; and at least 99% of the codes equal
    the oracle's own encoding.  groups: the routed experts to check (default
    all); shared rows are always checked.  Returns (rows checked, fraction
    of equal codes, largest scale deviation as a fraction of its bound)."""
    s = orc.shape
    xin, _ = orc.expert_input(x_store)
    T, k = xin.shape[0], s.k
    Tk = T * k
    offsets = np.asarray(tr["offsets"], np.int64)
    perm = np.asarray(tr["perm"], np.int64)
    zq, zs = np.asarray(tr["z_q"]), np.asarray(tr["z_s"])
    todo = []
    for e in (range(s.E) if groups is None else groups):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size:
            todo.append((orc.src.expert(e), rows, perm[rows], s.I))
    for j in range(s.S):
        todo.append((orc.src.shared(j), Tk + j * T + np.arange(T), np.arange(T), s.Is))
    c = max(4.0 * np.sqrt(s.h) * U32, 2.0 ** -8 / np.sqrt(s.h))
    n_rows = n_eq = n_el = 0
    worst = 0.0
    for mats, rows, toks, N in todo:
        G, U, _ = orc._weights(mats)
        xr = xin[toks]
        g, u = xr @ G.T, xr @ U.T
        sg, su = np.abs(xr) @ np.abs(G).T, np.abs(xr) @ np.abs(U).T
        z = O.silu(g) * u
        dz = 1.1 * np.abs(u) * c * sg + np.abs(O.silu(g)) * c * su + 4 * U32 * np.abs(z)
        z32 = z.astype(np.float32).astype(np.float64)
        q = zq[rows, :N]
        sc = zs[rows, :N // 128].astype(np.float64)
        R = len(rows)
        zg = z32.reshape(R, N // 128, 128)
        amax = np.abs(zg).max(axis=2)
        s_ref = (amax / 448.0).astype(np.float32).astype(np.float64)
        s_ref = np.where((amax == 0) | (s_ref == 0), 1.0, s_ref)
        ds = dz.reshape(R, N // 128, 128).max(axis=2) / 448.0 + 2 * U32 * s_ref
        worst = max(worst, float(np.max(np.abs(sc - s_ref) / ds)))
        assert np.all(np.abs(sc - s_ref) <= ds), \
            f"z scales off by {np.max(np.abs(sc - s_ref) / s_ref):.3e} relative"
        vals = O.e4m3_decode(q).reshape(R, N // 128, 128)
        nz = np.abs(vals).max(axis=2) > 0
        assert np.all(np.abs(vals).max(axis=2)[nz] == 448.0), "a group's largest code is not 448"
        deq = vals * sc[..., None]
        tol = (_e4m3_half_spacing(deq / sc[..., None]) * sc[..., None] * (1 + 1e-6)
               + 2 * dz.reshape(R, N // 128, 128))
        err = np.abs(deq - zg)
        assert np.all(err <= tol), f"dequantised z off by {np.max(err - tol):.3e} beyond its bound"
        own = O.e4m3_encode((zg / s_ref[..., None]).astype(np.float32)).reshape(R, N)
        n_eq += int(np.sum(own == q))
        n_el += q.size
        n_rows += R
    frac = n_eq / max(n_el, 1)
    assert frac >= 0.99, f"only {frac:.4f} of the z codes equal the oracle's"
    return n_rows, frac, worst


def check_routing(logits, beta, gpu_ids, k):
    """Assert the GPU ids are a valid top-k within the slack; return the
    boolean mask of tokens whose ids differ from the oracle's exactly."""
    T, E = logits.shape
    oracle_ids = O.select_topk(logits, k)
    g = np.asarray(gpu_ids, np.int64)
    assert g.shape == (T, k)
    assert np.all((g >= 0) & (g < E))
    for t in range(T):
        assert len(set(g[t].tolist())) == k, f"token {t}: repeated expert {g[t]}"
    lg = np.take_along_axis(logits, g, 1)
    bg = np.take_along_axis(beta, g, 1)
    # slot order: descending logit within the slack
    bad = lg[:, :-1] + bg[:, :-1] < lg[:, 1:] - bg[:, 1:]
    assert not bad.any(), f"slot order violated at tokens {np.nonzero(bad.any(1))[0][:10]}"
    # set: no unselected expert clearly above the last selected one
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, g, True, 1)
    floor = (lg[:, -1] + bg[:, -1])[:, None]
    above = (~sel) & (logits - beta > floor)
    assert not above.any(), f"top-k set violated at tokens {np.nonzero(above.any(1))[0][:10]}"
    return np.any(g != oracle_ids, axis=1)


def check_weights(gpu_w, ref_w, beta, gpu_ids, same):
    """Routing weights: with logit errors |d_i| <= beta_i, log w_j moves by at
    most 2 max_i beta_i, so |dw_j| <= w_j (exp(2 max beta) - 1) (+ fp32 rounding of the
    exp/sum/divide, at most about (k + 3) 2^-24 relative, covered by 1e-6)."""
    g = np.asarray(gpu_w, np.float64)[same]
    r = np.asarray(ref_w, np.float64)[same]
    bmax = np.take_along_axis(beta, np.asarray(gpu_ids, np.int64), 1)[same].max(axis=1,
                                                                                   keepdims=True)
    bound = r * np.expm1(2 * bmax) + 1e-6
    err = np.abs(g - r)
    assert np.all(err <= bound), f"weights off by {err.max():.3e} (max err/bound {np.max(err / bound):.2f})"
    return float(np.max(err / bound)) if err.size else 0.0


def check_dispatch(gpu_tr, E):
    ids = gpu_tr["topk_ids"]
    counts, offsets, perm, slot_row = O.dispatch(ids, E)
    assert np.array_equal(gpu_tr["counts"], counts)
    assert np.array_equal(gpu_tr["offsets"], offsets)
    assert np.array_equal(gpu_tr["perm"], perm)
    assert np.array_equal(gpu_tr["slot_row"], slot_row)


def check_outputs(gpu_out, ref_out, mode, keep=None):
    g = np.asarray(gpu_out, np.float64)
    r = np.asarray(ref_out, np.float64)
    if keep is not None:
        g, r = g[keep], r[keep]
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    mabs = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300)
    rel_tol, max_tol = TOL[mode]
    assert rel <= rel_tol, f"rel-L2 {rel:.3e} > {rel_tol}"
    if max_tol is not None:
        assert mabs <= max_tol, f"max-abs {mabs:.3e} > {max_tol} * max|ref|"
    return rel, mabs

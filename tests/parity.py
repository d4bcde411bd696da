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


def routing_slack(x64, wr64, b, h):
    s = np.abs(x64) @ np.abs(wr64).T
    if b is not None:
        s = s + np.abs(np.asarray(b, np.float64))[None, :]
    return (h + 2) * 2.0 ** -24 * s


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

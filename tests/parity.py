"""Shared helpers of the GPU parity tests: tolerances and comparison rules.

Tolerances (floating point):
  * fp32 path: max over rows of ||o - o_ref||_inf / ||o_ref||_inf <= 1e-4.
  * bf16 path: the same row metric <= 1e-2; lse absolute error <= 1e-2.
  * MXFP4-indexer end-to-end: <= 5e-2.
Top-k (integer result decided by floating point): with s* the oracle's k-th score and
tau = 1e-3 * max(1, |s*|), every index whose oracle score is above s* + tau must be
chosen, every chosen index must have an oracle score >= s* - tau, and the count is
min(k, n).  Outside that tie zone the sets are equal.
"""
from __future__ import annotations

import numpy as np

from oracle import codecs


def row_rel_err(o, o_ref) -> float:
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    D = o.shape[-1]
    a = np.abs(o - o_ref).reshape(-1, D).max(axis=1)
    b = np.abs(o_ref).reshape(-1, D).max(axis=1)
    b = np.where(b > 0, b, 1.0)
    return float((a / b).max()) if a.size else 0.0


def lse_abs_err(lse, lse_ref) -> float:
    lse = np.asarray(lse, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(lse - lse_ref))
    return float(d.max()) if d.size else 0.0


def check_topk(idx_gpu: np.ndarray, s_ref: np.ndarray, n: int, k: int, tau_rel: float = 1e-3):
    """Validate one row of GPU top-k indices against the oracle's float64 scores."""
    idx_gpu = np.asarray(idx_gpu)
    take = min(k, n)
    assert np.all(idx_gpu[take:] == -1), "padding must be -1"
    sel = idx_gpu[:take].astype(np.int64)
    assert np.all(np.diff(sel) > 0), "indices must be strictly ascending"
    assert np.all((sel >= 0) & (sel < n)), "indices must be visible blocks"
    if take == 0:
        return 0
    s = s_ref[:n]
    order = np.argsort(-s, kind="stable")
    s_star = s[order[take - 1]]
    tau = tau_rel * max(1.0, abs(s_star))
    must = np.nonzero(s > s_star + tau)[0]
    assert np.all(np.isin(must, sel)), "a block clearly above the k-th score is missing"
    assert np.all(s[sel] >= s_star - tau), "a block clearly below the k-th score was chosen"
    ref = np.sort(order[:take])
    return int(np.sum(~np.isin(sel, ref)))   # tie-zone swaps (allowed)


def check_mxfp4_rounding(codes, scales, y_ref, tol) -> None:
    """MXFP4 codes [.., C/2] and E8M0 scales [.., C/32] written by a GPU quantiser, against
    the oracle's values y_ref [.., C] and an error bound tol (per element, e.g. the fp32
    accumulation bound of a pooling): each group's shared exponent must be the OCP MX rule's
    exponent (floor(log2 amax) - 2, clamped to [-127, 127]; 0 for an all-zero group) of some
    group maximum within tol of the oracle's, and each element an E2M1 rounding (nearest-even,
    saturating at 6) at that exponent of some value within tol of y_ref.  With tol = 0 only
    the oracle's own encoding passes."""
    y = np.asarray(y_ref, np.float64)
    C = y.shape[-1]
    g = y.reshape(y.shape[:-1] + (C // 32, 32))
    t = np.broadcast_to(np.asarray(tol, np.float64), y.shape).reshape(g.shape)
    X = np.asarray(scales).astype(np.int64) - 127

    def rule(amax):
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
        return np.where(amax > 0, np.clip(e, -127, 127), 0).astype(np.int64)

    a_lo = np.maximum(np.abs(g) - t, 0.0).max(axis=-1)
    a_hi = (np.abs(g) + t).max(axis=-1)
    lo = np.where(a_lo > 0, rule(a_lo), -127)
    ok = ((X >= lo) & (X <= rule(a_hi))) | ((a_lo == 0) & (X == 0))
    assert np.all(ok), "shared exponent outside the range the values allow"
    step = np.ldexp(1.0, X)[..., None]

    def q(v):                                   # E2M1 rounding at the group's exponent, as values
        return codecs.decode_e2m1(codecs._e2m1_code(v / step)) * step

    got = codecs.decode_mxfp4(codes, scales).reshape(g.shape)
    assert np.all((got >= q(g - t)) & (got <= q(g + t))), "an element is not a rounding of its value"

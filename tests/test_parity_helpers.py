"""The comparison rules of the GPU parity tests, checked on the CPU: each accepts what the
oracle itself produces and rejects a planted mistake (planted in a copy of the oracle's
output, never in a GPU result)."""
import numpy as np
import pytest

from oracle import codecs, method
from tests.parity import check_mxfp4_rounding, check_topk, lse_abs_err, row_rel_err


def _values(seed=3):
    r = np.random.default_rng(seed)
    y = r.standard_normal((5, 4, 64)) * np.exp(r.standard_normal((5, 4, 1)) * 2)
    y[0, 0, :32] = 0.0                                # an all-zero group
    y[1, 1, 3] = 1e4                                  # saturation inside a group
    return y.astype(np.float32).astype(np.float64)


def test_mxfp4_rule_accepts_the_oracle_encoding():
    y = _values()
    codes, scales = codecs.encode_mxfp4(y.astype(np.float32))
    check_mxfp4_rounding(codes, scales, y, 0.0)
    # a small bound still accepts it, and accepts the neighbouring rounding of a midpoint
    check_mxfp4_rounding(codes, scales, y, 1e-9 * np.abs(y))


def test_mxfp4_rule_rejects_a_wrong_code_or_scale():
    y = _values()
    codes, scales = codecs.encode_mxfp4(y.astype(np.float32))
    bad = codes.copy()
    bad[2, 3, 5] ^= 0x01                              # one element one grid step off
    with pytest.raises(AssertionError):
        check_mxfp4_rounding(bad, scales, y, 1e-6 * np.abs(y))
    bad_s = scales.copy()
    bad_s[3, 2, 1] += 1                               # shared exponent one too large
    with pytest.raises(AssertionError):
        check_mxfp4_rounding(codes, bad_s, y, 1e-6 * np.abs(y))


def test_topk_rule_accepts_the_oracle_and_rejects_a_swap():
    r = np.random.default_rng(5)
    s = r.standard_normal((1, 1, 500))
    pos = np.array([[4 * 500 - 1]])
    idx = method.topk(s, pos, 4, 32)[0, 0]
    assert check_topk(idx, s[0, 0], 500, 32) == 0
    order = np.argsort(-s[0, 0])
    wrong = np.sort(np.concatenate([order[1:32], order[200:201]]))   # drops the best block
    with pytest.raises(AssertionError):
        check_topk(wrong, s[0, 0], 500, 32)


def test_row_and_lse_metrics():
    o_ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    o = o_ref + np.array([[0.02, 0.0, 0.0], [0.0, 0.0, 0.0]])
    assert row_rel_err(o, o_ref) == pytest.approx(0.01)
    assert lse_abs_err(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.5])) == pytest.approx(0.5)

"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test checks the oracle against a closed form, an invariant, a hand-worked
example (tests/golden/worked_examples.json), a library routine (torch's dtype
casts and scaled_dot_product_attention, numpy sorting), or the loop-based
restatement in oracle/brute.py — chosen so that a dropped term, a wrong sign,
a wrong index or a transposed operand in the oracle fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, codecs, method

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _rng(seed):
    return np.random.default_rng(seed)


# ============================================================ codecs
def test_bf16_decode_all_codes_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    got = codecs.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_encode_matches_torch_rne():
    r = _rng(1)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-39).astype(np.float32),          # subnormals
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.3895314e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.encode_bf16(x), ref)


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = codecs.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_in_range_and_saturates():
    r = _rng(2)
    x = np.concatenate([r.standard_normal(20000) * 30, r.standard_normal(2000) * 1e-3,
                        np.clip(r.standard_normal(2000) * 300, -448, 448)]).astype(np.float32)
    # every midpoint between neighbouring finite codes (exact ties)
    fin = codecs.decode_e4m3(np.arange(0, 127, dtype=np.uint8))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.encode_e4m3(x), ref)
    for v, c in GOLD["e4m3"]["pairs"]:
        assert int(codecs.encode_e4m3(np.array([v], np.float32))[0]) == c, v


def test_e2m1_table_and_mxfp4_worked_block():
    assert list(codecs.decode_e2m1(np.arange(8))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(codecs.decode_e2m1(np.arange(8, 16))) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    g = GOLD["mxfp4_block"]
    x = np.array(g["values"], np.float32)[None, :]
    packed, scales = codecs.encode_mxfp4(x)
    assert int(scales[0, 0]) == g["scale_byte"]
    codes = np.stack([packed[0] & 0xF, packed[0] >> 4], axis=-1).reshape(-1)
    assert list(codes) == g["codes"]


def test_mxfp4_is_nearest_grid_point():
    """Brute force: each decoded element is a nearest point of the block's grid (or +-6 scale)."""
    r = _rng(3)
    x = (r.standard_normal((64, 128)) * np.exp(r.standard_normal((64, 1)) * 3)).astype(np.float32)
    x[5, :32] = 0.0                                               # all-zero block -> scale byte 127
    packed, scales = codecs.encode_mxfp4(x)
    assert scales[5, 0] == 127
    dq = codecs.decode_mxfp4(packed, scales)
    for i in range(x.shape[0]):
        for blk in range(4):
            s = 2.0 ** (int(scales[i, blk]) - 127)
            amax = np.abs(x[i, blk * 32:(blk + 1) * 32]).max()
            if amax > 0:
                assert s == 2.0 ** (math.floor(math.log2(float(amax))) - 2)
            grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6]) * s
            for j in range(blk * 32, (blk + 1) * 32):
                a = abs(float(x[i, j]))
                best = np.abs(grid - a).min()
                assert abs(abs(dq[i, j]) - a) <= best + 1e-30 or (a > 6 * s and abs(dq[i, j]) == 6 * s)
                if dq[i, j] != 0:
                    assert np.sign(dq[i, j]) == np.sign(x[i, j])


def test_fp8_kv_rows_worked_example():
    """A K row of 4 code dims + 2 RoPE dims (D = 6, d_rope = 2) and a V row, decoded by the
    OCP E4M3 definition (bias 7, three mantissa bits, subnormals m * 2^-9) and the bf16
    definition: the scale multiplies the code dims only, bytes are little-endian."""
    k_row = np.array([[0x38, 0xB8, 0x4C, 0x01, 0x80, 0x3F, 0x40, 0xC0]], np.uint8)
    # 0x38 = +1.0, 0xB8 = -1.0, 0x4C = 2^(9-7) * (1 + 4/8) = 6.0, 0x01 = 2^-9;
    # bf16 0x3F80 = 1.0, 0xC040 = -3.0
    got = codecs.decode_fp8_k_rows(k_row, 6, 2, 0.25)
    assert list(got[0]) == [0.25, -0.25, 1.5, 2.0 ** -11, 1.0, -3.0]
    v_row = np.array([[0x7E, 0xFE, 0x08, 0x00]], np.uint8)          # +448, -448, 2^-6, 0
    assert list(codecs.decode_fp8_v_rows(v_row, 3.0)[0]) == [1344.0, -1344.0, 3.0 * 2.0 ** -6, 0.0]


def test_fp8_kv_rows_round_trip_and_rounding():
    """Values on the E4M3 grid (times a power-of-two scale) and bf16 values survive the
    encoder exactly; off-grid code dims land on a nearest grid point."""
    r = _rng(55)
    codes = r.integers(0, 256, size=(40, 448)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                             # no NaN codes
    k = np.concatenate([codecs.decode_e4m3(codes) * 2.0 ** -5,
                        codecs.decode_bf16(codecs.encode_bf16(r.standard_normal((40, 64))))], axis=1)
    rows = codecs.encode_fp8_k_rows(k.astype(np.float32), 64, 2.0 ** -5)
    assert rows.shape == (40, 576)
    assert np.array_equal(codecs.decode_fp8_k_rows(rows, 512, 64, 2.0 ** -5), k)
    v = r.standard_normal((40, 512)).astype(np.float32)
    dv = codecs.decode_fp8_v_rows(codecs.encode_fp8_v_rows(v, 0.5), 0.5)
    grid = np.unique(np.abs(codecs.decode_e4m3(np.arange(0, 127, dtype=np.uint8)))) * 0.5
    nearest = np.abs(np.abs(v.astype(np.float64))[..., None] - grid).min(axis=-1)
    assert np.all(np.abs(np.abs(dv) - np.abs(v)) <= nearest + 1e-12)


# ============================================================ compression
def _raw(seed, B, T, C):
    r = _rng(seed)
    return r.standard_normal((B, T, C)), r.standard_normal((B, T)), r.standard_normal(T) * 0.1


def test_compress_uniform_gate_is_mean():
    x, _, _ = _raw(10, 2, 64, 5)
    y = method.compress(x, np.full((2, 64), 0.7), np.zeros(4), 4)
    assert np.allclose(y, x.reshape(2, 16, 4, 5).mean(axis=2), rtol=0, atol=1e-14)


def test_compress_4x_then_32x_equals_128x_under_uniform_gates():
    x, _, _ = _raw(11, 2, 512, 6)
    gate = np.repeat(_rng(12).standard_normal((2, 4)), 128, axis=1)     # constant inside each 128-block
    y4 = method.compress(x, gate, np.zeros(4), 4)
    y432 = method.compress(y4, gate[:, ::4], np.zeros(32), 32)
    y128 = method.compress(x, gate, np.zeros(128), 128)
    assert np.allclose(y432, y128, rtol=0, atol=1e-13)


def test_compress_one_hot_gate_and_one_hot_bias_copy_a_token():
    x, _, _ = _raw(13, 1, 32, 3)
    gate = np.zeros((1, 32))
    gate[0, 4 * 2 + 3] = 60.0                                      # block 2, slot 3
    y = method.compress(x, gate, np.zeros(4), 4)
    assert np.allclose(y[0, 2], x[0, 11], atol=1e-20)
    bias = np.array([0.0, 0.0, 60.0, 0.0])                          # slot 2 of every block
    y = method.compress(x, np.zeros((1, 32)), bias, 4)
    assert np.allclose(y[0], x[0, 2::4], atol=1e-20)


def test_compress_worked_two_slot_example():
    g = GOLD["gate_two_slots"]
    x = np.array(g["x"])[None]
    y = method.compress(x, np.array(g["gate"])[None], np.zeros(2), 2)
    assert np.allclose(y[0, 0], g["y"], atol=1e-12)


def test_compress_shift_invariance_and_convexity():
    x, gate, _ = _raw(14, 2, 64, 7)
    bias = _rng(15).standard_normal(8)
    y = method.compress(x, gate, bias, 8)
    gate2 = gate + np.repeat(_rng(16).standard_normal((2, 8)), 8, axis=1)
    assert np.allclose(method.compress(x, gate2, bias, 8), y, atol=1e-13)
    blocks = x.reshape(2, 8, 8, 7)
    assert np.all(y <= blocks.max(axis=2) + 1e-12) and np.all(y >= blocks.min(axis=2) - 1e-12)


def test_compress_matches_brute_force():
    x, gate, _ = _raw(17, 2, 24, 3)
    bias = _rng(18).standard_normal(4) * 0.5
    y = method.compress(x, gate, bias, 4)
    yb = np.array(brute.compress(x.tolist(), gate.tolist(), bias.tolist(), 4))
    assert np.allclose(y, yb, atol=1e-13)


# ============================================================ indexer
def test_indexer_single_head_is_gemv():
    r = _rng(20)
    q = np.abs(r.standard_normal((1, 1, 1, 16)))
    k = np.abs(r.standard_normal((1, 40, 16)))
    s = method.index_scores(q, np.ones((1, 1, 1)), k, np.array([[159]]), 4)
    assert np.allclose(s[0, 0], np.dot(k[0], q[0, 0, 0]), rtol=1e-14)
    s_neg = method.index_scores(-q, np.ones((1, 1, 1)), k, np.array([[159]]), 4)
    assert np.all(s_neg[0, 0] == 0.0)
    s3 = method.index_scores(q, np.full((1, 1, 1), 3.0), k, np.array([[159]]), 4)
    assert np.allclose(s3, 3 * s)


def test_indexer_worked_example_and_visibility():
    g = GOLD["indexer_two_heads"]
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None]
    s = method.index_scores(q, np.array(g["w"])[None, None], k, np.array([[11]]), 4)
    assert np.allclose(s[0, 0], g["scores"])
    r = _rng(21)
    q = r.standard_normal((1, 2, 2, 4))
    k = r.standard_normal((1, 8, 4))
    s = method.index_scores(q, np.ones((1, 2, 2)), k, np.array([[13, 2]]), 4)
    assert np.all(np.isfinite(s[0, 0, :3])) and np.all(np.isneginf(s[0, 0, 3:]))   # floor(14/4) = 3
    assert np.all(np.isneginf(s[0, 1]))                                              # floor(3/4) = 0


def test_indexer_matches_brute_force():
    r = _rng(22)
    q = r.standard_normal((2, 2, 3, 5))
    w = r.random((2, 2, 3))
    k = r.standard_normal((2, 9, 5))
    pos = np.array([[35, 20], [7, 100]])
    s = method.index_scores(q, w, k, pos, 4)
    for b in range(2):
        for t in range(2):
            n = min(9, (pos[b, t] + 1) // 4)
            for j in range(9):
                if j < n:
                    assert math.isclose(s[b, t, j], brute.score(q[b, t].tolist(), w[b, t].tolist(), k[b, j].tolist()),
                                        rel_tol=1e-12, abs_tol=1e-12)
                else:
                    assert s[b, t, j] == -np.inf


def test_indexer_fp4_queries_hand_example_and_grid_identity():
    """FP4-query scores: a hand-quantised query, and queries already on the MXFP4 grid
    (each group's largest magnitude 4 or 6 times a power of two) pass unchanged."""
    # 0.3 alone in its group: shared exponent floor(log2 0.3) - 2 = -4, 0.3 / 2^-4 = 4.8 -> 4,
    # so the query becomes 0.25; key e0, weight 1: score relu(0.25) = 0.25
    q = np.zeros((1, 1, 1, 32), np.float32)
    q[0, 0, 0, 0] = 0.3
    k = np.zeros((1, 3, 32))
    k[0, :, 0] = [1.0, -2.0, 8.0]
    s, codes, scales = method.index_scores_fp4(q, np.ones((1, 1, 1)), k, np.array([[11]]), 4)
    assert np.allclose(s[0, 0], [0.25, 0.0, 2.0], rtol=0, atol=0)
    assert scales[0, 0, 0, 0] == 127 - 4 and (codes[0, 0, 0, 0] & 0xF) == 0b0110       # e2m1 code of 4.0
    r = _rng(23)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    q = grid[r.integers(0, 8, (2, 2, 3, 64))] * np.where(r.random((2, 2, 3, 64)) < 0.5, -1.0, 1.0)
    q[..., ::32] = np.where(r.random(q[..., ::32].shape) < 0.5, 4.0, 6.0)              # group maxima
    q = (q * np.exp2(r.integers(-3, 4, (2, 2, 3, 2))).repeat(32, axis=-1)).astype(np.float32)
    w = r.random((2, 2, 3))
    k = r.standard_normal((2, 9, 64))
    pos = np.array([[35, 20], [7, 100]])
    s4, _, _ = method.index_scores_fp4(q, w, k, pos, 4)
    assert np.array_equal(s4, method.index_scores(q, w, k, pos, 4))


# ============================================================ top-k
def test_topk_worked_ties():
    g = GOLD["topk_ties"]
    s = np.array(g["scores"])[None, None]
    idx = method.topk(s, np.array([[4 * len(g["scores"]) - 1]]), 4, g["k"])
    assert list(idx[0, 0]) == g["idx"]


def test_topk_matches_lexsort_with_many_ties():
    r = _rng(30)
    s = r.integers(0, 7, size=(3, 2, 200)).astype(np.float64)
    s[0, 0, 50:] = 0.0
    pos = np.array([[799, 400], [799, 799], [100, 3]])
    idx = method.topk(s, pos, 4, 17)
    for b in range(3):
        for t in range(2):
            n = min(200, (pos[b, t] + 1) // 4)
            sel = np.sort(np.lexsort((np.arange(n), -s[b, t, :n]))[: min(17, n)])
            exp = np.full(17, -1)
            exp[: len(sel)] = sel
            assert np.array_equal(idx[b, t], exp)
            assert list(idx[b, t]) == brute.select(s[b, t].tolist(), n, 17)


def test_topk_k_at_least_visible_takes_all():
    s = _rng(31).standard_normal((1, 1, 50))
    idx = method.topk(s, np.array([[4 * 10 + 2]]), 4, 16)
    assert list(idx[0, 0]) == list(range(10)) + [-1] * 6


def test_topk_storage_permutation_is_consistent():
    r = _rng(32)
    s = r.standard_normal((1, 1, 64))
    perm = r.permutation(64)
    a = set(method.topk(s, np.array([[999]]), 4, 9)[0, 0])
    b = set(perm[method.topk(s[:, :, perm], np.array([[999]]), 4, 9)[0, 0]])
    assert a == b


# ============================================================ attention
def _attn_case(seed, B=2, Q=2, H=3, D=8, N=24, L=10, m=4):
    r = _rng(seed)
    return dict(q=r.standard_normal((B, Q, H, D)), kc=r.standard_normal((B, N, D)), vc=r.standard_normal((B, N, D)),
                kw=r.standard_normal((B, L, D)), vw=r.standard_normal((B, L, D)),
                win_pos0=np.array([90, 85]), q_pos=np.array([[95, 99], [91, 94]]), m=m)


def _sdpa(q, K, V, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1),
        torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1), scale=scale)
    return out[0].numpy()


def test_csa_with_all_blocks_equals_dense_attention_plus_window():
    c = _attn_case(40)
    W, scale = 6, 0.3
    n = method.visible_blocks(c["q_pos"], c["m"], 24)
    idx = np.full((2, 2, 24), -1)
    for b in range(2):
        for t in range(2):
            idx[b, t, : n[b, t]] = np.arange(n[b, t])
    o, lse = method.csa_attend(c["q"], c["kc"], c["vc"], idx, c["kw"], c["vw"], c["win_pos0"], W, c["q_pos"], scale)
    for b in range(2):
        for t in range(2):
            p = c["q_pos"][b, t]
            wr = [r for r in range(10) if p - W < c["win_pos0"][b] + r <= p]
            K = np.concatenate([c["kc"][b, : n[b, t]], c["kw"][b, wr]])
            V = np.concatenate([c["vc"][b, : n[b, t]], c["vw"][b, wr]])
            assert np.allclose(o[b, t], _sdpa(c["q"][b, t], K, V, scale), atol=1e-12)
            z = scale * c["q"][b, t] @ K.T
            assert np.allclose(lse[b, t], np.log(np.exp(z).sum(axis=1)), atol=1e-12)
    o2, lse2 = method.hca_attend(c["q"], c["kc"], c["vc"], c["m"], c["kw"], c["vw"], c["win_pos0"], W, c["q_pos"], scale)
    assert np.allclose(o2, o, atol=1e-14) and np.allclose(lse2, lse, atol=1e-14)


def test_attention_closed_forms():
    c = _attn_case(41)
    W = 4
    idx = np.array([[[0, 3, 5, -1], [1, 2, 40, -7]], [[7, -1, -1, -1], [-1, -1, -1, -1]]])   # 40, -7 skipped
    vconst = np.broadcast_to(np.arange(8.0), c["vc"].shape).copy()
    o, _ = method.csa_attend(c["q"], c["kc"], vconst, idx, c["kw"], np.broadcast_to(np.arange(8.0), c["vw"].shape),
                             c["win_pos0"], W, c["q_pos"], 0.5)
    assert np.allclose(o, np.arange(8.0), atol=1e-12)                     # V == c  ->  o == c
    # q == 0: every logit is 0, so lse = log |S| (counts worked out by hand)
    _, lse = method.csa_attend(np.zeros_like(c["q"]), c["kc"], c["vc"], idx, c["kw"], c["vw"], c["win_pos0"], W,
                               c["q_pos"], 0.5)
    # b0: win rows pos 90..99; p=95 -> pos 92..95 (4 rows); p=99 -> 96..99 (4). b1: pos 85..94; p=91 -> 88..91; p=94 -> 91..94
    assert np.allclose(lse[0, 0], math.log(3 + 4)) and np.allclose(lse[0, 1], math.log(2 + 4))
    assert np.allclose(lse[1, 0], math.log(1 + 4)) and np.allclose(lse[1, 1], math.log(0 + 4))
    # identical keys -> plain mean of V over the set
    kc = np.broadcast_to(c["kc"][:, :1], c["kc"].shape)
    kw = np.broadcast_to(c["kc"][:, :1], c["kw"].shape)
    o, _ = method.csa_attend(c["q"], kc, c["vc"], idx, kw, c["vw"], c["win_pos0"], W, c["q_pos"], 0.5)
    mean = np.concatenate([c["vc"][0, [0, 3, 5]], c["vw"][0, 2:6]]).mean(axis=0)
    assert np.allclose(o[0, 0], mean, atol=1e-12)


def test_attention_empty_set():
    c = _attn_case(42)
    idx = np.full((2, 2, 3), -1)
    o, lse = method.csa_attend(c["q"], c["kc"], c["vc"], idx, c["kw"], c["vw"], np.array([1000, 1000]), 8,
                               c["q_pos"], 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_attention_matches_masked_brute_force():
    c = _attn_case(43, B=1, Q=2, H=2, D=4, N=12, L=6)
    idx = np.array([[[0, 2, 9, -1], [1, 4, 5, 6]]])
    c["win_pos0"] = np.array([40])
    c["q_pos"] = np.array([[43, 47]])
    o, lse = method.csa_attend(c["q"], c["kc"], c["vc"], idx, c["kw"], c["vw"], c["win_pos0"], 3, c["q_pos"], 0.7)
    for t in range(2):
        for h in range(2):
            ob, lb = brute.attend_masked(c["q"][0, t, h].tolist(), c["kc"][0].tolist(), c["vc"][0].tolist(),
                                         set(idx[0, t].tolist()), c["kw"][0].tolist(), c["vw"][0].tolist(),
                                         40, 3, int(c["q_pos"][0, t]), 0.7)
            assert np.allclose(o[0, t, h], ob, atol=1e-12) and math.isclose(lse[0, t, h], lb, abs_tol=1e-12)


# ============================================================ LSE merge
def test_lse_merge_of_disjoint_parts_reproduces_attention():
    r = _rng(50)
    q = r.standard_normal((4, 8))
    K = r.standard_normal((30, 8))
    V = r.standard_normal((30, 8))
    o, lse = method.attend_rows(q, K, V, 0.4)
    cuts = [0, 7, 8, 30]
    parts = [method.attend_rows(q, K[a:b], V[a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(method.attend_rows(q, K[:0], V[:0], 0.4))                # empty part (lse = -inf)
    om, lm = method.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(om, o, atol=1e-13) and np.allclose(lm, lse, atol=1e-13)
    o1, l1 = method.lse_merge(o[None], lse[None])
    assert np.allclose(o1, o, atol=1e-15) and np.allclose(l1, lse, atol=1e-15)
    oe, le = method.lse_merge(np.zeros((2, 4, 8)), np.full((2, 4), -np.inf))
    assert np.all(oe == 0) and np.all(np.isneginf(le))

"""GPU parity at the benchmark's full sizes and launch configuration, checked against the
float64 oracle on sampled rows / blocks (the oracle cannot afford every output of the
largest configurations in a test, but each sampled output is computed exactly).

* 1M-context CSA decode: B = 8, 262,144 compressed entries, MXFP4 indexer keys (8 heads,
  dim 128), top-1024, 64 heads x 512, 128-token window.
* 1M-context HCA decode: B = 8, 8,192 entries, every row checked; the fused window branch
  against compressed-only + window-only partials combined by lse_merge; the 128x
  compression pre-pass over the full 2^20-token raw stream on sampled blocks.
* 64K-context CSA decode: B = 4, 16,384 entries, bf16 indexer keys, top-512, every row.
* FP8 K|V rows: the 1M-context HCA decode and a 64K-context CSA decode over rows of 448
  E4M3 K codes + 64 bf16 RoPE dims and 512 E4M3 V codes, every row.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import codecs, method
from tests.parity import check_topk, lse_abs_err, row_rel_err

pytestmark = pytest.mark.gpu

L = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global L
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_25_amd as lib_mod
    lib_mod.lib()
    L = lib_mod
    yield
    torch.cuda.empty_cache()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(x32):
    bits = synth.bf16_bits(x32)
    return dev(bits.view(np.int16)).view(torch.bfloat16), bits


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_bf16(t):
    return codecs.decode_bf16(bits_of(t))


# ----------------------------------------------------------------------------------- c4
def test_csa_decode_1m_mxfp4_sampled_rows():
    B, N, HI, DI, k, H, D, Lw, W, m = 8, 262144, 8, 128, 1024, 64, 512, 128, 128, 4
    p = (1 << 20) - 1
    sampled = (0, 5)
    # indexer keys: sampled rows drawn on the host and encoded by the oracle (their codes
    # are what both sides read); the other rows drawn and quantised on the device
    ki = torch.empty((B, N, DI // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, N, DI // 32), dtype=torch.uint8, device="cuda")
    ref_codes = {}
    zero1 = dev(np.zeros(1, np.float32))
    for b in range(B):
        if b in sampled:
            k32 = synth.normal(4100 + b, synth.KI, (N, DI))
            codes, scales = codecs.encode_mxfp4(k32)
            # the library's quantiser on a slice of the same draws: identical bytes
            g = dev(np.zeros((1, 4096), np.float32))
            c_gpu, s_gpu = L.csa_compress(dev(k32[None, :4096]), g, zero1, 1, L.MXFP4_DTYPE)
            assert np.array_equal(c_gpu.cpu().numpy()[0], codes[:4096])
            assert np.array_equal(s_gpu.cpu().numpy()[0], scales[:4096])
            ki[b] = dev(codes)
            ks[b] = dev(scales)
            ref_codes[b] = (codes, scales)
            del k32
        else:
            k32 = synth.device_normal((1, N, DI), 4100 + b, torch.float32)
            L.csa_compress(k32, torch.zeros((1, N), device="cuda"), zero1, 1, L.MXFP4_DTYPE,
                           out=ki[b:b + 1], out_scale=ks[b:b + 1])
            del k32
    qi32 = synth.normal(4, synth.QI, (B, 1, HI, DI))
    qi, qi_bits = bf16_dev(qi32)
    wi = synth.uniform(4, synth.WI, (B, 1, HI))
    pos = np.full((B, 1), p, np.int32)
    idx = L.csa_index_topk(qi, dev(wi), ki, dev(pos), m, k, ki_scale=ks)
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()
    idx_ref = {}
    for b in sampled:
        kdec = codecs.decode_mxfp4(*ref_codes[b])
        s = method.index_scores(codecs.decode_bf16(qi_bits[b:b + 1]), wi[b:b + 1], kdec[None], pos[b:b + 1], m)
        assert check_topk(idx_g[b, 0], s[0, 0], N, k) == 0       # random scores: no tie swaps
        idx_ref[b] = method.topk(s, pos[b:b + 1], m, k)[0, 0]
        assert np.array_equal(idx_g[b, 0], idx_ref[b])
        del kdec
    # attention over the oracle's index set (sampled rows) in the bench's launch configuration
    kc = torch.empty((B, N, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty((B, N, D), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        kc[b] = synth.device_normal((N, D), 4200 + b, torch.bfloat16)
        vc[b] = synth.device_normal((N, D), 4300 + b, torch.bfloat16)
    q, q_bits = bf16_dev(synth.normal(4, synth.Q, (B, 1, H, D)))
    kw, kw_bits = bf16_dev(synth.normal(4, synth.KW, (B, Lw, D)))
    vw, vw_bits = bf16_dev(synth.normal(4, synth.VW, (B, Lw, D)))
    win_pos0 = np.full((B,), p + 1 - Lw, np.int32)
    idx_in = idx.clone()
    for b in sampled:
        idx_in[b, 0] = torch.from_numpy(idx_ref[b].astype(np.int32)).cuda()
    scale = 1.0 / math.sqrt(D)
    o, lse = L.csa_attend(q, kc, vc, idx_in, kw, vw, dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    for b in sampled:
        sel = torch.from_numpy(idx_ref[b].astype(np.int64)).cuda()
        kg, vg = dec(bits_of(kc[b][sel])), dec(bits_of(vc[b][sel]))
        o_r, lse_r = method.csa_attend(dec(q_bits[b:b + 1]), kg[None], vg[None], np.arange(k)[None, None],
                                       dec(kw_bits[b:b + 1]), dec(vw_bits[b:b + 1]), win_pos0[b:b + 1], W,
                                       pos[b:b + 1], scale)
        assert row_rel_err(host_bf16(o[b:b + 1]), o_r) <= 1e-2
        assert lse_abs_err(lse[b:b + 1].cpu().numpy(), lse_r) <= 1e-2
    del kc, vc, ki, ks


# ----------------------------------------------------------------------------------- c3
def test_hca_decode_1m_all_rows_and_lse_merge_of_branches():
    B, N, H, D, Lw, W, m = 8, 8192, 64, 512, 128, 128, 128
    p = (1 << 20) - 1
    kc = synth.device_normal((B, N, D), 3101, torch.bfloat16)
    vc = synth.device_normal((B, N, D), 3102, torch.bfloat16)
    q, q_bits = bf16_dev(synth.normal(3, synth.Q, (B, 1, H, D)))
    kw, kw_bits = bf16_dev(synth.normal(3, synth.KW, (B, Lw, D)))
    vw, vw_bits = bf16_dev(synth.normal(3, synth.VW, (B, Lw, D)))
    pos = np.full((B, 1), p, np.int32)
    win_pos0 = np.full((B,), p + 1 - Lw, np.int32)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.hca_attend(q, kc, vc, m, kw, vw, dev(win_pos0), W, dev(pos), scale)
    # the two branches separately, combined by lse_merge
    o_c, lse_c = L.hca_attend(q, kc, vc, m, kw, vw, dev(win_pos0), 0, dev(pos), scale)
    o_w, lse_w = L.hca_attend(q, kc, vc, m, kw, vw, dev(win_pos0), W, dev(pos), scale, N=0)
    R = B * H
    parts = torch.stack([o_c.reshape(R, D).float(), o_w.reshape(R, D).float()])
    lparts = torch.stack([lse_c.reshape(R), lse_w.reshape(R)])
    o_m, lse_m = L.lse_merge(parts, lparts)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    o_r, lse_r = method.hca_attend(dec(q_bits), dec(bits_of(kc)), dec(bits_of(vc)), m, dec(kw_bits), dec(vw_bits),
                                   win_pos0, W, pos, scale)
    assert row_rel_err(host_bf16(o), o_r) <= 1e-2
    assert lse_abs_err(lse.cpu().numpy(), lse_r) <= 1e-2
    assert row_rel_err(o_m.cpu().numpy().reshape(B, 1, H, D), o_r) <= 1e-2
    assert lse_abs_err(lse_m.cpu().numpy().reshape(B, 1, H), lse_r) <= 1e-2


def test_hca_compress_prepass_1m_sampled_blocks():
    """128x pooling over the full raw stream [8, 2^20, 512] bf16; 34 blocks per sequence
    (first, last and 32 seeded) checked against the oracle."""
    B, T, C, m = 8, 1 << 20, 512, 128
    x = synth.device_normal((B, T, C), 3201, torch.bfloat16)
    gate = synth.device_normal((B, T), 3202, torch.float32)
    bias32 = synth.normal(3, synth.BIAS, (m,), std=0.1)
    y = L.csa_compress(x, gate, dev(bias32), m, torch.bfloat16)
    torch.cuda.synchronize()
    assert y.shape == (B, T // m, C)
    rng = np.random.Generator(np.random.Philox(key=3203))
    for b in range(B):
        blocks = np.concatenate([[0, T // m - 1], rng.integers(1, T // m - 1, size=32)])
        for i in blocks:
            xs = host_bf16(x[b, i * m:(i + 1) * m])[None]
            gs = gate[b, i * m:(i + 1) * m].cpu().numpy()[None]
            y_r = method.compress(xs, gs, bias32, m)[0, 0]
            y_g = host_bf16(y[b, i])
            amax = np.abs(xs).max()
            ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(y_r), 2.0 ** -126))) - 7).astype(np.int64))
            assert np.all(np.abs(y_g - y_r) <= ulp + m * 2.0 ** -21 * amax), (b, i)
    del x, gate, y


# ----------------------------------------------------------------------------------- c2
def test_csa_decode_64k_bf16_all_rows():
    B, N, HI, DI, k, H, D, Lw, W, m = 4, 16384, 8, 128, 512, 64, 512, 128, 128, 4
    p = 65535
    ki, ki_bits = bf16_dev(synth.normal(2, synth.KI, (B, N, DI)))
    qi, qi_bits = bf16_dev(synth.normal(2, synth.QI, (B, 1, HI, DI)))
    wi = synth.uniform(2, synth.WI, (B, 1, HI))
    pos = np.full((B, 1), p, np.int32)
    idx = L.csa_index_topk(qi, dev(wi), ki, dev(pos), m, k)
    kc, kc_bits = bf16_dev(synth.normal(2, synth.KC, (B, N, D)))
    vc, vc_bits = bf16_dev(synth.normal(2, synth.VC, (B, N, D)))
    q, q_bits = bf16_dev(synth.normal(2, synth.Q, (B, 1, H, D)))
    kw, kw_bits = bf16_dev(synth.normal(2, synth.KW, (B, Lw, D)))
    vw, vw_bits = bf16_dev(synth.normal(2, synth.VW, (B, Lw, D)))
    win_pos0 = np.full((B,), p + 1 - Lw, np.int32)
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    s = method.index_scores(dec(qi_bits), wi, dec(ki_bits), pos, m)
    idx_r = method.topk(s, pos, m, k)
    idx_g = idx.cpu().numpy()
    for b in range(B):
        assert check_topk(idx_g[b, 0], s[b, 0], N, k) == 0
    assert np.array_equal(idx_g, idx_r)
    o, lse = L.csa_attend(q, kc, vc, idx, kw, vw, dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    o_r, lse_r = method.csa_attend(dec(q_bits), dec(kc_bits), dec(vc_bits), idx_r, dec(kw_bits), dec(vw_bits),
                                   win_pos0, W, pos, scale)
    assert row_rel_err(host_bf16(o), o_r) <= 1e-2
    assert lse_abs_err(lse.cpu().numpy(), lse_r) <= 1e-2


# ------------------------------------------------------------------- FP8 K|V rows (NEXT 2)
DR = 64      # bf16 RoPE dims at the end of an FP8 K row


def _fp8_rows(cfg, B, N, Lw, D, ks, vs):
    """K/V caches and windows as FP8 K|V byte rows made by the oracle's encoder, with the
    oracle's float64 decoding of those bytes."""
    kc = synth.normal(cfg, synth.KC, (B, N, D))
    vc = synth.normal(cfg, synth.VC, (B, N, D))
    kw = synth.normal(cfg, synth.KW, (B, Lw, D))
    vw = synth.normal(cfg, synth.VW, (B, Lw, D))
    rows = [codecs.encode_fp8_k_rows(kc, DR, ks), codecs.encode_fp8_v_rows(vc, vs),
            codecs.encode_fp8_k_rows(kw, DR, ks), codecs.encode_fp8_v_rows(vw, vs)]
    dec = [codecs.decode_fp8_k_rows(rows[0], D, DR, ks), codecs.decode_fp8_v_rows(rows[1], vs),
           codecs.decode_fp8_k_rows(rows[2], D, DR, ks), codecs.decode_fp8_v_rows(rows[3], vs)]
    return rows, dec


def test_hca_decode_1m_fp8kv_all_rows():
    """The bench's FP8 HCA decode: B = 8, 8,192 entries of 1,088-byte FP8 K|V rows plus a
    128-row FP8 window, 64 heads x 512, non-power-of-two scales; every row against the
    oracle attending over its decoding of the same bytes."""
    B, N, H, D, Lw, W, m = 8, 8192, 64, 512, 128, 128, 128
    ks, vs = 0.37, 1.9
    p = (1 << 20) - 1
    (kcb, vcb, kwb, vwb), (kcd, vcd, kwd, vwd) = _fp8_rows(31, B, N, Lw, D, ks, vs)
    q, q_bits = bf16_dev(synth.normal(31, synth.Q, (B, 1, H, D)))
    pos = np.full((B, 1), p, np.int32)
    win_pos0 = np.full((B,), p + 1 - Lw, np.int32)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.hca_attend_fp8kv(q, dev(kcb), dev(vcb), m, dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos), scale,
                                k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    o_r, lse_r = method.hca_attend(codecs.decode_bf16(q_bits), kcd, vcd, m, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host_bf16(o), o_r) <= 1e-2
    assert lse_abs_err(lse.cpu().numpy(), lse_r) <= 1e-2


def test_csa_decode_64k_fp8kv_all_rows():
    """CSA decode over FP8 K|V rows: B = 4, 16,384 entries, 512 selected per query (a
    seeded index set), 128-row FP8 window; every row against the oracle."""
    B, N, k, H, D, Lw, W = 4, 16384, 512, 64, 512, 128, 128
    ks, vs = 1.0, 0.55
    p = 65535
    (kcb, vcb, kwb, vwb), (kcd, vcd, kwd, vwd) = _fp8_rows(32, B, N, Lw, D, ks, vs)
    idx = synth.sorted_unique_indices(32, synth.IDX, B, N, k).reshape(B, 1, k)
    q, q_bits = bf16_dev(synth.normal(32, synth.Q, (B, 1, H, D)))
    pos = np.full((B, 1), p, np.int32)
    win_pos0 = np.full((B,), p + 1 - Lw, np.int32)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.csa_attend_fp8kv(q, dev(kcb), dev(vcb), dev(idx), dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos),
                                scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    o_r, lse_r = method.csa_attend(codecs.decode_bf16(q_bits), kcd, vcd, idx, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host_bf16(o), o_r) <= 1e-2
    assert lse_abs_err(lse.cpu().numpy(), lse_r) <= 1e-2


# ----------------------------------------------------------------------------------- c5
def _fp8_valid_rounding(codes, exact):
    """Each fp8 code is the nearest-even rounding of `exact` or one of its two neighbours
    (the library pools in fp32, the oracle in fp64)."""
    dec = codecs.decode_e4m3(codes)
    a = np.abs(exact)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = np.ldexp(1.0, (e - 3).astype(np.int64))
    return np.all(np.abs(dec - np.clip(exact, -448, 448)) <= ulp * 1.0001)


def test_prefill_chunk_csa_and_hca_layers_sampled_queries():
    """A 4096-token chunk against a 256K-token cache: compress the chunk (4x / 128x, fp8
    indexer keys), fp8 indexer + top-512 for 4096 queries, CSA and HCA attention with a
    4224-row window buffer.  Sampled query rows are checked against the oracle; the new
    compressed entries both sides read are the oracle's (the library's compression of the
    same chunk is checked separately)."""
    T, H, D, HI, DI, k, W, m = 4096, 64, 512, 8, 128, 512, 128, 4
    P0 = 262144                                   # cached raw tokens
    N0c, N0h = P0 // 4, P0 // 128                 # cached CSA / HCA entries
    Lw = 128 + T                                  # window buffer: positions [P0-128, P0+T)
    wpos0 = np.array([P0 - 128], np.int32)
    qpos = (P0 + np.arange(T, dtype=np.int32))[None]
    sampled = np.array([0, 1, 2, 3, 127, 128, 2047, 4094, 4095])
    scale = 1.0 / math.sqrt(D)
    dec = codecs.decode_bf16
    cfg = 5
    # ---------------- inputs shared by the two layers' windows
    gate = synth.normal(cfg, synth.GATE, (1, T))
    bias4 = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    bias128 = synth.normal(cfg + 10, synth.BIAS, (128,), std=0.1)

    # ================ CSA layer
    rk = synth.bf16_bits(synth.normal(cfg, synth.RAW_K, (1, T, D)))
    rv = synth.bf16_bits(synth.normal(cfg, synth.RAW_V, (1, T, D)))
    rki = synth.bf16_bits(synth.normal(cfg, synth.RAW_KI, (1, T, DI)))
    new_k = method.compress(dec(rk), gate, bias4, m)[0]           # [1024, D] fp64
    new_v = method.compress(dec(rv), gate, bias4, m)[0]
    new_ki = method.compress(dec(rki), gate, bias4, m)[0]
    # the library's compression of the same chunk
    g_d, b_d = dev(gate), dev(bias4)
    ck = L.csa_compress(dev(rk.view(np.int16)).view(torch.bfloat16), g_d, b_d, m, torch.bfloat16)
    cki = L.csa_compress(dev(rki.view(np.int16)).view(torch.bfloat16), g_d, b_d, m, torch.float8_e4m3fn)
    torch.cuda.synchronize()
    amax = np.abs(dec(rk)).reshape(T // m, m * D).max(axis=1)[:, None]
    ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(new_k), 2.0 ** -126))) - 7).astype(np.int64))
    assert np.all(np.abs(host_bf16(ck)[0] - new_k) <= ulp + m * 2.0 ** -21 * amax)
    assert _fp8_valid_rounding(cki.view(torch.uint8).cpu().numpy()[0], new_ki)
    # caches: cached part drawn, new part = the oracle's entries
    kc = torch.empty((1, N0c + T // m, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc[0, :N0c] = synth.device_normal((N0c, D), 5101, torch.bfloat16)
    vc[0, :N0c] = synth.device_normal((N0c, D), 5102, torch.bfloat16)
    nk_bits, nv_bits = codecs.encode_bf16(new_k), codecs.encode_bf16(new_v)
    kc[0, N0c:] = dev(nk_bits.view(np.int16)).view(torch.bfloat16)
    vc[0, N0c:] = dev(nv_bits.view(np.int16)).view(torch.bfloat16)
    ki_codes = np.concatenate([codecs.encode_e4m3(synth.normal(cfg, synth.KI, (N0c, DI))), codecs.encode_e4m3(new_ki)])
    ki = dev(ki_codes[None]).view(torch.float8_e4m3fn)
    qi_codes = codecs.encode_e4m3(synth.normal(cfg, synth.QI, (1, T, HI, DI)))
    qi = dev(qi_codes).view(torch.float8_e4m3fn)
    wi = synth.uniform(cfg, synth.WI, (1, T, HI))
    idx = L.csa_index_topk(qi, dev(wi), ki, dev(qpos), m, k)
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()
    s = method.index_scores(codecs.decode_e4m3(qi_codes[:, sampled]), wi[:, sampled],
                            codecs.decode_e4m3(ki_codes)[None], qpos[:, sampled], m)
    idx_r = method.topk(s, qpos[:, sampled], m, k)
    n_vis = method.visible_blocks(qpos[:, sampled], m, N0c + T // m)
    for j, qq in enumerate(sampled):
        assert check_topk(idx_g[0, qq], s[0, j], int(n_vis[0, j]), k) <= 2
    # window buffer: 128 cached raw rows then the chunk's raw rows
    kw_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.KW, (1, 128, D))), rk], axis=1)
    vw_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.VW, (1, 128, D))), rv], axis=1)
    q = synth.device_normal((1, T, H, D), 5103, torch.bfloat16)
    idx_in = idx.clone()
    idx_in[0, torch.from_numpy(sampled).cuda()] = torch.from_numpy(idx_r[0]).cuda()
    o, lse = L.csa_attend(q, kc, vc, idx_in, dev(kw_bits.view(np.int16)).view(torch.bfloat16),
                          dev(vw_bits.view(np.int16)).view(torch.bfloat16), dev(wpos0), W, dev(qpos), scale)
    torch.cuda.synchronize()
    kc_h = np.concatenate([host_bf16(kc[0, :N0c]), dec(nk_bits)])[None]
    vc_h = np.concatenate([host_bf16(vc[0, :N0c]), dec(nv_bits)])[None]
    o_r, lse_r = method.csa_attend(host_bf16(q[:, torch.from_numpy(sampled).cuda()]), kc_h, vc_h, idx_r,
                                   dec(kw_bits), dec(vw_bits), wpos0, W, qpos[:, sampled], scale)
    assert row_rel_err(host_bf16(o[:, torch.from_numpy(sampled).cuda()]), o_r) <= 1e-2
    assert lse_abs_err(lse[:, torch.from_numpy(sampled).cuda()].cpu().numpy(), lse_r) <= 1e-2
    del kc, vc, ki, qi, q, o

    # ================ HCA layer
    cfg = 6
    rk = synth.bf16_bits(synth.normal(cfg, synth.RAW_K, (1, T, D)))
    rv = synth.bf16_bits(synth.normal(cfg, synth.RAW_V, (1, T, D)))
    hn_k = method.compress(dec(rk), gate, bias128, 128)[0]        # [32, D]
    hn_v = method.compress(dec(rv), gate, bias128, 128)[0]
    hck = L.csa_compress(dev(rk.view(np.int16)).view(torch.bfloat16), g_d, dev(bias128), 128, torch.bfloat16)
    torch.cuda.synchronize()
    amax = np.abs(dec(rk)).reshape(T // 128, 128 * D).max(axis=1)[:, None]
    ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(np.abs(hn_k), 2.0 ** -126))) - 7).astype(np.int64))
    assert np.all(np.abs(host_bf16(hck)[0] - hn_k) <= ulp + 128 * 2.0 ** -21 * amax)
    hkc_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.KC, (N0h, D))), codecs.encode_bf16(hn_k)])[None]
    hvc_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.VC, (N0h, D))), codecs.encode_bf16(hn_v)])[None]
    kw_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.KW, (1, 128, D))), rk], axis=1)
    vw_bits = np.concatenate([synth.bf16_bits(synth.normal(cfg, synth.VW, (1, 128, D))), rv], axis=1)
    q = synth.device_normal((1, T, H, D), 6103, torch.bfloat16)
    b16 = lambda x: dev(x.view(np.int16)).view(torch.bfloat16)
    o, lse = L.hca_attend(q, b16(hkc_bits), b16(hvc_bits), 128, b16(kw_bits), b16(vw_bits), dev(wpos0), W, dev(qpos),
                          scale)
    torch.cuda.synchronize()
    sel = torch.from_numpy(sampled).cuda()
    o_r, lse_r = method.hca_attend(host_bf16(q[:, sel]), dec(hkc_bits), dec(hvc_bits), 128, dec(kw_bits),
                                   dec(vw_bits), wpos0, W, qpos[:, sampled], scale)
    assert row_rel_err(host_bf16(o[:, sel]), o_r) <= 1e-2
    assert lse_abs_err(lse[:, sel].cpu().numpy(), lse_r) <= 1e-2

"""GPU parity: every entry point of the C ABI against the float64 CPU oracle on the same
seeded inputs (small shapes that span several tiles and a ragged tail, edge cases)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import codecs, method
from tests.parity import check_mxfp4_rounding, check_topk, lse_abs_err, row_rel_err

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(x32):
    bits = synth.bf16_bits(x32)
    return dev(bits.view(np.int16)).view(torch.bfloat16), bits


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return codecs.decode_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def bf16_ulp(y):
    a = np.abs(np.asarray(y, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))


def compress_tol(x, m, y_ref):
    """One bf16 ulp of the exact value, plus the fp32 accumulation error of m weighted
    terms (about m * 2^-24 * max|x| of the block; 8x slack)."""
    B, T, C = x.shape
    amax = np.abs(np.asarray(x, np.float64)).reshape(B, T // m, m * C).max(axis=2)[..., None]
    return bf16_ulp(y_ref) + m * 2.0 ** -21 * amax


# ============================================================ compression
def test_compress_f32_c1_shapes():
    cfg = 101
    x = synth.normal(cfg, synth.RAW_K, (1, 4096, 128))
    gate = synth.normal(cfg, synth.GATE, (1, 4096))
    bias = synth.normal(cfg, synth.BIAS, (4,), std=0.1)
    y = L.csa_compress(dev(x), dev(gate), dev(bias), 4, torch.float32)
    torch.cuda.synchronize()
    y_ref = method.compress(x.astype(np.float64), gate, bias, 4)
    assert row_rel_err(host(y), y_ref) <= 1e-5


@pytest.mark.parametrize("m,C,nb,B", [(128, 512, 13, 2), (4, 128, 37, 3), (4, 512, 9, 1), (32, 64, 5, 2), (4, 1024, 1024, 1),
                                      (128, 1024, 3, 2)])
def test_compress_bf16_within_one_ulp(m, C, nb, B):
    cfg = 102
    T = m * nb
    x = synth.normal(cfg, synth.RAW_V, (B, T, C))
    gate = synth.normal(cfg, synth.GATE, (B, T))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    xd, xbits = dev_bf16(x)
    y = L.csa_compress(xd, dev(gate), dev(bias), m, torch.bfloat16)
    torch.cuda.synchronize()
    y_ref = method.compress(codecs.decode_bf16(xbits), gate, bias, m)
    err = np.abs(host(y) - y_ref)
    assert np.all(err <= compress_tol(codecs.decode_bf16(xbits), m, y_ref))


def test_compress_into_cache_tail_with_batch_stride():
    cfg = 103
    B, m, C, nb, cap = 2, 4, 128, 8, 20
    x = synth.normal(cfg, synth.RAW_K, (B, m * nb, C))
    gate = synth.normal(cfg, synth.GATE, (B, m * nb))
    bias = np.zeros(m, np.float32)
    xd, xbits = dev_bf16(x)
    cache = torch.zeros((B, cap, C), dtype=torch.bfloat16, device="cuda")
    L.csa_compress(xd, dev(gate), dev(bias), m, torch.bfloat16, out=cache[:, 12:])
    torch.cuda.synchronize()
    got = host(cache)
    assert np.all(got[:, :12] == 0)
    y_ref = method.compress(codecs.decode_bf16(xbits), gate, bias, m)
    assert np.all(np.abs(got[:, 12:] - y_ref) <= compress_tol(codecs.decode_bf16(xbits), m, y_ref))


@pytest.mark.parametrize("m,C,ydt", [(4, 1024, "bf16"), (128, 1024, "bf16"), (4, 128, "mxfp4"), (4, 64, "f32"),
                                     (4, 1024, "fp8kv"), (128, 1024, "fp8kv")])
def test_cache_append_decode_matches_prefix_compression(m, C, ydt):
    """Prefix / decode consistency: a prefix compressed in one call, then one token per
    step through kv_cache_append (the ring wraps twice, blocks complete at different steps
    per sequence) leaves the ring holding the last L raw rows at row position % L and the
    cache holding the oracle's pooled blocks of the whole sequence."""
    cfg = 150 + m
    B, W = 3, 16
    Lw = max(m, 40) if m < 128 else 256                     # a multiple of m, >= W
    T0 = np.array([5 * m, 5 * m + 1, 7 * m - 1])          # prefix lengths (ragged)
    S = 2 * Lw + 2 * m                                      # decode steps
    Tt = int(T0.max()) + S
    N = Tt // m + 2
    x32 = synth.normal(cfg, synth.RAW_K, (B, Tt, C))
    gate = synth.normal(cfg, synth.GATE, (B, Tt))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    if ydt == "f32":
        xd = dev(x32)
        x64 = x32.astype(np.float64)
    else:
        xd, xbits = dev_bf16(x32)
        x64 = codecs.decode_bf16(xbits)
    if ydt == "mxfp4":
        cache = torch.zeros((B, N, C // 2), dtype=torch.uint8, device="cuda")
        cscale = torch.zeros((B, N, C // 32), dtype=torch.uint8, device="cuda")
    elif ydt == "fp8kv":
        cache = torch.zeros((B, N, C + DR), dtype=torch.uint8, device="cuda")
        cscale = dev(np.array([127 - 1, 127 + 2], dtype=np.uint8))   # K codes of y * 2, V codes of y / 4
    else:
        cache = torch.zeros((B, N, C), dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device="cuda")
        cscale = None
    gd, bd = dev(gate), dev(bias)
    # prefix: complete blocks compressed in one call per sequence; the ring holds the last L rows
    win = torch.zeros((B, Lw, C), dtype=xd.dtype, device="cuda")
    wgate = torch.zeros((B, Lw), dtype=torch.float32, device="cuda")
    for b in range(B):
        nb0 = int(T0[b]) // m
        if nb0:
            kw = dict(out=cache[b:b + 1, :nb0])
            if ydt == "mxfp4":
                kw["out_scale"] = cscale[b:b + 1, :nb0]
            elif ydt == "fp8kv":
                kw["out_scale"] = cscale
            L.csa_compress(xd[b:b + 1, :nb0 * m], gd[b:b + 1, :nb0 * m].contiguous(), bd, m,
                           {"mxfp4": L.MXFP4_DTYPE, "fp8kv": L.FP8_KV_DTYPE}.get(ydt, cache.dtype), **kw)
        for q in range(max(0, int(T0[b]) - Lw), int(T0[b])):
            win[b, q % Lw] = xd[b, q]
            wgate[b, q % Lw] = gd[b, q]
    rows = torch.arange(B, device="cuda")
    for t in range(S):
        pd = dev((T0 + t).astype(np.int32))
        pl = pd.long()
        L.kv_cache_append(xd[rows, pl].contiguous(), gd[rows, pl].contiguous(), pd, win, wgate, bd, m, cache, cscale,
                          cache_dtype=L.FP8_KV_DTYPE if ydt == "fp8kv" else None)
    torch.cuda.synchronize()
    # ring: the last L positions at row position % L, bit for bit
    for b in range(B):
        last = int(T0[b]) + S - 1
        qs = torch.arange(last - Lw + 1, last + 1, device="cuda")
        assert torch.equal(win[b, qs % Lw], xd[b, qs])
        assert torch.equal(wgate[b, qs % Lw], gd[b, qs])
    # cache: every completed block equals the oracle's pooling of the whole sequence
    for b in range(B):
        nb = (int(T0[b]) + S) // m
        y_ref = method.compress(x64[b:b + 1, :nb * m], gate[b:b + 1, :nb * m], bias, m)[0]
        if ydt == "mxfp4":
            codes, scales = cache[b, :nb].cpu().numpy(), cscale[b, :nb].cpu().numpy()
            got = codecs.decode_mxfp4(codes, scales)
            step = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)   # 2^X per group
            assert np.all(np.abs(got - y_ref) <= 2 * step + 1e-6 * np.abs(y_ref))   # e2m1 rounding / saturation
        elif ydt == "fp8kv":
            x_b = x64[b:b + 1, :nb * m]
            _check_fp8kv_rows(cache[b, :nb].cpu().numpy(), y_ref, compress_tol(x_b, m, y_ref[None])[0] - bf16_ulp(y_ref),
                              ek=-1, ev=2)
        else:
            got = host(cache[b, :nb])
            if ydt == "f32":
                assert row_rel_err(got[None], y_ref[None]) <= 1e-5
            else:
                assert np.all(np.abs(got - y_ref) <= compress_tol(x64[b:b + 1, :nb * m], m, y_ref[None])[0])
        assert torch.count_nonzero(cache[b, nb:]) == 0


@pytest.mark.parametrize("csa", [True, False])
def test_attend_over_a_ring_window(csa):
    """win_pos0 = NULL: the window is a ring (position p in row p % L); the result equals
    the oracle on the same rows laid out linearly."""
    cfg = 170
    B, Q, H, D, N, m, Lw, W, k = 2, 3, 64, 512, 300, (4 if csa else 128), 256, 128, 64
    pmax = np.array([N * m + 40, N * m - 7])
    qpos = np.stack([pmax, pmax - 1, pmax - 90], axis=1).astype(np.int32)       # [B, Q]
    bits = lambda t, shape: synth.bf16_bits(synth.normal(cfg, t, shape))
    qb, kb, vb = bits(synth.Q, (B, Q, H, D)), bits(synth.KC, (B, N, D)), bits(synth.VC, (B, N, D))
    kwl, vwl = bits(synth.KW, (B, Lw, D)), bits(synth.VW, (B, Lw, D))       # linear: row r <-> wp0 + r
    wp0 = (pmax - Lw + 1).astype(np.int32)
    kwr, vwr = np.empty_like(kwl), np.empty_like(vwl)
    for b in range(B):
        rr = (wp0[b] + np.arange(Lw)) % Lw
        kwr[b, rr], vwr[b, rr] = kwl[b], vwl[b]
    tb = lambda x: dev(x.view(np.int16)).view(torch.bfloat16)
    dec = codecs.decode_bf16
    scale = 1.0 / math.sqrt(D)
    if csa:
        idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k).astype(np.int32)
        o, lse = L.csa_attend(tb(qb), tb(kb), tb(vb), dev(idx), tb(kwr), tb(vwr), None, W, dev(qpos), scale)
        o_r, lse_r = method.csa_attend(dec(qb), dec(kb), dec(vb), idx, dec(kwl), dec(vwl), wp0, W, qpos, scale)
    else:
        o, lse = L.hca_attend(tb(qb), tb(kb), tb(vb), m, tb(kwr), tb(vwr), None, W, dev(qpos), scale)
        o_r, lse_r = method.hca_attend(dec(qb), dec(kb), dec(vb), m, dec(kwl), dec(vwl), wp0, W, qpos, scale)
    torch.cuda.synchronize()
    assert row_rel_err(host(o), o_r) <= 1e-2
    assert lse_abs_err(lse.cpu().numpy(), lse_r) <= 1e-3


def _quant_inputs():
    r = np.random.default_rng(7)
    x = (r.standard_normal((3, 64, 128)) * np.exp(r.standard_normal((3, 64, 1)) * 2)).astype(np.float32)
    x[0, 0, :32] = 0.0
    x[0, 1, :32] = np.float32(1e-41)                       # subnormal group
    x[0, 2, :] = np.float32(1e4)                           # fp8 saturation
    fin = codecs.decode_e4m3(np.arange(0, 127, dtype=np.uint8))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)   # exact fp8 ties
    x[1, 0, :mids.size] = mids
    grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 7.0], np.float32)
    row = np.concatenate([grid, -grid, [6.0, 4.0], np.zeros(32 - 2 * len(grid) - 2, np.float32)]).astype(np.float32)
    x[1, 1, :32] = row                                       # amax 7 -> X = 0: e2m1 ties at the grid midpoints
    return x


def test_quantizers_bit_exact_against_oracle_encoders():
    x = _quant_inputs()
    B, T, C = x.shape
    gate = np.zeros((B, T), np.float32)
    one = np.zeros(1, np.float32)
    f8 = L.csa_compress(dev(x), dev(gate), dev(one), 1, torch.float8_e4m3fn)
    codes, scales = L.csa_compress(dev(x), dev(gate), dev(one), 1, L.MXFP4_DTYPE)
    torch.cuda.synchronize()
    assert np.array_equal(f8.view(torch.uint8).cpu().numpy(), codecs.encode_e4m3(x))
    p_ref, s_ref = codecs.encode_mxfp4(x)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), p_ref)
    # bf16 input through the same path
    xd, xbits = dev_bf16(x)
    codes, scales = L.csa_compress(xd, dev(gate), dev(one), 1, L.MXFP4_DTYPE)
    torch.cuda.synchronize()
    p_ref, s_ref = codecs.encode_mxfp4(codecs.decode_bf16(xbits).astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), p_ref) and np.array_equal(scales.cpu().numpy(), s_ref)


def test_compress_fp8_output_is_a_valid_rounding():
    cfg = 104
    x = synth.normal(cfg, synth.RAW_KI, (2, 4 * 50, 128)) * np.float32(20)
    gate = synth.normal(cfg, synth.GATE, (2, 200))
    bias = synth.normal(cfg, synth.BIAS, (4,), std=0.1)
    y = L.csa_compress(dev(x), dev(gate), dev(bias), 4, torch.float8_e4m3fn)
    torch.cuda.synchronize()
    got = y.view(torch.uint8).cpu().numpy()
    y32 = method.compress(x.astype(np.float64), gate, bias, 4).astype(np.float32)
    ref = codecs.encode_e4m3(y32)
    diff = got != ref
    # a code may differ only where the exact value sits next to a rounding midpoint
    lo = codecs.encode_e4m3(y32 * np.float32(1 - 1e-6))
    hi = codecs.encode_e4m3(y32 * np.float32(1 + 1e-6))
    assert np.all(~diff | (got == lo) | (got == hi))
    assert diff.mean() < 1e-3


def _check_fp8kv_rows(rows, y_ref, tol, ek=0, ev=0):
    """rows: FP8 K|V rows [.., C+64] uint8 written by the pooling; y_ref: the oracle's pooled
    values [.., C]; tol: the fp32 accumulation bound per element.  Code dims must be an
    E4M3 rounding (nearest-even, saturating) of a value within tol of y_ref * 2^-e; the
    bf16 dims must lie within tol of y_ref plus one bf16 ulp."""
    C = y_ref.shape[-1]
    D, DN = C // 2, C // 2 - DR
    tol = np.broadcast_to(tol, y_ref.shape)

    def codes_ok(codes, y, t, e):
        y = y * 2.0 ** -e
        t = t * 2.0 ** -e
        lo = codecs.decode_e4m3(codecs.encode_e4m3((y - t).astype(np.float32)))
        hi = codecs.decode_e4m3(codecs.encode_e4m3((y + t).astype(np.float32)))
        got = codecs.decode_e4m3(codes)
        return np.all((got >= lo) & (got <= hi))

    assert codes_ok(rows[..., :DN], y_ref[..., :DN], tol[..., :DN], ek)
    assert codes_ok(rows[..., D + DR:], y_ref[..., D:], tol[..., D:], ev)
    tail = np.ascontiguousarray(rows[..., DN:D + DR]).view("<u2")
    got = codecs.decode_bf16(tail)
    assert np.all(np.abs(got - y_ref[..., DN:D]) <= tol[..., DN:D] + bf16_ulp(y_ref[..., DN:D]))


@pytest.mark.parametrize("m,nb", [(4, 60), (128, 5)])
def test_compress_fp8kv_rows(m, nb):
    """Pooling K|V side by side straight into FP8 K|V rows (E4M3 codes with power-of-two
    scales from two E8M0 bytes, bf16 RoPE dims of K) against the oracle's pooled values."""
    cfg = 106 + m
    B, C = 2, 1024
    x32 = synth.normal(cfg, synth.RAW_K, (B, nb * m, C)) * np.float32(3)
    gate = synth.normal(cfg, synth.GATE, (B, nb * m))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    xd, xbits = dev_bf16(x32)
    sc = dev(np.array([127 - 2, 127 + 1], dtype=np.uint8))   # K codes of y * 2^2, V codes of y * 2^-1
    rows = L.csa_compress(xd, dev(gate), dev(bias), m, L.FP8_KV_DTYPE, out_scale=sc)
    torch.cuda.synchronize()
    x64 = codecs.decode_bf16(xbits)
    y_ref = method.compress(x64, gate, bias, m)
    tol = compress_tol(x64, m, y_ref) - bf16_ulp(y_ref)      # the accumulation part
    _check_fp8kv_rows(rows.cpu().numpy(), y_ref, tol, ek=-2, ev=1)


@pytest.mark.parametrize("fp8", [False, True])
def test_compress2_equals_two_compress_calls(fp8):
    """K|V rows and the indexer key pooled in one launch write the same bytes as two
    csa_compress calls (into the tail of caches with a batch stride)."""
    cfg = 109 + fp8
    B, m, nb, C, C2, N = 3, 4, 20, 1024, 128, 50
    T = nb * m
    x, _ = dev_bf16(synth.normal(cfg, synth.RAW_K, (B, T, C)))
    x2, _ = dev_bf16(synth.normal(cfg, synth.RAW_KI, (B, T, C2)))
    gate = dev(synth.normal(cfg, synth.GATE, (B, T)))
    bias = dev(synth.normal(cfg, synth.BIAS, (m,), std=0.1))
    width = C + DR if fp8 else C
    ydt = torch.uint8 if fp8 else torch.bfloat16
    y_a, y_b = torch.zeros((B, N, width), dtype=ydt, device="cuda"), torch.zeros((B, N, width), dtype=ydt, device="cuda")
    k_a, k_b = (torch.zeros((B, N, C2 // 2), dtype=torch.uint8, device="cuda") for _ in range(2))
    s_a, s_b = (torch.zeros((B, N, C2 // 32), dtype=torch.uint8, device="cuda") for _ in range(2))
    sc = dev(np.array([127 - 1, 127 + 1], dtype=np.uint8)) if fp8 else None
    L.csa_compress2(x, x2, gate, bias, m, y_a[:, N - nb:], k_a[:, N - nb:], s_a[:, N - nb:], out_scale=sc, fp8_kv=fp8)
    L.csa_compress(x, gate, bias, m, L.FP8_KV_DTYPE if fp8 else torch.bfloat16, out=y_b[:, N - nb:],
                   out_scale=sc)
    L.csa_compress(x2, gate, bias, m, L.MXFP4_DTYPE, out=k_b[:, N - nb:], out_scale=s_b[:, N - nb:])
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b) and torch.equal(k_a, k_b) and torch.equal(s_a, s_b)
    assert torch.count_nonzero(y_a[:, :N - nb]) == 0 and torch.count_nonzero(y_a[:, N - nb:]) > 0


@pytest.mark.parametrize("fp8", [False, True])
def test_compress2_against_the_oracle(fp8):
    """csa_compress2 (a CSA layer's K|V rows and indexer key pooled in one launch, the decode
    step's pooling call) against the oracle's pooling of the same bytes: bf16 K|V within one
    ulp plus the fp32 accumulation bound, FP8 K|V rows as valid E4M3 roundings with bf16 RoPE
    dims, MXFP4 keys as valid roundings group by group; rows outside the written range stay
    untouched."""
    cfg = 111 + fp8
    B, m, nb, C, C2, N = 3, 4, 24, 1024, 128, 60
    T = nb * m
    x32 = synth.normal(cfg, synth.RAW_K, (B, T, C)) * np.float32(2)
    x2_32 = synth.normal(cfg, synth.RAW_KI, (B, T, C2)) * np.exp(synth.normal(cfg + 50, synth.RAW_KI, (B, T, 1)))
    gate = synth.normal(cfg, synth.GATE, (B, T))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    x, xbits = dev_bf16(x32)
    x2, x2bits = dev_bf16(x2_32)
    width = C + DR if fp8 else C
    ydt = torch.uint8 if fp8 else torch.bfloat16
    y = torch.zeros((B, N, width), dtype=ydt, device="cuda")
    kc = torch.zeros((B, N, C2 // 2), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, N, C2 // 32), dtype=torch.uint8, device="cuda")
    sc = dev(np.array([127 - 1, 127 + 1], dtype=np.uint8)) if fp8 else None
    L.csa_compress2(x, x2, dev(gate), dev(bias), m, y[:, N - nb:], kc[:, N - nb:], ks[:, N - nb:], out_scale=sc,
                    fp8_kv=fp8)
    torch.cuda.synchronize()
    x64, x2_64 = codecs.decode_bf16(xbits), codecs.decode_bf16(x2bits)
    y_ref = method.compress(x64, gate, bias, m)
    k_ref = method.compress(x2_64, gate, bias, m)
    acc = compress_tol(x64, m, y_ref) - bf16_ulp(y_ref)            # the fp32 accumulation part
    if fp8:
        _check_fp8kv_rows(y[:, N - nb:].cpu().numpy(), y_ref, acc, ek=-1, ev=1)
    else:
        assert np.all(np.abs(host(y[:, N - nb:]) - y_ref) <= compress_tol(x64, m, y_ref))
    acc2 = compress_tol(x2_64, m, k_ref) - bf16_ulp(k_ref)
    check_mxfp4_rounding(kc[:, N - nb:].cpu().numpy(), ks[:, N - nb:].cpu().numpy(), k_ref, acc2)
    for t in (y, kc, ks):
        assert torch.count_nonzero(t[:, :N - nb]) == 0


def test_fp8kv_rows_from_pooling_feed_the_attention():
    """Pooling into FP8 K|V rows (K|V side by side, row stride C + 64) and HCA attention over
    such a cache.  Parity: the GPU attends over the oracle's own pooled-and-encoded rows and
    matches the oracle on them.  Layout: the GPU's pooled rows equal those bytes but for
    rare rounding midpoints, and attending over them gives the same result (GPU vs GPU)."""
    cfg = 108
    B, Q, H, D, m, nb, Lw, W = 2, 2, 64, 512, 128, 40, 128, 128
    x32 = synth.normal(cfg, synth.RAW_K, (B, nb * m, 2 * D))
    gate = synth.normal(cfg, synth.GATE, (B, nb * m))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    xd, xbits = dev_bf16(x32)
    kv_gpu = L.csa_compress(xd, dev(gate), dev(bias), m, L.FP8_KV_DTYPE)        # [B, nb, 1088]
    y_ref = method.compress(codecs.decode_bf16(xbits), gate, bias, m).astype(np.float32)
    rows = np.concatenate([codecs.encode_fp8_k_rows(y_ref[..., :D], DR, 1.0),
                           codecs.encode_fp8_v_rows(y_ref[..., D:], 1.0)], axis=-1)     # the oracle's rows
    torch.cuda.synchronize()
    gpu_rows = kv_gpu.cpu().numpy()
    x64 = codecs.decode_bf16(xbits)
    y64 = method.compress(x64, gate, bias, m)
    _check_fp8kv_rows(gpu_rows, y64, compress_tol(x64, m, y64) - bf16_ulp(y64))   # every code a valid rounding
    (_, _, kwb, vwb), (_, _, kwd, vwd) = _fp8_kv(cfg, B, 1, Lw, D, 1.0, 1.0)
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    qd, qb = dev_bf16(q)
    T = nb * m
    win_pos0 = np.array([T - Lw, T - Lw], dtype=np.int32)
    pos = np.array([[T - 1, T - 50], [T - 30, T - 100]], dtype=np.int32)
    KB = D + DR
    scale = 1.0 / math.sqrt(D)
    kv_ref = dev(rows)
    o, lse = L.hca_attend_fp8kv(qd, kv_ref[..., :KB], kv_ref[..., KB:], m, dev(kwb), dev(vwb), dev(win_pos0), W,
                                dev(pos), scale)
    o2, lse2 = L.hca_attend_fp8kv(qd, kv_gpu[..., :KB], kv_gpu[..., KB:], m, dev(kwb), dev(vwb), dev(win_pos0), W,
                                  dev(pos), scale)
    torch.cuda.synchronize()
    kd, vd = codecs.decode_fp8_k_rows(rows[..., :KB], D, DR, 1.0), codecs.decode_fp8_v_rows(rows[..., KB:], 1.0)
    o_r, lse_r = method.hca_attend(codecs.decode_bf16(qb), kd, vd, m, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_r) <= 1e-2
    assert lse_abs_err(host(lse), lse_r) <= 1e-2
    # end to end: the GPU's own pooled rows through the GPU attention, against the oracle's
    # pooling, encoding and attention
    assert row_rel_err(host(o2), o_r) <= 1e-2
    assert lse_abs_err(host(lse2), lse_r) <= 1e-2


# ============================================================ indexer + top-k
def _scores_oracle(qi64, w, ki64, q_pos, m):
    return method.index_scores(qi64, w, ki64, q_pos, m)


@pytest.mark.parametrize("HI,DI,Q", [(8, 128, 3), (4, 64, 5), (16, 128, 2), (8, 256, 1), (4, 32, 2)])
def test_index_topk_bf16(HI, DI, Q):
    cfg = 200 + HI + DI
    B, N, m, k = 2, 5000, 4, 512
    qi = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    ki = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = np.array([[4 * N - 1, 1000, 2, 4 * N + 77, 2047][:Q], [4 * N - 3, 4 * 600 + 1, 4 * N - 1, 3, 99][:Q]],
                   dtype=np.int32)
    qd, qbits = dev_bf16(qi)
    kd, kbits = dev_bf16(ki)
    idx, sc = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k, with_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_bf16(kbits), pos, m)
    nvis = method.visible_blocks(pos, m, N)
    for b in range(B):
        for q in range(Q):
            n = int(nvis[b, q])
            check_topk(idx[b, q], s_ref[b, q], n, k)
            take = min(k, n)
            sel = idx[b, q, :take]
            ref = s_ref[b, q, sel]
            tol = 1e-5 * np.abs(s_ref[b, q, :n]).max() if n else 0
            assert np.all(np.abs(sc[b, q, :take] - ref) <= tol + 1e-6)
            assert np.all(np.isneginf(sc[b, q, take:]))


def test_index_topk_mxfp4_keys():
    cfg = 210
    B, Q, HI, DI, N, m, k = 2, 1, 8, 128, 6000, 4, 256
    qi = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = np.array([[4 * N - 1], [4 * 3000 + 2]], dtype=np.int32)
    codes, scales = L.csa_compress(dev(k32), dev(np.zeros((B, N), np.float32)), dev(np.zeros(1, np.float32)), 1,
                                   L.MXFP4_DTYPE)
    p_ref, s_ref8 = codecs.encode_mxfp4(k32)
    assert np.array_equal(codes.cpu().numpy(), p_ref) and np.array_equal(scales.cpu().numpy(), s_ref8)
    qd, qbits = dev_bf16(qi)
    idx = L.csa_index_topk(qd, dev(w), codes, dev(pos), m, k, ki_scale=scales)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_mxfp4(p_ref, s_ref8), pos, m)
    nvis = method.visible_blocks(pos, m, N)
    for b in range(B):
        assert check_topk(idx[b, 0], s_ref[b, 0], int(nvis[b, 0]), k) <= 2


@pytest.mark.parametrize("DI", [128, 256])
def test_index_topk_fp4_queries_and_keys(DI):
    """FP4 x FP4 indexer: queries quantised by the library (bit-equal to the oracle's MXFP4
    encoder), keys in MXFP4; scores on the scaled FP4 MFMA against the oracle's FP4-query
    mode."""
    cfg = 215
    B, Q, HI, N, m, k = 2, 3, 8, 5000, 4, 256
    q32 = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = np.array([[4 * N - 1, 4 * 3000 + 2, 4 * 50], [4 * N - 3, 4 * N - 1, 7]], dtype=np.int32)
    kp, ks = codecs.encode_mxfp4(k32)
    R = B * Q * HI
    qbuf = torch.empty(R * DI // 2 + R * DI // 32, dtype=torch.uint8, device="cuda")
    qc, qs = qbuf[:R * DI // 2].view(1, R, DI // 2), qbuf[R * DI // 2:].view(1, R, DI // 32)
    L.csa_compress(dev(q32.reshape(1, R, DI)), dev(np.zeros((1, R), np.float32)), dev(np.zeros(1, np.float32)), 1,
                   L.MXFP4_DTYPE, out=qc, out_scale=qs)
    s_ref, qp_ref, qs_ref = method.index_scores_fp4(q32, w, codecs.decode_mxfp4(kp, ks), pos, m)
    assert np.array_equal(qc.cpu().numpy().reshape(qp_ref.shape), qp_ref)
    assert np.array_equal(qs.cpu().numpy().reshape(qs_ref.shape), qs_ref)
    idx, sc = L.csa_index_topk(qc.view(B, Q, HI, DI // 2), dev(w), dev(kp), dev(pos), m, k, ki_scale=dev(ks),
                               qi_scale=qs.view(B, Q, HI, DI // 32), with_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    nvis = method.visible_blocks(pos, m, N)
    for b in range(B):
        for q in range(Q):
            n = int(nvis[b, q])
            check_topk(idx[b, q], s_ref[b, q], n, k)
            take = min(k, n)
            ref = s_ref[b, q, idx[b, q, :take]]
            assert np.all(np.abs(sc[b, q, :take] - ref) <= 1e-5 * np.abs(s_ref[b, q, :n]).max() + 1e-6)


@pytest.mark.parametrize("HI,DI", [(8, 128), (16, 256), (4, 64)])
def test_index_topk_fp8(HI, DI):
    """fp8 queries and keys: DI >= 128 runs on the scaled 16x16x128 MFMA, DI = 64 on the
    16x16x32 one.  Both sides read the oracle's e4m3 codes; the library's quantiser is
    checked against the oracle's encoder separately."""
    cfg = 220 + DI
    B, Q, N, m, k = 1, 4, 3000, 4, 300
    q32 = synth.normal(cfg, synth.QI, (B, Q, HI, DI)) * np.float32(4)
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI)) * np.float32(4)
    pos = np.array([[4 * N - 1, 4 * N - 2, 5000, 40]], dtype=np.int32)
    zero1 = dev(np.zeros(1, np.float32))
    qc, kc = codecs.encode_e4m3(q32), codecs.encode_e4m3(k32)
    q8 = L.csa_compress(dev(q32.reshape(1, -1, DI)), dev(np.zeros((1, B * Q * HI), np.float32)), zero1, 1,
                        torch.float8_e4m3fn).view(B, Q, HI, DI)
    k8 = L.csa_compress(dev(k32), dev(np.zeros((B, N), np.float32)), zero1, 1, torch.float8_e4m3fn)
    assert np.array_equal(q8.view(torch.uint8).cpu().numpy(), qc)
    assert np.array_equal(k8.view(torch.uint8).cpu().numpy(), kc)
    idx = L.csa_index_topk(dev(qc).view(torch.float8_e4m3fn), dev(w), dev(kc).view(torch.float8_e4m3fn), dev(pos),
                           m, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_e4m3(qc), w, codecs.decode_e4m3(kc), pos, m)
    nvis = method.visible_blocks(pos, m, N)
    for q in range(Q):
        check_topk(idx[0, q], s_ref[0, q], int(nvis[0, q]), k)


def test_index_topk_ties_and_zero_scores():
    """Negated queries make every score 0: the selection must be the lowest indices."""
    B, Q, HI, DI, N, m, k = 1, 2, 4, 64, 2000, 4, 100
    qi = -np.abs(synth.normal(230, synth.QI, (B, Q, HI, DI)))
    ki = np.abs(synth.normal(230, synth.KI, (B, N, DI)))
    w = synth.uniform(230, synth.WI, (B, Q, HI))
    qi[0, 1, 0] = np.abs(qi[0, 1, 0])                      # query 1: head 0 positive -> real scores
    pos = np.array([[4 * N - 1, 4 * N - 1]], dtype=np.int32)
    qd, qbits = dev_bf16(qi)
    kd, kbits = dev_bf16(ki)
    idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k).cpu().numpy()
    assert list(idx[0, 0]) == list(range(k))
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_bf16(kbits), pos, m)
    check_topk(idx[0, 1], s_ref[0, 1], N, k)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "mxfp4"])
def test_index_topk_many_queries(kind):
    """Enough queries for the multi-query indexer path (several query tiles share each key
    tile); a ragged last query group and per-query visibility."""
    cfg = 260
    B, Q, HI, DI, N, m, k = 2, 37, 8, 128, 3000, 4, 100
    q32 = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = (np.arange(B * Q, dtype=np.int32).reshape(B, Q) * 311) % (4 * N + 50)
    zero1 = dev(np.zeros(1, np.float32))
    if kind == "bf16":
        qd, qb = dev_bf16(q32)
        kd, kb = dev_bf16(k32)
        q64, k64 = codecs.decode_bf16(qb), codecs.decode_bf16(kb)
        idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k)
    elif kind == "fp8":
        qc, kc = codecs.encode_e4m3(q32), codecs.encode_e4m3(k32)
        q64, k64 = codecs.decode_e4m3(qc), codecs.decode_e4m3(kc)
        idx = L.csa_index_topk(dev(qc).view(torch.float8_e4m3fn), dev(w), dev(kc).view(torch.float8_e4m3fn), dev(pos),
                               m, k)
    else:
        qd, qb = dev_bf16(q32)
        codes, scales = codecs.encode_mxfp4(k32)
        q64, k64 = codecs.decode_bf16(qb), codecs.decode_mxfp4(codes, scales)
        idx = L.csa_index_topk(qd, dev(w), dev(codes), dev(pos), m, k, ki_scale=dev(scales))
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s_ref = _scores_oracle(q64, w, k64, pos, m)
    nvis = method.visible_blocks(pos, m, N)
    for b in range(B):
        for q in range(Q):
            assert check_topk(idx[b, q], s_ref[b, q], int(nvis[b, q]), k) <= 2


def test_index_topk_many_rows_long_ranges():
    """300 query rows (a prefill-sized call): the selection scans 8192-key ranges instead of
    2048; ragged last range, per-query visibility, every row against the oracle."""
    cfg = 265
    B, Q, HI, DI, N, m, k = 1, 300, 4, 64, 20000, 4, 256
    q32 = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = (np.arange(Q, dtype=np.int32).reshape(B, Q) * 263 + 4 * N - 300 * 263) % (4 * N + 9)
    qd, qb = dev_bf16(q32)
    kd, kb = dev_bf16(k32)
    idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_bf16(qb), w, codecs.decode_bf16(kb), pos, m)
    nvis = method.visible_blocks(pos, m, N)
    assert nvis.max() > 16384                                # rows with more than two long ranges
    for q in range(Q):
        assert check_topk(idx[0, q], s_ref[0, q], int(nvis[0, q]), k) <= 2


def test_index_topk_many_queries_rows_past_2e17_keys():
    """A many-query call (several query tiles per workgroup) whose rows see 131,073 to
    262,144 keys: the row selection keeps its key bitmap on chip in the larger of its two
    layouts (rows of at most 2^17 keys take the smaller one, two workgroups to a CU).
    Sampled rows, including the shortest and the longest, against the oracle."""
    cfg = 266
    B, Q, HI, DI, N, m, k = 2, 32, 8, 128, 150000, 4, 512
    q32 = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = (4 * N - 1 - 4 * 600 * np.arange(Q, dtype=np.int32)[::-1]).reshape(1, Q).repeat(B, 0).astype(np.int32)
    qd, qb = dev_bf16(q32)
    kd, kb = dev_bf16(k32)
    print("index_topk many queries: N=150000 B=2 Q=32", flush=True)
    idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    nvis = method.visible_blocks(pos, m, N)
    assert nvis.min() > 1 << 17
    sel = [0, 13, Q - 1]
    q64, k64 = codecs.decode_bf16(qb), codecs.decode_bf16(kb)
    s_ref = _scores_oracle(q64[:, sel], w[:, sel], k64, pos[:, sel], m)
    for b in range(B):
        for j, q in enumerate(sel):
            assert check_topk(idx[b, q], s_ref[b, j], int(nvis[b, q]), k) <= 2


@pytest.mark.parametrize("N", [10000, 300000])
def test_index_topk_many_candidates(N):
    """All-zero scores put every key into the threshold bin: more candidates than the
    on-chip candidate buffer holds (and, at N > 2^18, a bitmap kept in the workspace)."""
    B, Q, HI, DI, m, k = 1, 2, 4, 64, 4, 1024
    qi = -np.abs(synth.normal(231, synth.QI, (B, Q, HI, DI)))
    ki = np.abs(synth.normal(231, synth.KI, (B, N, DI)))
    w = synth.uniform(231, synth.WI, (B, Q, HI))
    qi[0, 1] = synth.normal(232, synth.QI, (HI, DI))      # query 1: ordinary scores
    pos = np.array([[4 * N - 1, 4 * N - 5]], dtype=np.int32)
    qd, qbits = dev_bf16(qi)
    kd, kbits = dev_bf16(ki)
    idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k).cpu().numpy()
    assert list(idx[0, 0]) == list(range(k))
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_bf16(kbits), pos, m)
    check_topk(idx[0, 1], s_ref[0, 1], int(method.visible_blocks(pos, m, N)[0, 1]), k)


def test_index_topk_concentrated_winners():
    """Rows whose winners crowd into a few key chunks.  With 256 chunks of 256 keys each chunk
    keeps only its 32 best as candidates.  Sequence 0: five chunks of keys scaled by 5 hold
    more than 32 winners each, so those chunks are widened from the stored scores.
    Sequence 1: every score is 0 (negated queries, positive keys), so the winners are the
    4096 lowest indices, packed 256 to a chunk: widening them would exceed the on-chip room
    and the whole row is selected from the stored scores.  Both against the oracle."""
    cfg = 236
    B, Q, HI, DI, N, m, k = 2, 1, 8, 128, 65536, 4, 4096
    qi = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    ki = synth.normal(cfg, synth.KI, (B, N, DI))
    boosted = (3, 100, 101, 102, 103)
    for c in boosted:
        ki[0, c * 256:(c + 1) * 256] *= np.float32(5)
    qi[1] = -np.abs(qi[1])
    ki[1] = np.abs(ki[1])
    pos = np.array([[4 * N - 1], [4 * N - 2]], dtype=np.int32)
    qd, qbits = dev_bf16(qi)
    kd, kbits = dev_bf16(ki)
    idx, sc = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k, with_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_bf16(kbits), pos, m)
    assert check_topk(idx[0, 0], s_ref[0, 0], N, k) <= 2
    assert np.all(np.abs(sc[0, 0] - s_ref[0, 0, idx[0, 0]]) <= 1e-5 * np.abs(s_ref[0, 0]).max())
    per_chunk = np.bincount(idx[0, 0] // 256, minlength=N // 256)
    assert per_chunk[list(boosted)].min() > 32                  # those chunks had to be widened
    assert np.all(s_ref[1, 0, :N - 1] == 0) and list(idx[1, 0]) == list(range(k))   # (the last block is not visible)
    assert np.all(sc[1, 0] == 0)


@pytest.mark.parametrize("case", ["decode", "many_queries", "fp4_queries", "fp8_rows", "batch40", "batch256"])
def test_pool_index_topk_equals_compress2_then_index_topk(case):
    """csa_pool_index_topk (the newest block pooled inside the indexer launch) against
    csa_compress2 followed by csa_index_topk on copies of the same caches: the pooled K|V
    and key rows and the selection bit for bit; the pooled row anywhere in a chunk (here not
    the last row), several query groups per sequence, MXFP4 queries, FP8 K|V rows, and
    batches whose planned K|V split is packed into fewer workgroups (40) or kept (256)."""
    cfg = 250 + len(case)
    HI, DI, m = 8, 128, 4
    B, Q, N, k, row = {"decode": (8, 1, 20000, 512, 19999), "many_queries": (2, 37, 3000, 100, 1234),
                       "fp4_queries": (3, 1, 9000, 256, 5000), "fp8_rows": (2, 1, 6000, 128, 5999),
                       "batch40": (40, 1, 3000, 64, 2999), "batch256": (256, 1, 300, 32, 299)}[case]
    C, LW = 1024, 16
    fp8 = case == "fp8_rows"
    k32 = synth.normal(cfg, synth.KI, (B, N, DI))
    codes, scales = codecs.encode_mxfp4(k32)
    ki0, ks0 = dev(codes), dev(scales)
    if fp8:
        kv0 = dev(np.random.default_rng(cfg).integers(0, 120, (B, N, C + 64), dtype=np.uint8))
    else:
        kv0 = dev_bf16(synth.normal(cfg, synth.KC, (B, N, C)))[0]
    xw = dev_bf16(synth.normal(cfg, synth.KW, (B, LW, C)))[0]
    x2w = dev_bf16(synth.normal(cfg, synth.RAW_KI, (B, LW, DI)))[0]
    gate = dev(synth.normal(cfg, synth.GATE, (B, m)))
    bias = dev(synth.normal(cfg, synth.BIAS, (m,), std=0.1))
    wi = dev(synth.uniform(cfg, synth.WI, (B, Q, HI)))
    pos = dev((4 * N - 1 - (np.arange(B * Q, dtype=np.int32).reshape(B, Q) * 97) % (4 * N // 3)).astype(np.int32))
    sc8 = dev(np.array([125, 126], np.uint8)) if fp8 else None
    if case == "fp4_queries":
        qc, qs = codecs.encode_mxfp4(synth.normal(cfg, synth.QI, (B, Q, HI, DI)))
        qbuf = dev(np.concatenate([qc.reshape(-1), qs.reshape(-1)]))
        qi, q_scale = qbuf[:qc.size].view(qc.shape), qbuf[qc.size:].view(qs.shape)
    else:
        qi, q_scale = dev_bf16(synth.normal(cfg, synth.QI, (B, Q, HI, DI)))[0], None
    xs, x2s = xw[:, LW - m:], x2w[:, LW - m:]
    kv_a, ki_a, ks_a = kv0.clone(), ki0.clone(), ks0.clone()
    L.csa_compress2(xs, x2s, gate, bias, m, kv_a[:, row:row + 1], ki_a[:, row:row + 1], ks_a[:, row:row + 1],
                    out_scale=sc8, fp8_kv=fp8)
    ia, sa = L.csa_index_topk(qi, wi, ki_a, pos, m, k, ki_scale=ks_a, with_scores=True, qi_scale=q_scale)
    kv_b, ki_b, ks_b = kv0.clone(), ki0.clone(), ks0.clone()
    ib, sb = L.csa_pool_index_topk(xs, x2s, gate, bias, row, kv_b, qi, wi, ki_b, pos, m, k, ks_b,
                                   kv_cache_scale=sc8, fp8_kv=fp8, with_scores=True, qi_scale=q_scale)
    torch.cuda.synchronize()
    assert not torch.equal(kv_a, kv0) and not torch.equal(ki_a, ki0)       # the row was rewritten
    for name, a, b_ in (("kv", kv_a, kv_b), ("key codes", ki_a, ki_b), ("key scales", ks_a, ks_b), ("idx", ia, ib),
                        ("scores", sa, sb)):
        assert torch.equal(a, b_), name


def test_index_topk_very_long_rows():
    """Rows of more than 2^21 visible blocks: more key ranges in the selection's first pass
    than the second pass indexes directly, so candidates of the last ranges are found by
    walking the range counts."""
    B, Q, HI, DI, N, m, k = 1, 2, 4, 32, 2200000, 4, 2048
    qi = synth.normal(233, synth.QI, (B, Q, HI, DI))
    ki = synth.normal(233, synth.KI, (B, N, DI))
    w = synth.uniform(233, synth.WI, (B, Q, HI))
    pos = np.array([[4 * N - 1, 4 * 2150000 + 1]], dtype=np.int32)
    qd, qbits = dev_bf16(qi)
    kd, kbits = dev_bf16(ki)
    idx = L.csa_index_topk(qd, dev(w), kd, dev(pos), m, k).cpu().numpy()
    s_ref = _scores_oracle(codecs.decode_bf16(qbits), w, codecs.decode_bf16(kbits), pos, m)
    nvis = method.visible_blocks(pos, m, N)
    for q in range(Q):
        assert check_topk(idx[0, q], s_ref[0, q], int(nvis[0, q]), k) <= 2
    assert idx[0, 0].max() >= 2095104                     # the tail ranges contribute


def test_index_topk_f32_is_deterministic():
    cfg = 240
    B, Q, HI, DI, N, m, k = 1, 1, 4, 64, 1024, 4, 64
    qi = synth.normal(cfg, synth.QI, (B, Q, HI, DI))
    w = synth.uniform(cfg, synth.WI, (B, Q, HI))
    ki = synth.normal(cfg, synth.KI, (B, N, DI))
    pos = np.array([[4095]], dtype=np.int32)
    a = L.csa_index_topk(dev(qi), dev(w), dev(ki), dev(pos), m, k, with_scores=True)
    b = L.csa_index_topk(dev(qi), dev(w), dev(ki), dev(pos), m, k, with_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    s_ref = _scores_oracle(qi.astype(np.float64), w, ki.astype(np.float64), pos, m)
    check_topk(a[0].cpu().numpy()[0, 0], s_ref[0, 0], N, k)


# ============================================================ attention
def _attn_inputs(cfg, B, Q, H, D, N, L_, k=None):
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    kc = synth.normal(cfg, synth.KC, (B, N, D))
    vc = synth.normal(cfg, synth.VC, (B, N, D))
    kw = synth.normal(cfg, synth.KW, (B, L_, D))
    vw = synth.normal(cfg, synth.VW, (B, L_, D))
    return q, kc, vc, kw, vw


@pytest.mark.parametrize("H,D,Q", [(64, 512, 2), (16, 128, 3), (32, 256, 1)])
def test_csa_attend_bf16(H, D, Q):
    cfg = 300 + D
    B, N, L_, W, k = 2, 3000, 160, 128, 512
    q, kc, vc, kw, vw = _attn_inputs(cfg, B, Q, H, D, N, L_)
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    idx[0, 0, -7:] = -1                                        # short list
    idx[1, 0, 3] = N + 5                                       # out-of-range entries are skipped
    win_pos0 = np.array([40000, 7], dtype=np.int32)
    pos = np.array([[40000 + 150, 40000 + 20, 40000 + 159][:Q], [7 + 127, 7 + 300, 3][:Q]], dtype=np.int32)
    t = [dev_bf16(a) for a in (q, kc, vc, kw, vw)]
    (qd, qb), (kcd, kcb), (vcd, vcb), (kwd, kwb), (vwd, vwb) = t
    scale = 1.0 / math.sqrt(D)
    o, lse = L.csa_attend(qd, kcd, vcd, dev(idx), kwd, vwd, dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    o_ref, lse_ref = method.csa_attend(dec(qb), dec(kcb), dec(vcb), idx, dec(kwb), dec(vwb), win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


@pytest.mark.parametrize("H,D,N", [(64, 512, 1000), (16, 128, 77), (64, 512, 31)])
def test_hca_attend_bf16(H, D, N):
    cfg = 400 + N
    B, Q, L_, W, m = 2, 2, 128, 128, 128
    q, kc, vc, kw, vw = _attn_inputs(cfg, B, Q, H, D, N, L_)
    T = N * m
    win_pos0 = np.array([T - L_, T - L_ - 64], dtype=np.int32)
    pos = np.array([[T - 1, T - 100], [T - 65, 128 * 5 + 3]], dtype=np.int32)
    t = [dev_bf16(a) for a in (q, kc, vc, kw, vw)]
    (qd, qb), (kcd, kcb), (vcd, vcb), (kwd, kwb), (vwd, vwb) = t
    scale = 1.0 / math.sqrt(D)
    o, lse = L.hca_attend(qd, kcd, vcd, m, kwd, vwd, dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    o_ref, lse_ref = method.hca_attend(dec(qb), dec(kcb), dec(vcb), m, dec(kwb), dec(vwb), win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


@pytest.mark.parametrize("H,ring", [(64, False), (32, False), (64, True)])
def test_hca_attend_bf16_many_queries(H, ring):
    """Many queries per sequence (two per workgroup, their key lists merged): a run of
    consecutive positions, and positions far apart (disjoint windows, a query that sees no
    compressed entry, one whose window lies before the buffer); an odd query count."""
    cfg = 480 + H + ring
    B, Q, D, N, m, W = 2, 37, 512, 300, 128, 128
    Lw = 256 if ring else 600
    q, kc, vc, kwl, vwl = _attn_inputs(cfg, B, Q, H, D, N, Lw)
    T = N * m
    pos = np.zeros((B, Q), dtype=np.int32)
    pos[0] = T - Q + np.arange(Q)                                   # consecutive, the chunk's tail
    r = np.random.default_rng(cfg)
    pos[1] = np.sort(r.integers(T - 560, T, size=Q))               # scattered inside the window buffer
    pos[1, :3] = [5, 100, T - 900]                                  # no visible entry / window elsewhere
    if ring:
        pos[1] = T - 1 - np.sort(r.integers(0, 100, size=Q))[::-1]   # every window inside the ring's last L
    wp0 = np.full(B, T - Lw, dtype=np.int32)
    if ring:
        kwr, vwr = np.empty_like(kwl), np.empty_like(vwl)
        for b in range(B):
            rr = (wp0[b] + np.arange(Lw)) % Lw
            kwr[b, rr], vwr[b, rr] = kwl[b], vwl[b]
    else:
        kwr, vwr = kwl, vwl
    t = [dev_bf16(x) for x in (q, kc, vc, kwr, vwr)]
    (qd, qb), (kcd, kcb), (vcd, vcb), (kwd, _), (vwd, _) = t
    kwlb, vwlb = synth.bf16_bits(kwl), synth.bf16_bits(vwl)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.hca_attend(qd, kcd, vcd, m, kwd, vwd, None if ring else dev(wp0), W, dev(pos), scale)
    torch.cuda.synchronize()
    dec = codecs.decode_bf16
    o_ref, lse_ref = method.hca_attend(dec(qb), dec(kcb), dec(vcb), m, dec(kwlb), dec(vwlb), wp0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_attend_with_kv_side_by_side(dt):
    """K and V rows in one [.., 2D] buffer (caches and window), pooled by one csa_compress
    call; attention reads them through row strides and matches the separate-tensor call."""
    cfg = 470
    B, Q, H, D, N, L_, W, k, m = 2, 2, 16, 128, 900, 140, 128, 64, 4
    T = 4 * m
    q, kc, vc, kw, vw = _attn_inputs(cfg, B, Q, H, D, N, L_)
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    win_pos0 = np.array([2700, 2000], dtype=np.int32)
    pos = np.array([[2799, 2750], [2100, 2139]], dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    if dt == "bf16":
        cv = lambda a: dev_bf16(a)[0]
    else:
        cv = dev
    kvc = torch.cat([cv(kc), cv(vc)], dim=2)          # [B, N, 2D]
    kvw = torch.cat([cv(kw), cv(vw)], dim=2)          # [B, L, 2D]
    # the newest block of both K and V pooled in one call into the caches' last entry
    gate = dev(synth.normal(cfg, synth.GATE, (B, T)))
    bias = dev(synth.normal(cfg, synth.BIAS, (m,), std=0.1))
    g_blk = gate[:, :m].contiguous()
    L.csa_compress(kvw[:, L_ - T:L_ - T + m], g_blk, bias, m, kvc.dtype, out=kvc[:, N - 1:])
    qd = cv(q)
    o1, lse1 = L.csa_attend(qd, kvc[..., :D], kvc[..., D:], dev(idx), kvw[..., :D], kvw[..., D:], dev(win_pos0), W,
                            dev(pos), scale)
    o2, lse2 = L.csa_attend(qd, kvc[..., :D].contiguous(), kvc[..., D:].contiguous(), dev(idx),
                            kvw[..., :D].contiguous(), kvw[..., D:].contiguous(), dev(win_pos0), W, dev(pos), scale)
    h1, hl1 = L.hca_attend(qd, kvc[..., :D], kvc[..., D:], m, kvw[..., :D], kvw[..., D:], dev(win_pos0), W, dev(pos),
                           scale, N=300)
    h2, hl2 = L.hca_attend(qd, kvc[..., :D].contiguous(), kvc[..., D:].contiguous(), m, kvw[..., :D].contiguous(),
                           kvw[..., D:].contiguous(), dev(win_pos0), W, dev(pos), scale, N=300)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    assert torch.equal(h1, h2) and torch.equal(hl1, hl2)
    # the pooled entry: K and V halves each equal the oracle's pooling of their raw rows
    kv_h = host(kvc)
    raw = host(kvw)
    y_r = method.compress(raw[:, L_ - T:L_ - T + m], host(g_blk), host(bias), m)
    tol = compress_tol(raw[:, L_ - T:L_ - T + m], m, y_r) if dt == "bf16" else 1e-5 * np.abs(y_r).max()
    assert np.all(np.abs(kv_h[:, N - 1:N] - y_r) <= tol)
    # the strided attention against the oracle over the same rows, with the oracle's own
    # pooled entry in row N-1
    kc_r, vc_r = kv_h[..., :D].copy(), kv_h[..., D:].copy()
    kc_r[:, N - 1], vc_r[:, N - 1] = y_r[:, 0, :D], y_r[:, 0, D:]
    kw_r, vw_r = raw[..., :D], raw[..., D:]
    q_r = host(qd)
    o_r, lse_r = method.csa_attend(q_r, kc_r, vc_r, idx, kw_r, vw_r, win_pos0, W, pos, scale)
    h_r, hl_r = method.hca_attend(q_r, kc_r[:, :300], vc_r[:, :300], m, kw_r, vw_r, win_pos0, W, pos, scale)
    tol_o = 1e-2 if dt == "bf16" else 1e-4
    assert row_rel_err(host(o1), o_r) <= tol_o and lse_abs_err(host(lse1), lse_r) <= tol_o
    assert row_rel_err(host(h1), h_r) <= tol_o and lse_abs_err(host(hl1), hl_r) <= tol_o


@pytest.mark.parametrize("D,H", [(128, 16), (64, 4), (512, 2)])
def test_attend_f32_csa_and_hca(D, H):
    cfg = 450 + D
    B, Q, N, L_, W, k, m = 2, 2, 700, 150, 128, 96, 4
    q, kc, vc, kw, vw = _attn_inputs(cfg, B, Q, H, D, N, L_)
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    idx[1, 1, :10] = -1
    win_pos0 = np.array([2700, 2000], dtype=np.int32)
    pos = np.array([[2799, 2750], [2100, 2149]], dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    args = [dev(a) for a in (q, kc, vc)]
    o, lse = L.csa_attend(*args, dev(idx), dev(kw), dev(vw), dev(win_pos0), W, dev(pos), scale)
    oh, lseh = L.hca_attend(*args, m, dev(kw), dev(vw), dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    o_ref, lse_ref = method.csa_attend(f(q), f(kc), f(vc), idx, f(kw), f(vw), win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-4 and lse_abs_err(host(lse), lse_ref) <= 1e-4
    o_ref, lse_ref = method.hca_attend(f(q), f(kc), f(vc), m, f(kw), f(vw), win_pos0, W, pos, scale)
    assert row_rel_err(host(oh), o_ref) <= 1e-4 and lse_abs_err(host(lseh), lse_ref) <= 1e-4


@pytest.mark.parametrize("csa,B,Q,H", [(True, 8, 1, 64), (False, 8, 1, 64), (True, 16, 1, 32), (False, 4, 2, 64),
                                       (True, 32, 1, 64), (False, 11, 1, 48)])
def test_attend_decode_batches(csa, B, Q, H):
    """Decode batches of 4 to 32 sequences (key ranges split over the CUs, parts merged):
    against the oracle, with a sequence whose key set is empty and one with a short list; a
    second call on other inputs right after the first; the first call again, bitwise."""
    cfg = 520 + 7 * B + H + csa
    D, L_, W, m = 512, 160, 128, 128
    N = 3000 if csa else 1000
    k = 512
    scale = 1.0 / math.sqrt(D)
    dec = codecs.decode_bf16

    def inputs(c):
        q, kc, vc, kw, vw = _attn_inputs(c, B, Q, H, D, N, L_)
        T = N * (4 if csa else m)
        win_pos0 = np.full(B, T - L_, dtype=np.int32)
        pos = (T - 1 - np.arange(B * Q, dtype=np.int32) % 23).reshape(B, Q)
        win_pos0[0] = 10 ** 6                                   # sequence 0: window ahead of the query
        pos[0, :] = 5 if not csa else pos[0, :]                 # HCA: no visible entry either
        idx = synth.sorted_unique_indices(c, synth.IDX, B * Q, N, k).reshape(B, Q, k)
        if csa:
            idx[0] = -1                                         # CSA: empty list for sequence 0
            idx[B - 1, 0, 100:] = -1                            # a short list
        return (q, kc, vc, kw, vw), idx, win_pos0, pos

    def run(c):
        (q, kc, vc, kw, vw), idx, win_pos0, pos = inputs(c)
        t = [dev_bf16(a) for a in (q, kc, vc, kw, vw)]
        (qd, qb), (kcd, kcb), (vcd, vcb), (kwd, kwb), (vwd, vwb) = t
        if csa:
            o, lse = L.csa_attend(qd, kcd, vcd, dev(idx), kwd, vwd, dev(win_pos0), W, dev(pos), scale)
            ref = method.csa_attend(dec(qb), dec(kcb), dec(vcb), idx, dec(kwb), dec(vwb), win_pos0, W, pos, scale)
        else:
            o, lse = L.hca_attend(qd, kcd, vcd, m, kwd, vwd, dev(win_pos0), W, dev(pos), scale)
            ref = method.hca_attend(dec(qb), dec(kcb), dec(vcb), m, dec(kwb), dec(vwb), win_pos0, W, pos, scale)
        return o, lse, ref

    o1, lse1, ref1 = run(cfg)
    o2, lse2, ref2 = run(cfg + 1)
    o3, lse3, _ = run(cfg)
    torch.cuda.synchronize()
    for o, lse, (o_ref, lse_ref) in ((o1, lse1, ref1), (o2, lse2, ref2)):
        assert torch.all(o[0].float() == 0) and torch.all(torch.isneginf(lse[0]))
        assert row_rel_err(host(o), o_ref) <= 1e-2
        assert lse_abs_err(host(lse), lse_ref) <= 1e-2
    assert torch.equal(o1, o3) and torch.equal(lse1, lse3)


@pytest.mark.parametrize("B,Q,H,N", [(8, 1, 64, 1000), (3, 2, 48, 301), (2, 1, 16, 1)])
def test_hca_pool_attend_against_the_oracle(B, Q, H, N):
    """hca_pool_attend (the newest 128-token block pooled on free workgroups of the attention
    launch, its entry merged as a part of its own): the pooled cache row and the attention
    against the oracle (pooling, then dense attention over every visible entry and the
    window); a query that does not see the new entry; the call twice in a row, bitwise."""
    cfg = 560 + B + N
    D, m, Lw, W = 512, 128, 128, 128
    T = N * m
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    kv = synth.normal(cfg, synth.KC, (B, N, 2 * D))
    win = synth.normal(cfg, synth.KW, (B, Lw, 2 * D))                  # the newest Lw raw tokens (K|V)
    gate = synth.normal(cfg, synth.GATE, (B, m))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    wpos0 = np.full(B, T - Lw, np.int32)
    pos = np.tile((T - 1 - np.arange(Q, dtype=np.int32) * 3)[None], (B, 1))
    pos[B - 1, 0] = T - 2                                               # sees entries [0, N - 1) only
    (qd, qb), (kvd, kvb), (wd, wb) = dev_bf16(q), dev_bf16(kv), dev_bf16(win)
    scale = 1.0 / math.sqrt(D)
    outs = []
    for _ in range(2):
        o, lse = L.hca_pool_attend(wd[:, Lw - m:], dev(gate), dev(bias), qd, kvd[..., :D], kvd[..., D:], m, wd[..., :D],
                                   wd[..., D:], dev(wpos0), W, dev(pos), scale)
        outs.append((o.clone(), lse.clone(), kvd[:, N - 1].clone()))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b_) for a, b_ in zip(outs[0], outs[1]))
    dec = codecs.decode_bf16
    new = method.compress(dec(wb[:, Lw - m:]), gate, bias, m)[:, 0]       # [B, 2D] exact pooled entry
    row = host(outs[0][2])
    assert np.all(np.abs(row - new) <= compress_tol(dec(wb[:, Lw - m:]), m, new[:, None])[:, 0])
    rows = dec(kvb).copy()
    rows[:, N - 1] = row                                                # the cache as the call left it
    wr = dec(wb)
    o_ref, lse_ref = method.hca_attend(dec(qb), rows[..., :D], rows[..., D:], m, wr[..., :D], wr[..., D:], wpos0, W,
                                       pos, scale)
    assert row_rel_err(host(outs[0][0]), o_ref) <= 1e-2
    assert lse_abs_err(host(outs[0][1]), lse_ref) <= 1e-2


def test_attend_empty_key_set_and_determinism():
    B, Q, H, D, N, L_ = 1, 2, 64, 512, 64, 32
    q, kc, vc, kw, vw = _attn_inputs(500, B, Q, H, D, N, L_)
    t = [dev_bf16(a)[0] for a in (q, kc, vc, kw, vw)]
    win_pos0 = np.array([10000], dtype=np.int32)
    pos = np.array([[5, 100]], dtype=np.int32)                  # no visible block (m=128), window ahead
    o, lse = L.hca_attend(t[0], t[1], t[2], 128, t[3], t[4], dev(win_pos0), 16, dev(pos), 0.1)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))
    pos = np.array([[128 * 64 - 1, 128 * 30]], dtype=np.int32)
    r1 = L.hca_attend(t[0], t[1], t[2], 128, t[3], t[4], dev(win_pos0), 16, dev(pos), 0.1)
    r2 = L.hca_attend(t[0], t[1], t[2], 128, t[3], t[4], dev(win_pos0), 16, dev(pos), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


# ============================================================ FP8 K/V rows
DR = 64   # RoPE dims of a K row kept in bf16


def _fp8_kv(cfg, B, N, L_, D, k_scale, v_scale):
    """Seeded K/V caches and windows as FP8 byte rows (the oracle's encoder) and their
    float64 decoding (the oracle's decoder)."""
    _, kc, vc, kw, vw = _attn_inputs(cfg, B, 1, 1, D, N, L_)
    rows = [codecs.encode_fp8_k_rows(kc, DR, k_scale), codecs.encode_fp8_v_rows(vc, v_scale),
            codecs.encode_fp8_k_rows(kw, DR, k_scale), codecs.encode_fp8_v_rows(vw, v_scale)]
    dec = [codecs.decode_fp8_k_rows(rows[0], D, DR, k_scale), codecs.decode_fp8_v_rows(rows[1], v_scale),
           codecs.decode_fp8_k_rows(rows[2], D, DR, k_scale), codecs.decode_fp8_v_rows(rows[3], v_scale)]
    return rows, dec


@pytest.mark.parametrize("H,Q", [(64, 2), (32, 3)])
def test_csa_attend_fp8kv(H, Q):
    """Selected entries (short list, out-of-range entries) plus a linear window, with
    non-power-of-two scales; the oracle attends over the decoded rows."""
    cfg = 700 + H
    B, D, N, L_, W, k = 2, 512, 3000, 160, 128, 512
    ks, vs = 0.71, 1.37
    (kcb, vcb, kwb, vwb), (kcd, vcd, kwd, vwd) = _fp8_kv(cfg, B, N, L_, D, ks, vs)
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    idx[0, 0, -7:] = -1
    idx[1, 0, 3] = N + 5
    win_pos0 = np.array([40000, 7], dtype=np.int32)
    pos = np.array([[40000 + 150, 40000 + 20, 40000 + 159][:Q], [7 + 127, 7 + 300, 3][:Q]], dtype=np.int32)
    qd, qb = dev_bf16(q)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.csa_attend_fp8kv(qd, dev(kcb), dev(vcb), dev(idx), dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos),
                                scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    o_ref, lse_ref = method.csa_attend(codecs.decode_bf16(qb), kcd, vcd, idx, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


@pytest.mark.parametrize("N", [1000, 45])
def test_hca_attend_fp8kv_ring_window(N):
    """Every visible entry (several splits and a ragged tail, or fewer entries than one
    tile) plus a ring window (position p in row p % L)."""
    cfg = 720 + N
    B, Q, H, D, m, Lw, W = 2, 3, 64, 512, 128, 256, 128
    ks, vs = 2.0 ** -2, 3.1
    (kcb, vcb, kwl, vwl), (kcd, vcd, kwd, vwd) = _fp8_kv(cfg, B, N, Lw, D, ks, vs)
    pmax = np.array([N * m + 40, N * m - 7])
    qpos = np.stack([pmax, pmax - 1, pmax - 90], axis=1).astype(np.int32)   # windows inside the ring
    wp0 = (pmax - Lw + 1).astype(np.int32)
    kwr, vwr = np.empty_like(kwl), np.empty_like(vwl)
    for b in range(B):
        rr = (wp0[b] + np.arange(Lw)) % Lw
        kwr[b, rr], vwr[b, rr] = kwl[b], vwl[b]
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    qd, qb = dev_bf16(q)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.hca_attend_fp8kv(qd, dev(kcb), dev(vcb), m, dev(kwr), dev(vwr), None, W, dev(qpos), scale,
                                k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    o_ref, lse_ref = method.hca_attend(codecs.decode_bf16(qb), kcd, vcd, m, kwd, vwd, wp0, W, qpos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


def test_attend_fp8kv_side_by_side_and_every_code():
    """K and V rows side by side in one row of 576 + 512 bytes give the same bits as
    separate tensors; code bytes drawn over every finite E4M3 code (subnormals, zeros,
    +-448) still match the oracle."""
    cfg = 760
    B, Q, H, D, N, L_, W, k, m = 2, 2, 48, 512, 700, 140, 128, 256, 4
    ks, vs = 2.0 ** -6, 2.0 ** -5
    r = np.random.default_rng(cfg)

    def draw(shape):                      # any finite code (the two NaN codes become zero)
        c = r.integers(0, 256, size=shape).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0
        return c

    kcb = np.concatenate([draw((B, N, D - DR)), synth.bf16_bits(synth.normal(cfg, synth.KC, (B, N, DR)))
                          .astype("<u2").view(np.uint8).reshape(B, N, 2 * DR)], axis=2)
    kwb = np.concatenate([draw((B, L_, D - DR)), synth.bf16_bits(synth.normal(cfg, synth.KW, (B, L_, DR)))
                          .astype("<u2").view(np.uint8).reshape(B, L_, 2 * DR)], axis=2)
    vcb, vwb = draw((B, N, D)), draw((B, L_, D))
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    win_pos0 = np.array([2700, 2000], dtype=np.int32)
    pos = np.array([[2799, 2750], [2100, 2139]], dtype=np.int32)
    qd, qb = dev_bf16(q)
    scale = 1.0 / math.sqrt(D)
    kvc = dev(np.concatenate([kcb, vcb], axis=2))
    kvw = dev(np.concatenate([kwb, vwb], axis=2))
    KB = D + DR
    o1, l1 = L.csa_attend_fp8kv(qd, kvc[..., :KB], kvc[..., KB:], dev(idx), kvw[..., :KB], kvw[..., KB:],
                                dev(win_pos0), W, dev(pos), scale, k_scale=ks, v_scale=vs)
    o2, l2 = L.csa_attend_fp8kv(qd, dev(kcb), dev(vcb), dev(idx), dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos),
                                scale, k_scale=ks, v_scale=vs)
    h1, hl1 = L.hca_attend_fp8kv(qd, kvc[..., :KB], kvc[..., KB:], m, kvw[..., :KB], kvw[..., KB:], dev(win_pos0), W,
                                 dev(pos), scale, k_scale=ks, v_scale=vs, N=300)
    h2, hl2 = L.hca_attend_fp8kv(qd, dev(kcb), dev(vcb), m, dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos), scale,
                                 k_scale=ks, v_scale=vs, N=300)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(h1, h2) and torch.equal(hl1, hl2)
    kd, vd = codecs.decode_fp8_k_rows(kcb, D, DR, ks), codecs.decode_fp8_v_rows(vcb, vs)
    kwd, vwd = codecs.decode_fp8_k_rows(kwb, D, DR, ks), codecs.decode_fp8_v_rows(vwb, vs)
    o_ref, lse_ref = method.csa_attend(codecs.decode_bf16(qb), kd, vd, idx, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host(o1), o_ref) <= 1e-2
    assert lse_abs_err(host(l1), lse_ref) <= 1e-2
    h_ref, hl_ref = method.hca_attend(codecs.decode_bf16(qb), kd[:, :300], vd[:, :300], m, kwd, vwd, win_pos0, W,
                                      pos, scale)
    assert row_rel_err(host(h1), h_ref) <= 1e-2
    assert lse_abs_err(host(hl1), hl_ref) <= 1e-2


def test_csa_attend_fp8kv_many_queries():
    """Enough queries for one workgroup per query: each query's list of 1024 entries plus
    its window is cut into splits of at most 512 list slots (the FP8 kernel's index list)."""
    cfg = 790
    B, Q, H, D, N, L_, W, k = 1, 260, 16, 512, 5000, 400, 128, 1024
    ks, vs = 0.5, 1.75
    (kcb, vcb, kwb, vwb), (kcd, vcd, kwd, vwd) = _fp8_kv(cfg, B, N, L_, D, ks, vs)
    q = synth.normal(cfg, synth.Q, (B, Q, H, D))
    idx = synth.sorted_unique_indices(cfg, synth.IDX, B * Q, N, k).reshape(B, Q, k)
    idx[0, 5, 900:] = -1
    win_pos0 = np.array([80000], dtype=np.int32)
    pos = (80000 + 130 + np.arange(Q, dtype=np.int32))[None, :]
    qd, qb = dev_bf16(q)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.csa_attend_fp8kv(qd, dev(kcb), dev(vcb), dev(idx), dev(kwb), dev(vwb), dev(win_pos0), W, dev(pos),
                                scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    o_ref, lse_ref = method.csa_attend(codecs.decode_bf16(qb), kcd, vcd, idx, kwd, vwd, win_pos0, W, pos, scale)
    assert row_rel_err(host(o), o_ref) <= 1e-2
    assert lse_abs_err(host(lse), lse_ref) <= 1e-2


def test_attend_fp8kv_empty_key_sets():
    """No compressed entries and no window row in range: o = 0 and lse = -inf (CSA with N = 0
    and a list of slots, HCA before its first complete block)."""
    B, Q, H, D, L_ = 1, 2, 64, 512, 32
    (kcb, vcb, kwb, vwb), _ = _fp8_kv(780, B, 8, L_, D, 1.0, 1.0)
    q, _ = dev_bf16(synth.normal(780, synth.Q, (B, Q, H, D)))
    win_pos0 = np.array([10000], dtype=np.int32)
    pos = np.array([[5, 100]], dtype=np.int32)
    idx = np.zeros((B, Q, 16), dtype=np.int32)
    o, lse = L.csa_attend_fp8kv(q, dev(kcb), dev(vcb), dev(idx), dev(kwb), dev(vwb), dev(win_pos0), 16, dev(pos), 0.1,
                                N=0)
    h, hl = L.hca_attend_fp8kv(q, dev(kcb), dev(vcb), 128, dev(kwb), dev(vwb), dev(win_pos0), 16, dev(pos), 0.1)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(h.float() == 0) and torch.all(torch.isneginf(hl))


def test_lse_merge():
    r = np.random.default_rng(600)
    P, R, D = 5, 37, 512
    o = r.standard_normal((P, R, D)).astype(np.float32)
    lse = (r.standard_normal((P, R)) * 3).astype(np.float32)
    lse[2, :5] = -np.inf
    lse[:, 7] = -np.inf
    out, lo = L.lse_merge(dev(o), dev(lse), torch.float32)
    outb, _ = L.lse_merge(dev(o), dev(lse), torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, l_ref = method.lse_merge(o.astype(np.float64), lse.astype(np.float64))
    assert row_rel_err(host(out), o_ref) <= 1e-5
    assert row_rel_err(host(outb), o_ref) <= 1e-2
    assert lse_abs_err(host(lo), l_ref) <= 1e-5


# ============================================================ c1 end to end (fp32)
def test_c1_csa_decode_end_to_end_f32():
    """Tiny CSA decode: compress 4x, index, top-64, attend over selection + 128-token window."""
    cfg = 1
    T, D, DI, HI, H, m, k, W = 4096, 128, 64, 4, 16, 4, 64, 128
    rk = synth.normal(cfg, synth.RAW_K, (1, T, D))
    rv = synth.normal(cfg, synth.RAW_V, (1, T, D))
    rki = synth.normal(cfg, synth.RAW_KI, (1, T, DI))
    gate = synth.normal(cfg, synth.GATE, (1, T))
    bias = synth.normal(cfg, synth.BIAS, (m,), std=0.1)
    q = synth.normal(cfg, synth.Q, (1, 1, H, D))
    qi = synth.normal(cfg, synth.QI, (1, 1, HI, DI))
    w = synth.uniform(cfg, synth.WI, (1, 1, HI))
    pos = np.array([[T - 1]], dtype=np.int32)
    win_pos0 = np.array([T - W], dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    g, bb = dev(gate), dev(bias)
    kc = L.csa_compress(dev(rk), g, bb, m, torch.float32)
    vc = L.csa_compress(dev(rv), g, bb, m, torch.float32)
    kic = L.csa_compress(dev(rki), g, bb, m, torch.float32)
    idx = L.csa_index_topk(dev(qi), dev(w), kic, dev(pos), m, k)
    kw = dev(np.ascontiguousarray(rk[:, T - W:]))
    vw = dev(np.ascontiguousarray(rv[:, T - W:]))
    o, lse = L.csa_attend(dev(q), kc, vc, idx, kw, vw, dev(win_pos0), W, dev(pos), scale)
    torch.cuda.synchronize()
    # oracle chain from the raw inputs
    kc_r = method.compress(rk.astype(np.float64), gate, bias, m)
    vc_r = method.compress(rv.astype(np.float64), gate, bias, m)
    ki_r = method.compress(rki.astype(np.float64), gate, bias, m)
    o_r, lse_r, idx_r, s_r = method.csa_decode(q, kc_r, vc_r, qi, w, ki_r, rk[:, T - W:], rv[:, T - W:], win_pos0, W,
                                               pos, m, k, scale)
    idx_g = idx.cpu().numpy()
    assert check_topk(idx_g[0, 0], s_r[0, 0], T // m, k) == 0
    assert np.array_equal(idx_g, idx_r)
    assert row_rel_err(host(o), o_r) <= 1e-4
    assert lse_abs_err(host(lse), lse_r) <= 1e-4

"""The C ABI without a GPU: the library loads, exports every declared entry point, and
rejects bad arguments (and answers workspace-size queries) before touching the device."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library will share)

import long_context_attention_25_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsv4attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:dsv4_status|int|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"csa_compress", "csa_index_topk", "csa_attend", "hca_attend", "lse_merge",
                          "dsv4_last_error", "dsv4_status_string", "dsv4_version"}
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_debug_flags_release_and_debug_builds():
    """The release build answers dsv4_debug_flags with DSV4_ERR_UNSUPPORTED; the debug build
    exports every declared entry point too."""
    v = ctypes.c_uint32(7)
    assert L.lib().dsv4_debug_flags(ctypes.byref(v)) == 2 and v.value == 0
    assert L.lib().dsv4_debug_flags(None) == 1
    if os.path.exists(L.DEBUG_LIB_PATH):
        dbg = ctypes.CDLL(L.DEBUG_LIB_PATH)
        for n in declared_functions():
            assert hasattr(dbg, n), n


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.dsv4_version() >= 100
    assert lib.dsv4_status_string(0) == b"DSV4_OK"
    assert lib.dsv4_status_string(3) == b"DSV4_ERR_WORKSPACE"
    assert lib.dsv4_status_string(99) == b"DSV4_ERR_UNKNOWN"


P = ctypes.c_void_p(16)   # a non-NULL pointer that is never dereferenced (validation fails first)


def _compress(**kw):
    a = dict(x=P, x_dt=1, gate=P, bias=P, B=1, T=16, C=64, m=4, xbs=0, y=P, ysc=P, ydt=1, ybs=0)
    a.update(kw)
    return L.lib().csa_compress(a["x"], a["x_dt"], a["gate"], a["bias"], a["B"], a["T"], a["C"], a["m"], a["xbs"],
                                a["y"], a["ysc"], a["ydt"], a["ybs"], None)


def test_compress_validation():
    assert _compress(m=0) == 1
    assert _compress(T=18) == 1 and b"multiple of m" in L.lib().dsv4_last_error()
    assert _compress(x_dt=2) == 2
    assert _compress(C=12) == 2
    assert _compress(C=4096) == 2
    assert _compress(ydt=3, C=48) == 2
    assert _compress(x=None) == 1
    assert _compress(ydt=3, ysc=None) == 1
    assert _compress(xbs=8) == 1
    assert _compress(B=0) == 0                       # nothing to do: no launch
    assert L.lib().dsv4_last_error() == b""


def _append(**kw):
    a = dict(x=P, x_dt=1, g=P, pos=P, B=2, C=1024, win=P, wg=P, L=256, bias=P, m=128, y=P, ysc=None, ydt=1, N=64,
             ybs=0)
    a.update(kw)
    return L.lib().kv_cache_append(a["x"], a["x_dt"], a["g"], a["pos"], a["B"], a["C"], a["win"], a["wg"], a["L"],
                                   a["bias"], a["m"], a["y"], a["ysc"], a["ydt"], a["N"], a["ybs"], None)


def _compress2(**kw):
    a = dict(x=P, x2=P, x_dt=1, gate=P, bias=P, B=1, T=16, m=4, C=1024, xbs=0, y=P, ysc=None, ydt=1, ybs=0,
             C2=128, x2bs=0, y2=P, y2sc=P, y2dt=3, y2bs=0)
    a.update(kw)
    return L.lib().csa_compress2(a["x"], a["x2"], a["x_dt"], a["gate"], a["bias"], a["B"], a["T"], a["m"], a["C"],
                                 a["xbs"], a["y"], a["ysc"], a["ydt"], a["ybs"], a["C2"], a["x2bs"], a["y2"],
                                 a["y2sc"], a["y2dt"], a["y2bs"], None)


def test_compress2_validation():
    assert _compress2(B=0) == 0                              # nothing to pool: no launch
    assert _compress2(ydt=0) == 2                            # f32 K|V output: unsupported here
    assert _compress2(y2dt=1) == 2                           # the second job must be MXFP4
    assert _compress2(x_dt=0) == 2
    assert _compress2(y2sc=None) == 1                        # MXFP4 needs its scales
    assert _compress2(T=18) == 1
    assert _compress2(C2=48) == 2                            # MXFP4 groups of 32
    assert _compress2(x2=None) == 1


def test_cache_append_validation():
    assert _append(m=0) == 1
    assert _append(L=200) == 1 and b"multiple of m" in L.lib().dsv4_last_error()
    assert _append(L=64) == 1
    assert _append(x_dt=2) == 2
    assert _append(C=12) == 2
    assert _append(ydt=3, C=48) == 2
    assert _append(ydt=3, ysc=None) == 1
    assert _append(win=None) == 1
    assert _append(ybs=10) == 1
    assert _append(y=None, N=0, B=0) == 0             # nothing to do: no launch
    assert L.lib().dsv4_last_error() == b""


def _index(ws=None, n=None, **kw):
    a = dict(qi=P, qdt=1, wi=P, ki=P, ksc=None, kdt=1, qpos=P, B=8, Q=1, HI=8, DI=128, N=262144, kbs=0, m=4, k=1024,
             oi=P, osc=None)
    a.update(kw)
    n = ctypes.c_size_t(0) if n is None else n
    st = L.lib().csa_index_topk(a["qi"], a["qdt"], a["wi"], a["ki"], a["ksc"], a["kdt"], a["qpos"], a["B"], a["Q"],
                                a["HI"], a["DI"], a["N"], a["kbs"], a["m"], a["k"], a["oi"], a["osc"], ws,
                                ctypes.byref(n), None)
    return st, n.value


def test_index_topk_validation_and_workspace_query():
    st, n = _index()
    # a decode-shaped call: fp32 scores, then up to 64 candidates of each 4096-key chunk
    # (64 chunks per row) and one 16-byte record per chunk
    assert st == 0 and n == 8 * 262144 * 4 + 8 * 64 * 64 * 8 + 8 * 64 * 16
    # many queries per sequence: scores, row histograms, bitmaps and a candidate slot per key
    st, n = _index(B=1, Q=4096, N=65536)
    assert st == 0 and n >= 4096 * 65536 * 12
    assert _index(k=0)[0] == 1
    assert _index(k=5000)[0] == 1
    assert _index(HI=6)[0] == 2
    assert _index(DI=96)[0] == 2
    assert _index(qdt=0)[0] == 2                        # (F32, BF16) is not a supported pair
    assert _index(kdt=3)[0] == 1                        # MXFP4 keys need scales
    assert _index(kdt=3, ksc=P)[0] == 0
    assert _index(kbs=5)[0] == 1
    assert _index(m=0)[0] == 1
    st, _ = _index(ws=P, n=ctypes.c_size_t(100))
    assert st == 3 and b"smaller" in L.lib().dsv4_last_error()


def _attend(csa=True, ws=None, **kw):
    a = dict(q=P, kc=P, vc=P, dt=1, idx=P, k=1024, kw=P, vw=P, wp0=P, L=128, W=128, qpos=P, B=8, Q=1, H=64, D=512,
             N=262144, kvbs=0, kvrs=0, wrs=0, scale=0.044, out=P, lse=P, m=128)
    a.update(kw)
    n = ctypes.c_size_t(0)
    if csa:
        st = L.lib().csa_attend(a["q"], a["kc"], a["vc"], a["dt"], a["idx"], a["k"], a["kw"], a["vw"], a["wp0"],
                                a["L"], a["W"], a["qpos"], a["B"], a["Q"], a["H"], a["D"], a["N"], a["kvbs"],
                                a["kvrs"], a["wrs"], a["scale"], a["out"], a["lse"], ws, ctypes.byref(n), None)
    else:
        st = L.lib().hca_attend(a["q"], a["kc"], a["vc"], a["dt"], a["m"], a["kw"], a["vw"], a["wp0"], a["L"],
                                a["W"], a["qpos"], a["B"], a["Q"], a["H"], a["D"], a["N"], a["kvbs"], a["kvrs"],
                                a["wrs"], a["scale"], a["out"], a["lse"], ws, ctypes.byref(n), None)
    return st, n.value


def test_attend_validation_and_workspace_query():
    st, n = _attend()
    assert st == 0 and n > 0                            # split-K partials
    st, n = _attend(csa=False, N=8192)
    assert st == 0 and n > 0
    assert _attend(D=96)[0] == 2
    assert _attend(H=40)[0] == 2
    assert _attend(dt=2)[0] == 2
    assert _attend(idx=None)[0] == 1
    assert _attend(q=None)[0] == 1
    assert _attend(csa=False, m=0)[0] == 1
    assert _attend(kvbs=7)[0] == 1
    assert _attend(kvrs=1024, wrs=1024)[0] == 0          # K and V side by side
    assert _attend(kvrs=100)[0] == 1                     # narrower than D
    assert _attend(wrs=1028)[0] == 1                     # bf16 rows must stay 16-byte aligned
    assert _attend(scale=float("nan"))[0] == 1
    assert _attend(dt=0, D=128, H=16)[0] == 0           # f32 path needs no workspace
    assert _attend(dt=0, D=1024, H=16)[0] == 2
    assert _attend(wp0=None)[0] == 0                     # ring window (W <= L)
    assert _attend(wp0=None, W=256)[0] == 1 and b"ring" in L.lib().dsv4_last_error()


def test_attend_split_count_stays_within_the_merge_limit():
    """The split-K merge holds at most 1024 part weights: a key list longer than 1024 splits
    of the longest CSA chunk is rejected before any launch; a dense (HCA) list of any length
    is planned with longer splits instead."""
    win = 3_000_000
    st, _ = _attend(W=win, L=win)                                   # bf16 CSA: 2048-entry chunks
    assert st == 2 and b"1024 splits" in L.lib().dsv4_last_error()
    assert _attend_fp8(W=600_000, L=600_000)[0] == 2               # FP8 CSA: 512-entry chunks
    st, n = _attend(csa=False, N=40_000_000, W=128, L=256)          # HCA: longer splits, accepted
    assert st == 0 and n > 0
    assert _attend(W=1_000_000, L=1_000_000)[0] == 0                 # within 1024 x 2048

def _attend_fp8(csa=True, **kw):
    a = dict(q=P, kc=P, vc=P, idx=P, k=512, m=128, kw=P, vw=P, wp0=P, L=256, W=128, qpos=P, B=8, Q=1, H=64, D=512,
             dr=64, N=262144, kvbs=0, kvrs=0, wrs=0, ks=1.0, vs=1.0, scale=0.04, out=P, lse=P)
    a.update(kw)
    n = ctypes.c_size_t(0)
    lib = L.lib()
    if csa:
        st = lib.csa_attend_fp8kv(a["q"], a["kc"], a["vc"], a["idx"], a["k"], a["kw"], a["vw"], a["wp0"], a["L"],
                                  a["W"], a["qpos"], a["B"], a["Q"], a["H"], a["D"], a["dr"], a["N"], a["kvbs"],
                                  a["kvrs"], a["wrs"], a["ks"], a["vs"], a["scale"], a["out"], a["lse"], None,
                                  ctypes.byref(n), None)
    else:
        st = lib.hca_attend_fp8kv(a["q"], a["kc"], a["vc"], a["m"], a["kw"], a["vw"], a["wp0"], a["L"], a["W"],
                                  a["qpos"], a["B"], a["Q"], a["H"], a["D"], a["dr"], a["N"], a["kvbs"], a["kvrs"],
                                  a["wrs"], a["ks"], a["vs"], a["scale"], a["out"], a["lse"], None, ctypes.byref(n),
                                  None)
    return st, n.value


def test_attend_fp8kv_validation_and_workspace_query():
    st, n = _attend_fp8()
    assert st == 0 and n > 0
    st, n = _attend_fp8(csa=False, N=8192)
    assert st == 0 and n > 0
    assert _attend_fp8(D=256)[0] == 2                       # D = 512 only
    assert _attend_fp8(dr=32)[0] == 2                       # d_rope = 64 only
    assert _attend_fp8(H=40)[0] == 2
    assert _attend_fp8(kvrs=1088, wrs=1088)[0] == 0         # K and V side by side (576 + 512 bytes)
    assert _attend_fp8(kvrs=512)[0] == 1                    # narrower than a K row
    assert _attend_fp8(wrs=584)[0] == 1                     # not a multiple of 16 bytes
    assert _attend_fp8(kc=ctypes.c_void_p(24))[0] == 1      # not 16-byte aligned
    assert _attend_fp8(ks=float("inf"))[0] == 1
    assert _attend_fp8(vs=float("nan"))[0] == 1
    assert _attend_fp8(idx=None)[0] == 1
    assert _attend_fp8(csa=False, m=0)[0] == 1
    assert _attend_fp8(wp0=None, W=512)[0] == 1             # ring window needs W <= L


def test_lse_merge_validation():
    lib = L.lib()
    assert lib.lse_merge(P, P, 0, 4, 8, P, 0, P, None) == 1
    assert lib.lse_merge(P, P, 2, 4, 6, P, 0, P, None) == 1
    assert lib.lse_merge(P, P, 2, 4, 8, P, 2, P, None) == 2
    assert lib.lse_merge(P, P, 2, 0, 8, P, 0, P, None) == 0


def test_ceiling_probe_library_exports():
    """The benchmark's measurement helpers (HBM-read and MFMA-throughput kernels) build into a
    library of their own that exports its two entry points; nothing is launched here."""
    path = os.path.join(os.path.dirname(L.LIB_PATH), "libdsv4probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    probe = ctypes.CDLL(path)
    for name in ("dsv4probe_read", "dsv4probe_mfma"):
        assert hasattr(probe, name), name


def test_binding_rejects_strided_operands_before_any_call():
    """The kernels read packed row-major arrays: the binding raises ValueError for views whose
    rows are not packed (checked on host tensors, before the library is called)."""
    B, Q, HI, DI, N = 2, 1, 8, 128, 64
    qi = torch.zeros((B, Q, HI, DI), dtype=torch.bfloat16)
    wi = torch.zeros((B, Q, HI))
    qpos = torch.zeros((B, Q), dtype=torch.int32)
    ki = torch.zeros((B, N, 2 * DI), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ki rows"):
        L.csa_index_topk(qi, wi, ki[..., :DI], qpos, 4, 16)          # column slice: rows not packed
    with pytest.raises(ValueError, match="qi must be contiguous"):
        L.csa_index_topk(torch.zeros((B, Q, HI, 2 * DI), dtype=torch.bfloat16)[..., :DI], wi,
                         ki[..., :DI].contiguous(), qpos, 4, 16)
    H, D, k = 16, 128, 8
    q = torch.zeros((B, Q, H, D), dtype=torch.bfloat16)
    kc = torch.zeros((B, N, D), dtype=torch.bfloat16)
    kw = torch.zeros((B, 16, D), dtype=torch.bfloat16)
    wp0 = torch.zeros(B, dtype=torch.int32)
    idx = torch.zeros((B, Q, 2 * k), dtype=torch.int32)[..., ::2]
    with pytest.raises(ValueError, match="idx must be contiguous"):
        L.csa_attend(q, kc, kc, idx, kw, kw, wp0, 16, qpos, 0.1)
    with pytest.raises(ValueError, match="q must be contiguous"):
        L.hca_attend(torch.zeros((B, Q, H, 2 * D), dtype=torch.bfloat16)[..., :D], kc, kc, 4, kw, kw, wp0, 16,
                     qpos, 0.1)
    with pytest.raises(ValueError, match="out must be contiguous"):
        L.hca_attend(q, kc, kc, 4, kw, kw, wp0, 16, qpos, 0.1, out=torch.zeros((B, Q, H, 2 * D),
                                                                                dtype=torch.bfloat16)[..., :D])
    with pytest.raises(ValueError, match="o_parts must be contiguous"):
        L.lse_merge(torch.zeros((2, 8, 32))[..., :16], torch.zeros((2, 8)))


def test_noalloc_index_rejects_a_call_larger_than_its_scratch():
    """csa_index_topk_noalloc refuses, before touching the device, a call whose scratch need
    exceeds the library's 48 MiB array (here 2^28 keys of one query)."""
    lib = L.lib()
    st = lib.csa_index_topk_noalloc(P, 1, P, P, P, 3, P, 1, 1, 8, 128, 1 << 28, 0, 4, 64, P, None, None)
    assert st == 2 and b"static scratch" in lib.dsv4_last_error()
    assert lib.csa_index_topk_noalloc(P, 1, P, P, P, 3, P, 1, 1, 8, 128, 1000, 0, 4, 0, P, None, None) == 1

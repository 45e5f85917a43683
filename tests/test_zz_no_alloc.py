"""csa_index_topk_noalloc (csa_index_topk with its scratch in a library-owned static
array, for callers that cannot allocate) against csa_index_topk with a caller workspace:
identical index sets and scores, on two calls in a row, the second with a smaller input
(the array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(L, qi, qi_dt, wi, ki, ks, ki_dt, qpos, DI, N, m, k):
    B, Q, HI = qi.shape[:3]
    idx = torch.full((B, Q, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Q, k), 7.0, dtype=torch.float32, device="cuda")
    lib = L.lib()
    st = lib.csa_index_topk_noalloc(_p(qi), qi_dt, _p(wi), _p(ki), _p(ks), ki_dt, _p(qpos), B, Q, HI, DI, N, 0, m, k,
                                    _p(idx), _p(sc), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.dsv4_last_error().decode()
    return idx, sc


def test_noalloc_index_topk_matches_the_workspace_call_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_25_amd as L
    # call 1: the 1M-context decode shape (B = 8, 262,144 MXFP4 keys, top-1024)
    B, N, HI, DI, k, m = 8, 262144, 8, 128, 1024, 4
    print("noalloc call 1: B=8 N=262144 MXFP4 keys k=1024", flush=True)
    ki = torch.empty((B, N, DI // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, N, DI // 32), dtype=torch.uint8, device="cuda")
    z1 = torch.zeros(1, device="cuda")
    for b in range(B):
        k32 = synth.device_normal((1, N, DI), 7700 + b, torch.float32)
        L.csa_compress(k32, torch.zeros((1, N), device="cuda"), z1, 1, L.MXFP4_DTYPE, out=ki[b:b + 1],
                       out_scale=ks[b:b + 1])
    qi = synth.device_normal((B, 1, HI, DI), 7710, torch.bfloat16)
    wi = synth.device_uniform((B, 1, HI), 7711)
    qpos = torch.full((B, 1), 4 * N - 1, dtype=torch.int32, device="cuda")
    qpos[3, 0] = 4 * 1000 + 2                         # a short row
    ref = L.csa_index_topk(qi, wi, ki, qpos, m, k, ki_scale=ks, with_scores=True)
    got = _noalloc(L, qi, L.BF16, wi, ki, ks, L.MXFP4, qpos, DI, N, m, k)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    # call 2: smaller (B = 2, 50,000 bf16 keys, top-300, several queries)
    B, N, Q, k = 2, 50000, 3, 300
    print("noalloc call 2: B=2 N=50000 bf16 keys k=300 Q=3", flush=True)
    ki2 = synth.device_normal((B, N, DI), 7720, torch.bfloat16)
    qi2 = synth.device_normal((B, Q, HI, DI), 7721, torch.bfloat16)
    wi2 = synth.device_uniform((B, Q, HI), 7722)
    qpos2 = torch.tensor([[4 * N - 1, 4 * N - 9, 57], [4 * 20000, 4 * N - 1, 3]], dtype=torch.int32, device="cuda")
    ref = L.csa_index_topk(qi2, wi2, ki2, qpos2, m, k, with_scores=True)
    got = _noalloc(L, qi2, L.BF16, wi2, ki2, None, L.BF16, qpos2, DI, N, m, k)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    assert int((got[0][1, 0] >= 0).sum()) == k and int((got[0][0, 2] >= 0).sum()) == 14

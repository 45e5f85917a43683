#!/usr/bin/env python3
"""CSA + HCA decode at 1M-token context on one MI355X.

One step = one new token for each of B = 8 sequences through one CSA layer and one HCA
layer, every stage in the library's HIP kernels:
  CSA: compress the newest 4-token block (K, V and the indexer key, the key quantised to
       MXFP4) into the caches; indexer over all 262,144 MXFP4 keys + top-1024 selection;
       attention over the 1024 selected entries + the 128-token window.
  HCA: compress the newest 128-token block (K, V); dense attention over all 8,192
       entries + the 128-token window; split-K partials merged by log-sum-exp.
A new block completes only every 4 (CSA) or 128 (HCA) tokens; compressing one of each in
every step is the worst case.  value = queries/s, one query = one token of one sequence
through both layers (all 64 heads).  Inputs are seeded synthetic tensors resident in HBM;
three replicas of the streamed inputs rotate so that the 256 MB Infinity Cache does not
serve a step from the previous one.

python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

B, CTX, H, D = 8, 1 << 20, 64, 512
M_CSA, M_HCA = 4, 128
N_CSA, N_HCA = CTX // M_CSA, CTX // M_HCA
HI, DI, TOPK, W, LWIN = 8, 128, 1024, 128, 128
CFG_HCA, CFG_CSA = 3, 4            # config numbers used in the seeds
HBM_PEAK_GBS = 8000.0


def seed(cfg, tid, rep, b=0):
    return 1000 * cfg + tid + 50 * rep + 100000 * (b + 1)


def algorithmic_bytes():
    """Bytes the method must move once per step (inputs read once + outputs written once)."""
    keys = B * N_CSA * (DI // 2 + DI // 32)                       # MXFP4 codes + E8M0 scales
    q_idx = B * HI * DI * 2 + B * HI * 4                          # indexer query + head weights
    csa_rows = B * (TOPK + W) * 2 * D * 2                         # selected K/V rows + window rows
    hca_rows = B * (N_HCA + W) * 2 * D * 2                        # every entry + window rows
    q_o = 2 * (2 * B * H * D * 2 + B * H * 4)                     # q, o, lse for both layers
    compress = B * (M_CSA * (2 * D + DI) * 2 + M_CSA * 4 + 2 * D * 2 + (DI // 2 + DI // 32)) \
        + B * (M_HCA * 4 + 2 * D * 2)                             # HCA block rows are the window rows
    parts = dict(csa_index_keys=keys, csa_index_q=q_idx, csa_attend_rows=csa_rows, hca_attend_rows=hca_rows,
                 q_o_lse=q_o, compress=compress)
    return sum(parts.values()), parts


# Algorithmic bytes per launch of the three big kernels (what each must read once; the
# split-K partials, scores and histograms are excluded).
KERNEL_BYTES = {
    # MXFP4 key codes + E8M0 scales of every visible block, indexer queries, head weights,
    # and the pooling of the newest block done in the same launch (raw rows in, pooled rows out)
    "index_mfma_kernel": B * N_CSA * (DI // 2 + DI // 32) + B * HI * DI * 2 + B * HI * 4
    + B * (M_CSA * (2 * D + DI) * 2 + M_CSA * 4 + 2 * D * 2 + (DI // 2 + DI // 32)),
    # the selected K/V rows + window rows, q, the index list
    "attend_bf16_kernel (CSA)": B * (TOPK + W) * 2 * D * 2 + B * H * D * 2 + B * TOPK * 4,
    # every visible K/V entry + window rows, q, and the pooling of the newest block done in
    # the same launch (its 128 raw rows are the window rows, read a second time; gates; the
    # pooled row out)
    "attend_bf16_kernel (HCA)": B * (N_HCA + W) * 2 * D * 2 + B * H * D * 2
    + B * (M_HCA * 2 * D * 2 + M_HCA * 4 + 2 * D * 2),
}

# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs, each scaled by
# the counter's reading for a 256 MiB device copy (see profiles/).  An entry is used only
# while the kernel source it was measured on is unchanged (sha256 of the file).
MEASURED_TRAFFIC = {
    "index_mfma_kernel": {"bytes_per_launch": 151870796,
        "source_sha256": "bc3130e1f1eb6f0db2c6dc3ad925ae4439b373c456f0e70ef8a43d11749ae99f"},
    "attend_bf16_kernel (HCA)": {"bytes_per_launch": 157989339,
        "source_sha256": "d06b252d9fbb7db53c5156c03001dd0ebdbaea00a299f956ba8f58a9c8c628ae"},
    "attend_bf16_kernel (CSA)": {"bytes_per_launch": 32835048,
        "source_sha256": "d06b252d9fbb7db53c5156c03001dd0ebdbaea00a299f956ba8f58a9c8c628ae"},
}


class Workload:
    """Device tensors of the 1M-context decode step (three replicas of the streamed inputs)."""

    def __init__(self, L, torch, synth, replicas):
        dev = "cuda"
        bf = torch.bfloat16
        self.replicas = replicas
        self.q_pos = torch.full((B, 1), CTX - 1, dtype=torch.int32, device=dev)
        self.win_pos0 = torch.full((B,), CTX - LWIN, dtype=torch.int32, device=dev)
        # CSA compressed K/V cache (gathered rows only; one copy).  K and V of an entry sit
        # side by side in one [B, N, 2D] buffer, as do the raw K|V rows of the window, so
        # that one pooling call compresses both (they share the block's gate weights).
        self.kvc = torch.empty((B, N_CSA, 2 * D), dtype=bf, device=dev)
        self.kc, self.vc = self.kvc[..., :D], self.kvc[..., D:]
        for b in range(B):
            self.kc[b] = synth.device_normal((N_CSA, D), seed(CFG_CSA, synth.KC, 0, b), bf)
            self.vc[b] = synth.device_normal((N_CSA, D), seed(CFG_CSA, synth.VC, 0, b), bf)
        self.r = []
        zeros1 = torch.zeros(1, dtype=torch.float32, device=dev)
        for rep in range(replicas):
            t = {}
            t["q"] = synth.device_normal((B, 1, H, D), seed(CFG_CSA, synth.Q, rep), bf)
            t["qi"] = synth.device_normal((B, 1, HI, DI), seed(CFG_CSA, synth.QI, rep), bf)
            t["wi"] = synth.device_uniform((B, 1, HI), seed(CFG_CSA, synth.WI, rep))
            t["ki"] = torch.empty((B, N_CSA, DI // 2), dtype=torch.uint8, device=dev)
            t["ks"] = torch.empty((B, N_CSA, DI // 32), dtype=torch.uint8, device=dev)
            for b in range(B):
                k32 = synth.device_normal((1, N_CSA, DI), seed(CFG_CSA, synth.KI, rep, b), torch.float32)
                gz = torch.zeros((1, N_CSA), dtype=torch.float32, device=dev)
                L.csa_compress(k32, gz, zeros1, 1, L.MXFP4_DTYPE, out=t["ki"][b:b + 1], out_scale=t["ks"][b:b + 1])
                del k32, gz
            t["kvw"] = torch.cat([synth.device_normal((B, LWIN, D), seed(CFG_CSA, synth.KW, rep), bf),
                                  synth.device_normal((B, LWIN, D), seed(CFG_CSA, synth.VW, rep), bf)], dim=2)
            t["kw"], t["vw"] = t["kvw"][..., :D], t["kvw"][..., D:]
            t["kiw"] = synth.device_normal((B, LWIN, DI), seed(CFG_CSA, synth.RAW_KI, rep), bf)
            t["gate"] = synth.device_normal((B, LWIN), seed(CFG_CSA, synth.GATE, rep), torch.float32)
            t["bias"] = synth.device_normal((M_CSA,), seed(CFG_CSA, synth.BIAS, rep), torch.float32, std=0.1)
            # HCA layer
            t["hq"] = synth.device_normal((B, 1, H, D), seed(CFG_HCA, synth.Q, rep), bf)
            t["hkvc"] = torch.cat([synth.device_normal((B, N_HCA, D), seed(CFG_HCA, synth.KC, rep), bf),
                                   synth.device_normal((B, N_HCA, D), seed(CFG_HCA, synth.VC, rep), bf)], dim=2)
            t["hkc"], t["hvc"] = t["hkvc"][..., :D], t["hkvc"][..., D:]
            t["hkvw"] = torch.cat([synth.device_normal((B, LWIN, D), seed(CFG_HCA, synth.KW, rep), bf),
                                   synth.device_normal((B, LWIN, D), seed(CFG_HCA, synth.VW, rep), bf)], dim=2)
            t["hkw"], t["hvw"] = t["hkvw"][..., :D], t["hkvw"][..., D:]
            t["hgate"] = synth.device_normal((B, LWIN), seed(CFG_HCA, synth.GATE, rep), torch.float32)
            t["hbias"] = synth.device_normal((M_HCA,), seed(CFG_HCA, synth.BIAS, rep), torch.float32, std=0.1)
            # outputs
            t["idx"] = torch.empty((B, 1, TOPK), dtype=torch.int32, device=dev)
            t["o"] = torch.empty((B, 1, H, D), dtype=bf, device=dev)
            t["lse"] = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
            t["ho"] = torch.empty((B, 1, H, D), dtype=bf, device=dev)
            t["hlse"] = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
            self.r.append(t)
        torch.cuda.synchronize()


def marshal_step(L, torch, wl, rep):
    """The step as a list of (C function, argument tuple) with every pointer resolved."""
    lib = L.lib()
    t = wl.r[rep]
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    scale = 1.0 / math.sqrt(D)
    calls = []
    g4 = t["gate"][:, LWIN - M_CSA:].contiguous()
    t["g4"] = g4
    # CSA: the newest 4-token block -> entry N_CSA-1 of K|V (bf16, the 2D channels side by
    # side) and of the indexer key (MXFP4), pooled in the indexer launch, then indexer + top-k
    t["pool"] = L.BlockPool(P(t["kvw"][:, LWIN - M_CSA:]), P(t["kiw"][:, LWIN - M_CSA:]), P(g4), P(t["bias"]), 2 * D,
                            LWIN, LWIN, P(wl.kvc[:, N_CSA - 1]), None, L.BF16, N_CSA, N_CSA - 1)
    n = ctypes.c_size_t(0)
    idx_args = (ctypes.byref(t["pool"]), P(t["qi"]), L.BF16, P(t["wi"]), P(t["ki"]), P(t["ks"]), L.MXFP4,
                P(wl.q_pos), B, 1, HI, DI, N_CSA, 0, M_CSA, TOPK, P(t["idx"]), None)
    assert lib.csa_pool_index_topk(*idx_args, None, ctypes.byref(n), st) == 0
    t["ws_idx"] = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    t["ws_idx_n"] = ctypes.c_size_t(n.value)
    calls.append((lib.csa_pool_index_topk, idx_args + (P(t["ws_idx"]), ctypes.byref(t["ws_idx_n"]), st)))
    timed = {len(calls) - 1: "index_mfma_kernel"}
    # CSA attention
    att = (P(t["q"]), P(wl.kc), P(wl.vc), L.BF16, P(t["idx"]), TOPK, P(t["kw"]), P(t["vw"]), P(wl.win_pos0), LWIN, W,
           P(wl.q_pos), B, 1, H, D, N_CSA, 0, 2 * D, 2 * D, ctypes.c_float(scale), P(t["o"]), P(t["lse"]))
    assert lib.csa_attend(*att, None, ctypes.byref(n), st) == 0
    t["ws_csa"] = torch.empty(max(n.value, 1), dtype=torch.uint8, device="cuda")
    t["ws_csa_n"] = ctypes.c_size_t(n.value)
    calls.append((lib.csa_attend, att + (P(t["ws_csa"]), ctypes.byref(t["ws_csa_n"]), st)))
    timed[len(calls) - 1] = "attend_bf16_kernel (CSA)"
    # HCA: the newest 128-token block (the whole window) -> entry N_HCA-1 of K|V, pooled in
    # the attention launch, then dense attention over every entry and the window
    hatt = (P(t["hkvw"]), P(t["hgate"]), P(t["hbias"]), LWIN, P(t["hq"]), P(t["hkc"]), P(t["hvc"]), L.BF16, M_HCA,
            P(t["hkw"]), P(t["hvw"]), P(wl.win_pos0), LWIN, W, P(wl.q_pos), B, 1, H, D, N_HCA, 0, 2 * D, 2 * D,
            ctypes.c_float(scale), P(t["ho"]), P(t["hlse"]))
    assert lib.hca_pool_attend(*hatt, None, ctypes.byref(n), st) == 0
    t["ws_hca"] = torch.empty(max(n.value, 1), dtype=torch.uint8, device="cuda")
    t["ws_hca_n"] = ctypes.c_size_t(n.value)
    calls.append((lib.hca_pool_attend, hatt + (P(t["ws_hca"]), ctypes.byref(t["ws_hca_n"]), st)))
    timed[len(calls) - 1] = "attend_bf16_kernel (HCA)"
    return calls, timed


def time_cache_append(L, torch, wl, steps):
    """Average GPU time of one decode step of cache maintenance through kv_cache_append:
    the new token (position CTX-1, the last row of each 128-row window used as a ring)
    is appended to the CSA K|V, CSA indexer-key (MXFP4) and HCA K|V windows and completes
    a block of each layer (the worst case), which is pooled into entry N-1 of each cache.
    Outside the timed decode steps; the decode step pools with csa_compress instead (its
    cache row chosen on the host, so no kernel waits for a device-side position)."""
    lib = L.lib()
    t = wl.r[0]
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    new = {k: t[w][:, LWIN - 1].contiguous() for k, w in (("kv", "kvw"), ("ki", "kiw"), ("hkv", "hkvw"))}
    g_new, hg_new = t["gate"][:, LWIN - 1].contiguous(), t["hgate"][:, LWIN - 1].contiguous()
    calls = [
        (P(new["kv"]), L.BF16, P(g_new), P(wl.q_pos), B, 2 * D, P(t["kvw"]), P(t["gate"]), LWIN, P(t["bias"]), M_CSA,
         P(wl.kvc), None, L.BF16, N_CSA, 0, st),
        (P(new["ki"]), L.BF16, P(g_new), P(wl.q_pos), B, DI, P(t["kiw"]), P(t["gate"]), LWIN, P(t["bias"]), M_CSA,
         P(t["ki"]), P(t["ks"]), L.MXFP4, N_CSA, 0, st),
        (P(new["hkv"]), L.BF16, P(hg_new), P(wl.q_pos), B, 2 * D, P(t["hkvw"]), P(t["hgate"]), LWIN, P(t["hbias"]),
         M_HCA, P(t["hkvc"]), None, L.BF16, N_HCA, 0, st),
    ]

    def step():
        for a in calls:
            st_ = lib.kv_cache_append(*a)
            if st_ != 0:
                raise RuntimeError(lib.dsv4_last_error().decode())

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / steps


# The V4-Pro stack the pages describe: 61 layers, layers 0 and 1 HCA, layers 2 .. 60
# alternating CSA and HCA (CSA first), then an MTP block with sliding-window attention only.
SCHEDULE = ["hca", "hca"] + ["csa" if i % 2 == 0 else "hca" for i in range(2, 61)] + ["swa"]


def kv_bytes_per_token():
    """Stored cache bytes per token and layer type at this workload's storage formats (bf16
    K|V entries, MXFP4 indexer keys); the 128-row raw windows are per sequence, not per token."""
    csa = (2 * D * 2 + DI // 2 + DI // 32) / M_CSA            # K|V entry + indexer key, per 4 tokens
    hca = 2 * D * 2 / M_HCA                                   # K|V entry per 128 tokens
    return {"csa": csa, "hca": hca, "swa": 0.0}


def time_schedule(L, torch, marsh, steps):
    """One decode token for the 8 sequences through the whole layer schedule: the CSA and
    HCA layers run the decode step's calls (marsh: the marshalled step of each replica;
    replicas rotate layer by layer), the MTP layer attends over its window only.  Returns
    (us per token step, per-layer-type us)."""
    lib = L.lib()
    parts = [{"csa": c[:2], "hca": c[2:]} for c in marsh]
    # window-only attention: hca_attend with no compressed entries (the pooled HCA call's
    # arguments from q on, N = 0)
    lib_ = L.lib()
    for r, c in enumerate(marsh):
        fn, a = c[2]
        assert fn.__name__ == "hca_pool_attend"
        a = list(a[4:])
        a[15] = 0                                   # N
        parts[r]["swa"] = [(lib_.hca_attend, tuple(a))]

    def run(kinds):
        for i, kind in enumerate(kinds):
            for fn, a in parts[i % len(parts)][kind]:
                if fn(*a) != 0:
                    raise RuntimeError(lib.dsv4_last_error().decode())

    res = {}
    for name, kinds in (("schedule", SCHEDULE), ("csa", ["csa"] * 12), ("hca", ["hca"] * 12), ("swa", ["swa"] * 12)):
        run(kinds)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run(kinds)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1000.0 / (steps * len(kinds))
    return res["schedule"] * len(SCHEDULE), {k: round(res[k], 2) for k in ("csa", "hca", "swa")}


FP8_ROW = 2 * D + 64               # FP8 K|V row: 448 K codes + 64 bf16 K dims + 512 V codes
FP8_KERNEL_BYTES = {
    "attend_fp8kv_kernel (CSA)": B * (TOPK + W) * FP8_ROW + B * H * D * 2 + B * TOPK * 4,
    "attend_fp8kv_kernel (HCA)": B * (N_HCA + W) * FP8_ROW + B * H * D * 2,
}


def fp8_step_bytes():
    """Algorithmic bytes of the step with FP8 K|V rows (the bf16 step's, K/V rows at
    FP8_ROW bytes instead of 4D, pooled rows written at FP8_ROW bytes)."""
    total, parts = algorithmic_bytes()
    parts = dict(parts)
    parts["csa_attend_rows"] = B * (TOPK + W) * FP8_ROW
    parts["hca_attend_rows"] = B * (N_HCA + W) * FP8_ROW
    parts["compress"] -= 2 * B * (2 * D * 2 - FP8_ROW)          # the two pooled K|V rows
    return sum(parts.values()), parts


def run_fp8_kv(L, torch, wl, steps, warmup, every=10):
    """The decode step with the K/V caches and windows stored as FP8 K|V rows (E4M3 codes,
    bf16 RoPE dims of K): the K|V pooling writes FP8 rows, the attention reads them (the
    indexer and its MXFP4 keys as in the bf16 step).  The FP8 copies are made once by the
    library's own pooling with m = 1 (an exact per-row quantisation) before timing."""
    lib = L.lib()
    dev = "cuda"
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def to_fp8(x):                                             # [B, rows, 2D] bf16 -> [B, rows, FP8_ROW]
        out = torch.empty((x.shape[0], x.shape[1], FP8_ROW), dtype=torch.uint8, device=dev)
        for b in range(x.shape[0]):
            g = torch.zeros((1, x.shape[1]), dtype=torch.float32, device=dev)
            L.csa_compress(x[b:b + 1], g, torch.zeros(1, device=dev), 1, L.FP8_KV_DTYPE, out=out[b:b + 1])
        return out

    kvc8 = to_fp8(wl.kvc)
    KB = D + 64
    scale = 1.0 / math.sqrt(D)
    steps_calls = []
    timed = {}
    n = ctypes.c_size_t(0)
    for t in wl.r:
        t8 = {"kvw": to_fp8(t["kvw"]), "hkvc": to_fp8(t["hkvc"]), "hkvw": to_fp8(t["hkvw"])}
        calls = []
        # the newest block pooled into FP8 K|V row N_CSA-1 (and the MXFP4 key) in the indexer launch
        t8["pool"] = L.BlockPool(P(t["kvw"][:, LWIN - M_CSA:]), P(t["kiw"][:, LWIN - M_CSA:]), P(t["g4"]),
                                 P(t["bias"]), 2 * D, LWIN, LWIN, P(kvc8[:, N_CSA - 1]), None, L.FP8_KV, N_CSA,
                                 N_CSA - 1)
        idx_args = (ctypes.byref(t8["pool"]), P(t["qi"]), L.BF16, P(t["wi"]), P(t["ki"]), P(t["ks"]), L.MXFP4,
                    P(wl.q_pos), B, 1, HI, DI, N_CSA, 0, M_CSA, TOPK, P(t["idx"]), None)
        calls.append((lib.csa_pool_index_topk, idx_args + (P(t["ws_idx"]), ctypes.byref(t["ws_idx_n"]), st)))
        att = (P(t["q"]), P(kvc8), P(kvc8[..., KB:]), P(t["idx"]), TOPK, P(t8["kvw"]), P(t8["kvw"][..., KB:]),
               P(wl.win_pos0), LWIN, W, P(wl.q_pos), B, 1, H, D, 64, N_CSA, 0, FP8_ROW, FP8_ROW,
               ctypes.c_float(1.0), ctypes.c_float(1.0), ctypes.c_float(scale), P(t["o"]), P(t["lse"]))
        assert lib.csa_attend_fp8kv(*att, None, ctypes.byref(n), st) == 0
        t8["ws_csa"] = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
        t8["ws_csa_n"] = ctypes.c_size_t(n.value)
        calls.append((lib.csa_attend_fp8kv, att + (P(t8["ws_csa"]), ctypes.byref(t8["ws_csa_n"]), st)))
        timed[len(calls) - 1] = "attend_fp8kv_kernel (CSA)"
        calls.append((lib.csa_compress, (P(t["hkvw"]), L.BF16, P(t["hgate"]), P(t["hbias"]), B, M_HCA, 2 * D, M_HCA,
                                         LWIN, P(t8["hkvc"][:, N_HCA - 1:]), None, L.FP8_KV, N_HCA, st)))
        hatt = (P(t["hq"]), P(t8["hkvc"]), P(t8["hkvc"][..., KB:]), M_HCA, P(t8["hkvw"]), P(t8["hkvw"][..., KB:]),
                P(wl.win_pos0), LWIN, W, P(wl.q_pos), B, 1, H, D, 64, N_HCA, 0, FP8_ROW, FP8_ROW,
                ctypes.c_float(1.0), ctypes.c_float(1.0), ctypes.c_float(scale), P(t["ho"]), P(t["hlse"]))
        assert lib.hca_attend_fp8kv(*hatt, None, ctypes.byref(n), st) == 0
        t8["ws_hca"] = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
        t8["ws_hca_n"] = ctypes.c_size_t(n.value)
        calls.append((lib.hca_attend_fp8kv, hatt + (P(t8["ws_hca"]), ctypes.byref(t8["ws_hca_n"]), st)))
        timed[len(calls) - 1] = "attend_fp8kv_kernel (HCA)"
        t["fp8"] = t8
        steps_calls.append(calls)
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [{i: (ev.create(), ev.create()) for i in timed} for _ in range((steps + every - 1) // every)]
    for i in range(warmup):
        run_step(lib, steps_calls[i % len(steps_calls)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run_step(lib, steps_calls[i % len(steps_calls)], arm=pairs[i // every] if i % every == 0 else None)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kernels = {}
    for i, name in timed.items():
        k_ms = sum(ev.elapsed_ms(*p[i]) for p in pairs) / len(pairs)
        gbs = FP8_KERNEL_BYTES[name] / (k_ms / 1e3) / 1e9
        tr = MEASURED_TRAFFIC.get(name)
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_attention_25_amd", "csrc",
                           "attend.hip")
        kernels[name] = {"avg_launch_us": round(k_ms * 1e3, 2), "bytes_per_launch": FP8_KERNEL_BYTES[name],
                         "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": tr["bytes_per_launch"] if tr and tr["source_sha256"] == source_sha(src)
                         else None}
    total, _ = fp8_step_bytes()
    kv_tok = {"csa": (FP8_ROW + DI // 2 + DI // 32) / M_CSA, "hca": FP8_ROW / M_HCA}
    del kvc8
    for t in wl.r:
        t.pop("fp8", None)
    return {"ms_per_step": round(ms, 5), "queries_per_s": round(B / (ms / 1e3), 1), "bytes_per_step": total,
            "step_hbm_gbs": round(total / (ms / 1e3) / 1e9, 1), "kernels": kernels,
            "kv_bytes_per_token": {k: round(v, 2) for k, v in kv_tok.items()},
            "note": "the same step with K/V caches and windows as FP8 K|V rows (448 E4M3 K codes, 64 bf16 K dims, "
                    "512 E4M3 V codes per row; scales 1): pooling writes FP8 rows, attention decodes them in its "
                    "tile loop; measured after the bf16 steps, same replicas and indexer"}


class HipEvents:
    """Raw hipEvent_t pairs from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def measured_ceilings(torch):
    """Rates this GPU reaches on kernels that do nothing else (libdsv4probe.so): a 2 GiB
    streaming read with non-temporal loads (GB/s) and back-to-back dense MFMAs (TFLOP/s)
    for bf16, fp8 (16x16x32 and the scaled 16x16x128 form) and fp4.  Context for the
    roofline, whose peaks stay the published ones; None when the library is not built."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_attention_25_amd",
                        "libdsv4probe.so")
    if not os.path.exists(path):
        return None
    p = ctypes.CDLL(path)
    p.dsv4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    p.dsv4probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3          # seconds per call

    nbytes, blocks = 2 << 30, 512
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    s_read = timed(lambda: p.dsv4probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                            ctypes.c_void_p(sink.data_ptr()), blocks, st), 10)
    del buf
    res = {"hbm_read_gbs": round(nbytes / s_read / 1e9, 1), "mfma_tflops": {}}
    iters, mblocks = 4000, 1024
    for kind, name, flops in ((0, "bf16", 16 * 16 * 32 * 2), (1, "fp8 16x16x32", 16 * 16 * 32 * 2),
                              (2, "fp8 16x16x128", 16 * 16 * 128 * 2), (3, "fp4 16x16x128", 16 * 16 * 128 * 2),
                              (4, "bf16 16x16x16", 16 * 16 * 16 * 2)):
        sec = timed(lambda: p.dsv4probe_mfma(kind, iters, ctypes.c_void_p(sink.data_ptr()), mblocks, st), 10)
        res["mfma_tflops"][name] = round(mblocks * 4 * iters * 8 * flops / sec / 1e12, 1)
    torch.cuda.synchronize()
    return res


def run_step(lib, calls, arm=None):
    """One step; arm maps a call index to the (start, stop) events of its main kernel."""
    for i, (fn, args) in enumerate(calls):
        if arm is not None and i in arm:
            lib.dsv4_time_next_kernel(*arm[i])
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{fn.__name__}: {lib.dsv4_last_error().decode()}")


def time_graph_replay(L, torch, wl, replicas, steps):
    """The decode step captured once per replica into a HIP graph (on a side stream, with
    the calls marshalled for that stream) and replayed with the replicas rotating: ms per
    step.  The outputs of the last replay of each replica are compared with an eager run
    of the same step (bitwise)."""
    lib = L.lib()
    s = torch.cuda.Stream()
    graphs, outs = [], []
    with torch.cuda.stream(s):
        marsh = [marshal_step(L, torch, wl, r)[0] for r in range(replicas)]
        for r in range(replicas):
            run_step(lib, marsh[r])
        torch.cuda.synchronize()
        for r in range(replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                run_step(lib, marsh[r])
            graphs.append(g)
    torch.cuda.synchronize()
    for r in range(replicas):                                  # eager reference outputs
        run_step(lib, marsh[r])
        torch.cuda.synchronize()
        t = wl.r[r]
        outs.append([t[k].clone() for k in ("idx", "o", "lse", "ho", "hlse")])
    with torch.cuda.stream(s):                                 # replays and events on one stream
        for i in range(3 * replicas):
            graphs[i % replicas].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            graphs[i % replicas].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        same = True
        for r in range(replicas):
            graphs[r].replay()
            torch.cuda.synchronize()
            t = wl.r[r]
            same = same and all(torch.equal(t[k], o) for k, o in zip(("idx", "o", "lse", "ho", "hlse"), outs[r]))
    del graphs
    return ms, same


# ------------------------------------------------------------------------------------ oracle leg
def cpu_baseline(L, torch, synth, wl, budget_s, threads=1):
    """The float64 oracle on `threads` host threads (None: all of them; NumPy's BLAS runs the
    indexer's products on them, the rest of the oracle is single-threaded NumPy): whole
    decode steps of the sequences of replica 0 (both layers), cycling over the 8 sequences
    until ~budget_s of timed work.  Inputs are generated and decoded beforehand (untimed);
    the library is not used.  Returns (steps, seconds, BLAS threads used)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import codecs, method

    t = wl.r[0]

    def bits(x):
        return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    seqs = []
    for b in range(B):
        k32 = synth.device_normal((1, N_CSA, DI), seed(CFG_CSA, synth.KI, 0, b), torch.float32)[0].cpu().numpy()
        packed, scales = codecs.encode_mxfp4(k32)                 # the stored MXFP4 cache
        del k32
        seqs.append(dict(
            packed=packed, scales=scales,
            q=codecs.decode_bf16(bits(t["q"][b:b + 1])), qi=codecs.decode_bf16(bits(t["qi"][b:b + 1])),
            wi=t["wi"][b:b + 1].cpu().numpy(),
            kw=codecs.decode_bf16(bits(t["kw"][b:b + 1])), vw=codecs.decode_bf16(bits(t["vw"][b:b + 1])),
            kiw=codecs.decode_bf16(bits(t["kiw"][b:b + 1])), gate=t["gate"][b:b + 1].cpu().numpy(),
            bias=t["bias"].cpu().numpy(), hq=codecs.decode_bf16(bits(t["hq"][b:b + 1])),
            hk=codecs.decode_bf16(bits(t["hkc"][b:b + 1])), hv=codecs.decode_bf16(bits(t["hvc"][b:b + 1])),
            hkw=codecs.decode_bf16(bits(t["hkw"][b:b + 1])), hvw=codecs.decode_bf16(bits(t["hvw"][b:b + 1])),
            hgate=t["hgate"][b:b + 1].cpu().numpy(), hbias=t["hbias"].cpu().numpy(),
            kc=wl.kc[b], vc=wl.vc[b]))

    done, elapsed = 0, 0.0
    scale = 1.0 / math.sqrt(D)
    pos = np.array([[CTX - 1]])
    with threadpool_limits(limits=threads):
        used = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
        while elapsed < budget_s:
            sq = seqs[done % B]
            t0 = time.perf_counter()
            # ---- CSA: compress the newest block (K, V, indexer key -> MXFP4)
            g4 = sq["gate"][:, LWIN - M_CSA:]
            new_k = method.compress(sq["kw"][:, LWIN - M_CSA:], g4, sq["bias"], M_CSA)
            new_v = method.compress(sq["vw"][:, LWIN - M_CSA:], g4, sq["bias"], M_CSA)
            new_ki = method.compress(sq["kiw"][:, LWIN - M_CSA:], g4, sq["bias"], M_CSA)
            p_new, s_new = codecs.encode_mxfp4(new_ki[0].astype(np.float32))
            packed, scales = sq["packed"].copy(), sq["scales"].copy()
            packed[-1], scales[-1] = p_new[0], s_new[0]
            ki = codecs.Stored(packed[None], codecs.MXFP4, scales[None])
            s = method.index_scores(sq["qi"], sq["wi"], ki, pos, M_CSA)
            idx = method.topk(s, pos, M_CSA, TOPK)
            sel = idx[0, 0][idx[0, 0] >= 0]
            t_gather = time.perf_counter()
            old = sel[sel < N_CSA - 1]
            kg = codecs.decode_bf16(bits(sq["kc"][torch.from_numpy(old).cuda()]))
            vg = codecs.decode_bf16(bits(sq["vc"][torch.from_numpy(old).cuda()]))
            t_gather = time.perf_counter() - t_gather               # device-to-host gather: not timed
            if len(old) < len(sel):
                kg = np.concatenate([kg, new_k[0]])
                vg = np.concatenate([vg, new_v[0]])
            n_sel = len(sel)
            method.csa_attend(sq["q"], kg[None], vg[None], np.arange(n_sel)[None, None], sq["kw"], sq["vw"],
                              np.array([CTX - LWIN]), W, pos, scale)
            # ---- HCA: compress the newest block, dense attention
            hk, hv = sq["hk"].copy(), sq["hv"].copy()
            hk[0, -1] = method.compress(sq["hkw"], sq["hgate"], sq["hbias"], M_HCA)[0, 0]
            hv[0, -1] = method.compress(sq["hvw"], sq["hgate"], sq["hbias"], M_HCA)[0, 0]
            method.hca_attend(sq["hq"], hk, hv, M_HCA, sq["hkw"], sq["hvw"], np.array([CTX - LWIN]), W, pos, scale)
            elapsed += time.perf_counter() - t0 - t_gather
            done += 1
    return done, elapsed, used


def source_sha(path):
    import hashlib

    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# ------------------------------------------------------------------------------------ prefill
PF_T, PF_P0, PF_K = 4096, 262144, 512           # chunk tokens, cached raw tokens, top-k
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}


def time_index_kernel(L, torch, call, n):
    """Average duration (ms) of the indexer kernel of csa_index_topk over n calls, from HIP
    events attached to that kernel's launch; call(lib, i) issues the i-th csa_index_topk."""
    lib = L.lib()
    ev = HipEvents()
    for i in range(3):
        call(lib, i)
    torch.cuda.synchronize()
    pairs = [(ev.create(), ev.create()) for _ in range(n)]
    for i, p in enumerate(pairs):
        lib.dsv4_time_next_kernel(*p)
        call(lib, i)
    torch.cuda.synchronize()
    return sum(ev.elapsed_ms(*p) for p in pairs) / n


def fp4_index_decode(L, torch, wl):
    """The decode workload's indexer (8 x 262,144 MXFP4 keys) with MXFP4 queries on the
    scaled FP4 MFMA and, timed the same way, with the step's bf16 queries: main-kernel
    microseconds of calls on their own, the replicas' keys rotating as in the step (one
    replica's 143 MB of keys repeated would be served from the 256 MB Infinity Cache)."""
    R = B * HI
    qs = []
    for t in wl.r:
        qbuf = torch.empty(R * DI // 2 + R * DI // 32, dtype=torch.uint8, device="cuda")
        qc, qsc = qbuf[:R * DI // 2].view(1, R, DI // 2), qbuf[R * DI // 2:].view(1, R, DI // 32)
        L.csa_compress(t["qi"].view(1, R, DI).float(), torch.zeros((1, R), device="cuda"),
                       torch.zeros(1, device="cuda"), 1, L.MXFP4_DTYPE, out=qc, out_scale=qsc)
        qs.append((qbuf, qc.view(B, 1, HI, DI // 2), qsc.view(B, 1, HI, DI // 32)))
    idx = torch.empty((B, 1, TOPK), dtype=torch.int32, device="cuda")
    ws = torch.empty(wl.r[0]["ws_idx"].numel(), dtype=torch.uint8, device="cuda")   # same shapes as the step's call

    def fp4(lib, i):
        t, (_, qc, qsc) = wl.r[i % len(wl.r)], qs[i % len(wl.r)]
        L.csa_index_topk(qc, t["wi"], t["ki"], wl.q_pos, M_CSA, TOPK, ki_scale=t["ks"], qi_scale=qsc, out_idx=idx,
                         workspace=ws)

    def bf16(lib, i):
        t = wl.r[i % len(wl.r)]
        L.csa_index_topk(t["qi"], t["wi"], t["ki"], wl.q_pos, M_CSA, TOPK, ki_scale=t["ks"], out_idx=idx,
                         workspace=ws)
    return time_index_kernel(L, torch, fp4, 30) * 1e3, time_index_kernel(L, torch, bf16, 30) * 1e3


def prefill_flops():
    """Algorithmic flops of one CSA layer's indexer (fp8) and attention (bf16), and of one
    HCA layer's attention (bf16), for a 4096-token chunk against a 256K-token cache:
    2*HI*DI per (query, visible block) and 4*H*D per (query, key in the attended set)."""
    pos = PF_P0 + np.arange(PF_T, dtype=np.int64)
    n_csa = np.minimum(PF_P0 // 4 + PF_T // 4, (pos + 1) // 4)
    n_hca = np.minimum(PF_P0 // 128 + PF_T // 128, (pos + 1) // 128)
    idx = 2.0 * HI * DI * float(n_csa.sum())
    csa = 4.0 * H * D * PF_T * (PF_K + W)
    hca = 4.0 * H * D * float((n_hca + W).sum())
    return idx, csa, hca


def run_prefill(L, torch, synth, steps, warmup):
    """Chunked prefill: a 4-layer stack (CSA, HCA, CSA, HCA, independent seeds) over one
    4096-token chunk against a 256K-token cache; each layer compresses the chunk into its
    caches and attends (CSA: fp8 indexer + top-512 + window; HCA: dense + window)."""
    lib = L.lib()
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    T, P0 = PF_T, PF_P0
    Lw = W + T
    qpos = (P0 + torch.arange(T, dtype=torch.int32, device="cuda")).reshape(1, T)
    wpos0 = torch.tensor([P0 - W], dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    layers = []
    for li, kind in enumerate(("csa", "hca", "csa", "hca")):
        sd = lambda tid: seed(5 if kind == "csa" else 6, tid, li)
        t = {"kind": kind}
        m = M_CSA if kind == "csa" else M_HCA
        n0 = P0 // m
        n = n0 + T // m
        t["kc"] = synth.device_normal((1, n, D), sd(synth.KC), bf)
        t["vc"] = synth.device_normal((1, n, D), sd(synth.VC), bf)
        t["kw"] = synth.device_normal((1, Lw, D), sd(synth.KW), bf)       # window: 128 cached + chunk
        t["vw"] = synth.device_normal((1, Lw, D), sd(synth.VW), bf)
        t["gate"] = synth.device_normal((1, T), sd(synth.GATE), torch.float32)
        t["bias"] = synth.device_normal((m,), sd(synth.BIAS), torch.float32, std=0.1)
        t["q"] = synth.device_normal((1, T, H, D), sd(synth.Q), bf)
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((1, T, H), dtype=torch.float32, device="cuda")
        t["n0"], t["m"] = n0, m
        if kind == "csa":
            t["ki"] = synth.device_normal((1, n, DI), sd(synth.KI), f8)
            t["kiw"] = synth.device_normal((1, T, DI), sd(synth.RAW_KI), bf)
            t["qi"] = synth.device_normal((1, T, HI, DI), sd(synth.QI), f8)
            t["wi"] = synth.device_uniform((1, T, HI), sd(synth.WI))
            t["idx"] = torch.empty((1, T, PF_K), dtype=torch.int32, device="cuda")
        layers.append(t)
    torch.cuda.synchronize()
    ws = {}

    def layer(t, arm=None):
        m, n0 = t["m"], t["n0"]
        kwc, vwc = t["kw"][:, W:], t["vw"][:, W:]                      # the chunk's raw rows
        L.csa_compress(kwc, t["gate"], t["bias"], m, bf, out=t["kc"][:, n0:])
        L.csa_compress(vwc, t["gate"], t["bias"], m, bf, out=t["vc"][:, n0:])
        if t["kind"] == "csa":
            L.csa_compress(t["kiw"], t["gate"], t["bias"], m, f8, out=t["ki"][:, n0:])
            if arm:
                lib.dsv4_time_next_kernel(*arm[0])
            L.csa_index_topk(t["qi"], t["wi"], t["ki"], qpos, m, PF_K, out_idx=t["idx"],
                             workspace=ws.setdefault("idx", None))
            if arm:
                lib.dsv4_time_next_kernel(*arm[1])
            L.csa_attend(t["q"], t["kc"], t["vc"], t["idx"], t["kw"], t["vw"], wpos0, W, qpos, scale,
                         out=t["o"], lse=t["lse"])
        else:
            if arm:
                lib.dsv4_time_next_kernel(*arm[2])
            L.hca_attend(t["q"], t["kc"], t["vc"], m, t["kw"], t["vw"], wpos0, W, qpos, scale, out=t["o"],
                         lse=t["lse"])

    ev = HipEvents()
    for _ in range(warmup):
        for t in layers:
            layer(t)
    torch.cuda.synchronize()
    pairs = [[(ev.create(), ev.create()) for _ in range(3)] for _ in range(steps * 4)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        for j, t in enumerate(layers):
            layer(t, pairs[4 * i + j])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    f_idx, f_csa, f_hca = prefill_flops()
    k_idx = sum(ev.elapsed_ms(*pairs[4 * i + j][0]) for i in range(steps) for j in (0, 2)) / (2 * steps)
    k_csa = sum(ev.elapsed_ms(*pairs[4 * i + j][1]) for i in range(steps) for j in (0, 2)) / (2 * steps)
    k_hca = sum(ev.elapsed_ms(*pairs[4 * i + j][2]) for i in range(steps) for j in (1, 3)) / (2 * steps)
    ideal_ms = 2 * (f_idx / PEAK_TFLOPS["fp8"] + f_csa / PEAK_TFLOPS["bf16"] + f_hca / PEAK_TFLOPS["bf16"]) / 1e9
    kern = lambda f, kms, pk: {"avg_launch_ms": round(kms, 4), "tflops": round(f / kms / 1e9, 1),
                               "frac_of_peak": round(f / kms / 1e9 / PEAK_TFLOPS[pk], 4), "flops": f}
    # the CSA indexer again with MXFP4 queries and keys (scaled FP4 MFMA), same shapes
    t0 = layers[0]
    n = t0["ki"].shape[1]
    k4 = torch.empty((1, n, DI // 2), dtype=torch.uint8, device="cuda")
    k4s = torch.empty((1, n, DI // 32), dtype=torch.uint8, device="cuda")
    L.csa_compress(synth.device_normal((1, n, DI), seed(7, synth.KI, 0), bf), torch.zeros((1, n), device="cuda"),
                   torch.zeros(1, device="cuda"), 1, L.MXFP4_DTYPE, out=k4, out_scale=k4s)
    R = T * HI
    qbuf = torch.empty(R * DI // 2 + R * DI // 32, dtype=torch.uint8, device="cuda")
    qc, qs = qbuf[:R * DI // 2].view(1, R, DI // 2), qbuf[R * DI // 2:].view(1, R, DI // 32)
    L.csa_compress(synth.device_normal((1, R, DI), seed(7, synth.QI, 0), bf), torch.zeros((1, R), device="cuda"),
                   torch.zeros(1, device="cuda"), 1, L.MXFP4_DTYPE, out=qc, out_scale=qs)

    def fp4_call(lib_, i=0):
        L.csa_index_topk(qc.view(1, T, HI, DI // 2), t0["wi"], k4, qpos, M_CSA, PF_K, ki_scale=k4s,
                         qi_scale=qs.view(1, T, HI, DI // 32), out_idx=t0["idx"], workspace=ws.get("idx"))
    k_fp4 = time_index_kernel(L, torch, fp4_call, max(2, steps))
    ceil = measured_ceilings(torch)
    extra = {}
    if ceil is not None:
        mt = ceil["mfma_tflops"]
        # the stack at the measured MFMA rates of the instructions it uses (the indexer's fp8
        # keys on the scaled 16x16x128 form, attention on bf16 16x16x32 / 16x16x16)
        ideal_meas = 2 * (f_idx / mt["fp8 16x16x128"] + (f_csa + f_hca) / mt["bf16"]) / 1e9
        extra["measured_ceilings"] = {"mfma_tflops": mt, "ideal_ms_at_measured": round(ideal_meas, 4),
                                      "value_vs_measured": round(ideal_meas / ms, 4),
                                      "note": "back-to-back MFMAs on this GPU; context only, value uses the "
                                              "published peaks"}
    return {
        "metric": "chunked prefill MFMA utilisation (4-layer CSA/HCA stack, 4096-token chunk, 256K cache)",
        "value": round(ideal_ms / ms, 4), "unit": "fraction of dense MFMA peak", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+fp8", "data": "synthetic (seeded N(0,1) / U(0,1))",
        "config": {"workload": "chunked prefill: CSA, HCA, CSA, HCA layers; 4096 queries at positions "
                               "262144..266239; 64 heads x 512; fp8 indexer 8 x 128, top-512; window 128",
                   "chunk": T, "cache_tokens": P0},
        "ideal_ms_at_peak": round(ideal_ms, 4),
        "kernels": {"index_mfma_kernel (fp8)": kern(f_idx, k_idx, "fp8"),
                    "attend_bf16_kernel (CSA)": kern(f_csa, k_csa, "bf16"),
                    "attend_bf16_kernel (HCA)": kern(f_hca, k_hca, "bf16")},
        "fp4_indexer": dict(kern(f_idx, k_fp4, "fp4"), note="the CSA layer's indexer with MXFP4 queries and keys "
                            "on the scaled FP4 MFMA (outside the stack timing)"),
        **extra,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--time-every", type=int, default=10,
                    help="per-kernel event timing on every n-th timed step (event-timed launches cost "
                         "a few microseconds each, so timing every step would slow the step itself)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule", action="store_true", help="skip the 61-layer schedule timing")
    ap.add_argument("--no-fp8-kv", action="store_true", help="skip the step with FP8 K|V caches")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the chunked-prefill stack instead of decode (prints its own line)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill sub-object of the decode line")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing of the step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this size after warm-up (reference for traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: the path runs on a single MI355X and multi-GPU "
                         "sharding is not implemented. Use --gpus 1.\n")
        sys.exit(2)

    import torch

    import long_context_attention_25_amd as L
    import synth

    lib = L.lib()
    torch.cuda.set_device(0)
    if args.prefill:
        print(json.dumps(run_prefill(L, torch, synth, max(1, args.steps // 10), max(1, args.warmup // 5))), flush=True)
        return
    wl = Workload(L, torch, synth, args.replicas)
    steps = [marshal_step(L, torch, wl, r) for r in range(args.replicas)]
    timed = steps[0][1]
    ev = HipEvents()
    every = max(1, args.time_every)
    pairs = [{i: (ev.create(), ev.create()) for i in timed} for _ in range((args.steps + every - 1) // every)]

    for i in range(args.warmup):
        run_step(lib, steps[i % args.replicas][0])
    torch.cuda.synchronize()
    if args.copy_calibration_mib:
        # a plain device copy of known size: the reference reading for the traffic counters
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run_step(lib, steps[i % args.replicas][0], arm=pairs[i // every] if i % every == 0 else None)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    total_bytes, parts = algorithmic_bytes()
    qps = B / (ms / 1e3)
    kernels = {}
    for i, name in timed.items():
        k_ms = sum(ev.elapsed_ms(*p[i]) for p in pairs) / len(pairs)
        gbs = KERNEL_BYTES[name] / (k_ms / 1e3) / 1e9
        kernels[name] = {"avg_launch_us": round(k_ms * 1e3, 2), "bytes_per_launch": KERNEL_BYTES[name],
                         "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(kernels, key=lambda n: kernels[n]["avg_launch_us"])
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_attention_25_amd", "csrc",
                       "index_topk.hip" if dom.startswith("index") else "attend.hip")
    tr = MEASURED_TRAFFIC.get(dom)
    traffic = tr["bytes_per_launch"] if tr and tr["source_sha256"] == source_sha(src) else None
    k = kernels[dom]
    out = {
        "metric": "CSA+HCA decode queries/s at 1M ctx + achieved HBM GB/s vs peak",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) / U(0,1); MXFP4 indexer keys, bf16 KV)",
        "config": {"workload": "CSA decode (MXFP4 indexer, top-1024 of 262144 + 128 window) + HCA decode "
                               "(8192 entries at 128x + 128 window) at 1M context, new block compressed each step",
                   "batch": B, "context": CTX, "heads": H, "head_dim": D, "csa_entries": N_CSA,
                   "hca_entries": N_HCA, "topk": TOPK, "window": W, "indexer_heads": HI, "indexer_dim": DI,
                   "replicas": args.replicas},
        "step_hbm_gbs": round(total_bytes / (ms / 1e3) / 1e9, 1),
        "step_hbm_frac": round(total_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_step": total_bytes,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": k["achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": k["frac"], "traffic": traffic,
                     "bytes_per_launch": k["bytes_per_launch"], "avg_launch_us": k["avg_launch_us"],
                     "timed_launches": len(pairs)},
        "kernels": kernels,
    }
    if not args.no_graph:
        g_ms, g_same = time_graph_replay(L, torch, wl, args.replicas, max(20, args.steps // 2))
        out["graph_replay"] = {"ms_per_step": round(g_ms, 5), "eager_ms_per_step": round(ms, 5),
                               "queries_per_s": round(B / (g_ms / 1e3), 1), "outputs_equal_eager": g_same,
                               "note": "the same step captured once per replica into a HIP graph and replayed "
                                       "(replicas rotating); value stays the eager rate"}
    us_fp4, us_bf16 = fp4_index_decode(L, torch, wl)
    out["fp4_indexer"] = {"avg_launch_us": round(us_fp4, 2), "bf16_query_avg_launch_us": round(us_bf16, 2),
                          "note": "the same 8 x 262144 MXFP4 keys with MXFP4 queries (scaled FP4 MFMA) and, timed "
                                  "alike, with bf16 queries: csa_index_topk calls on their own after the timed steps, "
                                  "main kernel only, keys of the three replicas rotating"}
    if not args.no_fp8_kv:
        out["fp8_kv"] = run_fp8_kv(L, torch, wl, args.steps, args.warmup, every)
    out["cache_append"] = {"us_per_step": round(time_cache_append(L, torch, wl, 50), 2), "calls_per_step": 3,
                           "note": "kv_cache_append for CSA K|V, CSA indexer key (MXFP4) and HCA K|V, each new "
                                   "token completing a block (worst case); measured after the timed steps"}
    if not args.no_schedule:
        us_tok, per_layer = time_schedule(L, torch, [c for c, _ in steps], 5)
        kvb = kv_bytes_per_token()
        counts = {k: SCHEDULE.count(k) for k in ("csa", "hca", "swa")}
        out["schedule_61"] = {
            "layers": counts, "us_per_token_step": round(us_tok, 1), "queries_per_s": round(B / (us_tok / 1e6), 1),
            "per_layer_us": per_layer,
            "kv_bytes_per_token": round(sum(counts[k] * kvb[k] for k in counts), 1),
            "note": "layers 0-1 HCA, 2-60 alternating CSA/HCA, MTP block window-only; each layer is one decode "
                    "step of this workload (new block pooled every step); caches rotate over the replicas"}
    ceil = measured_ceilings(torch)
    if ceil is not None:
        out["measured_ceilings"] = dict(ceil, roofline_frac_of_read=round(k["achieved_gbs"] / ceil["hbm_read_gbs"], 4),
                                        note="2 GiB streaming read (non-temporal loads) and back-to-back MFMAs on "
                                             "this GPU; context only, the roofline uses the published peaks")
    if not args.no_prefill:
        pf = run_prefill(L, torch, synth, max(1, args.steps // 10), max(1, args.warmup // 5))
        out["prefill"] = {k: pf[k] for k in ("metric", "value", "unit", "ms_per_step", "ideal_ms_at_peak", "kernels",
                                              "fp4_indexer", "config") if k in pf}
    if not args.no_cpu_baseline:
        done, el, used = cpu_baseline(L, torch, synth, wl, args.cpu_seconds, threads=None)
        done1, el1, _ = cpu_baseline(L, torch, synth, wl, args.cpu_seconds, threads=1)
        sample = (f"decode steps of single sequences (both layers; cycling over the {B} sequences of replica 0), "
                  f"float64 NumPy oracle")
        out["cpu_baseline"] = {"value": round(done / el, 3), "unit": "queries/s", "cores": used, "kind": "oracle",
                               "host_cpus": os.cpu_count(),
                               "sample": f"{done} {sample}, {el:.1f} s, BLAS on {used} threads"}
        out["cpu_baseline_1_thread"] = {"value": round(done1 / el1, 3), "unit": "queries/s", "cores": 1,
                                        "kind": "oracle", "sample": f"{done1} {sample}, {el1:.1f} s on 1 thread"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module holds no arithmetic of the attention method: it only draws
random numbers and hands them over in the storage dtypes the method reads
(float32, or bfloat16 via torch's own round-to-nearest-even cast).  The
quantised forms (fp8 e4m3, MXFP4) are *not* produced here: each side (the
HIP library and the oracle) quantises the float32 draws with its own code.

Seeding: every tensor of a workload gets its own counter-based stream,
``numpy.random.Generator(Philox(key=1000*config + tensor_id))`` on the host,
or a ``torch.Generator`` seeded with the same number when the tensor is too
large to draw on the host and is drawn on the device instead.
"""
from __future__ import annotations

import numpy as np

# tensor ids (fixed so that a tensor's stream never depends on call order)
Q, KC, VC, KW, VW, QI, WI, KI, GATE, BIAS, RAW_K, RAW_V, RAW_KI, IDX = range(14)


def rng(config: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=1000 * int(config) + int(tensor_id)))


def normal(config: int, tensor_id: int, shape, std: float = 1.0) -> np.ndarray:
    g = rng(config, tensor_id)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def uniform(config: int, tensor_id: int, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    g = rng(config, tensor_id)
    return (g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def sorted_unique_indices(config: int, tensor_id: int, rows: int, n: int, k: int) -> np.ndarray:
    """rows x k int32: k distinct values from [0, n), ascending; -1 padding when k > n."""
    g = rng(config, tensor_id)
    out = np.full((rows, k), -1, dtype=np.int32)
    take = min(k, n)
    for r in range(rows):
        out[r, :take] = np.sort(g.choice(n, size=take, replace=False)).astype(np.int32)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 draws as bfloat16 (torch's RNE cast); returns the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def device_normal(shape, seed: int, dtype, device="cuda", std: float = 1.0):
    """Large draws made on the device with a seeded torch generator (too big for the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def device_uniform(shape, seed: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)

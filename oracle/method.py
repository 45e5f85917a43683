"""The CSA / HCA attention path in float64, step by step, as the pages describe it.

Page citations use the page address and the section title on that page:

[CSA]  honbul.tistory.com/221 §"CSA: 압축한 뒤, 필요한 기억만 골라서 보기" — several
       tokens are bundled into one compressed KV entry; a small indexer picks the
       compressed entries most relevant to the current token; only those go into
       attention; recent tokens are kept by a separate sliding window, and the
       compressed long-range memory and the recent raw memory are used together.
[HCA]  honbul.tistory.com/221 §"HCA: 더 강하게 압축하고, 압축된 전체를 보기" — a
       stronger compression, no sparse selection, attention over every compressed
       entry.
[KVC]  honbul.tistory.com/221 §"KV cache를 줄이는 방식" — separate caches for the
       compressed entries, the sliding window, and the tail tokens not yet enough
       to compress.
[P2§4] pogovet.com, 상세 정리 §4 — CSA compresses KV 4x along the sequence by
       softmax-gated pooling with a learned positional bias; an FP4 lightning
       indexer picks the top-k compressed blocks per query; a sliding-window
       branch handles recent tokens; HCA compresses 128x and attends densely.

Readings of what the prose leaves open (each one is listed with its reason in the
design notes of the repository):
  * one scalar gate logit per raw token, one learned bias scalar per slot of a block;
  * blocks are disjoint, stride m, aligned to position 0; a block is visible to a
    query at position p once it is complete: j < floor((p+1)/m);
  * indexer score s_j = sum_h w_h * max(0, q_h . k_j) over visible j only;
  * top-k: larger score first, equal scores -> lower index; output ascending, -1 pad;
  * the selected compressed entries and the window rows (positions in (p-W, p])
    share ONE softmax; a recent token may appear both compressed and raw;
  * empty key set -> o = 0, lse = -inf; lse is the natural log and includes scale.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_mxfp4, encode_mxfp4, rows


# --------------------------------------------------------------------------- compression
def compress(x: np.ndarray, gate: np.ndarray, pos_bias: np.ndarray, m: int) -> np.ndarray:
    """Softmax-gated pooling of disjoint blocks of m raw tokens  [CSA], [HCA], [P2§4].

    x [B,T,C], gate [B,T] (one logit per raw token), pos_bias [m] (one per slot).
    y[b,i,:] = sum_j a_j x[b,i*m+j,:],  a = softmax_j(gate[b,i*m+j] + pos_bias[j]).
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    assert T % m == 0
    nb = T // m
    z = np.asarray(gate, dtype=np.float64).reshape(B, nb, m) + np.asarray(pos_bias, np.float64)[None, None, :]
    z = z - z.max(axis=2, keepdims=True)
    e = np.exp(z)
    a = e / e.sum(axis=2, keepdims=True)
    return np.einsum("bim,bimc->bic", a, x.reshape(B, nb, m, C))


# --------------------------------------------------------------------------- indexer
def visible_blocks(q_pos, m: int, N: int):
    """Number of complete compressed blocks at or before position p: min(N, floor((p+1)/m))."""
    return np.minimum(N, (np.asarray(q_pos, dtype=np.int64) + 1) // m)


def index_scores(qi, wi, ki, q_pos, m: int) -> np.ndarray:
    """Lightning-indexer scores for every (query, compressed block)  [CSA], [P2§4].

    qi [B,Q,HI,DI], wi [B,Q,HI], ki [B,N,DI] (array or codecs.Stored), q_pos [B,Q].
    s[b,q,j] = sum_h wi[b,q,h] * relu(qi[b,q,h,:] . ki[b,j,:]) for j < n(q_pos), else -inf.
    """
    qi = np.asarray(qi, dtype=np.float64)
    wi = np.asarray(wi, dtype=np.float64)
    B, Q, HI, DI = qi.shape
    N = ki.shape[1]
    n_vis = visible_blocks(q_pos, m, N)
    s = np.full((B, Q, N), -np.inf)
    for b in range(B):
        nmax = int(n_vis[b].max()) if Q else 0
        if nmax == 0:
            continue
        kb = rows(ki, b, slice(0, nmax))                    # [n, DI]
        for q in range(Q):
            n = int(n_vis[b, q])
            dots = qi[b, q] @ kb[:n].T                       # [HI, n]
            s[b, q, :n] = wi[b, q] @ np.maximum(dots, 0.0)
    return s


def index_scores_fp4(qi32, wi, ki, q_pos, m: int):
    """Indexer scores with FP4 queries as well as FP4 keys  [P2§4] (FP4 lightning indexer),
    [P2§5]: the queries go through the MXFP4 quantiser (codecs.encode_mxfp4, per 32-element
    group of each head row) and the scores are then those of index_scores on the decoded
    values.  Returns (scores, query codes, query scales): the codes and scales are the
    bytes the quantised queries are stored as.
    """
    codes, scales = encode_mxfp4(np.asarray(qi32, dtype=np.float32))
    return index_scores(decode_mxfp4(codes, scales), wi, ki, q_pos, m), codes, scales


def topk(s: np.ndarray, q_pos, m: int, k: int) -> np.ndarray:
    """Top-k compressed blocks per query  [CSA] (Top-k Selector), [P2§4].

    Among the visible blocks, larger score first and equal scores to the lower index;
    the selected indices are returned in ascending order, padded with -1.
    """
    B, Q, N = s.shape
    n_vis = visible_blocks(q_pos, m, N)
    out = np.full((B, Q, k), -1, dtype=np.int32)
    for b in range(B):
        for q in range(Q):
            n = int(n_vis[b, q])
            take = min(k, n)
            if take == 0:
                continue
            order = np.argsort(-s[b, q, :n], kind="stable")  # stable: ties keep index order
            out[b, q, :take] = np.sort(order[:take])
    return out


# --------------------------------------------------------------------------- attention
def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of H query heads over an explicit key list (MQA: K, V shared).

    q [H,D], K/V [n,D] -> o [H,D], lse [H] with lse = log sum_j exp(scale * q.k_j).
    """
    H, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    z = scale * (q @ K.T)
    mx = z.max(axis=1, keepdims=True)
    e = np.exp(z - mx)
    ssum = e.sum(axis=1, keepdims=True)
    return (e @ V) / ssum, (mx + np.log(ssum))[:, 0]


def window_rows(p: int, win_pos0: int, L: int, W: int) -> np.ndarray:
    """Rows r of the window buffer (row r holds position win_pos0 + r) with p-W < pos <= p."""
    lo = max(0, p - W + 1 - win_pos0)
    hi = min(L, p + 1 - win_pos0)
    return np.arange(lo, hi) if hi > lo else np.arange(0)


def csa_attend(q, kc, vc, idx, kw, vw, win_pos0, W: int, q_pos, scale: float):
    """CSA attention: one softmax over the selected compressed entries and the window
    rows  [CSA], [P2§4].  idx entries outside [0, N) are skipped.

    q [B,Q,H,D]; kc/vc [B,N,D]; idx [B,Q,k]; kw/vw [B,L,D]; win_pos0 [B]; q_pos [B,Q].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Q, H, D = q.shape
    N = kc.shape[1]
    L = kw.shape[1]
    o = np.zeros((B, Q, H, D))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        for t in range(Q):
            sel = np.asarray(idx[b, t], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel < N)]
            wr = window_rows(int(q_pos[b, t]), int(win_pos0[b]), L, W)
            K = np.concatenate([rows(kc, b, sel), rows(kw, b, wr)], axis=0)
            V = np.concatenate([rows(vc, b, sel), rows(vw, b, wr)], axis=0)
            o[b, t], lse[b, t] = attend_rows(q[b, t], K, V, scale)
    return o, lse


def hca_attend(q, kc, vc, m: int, kw, vw, win_pos0, W: int, q_pos, scale: float):
    """HCA attention: one softmax over every visible compressed entry and the window
    rows  [HCA], [P2§4]."""
    q = np.asarray(q, dtype=np.float64)
    B, Q, H, D = q.shape
    N = kc.shape[1]
    n_vis = visible_blocks(q_pos, m, N)
    idx = np.full((B, Q, max(1, int(n_vis.max()) if n_vis.size else 1)), -1, dtype=np.int64)
    for b in range(B):
        for t in range(Q):
            idx[b, t, : n_vis[b, t]] = np.arange(n_vis[b, t])
    return csa_attend(q, kc, vc, idx, kw, vw, win_pos0, W, q_pos, scale)


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge attention results over disjoint key sets by their log-sum-exp.

    o_parts [P,R,D], lse_parts [P,R] -> o [R,D], lse [R].  A part with lse = -inf is
    empty; if every part is empty the result is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_parts - safe[None, :])                  # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.einsum("pr,prd->rd", w, o_parts) / tot[:, None]
        lse = safe + np.log(tot)
    empty = ~np.isfinite(M)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


# --------------------------------------------------------------------------- whole decode step
def csa_decode(q, kc, vc, qi, wi, ki, kw, vw, win_pos0, W, q_pos, m, k, scale):
    """Index, select and attend for CSA: returns (o, lse, idx, scores)."""
    s = index_scores(qi, wi, ki, q_pos, m)
    idx = topk(s, q_pos, m, k)
    o, lse = csa_attend(q, kc, vc, idx, kw, vw, win_pos0, W, q_pos, scale)
    return o, lse, idx, s

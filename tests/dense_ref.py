"""Dense n x n references used to pin the oracle (numpy, float64).

These restate SER and SEA as textbook dense linear algebra, independently of
the oracle's sparse loops:

* SER (page "Graph Machine: Towards Better Pretraining via Edges", ai.info,
  Key Contributions 2-3): the edges of a row are the non-zeros of a soft
  sparse adjacency matrix, and referral is the matrix product A1 A2 followed
  by keeping the s1 largest entries of each row.
* SEA (same page, Key Contributions 3 and Methodology): causal attention whose
  logits are scale * Q K^T plus the log of the (summed) edge weight, with
  -inf where a row has no edge to a column.
"""
from __future__ import annotations

import numpy as np


def adjacency(idx, w, b, h, n):
    """Dense A[i, j] = sum of the weights of row i's slots pointing at j."""
    A = np.zeros((n, n), np.float64)
    rows = np.repeat(np.arange(n), idx.shape[-1])
    np.add.at(A, (rows, idx[b, :, h, :].reshape(-1).astype(np.int64)),
              w[b, :, h, :].reshape(-1).astype(np.float64))
    return A


def ser_forward(idx1, w1, idx2, w2, s1):
    """Top-s1 of each row of A1 A2 over its positive fp32-rounded entries.

    Returns (idx, w, kth, next): ``kth``/``next`` are the s1-th and (s1+1)-th
    largest keys of each row (0 when absent), for the near-tie rule.
    """
    B, n, hkv, _ = idx1.shape
    io = np.zeros((B, n, hkv, s1), np.int32)
    wo = np.zeros((B, n, hkv, s1), np.float32)
    kth = np.zeros((B, n, hkv), np.float64)
    nxt = np.zeros((B, n, hkv), np.float64)
    for b in range(B):
        for h in range(hkv):
            C = adjacency(idx1, w1, b, h, n) @ adjacency(idx2, w2, b, h, n)
            key = C.astype(np.float32)
            for i in range(n):
                cols = np.nonzero(key[i] > 0)[0]
                order = cols[np.lexsort((cols, -key[i, cols].astype(np.float64)))]
                keep = order[:s1]
                io[b, i, h, :len(keep)] = keep
                wo[b, i, h, :len(keep)] = key[i, keep]
                if len(order) >= s1:
                    kth[b, i, h] = key[i, order[s1 - 1]]
                if len(order) > s1:
                    nxt[b, i, h] = key[i, order[s1]]
    return io, wo, kth, nxt


def ser_backward(idx1, w1, idx2, w2, idx_out, w_out, dw_out):
    """dA1 = (M o dW') A2^T and dA2 = A1^T (M o dW'), read at the slots.

    M is the mask of retained entries of A' (positive slots); zero-weight
    input slots are padding and read 0.
    """
    B, n, hkv, s2 = idx1.shape
    dw1 = np.zeros(idx1.shape, np.float64)
    dw2 = np.zeros(idx2.shape, np.float64)
    for b in range(B):
        for h in range(hkv):
            A1 = adjacency(idx1, w1, b, h, n)
            A2 = adjacency(idx2, w2, b, h, n)
            G = adjacency(idx_out, np.where(w_out > 0, dw_out, 0.0), b, h, n)
            dA1 = G @ A2.T
            dA2 = A1.T @ G
            for i in range(n):
                for a in range(s2):
                    if w1[b, i, h, a] > 0:
                        dw1[b, i, h, a] = dA1[i, idx1[b, i, h, a]]
                for c in range(idx2.shape[-1]):
                    if w2[b, i, h, c] > 0:
                        dw2[b, i, h, c] = dA2[i, idx2[b, i, h, c]]
    return dw1, dw2


def sea_probs(q, k, idx, w, scale=None):
    """Dense attention probabilities P [B, hq, n, n] of the masked causal
    attention with bias ln W (rows with no live edge are 0)."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    P = np.zeros((B, hq, n, n))
    for b in range(B):
        for h in range(hkv):
            W = adjacency(idx, np.where(w > 0, w, 0.0), b, h, n)
            with np.errstate(divide="ignore"):
                bias = np.where(W > 0, np.log(np.where(W > 0, W, 1.0)), -np.inf)
            for g in range(G):
                S = scale * q[b, :, h * G + g, :] @ k[b, :, h, :].T + bias
                mx = S.max(axis=1, keepdims=True)
                alive = np.isfinite(mx)
                E = np.where(alive, np.exp(S - np.where(alive, mx, 0.0)), 0.0)
                Z = E.sum(axis=1, keepdims=True)
                P[b, h * G + g] = np.where(Z > 0, E / np.where(Z > 0, Z, 1.0), 0.0)
    return P


def sea(q, k, v, idx, w, dout=None, scale=None):
    """Dense masked attention with additive bias ln W; optional backward.

    Returns o, or (o, dq, dk, dv, dw) when ``dout`` is given; dw is dS/W
    summed over the query heads of the group, read at each live slot.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.zeros_like(q)
    if dout is not None:
        dout = np.asarray(dout, np.float64)
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        dw = np.zeros(idx.shape, np.float64)
    for b in range(B):
        for h in range(hkv):
            W = adjacency(idx, np.where(w > 0, w, 0.0), b, h, n)
            with np.errstate(divide="ignore"):
                bias = np.where(W > 0, np.log(np.where(W > 0, W, 1.0)), -np.inf)
            K = k[b, :, h, :]; V = v[b, :, h, :]
            dW = np.zeros((n, n))
            for g in range(G):
                hh = h * G + g
                S = scale * q[b, :, hh, :] @ K.T + bias
                mx = S.max(axis=1, keepdims=True)
                alive = np.isfinite(mx)
                E = np.where(alive, np.exp(S - np.where(alive, mx, 0.0)), 0.0)
                Z = E.sum(axis=1, keepdims=True)
                P = np.where(Z > 0, E / np.where(Z > 0, Z, 1.0), 0.0)
                o[b, :, hh, :] = P @ V
                if dout is not None:
                    dO = dout[b, :, hh, :]
                    dP = dO @ V.T
                    dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
                    dq[b, :, hh, :] = scale * dS @ K
                    dk[b, :, h, :] += scale * dS.T @ q[b, :, hh, :]
                    dv[b, :, h, :] += P.T @ dO
                    dW += np.where(W > 0, dS / np.where(W > 0, W, 1.0), 0.0)
            if dout is not None:
                for i in range(n):
                    for t in range(idx.shape[-1]):
                        if w[b, i, h, t] > 0:
                            dw[b, i, h, t] = dW[i, idx[b, i, h, t]]
    if dout is None:
        return o
    return o, dq, dk, dv, dw


def leg_mix(idx, w, alpha, s):
    """Leg construction as dense rows: L[i] = sum_k alpha[h, k] w[i, k]
    e_{idx[i, k]}; top-s of each row over its positive fp32-rounded entries.
    Returns (idx, w, kth, next) like ser_forward."""
    B, n, hkv, K = idx.shape
    io = np.zeros((B, n, hkv, s), np.int32)
    wo = np.zeros((B, n, hkv, s), np.float32)
    kth = np.zeros((B, n, hkv), np.float64)
    nxt = np.zeros((B, n, hkv), np.float64)
    for b in range(B):
        for h in range(hkv):
            mixed = w[b, :, h, :].astype(np.float64) * np.asarray(alpha, np.float64)[h][None, :]
            L = np.zeros((n, n), np.float64)
            rows = np.repeat(np.arange(n), K)
            np.add.at(L, (rows, idx[b, :, h, :].reshape(-1).astype(np.int64)), mixed.reshape(-1))
            key = L.astype(np.float32)
            for i in range(n):
                cols = np.nonzero(key[i] > 0)[0]
                order = cols[np.lexsort((cols, -key[i, cols].astype(np.float64)))]
                keep = order[:s]
                io[b, i, h, :len(keep)] = keep
                wo[b, i, h, :len(keep)] = key[i, keep]
                if len(order) >= s:
                    kth[b, i, h] = key[i, order[s - 1]]
                if len(order) > s:
                    nxt[b, i, h] = key[i, order[s]]
    return io, wo, kth, nxt


def leg_mix_backward(idx, w, alpha, idx_out, w_out, dleg):
    """Through the dense mixture: dL = M o dLeg (retained entries); then
    dw[i, k] = alpha[h, k] dL[i, idx[i, k]] and dalpha[h, k] = sum_i w[i, k]
    dL[i, idx[i, k]], over slots with alpha > 0 and w > 0."""
    B, n, hkv, K = idx.shape
    alpha = np.asarray(alpha, np.float64)
    dw = np.zeros(idx.shape, np.float64)
    da = np.zeros((hkv, K), np.float64)
    for b in range(B):
        for h in range(hkv):
            G = adjacency(idx_out, np.where(w_out > 0, dleg, 0.0), b, h, n)
            for i in range(n):
                for k in range(K):
                    if w[b, i, h, k] > 0 and alpha[h, k] > 0:
                        g = G[i, idx[b, i, h, k]]
                        dw[b, i, h, k] = alpha[h, k] * g
                        da[h, k] += w[b, i, h, k] * g
    return dw, da

"""fp64 reference for jagged exact softmax attention (test infrastructure only).

What is computed (per sequence b and head h, with local indices i for queries
and j for keys/values):

  S_ij = Q_i . K_j / sqrt(D) + beta[h, clip(i - j, -R, R) + R]      (bias optional)
  causal: key j is visible to query i iff j <= i (top-left alignment)
  P_ij = softmax_j(S_ij),  O_i = sum_j P_ij V_j,  lse_i = log sum_j exp(S_ij)
  no keys (Lk = 0): O_i = 0, lse_i = -inf

Sources:
  * exact attention as score matrix -> row softmax -> weighted sum of values,
    computed without padding over variable-length sequences:
    "TLX-Optimized Jagged Flash Attention: Approaching FA4-Level Performance on
    Blackwell", section "Why Jagged Flash Attention Deserves Attention";
    "Jagged Flash Attention (JFA)" (sysdesign-wiki), section "Definition".
  * custom attention biases and asymmetric query / key-value lengths: same
    "Definition" section. The pages give no form for the bias; the relative
    position table beta[h, clip(i-j)] is the reading used here.
  * backward passes: "Jagged Flash Attention (JFA)", "Four generations" item 2.
    The pages state no gradient formulas; the ones below are the matrix
    calculus of the definition above:
      dV = P^T dO;  dP = dO V^T;  Delta_i = sum_d dO_id O_id = sum_j P_ij dP_ij
      dS = P * (dP - Delta);  dQ = dS K / sqrt(D);  dK = dS^T Q / sqrt(D)
    and, as beta[h, r] is added to every score with clip(i - j) + R = r,
      dbeta[h, r] = sum over b and visible (i, j) of that bin of dS_ij

This is the plain definition evaluated sequence by sequence in fp64, with the
query rows cut into blocks only to bound memory (each block is exact: causal
blocks use the key prefix their last row can see). It is not the tiled,
online-softmax algorithm and shares nothing with the GPU path.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

BIAS_RADIUS = 128


def _lens(offsets) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    return off[1:] - off[:-1]


def valid_pairs(q_offsets, kv_offsets, causal: bool) -> int:
    """Number of (query, key) pairs the attention actually uses, per head."""
    total = 0
    for lq, lk in zip(_lens(q_offsets), _lens(kv_offsets)):
        lq, lk = int(lq), int(lk)
        if not causal:
            total += lq * lk
        else:
            # sum_i min(i + 1, lk) for i in [0, lq)
            m = min(lq, lk)
            total += m * (m + 1) // 2 + (lq - m) * lk
    return total


def _scores(Qb, K, h, r0, r1, ncol, scale, bias, causal):
    S = scale * (Qb @ K[:ncol].T)
    if bias is not None or causal:
        i = np.arange(r0, r1)[:, None]
        j = np.arange(ncol)[None, :]
        if bias is not None:
            S = S + bias[h].astype(np.float64)[np.clip(i - j, -BIAS_RADIUS, BIAS_RADIUS) + BIAS_RADIUS]
        if causal:
            S = np.where(j <= i, S, -np.inf)
    return S


def _selected(B: int, H: int, pairs: Optional[Iterable[Tuple[int, int]]]):
    if pairs is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return sorted(set((int(b), int(h)) for b, h in pairs))


def forward(q, k, v, q_offsets, kv_offsets, bias=None, causal: bool = False,
            scale: Optional[float] = None, pairs=None, row_block: int = 512):
    """Exact attention over jagged sequences.

    q: [Tq, H, D]; k, v: [Tk, H, D] (any float dtype, upcast to fp64 per slice);
    offsets: int [B+1]; bias: None or [H, 2R+1]. ``pairs`` restricts the work to
    a list of (b, h); rows outside it are left at O = 0, lse = nan.
    Returns (out [Tq, H, D] fp64, lse [Tq, H] fp64).
    """
    Tq, H, D = q.shape
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    B = len(qo) - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((Tq, H, D), dtype=np.float64)
    lse = np.full((Tq, H), np.nan, dtype=np.float64)
    for b, h in _selected(B, H, pairs):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        Lq, Lk = qe - qs, ke - ks
        if Lq == 0:
            continue
        if Lk == 0:
            out[qs:qe, h] = 0.0
            lse[qs:qe, h] = -np.inf
            continue
        Q = q[qs:qe, h].astype(np.float64)
        K = k[ks:ke, h].astype(np.float64)
        V = v[ks:ke, h].astype(np.float64)
        for r0 in range(0, Lq, row_block):
            r1 = min(r0 + row_block, Lq)
            ncol = min(Lk, r1) if causal else Lk
            S = _scores(Q[r0:r1], K, h, r0, r1, ncol, scale, bias, causal)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1)
            out[qs + r0:qs + r1, h] = (E @ V[:ncol]) / l[:, None]
            lse[qs + r0:qs + r1, h] = m[:, 0] + np.log(l)
    return out, lse


def backward(q, k, v, dout, q_offsets, kv_offsets, bias=None, causal: bool = False,
             scale: Optional[float] = None, pairs=None, row_block: int = 512,
             out=None, lse=None):
    """Gradients of sum(dout * O) with respect to q, k and v (fp64).

    ``out``/``lse`` may be passed from :func:`forward`; otherwise they are
    recomputed here. Returns (dq, dk, dv) with the shapes of q, k, v.
    """
    Tq, H, D = q.shape
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    B = len(qo) - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None or lse is None:
        out, lse = forward(q, k, v, qo, ko, bias, causal, scale, pairs, row_block)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b, h in _selected(B, H, pairs):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        Lq, Lk = qe - qs, ke - ks
        if Lq == 0 or Lk == 0:
            continue
        Q = q[qs:qe, h].astype(np.float64)
        K = k[ks:ke, h].astype(np.float64)
        V = v[ks:ke, h].astype(np.float64)
        dO = dout[qs:qe, h].astype(np.float64)
        O = np.asarray(out[qs:qe, h], dtype=np.float64)
        L = np.asarray(lse[qs:qe, h], dtype=np.float64)
        dK = np.zeros((Lk, D))
        dV = np.zeros((Lk, D))
        for r0 in range(0, Lq, row_block):
            r1 = min(r0 + row_block, Lq)
            ncol = min(Lk, r1) if causal else Lk
            S = _scores(Q[r0:r1], K, h, r0, r1, ncol, scale, bias, causal)
            P = np.exp(S - L[r0:r1, None])
            dOb = dO[r0:r1]
            dV[:ncol] += P.T @ dOb
            dP = dOb @ V[:ncol].T
            delta = (dOb * O[r0:r1]).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dq[qs + r0:qs + r1, h] = scale * (dS @ K[:ncol])
            dK[:ncol] += scale * (dS.T @ Q[r0:r1])
        dk[ks:ke, h] = dK
        dv[ks:ke, h] = dV
    return dq, dk, dv


def bias_grad(q, k, v, dout, q_offsets, kv_offsets, bias, causal: bool = False,
              scale: Optional[float] = None, pairs=None, row_block: int = 512, out=None, lse=None):
    """Gradient of sum(dout * O) with respect to the bias table (fp64, [H, 2R+1]).

    beta[h, r] enters every score S_ij of head h whose relative position falls
    in bin r = clip(i - j, -R, R) + R, so its gradient is the sum of dS_ij
    (the gradient with respect to S_ij) over those pairs, over all sequences.
    Pairs the causal mask hides have P = 0, hence dS = 0.
    """
    Tq, H, D = q.shape
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    B = len(qo) - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None or lse is None:
        out, lse = forward(q, k, v, qo, ko, bias, causal, scale, pairs, row_block)
    nbins = 2 * BIAS_RADIUS + 1
    dbias = np.zeros((H, nbins), dtype=np.float64)
    for b, h in _selected(B, H, pairs):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        Lq, Lk = qe - qs, ke - ks
        if Lq == 0 or Lk == 0:
            continue
        Q = q[qs:qe, h].astype(np.float64)
        K = k[ks:ke, h].astype(np.float64)
        V = v[ks:ke, h].astype(np.float64)
        dO = dout[qs:qe, h].astype(np.float64)
        O = np.asarray(out[qs:qe, h], dtype=np.float64)
        L = np.asarray(lse[qs:qe, h], dtype=np.float64)
        for r0 in range(0, Lq, row_block):
            r1 = min(r0 + row_block, Lq)
            ncol = min(Lk, r1) if causal else Lk
            S = _scores(Q[r0:r1], K, h, r0, r1, ncol, scale, bias, causal)
            P = np.exp(S - L[r0:r1, None])
            dP = dO[r0:r1] @ V[:ncol].T
            delta = (dO[r0:r1] * O[r0:r1]).sum(axis=1)
            dS = P * (dP - delta[:, None])
            i = np.arange(r0, r1)[:, None]
            j = np.arange(ncol)[None, :]
            bins = np.clip(i - j, -BIAS_RADIUS, BIAS_RADIUS) + BIAS_RADIUS
            dbias[h] += np.bincount(bins.ravel(), weights=dS.ravel(), minlength=nbins)
    return dbias

"""fp64 reference for the attention variants: additive logit bias and its
gradient, logit soft-capping (a score modification), a per-head sink logit
and its gradient, and the per-head maximum logit.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, float64,
dense [Sq, Skv] matrices, one (batch row, query head) at a time; each
quantity is its definition written out.

The pages only name these variants.  The TransformerEngine page on fused
attention backward sharding ("[JAX] Align fused attn backward output
gradient sharding and other test strengthening") runs backward cases with
max-logit and score-mod (Changes 5) and returns optional bias gradients
beside the Q/K/V gradients (Diagram; Changes 5 and 6 reduce dBias across
data-parallel axes); the TransformerEngine page "[JAX] Make all jax
attention calls use non-packed common calls" links a change adding sink
attention.  None of them writes the equations, so the readings below are the
plainest ones in common use:

  * logits:   X_ij = scale * <q_i, k_j> + bias[b', h, i, j]
              (bias [Bb, Hq, Sq, Skv], Bb = 1 shared by every batch row or
              Bb = B; b' = b or 0)
  * score modification (soft-capping, c > 0):
              S_ij = c * tanh(X_ij / c), else S_ij = X_ij
  * sink:     one extra softmax term per query with logit sink[h] and no
              value:  P_ij = exp(S_ij) / (exp(sink[h]) + sum_allowed exp(S_ij)),
              LSE_i = log(exp(sink[h]) + sum_allowed exp(S_ij));
              a row that attends no key then has O = 0 and LSE = sink[h]
  * max logit: per query head, the largest S_ij over batch rows and allowed
              pairs (the sink is not a pair); -inf when there is none
  * gradients: dS = P (dP - Delta) as without variants, dX = dS * dS/dX
              (1 - (S / c)^2 under soft-capping), dQ = scale dX K,
              dK = scale dX^T Q, dbias = dX summed over the batch rows that
              share a bias row, dsink[h] = - sum_{b,i} P_sink(b,i) Delta(b,i)
              with P_sink = exp(sink[h] - LSE).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _check_shapes, _heads, allowed_mask, kv_head_of, resolve_segments


def _bias_row(bias, b):
    """The bias slab [Hq, Sq, Skv] batch row b reads (None without bias)."""
    if bias is None:
        return None
    return bias[b if bias.shape[0] > 1 else 0]


def _logits(qh, kh, scale, bias_h, softcap):
    """(X, S): the biased, scaled logits and the score-modified ones."""
    X = scale * (qh @ kh.T)
    if bias_h is not None:
        X = X + bias_h
    if softcap:
        S = softcap * np.tanh(X / softcap)
    else:
        S = X
    return X, S


def _softmax_with_sink(S, mask, sink_h):
    """Probabilities over the allowed keys plus an optional sink term.

    Returns (P, lse, p_sink).  P is 0 where masked; a row whose terms are all
    exp(-inf) (no allowed key and no sink) gets P = 0, LSE = -inf.
    """
    Sq = S.shape[0]
    Z = np.where(mask, S, -np.inf)
    m = Z.max(axis=1) if S.shape[1] else np.full(Sq, -np.inf)
    if sink_h is not None:
        m = np.maximum(m, sink_h)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    with np.errstate(under="ignore"):
        E = np.exp(Z - m0[:, None])
        e_sink = np.exp(sink_h - m0) if sink_h is not None else np.zeros(Sq)
    den = E.sum(axis=1) + e_sink
    den_safe = np.where(live, den, 1.0)
    P = np.where(live[:, None], E / den_safe[:, None], 0.0)
    lse = np.where(live, m0 + np.log(den_safe), -np.inf)
    p_sink = np.where(live, e_sink / den_safe, 0.0)
    return P, lse, p_sink


def _prep(q, k, v, scale, bias, softcap, sink):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Skv, Hq, Hkv, Dqk, Dv = _check_shapes(q, k, v)
    scale = 1.0 / math.sqrt(Dqk) if scale is None else float(scale)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
        if bias.ndim != 4 or bias.shape[0] not in (1, B) or bias.shape[1:] != (Hq, Sq, Skv):
            raise ValueError("bias must be [1 or B, Hq, Sq, Skv]")
    softcap = float(softcap) if softcap else 0.0
    if softcap < 0:
        raise ValueError("softcap must be >= 0")
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64)
        if sink.shape != (Hq,):
            raise ValueError("sink must be [Hq]")
    return q, k, v, (B, Sq, Skv, Hq, Hkv, Dqk, Dv), scale, bias, softcap, sink


def forward_ex(q, k, v, *, causal: bool, scale=None, segments=None, heads=None, bias=None, softcap=0.0,
               sink=None):
    """O, LSE and the per-head maximum logit with the variants applied.

    Returns a dict with O [B,Sq,Hq,Dv], LSE [B,Hq,Sq], max_logit [Hq]
    (NaN for heads outside ``heads``) and count [B,Sq].
    """
    q, k, v, dims, scale, bias, softcap, sink = _prep(q, k, v, scale, bias, softcap, sink)
    B, Sq, Skv, Hq, Hkv, Dqk, Dv = dims
    seg = resolve_segments(segments, B, Sq, Skv)
    O = np.full((B, Sq, Hq, Dv), np.nan)
    LSE = np.full((B, Hq, Sq), np.nan)
    max_logit = np.full(Hq, np.nan)
    count = np.zeros((B, Sq), dtype=np.int64)
    for h in _heads(heads, Hq):
        max_logit[h] = -np.inf
    for b in range(B):
        mask = allowed_mask(b, Sq, Skv, causal, seg)
        count[b] = mask.sum(axis=1)
        brow = _bias_row(bias, b)
        for h in _heads(heads, Hq):
            c = kv_head_of(h, Hq, Hkv)
            _, S = _logits(q[b, :, h, :], k[b, :, c, :], scale, None if brow is None else brow[h], softcap)
            if mask.any():
                max_logit[h] = max(max_logit[h], float(S[mask].max()))
            P, lse, _ = _softmax_with_sink(S, mask, None if sink is None else sink[h])
            O[b, :, h, :] = P @ v[b, :, c, :]
            LSE[b, h] = lse
    return {"O": O, "LSE": LSE, "max_logit": max_logit, "count": count}


def backward_ex(q, k, v, do, *, causal: bool, scale=None, segments=None, heads=None, bias=None, softcap=0.0,
                sink=None, return_p=False):
    """Gradients of O with respect to Q, K, V, the bias and the sink logits
    for upstream dO.

    ``heads`` restricts the work to a subset of query heads; dK/dV of a
    key/value head are complete only when its whole group is in the subset
    (otherwise NaN), dbias and dsink of heads outside it are NaN.  Returns
    dQ, dK, dV, dbias (bias's shape, None without bias), dsink ([Hq], None
    without sink), and O, LSE, Delta of the heads computed (with
    ``return_p`` also the probabilities P [B, Hq, Sq, Skv], for error
    bounds that scale with them).
    """
    q, k, v, dims, scale, bias, softcap, sink = _prep(q, k, v, scale, bias, softcap, sink)
    B, Sq, Skv, Hq, Hkv, Dqk, Dv = dims
    do = np.asarray(do, dtype=np.float64)
    if do.shape != (B, Sq, Hq, Dv):
        raise ValueError("do must be [B, Sq, Hq, Dv]")
    seg = resolve_segments(segments, B, Sq, Skv)
    hs = list(_heads(heads, Hq))
    g = Hq // Hkv
    dQ = np.full(q.shape, np.nan)
    dK = np.full(k.shape, np.nan)
    dV = np.full(v.shape, np.nan)
    dbias = None if bias is None else np.full(bias.shape, np.nan)
    dsink = None if sink is None else np.full(Hq, np.nan)
    O = np.full((B, Sq, Hq, Dv), np.nan)
    LSE = np.full((B, Hq, Sq), np.nan)
    Delta = np.full((B, Hq, Sq), np.nan)
    Pall = np.full((B, Hq, Sq, Skv), np.nan) if return_p else None
    for h in hs:
        if dbias is not None:
            dbias[:, h] = 0.0
        if dsink is not None:
            dsink[h] = 0.0
    complete = [c for c in range(Hkv) if all(h in hs for h in range(c * g, c * g + g))]
    for b in range(B):
        mask = allowed_mask(b, Sq, Skv, causal, seg)
        brow = _bias_row(bias, b)
        for c in {kv_head_of(h, Hq, Hkv) for h in hs}:
            dK[b, :, c, :] = 0.0
            dV[b, :, c, :] = 0.0
        for h in hs:
            c = kv_head_of(h, Hq, Hkv)
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, c, :], v[b, :, c, :], do[b, :, h, :]
            _, S = _logits(qh, kh, scale, None if brow is None else brow[h], softcap)
            P, lse, p_sink = _softmax_with_sink(S, mask, None if sink is None else sink[h])
            dP = doh @ vh.T
            delta = (P * dP).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dX = dS * (1.0 - (S / softcap) ** 2) if softcap else dS
            dQ[b, :, h, :] = scale * (dX @ kh)
            dK[b, :, c, :] += scale * (dX.T @ qh)
            dV[b, :, c, :] += P.T @ doh
            if dbias is not None:
                dbias[b if bias.shape[0] > 1 else 0, h] += dX
            if dsink is not None:
                dsink[h] += float(-(p_sink * delta).sum())
            O[b, :, h, :] = P @ vh
            LSE[b, h] = lse
            Delta[b, h] = delta
            if return_p:
                Pall[b, h] = P
    for c in range(Hkv):
        if c not in complete:
            dK[:, :, c, :] = np.nan
            dV[:, :, c, :] = np.nan
    out = {"dQ": dQ, "dK": dK, "dV": dV, "dbias": dbias, "dsink": dsink, "O": O, "LSE": LSE, "Delta": Delta}
    if return_p:
        out["P"] = Pall
    return out

"""fp64 reference for masked scaled-dot-product attention and its gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, float64
throughout, dense [Sq, Skv] matrices, one (batch row, query head) at a time.
No tiling, no online softmax, no recompute from a stored log-sum-exp: each
quantity is the definition written out.

Notation (shared with the tests):
  q  [B, Sq,  Hq,  Dqk]   k [B, Skv, Hkv, Dqk]   v [B, Skv, Hkv, Dv]
  do [B, Sq,  Hq,  Dv]    (upstream gradient of the output O)
  segments: dict with "ids_q", "pos_q", "ids_kv", "pos_kv", each int32
  [B, S] or None.  ids 0 marks padding.

Readings of points the pages leave open:
  * id 0 is padding: a query with id 0 attends nothing, a key with id 0 is
    attended by nothing.
  * with segment metadata, causal compares positions, pos_kv[j] <= pos_q[i],
    not raw token indices; without metadata it compares indices and needs
    Sq == Skv.
  * a query row that attends nothing has O = 0 and LSE = -inf, and adds
    nothing to any gradient; its dQ row is 0.  A key attended by nothing has
    dK = dV = 0.
  * LSE is the natural-log log-sum-exp of the scaled logits, [B, Hq, Sq].
  * GQA maps query head h to key/value head h // (Hq // Hkv).
  * the default softmax scale is 1 / sqrt(Dqk).
"""

from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Segment metadata
# ---------------------------------------------------------------------------

def derive_pos(ids) -> np.ndarray:
    """Position of each token inside the contiguous run of equal ids that
    holds it (first token of a run has position 0).

    This is the plain reading of the helper that builds segment positions
    from segment ids alone ("[JAX] Fix batcher in FusedAttn primitive ...",
    Description: from_segment_ids_and_pos() generates segment_pos
    internally).  Written as an explicit scan so it can be read at a glance.
    """
    ids = np.asarray(ids)
    B, S = ids.shape
    pos = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        start = 0
        for i in range(S):
            if i > 0 and ids[b, i] != ids[b, i - 1]:
                start = i
            pos[b, i] = i - start
    return pos


def resolve_segments(segments, B: int, Sq: int, Skv: int):
    """Fill in the defaults of a metadata dict.

    * no dict: plain BSHD, returns None;
    * ids_q is required; pos_q None -> derived from ids_q;
    * ids_kv None -> self-attention, KV metadata is Q's (needs Sq == Skv);
    * pos_kv None -> derived from ids_kv.
    Metadata are [batch, seqlen] pairs for Q and for KV ("[JAX] Fix batcher
    ...", Description; "[JAX] Align fused attn backward ...", Changes 3-4).
    """
    if segments is None:
        return None
    ids_q = np.asarray(segments["ids_q"], dtype=np.int64)
    if ids_q.shape != (B, Sq):
        raise ValueError("ids_q must be [B, Sq]")
    pos_q = segments.get("pos_q")
    pos_q = derive_pos(ids_q) if pos_q is None else np.asarray(pos_q, dtype=np.int64)
    if pos_q.shape != (B, Sq):
        raise ValueError("pos_q must be [B, Sq]")
    ids_kv = segments.get("ids_kv")
    if ids_kv is None:
        if Sq != Skv:
            raise ValueError("self-attention metadata needs Sq == Skv")
        return ids_q, pos_q, ids_q, pos_q
    ids_kv = np.asarray(ids_kv, dtype=np.int64)
    if ids_kv.shape != (B, Skv):
        raise ValueError("ids_kv must be [B, Skv]")
    pos_kv = segments.get("pos_kv")
    pos_kv = derive_pos(ids_kv) if pos_kv is None else np.asarray(pos_kv, dtype=np.int64)
    if pos_kv.shape != (B, Skv):
        raise ValueError("pos_kv must be [B, Skv]")
    return ids_q, pos_q, ids_kv, pos_kv


def allowed_mask(b: int, Sq: int, Skv: int, causal: bool, seg) -> np.ndarray:
    """Boolean [Sq, Skv]: may query i of batch row b attend key j.

    Without metadata: every pair, or j <= i when causal.
    With metadata (seg = resolve_segments(...)): same nonzero segment id, and
    when causal pos_kv[j] <= pos_q[i].
    """
    if seg is None:
        if not causal:
            return np.ones((Sq, Skv), dtype=bool)
        if Sq != Skv:
            raise ValueError("causal attention without metadata needs Sq == Skv")
        return np.tril(np.ones((Sq, Skv), dtype=bool))
    ids_q, pos_q, ids_kv, pos_kv = seg
    iq = ids_q[b][:, None]
    ik = ids_kv[b][None, :]
    mask = (iq != 0) & (iq == ik)
    if causal:
        mask &= pos_kv[b][None, :] <= pos_q[b][:, None]
    return mask


def fast_route_eligible(segments, B: int, Sq: int, Skv: int) -> np.ndarray:
    """Per batch row: may the boundary-only (fast) mask replace the general
    metadata compare without changing the set of allowed pairs.

    "[JAX] Align fused attn backward ..." (Changes 3 and 4, Diagram): the
    fast path is taken only when Q and KV describe matching token metadata;
    otherwise the general path.  The condition used here, per row:
      * Sq == Skv, ids_q == ids_kv and pos_q == pos_kv elementwise;
      * every run of a nonzero id has an id larger than every nonzero id
        before it (so each nonzero id is one contiguous run);
      * pos equals the offset of the token inside its run.
    Under these, "same id" equals "same run", and pos order equals index
    order, so the mask is decided by run boundaries alone.
    """
    seg = resolve_segments(segments, B, Sq, Skv)
    out = np.zeros(B, dtype=bool)
    if seg is None or Sq != Skv:
        return out
    ids_q, pos_q, ids_kv, pos_kv = seg
    for b in range(B):
        if not (np.array_equal(ids_q[b], ids_kv[b]) and np.array_equal(pos_q[b], pos_kv[b])):
            continue
        ok = True
        best = None          # largest nonzero id seen so far
        start = 0
        for i in range(Sq):
            cur = int(ids_q[b, i])
            if i == 0 or cur != int(ids_q[b, i - 1]):
                start = i
                if cur != 0:
                    if best is not None and cur <= best:
                        ok = False
                        break
                    best = cur
            if cur != 0 and int(pos_q[b, i]) != i - start:
                ok = False
                break
        out[b] = ok
    return out


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """GQA grouping: the g = Hq / Hkv query heads h = g*c .. g*c+g-1 share
    key/value head c (maxdiffusion PR 485, Code Review of the fused backward:
    q_heads_per_kv_head, q_head_in_group)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


# ---------------------------------------------------------------------------
# Forward and backward
# ---------------------------------------------------------------------------

def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, Sq, Hq, Dqk = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != Dqk or v.shape[:3] != (B, Skv, Hkv):
        raise ValueError("inconsistent q/k/v shapes")
    if Hq < 1 or Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return B, Sq, Skv, Hq, Hkv, Dqk, v.shape[3]


def _probabilities(qh, kh, mask, scale):
    """Softmax of the masked, scaled logits of one (row, head).

    Returns (S, P, n, lse): S the scaled logits [Sq, Skv], P the attention
    probabilities (0 where masked, whole row 0 when nothing is allowed),
    n the allowed count per query, lse the natural log-sum-exp (-inf for
    an empty row).
    """
    S = scale * (qh @ kh.T)
    n = mask.sum(axis=1)
    masked = np.where(mask, S, -np.inf)
    m = masked.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    m_safe = np.where(n > 0, m, 0.0)
    with np.errstate(under="ignore"):
        E = np.exp(np.where(mask, S - m_safe[:, None], -np.inf))
    den = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(n[:, None] > 0, E / np.where(den > 0, den, 1.0)[:, None], 0.0)
        lse = np.where(n > 0, m_safe + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return S, P, n, lse


def _heads(heads, Hq):
    return range(Hq) if heads is None else sorted(set(int(h) for h in heads))


def forward(q, k, v, *, causal: bool, scale=None, segments=None, heads=None):
    """O = softmax(scale * Q K^T + mask) V and LSE, in float64.

    ``heads`` restricts the work to a subset of query heads (other heads'
    outputs are NaN) so that full-size inputs can be checked on a sample.
    Returns a dict with O [B,Sq,Hq,Dv], LSE [B,Hq,Sq] and count [B,Sq]
    (number of keys each query attends).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Skv, Hq, Hkv, Dqk, Dv = _check_shapes(q, k, v)
    scale = 1.0 / math.sqrt(Dqk) if scale is None else float(scale)
    seg = resolve_segments(segments, B, Sq, Skv)
    O = np.full((B, Sq, Hq, Dv), np.nan)
    LSE = np.full((B, Hq, Sq), np.nan)
    count = np.zeros((B, Sq), dtype=np.int64)
    for b in range(B):
        mask = allowed_mask(b, Sq, Skv, causal, seg)
        count[b] = mask.sum(axis=1)
        for h in _heads(heads, Hq):
            c = kv_head_of(h, Hq, Hkv)
            _, P, _, lse = _probabilities(q[b, :, h, :], k[b, :, c, :], mask, scale)
            O[b, :, h, :] = P @ v[b, :, c, :]
            LSE[b, h] = lse
    return {"O": O, "LSE": LSE, "count": count}


def backward(q, k, v, do, *, causal: bool, scale=None, segments=None, heads=None):
    """Analytic gradient of O with respect to Q, K, V for upstream dO.

    For one (row, head):  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,
    dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q,
    dV = P^T dO.  dK and dV of a key/value head sum over the query heads of
    its group (maxdiffusion PR 485, Key Features: dK/dV accumulated across
    GQA heads).  P is recomputed from the definition, not from a stored LSE.

    ``heads`` restricts the work to a subset of query heads; dK/dV of a
    key/value head are complete only when its whole group is in the subset
    (otherwise NaN).  Returns dQ, dK, dV and, for diagnostics, O, LSE and
    Delta of the heads computed.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Sq, Skv, Hq, Hkv, Dqk, Dv = _check_shapes(q, k, v)
    if do.shape != (B, Sq, Hq, Dv):
        raise ValueError("do must be [B, Sq, Hq, Dv]")
    scale = 1.0 / math.sqrt(Dqk) if scale is None else float(scale)
    seg = resolve_segments(segments, B, Sq, Skv)
    hs = list(_heads(heads, Hq))
    g = Hq // Hkv
    dQ = np.full(q.shape, np.nan)
    dK = np.full(k.shape, np.nan)
    dV = np.full(v.shape, np.nan)
    O = np.full((B, Sq, Hq, Dv), np.nan)
    LSE = np.full((B, Hq, Sq), np.nan)
    Delta = np.full((B, Hq, Sq), np.nan)
    complete = [c for c in range(Hkv) if all(h in hs for h in range(c * g, c * g + g))]
    for b in range(B):
        mask = allowed_mask(b, Sq, Skv, causal, seg)
        for c in {kv_head_of(h, Hq, Hkv) for h in hs}:
            dK[b, :, c, :] = 0.0
            dV[b, :, c, :] = 0.0
        for h in hs:
            c = kv_head_of(h, Hq, Hkv)
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, c, :], v[b, :, c, :], do[b, :, h, :]
            _, P, _, lse = _probabilities(qh, kh, mask, scale)
            dP = doh @ vh.T
            delta = (P * dP).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dQ[b, :, h, :] = scale * (dS @ kh)
            dK[b, :, c, :] += scale * (dS.T @ qh)
            dV[b, :, c, :] += P.T @ doh
            O[b, :, h, :] = P @ vh
            LSE[b, h] = lse
            Delta[b, h] = delta
    for c in range(Hkv):
        if c not in complete:          # partial group sums are not results
            dK[:, :, c, :] = np.nan
            dV[:, :, c, :] = np.nan
    return {"dQ": dQ, "dK": dK, "dV": dV, "O": O, "LSE": LSE, "Delta": Delta}

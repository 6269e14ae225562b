"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function returns the largest discrepancy it finds; the tests
in ``test_oracle_pins.py`` assert it is below a bound, and
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and
asserts that at least one pin then fails.  Nothing here imports the HIP
path.
"""

from __future__ import annotations

import math

import numpy as np
import scipy.special

import oracle
from oracle import attention as oa


def rng_arrays(seed, B, Sq, Skv, Hq, Hkv, Dqk, Dv):
    r = np.random.default_rng([seed, 99])
    q = r.standard_normal((B, Sq, Hq, Dqk))
    k = r.standard_normal((B, Skv, Hkv, Dqk))
    v = r.standard_normal((B, Skv, Hkv, Dv))
    do = r.standard_normal((B, Sq, Hq, Dv))      # nonuniform upstream gradient
    return q, k, v, do


# Small metadata cases used by several pins -------------------------------

def seg_packed_padded():
    # two segments and a padded tail on row 0; three segments on row 1
    ids = np.array([[1, 1, 1, 1, 2, 2, 2, 0, 0, 0],
                    [1, 1, 2, 2, 2, 2, 3, 3, 3, 3]], dtype=np.int32)
    return {"ids_q": ids, "pos_q": oa.derive_pos(ids), "ids_kv": None, "pos_kv": None}


def seg_cross_rotated():
    # independent Q / KV segmentations, KV rotated by 3 (splits segment 3),
    # Q id 4 has no keys (empty rows), KV id 5 has no queries
    ids_q = np.array([[1, 1, 1, 2, 2, 3, 3, 3, 4, 4]], dtype=np.int32)
    ids_kv0 = np.array([1, 1, 2, 2, 2, 3, 3, 3, 5, 5, 5], dtype=np.int32)
    pos_kv0 = oa.derive_pos(ids_kv0[None])[0]
    ids_kv = np.roll(ids_kv0, 3)[None]
    pos_kv = np.roll(pos_kv0, 3)[None]
    return {"ids_q": ids_q, "pos_q": oa.derive_pos(ids_q), "ids_kv": ids_kv, "pos_kv": pos_kv}


def _lse_diff(a, b):
    """Largest difference of two LSE arrays; -inf entries must coincide."""
    if not np.array_equal(np.isneginf(a), np.isneginf(b)):
        return np.inf
    fin = np.isfinite(a)
    return float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0


def loss(q, k, v, do, **kw):
    o = oracle.forward(q, k, v, **kw)["O"]
    return float(np.sum(o * do))


def pin_finite_differences(q, k, v, do, h=1e-6, **kw):
    """Largest |analytic - central difference| over every input element,
    relative to max(1, |analytic|), for L = sum(O * dO)."""
    g = oracle.backward(q, k, v, do, **kw)
    worst = 0.0
    for name, arr, grad in (("q", q, g["dQ"]), ("k", k, g["dK"]), ("v", v, g["dV"])):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(q, k, v, do, **kw)
            arr[idx] = old - h
            lm = loss(q, k, v, do, **kw)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - grad[idx]) / max(1.0, abs(grad[idx])))
    return worst


def probs_scipy(q, k, b, h, Hq, Hkv, mask, scale):
    """Attention probabilities of one (row, head) from scipy's softmax of the
    masked logits (empty rows set to 0)."""
    c = h // (Hq // Hkv)
    s = scale * (q[b, :, h, :] @ k[b, :, c, :].T)
    s = np.where(mask, s, -np.inf)
    with np.errstate(invalid="ignore"):
        p = scipy.special.softmax(s, axis=1)
    return np.where(mask.any(axis=1)[:, None], p, 0.0)


def pin_dv_is_pt_do(q, k, v, do, *, causal, segments=None):
    """dV == sum over the group's heads of P^T dO, with P from scipy."""
    B, Sq, Hq, Dqk = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(Dqk)
    seg = oa.resolve_segments(segments, B, Sq, Skv)
    g = oracle.backward(q, k, v, do, causal=causal, segments=segments)
    worst = 0.0
    for b in range(B):
        mask = oa.allowed_mask(b, Sq, Skv, causal, seg)
        ref = np.zeros((Skv, Hkv, v.shape[3]))
        for h in range(Hq):
            p = probs_scipy(q, k, b, h, Hq, Hkv, mask, scale)
            ref[:, h // (Hq // Hkv), :] += p.T @ do[b, :, h, :]
        worst = max(worst, float(np.max(np.abs(ref - g["dV"][b]))))
    return worst


def pin_row_sums(q, k, *, causal, segments=None):
    """With V = 1 every output element is the row sum of P: 1 for rows that
    attend something, 0 for empty rows."""
    B, Sq = q.shape[:2]
    Skv, Hkv = k.shape[1], k.shape[2]
    ones = np.ones((B, Skv, Hkv, 3))
    f = oracle.forward(q, k, ones, causal=causal, segments=segments)
    expect = (f["count"] > 0).astype(np.float64)[:, :, None, None]
    return float(np.max(np.abs(f["O"] - expect)))


def pin_delta_identity(q, k, v, do, *, causal, segments=None):
    """sum_j P_ij dP_ij == sum_d O_id dO_id for every row."""
    g = oracle.backward(q, k, v, do, causal=causal, segments=segments)
    rhs = np.einsum("bshd,bshd->bhs", g["O"], do)
    return float(np.max(np.abs(g["Delta"] - rhs)))


def pin_dk_zero_sum(q, k, v, do, *, causal, segments):
    """Softmax gradients sum to zero over each query's allowed keys, so dK
    summed over the keys of one self-attention segment (or over all keys
    without metadata) vanishes."""
    B, Sq = q.shape[:2]
    g = oracle.backward(q, k, v, do, causal=causal, segments=segments)
    worst = 0.0
    for b in range(B):
        if segments is None:
            groups = [np.arange(k.shape[1])]
        else:
            ids = np.asarray(segments["ids_q"])[b]
            groups = [np.nonzero(ids == s)[0] for s in np.unique(ids) if s != 0]
        for idx in groups:
            worst = max(worst, float(np.max(np.abs(g["dK"][b, idx].sum(axis=0)))))
    return worst


def pin_closed_forms(seed=0):
    """Q = 0 makes every allowed logit equal: O is the mean of the allowed
    values and LSE = ln(n).  The first token of a causal segment sees only
    itself: O = v, LSE = its own scaled logit, dQ = 0."""
    seg = seg_packed_padded()
    q, k, v, do = rng_arrays(seed, 2, 10, 10, 2, 1, 6, 4)
    worst = 0.0
    f = oracle.forward(np.zeros_like(q), k, v, causal=True, segments=seg)
    ids = seg["ids_q"]
    pos = seg["pos_q"]
    for b in range(2):
        for i in range(10):
            allowed = [j for j in range(10) if ids[b, i] != 0 and ids[b, j] == ids[b, i] and pos[b, j] <= pos[b, i]]
            for h in range(2):
                if allowed:
                    mean = v[b, allowed, 0, :].mean(axis=0)
                    worst = max(worst, float(np.max(np.abs(f["O"][b, i, h] - mean))))
                    worst = max(worst, abs(f["LSE"][b, h, i] - math.log(len(allowed))))
                else:
                    worst = max(worst, float(np.max(np.abs(f["O"][b, i, h]))))
                    if f["LSE"][b, h, i] != -np.inf:
                        worst = max(worst, 1.0)
    f = oracle.forward(q, k, v, causal=True, segments=seg)
    g = oracle.backward(q, k, v, do, causal=True, segments=seg)
    scale = 1.0 / math.sqrt(6)
    for b in range(2):
        for i in range(10):
            if ids[b, i] != 0 and pos[b, i] == 0:
                for h in range(2):
                    worst = max(worst, float(np.max(np.abs(f["O"][b, i, h] - v[b, i, 0]))))
                    s = scale * float(q[b, i, h] @ k[b, i, 0])
                    worst = max(worst, abs(f["LSE"][b, h, i] - s))
                    worst = max(worst, float(np.max(np.abs(g["dQ"][b, i, h]))))
    return worst


def pin_packed_equals_separate(seed=0):
    """Each causal segment of a packed row, run alone as plain causal
    attention, gives the packed result on its tokens; padded tokens get
    O = 0, LSE = -inf and zero gradients."""
    seg = seg_packed_padded()
    q, k, v, do = rng_arrays(seed, 2, 10, 10, 2, 1, 6, 4)
    f = oracle.forward(q, k, v, causal=True, segments=seg)
    g = oracle.backward(q, k, v, do, causal=True, segments=seg)
    worst = 0.0
    for b in range(2):
        ids = seg["ids_q"][b]
        for s in np.unique(ids):
            idx = np.nonzero(ids == s)[0]
            if s == 0:
                worst = max(worst, float(np.max(np.abs(f["O"][b, idx]))))
                if not np.all(f["LSE"][b][:, idx] == -np.inf):
                    worst = max(worst, 1.0)
                for key in ("dQ", "dK", "dV"):
                    worst = max(worst, float(np.max(np.abs(g[key][b, idx]))))
                continue
            sl = slice(idx[0], idx[-1] + 1)
            fs = oracle.forward(q[b:b + 1, sl], k[b:b + 1, sl], v[b:b + 1, sl], causal=True)
            gs = oracle.backward(q[b:b + 1, sl], k[b:b + 1, sl], v[b:b + 1, sl], do[b:b + 1, sl], causal=True)
            worst = max(worst, float(np.max(np.abs(fs["O"][0] - f["O"][b, sl]))))
            worst = max(worst, float(np.max(np.abs(fs["LSE"][0] - f["LSE"][b][:, sl]))))
            for key in ("dQ", "dK", "dV"):
                worst = max(worst, float(np.max(np.abs(gs[key][0] - g[key][b, sl]))))
    return worst


def pin_gqa_equals_mha(seed=0, causal=True, segments=None, B=1, S=9, Hq=4, Hkv=2):
    """GQA equals MHA on K/V heads repeated g times (head h uses K/V head
    h // g); the GQA dK/dV is the MHA dK/dV summed over each group."""
    q, k, v, do = rng_arrays(seed, B, S, S, Hq, Hkv, 5, 3)
    g = Hq // Hkv
    kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    f1 = oracle.forward(q, k, v, causal=causal, segments=segments)
    f2 = oracle.forward(q, kr, vr, causal=causal, segments=segments)
    g1 = oracle.backward(q, k, v, do, causal=causal, segments=segments)
    g2 = oracle.backward(q, kr, vr, do, causal=causal, segments=segments)
    dk2 = g2["dK"].reshape(B, S, Hkv, g, 5).sum(axis=3)
    dv2 = g2["dV"].reshape(B, S, Hkv, g, 3).sum(axis=3)
    return max(float(np.max(np.abs(f1["O"] - f2["O"]))),
               _lse_diff(f1["LSE"], f2["LSE"]),
               float(np.max(np.abs(g1["dQ"] - g2["dQ"]))),
               float(np.max(np.abs(g1["dK"] - dk2))),
               float(np.max(np.abs(g1["dV"] - dv2))))


def pin_padding_garbage(seed=0):
    """Padded tail tokens set to 1000.0 in Q, K, V and dO change nothing
    else (bit for bit) and get exactly zero gradients."""
    seg = seg_packed_padded()
    q, k, v, do = rng_arrays(seed, 2, 10, 10, 2, 1, 6, 4)
    ids = seg["ids_q"]
    pad = ids == 0
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for a in (q2, k2, v2, do2):
        a[pad] = 1000.0
    f1 = oracle.forward(q, k, v, causal=True, segments=seg)
    f2 = oracle.forward(q2, k2, v2, causal=True, segments=seg)
    g2 = oracle.backward(q2, k2, v2, do2, causal=True, segments=seg)
    g1 = oracle.backward(q, k, v, do, causal=True, segments=seg)
    worst = 0.0
    keep = ~pad
    for b in range(2):
        worst = max(worst, float(np.max(np.abs(f1["O"][b, keep[b]] - f2["O"][b, keep[b]]))))
        for key in ("dQ", "dK", "dV"):
            worst = max(worst, float(np.max(np.abs(g1[key][b, keep[b]] - g2[key][b, keep[b]]))))
            if pad[b].any():
                worst = max(worst, float(np.max(np.abs(g2[key][b, pad[b]]))))
    return worst


def pin_kv_permutation(seed=0, causal=False):
    """Permuting KV tokens together with their metadata leaves O and LSE
    unchanged and permutes dK and dV the same way (the mask depends on ids
    and positions only, never on token order)."""
    seg = seg_cross_rotated()
    Sq, Skv = seg["ids_q"].shape[1], seg["ids_kv"].shape[1]
    q, k, v, do = rng_arrays(seed, 1, Sq, Skv, 4, 2, 6, 5)
    perm = np.random.default_rng([seed, 7]).permutation(Skv)
    seg2 = dict(seg)
    seg2["ids_kv"] = seg["ids_kv"][:, perm]
    seg2["pos_kv"] = seg["pos_kv"][:, perm]
    f1 = oracle.forward(q, k, v, causal=causal, segments=seg)
    f2 = oracle.forward(q, k[:, perm], v[:, perm], causal=causal, segments=seg2)
    g1 = oracle.backward(q, k, v, do, causal=causal, segments=seg)
    g2 = oracle.backward(q, k[:, perm], v[:, perm], do, causal=causal, segments=seg2)
    return max(float(np.max(np.abs(f1["O"] - f2["O"]))),
               _lse_diff(f1["LSE"], f2["LSE"]),
               float(np.max(np.abs(g1["dQ"] - g2["dQ"]))),
               float(np.max(np.abs(g1["dK"][:, perm] - g2["dK"]))),
               float(np.max(np.abs(g1["dV"][:, perm] - g2["dV"]))))


def pin_shard_merge(seed=0, nshards=3):
    """Splitting KV into shards and merging the shard outputs by their
    log-sum-exp (the ring-attention combination) gives the unsplit result."""
    seg = seg_cross_rotated()
    Sq, Skv = seg["ids_q"].shape[1], seg["ids_kv"].shape[1]
    q, k, v, _ = rng_arrays(seed, 1, Sq, Skv, 2, 1, 6, 5)
    full = oracle.forward(q, k, v, causal=False, segments=seg)
    bounds = np.linspace(0, Skv, nshards + 1).astype(int)
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        s = {"ids_q": seg["ids_q"], "pos_q": seg["pos_q"],
             "ids_kv": seg["ids_kv"][:, a:b], "pos_kv": seg["pos_kv"][:, a:b]}
        f = oracle.forward(q, k[:, a:b], v[:, a:b], causal=False, segments=s)
        outs.append(f["O"])
        lses.append(f["LSE"])
    L = np.stack(lses)                                   # [n, B, H, Sq]
    with np.errstate(invalid="ignore"):
        lse = scipy.special.logsumexp(L, axis=0)
        w = np.where(np.isfinite(L), np.exp(L - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    merged = sum(np.transpose(w[i], (0, 2, 1))[..., None] * outs[i] for i in range(nshards))
    worst = float(np.max(np.abs(merged - full["O"])))
    same_inf = np.array_equal(np.isneginf(lse), np.isneginf(full["LSE"]))
    fin = np.isfinite(full["LSE"])
    worst = max(worst, float(np.max(np.abs(lse[fin] - full["LSE"][fin]))))
    return worst if same_inf else max(worst, 1.0)


def pin_torch_sdpa(seed=0, causal=True, Sq=12, Skv=12, Hq=4, Hkv=2, Dqk=8, Dv=6, segments=None):
    """Forward against torch's scaled_dot_product_attention and gradients
    against torch autograd through it, float64 on the CPU.  Only cases where
    every query attends something (SDPA gives NaN on empty rows)."""
    import torch
    q, k, v, do = rng_arrays(seed, 1, Sq, Skv, Hq, Hkv, Dqk, Dv)
    g = Hq // Hkv
    seg = oa.resolve_segments(segments, 1, Sq, Skv)
    mask = oa.allowed_mask(0, Sq, Skv, causal, seg)
    assert mask.any(axis=1).all()
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    qq = tq.permute(0, 2, 1, 3)
    kk = tk.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vv = tv.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.tensor(mask))
    o = o.permute(0, 2, 1, 3)
    (o * torch.tensor(do)).sum().backward()
    f = oracle.forward(q, k, v, causal=causal, segments=segments)
    gr = oracle.backward(q, k, v, do, causal=causal, segments=segments)
    return max(float(np.max(np.abs(o.detach().numpy() - f["O"]))),
               float(np.max(np.abs(tq.grad.numpy() - gr["dQ"]))),
               float(np.max(np.abs(tk.grad.numpy() - gr["dK"]))),
               float(np.max(np.abs(tv.grad.numpy() - gr["dV"]))))

"""Pins that tie the fp64 variant oracle (bias, soft-capping, sink, max
logit) to something other than itself.

Each ``pin_*`` takes the variants module to check (the oracle's, or a
planted-mistake copy of it in ``test_oracle_variant_pins.py``) and returns the
largest discrepancy it finds.  Nothing here imports the HIP path.
"""

from __future__ import annotations

import math

import numpy as np

import oracle
from oracle import attention as oa
from oracle import variants as ov_default
from tests.oracle_pins import _lse_diff, rng_arrays, seg_packed_padded


def variant_case(seed=0, B=2, S=6, Hq=2, Hkv=1, Dqk=3, Dv=2, bias_batch=1, softcap=1.5, sink=True):
    """Tiny inputs with every variant switched on; logits of order 1-3 so
    that soft-capping is far from linear.  Row 0 ends in a padded query (it
    attends nothing, only the sink)."""
    q, k, v, do = rng_arrays(seed, B, S, S, Hq, Hkv, Dqk, Dv)
    r = np.random.default_rng([seed, 5])
    q *= 1.7
    bias = r.standard_normal((bias_batch, Hq, S, S))
    sk = r.standard_normal(Hq) if sink else None
    ids = np.ones((B, S), dtype=np.int32)
    ids[0, S - 1] = 0
    ids[-1, S // 2:] = 2
    seg = {"ids_q": ids}
    return q, k, v, do, bias, sk, softcap, seg


def _loss(ov, q, k, v, do, bias, sink, **kw):
    o = ov.forward_ex(q, k, v, bias=bias, sink=sink, **kw)["O"]
    return float(np.sum(o * do))


def pin_finite_differences(ov=ov_default, h=1e-6, **case_kw):
    """Largest |analytic - central difference| over every element of q, k,
    v, the bias and the sink logits, relative to max(1, |analytic|), for
    L = sum(O * dO), with bias, soft-capping, sink, causal packed metadata
    and GQA all on."""
    q, k, v, do, bias, sink, softcap, seg = variant_case(**case_kw)
    kw = dict(causal=True, segments=seg, softcap=softcap)
    g = ov.backward_ex(q, k, v, do, bias=bias, sink=sink, **kw)
    worst = 0.0
    items = [(q, g["dQ"]), (k, g["dK"]), (v, g["dV"]), (bias, g["dbias"])]
    if sink is not None:
        items.append((sink, g["dsink"]))
    for arr, grad in items:
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(ov, q, k, v, do, bias, sink, **kw)
            arr[idx] = old - h
            lm = _loss(ov, q, k, v, do, bias, sink, **kw)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - grad[idx]) / max(1.0, abs(grad[idx])))
    return worst


def pin_reduces_to_plain(ov=ov_default, seed=1):
    """Zero bias, no soft-capping and no sink give the plain oracle's
    results (forward and backward), on packed causal metadata with GQA."""
    seg = seg_packed_padded()
    q, k, v, do = rng_arrays(seed, 2, 10, 10, 4, 2, 6, 4)
    zero = np.zeros((2, 4, 10, 10))
    f0 = oracle.forward(q, k, v, causal=True, segments=seg)
    g0 = oracle.backward(q, k, v, do, causal=True, segments=seg)
    f1 = ov.forward_ex(q, k, v, causal=True, segments=seg, bias=zero)
    g1 = ov.backward_ex(q, k, v, do, causal=True, segments=seg, bias=zero)
    worst = max(float(np.max(np.abs(f0["O"] - f1["O"]))), _lse_diff(f0["LSE"], f1["LSE"]))
    for key in ("dQ", "dK", "dV"):
        worst = max(worst, float(np.max(np.abs(g0[key] - g1[key]))))
    return worst


def pin_sink_is_zero_key(ov=ov_default, seed=2):
    """A sink behaves as one more key with zero key and value vectors whose
    bias is the sink logit: same O and LSE, dsink equals the gradient of
    that key's bias column, and the other gradients are unchanged."""
    B, S, Hq, Hkv = 1, 7, 2, 1
    q, k, v, do = rng_arrays(seed, B, S, S + 1, Hq, Hkv, 4, 3)
    k[:, S] = 0.0
    v[:, S] = 0.0
    sink = np.array([0.7, -1.3])
    bias = np.random.default_rng([seed, 3]).standard_normal((1, Hq, S, S + 1))
    bias[0, :, :, S] = sink[:, None]
    fa = ov.forward_ex(q, k, v, causal=False, bias=bias)
    ga = ov.backward_ex(q, k, v, do, causal=False, bias=bias)
    fs = ov.forward_ex(q, k[:, :S], v[:, :S], causal=False, bias=bias[..., :S], sink=sink)
    gs = ov.backward_ex(q, k[:, :S], v[:, :S], do, causal=False, bias=bias[..., :S], sink=sink)
    worst = max(float(np.max(np.abs(fa["O"] - fs["O"]))), _lse_diff(fa["LSE"], fs["LSE"]))
    worst = max(worst, float(np.max(np.abs(ga["dQ"] - gs["dQ"]))))
    worst = max(worst, float(np.max(np.abs(ga["dK"][:, :S] - gs["dK"]))))
    worst = max(worst, float(np.max(np.abs(ga["dV"][:, :S] - gs["dV"]))))
    worst = max(worst, float(np.max(np.abs(ga["dbias"][..., :S] - gs["dbias"]))))
    worst = max(worst, float(np.max(np.abs(ga["dbias"][0, :, :, S].sum(axis=1) - gs["dsink"]))))
    return worst


def pin_softcap_limit(ov=ov_default, seed=3):
    """A soft cap far above every logit changes nothing (tanh(x) ~ x)."""
    q, k, v, do, bias, sink, _, seg = variant_case(seed)
    kw = dict(causal=True, segments=seg, bias=bias, sink=sink)
    f0 = ov.forward_ex(q, k, v, **kw)
    f1 = ov.forward_ex(q, k, v, softcap=1e7, **kw)
    g0 = ov.backward_ex(q, k, v, do, **kw)
    g1 = ov.backward_ex(q, k, v, do, softcap=1e7, **kw)
    worst = max(float(np.max(np.abs(f0["O"] - f1["O"]))), _lse_diff(f0["LSE"], f1["LSE"]),
                float(np.max(np.abs(f0["max_logit"] - f1["max_logit"]))))
    for key in ("dQ", "dK", "dV", "dbias", "dsink"):
        worst = max(worst, float(np.max(np.abs(g0[key] - g1[key]))))
    return worst


def pin_max_logit_bruteforce(ov=ov_default, seed=4, softcap=1.5):
    """Per-head maximum logit against scalar loops over every (row, query,
    key) triple that the mask allows."""
    q, k, v, do, bias, sink, _, seg = variant_case(seed, B=2, S=6, Hq=4, Hkv=2, bias_batch=2)
    ids = seg["ids_q"]
    pos = oa.derive_pos(ids)
    B, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    scale = 1.0 / math.sqrt(D)
    expect = [-math.inf] * Hq
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                for j in range(S):
                    if ids[b, i] == 0 or ids[b, j] != ids[b, i] or pos[b, j] > pos[b, i]:
                        continue
                    x = scale * sum(q[b, i, h, d] * k[b, j, h // g, d] for d in range(D)) + bias[b, h, i, j]
                    s = softcap * math.tanh(x / softcap)
                    expect[h] = max(expect[h], s)
    got = ov.forward_ex(q, k, v, causal=True, segments=seg, bias=bias, sink=sink, softcap=softcap)["max_logit"]
    return float(np.max(np.abs(np.array(expect) - got)))


def pin_bias_row_shift(ov=ov_default, seed=5):
    """A bias constant along each query row leaves O unchanged and shifts
    LSE by that constant (softmax shift invariance)."""
    seg = seg_packed_padded()
    q, k, v, _ = rng_arrays(seed, 2, 10, 10, 2, 1, 6, 4)
    c = np.random.default_rng([seed, 1]).standard_normal((2, 2, 10))
    bias = np.broadcast_to(c[..., None], (2, 2, 10, 10)).copy()
    f0 = ov.forward_ex(q, k, v, causal=True, segments=seg)
    f1 = ov.forward_ex(q, k, v, causal=True, segments=seg, bias=bias)
    return max(float(np.max(np.abs(f0["O"] - f1["O"]))), _lse_diff(f0["LSE"] + c, f1["LSE"]))


def pin_bias_as_mask(ov=ov_default, seed=6):
    """A bias of -inf above the diagonal turns plain attention into the
    causal mask (compared with the plain oracle)."""
    q, k, v, do = rng_arrays(seed, 1, 8, 8, 2, 2, 5, 3)
    bias = np.where(np.tril(np.ones((8, 8), dtype=bool)), 0.0, -np.inf)[None, None].repeat(2, axis=1)
    f0 = oracle.forward(q, k, v, causal=True)
    g0 = oracle.backward(q, k, v, do, causal=True)
    f1 = ov.forward_ex(q, k, v, causal=False, bias=bias)
    g1 = ov.backward_ex(q, k, v, do, causal=False, bias=bias)
    worst = max(float(np.max(np.abs(f0["O"] - f1["O"]))), _lse_diff(f0["LSE"], f1["LSE"]))
    for key in ("dQ", "dK", "dV"):
        worst = max(worst, float(np.max(np.abs(g0[key] - g1[key]))))
    return worst


def pin_dbias_dsink_balance(ov=ov_default, seed=7):
    """Without soft-capping the logit gradients of a query sum to zero over
    its keys and the sink (softmax gradients are orthogonal to the ones
    vector), so the whole dbias of a head equals -dsink."""
    q, k, v, do, bias, sink, _, seg = variant_case(seed, Hq=2, Hkv=2, bias_batch=1)
    g = ov.backward_ex(q, k, v, do, causal=True, segments=seg, bias=bias, sink=sink)
    return float(np.max(np.abs(g["dbias"].sum(axis=(0, 2, 3)) + g["dsink"])))


def pin_empty_row_with_sink(ov=ov_default, seed=8):
    """A query that attends no key puts all weight on the sink: O = 0,
    LSE = sink, and it adds nothing to any gradient."""
    q, k, v, do, bias, sink, softcap, seg = variant_case(seed, bias_batch=2)
    kw = dict(causal=True, segments=seg, bias=bias, sink=sink, softcap=softcap)
    f = ov.forward_ex(q, k, v, **kw)
    g = ov.backward_ex(q, k, v, do, **kw)
    S = q.shape[1]
    worst = float(np.max(np.abs(f["O"][0, S - 1])))
    worst = max(worst, float(np.max(np.abs(f["LSE"][0, :, S - 1] - sink))))
    worst = max(worst, float(np.max(np.abs(g["dQ"][0, S - 1]))))
    worst = max(worst, float(np.max(np.abs(g["dbias"][0, :, S - 1, :]))))
    return worst


def pin_torch_sdpa_bias(ov=ov_default, seed=9):
    """Forward and gradients (dQ, dK, dV and dbias) against torch's
    scaled_dot_product_attention with an additive float mask and autograd,
    float64 on the CPU, bias shared by the batch (its gradient sums over
    the batch rows)."""
    import torch
    B, S, Hq, Hkv, D, Dv = 2, 9, 4, 2, 6, 5
    q, k, v, do = rng_arrays(seed, B, S, S, Hq, Hkv, D, Dv)
    bias = np.random.default_rng([seed, 2]).standard_normal((1, Hq, S, S))
    g = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    tb = torch.tensor(bias, requires_grad=True)
    qq = tq.permute(0, 2, 1, 3)
    kk = tk.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vv = tv.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=tb.expand(B, Hq, S, S))
    o = o.permute(0, 2, 1, 3)
    (o * torch.tensor(do)).sum().backward()
    f = ov.forward_ex(q, k, v, causal=False, bias=bias)
    gr = ov.backward_ex(q, k, v, do, causal=False, bias=bias)
    return max(float(np.max(np.abs(o.detach().numpy() - f["O"]))),
               float(np.max(np.abs(tq.grad.numpy() - gr["dQ"]))),
               float(np.max(np.abs(tk.grad.numpy() - gr["dK"]))),
               float(np.max(np.abs(tv.grad.numpy() - gr["dV"]))),
               float(np.max(np.abs(tb.grad.numpy() - gr["dbias"]))))


def all_pins(ov=ov_default):
    """(name, value, bound) of every pin, for the tests and the mutants."""
    return [
        ("finite_differences_shared_bias", pin_finite_differences(ov), 1e-6),
        ("finite_differences_batch_bias", pin_finite_differences(ov, seed=11, bias_batch=2, Hq=4, Hkv=2), 1e-6),
        ("reduces_to_plain", pin_reduces_to_plain(ov), 1e-12),
        ("sink_is_zero_key", pin_sink_is_zero_key(ov), 1e-12),
        ("softcap_limit", pin_softcap_limit(ov), 1e-9),
        ("max_logit_bruteforce", pin_max_logit_bruteforce(ov), 1e-12),
        ("bias_row_shift", pin_bias_row_shift(ov), 1e-12),
        ("bias_as_mask", pin_bias_as_mask(ov), 1e-12),
        ("dbias_dsink_balance", pin_dbias_dsink_balance(ov), 1e-12),
        ("empty_row_with_sink", pin_empty_row_with_sink(ov), 1e-12),
        ("torch_sdpa_bias", pin_torch_sdpa_bias(ov), 1e-12),
    ]

"""GPU parity of the attention variants (attn_fwd_ex / attn_bwd_ex through the
C ABI) against the fp64 variant oracle on the same seeded inputs: additive
bias and its gradient, soft-capping, sink logits and their gradient, and the
per-head maximum logit, on every route and both element types."""

import numpy as np
import pytest

import oracle
from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run_gpu(case, var, *, max_logit=True, flags=0):
    import torch
    import bwd_packed_segments_amd as bps
    dt = case["dtype"]
    t = {k: G.to_dev(case[k], dt) for k in ("q", "k", "v", "do")}
    seg = G.seg_to_dev(case["segments"])
    bias = G.to_dev(var["bias"], dt) if var["bias"] is not None else None
    sink = torch.from_numpy(var["sink"]).to("cuda") if var["sink"] is not None else None
    kw = dict(causal=case["causal"], segments=seg, bias=bias, softcap=var["softcap"], sink=sink, flags=flags)
    o, lse, ml = bps.attn_fwd_ex(t["q"], t["k"], t["v"], return_max_logit=True, **kw)
    dq, dk, dv, dbias, dsink = bps.attn_bwd_ex(t["q"], t["k"], t["v"], o, lse, t["do"], **kw)
    torch.cuda.synchronize()
    out = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}
    if max_logit:
        out["max_logit"] = ml
    if dbias is not None:
        out["dbias"] = dbias
    if dsink is not None:
        out["dsink"] = dsink
    return G.numpy_out(out)


def _run_oracle(case, var, heads=None):
    kw = dict(causal=case["causal"], segments=case["segments"], heads=heads, bias=var["bias"],
              softcap=var["softcap"], sink=var["sink"])
    f = oracle.forward_ex(case["q"], case["k"], case["v"], **kw)
    g = oracle.backward_ex(case["q"], case["k"], case["v"], case["do"], return_p=var["bias"] is not None, **kw)
    ref = {"O": f["O"], "LSE": f["LSE"], "max_logit": f["max_logit"], "dQ": g["dQ"], "dK": g["dK"], "dV": g["dV"]}
    if g["dbias"] is not None:
        ref["dbias"] = g["dbias"]
        ref["P"] = g["P"]
    if g["dsink"] is not None:
        ref["dsink"] = g["dsink"]
    return ref


# Unit roundoff of the saved output O: the backward forms Delta = <dO, O>
# from O as stored (the forward saves its output for the backward), so
# Delta_i is off by up to u * sum_d |dO_id O_id|, and dx_ij = P_ij (dP_ij -
# Delta_i) dS/dx inherits P_ij times that (dS/dx <= 1).  dQ, dK and dV
# average this over many pairs; dbias shows it element by element.
# u is the unit roundoff of round-to-nearest, half the spacing of the format
# at 1: bf16 keeps 8 significant bits (spacing 2^-7 in [1, 2), so 2^-8), fp32
# keeps 24 (2^-24).  The forward's own error in O (P rounded to bf16 before
# the P V product) is left to the base tolerance.
U_OUT = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -24}


def _check_dbias(case, gpu, ref):
    tol = G.TOL[case["dtype"]]
    a = np.abs(case["do"].astype(np.float64) * ref["O"]).sum(axis=-1).transpose(0, 2, 1)   # [B, Hq, Sq]
    extra = U_OUT[case["dtype"]] * ref["P"] * a[..., None]                                  # [B, Hq, Sq, Skv]
    if ref["dbias"].shape[0] == 1:
        extra = extra.sum(axis=0, keepdims=True)      # one slab shared by the batch rows
    r, g = ref["dbias"], gpu["dbias"]
    fin = np.isfinite(r)
    assert np.all(np.isfinite(g[fin])), "dbias: non-finite GPU values"
    err = np.abs(g[fin] - r[fin])
    bound = tol * np.maximum(1.0, np.abs(r[fin])) + extra[fin]
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), (f"dbias: error {err[worst]:.3e} > bound {bound[worst]:.3e} "
                                  f"(gpu {g[fin][worst]!r} vs ref {r[fin][worst]!r})")
    rel_l2 = float(np.linalg.norm(g[fin] - r[fin]) / max(np.linalg.norm(r[fin]), 1e-30))
    assert rel_l2 <= 1e-2, f"dbias: relative L2 error {rel_l2:.3e}"
    return {"max_abs": float(err.max()), "rel_l2": rel_l2}


def _check_dsink(case, var, gpu, ref, heads=None):
    """dsink[h] = -sum_{b,i} P_sink Delta sums the same Delta error over the
    rows, weighted by the sink's share P_sink = exp(sink - LSE)."""
    tol = G.TOL[case["dtype"]]
    a = np.abs(case["do"].astype(np.float64) * ref["O"]).sum(axis=-1).transpose(0, 2, 1)   # [B, Hq, Sq]
    p_sink = np.exp(var["sink"].astype(np.float64)[None, :, None] - ref["LSE"])
    extra = U_OUT[case["dtype"]] * (p_sink * a).sum(axis=(0, 2))
    hs = np.arange(len(var["sink"])) if heads is None else np.asarray(heads)
    r, g = ref["dsink"][hs], gpu["dsink"][hs]
    err = np.abs(g - r)
    bound = tol * np.maximum(1.0, np.abs(r)) + extra[hs]
    assert np.all(err <= bound), f"dsink: errors {err} > bounds {bound} (gpu {g} vs ref {r})"
    return {"max_abs": float(err.max())}


def _check(case, var, flags=0):
    print(f"[variants] {case['workload']} seed={case['seed']} softcap={var['softcap']} "
          f"bias={None if var['bias'] is None else var['bias'].shape} sink={var['sink'] is not None}", flush=True)
    gpu = _run_gpu(case, var, flags=flags)
    ref = _run_oracle(case, var)
    out = G.check_all(case, gpu, ref, keys=("O", "LSE", "max_logit", "dQ", "dK", "dV"))
    if "dbias" in ref:
        out["dbias"] = _check_dbias(case, gpu, ref)
    if "dsink" in ref:
        out["dsink"] = _check_dsink(case, var, gpu, ref)
    return out, gpu, ref


def _var(w, seed, softcap=0.0, **kw):
    v = inputs.variant_inputs(w, seed, **kw)
    v["softcap"] = softcap
    return v


@pytest.mark.parametrize("seed", [0, 1])
def test_packed_causal_bias_softcap_sink(seed):
    """Fast route, per-row bias, soft-capping far from linear, sink."""
    w = inputs.workload("thd_packed_8k", B=2, S=700, Hq=4, Hkv=2, seg_lo=16, seg_hi=300)
    case = inputs.make_case(w, seed)
    _check(case, _var(w, seed, softcap=2.0, bias_batch=2, sink=True))


@pytest.mark.parametrize("seed", [0, 1])
def test_gqa_causal_shared_bias_sink(seed):
    """Dense causal route, GQA 8/2, one bias slab for both batch rows (dbias
    summed over rows), sink, ragged length."""
    w = inputs.workload("gqa_causal_8k", B=2, S=520, Hq=8, Hkv=2)
    case = inputs.make_case(w, seed)
    _check(case, _var(w, seed, bias_batch=1, sink=True))


def test_cross_general_all_variants():
    """General route (independent rotated metadata, Dqk 192 / Dv 128): bias,
    soft-capping, sink."""
    w = inputs.workload("thd_cross_ring_4k", Sq=600, Skv=700, Hq=4, Hkv=2, seg_lo=32, seg_hi=256)
    case = inputs.make_case(w, 3)
    _check(case, _var(w, 3, softcap=5.0, bias_batch=1, sink=True))


def test_fp32_all_variants():
    w = inputs.workload("tiny_fp32", B=2, Sq=260, Skv=260, causal=True, Hq=2, Hkv=1)
    case = inputs.make_case(w, 4)
    _check(case, _var(w, 4, softcap=3.0, bias_batch=2, sink=True))


def test_bias_with_neg_inf_and_empty_rows():
    """A bias that masks a fifth of the pairs with -inf on packed metadata
    with a padded tail: rows left with no key put all weight on the sink
    (O = 0, LSE = sink)."""
    w = inputs.workload("thd_packed_8k", B=2, S=400, Hq=2, Hkv=1, seg_lo=1, seg_hi=40)
    case = inputs.make_case(w, 5)
    _check(case, _var(w, 5, bias_batch=2, bias_neg_inf=0.2, sink=True))


def test_softcap_only_and_max_logit_plain():
    """Soft-capping with no bias and no sink on plain non-causal BSHD."""
    w = inputs.workload("bshd_causal_2k", B=1, S=333, Hq=4, Hkv=4, causal=False)
    case = inputs.make_case(w, 6)
    _check(case, _var(w, 6, softcap=1.5))


def test_sink_row_with_no_keys_only():
    """Cross metadata where a query segment has no keys: LSE = sink there."""
    w = inputs.workload("thd_cross_ring_4k", Sq=300, Skv=260, Hq=2, Hkv=1, Dqk=128, seg_lo=20, seg_hi=60)
    case = inputs.make_case(w, 7)
    var = _var(w, 7, sink=True)
    out, gpu, ref = _check(case, var)
    assert np.isfinite(gpu["LSE"]).all()


def test_no_variant_equals_plain_bitwise():
    """attn_fwd_ex / attn_bwd_ex with nothing requested run the plain
    kernels: bitwise the results of attn_fwd / attn_bwd."""
    import torch
    import bwd_packed_segments_amd as bps
    case = G.small_case("thd_packed_8k", 8, B=2, S=500, Hq=4, Hkv=2, seg_lo=16, seg_hi=200)
    t = {k: G.to_dev(case[k], "bf16") for k in ("q", "k", "v", "do")}
    seg = G.seg_to_dev(case["segments"])
    print("[variants] none vs plain", flush=True)
    o1, l1 = bps.attn_fwd(t["q"], t["k"], t["v"], causal=True, segments=seg)
    o2, l2 = bps.attn_fwd_ex(t["q"], t["k"], t["v"], causal=True, segments=seg)
    g1 = bps.attn_bwd(t["q"], t["k"], t["v"], o1, l1, t["do"], causal=True, segments=seg)
    g2 = bps.attn_bwd_ex(t["q"], t["k"], t["v"], o1, l1, t["do"], causal=True, segments=seg)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2[:3]):
        assert torch.equal(a, b)
    assert g2[3] is None and g2[4] is None


def test_variants_deterministic_and_schedule_free():
    """Two runs, and a run with the workgroup schedule reversed, give
    bitwise equal results (shared-bias dbias partials and dsink included)."""
    w = inputs.workload("gqa_causal_8k", B=2, S=300, Hq=4, Hkv=2)
    case = inputs.make_case(w, 9)
    var = _var(w, 9, softcap=4.0, bias_batch=1, sink=True)
    print("[variants] determinism", flush=True)
    a = _run_gpu(case, var)
    b = _run_gpu(case, var)
    c = _run_gpu(case, var, flags=2)      # ATTN_REVERSE_SCHEDULE
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
        assert np.array_equal(a[k], c[k], equal_nan=True), k


def test_full_size_softcap_sink_sampled_heads():
    """The 8K causal GQA workload (B=1, Hq=64, Hkv=8, S=8192) with
    soft-capping, sink and max logit, checked on two query heads the oracle
    computes exactly (O, LSE, dQ, max logit and dsink of those heads)."""
    import torch
    import bwd_packed_segments_amd as bps
    w = inputs.WORKLOADS["gqa_causal_8k"]
    case = inputs.make_case(w, 0)
    var = _var(w, 0, softcap=6.0, sink=True)
    print("[variants] full size gqa_causal_8k", flush=True)
    gpu = _run_gpu(case, var)
    heads = [0, 37]
    ref = _run_oracle(case, var, heads=heads)
    tol = G.TOL["bf16"]
    sel_h = np.zeros(64, dtype=bool)
    sel_h[heads] = True
    G.compare("O", gpu["O"][:, :, heads], ref["O"][:, :, heads], tol)
    G.compare("LSE", gpu["LSE"][:, heads], ref["LSE"][:, heads], tol)
    G.compare("dQ", gpu["dQ"][:, :, heads], ref["dQ"][:, :, heads], tol)
    G.compare("max_logit", gpu["max_logit"][sel_h], ref["max_logit"][sel_h], tol)
    _check_dsink(case, var, gpu, ref, heads=heads)
    torch.cuda.synchronize()

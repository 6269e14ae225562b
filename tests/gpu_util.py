"""Helpers of the GPU tests: move a seeded case to the device, run the HIP
path through the C ABI, run the oracle on the same values, compare."""

from __future__ import annotations

import os

import numpy as np

import oracle
from bwd_packed_segments_amd import inputs

# Tolerance per dtype: |gpu - ref| <= TOL * max(1, |ref|) element by element
# (absolute below 1, relative above; a bf16 result alone carries a relative
# rounding of 2^-9, so a purely absolute 2e-2 cannot hold for values of 8 and
# more, which summed GQA gradients reach).
TOL = {"bf16": 2e-2, "fp32": 1e-4}

# Every comparison's statistics, for the margin summary printed at the end of
# the session (conftest.pytest_terminal_summary).
RECORD = []


def rel_l2_limit(tol):
    """Bound on ||gpu - ref||_2 / ||ref||_2: 1e-2 for bf16 outputs (an error
    spread over a whole tensor, beyond rounding, shows here long before any
    single element leaves the elementwise band), the elementwise tolerance
    itself for fp32."""
    return 1e-2 if tol >= 1e-2 else tol


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def seg_to_dev(segments):
    import torch
    from bwd_packed_segments_amd import Segments
    if segments is None:
        return None

    def t(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")
    return Segments(t(segments["ids_q"]), t(segments.get("pos_q")), t(segments.get("ids_kv")),
                    t(segments.get("pos_kv")))


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(case, flags=0, bwd=True, tensors=None):
    """Forward (and backward) on the GPU.  Returns numpy float64 arrays."""
    import torch
    import bwd_packed_segments_amd as bps
    dt = case["dtype"]
    if tensors is None:
        tensors = {k: to_dev(case[k], dt) for k in ("q", "k", "v", "do") if k in case}
    seg = seg_to_dev(case["segments"])
    o, lse, route = bps.attn_fwd(tensors["q"], tensors["k"], tensors["v"], causal=case["causal"],
                                 segments=seg, flags=flags, return_route=True)
    out = {"O": o, "LSE": lse, "route": route}
    if bwd:
        do = tensors["do"]
        if do.stride() != o.stride():
            do = do.contiguous()
        dq, dk, dv = bps.attn_bwd(tensors["q"], tensors["k"], tensors["v"], o, lse, do, causal=case["causal"],
                                  segments=seg, flags=flags)
        out.update({"dQ": dq, "dK": dk, "dV": dv})
    torch.cuda.synchronize()
    return out


def numpy_out(out):
    return {k: (to_np(v) if k != "route" else v) for k, v in out.items()}


def run_oracle(case, heads=None, bwd=True):
    f = oracle.forward(case["q"], case["k"], case["v"], causal=case["causal"], segments=case["segments"],
                       heads=heads)
    if not bwd:
        return f
    g = oracle.backward(case["q"], case["k"], case["v"], case["do"], causal=case["causal"],
                        segments=case["segments"], heads=heads)
    f.update({"dQ": g["dQ"], "dK": g["dK"], "dV": g["dV"]})
    return f


def compare(name, gpu, ref, tol, where=None):
    """Elementwise |gpu - ref| <= tol * max(1, |ref|) over the entries where
    ref is finite (and `where` selects); -inf in ref must be -inf in gpu.
    Returns a dict of statistics; raises AssertionError on failure."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sel = ~np.isnan(ref)
    if where is not None:
        sel &= where
    ninf = sel & np.isneginf(ref)
    assert np.all(np.isneginf(gpu[ninf])), f"{name}: -inf entries differ"
    fin = sel & np.isfinite(ref)
    assert np.all(np.isfinite(gpu[fin])), f"{name}: non-finite GPU values where the oracle is finite"
    if not fin.any():
        return {"max_abs": 0.0, "max_scaled": 0.0, "rel_l2": 0.0}
    g, r = gpu[fin], ref[fin]
    err = np.abs(g - r)
    scaled = err / np.maximum(1.0, np.abs(r))
    worst = int(np.argmax(scaled))
    norm_r = float(np.linalg.norm(r))
    rel_l2 = float(np.linalg.norm(g - r) / max(norm_r, 1e-30))
    stats = {"max_abs": float(err.max()), "max_scaled": float(scaled.max()), "rel_l2": rel_l2}
    RECORD.append({"test": os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], "out": name,
                   "max_scaled": stats["max_scaled"], "tol": tol, "rel_l2": rel_l2, "n": int(g.size)})
    assert scaled.max() <= tol, (f"{name}: max scaled error {scaled.max():.3e} > {tol} "
                                 f"(gpu {g[worst]!r} vs ref {r[worst]!r}); {stats}")
    if norm_r > 1e-6:
        assert rel_l2 <= rel_l2_limit(tol), f"{name}: relative L2 error {rel_l2:.3e} > {rel_l2_limit(tol)}; {stats}"
    return stats


def check_all(case, gpu, ref, keys=("O", "LSE", "dQ", "dK", "dV")):
    tol = TOL[case["dtype"]]
    out = {}
    for k in keys:
        if k in gpu and k in ref:
            out[k] = compare(k, gpu[k], ref[k], tol)
    return out


def small_case(name, seed, **over):
    return inputs.make_case(inputs.workload(name, **over), seed)

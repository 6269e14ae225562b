"""One-GPU ring emulation (attn_ring_fwd / attn_ring_bwd) against the fp64
oracle run on the whole, unsharded sequence.

Shard sizes follow the ring test of the maxdiffusion backward page
(Testing: local shards of 650 queries and 733 keys); segments are long
enough to cross shard boundaries, so global positions and the log-sum-exp
merge are both exercised."""

import numpy as np
import pytest

from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _ring_gpu(case, cp):
    import torch
    import bwd_packed_segments_amd as bps
    dt = case["dtype"]
    t = {k: G.to_dev(case[k], dt) for k in ("q", "k", "v", "do")}
    seg = G.seg_to_dev(case["segments"])
    o, lse = bps.attn_ring_fwd(t["q"], t["k"], t["v"], cp=cp, causal=case["causal"], segments=seg)
    dq, dk, dv = bps.attn_ring_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], cp=cp, causal=case["causal"],
                                   segments=seg)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}


def _check_ring(case, cp):
    print(f"[ring] {case['workload']} cp={cp} seed={case['seed']}", flush=True)
    gpu = G.numpy_out(_ring_gpu(case, cp))
    ref = G.run_oracle(case)
    G.check_all(case, gpu, ref)


@pytest.mark.parametrize("cp", [2, 4])
def test_ring_cross_rotated_gqa(cp):
    """Cross-attention with independent, rotated KV metadata (the ring-step
    recipe), GQA 4/2, Dqk 192, Dv 128, non-causal."""
    w = inputs.workload("thd_cross_ring_4k", Sq=650 * cp, Skv=733 * cp, Hq=4, Hkv=2, seg_lo=200, seg_hi=900)
    _check_ring(inputs.make_case(w, cp), cp)


def test_ring_packed_causal_derived_positions():
    """Packed causal self-attention, positions derived from the ids on the
    whole row (segments cut by shard boundaries keep their positions)."""
    w = inputs.workload("thd_packed_8k", B=2, S=1300, Hq=2, Hkv=2, seg_lo=150, seg_hi=700)
    case = inputs.make_case(w, 5)
    case["segments"] = dict(case["segments"], pos_q=None)
    _check_ring(case, 4)


def test_ring_index_causal_no_metadata():
    w = inputs.workload("bshd_causal_2k", B=1, S=1300, Hq=2, Hkv=1)
    _check_ring(inputs.make_case(w, 6), 2)


def test_ring_fp32():
    w = inputs.workload("tiny_fp32", Sq=260, Skv=390, causal=False, Hq=2, Hkv=1)
    _check_ring(inputs.make_case(w, 7), 2)


def test_ring_single_shard_equals_monolithic():
    """cp = 1 is one step whose partials are the whole result: bitwise the
    plain forward and backward."""
    import torch
    case = inputs.make_case(inputs.workload("thd_packed_8k", B=1, S=700, Hq=2, Hkv=1, seg_lo=100, seg_hi=400), 8)
    print("[ring] cp=1 vs monolithic", flush=True)
    a = _ring_gpu(case, 1)
    b = G.run_gpu(case)
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        assert torch.equal(a[k], b[k]), k


def test_ring_deterministic():
    import torch
    w = inputs.workload("thd_cross_ring_4k", Sq=650 * 2, Skv=733 * 2, Hq=4, Hkv=2, seg_lo=200, seg_hi=900)
    case = inputs.make_case(w, 9)
    print("[ring] determinism", flush=True)
    a = _ring_gpu(case, 2)
    b = _ring_gpu(case, 2)
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        assert torch.equal(a[k], b[k]), k

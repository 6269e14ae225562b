"""attn_bwd_noalloc: the backward without a workspace argument, against
attn_bwd on the same inputs, over consecutive calls of decreasing size (the
per-GPU scratch array keeps the previous call's contents, which must not
matter), plus its host validation."""

import os

import numpy as np
import pytest

from bwd_packed_segments_amd import binding as B
from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.skipif(not os.path.exists(B.library_path()),
                                reason="libbps_attn.so not built (run __graft_entry__.build())")


def test_noalloc_validation_before_any_hip_call():
    big = B.make_desc(B=64, Sq=8192, Skv=8192, Hq=16, Hkv=8, Dqk=128, Dv=128, causal=True)   # 8.4M rows
    st, text = B.validate_bwd_noalloc(big)
    assert st == B.ATTN_E_WORKSPACE and "scratch" in text
    fused = B.make_desc(B=1, Sq=256, Skv=256, Hq=2, Hkv=1, Dqk=128, Dv=128, flags=B.ATTN_FUSED_BWD)
    st, text = B.validate_bwd_noalloc(fused)
    assert st == B.ATTN_E_UNSUPPORTED and "FUSED" in text
    st, text = B.validate_bwd_noalloc(B.make_desc(B=1, Sq=256, Skv=256, Hq=2, Hkv=1, Dqk=128, Dv=128), ptr=None)
    assert st == B.ATTN_E_INVALID and "NULL" in text


CASES = [
    # (workload, overrides, seed, bitwise): at least 512 key tiles -> attn_bwd does not split either
    ("gqa_causal_8k", dict(Hq=16, Hkv=8), 0, True),
    ("thd_packed_8k", dict(B=2, S=700, Hq=4, Hkv=2, seg_lo=16, seg_hi=300), 1, False),
    ("thd_cross_ring_4k", dict(Sq=300, Skv=260, Hq=4, Hkv=2, seg_lo=32, seg_hi=128), 2, False),
]


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_over_consecutive_calls():
    import torch
    import bwd_packed_segments_amd as bps
    sizes = []
    for name, over, seed, bitwise in CASES:
        case = G.small_case(name, seed, **over)
        w = case["workload"]
        sizes.append(w.B * w.Hq * w.Sq)
        print(f"[noalloc] {w} seed={seed}", flush=True)
        t = {k: G.to_dev(case[k], w.dtype) for k in ("q", "k", "v", "do")}
        seg = G.seg_to_dev(case["segments"])
        o, lse = bps.attn_fwd(t["q"], t["k"], t["v"], causal=w.causal, segments=seg)
        ref = bps.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, segments=seg)
        got = bps.attn_bwd_noalloc(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, segments=seg)
        again = bps.attn_bwd_noalloc(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, segments=seg)
        torch.cuda.synchronize()
        for name_, a, b, c in zip(("dQ", "dK", "dV"), ref, got, again):
            assert torch.equal(b, c), f"{name_}: noalloc not reproducible"
            if bitwise:
                assert torch.equal(a, b), f"{name_}: noalloc differs from attn_bwd"
            else:
                G.compare(f"{name_} noalloc vs attn_bwd", G.to_np(b), G.to_np(a), G.TOL[w.dtype])
        if not bitwise:
            oracle_ref = G.run_oracle(case)
            for name_, b in zip(("dQ", "dK", "dV"), got):
                G.compare(name_, G.to_np(b), oracle_ref[name_], G.TOL[w.dtype])
    assert sizes[0] > sizes[1] > sizes[2]     # each call smaller than the one before

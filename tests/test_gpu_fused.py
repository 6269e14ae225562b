"""GPU parity of the single-pass backward (ATTN_FUSED_BWD): dK/dV kernel
that also writes per-key-tile dQ partials, then a fixed-order sum.

Against the fp64 oracle on the same seeded inputs (every route, GQA, head
dims, ragged and empty cases, the 8K GQA workload at full size on a group of
heads); against the two-kernel backward: dK and dV bitwise equal, dQ within
the bf16 tolerance; and bitwise reproducible under a reversed workgroup
schedule and when run phase by phase."""

import numpy as np
import pytest

from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _fused_flags():
    import bwd_packed_segments_amd as bps
    return bps.ATTN_FUSED_BWD


def _parity(case, heads=None, flags=0):
    flags |= _fused_flags()
    print(f"[fused] {case['workload']} seed={case['seed']} flags={flags}", flush=True)
    gpu = G.numpy_out(G.run_gpu(case, flags=flags))
    ref = G.run_oracle(case, heads=heads)
    return G.check_all(case, gpu, ref), gpu, ref


@pytest.mark.parametrize("causal", [True, False])
def test_fused_bshd_small(causal):
    case = G.small_case("bshd_causal_2k", 0, B=2, S=300, Hq=4, Hkv=4, causal=causal)
    _parity(case)


@pytest.mark.parametrize("seed", [0, 1])
def test_fused_thd_packed_small(seed):
    case = G.small_case("thd_packed_8k", seed, B=2, S=700, Hq=4, Hkv=4, seg_lo=16, seg_hi=300)
    _, gpu, _ = _parity(case)
    assert gpu["route"] == "fast"


@pytest.mark.parametrize("seed", [0, 1])
def test_fused_gqa_causal_small(seed):
    case = G.small_case("gqa_causal_8k", seed, S=520, Hq=8, Hkv=2)
    _parity(case)


def test_fused_thd_cross_general():
    case = G.small_case("thd_cross_ring_4k", 2, Sq=600, Skv=700, Hq=4, Hkv=2, Dqk=128, seg_lo=32, seg_hi=256)
    _, gpu, _ = _parity(case)
    assert gpu["route"] == "general"


def test_fused_cross_causal_positions():
    case = G.small_case("thd_cross_ring_4k", 3, Sq=500, Skv=500, Hq=4, Hkv=1, Dqk=128, seg_lo=32, seg_hi=200,
                        causal=True)
    _parity(case)


@pytest.mark.parametrize("dqk,dv", [(64, 64), (64, 128), (128, 64)])
def test_fused_head_dims(dqk, dv):
    case = G.small_case("gqa_causal_8k", 4, S=200, Hq=4, Hkv=2, Dqk=dqk, Dv=dv)
    _parity(case)


def test_fused_odd_lengths():
    """Non-divisible lengths (1350 queries, 1777 keys), dense non-causal and cross metadata."""
    _parity(G.small_case("bshd_causal_2k", 5, B=1, Sq=1350, Skv=1777, Hq=2, Hkv=1, causal=False))
    _parity(G.small_case("thd_cross_ring_4k", 5, Sq=1350, Skv=1777, Hq=4, Hkv=2, Dqk=128, seg_lo=64,
                         seg_hi=700))


def test_fused_all_padding_row_and_single_token():
    case = G.small_case("thd_packed_8k", 10, B=2, S=300, Hq=2, Hkv=2, seg_lo=16, seg_hi=100)
    ids = np.array(case["segments"]["ids_q"])
    ids[1] = 0
    case["segments"] = {"ids_q": ids, "pos_q": np.zeros_like(ids)}
    _, gpu, _ = _parity(case)
    for k in ("dQ", "dK", "dV"):
        assert np.all(gpu[k][1] == 0)
    _parity(G.small_case("bshd_causal_2k", 11, B=1, S=1, Hq=2, Hkv=1))


def test_fused_empty_kv_and_empty_q():
    import torch
    import bwd_packed_segments_amd as bps
    F = _fused_flags()
    print("[fused] empty kv / empty q", flush=True)
    q = torch.randn(1, 70, 2, 64, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 0, 1, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = bps.attn_fwd(q, k, k, causal=False)
    dq, dk, dv = bps.attn_bwd(q, k, k, o, lse, torch.randn_like(o), causal=False, flags=F)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0
    q0 = torch.zeros(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    k1 = torch.randn(1, 9, 1, 64, device="cuda").to(torch.bfloat16)
    o0, lse0 = bps.attn_fwd(q0, k1, k1, causal=False)
    dq0, dk0, dv0 = bps.attn_bwd(q0, k1, k1, o0, lse0, o0, causal=False, flags=F)
    torch.cuda.synchronize()
    assert torch.all(dk0 == 0) and torch.all(dv0 == 0)


def _bwd_pair(case, extra_flags=0):
    """Two-kernel and fused backward on the same forward outputs."""
    import torch
    import bwd_packed_segments_amd as bps
    dt = case["dtype"]
    t = {k: G.to_dev(case[k], dt) for k in ("q", "k", "v", "do")}
    seg = G.seg_to_dev(case["segments"])
    o, lse = bps.attn_fwd(t["q"], t["k"], t["v"], causal=case["causal"], segments=seg)
    args = (t["q"], t["k"], t["v"], o, lse, t["do"])
    two = bps.attn_bwd(*args, causal=case["causal"], segments=seg)
    one = bps.attn_bwd(*args, causal=case["causal"], segments=seg, flags=bps.ATTN_FUSED_BWD | extra_flags)
    torch.cuda.synchronize()
    return args, seg, two, one


@pytest.mark.parametrize("name,over", [
    ("gqa_causal_8k", dict(S=777, Hq=8, Hkv=2)),
    ("thd_packed_8k", dict(B=2, S=900, Hq=4, Hkv=4, seg_lo=16, seg_hi=300)),
    ("thd_cross_ring_4k", dict(Sq=600, Skv=700, Hq=4, Hkv=2, Dqk=128, seg_lo=32, seg_hi=256)),
], ids=["dense", "fast", "general"])
def test_fused_matches_two_kernel_backward(name, over):
    """dK, dV bitwise equal to the two-kernel backward (the same kernel
    computes them); dQ differs only in fp32 summation order."""
    import torch
    case = G.small_case(name, 12, **over)
    print(f"[fused] vs two-kernel {name}", flush=True)
    _, _, two, one = _bwd_pair(case)
    assert torch.equal(one[1], two[1]) and torch.equal(one[2], two[2])
    G.compare("dQ fused vs two-kernel", G.to_np(one[0]), G.to_np(two[0]), G.TOL["bf16"])


def test_fused_deterministic_and_schedule_free():
    """Bitwise equal outputs on a repeat, under a reversed workgroup
    schedule, and when the phases run as separate calls."""
    import torch
    import bwd_packed_segments_amd as bps
    case = G.small_case("thd_packed_8k", 13, B=2, S=1100, Hq=8, Hkv=2, seg_lo=16, seg_hi=400, causal=True)
    print("[fused] determinism", flush=True)
    args, seg, _, one = _bwd_pair(case)
    again = bps.attn_bwd(*args, causal=True, segments=seg, flags=bps.ATTN_FUSED_BWD)
    rev = bps.attn_bwd(*args, causal=True, segments=seg, flags=bps.ATTN_FUSED_BWD | bps.ATTN_REVERSE_SCHEDULE)
    plan = bps.BwdPlan(*args, causal=True, segments=seg, flags=bps.ATTN_FUSED_BWD)
    plan.run(bps.ATTN_BWD_PREPARE)
    plan.run(bps.ATTN_BWD_DKDV)
    plan.run(bps.ATTN_BWD_DQ)
    torch.cuda.synchronize()
    for got in (again, rev, (plan.dq, plan.dk, plan.dv)):
        for a, b in zip(got, one):
            assert torch.equal(a, b)


def test_fused_with_sink():
    """A sink enters the backward only through the saved LSE: the fused form
    takes it (attn_bwd_ex), with dsink unchanged and dQ/dK/dV against the
    oracle."""
    import torch
    import oracle
    import bwd_packed_segments_amd as bps
    case = G.small_case("gqa_causal_8k", 14, S=300, Hq=4, Hkv=2)
    sink = np.linspace(-1.0, 2.0, 4)
    print("[fused] sink", flush=True)
    t = {k: G.to_dev(case[k], "bf16") for k in ("q", "k", "v", "do")}
    st = torch.from_numpy(sink.astype(np.float32)).cuda()
    o, lse = bps.attn_fwd_ex(t["q"], t["k"], t["v"], causal=True, sink=st)
    args = (t["q"], t["k"], t["v"], o, lse, t["do"])
    one = bps.attn_bwd_ex(*args, causal=True, sink=st, flags=bps.ATTN_FUSED_BWD)
    two = bps.attn_bwd_ex(*args, causal=True, sink=st)
    torch.cuda.synchronize()
    assert torch.equal(one[1], two[1]) and torch.equal(one[2], two[2]) and torch.equal(one[4], two[4])
    ref = oracle.backward_ex(case["q"], case["k"], case["v"], case["do"], causal=True, sink=sink)
    for k, i in (("dQ", 0), ("dK", 1), ("dV", 2)):
        G.compare(k, G.to_np(one[i]), ref[k], G.TOL["bf16"])


def test_fused_full_size_gqa_group():
    """The 8K causal GQA workload at full size in the launch configuration
    the bench times with --fused-bwd; the oracle computes the whole group of
    KV head 0 (query heads 0-7)."""
    case = inputs.make_case("gqa_causal_8k", 0)
    _parity(case, heads=list(range(8)))

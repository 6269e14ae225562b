"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element.

Small shapes span several tiles and a ragged tail so the oracle finishes in
seconds; the full benchmark shapes are compared on a sample of heads the
oracle computes exactly (for dK/dV: whole GQA groups)."""

import numpy as np
import pytest

from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 2]


def _parity(case, heads=None, flags=0):
    print(f"[parity] {case['workload']} seed={case['seed']} flags={flags}", flush=True)
    gpu = G.numpy_out(G.run_gpu(case, flags=flags))
    ref = G.run_oracle(case, heads=heads)
    return G.check_all(case, gpu, ref), gpu, ref


@pytest.mark.parametrize("seed", SEEDS)
def test_tiny_fp32(seed):
    case = inputs.make_case("tiny_fp32", seed)
    _parity(case)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("causal", [True, False])
def test_bshd_small(seed, causal):
    case = G.small_case("bshd_causal_2k", seed, B=2, S=300, Hq=4, Hkv=4, causal=causal)
    _parity(case)


@pytest.mark.parametrize("seed", SEEDS)
def test_thd_packed_small(seed):
    case = G.small_case("thd_packed_8k", seed, B=2, S=700, Hq=4, Hkv=4, seg_lo=16, seg_hi=300)
    stats, gpu, _ = _parity(case)
    assert gpu["route"] == "fast"


@pytest.mark.parametrize("seed", SEEDS)
def test_gqa_causal_small(seed):
    case = G.small_case("gqa_causal_8k", seed, S=520, Hq=8, Hkv=2)
    _parity(case)


@pytest.mark.parametrize("seed", SEEDS)
def test_thd_cross_small(seed):
    case = G.small_case("thd_cross_ring_4k", seed, Sq=600, Skv=700, Hq=4, Hkv=2, seg_lo=32, seg_hi=256)
    stats, gpu, _ = _parity(case)
    assert gpu["route"] == "general"


@pytest.mark.parametrize("seed", [0, 1])
def test_thd_cross_causal_positions(seed):
    """Cross metadata with a causal mask over positions (general route)."""
    case = G.small_case("thd_cross_ring_4k", seed, Sq=500, Skv=500, Hq=4, Hkv=1, seg_lo=32, seg_hi=200,
                        causal=True)
    _parity(case)


@pytest.mark.parametrize("dqk,dv", [(64, 64), (64, 128), (128, 64), (192, 64), (192, 128)])
def test_head_dims_bf16(dqk, dv):
    case = G.small_case("gqa_causal_8k", 3, S=200, Hq=4, Hkv=2, Dqk=dqk, Dv=dv)
    _parity(case)


@pytest.mark.parametrize("dqk,dv,causal", [(128, 128, True), (64, 128, False), (128, 64, True)])
def test_head_dims_fp32(dqk, dv, causal):
    case = G.small_case("tiny_fp32", 4, S=190, Hq=2, Hkv=1, Dqk=dqk, Dv=dv, causal=causal)
    _parity(case)


@pytest.mark.parametrize("dqk,dv", [(128, 128), (64, 64), (128, 64)])
@pytest.mark.parametrize("force_general", [False, True])
def test_packed_gqa(dqk, dv, force_general):
    """Packed self-attention with GQA groups of 4, causal inside segments:
    the head-pair forward and dQ and the gradient-split dK/dV with segment
    boundaries inside their tiles, on the fast route and with every row
    forced onto the general one."""
    import bwd_packed_segments_amd as bps
    case = G.small_case("thd_packed_8k", 16, B=2, S=700, Hq=8, Hkv=2, Dqk=dqk, Dv=dv, seg_lo=16, seg_hi=300)
    stats, gpu, _ = _parity(case, flags=bps.ATTN_FORCE_GENERAL if force_general else 0)
    assert gpu["route"] == ("general" if force_general else "fast")


def test_many_batch_rows_packed():
    """Sixteen batch rows of packed segments (one metadata workgroup and one
    route per row), GQA groups of 2, causal inside segments."""
    case = G.small_case("thd_packed_8k", 17, B=16, S=300, Hq=4, Hkv=2, seg_lo=16, seg_hi=200)
    stats, gpu, _ = _parity(case)
    assert gpu["route"] == "fast"


def test_cross_causal_unequal_lengths():
    """Cross attention on the general route with Sq != Skv and a causal mask
    over positions (allowed with metadata: causal compares positions, not
    token indices), GQA groups of 2."""
    case = G.small_case("thd_cross_ring_4k", 18, Sq=600, Skv=900, Hq=4, Hkv=2, Dqk=128, seg_lo=32, seg_hi=256,
                        causal=True)
    stats, gpu, _ = _parity(case)
    assert gpu["route"] == "general"


@pytest.mark.parametrize("S,H,causal,parts", [(1024, 50, True, 2), (1024, 32, False, 3)])
def test_split_dkdv_walks(S, H, causal, parts):
    """bf16 dK/dV grids of fewer than 512 key tiles cut each key tile's walk
    over query tiles into parts whose fp32 partials a second kernel adds in
    part order.  These shapes (400 and 256 key tiles) take 2 and 3 parts; the
    workspace, which holds one partial per part, shows which."""
    from bwd_packed_segments_amd import binding
    n_kt = H * ((S + 127) // 128)
    per_part = n_kt * 128 * (128 + 128) * 4
    ws = binding.bwd_workspace_size(binding.make_desc(B=1, Sq=S, Skv=S, Hq=H, Hkv=H, Dqk=128, Dv=128, causal=causal))
    assert parts * per_part <= ws < (parts + 1) * per_part
    case = G.small_case("bshd_causal_2k", 15, B=1, S=S, Hq=H, Hkv=H, causal=causal)
    _parity(case)


def test_odd_lengths_cross():
    """Non-divisible lengths (1350 queries, 1777 keys), GQA."""
    case = G.small_case("thd_cross_ring_4k", 5, Sq=1350, Skv=1777, Hq=4, Hkv=2, Dqk=128, seg_lo=64, seg_hi=700)
    _parity(case)


def test_odd_lengths_dense():
    case = G.small_case("bshd_causal_2k", 6, B=1, Sq=1350, Skv=1777, Hq=2, Hkv=1, causal=False)
    _parity(case)


def test_packed_pos_derived_on_device():
    """pos omitted: derived on the device from ids."""
    case = G.small_case("thd_packed_8k", 7, B=2, S=400, Hq=2, Hkv=2, seg_lo=16, seg_hi=200)
    seg = dict(case["segments"])
    seg["pos_q"] = None
    case["segments"] = seg
    _parity(case)


def test_unsorted_ids_take_general_route():
    """Ids that reappear in two runs are not fast-route eligible; results
    still match the oracle."""
    case = G.small_case("thd_packed_8k", 8, B=1, S=256, Hq=2, Hkv=2, seg_lo=16, seg_hi=64)
    ids = np.array(case["segments"]["ids_q"])
    ids[0, 200:230] = 1                     # id 1 again, far from its first run
    from oracle import derive_pos
    case["segments"] = {"ids_q": ids, "pos_q": derive_pos(ids)}
    stats, gpu, _ = _parity(case)


def test_strided_packed_qkv():
    """Q, K, V as views into one packed [B, S, 3, H, D] buffer (element strides)."""
    import torch
    case = G.small_case("bshd_causal_2k", 9, B=2, S=260, Hq=4, Hkv=4)
    qkv = np.stack([case["q"], case["k"], case["v"]], axis=2)           # [B, S, 3, H, D]
    t = G.to_dev(qkv, "bf16")
    tensors = {"q": t[:, :, 0], "k": t[:, :, 1], "v": t[:, :, 2], "do": G.to_dev(case["do"], "bf16")}
    print("[parity] strided packed qkv", flush=True)
    gpu = G.numpy_out(G.run_gpu(case, tensors=tensors))
    ref = G.run_oracle(case)
    G.check_all(case, gpu, ref)
    assert tensors["q"].stride()[1] == 3 * 4 * 128


def test_empty_kv_and_empty_q():
    import torch
    import bwd_packed_segments_amd as bps
    print("[edge] empty kv", flush=True)
    q = torch.randn(1, 70, 2, 64, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 0, 1, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.zeros(1, 0, 1, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = bps.attn_fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    do = torch.randn_like(o)
    dq, dk, dv = bps.attn_bwd(q, k, v, o, lse, do, causal=False)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0
    print("[edge] empty q", flush=True)
    q0 = torch.zeros(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    k1 = torch.randn(1, 9, 1, 64, device="cuda").to(torch.bfloat16)
    o0, lse0 = bps.attn_fwd(q0, k1, k1, causal=False)
    dq0, dk0, dv0 = bps.attn_bwd(q0, k1, k1, o0, lse0, o0, causal=False)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.all(dk0 == 0) and torch.all(dv0 == 0)


def test_all_padding_row():
    """A batch row made only of padding: O = 0, LSE = -inf, all gradients 0."""
    case = G.small_case("thd_packed_8k", 10, B=2, S=300, Hq=2, Hkv=2, seg_lo=16, seg_hi=100)
    ids = np.array(case["segments"]["ids_q"])
    ids[1] = 0
    case["segments"] = {"ids_q": ids, "pos_q": np.zeros_like(ids)}
    stats, gpu, _ = _parity(case)
    assert np.all(gpu["O"][1] == 0) and np.all(np.isneginf(gpu["LSE"][1]))
    for k in ("dQ", "dK", "dV"):
        assert np.all(gpu[k][1] == 0)


def test_single_token():
    case = G.small_case("bshd_causal_2k", 11, B=1, S=1, Hq=2, Hkv=1)
    _parity(case)


# ------------------------------------------------------------ full sizes

FULL = [
    ("bshd_causal_2k", [0, 15], 0),
    ("thd_packed_8k", [0, 31], 0),
    ("gqa_causal_8k", list(range(8)), 0),      # whole group of KV head 0
    ("gqa_causal_8k", list(range(56, 64)), 1),  # whole group of KV head 7
    ("gqa_causal_8k", list(range(24, 32)), 2),  # whole group of KV head 3
    ("thd_cross_ring_4k", list(range(4)), 0),  # whole group of KV head 0
    ("thd_cross_ring_4k", list(range(28, 32)), 1),
    ("thd_cross_ring_4k", list(range(12, 16)), 2),
]


@pytest.mark.parametrize("name,heads,seed", FULL, ids=[f"{f[0]}-seed{f[2]}" for f in FULL])
def test_full_size_sampled_heads(name, heads, seed):
    """The benchmark workloads at full size, in the launch configuration the
    bench times; the oracle computes a sample of heads exactly (for dK/dV a
    whole GQA group), three seeds for the GQA and cross workloads."""
    case = inputs.make_case(name, seed)
    _parity(case, heads=heads)


EXPECTED_ROUTE = {"thd_packed_8k": "fast", "thd_cross_ring_4k": "general", "gqa_causal_8k": "dense",
                  "bshd_causal_2k": "dense"}


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("name", sorted(EXPECTED_ROUTE))
def test_effective_route_full_size(name, seed):
    """The route each batch row takes on the device at full size: every row
    of the packed workload on the fast route (every row is eligible), every
    row of the cross workload on the general one.  The cross workload has
    equal lengths, so the host requests the fast route and the device check
    turns it down: independent, rotated KV metadata must take the general
    path (TransformerEngine PR 3516, Changes 3 and 4).  Rows agree with the
    oracle's eligibility test, and ATTN_FORCE_GENERAL sends every row of the
    packed workload to the general route."""
    import oracle
    import bwd_packed_segments_amd as bps
    case = inputs.make_case(inputs.workload(name, Hq=inputs.WORKLOADS[name].Hkv), seed)
    w = case["workload"]
    print(f"[route] {name} seed={seed}", flush=True)
    t = {k: G.to_dev(case[k], w.dtype) for k in ("q", "k", "v")}
    seg = G.seg_to_dev(case["segments"])
    _, _, req, rows = bps.attn_fwd(t["q"], t["k"], t["v"], causal=w.causal, segments=seg, return_route=True,
                                   return_route_rows=True)
    rows = rows.cpu().numpy()
    expect = {"dense": 0, "fast": 1, "general": 2}[EXPECTED_ROUTE[name]]
    assert np.all(rows == expect), (name, rows)
    if case["segments"] is not None:
        elig = oracle.fast_route_eligible(case["segments"], w.B, w.Sq, w.Skv)
        assert np.array_equal(rows == 1, elig), (rows, elig)
        assert req == "fast"       # shared metadata, or equal lengths that may match
        _, _, req_g, rows_g = bps.attn_fwd(t["q"], t["k"], t["v"], causal=w.causal, segments=seg,
                                           flags=bps.ATTN_FORCE_GENERAL, return_route=True, return_route_rows=True)
        assert req_g == "general" and np.all(rows_g.cpu().numpy() == 2)
    else:
        assert req == "dense"


def test_kv_packed_views():
    """K and V as views into one packed [B, S, 2, Hkv, D] buffer, the
    KV-packed layout whose V offset the TransformerEngine page on non-packed
    common calls (PR 2358, review of the KV-packed stride) works out from the
    value head dim; GQA, causal, ragged length."""
    case = G.small_case("gqa_causal_8k", 12, S=333, Hq=4, Hkv=2)
    kv = np.stack([case["k"], case["v"]], axis=2)                       # [B, S, 2, Hkv, D]
    t = G.to_dev(kv, "bf16")
    tensors = {"q": G.to_dev(case["q"], "bf16"), "k": t[:, :, 0], "v": t[:, :, 1], "do": G.to_dev(case["do"], "bf16")}
    assert tensors["k"].stride()[1] == 2 * 2 * 128 and tensors["v"].data_ptr() - tensors["k"].data_ptr() == 2 * 2 * 128
    print("[parity] kv packed views", flush=True)
    gpu = G.numpy_out(G.run_gpu(case, tensors=tensors))
    ref = G.run_oracle(case)
    G.check_all(case, gpu, ref)


def test_do_layout_must_match_o():
    """dO must share O's strides (the output gradient takes the saved
    output's layout, TransformerEngine PR 3516, Changes 1): a dO in another
    layout is refused before anything runs, by attn_bwd and by BwdPlan."""
    import torch
    import bwd_packed_segments_amd as bps
    case = G.small_case("gqa_causal_8k", 13, S=128, Hq=4, Hkv=2)
    t = {k: G.to_dev(case[k], "bf16") for k in ("q", "k", "v", "do")}
    o, lse = bps.attn_fwd(t["q"], t["k"], t["v"], causal=True)
    do_bhsd = t["do"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # same shape, BHSD strides
    assert do_bhsd.shape == o.shape and do_bhsd.stride() != o.stride()
    with pytest.raises(ValueError, match="strides of O"):
        bps.attn_bwd(t["q"], t["k"], t["v"], o, lse, do_bhsd, causal=True)
    with pytest.raises(ValueError, match="strides of O"):
        bps.BwdPlan(t["q"], t["k"], t["v"], o, lse, do_bhsd, causal=True)
    dq, dk, dv = bps.attn_bwd(t["q"], t["k"], t["v"], o, lse, do_bhsd.contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all()


def test_long_shard_sampled_rows_and_sums():
    """The long-sequence shard (18,900 queries x 75,600 keys, H=40, D=128,
    non-causal) at full size.  Without a mask the query rows are
    independent, so O, LSE and dQ of sampled rows are checked against the
    oracle run on those rows alone (two heads); dK and dV are checked at
    every key through identities that hold at any size: the keys' dV sum to
    the queries' dO sum (softmax rows sum to one) and the keys' dK sum to
    zero (each row of dS sums to zero)."""
    import oracle
    case = inputs.make_case("wan_cp_shard", 0)
    w = case["workload"]
    print(f"[parity] {w} sampled rows + sums", flush=True)
    gpu = G.numpy_out(G.run_gpu(case))
    rows = np.r_[0:16, 9000:9016, w.Sq - 16:w.Sq]
    sub = dict(case)
    sub["q"] = case["q"][:, rows]
    sub["do"] = case["do"][:, rows]
    heads = [0, 39]
    ref = G.run_oracle(sub, heads=heads)
    tol = G.TOL["bf16"]
    for key in ("O", "dQ"):
        g = gpu[key][:, rows][:, :, heads]
        r = ref[key][:, :, heads]
        assert np.all(np.abs(g - r) <= tol * np.maximum(1.0, np.abs(r))), key
    g = gpu["LSE"][:, heads][:, :, rows]
    r = ref["LSE"][:, heads]
    assert np.all(np.abs(g - r) <= tol * np.maximum(1.0, np.abs(r))), "LSE"
    # sums over all keys, every head
    do_sum = case["do"].astype(np.float64).sum(axis=1)          # [B, H, Dv]
    dv_sum = gpu["dV"].sum(axis=1)
    scale = np.abs(gpu["dV"]).sum(axis=1) + 1.0
    assert np.max(np.abs(dv_sum - do_sum) / scale) < 1e-2
    dk_sum = gpu["dK"].sum(axis=1)
    scale = np.abs(gpu["dK"]).sum(axis=1) + 1.0
    assert np.max(np.abs(dk_sum) / scale) < 1e-2


def test_long_shard_dkdv_elementwise():
    """dK and dV of one head of the 18,900 x 75,600 shard, element by element.
    Without a mask every query row's softmax is independent of the others, so
    the oracle runs over disjoint chunks of query rows, each against all
    75,600 keys, and each chunk's contribution to dK and dV (sums over its
    rows) is added in fp64: that is the exact gradient, computed in pieces."""
    case = inputs.make_case("wan_cp_shard", 0)
    w = case["workload"]
    print(f"[parity] {w} dK/dV head 0, all keys", flush=True)
    gpu = G.numpy_out(G.run_gpu(case))
    head = 0
    dk = np.zeros((w.B, w.Skv, w.Dqk))
    dv = np.zeros((w.B, w.Skv, w.Dv))
    step = 1575
    import oracle
    for r0 in range(0, w.Sq, step):
        ref = oracle.backward(case["q"][:, r0:r0 + step], case["k"], case["v"], case["do"][:, r0:r0 + step],
                              causal=False, heads=[head])
        dk += ref["dK"][:, :, head]
        dv += ref["dV"][:, :, head]
    tol = G.TOL["bf16"]
    G.compare("dK", gpu["dK"][:, :, head], dk, tol)
    G.compare("dV", gpu["dV"][:, :, head], dv, tol)

"""GPU mask and segment logic, bit-exact against the oracle, and the
determinism of the gradients."""

import math

import numpy as np
import pytest

import oracle
from bwd_packed_segments_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _mask_cases():
    rng = np.random.default_rng(0)
    out = []
    # packed self-attention, fast route
    ids = np.array([[1] * 40 + [2] * 70 + [3] * 5 + [0] * 15, [5] * 60 + [9] * 70], dtype=np.int32)
    out.append(("packed_self", {"ids_q": ids, "pos_q": oracle.derive_pos(ids)}, 130, 130, True))
    out.append(("packed_self_nopos", {"ids_q": ids}, 130, 130, True))
    # unsorted ids / repeated id: general route
    ids2 = ids.copy()
    ids2[0, 120:125] = 1
    out.append(("repeated_id", {"ids_q": ids2}, 130, 130, True))
    # wrong positions: general
    pos = oracle.derive_pos(ids)
    pos[1, 10] += 1
    out.append(("bad_pos", {"ids_q": ids, "pos_q": pos}, 130, 130, True))
    # cross, rotated, unequal lengths
    w = inputs.workload("thd_cross_ring_4k", Sq=150, Skv=170, seg_lo=10, seg_hi=60, B=2)
    seg = inputs.segments_for(w, 3)
    out.append(("cross_rotated", seg, 150, 170, False))
    out.append(("cross_rotated_causal", seg, 150, 170, True))
    # equal-length cross with independent metadata
    w = inputs.workload("thd_cross_ring_4k", Sq=160, Skv=160, seg_lo=10, seg_hi=60, B=1)
    out.append(("cross_equal_len", inputs.segments_for(w, 4), 160, 160, True))
    # equal metadata passed as separate buffers: fast after the device compare
    out.append(("self_separate_buffers", {"ids_q": ids, "pos_q": pos * 0 + oracle.derive_pos(ids),
                                          "ids_kv": ids.copy(), "pos_kv": oracle.derive_pos(ids)}, 130, 130, True))
    # random ids, lots of zeros
    idr = rng.integers(0, 4, size=(2, 97)).astype(np.int32)
    out.append(("random_ids", {"ids_q": idr}, 97, 97, True))
    return out


MASK_CASES = _mask_cases()


@pytest.mark.parametrize("name,seg,Sq,Skv,causal", MASK_CASES, ids=[c[0] for c in MASK_CASES])
@pytest.mark.parametrize("force_general", [False, True])
def test_debug_mask_bit_exact(name, seg, Sq, Skv, causal, force_general):
    import bwd_packed_segments_amd as bps
    import torch
    print(f"[mask] {name} force_general={force_general}", flush=True)
    B = np.asarray(seg["ids_q"]).shape[0]
    flags = bps.ATTN_FORCE_GENERAL if force_general else 0
    mask, routes = bps.attn_debug_mask(B=B, Sq=Sq, Skv=Skv, causal=causal, segments=G.seg_to_dev(seg), flags=flags)
    torch.cuda.synchronize()
    mask = mask.cpu().numpy().astype(bool)
    res = oracle.resolve_segments(seg, B, Sq, Skv)
    for b in range(B):
        assert np.array_equal(mask[b], oracle.allowed_mask(b, Sq, Skv, causal, res)), f"row {b}"
    expect = oracle.fast_route_eligible(seg, B, Sq, Skv)
    if force_general:
        expect[:] = False
    assert np.array_equal(routes.cpu().numpy(), np.where(expect, 1, 2))


def _at_offset(x, off):
    """x as a contiguous int32 device tensor that starts `off` int32 past a
    16-byte boundary (a view into a larger buffer)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.int32)
    buf = torch.zeros(x.size + 4, dtype=torch.int32, device="cuda")
    assert buf.data_ptr() % 16 == 0
    v = buf[off:off + x.size].view(x.shape)
    v.copy_(torch.from_numpy(x).to("cuda"))
    return v


@pytest.mark.parametrize("off", [1, 2, 3])
@pytest.mark.parametrize("sep", [False, True])
def test_metadata_at_unaligned_addresses(off, sep):
    """Metadata tensors 4, 8 or 12 bytes past a 16-byte boundary: the metadata
    kernel reads and writes them element by element instead of 16 bytes at a
    time, and the mask and the routes are still the oracle's, bit for bit."""
    import bwd_packed_segments_amd as bps
    import torch
    w = inputs.workload("thd_packed_8k", B=2, S=1000, seg_lo=20, seg_hi=300)
    seg = inputs.segments_for(w, 6)
    if sep:   # equal metadata in separate KV buffers: fast after the device compare
        seg = {"ids_q": seg["ids_q"], "pos_q": seg["pos_q"], "ids_kv": seg["ids_q"].copy(),
               "pos_kv": seg["pos_q"].copy()}
    print(f"[mask] unaligned metadata off={off} sep={sep}", flush=True)
    dev = bps.Segments(*[None if seg.get(k) is None else _at_offset(seg[k], off)
                         for k in ("ids_q", "pos_q", "ids_kv", "pos_kv")])
    assert dev.ids_q.data_ptr() % 16 == 4 * off
    for causal in (True, False):
        mask, routes = bps.attn_debug_mask(B=2, Sq=1000, Skv=1000, causal=causal, segments=dev)
        torch.cuda.synchronize()
        res = oracle.resolve_segments(seg, 2, 1000, 1000)
        for b in range(2):
            ref = oracle.allowed_mask(b, 1000, 1000, causal, res)
            assert np.array_equal(mask[b].cpu().numpy().astype(bool), ref), f"row {b} causal={causal}"
        expect = oracle.fast_route_eligible(seg, 2, 1000, 1000)
        assert np.array_equal(routes.cpu().numpy(), np.where(expect, 1, 2))


def test_debug_mask_dense():
    import bwd_packed_segments_amd as bps
    import torch
    for causal, Sq, Skv in ((True, 77, 77), (False, 50, 90)):
        mask, routes = bps.attn_debug_mask(B=1, Sq=Sq, Skv=Skv, causal=causal)
        torch.cuda.synchronize()
        assert np.array_equal(mask.cpu().numpy()[0].astype(bool), oracle.allowed_mask(0, Sq, Skv, causal, None))
        assert int(routes.cpu()[0]) == 0


COUNT_CASES = [
    ("tiny_fp32", {}),
    ("bshd_causal_2k", {}),
    ("thd_packed_8k", {}),
    ("gqa_causal_8k", {"Hq": 8, "Hkv": 1}),
    ("thd_cross_ring_4k", {}),
    ("thd_cross_ring_4k", {"Sq": 1350, "Skv": 1777, "Hq": 4, "Hkv": 1, "causal": True}),
]


@pytest.mark.parametrize("name,over", COUNT_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(COUNT_CASES)])
def test_lse_counts_through_kernels(name, over):
    """With Q = 0 every allowed score is 0, so exp(LSE) is the number of keys
    a query attends: the allowed set of the real kernels, checked against the
    oracle's mask count for every query (and -inf exactly where it is 0)."""
    import torch
    w = inputs.workload(name, **over)
    case = inputs.make_case(w, 0, with_do=False)
    print(f"[count] {w}", flush=True)
    case["q"] = np.zeros_like(case["q"])
    gpu = G.run_gpu(case, bwd=False)
    lse = G.to_np(gpu["LSE"])
    res = oracle.resolve_segments(case["segments"], w.B, w.Sq, w.Skv)
    for b in range(w.B):
        n = oracle.allowed_mask(b, w.Sq, w.Skv, w.causal, res).sum(axis=1)
        for h in range(w.Hq):
            row = lse[b, h]
            assert np.array_equal(np.isneginf(row), n == 0)
            got = np.rint(np.exp(row[n > 0])).astype(np.int64)
            assert np.array_equal(got, n[n > 0]), f"row {b} head {h}"


def test_fast_equals_general_bitwise_full_size():
    """The packed workload at full size: the fast and the forced general
    route give bitwise identical O, LSE, dQ, dK, dV."""
    import torch
    case = inputs.make_case("thd_packed_8k", 1)
    print("[route] fast vs general", flush=True)
    a = G.run_gpu(case)
    b = G.run_gpu(case, flags=1)
    assert a["route"] == "fast" and b["route"] == "general"
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["gqa_causal_8k", "thd_cross_ring_4k", "thd_packed_8k"])
def test_deterministic_and_schedule_independent(name):
    """Gradients are bitwise identical across runs and under a reversed
    workgroup schedule (no atomics, fixed reduction order)."""
    import torch
    import bwd_packed_segments_amd as bps
    over = {"Hq": 16, "Hkv": 2} if name == "gqa_causal_8k" else {}
    case = inputs.make_case(inputs.workload(name, **over), 2)
    print(f"[determinism] {name}", flush=True)
    a = G.run_gpu(case)
    b = G.run_gpu(case)
    c = G.run_gpu(case, flags=bps.ATTN_REVERSE_SCHEDULE)
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        assert torch.equal(a[k], b[k]), f"repeat {k}"
        assert torch.equal(a[k], c[k]), f"reversed {k}"


def test_padding_garbage_isolation():
    """1000.0 in every padded token of Q, K, V and dO: valid outputs are
    bitwise unchanged and padded rows get exact zeros."""
    import torch
    case = inputs.make_case(inputs.workload("thd_packed_8k", B=2, S=1000, Hq=4, Hkv=4, seg_lo=50, seg_hi=400), 3)
    print("[garbage] padded tail = 1000", flush=True)
    pad = np.asarray(case["segments"]["ids_q"]) == 0
    assert pad.any()
    g = dict(case)
    for k in ("q", "k", "v", "do"):
        arr = np.array(case[k])
        arr[pad] = 1000.0
        g[k] = arr
    a = G.numpy_out(G.run_gpu(case))
    b = G.numpy_out(G.run_gpu(g))
    keep = ~pad
    for k in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(a[k][keep], b[k][keep]), k
        assert np.all(b[k][pad] == 0), k
    assert np.array_equal(a["LSE"].transpose(0, 2, 1)[keep], b["LSE"].transpose(0, 2, 1)[keep])


def test_dk_zero_sum_per_segment():
    """Softmax gradients sum to zero per query, so the GPU dK summed over
    each segment is ~0 (relative to its scale)."""
    case = inputs.make_case(inputs.workload("thd_packed_8k", B=1, S=2048, Hq=4, Hkv=4, seg_lo=100, seg_hi=900), 4)
    gpu = G.numpy_out(G.run_gpu(case))
    ids = np.asarray(case["segments"]["ids_q"])[0]
    for s in np.unique(ids[ids != 0]):
        idx = ids == s
        tot = gpu["dK"][0, idx].sum(axis=0)
        scale = np.abs(gpu["dK"][0, idx]).sum(axis=0) + 1e-6
        assert np.max(np.abs(tot) / scale) < 0.05


def _long_row_metadata():
    """Two rows of 8192 + 3000 tokens, longer than one 8192-token scan round
    of the metadata kernel.  Row 0: packed segments with one run straddling
    token 8192 (fast-route eligible).  Row 1: the same, but the id of an
    early run appears again after token 8192 (not eligible: the general
    route must take it)."""
    S = 8192 + 3000
    cuts = [0, 700, 2500, 2600, 5000, 7900, 8500, 9000, 10400, 11100]   # run [7900, 8500) straddles 8192
    ids = np.zeros((2, S), dtype=np.int32)
    for r, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        ids[:, a:b] = r + 1
    ids[:, 11100:] = 0                      # padded tail
    ids[1, 9000:9100] = 2                    # id 2 again, in the second round
    return S, {"ids_q": ids, "pos_q": oracle.derive_pos(ids)}


@pytest.mark.parametrize("causal", [True, False])
def test_long_rows_across_scan_rounds(causal):
    """Metadata rows longer than one scan round of the metadata kernel: the
    run bounds and summaries carried from one round to the next give the
    oracle's mask bit for bit, and each row takes the route the oracle's
    eligibility test names (fast for row 0, general for row 1)."""
    import bwd_packed_segments_amd as bps
    import torch
    S, seg = _long_row_metadata()
    print(f"[mask] long rows S={S} causal={causal}", flush=True)
    mask, routes = bps.attn_debug_mask(B=2, Sq=S, Skv=S, causal=causal, segments=G.seg_to_dev(seg))
    torch.cuda.synchronize()
    elig = oracle.fast_route_eligible(seg, 2, S, S)
    assert list(elig) == [True, False]
    assert routes.cpu().tolist() == [1, 2]
    rs = oracle.resolve_segments(seg, 2, S, S)
    for b in range(2):
        ref = oracle.allowed_mask(b, S, S, causal, rs)
        got = mask[b].cpu().numpy().astype(bool)
        assert np.array_equal(got, ref), f"row {b}: {np.count_nonzero(got != ref)} mask bits differ"


def _repeating_meta(S, period, n_ids):
    """Ids 1..n_ids, a new id every `period` tokens, repeating over the whole
    row (each id in many separate runs: general route); positions from the
    index."""
    idx = np.arange(S)
    ids = ((idx // period) % n_ids + 1).astype(np.int32)[None, :]
    return ids, idx.astype(np.int32)[None, :]


@pytest.mark.parametrize("Sq,Skv,Hq,Hkv", [(70_000, 512, 2, 1), (70_000, 512, 1, 1), (512, 70_000, 2, 1)],
                         ids=["long_q_gqa", "long_q", "long_kv"])
def test_walks_longer_than_class_table(Sq, Skv, Hq, Hkv):
    """Walks of more than 1024 tiles (the per-workgroup table of tile classes
    holds the first 1024; later tiles are classified on the fly): 70,000
    queries against 512 keys make the dK/dV walks that long, 512 queries
    against 70,000 keys the forward and dQ walks.  Cross-attention metadata
    whose ids repeat all along both rows (general route), non-causal, against
    the oracle.  The 70,000-token rows also span nine scan rounds of the
    metadata kernel."""
    w = inputs.workload("thd_cross_ring_4k", Sq=Sq, Skv=Skv, Hq=Hq, Hkv=Hkv, Dqk=64, Dv=64)
    case = inputs.make_case(w, 5)
    # 20 query ids against 5 key ids: each key is attended by one query in
    # twenty (about 7,000 terms per dK/dV element on the long query row,
    # whose ids 6..20 match nothing, so those tiles are skipped), which keeps
    # the reductions at the length of the workloads' own.
    iq, pq = _repeating_meta(Sq, 600, 20)
    ik, pk = _repeating_meta(Skv, 100, 5)
    case["segments"] = {"ids_q": iq, "pos_q": pq, "ids_kv": ik, "pos_kv": pk}
    print(f"[parity] long walks Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv}", flush=True)
    gpu = G.numpy_out(G.run_gpu(case))
    assert gpu["route"] == "general"
    ref = G.run_oracle(case)
    G.check_all(case, gpu, ref)


def test_log_route_reports_downgrades(capfd):
    """ATTN_LOG_ROUTE writes one stderr line per batch row that the device
    moved from the requested fast route to the general one (cross metadata
    that differ from Q's), in the forward and in the backward's prepare
    phase, and nothing for rows that keep the fast route (TransformerEngine
    PR 3516, review: a warning when the fast path is not taken)."""
    import torch
    import bwd_packed_segments_amd as bps
    cross = inputs.make_case(inputs.workload("thd_cross_ring_4k", B=2, Sq=600, Skv=600, Hq=2, Hkv=1, Dqk=64, Dv=64,
                                             seg_lo=50, seg_hi=300), 4)
    packed = inputs.make_case(inputs.workload("thd_packed_8k", B=2, S=600, Hq=2, Hkv=2, Dqk=64, Dv=64, seg_lo=50,
                                              seg_hi=300), 4)
    for name, case, expect_moved in (("cross", cross, None), ("packed", packed, 0)):
        print(f"[log route] {name}", flush=True)
        t = {k: G.to_dev(case[k], "bf16") for k in ("q", "k", "v", "do")}
        seg = G.seg_to_dev(case["segments"])
        capfd.readouterr()
        o, lse, req, rows = bps.attn_fwd(t["q"], t["k"], t["v"], causal=case["causal"], segments=seg,
                                         flags=bps.ATTN_LOG_ROUTE, return_route=True, return_route_rows=True)
        torch.cuda.synchronize()
        err_f = capfd.readouterr().err
        bps.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=case["causal"], segments=seg,
                     flags=bps.ATTN_LOG_ROUTE)
        torch.cuda.synchronize()
        err_b = capfd.readouterr().err
        moved = int((rows.cpu().numpy() == 2).sum())
        assert req == "fast"
        if expect_moved is not None:
            assert moved == expect_moved
        else:
            assert moved > 0
        for err, call in ((err_f, "forward"), (err_b, "backward")):
            lines = [l for l in err.splitlines() if "takes the general route" in l]
            assert len(lines) == moved, (call, err)
            assert all(f"bps_attn: {call}:" in l for l in lines), err

"""CPU checks that pin the fp64 oracle to the mathematics (no GPU needed)."""

import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_cases.txt")


# ---------------------------------------------------------------- golden masks

def _parse_golden():
    cases, derive, fast = [], {}, []
    cur = None
    with open(GOLDEN) as f:
        lines = [l.rstrip("\n") for l in f]
    i = 0
    while i < len(lines):
        line = lines[i].strip()
        i += 1
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            cur = {"name": line.split()[1]}
            cases.append(cur)
        elif line.startswith("derive "):
            _, key, *vals = line.split()
            derive[key] = np.array([int(x) for x in vals], dtype=np.int32)
        elif line.startswith("fast "):
            parts = [p.strip() for p in line.split("|")]
            flag = int(parts[0].split()[1])
            ids = np.array([int(x) for x in parts[1].split()[1:]], dtype=np.int32)
            pos = np.array([int(x) for x in parts[2].split()[1:]], dtype=np.int32)
            fast.append((flag, ids, pos))
        elif line == "mask":
            rows = []
            while i < len(lines) and lines[i].strip() and not lines[i].startswith("#"):
                rows.append([int(c) for c in lines[i].strip()])
                i += 1
            cur["mask"] = np.array(rows, dtype=bool)
        else:
            key, *vals = line.split()
            cur[key] = vals
    return cases, derive, fast


CASES, DERIVE, FAST = _parse_golden()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_mask(case):
    causal = bool(int(case["causal"][0]))
    mask = case["mask"]
    Sq, Skv = mask.shape
    if case["ids_q"] == ["none"]:
        seg = None
    else:
        ids_q = np.array([[int(x) for x in case["ids_q"]]], dtype=np.int32)
        pos_q = np.array([[int(x) for x in case["pos_q"]]], dtype=np.int32)
        if case["ids_kv"] == ["same"]:
            segments = {"ids_q": ids_q, "pos_q": pos_q}
        else:
            segments = {"ids_q": ids_q, "pos_q": pos_q,
                        "ids_kv": np.array([[int(x) for x in case["ids_kv"]]], dtype=np.int32),
                        "pos_kv": np.array([[int(x) for x in case["pos_kv"]]], dtype=np.int32)}
        seg = oa.resolve_segments(segments, 1, Sq, Skv)
    got = oa.allowed_mask(0, Sq, Skv, causal, seg)
    assert np.array_equal(got, mask)


def test_golden_derive_pos():
    assert np.array_equal(oa.derive_pos(DERIVE["ids"][None])[0], DERIVE["pos"])


@pytest.mark.parametrize("k", range(len(FAST)))
def test_golden_fast_route(k):
    flag, ids, pos = FAST[k]
    S = ids.size
    got = oa.fast_route_eligible({"ids_q": ids[None], "pos_q": pos[None]}, 1, S, S)
    assert bool(got[0]) == bool(flag)


def test_fast_route_needs_equal_metadata():
    ids = np.array([[1, 1, 2, 2]], dtype=np.int32)
    same_values = {"ids_q": ids, "pos_q": None, "ids_kv": ids.copy(), "pos_kv": None}
    assert oa.fast_route_eligible(same_values, 1, 4, 4)[0]
    other = {"ids_q": ids, "ids_kv": np.array([[1, 2, 2, 2]], dtype=np.int32)}
    assert not oa.fast_route_eligible(other, 1, 4, 4)[0]
    assert not oa.fast_route_eligible({"ids_q": ids, "ids_kv": np.ones((1, 5), np.int32)}, 1, 4, 5)[0]


def test_fast_route_mask_is_run_boundaries():
    """Where the fast route is eligible, the mask built from run boundaries
    alone (same run, and j <= i when causal) equals the id/pos mask."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        S = int(rng.integers(1, 40))
        ids = np.zeros(S, dtype=np.int32)
        i, sid = 0, 1
        while i < S:
            L = int(rng.integers(1, 8))
            if rng.random() < 0.3:
                ids[i:i + L] = 0
            else:
                ids[i:i + L] = sid
                sid += int(rng.integers(1, 3))
            i += L
        seg = {"ids_q": ids[None]}
        assert oa.fast_route_eligible(seg, 1, S, S)[0]
        res = oa.resolve_segments(seg, 1, S, S)
        start = np.zeros(S, int)
        end = np.zeros(S, int)
        for t in range(S):
            start[t] = t if t == 0 or ids[t] != ids[t - 1] else start[t - 1]
        for t in range(S - 1, -1, -1):
            end[t] = t + 1 if t == S - 1 or ids[t] != ids[t + 1] else end[t + 1]
        for causal in (False, True):
            m = oa.allowed_mask(0, S, S, causal, res)
            for a in range(S):
                for b in range(S):
                    expect = ids[a] != 0 and start[a] <= b < end[a] and (not causal or b <= a)
                    assert m[a, b] == expect


# --------------------------------------------------------------------- pins

def test_fd_causal_packed_padded():
    seg = P.seg_packed_padded()
    q, k, v, do = P.rng_arrays(1, 2, 10, 10, 2, 1, 6, 4)
    assert P.pin_finite_differences(q, k, v, do, causal=True, segments=seg) < 1e-6


def test_fd_cross_rotated_gqa_unequal_dims():
    seg = P.seg_cross_rotated()
    q, k, v, do = P.rng_arrays(2, 1, 10, 11, 4, 2, 6, 5)
    assert P.pin_finite_differences(q, k, v, do, causal=False, segments=seg) < 1e-6
    assert P.pin_finite_differences(q, k, v, do, causal=True, segments=seg) < 1e-6


def test_fd_plain():
    q, k, v, do = P.rng_arrays(3, 1, 7, 7, 2, 2, 4, 3)
    assert P.pin_finite_differences(q, k, v, do, causal=False) < 1e-6
    assert P.pin_finite_differences(q, k, v, do, causal=True) < 1e-6


def test_fd_nondefault_scale():
    q, k, v, do = P.rng_arrays(4, 1, 6, 8, 2, 1, 4, 3)
    assert P.pin_finite_differences(q, k, v, do, causal=False, scale=0.37) < 1e-6


@pytest.mark.parametrize("which", ["plain_causal", "packed", "cross"])
def test_dv_is_pt_do(which):
    if which == "plain_causal":
        q, k, v, do = P.rng_arrays(0, 2, 9, 9, 4, 2, 5, 3)
        assert P.pin_dv_is_pt_do(q, k, v, do, causal=True) < 1e-12
    elif which == "packed":
        q, k, v, do = P.rng_arrays(0, 2, 10, 10, 4, 2, 5, 3)
        assert P.pin_dv_is_pt_do(q, k, v, do, causal=True, segments=P.seg_packed_padded()) < 1e-12
    else:
        q, k, v, do = P.rng_arrays(0, 1, 10, 11, 4, 1, 5, 3)
        assert P.pin_dv_is_pt_do(q, k, v, do, causal=False, segments=P.seg_cross_rotated()) < 1e-12


def test_row_sums():
    q, k, _, _ = P.rng_arrays(0, 2, 10, 10, 2, 1, 6, 4)
    assert P.pin_row_sums(q, k, causal=True, segments=P.seg_packed_padded()) < 1e-12
    q, k, _, _ = P.rng_arrays(0, 1, 10, 11, 2, 1, 6, 4)
    assert P.pin_row_sums(q, k, causal=False, segments=P.seg_cross_rotated()) < 1e-12


def test_delta_identity():
    q, k, v, do = P.rng_arrays(0, 2, 10, 10, 2, 1, 6, 4)
    assert P.pin_delta_identity(q, k, v, do, causal=True, segments=P.seg_packed_padded()) < 1e-12


def test_dk_zero_sum():
    q, k, v, do = P.rng_arrays(0, 2, 10, 10, 4, 2, 6, 4)
    assert P.pin_dk_zero_sum(q, k, v, do, causal=True, segments=P.seg_packed_padded()) < 1e-12
    q, k, v, do = P.rng_arrays(1, 1, 9, 9, 2, 2, 6, 4)
    assert P.pin_dk_zero_sum(q, k, v, do, causal=True, segments=None) < 1e-12


def test_closed_forms():
    assert P.pin_closed_forms() < 1e-12


def test_packed_equals_separate():
    assert P.pin_packed_equals_separate() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha(causal):
    assert P.pin_gqa_equals_mha(causal=causal) < 1e-12
    ids = np.array([[1, 1, 1, 2, 2, 2, 2, 0, 0]], dtype=np.int32)
    assert P.pin_gqa_equals_mha(causal=causal, segments={"ids_q": ids}) < 1e-12


def test_padding_garbage():
    assert P.pin_padding_garbage() == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_kv_permutation(causal):
    assert P.pin_kv_permutation(causal=causal) < 1e-12


def test_shard_merge():
    assert P.pin_shard_merge() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa(causal):
    assert P.pin_torch_sdpa(causal=causal) < 1e-12
    assert P.pin_torch_sdpa(causal=False, Sq=5, Skv=9) < 1e-12
    ids = np.array([[1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 3]], dtype=np.int32)
    assert P.pin_torch_sdpa(causal=causal, segments={"ids_q": ids}) < 1e-12


def test_empty_rows_and_empty_kv():
    """A query with no keys gets O = 0, LSE = -inf, dQ = 0; an empty key
    sequence makes every row empty."""
    seg = P.seg_cross_rotated()
    q, k, v, do = P.rng_arrays(0, 1, 10, 11, 2, 1, 6, 5)
    f = oracle.forward(q, k, v, causal=False, segments=seg)
    g = oracle.backward(q, k, v, do, causal=False, segments=seg)
    empty = f["count"][0] == 0
    assert empty.any()
    assert np.all(f["O"][0, empty] == 0) and np.all(f["LSE"][0][:, empty] == -np.inf)
    assert np.all(g["dQ"][0, empty] == 0)
    unattended = ~oa.allowed_mask(0, 10, 11, False, oa.resolve_segments(seg, 1, 10, 11)).any(axis=0)
    assert unattended.any()
    assert np.all(g["dK"][0, unattended] == 0) and np.all(g["dV"][0, unattended] == 0)
    f0 = oracle.forward(q, k[:, :0], v[:, :0], causal=False)
    assert np.all(f0["O"] == 0) and np.all(f0["LSE"] == -np.inf)


def test_head_subset_matches_full():
    q, k, v, do = P.rng_arrays(0, 1, 9, 9, 4, 2, 5, 3)
    full = oracle.backward(q, k, v, do, causal=True)
    part = oracle.backward(q, k, v, do, causal=True, heads=[2, 3])
    assert np.array_equal(part["dQ"][:, :, 2:], full["dQ"][:, :, 2:])
    assert np.array_equal(part["dK"][:, :, 1], full["dK"][:, :, 1])
    assert np.all(np.isnan(part["dK"][:, :, 0]))


def test_oracle_input_validation():
    q, k, v, do = P.rng_arrays(0, 1, 4, 5, 2, 1, 4, 3)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, causal=True)          # causal needs Sq == Skv
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, causal=False, segments={"ids_q": np.ones((1, 4), np.int32)})
    with pytest.raises(ValueError):
        oracle.forward(q, k[:, :, :0], v[:, :, :0], causal=False)

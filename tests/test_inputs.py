"""The seeded input generators: seed required, deterministic, and the
segment recipes hold the properties the workloads state."""

import numpy as np
import pytest
import torch

from bwd_packed_segments_amd import inputs


def test_seed_required():
    with pytest.raises(ValueError):
        inputs.make_case("tiny_fp32", None)


def test_deterministic_and_seed_sensitive():
    a = inputs.make_case(inputs.workload("thd_packed_8k", S=512, Hq=2, Hkv=2, seg_lo=16, seg_hi=200), 3)
    b = inputs.make_case(inputs.workload("thd_packed_8k", S=512, Hq=2, Hkv=2, seg_lo=16, seg_hi=200), 3)
    c = inputs.make_case(inputs.workload("thd_packed_8k", S=512, Hq=2, Hkv=2, seg_lo=16, seg_hi=200), 4)
    for key in ("q", "k", "v", "do"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert np.array_equal(a["segments"]["ids_q"], b["segments"]["ids_q"])
    # dO is a nonuniform draw, not a constant
    assert np.std(a["do"]) > 0.5


def test_bf16_round_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    ours = inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_packed_recipe():
    w = inputs.WORKLOADS["thd_packed_8k"]
    for seed in range(5):
        seg = inputs.segments_for(w, seed)
        ids, pos = seg["ids_q"], seg["pos_q"]
        assert ids.shape == (2, 8192)
        for b in range(2):
            assert ids[b, -1] == 0                      # padded tail of at least one token
            nz = ids[b][ids[b] != 0]
            sids = np.unique(nz)
            assert np.array_equal(sids, np.arange(1, sids.size + 1))
            for s in sids:
                idx = np.nonzero(ids[b] == s)[0]
                assert idx[-1] - idx[0] + 1 == idx.size   # contiguous
                assert 128 <= idx.size <= 4096
                assert np.array_equal(pos[b, idx], np.arange(idx.size))
            tail = np.nonzero(ids[b] == 0)[0]
            assert tail[0] == nz.size and np.all(pos[b, tail] == 0)


def test_cross_recipe():
    w = inputs.WORKLOADS["thd_cross_ring_4k"]
    for seed in range(5):
        seg = inputs.segments_for(w, seed)
        assert np.all(seg["ids_q"] != 0) and np.all(seg["ids_kv"] != 0)     # no padding
        # the rotation splits one KV segment across the row's wrap
        ids = seg["ids_kv"][0]
        assert ids[0] == ids[-1]
        runs = 1 + np.count_nonzero(ids[1:] != ids[:-1])
        assert runs == np.unique(ids).size + 1
        for s in np.unique(seg["ids_q"][0])[:-1]:
            n = np.count_nonzero(seg["ids_q"][0] == s)
            assert 256 <= n <= 2048


def test_workload_table():
    w = inputs.WORKLOADS
    assert (w["gqa_causal_8k"].Hq, w["gqa_causal_8k"].Hkv, w["gqa_causal_8k"].Sq) == (64, 8, 8192)
    assert (w["thd_cross_ring_4k"].Dqk, w["thd_cross_ring_4k"].Dv) == (192, 128)
    assert w["tiny_fp32"].dtype == "fp32"
    assert inputs.workload("gqa_causal_8k", S=300).Skv == 300

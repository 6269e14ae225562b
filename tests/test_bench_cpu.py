"""bench.py's host-side accounting: allowed-pair counts against the oracle's
mask, FLOP formulas, and the single-GPU guard."""

import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from bwd_packed_segments_amd import inputs

CASES = [
    ("thd_packed_8k", dict(S=600, seg_lo=20, seg_hi=200)),
    ("thd_cross_ring_4k", dict(Sq=300, Skv=340, seg_lo=20, seg_hi=100)),
    ("thd_cross_ring_4k", dict(Sq=300, Skv=300, seg_lo=20, seg_hi=100, causal=True)),
    ("gqa_causal_8k", dict(S=100, Hq=4, Hkv=1)),
    ("bshd_causal_2k", dict(B=1, Sq=50, Skv=70, causal=False)),
]


@pytest.mark.parametrize("name,over", CASES)
def test_allowed_pairs_match_oracle_mask(name, over):
    w = inputs.workload(name, **over)
    c = inputs.make_case(w, 1, with_do=False)
    f = oracle.forward(c["q"][:, :, :1], c["k"][:, :, :1], c["v"][:, :, :1], causal=w.causal,
                       segments=c["segments"])
    assert bench.allowed_pairs(w, c["segments"]) == int(f["count"].sum()) * w.Hq


def test_flops_gqa_8k():
    w = inputs.WORKLOADS["gqa_causal_8k"]
    n = bench.allowed_pairs(w, None)
    assert n == 64 * 8192 * 8193 // 2
    F = bench.flops(w, n)
    assert abs((F["fwd"] + F["bwd"]) / 1e12 - 3.8488) < 1e-3
    assert F["k_fwd"] + F["k_dkdv"] + F["k_dq"] == 2.0 * n * (5 * 128 + 4 * 128)


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_functions_name_only_defined_globals():
    """Every global name a function in bench.py reads is bound at module
    level or is a builtin (a name left over from another function's body
    would only fail on the GPU, in the middle of a run)."""
    import builtins
    import symtable
    with open(bench.__file__) as f:
        table = symtable.symtable(f.read(), bench.__file__, "exec")
    known = set(vars(bench)) | set(dir(builtins))
    missing = []

    def walk(t):
        if t.get_type() == "function":
            for s in t.get_symbols():
                if s.is_referenced() and s.is_global() and s.get_name() not in known:
                    missing.append(f"{t.get_name()}: {s.get_name()}")
        for c in t.get_children():
            walk(c)
    walk(table)
    assert not missing, missing

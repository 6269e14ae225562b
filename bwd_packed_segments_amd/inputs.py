"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws tensors and segment
metadata.  Both the fp64 oracle and the HIP path receive exactly the arrays
made here (bf16 workloads are drawn in fp32 and rounded once to bf16, so the
oracle sees the very values the GPU reads).

Workloads (sizes as the pages' discussion and the benchmark contract set
them; every one is synthetic, iid N(0, 1) tensors):

  tiny_fp32          B=1, H=1, S=128, D=64, fp32, no mask
  bshd_causal_2k     B=2, Hq=Hkv=16, S=2048, D=128, bf16, causal
  thd_packed_8k      2 rows x 8192 tokens, H=32, D=128, bf16, causal inside
                     segments; segment lengths uniform in [128, 4096] with a
                     padded tail (id 0)
  gqa_causal_8k      B=1, Hq=64, Hkv=8, S=8192, D=128, bf16, causal
  thd_cross_ring_4k  4096 Q and 4096 KV tokens, Hq=32, Hkv=8, Dqk=192,
                     Dv=128, bf16, non-causal; independent Q and KV
                     segmentations (lengths uniform in [256, 2048]), the KV
                     one rotated by a random offset like a ring-attention
                     step

Seeds: each tensor comes from its own stream,
numpy.random.default_rng([seed, k]) with k = 0 (Q), 1 (K), 2 (V), 3 (dO),
4 (Q metadata), 5 (KV metadata), 6 (rotation).  A seed is required: the
output gradient must be a deterministic nonuniform draw ("[JAX] Align fused
attn backward output gradient sharding ...", Changes 2 and 5.1: uniform
output gradients hide permutation errors, and the runner rejects a missing
seed).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    Skv: int
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    dtype: str            # "bf16" or "fp32"
    causal: bool
    meta: str             # "none", "packed_self" or "cross_rotated"
    seg_lo: int = 0       # segment length range (inclusive)
    seg_hi: int = 0

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 128, 128, 1, 1, 64, 64, "fp32", False, "none"),
    "bshd_causal_2k": Workload("bshd_causal_2k", 2, 2048, 2048, 16, 16, 128, 128, "bf16", True, "none"),
    "thd_packed_8k": Workload("thd_packed_8k", 2, 8192, 8192, 32, 32, 128, 128, "bf16", True,
                              "packed_self", 128, 4096),
    "gqa_causal_8k": Workload("gqa_causal_8k", 1, 8192, 8192, 64, 8, 128, 128, "bf16", True, "none"),
    "thd_cross_ring_4k": Workload("thd_cross_ring_4k", 1, 4096, 4096, 32, 8, 192, 128, "bf16", False,
                                  "cross_rotated", 256, 2048),
    # One context-parallel shard of the long-sequence benchmark on the
    # maxdiffusion ring-attention page (75,600 tokens, 40 heads, head dim
    # 128, four shards): the local 18,900 queries against all 75,600 keys,
    # non-causal, no padding mask.
    "wan_cp_shard": Workload("wan_cp_shard", 1, 18900, 75600, 40, 40, 128, 128, "bf16", False, "none"),
    # The whole 75,600-token sequence of that benchmark (for the one-GPU
    # ring emulation with four shards of 18,900 tokens).
    "wan_full_76k": Workload("wan_full_76k", 1, 75600, 75600, 40, 40, 128, 128, "bf16", False, "none"),
}

# Order of the workloads as the benchmark contract lists them.
WORKLOAD_ORDER = ["tiny_fp32", "bshd_causal_2k", "thd_packed_8k", "gqa_causal_8k", "thd_cross_ring_4k"]


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with some fields replaced (smaller
    shapes for parity tests that the oracle finishes in seconds)."""
    w = WORKLOADS[name]
    if "S" in overrides:
        s = overrides.pop("S")
        overrides.setdefault("Sq", s)
        overrides.setdefault("Skv", s)
    return dataclasses.replace(w, **overrides)


def _stream(seed: int, k: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(k)])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and
    return them as float32.  Inputs are finite draws, so no NaN care."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def normal(seed: int, k: int, shape, dtype: str) -> np.ndarray:
    a = _stream(seed, k).standard_normal(size=shape, dtype=np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def packed_rows(rng: np.random.Generator, B: int, S: int, lo: int, hi: int):
    """Rows of S tokens cut into segments with lengths uniform in [lo, hi];
    segments are added while they fit with at least one token to spare, and
    the rest of the row is a padded tail (id 0, pos 0).  Ids count 1, 2, ...
    per row; pos restarts at 0 in every segment."""
    ids = np.zeros((B, S), dtype=np.int32)
    pos = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        cum, sid = 0, 1
        while True:
            L = int(rng.integers(lo, hi + 1))
            if cum + L >= S:
                break
            ids[b, cum:cum + L] = sid
            pos[b, cum:cum + L] = np.arange(L, dtype=np.int32)
            cum += L
            sid += 1
    return ids, pos


def exact_rows(rng: np.random.Generator, B: int, S: int, lo: int, hi: int):
    """Rows of S tokens cut into segments with lengths uniform in [lo, hi],
    the last one truncated so the row is exactly full (no padding)."""
    ids = np.zeros((B, S), dtype=np.int32)
    pos = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        cum, sid = 0, 1
        while cum < S:
            L = min(int(rng.integers(lo, hi + 1)), S - cum)
            ids[b, cum:cum + L] = sid
            pos[b, cum:cum + L] = np.arange(L, dtype=np.int32)
            cum += L
            sid += 1
    return ids, pos


def segments_for(w: Workload, seed: int):
    """Segment metadata of a workload (None for plain BSHD)."""
    if w.meta == "none":
        return None
    if w.meta == "packed_self":
        ids, pos = packed_rows(_stream(seed, 4), w.B, w.Sq, w.seg_lo, w.seg_hi)
        return {"ids_q": ids, "pos_q": pos, "ids_kv": None, "pos_kv": None}
    if w.meta == "cross_rotated":
        ids_q, pos_q = exact_rows(_stream(seed, 4), w.B, w.Sq, w.seg_lo, w.seg_hi)
        ids_kv, pos_kv = exact_rows(_stream(seed, 5), w.B, w.Skv, w.seg_lo, w.seg_hi)
        rot = _stream(seed, 6)
        for b in range(w.B):
            r = int(rot.integers(1, max(w.Skv, 2)))
            ids_kv[b] = np.roll(ids_kv[b], r)
            pos_kv[b] = np.roll(pos_kv[b], r)
        return {"ids_q": ids_q, "pos_q": pos_q, "ids_kv": ids_kv, "pos_kv": pos_kv}
    raise ValueError(f"unknown metadata recipe {w.meta!r}")


def make_case(w, seed, *, with_do: bool = True):
    """All inputs of one workload instance.

    Returns a dict: q [B,Sq,Hq,Dqk], k [B,Skv,Hkv,Dqk], v [B,Skv,Hkv,Dv],
    do [B,Sq,Hq,Dv] (float32 arrays holding bf16-exact values for bf16
    workloads), segments (dict or None), causal, dtype, workload.
    """
    if seed is None:
        raise ValueError("a seed is required (inputs must be reproducible)")
    if isinstance(w, str):
        w = WORKLOADS[w]
    case = {
        "q": normal(seed, 0, (w.B, w.Sq, w.Hq, w.Dqk), w.dtype),
        "k": normal(seed, 1, (w.B, w.Skv, w.Hkv, w.Dqk), w.dtype),
        "v": normal(seed, 2, (w.B, w.Skv, w.Hkv, w.Dv), w.dtype),
        "segments": segments_for(w, seed),
        "causal": w.causal,
        "dtype": w.dtype,
        "workload": w,
        "seed": seed,
    }
    if with_do:
        case["do"] = normal(seed, 3, (w.B, w.Sq, w.Hq, w.Dv), w.dtype)
    return case


def variant_inputs(w, seed, *, bias_batch=None, bias_scale=1.0, bias_neg_inf=0.0, sink=False, sink_scale=1.0):
    """Seeded inputs of the attention variants for workload w: an additive
    bias [bias_batch, Hq, Sq, Skv] (None when bias_batch is None) drawn from
    N(0, bias_scale^2), rounded to the workload's dtype, with a fraction
    bias_neg_inf of its entries set to -inf; sink logits [Hq] (fp32, None
    unless sink) drawn from N(0, sink_scale^2).  Streams 7, 8 and 9 of the
    seed, apart from those of make_case."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    out = {"bias": None, "sink": None}
    if bias_batch is not None:
        bias = normal(seed, 7, (bias_batch, w.Hq, w.Sq, w.Skv), "fp32") * np.float32(bias_scale)
        if w.dtype == "bf16":
            bias = bf16_round(bias)
        if bias_neg_inf > 0:
            bias[_stream(seed, 9).random(bias.shape) < bias_neg_inf] = -np.inf
        out["bias"] = bias
    if sink:
        out["sink"] = normal(seed, 8, (w.Hq,), "fp32") * np.float32(sink_scale)
    return out

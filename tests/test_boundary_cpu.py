"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host validation rejects bad arguments before any HIP call
(so these run without a GPU; nothing here launches a kernel)."""

import ctypes
import os
import re

import pytest

import bwd_packed_segments_amd as bps
from bwd_packed_segments_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bps_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.library_path()),
                                reason="libbps_attn.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = B.lib()
    declared = header_functions()
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_error_string():
    L = B.lib()
    assert b"gfx950" in L.attn_version()
    assert isinstance(L.attn_last_error(), bytes)


def good(**kw):
    base = dict(B=2, Sq=300, Skv=300, Hq=4, Hkv=2, Dqk=128, Dv=128, causal=True)
    base.update(kw)
    return B.make_desc(**base)


def test_workspace_sizes():
    d = good()
    assert B.fwd_workspace_size(d) == 0                       # no metadata: no workspace
    assert B.bwd_workspace_size(d) >= 2 * 2 * 4 * 300 * 4      # delta + lse2
    seg = B.attn_segments(0x1000, None, None, None)
    assert B.fwd_workspace_size(d, seg) > 0
    seg2 = B.attn_segments(0x1000, 0x2000, 0x3000, 0x4000)
    assert B.fwd_workspace_size(d, seg2) > B.fwd_workspace_size(d, B.attn_segments(0x1000, 0x2000, None, None))
    bad = good(Hq=3)
    assert B.fwd_workspace_size(bad) == 0


CASES = [
    ("hq_not_multiple", dict(Hq=6, Hkv=4), None, B.ATTN_E_INVALID, "multiple"),
    ("zero_heads", dict(Hkv=0), None, B.ATTN_E_INVALID, "positive"),
    ("neg_len", dict(Sq=-1), None, B.ATTN_E_INVALID, "positive"),
    ("dims", dict(Dqk=96), None, B.ATTN_E_UNSUPPORTED, "head dims"),
    ("dims_fp32_192", dict(Dqk=192, dtype=B.ATTN_FP32), None, B.ATTN_E_UNSUPPORTED, "head dims"),
    ("dtype", dict(dtype=7), None, B.ATTN_E_INVALID, "dtype"),
    ("causal_value", dict(causal=True), None, None, None),
    ("causal_unequal_nometa", dict(Skv=200), None, B.ATTN_E_UNSUPPORTED, "Sq == Skv"),
    ("scale_nan", dict(scale=float("nan")), None, B.ATTN_E_INVALID, "scale"),
    ("scale_neg", dict(scale=-1.0), None, B.ATTN_E_INVALID, "scale"),
    ("flags", dict(flags=1 << 7), None, B.ATTN_E_INVALID, "flag"),
    ("stride_align", dict(q=(300 * 4 * 128, 4 * 128, 124)), None, B.ATTN_E_UNSUPPORTED, "multiples"),
    ("stride_neg", dict(k=(-1, 256, 128)), None, B.ATTN_E_INVALID, "non-negative"),
    ("meta_no_ids", dict(), B.attn_segments(None, 0x1000, None, None), B.ATTN_E_INVALID, "ids_q"),
    ("meta_pos_kv_alone", dict(), B.attn_segments(0x1000, None, None, 0x2000), B.ATTN_E_INVALID, "pairs"),
    ("meta_self_unequal", dict(Skv=200), B.attn_segments(0x1000, None, None, None), B.ATTN_E_INVALID, "Sq == Skv"),
]


@pytest.mark.parametrize("name,kw,seg,status,msg", CASES, ids=[c[0] for c in CASES])
def test_validation(name, kw, seg, status, msg):
    d = good(**kw)
    if status is None:
        d.causal = 2
        status, msg = B.ATTN_E_INVALID, "causal"
    st, text = B.validate_fwd(d, seg)
    assert st == status, text
    assert msg in text
    st, text = B.validate_bwd(d, seg)
    assert st == status, text


def test_null_pointers_rejected():
    st, text = B.validate_fwd(good(), q=None)
    assert st == B.ATTN_E_INVALID and "NULL" in text
    st, text = B.validate_bwd(good(), dq=None)
    assert st == B.ATTN_E_INVALID and "NULL" in text


def test_misaligned_pointer_rejected():
    st, text = B.validate_fwd(good(), q=(1 << 12) + 2)
    assert st == B.ATTN_E_UNSUPPORTED and "aligned" in text


def test_workspace_checks():
    seg = B.attn_segments(0x1000, None, None, None)
    d = good()
    need = B.fwd_workspace_size(d, seg)
    st, text = B.validate_fwd(d, seg, ws=1 << 20, ws_bytes=need - 1)
    assert st == B.ATTN_E_WORKSPACE and "smaller" in text
    st, text = B.validate_fwd(d, seg, ws=None, ws_bytes=need)
    assert st == B.ATTN_E_WORKSPACE and "NULL" in text
    st, text = B.validate_fwd(d, seg, ws=(1 << 20) + 64, ws_bytes=need)
    assert st == B.ATTN_E_WORKSPACE and "aligned" in text
    st, text = B.validate_bwd(d, seg, ws=1 << 20, ws_bytes=B.bwd_workspace_size(d, seg) - 1)
    assert st == B.ATTN_E_WORKSPACE


def test_null_desc():
    L = B.lib()
    st = L.attn_fwd(None, None, 1, 1, 1, 1, 1, None, 0, None, None)
    assert st == B.ATTN_E_INVALID
    assert L.attn_fwd_workspace_size(None, None) == 0


def test_error_is_thread_local():
    import threading
    B.validate_fwd(good(Hq=6, Hkv=4))
    seen = {}

    def other():
        seen["msg"] = B.lib().attn_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == b""
    assert b"multiple" in B.lib().attn_last_error()


def test_product_path_has_no_oracle_import():
    """The binding and the package never import the oracle (test-only)."""
    pkg = os.path.join(ROOT, "bwd_packed_segments_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py") and fn != "inputs.py":
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle)", ""), fn


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setenv("BPS_ATTN_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        B.lib()
    monkeypatch.setattr(B, "_lib", None)


def test_ring_validation():
    d = good(Sq=300, Skv=300)
    st, text = B.validate_ring_fwd(d, None, 0)
    assert st == B.ATTN_E_INVALID and "cp" in text
    st, text = B.validate_ring_fwd(d, None, 7)
    assert st == B.ATTN_E_INVALID and "multiples of cp" in text
    st, text = B.validate_ring_fwd(good(Hq=6, Hkv=4), None, 2)        # descriptor errors come first
    assert st == B.ATTN_E_INVALID and "multiple" in text
    st, text = B.validate_ring_fwd(good(Skv=200), None, 2)            # causal without metadata needs Sq == Skv
    assert st == B.ATTN_E_UNSUPPORTED
    fwd, bwd = B.ring_workspace_sizes(d, None, 3)
    st, text = B.validate_ring_fwd(d, None, 3, ws=1 << 20, ws_bytes=fwd - 1)
    assert st == B.ATTN_E_WORKSPACE and "smaller" in text


def test_ring_workspace_sizes():
    d = good(Sq=600, Skv=600)
    f1, b1 = B.ring_workspace_sizes(d, None, 1)
    f3, b3 = B.ring_workspace_sizes(d, None, 3)
    assert f1 > 0 and b1 > 0
    # cp partial copies of O (forward) or of dQ, dK, dV (backward)
    o_bytes = 2 * 600 * 4 * 128 * 2
    qkv_bytes = (2 * 600 * 4 * 128 + 2 * 2 * 600 * 2 * 128) * 2
    assert f1 >= o_bytes and f3 >= 3 * o_bytes
    assert b1 >= qkv_bytes and b3 >= 3 * qkv_bytes
    assert B.ring_workspace_sizes(d, None, 7) == (0, 0)


def _var(**kw):
    f = dict(bias=None, bias_batch=1, softcap=0.0, sink=None, max_logit=None, dbias=None, dsink=None)
    f.update(kw)
    return B.attn_variant(f["bias"], f["bias_batch"], f["softcap"], f["sink"], f["max_logit"], f["dbias"],
                          f["dsink"])


def test_variant_validation():
    d = good()                                   # B = 2
    ptr = 1 << 12
    cases = [
        (_var(bias=ptr, bias_batch=3), False, B.ATTN_E_INVALID, "bias_batch"),
        (_var(bias=ptr, bias_batch=0), False, B.ATTN_E_INVALID, "bias_batch"),
        (_var(softcap=-1.0), False, B.ATTN_E_INVALID, "softcap"),
        (_var(softcap=float("inf")), False, B.ATTN_E_INVALID, "softcap"),
        (_var(softcap=float("nan")), False, B.ATTN_E_INVALID, "softcap"),
        (_var(dbias=ptr), True, B.ATTN_E_INVALID, "dbias"),
        (_var(dsink=ptr), True, B.ATTN_E_INVALID, "dsink"),
        (_var(bias=ptr + 2), False, B.ATTN_E_UNSUPPORTED, "aligned"),
        (_var(bias=ptr, dbias=ptr + 8), True, B.ATTN_E_UNSUPPORTED, "aligned"),
        (_var(sink=ptr + 2), False, B.ATTN_E_INVALID, "aligned"),
    ]
    for var, bwd, status, word in cases:
        st, text = B.validate_ex(d, var, bwd=bwd)
        assert st == status and word in text, (st, text)
    # descriptor errors come first, and a too-small workspace is refused
    st, text = B.validate_ex(good(Hq=6, Hkv=4), _var(softcap=1.0))
    assert st == B.ATTN_E_INVALID and "multiple" in text
    fwd, _ = B.ex_workspace_sizes(d, _var(max_logit=ptr))
    st, text = B.validate_ex(d, _var(max_logit=ptr), ws=1 << 20, ws_bytes=fwd - 1)
    assert st == B.ATTN_E_WORKSPACE


def test_variant_workspace_sizes():
    d = good(B=2, Sq=300, Skv=300, Hq=4, Hkv=2)
    plain = (B.fwd_workspace_size(d), B.bwd_workspace_size(d))
    ptr = 1 << 12
    assert B.ex_workspace_sizes(d, None) == plain
    assert B.ex_workspace_sizes(d, _var()) == plain
    assert B.ex_workspace_sizes(d, _var(softcap=2.0, sink=ptr, bias=ptr, bias_batch=2)) == plain
    f, b = B.ex_workspace_sizes(d, _var(max_logit=ptr))
    assert f >= plain[0] + 4 * 2 * 3 * 4 * 4 and b == plain[1]        # [Hq][B][3 query tiles][4 waves] fp32
    f, b = B.ex_workspace_sizes(d, _var(sink=ptr, dsink=ptr))
    assert f == plain[0] and b >= plain[1] + 2 * 4 * 300 * 4          # one fp32 term per row
    f, b = B.ex_workspace_sizes(d, _var(bias=ptr, bias_batch=1, dbias=ptr))
    assert b >= plain[1] + 2 * 4 * 300 * 300 * 4                     # fp32 partials per batch row
    f, b = B.ex_workspace_sizes(d, _var(bias=ptr, bias_batch=2, dbias=ptr))
    assert b == plain[1]                                              # written in place
    assert B.ex_workspace_sizes(d, _var(softcap=-1.0)) == (0, 0)


def test_fused_bwd_validation_and_workspace():
    F = B.ATTN_FUSED_BWD
    d = good(B=2, Sq=300, Skv=260, Hq=4, Hkv=2, Dqk=128, Dv=64, causal=False)
    plain = B.bwd_workspace_size(d)
    fused = B.bwd_workspace_size(good(B=2, Sq=300, Skv=260, Hq=4, Hkv=2, Dqk=128, Dv=64, causal=False, flags=F))
    # one fp32 partial of 32 queries x Dqk per (row, head, key tile of 128, query block of 32),
    # query blocks padded to whole 64-row tiles: 3 key tiles, 10 query blocks
    assert fused >= plain + 2 * 4 * 3 * 10 * 32 * 128 * 4
    assert fused < plain + 2 * 4 * 3 * 10 * 32 * 128 * 4 + 512
    assert B.fwd_workspace_size(good(flags=F)) == B.fwd_workspace_size(good())   # the forward ignores it
    for kw, word in ((dict(dtype=B.ATTN_FP32, Dqk=64, Dv=64), "bf16"), (dict(Dqk=192), "Dqk")):
        st, text = B.validate_bwd(good(flags=F, **kw))
        assert st == B.ATTN_E_UNSUPPORTED and word in text, (st, text)
        assert B.bwd_workspace_size(good(flags=F, **kw)) == 0
    # no bias or soft cap in the fused form; a sink (read through the LSE) is fine
    ptr = 1 << 12
    st, text = B.validate_ex(good(flags=F), _var(softcap=2.0), bwd=True)
    assert st == B.ATTN_E_UNSUPPORTED and "fused" in text
    st, text = B.validate_ex(good(flags=F), _var(bias=ptr, bias_batch=2), bwd=True)
    assert st == B.ATTN_E_UNSUPPORTED and "fused" in text
    assert B.ex_workspace_sizes(good(flags=F), _var(sink=ptr))[1] == B.bwd_workspace_size(good(flags=F))
    st, text = B.validate_ring_fwd(good(flags=F), None, 2)
    assert st == B.ATTN_E_UNSUPPORTED and "ring" in text
    st, text = B.validate_bwd(good(flags=1 << 4))
    assert st == B.ATTN_E_INVALID and "flag" in text


def test_split_dkdv_workspace():
    """bf16 dK/dV grids of fewer than 512 key tiles split each key tile's
    walk (2 to 4 ways, about 768 parts in all) into fp32 partials held in
    the workspace."""
    row = 2 * 4 * 300 * 4                                   # one fp32 per (batch row, head, query)
    small = good(B=2, Sq=300, Skv=300, Hq=4, Hkv=2)         # 2 x 2 x 3 = 12 key tiles -> 4 parts
    assert B.bwd_workspace_size(small) >= 2 * row + 12 * 4 * 128 * 256 * 4
    fp32 = good(B=2, Sq=300, Skv=300, Hq=4, Hkv=2, Dqk=64, Dv=64, dtype=B.ATTN_FP32)
    assert B.bwd_workspace_size(fp32) < 2 * row + 1024      # fp32 kernels never split
    big = good(B=1, Sq=8192, Skv=8192, Hq=64, Hkv=8)        # 8 x 64 = 512 key tiles: no split
    assert B.bwd_workspace_size(big) < 2 * 64 * 8192 * 4 + 1024
    mid = good(B=1, Sq=4096, Skv=4096, Hq=32, Hkv=8, Dqk=192)   # 256 key tiles -> 3 parts
    extra = B.bwd_workspace_size(mid) - 2 * 32 * 4096 * 4
    assert 256 * 3 * 128 * (192 + 128) * 4 <= extra < 256 * 3 * 128 * (192 + 128) * 4 + 1024
    wide = good(B=1, Sq=4096, Skv=4096, Hq=48, Hkv=12, Dqk=128)  # 384 key tiles -> 2 parts
    extra = B.bwd_workspace_size(wide) - 2 * 48 * 4096 * 4
    assert 384 * 2 * 128 * 256 * 4 <= extra < 384 * 2 * 128 * 256 * 4 + 1024


def test_overlapping_output_strides_rejected():
    """Strides the library writes through must not alias: O in both calls,
    and Q, K, V in the backward (dQ, dK, dV share them).  An expanded K
    (head stride 0 over two KV heads) may be read, but its gradient would be
    stored by several workgroups to the same memory."""
    d = good(o=(300 * 4 * 128, 64, 128))                    # token stride 64 < head span 4 x 128
    st, text = B.validate_fwd(d)
    assert st == B.ATTN_E_UNSUPPORTED and "overlap" in text
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_UNSUPPORTED and "overlap" in text
    d = good(k=(300 * 128, 128, 0))                         # both KV heads at one address
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_UNSUPPORTED and "k (and dK)" in text
    d = good(q=(0, 4 * 128, 128))                           # both batch rows at one address
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_UNSUPPORTED and "q (and dQ)" in text
    d = good(v=(300 * 2 * 128, 2 * 128, 128), B=2, Hkv=2)   # disjoint: validation reaches the workspace check
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_WORKSPACE, text


def test_kv_token_stride_limit():
    """K and V token strides above 2^24 elements are rejected before any
    HIP call (the kernels address key tile rows with 32-bit offsets); the
    limit itself passes on to the workspace check."""
    big = (1 << 24) + 128
    for which in ("k", "v"):
        d = good(B=1, **{which: (300 * big, big, 128)})
        st, text = B.validate_fwd(d)
        assert st == B.ATTN_E_UNSUPPORTED and "token strides" in text, text
    lim = 1 << 24
    d = good(B=1, k=(300 * lim, lim, 128), v=(300 * lim, lim, 128))
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_WORKSPACE, text


def test_log_route_flag_accepted_and_unknown_bits_rejected():
    """ATTN_LOG_ROUTE is a known flag (validation goes on to the missing
    workspace); bit 4 is not."""
    seg = B.attn_segments(0x1000, None, None, None)
    st, text = B.validate_fwd(good(flags=B.ATTN_LOG_ROUTE), seg)
    assert st == B.ATTN_E_WORKSPACE, text
    st, text = B.validate_bwd(good(flags=B.ATTN_LOG_ROUTE | B.ATTN_FORCE_GENERAL), seg)
    assert st == B.ATTN_E_WORKSPACE, text
    st, text = B.validate_fwd(good(flags=1 << 4), seg)
    assert st == B.ATTN_E_INVALID and "unknown flag" in text, text


def test_disjoint_packed_views_pass_the_stride_check():
    """Packed QKV [B, S, 3, H, D] and KV [B, S, 2, Hkv, D] views are disjoint
    per tensor: validation passes the stride checks and stops at the missing
    workspace, which is checked after them."""
    S, H, D = 300, 4, 128
    qkv = (S * 3 * H * D, 3 * H * D, D)
    kv = (S * 2 * 2 * D, 2 * 2 * D, D)
    d = good(q=qkv, k=kv, v=kv, o=(S * H * D, H * D, D))
    st, text = B.validate_bwd(d)
    assert st == B.ATTN_E_WORKSPACE, text


def test_route_rows_validation():
    L = B.lib()
    seg = B.attn_segments(0x1000, None, None, None)
    d = good()
    st = L.attn_route_rows(ctypes.byref(d), ctypes.byref(seg), 1 << 20, 1 << 20, None, None)
    assert st == B.ATTN_E_INVALID and b"route_rows" in L.attn_last_error()
    need = B.fwd_workspace_size(d, seg)
    st = L.attn_route_rows(ctypes.byref(d), ctypes.byref(seg), 1 << 20, need - 1, 1 << 12, None)
    assert st == B.ATTN_E_WORKSPACE
    bad = good(Hq=3)
    st = L.attn_route_rows(ctypes.byref(bad), None, None, 0, 1 << 12, None)
    assert st == B.ATTN_E_INVALID

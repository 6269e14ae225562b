"""The backward's dK/dV and dQ phases launched on two streams at once
(after the prepare phase) give bitwise the outputs of the one-stream
backward: the two phases read the prepared workspace and write disjoint
outputs, so any overlap of them is a legal schedule.  The benchmark uses it
where it measured faster."""

import numpy as np
import pytest

from bwd_packed_segments_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    # fast route, work-split dK/dV, one query head per KV head
    ("thd_packed_8k", dict(B=2, S=1000, Hq=4, Hkv=4, seg_lo=50, seg_hi=400), None),
    # general route, dK/dV walks split into parts (fp32 partials and their sum)
    ("thd_cross_ring_4k", dict(Sq=700, Skv=900, Hq=4, Hkv=2, seg_lo=32, seg_hi=256), None),
    # dense causal GQA: gradient-split dK/dV and dQ over head pairs
    ("gqa_causal_8k", dict(S=1000, Hq=8, Hkv=2), None),
    # soft cap and a bias slab shared by two batch rows (dbias partials summed in the dK/dV phase)
    ("bshd_causal_2k", dict(B=2, S=400, Hq=4, Hkv=2), "bias_softcap"),
]


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("name,over,variant", CASES, ids=[c[0] for c in CASES])
def test_two_stream_backward_is_bitwise_one_stream(name, over, variant):
    import torch
    import bwd_packed_segments_amd as bps
    from tests import gpu_util as G
    w = inputs.workload(name, **over)
    case = inputs.make_case(w, 21)
    print(f"[schedule] {name} {over} variant={variant}", flush=True)
    dev = {k: torch.from_numpy(case[k]).to("cuda").to(torch.bfloat16) for k in ("q", "k", "v", "do")}
    seg = G.seg_to_dev(case["segments"])
    var = {}
    if variant == "bias_softcap":
        bias = inputs.variant_inputs(w, 21, bias_batch=1)["bias"]
        var = dict(bias=torch.from_numpy(bias).to("cuda").to(torch.bfloat16), softcap=4.0)
    fwd = bps.FwdPlan(dev["q"], dev["k"], dev["v"], causal=w.causal, segments=seg, **var)
    fwd.run()

    def plan():
        return bps.BwdPlan(dev["q"], dev["k"], dev["v"], fwd.o, fwd.lse, dev["do"], causal=w.causal, segments=seg,
                           **var)

    def outs(p):
        return [p.dq, p.dk, p.dv] + ([p.dbias] if p.dbias is not None else [])

    one = plan()
    one.run(bps.ATTN_BWD_ALL)
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs(one)]

    two = plan()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for rep in range(3):
        for t in outs(two):
            t.fill_(float("nan"))
        two.run(bps.ATTN_BWD_PREPARE, stream=main)
        forked = torch.cuda.Event()
        forked.record(main)
        side.wait_event(forked)
        two.run(bps.ATTN_BWD_DQ, stream=side)
        two.run(bps.ATTN_BWD_DKDV, stream=main)
        joined = torch.cuda.Event()
        joined.record(side)
        main.wait_event(joined)
        torch.cuda.synchronize()
        for name_o, a, b in zip(("dQ", "dK", "dV", "dbias"), ref, outs(two)):
            diff = int((a != _bits(b)).sum())
            assert diff == 0, f"{name_o}: {diff} elements differ from the one-stream backward (repeat {rep})"
    assert np.isfinite(one.dq.float().cpu().numpy()).all()

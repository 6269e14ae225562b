"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  A mutant is the oracle's source with one textual change,
loaded as a separate module; the pins are then run against it."""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from tests import oracle_pins as P
from tests.test_oracle_pins import CASES, FAST

SRC = open(os.path.join(os.path.dirname(oa.__file__), "attention.py")).read()

MUTATIONS = {
    "gqa_modulo": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "causal_flipped": ("return np.tril(np.ones((Sq, Skv), dtype=bool))",
                       "return np.triu(np.ones((Sq, Skv), dtype=bool))"),
    "pos_vs_index": ("mask &= pos_kv[b][None, :] <= pos_q[b][:, None]",
                     "mask &= np.arange(Skv)[None, :] <= np.arange(Sq)[:, None]"),
    "padding_attends": ("mask = (iq != 0) & (iq == ik)", "mask = (iq == ik)"),
    "dk_no_scale": ("dK[b, :, c, :] += scale * (dS.T @ qh)", "dK[b, :, c, :] += (dS.T @ qh)"),
    "ds_sign": ("dS = P * (dP - delta[:, None])", "dS = P * (delta[:, None] - dP)"),
    "dv_transposed": ("dV[b, :, c, :] += P.T @ doh", "dV[b, :, c, :] += P @ doh"),
    "delta_dropped": ("dS = P * (dP - delta[:, None])", "dS = P * dP"),
    "lse_log2": ("m_safe + np.log(np.where(den > 0, den, 1.0))",
                 "m_safe + np.log2(np.where(den > 0, den, 1.0))"),
    "default_scale": ("scale = 1.0 / math.sqrt(Dqk) if scale is None else float(scale)",
                      "scale = 1.0 / Dqk if scale is None else float(scale)"),
    "dq_uses_q": ("dQ[b, :, h, :] = scale * (dS @ kh)", "dQ[b, :, h, :] = scale * (dS @ qh)"),
    "derive_pos_off_by_one": ("pos[b, i] = i - start", "pos[b, i] = i - start + 1"),
    "max_unmasked": ("masked = np.where(mask, S, -np.inf)", "masked = S"),
    "dk_overwrites_group": ("dK[b, :, c, :] += scale * (dS.T @ qh)", "dK[b, :, c, :] = scale * (dS.T @ qh)"),
    "dv_overwrites_group": ("dV[b, :, c, :] += P.T @ doh", "dV[b, :, c, :] = P.T @ doh"),
    "fast_route_nonstrict": ("if best is not None and cur <= best:", "if best is not None and cur < best:"),
    "fast_route_ignores_pos": ("if cur != 0 and int(pos_q[b, i]) != i - start:", "if False:"),
    "empty_row_lse_zero": ("lse = np.where(n > 0, m_safe + np.log(np.where(den > 0, den, 1.0)), -np.inf)",
                           "lse = np.where(n > 0, m_safe + np.log(np.where(den > 0, den, 1.0)), 0.0)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) >= 1, name
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _all_pins_pass():
    """True when every pin passes under the current oracle."""
    try:
        for case in CASES:
            causal = bool(int(case["causal"][0]))
            mask = case["mask"]
            Sq, Skv = mask.shape
            if case["ids_q"] == ["none"]:
                seg = None
            else:
                ids_q = np.array([[int(x) for x in case["ids_q"]]], dtype=np.int32)
                pos_q = np.array([[int(x) for x in case["pos_q"]]], dtype=np.int32)
                segs = {"ids_q": ids_q, "pos_q": pos_q}
                if case["ids_kv"] != ["same"]:
                    segs["ids_kv"] = np.array([[int(x) for x in case["ids_kv"]]], dtype=np.int32)
                    segs["pos_kv"] = np.array([[int(x) for x in case["pos_kv"]]], dtype=np.int32)
                seg = oracle.resolve_segments(segs, 1, Sq, Skv)
            if not np.array_equal(oracle.allowed_mask(0, Sq, Skv, causal, seg), mask):
                return False
        for flag, fids, fpos in FAST:
            if bool(oracle.fast_route_eligible({"ids_q": fids[None], "pos_q": fpos[None]}, 1, fids.size,
                                               fids.size)[0]) != bool(flag):
                return False
        ids = np.array([[1, 1, 1, 2, 2, 0, 0, 3, 3, 1]], dtype=np.int32)
        if not np.array_equal(oracle.derive_pos(ids)[0], [0, 1, 2, 0, 1, 0, 1, 0, 1, 0]):
            return False
        q, k, v, do = P.rng_arrays(1, 1, 6, 6, 2, 1, 3, 2)
        ids6 = np.array([[1, 1, 1, 2, 2, 0]], dtype=np.int32)
        if P.pin_finite_differences(q, k, v, do, causal=True, segments={"ids_q": ids6}) > 1e-6:
            return False
        checks = [
            P.pin_closed_forms() < 1e-12,
            P.pin_packed_equals_separate() < 1e-12,
            P.pin_gqa_equals_mha(causal=True) < 1e-12,
            P.pin_padding_garbage() == 0.0,
            P.pin_torch_sdpa(causal=True) < 1e-12,
            P.pin_torch_sdpa(causal=False, Sq=5, Skv=9) < 1e-12,
            P.pin_row_sums(*P.rng_arrays(0, 2, 10, 10, 2, 1, 6, 4)[:2], causal=True,
                           segments=P.seg_packed_padded()) < 1e-12,
        ]
        return all(checks)
    except Exception:
        return False


def _install(monkeypatch, mod):
    for name in ("forward", "backward", "allowed_mask", "derive_pos", "resolve_segments",
                 "fast_route_eligible", "kv_head_of"):
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    for name in dir(mod):
        if not name.startswith("__"):
            monkeypatch.setattr(oa, name, getattr(mod, name), raising=False)


def test_unmutated_oracle_passes():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    _install(monkeypatch, _mutant(name))
    assert not _all_pins_pass(), f"planted mistake {name!r} went unnoticed"

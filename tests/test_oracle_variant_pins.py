"""The variant oracle against its pins, and planted mistakes in it that the
pins must catch (on the CPU)."""

import os
import types

import pytest

from oracle import variants as ov
from tests import oracle_variant_pins as VP

SRC = open(os.path.join(os.path.dirname(ov.__file__), "variants.py")).read()

MUTATIONS = {
    "sink_not_in_denominator": ("den = E.sum(axis=1) + e_sink", "den = E.sum(axis=1)"),
    "softcap_no_derivative": ("dX = dS * (1.0 - (S / softcap) ** 2) if softcap else dS", "dX = dS"),
    "softcap_derivative_sign": ("(1.0 - (S / softcap) ** 2)", "(1.0 + (S / softcap) ** 2)"),
    "dsink_sign": ("dsink[h] += float(-(p_sink * delta).sum())", "dsink[h] += float((p_sink * delta).sum())"),
    "bias_scaled": ("X = X + bias_h", "X = X + scale * bias_h"),
    "softcap_unscaled": ("S = softcap * np.tanh(X / softcap)", "S = np.tanh(X / softcap)"),
    "dbias_from_ds": ("dbias[b if bias.shape[0] > 1 else 0, h] += dX", "dbias[b if bias.shape[0] > 1 else 0, h] += dS"),
    "dbias_first_row_only": ("dbias[b if bias.shape[0] > 1 else 0, h] += dX",
                             "dbias[b if bias.shape[0] > 1 else 0, h] = dX"),
    "bias_row_zero": ("return bias[b if bias.shape[0] > 1 else 0]", "return bias[0]"),
    "max_logit_unmasked": ("max_logit[h] = max(max_logit[h], float(S[mask].max()))",
                           "max_logit[h] = max(max_logit[h], float(S.max()))"),
    "max_logit_before_softcap": ("_, S = _logits(q[b, :, h, :]", "S, _ = _logits(q[b, :, h, :]"),
    "dq_from_ds": ("dQ[b, :, h, :] = scale * (dX @ kh)", "dQ[b, :, h, :] = scale * (dS @ kh)"),
    "sink_lse_dropped": ("lse = np.where(live, m0 + np.log(den_safe), -np.inf)",
                         "lse = np.where(live, m0 + np.log(den_safe - e_sink + 1e-300), -np.inf)"),
    "bias_after_softcap": ("    if bias_h is not None:\n        X = X + bias_h\n    if softcap:\n"
                           "        S = softcap * np.tanh(X / softcap)\n    else:\n        S = X\n",
                           "    if softcap:\n        S = softcap * np.tanh(X / softcap)\n    else:\n        S = X\n"
                           "    if bias_h is not None:\n        X = X + bias_h\n        S = S + bias_h\n"),
    "sink_base2": ("e_sink = np.exp(sink_h - m0)", "e_sink = np.exp2(sink_h - m0)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    mod = types.ModuleType(f"oracle_variants_mutant_{name}")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,value,bound", VP.all_pins(), ids=lambda x: x if isinstance(x, str) else "")
def test_variant_pin(name, value, bound):
    assert value <= bound, f"{name}: {value} > {bound}"


def _fails_some_pin(mod):
    try:
        return any(not (value <= bound) for _, value, bound in VP.all_pins(mod))
    except Exception:
        return True


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_variant_mutation_is_caught(name):
    assert _fails_some_pin(_mutant(name)), f"planted mistake {name!r} went unnoticed"

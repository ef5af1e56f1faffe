"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (on the CPU, in memory),
loads the copy as a module, points the pin tests at it and requires at least one pin to
fail.  The committed oracle is never modified.
"""
import importlib.util
import os
import types

import pytest

import oracle.polar_oracle as good
from tests import test_oracle as pins

SRC = open(good.__file__).read()

MUTATIONS = {
    "S2 without the square": ("s2 = (p * p).sum(axis=1)", "s2 = p.sum(axis=1)"),
    "n_eff as S1/S2": ("n_eff = s1 * s1 / s2", "n_eff = s1 / s2"),
    "temperature linear in n": ("return 1.0 + tau * np.log(_f64(n))", "return 1.0 + tau * _f64(n)"),
    "temperature off by one": ("return 1.0 + tau * np.log(_f64(n))", "return 1.0 + tau * np.log(_f64(n) + 1)"),
    "causal mask off by one": ("return np.minimum(i + 1 + (tk - tq), tk)", "return np.minimum(i + (tk - tq), tk)"),
    "scale 1/d": ("scale = 1.0 / np.sqrt(d) if", "scale = 1.0 / d if"),
    "temperature on keys only": ("s = (lam * scale)[:, None] * raw", "s = scale * raw"),
    "values replaced by keys": ("acc = p @ v[b, hk, :last]", "acc = p @ k[b, hk, :last]"),
    "floor sign of m": ("z = f - m - np.log(s1)", "z = f + m - np.log(s1)"),
    "floor without S1": ("z = f - m - np.log(s1)", "z = f - m"),
    "floor without temperature": ("return _f64(lam) * np.sqrt(2.0 * np.log(_f64(n))) + beta",
                                  "return np.sqrt(2.0 * np.log(_f64(n))) + beta"),
    "floor sqrt(ln n)": ("return _f64(lam) * np.sqrt(2.0 * np.log(_f64(n))) + beta",
                         "return _f64(lam) * np.sqrt(np.log(_f64(n))) + beta"),
    "saturation scale inverted": ("np.tanh(np.log(n_eff) / kappa)", "np.tanh(np.log(n_eff) * kappa)"),
    "saturation without log": ("np.tanh(np.log(n_eff) / kappa)", "np.tanh(n_eff / kappa)"),
    "count without confidence": ("count = conf * np.tanh", "count = np.tanh"),
    "merge weight on S2 not squared": ("s2 += w * w * b2", "s2 += w * b2"),
    "merge weight on acc squared": ("acc = acc + w * c", "acc = acc + w * w * c"),
    "kv head mapping modulo": ("hk = h // group", "hk = h % Hkv"),
    "direction divided by S1": ("direction = np.where(norm[:, None] == 0.0, 0.0, acc / safe[:, None])",
                                "direction = acc / s1[:, None]"),
    "max not subtracted consistently": ("p = np.exp(s - m[:, None])", "p = np.exp(s)"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not (name.startswith("test_") and isinstance(fn, types.FunctionType)):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        combos = [{}]
        for m in params:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            new = []
            for c in combos:
                for val in m.args[1]:
                    vals = val if len(argnames) > 1 else (val,)
                    new.append({**c, **dict(zip(argnames, vals))})
            combos = new
        calls += [(fn, kw) for kw in combos]
    return calls


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_pins_catch_mutation(label, monkeypatch):
    mod = _mutant(*MUTATIONS[label])
    for name in ("finish_rows", "length_temperature", "merge_reference", "merge_statistics",
                 "null_floor", "polar_attention", "split_statistics", "visible_count"):
        monkeypatch.setattr(pins, name, getattr(mod, name))
    caught = []
    for fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            caught.append(f"{fn.__name__}{kw}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake '{label}'"


def test_unmutated_oracle_passes_all_pins():
    for fn, kw in _pin_calls():
        fn(**kw)

"""The backward oracle's finite-difference pin must catch plausible mistakes planted in
copies of its source (in memory; the committed oracle is never modified)."""
import importlib.util

import pytest

import oracle.polar_backward as good
from tests.test_backward_oracle import CASES, VARIANT_CASES, fd_check

SRC = open(good.__file__).read()

MUTATIONS = {
    "S2 term without the factor 2": ("c1[:, None] + 2.0 * c2[:, None] * p", "c1[:, None] + c2[:, None] * p"),
    "direction gradient not projected": ("(g_u - u * np.sum(u * g_u, axis=-1, keepdims=True))", "g_u"),
    "dk without the temperature": ("dk[b, hk] += (ls[:, None] * ds).T @ q[b, h]", "dk[b, hk] += ds.T @ q[b, h]"),
    "dv weighted by ds": ("dv[b, hk] += p.T @ w", "dv[b, hk] += ds.T @ w"),
    "n_eff derivative sign": ("c2 = -g_neff * n_eff / s2", "c2 = g_neff * n_eff / s2"),
    "confidence derivative without (1 - conf)": ("dconf_dz1 = conf * (1.0 - conf)", "dconf_dz1 = conf"),
    "count ignores the saturation slope": ("g_neff = g_n + g_k * conf * slope", "g_neff = g_n"),
    "log1p saturation with the slope of ln": ("slope = (1.0 - t * t) / (kappa * (1.0 + n_eff))",
                                              "slope = (1.0 - t * t) / (kappa * n_eff)"),
    "variant temperature ignored": ("lam = np.array([temperature(int(ni), tau, var) for ni in n])",
                                    "lam = length_temperature(n, tau)"),
    "gumbel2 floor level ignored": ("f = lam * np.array([floor_level(int(ni), var) for ni in n]) + beta",
                                    "f = None"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle.backward_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_finite_differences_catch(name):
    mod = _mutant(*MUTATIONS[name])
    caught = False
    for variant, case in [(None, c) for c in CASES] + VARIANT_CASES:
        try:
            fd_check(mod, case, variant=variant)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught: {name}"

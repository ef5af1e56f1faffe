"""The variant oracle's pins must catch plausible mistakes planted in copies of its
source (in memory; the committed oracle is never modified)."""
import importlib.util

import pytest

import oracle.polar_variants as good
from tests.test_oracle_variants import CHECKS

SRC = open(good.__file__).read()

MUTATIONS = {
    "ssmax keeps the 1 +": ("return tau * ln_n\n", "return 1.0 + tau * ln_n\n"),
    "train ratio inverted": ("return ln_n / math.log(var[\"train_len\"])", "return math.log(var[\"train_len\"]) / ln_n"),
    "gumbel correction sign": ("b = r - (math.log(math.log(n))", "b = r + (math.log(math.log(n))"),
    "gumbel without the gamma term": ("return b + EULER_GAMMA / r", "return b"),
    "gumbel with ln 2 pi": ("math.log(4.0 * math.pi)", "math.log(2.0 * math.pi)"),
    "qnorm without the softmax scale": ("return scale * float(np.sqrt(q_row @ q_row))", "return float(np.sqrt(q_row @ q_row))"),
    "soft floor not clipped": ("np.maximum(p - math.exp(f - m), 0.0)", "p - math.exp(f - m)"),
    "soft floor against the maximum": ("np.maximum(p - math.exp(f - m), 0.0)", "np.maximum(p - math.exp(f), 0.0)"),
    "gate inclusive of the maximum only": ("np.where(s > f, p, 0.0)", "np.where(s >= m, p, 0.0)"),
    "log1p saturation as log": ("x = math.log1p(n_eff) if", "x = math.log(n_eff) if"),
    "window one key short": ("lo = max(0, hi - window) if window else 0", "lo = max(0, hi - window + 1) if window else 0"),
    "window count from the causal row": ("return lo, hi, hi - lo", "return lo, hi, hi"),
    "merge weight not squared": ("s2 += wgt * wgt * b2", "s2 += wgt * b2"),
    "floor ignores the temperature": ("return lam * sigma * floor_level(n, var)", "return sigma * floor_level(n, var)"),
    "confidence without the floor": ("conf = 1.0 / (1.0 + math.exp(f - m - math.log(s1)))",
                                     "conf = 1.0 / (1.0 + math.exp(-m - math.log(s1)))"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle.variant_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "variant_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for check in CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, ZeroDivisionError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutation '{name}'"

"""CPU checks of the stored oracle self-sensitivity floors (tests/golden)."""
import json
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "oracle_sensitivity.json")


def _samples():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mos", os.path.join(HERE, "golden", "make_oracle_sensitivity.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)          # defines constants only; main() is not run
    return mod.SAMPLES, mod.EPS


def test_floors_cover_the_sampled_rows_and_steps():
    samples, eps = _samples()
    data = json.load(open(GOLDEN))
    for name, (rows, steps) in samples.items():
        entry = data[name]
        assert entry["rows"] == rows and entry["steps"] == steps and entry["eps"] == eps
        for r in entry["max_abs_dlogit"]:
            assert len(r) == len(steps)
            # a float32-sized perturbation moves the logits, but by a few percent at most
            assert all(0.0 < x < 0.1 for x in r), (name, r)


@pytest.mark.parametrize("name", ["opt1.3b", "opt6.7b", "opt13b"])
def test_floor_grows_with_depth_not_beyond_reason(name):
    data = json.load(open(GOLDEN))
    worst = max(max(r) for r in data[name]["max_abs_dlogit"])
    rms = max(max(r) for r in data[name]["logit_rms"])
    assert worst < 0.05 * rms + 0.02

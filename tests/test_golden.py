"""CPU checks of the stored oracle self-sensitivity floors (tests/golden), and of the
properties the GPU tests' bound takes from them (gpu_util.oracle_floor)."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "oracle_sensitivity.json")


def _script():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mos", os.path.join(HERE, "golden", "make_oracle_sensitivity.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)          # defines constants and functions only; main() is not run
    return mod


def _entries():
    mod = _script()
    data = json.load(open(GOLDEN))
    return mod, [(name, data[name]) for name in mod.SAMPLES]


def test_floors_cover_the_sampled_rows_and_steps():
    mod, entries = _entries()
    for name, e in entries:
        rows, steps = mod.SAMPLES[name]
        assert e["rows"] == rows and e["steps"] == steps
        assert e["eps"] == mod.EPS and e["eps_gpu"] == mod.EPS_GPU and e["eps_small"] == mod.EPS_SMALL
        a = np.asarray(e["per_copy_max_abs_dlogit"])
        b = np.asarray(e["gpu_per_copy_max_abs_dlogit"])
        assert a.shape == (mod.N_EPS, len(rows), len(steps)) and b.shape == (mod.N_GPU, len(rows), len(steps))
        # a float32-sized perturbation moves the logits, by a few percent of their scale at most
        assert (a > 0).all() and (b > 0).all() and a.max() < 0.1 and b.max() < 0.1, name


@pytest.mark.parametrize("name", ["opt1.3b", "opt6.7b", "opt13b", "opt6.7b-2l", "opt13b-2l"])
def test_floor_is_a_tight_level_set_by_the_storage_points(name):
    """The bound's premise: across independently perturbed copies the largest logit
    difference scatters little about its mean (coefficient of variation well below
    0.25), and a perturbation 256 times larger (2^-16 against 2^-24) raises the level
    by a small factor only -- the level is set by the bf16 storage points, not by the
    size of the first difference."""
    _, entries = _entries()
    e = dict(entries)[name]
    a = np.asarray(e["per_copy_max_abs_dlogit"])
    b = np.asarray(e["gpu_per_copy_max_abs_dlogit"])
    allc = np.concatenate([a, b])
    cv = (allc / allc.mean(axis=0, keepdims=True)).std(ddof=1)
    assert cv < 0.25, cv
    ratio = b.mean() / a.mean()
    assert 0.8 < ratio < 1.6, ratio
    rms = np.asarray(e["logit_rms"]).max()
    assert allc.max() < 0.05 * rms + 0.02


def test_floor_bound_matches_its_definition():
    """gpu_util.oracle_floor = m (1 + FLOOR_SIGMAS c), recomputed here from the file."""
    import sys
    sys.path.insert(0, HERE)
    import gpu_util as G
    _, entries = _entries()
    for name, e in entries:
        a = np.asarray(e["per_copy_max_abs_dlogit"])
        b = np.asarray(e["gpu_per_copy_max_abs_dlogit"])
        allc = np.concatenate([a, b])
        c = (allc / allc.mean(axis=0, keepdims=True)).std(ddof=1)
        for i, r in enumerate(e["rows"]):
            for k, s in enumerate(e["steps"]):
                m = max(a[:, i, k].mean(), b[:, i, k].mean())
                assert G.oracle_floor(name, r, s) == pytest.approx(m * (1 + G.FLOOR_SIGMAS * c), rel=1e-12)
        assert G.oracle_floor(name, -1, 0) is None

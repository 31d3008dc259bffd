"""Pins of the weight-only FP8 oracle (oracle/fp8.py): E4M3 rounding against torch's
float8_e4m3fn conversion and the format's closed forms, the per-channel quantiser's
bounds, and the decode model with FP8 weights reducing to the bf16 one when the
weights are exactly representable."""
import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as F
from oracle import opt_he as O


def _torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).float().double().numpy()


def _all_finite_codes():
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return np.unique(v[np.isfinite(v)])


def test_e4m3_round_matches_torch_random():
    rng = np.random.default_rng(8)
    x = (rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-13, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(F.e4m3_round(x), _torch_e4m3(x))


def test_e4m3_round_ties_fixed_points_and_subnormals():
    vals = _all_finite_codes()
    assert len(vals) == 253 and vals.max() == 448 and vals[vals > 0].min() == 2.0 ** -9
    np.testing.assert_array_equal(F.e4m3_round(vals), vals)          # the grid maps to itself
    pos = vals[vals >= 0]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)             # exact halfway points
    np.testing.assert_array_equal(F.e4m3_round(mids), _torch_e4m3(mids))
    np.testing.assert_array_equal(F.e4m3_round(-mids), _torch_e4m3(-mids))
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25; subnormal 2^-10 -> 0
    assert F.e4m3_round(1 + 1 / 16) == 1.0 and F.e4m3_round(1 + 3 / 16) == 1.25
    assert F.e4m3_round(2.0 ** -10) == 0.0 and F.e4m3_round(3 * 2.0 ** -10) == 2 * 2.0 ** -9
    # saturation (where torch's conversion gives NaN instead)
    assert F.e4m3_round(460.0) == 448 and F.e4m3_round(1e6) == 448 and F.e4m3_round(-500.0) == -448


def test_quantize_rows_bounds():
    rng = np.random.default_rng(2)
    W = torch.from_numpy(rng.normal(0, 0.02, (64, 512)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    W[3] = 0.0
    W[5, 7] = -0.5                                  # an outlier row
    q, s = F.quantize_rows(W)
    assert s.dtype == np.float32 and s[3] == 1.0 and (q[3] == 0).all()
    amax_idx = np.abs(W).argmax(axis=1)
    live = np.abs(W).max(axis=1) > 0
    assert (np.abs(q[np.arange(64), amax_idx])[live] == 448).all()  # the row maximum lands on 448
    assert set(np.unique(np.abs(q))) <= set(_all_finite_codes())
    # error within half a spacing of the E4M3 grid at each quotient
    y = (W.astype(np.float32) / s[:, None]).astype(np.float64)
    _, ex = np.frexp(np.where(np.abs(y) > 0, np.abs(y), 1.0))
    half = np.exp2(np.maximum(ex - 1, -6) - 3) / 2
    assert (np.abs(q - y) <= half).all()
    Wq = F.dequantize(q, s)
    assert np.abs(Wq - W).max() <= np.abs(W).max() * 2.0 ** -4


def test_fp8_decode_equals_bf16_when_weights_are_representable():
    """Rows built from E4M3 values times 2^-12 with 448 in every row quantise exactly,
    so the FP8 decode equals the plain one; generic weights do not."""
    wl = synth.WORKLOADS["tiny"]
    params = synth.model_params(wl.actor)
    rng = np.random.default_rng(6)
    codes = _all_finite_codes()
    exact = dict(params)
    for i in range(wl.actor.n_layers):
        for name in ("qkv", "out", "fc1", "fc2"):
            W = params[f"L{i}.{name}.w"]
            v = rng.choice(codes, size=W.shape) * 2.0 ** -12
            v[:, 0] = 448 * 2.0 ** -12
            exact[f"L{i}.{name}.w"] = torch.from_numpy(v.astype(np.float32))
    prompts = synth.prompts(wl).numpy()
    forced = synth.forced_tokens(wl).numpy()

    def run(p, fp8):
        om = O.OracleModel(wl.actor, p, O.Precision("fp32"), fp8_decode=fp8)
        return O.greedy_generate(om, prompts, 6, wl.max_seq, forced=forced)[1]

    for a, b in zip(run(exact, True), run(exact, False)):
        np.testing.assert_array_equal(a, b)
    diff = max(np.abs(a - b).max() for a, b in zip(run(params, True)[1:], run(params, False)[1:]))
    assert diff > 1e-6
    # the prompt pass is untouched by the FP8 decode weights
    np.testing.assert_array_equal(run(params, True)[0], run(params, False)[0])

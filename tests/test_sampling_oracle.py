"""Pins of the sampling / log-probability oracle (oracle/sampling.py) against what
does not depend on it: numpy's own Philox4x64-10 bit generator, scipy's logsumexp,
the distribution the Gumbel-max rule must produce, and the greedy oracle."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import synth
from oracle import opt_he as O
from oracle import sampling as SM


def _numpy_philox_block(counter, key):
    """numpy's Philox (4x64, 10 rounds) output block for `counter` exactly: numpy
    increments the stored counter before producing its first block."""
    c = [int(x) for x in counter]
    prev = list(c)
    i = 0
    while True:                      # counter - 1 with borrow
        if prev[i] > 0:
            prev[i] -= 1
            break
        prev[i] = 2 ** 64 - 1
        i += 1
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return bg.random_raw(4)


def test_philox_matches_numpy_bit_generator():
    rng = np.random.default_rng(7)
    for _ in range(25):
        key = [int(x) for x in rng.integers(0, 2 ** 63, size=2, dtype=np.int64)]
        ctr = [int(x) for x in rng.integers(1, 2 ** 63, size=4, dtype=np.int64)]
        ref = _numpy_philox_block(ctr, key)
        got = SM.philox4x64_10([np.array([x], dtype=np.uint64) for x in ctr], key)[:, 0]
        assert np.array_equal(ref, got), (key, ctr)
    # carries through the top bits of the key schedule and counter words
    ctr = [2 ** 64 - 1, 2 ** 64 - 1, 5, 0]
    key = [2 ** 64 - 1, 2 ** 64 - 1]
    assert np.array_equal(_numpy_philox_block(ctr, key),
                          SM.philox4x64_10([np.array([x], dtype=np.uint64) for x in ctr], key)[:, 0])


def test_uniforms_open_interval_and_moments():
    u = SM.uniforms(11, np.arange(8), 300, 4096).astype(np.float64)
    assert u.dtype == np.float64 and (u > 0).all() and (u < 1).all()
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005
    # different positions, rows and seeds give different streams
    assert not np.array_equal(SM.uniforms(11, np.arange(2), 300, 64), SM.uniforms(11, np.arange(2), 301, 64))
    assert not np.array_equal(SM.uniforms(11, np.array([0]), 300, 64), SM.uniforms(11, np.array([1]), 300, 64))
    assert not np.array_equal(SM.uniforms(11, np.arange(2), 300, 64), SM.uniforms(12, np.arange(2), 300, 64))


def test_uniform_extremes_stay_inside_the_interval():
    """The smallest and largest words map to 2^-24 and 1 - 2^-24 exactly, so G is
    finite for every word; neighbouring top values stay distinct."""
    w = np.array([0, (1 << 41) - 1, 1 << 41, (1 << 64) - 1, ((1 << 64) - 1) ^ (1 << 41)], dtype=np.uint64)
    u = SM.word_uniform(w)
    assert u.dtype == np.float32
    assert u[0] == np.float32(2.0 ** -24) and u[1] == u[0]
    assert u[2] == np.float32(3 * 2.0 ** -24)
    assert u[3] == np.float32(1 - 2.0 ** -24) and u[4] < u[3]
    assert np.isfinite(SM.gumbel(u)).all()


def test_logsumexp_matches_scipy():
    rng = np.random.default_rng(3)
    for scale in (0.1, 1.0, 30.0):
        x = rng.normal(size=(5, 777)) * scale
        np.testing.assert_allclose(SM.logsumexp(x, axis=1), scipy.special.logsumexp(x, axis=1), rtol=1e-13, atol=1e-13)


def test_gumbel_max_draws_the_softmax_distribution():
    """Over many independent counters (positions), the Gumbel-max pick of fixed logits
    is distributed as softmax(logits / T): chi-square goodness of fit."""
    logits = np.array([[0.3, -1.2, 2.0, 0.0, 1.1, -0.4]])
    T = 0.8
    p = scipy.special.softmax(logits[0] / T)
    n = 40000
    counts = np.zeros(logits.shape[1])
    for pos in range(n):
        tok, _, _ = SM.pick(logits, T, 5, np.array([3]), pos)
        counts[tok[0]] += 1
    chi2 = scipy.stats.chisquare(counts, n * p)
    assert chi2.pvalue > 1e-3, (counts / n, p)


def test_low_temperature_is_greedy_and_logprobs_normalise():
    rng = np.random.default_rng(9)
    lg = rng.normal(size=(4, 500))
    tok, _, _ = SM.pick(lg, 1e-7, 1, np.arange(4), 10)
    assert np.array_equal(tok, O.argmax_lowest(lg))
    for T in (0.0, 0.7, 1.3):
        scaled = lg / (T if T > 0 else 1.0)
        lp_all = scaled - SM.logsumexp(scaled, axis=1)[:, None]
        np.testing.assert_allclose(np.exp(lp_all).sum(axis=1), 1.0, rtol=1e-12)
        tok, lp, _ = SM.pick(lg, T, 2, np.arange(4), 10)
        np.testing.assert_allclose(lp, lp_all[np.arange(4), tok], rtol=0, atol=1e-12)


def test_zero_temperature_generation_is_the_greedy_oracle():
    wl = synth.WORKLOADS["tiny"]
    params = synth.model_params(wl.actor)
    prompts = synth.prompts(wl).numpy()
    om = O.OracleModel(wl.actor, params, O.Precision("fp32"))
    picks, logits = O.greedy_generate(om, prompts, wl.gen_len, wl.max_seq)
    om2 = O.OracleModel(wl.actor, params, O.Precision("fp32"))
    toks, lps, _, lg2 = SM.sampled_generate(om2, prompts, wl.gen_len, wl.max_seq, 0.0, 0)
    assert np.array_equal(toks, picks)
    for j in range(wl.gen_len):
        np.testing.assert_allclose(lps[:, j], (logits[j] - SM.logsumexp(logits[j], axis=1)[:, None])[
            np.arange(len(prompts)), picks[:, j]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_sampled_generation_is_reproducible_and_seed_dependent(T):
    wl = synth.WORKLOADS["tiny"]
    params = synth.model_params(wl.actor)
    prompts = synth.prompts(wl).numpy()
    om = lambda: O.OracleModel(wl.actor, params, O.Precision("fp32"))
    a = SM.sampled_generate(om(), prompts, wl.gen_len, wl.max_seq, T, 42)[0]
    b = SM.sampled_generate(om(), prompts, wl.gen_len, wl.max_seq, T, 42)[0]
    c = SM.sampled_generate(om(), prompts, wl.gen_len, wl.max_seq, T, 43)[0]
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


# ------------------------------------------------------------------------------------
# top-p (nucleus)
# ------------------------------------------------------------------------------------

def test_nucleus_is_the_smallest_set_reaching_p_brute_force():
    """Over every subset of a 7-token vocabulary: the nucleus is the subset of fewest
    tokens whose probability reaches p (the most probable one among those)."""
    import itertools
    rng = np.random.default_rng(21)
    V = 7
    for trial in range(60):
        lg = rng.normal(size=(1, V)) * rng.uniform(0.3, 3.0)
        p = rng.uniform(0.05, 0.98)
        prob = scipy.special.softmax(lg[0])
        best = None
        for k in range(1, V + 1):
            sets = [c for c in itertools.combinations(range(V), k) if prob[list(c)].sum() >= p]
            if sets:
                best = max(sets, key=lambda c: prob[list(c)].sum())
                break
        mask, margin = SM.nucleus(lg, p)
        assert set(np.nonzero(mask[0])[0]) == set(best), (trial, p, prob)
        assert margin[0] > 0


def test_nucleus_includes_ties_and_limits():
    lg = np.log(np.array([[0.4, 0.2, 0.2, 0.1, 0.1]]))
    mask, margin = SM.nucleus(lg, 0.5)          # 0.4 + 0.2 reaches 0.5; the other 0.2 is tied
    assert mask[0].tolist() == [True, True, True, False, False]
    mask, _ = SM.nucleus(lg, 0.3)
    assert mask[0].tolist() == [True, False, False, False, False]
    rng = np.random.default_rng(4)
    x = rng.normal(size=(6, 300))
    # p -> 0 keeps only the most probable token: sampling becomes greedy
    tok, _, _ = SM.pick(x, 0.9, 3, np.arange(6), 17, top_p=1e-9)
    assert np.array_equal(tok, O.argmax_lowest(x))
    # p = 1 is plain sampling, bit for bit
    a = SM.pick(x, 0.9, 3, np.arange(6), 17, top_p=1.0)
    b = SM.pick(x, 0.9, 3, np.arange(6), 17)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    # the reported log-probability is that of the untruncated distribution
    tok, lp, _ = SM.pick(x, 0.9, 3, np.arange(6), 17, top_p=0.3)
    full = x / 0.9 - SM.logsumexp(x / 0.9, axis=1)[:, None]
    np.testing.assert_allclose(lp, full[np.arange(6), tok], rtol=0, atol=1e-12)


def test_top_p_draws_the_renormalised_nucleus():
    """Chi-square over many positions: picks follow softmax(logits / T) restricted to
    the nucleus and renormalised; nothing outside it is ever drawn."""
    logits = np.array([[0.3, -1.2, 2.0, 0.0, 1.1, -0.4]])
    T, p = 0.8, 0.7
    prob = scipy.special.softmax(logits[0] / T)
    mask, _ = SM.nucleus(logits / T, p)
    want = np.where(mask[0], prob, 0.0)
    want /= want.sum()
    n = 30000
    counts = np.zeros(logits.shape[1])
    for pos in range(n):
        tok, _, _ = SM.pick(logits, T, 9, np.array([1]), pos, top_p=p)
        counts[tok[0]] += 1
    assert counts[~mask[0]].sum() == 0
    chi2 = scipy.stats.chisquare(counts[mask[0]], n * want[mask[0]])
    assert chi2.pvalue > 1e-3, (counts / n, want)

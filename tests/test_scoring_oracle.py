"""Pins of the teacher-forced scoring oracle (oracle/scoring.py) against what does not
depend on its own arithmetic: Hugging Face's OPT language-model loss (which shifts
labels against logits by itself), the cached generation route of the oracle
(prefill + decode, a different code path from the full causal pass), a brute-force
normalisation over every possible next token, and causality."""
import numpy as np
import pytest
import torch

import synth
from oracle import opt_he as O
from oracle import sampling as SM
from oracle import scoring as SC
from test_oracle_pins import _hf_opt, fp64_softmax  # noqa: F401  (fixture)

TINY = synth.WORKLOADS["tiny"]


def _experience(wl, batch=None):
    return torch.cat([synth.prompts(wl, batch=batch), synth.forced_tokens(wl, batch=batch)], dim=1).numpy()


@pytest.fixture(scope="module")
def tiny():
    params = synth.model_params(TINY.actor)
    lora = synth.lora_params(TINY.actor, TINY.lora_rank)
    return params, lora


def test_matches_hf_language_model_loss_per_token(tiny, fp64_softmax):
    """Hugging Face's causal-LM loss with every label but one masked out is minus the
    log-probability of that one token given its prefix.  The library casts the logits
    to float32 before its cross-entropy, so agreement is to float32 rounding; a
    position or sign error is off by O(1)."""
    params, lora = tiny
    seq = _experience(TINY)
    S_p = TINY.prompt_len
    om = O.OracleModel(TINY.actor, params, O.Precision("fp64"), lora=lora, lora_scale=TINY.lora_scale)
    got = SC.teacher_forced_logprobs(om, seq, S_p)
    hf = _hf_opt(TINY.actor, params, lora=lora, scale=TINY.lora_scale, unfused_lora=True)
    ids = torch.from_numpy(seq).long()
    with torch.no_grad():
        for b in range(seq.shape[0]):
            for j in (0, 1, 7, seq.shape[1] - S_p - 1):
                labels = torch.full_like(ids[b:b + 1], -100)
                labels[0, S_p + j] = ids[b, S_p + j]
                loss = hf(input_ids=ids[b:b + 1], labels=labels).loss.item()
                assert abs(-loss - got[b, j]) <= 2e-6 * max(1.0, abs(loss)), (b, j, -loss, got[b, j])


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_equals_cached_generation_logprobs(tiny, T):
    """On the oracle's own generated answer, the full causal pass gives the
    log-probabilities the cached generation route reported at temperature 1 (greedy
    reports them at T' = 1 too)."""
    params, lora = tiny
    prompts = synth.prompts(TINY).numpy()
    mk = lambda: O.OracleModel(TINY.actor, params, O.Precision("fp32"), lora=lora, lora_scale=TINY.lora_scale)
    toks, lps, _, _ = SM.sampled_generate(mk(), prompts, TINY.gen_len, TINY.max_seq, T, 31)
    seq = np.concatenate([prompts, toks], axis=1)
    got = SC.teacher_forced_logprobs(mk(), seq, TINY.prompt_len)
    np.testing.assert_allclose(got, lps, rtol=0, atol=1e-9)


def test_next_token_distribution_normalises(tiny):
    """Brute force over the vocabulary: with the last token of the sequence set to
    each of the V values in turn, exp(lp) of the last position sums to 1.  A
    log-probability read from the wrong position (one that sees the token itself)
    breaks this."""
    params, _ = tiny
    om = O.OracleModel(TINY.actor, params, O.Precision("fp64"))
    base = _experience(TINY, batch=1)[:, :10]
    V = TINY.actor.vocab
    seqs = np.repeat(base, V, axis=0)
    seqs[:, -1] = np.arange(V)
    lp = SC.teacher_forced_logprobs(om, seqs, 9)[:, 0]
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    # and a different prefix gives a different distribution
    seqs[:, 5] = (seqs[:, 5] + 1) % V
    lp2 = SC.teacher_forced_logprobs(om, seqs, 9)[:, 0]
    assert np.abs(lp2 - lp).max() > 1e-6


def test_causal_and_prompt_length_consistent(tiny):
    """Changing a later token leaves earlier log-probabilities unchanged, and the
    split point only selects which positions are reported."""
    params, _ = tiny
    om = O.OracleModel(TINY.actor, params, O.Precision("fp64"))
    seq = _experience(TINY)
    a = SC.teacher_forced_logprobs(om, seq, 4)
    seq2 = seq.copy()
    seq2[:, 20] = (seq2[:, 20] + 3) % TINY.actor.vocab
    b = SC.teacher_forced_logprobs(om, seq2, 4)
    np.testing.assert_array_equal(a[:, :20 - 4], b[:, :20 - 4])
    assert np.abs(a[:, 20 - 4] - b[:, 20 - 4]).max() > 1e-6
    c = SC.teacher_forced_logprobs(om, seq, 11)
    np.testing.assert_allclose(c, a[:, 11 - 4:], rtol=0, atol=1e-12)
    assert (a < 0).all()


def test_one_answer_token_is_the_prompt_pass_head(tiny):
    """S = S_p + 1: the log-softmax of the prompt pass's last logits at the token."""
    params, _ = tiny
    om = O.OracleModel(TINY.actor, params, O.Precision("fp32"))
    seq = _experience(TINY)[:, :TINY.prompt_len + 1]
    lg, _ = O.OracleModel(TINY.actor, params, O.Precision("fp32")).prefill(seq[:, :-1], TINY.max_seq)
    lse = np.log(np.exp(lg - lg.max(axis=1, keepdims=True)).sum(axis=1)) + lg.max(axis=1)
    want = lg[np.arange(len(seq)), seq[:, -1]] - lse
    np.testing.assert_allclose(SC.teacher_forced_logprobs(om, seq, TINY.prompt_len)[:, 0], want, rtol=0, atol=1e-10)


def test_rejects_bad_split(tiny):
    params, _ = tiny
    om = O.OracleModel(TINY.actor, params, O.Precision("fp64"))
    seq = _experience(TINY)
    for sp in (0, seq.shape[1]):
        with pytest.raises(ValueError):
            SC.teacher_forced_logprobs(om, seq, sp)

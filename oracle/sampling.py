"""Oracle for the sampling and log-probability extension of the generation step.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; the product path never calls it.

The experience the actor generates is "sampled" autoregressively (DeepSpeed-Chat
paper summary, section on the RLHF pipeline: the actor produces answers to the
queries), and the PPO step that follows needs the log-probability of every generated
token under the actor.  The pages give no sampler.  Reading taken here:

* temperature T > 0: the next token is drawn from softmax(logits / T) by the
  Gumbel-max rule, token = argmax_n (logit_n / T + G_n) with G_n = -log(-log U_n),
  which yields exactly that distribution for i.i.d. uniform U_n;  T = 0 is greedy
  (lowest index on ties);
* U_n comes from the counter-based generator Philox4x64-10 (Salmon, Moraes, Dror,
  Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): one block per four
  columns, counter (n div 4, row, position of the generated token, 0), key (seed, 0),
  output word n mod 4; U = (top 23 bits of that word + 1/2) / 2^23, exact in single
  precision (with 24 bits the float32 sum k + 1/2 rounds the largest k up to 2^24,
  giving U = 1 and an infinite G), so U lies in [2^-24, 1 - 2^-24];
* the log-probability reported for a token t is logit_t / T' - logsumexp(logits / T')
  with T' = T (T' = 1 for greedy), computed here in float64;
* top-p (nucleus) sampling with 0 < p < 1 (T > 0): the pick is restricted to the
  nucleus, the smallest set of most probable tokens whose probability under
  softmax(logits / T) reaches p (Holtzman et al., "The curious case of neural text
  degeneration", ICLR 2020), with every token tied with the least probable member
  included; Gumbel-max over the nucleus draws from the renormalised distribution.
  The same uniforms are used, and the reported log-probability stays that of the
  untruncated softmax(logits / T).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from oracle import opt_he as O

M32 = np.uint64(0xFFFFFFFF)
# Philox4x64 round multipliers and Weyl key increments (Salmon et al., 2011)
PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
PHILOX_M1 = np.uint64(0xCA5A826395121157)
PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)
PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)


def _mulhilo64(a: np.uint64, b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(high, low) 64-bit halves of the 128-bit product a * b, elementwise."""
    b = np.asarray(b, dtype=np.uint64)
    a0, a1 = a & M32, a >> np.uint64(32)
    b0, b1 = b & M32, b >> np.uint64(32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1     # each < 2^64
    mid = (p00 >> np.uint64(32)) + (p01 & M32) + (p10 & M32)
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    lo = a * b                                                   # wraps mod 2^64
    return hi, lo


def philox4x64_10(counter, key) -> np.ndarray:
    """Ten rounds of Philox4x64 on counters [4, ...] with key (k0, k1); returns [4, ...]."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) for x in counter)
        k0, k1 = np.uint64(key[0]), np.uint64(key[1])
        for _ in range(10):
            hi0, lo0 = _mulhilo64(PHILOX_M0, c0)
            hi1, lo1 = _mulhilo64(PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0, k1 = k0 + PHILOX_W0, k1 + PHILOX_W1
    return np.stack([c0, c1, c2, c3])


def uniforms(seed: int, rows: np.ndarray, position: int, V: int) -> np.ndarray:
    """U[b, n] in (0, 1), float32, for batch rows `rows` generating at `position`."""
    rows = np.asarray(rows, dtype=np.uint64)
    nb = (V + 3) // 4
    n4 = np.arange(nb, dtype=np.uint64)
    ctr = (np.broadcast_to(n4[None, :], (len(rows), nb)),
           np.broadcast_to(rows[:, None], (len(rows), nb)),
           np.full((len(rows), nb), position, dtype=np.uint64),
           np.zeros((len(rows), nb), dtype=np.uint64))
    w = philox4x64_10(ctr, (np.uint64(seed), np.uint64(0)))       # [4, rows, nb]
    w = np.moveaxis(w, 0, -1).reshape(len(rows), 4 * nb)[:, :V]    # column n = word n % 4 of block n // 4
    return word_uniform(w)


def word_uniform(w) -> np.ndarray:
    """U = (top 23 bits of the 64-bit word + 1/2) / 2^23 in float32 (exact)."""
    top = (np.asarray(w, dtype=np.uint64) >> np.uint64(41)).astype(np.float32)
    return (top + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel(u: np.ndarray) -> np.ndarray:
    """G = -log(-log U) in float32."""
    u = np.asarray(u, dtype=np.float32)
    return -np.log(-np.log(u))


def logsumexp(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """log(sum(exp(x))) along axis, float64, shifted by the maximum."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)


def nucleus(scaled: np.ndarray, top_p: float) -> Tuple[np.ndarray, np.ndarray]:
    """Nucleus of each row of tempered logits [B, V] (float64) for 0 < top_p < 1.

    Tokens sorted by probability, the nucleus is the first k of them whose cumulative
    probability reaches top_p, plus every token tied with the k-th.  Returns (mask
    [B, V], margin [B]): the margin is how far top_p is from the cumulative
    probability of the first k - 1 and of the first k tokens, the room a rounding
    change has before k moves.
    """
    scaled = np.asarray(scaled, dtype=np.float64)
    prob = np.exp(scaled - logsumexp(scaled, axis=1)[:, None])
    order = np.argsort(-prob, axis=1, kind="stable")
    sp = np.take_along_axis(prob, order, axis=1)
    cum = np.cumsum(sp, axis=1)
    hit = cum >= top_p
    # index of the k-th token (0-based); the whole row if rounding keeps the total below p
    k = np.where(hit.any(axis=1), np.argmax(hit, axis=1), scaled.shape[1] - 1)
    rows = np.arange(len(scaled))
    kth = scaled[rows, order[rows, k]]
    mask = scaled >= kth[:, None]
    below = np.where(k > 0, cum[rows, np.maximum(k - 1, 0)], 0.0)
    margin = np.minimum(top_p - below, cum[rows, k] - top_p)
    return mask, margin


def pick(logits: np.ndarray, temperature: float, seed: int, rows: np.ndarray,
         position: int, top_p: float = 1.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One step for rows of logits [B, V] (float64).

    Returns (tokens [B], log-probabilities [B], decision margin [B]): the margin is the
    gap between the best and second-best of the quantity maximised (logits for greedy,
    logit / T + G for sampling, over the nucleus under top-p), the part of the decision
    a rounding change can flip.  The nucleus's own margin (in probability mass) is
    the second value of ``nucleus``.
    """
    logits = np.asarray(logits, dtype=np.float64)
    if temperature > 0:
        scaled = logits / temperature
        y = scaled + gumbel(uniforms(seed, rows, position, logits.shape[1])).astype(np.float64)
        if 0 < top_p < 1:
            mask, _ = nucleus(scaled, top_p)
            y = np.where(mask, y, -np.inf)
    else:
        scaled = logits
        y = logits
    tok = O.argmax_lowest(y)
    top2 = np.sort(y, axis=1)[:, -2:]
    lp = scaled[np.arange(len(tok)), tok] - logsumexp(scaled, axis=1)
    return tok, lp, top2[:, 1] - top2[:, 0]


def sampled_generate(model: O.OracleModel, prompts, gen_len: int, max_seq: int, temperature: float,
                     seed: int, forced=None, top_p: float = 1.0
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, List[np.ndarray]]:
    """Generate gen_len tokens per row (the greedy loop of opt_he.greedy_generate with
    `pick` as the rule).  Token j of every row is generated at position S + j.
    Returns (tokens [B, gen_len], log-probabilities [B, gen_len], margins [B, gen_len],
    logits per step)."""
    prompts = np.asarray(prompts)
    B, S = prompts.shape
    rows = np.arange(B)
    toks = np.zeros((B, gen_len), dtype=np.int64)
    lps = np.zeros((B, gen_len))
    margins = np.zeros((B, gen_len))
    lg, cache = model.prefill(prompts, max_seq)
    logits = [lg]
    toks[:, 0], lps[:, 0], margins[:, 0] = pick(lg, temperature, seed, rows, S, top_p)
    for j in range(1, gen_len):
        fed = toks[:, j - 1] if forced is None else np.asarray(forced)[:, j - 1]
        lg = model.decode(fed, cache)
        logits.append(lg)
        toks[:, j], lps[:, j], margins[:, j] = pick(lg, temperature, seed, rows, S + j, top_p)
    return toks, lps, margins, logits

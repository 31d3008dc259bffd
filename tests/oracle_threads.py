"""Run the oracle's definition-mode forward over many rows in parallel threads.

Test infrastructure: it calls only the oracle's own pieces (OracleModel.embed,
layer, layer_forward, lm_logits) in the order OracleModel.hidden does, for
independent row chunks at once.  Every chunk goes through the same layer weights,
converted (and LoRA-folded) once per layer and dropped after it; numpy releases the
GIL in its array kernels, so the chunks' elementwise work runs on several cores.
BLAS runs one thread per chunk meanwhile.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np
from threadpoolctl import threadpool_limits

from oracle import opt_he as O


def cores() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def logits_at(shape, params, prec, seqs: np.ndarray, cols: Sequence[int], lora=None, lora_scale=1.0,
              chunks: Optional[int] = None, keep: Optional[dict] = None) -> np.ndarray:
    """Definition-mode logits of every row of seqs [B, T] at positions `cols`:
    [B, len(cols), V] float64, rows split into `chunks` (default: the core count).
    keep: a dict that receives every converted layer (for a later cached-mode run
    through OracleModel._layers); by default each layer is dropped after use."""
    return _run(shape, params, prec, seqs, lambda om, h: om.lm_logits(h[:, list(cols)]), lora, lora_scale,
                chunks, np.concatenate, keep)


def reward_at_last(shape, params, prec, seqs: np.ndarray, chunks: Optional[int] = None):
    """The scalar head of a reward model at the last position of every row:
    (y [B, d_embed], reward [B]) float64."""
    return _run(shape, params, prec, seqs, lambda om, h: om.scalar_head(h[:, -1]), None, 1.0, chunks,
                lambda outs: tuple(np.concatenate(o) for o in zip(*outs)))


def _run(shape, params, prec, seqs, head, lora, lora_scale, chunks, join, keep=None, ahead=4):
    seqs = np.asarray(seqs)
    n = min(len(seqs), chunks or cores())
    parts = [p for p in np.array_split(seqs, n) if len(p)]
    shared = {} if keep is None else keep

    def model():
        om = O.OracleModel(shape, params, prec, lora=lora, lora_scale=lora_scale, cache_layers=True)
        om._layers = shared                    # one converted copy of each layer
        return om

    models = [model() for _ in parts]
    L = shape.n_layers
    with ThreadPoolExecutor(len(models)) as pool, ThreadPoolExecutor(ahead) as conv, threadpool_limits(1):
        # layers are converted (LoRA-folded) `ahead` at a time in the background
        pending = {i: conv.submit(model().layer, i) for i in range(min(ahead, L))}
        hs = list(pool.map(lambda a: a[0].embed(a[1], 0), zip(models, parts)))
        for i in range(L):
            pending.pop(i).result()
            if i + ahead < L:
                pending[i + ahead] = conv.submit(model().layer, i + ahead)
            hs = list(pool.map(lambda a: a[0].layer_forward(i, a[1], 0, None), zip(models, hs)))
            if keep is None:
                shared.pop(i)
        out = list(pool.map(lambda a: head(a[0], a[1]), zip(models, hs)))
    return join(out)

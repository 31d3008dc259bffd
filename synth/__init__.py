"""Seeded synthetic inputs for Hybrid-Engine experience generation.

This module draws random numbers and nothing else: it holds the model shapes
of the five workloads, draws the parameters, LoRA adapters, prompts and forced
token streams from a seed, and stores them in the model's storage type.  It
holds none of the method's arithmetic.  Both the CPU oracle and the GPU
library consume what it returns, and neither of them is imported here.

Every tensor is drawn from its own counter-style stream,
``numpy.random.Generator(PCG64(SeedSequence([seed, crc32(name), chunk])))``,
in fixed-size chunks, so any tensor (or chunk of one) can be regenerated alone
and large tensors are drawn by several threads at once.  Values are drawn in
float32; bf16 tensors are then converted with ``torch.Tensor.to(bfloat16)``
(round to nearest even).

Parameter recipe (the pages give none; see the configuration notes):
  * weight matrices, embeddings, position tables:  N(0, 0.02)
  * biases and LayerNorm beta:                     N(0, 0.02)
  * LayerNorm gamma:                               1 + N(0, 0.02)
  * LoRA A and B:                                  N(0, 0.02)  (B is not zero)
  * prompts and forced tokens:                     uniform integers in [0, V)
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

STD = 0.02
CHUNK = 1 << 22          # elements per independent stream chunk

PROJ_NAMES = ("q", "k", "v", "out", "fc1", "fc2")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape of one OPT-style decoder (actor or reward model)."""
    n_layers: int
    d_model: int
    n_heads: int
    d_ffn: int
    vocab: int
    max_pos: int                 # learned-position table has max_pos + 2 rows
    dtype: str                   # "fp32" or "bf16": storage type
    norm: str = "pre"            # "pre" (actor) or "post" (reward model)
    d_embed: int = 0             # word-embedding width; 0 means d_model
    head: str = "lm"             # "lm" (tied LM head) or "scalar" (reward head)

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def embed_dim(self) -> int:
        return self.d_embed or self.d_model

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


@dataclasses.dataclass(frozen=True)
class Workload:
    """One experience-generation workload: actor shape, LoRA, batch, lengths."""
    name: str
    actor: ModelShape
    lora_rank: int
    lora_alpha: float
    batch: int
    prompt_len: int
    gen_len: int
    max_seq: int
    reward: Optional[ModelShape] = None
    rounds: int = 1

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_rank


def _opt(L, d, H, F, max_pos=2048, dtype="bf16", V=50272):
    return ModelShape(n_layers=L, d_model=d, n_heads=H, d_ffn=F, vocab=V,
                      max_pos=max_pos, dtype=dtype)


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 decoder: 2 layers, d 64, 4 heads, FFN 256, vocab 512, 64 positions
    "tiny": Workload("tiny", _opt(2, 64, 4, 256, max_pos=64, dtype="fp32", V=512),
                     lora_rank=4, lora_alpha=8.0, batch=2, prompt_len=16,
                     gen_len=16, max_seq=32),
    "opt125m": Workload("opt125m", _opt(12, 768, 12, 3072), lora_rank=8,
                        lora_alpha=16.0, batch=16, prompt_len=256, gen_len=256,
                        max_seq=512),
    "opt1.3b": Workload("opt1.3b", _opt(24, 2048, 32, 8192), lora_rank=8,
                        lora_alpha=16.0, batch=32, prompt_len=256, gen_len=256,
                        max_seq=512),
    "opt6.7b": Workload("opt6.7b", _opt(32, 4096, 32, 16384), lora_rank=16,
                        lora_alpha=32.0, batch=64, prompt_len=256, gen_len=256,
                        max_seq=512),
    "opt13b": Workload("opt13b", _opt(40, 5120, 40, 20480), lora_rank=16,
                       lora_alpha=32.0, batch=128, prompt_len=256, gen_len=256,
                       max_seq=512,
                       reward=ModelShape(n_layers=24, d_model=1024, n_heads=16,
                                         d_ffn=4096, vocab=50272, max_pos=2048,
                                         dtype="bf16", norm="post", d_embed=512,
                                         head="scalar"),
                       rounds=2),
}


def _stream(seed: int, name: str, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, zlib.crc32(name.encode()), chunk])
    return np.random.Generator(np.random.PCG64(ss))


def _normal_f32(seed: int, name: str, n: int, pool: Optional[ThreadPoolExecutor]) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range((n + CHUNK - 1) // CHUNK)]

    def fill(item):
        c, a, b = item
        _stream(seed, name, c).standard_normal(b - a, dtype=np.float32, out=out[a:b])

    if pool is None or len(chunks) == 1:
        for item in chunks:
            fill(item)
    else:
        list(pool.map(fill, chunks))
    return out


def normal(seed: int, name: str, shape, std: float = STD, mean: float = 0.0,
           dtype=torch.bfloat16, pool: Optional[ThreadPoolExecutor] = None) -> torch.Tensor:
    """N(mean, std) tensor of ``shape`` in ``dtype`` (CPU), from stream ``name``."""
    n = int(np.prod(shape))
    x = _normal_f32(seed, name, n, pool)
    x *= np.float32(std)
    if mean:
        x += np.float32(mean)
    t = torch.from_numpy(x).reshape(shape)
    return t if dtype == torch.float32 else t.to(dtype)


def tokens(seed: int, name: str, shape, vocab: int) -> torch.Tensor:
    """Uniform int32 token ids in [0, vocab)."""
    g = _stream(seed, name, 0)
    return torch.from_numpy(g.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32))


def sample_logits(B: int, V: int, seed: int = 0, spread: float = 2.0, head: float = 1.1) -> torch.Tensor:
    """[B, V] float32 logits shaped like a language model's: N(0, spread) noise on a
    Zipf-like profile -head * log(1 + rank) over a seeded permutation of the columns
    (a few likely tokens, a long tail)."""
    g = _stream(seed, "logit_ranks", 0)
    rank = g.permutation(V).astype(np.float32)
    base = (-np.float32(head) * np.log1p(rank)).astype(np.float32)
    x = normal(seed, "logits", (B, V), std=spread, dtype=torch.float32).numpy()
    return torch.from_numpy((x + base[None, :]).astype(np.float32))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def model_params(shape: ModelShape, seed: int = 0, prefix: str = "") -> Dict[str, torch.Tensor]:
    """All parameters of an OPT-style decoder, as CPU tensors in the storage type.

    Names: ``E`` [V, d_embed], ``P`` [max_pos+2, d], ``lnf.g``/``lnf.b`` (pre-LN
    only), ``proj_in`` [d, d_embed] / ``proj_out`` [d_embed, d] (when d_embed !=
    d), ``score`` [d_embed] (scalar head), and per layer i: ``L{i}.ln1.g``,
    ``L{i}.ln1.b``, ``L{i}.qkv.w`` [3d, d] (rows q, then k, then v),
    ``L{i}.qkv.b`` [3d], ``L{i}.out.w`` [d, d], ``L{i}.out.b``, ``L{i}.ln2.g``,
    ``L{i}.ln2.b``, ``L{i}.fc1.w`` [F, d], ``L{i}.fc1.b`` [F], ``L{i}.fc2.w``
    [d, F], ``L{i}.fc2.b`` [d].  Linear weights are [out, in] row-major.
    """
    d, F, V, de = shape.d_model, shape.d_ffn, shape.vocab, shape.embed_dim
    dt = shape.torch_dtype
    p: Dict[str, torch.Tensor] = {}
    with ThreadPoolExecutor(_threads()) as pool:
        def w(name, shp, mean=0.0):
            p[name] = normal(seed, prefix + name, shp, mean=mean, dtype=dt, pool=pool)

        w("E", (V, de))
        w("P", (shape.max_pos + 2, d))
        if shape.norm == "pre":
            w("lnf.g", (d,), mean=1.0)
            w("lnf.b", (d,))
        if de != d:
            w("proj_in", (d, de))
            w("proj_out", (de, d))
        if shape.head == "scalar":
            w("score", (de,))
        for i in range(shape.n_layers):
            w(f"L{i}.ln1.g", (d,), mean=1.0)
            w(f"L{i}.ln1.b", (d,))
            w(f"L{i}.qkv.w", (3 * d, d))
            w(f"L{i}.qkv.b", (3 * d,))
            w(f"L{i}.out.w", (d, d))
            w(f"L{i}.out.b", (d,))
            w(f"L{i}.ln2.g", (d,), mean=1.0)
            w(f"L{i}.ln2.b", (d,))
            w(f"L{i}.fc1.w", (F, d))
            w(f"L{i}.fc1.b", (F,))
            w(f"L{i}.fc2.w", (d, F))
            w(f"L{i}.fc2.b", (d,))
    return p


def proj_dims(shape: ModelShape, proj: str):
    """(d_out, d_in) of an adapted projection."""
    d, F = shape.d_model, shape.d_ffn
    return {"q": (d, d), "k": (d, d), "v": (d, d), "out": (d, d),
            "fc1": (F, d), "fc2": (d, F)}[proj]


def lora_params(shape: ModelShape, rank: int, seed: int = 0,
                tag: str = "lora") -> Dict[str, torch.Tensor]:
    """LoRA pairs for q, k, v, out, fc1, fc2 of every layer.

    ``{tag}.L{i}.{proj}.A`` is [rank, d_in] and ``{tag}.L{i}.{proj}.B`` is
    [d_out, rank], both N(0, 0.02) in the storage type.
    """
    dt = shape.torch_dtype
    p: Dict[str, torch.Tensor] = {}
    with ThreadPoolExecutor(_threads()) as pool:
        for i in range(shape.n_layers):
            for proj in PROJ_NAMES:
                dout, din = proj_dims(shape, proj)
                base = f"{tag}.L{i}.{proj}"
                p[base + ".A"] = normal(seed, base + ".A", (rank, din), dtype=dt, pool=pool)
                p[base + ".B"] = normal(seed, base + ".B", (dout, rank), dtype=dt, pool=pool)
    return p


def prompts(wl: Workload, seed: int = 0, batch: Optional[int] = None) -> torch.Tensor:
    """[B, prompt_len] int32 prompt ids."""
    return tokens(seed, "prompts", (batch or wl.batch, wl.prompt_len), wl.actor.vocab)


def forced_tokens(wl: Workload, seed: int = 0, batch: Optional[int] = None) -> torch.Tensor:
    """[B, gen_len] int32 token stream fed in place of the model's own picks."""
    return tokens(seed, "forced", (batch or wl.batch, wl.gen_len), wl.actor.vocab)

"""Plain CPU oracle of Hybrid-Engine experience generation for an OPT actor.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  Nothing here is shared with
the GPU library, and nothing here imports it.

What it computes, and where the pages define it:

* LoRA folding -- "DeepSpeed-Chat: Easy, Fast and Affordable RLHF Training of
  ChatGPT-like Models at All Scales" (paper summary, page 1), section
  "Training Mode: ZeRO and LoRA Optimizations": a frozen W in R^{d x k} gets a
  trainable update B A with B in R^{d x r}, A in R^{r x k}.  The Hybrid
  Engine folds the adapter into the weight before generation and takes it out
  afterwards (DeepSpeed-Chat selection guide, page 2, section 3 "engine
  internals": fuse_lora_weight before generate, unfuse_lora_weight after).
  Reading: the update carries the usual scale s = alpha / r.
* Generation -- page 1, section "The Three-Step RLHF Training Pipeline in
  Algorithmic Detail", item 1 (generation phase): 256-token prompts, 256
  generated tokens per sequence, autoregressively.  Reading: greedy choice
  (argmax, lowest index on ties), fixed length, no stop token.
* KV cache -- page 1, section "Inference Mode: Generation Phase
  Optimizations", Optimization 2: the keys and values of earlier tokens are
  kept and the current step's are appended instead of recomputing the whole
  sequence.  The cached mode below does that; the definition mode recomputes
  the full sequence for every token, and the two must agree.
* Operator set -- page 2, section 3: the inference containers replace the
  transformer layer, Linear, Embedding, LayerNorm and the OPT positional
  embedding.  Architecture constants (pre-LN, ReLU FFN, learned positions
  with offset 2, tied LM head, and the post-LN reward model with a 512-wide
  embedding projection) follow the OPT family named on page 1, section
  "The Three-Step RLHF Training Pipeline in Algorithmic Detail" (OPT actors,
  OPT-350M reward model).

Everything is computed in float64.  ``Precision`` decides what happens at the
points where the GPU stores a value in its storage type: nothing ("fp64"),
rounding to float32 ("fp32") or rounding to bfloat16, ties to even ("bf16").
The bf16 storage points are: the fused weights; every GEMM input activation
(LayerNorm outputs, the attention output, the ReLU output, the final
normalised state); q after bias and scale; k and v as stored in the cache.
Accumulations, bias adds, the residual stream, LayerNorm statistics,
attention scores, softmax and logits stay wide.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

LN_EPS = 1e-5          # OPT's LayerNorm epsilon (the pages give none)
POS_OFFSET = 2         # OPT learned positions: row t + 2 for position t

_PROJ = ("q", "k", "v", "out", "fc1", "fc2")


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even; result in float64.

    bfloat16 keeps 8 significant bits and float32's exponent range.  For x in
    [2^(e-1), 2^e) the spacing is 2^(e-8); below 2^-126 the spacing stays
    2^-133 (subnormals).  Values at or above 2^128 after rounding overflow to
    infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    # Normal range: float64 keeps 52 fraction bits, bfloat16 7, so round the bit
    # pattern at bit 45, ties to even (add 2^44 - 1 plus the kept lowest bit, then
    # clear the 45 dropped bits; a carry moves into the exponent as it should).
    u = np.ascontiguousarray(x).view(np.uint64)
    keep_lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = ((u + (np.uint64((1 << 44) - 1) + keep_lsb)) & ~np.uint64((1 << 45) - 1)).view(np.float64)
    r = r.reshape(x.shape)
    ax = np.abs(x)
    odd = ((ax < 2.0 ** -126) & (ax > 0)) | (np.abs(r) >= 2.0 ** 128) | ~np.isfinite(x)
    if np.any(odd):
        xo = x[odd]
        _, e = np.frexp(xo)
        qe = np.maximum(e - 8, -133)
        ro = np.ldexp(np.rint(np.ldexp(xo, -qe)), qe)   # np.rint: half to even
        ro = np.where(np.abs(ro) >= 2.0 ** 128, np.copysign(np.inf, xo), ro)
        ro = np.where(np.isfinite(xo), ro, xo)
        r = r.copy()
        r[odd] = ro
    return r


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (2^-133 at zero)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def round_fp32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


class Precision:
    """Where values are rounded: "fp64" (never), "fp32" or "bf16"."""

    def __init__(self, kind: str):
        if kind not in ("fp64", "fp32", "bf16"):
            raise ValueError(kind)
        self.kind = kind

    def store(self, x) -> np.ndarray:
        if self.kind == "bf16":
            return round_bf16(x)
        if self.kind == "fp32":
            return round_fp32(x)
        return np.asarray(x, dtype=np.float64)

    def __repr__(self):
        return f"Precision({self.kind!r})"


def f64(t) -> np.ndarray:
    """A torch tensor or array as a float64 numpy array (bf16 widens exactly)."""
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


# ----------------------------------------------------------------------------
# LoRA (page 1, "Training Mode: ZeRO and LoRA Optimizations"; page 2, section 3)
# ----------------------------------------------------------------------------

def lora_delta(A: np.ndarray, B: np.ndarray, scale: float) -> np.ndarray:
    """The adapter's update s * B A, B [d_out, r], A [r, d_in], in float64."""
    return scale * (B @ A)


def lora_fuse(W, A, B, scale: float, prec: Precision) -> np.ndarray:
    """Fold the adapter into the weight: W' = store(W + s B A)."""
    return prec.store(f64(W) + lora_delta(f64(A), f64(B), scale))


def lora_unfuse(Wf, A, B, scale: float, prec: Precision) -> np.ndarray:
    """Take the adapter out again: W'' = store(W' - s B A), same update."""
    return prec.store(f64(Wf) - lora_delta(f64(A), f64(B), scale))


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------

def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = LN_EPS,
               wide=None) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the last axis, biased variance.

    ``wide`` (default None: nothing) is applied to the two statistics as they are
    formed; see OracleModel.wide."""
    mu = x.mean(axis=-1, keepdims=True)
    if wide is not None:
        mu = wide(mu)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    if wide is not None:
        var = wide(var)
    return (x - mu) / np.sqrt(var + eps) * g + b


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     q_pos0: int) -> Tuple[np.ndarray, np.ndarray]:
    """Causal softmax attention of one sequence.

    q: [H, Tq, D], already scaled by D^-1/2; k, v: [H, Tk, D].  Query i sits at
    absolute position q_pos0 + i and sees keys 0 .. q_pos0 + i.  Returns the
    output [H, Tq, D] and the probabilities [H, Tq, Tk]; masked entries are
    exactly zero.
    """
    Tq, Tk = q.shape[1], k.shape[1]
    s = q @ np.swapaxes(k, 1, 2)
    seen = np.arange(Tk)[None, :] <= (q_pos0 + np.arange(Tq))[:, None]
    s = np.where(seen[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v, p


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the largest value along the last axis; the lowest index wins ties."""
    logits = np.asarray(logits)
    m = logits.max(axis=-1, keepdims=True)
    hit = logits == m
    return hit.argmax(axis=-1).astype(np.int64)


# ----------------------------------------------------------------------------
# the decoder
# ----------------------------------------------------------------------------

class KVCache:
    """Per-layer keys and values of one batch: [L][B, H, S_max, D] float64."""

    def __init__(self, n_layers, B, H, S_max, D):
        self.k = [np.zeros((B, H, S_max, D)) for _ in range(n_layers)]
        self.v = [np.zeros((B, H, S_max, D)) for _ in range(n_layers)]
        self.length = 0


class OracleModel:
    """An OPT-style decoder whose adapted weights are W + s B A.

    ``params`` and ``lora`` are name -> tensor maps in the layout the seeded
    generator produces (Linear weights [out, in]; q, k, v packed as the rows of
    ``L{i}.qkv.w``).  With ``lora`` given, every adapted projection is folded
    (``lora_fuse``) before use; without it the base weights run.

    ``wide`` is None for the method itself.  For measuring how sensitive the result
    is to the last bits of the wide arithmetic (test infrastructure), it may be set
    to a function that is applied to every value an implementation forms by a
    float32 accumulation or add: the embedding sum, each projection's product
    before its bias, the attention output before it is stored, the LayerNorm
    statistics, the residual stream after each add, and the head's logits.
    """

    def __init__(self, shape, params: Dict, prec: Precision, lora: Optional[Dict] = None,
                 lora_scale: float = 1.0, lora_tag: str = "lora", cache_layers: bool = True,
                 eps: float = LN_EPS, fp8_decode: bool = False):
        self.shape = shape
        self.params = params
        self.prec = prec
        self.lora = lora
        self.lora_scale = lora_scale
        self.lora_tag = lora_tag
        self.eps = eps
        self.cache_layers = cache_layers
        self._layers: Dict[int, Dict[str, np.ndarray]] = {}
        self._glob: Dict[str, np.ndarray] = {}
        # weight-only FP8 for the decode steps' projections (oracle/fp8.py)
        self.fp8_decode = fp8_decode
        self._in_decode = False
        self._layers_q: Dict[int, Dict[str, np.ndarray]] = {}
        self.wide = None

    def _w(self, x: np.ndarray) -> np.ndarray:
        return x if self.wide is None else self.wide(x)

    # -- parameters -----------------------------------------------------------
    def g(self, name: str) -> np.ndarray:
        if name not in self._glob:
            self._glob[name] = f64(self.params[name])
        return self._glob[name]

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        if self.fp8_decode and self._in_decode:
            return self._layer_fp8(i)
        return self._layer_full(i)

    def _layer_fp8(self, i: int) -> Dict[str, np.ndarray]:
        """Layer i with its four projection weights replaced by their FP8 versions."""
        from oracle import fp8
        if i not in self._layers_q:
            lw = dict(self._layer_full(i))
            for name in ("qkv.w", "out.w", "fc1.w", "fc2.w"):
                lw[name] = fp8.fp8_weight(lw[name])
            if not self.cache_layers:
                return lw
            self._layers_q[i] = lw
        return self._layers_q[i]

    def _layer_full(self, i: int) -> Dict[str, np.ndarray]:
        if i in self._layers:
            return self._layers[i]
        d = self.shape.d_model
        p = self.params
        wqkv = f64(p[f"L{i}.qkv.w"])
        W = {"q": wqkv[:d], "k": wqkv[d:2 * d], "v": wqkv[2 * d:],
             "out": f64(p[f"L{i}.out.w"]), "fc1": f64(p[f"L{i}.fc1.w"]),
             "fc2": f64(p[f"L{i}.fc2.w"])}
        if self.lora is not None:
            for proj in _PROJ:
                base = f"{self.lora_tag}.L{i}.{proj}"
                W[proj] = lora_fuse(W[proj], self.lora[base + ".A"], self.lora[base + ".B"],
                                    self.lora_scale, self.prec)
        lw = {
            "ln1.g": f64(p[f"L{i}.ln1.g"]), "ln1.b": f64(p[f"L{i}.ln1.b"]),
            "qkv.w": np.concatenate([W["q"], W["k"], W["v"]], axis=0),
            "qkv.b": f64(p[f"L{i}.qkv.b"]),
            "out.w": W["out"], "out.b": f64(p[f"L{i}.out.b"]),
            "ln2.g": f64(p[f"L{i}.ln2.g"]), "ln2.b": f64(p[f"L{i}.ln2.b"]),
            "fc1.w": W["fc1"], "fc1.b": f64(p[f"L{i}.fc1.b"]),
            "fc2.w": W["fc2"], "fc2.b": f64(p[f"L{i}.fc2.b"]),
        }
        if self.cache_layers:
            self._layers[i] = lw
        return lw

    # -- pieces ---------------------------------------------------------------
    def embed(self, ids: np.ndarray, pos0: int) -> np.ndarray:
        """Token embedding plus learned position (row t + 2) -> [B, T, d]."""
        ids = np.asarray(ids)
        T = ids.shape[1]
        P = self.g("P")
        pos = P[pos0 + POS_OFFSET: pos0 + POS_OFFSET + T]
        if T and pos0 + POS_OFFSET + T > P.shape[0]:
            raise IndexError("position beyond the learned-position table")
        e = self.g("E")[ids]
        if "proj_in" in self.params:
            e = self.prec.store(e) @ self.g("proj_in").T
        return self._w(e + pos[None])

    def _attend(self, i: int, lw, x: np.ndarray, pos0: int,
                cache: Optional[KVCache]) -> np.ndarray:
        """Self-attention block on a bf16/fp32-stored input x [B, T, d]."""
        st = self.prec.store
        B, T, d = x.shape
        H, D = self.shape.n_heads, self.shape.head_dim
        qkv = self._w(x @ lw["qkv.w"].T) + lw["qkv.b"]
        q = st(qkv[..., :d] * (1.0 / np.sqrt(D)))
        k = st(qkv[..., d:2 * d])
        v = st(qkv[..., 2 * d:])
        q = q.reshape(B, T, H, D).transpose(0, 2, 1, 3)
        k = k.reshape(B, T, H, D).transpose(0, 2, 1, 3)
        v = v.reshape(B, T, H, D).transpose(0, 2, 1, 3)
        if cache is not None:
            cache.k[i][:, :, pos0:pos0 + T] = k
            cache.v[i][:, :, pos0:pos0 + T] = v
            k = cache.k[i][:, :, :pos0 + T]
            v = cache.v[i][:, :, :pos0 + T]
            kpos0 = pos0
        else:
            if pos0 != 0:
                raise ValueError("without a cache the block must start at position 0")
            kpos0 = 0
        o = np.empty((B, H, T, D))
        for b in range(B):
            o[b], _ = causal_attention(q[b], k[b], v[b], kpos0)
        o = st(self._w(o.transpose(0, 2, 1, 3).reshape(B, T, d)))
        return self._w(o @ lw["out.w"].T) + lw["out.b"]

    def _ffn(self, lw, x: np.ndarray) -> np.ndarray:
        a = self.prec.store(np.maximum(self._w(x @ lw["fc1.w"].T) + lw["fc1.b"], 0.0))
        return self._w(a @ lw["fc2.w"].T) + lw["fc2.b"]

    def layer_forward(self, i: int, h: np.ndarray, pos0: int,
                      cache: Optional[KVCache] = None) -> np.ndarray:
        """One decoder layer on the residual stream h [B, T, d] (float64)."""
        lw = self.layer(i)
        st = self.prec.store
        w = self._w
        if self.shape.norm == "pre":
            h = w(h + self._attend(i, lw, st(layer_norm(h, lw["ln1.g"], lw["ln1.b"], self.eps, self.wide)),
                                   pos0, cache))
            h = w(h + self._ffn(lw, st(layer_norm(h, lw["ln2.g"], lw["ln2.b"], self.eps, self.wide))))
        else:   # post-LN: normalise after each residual add; the normalised value is the stream
            h = layer_norm(w(h + self._attend(i, lw, st(h), pos0, cache)),
                           lw["ln1.g"], lw["ln1.b"], self.eps, self.wide)
            h = layer_norm(w(h + self._ffn(lw, st(h))), lw["ln2.g"], lw["ln2.b"], self.eps, self.wide)
        return h

    def hidden(self, ids, pos0: int = 0, cache: Optional[KVCache] = None) -> np.ndarray:
        h = self.embed(ids, pos0)
        for i in range(self.shape.n_layers):
            h = self.layer_forward(i, h, pos0, cache)
        return h

    def lm_logits(self, h: np.ndarray) -> np.ndarray:
        """Final LayerNorm, then the tied head: logits = z E^T."""
        z = self.prec.store(layer_norm(h, self.g("lnf.g"), self.g("lnf.b"), self.eps, self.wide))
        return self._w(z @ self.g("E").T)

    # -- the two modes ----------------------------------------------------------
    def forward_full(self, ids) -> np.ndarray:
        """Definition mode: logits [B, T, V] for every position, no cache."""
        return self.lm_logits(self.hidden(np.asarray(ids), 0, None))

    def prefill(self, ids, max_seq: int) -> Tuple[np.ndarray, KVCache]:
        """Cached mode, prompt pass: logits [B, V] at the last prompt position."""
        ids = np.asarray(ids)
        B, T = ids.shape
        cache = KVCache(self.shape.n_layers, B, self.shape.n_heads, max_seq, self.shape.head_dim)
        h = self.hidden(ids, 0, cache)
        cache.length = T
        return self.lm_logits(h[:, -1]), cache

    def decode(self, ids_step, cache: KVCache) -> np.ndarray:
        """Cached mode, one step: feed ids [B] at the next position, logits [B, V]."""
        ids = np.asarray(ids_step).reshape(-1, 1)
        pos = cache.length
        if pos >= cache.k[0].shape[2]:
            raise IndexError("KV cache full")
        self._in_decode = True
        try:
            h = self.hidden(ids, pos, cache)
        finally:
            self._in_decode = False
        cache.length = pos + 1
        return self.lm_logits(h[:, -1])

    # -- reward model -------------------------------------------------------------
    def score(self, ids) -> np.ndarray:
        """Scalar reward at the last position of each row: (h_last P_out^T) . w."""
        return self.score_y(ids)[1]

    def score_y(self, ids) -> Tuple[np.ndarray, np.ndarray]:
        """(y, reward): y = h_last P_out^T [B, d_embed] and reward = y . w [B]."""
        return self.scalar_head(self.hidden(np.asarray(ids), 0, None)[:, -1])

    def scalar_head(self, h_last: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """The reward head on the last position's stream [B, d]: (y, y . w)."""
        y = self.prec.store(h_last) @ self.g("proj_out").T
        return y, y @ self.g("score")


def greedy_generate(model: OracleModel, prompts, gen_len: int, max_seq: int,
                    forced=None, mode: str = "cached") -> Tuple[np.ndarray, List[np.ndarray]]:
    """Generate gen_len tokens per row.

    The first token comes from the prompt pass; step j = 1 .. gen_len-1 feeds
    token j-1 at position prompt_len + j - 1.  The fed token is the model's own
    previous pick, or ``forced[:, j-1]`` when a forced stream is given.
    Returns (picks [B, gen_len], logits per step [gen_len][B, V]).
    """
    prompts = np.asarray(prompts)
    B, S = prompts.shape
    picks = np.zeros((B, gen_len), dtype=np.int64)
    logits: List[np.ndarray] = []
    if mode == "cached":
        lg, cache = model.prefill(prompts, max_seq)
    elif mode == "definition":
        lg = model.forward_full(prompts)[:, -1]
        seq = prompts.astype(np.int64)
    else:
        raise ValueError(mode)
    logits.append(lg)
    picks[:, 0] = argmax_lowest(lg)
    for j in range(1, gen_len):
        fed = picks[:, j - 1] if forced is None else np.asarray(forced)[:, j - 1]
        if mode == "cached":
            lg = model.decode(fed, cache)
        else:
            seq = np.concatenate([seq, np.asarray(fed, dtype=np.int64)[:, None]], axis=1)
            lg = model.forward_full(seq)[:, -1]
        logits.append(lg)
        picks[:, j] = argmax_lowest(lg)
    return picks, logits

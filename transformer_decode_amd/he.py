"""ctypes binding of libhe (include/he.h): same names, argument marshalling only.

Every step of the path runs in the HIP kernels of ``libhe.so``; this module only
converts Python/torch arguments to the C ABI.  PyTorch provides device memory
and streams.  If the library has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# HE_LIB names another build of the same library (the host-side AddressSanitizer
# build of the CPU tests); by default the in-tree libhe.so
LIB_PATH = os.environ.get("HE_LIB") or os.path.join(_PKG, "libhe.so")

# status codes
HE_OK, HE_E_ARG, HE_E_STATE, HE_E_NOCACHE, HE_E_RANGE, HE_E_OOM, HE_E_HIP, HE_E_UNSUPPORTED = (
    0, -1, -2, -3, -4, -5, -6, -7)
HE_DTYPE_F32, HE_DTYPE_BF16 = 0, 1
HE_NORM_PRE, HE_NORM_POST = 0, 1
HE_HEAD_LM, HE_HEAD_SCALAR = 0, 1
HE_FLAG_VALIDATE_ONLY = 1
HE_PROJ_Q, HE_PROJ_K, HE_PROJ_V, HE_PROJ_OUT, HE_PROJ_FC1, HE_PROJ_FC2, HE_N_PROJ = range(7)
(HE_K_LORA, HE_K_EMBED_NORM, HE_K_GEMM_PREFILL, HE_K_ATTN_PREFILL, HE_K_GEMV_DECODE,
 HE_K_ATTN_DECODE, HE_K_LMHEAD, HE_K_SCORE, HE_K_VOCAB, HE_K_COUNT) = range(10)
HE_DBG_FAIL_NEXT_ALLOC, HE_DBG_FAIL_NEXT_STEP = 1, 2

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class he_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("d_model", _i32), ("n_heads", _i32), ("d_ffn", _i32),
                ("vocab", _i32), ("max_pos", _i32), ("dtype", _i32), ("norm", _i32),
                ("head", _i32), ("d_embed", _i32), ("ln_eps", ctypes.c_float),
                ("tp_size", _i32), ("use_graph", _i32), ("flags", _i32)]


class he_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_out", "b_out",
                                   "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class he_weight_table(ctypes.Structure):
    _fields_ = [("tok_emb", _vp), ("pos_emb", _vp), ("lnf_g", _vp), ("lnf_b", _vp),
                ("proj_in", _vp), ("proj_out", _vp), ("score_w", _vp),
                ("layers", ctypes.POINTER(he_layer_weights))]


class he_lora_pair(ctypes.Structure):
    _fields_ = [("A", _vp), ("B", _vp)]


class he_lora_table(ctypes.Structure):
    _fields_ = [("rank", _i32), ("alpha", ctypes.c_float), ("pairs", ctypes.POINTER(he_lora_pair))]


class he_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("seed", ctypes.c_uint64), ("top_p", ctypes.c_float)]


class he_kernel_stat(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


_lib = None

_SIGS = {
    "he_create": (_i32, [ctypes.POINTER(he_model_desc), ctypes.POINTER(he_weight_table), _vp,
                         ctypes.POINTER(_vp)]),
    "he_destroy": (_i32, [_vp]),
    "he_fuse_lora": (_i32, [_vp, ctypes.POINTER(he_lora_table)]),
    "he_unfuse_lora": (_i32, [_vp, ctypes.POINTER(he_lora_table)]),
    "he_retake_cache": (_i32, [_vp, _i32, _i32]),
    "he_release_cache": (_i32, [_vp]),
    "he_prefill": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "he_decode_step": (_i32, [_vp, _vp, _vp, _vp]),
    "he_generate": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "he_generate_ex": (_i32, [_vp, _vp, _i32, _i32, _i32, ctypes.POINTER(he_sampling), _vp, _vp]),
    "he_score": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "he_sample": (_i32, [_vp, _vp, _i32, _i32, ctypes.POINTER(he_sampling), _vp, _vp]),
    "he_sample_static": (_i32, [_vp, _vp, _i32, _i32, ctypes.POINTER(he_sampling), _vp, _vp]),
    "he_set_fp8_decode": (_i32, [_vp, _i32]),
    "he_fp8_export": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "he_logprobs": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "he_sync": (_i32, [_vp]),
    "he_last_error": (ctypes.c_char_p, [_vp]),
    "he_status_str": (ctypes.c_char_p, [_i32]),
    "he_kernel_timer": (_i32, [_vp, _i32, _i32]),
    "he_kernel_stats": (_i32, [_vp, _i32, ctypes.POINTER(he_kernel_stat)]),
    "he_build_info": (ctypes.c_char_p, []),
    "he_debug": (_i32, [_vp, _i32, ctypes.c_int64]),
}


def lib():
    """Load libhe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m transformer_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class HEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{lib().he_status_str(status).decode()}: {msg}")
        self.status = status


def _check(status: int, ctx) -> int:
    if status != HE_OK:
        msg = lib().he_last_error(ctx).decode() if ctx else ""
        raise HEError(status, msg)
    return status


# ---- the C ABI, name for name ------------------------------------------------------------

def he_create(desc: he_model_desc, table: he_weight_table, stream: int):
    out = _vp()
    _check(lib().he_create(ctypes.byref(desc), ctypes.byref(table), _vp(stream), ctypes.byref(out)), None)
    return out


def he_destroy(ctx):
    return lib().he_destroy(ctx)


def he_fuse_lora(ctx, table: he_lora_table):
    return _check(lib().he_fuse_lora(ctx, ctypes.byref(table)), ctx)


def he_unfuse_lora(ctx, table: he_lora_table):
    return _check(lib().he_unfuse_lora(ctx, ctypes.byref(table)), ctx)


def he_retake_cache(ctx, max_batch: int, max_seq: int):
    return _check(lib().he_retake_cache(ctx, max_batch, max_seq), ctx)


def he_release_cache(ctx):
    return _check(lib().he_release_cache(ctx), ctx)


def he_prefill(ctx, d_ids: int, B: int, S: int, d_next: int, d_logits: int = 0):
    return _check(lib().he_prefill(ctx, _vp(d_ids), B, S, _vp(d_next), _vp(d_logits or None)), ctx)


def he_decode_step(ctx, d_in: int, d_next: int, d_logits: int = 0):
    return _check(lib().he_decode_step(ctx, _vp(d_in), _vp(d_next), _vp(d_logits or None)), ctx)


def he_generate(ctx, d_prompt: int, B: int, S: int, S_g: int, d_out: int):
    return _check(lib().he_generate(ctx, _vp(d_prompt), B, S, S_g, _vp(d_out)), ctx)


def he_generate_ex(ctx, d_prompt: int, B: int, S: int, S_g: int, smp, d_out: int, d_logprobs: int = 0):
    """smp: he_sampling or None (greedy)."""
    p = ctypes.byref(smp) if smp is not None else None
    return _check(lib().he_generate_ex(ctx, _vp(d_prompt), B, S, S_g, p, _vp(d_out), _vp(d_logprobs or None)), ctx)


def he_sample(ctx, d_logits: int, B: int, position: int, smp, d_tokens: int, d_logprobs: int = 0):
    """smp: he_sampling or None (greedy)."""
    p = ctypes.byref(smp) if smp is not None else None
    return _check(lib().he_sample(ctx, _vp(d_logits), B, position, p, _vp(d_tokens), _vp(d_logprobs or None)), ctx)


def he_sample_static(ctx, d_logits: int, B: int, position: int, smp, d_tokens: int, d_logprobs: int = 0):
    """he_sample on the library's static device scratch: no workspace, no allocation."""
    p = ctypes.byref(smp) if smp is not None else None
    return _check(lib().he_sample_static(ctx, _vp(d_logits), B, position, p, _vp(d_tokens),
                                         _vp(d_logprobs or None)), ctx)


def he_set_fp8_decode(ctx, enable: bool):
    return _check(lib().he_set_fp8_decode(ctx, 1 if enable else 0), ctx)


def he_fp8_export(ctx, layer: int, proj: int, d_codes: int, d_scales: int):
    return _check(lib().he_fp8_export(ctx, layer, proj, _vp(d_codes), _vp(d_scales)), ctx)


def he_score(ctx, d_ids: int, B: int, S: int, d_reward: int, d_y: int = 0):
    return _check(lib().he_score(ctx, _vp(d_ids), B, S, _vp(d_reward), _vp(d_y)), ctx)


def he_logprobs(ctx, d_seq: int, B: int, S: int, S_p: int, d_logprobs: int):
    return _check(lib().he_logprobs(ctx, _vp(d_seq), B, S, S_p, _vp(d_logprobs)), ctx)


def he_sync(ctx):
    return _check(lib().he_sync(ctx), ctx)


def he_last_error(ctx) -> str:
    return lib().he_last_error(ctx).decode()


def he_status_str(s: int) -> str:
    return lib().he_status_str(s).decode()


def he_kernel_timer(ctx, kernel_class: int, enable: bool):
    return _check(lib().he_kernel_timer(ctx, kernel_class, int(bool(enable))), ctx)


def he_kernel_stats(ctx, kernel_class: int) -> he_kernel_stat:
    st = he_kernel_stat()
    _check(lib().he_kernel_stats(ctx, kernel_class, ctypes.byref(st)), ctx)
    return st


def he_build_info() -> str:
    return lib().he_build_info().decode()


def he_debug(ctx, what: int, value: int):
    return _check(lib().he_debug(ctx, what, value), ctx)


# ---- convenience: marshal a name -> tensor map into the tables ------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def model_desc(shape, use_graph: bool = True, flags: int = 0, ln_eps: float = 1e-5) -> he_model_desc:
    return he_model_desc(
        n_layers=shape.n_layers, d_model=shape.d_model, n_heads=shape.n_heads, d_ffn=shape.d_ffn,
        vocab=shape.vocab, max_pos=shape.max_pos,
        dtype=HE_DTYPE_F32 if shape.dtype == "fp32" else HE_DTYPE_BF16,
        norm=HE_NORM_PRE if shape.norm == "pre" else HE_NORM_POST,
        head=HE_HEAD_LM if shape.head == "lm" else HE_HEAD_SCALAR,
        d_embed=shape.embed_dim, ln_eps=ln_eps, tp_size=1, use_graph=int(use_graph), flags=flags)


def weight_table(shape, p: Dict) -> tuple:
    """(he_weight_table, keepalive) from the seeded generator's parameter names."""
    layers = (he_layer_weights * max(1, shape.n_layers))()
    for i in range(shape.n_layers):
        lw = layers[i]
        for field, name in (("ln1_g", "ln1.g"), ("ln1_b", "ln1.b"), ("w_qkv", "qkv.w"),
                            ("b_qkv", "qkv.b"), ("w_out", "out.w"), ("b_out", "out.b"),
                            ("ln2_g", "ln2.g"), ("ln2_b", "ln2.b"), ("w_fc1", "fc1.w"),
                            ("b_fc1", "fc1.b"), ("w_fc2", "fc2.w"), ("b_fc2", "fc2.b")):
            setattr(lw, field, _ptr(p[f"L{i}.{name}"]))
    t = he_weight_table(tok_emb=_ptr(p["E"]), pos_emb=_ptr(p["P"]), lnf_g=_ptr(p.get("lnf.g")),
                        lnf_b=_ptr(p.get("lnf.b")), proj_in=_ptr(p.get("proj_in")),
                        proj_out=_ptr(p.get("proj_out")), score_w=_ptr(p.get("score")),
                        layers=layers)
    return t, layers


def lora_table(shape, lora: Dict, rank: int, alpha: float, tag: str = "lora") -> tuple:
    pairs = (he_lora_pair * max(1, shape.n_layers * HE_N_PROJ))()
    names = ("q", "k", "v", "out", "fc1", "fc2")
    for i in range(shape.n_layers):
        for j, proj in enumerate(names):
            base = f"{tag}.L{i}.{proj}"
            if base + ".A" in lora:
                pairs[i * HE_N_PROJ + j] = he_lora_pair(_ptr(lora[base + ".A"]), _ptr(lora[base + ".B"]))
    return he_lora_table(rank=rank, alpha=alpha, pairs=pairs), pairs


class Engine:
    """One libhe context over device-resident parameters (a name -> tensor map).

    The tensors must stay alive and unmodified while the engine exists (the
    library borrows them); fuse/unfuse write the projection weights in place.
    All work runs on ``self.stream`` (a torch CUDA stream).
    """

    def __init__(self, shape, params: Dict, use_graph: bool = True, validate_only: bool = False,
                 stream=None):
        import torch
        self.shape = shape
        self.params = params
        self.validate_only = validate_only
        if validate_only:
            self.stream = None
            handle = 0
        else:
            self.stream = stream if stream is not None else torch.cuda.Stream()
            handle = self.stream.cuda_stream
        self.desc = model_desc(shape, use_graph=use_graph,
                               flags=HE_FLAG_VALIDATE_ONLY if validate_only else 0)
        self.table, self._keep = weight_table(shape, params)
        self.ctx = he_create(self.desc, self.table, handle)

    def close(self):
        if self.ctx:
            he_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lora(self, lora: Dict, rank: int, alpha: float, tag: str = "lora"):
        return lora_table(self.shape, lora, rank, alpha, tag)

    def sync(self):
        he_sync(self.ctx)

"""Host-side checks of the C ABI: the library loads, exports every declared call,
and its argument and state checks behave as documented (validate-only contexts,
which make no GPU calls at all)."""
import ctypes
import os
import re

import pytest

import synth
from transformer_decode_amd import he

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(he.LIB_PATH):
        from transformer_decode_amd import build
        build.build(verbose=False)
    return he.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "he.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(he_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_call():
    names = _declared()
    assert "he_generate" in names and "he_generate_ex" in names and "he_fuse_lora" in names
    assert "he_logprobs" in names and "he_sample" in names
    assert len(names) >= 20
    L = ctypes.CDLL(he.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_build_info_names_gfx950():
    assert "gfx950" in he.he_build_info()


def test_status_strings():
    assert he.he_status_str(he.HE_E_NOCACHE) == "HE_E_NOCACHE"
    assert he.he_status_str(0) == "HE_OK"


# ---- validate-only contexts: fake but non-null device pointers, no GPU work -------------

class _Fake:
    """Stands in for a tensor: only data_ptr() is read, never dereferenced."""
    def __init__(self, p):
        self.p = p

    def data_ptr(self):
        return self.p


def _fake_params(shape):
    names = ["E", "P", "lnf.g", "lnf.b"]
    if shape.embed_dim != shape.d_model:
        names += ["proj_in", "proj_out"]
    if shape.head == "scalar":
        names += ["score"]
    for i in range(shape.n_layers):
        names += [f"L{i}.{n}" for n in ("ln1.g", "ln1.b", "qkv.w", "qkv.b", "out.w", "out.b",
                                        "ln2.g", "ln2.b", "fc1.w", "fc1.b", "fc2.w", "fc2.b")]
    return {n: _Fake(0x10000 + 0x100 * k) for k, n in enumerate(names)}


def _fake_lora(shape):
    out = {}
    for i in range(shape.n_layers):
        for p in synth.PROJ_NAMES:
            out[f"lora.L{i}.{p}.A"] = _Fake(0x90000 + 0x100 * i)
            out[f"lora.L{i}.{p}.B"] = _Fake(0xa0000 + 0x100 * i)
    return out


def _engine(shape=None):
    shape = shape or synth.WORKLOADS["tiny"].actor
    return he.Engine(shape, _fake_params(shape), validate_only=True)


def _status(fn, *a):
    try:
        fn(*a)
        return he.HE_OK
    except he.HEError as e:
        return e.status


def test_state_machine_generation_cycle():
    wl = synth.WORKLOADS["tiny"]
    e = _engine()
    ctx, P = e.ctx, 0x1234
    lt, _k = e.lora(_fake_lora(wl.actor), wl.lora_rank, wl.lora_alpha)
    # nothing before the workspace
    assert _status(he.he_prefill, ctx, P, 2, 16, P) == he.HE_E_NOCACHE
    assert _status(he.he_decode_step, ctx, P, P) == he.HE_E_NOCACHE
    assert _status(he.he_generate, ctx, P, 2, 16, 16, P) == he.HE_E_NOCACHE
    # fuse / unfuse pairing
    assert _status(he.he_unfuse_lora, ctx, lt) == he.HE_E_STATE
    he.he_fuse_lora(ctx, lt)
    assert _status(he.he_fuse_lora, ctx, lt) == he.HE_E_STATE
    he.he_retake_cache(ctx, 2, 32)
    assert _status(he.he_retake_cache, ctx, 2, 32) == he.HE_E_STATE
    # decode before prefill
    assert _status(he.he_decode_step, ctx, P, P) == he.HE_E_STATE
    he.he_prefill(ctx, P, 2, 16, P)
    for _ in range(16):
        he.he_decode_step(ctx, P, P)
    assert _status(he.he_decode_step, ctx, P, P) == he.HE_E_RANGE     # position 32 == max_seq
    he.he_generate(ctx, P, 2, 16, 17, P)                               # 16 + 17 - 1 = 32 fits
    assert _status(he.he_generate, ctx, P, 2, 16, 18, P) == he.HE_E_RANGE
    he.he_unfuse_lora(ctx, lt)
    he.he_generate(ctx, P, 2, 16, 16, P)                               # base weights, unfused
    he.he_release_cache(ctx)
    he.he_release_cache(ctx)                                           # no-op
    assert _status(he.he_decode_step, ctx, P, P) == he.HE_E_NOCACHE
    e.close()


def test_top_p_vocabulary_limit():
    """The nucleus kernel holds a row of at most 53248 logits in registers."""
    import dataclasses
    shape = dataclasses.replace(synth.WORKLOADS["opt125m"].actor, n_layers=1, vocab=53264)
    e = he.Engine(shape, _fake_params(shape), validate_only=True)
    ctx, P = e.ctx, 0x1234
    he.he_retake_cache(ctx, 2, 32)
    assert _status(he.he_generate_ex, ctx, P, 2, 16, 8, he.he_sampling(0.7, 1, 0.9), P, P) == he.HE_E_UNSUPPORTED
    he.he_generate_ex(ctx, P, 2, 16, 8, he.he_sampling(0.7, 1, 1.0), P, P)     # top-p off: fine
    e.close()


def test_unsupported_bf16_decode_shapes():
    """bf16 generation models need d and d_ffn divisible by 128 and vocab by 16."""
    import dataclasses
    base = synth.WORKLOADS["opt125m"].actor
    for bad in (dict(vocab=50270), dict(d_model=800, n_heads=10), dict(d_ffn=3104)):
        shape = dataclasses.replace(base, n_layers=1, **bad)
        with pytest.raises(he.HEError) as ei:
            he.Engine(shape, _fake_params(shape), validate_only=True)
        assert ei.value.status == he.HE_E_UNSUPPORTED


def test_argument_checks():
    e = _engine()
    ctx, P = e.ctx, 0x1234
    assert _status(he.he_retake_cache, ctx, 0, 32) == he.HE_E_ARG
    assert _status(he.he_retake_cache, ctx, 2, 65) == he.HE_E_RANGE   # 64 learned positions
    he.he_retake_cache(ctx, 2, 32)
    assert _status(he.he_prefill, ctx, P, 3, 16, P) == he.HE_E_ARG    # batch > max_batch
    assert _status(he.he_prefill, ctx, P, 0, 16, P) == he.HE_E_ARG
    assert _status(he.he_prefill, ctx, P, 2, 0, P) == he.HE_E_ARG
    assert _status(he.he_prefill, ctx, P, 2, 33, P) == he.HE_E_RANGE
    assert _status(he.he_prefill, ctx, 0, 2, 16, P) == he.HE_E_ARG    # NULL ids
    assert _status(he.he_score, ctx, P, 2, 16, P) == he.HE_E_UNSUPPORTED
    assert _status(he.he_generate, ctx, P, 2, 16, 0, P) == he.HE_E_ARG
    # sampled generation: temperature must be finite and >= 0; NULL rule = greedy
    for t in (-0.5, float("nan"), float("inf"), 1e-45):
        assert _status(he.he_generate_ex, ctx, P, 2, 16, 8, he.he_sampling(t, 1), P, P) == he.HE_E_ARG
    he.he_generate_ex(ctx, P, 2, 16, 8, None, P, P)
    he.he_generate_ex(ctx, P, 2, 16, 8, he.he_sampling(0.7, 123), P, 0)
    assert _status(he.he_generate_ex, ctx, P, 2, 16, 18, he.he_sampling(1.0, 1), P, P) == he.HE_E_RANGE
    assert _status(he.he_generate_ex, ctx, 0, 2, 16, 8, he.he_sampling(1.0, 1), P, P) == he.HE_E_ARG
    # top-p: negative or NaN rejected; 0 and >= 1 mean off
    for tp in (-0.1, float("nan")):
        assert _status(he.he_generate_ex, ctx, P, 2, 16, 8, he.he_sampling(0.7, 1, tp), P, P) == he.HE_E_ARG
    for tp in (0.0, 0.9, 1.0, 5.0):
        he.he_generate_ex(ctx, P, 2, 16, 8, he.he_sampling(0.7, 1, tp), P, P)
    # sampling caller logits
    he.he_sample(ctx, P, 2, 0, None, P, 0)
    he.he_sample(ctx, P, 1, 31, he.he_sampling(0.8, 3, 0.5), P, P)
    for args, st in (((0, 2, 5, None, P, 0), he.HE_E_ARG), ((P, 2, 5, None, 0, 0), he.HE_E_ARG),
                     ((P, 3, 5, None, P, 0), he.HE_E_ARG), ((P, 2, -1, None, P, 0), he.HE_E_ARG),
                     ((P, 2, 5, he.he_sampling(-1.0, 0), P, 0), he.HE_E_ARG)):
        assert _status(he.he_sample, ctx, *args) == st, args
    # teacher-forced scoring: 1 <= S_p < S <= max_seq, buffers non-NULL
    he.he_logprobs(ctx, P, 2, 32, 16, P)
    he.he_logprobs(ctx, P, 1, 2, 1, P)
    for args, st in (((P, 2, 32, 0, P), he.HE_E_ARG), ((P, 2, 32, 32, P), he.HE_E_ARG),
                     ((P, 2, 33, 16, P), he.HE_E_RANGE), ((P, 3, 32, 16, P), he.HE_E_ARG),
                     ((0, 2, 32, 16, P), he.HE_E_ARG), ((P, 2, 32, 16, 0), he.HE_E_ARG)):
        assert _status(he.he_logprobs, ctx, *args) == st, args
    bad = he.he_lora_table(rank=0, alpha=1.0, pairs=(he.he_lora_pair * 12)())
    assert _status(he.he_fuse_lora, ctx, bad) == he.HE_E_ARG
    assert "rank" in he.he_last_error(ctx)
    e.close()


def test_create_rejects_bad_descriptions():
    shape = synth.WORKLOADS["tiny"].actor
    params = _fake_params(shape)
    table, keep = he.weight_table(shape, params)
    d = he.model_desc(shape, flags=he.HE_FLAG_VALIDATE_ONLY)
    d.tp_size = 2
    with pytest.raises(he.HEError) as ei:
        he.he_create(d, table, 0)
    assert ei.value.status == he.HE_E_UNSUPPORTED
    d = he.model_desc(shape, flags=he.HE_FLAG_VALIDATE_ONLY)
    d.n_heads = 3                                   # 64 % 3 != 0
    with pytest.raises(he.HEError):
        he.he_create(d, table, 0)
    d = he.model_desc(shape, flags=he.HE_FLAG_VALIDATE_ONLY)
    table.tok_emb = None
    with pytest.raises(he.HEError) as ei:
        he.he_create(d, table, 0)
    assert ei.value.status == he.HE_E_ARG


def test_injected_allocation_failure_then_retake():
    e = _engine()
    he.he_debug(e.ctx, he.HE_DBG_FAIL_NEXT_ALLOC, 1)
    assert _status(he.he_retake_cache, e.ctx, 2, 32) == he.HE_E_OOM
    he.he_retake_cache(e.ctx, 2, 32)                 # the next attempt succeeds
    e.close()


def test_injected_step_failure_leaves_unfuse_and_release():
    wl = synth.WORKLOADS["tiny"]
    e = _engine()
    ctx, P = e.ctx, 0x1234
    lt, _k = e.lora(_fake_lora(wl.actor), wl.lora_rank, wl.lora_alpha)
    he.he_fuse_lora(ctx, lt)
    he.he_retake_cache(ctx, 2, 32)
    he.he_debug(ctx, he.HE_DBG_FAIL_NEXT_STEP, 1)
    assert _status(he.he_generate, ctx, P, 2, 16, 16, P) == he.HE_E_HIP
    # failed state: compute calls refuse, unfuse and release still run
    assert _status(he.he_prefill, ctx, P, 2, 16, P) == he.HE_E_HIP
    assert _status(he.he_fuse_lora, ctx, lt) == he.HE_E_HIP
    he.he_unfuse_lora(ctx, lt)
    he.he_release_cache(ctx)
    e.close()


def test_reward_model_only_scores():
    wl = synth.WORKLOADS["opt13b"]
    e = _engine(wl.reward)
    ctx, P = e.ctx, 0x1234
    he.he_retake_cache(ctx, 128, 512)
    he.he_score(ctx, P, 128, 512, P, P)
    assert _status(he.he_prefill, ctx, P, 2, 16, P) == he.HE_E_UNSUPPORTED
    assert _status(he.he_logprobs, ctx, P, 2, 16, 8, P) == he.HE_E_UNSUPPORTED
    assert _status(he.he_sample, ctx, P, 2, 0, None, P, 0) == he.HE_E_UNSUPPORTED
    assert _status(he.he_score, ctx, P, 129, 512, P) == he.HE_E_ARG
    e.close()


def test_fp8_decode_switch():
    """Weight-only FP8 decode: bf16 LM-head models with d and d_ffn divisible by 256;
    the export needs it on and a layer / projection in range."""
    import dataclasses
    P = 0x1234
    shape = dataclasses.replace(synth.WORKLOADS["opt125m"].actor, n_layers=2)
    e = he.Engine(shape, _fake_params(shape), validate_only=True)
    ctx = e.ctx
    assert _status(he.he_fp8_export, ctx, 0, 0, P, P) == he.HE_E_STATE
    he.he_set_fp8_decode(ctx, True)
    he.he_fp8_export(ctx, 1, 3, P, P)
    for args in ((2, 0, P, P), (0, 4, P, P), (-1, 0, P, P), (0, 0, 0, P), (0, 0, P, 0)):
        assert _status(he.he_fp8_export, ctx, *args) == he.HE_E_ARG, args
    he.he_set_fp8_decode(ctx, False)
    assert _status(he.he_fp8_export, ctx, 0, 0, P, P) == he.HE_E_STATE
    e.close()
    # a refused switch changes nothing: the prompt pass still stands for a decode step
    tiny = synth.WORKLOADS["tiny"].actor
    e = he.Engine(tiny, _fake_params(tiny), validate_only=True)
    he.he_retake_cache(e.ctx, 2, 32)
    he.he_prefill(e.ctx, P, 2, 16, P)
    assert _status(he.he_set_fp8_decode, e.ctx, True) == he.HE_E_UNSUPPORTED
    he.he_decode_step(e.ctx, P, P, 0)
    e.close()
    for bad in (synth.WORKLOADS["tiny"].actor,                                          # fp32
                dataclasses.replace(shape, d_model=640, n_heads=10),                     # d % 256
                dataclasses.replace(shape, d_ffn=2944),                                  # d_ffn % 256
                synth.WORKLOADS["opt13b"].reward):                                       # scalar head
        e = he.Engine(bad, _fake_params(bad), validate_only=True)
        assert _status(he.he_set_fp8_decode, e.ctx, True) == he.HE_E_UNSUPPORTED, bad
        e.close()

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.  Tolerances: fp32 workload 1e-3 relative on logits, bf16 workloads
3e-2 absolute on logits, greedy picks identical wherever the oracle's top-2 gap
exceeds 1e-2, LoRA fold/unfold within one bf16 spacing."""
import numpy as np
import pytest
import torch

import synth
from oracle import opt_he as O
from transformer_decode_amd import he

from gpu_util import (GpuRun, check_logits, greedy_prefix_agrees, log, precision)
from layout import from_inference, to_inference

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
C2 = synth.WORKLOADS["opt125m"]


def _oracle(wl, params, lora, cache_layers=True):
    return O.OracleModel(wl.actor, params, precision(wl.actor), lora=lora,
                         lora_scale=wl.lora_scale, cache_layers=cache_layers)


# ------------------------------------------------------------------------------------
# LoRA fold / unfold
# ------------------------------------------------------------------------------------

def _fused_ref(wl, params, lora, i, key, prec):
    """The oracle's folded weight for one stored matrix (q, k, v packed in qkv.w)."""
    d = wl.actor.d_model
    W = params[f"L{i}.{key}"]
    if key == "qkv.w":
        return np.concatenate([
            O.lora_fuse(W[j * d:(j + 1) * d], lora[f"lora.L{i}.{p}.A"], lora[f"lora.L{i}.{p}.B"],
                        wl.lora_scale, prec) for j, p in enumerate(("q", "k", "v"))], axis=0)
    p = key.split(".")[0]
    return O.lora_fuse(W, lora[f"lora.L{i}.{p}.A"], lora[f"lora.L{i}.{p}.B"], wl.lora_scale, prec)


def _fused_ref_abs(wl, lora, i, key):
    """|B| |A| for the adapters of one stored matrix (float32 error scale of the update)."""
    def one(p):
        A = lora[f"lora.L{i}.{p}.A"].double().abs().numpy()
        B = lora[f"lora.L{i}.{p}.B"].double().abs().numpy()
        return B @ A
    if key == "qkv.w":
        return np.concatenate([one(p) for p in ("q", "k", "v")], axis=0)
    return one(key.split(".")[0])


@pytest.mark.parametrize("name", ["tiny", "opt125m"])
def test_lora_fuse_and_unfuse(name):
    wl = synth.WORKLOADS[name]
    log(f"lora fuse/unfuse {name}")
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    prec = precision(wl.actor)
    keys = ("qkv.w", "out.w", "fc1.w", "fc2.w")
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_sync(run.ctx)
    fused_ref = {}
    bf = wl.actor.dtype == "bf16"
    if bf:   # the tied embedding (LM head weight) only changes layout
        E0 = params["E"].double().numpy()
        assert np.array_equal(run.dev["E"].double().cpu().numpy(), to_inference(E0))
    for i in range(wl.actor.n_layers):
        for key in keys:
            ref = _fused_ref(wl, params, lora, i, key, prec)
            fused_ref[i, key] = ref
            got = run.dev[f"L{i}.{key}"].double().cpu().numpy()
            if bf:   # bf16 weights are held in the inference layout while fused
                got = from_inference(got)
            if wl.actor.dtype == "bf16":
                # The oracle rounds W + s B A once from the exact sum; the kernel sums the
                # rank-r update in float32 (error <= r 2^-24 s (|B| |A|)), adds it to W in
                # float32 (2^-24 |W'|) and rounds to bf16.  So one bf16 spacing plus the
                # float32 terms, which only matter where W and s B A nearly cancel.
                Wabs = _fused_ref_abs(wl, lora, i, key)
                bound = O.ulp_bf16(ref) + wl.lora_rank * 2.0 ** -24 * wl.lora_scale * Wabs \
                    + 2.0 ** -24 * np.abs(ref)
                assert (np.abs(got - ref) <= bound).all(), f"L{i}.{key} fused beyond the bound"
                assert (got != ref).mean() < 1e-3, f"L{i}.{key}: too many 1-ulp differences"
            else:
                np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)
    with torch.cuda.stream(run.stream):
        he.he_unfuse_lora(run.ctx, lt)
        he.he_sync(run.ctx)
    if bf:
        assert np.array_equal(run.dev["E"].double().cpu().numpy(), E0)
    for i in range(wl.actor.n_layers):
        for key in keys:
            W0 = params[f"L{i}.{key}"].double().numpy()
            Wr = run.dev[f"L{i}.{key}"].double().cpu().numpy()
            if wl.actor.dtype == "bf16":
                bound = O.ulp_bf16(np.maximum(np.abs(W0), np.abs(fused_ref[i, key])))
                assert (np.abs(Wr - W0) <= bound).all(), f"L{i}.{key} round trip beyond 1 ulp"
                assert (Wr == W0).mean() > 0.8, f"L{i}.{key}: too few bit-exact elements"
            else:
                np.testing.assert_allclose(Wr, W0, rtol=0, atol=1e-6)
    run.close()


# ------------------------------------------------------------------------------------
# tiny fp32 workload
# ------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_inputs():
    params = synth.model_params(TINY.actor)
    lora = synth.lora_params(TINY.actor, TINY.lora_rank)
    return params, lora, synth.prompts(TINY), synth.forced_tokens(TINY)


def test_tiny_teacher_forced_logits(tiny_inputs):
    params, lora, prompts, forced = tiny_inputs
    log("tiny teacher-forced")
    om = _oracle(TINY, params, lora)
    _, ref = O.greedy_generate(om, prompts.numpy(), TINY.gen_len, TINY.max_seq, forced=forced.numpy())
    run = GpuRun(TINY, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, TINY.batch, TINY.max_seq)
    got = run.teacher_forced(prompts, forced, TINY.gen_len)
    for j in range(TINY.gen_len):
        check_logits(got[j], ref[j], TINY.actor, f"step {j}")
    run.close()


def test_tiny_generate_matches_oracle(tiny_inputs):
    params, lora, prompts, _ = tiny_inputs
    om = _oracle(TINY, params, lora)
    picks, lg = O.greedy_generate(om, prompts.numpy(), TINY.gen_len, TINY.max_seq)
    for use_graph in (True, False):
        run = GpuRun(TINY, params, use_graph=use_graph)
        lt = run.lora(lora)
        with torch.cuda.stream(run.stream):
            he.he_fuse_lora(run.ctx, lt)
            he.he_retake_cache(run.ctx, TINY.batch, TINY.max_seq)
        got = run.generate(prompts, TINY.gen_len)
        n = greedy_prefix_agrees(got, picks, lg)
        assert n >= TINY.batch * 4
        run.close()


# ------------------------------------------------------------------------------------
# OPT-125m shape, bf16
# ------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c2_inputs():
    params = synth.model_params(C2.actor)
    lora = synth.lora_params(C2.actor, C2.lora_rank)
    return params, lora, synth.prompts(C2), synth.forced_tokens(C2)


ROWS_C2 = [0, 7, 15]


def test_opt125m_teacher_forced_logits(c2_inputs):
    params, lora, prompts, forced = c2_inputs
    log("opt125m teacher-forced: GPU")
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, C2.batch, C2.max_seq)
    steps = [0, 1, 2, 64, 128, 200, 255]
    got = run.teacher_forced(prompts, forced, C2.gen_len, want_rows=ROWS_C2, want_steps=set(steps))
    run.close()
    log("opt125m teacher-forced: oracle")
    om = _oracle(C2, params, lora)
    seq = np.concatenate([prompts.numpy()[ROWS_C2], forced.numpy()[ROWS_C2, :C2.gen_len - 1]], axis=1)
    full = om.forward_full(seq)                        # logits after every prefix
    S = C2.prompt_len
    worst = 0.0
    for j in steps:
        worst = max(worst, check_logits(got[j], full[:, S - 1 + j], C2.actor, f"step {j}"))
    log(f"opt125m max |dlogit| {worst:.3e}")


def test_opt125m_generate_greedy(c2_inputs):
    params, lora, prompts, _ = c2_inputs
    log("opt125m greedy: GPU")
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, C2.batch, C2.max_seq)
    got = run.generate(prompts, C2.gen_len)
    got2 = run.generate(prompts, C2.gen_len)
    assert np.array_equal(got, got2), "generation is not deterministic"
    run.close()
    run = GpuRun(C2, params, use_graph=False)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, C2.batch, C2.max_seq)
    got3 = run.generate(prompts, C2.gen_len)
    run.close()
    assert np.array_equal(got, got3), "graph replay differs from direct launches"
    log("opt125m greedy: oracle (3 rows, 64 steps)")
    om = _oracle(C2, params, lora)
    G = 64
    picks, lg = O.greedy_generate(om, prompts.numpy()[ROWS_C2], G, C2.max_seq)
    n = greedy_prefix_agrees(got[ROWS_C2, :G], picks, lg)
    log(f"opt125m greedy: {n} picks compared")
    assert n >= 8


def test_opt125m_unfused_base_weights(c2_inputs):
    """Generation with the adapters not folded runs the base weights (row-major):
    first a folded run captures the decode graph in the inference layout, then after
    the unfold the same context must re-capture and match the adapter-free oracle."""
    params, lora, prompts, forced = c2_inputs
    log("opt125m unfused: GPU")
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_retake_cache(run.ctx, C2.batch, C2.max_seq)
        he.he_fuse_lora(run.ctx, lt)
    run.generate(prompts, 8)
    with torch.cuda.stream(run.stream):
        he.he_unfuse_lora(run.ctx, lt)
    steps = [0, 1, 100, 255]
    got = run.teacher_forced(prompts, forced, C2.gen_len, want_rows=ROWS_C2, want_steps=set(steps))
    run.close()
    log("opt125m unfused: oracle without adapters")
    om = _oracle(C2, params, None)
    seq = np.concatenate([prompts.numpy()[ROWS_C2], forced.numpy()[ROWS_C2, :C2.gen_len - 1]], axis=1)
    full = om.forward_full(seq)
    S = C2.prompt_len
    for j in steps:
        check_logits(got[j], full[:, S - 1 + j], C2.actor, f"unfused step {j}")


def test_opt125m_ragged_prompt_pass(c2_inputs):
    """A prompt pass whose B*S is a multiple of neither 16 nor 256 (3 x 37 = 111 rows):
    the projections run the small-tile GEMM on activations in the inference layout with
    a partial last 16-row block; then two decode steps at batch 3."""
    params, lora, prompts, forced = c2_inputs
    B, S = 3, 37
    ids, fc = prompts[:B, :S].contiguous(), forced[:B].contiguous()
    log("opt125m ragged prompt pass: GPU")
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, C2.batch, C2.max_seq)
    got = run.teacher_forced(ids, fc, 3)
    run.close()
    log("opt125m ragged prompt pass: oracle")
    om = _oracle(C2, params, lora)
    seq = np.concatenate([ids.numpy(), fc.numpy()[:, :2]], axis=1)
    full = om.forward_full(seq)
    for j in range(3):
        check_logits(got[j], full[:, S - 1 + j], C2.actor, f"ragged step {j}")


def test_opt125m_debug_mode_waits_after_every_launch(c2_inputs, monkeypatch):
    """HE_DEBUG=1 (read at he_create): every launch is followed by a stream wait and an
    error check, graph replay is off.  A generation, a teacher-forced step with logits
    and a scoring pass then give the same bits as the ordinary graph-replayed run."""
    params, lora, prompts, forced = c2_inputs
    B, S, G = C2.batch, C2.prompt_len, 12
    outs = {}
    for mode in ("normal", "debug"):
        if mode == "debug":
            monkeypatch.setenv("HE_DEBUG", "1")
        run = GpuRun(C2, params)
        monkeypatch.delenv("HE_DEBUG", raising=False)
        lt = run.lora(lora)
        with torch.cuda.stream(run.stream):
            he.he_fuse_lora(run.ctx, lt)
            he.he_retake_cache(run.ctx, B, C2.max_seq)
        gen = run.generate(prompts, G)
        lg = run.teacher_forced(prompts, forced, 3, want_steps={2})[2]
        seq = torch.cat([prompts, forced[:, :8]], dim=1).to(torch.int32).cuda()
        lp = torch.empty(B, 8, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(run.stream):
            he.he_logprobs(run.ctx, seq.data_ptr(), B, S + 8, S, lp.data_ptr())
            he.he_sync(run.ctx)
        outs[mode] = (gen, lg, lp.cpu().numpy())
        run.close()
    log("debug mode: generation, logits and log-probabilities compared bit for bit")
    assert np.array_equal(outs["normal"][0], outs["debug"][0])
    assert np.array_equal(outs["normal"][1].view(np.uint32), outs["debug"][1].view(np.uint32))
    assert np.array_equal(outs["normal"][2].view(np.uint32), outs["debug"][2].view(np.uint32))


def test_opt125m_wide_ragged_batch(c2_inputs):
    """A batch of 100 rows: decode runs the plans for 65-128 rows (activation tiles of
    128 rows, 100 live; three or four weight fragments per wave, the last fragment group
    clamped at the matrix edge) and the prompt pass a 6400-row GEMM.  Teacher-forced
    logits on rows {0, 63, 64, 99} against the oracle, then free-running greedy picks on
    rows {0, 99} and graph replay against direct launches."""
    params, lora, _, _ = c2_inputs
    B, S, G = 100, 64, 16
    prompts = synth.tokens(0, "wide.prompts", (B, S), C2.actor.vocab)
    forced = synth.tokens(0, "wide.forced", (B, G), C2.actor.vocab)
    rows = [0, 63, 64, 99]
    log("opt125m batch 100: GPU")
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, B, S + G)
    steps = [0, 1, 8, 15]
    got = run.teacher_forced(prompts, forced, G, want_rows=rows, want_steps=set(steps))
    gen = run.generate(prompts, G)
    run.close()
    run = GpuRun(C2, params, use_graph=False)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, B, S + G)
    gen2 = run.generate(prompts, G)
    run.close()
    assert np.array_equal(gen, gen2), "graph replay differs from direct launches"
    log("opt125m batch 100: oracle")
    om = _oracle(C2, params, lora)
    seq = np.concatenate([prompts.numpy()[rows], forced.numpy()[rows, :G - 1]], axis=1)
    full = om.forward_full(seq)
    for j in steps:
        check_logits(got[j], full[:, S - 1 + j], C2.actor, f"batch 100 step {j}")
    picks, lg = O.greedy_generate(om, prompts.numpy()[[0, 99]], G, S + G)
    n = greedy_prefix_agrees(gen[[0, 99]], picks, lg)
    log(f"opt125m batch 100: {n} picks compared")
    assert n >= 2

"""GPU parity of weight-only FP8 decode (he_set_fp8_decode) against the oracle
(oracle/fp8.py, OracleModel(fp8_decode=True)) on the same seeded inputs.

Codes and scales are byte work: they must match the oracle's bit for bit.  They are
compared on weights both sides hold exactly: the base weights (row-major), and their
fuse with all-zero adapters (the oracle's fused values; the GPU then holds them in the
inference layout).
Logits of decode steps with FP8 weights are floating point: within the bf16 logit
bound of the other parity tests (3e-2), at OPT-125m and at the OPT-6.7B layer shapes
(two layers, the full batch of 64, the decode plans the bench runs)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as F
from oracle import opt_he as O
from transformer_decode_amd import he

from gpu_util import BF16_ABS_TOL, GpuRun, check_logits, log, precision

pytestmark = pytest.mark.gpu

PROJ = ("qkv", "out", "fc1", "fc2")


def _codes(q):
    return torch.from_numpy(np.asarray(q, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _export(run, layer, proj, N, K):
    codes = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(N, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(run.stream):
        he.he_fp8_export(run.ctx, layer, proj, codes.data_ptr(), scales.data_ptr())
        he.he_sync(run.ctx)
    return codes.cpu().numpy(), scales.cpu().numpy()


def _check_codes(wl, params, layers, fused):
    shape = wl.actor
    d, Fd = shape.d_model, shape.d_ffn
    dims = {"qkv": (3 * d, d), "out": (d, d), "fc1": (Fd, d), "fc2": (d, Fd)}
    run = GpuRun(wl, params)
    lora = None
    if fused:       # all-zero adapters: the weights change layout, and -0 becomes +0 (W + 0)
        lora = {k: (torch.zeros_like(v) if k.endswith(".B") else v)
                for k, v in synth.lora_params(shape, wl.lora_rank).items()}
        with torch.cuda.stream(run.stream):
            he.he_fuse_lora(run.ctx, run.lora(lora))
    om = O.OracleModel(shape, params, O.Precision("bf16"), lora=lora, lora_scale=wl.lora_scale,
                       cache_layers=False)
    with torch.cuda.stream(run.stream):
        he.he_set_fp8_decode(run.ctx, True)
    for l in layers:
        lw = om.layer(l)                           # the weights the decode step uses
        for j, p in enumerate(PROJ):
            N, K = dims[p]
            got_c, got_s = _export(run, l, j, N, K)
            q, s = F.quantize_rows(lw[f"{p}.w"])
            assert np.array_equal(got_s.view(np.uint32), s.view(np.uint32)), (l, p, "scales")
            want_c = _codes(q)
            bad = np.count_nonzero(got_c != want_c)
            assert bad == 0, (l, p, bad, np.argwhere(got_c != want_c)[:4])
    log(f"{wl.name}: E4M3 codes and scales of layers {layers} bit-exact (fused={fused})")
    run.close()


@pytest.mark.parametrize("fused", [False, True])
def test_opt125m_fp8_codes_bit_exact(fused):
    wl = synth.WORKLOADS["opt125m"]
    _check_codes(wl, synth.model_params(wl.actor), [0, wl.actor.n_layers - 1], fused)


def test_opt6_7b_fp8_codes_bit_exact_sampled_layers():
    """Full-size projection shapes (4096 x 4096 up to 16384 x 4096 and 4096 x 16384)."""
    wl = synth.WORKLOADS["opt6.7b"]
    shape = dataclasses.replace(wl.actor, n_layers=2)
    _check_codes(dataclasses.replace(wl, actor=shape), synth.model_params(shape), [0, 1], True)


def _decode_parity(wl, rows, steps):
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts, forced = synth.prompts(wl), synth.forced_tokens(wl)
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_set_fp8_decode(run.ctx, True)
        he.he_retake_cache(run.ctx, wl.batch, wl.max_seq)
    last = max(steps) + 1
    log(f"{wl.name}: GPU teacher-forced, FP8 decode weights")
    got = run.teacher_forced(prompts, forced, last, want_rows=rows, want_steps=set(steps))
    with torch.cuda.stream(run.stream):
        he.he_set_fp8_decode(run.ctx, False)
    ref16 = run.teacher_forced(prompts, forced, last, want_rows=rows, want_steps=set(steps))
    run.close()
    log(f"{wl.name}: oracle rows {rows}")
    om = O.OracleModel(wl.actor, params, precision(wl.actor), lora=lora, lora_scale=wl.lora_scale,
                       fp8_decode=True)
    _, lg = O.greedy_generate(om, prompts.numpy()[rows], last, wl.max_seq, forced=forced.numpy()[rows])
    worst = 0.0
    for j in steps:
        worst = max(worst, check_logits(got[j], lg[j], wl.actor, f"{wl.name} fp8 step {j}"))
    moved = max(float(np.abs(got[j] - ref16[j]).max()) for j in steps if j > 0)
    log(f"{wl.name}: FP8 vs oracle max |dlogit| {worst:.3e}; FP8 vs bf16 decode {moved:.3e}")
    assert moved > BF16_ABS_TOL / 100   # the decode really ran on other weights
    # the prompt pass keeps bf16: step 0 is the same with and without FP8 decode
    np.testing.assert_array_equal(got[0], ref16[0])


def test_opt125m_fp8_decode_matches_oracle():
    wl = synth.WORKLOADS["opt125m"]
    _decode_parity(wl, rows=[0, wl.batch - 1], steps=[0, 1, 5, 31])


def test_opt125m_fp8_decode_batch_100():
    """100 batch rows: activation tiles of 128 rows, 100 live, with E4M3 weights (the
    plans for 65-128 rows of the FP8 path)."""
    wl = dataclasses.replace(synth.WORKLOADS["opt125m"], batch=100, prompt_len=64, gen_len=16, max_seq=80)
    _decode_parity(wl, rows=[0, 63, 64, 99], steps=[0, 1, 8, 15])


def test_opt6_7b_shape_fp8_decode_matches_oracle():
    """Two layers of the 6.7B shape at the full batch of 64: the bench's decode plans."""
    wl = synth.WORKLOADS["opt6.7b"]
    wl = dataclasses.replace(wl, actor=dataclasses.replace(wl.actor, n_layers=2))
    _decode_parity(wl, rows=[0, wl.batch - 1], steps=[0, 1, 7])


def test_opt125m_fp8_generation_graph_replay_and_requantisation():
    """Graph replay equals direct launches; switching FP8 on before the fuse (the fuse
    remakes the copies) equals switching it on after; off again is the bf16 decode."""
    wl = synth.WORKLOADS["opt125m"]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts = synth.prompts(wl)
    outs = {}
    for name, use_graph, before in (("graph", True, True), ("direct", False, True), ("after", True, False)):
        run = GpuRun(wl, params, use_graph=use_graph)
        lt = run.lora(lora)
        with torch.cuda.stream(run.stream):
            if before:
                he.he_set_fp8_decode(run.ctx, True)
            he.he_fuse_lora(run.ctx, lt)
            if not before:
                he.he_set_fp8_decode(run.ctx, True)
            he.he_retake_cache(run.ctx, wl.batch, wl.max_seq)
        outs[name] = run.generate(prompts, 24)
        if name == "after":
            with torch.cuda.stream(run.stream):
                he.he_set_fp8_decode(run.ctx, False)
            outs["bf16"] = run.generate(prompts, 24)
        run.close()
    assert np.array_equal(outs["graph"], outs["direct"])
    assert np.array_equal(outs["graph"], outs["after"])
    assert not np.array_equal(outs["graph"], outs["bf16"])


def test_opt125m_fp8_top_p_generation_follows_the_rule_each_step():
    """FP8 decode with top-p sampling: the loop's picks and log-probabilities equal
    he_sample applied to the teacher-forced FP8 decode logits, step by step."""
    wl = synth.WORKLOADS["opt125m"]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    B, S, G = wl.batch, wl.prompt_len, 10
    smp = he.he_sampling(0.9, 404, 0.9)
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    prompts = synth.prompts(wl).cuda()
    toks = torch.empty(B, G, dtype=torch.int32, device="cuda")
    lps = torch.empty(B, G, dtype=torch.float32, device="cuda")
    lg = torch.empty(B, wl.actor.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    rt = torch.empty(B, dtype=torch.int32, device="cuda")
    rl = torch.empty(B, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    bt, bl = [], []
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_set_fp8_decode(run.ctx, True)
        he.he_retake_cache(run.ctx, B, wl.max_seq)
        he.he_generate_ex(run.ctx, prompts.data_ptr(), B, S, G, smp, toks.data_ptr(), lps.data_ptr())
        he.he_prefill(run.ctx, prompts.data_ptr(), B, S, nxt.data_ptr(), lg.data_ptr())
        for j in range(G):
            if j:
                col = toks[:, j - 1].contiguous()
                he.he_decode_step(run.ctx, col.data_ptr(), nxt.data_ptr(), lg.data_ptr())
            he.he_sample(run.ctx, lg.data_ptr(), B, S + j, smp, rt.data_ptr(), rl.data_ptr())
            he.he_sync(run.ctx)
            bt.append(rt.cpu().numpy().copy())
            bl.append(rl.cpu().numpy().copy())
    a_t, a_l = toks.cpu().numpy(), lps.cpu().numpy()
    run.close()
    assert np.array_equal(a_t, np.stack(bt, axis=1))
    assert np.array_equal(a_l.view(np.uint32), np.stack(bl, axis=1).view(np.uint32))


def test_opt125m_fp8_toggle_recaptures_graph():
    """FP8 on -> generate -> off -> on -> generate: switching FP8 decode off frees the E4M3
    copy and switching it on makes a new one at new addresses, so a decode graph captured
    before must not be replayed.  Between off and on the freed memory is taken by a
    buffer of NaN codes (0xFF), so a replayed stale graph would read them.  Graph replay
    must equal direct launches bit for bit, both generations."""
    wl = synth.WORKLOADS["opt125m"]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts = synth.prompts(wl)
    d, F_ = wl.actor.d_model, wl.actor.d_ffn
    f8_bytes = wl.actor.n_layers * (4 * d * d + 2 * d * F_ + 4 * (6 * d + F_))
    outs = {}
    for name, use_graph in (("graph", True), ("direct", False)):
        run = GpuRun(wl, params, use_graph=use_graph)
        lt = run.lora(lora)
        with torch.cuda.stream(run.stream):
            he.he_fuse_lora(run.ctx, lt)
            he.he_retake_cache(run.ctx, wl.batch, wl.max_seq)
            he.he_set_fp8_decode(run.ctx, True)
        first = run.generate(prompts, 16)
        with torch.cuda.stream(run.stream):
            he.he_set_fp8_decode(run.ctx, False)
            he.he_sync(run.ctx)
        junk = torch.full((f8_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(run.stream):
            he.he_set_fp8_decode(run.ctx, True)
        second = run.generate(prompts, 16)
        del junk
        outs[name] = (first, second)
        run.close()
    log("fp8 toggle: graph and direct generations compared")
    assert np.array_equal(outs["graph"][0], outs["direct"][0])
    assert np.array_equal(outs["graph"][1], outs["direct"][1])
    assert np.array_equal(outs["graph"][0], outs["graph"][1])

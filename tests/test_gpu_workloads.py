"""GPU parity at the workloads' own sizes, on sampled outputs the oracle can
compute one by one, plus the mode-switch sequence (two generation rounds with the
workspace released and re-taken between them) and reward scoring."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import opt_he as O
from oracle import scoring as SC
from transformer_decode_amd import he

from gpu_util import (BF16_ABS_TOL, FLOOR_FACTOR, GpuRun, check_logits, greedy_prefix_agrees, log,
                      oracle_floor, precision, to_dev)

pytestmark = pytest.mark.gpu


def _sampled_teacher_forced(wl, rows, steps):
    """Full batch on the GPU (prefill + 255 forced steps, graph replay); the oracle
    recomputes the sampled rows from scratch (definition mode, no cache).  Then the
    scoring pass (he_logprobs) over the full batch of prompt + 256 forced tokens, the
    workload's own 512-token experience, checked on the same rows at every answer
    position: its log-probabilities need the oracle's logits at positions
    prompt_len - 1 .. prompt_len + 254, which the definition-mode pass already has.
    Bound: twice the row's logit bound (the larger of 3e-2 and 1.5 x the oracle's
    measured self-sensitivity over its recorded steps)."""
    log(f"{wl.name}: inputs")
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts, forced = synth.prompts(wl), synth.forced_tokens(wl)
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, wl.batch, wl.max_seq)
    log(f"{wl.name}: GPU teacher-forced run")
    got = run.teacher_forced(prompts, forced, wl.gen_len, want_rows=rows, want_steps=set(steps))
    log(f"{wl.name}: GPU scoring pass")
    B, S_p, n = wl.batch, wl.prompt_len, wl.gen_len
    exp = torch.cat([prompts, forced], dim=1).to(torch.int32).cuda()
    lp = torch.full((B, n), float("nan"), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(run.stream):
        he.he_logprobs(run.ctx, exp.data_ptr(), B, S_p + n, S_p, lp.data_ptr())
        he.he_sync(run.ctx)
    lp = lp.cpu().numpy()
    assert np.isfinite(lp).all()
    run.close()
    del run
    torch.cuda.empty_cache()
    log(f"{wl.name}: oracle on rows {rows}")
    om = O.OracleModel(wl.actor, params, precision(wl.actor), lora=lora, lora_scale=wl.lora_scale,
                       cache_layers=False)
    last = max(steps)
    seq = np.concatenate([prompts.numpy()[rows], forced.numpy()[rows, :last]], axis=1)
    full = om.forward_full(seq)
    S = wl.prompt_len
    worst = 0.0
    for j in steps:
        floors = [oracle_floor(wl.name, r, j) for r in rows]
        worst = max(worst, check_logits(got[j], full[:, S - 1 + j], wl.actor, f"{wl.name} step {j}", floors))
    log(f"{wl.name}: max |dlogit| {worst:.3e}")
    want = SC.logprobs_from_logits(full[:, S - 1:S - 1 + n], forced.numpy()[rows, :n])
    for i, r in enumerate(rows):
        fl = [oracle_floor(wl.name, r, j) for j in steps]
        bound = 2 * max([BF16_ABS_TOL] + [FLOOR_FACTOR * f for f in fl if f is not None])
        err = np.abs(lp[r].astype(np.float64) - want[i])
        log(f"{wl.name} scoring row {r}: {n} log-probs, max |d| {err.max():.3e} (bound {bound:.2e})")
        assert err.max() <= bound, f"row {r}: max |dlogprob| {err.max():.3e} at answer token {err.argmax()}"


def test_opt1_3b_sampled_rows():
    wl = synth.WORKLOADS["opt1.3b"]
    _sampled_teacher_forced(wl, rows=[0, wl.batch - 1], steps=[0, 1, 255])


def test_opt6_7b_sampled_rows():
    wl = synth.WORKLOADS["opt6.7b"]
    _sampled_teacher_forced(wl, rows=[wl.batch - 1], steps=[0, 255])


def test_opt13b_sampled_rows():
    wl = synth.WORKLOADS["opt13b"]
    _sampled_teacher_forced(wl, rows=[wl.batch - 1], steps=[0, 255])


def test_two_rounds_release_retake():
    """fuse -> generate -> unfuse -> release, new adapters ("training"), retake ->
    fuse -> generate -> unfuse -> release.  Round 2 must match the oracle with the
    new adapters, and the base weights must survive both round trips."""
    wl = synth.WORKLOADS["opt125m"]
    params = synth.model_params(wl.actor)
    lora1 = synth.lora_params(wl.actor, wl.lora_rank, tag="lora")
    lora2 = synth.lora_params(wl.actor, wl.lora_rank, seed=1, tag="lora")
    prompts = synth.prompts(wl)
    run = GpuRun(wl, params)
    lt1 = run.lora(lora1)
    keep1 = (run.lora_dev, run._keep)
    out = []
    free = []
    for rnd, lt in ((1, lt1), (2, None)):
        if rnd == 2:
            lt = run.lora(lora2)
        with torch.cuda.stream(run.stream):
            he.he_retake_cache(run.ctx, wl.batch, wl.max_seq)
            he.he_fuse_lora(run.ctx, lt)
        out.append(run.generate(prompts, wl.gen_len))
        with torch.cuda.stream(run.stream):
            he.he_unfuse_lora(run.ctx, lt)
            he.he_release_cache(run.ctx)
            he.he_sync(run.ctx)
        free.append(torch.cuda.mem_get_info()[0])
    kv_bytes = 2 * wl.actor.n_layers * wl.batch * wl.max_seq * wl.actor.d_model * 2
    assert free[1] >= free[0] - kv_bytes // 8, "workspace memory not returned"
    for i in range(wl.actor.n_layers):
        for k in ("qkv.w", "out.w", "fc1.w", "fc2.w"):
            W0 = params[f"L{i}.{k}"].double().numpy()
            Wr = run.dev[f"L{i}.{k}"].double().cpu().numpy()
            # two fold/unfold trips, each within one spacing of max(|W|, |W'|) (|W'| <= 2|W| + 0.01 here)
            bound = 2 * O.ulp_bf16(np.maximum(np.abs(W0), 2 * np.abs(W0) + 0.01))
            assert (np.abs(Wr - W0) <= bound).all()
    run.close()
    rows = [0, 15]
    om = O.OracleModel(wl.actor, params, precision(wl.actor), lora=lora2, lora_scale=wl.lora_scale)
    picks, lg = O.greedy_generate(om, prompts.numpy()[rows], 48, wl.max_seq)
    n = greedy_prefix_agrees(out[1][rows, :48], picks, lg)
    log(f"round 2: {n} picks compared")
    assert n >= 4
    assert not np.array_equal(out[0], out[1])


def _rm_check(B, S, rows):
    wl = synth.WORKLOADS["opt13b"]
    shape = wl.reward
    log(f"reward model {B}x{S}: inputs")
    params = synth.model_params(shape, prefix="rm.")
    ids = synth.tokens(0, "rm.ids", (B, S), shape.vocab)
    dev = to_dev(params)
    eng = he.Engine(shape, dev)
    d_ids = ids.cuda()
    rew = torch.empty(B, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(eng.stream):
        he.he_retake_cache(eng.ctx, B, S)
        he.he_score(eng.ctx, d_ids.data_ptr(), B, S, rew.data_ptr())
        he.he_sync(eng.ctx)
    got = rew.cpu().numpy()
    eng.close()
    log("reward model: oracle")
    om = O.OracleModel(shape, params, O.Precision("bf16"))
    ref = om.score(ids.numpy()[rows])
    err = np.abs(got[rows] - ref)
    log(f"reward model: rewards {ref}, max |diff| {err.max():.3e}")
    assert (err <= 3e-2).all(), (got[rows], ref)
    assert np.isfinite(got).all()


def test_reward_model_small_batch():
    _rm_check(4, 96, [0, 1, 2, 3])


def test_reward_model_full_size_sampled_rows():
    _rm_check(128, 512, [0, 127])

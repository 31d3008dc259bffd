"""GPU parity at the workloads' own sizes, on sampled outputs the oracle can
compute one by one, plus the mode-switch sequences (generation rounds with the
workspace released and re-taken between them) and reward scoring.

Full depth: rows {0, 1, B/2, B-1} at decode steps {0, 1, 128, 255}, teacher-forced,
against the larger of 3e-2 and the oracle's own measured sensitivity bound
(gpu_util.oracle_floor).  Full width at two layers: every row of the batch at the
same steps against the same kind of bound (the oracle's sensitivity at two layers),
and free-running greedy picks against the oracle's own greedy decoding."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle_threads as OT
import synth
from oracle import opt_he as O
from oracle import scoring as SC
from transformer_decode_amd import he

from gpu_util import (BF16_ABS_TOL, GpuRun, check_logits, greedy_prefix_agrees, log, oracle_floor,
                      oracle_floor_pooled, precision, to_dev, top2_margin)

pytestmark = pytest.mark.gpu

STEPS = [0, 1, 128, 255]


def rows4(B):
    return [0, 1, B // 2, B - 1]


def _oracle_greedy(om, prompts, max_steps, max_seq, stop_margin):
    """The oracle's own greedy decoding (cached mode) of `prompts`, stopped once every
    row has met a step whose top-2 gap is <= stop_margin (or after max_steps):
    (picks [R, n], logits per step)."""
    lg, cache = om.prefill(prompts, max_seq)
    picks, logits = [O.argmax_lowest(lg)], [lg]
    done = top2_margin(lg) <= stop_margin
    while len(picks) < max_steps and not done.all():
        lg = om.decode(picks[-1], cache)
        picks.append(O.argmax_lowest(lg))
        logits.append(lg)
        done |= top2_margin(lg) <= stop_margin
    return np.stack(picks, axis=1), logits


def _sampled_teacher_forced(wl, rows, steps, free_rows=(), free_cap=0):
    """Full batch on the GPU (prefill + 255 forced steps, graph replay); the oracle
    recomputes the sampled rows from scratch (definition mode, no cache).  Then the
    scoring pass (he_logprobs) over the full batch of prompt + 256 forced tokens, the
    workload's own 512-token experience, checked on the same rows at every answer
    position against the oracle's logits at positions prompt_len - 1 .. prompt_len +
    254.  Bound: twice the row's logit bound (a log-probability is a logit minus a
    logsumexp).  With free_rows, also he_generate's free-running picks on those rows
    against the oracle's own greedy decoding, compared up to the first step whose
    top-2 gap is at most twice the row's logit bound (below that gap a pick may
    legitimately differ), at most free_cap steps."""
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
    gen = run.generate(prompts, wl.gen_len) if free_rows else None
    log(f"{wl.name}: GPU scoring pass")
    B, S, n = wl.batch, wl.prompt_len, wl.gen_len
    exp = torch.cat([prompts, forced], dim=1).to(torch.int32).cuda()
    lp = torch.full((B, n), float("nan"), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(run.stream):
        he.he_logprobs(run.ctx, exp.data_ptr(), B, S + n, S, lp.data_ptr())
        he.he_sync(run.ctx)
    lp = lp.cpu().numpy()
    assert np.isfinite(lp).all()
    run.close()
    del run
    torch.cuda.empty_cache()
    log(f"{wl.name}: oracle on rows {rows}")
    prec = precision(wl.actor)
    seq = np.concatenate([prompts.numpy()[rows], forced.numpy()[rows, :n - 1]], axis=1)
    keep = {} if free_rows else None
    full = OT.logits_at(wl.actor, params, prec, seq, range(S - 1, S - 1 + n), lora=lora,
                        lora_scale=wl.lora_scale, keep=keep)                # [rows, n, V]
    bounds = {}
    for j in steps:
        floors = [oracle_floor(wl.name, r, j) for r in rows]
        check_logits(got[j], full[:, j], wl.actor, f"{wl.name} step {j}", floors)
        for r, f in zip(rows, floors):
            bounds[r] = max(bounds.get(r, BF16_ABS_TOL), f or 0.0)
    want = SC.logprobs_from_logits(full, forced.numpy()[rows, :n])
    for i, r in enumerate(rows):
        err = np.abs(lp[r].astype(np.float64) - want[i])
        log(f"{wl.name} scoring row {r}: {n} log-probs, max |d| {err.max():.3e} (bound {2 * bounds[r]:.2e})")
        assert err.max() <= 2 * bounds[r], f"row {r}: max |dlogprob| {err.max():.3e} at answer token {err.argmax()}"
    if free_rows:
        del full
        om = O.OracleModel(wl.actor, params, prec, lora=lora, lora_scale=wl.lora_scale, cache_layers=True)
        om._layers = keep
        stop = 2 * max(bounds[r] for r in free_rows)
        picks, lgs = _oracle_greedy(om, prompts.numpy()[list(free_rows)], free_cap, wl.max_seq, stop)
        nc = greedy_prefix_agrees(gen[list(free_rows), :picks.shape[1]], picks, lgs, margin=stop)
        log(f"{wl.name}: free-running greedy, rows {list(free_rows)}: {nc} picks equal the oracle's "
            f"(compared up to the first gap <= {stop:.3f}, {picks.shape[1]} oracle steps)")
        keep.clear()


def test_opt1_3b_sampled_rows():
    wl = synth.WORKLOADS["opt1.3b"]
    _sampled_teacher_forced(wl, rows=rows4(wl.batch), steps=STEPS)


def test_opt6_7b_sampled_rows_and_free_running():
    wl = synth.WORKLOADS["opt6.7b"]
    _sampled_teacher_forced(wl, rows=rows4(wl.batch), steps=STEPS, free_rows=(0, wl.batch - 1), free_cap=24)


def _two_layers(name, free_running):
    """The workload's full width (d, F, V, H, batch) at two layers: every row at the
    decode steps STEPS, teacher-forced, against the bf16 bound (3e-2, or the oracle's
    own sensitivity bound at two layers where that is larger, pooled over its sampled
    rows); with free_running, he_generate's picks of every row against the oracle's own
    greedy decoding up to the first step whose top-2 gap is at most twice that bound."""
    wl = synth.WORKLOADS[name]
    wl = dataclasses.replace(wl, actor=dataclasses.replace(wl.actor, n_layers=2))
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts, forced = synth.prompts(wl), synth.forced_tokens(wl)
    B, S, n = wl.batch, wl.prompt_len, wl.gen_len
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, B, wl.max_seq)
    log(f"{name} width, 2 layers: GPU teacher-forced run, all {B} rows")
    got = run.teacher_forced(prompts, forced, n, want_steps=set(STEPS))
    gen = run.generate(prompts, n) if free_running else None
    run.close()
    del run
    torch.cuda.empty_cache()
    log(f"{name} width, 2 layers: oracle, all rows")
    prec = precision(wl.actor)
    seq = np.concatenate([prompts.numpy(), forced.numpy()[:, :max(STEPS)]], axis=1)
    keep = {} if free_running else None
    full = OT.logits_at(wl.actor, params, prec, seq, [S - 1 + j for j in STEPS], lora=lora,
                        lora_scale=wl.lora_scale, keep=keep)
    bound = BF16_ABS_TOL
    for i, j in enumerate(STEPS):
        f = oracle_floor_pooled(name + "-2l", j)
        bound = max(bound, f or 0.0)
        check_logits(got[j], full[:, i], wl.actor, f"{name} 2 layers step {j}", [f] * B)
    if free_running:
        om = O.OracleModel(wl.actor, params, prec, lora=lora, lora_scale=wl.lora_scale, cache_layers=True)
        om._layers = keep
        stop = 2 * bound
        picks, lgs = _oracle_greedy(om, prompts.numpy(), n, wl.max_seq, stop)
        nc = greedy_prefix_agrees(gen[:, :picks.shape[1]], picks, lgs, margin=stop)
        log(f"{name} width, 2 layers: free-running greedy, {nc} picks over {B} rows equal the oracle's "
            f"(compared up to the first gap <= {stop:.3f}; {picks.shape[1]} oracle steps)")
        assert nc >= B


def test_opt6_7b_width_two_layers_all_rows():
    _two_layers("opt6.7b", free_running=True)


def test_opt13b_width_two_layers_all_rows():
    _two_layers("opt13b", free_running=False)


def _rm_check(ids, rows, what):
    """he_score on ids [B, S] of the largest workload's reward model (OPT-350m shape,
    post-LN): y = h_last P_out^T element-wise within 3e-2 (it is unit-scale) and the
    rewards within 3e-2 * |w| (the y bound carried through the head w) on `rows`."""
    wl = synth.WORKLOADS["opt13b"]
    shape = wl.reward
    B, S = ids.shape
    params = synth.model_params(shape, prefix="rm.")
    dev = to_dev(params)
    eng = he.Engine(shape, dev)
    d_ids = ids.to(torch.int32).cuda()
    rew = torch.empty(B, dtype=torch.float32, device="cuda")
    rew2 = torch.empty(B, dtype=torch.float32, device="cuda")
    ys = torch.empty(B, shape.embed_dim, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(eng.stream):
        he.he_retake_cache(eng.ctx, B, S)
        he.he_score(eng.ctx, d_ids.data_ptr(), B, S, rew.data_ptr(), ys.data_ptr())
        he.he_score(eng.ctx, d_ids.data_ptr(), B, S, rew2.data_ptr())
        he.he_sync(eng.ctx)
    got, got2, gy = rew.cpu().numpy(), rew2.cpu().numpy(), ys.cpu().numpy()
    eng.close()
    assert np.isfinite(got).all() and np.isfinite(gy).all()
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32)), "reward scoring is not reproducible"
    log(f"{what}: oracle on rows {rows}")
    y, ref = OT.reward_at_last(shape, params, O.Precision("bf16"), ids.numpy()[rows])
    w = O.f64(params["score"])
    ey = np.abs(gy[rows] - y).max(axis=1)
    er = np.abs(got[rows] - ref)
    rb = BF16_ABS_TOL * float(np.linalg.norm(w))
    log(f"{what}: y max |diff| per row {ey} (|y| ~ {np.abs(y).mean():.3f}); rewards {ref}, |diff| {er} (bound {rb:.3e})")
    assert (ey <= BF16_ABS_TOL).all()
    assert (er <= rb).all()
    # y.w recomputed from the GPU's own y: the head's dot product
    assert np.allclose(gy.astype(np.float64) @ w, got, atol=1e-4)
    return got


def test_reward_model_small_batch():
    _rm_check(synth.tokens(0, "rm.ids", (4, 96), synth.WORKLOADS["opt13b"].reward.vocab), [0, 1, 2, 3],
              "reward model 4x96")


def test_reward_model_full_size_sampled_rows():
    _rm_check(synth.tokens(0, "rm.ids", (128, 512), synth.WORKLOADS["opt13b"].reward.vocab), rows4(128),
              "reward model 128x512")


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


def test_opt13b_two_rounds_and_reward_scoring():
    """The largest workload's sequence: round 1 (fuse, generate 256 tokens for 128
    prompts, unfuse, release the 53.7 GB KV workspace), round 2 (retake, fuse,
    teacher-forced pass + generation, unfuse, release), then reward scoring of the
    round-2 sequences (prompt + answer, 512 tokens) by the OPT-350m-shape reward model.
    Checks: the workspace's memory comes back on release; round 2's logits at rows
    {0, 1, 64, 127}, steps {0, 1, 128, 255} match the oracle; the base weights survive
    both round trips; the rewards of the generated experience are finite and
    reproducible.  Round 2's fold starts from the unfolded weights, which are the
    originals only to within one bf16 spacing; folding them again reproduces round 1's
    fused weights except on a few elements in 10^7, each one spacing apart (checked
    here).  That is enough for free-running picks to part from round 1's at a near-tie,
    so round 2's tokens are compared with round 1's only as a logged statistic."""
    wl = synth.WORKLOADS["opt13b"]
    a = wl.actor
    B, S, n = wl.batch, wl.prompt_len, wl.gen_len
    rows = rows4(B)
    log("opt13b sequence: inputs")
    params = synth.model_params(a)
    lora = synth.lora_params(a, wl.lora_rank)
    prompts, forced = synth.prompts(wl), synth.forced_tokens(wl)
    run = GpuRun(wl, params)
    lt = run.lora(lora)
    ws_bytes = 2 * a.n_layers * B * wl.max_seq * a.d_model * 2
    torch.cuda.synchronize()
    gens, got, fused1 = [], None, None
    wkeys = [k for k in run.dev if k.endswith(".w")]
    for rnd in (1, 2):
        # free device memory as the library sees it: the test's own transient tensors
        # are handed back by torch's caching allocator before each reading
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        free0 = torch.cuda.mem_get_info()[0]
        with torch.cuda.stream(run.stream):
            he.he_retake_cache(run.ctx, B, wl.max_seq)
            he.he_fuse_lora(run.ctx, lt)
            he.he_sync(run.ctx)
        free1 = torch.cuda.mem_get_info()[0]
        if rnd == 1:          # round 1's fused weights, kept in host memory
            fused1 = {k: run.dev[k].cpu() for k in wkeys}
        else:                 # compared one matrix at a time on the GPU
            nd = tot = 0
            for k in wkeys:
                ref = fused1.pop(k).cuda()
                dv = (run.dev[k].view(torch.int16).int() - ref.view(torch.int16).int()).abs()
                nz = dv[dv != 0]
                assert (nz == 1).all(), f"{k}: a refolded weight is more than one bf16 spacing from round 1's"
                nd += int(nz.numel())
                tot += dv.numel()
                del ref, dv, nz
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            log(f"opt13b sequence: round 2's fused weights differ from round 1's on {nd} of {tot} elements")
            assert nd <= 1e-6 * tot
            free1 = torch.cuda.mem_get_info()[0]
            log("opt13b sequence: round 2 teacher-forced run")
            got = run.teacher_forced(prompts, forced, n, want_rows=rows, want_steps=set(STEPS))
        log(f"opt13b sequence: round {rnd} generation")
        gens.append(run.generate(prompts, n))
        with torch.cuda.stream(run.stream):
            he.he_unfuse_lora(run.ctx, lt)
            he.he_release_cache(run.ctx)
            he.he_sync(run.ctx)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        free2 = torch.cuda.mem_get_info()[0]
        log(f"opt13b sequence: round {rnd}: retake took {(free0 - free1) / 1e9:.2f} GB, release returned "
            f"{(free2 - free1) / 1e9:.2f} GB (KV cache {ws_bytes / 1e9:.2f} GB)")
        assert free0 - free1 >= ws_bytes, "the workspace is smaller than the KV cache"
        assert free2 - free1 >= ws_bytes and free2 >= free0 - (64 << 20), "workspace memory not returned"
    same = gens[0] == gens[1]
    first = np.where(same.all(axis=1), n, np.argmin(same, axis=1))
    log(f"opt13b sequence: rounds 1 and 2 generate the same first token on {int(same[:, 0].sum())}/{B} rows; "
        f"identical prefixes of median {int(np.median(first))} tokens, {int((first == n).sum())} rows identical")
    for i in (0, a.n_layers - 1):
        for k in ("qkv.w", "fc2.w"):
            W0 = params[f"L{i}.{k}"].double().numpy()
            Wr = run.dev[f"L{i}.{k}"].double().cpu().numpy()
            bound = 2 * O.ulp_bf16(np.maximum(np.abs(W0), 2 * np.abs(W0) + 0.05))
            assert (np.abs(Wr - W0) <= bound).all(), (i, k)
    run.close()
    del run
    torch.cuda.empty_cache()
    log("opt13b sequence: reward scoring of the round-2 experience")
    exp = torch.from_numpy(np.concatenate([prompts.numpy(), gens[1]], axis=1).astype(np.int32))
    shape = wl.reward
    eng = he.Engine(shape, to_dev(synth.model_params(shape, prefix="rm.")))
    d_exp = exp.cuda()
    r1 = torch.empty(B, dtype=torch.float32, device="cuda")
    r2 = torch.empty(B, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(eng.stream):
        he.he_retake_cache(eng.ctx, B, S + n)
        he.he_score(eng.ctx, d_exp.data_ptr(), B, S + n, r1.data_ptr())
        he.he_score(eng.ctx, d_exp.data_ptr(), B, S + n, r2.data_ptr())
        he.he_release_cache(eng.ctx)
        he.he_sync(eng.ctx)
    rw1, rw2 = r1.cpu().numpy(), r2.cpu().numpy()
    eng.close()
    log(f"opt13b sequence: rewards of the experience, mean {rw1.mean():.4f} sd {rw1.std():.4f}")
    assert np.isfinite(rw1).all() and np.array_equal(rw1.view(np.uint32), rw2.view(np.uint32))
    log(f"opt13b sequence: oracle on rows {rows}")
    seq = np.concatenate([prompts.numpy()[rows], forced.numpy()[rows, :max(STEPS)]], axis=1)
    full = OT.logits_at(a, params, precision(a), seq, [S - 1 + j for j in STEPS], lora=lora,
                        lora_scale=wl.lora_scale)
    for i, j in enumerate(STEPS):
        check_logits(got[j], full[:, i], a, f"opt13b round 2 step {j}", [oracle_floor(wl.name, r, j) for r in rows])

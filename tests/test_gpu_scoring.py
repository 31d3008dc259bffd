"""GPU parity of the teacher-forced scoring pass (he_logprobs) against the oracle
(oracle/scoring.py) on the same seeded inputs.

The sequence is given, so nothing feeds back and every position is compared.  A
log-probability is one logit minus the row's logsumexp, so its error is at most twice
the workload's logit error bound: 2e-3 * max|logit| for the fp32 workload, 6e-2 for
bf16 (twice the 3e-2 logit bound of the other parity tests)."""
import numpy as np
import pytest
import torch

import synth
from oracle import opt_he as O
from oracle import scoring as SC
from transformer_decode_amd import he

from gpu_util import BF16_ABS_TOL, FP32_REL_TOL, GpuRun, log, precision

pytestmark = pytest.mark.gpu

BF16_LP_TOL = 2 * BF16_ABS_TOL


def _experience(wl, prompt_len, answer_len):
    return torch.cat([synth.prompts(wl)[:, :prompt_len], synth.forced_tokens(wl)[:, :answer_len]], dim=1)


def _gpu_logprobs(run, seq, S_p, fuse=True, lora_cpu=None):
    B, S = seq.shape
    out = torch.full((B, S - S_p), float("nan"), dtype=torch.float32, device="cuda")
    ids = seq.to(torch.int32).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(run.stream):
        if fuse:
            he.he_fuse_lora(run.ctx, run.lora(lora_cpu))
        he.he_retake_cache(run.ctx, run.wl.batch, run.wl.max_seq)
        he.he_logprobs(run.ctx, ids.data_ptr(), B, S, S_p, out.data_ptr())
        he.he_sync(run.ctx)
    return out.cpu().numpy()


def _compare(got, want, bound, what):
    err = np.abs(got.astype(np.float64) - want)
    log(f"{what}: {err.size} log-probs, max |d| {err.max():.3e} (bound {bound:.1e})")
    assert np.isfinite(got).all()
    assert err.max() <= bound, f"{what}: max |dlogprob| {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


# ------------------------------------------------------------------------------------
# tiny fp32 workload: all rows, all positions
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("S_p,S", [(16, 32), (5, 23), (31, 32), (1, 2)])
def test_tiny_logprobs_match_oracle(S_p, S):
    wl = synth.WORKLOADS["tiny"]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    seq = _experience(wl, wl.prompt_len, wl.gen_len)[:, :S]
    run = GpuRun(wl, params)
    got = _gpu_logprobs(run, seq, S_p, lora_cpu=lora)
    run.close()
    om = O.OracleModel(wl.actor, params, precision(wl.actor), lora=lora, lora_scale=wl.lora_scale)
    want = SC.teacher_forced_logprobs(om, seq.numpy(), S_p)
    scale = float(np.abs(om.lm_logits(om.hidden(seq.numpy(), 0, None))).max())
    _compare(got, want, 2 * FP32_REL_TOL * max(1.0, scale), f"tiny S_p={S_p} S={S}")


# ------------------------------------------------------------------------------------
# OPT-125m shape, bf16: the full batch of 16 on the GPU, sampled rows in the oracle
# ------------------------------------------------------------------------------------

C2 = synth.WORKLOADS["opt125m"]


@pytest.fixture(scope="module")
def c2():
    return synth.model_params(C2.actor), synth.lora_params(C2.actor, C2.lora_rank)


@pytest.mark.parametrize("fuse", [True, False])
def test_opt125m_logprobs_two_chunks(c2, fuse):
    """S = 512, S_p = 200: 16 x 312 = 4992 scored positions, one full chunk of 4096
    logit rows and a ragged one of 896; row 13 straddles the chunk boundary.
    Unfused, the base weights run from their row-major layout."""
    params, lora = c2
    S_p, S = 200, 512
    seq = _experience(C2, C2.prompt_len, C2.gen_len)[:, :S]
    run = GpuRun(C2, params)
    got = _gpu_logprobs(run, seq, S_p, fuse=fuse, lora_cpu=lora)
    run.close()
    rows = [0, 13, 15]
    om = O.OracleModel(C2.actor, params, precision(C2.actor), lora=lora if fuse else None,
                       lora_scale=C2.lora_scale)
    want = SC.teacher_forced_logprobs(om, seq.numpy()[rows], S_p)
    _compare(got[rows], want, BF16_LP_TOL, f"opt125m fused={fuse}")


def test_opt125m_logprobs_ragged_rows(c2):
    """Three sequences of 301 tokens, S_p = 200: the prompt layers run on 903 rows and
    the scored norm on 303 (row groups of 101). Both are above the size where the
    LayerNorm takes one wave per row, and neither is a multiple of that kernel's four
    rows per WG, so the last WG is partly empty. Every position is checked."""
    params, lora = c2
    S_p, S = 200, 301
    seq = _experience(C2, C2.prompt_len, C2.gen_len)[:3, :S].contiguous()
    run = GpuRun(C2, params)
    got = _gpu_logprobs(run, seq, S_p, lora_cpu=lora)
    run.close()
    om = O.OracleModel(C2.actor, params, precision(C2.actor), lora=lora, lora_scale=C2.lora_scale)
    want = SC.teacher_forced_logprobs(om, seq.numpy(), S_p)
    _compare(got, want, BF16_LP_TOL, "opt125m 3 x 301 rows")


def test_opt125m_scoring_reproduces_generation_logprobs(c2):
    """Sampling at T = 1 reports log softmax(logits) of each pick from the decode
    route; scoring the finished sequence recomputes them from the prompt-pass route.
    Each is within the bf16 log-prob bound of the oracle, so they agree within twice
    that."""
    params, lora = c2
    G = 48
    run = GpuRun(C2, params)
    lt = run.lora(lora)
    B, S_p = C2.batch, C2.prompt_len
    prompts = synth.prompts(C2).cuda()
    toks = torch.empty(B, G, dtype=torch.int32, device="cuda")
    lp_gen = torch.empty(B, G, dtype=torch.float32, device="cuda")
    lp_tf = torch.empty(B, G, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(run.stream):
        he.he_fuse_lora(run.ctx, lt)
        he.he_retake_cache(run.ctx, B, C2.max_seq)
        he.he_generate_ex(run.ctx, prompts.data_ptr(), B, S_p, G, he.he_sampling(1.0, 99), toks.data_ptr(),
                          lp_gen.data_ptr())
        seq = torch.cat([prompts, toks], dim=1).contiguous()
        he.he_logprobs(run.ctx, seq.data_ptr(), B, S_p + G, S_p, lp_tf.data_ptr())
        he.he_sync(run.ctx)
    a, b = lp_gen.cpu().numpy(), lp_tf.cpu().numpy()
    run.close()
    _compare(b, a.astype(np.float64), 2 * BF16_LP_TOL, "opt125m generation vs scoring")
    # a token the model itself sampled is rarely very unlikely
    assert np.median(b) > -20


def test_head_128_two_window_attention():
    """Head size 128 with S = 400: the prompt-pass attention holds 256 keys of a head in
    LDS at once, so queries past 256 run over two staged windows (the second ragged,
    144 keys).  A two-layer bf16 model of that head size, every position scored."""
    import dataclasses
    shape = dataclasses.replace(C2.actor, n_layers=2, d_model=256, n_heads=2, d_ffn=512)
    wl = dataclasses.replace(C2, name="head128", actor=shape, batch=2, max_seq=512)
    params = synth.model_params(shape, seed=5)
    lora = synth.lora_params(shape, wl.lora_rank, seed=5)
    S_p, S = 100, 400
    seq = _experience(wl, wl.prompt_len, wl.gen_len)[:, :S]
    run = GpuRun(wl, params)
    got = _gpu_logprobs(run, seq, S_p, lora_cpu=lora)
    run.close()
    om = O.OracleModel(shape, params, precision(shape), lora=lora, lora_scale=wl.lora_scale)
    want = SC.teacher_forced_logprobs(om, seq.numpy(), S_p)
    _compare(got, want, BF16_LP_TOL, "head 128, S = 400")


def test_opt125m_scoring_batch_one_and_fp8_mode(c2):
    """B = 1 with a one-token prompt and a two-token answer against the oracle; and the
    scoring pass (a prompt pass: bf16 weights) is bit-for-bit the same whether or not
    FP8 decode weights are switched on."""
    params, lora = c2
    seq = _experience(C2, C2.prompt_len, C2.gen_len)
    run = GpuRun(C2, params)
    got1 = _gpu_logprobs(run, seq[:1, :3], 1, lora_cpu=lora)
    om = O.OracleModel(C2.actor, params, precision(C2.actor), lora=lora, lora_scale=C2.lora_scale)
    _compare(got1, SC.teacher_forced_logprobs(om, seq.numpy()[:1, :3], 1), BF16_LP_TOL, "opt125m B=1 S=3")
    B, S, S_p = C2.batch, 300, 200
    ids = seq[:, :S].to(torch.int32).cuda()
    outs = []
    for f8 in (False, True):
        out = torch.empty(B, S - S_p, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(run.stream):
            he.he_set_fp8_decode(run.ctx, f8)
            he.he_logprobs(run.ctx, ids.data_ptr(), B, S, S_p, out.data_ptr())
            he.he_sync(run.ctx)
        outs.append(out.cpu().numpy())
    run.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))

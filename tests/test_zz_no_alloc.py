"""he_sample_static (the pick rule on the library's static device scratch, for callers
that cannot allocate) against he_sample (the same rule on the workspace) through the
C ABI: the same tokens and log-probabilities bit for bit, on two calls in a row, the
second with a smaller batch, for greedy, sampled and top-p rules."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from transformer_decode_amd import he

from gpu_util import GpuRun, log

pytestmark = pytest.mark.gpu


def _pick(fn, run, x, B, pos, smp):
    tok = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lp = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(run.stream):
        fn(run.ctx, x.data_ptr(), B, pos, smp, tok.data_ptr(), lp.data_ptr())
        he.he_sync(run.ctx)
    return tok.cpu().numpy(), lp.cpu().numpy()


@pytest.mark.parametrize("T,P", [(0.0, 0.0), (0.8, 0.0), (1.0, 0.9)])
def test_static_scratch_pick_equals_workspace_pick(T, P):
    wl = synth.WORKLOADS["opt6.7b"]
    shape = dataclasses.replace(wl.actor, n_layers=0)
    wl = dataclasses.replace(wl, actor=shape)
    V = shape.vocab
    smp = he.he_sampling(T, 31337, P) if T > 0 else None
    # the allocation-free call first, on a context with no workspace at all
    free = GpuRun(wl, synth.model_params(shape))
    ws = GpuRun(wl, synth.model_params(shape))
    with torch.cuda.stream(ws.stream):
        he.he_retake_cache(ws.ctx, 128, 16)
        he.he_sync(ws.ctx)
    for call, (B, pos) in enumerate(((128, 300), (37, 301))):
        x = synth.sample_logits(B, V, seed=11 + call).cuda()
        a_t, a_l = _pick(he.he_sample_static, free, x, B, pos, smp)
        b_t, b_l = _pick(he.he_sample, ws, x, B, pos, smp)
        log(f"static scratch T={T} p={P} call {call} (batch {B}): {np.count_nonzero(a_t == b_t)}/{B} picks equal")
        assert (a_t >= 0).all() and (a_t < V).all()
        assert np.array_equal(a_t, b_t)
        assert np.array_equal(a_l.view(np.uint32), b_l.view(np.uint32))
    with pytest.raises(he.HEError):
        x = synth.sample_logits(1, V, seed=5).cuda()
        _pick(he.he_sample_static, free, x, 167, 0, smp)    # 167 rows x 393 blocks > 65536
    free.close()
    ws.close()

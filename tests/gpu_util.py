"""Shared helpers of the GPU parity tests (inputs, uploads, tolerances)."""
import json
import os
import sys
import time

import numpy as np
import torch

import synth
from oracle import opt_he as O
from transformer_decode_amd import he

BF16_ABS_TOL = 3e-2       # bf16 workloads: max |logit difference| per row and step
FP32_REL_TOL = 1e-3       # fp32 workload: max |difference| <= 1e-3 * max |oracle logit|
MARGIN = 1e-2             # greedy picks are compared where the oracle's top-2 gap exceeds this
# Full-depth bf16 workloads: where the oracle's own sensitivity to float32-sized errors
# in its wide arithmetic exceeds BF16_ABS_TOL, the bound is the level a further
# float32-accurate evaluation stays under: the measured mean m of the perturbed
# copies' largest logit differences at that row and step, plus FLOOR_SIGMAS standard
# deviations (m times the coefficient of variation c pooled over the workload's
# copies, rows and steps).  A largest difference over 50272 logits follows an
# extreme-value (Gumbel) law, under which mean + 6 sd is exceeded with probability
# about 2.6e-4 per comparison.
FLOOR_SIGMAS = 6.0
_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_sensitivity.json")


def _floor_entry(name):
    if not os.path.exists(_GOLDEN):
        return None
    return json.load(open(_GOLDEN)).get(name)


def floor_stats(name):
    """(means [rows][steps], pooled coefficient of variation) of a workload's stored
    perturbed copies, or None.  means: the larger of the 2^-24 and 2^-16 groups' means."""
    e = _floor_entry(name)
    if not e or "per_copy_max_abs_dlogit" not in e:
        return None
    a = np.asarray(e["per_copy_max_abs_dlogit"], dtype=np.float64)        # [copies, rows, steps]
    b = np.asarray(e["gpu_per_copy_max_abs_dlogit"], dtype=np.float64)
    allc = np.concatenate([a, b], axis=0)
    rel = allc / allc.mean(axis=0, keepdims=True)
    c = float(rel.std(ddof=1))
    return np.maximum(a.mean(axis=0), b.mean(axis=0)), c, e["rows"], e["steps"]


def oracle_floor(name, row, step):
    """The logit bound the oracle's own sensitivity sets at (row, step), or None."""
    st_ = floor_stats(name)
    if st_ is None:
        return None
    means, c, rows, steps = st_
    if row not in rows or step not in steps:
        return None
    return float(means[rows.index(row), steps.index(step)] * (1.0 + FLOOR_SIGMAS * c))


def oracle_floor_pooled(name, step):
    """The largest oracle_floor over the workload's stored rows at `step` (for rows
    that were not sampled: the level is a property of the model, not of the row), or
    None."""
    st_ = floor_stats(name)
    if st_ is None or step not in st_[3]:
        return None
    return max(oracle_floor(name, r, step) for r in st_[2])


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(p):
    out = {k: v.to("cuda", non_blocking=False).contiguous() for k, v in p.items()}
    torch.cuda.synchronize()      # uploads done before the library's stream reads them
    return out


def precision(shape):
    return O.Precision("fp32" if shape.dtype == "fp32" else "bf16")


def top2_margin(logits):
    s = np.sort(np.asarray(logits, dtype=np.float64), axis=-1)
    return s[..., -1] - s[..., -2]


def check_logits(gpu, ref, shape, what="", floors=None):
    """Max |logit difference| per row against the workload's bound, and greedy picks.
    floors: per row, the oracle-sensitivity bound (oracle_floor) or None; the bf16
    bound is the larger of BF16_ABS_TOL and it.  Picks are compared where the oracle's
    top-2 gap exceeds MARGIN and twice the row's measured largest difference: a pick
    can only change where the gap is at most twice the largest change of a logit."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref).max(axis=-1)
    if shape.dtype == "fp32":
        bound = FP32_REL_TOL * np.abs(ref).max(axis=-1)
    else:
        bound = np.full(err.shape, BF16_ABS_TOL)
        if floors is not None:
            bound = np.maximum(bound, np.array([f if f is not None else 0.0 for f in floors]))
    bad = err > bound
    log(f"{what}: max |dlogit| {err.max():.3e} per row {np.array2string(err, precision=4)} "
        f"(bounds {np.array2string(bound, precision=4)})")
    assert not bad.any(), f"{what}: max |dlogit| {err.max():.3e} over bound at rows {np.nonzero(bad)}"
    clear = top2_margin(ref) > np.maximum(MARGIN, 2 * err)
    assert (gpu.argmax(-1)[clear] == ref.argmax(-1)[clear]).all(), f"{what}: argmax mismatch"
    return float(err.max())


class GpuRun:
    """Engine over uploaded parameters plus device buffers for one workload."""

    def __init__(self, wl, params, use_graph=True):
        self.wl = wl
        self.dev = to_dev(params)
        self.eng = he.Engine(wl.actor, self.dev, use_graph=use_graph)
        self.ctx = self.eng.ctx
        self.stream = self.eng.stream

    def lora(self, lora_cpu):
        self.lora_dev = to_dev(lora_cpu)
        self.lt, self._keep = self.eng.lora(self.lora_dev, self.wl.lora_rank, self.wl.lora_alpha)
        return self.lt

    def teacher_forced(self, prompts, forced, steps, want_rows=None, want_steps=None):
        """Prefill + `steps - 1` decode steps fed with `forced`; logits per step [B, V]."""
        B, S = prompts.shape
        V = self.wl.actor.vocab
        ids = prompts.to("cuda")
        fd = forced.to("cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.empty(B, V, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        out = {}
        with torch.cuda.stream(self.stream):
            he.he_prefill(self.ctx, ids.data_ptr(), B, S, nxt.data_ptr(), lg.data_ptr())
            he.he_sync(self.ctx)
            if want_steps is None or 0 in want_steps:
                out[0] = lg.cpu().numpy()[want_rows if want_rows is not None else slice(None)]
            for j in range(1, steps):
                col = fd[:, j - 1].contiguous()
                want = want_steps is None or j in want_steps
                he.he_decode_step(self.ctx, col.data_ptr(), nxt.data_ptr(), lg.data_ptr() if want else 0)
                if want:
                    he.he_sync(self.ctx)
                    out[j] = lg.cpu().numpy()[want_rows if want_rows is not None else slice(None)]
            he.he_sync(self.ctx)
        return out

    def generate(self, prompts, gen_len):
        B, S = prompts.shape
        ids = prompts.to("cuda")
        out = torch.empty(B, gen_len, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            he.he_generate(self.ctx, ids.data_ptr(), B, S, gen_len, out.data_ptr())
            he.he_sync(self.ctx)
        return out.cpu().numpy()

    def close(self):
        self.eng.close()


def greedy_prefix_agrees(gpu_picks, oracle_picks, oracle_logits, margin=MARGIN):
    """Free-running picks must agree up to the first step where the oracle's own
    choice is not clear (top-2 gap <= margin); returns the number compared."""
    compared = 0
    B, G = oracle_picks.shape
    for b in range(B):
        for j in range(G):
            if top2_margin(oracle_logits[j][b]) <= margin:
                break
            assert gpu_picks[b, j] == oracle_picks[b, j], f"row {b} step {j}: {gpu_picks[b, j]} vs {oracle_picks[b, j]}"
            compared += 1
    return compared

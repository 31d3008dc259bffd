"""Measure how far the oracle's own logits move when its wide arithmetic is
perturbed by float32-sized errors.

For the large bf16 workloads the parity tests compare the GPU with the oracle at
sampled rows and decode steps.  Both round to bfloat16 at the same storage points,
but a value that lands next to a rounding boundary rounds either way depending on
the last bits of its float32 (GPU) or float64 (oracle) accumulation.  Each such
one-spacing flip moves the next layer's products enough to flip others, so over
32-40 layers any two evaluations that differ at all drift apart to a level set by
the bf16 storage points themselves, not by the size of the first difference.

This script measures that level on the oracle alone.  Every value the GPU forms by
a float32 accumulation or add (OracleModel.wide: embedding sum, each projection's
product, the attention output, the LayerNorm statistics, the residual stream after
each add, the logits) is multiplied by (1 + eps * N(0, 1)), independently per
element.  A batch holds several copies of the sampled rows: an unperturbed copy
and perturbed copies, each with its own noise, at eps = 2^-24 (one float32
rounding), at eps = 2^-16 (the coarsest wide value the GPU forms: prompt-pass
attention feeds its probabilities to the value product as two bf16 parts, about 16
significant bits) and one at eps = 2^-32, which shows how far the level depends on
the size of the perturbation.  Rows are independent, so each copy is a separate
evaluation; the largest |logit difference| of every perturbed copy against the
unperturbed one of its batch is recorded per row and decode step.  Copies are run
in groups (each with its own unperturbed copy) to bound memory; within a group the
copies run in parallel threads.  It imports only the input generators and the
oracle.

    python tests/golden/make_oracle_sensitivity.py [workload ...]

writes tests/golden/oracle_sensitivity.json (merged with what is there).
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth                         # noqa: E402
from oracle import opt_he as O       # noqa: E402

STEPS = [0, 1, 128, 255]
# rows {0, 1, B/2, B-1} of each workload's batch, the rows the GPU tests sample
SAMPLES = {
    "opt1.3b": ([0, 1, 16, 31], STEPS),
    "opt6.7b": ([0, 1, 32, 63], STEPS),
    "opt13b": ([0, 1, 64, 127], STEPS),
    # the same widths and batches at two layers (the full-width shallow tests)
    "opt6.7b-2l": ([0, 1, 32, 63], STEPS),
    "opt13b-2l": ([0, 1, 64, 127], STEPS),
}


def workload(name):
    """A workload by name; "<name>-2l" is that workload with two decoder layers."""
    import dataclasses
    base, _, var = name.partition("-")
    wl = synth.WORKLOADS[base]
    if var == "2l":
        wl = dataclasses.replace(wl, actor=dataclasses.replace(wl.actor, n_layers=2))
    return wl
EPS = 2.0 ** -24
EPS_GPU = 2.0 ** -16                  # the GPU's coarsest wide rounding (two-part P)
EPS_SMALL = 2.0 ** -32
N_EPS, N_GPU = 6, 4                   # perturbed copies at EPS and at EPS_GPU
GROUP = 6                             # perturbed copies per group (plus the unperturbed one)
NOISE_SEED = 20241
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_sensitivity.json")


def copy_eps():
    """eps of every perturbed copy, in order."""
    return [EPS] * N_EPS + [EPS_GPU] * N_GPU + [EPS_SMALL]


def _copies(wl, params, lora, seq, eps, steps, seed):
    """Logit deviations [len(eps), rows, steps] of the perturbed copies against an
    unperturbed copy of the same rows, and that copy's logit RMS.  Each copy is its own
    OracleModel (its own noise stream) over the same converted layer weights; the copies
    advance layer by layer in parallel threads (numpy releases the GIL; BLAS runs one
    thread per copy)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    R = seq.shape[0]
    shared = {}
    models = []
    for c, e in enumerate([0.0] + list(eps)):
        om = O.OracleModel(wl.actor, params, O.Precision("bf16"), lora=lora,
                           lora_scale=wl.lora_scale, cache_layers=True)
        om._layers = shared                                # one converted copy of each layer
        if e:
            rng = np.random.default_rng(seed + c)
            # float64 eps: with a Python float NumPy would keep 1 + eps n in float32
            om.wide = (lambda r, e_: (lambda x: x * (1.0 + e_ * r.standard_normal(x.shape, dtype=np.float32))))(
                rng, np.float64(e))
        models.append(om)
    threads = min(len(models), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as pool, threadpool_limits(1):
        hs = list(pool.map(lambda om: om.embed(seq, 0), models))
        for i in range(wl.actor.n_layers):
            models[0].layer(i)                             # LoRA fold of layer i, once
            hs = list(pool.map(lambda a: a[0].layer_forward(i, a[1], 0, None), zip(models, hs)))
            shared.pop(i)
        S = wl.prompt_len
        cols = [S - 1 + j for j in steps]
        lg = list(pool.map(lambda a: a[0].lm_logits(a[1][:, cols]), zip(models, hs)))
    lg = np.stack(lg)                                      # [copies + 1, R, steps, V]
    dev = np.abs(lg[1:] - lg[0][None]).max(axis=-1)
    rms = np.sqrt((lg[0] ** 2).mean(axis=-1))
    return dev, rms


def measure(name):
    wl = workload(name)
    rows, steps = SAMPLES[name]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts, forced = synth.prompts(wl).numpy(), synth.forced_tokens(wl).numpy()
    seq = np.concatenate([prompts[rows], forced[rows, :max(steps)]], axis=1)
    eps = copy_eps()
    t0 = time.time()
    devs, rms = [], None
    for g0 in range(0, len(eps), GROUP):
        dev, rms = _copies(wl, params, lora, seq, eps[g0:g0 + GROUP], steps, NOISE_SEED + 100 * g0)
        devs.append(dev)
        print(f"{name}: copies {g0}..{g0 + len(dev) - 1} done at {time.time() - t0:.0f}s", flush=True)
    dev = np.concatenate(devs, axis=0)
    a, b = N_EPS, N_EPS + N_GPU
    entry = {"rows": rows, "steps": steps, "noise_seed": NOISE_SEED,
             "eps": EPS, "per_copy_max_abs_dlogit": dev[:a].tolist(),
             "max_abs_dlogit": dev[:a].max(axis=0).tolist(),
             "eps_gpu": EPS_GPU, "gpu_per_copy_max_abs_dlogit": dev[a:b].tolist(),
             "eps_small": EPS_SMALL, "small_max_abs_dlogit": dev[b].tolist(),
             "logit_rms": rms.tolist(), "seconds": round(time.time() - t0, 1)}
    print(name, json.dumps(entry), flush=True)
    return entry


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["_about"] = ("max |logit difference| of the oracle against itself with every float32-formed "
                      "value (embedding sum, projection products, attention output, LayerNorm "
                      "statistics, residual adds, logits) multiplied by 1 + eps N(0, 1); written by "
                      "tests/golden/make_oracle_sensitivity.py")
    for name in names:
        data[name] = measure(name)
        json.dump(data, open(OUT, "w"), indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or list(SAMPLES))

"""Measure how far the oracle's own logits move under a float32-sized perturbation.

For the large bf16 workloads the parity tests compare the GPU with the oracle at a
few sampled rows and decode steps.  Both round to bfloat16 at the same storage
points, but a value that lands next to a rounding boundary can round either way
depending on the last bits of its float32 (GPU) or float64 (oracle) accumulation,
and such one-ulp flips grow over 32-40 layers.  This script measures that floor
on the oracle alone: it perturbs the embedding output of each sampled row by
independent relative noise of 2^-24 (one float32 rounding error) and records the
largest |logit difference| against the unperturbed oracle, per row and step, over
two noise seeds.  It imports only the input generators and the oracle.

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

# rows and decode steps the GPU tests sample, per workload
SAMPLES = {
    "opt1.3b": ([0, 31], [0, 1, 255]),
    "opt6.7b": ([63], [0, 255]),
    "opt13b": ([127], [0, 255]),
}
EPS = 2.0 ** -24
SEEDS = (1, 2)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_sensitivity.json")


def measure(name):
    wl = synth.WORKLOADS[name]
    rows, steps = SAMPLES[name]
    params = synth.model_params(wl.actor)
    lora = synth.lora_params(wl.actor, wl.lora_rank)
    prompts, forced = synth.prompts(wl).numpy(), synth.forced_tokens(wl).numpy()
    S, last = wl.prompt_len, max(steps)
    seq = np.concatenate([prompts[rows], forced[rows, :last]], axis=1)
    cols = [S - 1 + j for j in steps]

    def run(seed):
        om = O.OracleModel(wl.actor, params, O.Precision("bf16"), lora=lora,
                           lora_scale=wl.lora_scale, cache_layers=False)
        if seed:
            rng = np.random.default_rng(seed)
            embed = om.embed
            om.embed = lambda ids, pos0: (lambda e: e * (1.0 + EPS * rng.standard_normal(e.shape)))(embed(ids, pos0))
        h = om.hidden(seq, 0, None)
        return om.lm_logits(h[:, cols])            # [rows, steps, V]

    t0 = time.time()
    ref = run(0)
    worst = np.zeros((len(rows), len(steps)))
    for seed in SEEDS:
        worst = np.maximum(worst, np.abs(run(seed) - ref).max(axis=-1))
    rms = np.sqrt((ref ** 2).mean(axis=-1))
    entry = {"rows": rows, "steps": steps, "eps": EPS, "seeds": list(SEEDS),
             "max_abs_dlogit": worst.tolist(), "logit_rms": rms.tolist(),
             "seconds": round(time.time() - t0, 1)}
    print(name, json.dumps(entry), flush=True)
    return entry


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["_about"] = ("max |logit difference| of the oracle against itself with its embedding "
                      "output perturbed by relative N(0, 2^-24) noise; written by "
                      "tests/golden/make_oracle_sensitivity.py")
    for name in names:
        data[name] = measure(name)
        json.dump(data, open(OUT, "w"), indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or list(SAMPLES))

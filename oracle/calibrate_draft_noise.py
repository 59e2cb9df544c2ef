"""Write synth/draft_noise.json: draft-noise std for a target acceptance rate.

TEST INFRASTRUCTURE (uses only the oracle and the seeded generators).

The workloads build draft logits as target logits plus sigma * N(0, 1). For
each logit distribution used by a workload, this script bisects sigma until
the mean acceptance rate alpha = sum_x min(p(x), q(x)) ("Speculative
Decoding: Two Models, One Voice", Appendix tool 1) over a seeded sample of
rows hits the target. Run:

    python -m oracle.calibrate_draft_noise
"""

import json
import os

import numpy as np

import synth
from .softmax import softmax_rows

# (key, logit std, vocabulary, target alphas). The lm-head logits of the
# Llama-shaped stacks are sums of d_in products of N(0,1) activations and
# N(0, 0.02^2) weights, so their std is 0.02 * sqrt(d_in).
TARGETS = [
    ("llama8b_lm_head", 0.02 * 4096 ** 0.5, 128256, [0.8]),
    ("llama70b_lm_head", 0.02 * 8192 ** 0.5, 128256, [0.8]),
    ("stress_std3", 3.0, 128256, [0.6, 0.81, 0.9]),
]
ROWS = 32
SEED = 20260718


def mean_alpha(logits, noise, sigma):
    p, _, _ = softmax_rows(logits)
    q, _, _ = softmax_rows((logits + np.float32(sigma) * noise).astype(np.float32))
    return float(np.minimum(p, q).sum(axis=-1).mean()), np.minimum(p, q).sum(axis=-1)


def calibrate(logit_std, V, alpha, rows=ROWS, seed=SEED):
    logits = synth.normals(seed, f"calib.logits.{V}.{logit_std:.6f}", (rows, V), logit_std)
    noise = synth.normals(seed, f"calib.noise.{V}.{logit_std:.6f}", (rows, V), 1.0)
    lo, hi = 0.0, 8.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        a, _ = mean_alpha(logits, noise, mid)
        if a > alpha:
            lo = mid
        else:
            hi = mid
    sigma = 0.5 * (lo + hi)
    a, per_row = mean_alpha(logits, noise, sigma)
    return sigma, a, float(per_row.min()), float(per_row.max())


def main():
    out = {"recipe": (f"sigma bisected so that the mean of sum_x min(p, q) over {ROWS} "
                      f"seeded rows (seed {SEED}) of i.i.d. N(0, std^2) logits, with "
                      "q = softmax(logits + sigma * N(0,1)), equals alpha")}
    for key, std, V, alphas in TARGETS:
        rows = []
        for alpha in alphas:
            sigma, a, amin, amax = calibrate(std, V, alpha)
            rows.append({"alpha": alpha, "sigma": sigma, "achieved": a,
                         "row_min": amin, "row_max": amax})
            print(f"{key} alpha={alpha}: sigma={sigma:.6f} achieved={a:.6f} "
                  f"rows [{amin:.4f}, {amax:.4f}]", flush=True)
        out[key] = {"logit_std": std, "V": V, "rows": ROWS, "seed": SEED, "sigmas": rows}
    path = os.path.join(os.path.dirname(os.path.abspath(synth.__file__)), "draft_noise.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

"""Error of the 4-bit checkpoint recipe's activation quantisation, from the
oracle alone (no GPU, no HIP code): over 48 layers (4 shapes x 4 batch sizes
including a single token x 3 seeds) it compares the binary64 oracle that
round-trips x and h through MXFP8 (E4M3 elements, one E8M0 scale per 32
channels: what the 4-bit kernels compute) with the binary64 oracle on the
same MXFP4 weights and unquantised activations, and records max|a - b| /
max|b| per layer.  That distance is the recipe's own cost, so a bar on the
GPU output against the weight-only oracle has to sit above the largest of
these plus the GPU-versus-emulation allowance.

The 4-bit form stands in for the NVFP4 checkpoint the pages mention ("Hugging
Face releases Beam ...", checkpoint paragraph; "Reflection Beam", section
"Where to run it").

    python tests/golden/mx_recipe_study.py      # rewrites mx_recipe_study.json
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle                                   # noqa: E402
from synth import WORKLOADS, make_inputs, small_shape   # noqa: E402

SHAPES = [(512, 256, 64), (1024, 512, 32), (2048, 1024, 16), (384, 384, 64)]
TOKENS = (1, 2, 7, 33)
SEEDS = (0, 1, 2)


def configs():
    for (H, I, E) in SHAPES:
        for T in TOKENS:
            for seed in SEEDS:
                yield H, I, E, T, seed


def study_one(H, I, E, T, seed):
    """(whole-layer error, worst single-row error) of the MXFP8 emulation
    against the weight-only oracle for one layer."""
    sh = small_shape(hidden=H, intermediate=I, n_experts=E)
    inp = make_inputs(WORKLOADS["mxfp4_8k"], tokens=T, shape=sh,
                      seed=1000 + 37 * seed + T)
    lg = oracle.logits(sh, inp.x, inp.w_router)
    idx, w, _ = oracle.route(sh, lg, inp.bias.numpy())
    toks = np.arange(T)
    args = (sh, toks, inp.x, idx, w, inp.w_gate_up, inp.w_down, inp.s_gate_up,
            inp.s_down)
    ref = oracle.forward_tokens(*args, act_quant=False)
    emu = oracle.forward_tokens(*args, act_quant=True)
    whole = float(np.abs(emu - ref).max() / np.abs(ref).max())
    rows = max(float(np.abs(emu[i] - ref[i]).max() / np.abs(ref[i]).max())
               for i in range(T))
    return whole, rows


def main():
    cases = []
    for H, I, E, T, seed in configs():
        whole, rows = study_one(H, I, E, T, seed)
        cases.append({"H": H, "I": I, "E": E, "T": T, "seed": seed,
                      "layer_err": whole, "worst_row_err": rows})
        print(cases[-1], flush=True)
    errs = np.array([c["layer_err"] for c in cases])
    out = {
        "what": "max|emu - ref| / max|ref| per layer: emu = binary64 oracle with x and "
                "h round-tripped through MXFP8, ref = binary64 oracle with unquantised "
                "activations, both on the same MXFP4 weights",
        "script": "tests/golden/mx_recipe_study.py",
        "n": len(cases),
        "max": float(errs.max()),
        "mean": float(errs.mean()),
        "cases": cases,
    }
    with open(os.path.join(HERE, "mx_recipe_study.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(f"n={len(cases)} max {errs.max():.4e} mean {errs.mean():.4e}")


if __name__ == "__main__":
    main()

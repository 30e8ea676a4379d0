"""Writes tests/golden/tiny_greedy.json: the oracle's greedy run of the tiny
config (seeded prompt prefilled through the decode step, then 16 greedy
steps).  Calls only the oracle and the seeded generator."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def tiny_run():
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    o = oracle.Oracle(m, nthreads=1)
    p = synth.prompt(cfg)
    o.prefill(p[:-1])
    tok, logits = o.step(int(p[-1]), len(p) - 1)
    toks, maxes = [tok], [float(np.max(logits))]
    for i in range(cfg.decode_steps):
        tok, logits = o.step(toks[-1], cfg.prompt_len + i)
        toks.append(tok)
        maxes.append(float(np.max(logits)))
    return {"config": "tiny", "prompt": [int(t) for t in p], "greedy": toks, "max_logit": maxes}


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_greedy.json")
    with open(out, "w") as f:
        json.dump(tiny_run(), f, indent=1)
    print("wrote", out)

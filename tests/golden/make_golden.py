"""Writes tests/golden/tiny_oracle_greedy.json by calling only the oracle and the input generator.

The pages print no worked numeric example of a decode step, so the fixtures here are not
values from the pages; this one records the oracle's own greedy run on the tiny workload
(2 layers, hidden 256, 4/2 heads of 64, FFN 688, vocab 1024, fp16, 16-token prompt, 32
steps) so that any later change of the oracle's arithmetic shows up as a diff.  Regenerate
only together with a commit that names the passage or reading that justifies the change.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthgen  # noqa: E402


def run():
    w = synthgen.WORKLOADS["tiny"]
    wts = synthgen.make_weights(w)
    m = oracle.OracleModel(wts)
    prompt = synthgen.make_prompt(w)
    tok, lg = m.prefill(prompt)
    toks, heads = [tok], {"prefill": [float(v) for v in lg[:8]]}
    for i in range(w.steps):
        tok, lg = m.step(toks[-1])
        toks.append(tok)
        if i in (0, 15, 31):
            heads[f"step{i}"] = [float(v) for v in lg[:8]]
    return {"workload": "tiny", "prompt": [int(t) for t in prompt], "tokens": [int(t) for t in toks],
            "logits_head": heads}


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_greedy.json")
    with open(out, "w") as f:
        json.dump(run(), f, indent=1)
    print("wrote", out)

#!/usr/bin/env python3
"""Write tests/golden/qwen7b_2k_oracle.json: the oracle's values for the substitute-draft
workload at its own 2048-token context (7B-shaped bf16 target, seeded random-init
weights, 2048 seeded random prompt ids; its 4-bit group-64 substitute draft).

Calls only the oracle (oracle/) and the seeded input generators.  Float64 throughout;
takes about ten minutes and ~30 GB of host memory.

Stored (sampled columns: 512 seeded indices plus each row's top 8):
  saved_next   logits of the prompt's last position (the prefill's output row);
  rows[i]      logits after the oracle's own greedy tokens g_1..g_(i+1) (i = 0..7), one
               token at a time: row i predicts g_(i+2); rows[i] is what row i of an
               8-row verify block over [g_1..g_8] must produce;
  q4_step      logits of the 4-bit substitute draft's one-token step on g_1 at position
               2048 over the target's prefilled cache (the shared-cache draft step of
               the "SubSpec" summary, sections 4.1.1-4.1.3).
Each row also stores its argmax and top-2 margin.

Usage: python tests/golden/make_qwen7b_goldens.py [out.json]
"""
from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from block_verify_amd.shapes import QWEN_7B, SEED_TARGET  # noqa: E402
from block_verify_amd.synth import make_prompt, make_q4_draft, make_weights  # noqa: E402
from oracle.accept import argmax_lowest, top2_margin  # noqa: E402
from oracle.model import OracleCache, OracleWeights, forward, prefill  # noqa: E402

P, N_ROWS, N_COLS, TOP = 2048, 8, 512, 8
COL_SEED = 77


def row_record(logits, base_cols):
    logits = np.asarray(logits, np.float64)
    top = np.argsort(-logits, kind="stable")[:TOP]
    cols = sorted(set(int(c) for c in base_cols) | set(int(c) for c in top))
    return {"argmax": argmax_lowest(logits), "margin": top2_margin(logits), "cols": cols,
            "values": [float(np.float32(logits[c])) for c in cols]}


def main(out_path):
    S = QWEN_7B
    t0 = time.time()
    w = make_weights(S, SEED_TARGET)
    prompt = make_prompt(S.vocab, P)
    print(f"weights {time.time() - t0:.0f} s", flush=True)
    ow = OracleWeights(S, w, cache=False)
    cache = OracleCache(S, P + N_ROWS + 8)
    t0 = time.time()
    saved = prefill(ow, cache, prompt)
    print(f"prefill {time.time() - t0:.0f} s", flush=True)
    base_cols = np.random.default_rng(COL_SEED).choice(S.vocab, N_COLS, replace=False)

    # the 4-bit draft's step on g_1 over the prefilled shared cache (a copy: the target continues)
    q4t = make_q4_draft(S, w)
    qw_tensors = list(w)
    for i, t in enumerate(q4t):
        if isinstance(t, tuple):
            qw_tensors[i] = t
    qw = OracleWeights(S, qw_tensors, cache=False)
    g = [argmax_lowest(saved)]
    t0 = time.time()
    q4_logits = forward(qw, cache.clone(), [g[0]])[0]
    print(f"4-bit draft step {time.time() - t0:.0f} s", flush=True)

    rows = []
    for i in range(N_ROWS):
        t0 = time.time()
        lg = forward(ow, cache, [g[-1]])[0]
        rows.append(lg)
        g.append(argmax_lowest(lg))
        print(f"step {i}: token {g[-2]} -> next {g[-1]}  {time.time() - t0:.0f} s", flush=True)

    out = {
        "source": ("Oracle (oracle/model.py, float64, bf16-rounded K/V) on the 7B-shaped random-init target "
                   "(seed 0), the 2048-token seeded prompt (seed 20) and its 4-bit group-64 substitute draft; "
                   "written by tests/golden/make_qwen7b_goldens.py, which calls only oracle/ and the seeded "
                   "input generators."),
        "command": "python tests/golden/make_qwen7b_goldens.py",
        "shape": S.name, "prompt_len": P, "weights_seed": SEED_TARGET,
        "tokens": g[:N_ROWS],
        "next_after_rows": g[N_ROWS],
        "saved_next": row_record(saved, base_cols),
        "rows": [row_record(r, base_cols) for r in rows],
        "q4_step": row_record(q4_logits, base_cols),
    }
    with open(out_path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
    print(f"wrote {out_path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "qwen7b_2k_oracle.json"))

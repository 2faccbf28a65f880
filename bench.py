#!/usr/bin/env python3
"""Committed tok/s of block-verify speculative decoding on one MI355X.

Workload (default): a Qwen2.5-1.5B-shaped random-init bf16 target at a
2048-token context (prompt of 2048 seeded random ids, prefilled once), k = 4
drafts per round from the synthetic table (the target's own greedy
continuation with each position replaced with probability 0.46, seed 1),
64 committed tokens per job.  One "step" is one job: reset to the
post-prefill state, then rounds (draft provision, block verify, greedy
acceptance, trim, repair) until 64 tokens are committed.  Inputs are
resident in HBM before the timed region.

Prints one JSON line.  `value` = committed tokens / second over the timed
jobs (schedule B by default: the (k+1)-row verify pass; schedule A, the
k-row verify plus a one-token repair forward, is reported beside it).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "committed tok/s, k=4, 1.5B-shape @2K/8K ctx; verify HBM GB/s vs 8 TB/s peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """A ring of hipEvent_t created through the HIP runtime (timing only)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), 0)
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.arr[i] = ev.value
        self.n = n

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[a], self.arr[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(out.value)


def verify_bytes(shape, T: int, M: int) -> int:
    """Algorithmic HBM bytes of one forward of M rows at context T.

    Weights read once (every linear incl. the LM head, the norm gains), the
    K/V of the T cached positions and of the M new ones read by attention,
    the M new K/V written, the M logits rows written, the M embedding rows.
    """
    w = shape.weight_bytes_bf16() - 2 * shape.vocab * shape.hidden   # embedding table is gathered, not streamed
    kv_pos = shape.kv_bytes_per_token()
    return w + kv_pos * (T + M) + kv_pos * M + 4 * shape.vocab * M + 2 * shape.hidden * M


def gpu_ar(b, model, shape, prompt_t, n, max_len, torch):
    """Greedy AR with the same kernels (M=1 steps chained on the device)."""
    cache = b.Cache(shape, max_len)
    ws = b.Workspace(shape, max_len)
    toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    b.prefill(model, cache, prompt_t, ws, logits=logits, argmax=toks[0:1])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n - 1):
        b.decode_step(model, cache, toks[i:i + 1], ws, logits=logits, argmax=toks[i + 1:i + 2])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if ws.error_bits():
        raise RuntimeError(f"AR: device error bits {ws.error_bits()}")
    return [int(x) for x in toks[:n].cpu().numpy()], dt


def run_spec(b, model, shape, prompt, table, k, schedule, steps, warmup, n_new, max_len, torch, **round_kw):
    """Timed jobs replay the captured round.  The job time (the throughput) comes from
    the untimed replay, one HIP graph per round.  The per-term costs (draft, verify,
    accept, repair) come from a second handle on the same job that replays the round
    as its four segment graphs with the library's events between them, into a ring
    large enough that every timed round keeps its own timestamps; that replay pays
    one graph launch per segment, reported as its own job time beside the first."""
    r = b.Round(model, k, schedule=schedule, table=table, max_len=max_len, **round_kw)
    r.prefill(prompt)
    r.capture()
    for _ in range(warmup):
        r.run(n_new, graph=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks_all = []
    rounds = 0
    acc = 0
    for _ in range(steps):
        st, toks = r.run(n_new, graph=True)
        rounds += st.round
        acc += st.accepted_total
        toks_all.append(list(toks[:n_new]))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if r.ws.error_bits():
        raise RuntimeError(f"spec: device error bits {r.ws.error_bits()}")
    del r

    nvar = (n_new + 1) * max(steps, 1)
    ev = HipEvents(5 * nvar)
    rt = b.Round(model, k, schedule=schedule, table=table, max_len=max_len, events=ev.arr, n_events=5 * nvar,
                 **round_kw)
    rt.prefill(prompt)
    rt.capture()
    for _ in range(warmup):
        rt.run(n_new, graph=True)
    torch.cuda.synchronize()
    start_calls = rt.calls()
    t1 = time.perf_counter()
    for _ in range(steps):
        st, toks = rt.run(n_new, graph=True)
        toks_all.append(list(toks[:n_new]))
    torch.cuda.synchronize()
    dt_seg = time.perf_counter() - t1
    end_calls = rt.calls()
    terms = {"draft": [], "verify": [], "accept": [], "repair": [], "round": []}
    for c in range(start_calls, end_calls):
        base = (c % nvar) * 5
        rd = ev.ms(base, base + 4)
        if ev.ms(base + 1, base + 2) < 0.05:     # a launched round past the target returns at once
            continue
        terms["draft"].append(ev.ms(base, base + 1))
        terms["verify"].append(ev.ms(base + 1, base + 2))
        terms["accept"].append(ev.ms(base + 2, base + 3))
        terms["repair"].append(ev.ms(base + 3, base + 4))
        terms["round"].append(rd)
    if rt.ws.error_bits():
        raise RuntimeError(f"spec (timed replay): device error bits {rt.ws.error_bits()}")
    return dict(seconds=dt, seconds_segmented=dt_seg, rounds=rounds, accepted=acc, tokens=toks_all, terms=terms,
                prompt_len=len(prompt), t_len=rt.tcache.length())


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "verify_forward_1.5b_2k_traffic.md")


def measured_traffic():
    """HBM bytes per 5-row verify forward at a 2048-token context, from the committed
    FETCH_SIZE / WRITE_SIZE summary; None once a kernel source it lists has changed."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    val = None
    for line in text.splitlines():
        f = line.split()
        if len(f) == 3 and f[0] == "traffic_bytes_per_forward":
            val = int(f[2])
        elif len(f) == 3 and f[0] == "sha256":
            with open(os.path.join(ROOT, f[1]), "rb") as fh:
                if hashlib.sha256(fh.read()).hexdigest() != f[2]:
                    return None
    return val


def profile_forwards(b, model, shape, prompt_t, rows, n, max_len, torch):
    """Verify forwards at the prompt's context (trimmed back after each), timed with
    hipEvents, then a plain 256 MiB device-to-device copy (calibrates traffic counters)."""
    cache = b.Cache(shape, max_len)
    ws = b.Workspace(shape, max_len)
    logits = torch.empty((rows, shape.vocab), dtype=torch.float32, device="cuda")
    b.prefill(model, cache, prompt_t, ws, logits=logits[0])
    P = int(prompt_t.numel())
    toks = torch.arange(rows, dtype=torch.int32, device="cuda") * 977 + 13
    ev = HipEvents(2 * n)
    hip = ev.hip
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(n):
        hip.hipEventRecord(ev.arr[2 * i], stream)
        b.decode_step(model, cache, toks, ws, logits=logits)
        hip.hipEventRecord(ev.arr[2 * i + 1], stream)
        cache.trim(P, ws)
    torch.cuda.synchronize()
    us = [1e3 * ev.ms(2 * i, 2 * i + 1) for i in range(n)]
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    vb = verify_bytes(shape, P, rows)
    print(json.dumps({"mode": "forward-only", "rows": rows, "context": P, "forwards": n,
                      "us_per_forward_median": float(np.median(us)), "algorithmic_bytes": vb,
                      "copy_bytes": 256 << 20, "error_bits": ws.error_bits()}), flush=True)


def cpu_baseline(shape, weights, k, tau, budget_s=15.0, context=2048):
    """Time the oracle's schedule-B round (k+1-row verify forward + greedy accept + trim).

    Bounded sample: the oracle's cache holds `context` positions of seeded
    random K/V (the forward's cost does not depend on their values); the
    oracle's tokens/second = tau (tokens per round, measured on the GPU job)
    / oracle seconds per round.
    """
    from oracle.accept import greedy_accept, argmax_lowest
    from oracle.model import OracleCache, OracleWeights, forward
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    w = OracleWeights(shape, weights)
    cache = OracleCache(shape, context + 4 * (k + 1) + 8)
    rng = np.random.default_rng(5)
    for l in range(shape.n_layers):
        cache.k[l][:, :context] = rng.standard_normal((shape.n_kv_heads, context, shape.head_dim))
        cache.v[l][:, :context] = rng.standard_normal((shape.n_kv_heads, context, shape.head_dim))
    cache.length = context
    toks = rng.integers(0, shape.vocab, k + 1)

    def one_round():
        t = cache.length
        rows = forward(w, cache, toks)
        v = [argmax_lowest(rr) for rr in rows]
        m, com = greedy_accept(v, list(toks[1:]), True)
        cache.trim(t)

    t0 = time.perf_counter()
    one_round()             # first round also upcasts the weights (not timed)
    log(f"cpu baseline: warm-up round {time.perf_counter() - t0:.1f} s")
    n, t0 = 0, time.perf_counter()
    while True:
        one_round()
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s or n >= 50:
            break
    per_round = el / n
    return {"value": tau / per_round, "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{n} oracle schedule-B rounds (verify forward of {k + 1} rows, float64, at a "
                       f"{context}-position cache of seeded random K/V + greedy accept + trim), "
                       f"{per_round:.3f} s/round; tok/s = {tau:.3f} tokens/round (GPU job) / s per round")}


def run_substitute(args, torch):
    """Substitute-draft job at the 7B shape: depth-8 4-bit self-draft on the shared
    cache, 2048-token context, greedy, 64 tokens (schedule A).  Prints one JSON
    line of its own (a measurement of the 4-bit draft step, not the headline)."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_7B as S, SEED_TARGET
    from block_verify_amd.synth import make_prompt, make_q4_draft, make_weights
    D, P = 8, 2048
    max_len = P + args.n_new + 4 * (D + 2) + 64
    t0 = time.perf_counter()
    w = make_weights(S, SEED_TARGET)
    qt = make_q4_draft(S, w)
    model = b.Model(S, w)
    qmodel = b.Model(S, qt, weight_format=b.W_Q4G64, share=model)
    torch.cuda.synchronize()
    log(f"7B target + 4-bit draft ready in {time.perf_counter() - t0:.1f} s")
    prompt = make_prompt(S.vocab, P)
    ar_toks, ar_s = gpu_ar(b, model, S, torch.from_numpy(prompt).cuda(), args.n_new + D + 2, max_len, torch)
    ar_tok_s = (args.n_new + D + 1) / ar_s
    res = run_spec(b, model, S, prompt, None, D, 0, args.steps, args.warmup, args.n_new, max_len, torch,
                   draft_source=b.DRAFT_Q4_SELF, draft=qmodel)
    for toks in res["tokens"]:
        if toks != ar_toks[:args.n_new]:
            raise RuntimeError("substitute draft: committed tokens differ from the GPU AR decode")
    t = {k2: float(np.mean(v)) for k2, v in res["terms"].items()}
    kv_tok = S.kv_bytes_per_token()
    q4_lin = 0
    for rows, kk in [((S.n_q_heads + 2 * S.n_kv_heads) * S.head_dim, S.hidden), (S.hidden, S.n_q_heads * S.head_dim),
                     (2 * S.ffn, S.hidden), (S.hidden, S.ffn)]:
        nb = -(-kk // 128)
        q4_lin += S.n_layers * (rows * nb * 64 + rows * nb * 8)
    ctx = P + args.n_new // 2
    step_bytes = q4_lin + S.vocab * S.hidden * 2 + kv_tok * ctx + 4 * S.vocab
    step_ms = t["draft"] / (D - 1)
    out = {"mode": "substitute-7b", "workload": f"7B-shape target, 4-bit group-64 substitute draft (shared cache, "
                                                f"shared bf16 embedding / LM head), depth {D}, {P}-token context, "
                                                f"{args.n_new} tokens, greedy, schedule A",
           "tok_s": round(args.n_new * args.steps / res["seconds"], 2), "ar_tok_s": round(ar_tok_s, 2),
           "rounds_per_job": res["rounds"] / args.steps,
           "accepted_per_round": round(res["accepted"] / max(res["rounds"], 1), 3),
           "terms_ms": t, "q4_draft_step_ms": round(step_ms, 4),
           "q4_draft_step_bytes": int(step_bytes),
           "q4_draft_step_gbs": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
           "q4_linear_bytes": int(q4_lin)}
    print(json.dumps(out), flush=True)


def run_draft_model(b, model, S, args, torch, P=8192, corrupt=0.51, draft=None):
    """The draft-model leg: the same 1.5B-shape target with a 0.5B-shape draft model on
    its own cache (k draft steps per round, tokens from the corrupted-greedy table),
    schedule B, 64 tokens per job, at a P-token context."""
    from block_verify_amd.shapes import QWEN_0_5B, SEED_DRAFT
    from block_verify_amd.synth import make_draft_table, make_prompt, make_weights
    k = 4
    max_len = P + args.n_new + 4 * (k + 2) + 64
    if draft is None:
        draft = b.Model(QWEN_0_5B, make_weights(QWEN_0_5B, SEED_DRAFT))
    prompt = make_prompt(S.vocab, P)
    ar_toks, ar_s = gpu_ar(b, model, S, torch.from_numpy(prompt).cuda(), args.n_new + k + 2, max_len, torch)
    ar_tok_s = (args.n_new + k + 1) / ar_s
    table = make_draft_table(np.array(ar_toks), S.vocab, corrupt)
    r = run_spec(b, model, S, prompt, table, k, 1, args.steps, args.warmup, args.n_new, max_len, torch,
                 draft_source=b.DRAFT_MODEL, draft=draft)
    for toks in r["tokens"]:
        if toks != ar_toks[:args.n_new]:
            raise RuntimeError(f"{P}-token draft-model job: committed tokens differ from the GPU AR decode")
    t = {k2: float(np.mean(v)) for k2, v in r["terms"].items()}
    vb = verify_bytes(S, P + args.n_new // 2, k + 1)
    gbs = vb / (t["verify"] * 1e-3) / 1e9
    tok_s = args.n_new * args.steps / r["seconds"]
    log(f"{P}-token draft-model job: {tok_s:.1f} tok/s, verify {t['verify'] * 1e3:.1f} us")
    return draft, {"workload": f"1.5B-shape target, {P}-token context, 0.5B-shape draft model on its own cache, k={k}, "
                        f"{args.n_new} committed tokens, table drafts corrupt p={corrupt}, greedy, schedule B",
            "tok_s": round(tok_s, 2), "ar_tok_s": round(ar_tok_s, 2), "R_spec_over_ar": round(tok_s / ar_tok_s, 3),
            "rounds_per_job": r["rounds"] / args.steps, "terms_ms": t,
            "draft_step_ms": round(t["draft"] / k, 4),
            # the pages' ratio for this workload shape (RTX 4060 Laptop, trained Qwen2.5-1.5B / 0.5B): context only
            "pages_R_spec_over_ar": {2048: 0.531, 4096: 0.485, 8192: 0.522}.get(P),
            "verify_gbs": round(gbs, 1), "verify_frac": round(gbs / PEAK_HBM_GBS, 4), "verify_bytes": vb}


def run_stochastic_4k(b, model, S, args, torch):
    """The 4096-token stochastic leg: modified rejection sampling with the noisy
    self-draft (q = softmax(target logits + N(0,1) noise), Philox seed 3),
    schedule A, k = 4, 64 tokens per job."""
    from block_verify_amd.synth import make_noise, make_prompt
    k, P = 4, 4096
    max_len = P + args.n_new + 4 * (k + 2) + 64
    prompt = make_prompt(S.vocab, P)
    noise = make_noise(args.n_new + 2 * k + 2, S.vocab)
    r = run_spec(b, model, S, prompt, None, k, 0, args.steps, args.warmup, args.n_new, max_len, torch,
                 mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=3)
    if any(t != r["tokens"][0] for t in r["tokens"]):
        raise RuntimeError("stochastic leg: jobs with the same seeds committed different tokens")
    t = {k2: float(np.mean(v)) for k2, v in r["terms"].items()}
    tok_s = args.n_new * args.steps / r["seconds"]
    log(f"4K stochastic: {tok_s:.1f} tok/s, accept {t['accept'] * 1e3:.1f} us")
    return {"workload": f"1.5B-shape target, {P}-token context, modified rejection sampling, noisy self-draft "
                        f"(N(0,1) logit noise, seed 2; Philox seed 3), k={k}, {args.n_new} tokens, schedule A",
            "tok_s": round(tok_s, 2), "rounds_per_job": r["rounds"] / args.steps,
            "accepted_per_round": round(r["accepted"] / max(r["rounds"], 1), 3), "terms_ms": t,
            "accept_us": round(t["accept"] * 1e3, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--schedule", choices=["A", "B"], default="B")
    ap.add_argument("--context", type=int, default=2048)
    ap.add_argument("--n-new", type=int, default=64)
    ap.add_argument("--corrupt", type=float, default=0.46)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward-only", type=int, default=0,
                    help="profiling mode: after the prefill run this many verify forwards of k+1 rows "
                         "(no jobs), then one 256 MiB device copy of known size for counter calibration")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-8k", action="store_true", help="skip the 8192-token leg")
    ap.add_argument("--no-stochastic", action="store_true", help="skip the 4096-token stochastic leg")
    ap.add_argument("--substitute-7b", action="store_true",
                    help="measure the 7B substitute-draft job (4-bit draft steps) instead of the headline job")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    if args.substitute_7b:
        run_substitute(args, torch)
        return
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_1_5B as S, SEED_TARGET
    from block_verify_amd.synth import make_draft_table, make_prompt, make_weights

    k = 4
    P = args.context
    max_len = P + args.n_new + 4 * (k + 2) + 64
    t0 = time.perf_counter()
    weights = make_weights(S, SEED_TARGET)
    model = b.Model(S, weights)
    torch.cuda.synchronize()
    log(f"model ready in {time.perf_counter() - t0:.1f} s")
    prompt = make_prompt(S.vocab, P)
    prompt_t = torch.from_numpy(prompt).cuda()

    if args.forward_only:
        profile_forwards(b, model, S, prompt_t, k + 1, args.forward_only, max_len, torch)
        return
    ar_toks, ar_s = gpu_ar(b, model, S, prompt_t, args.n_new + k + 2, max_len, torch)
    ar_tok_s = (args.n_new + k + 1) / ar_s
    log(f"AR: {ar_tok_s:.1f} tok/s")
    table = make_draft_table(np.array(ar_toks), S.vocab, args.corrupt)

    res = {}
    for sched in ("A", "B"):
        res[sched] = run_spec(b, model, S, prompt, table, k, 0 if sched == "A" else 1, args.steps, args.warmup,
                              args.n_new, max_len, torch)
        for toks in res[sched]["tokens"]:
            if toks != ar_toks[:args.n_new]:
                raise RuntimeError(f"schedule {sched}: committed tokens differ from the GPU AR decode")
        log(f"schedule {sched}: {args.n_new * args.steps / res[sched]['seconds']:.1f} tok/s, "
            f"{res[sched]['rounds'] / args.steps:.1f} rounds/job")

    main_r = res[args.schedule]
    value = args.n_new * args.steps / main_r["seconds"]
    terms = {s: {t: float(np.mean(v)) for t, v in res[s]["terms"].items()} for s in res}
    rows = k + (1 if args.schedule == "B" else 0)
    vb = verify_bytes(S, P + args.n_new // 2, rows)
    v_ms = float(np.mean(main_r["terms"]["verify"]))
    achieved = vb / (v_ms * 1e-3) / 1e9
    traffic = measured_traffic() if (P == 2048 and rows == 5 and k == 4) else None
    rounds_per_job = main_r["rounds"] / args.steps
    tau = args.n_new / rounds_per_job
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(main_r["seconds"] * 1e3 / args.steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, random prompt ids, corrupted greedy-continuation drafts)",
        "config": {"workload": f"1.5B-shape target, {P}-token context, k={k}, {args.n_new} committed tokens, "
                               f"table drafts corrupt p={args.corrupt}, greedy, schedule {args.schedule}",
                   "context": P, "k": k, "n_new": args.n_new, "schedule": args.schedule},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": f"verify forward ({rows} rows), {vb} algorithmic bytes, {v_ms * 1e3:.1f} us avg"},
        "terms_ms": terms,
        "terms_replay": "four segment graphs per round with events between them",
        "segmented_tok_s": {s_: round(args.n_new * args.steps / res[s_]["seconds_segmented"], 2) for s_ in res},
        "schedule_A_tok_s": round(args.n_new * args.steps / res["A"]["seconds"], 2),
        "schedule_B_tok_s": round(args.n_new * args.steps / res["B"]["seconds"], 2),
        "ar_tok_s": round(ar_tok_s, 2),
        "R_spec_over_ar": round(value / ar_tok_s, 3),
        "rounds_per_job": round(rounds_per_job, 2),
        "acceptance_per_drafted": round(main_r["accepted"] / (k * main_r["rounds"]), 4),
        "tokens_per_round": round(tau, 3),
    }
    if not args.no_8k:
        # the draft model's cost at the headline context (the pages' 2K comparison) and at 8K
        draft, out["draft_model_2k"] = run_draft_model(b, model, S, args, torch, P=2048, corrupt=args.corrupt)
        _, out["context_8k"] = run_draft_model(b, model, S, args, torch, P=8192, corrupt=0.51, draft=draft)
    if not args.no_stochastic:
        out["stochastic_4k"] = run_stochastic_4k(b, model, S, args, torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(S, weights, k, tau, args.cpu_budget, P)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

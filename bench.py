"""Rollout throughput of the self-speculative step vs plain autoregressive decoding.

Workload (defaults): Qwen2.5-7B-shaped decoder in bf16, random init N(0, 0.02),
W4 group-128 asymmetric self-drafter, 256 prompts of 512 uniform tokens,
per-sequence stop lengths lognormal(median 2048, sigma 0.75) capped at 16384,
so the active batch shrinks from 256 to 1; temperature 1, top-p 1, gamma
adaptive in 1..8 (roofline toggle + EMA of the acceptance rate).

A step is one pass of the whole hot path over the live batch: the controller
picks AR or SD (and gamma), then draft -> verify -> rejection sample -> KV
commit/rollback.

Default (--steps K, --warmup W): the shrinking-batch sweep.  The stop-length
draw fixes, for every batch bin of the rollout (129-256, 65-128, ..., 2, 1),
how many steps it takes, how many tokens it emits, its mean live batch and
its mean context (one token per sequence per step: at step k the live batch
is #{stop - 1 > k} and every live sequence holds 512 + k keys).  Each bin is
prefilled at its mean batch and context, then runs W untimed and K timed
steps in each of SD-auto (the roofline toggle), forced SD and AR; an
untimed pass of K steps per mode then brackets every kernel launch with HIP
events (the roofline object and the per-bin draft / verify HBM fractions).
`value` is SD-auto tokens / seconds over its timed steps of all bins; the
rollout figures compose the bins' rates with their token counts.

--rollout (or --steps 0) runs the whole 256 -> 1 rollout to completion in
SD-auto and AR instead; --crossover runs the fixed-batch sweep.

Prints one JSON line (N = 1 only: the library runs on one GPU).
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import re
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rollout tokens/s SD vs AR, batch 256→1; verify/draft HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFS = 2500.0  # dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def no_gc():
    """Timed loops run without the cyclic garbage collector (collected just before): a full
    collection over the interpreter's objects takes tens of milliseconds, which would otherwise
    land inside whichever timed step triggers it.  Reference counting still frees as usual."""
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps per batch bin and mode (0 = run the rollout to completion)")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps per batch bin and mode")
    ap.add_argument("--rollout", action="store_true", help="the whole 256 -> 1 rollout instead of the bin sweep")
    ap.add_argument("--history", action="store_true",
                    help="the history drafter: an untimed earlier rollout of the prompts fills its cache, then "
                         "the same prompts are timed under ER_POLICY_HISTORY and AR")
    ap.add_argument("--history-new", type=int, default=256, help="tokens per sequence in --history")
    ap.add_argument("--history-gamma", type=int, default=4)
    ap.add_argument("--history-prefix", type=int, default=4)
    ap.add_argument("--group", type=int, default=0,
                    help="GRPO-style groups: every G sequences of a bin share their prefilled context's KV blocks")
    ap.add_argument("--config", default="", help="model shape (default qwen2.5-7b; qwen2.5-14b with --crossover)")
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--prompt-len", type=int, default=512)
    ap.add_argument("--median", type=float, default=2048)
    ap.add_argument("--cap", type=int, default=16384)
    ap.add_argument("--gamma-max", type=int, default=8)
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--top-p", type=float, default=1.0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--mode", choices=["both", "sd", "ar", "force-sd", "timing", "both+timing"], default="both",
                    help="rollouts to run: SD-auto (roofline toggle) and AR by default; 'timing' runs the "
                         "measured-timing guard policy")
    ap.add_argument("--gamma", type=int, default=0, help="pin gamma (0 = adaptive)")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (testing only)")
    ap.add_argument("--kv-blocks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-profile", action="store_true")
    ap.add_argument("--persistent", action="store_true",
                    help="run forwards of <= 16 rows as the persistent decode kernel (default: kernel sequence)")
    ap.add_argument("--library-gemm", type=int, default=-1,
                    help="library GEMMs for the target's projections: -1 from each shape's measured row threshold, "
                         "N > 0 from N rows for every shape, 0 never")
    ap.add_argument("--graphs", type=int, default=16,
                    help="replay recorded graphs for steps of at most this many sequences (0: every step eager)")
    ap.add_argument("--kprof-every", type=int, default=4,
                    help="bracket the attention launches of every this many steps of the timed rollout with HIP "
                         "events (events on every launch slow each step by ~0.3 ms)")
    ap.add_argument("--progress", type=float, default=20.0, help="seconds between progress lines")
    ap.add_argument("--crossover", action="store_true",
                    help="fixed-batch SD/AR sweep instead of the rollout: every sequence at --context keys, "
                         "batches --batches, gamma in --gammas and AR (default config qwen2.5-14b)")
    ap.add_argument("--batches", default="1,2,4,8,16,32,64,128")
    ap.add_argument("--gammas", default="2,4,6,8")
    ap.add_argument("--context", type=int, default=8192)
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only copy this many bytes device-to-device 10 times and exit (calibrates HBM byte counters)")
    return ap.parse_args()


def shape_is_bf16(eng):
    return getattr(eng.shape, "dtype", "bf16") == "bf16"


def engine_options(eng, args):
    """The launch options every bench engine runs with."""
    if args.persistent:
        eng.set_persistent(True)
    if args.graphs:
        eng.set_graphs(args.graphs)
    if args.library_gemm != -1 and shape_is_bf16(eng):
        eng.set_library_gemm(args.library_gemm)


def make_engine(args, shape, wts, policy):
    from speculative_decoding_rl_amd import Engine

    max_ctx = args.prompt_len + args.cap + args.gamma_max + 16
    max_ctx = (max_ctx + 15) // 16 * 16
    if args.kv_blocks:
        kv_blocks = args.kv_blocks
    else:
        # peak live KV of the shrinking batch is far below batch * max_ctx; size the pool
        # for the expected peak with margin (the lognormal tail is long, the batch is not)
        exp_len = args.prompt_len + args.median * math.exp(0.75 ** 2 / 2)
        kv_blocks = int(args.batch * (exp_len / 16 + 2) * 1.6) + 2 * (max_ctx // 16)
    eng = Engine(shape, wts, shape.quant, seed=args.seed, temperature=args.temperature, top_p=args.top_p,
                 gamma_init=4, gamma_min=1, gamma_max=args.gamma_max, policy=policy, max_seqs=args.batch + 64,
                 max_batch=args.batch, max_ctx=max_ctx, prefill_chunk=8192, kv_blocks=kv_blocks)
    engine_options(eng, args)
    return eng


def run_rollout(eng, args, prompts, stops, label):
    """Prefill, then steps until done (or K steps). Returns per-step records and totals."""
    import torch

    n = len(prompts)
    ids = eng.kv_alloc([args.prompt_len] * n, stops)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first = eng.prefill(ids, list(prompts))
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    log(f"[{label}] prefill {n}x{args.prompt_len} tokens: {t_prefill:.2f} s")
    gen = {int(i): 1 for i in ids}                 # the prefill token counts toward the stop length
    stop = {int(i): int(s) for i, s in zip(ids, stops)}
    active = [int(i) for i in ids if gen[int(i)] < stop[int(i)]]
    recs = []
    eng.reset_stats()
    from speculative_decoding_rl_amd import _lib
    prof = not args.no_kernel_profile
    if prof:
        eng.reset_kernel_profile()
    gc.collect()
    gc_was = gc.isenabled()
    gc.disable()   # as no_gc(): no collection pause inside a timed step
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    t_last = t_start
    k = 0
    while active and (args.steps == 0 or k < args.steps):
        B = len(active)
        if prof:   # the dominant kernel (attention), timed live on a sample of the steps
            eng.set_kernel_profile(_lib.ER_KPROF_ATTENTION if k % args.kprof_every == 0 else _lib.ER_KPROF_OFF)
        cbar = args.prompt_len + sum(gen[a] for a in active) / B - 1   # committed keys before this step
        ts = time.perf_counter()
        tok, ne, info = eng.step(active)
        te = time.perf_counter()
        recs.append((B, int(info.mode), int(info.gamma), int(ne.sum()), te - ts, int(info.accepted), cbar))
        for b, a in enumerate(active):
            gen[a] += int(ne[b])
        active = [a for a in active if gen[a] < stop[a]]
        k += 1
        if te - t_last > args.progress:
            done = sum(r[3] for r in recs)
            log(f"[{label}] step {k}: active {len(active)}, tokens {done}, "
                f"{done / (te - t_start):.0f} tok/s, mode {'SD' if info.mode else 'AR'} gamma {info.gamma}")
            t_last = te
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    if gc_was:
        gc.enable()
    kprof = eng.kernel_profile() if prof else []
    if prof:
        eng.set_kernel_profile(False)
    stats = eng.stats()
    left = [a for a in ids if gen[int(a)] < stop[int(a)]]
    eng.kv_free(ids)
    tokens = sum(r[3] for r in recs)
    log(f"[{label}] {k} steps, {tokens} tokens in {t_total:.2f} s -> {tokens / t_total:.1f} tok/s")
    return dict(recs=recs, t=t_total, tokens=tokens, steps=k, prefill_s=t_prefill, kprof=kprof, stats=stats,
                unfinished=len(left))


class Roofline:
    """Per-step roofline time of the method's algorithmic work (bytes at 8 TB/s, flops at 2.5 PFLOP/s).

    AR step: bytes 2*P_lin + B*C*kvb + B*kvb + 4*B*V, flops 2*P_lin*B + 4*B*C*hq*hd*L.  SD step: gamma
    drafter forwards (b_q*P_lin + B*C*kvb + B*kvb + 4*B*V bytes each) plus one verify forward over B*(gamma+1)
    rows.  C = committed keys per sequence; each forward is priced at max(bytes/BW, flops/FLOPS).
    """

    def __init__(self, shape):
        d, hq, hkv, hd, F, L, V = (shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                                   shape.n_layers, shape.vocab)
        self.P = L * (d * (hq + 2 * hkv) * hd + hq * hd * d + 3 * F * d) + V * d
        el = 2 if shape.dtype == "bf16" else 4
        self.wb = el
        self.qb = 0.5 + 3.0 / 128 if shape.quant == "w4" else 1.0
        self.kvb = L * 2 * hkv * hd * el
        self.att = 4.0 * hq * hd * L
        self.V = V

    def fwd(self, wbytes, rows, B, C):
        by = wbytes * self.P + B * C * self.kvb + rows * self.kvb + 4.0 * rows * self.V
        fl = 2.0 * self.P * rows + rows * C * self.att
        return max(by / (HBM_PEAK_GBS * 1e9), fl / (MFMA_PEAK_TFS * 1e12))

    def step(self, mode, gamma, B, C):
        if mode == 0:
            return self.fwd(self.wb, B, B, C)
        return gamma * self.fwd(self.qb, B, B, C) + self.fwd(self.wb, B * (gamma + 1), B, C)


def bins(recs, roof=None):
    edges = [256, 128, 64, 32, 16, 8, 4, 2, 1]
    out = []
    for hi, lo in zip(edges[:-1] + [1], edges[1:] + [0]):
        sel = [r for r in recs if lo < r[0] <= hi]
        if not sel:
            continue
        tok = sum(r[3] for r in sel)
        t = sum(r[4] for r in sel)
        sd = sum(1 for r in sel if r[1] == 1)
        row = dict(batch=f"{lo + 1}-{hi}", steps=len(sel), tokens=tok, seconds=round(t, 4),
                   tok_per_s=round(tok / t, 1) if t > 0 else None, sd_steps=sd)
        if roof is not None and t > 0:
            # the same steps at the roofline: how much of the HBM / MFMA bound the step time reaches
            row["roofline_frac"] = round(sum(roof.step(r[1], r[2], r[0], r[6]) for r in sel) / t, 4)
        out.append(row)
    return out


LINEAR_KERNELS = ("k_skinny", "k_linear_mfma", "k_linear_valu", "k_wgemm", "k_gemm2", "k_gemm_bf16")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from a committed counter summary under profiles/, or None.

    A summary names its kernel and the source files its traffic depends on, each with its sha256 when the
    counters were taken; a summary any of whose sources has changed since is ignored (the counters
    describe other code).
    """
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        fields, sources = {}, []
        for line in open(path):
            k, sep, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if not sep:
                continue
            if k == "source":
                sources.append([v, None])
            elif k == "source_sha256" and sources:
                sources[-1][1] = v
            elif k in ("kernel", "traffic_bytes_per_launch"):
                fields[k] = v
        if fields.get("kernel") != kernel or not sources:
            continue
        ok = True
        for rel, sha in sources:
            src = os.path.join(ROOT, rel)
            if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != sha:
                ok = False
        if not ok:
            continue
        try:
            return float(fields["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            continue
    return None


def kernel_pass(eng, args, prompts, n, policy, steps=32):
    """Every linear and attention launch timed with HIP events, outside the timed rollouts:
    prefill of the first n prompts, then `steps` steps under `policy` at that batch (forced
    speculation makes the drafter's and the verify pass's kernels appear)."""
    from speculative_decoding_rl_amd import _lib
    n = min(n, len(prompts))
    eng.set_policy(policy)
    ids = eng.kv_alloc([args.prompt_len] * n, [steps * (args.gamma_max + 1) + 8] * n)
    eng.prefill(ids, list(prompts[:n]))
    eng.reset_kernel_profile()
    eng.set_kernel_profile(_lib.ER_KPROF_ALL)
    act = [int(i) for i in ids]
    for _ in range(steps):
        act = [a for a in act if not eng.seq_info(a)[2]]
        if not act:
            break
        eng.step(act)
    kprof = eng.kernel_profile()
    eng.set_kernel_profile(_lib.ER_KPROF_OFF)
    eng.kv_free(ids)
    return kprof


def roofline_from(kprof):
    """Roofline object of the dominant kernel (largest total time over the timed region).

    achieved = algorithmic bytes (or flops) per launch / average launch time, both from the
    HIP events the library records around each launch on its stream.  A kernel whose
    algorithmic intensity is above the ridge (2.5 PFLOP/s / 8 TB/s) is priced against bf16
    MFMA peak, otherwise against HBM.
    """
    if not kprof:
        return None, None
    top = max(kprof, key=lambda k: k["ms"])
    sec = top["ms"] * 1e-3
    intensity = top["flops"] / top["bytes"] if top["bytes"] > 0 else 0.0
    if intensity > MFMA_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        tfs = top["flops"] / sec / 1e12
        rf = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s",
              "frac": round(tfs / MFMA_PEAK_TFS, 4), "traffic": None}
    else:
        gbs = top["bytes"] / sec / 1e9
        tr = measured_traffic(top["name"])
        rf = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": round(tr) if tr is not None else None}
    detail = {"kernel": top["name"], "launches": top["launches"], "avg_us": round(top["ms"] * 1e3 / top["launches"], 2),
              "avg_bytes": round(top["bytes"] / top["launches"]), "avg_flops": round(top["flops"] / top["launches"]),
              "share_of_profiled_time": round(top["ms"] / sum(k["ms"] for k in kprof), 4)}
    # the dominant linear kernel too (the verify / draft GEMV path)
    lin = [k for k in kprof if any(n in k["name"] for n in LINEAR_KERNELS)]
    if lin:
        tl = max(lin, key=lambda k: k["ms"])
        g = tl["bytes"] / (tl["ms"] * 1e-3) / 1e9
        detail["top_linear"] = {"kernel": tl["name"], "avg_us": round(tl["ms"] * 1e3 / tl["launches"], 2),
                                "achieved_gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4)}
    return rf, detail


def kernel_role(name):
    """draft: the quantized drafter's linears (W8 / W4 formats); target: the bf16 target's linears
    (the verify pass and the AR step); attention serves both (the drafter reads the target's KV)."""
    if name.startswith("er::k_attn"):
        return "attention"
    m = re.match(r"er::k_(skinny|linear_mfma)<(\d+)", name)
    if m:
        return "draft" if int(m.group(2)) in (2, 3) else "target"
    # the weight-streaming GEMM names its format first only for the quantized weights (five arguments)
    m = re.match(r"er::k_wgemm<([^>]*)>", name)
    if m and len(m.group(1).split(",")) == 5:
        return "draft" if int(m.group(1).split(",")[0]) in (2, 3) else "target"
    return "target"


def kernel_table(kprof):
    rows = []
    for k in sorted(kprof, key=lambda k: -k["ms"]):
        gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9 if k["ms"] > 0 else 0.0
        rows.append(dict(name=k["name"], role=kernel_role(k["name"]), launches=k["launches"], ms=round(k["ms"], 2),
                         avg_us=round(k["ms"] * 1e3 / max(1, k["launches"]), 2), gbs=round(gbs, 1),
                         frac_hbm=round(gbs / HBM_PEAK_GBS, 3)))
    return rows


def cpu_baseline(shape_name, args):
    """The oracle (fp64 NumPy, per sequence) timed on the host, on all its BLAS threads and on one:

    - the tiny fp32 decoder (4 prompts x 32 uniform tokens, 64 new, gamma 4, W8 drafter): the full
      SD and AR rollouts;
    - the workload's model shape at batch 1 and 8 from a 512-token context, gamma 4: SD and AR steps,
      each bounded by a time budget, on a 2-layer full-width slice (vocab, widths and heads as the
      workload), per-step time scaled to the full depth by the ratio of streamed linear parameters
      (the oracle is bound by reading its fp64 weights), so those figures are extrapolated.  The
      batch-8 states are copies of one prefilled state under eight sequence ids (the oracle's cost
      does not depend on the KV contents).

    value: SD tokens/s of the workload shape at batch 1 on all threads (the unit of the GPU line).
    """
    import copy

    import synth
    from oracle import spec as OSP
    from oracle.controller import ModelCost
    from oracle.model import config_from, weights_from
    from threadpoolctl import threadpool_info, threadpool_limits

    threads_all = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    sp = OSP.SamplingParams(seed=args.seed, temperature=args.temperature, top_p=args.top_p)
    runs = []

    # the tiny decoder, whole rollouts
    ts = synth.shape("tiny")
    tw = synth.weights(ts, seed=args.seed)
    tcfg = config_from(ts)
    TW = weights_from(tcfg, {k: v.float().numpy() for k, v in tw.items()})
    TD = OSP.build_drafter(TW, "w8")
    tpr = [list(p) for p in synth.prompts(4, 32, ts.vocab, seed=args.seed)]
    for nthr in (threads_all, 1):
        with threadpool_limits(limits=nthr):
            t0 = time.perf_counter()
            out = OSP.rollout_spec(tcfg, TW, TD, tpr, [64] * 4, 4, sp)
            t_sd = time.perf_counter() - t0
            t0 = time.perf_counter()
            out_ar = OSP.rollout_ar(tcfg, TW, tpr, [64] * 4, sp)
            t_ar = time.perf_counter() - t0
        n_tok = sum(len(o) for o in out)
        runs.append(dict(model="tiny", threads=nthr, batch=4, kind="full rollout", sd_tok_s=round(n_tok / t_sd, 2),
                         ar_tok_s=round(sum(len(o) for o in out_ar) / t_ar, 2), seconds=round(t_sd + t_ar, 2)))

    # the workload's shape, a 2-layer slice, bounded step samples
    full = synth.shape(shape_name)
    sl = synth.shape(shape_name, n_layers=2)
    t0 = time.perf_counter()
    wts = synth.weights(sl, seed=args.seed)
    cfg = config_from(sl)
    W = weights_from(cfg, {k: v.float().numpy() for k, v in wts.items()})
    del wts
    D = OSP.build_drafter(W, sl.quant)
    ctx, gamma = 512, 4
    budget_sd, budget_ar, max_steps = 3.0, 1.5, 64
    cap = ctx + (gamma + 1) * max_steps * 2 + 8
    base = OSP.prefill(cfg, W, 0, list(synth.prompts(1, ctx, sl.vocab, seed=args.seed)[0]), 10**6, cap, sp)
    setup = time.perf_counter() - t0
    mc = lambda s: ModelCost(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab, 2, 0.52, 2)
    scale = mc(full).p_lin / mc(sl).p_lin
    for nthr in (threads_all, 1):
        for B in (1, 8):
            states = []
            for b in range(B):
                st = copy.copy(base)
                st.kv = base.kv.copy()
                st.generated = list(base.generated)
                st.seq_id = b
                states.append(st)
            with threadpool_limits(limits=nthr):
                t0 = time.perf_counter()
                n_sd = tok_sd = 0
                while n_sd < 1 or (time.perf_counter() - t0 < budget_sd and n_sd < max_steps):
                    for st in states:
                        tok_sd += len(OSP.spec_step(cfg, W, D, st, gamma, sp).emitted)
                    n_sd += 1
                t_sd = (time.perf_counter() - t0) / n_sd
                t0 = time.perf_counter()
                n_ar = 0
                while n_ar < 1 or (time.perf_counter() - t0 < budget_ar and n_ar < max_steps):
                    for st in states:
                        OSP.ar_step(cfg, W, st, sp)
                    n_ar += 1
                t_ar = (time.perf_counter() - t0) / n_ar
            runs.append(dict(model=f"{shape_name} (2 of {full.n_layers} layers, extrapolated x{scale:.2f})",
                             threads=nthr, batch=B, context=ctx, gamma=gamma, sd_steps=n_sd, ar_steps=n_ar,
                             tokens_per_seq_sd_step=round(tok_sd / (n_sd * B), 3),
                             sd_tok_s=round((tok_sd / n_sd) / (t_sd * scale), 4),
                             ar_tok_s=round(B / (t_ar * scale), 4), seconds=round(t_sd * n_sd + t_ar * n_ar, 2)))
    head = next(r for r in runs if r["model"] != "tiny" and r["threads"] == threads_all and r["batch"] == 1)
    return {"value": head["sd_tok_s"], "unit": "tokens/s", "cores": int(threads_all), "kind": "oracle",
            "sample": (f"oracle (fp64 numpy, one sequence at a time): {shape_name} at batch 1, context {ctx}, "
                       f"gamma {gamma}, SD steps for {budget_sd:.0f} s on a 2-layer full-width slice, per-step time "
                       f"scaled to {full.n_layers} layers by streamed parameters (x{scale:.2f}, extrapolated); "
                       f"also batch 8, one thread, and the tiny decoder's full rollouts (runs); setup "
                       f"{setup:.0f} s untimed"),
            "host_cpu_count": os.cpu_count(), "ar_value": head["ar_tok_s"],
            "measured_s": round(sum(r["seconds"] for r in runs), 2), "runs": runs}


BIN_EDGES = (256, 128, 64, 32, 16, 8, 4, 2, 1)


def bin_plan(stops, prompt_len, batch):
    """The batch bins of the shrinking-batch rollout, paced one token per sequence per step: at step k
    the live batch is #{i : stop_i - 1 > k} (the prefill token counts toward the stop length) and every
    live sequence holds prompt_len + k committed keys.  Per bin (lo, hi]: its steps, its tokens, the
    step-mean live batch and the step-mean context."""
    act = np.asarray(stops, dtype=np.int64) - 1
    ks = np.arange(int(act.max()))
    B = np.searchsorted(np.sort(act), ks, side="right")
    B = len(act) - B                                   # #{act > k}
    edges = [e for e in BIN_EDGES if e < batch]
    out = []
    for hi, lo in zip([batch] + edges, edges + [0]):
        sel = (B > lo) & (B <= hi)
        n = int(sel.sum())
        if n == 0:
            continue
        tok = int(B[sel].sum())
        out.append(dict(bin=f"{lo + 1}-{hi}" if hi > lo + 1 else f"{hi}", lo=lo, hi=hi, plan_steps=n,
                        plan_tokens=tok, batch=max(1, int(round(tok / n))),
                        context=int(round(prompt_len + ks[sel].mean()))))
    return out


def merge_kprof(lists):
    """Sum kernel-profile records (one list per pass) by kernel name."""
    acc = {}
    for lst in lists:
        for k in lst:
            a = acc.setdefault(k["name"], dict(name=k["name"], launches=0, ms=0.0, bytes=0.0, flops=0.0))
            a["launches"] += k["launches"]
            a["ms"] += k["ms"]
            a["bytes"] += k["bytes"]
            a["flops"] += k["flops"]
    return list(acc.values())


def role_tops(kprof):
    """The largest-time kernel of each role with its achieved HBM rate."""
    out = {}
    for role in ("draft", "target", "attention"):
        ks = [k for k in kprof if kernel_role(k["name"]) == role and k["ms"] > 0]
        if not ks:
            continue
        k = max(ks, key=lambda k: k["ms"])
        gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
        out[role] = dict(kernel=k["name"], avg_us=round(k["ms"] * 1e3 / k["launches"], 2), gbs=round(gbs, 1),
                         frac_hbm=round(gbs / HBM_PEAK_GBS, 4), share=round(k["ms"] / sum(x["ms"] for x in kprof), 4))
    return out


SWEEP_MODES = (("sd", "SD-auto"), ("force-sd", "forced SD"), ("ar", "AR"))


def sweep(args, shape, wts, stops):
    """The timed measurement: every batch bin of the rollout at its mean batch and context, W
    untimed and K timed steps per mode, then an untimed all-launch profile pass (see the module notes)."""
    import torch

    import synth
    from speculative_decoding_rl_amd import Engine, _lib

    plan = bin_plan(stops, args.prompt_len, args.batch)
    K, Wm = args.steps, args.warmup
    per_step = args.gamma_max + 1
    room = (len(SWEEP_MODES) * (Wm + 2 * K)) * per_step + 16      # keys a sequence may gain in its bin
    max_ctx = (max(b["context"] for b in plan) + room + 32 + 15) // 16 * 16
    kv_blocks = max(b["batch"] * ((b["context"] + room + 15) // 16 + 2) for b in plan) + 64
    eng = Engine(shape, wts, shape.quant, seed=args.seed, temperature=args.temperature, top_p=args.top_p,
                 gamma_init=4, gamma_min=1, gamma_max=args.gamma_max, policy=_lib.ER_POLICY_AUTO,
                 max_seqs=max(b["batch"] for b in plan) + 8, max_batch=max(b["batch"] for b in plan),
                 max_ctx=max_ctx, prefill_chunk=8192, kv_blocks=kv_blocks)
    engine_options(eng, args)
    if args.gamma:
        eng.set_gamma(args.gamma)
    pol = {"sd": _lib.ER_POLICY_AUTO, "force-sd": _lib.ER_POLICY_FORCE_SD, "ar": _lib.ER_POLICY_FORCE_AR}
    roof = Roofline(shape)
    rows, all_kprof, timed_recs = [], [], {m: [] for m, _ in SWEEP_MODES}
    t_prefill = 0.0
    for bi, b in enumerate(plan):
        B, C = b["batch"], b["context"]
        if args.group > 1:   # one prompt per group, its members share the prompt's blocks
            gp = synth.prompts((B + args.group - 1) // args.group, C, shape.vocab, seed=args.seed + 101 * (bi + 1))
            prompts = [gp[i // args.group] for i in range(B)]
            ids = eng.kv_alloc([C] * B, [room] * B, share_group=[i // args.group for i in range(B)])
        else:
            prompts = synth.prompts(B, C, shape.vocab, seed=args.seed + 101 * (bi + 1))
            ids = eng.kv_alloc([C] * B, [room] * B)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.prefill(ids, list(prompts))
        torch.cuda.synchronize()
        t_prefill += time.perf_counter() - t0
        act = [int(i) for i in ids]
        row = dict(bin=b["bin"], batch=B, context=C, plan_steps=b["plan_steps"], plan_tokens=b["plan_tokens"])
        for m, _ in SWEEP_MODES:
            eng.set_policy(pol[m])
            for _ in range(Wm):
                eng.step(act)
            recs = []
            cbar = sum(eng.seq_info(a)[1] for a in act) / B     # committed keys, tracked from the emitted counts
            with no_gc():
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(K):
                    ts = time.perf_counter()
                    tok, ne, info = eng.step(act)
                    te = time.perf_counter()
                    n_em = int(ne.sum())
                    recs.append((B, int(info.mode), int(info.gamma), n_em, te - ts, int(info.accepted), cbar))
                    cbar += n_em / B
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
            tokens = sum(r[3] for r in recs)
            timed_recs[m].extend(recs)
            row[m] = dict(tok_s=round(tokens / dt, 1), ms_per_step=round(dt * 1e3 / K, 3), tokens=tokens,
                          seconds=round(dt, 4), sd_steps=sum(1 for r in recs if r[1] == 1),
                          mean_gamma=round(float(np.mean([r[2] for r in recs if r[1] == 1])), 2)
                          if any(r[1] == 1 for r in recs) else None,
                          roofline_frac=round(sum(roof.step(r[1], r[2], r[0], r[6]) for r in recs) / dt, 4))
        row["sd_over_ar"] = round(row["sd"]["tok_s"] / row["ar"]["tok_s"], 4)
        row["force_sd_over_ar"] = round(row["force-sd"]["tok_s"] / row["ar"]["tok_s"], 4)
        # untimed: the same steps again with every launch bracketed by HIP events
        kp_bin = []
        if not args.no_kernel_profile:
            for m, _ in SWEEP_MODES:
                eng.set_policy(pol[m])
                eng.reset_kernel_profile()
                eng.set_kernel_profile(_lib.ER_KPROF_ALL)
                for _ in range(K):
                    eng.step(act)
                kp_bin.append(eng.kernel_profile())
                eng.set_kernel_profile(_lib.ER_KPROF_OFF)
            all_kprof.extend(kp_bin)
            row["kernels"] = role_tops(merge_kprof(kp_bin))
        eng.kv_free(ids)
        st = eng.stats()
        row["alpha_ema"] = round(st["alpha_ema"], 4)
        log(f"[sweep] bin {b['bin']:>7s} B={B:3d} C={C:5d}: SD-auto {row['sd']['tok_s']:9.1f} tok/s "
            f"({row['sd']['sd_steps']}/{K} SD), forced SD {row['force-sd']['tok_s']:9.1f}, AR {row['ar']['tok_s']:9.1f}"
            f" -> SD-auto/AR {row['sd_over_ar']:.3f}")
        rows.append(row)
    eng.set_policy(_lib.ER_POLICY_AUTO)
    st = eng.stats()
    cm = eng.cost_model()
    eng.close()

    def composed(m):   # rollout seconds: each bin's planned tokens at its measured rate
        t = sum(r["plan_tokens"] / r[m]["tok_s"] for r in rows)
        return sum(r["plan_tokens"] for r in rows) / t

    comp = {m: round(composed(m), 1) for m, _ in SWEEP_MODES}
    return dict(rows=rows, recs=timed_recs, kprof=merge_kprof(all_kprof), composed=comp, stats=st, cost=cm,
                prefill_s=t_prefill)


def crossover(args, shape, wts):
    """Fixed-batch SD vs AR at a fixed context: every sequence holds `context` keys; for each batch B
    (largest first, so the pool holds the largest batch before any growth) run AR and SD at each pinned
    gamma for a few steps and time them.  Reports tokens/s, tokens per step, the SD/AR ratio, the batch
    where SD stops paying (measured), and the same ratio predicted by the roofline with the measured mean
    tokens per step."""
    import torch

    import synth
    from speculative_decoding_rl_amd import Engine, _lib

    batches = sorted({int(b) for b in args.batches.split(",")}, reverse=True)
    gammas = [int(g) for g in args.gammas.split(",")]
    warm = 1

    def timed_steps(B):  # more steps where few sequences average the acceptance
        return 12 if B <= 4 else 6 if B <= 16 else 3

    def growth(i):  # keys sequence i gains over the sweep (it runs in every batch larger than i)
        return sum((warm + timed_steps(b)) * (max(gammas) + 1) * (len(gammas) + 1) for b in batches if b > i)

    C = args.context
    max_ctx = (C + growth(0) + 32 + 15) // 16 * 16
    Bmax = batches[0]
    kv_blocks = sum((C + growth(i) + 32) // 16 + 2 for i in range(Bmax))
    eng = Engine(shape, wts, shape.quant, seed=args.seed, temperature=args.temperature, top_p=args.top_p,
                 gamma_init=min(4, max(gammas)), gamma_min=1, gamma_max=max(gammas), policy=_lib.ER_POLICY_FORCE_AR,
                 max_seqs=Bmax,
                 max_batch=Bmax, max_ctx=max_ctx, prefill_chunk=8192, kv_blocks=kv_blocks)
    engine_options(eng, args)
    prompts = synth.prompts(Bmax, C, shape.vocab, seed=args.seed)
    ids = [int(i) for i in eng.kv_alloc([C] * Bmax, [max_ctx - C - 16] * Bmax)]
    t0 = time.perf_counter()
    eng.prefill(ids, list(prompts))
    torch.cuda.synchronize()
    log(f"[crossover] prefill {Bmax} x {C} tokens in {time.perf_counter() - t0:.1f} s")
    roof = Roofline(shape)
    rows = []
    for bi, B in enumerate(batches):
        act = ids[:B]
        res = {}
        for g in [0] + gammas:
            if g == 0:
                eng.set_policy(_lib.ER_POLICY_FORCE_AR)
            else:
                eng.set_policy(_lib.ER_POLICY_FORCE_SD)
                eng.set_gamma(g)
            for _ in range(warm):
                eng.step(act)
            torch.cuda.synchronize()
            timed = timed_steps(B)
            with no_gc():
                ts = time.perf_counter()
                tok = 0
                for _ in range(timed):
                    _, ne, _ = eng.step(act)
                    tok += int(ne.sum())
                torch.cuda.synchronize()
                dt = (time.perf_counter() - ts) / timed
            cbar = C + sum(eng.seq_info(a)[1] - C for a in act) / B
            en = tok / timed / B
            t_roof = roof.step(0 if g == 0 else 1, g, B, cbar)
            res[g] = dict(ms_per_step=dt * 1e3, tok_per_step=en, tok_s=tok / timed / dt, roof_tok_s=B * en / t_roof)
            log(f"[crossover] B={B:4d} gamma={g} {dt * 1e3:8.2f} ms/step {en:.2f} tokens/seq/step "
                f"{res[g]['tok_s']:9.1f} tok/s (roofline {res[g]['roof_tok_s']:9.1f})")
        for g in gammas:
            rows.append(dict(batch=B, gamma=g, sd_tok_s=round(res[g]["tok_s"], 1), ar_tok_s=round(res[0]["tok_s"], 1),
                             sd_over_ar=round(res[g]["tok_s"] / res[0]["tok_s"], 4),
                             tokens_per_seq_step=round(res[g]["tok_per_step"], 3),
                             sd_ms_per_step=round(res[g]["ms_per_step"], 3), ar_ms_per_step=round(res[0]["ms_per_step"], 3),
                             roofline_sd_over_ar=round(res[g]["roof_tok_s"] / res[0]["roof_tok_s"], 4),
                             roofline_frac_sd=round(res[g]["tok_s"] / res[g]["roof_tok_s"], 4),
                             roofline_frac_ar=round(res[0]["tok_s"] / res[0]["roof_tok_s"], 4)))
        nxt = batches[bi + 1] if bi + 1 < len(batches) else 0
        if nxt < B:
            eng.kv_free(ids[nxt:B])

    def bstar(key):
        out = {}
        for g in gammas:
            won = [r["batch"] for r in rows if r["gamma"] == g and r[key] > 1.0]
            out[str(g)] = max(won) if won else 0
        return out

    st = eng.stats()
    return {"metric": "fixed-batch SD vs AR tokens/s at fixed context (crossover sweep)", "unit": "tokens/s",
            "config": {"workload": f"{shape.name}-shaped decoder, {shape.quant.upper()} self-drafter, every sequence "
                                   f"at {C} keys, T={args.temperature}, top-p={args.top_p}",
                       "batches": batches, "gammas": gammas, "steps_timed": {b: timed_steps(b) for b in batches}},
            "data": "synthetic (random-init weights N(0,0.02), uniform prompts)",
            "alpha_ema_end": round(st["alpha_ema"], 4),
            "crossover_batch_measured": bstar("sd_over_ar"), "crossover_batch_roofline": bstar("roofline_sd_over_ar"),
            "rows": rows}


def history_line(args, shape, wts):
    """Drafts copied from an earlier rollout of the same prompts (the history drafter): the batch's
    prompts are rolled out once under AR (untimed) and recorded with reward 1; the same prompts are then
    rolled out again, timed, under ER_POLICY_HISTORY and under AR, each sequence to --history-new
    tokens.  Under sampling the second rollout differs from the first, and a copied draft is accepted
    with probability p(draft); at temperature 0 it repeats the first."""
    import torch

    import synth
    from speculative_decoding_rl_amd import Engine, History, _lib

    B, P, N, g = args.batch, args.prompt_len, args.history_new, args.history_gamma
    max_ctx = (P + N + args.gamma_max + 32 + 15) // 16 * 16
    eng = Engine(shape, wts, shape.quant, seed=args.seed, temperature=args.temperature, top_p=args.top_p,
                 gamma_init=4, gamma_min=1, gamma_max=args.gamma_max, policy=_lib.ER_POLICY_FORCE_AR,
                 max_seqs=B + 4, max_batch=B, max_ctx=max_ctx, prefill_chunk=8192,
                 kv_blocks=B * (max_ctx // 16 + 2) + 64)
    engine_options(eng, args)
    hist = History(args.history_prefix)
    eng.set_history(hist, gamma=g, max_batch=max(B, 1))
    prompts = [list(p) for p in synth.prompts(B, P, shape.vocab, seed=args.seed)]

    def rollout(policy, timed):
        eng.set_policy(policy)
        eng.reset_stats()
        ids = [int(i) for i in eng.kv_alloc([P] * B, [N] * B)]
        first = eng.prefill(ids, prompts)
        out = {i: [int(first[k])] for k, i in enumerate(ids)}
        act = list(ids)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps = 0
        while act:
            tok, ne, _ = eng.step(act)
            for k, i in enumerate(act):
                out[i] += [int(t) for t in tok[k, :ne[k]]]
            act = [i for i in act if not eng.seq_info(i)[2]]
            steps += 1
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st = eng.stats()
        eng.kv_free(ids)
        return [out[i] for i in ids], dt, steps, st

    first, _, _, _ = rollout(_lib.ER_POLICY_FORCE_AR, False)
    for p_, r_ in zip(prompts, first):
        hist.add(p_, r_, 1.0)
    toks_h, t_h, steps_h, st_h = rollout(_lib.ER_POLICY_HISTORY, True)
    toks_a, t_a, steps_a, _ = rollout(_lib.ER_POLICY_FORCE_AR, True)
    n_tok = sum(len(t) - 1 for t in toks_h)
    eng.close()
    hist.close()
    return {"metric": "history drafter: tokens/s of a second rollout of the same prompts vs AR", "unit": "tokens/s",
            "value": round(n_tok / t_h, 2), "ar_value": round(sum(len(t) - 1 for t in toks_a) / t_a, 2),
            "history_over_ar": round((n_tok / t_h) / (sum(len(t) - 1 for t in toks_a) / t_a), 4),
            "steps": {"history": steps_h, "ar": steps_a},
            "acceptance": {"history_drafted": st_h["history_drafted"], "history_accepted": st_h["history_accepted"],
                           "per_draft": round(st_h["history_accepted"] / max(1, st_h["history_drafted"]), 4),
                           "tokens_per_sequence_step": round(n_tok / max(1, steps_h) / B, 3)},
            "second_rollout_repeats_first": toks_h == first,
            "config": {"workload": f"{args.config}-shaped decoder, batch {B}, prompts {P} tokens, {N} tokens per "
                                   f"sequence, T={args.temperature}, top-p={args.top_p}, history gamma {g}, "
                                   f"prefix {args.history_prefix}"},
            "data": "synthetic (random-init weights N(0,0.02), uniform prompts)"}


def sweep_line(args, shape, wts, stops):
    """The JSON line of the bin sweep."""
    t0 = time.perf_counter()
    sw = sweep(args, shape, wts, stops)
    log(f"[sweep] done in {time.perf_counter() - t0:.1f} s (prefill {sw['prefill_s']:.1f} s untimed)")
    rows, recs = sw["rows"], sw["recs"]
    t_sd = sum(r["sd"]["seconds"] for r in rows)
    tok_sd = sum(r["sd"]["tokens"] for r in rows)
    t_ar = sum(r["ar"]["seconds"] for r in rows)
    tok_ar = sum(r["ar"]["tokens"] for r in rows)
    n_steps = len(rows) * args.steps
    rf, rf_detail = roofline_from(sw["kprof"])
    roof = Roofline(shape)
    st = sw["stats"]
    bins_desc = ", ".join(f"{r['bin']}: B={r['batch']} C={r['context']}" for r in rows)
    out = {
        "metric": METRIC,
        "value": round(tok_sd / t_sd, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_sd * 1e3 / n_steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (random-init weights N(0,0.02), uniform prompts, lognormal stop lengths)",
        "config": {"workload": (f"{args.config}-shaped decoder{'' if not args.layers else f' ({args.layers} layers)'}, "
                                f"{shape.quant.upper()} self-drafter, {args.batch} prompts x {args.prompt_len} tokens, "
                                f"stop lengths lognormal(median {int(args.median)}, sigma 0.75) cap {args.cap}, "
                                f"T={args.temperature}, top-p={args.top_p}, gamma "
                                f"{'adaptive 1..%d' % args.gamma_max if not args.gamma else args.gamma}; "
                                f"the {len(rows)} batch bins of its 256->1 rollout, each prefilled at the bin's mean "
                                f"batch B and mean context C ({bins_desc}), {args.warmup} untimed + {args.steps} "
                                f"timed steps per bin in SD-auto, forced SD and AR; value = SD-auto tokens / "
                                f"seconds over its {n_steps} timed steps, ms_per_step their mean"
                                + (f"; groups of {args.group} sequences share their bin's prefilled context"
                                   if args.group > 1 else "")),
                   "mode": "SD-auto (roofline toggle)", "global_batch": args.batch, "seq_len": args.prompt_len,
                   "parallelism": "none (1 GPU)", "graphs": args.graphs,
                   "library_gemm_rows": args.library_gemm},
        "roofline": rf,
        "ar_value": round(tok_ar / t_ar, 2),
        "sd_over_ar": round((tok_sd / t_sd) / (tok_ar / t_ar), 4),
        "force_sd_value": round(sum(r["force-sd"]["tokens"] for r in rows) /
                                sum(r["force-sd"]["seconds"] for r in rows), 2),
        "rollout_composed": {"note": "each bin's planned tokens at its measured rate: tokens / sum(bin tokens / "
                                     "bin tok/s) over the bins of the stop-length draw",
                             "tokens": sum(r["plan_tokens"] for r in rows),
                             "sd_auto_tok_s": sw["composed"]["sd"], "forced_sd_tok_s": sw["composed"]["force-sd"],
                             "ar_tok_s": sw["composed"]["ar"],
                             "sd_auto_over_ar": round(sw["composed"]["sd"] / sw["composed"]["ar"], 4),
                             "forced_sd_over_ar": round(sw["composed"]["force-sd"] / sw["composed"]["ar"], 4)},
        "by_bin": rows,
    }
    out["acceptance"] = {"alpha_ema_end": round(st["alpha_ema"], 4),
                         "accepted_per_draft": round(st["accepted"] / st["drafted"], 4) if st["drafted"] else None,
                         "mean_emitted_per_sd_seq_step": round(1.0 + st["accepted"] / st["predict_times"], 4)
                         if st["predict_times"] else None,
                         "sd_steps": sum(r["sd"]["sd_steps"] for r in rows),
                         "sd_steps_all_modes": st["sd_steps"], "ar_steps_all_modes": st["ar_steps"],
                         "effective_length": round(st["effective_length"], 4),
                         "effective_percent": round(st["effective_percent"], 4)}
    cm = sw["cost"]
    out["controller"] = {"hbm_gbs": round(cm["hbm_bytes_per_s"] / 1e9, 1), "tflops": round(cm["flops_per_s"] / 1e12, 1),
                         "t_fwd_ms": round(cm["t_fwd_s"] * 1e3, 3),
                         "t_row_draft_us": round(cm["t_row_draft_s"] * 1e6, 2),
                         "t_row_target_us": round(cm["t_row_target_s"] * 1e6, 2)}
    out["roofline_frac_timed"] = {m: round(sum(roof.step(x[1], x[2], x[0], x[6]) for x in recs[m]) /
                                           sum(x[4] for x in recs[m]), 4) for m, _ in SWEEP_MODES}
    out["prefill_s"] = round(sw["prefill_s"], 3)
    if rf_detail:
        rf_detail["from"] = ("untimed pass: the same bins and modes, every launch bracketed with HIP events on "
                             "the library's stream")
        out["roofline_kernel"] = rf_detail
        out["kernels_top"] = kernel_table(sw["kprof"])[:12]
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(args.config, args)
        except Exception as e:  # reported, not fatal
            out["cpu_baseline"] = {"error": repr(e)}
    return out


def main():
    args = parse()
    args.kprof_every = max(1, args.kprof_every)
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (sharding sequences "
                                   "across GPUs is not built)"}))
        sys.exit(2)
    import torch

    import synth
    from speculative_decoding_rl_amd import _lib

    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "copies": 10}))
        return
    over = {"n_layers": args.layers} if args.layers else {}
    if not args.config:
        args.config = "qwen2.5-14b" if args.crossover else "qwen2.5-7b"
    shape = synth.shape(args.config, **over)
    t0 = time.perf_counter()
    wts = synth.weights(shape, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    log(f"weights {sum(v.numel() for v in wts.values()) / 1e9:.2f} B params on device in {time.perf_counter() - t0:.1f} s")
    if args.crossover:
        print(json.dumps(crossover(args, shape, wts)), flush=True)
        return
    if args.history:
        print(json.dumps(history_line(args, shape, wts)), flush=True)
        return
    prompts = synth.prompts(args.batch, args.prompt_len, shape.vocab, seed=args.seed)
    stops = synth.stop_lengths(args.batch, args.median, args.cap, seed=args.seed)
    log(f"stop lengths: sum {int(stops.sum())}, max {int(stops.max())}, median {int(np.median(stops))}")
    if args.steps > 0 and not args.rollout:
        print(json.dumps(sweep_line(args, shape, wts, stops)), flush=True)
        return
    args.steps = 0

    t0 = time.perf_counter()
    eng = make_engine(args, shape, wts, _lib.ER_POLICY_AUTO)
    torch.cuda.synchronize()
    log(f"engine init (drafter quantization + calibration) {time.perf_counter() - t0:.1f} s")
    if args.gamma:
        eng.set_gamma(args.gamma)

    # warm-up: a few steps of each mode on a small side batch (untimed)
    if args.warmup > 0:
        nw = min(8, args.batch)
        wp = synth.prompts(nw, 64, shape.vocab, seed=args.seed + 1)
        for pol in (_lib.ER_POLICY_FORCE_SD, _lib.ER_POLICY_FORCE_AR):
            eng.set_policy(pol)
            wid = eng.kv_alloc([64] * nw, [args.warmup + 2] * nw)
            eng.prefill(wid, list(wp))
            for _ in range(args.warmup):
                act = [int(a) for a in wid if not eng.seq_info(int(a))[2]]
                if act:
                    eng.step(act)
            eng.kv_free(wid)
        torch.cuda.synchronize()

    res = {}
    modes = {"both": ["sd", "ar"], "sd": ["sd"], "ar": ["ar"], "force-sd": ["force-sd"], "timing": ["timing"],
             "both+timing": ["sd", "ar", "timing"]}[args.mode]
    for m in modes:
        eng.set_policy({"sd": _lib.ER_POLICY_AUTO, "ar": _lib.ER_POLICY_FORCE_AR,
                        "force-sd": _lib.ER_POLICY_FORCE_SD, "timing": _lib.ER_POLICY_TIMING}[m])
        res[m] = run_rollout(eng, args, prompts, stops, m)

    main_run = res.get("sd") or res.get("force-sd") or res.get("timing") or res["ar"]
    value = main_run["tokens"] / main_run["t"]
    rf, rf_detail = roofline_from(main_run["kprof"])
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": main_run["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(main_run["t"] * 1e3 / max(1, main_run["steps"]), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (random-init weights N(0,0.02), uniform prompts, lognormal stop lengths)",
        "config": {"workload": (f"{args.config}-shaped decoder{'' if not args.layers else f' ({args.layers} layers)'}"
                                f", {shape.quant.upper()} self-drafter, {args.batch} prompts x {args.prompt_len} "
                                f"tokens, stop lengths lognormal(median {int(args.median)}, sigma 0.75) cap "
                                f"{args.cap}, T={args.temperature}, top-p={args.top_p}, gamma "
                                f"{'adaptive 1..%d' % args.gamma_max if not args.gamma else args.gamma}, "
                                f"{'full rollout 256->1' if args.steps == 0 else f'first {args.steps} steps'}"),
                   "mode": "SD-auto (roofline toggle)" if "sd" in res else modes[0],
                   "global_batch": args.batch, "seq_len": args.prompt_len, "parallelism": "none (1 GPU)",
                   "graphs": args.graphs, "library_gemm_rows": args.library_gemm},
        "roofline": rf,
    }
    if "ar" in res and main_run is not res["ar"]:
        ar_v = res["ar"]["tokens"] / res["ar"]["t"]
        out["ar_value"] = round(ar_v, 2)
        out["sd_over_ar"] = round(value / ar_v, 4)
    if "timing" in res and main_run is not res["timing"]:
        tr = res["timing"]
        out["timing_guard"] = {"value": round(tr["tokens"] / tr["t"], 2), "sd_steps": tr["stats"]["sd_steps"],
                               "ar_steps": tr["stats"]["ar_steps"]}
    st = main_run["stats"]
    out["acceptance"] = {"alpha_ema_end": round(st["alpha_ema"], 4),
                         "accepted_per_draft": round(st["accepted"] / st["drafted"], 4) if st["drafted"] else None,
                         # each speculative sequence-step emits its accepted drafts plus one token
                         "mean_emitted_per_sd_seq_step": round(1.0 + st["accepted"] / st["predict_times"], 4)
                         if st["predict_times"] else None,
                         "sd_steps": st["sd_steps"], "ar_steps": st["ar_steps"],
                         "effective_length": round(st["effective_length"], 4),
                         "effective_percent": round(st["effective_percent"], 4)}
    cm = eng.cost_model()
    out["controller"] = {"hbm_gbs": round(cm["hbm_bytes_per_s"] / 1e9, 1), "tflops": round(cm["flops_per_s"] / 1e12, 1),
                         "t_fwd_ms": round(cm["t_fwd_s"] * 1e3, 3),
                         "t_row_draft_us": round(cm["t_row_draft_s"] * 1e6, 2),
                         "t_row_target_us": round(cm["t_row_target_s"] * 1e6, 2)}
    out["prefill_s"] = round(main_run["prefill_s"], 3)
    roof = Roofline(shape)
    out["by_batch"] = {m: bins(r["recs"], roof) for m, r in res.items()}
    out["roofline_frac_rollout"] = {m: round(sum(roof.step(x[1], x[2], x[0], x[6]) for x in r["recs"]) / r["t"], 4)
                                    for m, r in res.items()}
    if rf_detail:
        rf_detail.pop("share_of_profiled_time", None)   # only attention launches are bracketed here
        rf_detail["sampled_every_steps"] = args.kprof_every
        out["roofline_kernel"] = rf_detail
    if not args.no_kernel_profile:
        kp = kernel_pass(eng, args, prompts, 64, _lib.ER_POLICY_AUTO)
        out["kernels_top"] = {"pass": "untimed: prefill 64 prompts, 32 SD-auto steps, every launch timed",
                              "kernels": kernel_table(kp)}
        out["kernels_sd"] = {}
        for n in (64, 4):
            ks = kernel_pass(eng, args, prompts, n, _lib.ER_POLICY_FORCE_SD)
            out["kernels_sd"][f"b{n}"] = {"pass": f"untimed: prefill {n} prompts, 32 forced SD steps, every "
                                                  "launch timed", "kernels": kernel_table(ks)}
        eng.set_policy(_lib.ER_POLICY_AUTO)
        lin = [k for k in kp if any(n in k["name"] for n in LINEAR_KERNELS)]
        if lin and rf_detail:
            tl = max(lin, key=lambda k: k["ms"])
            g = tl["bytes"] / (tl["ms"] * 1e-3) / 1e9
            rf_detail["top_linear"] = {"kernel": tl["name"], "avg_us": round(tl["ms"] * 1e3 / tl["launches"], 2),
                                       "achieved_gbs": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                                       "from": "the untimed kernel pass"}
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(args.config, args)
        except Exception as e:  # reported, not fatal
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

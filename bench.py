"""Throughput of one Medusa verify step on one MI355X.

A step is one pass of the whole hot path over one batch, as one composite
medusa_step call: heads (residual block + vocabulary projection with fused
top-s) -> candidate tree -> verify forward (QKV + RoPE, split-KV tree
attention, output projection, LM head with row statistics) -> posterior
(typical acceptance) -> commit. The
workload is the Vicuna-7B-shaped step (d 4096, V 32000, 5 heads, 45-node
top-(3,2,2,1,1) tree, 2048-token prefix, typical acceptance eps 0.09,
delta 0.3, tau 0.7) on seeded synthetic inputs resident in HBM.

Prints one JSON line: steps/s, the roofline of the dominant kernel (the
W2 vocabulary projection with the fused top-s, timed with HIP events on its
own stream inside the timed region) and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload NAME] [--headline-only]

By default the line also carries other_workloads: the same whole-step
timing (K/4 steps, at least 20) of the 13B shapes with a 136-node tree and a
4k prefix, of eight 7B sequences with ragged prefixes and greedy acceptance,
and of the 7B shapes with exact p/q acceptance, each with its HBM and
combined (HBM + MFMA) roofline fraction. --workload times one of them alone
with the full line; the CPU baseline is taken on the 7B workload only.

With --decode it prints a different line instead: the decoding loop
(medusa_generate) on planted agreement — accepted tokens per step A for a
Cartesian and a calibrated sparse tree against the tail-sum prediction —
and the step-cost ratio r of the 7B step to a plain one-token step made of
the same kernels.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "vicuna7b_typical"
HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth


def algorithmic_bytes(w, T, L_total):
    """Bytes the step must move (bf16 weights and KV, fp32 activations)."""
    d, V, K, B, H, Dh = w.d, w.V, w.K, w.B, w.H, w.Dh
    wb = 2
    weights = wb * (K * d * d + K * V * d + V * d + 4 * d * d)
    kv = wb * 2 * H * Dh * L_total
    emb = wb * d * B * T
    act = 4 * d * B
    logits = 2 * 4 * K * V * B if w.mode == "exact" else 0   # head logits written, then read
    return weights + kv + emb + act + logits


def w2_kernel_bytes(w):
    """Algorithmic bytes of one vocabulary-projection launch: the K*V*d bf16
    weights plus the K fp32 input vectors per sequence, and in exact mode the
    fp32 head logits it writes for drafting."""
    extra = 4 * w.B * w.K * w.V if w.mode == "exact" else 0
    return 2 * w.K * w.V * w.d + 4 * w.B * w.K * w.d + extra


MFMA_BF16_PEAK_FLOPS = 2.5e15   # MI355X dense bf16 matrix peak


def combined_roofline_us(w, T, L_total):
    """Sum over the step's stages of max(bytes / HBM peak, flops / bf16 MFMA
    peak): the floor when the node GEMMs reach the ridge (many tree rows)."""
    d, V, K, B, H, Dh = w.d, w.V, w.K, w.B, w.H, w.Dh
    M = B * T
    logits = 2 * 4 * K * V * B if w.mode == "exact" else 0
    stages = [  # (bytes, flops)
        (2 * K * d * d, 2 * B * K * d * d),                  # W1
        (2 * K * V * d + logits, 2 * B * K * V * d),         # W2
        (2 * 3 * d * d + 2 * d * M, 2 * M * 3 * d * d),      # QKV (+ E rows)
        (2 * 2 * H * Dh * L_total, 4 * H * Dh * T * L_total),  # prefix attention
        (2 * d * d, 2 * M * d * d),                          # output projection
        (2 * V * d, 2 * M * V * d),                          # LM head
    ]
    return sum(max(b / (HBM_PEAK_GBS * 1e9), f / MFMA_BF16_PEAK_FLOPS) for b, f in stages) * 1e6


def _oracle_rest(w, inp, topk):
    """Everything after the heads for every sequence: candidate tree,
    verifier forward, typical acceptance, posterior and commit."""
    from oracle import posterior as OP, tree as OT, verifier as OV
    from oracle.numerics import widen
    topo = OT.topology(inp["ranks"], w.K)
    for b in range(w.B):
        L = int(inp["kv_len"][b])
        tok = OT.draft_tokens_topk(topo, int(inp["root"][b]), topk[b])
        pos = OT.position_ids(topo, L)
        vf = OV.verifier_forward(inp["E"], inp["W_qkv"], inp["W_o"], inp["W_lm"], tok, pos,
                                 topo.mask, inp["k_cache"][b], inp["v_cache"][b], L, w.H, w.Dh,
                                 w.rope_theta, True)
        p, ent, am = OV.row_distribution(vf["logits"], w.tau)
        acc = OP.accept_typical(topo, tok, p, ent, w.eps, w.delta)
        post = OP.posterior_deterministic(topo, tok, acc, am)
        OP.commit(topo, post["last_node"], vf["k"], vf["v"], vf["y"], widen(inp["k_cache"][b]),
                  widen(inp["v_cache"][b]), L)


def cpu_baseline(w, inp, budget_s: float = 10.0):
    """The oracle, as it stands, timed on the host cores.

    First a bounded sample: the head stage for head 0 alone (W1 and W2 of one
    head) and everything after the heads for the full step, which estimates
    the step as K * head + rest. When that estimate fits the budget (a fast
    host), whole oracle steps -- all K heads, then the rest on their own
    top-s pools -- are run back to back until the budget has elapsed, and
    their rate is reported; otherwise the estimate is.
    """
    from threadpoolctl import threadpool_info
    from oracle import heads as OH
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    cores = f"float64 NumPy, BLAS threads {threads}, affinity cores {len(os.sched_getaffinity(0))}"
    h = np.asarray(inp["h"], dtype=np.float64)
    t0 = time.perf_counter()
    _, hl = OH.heads_forward(h, inp["W1"][:1], inp["W2"][:1], inp.get("b1"))
    t_head = time.perf_counter() - t0
    # the rest of the step, with head 0's top-s pool standing in for every depth
    ids, _, _ = OH.heads_topk(hl, w.s_max)
    t1 = time.perf_counter()
    _oracle_rest(w, inp, np.repeat(ids, w.K, axis=1))
    t_rest = time.perf_counter() - t1
    est = w.K * t_head + t_rest
    if est <= 1.2 * budget_s:
        n = 0
        t2 = time.perf_counter()
        while n == 0 or time.perf_counter() - t2 < budget_s:
            _, hl = OH.heads_forward(h, inp["W1"], inp["W2"], inp.get("b1"))
            ids, _, _ = OH.heads_topk(hl, w.s_max)
            _oracle_rest(w, inp, ids)
            n += 1
        el = time.perf_counter() - t2
        return {"value": n / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{w.name}: {n} whole oracle steps back to back ({el:.1f} s; all "
                          f"{w.K} heads, tree, verifier, typical acceptance, posterior, commit) "
                          f"({cores})"}
    return {"value": 1.0 / est, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name}: head stage for 1 of {w.K} heads ({t_head:.1f} s) + tree, "
                      f"verifier, typical acceptance, posterior and commit of the step "
                      f"({t_rest:.1f} s); step estimated as {w.K} x head + rest = {est:.1f} s "
                      f"({cores})"}


# HBM traffic of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counters, recorded in a committed profile summary together with a digest
# of the kernel's sources; reported only while the sources still match.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "heads_w2_vicuna7b_hbm_counters.md")
W2_SOURCES = ["medusa_tree_verification_forward_amd/csrc/heads.hip",
              "medusa_tree_verification_forward_amd/csrc/select.h",
              "medusa_tree_verification_forward_amd/csrc/common.h",
              "medusa_tree_verification_forward_amd/csrc/kernels.h"]


def w2_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in W2_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Bytes per launch from the counter summary, or None if absent or stale."""
    import re
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    dig = re.search(r"source digest: `([0-9a-f]+)`", text)
    val = re.search(r"HBM bytes per launch: `([0-9.e+]+)`", text)
    if not dig or not val or dig.group(1) != w2_source_digest():
        return None
    return float(val.group(1))


# Synthetic calibration table for the decoding report: P(rank i) of head k's
# true continuation (top-1 decaying with depth, as the heads' accuracy does).
DECODE_A = np.array([[0.60, 0.15, 0.06], [0.45, 0.13, 0.06], [0.35, 0.12, 0.05],
                     [0.28, 0.10, 0.05], [0.22, 0.09, 0.04]])


def decode_report(steps):
    """The decoding loop on planted agreement and the step-cost ratio."""
    import torch
    import medusa_tree_verification_forward_amd._lib as L
    from medusa_tree_verification_forward_amd.step import VerifyStep, to_host
    from workloads import WORKLOADS, cartesian_ranks, make_inputs, planted_inputs

    a = DECODE_A
    K, S = a.shape
    sparse, sparse_w, _ = L.sparse_tree(a, 45)
    trees = {"cartesian (3,2,2,1,1), 45 nodes": cartesian_ranks((3, 2, 2, 1, 1)),
             "calibrated sparse, 45 nodes": sparse}
    out = {}
    for name, spec in trees.items():
        paths = [tuple(int(x) for x in row if x >= 0) for row in spec]
        predicted = 1.0 + sum(float(np.prod([a[j, r] for j, r in enumerate(p)])) for p in paths)
        B, V = 8, 4096
        full = planted_inputs(a, spec, V=V, H=32, Dh=128, n_steps=steps, B=B, L=64)
        inp = {k: v for k, v in full.items() if k not in ("pi", "true_rank")}
        t_first = np.argmax(inp["h"], axis=1)
        st = VerifyStep(inp, H=32, Dh=128, s_max=S, mode="typical", tau=0.7, eps=0.09,
                        delta=0.3, theta=10000.0)
        toks, acc = st.generate(steps)
        torch.cuda.synchronize()
        toks, acc = to_host(toks), to_host(acc)
        # depth the planted ranks allow for the token each step starts from
        pset, rank = set(paths), full["true_rank"]
        closed = np.zeros_like(acc)
        for b in range(B):
            t = int(t_first[b])
            for i in range(steps):
                dep = 0
                while dep < K and tuple(int(rank[j, t]) for j in range(dep + 1)) in pset:
                    dep += 1
                closed[i, b] = dep
                t = int(toks[i, b, acc[i, b]])
        out[name] = {"nodes": len(paths), "A_measured": float(np.mean(acc + 1)),
                     "A_tail_sum_prediction": predicted,
                     "A_closed_form_on_visited_tokens": float(np.mean(closed + 1)),
                     "steps": steps, "sequences": B,
                     "distinct_start_tokens": int(len({int(x) for x in toks[:, :, 0].ravel()}))}
    # step cost: the 7B composite step against a plain one-token step
    w = WORKLOADS[WORKLOAD]
    inp = make_inputs(w)
    st = VerifyStep(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                    delta=w.delta, theta=w.rope_theta)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(20):
        st.run_step(keep_kv_len=True)
    e0.record()
    for _ in range(100):
        st.run_step(keep_kv_len=True)
    e1.record()
    torch.cuda.synchronize()
    t_medusa = e0.elapsed_time(e1) / 100 * 1e3
    plain_inp = dict(inp)
    plain_inp["ranks"] = np.zeros((0, K), dtype=np.int32)
    del st
    pl = VerifyStep(plain_inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau,
                    eps=w.eps, delta=w.delta, theta=w.rope_theta)

    def plain():   # root-only tree: draft nothing, verify the root, commit one token
        pl.tree()
        pl.verify()
        pl.posterior()
        pl.commit()
    for _ in range(10):
        plain()
    pl.reset_kv_len()   # the cache has room for ~60 one-token commits past the prefix
    e0.record()
    for _ in range(40):
        plain()
    e1.record()
    torch.cuda.synchronize()
    t_plain = e0.elapsed_time(e1) / 40 * 1e3
    r = t_medusa / t_plain
    print(json.dumps({
        "metric": "decoding loop: accepted tokens per step A (planted agreement) and A/r",
        "trees": out, "t_medusa_step_us": t_medusa, "t_plain_step_us": t_plain, "r": r,
        "A_over_r": {k: v["A_measured"] / r for k, v in out.items()},
        "data": "synthetic: planted agreement (permutation language, one-hot embeddings, "
                "V=d=4096, head ranks drawn from a synthetic calibration table); step times "
                "at the 7B shapes with seeded random weights",
        "note": "the verifier is one transformer layer plus the LM head, so r here weighs "
                "the heads against one layer, not against a whole base model"}))


def time_step(w, steps, warmup, reset_kv_len=False, graph=False, copy_bytes=0,
              min_warm_s=None):
    """Time `steps` whole steps of workload w (inputs resident in HBM), then
    the dominant kernel in a second pass of the same steps. Returns a dict
    with the step object and the timings."""
    import torch
    from medusa_tree_verification_forward_amd.step import VerifyStep
    from workloads import make_inputs

    inp = make_inputs(w)
    st = VerifyStep(inp, H=w.H, Dh=w.Dh, s_max=w.s_max, mode=w.mode, tau=w.tau, eps=w.eps,
                    delta=w.delta, theta=w.rope_theta)
    stream = torch.cuda.current_stream()

    def step():
        # stream=None: the calls go to torch's current stream (the capture
        # stream while a graph is being recorded). By default the commit
        # writes the advanced prefix lengths to a buffer of their own, so
        # every step runs over the same prefix; reset_kv_len instead
        # advances kv_len in place and restores it before each step.
        if reset_kv_len:
            st.reset_kv_len()
            st.run_step()
        else:
            st.run_step(keep_kv_len=True)

    # W untimed warm-up steps, continued until the GPU has been busy for at
    # least MIN_WARM_S: a 5-step warm-up left the first timed steps ~2-4%
    # slower than steady state (clocks and caches still settling), which a
    # serving loop never sees. The timed region below is unaffected.
    min_warm_s = MIN_WARM_S if min_warm_s is None else min_warm_s
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < min_warm_s:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()   # the wall clock follows the GPU
    torch.cuda.synchronize()
    g = None
    if graph:
        # one step (prefix-length reset + medusa_step) recorded once and replayed
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
    run_one = g.replay if g is not None else step
    if copy_bytes > 0:
        src = torch.empty(copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # whole steps, bracketed by synchronisation
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(steps):
        run_one()
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_stop) / steps

    # dominant kernel: the same steps again, with HIP events recorded on the
    # kernel's stream right around the vocabulary projection of every step
    # (kept out of the whole-step loop: each event record costs a few us)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:       # create the underlying events before handing them over
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        if reset_kv_len:
            st.reset_kv_len()
        st.run_step(keep_kv_len=not reset_kv_len, w2_events=evs[i])
    torch.cuda.synchronize()
    w2_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return dict(inp=inp, st=st, T=st.T, L_total=int(np.sum(inp["kv_len"])), ms_step=ms_step,
                w2_ms=w2_ms, graph=g is not None)


OTHER_WORKLOADS = ["vicuna13b_typical", "vicuna7b_batch8_ragged", "vicuna7b_exact"]
MIN_WARM_S = 0.3   # untimed steps before the timed ones, at least this long (and W of them)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reset-kv-len", action="store_true",
                    help="advance kv_len in place and restore it with a fill kernel before "
                         "every step (default: the advanced lengths go to a separate buffer)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one recorded step graph instead of eager launches "
                         "(measured slower on this stack: per-node overhead)")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the W2 kernel source digest (for the counter summary) and exit")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before the timed loop, run a plain device-to-device copy of this "
                         "many bytes 3 times (a known-size kernel for scaling HBM counters)")
    ap.add_argument("--workload", default=None,
                    choices=["vicuna7b_typical"] + OTHER_WORKLOADS,
                    help="time this workload alone (default: the 7B typical-acceptance step, "
                         "followed by the other workloads under other_workloads)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the 7B step alone (no other_workloads)")
    ap.add_argument("--min-warm", type=float, default=MIN_WARM_S,
                    help="continue the untimed warm-up until this many seconds of GPU work "
                         "(0: exactly W steps, for profiling runs that count launches)")
    ap.add_argument("--decode", action="store_true",
                    help="print the decoding-loop report (A, A/r) instead of the step line")
    args = ap.parse_args()
    if args.decode:
        decode_report(max(args.steps, 8))
        return
    if args.print_digest:
        print(w2_source_digest())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the verify step runs on a single MI355X; "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS

    name = args.workload or WORKLOAD
    w = WORKLOADS[name]
    r = time_step(w, args.steps, args.warmup, args.reset_kv_len, args.graph, args.copy_bytes,
                  args.min_warm)
    ms_step, T, L_total = r["ms_step"], r["T"], r["L_total"]
    alg = algorithmic_bytes(w, T, L_total)
    w2b = w2_kernel_bytes(w)
    achieved = w2b / (r["w2_ms"] * 1e-3) / 1e9
    res = r["st"].results()
    comb_us = combined_roofline_us(w, T, L_total)
    accept = {"typical": f"typical eps={w.eps} delta={w.delta} tau={w.tau}",
              "greedy": "greedy", "exact": f"exact p/q rejection, tau={w.tau}"}[w.mode]
    metric = ("Medusa verify-steps/sec at 7B shapes (K=5, 45-node tree, 2k KV); % HBM roofline"
              if w.name == WORKLOAD else f"Medusa verify-steps/sec, {w.name}; % HBM roofline")
    line = {
        "metric": metric,
        "value": 1000.0 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded Gaussian weights and KV, {w.name} shapes)",
        "timing": (("replays of one recorded graph" if r["graph"] else "eager launches")
                   + (" (prefix-length reset + medusa_step)" if args.reset_kv_len else
                      " (medusa_step; advanced prefix lengths written to a separate buffer, "
                      "so every step runs over the same prefix)")
                   + f"; untimed warm-up: the W steps, continued to at least {args.min_warm} s "
                     "of GPU work"),
        "config": {"workload": w.name, "batch": w.B, "d": w.d, "V": w.V, "heads": w.K,
                   "tree": f"top-{w.s}".replace(" ", ""), "tree_nodes": T - 1,
                   "prefix_kv": L_total, "attn": f"{w.H}x{w.Dh}", "accept": accept},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": alg,
                          "achieved_GBs": alg / (ms_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                          "frac": alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "combined_floor_us": comb_us,
                          "combined_frac": comb_us / (ms_step * 1e3)},
        "roofline": {"kernel": "heads_w2 (vocabulary projection + fused top-s)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic() if w.name == WORKLOAD else None,
                     "avg_us": r["w2_ms"] * 1e3, "bytes_per_launch": w2b,
                     "timing": "HIP events recorded on the launch stream around every W2 "
                               "launch, over a second pass of the K timed steps"},
        "accept_len": [int(x) for x in res["accept_len"]],
    }
    cpu = None
    if not args.no_cpu_baseline and w.name == WORKLOAD:
        cpu = cpu_baseline(w, r["inp"])
    del r, res
    torch.cuda.empty_cache()
    if args.workload is None and not args.headline_only:
        # the other workloads, same step and timing (fewer steps), no CPU baseline
        others = []
        for oname in OTHER_WORKLOADS:
            ow = WORKLOADS[oname]
            # at least 50 steps (~25 ms of GPU work): 20-step regions of these
            # workloads read 2-5 us a step above longer ones
            n = max(50, args.steps // 4)
            o = time_step(ow, n, max(5, args.warmup // 4), min_warm_s=args.min_warm)
            oalg = algorithmic_bytes(ow, o["T"], o["L_total"])
            ocomb = combined_roofline_us(ow, o["T"], o["L_total"])
            others.append({
                "workload": oname, "value": 1000.0 / o["ms_step"], "unit": "steps/s",
                "ms_per_step": o["ms_step"], "steps": n, "batch": ow.B, "tree_nodes": o["T"] - 1,
                "prefix_kv": o["L_total"], "accept": ow.mode,
                "algorithmic_bytes": oalg,
                "hbm_frac": oalg / (o["ms_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "combined_floor_us": ocomb, "combined_frac": ocomb / (o["ms_step"] * 1e3),
                "w2_avg_us": o["w2_ms"] * 1e3})
            del o
            torch.cuda.empty_cache()
        line["other_workloads"] = others
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

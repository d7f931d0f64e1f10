#!/usr/bin/env python3
"""Benchmark of the single-forward speculative verification step on one GPU.

One step = the whole hot path on one batch of synthetic input already
resident in HBM: masked GQA attention of the 2B response rows with the
copy-aligned RoPE fused into its loads (spec_verify_attn), then the
verification epilogue (spec_verify_accept: per-slot softmax normaliser,
acceptance in draft order, residual resample).  Metric: verified draft slots
per second = batch * gamma / step time.

Default workload: batch 32, cached prefix 2048, block B = gamma = 32, 32
query / 8 KV heads, head_dim 128, vocab 151936, bf16 attention inputs,
float32 logits.  Two copies of the inputs live in HBM and steps alternate
between them, so a step never finds the previous step's data in the 256 MB
last-level cache.

Prints ONE JSON line (rank 0, N = 1).  Every call is launched from Python
(--launch graph instead captures each input set's step once in a HIP graph
and replays it: the same time, since the step is GPU-bound).  After W
untimed steps, K steps are timed with events only at their two ends
(value, ms_per_step); the same K steps then run again, launched call by call
with HIP events on the launch stream around every call, which gives the
per-call durations.  `roofline` is the step's: every call at
its bound (HBM bytes at 8 TB/s, or bf16 MFMA flops at 2.5 PFLOP/s when they
take longer) against the timed step; `roofline.dominant_kernel` gives the
dominant call's own rate against its bound.  Same-run peak microbenchmarks
run before the warmup steps (their load lets the clocks settle).  Also
reports the CPU oracle timed on this host over the same workload, and how
the GPU's acceptance outputs agree with the oracle's (ties counted).

--verify coupled | greedy replaces the epilogue by shared-noise verification
(spec_verify_accept_coupled at --temperature, default 1) or its greedy form
(T = 0); the default, rejection, is the headline step (at --temperature T
other than 1 through spec_verify_accept_temperature).  --route margin |
entropy adds S2D2's verify-routing estimate (spec_verify_route, parameter
--route-param) in front of each step.  --copies C runs SPOT's multi-copy
verification step instead: attention over C copies of the block (the root
state and D = C - 1 draft states, spec_verify_attn_copies) followed by
shared-noise (or, with --verify greedy, greedy) verification of the D draft
steps; gamma = D.  --copies C --tree verifies a tree of the C block states
instead of a chain (spec_verify_tree_states: the target's own next commit at
every state from the logits of every slot of every copy, C * B rows per
sequence; --threshold t < 1 commits every slot whose confidence exceeds t,
the dynamic-threshold decoder).  --paged PS keeps the prompt caches in pages of PS rows
(spec_verify_attn_paged; --ragged gives each sequence its own prompt length)
and ends each step with the commit step and the cache append of finished
blocks (spec_verify_commit, spec_verify_kv_append); the prompt lengths and the
block are restored at the start of every step so that each step does the same
work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft slots/sec (attn+accept), B=32 prefix 2048; % of roofline"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def attn_bytes(c, copies: int = 0, prompt_rows=None) -> float:
    """Algorithmic HBM bytes of one attention call: prompt K/V cache, Q,
    response K/V and the output, each read or written once (2B response rows,
    or copies * B for the multi-copy layout).  prompt_rows: the prompt rows of
    the whole batch (default batch * prefix)."""
    e = 2 if c.dtype == "bf16" else 4
    R = copies * c.block if copies else 2 * c.block
    pr = c.batch * c.prefix_len if prompt_rows is None else prompt_rows
    return e * (2 * c.n_kvh * pr * c.head_dim
                + c.batch * R * c.n_qh * c.head_dim * 2
                + 2 * c.batch * R * c.n_kvh * c.head_dim)


def attn_flops(c, copies: int = 0, prompt_rows=None) -> float:
    """Algorithmic FLOPs: every response row attends to exactly P + B keys
    (QK^T and PV, 2 flops per multiply-add): the paired layout's D rows see
    P + (keys of earlier steps and their own), its mask rows as many, and
    every copy row sees the prompt and its own copy's B keys."""
    R = copies * c.block if copies else 2 * c.block
    pr = c.batch * c.prefix_len if prompt_rows is None else prompt_rows
    return 4.0 * R * c.n_qh * c.head_dim * (pr + c.batch * c.block)


def commit_bytes(c, n_appended: int) -> float:
    """Algorithmic HBM bytes of the commit step and the append: out_tokens and
    the block read, the block written, four per-sequence outputs, plus the K
    and V rows of each appended block read and written once."""
    e = 2 if c.dtype == "bf16" else 4
    return c.batch * (c.block * 4 * 3 + 4 * 6) + n_appended * 4 * c.block * c.n_kvh * c.head_dim * e


def accept_bytes(c, n_rejecting: int) -> float:
    """Algorithmic HBM bytes of one epilogue call: the float32 target logits
    of every verified slot once, plus for each sequence that rejects the
    target and draft rows of the rejected slot, plus the per-step gathers
    (logit and draft probability of each draft token), tau, tokens,
    uniforms and outputs."""
    V = c.vocab
    small = c.batch * (c.block * 4 * 3 + (c.gamma + 1) * 4 + c.gamma * 4 * 3 + 4)
    return 4.0 * c.batch * c.gamma * V + n_rejecting * 2 * 4.0 * V + small


def coupled_bytes(c, greedy: bool) -> float:
    """Algorithmic HBM bytes of one shared-noise verification call: the
    float32 target logits of every verified slot once, the float32 noise row
    of every verified slot once (not read when greedy), plus tau, draft
    tokens and the outputs."""
    rows = 4.0 * c.batch * c.gamma * c.vocab
    small = c.batch * (c.block * 4 * 4 + 4)
    return rows * (1 if greedy else 2) + small


def states_bytes(c, state, greedy: bool) -> float:
    """Algorithmic HBM bytes of one verification of trees of block states:
    the float32 logits row of every masked slot of every copy once, the
    noise row of every slot masked in at least one copy once (shared by the
    copies; not read when greedy), plus the states, parents and outputs."""
    masked = state < 0                                   # [batch][N][B]
    rows = 4.0 * c.vocab * int(masked.sum())
    noise = 0.0 if greedy else 4.0 * c.vocab * int(masked.any(axis=1).sum())
    return rows + noise + c.batch * (c.n_copies * (c.block + 2) * 4 + c.block * 4 + 4)


def route_bytes(c) -> float:
    """Algorithmic HBM bytes of one routing call: the float32 draft
    distribution of every verified slot once, plus tau and the outputs."""
    return 4.0 * c.batch * c.gamma * c.vocab + c.batch * (c.block * 4 + c.gamma * 4 + 4)


def measured_traffic(call: str):
    """HBM bytes per launch of `call` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain-copy calibration),
    or None when that summary is missing or the kernel source has changed
    since the counters were taken (its sha256 no longer matches)."""
    path = os.path.join(ROOT, "profiles", "headline_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == call:
            src = os.path.join(ROOT, "diffusion_speculative_verification_amd", "csrc", f[3])
            if not os.path.exists(src):
                return None
            digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
            return int(f[2]) if digest == f[4] else None
    return None


def oracle_agreement(o, inp, gamma, temperature, L_o, tok_o, al_o, rs_o, gpu) -> dict:
    """Agreement of the GPU's rejection-sampling outputs `gpu` = (accept_len,
    out_tokens) with the oracle's on the same inputs: sequences equal, and
    sequences that differ only where the decision is a tie (|u - alpha| <
    1e-6 for the first differing acceptance test; u * Z within 1e-6 * Z of a
    running-sum boundary for the resampled token).  Anything else is counted
    as a mismatch."""
    import numpy as np
    L_g, tok_g = gpu
    u = inp["uniforms"]
    lt = inp["target_logits"]
    if temperature != 1.0:
        lt = lt * (np.float32(1.0) / np.float32(temperature))
    equal = ties = mismatch = 0
    for b in range(len(L_o)):
        if int(L_g[b]) == int(L_o[b]) and np.array_equal(tok_g[b], tok_o[b]):
            equal += 1
            continue
        if int(L_g[b]) != int(L_o[b]):
            r = min(int(L_g[b]), int(L_o[b]))
            ok = abs(float(u[b, r]) - float(al_o[b, r])) < 1e-6
        else:
            diff = np.nonzero(tok_g[b] != tok_o[b])[0].tolist()
            slot = int(rs_o[b])
            ok = diff == [slot]
            if ok:
                v = int(tok_g[b, slot])
                _, cdf, Z, _ = o.residual(lt[b, slot], inp["draft_probs"][b, slot], float(u[b, gamma]))
                thr = float(u[b, gamma]) * Z
                lo_b = cdf[v - 1] if v > 0 else 0.0
                ok = 0 <= v < len(cdf) and lo_b - 1e-6 * Z <= thr <= cdf[v] + 1e-6 * Z
        ties += int(ok)
        mismatch += int(not ok)
    return {"sequences": len(L_o), "equal": equal, "ties": ties, "mismatches": mismatch}


def cpu_baseline(case, inp, verify="rejection", temperature=1.0, route="none", rparam=0.0, copies=0,
                 paged=False, tree=False, attn_budget_s=20.0, gpu_accept=None, threshold=1.0,
                 gpu_attn=None) -> dict:
    """The CPU oracle on this host over the same workload (one step).  The
    attention is timed over the first sequences of the batch until
    `attn_budget_s` has passed and scaled to the whole batch.  With
    `gpu_accept` (the GPU's accept_len and out_tokens of the same inputs) the
    oracle's acceptance outputs are also compared with the GPU's
    (oracle_agreement), and with `gpu_attn` (the GPU's attention output of
    the same inputs, one entry per sequence) the oracle's attention rows of
    the timed sequences are compared with it, both outside the timed part."""
    import oracle
    o = oracle.Oracle()
    threads = o.max_threads()
    cpu_model = "unknown"
    if os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    t = time.perf_counter()
    if route != "none":
        o.route(inp["draft_probs"], inp["tau"], case.gamma, route, rparam)
    t_route = time.perf_counter() - t
    t = time.perf_counter()
    n_seq = 0
    attn_o = []
    for b in range(case.batch):
        if paged:
            sl = slice(b, b + 1)
            ref = o.attention_paged(inp["q"][sl], inp["k_new"][sl], inp["v_new"][sl], inp["k_pages"], inp["v_pages"],
                              inp["block_table"][sl], inp["prefix_lens"][sl], inp["tau"][sl], case.page_size,
                              case.theta)[0]
        elif copies:
            ref = o.attention_copies(inp["q_c"][b], inp["k_new_c"][b], inp["v_new_c"][b], inp["k_cache"][b],
                               inp["v_cache"][b], copies, case.theta)
        else:
            ref = o.attention(inp["q"][b], inp["k_new"][b], inp["v_new"][b], inp["k_cache"][b], inp["v_cache"][b],
                              inp["tau"][b], case.theta)
        if gpu_attn is not None:
            attn_o.append(ref)
        n_seq += 1
        if time.perf_counter() - t > attn_budget_s:
            break
    t_attn = (time.perf_counter() - t) * case.batch / n_seq
    t = time.perf_counter()
    if tree:
        o.tree_states(inp["st_logits"], inp["st_gumbel"] if temperature > 0 else None, inp["st_parent"],
                      inp["st_state"], temperature, threshold)
        out_tokens = None
    elif verify == "rejection":
        acc_o = o.accept(inp["target_logits"], inp["draft_probs"], inp["draft_tokens"], inp["tau"],
                         inp["uniforms"], case.gamma, temperature)
        out_tokens = acc_o[1]
    else:
        out_tokens = o.accept_coupled(inp["target_logits"], inp["gumbel"] if temperature > 0 else None,
                                      inp["coupled_tokens"], inp["tau"], case.gamma, temperature)[1]
    t_acc = time.perf_counter() - t
    t_commit = 0.0
    if paged:
        t = time.perf_counter()
        n_app = o.commit(out_tokens, inp["block_tokens"], case.gamma)[3]
        o.kv_append(inp["k_new"], inp["v_new"], n_app, inp["k_pages"], inp["v_pages"], inp["block_table"],
                    inp["prefix_lens"], case.page_size, case.theta)
        t_commit = time.perf_counter() - t
    total = t_route + t_attn + t_acc + t_commit
    agreement = None
    if gpu_accept is not None and verify == "rejection" and not tree:
        agreement = oracle_agreement(o, inp, case.gamma, temperature, *acc_o, gpu_accept)
    attn_agreement = None
    if gpu_attn is not None:
        import numpy as np
        mx = err2 = ref2 = 0.0
        for b, ref in enumerate(attn_o):
            d = gpu_attn[b].astype(np.float64) - ref
            mx = max(mx, float(np.abs(d).max()))
            err2 += float((d * d).sum())
            ref2 += float((ref * ref).sum())
        attn_agreement = {"sequences": n_seq, "max_abs_err": mx,
                          "rel_rms_err": (err2 / ref2) ** 0.5 if ref2 > 0 else 0.0}
    attn_what = (f"attention {t_attn:.2f} s" if n_seq == case.batch else
                 f"attention {t_attn:.2f} s (timed on {n_seq} of {case.batch} sequences, scaled)")
    return {"value": case.batch * case.gamma / total, "unit": "slots/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"one step of the same workload ({case.batch} sequences): "
                      + (f"routing {t_route:.2f} s + " if route != "none" else "") +
                      f"{attn_what} + accept {t_acc:.2f} s"
                      + (f" + commit and append {t_commit:.2f} s" if paged else "") +
                      f" on {threads} OpenMP threads "
                      f"(host reports {os.cpu_count()} CPUs); input generation excluded",
            "agreement": agreement, "attn_agreement": attn_agreement}


def measured_peaks(torch, keep: list) -> dict:
    """Microbenchmarks on the same device in the same run, beside the
    datasheet peaks: a 1 GiB device copy (bytes read + written), a 1 GiB
    read-only pass (row sums of 4096 floats: the best read rate among
    torch's reductions here), and a bf16 16384 x 16384 x 8192 GEMM through
    torch (hipBLASLt).  Their buffers go into `keep`: the caller frees them
    after its timed steps (freeing device memory just before the warmup
    slowed the following 20 steps by ~3%)."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps * 1e-3

    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    t_copy = timed(lambda: b.copy_(a), 10)
    t_read = timed(lambda: a.view(-1, 4096).sum(1), 10)
    keep.append(b)
    del b
    m, n, k = 16384, 16384, 8192
    x = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.mm(x, y), 10)
    keep.extend([a, x, y])
    return {"hbm_copy_gbs": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "hbm_read_gbs": round((1 << 30) / t_read / 1e9, 1),
            "bf16_gemm_tflops": round(2 * m * n * k / t_mm / 1e12, 1),
            "what": "1 GiB device copy (read + write bytes), 1 GiB of float32 row sums, bf16 16384x16384x8192 "
                    "torch.mm"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the clocks need ~20 ms of load to settle)")
    ap.add_argument("--config", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--verify", choices=("rejection", "coupled", "greedy"), default=None,
                    help="epilogue: rejection sampling (headline), shared-noise or greedy verification "
                         "(default: rejection; coupled with --copies)")
    ap.add_argument("--paged", type=int, default=0, metavar="PS",
                    help="prompt caches in pages of PS rows, plus the commit step and the cache append")
    ap.add_argument("--ragged", action="store_true", help="with --paged: per-sequence prompt lengths")
    ap.add_argument("--tree", action="store_true",
                    help="with --copies: verify a tree of the C block states instead of a chain")
    ap.add_argument("--threshold", type=float, default=1.0,
                    help="with --tree: commit every slot whose confidence exceeds it (>= 1: one commit per step)")
    ap.add_argument("--copies", type=int, default=0,
                    help="SPOT multi-copy verification over C copies of the block (root + C-1 draft states)")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="sampling temperature (rejection: spec_verify_accept_temperature when not 1)")
    ap.add_argument("--route", choices=("none", "margin", "entropy"), default="none",
                    help="add the S2D2 verify-routing estimate in front of each step")
    ap.add_argument("--route-param", type=float, default=None,
                    help="margin threshold (default 0.05) or entropy beta (default 1.0)")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="launch every call from Python (default), or replay each input set's step captured in a "
                         "HIP graph (the same time at every workload measured: the step is GPU-bound)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the verification step shards across GPUs without communication, but only one GPU is used here)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibrate:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "reps": 5}))
        return

    from diffusion_speculative_verification_amd import synth
    from diffusion_speculative_verification_amd.device import StepBuffers

    case = synth.config_by_name(args.config)
    copies = args.copies
    verify = args.verify or ("coupled" if copies else "rejection")
    if copies:
        if verify == "rejection" or args.route != "none":
            print("--copies verifies by state equality (--verify coupled or greedy), without routing", file=sys.stderr)
            sys.exit(2)
        if not 2 <= copies <= case.block + 1 or copies * case.block > 1024:
            print(f"--copies must lie in [2, {min(case.block + 1, 1024 // case.block)}] for block {case.block}",
                  file=sys.stderr)
            sys.exit(2)
        case = case.with_(n_copies=copies, gamma=copies - 1)
    tree = bool(args.tree)
    if tree and not copies:
        print("--tree verifies the draft states of --copies C", file=sys.stderr)
        sys.exit(2)
    paged = args.paged > 0
    if paged:
        if copies or args.route != "none" or args.paged % 64:
            print("--paged takes a page size that is a multiple of 64, without --copies or --route", file=sys.stderr)
            sys.exit(2)
        case = case.with_(page_size=args.paged, ragged=args.ragged)
    T = 0.0 if verify == "greedy" else args.temperature
    parts = ("attn", "accept") if verify == "rejection" else ("attn", "coupled")
    if copies:
        parts = ("copies", "states") if tree else ("copies", "coupled")
    if paged:
        parts = parts + ("paged",)
    route = args.route
    rparam = args.route_param if args.route_param is not None else (0.05 if route == "margin" else 1.0)
    if verify != "rejection":
        case = case.with_(temperature=T)
    if tree:
        case = case.with_(threshold=args.threshold)
    gen_parts = parts + (("accept",) if route != "none" and "accept" not in parts else ())
    inp = synth.make_inputs(case, parts=gen_parts)
    if route != "none":
        parts = parts + ("route",)
    # enough input sets in rotation that a step never finds the previous
    # steps' data in the 256 MB last-level cache (at least 1 GiB in rotation)
    set_bytes = sum(v.nbytes for v in inp.values() if hasattr(v, "nbytes"))
    n_sets = int(min(8, max(2, -(-(1 << 30) // max(1, set_bytes)))))
    sets = [StepBuffers(case, inp, parts=parts) for _ in range(n_sets)]
    stream = torch.cuda.current_stream()

    def attend(s):
        if copies:
            s.attn_copies()
        elif paged:
            s.attn_paged()
        else:
            s.attn()

    def commit(s):
        s.commit(s.out_tokens if verify == "rejection" else s.cpl_out_tokens)
        s.kv_append(s.k_new, s.v_new, 2 * case.block)   # a finished block's D rows, positions P_b ..
        # the next step on this input set starts from the same prompt lengths
        # and a fresh block (two small device copies, timed with the commit)
        s.prefix_lens.copy_(s.prefix_lens0)
        s.block_tokens.copy_(s.block_tokens0)

    def epilogue(s):
        if tree:
            s.tree_states(details=False)
        elif verify == "rejection":
            s.accept(temperature=None if T == 1.0 else T)
        else:
            s.accept_coupled(temperature=T)

    def step(s, e=None):
        """One step; with e (five events) each call is bracketed for its time."""
        if e:
            e[3].record(stream)
        if route != "none":
            s.route(route, rparam)
        if e:
            e[0].record(stream)
        attend(s)
        if e:
            e[1].record(stream)
        epilogue(s)
        if e:
            e[2].record(stream)
        if paged:
            commit(s)
        if e:
            e[4].record(stream)

    # one graph per input set: the step's calls captured once (every call
    # allocates nothing, sets no memory with memset and never synchronises),
    # after an eager step on a side stream as capture requires
    graphs = None
    if args.launch == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for s_ in sets:
                step(s_)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for s_ in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(s_)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % n_sets].replay()
        else:
            step(sets[i % n_sets])

    # the same-run peak microbenchmarks go first: after the idle time of the
    # input generation they put the GPU under load (~0.1 s) before the warmup
    # steps, so that a short warmup starts closer to steady clocks
    peak_buffers = []
    peaks = measured_peaks(torch, peak_buffers)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    # timed pass: K steps with events only at its two ends (an event between
    # two calls costs a few microseconds of the step)
    K = args.steps
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(K):
        run_step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_begin.elapsed_time(t_end)

    # per-call pass: the same K steps again with every call bracketed by
    # events on the launch stream; the per-call durations for the roofline
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    for i in range(K):
        step(sets[i % n_sets], ev[i])
    torch.cuda.synchronize()
    peak_buffers.clear()
    torch.cuda.empty_cache()

    commit_ms = sum(ev[i][2].elapsed_time(ev[i][4]) for i in range(K)) / K if paged else 0.0
    route_ms = sum(ev[i][3].elapsed_time(ev[i][0]) for i in range(K)) / K if route != "none" else 0.0
    ms_step = total_ms / K
    attn_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(K)) / K
    acc_ms = sum(ev[i][1].elapsed_time(ev[i][2]) for i in range(K)) / K
    L = (sets[0].st_path_len if tree else sets[0].accept_len if verify == "rejection" else sets[0].cpl_accept_len).cpu()
    n_rej = int((L < case.gamma).sum())
    slots = case.batch * case.gamma
    value = slots / (ms_step * 1e-3)

    prompt_rows = int(inp["prefix_lens"].sum()) if paged else None
    a_bytes, a_flops = attn_bytes(case, copies, prompt_rows), attn_flops(case, copies, prompt_rows)
    attn_call = "spec_verify_attn_copies" if copies else "spec_verify_attn_paged" if paged else "spec_verify_attn"
    if tree:
        c_bytes, acc_call = states_bytes(case, inp["st_state"], T == 0), "spec_verify_tree_states"
    else:
        c_bytes = accept_bytes(case, n_rej) if verify == "rejection" else coupled_bytes(case, T == 0)
        acc_call = "spec_verify_accept" if verify == "rejection" else "spec_verify_accept_coupled"
    # the attention is bound by whichever of HBM bytes and bf16 MFMA flops
    # takes longer at peak (the multi-copy layout does B-fold more flops per
    # prompt byte and crosses into the MFMA-bound side)
    if a_flops / (BF16_PEAK_TFLOPS * 1e12) > a_bytes / (HBM_PEAK_GBS * 1e9):
        rl_attn = {"bound": "mfma", "achieved": a_flops / (attn_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "gbs": a_bytes / (attn_ms * 1e-3) / 1e9, "ms": attn_ms, "bytes": a_bytes,
                   "flops": a_flops}
    else:
        rl_attn = {"bound": "hbm", "achieved": a_bytes / (attn_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "tflops": a_flops / (attn_ms * 1e-3) / 1e12, "bf16_peak_tflops": BF16_PEAK_TFLOPS,
                   "ms": attn_ms, "bytes": a_bytes}
    rl_acc = {"bound": "hbm", "achieved": c_bytes / (acc_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "ms": acc_ms, "bytes": c_bytes}
    for r in (rl_attn, rl_acc):
        r["frac"] = r["achieved"] / r["peak"]
    dom = (acc_call, rl_acc) if acc_ms >= attn_ms else (attn_call, rl_attn)
    rl_route = None
    if route != "none":
        r_bytes = route_bytes(case)
        rl_route = {"bound": "hbm", "achieved": r_bytes / (route_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "ms": route_ms, "bytes": r_bytes, "estimator": route, "param": rparam}
        rl_route["frac"] = rl_route["achieved"] / rl_route["peak"]
        rl_route["traffic"] = measured_traffic("spec_verify_route") if case.name == "headline" else None
        if route_ms > max(acc_ms, attn_ms):
            dom = ("spec_verify_route", rl_route)
    rl_commit = None
    if paged:
        n_appended = int((sets[(K - 1) % n_sets].n_append > 0).sum())
        m_bytes = commit_bytes(case, n_appended)
        rl_commit = {"bound": "latency", "ms": commit_ms, "bytes": m_bytes, "appended_blocks": n_appended,
                     "achieved": m_bytes / (commit_ms * 1e-3) / 1e9, "unit": "GB/s"}
    roof_step_s = max(a_bytes / (HBM_PEAK_GBS * 1e9), a_flops / (BF16_PEAK_TFLOPS * 1e12)) + \
        c_bytes / (HBM_PEAK_GBS * 1e9) + (route_bytes(case) / (HBM_PEAK_GBS * 1e9) if route != "none" else 0.0) + \
        (rl_commit["bytes"] / (HBM_PEAK_GBS * 1e9) if paged else 0.0)
    # counter lines exist for the headline workload's variants and for the
    # plain step of the long-prefix and wide workloads
    headline = case.name == "headline"
    # counter lines are per workload: the copies step verifies gamma = D slots;
    # the paged step's verification is the plain step's
    acc_tag = f"_c{copies}" if copies else ""
    attn_tag = acc_tag if copies else (f"_p{args.paged}{'r' if args.ragged else ''}" if paged else "")
    if headline:
        rl_attn["traffic"] = measured_traffic(attn_call + attn_tag)
        # the tempered rejection path runs its own instantiation of the
        # normaliser pass, with a counter line of its own
        rl_acc["traffic"] = measured_traffic(acc_call + ("_greedy" if T == 0 and verify != "rejection" else "") +
                                             ("_tempered" if verify == "rejection" and T != 1.0 else "") + acc_tag)
    elif not (copies or paged or route != "none" or verify != "rejection" or T != 1.0):
        # the plain step of another workload has its own counter lines
        rl_attn["traffic"] = measured_traffic(f"{attn_call}_{case.name}")
        rl_acc["traffic"] = measured_traffic(f"{acc_call}_{case.name}")
    else:
        rl_attn["traffic"] = rl_acc["traffic"] = None
    # the dominant call: algorithmic work per launch over its event-timed
    # average launch
    dom_rl = {"call": dom[0], "bound": dom[1]["bound"], "achieved": round(dom[1]["achieved"], 1),
              "peak": dom[1]["peak"], "unit": dom[1]["unit"], "frac": round(dom[1]["frac"], 4),
              "traffic": dom[1]["traffic"], "traffic_unit": "bytes/launch", "ms_per_launch": round(dom[1]["ms"], 5)}
    dom_rl["frac_of_measured_peak"] = round(dom[1]["achieved"] / (peaks["bf16_gemm_tflops"] if
                                                                  dom[1]["unit"] == "TFLOP/s" else
                                                                  peaks["hbm_read_gbs"]), 4)
    # the metric's roofline is the step's: its calls back to back at their
    # bounds (roof_step_s) against the timed step.  When every call is bound
    # by HBM the step is too, and its rate is the step's algorithmic bytes
    # per timed step; a step whose attention is bound by the MFMA reports the
    # two times instead.
    step_bytes = a_bytes + c_bytes + (route_bytes(case) if route != "none" else 0.0) + \
        (rl_commit["bytes"] if paged else 0.0)
    hbm_step = rl_attn["bound"] == "hbm"
    parts_traffic = [rl_attn["traffic"], rl_acc["traffic"]] + ([rl_route["traffic"]] if rl_route else [])
    if hbm_step:
        roofline = {"bound": "hbm", "achieved": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(roof_step_s / (ms_step * 1e-3), 4),
                    "traffic": (sum(parts_traffic) if all(t is not None for t in parts_traffic) and not paged
                                else None),
                    "traffic_unit": "bytes/step", "algorithmic_bytes": round(step_bytes)}
    else:
        roofline = {"bound": "mfma+hbm", "achieved": round(roof_step_s * 1e6, 2), "peak": round(ms_step * 1e3, 2),
                    "unit": "us (step at its bounds / timed step)", "frac": round(roof_step_s / (ms_step * 1e-3), 4),
                    "traffic": None, "traffic_unit": "bytes/step"}
    roofline["what"] = "whole step (every call at its roofline) vs the timed step"
    roofline["dominant_kernel"] = dom_rl
    cpu = None
    if not args.no_cpu_baseline:
        gpu_acc = None
        if verify == "rejection" and not tree and not paged:
            # the GPU's outputs of the inputs in `inp` (every input set holds them)
            gpu_acc = (sets[0].accept_len.cpu().numpy(), sets[0].out_tokens.cpu().numpy())
        # the GPU's attention output of the same inputs
        gpu_out = sets[0].out_c if copies else sets[0].out_paged if paged else sets[0].out
        cpu = cpu_baseline(case, inp, verify, T, route, rparam, copies, paged, tree, gpu_accept=gpu_acc,
                           threshold=case.threshold, gpu_attn=gpu_out.float().cpu().numpy())

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "slots/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{case.name} SPOT multi-copy verify step: {copies} copies (root + D={copies - 1} "
                                f"draft states" + (" in a tree of block states" +
                                                   (f", commit threshold {case.threshold:g}"
                                                    if case.threshold < 1 else ", one commit per step")
                                                   if tree else "") + "), gamma=D"
                                if copies else f"{case.name} verify step") +
                               f": batch {case.batch}, prefix {case.prefix_len}, "
                               f"B={case.block}, gamma={case.gamma}, {case.n_qh}/{case.n_kvh} heads, "
                               f"head_dim {case.head_dim}, "
                               f"vocab {case.vocab}, {case.dtype} attention, fp32 logits" +
                               ("" if verify == "rejection" else
                                f"; {'greedy' if T == 0 else f'shared-noise (T={T:g})'} verification") +
                               (f"; rejection sampling at T={T:g}" if verify == "rejection" and T != 1.0 else "") +
                               ("" if route == "none" else f"; S2D2 routing estimate ({route}, {rparam:g}) first") +
                               ("" if not paged else f"; prompt cache in pages of {case.page_size} rows"
                                + (", ragged prompt lengths (mean %.0f)" % inp["prefix_lens"].mean() if case.ragged
                                   else "") + ", then commit and cache append"),
                   "route": None if route == "none" else {"estimator": route, "param": rparam},
                   "verify": verify, "temperature": None if verify == "rejection" and T == 1.0 else T,
                   "copies": copies or None, "tree": tree if copies else None,
                   "threshold": case.threshold if tree else None,
                   "page_size": case.page_size if paged else None, "ragged": bool(case.ragged) if paged else None,
                   "batch": case.batch, "prefix_len": case.prefix_len, "block": case.block, "gamma": case.gamma,
                   "n_qh": case.n_qh, "n_kvh": case.n_kvh, "head_dim": case.head_dim, "vocab": case.vocab,
                   "parallelism": "single GPU", "launch": args.launch},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "input_sets": n_sets,
            "measured_peaks": peaks,
            "attn": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in rl_attn.items()},
            "accept": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in rl_acc.items()},
            "commit": None if rl_commit is None else
            {k: (round(v, 5) if isinstance(v, float) else v) for k, v in rl_commit.items()},
            "route": None if rl_route is None else
            {k: (round(v, 5) if isinstance(v, float) else v) for k, v in rl_route.items()},
            "step_roofline_us": round(roof_step_s * 1e6, 2),
            "frac_of_step_roofline": round(roof_step_s / (ms_step * 1e-3), 4),
            "wall_s": round(wall, 4),
            "mean_accept_len": float(L.float().mean()),
            "rejecting_sequences": n_rej,
            # acceptance outputs of the GPU against the oracle on the same inputs
            # (counted ties are decisions within 1e-6 of their threshold)
            "oracle_agreement": cpu["agreement"] if cpu else None,
            # attention rows of the oracle's timed sequences against the GPU's
            # (max abs and relative RMS error)
            "attn_oracle_agreement": cpu["attn_agreement"] if cpu else None,
        },
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

"""Throughput of batched speculative-sampling verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the whole hot path on the headline workload (B = 256 sequences,
gamma = 8 draft tokens, V = 128256 bf16 logits, half the sequences greedy and
half at T = 1): verification (accept prefix + bonus token) and the F = 4 SSD
bonus candidates per position, as one specv_verify_topk call (one kernel that
reads every target and draft row once). Inputs are seeded synthetic logits
already resident in HBM when timing starts, in four identical copies that the
calls use in turn, so that no call finds its rows in the Infinity Cache.

Prints one JSON line: verified rows/s (B * (gamma + 1) per step), the step
kernel's roofline (algorithmic HBM bytes / its average duration, measured with
HIP events on the launch stream), the separate specv_verify and
specv_bonus_topk kernels for reference, and the oracle timed on the host cores
(a process pool over the workload's sequences, run before the GPU is used),
with its outcome compared to the step's on every sequence. A `tree` field
times token-tree verification (MSS) on 32 trees of 64 nodes over V = 152064
(--no-tree skips); `configs` times specv_verify on the B = 8, V = 32000 fp32
and B = 64, V = 128256 peaked bf16 workloads.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOAD = "v128256_bf16_b256_g8"
TREE_WORKLOAD = "tree_v152064_n64"
METRIC = "verified vocab rows/sec + achieved HBM GB/s (% peak) at V=128256, B=256, γ=8"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "speculative_sampling_verification_04_amd", "csrc")
COPY_BYTES = 1 << 30
SETTLE_S = 0.2
# Every timed loop cycles through this many identical copies of its inputs in
# HBM, so that no call finds the previous call's rows in the 256 MB Infinity
# Cache: rows streamed with ordinary loads stay there from one call to the
# next, and re-reading one input set back to back measured ~4% faster than
# reading inputs that were not read just before. A serving loop verifies new
# logits every step.
INPUT_SETS = 4


def algorithmic_bytes(w):
    """Logit bytes each call must read at least once (rows of V bf16):
    verify: every target row, and a draft row only for T > 0 sequences
    (greedy rows never read the draft); top-F: every draft row; the fused
    step: every target row and every draft row."""
    row = w.V * 2
    n_sampled = int((w.temperature > 0).sum())
    verify = w.B * (w.gamma + 1) * row + n_sampled * w.gamma * row
    topf = w.B * (w.gamma + 1) * row
    step = 2 * w.B * (w.gamma + 1) * row
    return verify, topf, step


def step_bytes_of(w):
    return algorithmic_bytes(w)[2]


def tree_algorithmic_bytes(tw):
    """Logit bytes of one tree call: every node's target row, plus the draft
    row of every node that has children when T > 0 (greedy trees read none)."""
    row = tw.V * 2
    total = 0
    for b in range(tw.B):
        internal = len(set(int(p) for p in tw.parent[b, 1:]))
        total += tw.N * row + (internal * row if tw.temperature[b] > 0 else 0)
    return total


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "bench_kernels_v128256_b256_g8_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# The workload the CPU baseline's worker processes read (inherited through
# fork: the pool is started before anything touches the GPU).
_CPU_W = None


def _oracle_sequence(b):
    """The oracle, as written, on sequence b of the workload: verification
    and top-F."""
    import oracle

    w = _CPU_W
    u, v = oracle.philox.chain_uniforms(w.seed, w.offset, b, w.gamma)
    r = oracle.sampling.verify_sequence(w.target[b].astype(np.float64), w.draft[b].astype(np.float64),
                                        w.draft_tokens[b], float(w.temperature[b]), u, v)
    ids, _ = oracle.topf.bonus_topf_batch(w.draft[b:b + 1].astype(np.float64), w.draft_tokens[b:b + 1], w.F)
    toks = np.full(w.gamma + 1, -1, np.int64)
    toks[:len(r.tokens)] = r.tokens
    return b, int(r.k), toks, bool(r.near_tie), ids[0]


def _warm(_):
    import oracle  # noqa: F401
    return os.getpid()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, reps=3, max_workers=16):
    """The oracle over every sequence of the workload (verify + top-F), in a
    pool of worker processes, one sequence per task, on the host cores
    available to this process (at most max_workers: the host's share for
    one GPU); the median of `reps` runs. Must run before the GPU is used (the
    pool forks). Returns (line, per-sequence oracle results)."""
    import multiprocessing

    global _CPU_W
    _CPU_W = w
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    ctx = multiprocessing.get_context("fork")
    times, results = [], None
    with ctx.Pool(workers) as pool:
        pool.map(_warm, range(workers))
        for _ in range(reps):
            t0 = time.perf_counter()
            res = pool.map(_oracle_sequence, range(w.B), chunksize=1)
            times.append(time.perf_counter() - t0)
            results = results or res
    dt = float(np.median(times))
    rows = w.B * (w.gamma + 1)
    line = {"value": rows / dt, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": f"all {w.B} sequences of the workload (half greedy, half T=1), verify + top-F, {rows} rows, "
                      f"one sequence per task over {workers} worker processes (numpy fp64); median of {reps} runs "
                      f"of {', '.join(f'{t:.2f}' for t in times)} s",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "gbps": 2 * rows * w.V * 2 / dt / 1e9}
    return line, results


def parity_of(results, gpu):
    """The fused step's outcome (k, tokens) and top-F ids against the
    oracle's, sequence by sequence."""
    equal = near = differ = topf_equal = 0
    for b, k, toks, near_tie, ids in results:
        same = int(gpu["num_accepted"][b]) == k and np.array_equal(gpu["tokens"][b], toks)
        if near_tie:
            near += 1
        elif same:
            equal += 1
        else:
            differ += 1
        topf_equal += int(np.array_equal(gpu["topk"][b], ids))
    return {"sequences": len(results), "outcome_equal": equal, "near_ties": near, "outcome_differs": differ,
            "topf_equal": topf_equal,
            "note": "the fused step's outcome (k, tokens) and top-F ids against the oracle's on every sequence; "
                    "near ties are decisions within 1e-6 of a tie"}


def verify_bytes_of(w):
    """Logit bytes specv_verify must read: every target row, and a draft row
    of each T > 0 sequence's gamma positions."""
    esz = 2 if w.dtype == "bf16" else 4
    n_sampled = int((w.temperature > 0).sum())
    return (w.B * (w.gamma + 1) + n_sampled * w.gamma) * w.V * esz


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-tree", action="store_true", help="skip the token-tree measurement")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the verification library has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import workloads

    w = workloads.make_workload(WORKLOAD)
    # The CPU baseline first: its worker processes are forked before this
    # process touches the GPU.
    cpu_line, cpu_results = (None, None) if args.no_cpu_baseline else cpu_baseline(w, args.cpu_reps)

    import torch

    from speculative_sampling_verification_04_amd import binding

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.load_library()
    target = torch.from_numpy(w.target).to(dev).to(torch.bfloat16)
    draft = torch.from_numpy(w.draft).to(dev).to(torch.bfloat16)
    sets = [(target, draft)] + [(target.clone(), draft.clone()) for _ in range(INPUT_SETS - 1)]
    tokens = torch.from_numpy(w.draft_tokens).to(dev)
    temp = torch.from_numpy(w.temperature).to(dev)
    B, gamma, F = w.B, w.gamma, w.F
    out = dict(tokens=torch.empty((B, gamma + 1), dtype=torch.int32, device=dev),
               num_accepted=torch.empty((B,), dtype=torch.int32, device=dev),
               probs=torch.empty((B, gamma, 2), dtype=torch.float32, device=dev),
               bonus_mass=torch.empty((B,), dtype=torch.float32, device=dev),
               topk=torch.empty((B, gamma + 1, F), dtype=torch.int32, device=dev),
               topk_logits=torch.empty((B, gamma + 1, F), dtype=torch.float32, device=dev))
    ws = torch.zeros(binding.verify_topk_workspace_bytes(B, gamma, w.V), dtype=torch.uint8, device=dev)

    def step(i):
        t, d = sets[i % INPUT_SETS]
        binding.verify_topk(t, d, tokens, temp, F, w.seed, i, workspace=ws, out=out)

    # Settle: the GPU's clocks take tens of milliseconds to ramp up from idle,
    # so the step is run for SETTLE_S of wall time before the W warm-up steps
    # (untimed, and reported as settle_ms).
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(20):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record()
        step(args.warmup + i)
        events[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_times = np.array([e[0].elapsed_time(e[1]) for e in events])
    step_kernel_ms = float(step_times.mean())
    step_pct = {f"p{q}_ms": float(np.percentile(step_times, q)) for q in (10, 50, 90)}
    mean_accepted = float(out["num_accepted"].float().mean().item())

    # Reference: the two entry points run separately (not part of the step).
    def timed(fn, n=50):
        # Same settle as the step: building each line's inputs leaves the GPU
        # idle for seconds, and the first calls after that run at low clocks.
        t_s, i = time.perf_counter(), 0
        while time.perf_counter() - t_s < SETTLE_S / 2:
            for _ in range(10):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    vws = torch.zeros(binding.verify_workspace_bytes(B, gamma, w.V), dtype=torch.uint8, device=dev)
    vout = {k: out[k] for k in ("tokens", "num_accepted", "probs", "bonus_mass")}
    verify_ms = timed(lambda i: binding.verify(*sets[i % INPUT_SETS], tokens, temp, w.seed, i, workspace=vws, out=vout))
    topf_ms = timed(lambda i: binding.bonus_topk(sets[i % INPUT_SETS][1], tokens, F,
                                                 out=(out["topk"], out["topk_logits"])))

    # SSD cache verification on the same rows: Theorem 12 fan-outs for a
    # budget of (gamma + 1) * F candidates (a = 0.6, r = 1), Saguaro sampling
    # with C = 47/147, exact rule (not part of the step).
    fan = binding.geometric_fanout(gamma, 0.6, 1.0, (gamma + 1) * F)
    cws = torch.zeros(binding.verify_cache_workspace_bytes(B, gamma, w.V), dtype=torch.uint8, device=dev)
    cout = binding.verify_cache(target, draft, tokens, temp, fan, w.seed, 0, saguaro_C=47 / 147, workspace=cws)
    cache_ms = timed(lambda i: binding.verify_cache(*sets[i % INPUT_SETS], tokens, temp, fan, w.seed, i,
                                                    saguaro_C=47 / 147, workspace=cws, out=cout))
    cache = {"entry": "specv_verify_cache", "fanout": fan, "saguaro_C": 47 / 147, "lenience": 1.0,
             "avg_ms": cache_ms, "algorithmic_bytes": step_bytes_of(w),
             "gbps": step_bytes_of(w) / (cache_ms * 1e-3) / 1e9,
             "hit_rate": float(cout["hit"].float().mean().item())}

    # Ragged batch over the same rows: sequence b drafts gamma_b in 1..gamma
    # tokens (seeded), rows packed; with draft logits, then without (n-gram
    # style drafts). Not part of the step.
    counts = np.random.default_rng(1234).integers(1, gamma + 1, B)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t_rows = [torch.cat([t[b, :counts[b] + 1] for b in range(B)]) for t, _ in sets]
    d_rows = [torch.cat([d[b, :counts[b]] for b in range(B)]) for _, d in sets]
    r_tok = torch.cat([tokens[b, :counts[b]] for b in range(B)])
    r_off = torch.from_numpy(offs).to(dev)
    ragged = {}
    for mode, dr in (("with_draft", d_rows), ("no_draft", None)):
        rws = torch.zeros(binding.verify_ragged_workspace_bytes(B, gamma, w.V, dr is not None), dtype=torch.uint8,
                          device=dev)
        rout = binding.verify_ragged(t_rows[0], dr[0] if dr else None, r_off, r_tok, temp, gamma, w.seed, 0,
                                     workspace=rws)
        r_ms = timed(lambda i: binding.verify_ragged(t_rows[i % INPUT_SETS], dr[i % INPUT_SETS] if dr else None, r_off,
                                                     r_tok, temp, gamma, w.seed, i, workspace=rws, out=rout))
        n_rows = int((counts + 1).sum()) + (int(counts[w.temperature > 0].sum()) if dr is not None else 0)
        r_bytes = n_rows * w.V * 2
        ragged[mode] = {"avg_ms": r_ms, "rows_read": n_rows, "algorithmic_bytes": r_bytes,
                        "gbps": r_bytes / (r_ms * 1e-3) / 1e9,
                        "mean_accepted": float(rout["num_accepted"].float().mean().item())}
    ragged["draft_counts"] = "uniform in 1..gamma, seed 1234"
    del t_rows, d_rows

    # Token-tree verification (MSS, T = 1) on its own workload: B = 32 trees of
    # N = 64 nodes over V = 152064 bf16 logits (not part of the step).
    tree = None
    if not args.no_tree:
        tw = workloads.make_workload(TREE_WORKLOAD)
        tt = torch.from_numpy(tw.target).to(dev).to(torch.bfloat16)
        td = torch.from_numpy(tw.draft).to(dev).to(torch.bfloat16)
        tsets = [(tt, td)] + [(tt.clone(), td.clone()) for _ in range(INPUT_SETS - 1)]
        tpar = torch.from_numpy(tw.parent).to(dev)
        ttok = torch.from_numpy(tw.tokens).to(dev)
        ttemp = torch.from_numpy(tw.temperature).to(dev)
        tws = torch.zeros(binding.tree_workspace_bytes(tw.B, tw.N, tw.V), dtype=torch.uint8, device=dev)
        tout = binding.tree_verify(tt, td, tpar, ttok, ttemp, tw.seed, 0, workspace=tws)
        tree_ms = timed(lambda i: binding.tree_verify(*tsets[i % INPUT_SETS], tpar, ttok, ttemp, tw.seed, i,
                                                      workspace=tws, out=tout))
        tree_bytes = tree_algorithmic_bytes(tw)
        tree = {"workload": TREE_WORKLOAD, "kernels": "tree_fused_kernel (rows and walks in one launch)", "B": tw.B, "N": tw.N, "V": tw.V,
                "avg_ms": tree_ms, "algorithmic_bytes": tree_bytes, "gbps": tree_bytes / (tree_ms * 1e-3) / 1e9,
                "trees_per_s": tw.B / (tree_ms * 1e-3),
                "mean_accepted": float(tout["num_accepted"].float().mean().item())}
        del tt, td, tsets, tws

    # Configurations 2 and 3: specv_verify alone, on enough copies of the
    # inputs that the calls in turn read past the 256 MB Infinity Cache
    # (config 2's 9.2 MB, config 3's 180.6 MB). Not part of the step.
    configs = {}
    for cname, n_sets in (("v32000_f32", 32), ("v128256_bf16_peaked", 4)):
        wc = workloads.make_workload(cname)
        cdt = torch.bfloat16 if wc.dtype == "bf16" else torch.float32
        ct = torch.from_numpy(wc.target).to(dev).to(cdt)
        cd = torch.from_numpy(wc.draft).to(dev).to(cdt)
        csets = [(ct, cd)] + [(ct.clone(), cd.clone()) for _ in range(n_sets - 1)]
        ctok = torch.from_numpy(wc.draft_tokens).to(dev)
        ctemp = torch.from_numpy(wc.temperature).to(dev)
        cws_v = torch.zeros(binding.verify_workspace_bytes(wc.B, wc.gamma, wc.V), dtype=torch.uint8, device=dev)
        cvout = binding.verify(ct, cd, ctok, ctemp, wc.seed, 0, workspace=cws_v)
        c_ms = timed(lambda i: binding.verify(*csets[i % n_sets], ctok, ctemp, wc.seed, i, workspace=cws_v,
                                              out=cvout), n=100)
        c_bytes = verify_bytes_of(wc)
        c_rows = wc.B * (wc.gamma + 1)
        configs[cname] = {"entry": "specv_verify", "B": wc.B, "gamma": wc.gamma, "V": wc.V, "logits": wc.dtype,
                          "input_sets": n_sets, "avg_ms": c_ms, "rows_per_s": c_rows / (c_ms * 1e-3),
                          "algorithmic_bytes": c_bytes, "gbps": c_bytes / (c_ms * 1e-3) / 1e9,
                          "frac": c_bytes / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "mean_accepted": float(cvout["num_accepted"].float().mean().item())}
        del ct, cd, csets, cws_v

    # Yardstick for the memory counters and for what a plain streaming kernel
    # reaches: torch's elementwise negation of 1 GiB of int32 (reads 1 GiB, writes
    # 1 GiB; larger than the 256 MB last-level cache), outside the timed region.
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda i: torch.neg(src, out=dst))
    del src, dst

    ms_per_step = elapsed * 1e3 / args.steps
    rows = B * (gamma + 1)
    verify_bytes, topf_bytes, step_bytes = algorithmic_bytes(w)
    achieved = step_bytes / (step_kernel_ms * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = measured_traffic("verify_topf_kernel")

    line = {
        "metric": METRIC,
        "value": rows / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": settle_ms,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "gamma": gamma, "V": w.V, "logits": "bf16",
                   "F": F, "greedy_sequences": int((w.temperature == 0).sum()),
                   "step": "specv_verify_topk", "parallelism": "none", "input_sets": INPUT_SETS},
        "hbm_gbps": step_gbps,
        "hbm_pct_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": "verify_topf_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes": step_bytes, "avg_ms": step_kernel_ms, **step_pct},
        "separate_kernels": {
            "chain_verify_kernel": {"avg_ms": verify_ms, "algorithmic_bytes": verify_bytes,
                                    "gbps": verify_bytes / (verify_ms * 1e-3) / 1e9},
            "topf_kernel": {"avg_ms": topf_ms, "algorithmic_bytes": topf_bytes,
                            "gbps": topf_bytes / (topf_ms * 1e-3) / 1e9}},
        "copy_yardstick": {"kernel": "torch.neg int32", "read_bytes": COPY_BYTES, "write_bytes": COPY_BYTES,
                           "avg_ms": copy_ms, "gbps": 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9},
        "mean_accepted": mean_accepted,
        "cache": cache,
        "ragged": ragged,
        "tree": tree,
        "configs": configs,
    }
    if cpu_line is not None:
        ref_out = binding.verify_topk(target, draft, tokens, temp, F, w.seed, w.offset)
        torch.cuda.synchronize()
        gpu = {k: ref_out[k].cpu().numpy() for k in ("tokens", "num_accepted", "topk")}
        cpu_line["parity"] = parity_of(cpu_results, gpu)
        line["cpu_baseline"] = cpu_line
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one pass of the whole verify path over one batch: the LM-head
contraction of the K+1 verify positions, the softmax statistics, and the
acceptance of every sequence (greedy or sampled, by the workload's per-row
mode), including the residual or bonus draw.  By default the step is one
spec_verify_step call (spec_verify_step_ragged for packed batches,
spec_tree_verify_step for draft trees; --path fused); --path separate runs
spec_verify_logits then the accept calls (spec_accept_sample /
spec_accept_greedy, their ragged forms, or spec_tree_accept_greedy).  Inputs
(weights, hidden states, draft logits, per-round draft tokens and seeds) are
resident in HBM before the timed region; each timed step uses the next
pre-drawn draft set and seed.

Prints one JSON line: verified positions per second (B*(K+1) / step time) and
the step time, with the roofline of the dominant kernel (the LM-head
contraction, timed with HIP events on the stream it runs on) and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload b1_k5_h4096_v128256]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "verified positions/sec + verify-step µs (B=1,K=5); % HBM / MFMA peak"
GEMM_SRC = os.path.join(ROOT, "speculative_decoding_verification_02_amd", "csrc", "lmhead_gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b1_k5_h4096_v128256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="headline workload only (by default its line also carries the other benchmark workloads)")
    ap.add_argument("--record-rounds", type=int, default=512,
                    help="further rounds, drafts redrawn each, whose accepted lengths give the acceptance by "
                         "position (0 leaves it out, e.g. for profiler runs)")
    ap.add_argument("--path", choices=["fused", "separate"], default="fused",
                    help="fused: spec_verify_step, the one-call step (statistics in the LM-head kernel where "
                         "it can compute them); separate: spec_verify_logits then the accept calls")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the run, copy a buffer of this many MiB 3 times (untimed), so a counter "
                         "profile of this command holds a plain copy kernel of known size")
    ap.add_argument("--traffic-kernel", default="lmhead_coop_bf16", help="LM-head kernel the counters cover")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then WRITE_SIZE, of a "
                         "run with --copy-calibration-mib) into profiles/lmhead_traffic_<workload>.json and exit")
    return ap.parse_args()


# Source section of each LM-head kernel in lmhead_gemm.hip (text from its
# banner comment to the next one: the kernel, its configuration and its
# launcher), so that stored counter readings stay tied to the kernel they
# were taken on.
_SECTIONS = {"lmhead_coop_bf16": "small M, cooperative", "lmhead_big_bf16": "big M",
             "lmhead_skinny_bf16": "small M",
             "lmhead_tiled_bf16": "large M", "lmhead_f32": "fp32"}


def kernel_source_sha(kernel: str) -> str:
    """sha256 of the code of the kernel's source section (kernel,
    configuration and launcher; comments and blank lines dropped), so edits
    elsewhere in the file, or to comments, keep stored readings valid."""
    lines = open(GEMM_SRC).read().splitlines()
    banners = [i for i, ln in enumerate(lines) if ln.startswith("// ---")]
    i = next(i for i in banners if lines[i].strip("/ -") == _SECTIONS[kernel])
    j = next((k for k in banners if k > i), len(lines))
    code = []
    for ln in lines[i:j]:
        ln = ln.split("//", 1)[0].rstrip()
        if ln.strip():
            code.append(ln)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the LM-head kernel from the committed counter
    summary, or None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "lmhead_traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel") != kernel or rec.get("source_sha") != kernel_source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(path, counter):
    import csv
    out = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") == counter:
            out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


# position of the statistics flag among each LM-head kernel's template
# arguments (cooperative <RPL, MAXST, NW, STATS, STASH>; direct-to-LDS
# <BK, SLOTS, NA, NB, STATS, NW, HS>)
_STATS_ARG = {"lmhead_coop_bf16": 3, "lmhead_big_bf16": 4}


def _stats_variant(name):
    base = name.split("(")[0]
    for k, i in _STATS_ARG.items():
        if k in base and "<" in base:
            args = [a.strip() for a in base[base.index("<") + 1:base.rindex(">")].split(",")]
            return len(args) > i and args[i] == "true"
    return False


def ingest_traffic(args):
    """HBM bytes per launch of the LM-head kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled so that the calibration copy of known size
    reads and writes exactly its size."""
    fetch = _counter_rows(args.ingest_traffic[0], "FETCH_SIZE")
    write = _counter_rows(args.ingest_traffic[1], "WRITE_SIZE")
    size = args.copy_calibration_mib * (1 << 20)
    if size <= 0:
        sys.exit("--ingest-traffic needs --copy-calibration-mib of the profiled run")

    def median_of(rows, pred):
        vals = sorted(v for n, v in rows if pred(n))
        if not vals:
            sys.exit("no matching dispatch in the counter file")
        return vals[len(vals) // 2]

    # the calibration copy is a contiguous same-type copy: the runtime's blit
    # kernel; take its largest dispatches (the calibration is the biggest copy)
    is_copy = lambda n: "copyBuffer" in n
    # the LM-head launches without the statistics option: the ones the
    # event-timed loop measures (the fused step runs the other variant)
    is_gemm = lambda n: "sv::lmhead" in n and not _stats_variant(n)

    def calib(rows):
        vals = sorted((v for n, v in rows if is_copy(n)), reverse=True)[:3]
        if not vals:
            sys.exit("no calibration copy in the counter file")
        return vals[len(vals) // 2]

    f_copy = calib(fetch)
    w_copy = calib(write)
    f_scale = size / (f_copy * 1024.0)
    w_scale = size / (w_copy * 1024.0)
    f_gemm = median_of(fetch, is_gemm) * 1024.0 * f_scale
    w_gemm = median_of(write, is_gemm) * 1024.0 * w_scale
    kernel = args.traffic_kernel
    rec = {"workload": args.workload, "kernel": kernel, "source_sha": kernel_source_sha(kernel),
           "fetch_bytes_per_launch": f_gemm, "write_bytes_per_launch": w_gemm,
           "hbm_bytes_per_launch": f_gemm + w_gemm, "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration": "torch copy of %d MiB: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB"
                          % (args.copy_calibration_mib, f_copy, w_copy)}
    path = os.path.join(ROOT, "profiles", "lmhead_traffic_%s.json" % args.workload)
    json.dump(rec, open(path, "w"), indent=1)
    print(json.dumps(rec))


def main():
    args = parse()
    if args.ingest_traffic:
        ingest_traffic(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the verify path here has no multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_decoding_verification_02_amd as sv
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.load_library()
    if args.workload in synth.NGRAM_WORKLOADS:
        print(json.dumps(bench_ngram(args, dev, synth.NGRAM_WORKLOADS[args.workload],
                                     cpu=not args.no_cpu_baseline, steps=args.steps)), flush=True)
        return
    res = measure(synth.WORKLOADS[args.workload], args, dev, args.steps, args.warmup,
                  cpu=not args.no_cpu_baseline, record_rounds=args.record_rounds)
    if args.workload == HEADLINE and not args.no_other_configs:
        # the other benchmark workloads, under the same clock: a few steps
        # each, no CPU baseline
        others = []
        for name in OTHER_CONFIGS:
            r = measure(synth.WORKLOADS[name], args, dev, min(args.steps, 10), 3, cpu=False)
            others.append({k: r[k] for k in ("config", "ms_per_step", "value", "unit", "step_us_median",
                                               "step_roofline", "roofline", "path")})
            torch.cuda.empty_cache()
        res["other_configs"] = others
        # the rows built beyond the five workloads: long blocks, per-sequence
        # draft counts, draft trees, and the prompt-lookup drafter
        widened = []
        for name in WIDENED:
            r = measure(synth.WORKLOADS[name], args, dev, min(args.steps, 10), 3, cpu=False)
            widened.append({k: r[k] for k in ("config", "ms_per_step", "value", "unit", "step_us_median",
                                               "step_roofline", "roofline", "path")})
            torch.cuda.empty_cache()
        r = bench_ngram(args, dev, synth.NGRAM_WORKLOADS["ngram_b256_l131072"], cpu=False, steps=min(args.steps, 20))
        widened.append({k: r[k] for k in ("config", "ms_per_step", "value", "unit", "step_us_median", "roofline")})
        res["widened_rows"] = widened
    print(json.dumps(res), flush=True)


HEADLINE = "b1_k5_h4096_v128256"
OTHER_CONFIGS = ("b64_k4_h4096_v128256", "b256_k8_h8192_v152064", "b512_k3_h5120_v262144")
WIDENED = ("b32_k15_h4096_v151936", "b64_k0to7_h4096_v128256", "b8_tree63_h4096_v128256")


def measure(wl, args, dev, n_steps, n_warmup, cpu=False, record_rounds=0):
    """Time one workload: n_warmup untimed steps, n_steps timed steps, the
    LM-head kernel alone under HIP events, the step distribution; with cpu,
    the oracle on a bounded sample of the same rounds; with record_rounds,
    the accepted lengths of that many further rounds (acceptance by draft
    position, and the rounds the CPU leg compares against the oracle)."""
    import torch

    import speculative_decoding_verification_02_amd as sv
    import synth

    B, K, H, V, T = wl.B, wl.K, wl.H, wl.V, wl.temperature
    M = wl.M
    print("bench: %s, generating inputs" % wl.name, file=sys.stderr, flush=True)
    W = synth.weights(wl, dev)
    hidden = synth.hidden_states(wl, dev)
    zd = synth.draft_logits(wl, synth.base_logits(hidden, W))
    smask = synth.sampled_mask(wl)
    n_sets = 16
    drafts = [synth.draft_tokens(zd, smask, T, seed=wl.data_seed * 104729 + r) for r in range(n_sets)]
    row_start = None
    tree = None
    if wl.tree:
        # draft trees of K nodes: parents fixed, node tokens redrawn per set
        par = synth.tree_parents(B, K, seed=wl.data_seed)
        base = synth.base_logits(hidden, W)
        tree = (torch.as_tensor(par, device=dev),
                [synth.tree_tokens(base, par, seed=wl.data_seed + 1 + r, sigma=wl.draft_sigma[0]).to(dev)
                 for r in range(n_sets)],
                torch.empty((B, K + 1), dtype=torch.int32, device=dev))
        drafts = [t.cpu() for t in tree[1]]
        del base
    if wl.ragged:
        # per-sequence draft counts: pack every input, K is the bound K_max
        counts = synth.draft_counts(B, K, wl.data_seed)
        rs = synth.row_start(counts)
        M = int(rs[-1])
        hidden = synth.pack_rows(hidden, counts).contiguous().view(M, 1, H)
        zd = synth.pack_rows(zd, counts, True).contiguous()
        drafts = [synth.pack_rows(d, counts, True).contiguous() for d in drafts]
        row_start = torch.as_tensor(rs, device=dev)
    n_seed_sets = n_warmup + n_steps + record_rounds
    seeds = [torch.from_numpy(synth.seeds(wl, r).view(np.int64).copy()).to(dev) for r in range(n_seed_sets)]
    greedy_rows = torch.as_tensor(np.nonzero(~smask)[0].astype(np.int32), device=dev)
    sampled_rows = torch.as_tensor(np.nonzero(smask)[0].astype(np.int32), device=dev)
    all_sampled, all_greedy = bool(smask.all()), bool((~smask).all())

    logits = torch.empty(tuple(hidden.shape[:2]) + (V,), dtype=torch.float32, device=dev)
    ws = torch.empty(sv.spec_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty(tuple(hidden.shape[:2]), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    step_ws = None
    if args.path == "fused":
        nbytes = (sv.spec_verify_step_ragged_workspace_bytes(B, K, V) if row_start is not None
                  else sv.spec_verify_step_workspace_bytes(B, K, V))
        step_ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        g_arg = None if not len(greedy_rows) else ("all" if all_greedy else greedy_rows)
        s_arg = None if not len(sampled_rows) else ("all" if all_sampled else sampled_rows)

    def step(r):
        d = drafts[r % n_sets]
        if step_ws is not None and tree is not None:
            sv.spec_tree_verify_step(hidden, W, logits, tree[0], tree[1][r % n_sets], acc, out, step_ws,
                                     out_nodes=tree[2], stream=stream)
            return
        if step_ws is not None and row_start is not None:
            sv.spec_verify_step_ragged(hidden.view(M, H), W, logits.view(M, V), row_start, K, acc, out.view(M),
                                       step_ws, draft_logits=zd, draft_tokens=d, temperature=T, seeds=seeds[r],
                                       greedy_rows=g_arg, sampled_rows=s_arg, stream=stream)
            return
        if step_ws is not None:
            sv.spec_verify_step(hidden, W, logits, acc, out, step_ws, draft_logits=zd, draft_tokens=d, temperature=T,
                                seeds=seeds[r], greedy_rows=g_arg, sampled_rows=s_arg, stream=stream)
            return
        sv.spec_verify_logits(hidden, W, logits, stream=stream)
        if tree is not None:
            sv.spec_tree_accept_greedy(logits, tree[0], tree[1][r % n_sets], acc, out, ws, out_nodes=tree[2],
                                       stream=stream)
        elif row_start is not None:
            lg, o = logits.view(M, V), out.view(M)
            if len(greedy_rows):
                sv.spec_accept_greedy_ragged(lg, d, row_start, K, acc, o, ws, rows=greedy_rows, stream=stream)
            if len(sampled_rows):
                sv.spec_accept_sample_ragged(lg, zd, d, row_start, K, T, seeds[r], acc, o, ws, rows=sampled_rows,
                                             stream=stream)
        elif all_sampled:
            sv.spec_accept_sample(logits, zd, d, T, seeds[r], acc, out, ws, stream=stream)
        elif all_greedy:
            sv.spec_accept_greedy(logits, d, acc, out, ws, stream=stream)
        else:
            sv.spec_accept_greedy(logits, d, acc, out, ws, rows=greedy_rows, stream=stream)
            sv.spec_accept_sample(logits, zd, d, T, seeds[r], acc, out, ws, rows=sampled_rows, stream=stream)

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print("bench: warmup %d" % n_warmup, file=sys.stderr, flush=True)
    for r in range(n_warmup):
        step(r)
    torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n_steps):
        step(n_warmup + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / n_steps
    accepted = acc.cpu().numpy()

    # the dominant kernel on its own: HIP events around each LM-head launch on
    # the stream it runs on (a separate loop, so the step timing above carries
    # no event overhead)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    for a, b in evs:
        a.record(stream)
        sv.spec_verify_logits(hidden, W, logits, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    print("bench: %d steps, %.1f us/step, LM-head kernel %.1f us" % (n_steps, step_s * 1e6, gemm_ms * 1e3),
          file=sys.stderr, flush=True)

    # the distribution of single steps (HIP events around each step, in a
    # loop of its own) and the tokens each commits: sum over sequences of
    # accepted length + 1
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    acc_hist = torch.empty((n_steps, B), dtype=torch.int32, device=dev)
    for k, (a, b) in enumerate(sev):
        a.record(stream)
        step(n_warmup + k)
        b.record(stream)
        acc_hist[k].copy_(acc)
    torch.cuda.synchronize()
    step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in sev])
    hist = acc_hist.cpu().numpy()
    committed = np.where(hist >= 0, hist + 1, 0).sum(axis=1)   # a faulted sequence (-1) commits nothing

    # algorithmic bytes / flops of one LM-head launch
    wbytes = 2 if wl.dtype == "bf16" else 4
    gemm_bytes = V * H * wbytes + M * H * wbytes + M * V * 4
    gemm_flops = 2.0 * M * V * H
    intensity = gemm_flops / gemm_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    t_gemm = gemm_ms * 1e-3
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": gemm_bytes / t_gemm / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gemm_flops / t_gemm / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if wl.dtype != "bf16":
        roof["kernel"] = "lmhead_f32"
    elif M <= 16 and H <= 4096:
        roof["kernel"] = "lmhead_coop_bf16"
    elif M <= 16:
        roof["kernel"] = "lmhead_skinny_bf16"
    elif H % 64 == 0 and V * H < 2 ** 32 and M * H < 2 ** 32:
        roof["kernel"] = "lmhead_big_bf16"
    else:
        roof["kernel"] = "lmhead_tiled_bf16"
    roof["traffic"] = load_traffic(wl.name, roof["kernel"])
    roof["algorithmic_bytes"] = gemm_bytes
    roof["algorithmic_flops"] = gemm_flops
    roof["avg_kernel_us"] = gemm_ms * 1e3

    # algorithmic bytes of one whole step (each tensor of the three-stage
    # interface once: W, hidden, logits written and read back, draft logits of
    # the sampled rows, two terminal rows per sampled sequence)
    n_sampled = int(smask.sum())
    if row_start is not None:
        rs_np = row_start.cpu().numpy()
        draft_rows = int(sum(rs_np[b + 1] - rs_np[b] - 1 for b in range(B) if smask[b]))
    else:
        draft_rows = 0 if tree is not None else n_sampled * K
    step_bytes = gemm_bytes + M * V * 4 + draft_rows * V * 4 + n_sampled * 2 * V * 4
    step_roof = {"algorithmic_bytes": step_bytes, "frac_hbm": step_bytes / step_s / (HBM_PEAK_GBS * 1e9),
                 "fused_minimal_bytes": step_bytes - M * V * 4,
                 "frac_hbm_fused_minimal": (step_bytes - M * V * 4) / step_s / (HBM_PEAK_GBS * 1e9)}

    positions = M
    res = {
        "metric": METRIC,
        "value": positions / step_s,
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": n_warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "K": K, "H": H, "V": V, "temperature": T,
                   "sampled_rows": int(smask.sum()), "greedy_rows": int((~smask).sum())},
        **({"verify_rows": M, "draft_counts": "K_b ~ U{0..%d}, packed" % K} if row_start is not None else {}),
        **({"tree_nodes": K, "mean_kept_depth": float(np.mean(accepted))} if tree is not None else {}),
        "verify_step_us": step_s * 1e6,
        "path": ("spec_tree_verify_step" if tree is not None else
                 "spec_verify_step_ragged" if row_start is not None else "spec_verify_step") if step_ws is not None
                else "separate calls",
        "step_us_median": float(np.median(step_us)),
        "step_us_p90": float(np.percentile(step_us, 90)),
        "committed_tokens_per_s": float(np.mean(committed / (step_us * 1e-6))),
        "step_roofline": step_roof,
        # the whole step's fraction of HBM peak (algorithmic bytes of the
        # step / step time); "roofline" below is the dominant kernel alone
        "headline_frac": step_roof["frac_hbm"],
        "roofline": roof,
    }

    # further rounds, untimed, with their outputs kept: the acceptance rate
    # by draft position, and the rounds the CPU leg checks against the oracle
    rec = None
    if record_rounds and tree is None and row_start is None:
        # each recorded round draws its own drafts (the timed steps cycle
        # through n_sets pre-drawn sets, which would tie the acceptance rates
        # to those few draws)
        r0 = n_warmup + n_steps
        rec_acc = torch.empty((record_rounds, B), dtype=torch.int32, device=dev)
        rec_out = torch.empty((record_rounds,) + tuple(out.shape), dtype=torch.int32, device=dev)
        rec_d = []
        for k in range(record_rounds):
            d = synth.draft_tokens(zd, smask, T, seed=wl.data_seed * 104729 + r0 + k)
            rec_d.append(d)
            drafts[(r0 + k) % n_sets] = d
            step(r0 + k)
            rec_acc[k].copy_(acc)
            rec_out[k].copy_(out)
        torch.cuda.synchronize()
        rec = dict(first_round=r0, acc=rec_acc.cpu().numpy(), out=rec_out.cpu().numpy(),
                   drafts=[d.cpu().numpy() for d in rec_d],
                   seeds=[synth.seeds(wl, r0 + k) for k in range(record_rounds)])
        s_rows = np.nonzero(smask)[0]
        if len(s_rows):
            n = rec["acc"][:, s_rows].reshape(-1)
            res["accept_by_position"] = [
                {"position": i, "reached": int((n >= i).sum()), "accepted": int((n > i).sum()),
                 "rate": float((n > i).sum() / max(1, (n >= i).sum()))} for i in range(K)]

    if cpu:
        rs_np = None if row_start is None else row_start.cpu().numpy()
        par_np = None if tree is None else tree[0].cpu().numpy()
        res["cpu_baseline"] = cpu_baseline(wl, W, hidden, zd, drafts, smask, args.cpu_seconds, rs_np, par_np, rec,
                                           res.get("accept_by_position"))
    return res




NEAR_TIE = 1e-4   # the stated rule: a decision whose margin is below this may differ


def _count_decisions(tally, kind, margins, same_upto, n_cmp):
    """One sequence's decisions of one kind: margins in order, the first
    differing decision index (or None); counts decisions, near-ties, flips
    (a difference at a near-tie; the sequence stops there) and violations
    (a difference at a clear margin)."""
    t = tally.setdefault(kind, {"decisions": 0, "near_ties": 0, "flips": 0, "violations": 0})
    for i in range(n_cmp):
        m = float(margins[i])
        t["decisions"] += 1
        t["near_ties"] += int(m < NEAR_TIE)
        if same_upto is not None and i == same_upto:
            t["flips" if m < NEAR_TIE else "violations"] += 1
            return True
    return False


def _parity_round(tally, og, os_, g_rows, s_rows, acc, out):
    """The GPU's outputs of one round against the oracle's (end to end: the
    oracle's own fp64 logits), per decision type."""
    K = out.shape[1] - 1
    if og is not None:
        for b in g_rows:
            o_n, g_n = int(og.accepted_len[b]), int(acc[b])
            first = None
            for i in range(min(o_n, g_n) + 1):
                if out[b, i] != og.out_tokens[b, i] or (i < o_n) != (i < g_n):
                    first = i
                    break
            _count_decisions(tally, "greedy", og.margin[b], first, (first + 1) if first is not None else o_n + 1)
    if os_ is not None:
        for b in s_rows:
            o_n, g_n = int(os_.accepted_len[b]), int(acc[b])
            if o_n < 0 or g_n < 0:
                t = tally.setdefault("faulted", {"both": 0, "one_side": 0})
                t["both" if o_n == g_n else "one_side"] += 1
                continue
            n_acc = min(o_n, K - 1) + 1 if K else 0
            first = None
            for i in range(n_acc):
                if (i < o_n) != (i < g_n):
                    first = i
                    break
                if i >= o_n:
                    break
            if _count_decisions(tally, "accept", os_.accept_margin[b], first,
                                (first + 1) if first is not None else min(n_acc, o_n + 1)):
                continue
            same = out[b, o_n] == os_.out_tokens[b, o_n]
            _count_decisions(tally, "terminal", [os_.terminal_margin[b]], None if same else 0, 1)


def cpu_baseline(wl, W, hidden, zd, drafts, smask, budget_s, rs=None, parents=None, rec=None, by_pos=None):
    """The oracle, as it stands, timed on this host on the same inputs: whole
    verify steps (fp64 logits of all K+1 positions + acceptance) until about
    budget_s seconds have been spent (at least one step).  With rec (rounds
    the GPU ran, outputs kept) the oracle takes those rounds, and its results
    are compared with the GPU's decision by decision under the stated 1e-4
    rule (near-ties and flips per decision type, end to end), and the
    oracle's acceptance probability alpha_i = sum_v min(q_i, p_i) is added to
    by_pos."""
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    cores = min(len(os.sched_getaffinity(0)), 16)
    print("bench: cpu baseline (oracle) on %d threads" % cores, file=sys.stderr, flush=True)
    w64 = oracle.widen_bf16(W.cpu().view(torch.int16).numpy().view(np.uint16)) if wl.dtype == "bf16" \
        else W.cpu().double().numpy()
    h = hidden.cpu()
    M = wl.M if rs is None else int(rs[-1])
    h64 = (oracle.widen_bf16(h.view(torch.int16).numpy().view(np.uint16)) if wl.dtype == "bf16"
           else h.double().numpy()).reshape(M, wl.H)
    zd64 = zd.cpu().numpy()
    ds = [d.cpu().numpy() for d in drafts]
    g_rows = np.nonzero(~smask)[0]
    s_rows = np.nonzero(smask)[0]
    times, t_logits = [], []
    tally, alphas = {}, []
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        t_start = time.perf_counter()
        r = 0
        while True:
            t0 = time.perf_counter()
            z = oracle.lm_head_logits(h64, w64)
            t_logits.append(time.perf_counter() - t0)
            if rec is not None:
                d, sd = rec["drafts"][r % len(rec["drafts"])], rec["seeds"][r % len(rec["seeds"])]
            else:
                d, sd = ds[r % len(ds)], synth_seeds(wl, r)
            og = os_ = None
            if parents is not None:
                oracle.tree_accept_greedy(z.reshape(wl.B, wl.K + 1, wl.V), parents, d)
            elif rs is not None:
                if len(g_rows):
                    oracle.accept_greedy_ragged(z, d, rs, wl.K, rows=g_rows)
                if len(s_rows):
                    oracle.accept_sample_ragged(z, zd64, d, rs, wl.K, wl.temperature, sd, rows=s_rows)
            else:
                z = z.reshape(wl.B, wl.K + 1, wl.V)
                if len(g_rows):
                    og = oracle.accept_greedy(z, d, rows=g_rows)
                if len(s_rows):
                    os_ = oracle.accept_sample(z, zd64, d, wl.temperature, sd, rows=s_rows)
            times.append(time.perf_counter() - t0)
            if rec is not None and r < len(rec["acc"]):
                _parity_round(tally, og, os_, g_rows, s_rows, rec["acc"][r], rec["out"][r])
                if os_ is not None:
                    alphas.append(os_.alpha[s_rows])
            r += 1
            if time.perf_counter() - t_start > budget_s:
                break
    t = float(np.mean(times))
    tl = float(np.mean(t_logits))
    out = {"value": M / t, "unit": "verified positions/s", "cores": int(min(used, cores)), "kind": "oracle",
           "logits_s_per_step": tl, "accept_s_per_step": t - tl,
           "sample": "%d whole verify steps of %s (fp64 logits of all %d positions over V=%d, then acceptance), "
                     "same inputs as the GPU run; %.2f s per step" % (len(times), wl.name, M, wl.V, t)}
    if tally:
        out["parity"] = dict(rounds=min(len(times), len(rec["acc"])), mode="end to end (the oracle's fp64 logits)",
                             rule="a decision may differ only below a margin of %g" % NEAR_TIE, **tally)
    if alphas and by_pos is not None:
        a = np.concatenate(alphas).reshape(-1, wl.K).mean(axis=0)
        for x in by_pos:
            x["alpha"] = float(a[x["position"]])
    return out


def bench_ngram(args, dev, wl, cpu=True, steps=50):
    """The prompt-lookup drafter on its own: one step = one
    spec_ngram_propose call over every history of the workload."""
    import torch

    import speculative_decoding_verification_02_amd as sv
    import synth

    print("bench: %s, generating histories" % wl.name, file=sys.stderr, flush=True)
    hist = synth.histories(wl.B, wl.L, wl.V, wl.data_seed, wl.copy_frac)
    starts = np.concatenate([[0], np.cumsum([len(h) for h in hist])]).astype(np.int64)
    n_tok = int(starts[-1])
    flat = torch.from_numpy(np.concatenate(hist).astype(np.int32)).to(dev)
    hs = torch.from_numpy(starts).to(dev)
    # copies of the history set, rotated between calls, more bytes in all than
    # the 256 MB last-level cache holds: each call reads its histories from HBM
    set_bytes = n_tok * 4
    n_copies = max(2, -(-(384 << 20) // set_bytes))
    copies = [flat] + [flat.clone() for _ in range(n_copies - 1)]
    max_len = max(len(h) for h in hist)
    drafts = torch.empty((wl.B, wl.n_drafts), dtype=torch.int32, device=dev)
    count = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    rs = torch.empty((wl.B + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty(sv.spec_ngram_workspace_bytes(wl.B, max_len), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        sv.spec_ngram_propose(copies[i % n_copies], hs, max_len, wl.max_ngram, wl.n_drafts, drafts, count, ws,
                              row_start=rs, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    call_ms = float(np.mean(call_us)) * 1e-3
    # algorithmic bytes: every history token read once, the drafts, counts
    # and offsets written once
    alg = n_tok * 4 + wl.B * (wl.n_drafts + 2) * 4 + (wl.B + 1) * 8
    roof = {"bound": "hbm", "achieved": alg / (call_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "kernel": "spec_ngram_propose (scan + finalize)", "traffic": None, "algorithmic_bytes": alg,
            "avg_call_us": call_ms * 1e3,
            "method": "history set of %.1f MB rotated over %d copies (%.0f MB in all, more than the 256 MB "
                      "last-level cache) between calls" % (set_bytes / 1e6, n_copies, n_copies * set_bytes / 1e6)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    res = {"metric": "history tokens scanned/s (prompt-lookup drafter)", "value": n_tok / step_s,
           "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "int32", "data": "synthetic",
           "config": {"workload": wl.name, "B": wl.B, "max_len": max_len, "tokens": n_tok, "V": wl.V,
                      "max_ngram": wl.max_ngram, "n_drafts": wl.n_drafts},
           "step_us_median": float(np.median(call_us)), "step_us_p90": float(np.percentile(call_us, 90)),
           "mean_drafts": float(count.float().mean().item()), "roofline": roof}
    if cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while n < wl.B:
            oracle.ngram_propose_one(hist[n], wl.n_drafts, wl.max_ngram)
            n += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        t = time.perf_counter() - t0
        scanned = sum(len(h) for h in hist[:n])
        res["cpu_baseline"] = {"value": scanned / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": "%d of the %d histories (%d tokens), one thread (numpy)" % (n, wl.B, scanned)}
    return res


def synth_seeds(wl, r):
    import synth
    return synth.seeds(wl, r)


if __name__ == "__main__":
    main()

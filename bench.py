"""Benchmark of the k-pool indexer selection on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload sq524288] [--overlap off|on]
                    [--kpool K] [--budget B] [--workspace-mib M] [--no-cpu-baseline]

One step is the whole path (pool the keys, score + select every row through
the 2 GiB chunk loop, expand to token ids) over the workload's rows, on
synthetic seeded inputs already resident in HBM.  By default one chunk buffer
holds at most 2 GiB of fp32 scores, the pages' cap, and chunks run one after
the other on one stream.  Prints ONE JSON line:

  value       visible (row, pool) scores per second of whole-path wall time
  ms_per_step selection wall time of one step
  roofline    the score kernel (the dominant kernel): algorithmic MFMA flops
              (2*H*D per visible pair) over its average launch time, against
              the 2.5 PFLOP/s dense bf16 peak.  Launch times come from HIP
              events that the library records around each launch on its
              stream, in a kernel pass of the same K steps run right after the
              timed region with every launch alone on one stream (with the
              chunk overlap on, overlapped launches share the CUs and their
              event spans would include the other stream's kernels)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
              workload's rows, extrapolated to the whole job by visible pairs
  probe_peaks what this machine reaches on plain work, measured after the kernel
              pass: a 1 GiB device-to-device copy (HBM) and a large bf16 GEMM
              through torch.matmul (the vendor BLAS), with the score and top-k
              rates as fractions of them beside the nominal-peak fractions

The pages' own figure for this workload (KPool selection at 512k tokens on
one B200, 21.07 s) is reported as context only.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PAGES_B200_SELECTION_S = {"sq524288": 21.07, "sq524288_slice": 2.63}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(cu, q_lo, q_hi, kpool):
    """Number of (row, pool) pairs with p*kpool <= t over rows [q_lo, q_hi)."""
    tot = 0
    for s in range(len(cu) - 1):
        a, b = max(q_lo, int(cu[s])), min(q_hi, int(cu[s + 1]))
        if a >= b:
            continue
        t0, t1 = a - int(cu[s]), b - int(cu[s])          # local positions [t0, t1)
        t = np.arange(t0, t1, dtype=np.int64)
        tot += int((t // kpool + 1).sum())
    return tot


def cpu_baseline(wl, inp, total_pairs, seed, budget_s=15.0):
    """Oracle on sampled rows of the same workload; rate extrapolated by visible pairs.

    The oracle reads the same seeded inputs (copied back from the device
    tensors the generator filled) and runs pool -> score -> select -> expand
    for each sampled row, as it stands.
    """
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 0) for d in threadpool_info()] or [cores])
    except Exception:
        threads = cores
    cu = np.asarray(inp["cu_seqlens"])
    lo, hi = wl.rows
    k = inp["k"].cpu().numpy().view(np.uint16)
    if wl.pooling == "gated":
        g = inp["g"].cpu().numpy().view(np.uint16)
        ape = inp["ape"].cpu().numpy()
        t0 = time.perf_counter()
        kp = oracle.pool_keys_gated(k, g, ape, cu, wl.kpool)
    else:
        t0 = time.perf_counter()
        kp = oracle.pool_keys(k, cu, wl.kpool)
    t_pool = time.perf_counter() - t0
    cu_pools, _ = oracle.count_pools(cu, wl.kpool)
    # 64 evenly spaced rows (always the first and last), then random rows until the time budget
    first = np.unique(np.linspace(lo, hi - 1, 64).astype(np.int64))
    extra = np.random.default_rng(seed).permutation(np.arange(lo, hi))[:8192]
    batches = [first] + [np.sort(extra[i:i + 32]) for i in range(0, len(extra), 32)]
    sample_pairs = nrows = 0
    t_rows = 0.0
    for batch in batches:
        idx = torch.from_numpy(batch).to(inp["q"].device)
        qs = inp["q"].index_select(0, idx).cpu().numpy().view(np.uint16)
        ws = inp["w"].index_select(0, idx).cpu().numpy()
        t1 = time.perf_counter()
        seq, t = oracle.row_positions(batch, cu)
        for i in range(len(batch)):
            sc = oracle.row_scores(qs[i:i + 1], ws[i:i + 1], kp, cu_pools, seq[i:i + 1], t[i:i + 1],
                                   wl.kpool)
            n = int(t[i] // wl.kpool + 1)
            ids = oracle.select_row(sc[0, :n], wl.budget)
            oracle.expand_row(ids, int(t[i]), wl.kpool)
            sample_pairs += n
        t_rows += time.perf_counter() - t1
        nrows += len(batch)
        if t_rows + t_pool >= budget_s:
            break
    est_full_s = t_pool + t_rows * (total_pairs / max(sample_pairs, 1))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": total_pairs / est_full_s,
        "unit": "scores/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{nrows} rows of {wl.name} (64 evenly spaced incl. first and last, then random), "
                   f"{sample_pairs} visible pairs scored, selected and expanded in {t_rows:.1f} s, "
                   f"plus pooling all {wl.T} keys in {t_pool:.1f} s; whole-job time extrapolated "
                   f"by visible pairs = {est_full_s:.0f} s; host {cpu_model or platform.processor()}, "
                   f"{cores} cores visible, BLAS threads {threads}"),
    }


def probe_peaks(reps: int = 10):
    """Achievable rates on this machine: HBM by a plain device copy, bf16 MFMA by a GEMM.

    Both run after the timed region and the kernel pass, so they change nothing
    the bench line times.  The copy moves 1 GiB (read) + 1 GiB (write) per rep;
    the GEMM is [16384, 16384] x [16384, 16384] in bf16 with fp32 accumulation
    (2 * 16384^3 flop per rep), both operands contiguous.
    """
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * a.numel() * 4 * reps / (e0.elapsed_time(e1) / 1000.0) / 1e9
    del a, b
    n = 16384  # (of 4096, 8192, 12288, 16384 the fastest on this chip)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    y = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    z = torch.matmul(x, y)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        z = torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) / 1000.0) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": copy_gbs, "bf16_gemm_TFLOPs": gemm_tflops,
            "how": (f"{reps} x 1 GiB device-to-device copy (2 GiB moved each); {reps} x "
                    f"torch.matmul bf16 [{n},{n}] x [{n},{n}]; HIP events")}


COUNTER_SOURCES = ("score.hip", "topk.hip", "api.hip")


def committed_counters(workload: str):
    """Per-launch counter figures from the committed summary profiles/counters_<workload>.md.

    The summary holds, per kernel, the FETCH_SIZE / WRITE_SIZE bytes per launch
    (scaled by a plain-copy calibration) and the score kernel's MFMA-busy share,
    from rocprofv3 --pmc runs of this script, together with the sha256 of the
    sources they were measured on (score.hip, topk.hip and api.hip, which plans
    the launches; the score kernel's cache policy also decides what the top-k
    finds in the caches).  Any changed source makes the figures stale: None.
    """
    import hashlib
    prof = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    csrc = os.path.join(ROOT, "pool_score_top_amd", "csrc")
    if not os.path.exists(prof):
        return None
    vals = {}
    for line in open(prof):
        line = line.strip()
        if ":" in line and line.split(":", 1)[0].startswith(("sha256_", "score_", "topk_")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    for name in COUNTER_SOURCES:
        sha = hashlib.sha256(open(os.path.join(csrc, name), "rb").read()).hexdigest()
        if vals.get(f"sha256_{name}") != sha:
            return None
    try:
        return {k: float(v) for k, v in vals.items() if not k.startswith("sha256_")}
    except ValueError:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="sq524288")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kpool", type=int, default=None,
                    help="override the workload's pool size (the workload is then named "
                         "<workload>_kpool<K>_budget<B>)")
    ap.add_argument("--budget", type=int, default=None,
                    help="override the workload's pools kept per row (1..2048)")
    ap.add_argument("--overlap", choices=("on", "off"), default="off",
                    help="chunk overlap in the timed region: on = two chunk buffers of up to 2 GiB "
                         "each on two streams (KPOOL_FLAG_OVERLAP); off (default) = one chunk "
                         "buffer, so all fp32 scores in flight stay within the 2 GiB cap")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workspace-mib", type=int, default=None,
                    help="cap the score workspace (default: one 2 GiB chunk buffer, two with "
                         "--overlap on); smaller workspaces mean shorter chunks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 4 times (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 4 x 1 GiB device copies")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the selection would "
              "shard by query rows with one int32 all-gather; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from pool_score_top_amd import kpool as K
    from pool_score_top_amd import synth

    over = {k: v for k, v in (("kpool", args.kpool), ("budget", args.budget)) if v is not None}
    wl = synth.workload(args.workload, **over)
    if over:
        wl = synth.Workload(**{**wl.__dict__,
                               "name": f"{args.workload}_kpool{wl.kpool}_budget{wl.budget}"})
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {wl.name} inputs (T={wl.T}, H={wl.H}, D={wl.D})")
    t0 = time.time()
    inp = synth.device_inputs(wl, args.seed, device=dev)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    cu = inp["cu_seqlens"]
    q_lo, q_hi = wl.rows
    overlap = args.overlap == "on"
    sel = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D, device=dev, q_lo=q_lo, q_hi=q_hi,
                     workspace_cap=None if args.workspace_mib is None else args.workspace_mib << 20,
                     overlap=overlap)
    pairs = visible_pairs(cu, q_lo, q_hi, wl.kpool)
    flops = 2.0 * wl.H * wl.D * pairs

    for i in range(args.warmup):
        sel.run(inp["q"], inp["k"], inp["w"], g=inp.get("g"), ape=inp.get("ape"))
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i} done")

    # timed region: K whole steps, nothing else on the GPU.  Events on the stream the
    # steps run on (the library joins its helper stream back into it) split the region
    # into steps without a synchronization inside it.
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ev[0].record()
    for i in range(args.steps):
        sel.run(inp["q"], inp["k"], inp["w"], g=inp.get("g"), ape=inp.get("ape"))
        step_ev[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1000.0 * elapsed / args.steps
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)]
    log(f"[bench] {args.steps} steps, {ms_step:.2f} ms/step (overlap {args.overlap})")

    # kernel pass: the same steps with every launch alone on one stream (flags = 0; the
    # same workspace gives the same chunks), each bracketed by HIP events on that stream
    K.profile_enable(True)
    K.profile_collect()  # reset
    torch.cuda.synchronize()
    tk = time.perf_counter()
    for i in range(args.steps):
        sel.run(inp["q"], inp["k"], inp["w"], overlap=False, g=inp.get("g"), ape=inp.get("ape"))
    torch.cuda.synchronize()
    ms_serial = 1000.0 * (time.perf_counter() - tk) / args.steps
    prof = K.profile_collect()
    K.profile_enable(False)
    log(f"[bench] kernel pass: {args.steps} steps, {ms_serial:.2f} ms/step (overlap off, events on)")

    score_ms, score_n = prof["score"]
    topk_ms, topk_n = prof["topk"]
    pool_ms, _ = prof["pool_keys"]
    exp_ms, _ = prof["expand"]
    S = args.steps
    rows = q_hi - q_lo
    score_tflops = flops * S / (score_ms / 1000.0) / 1e12
    topk_bytes = 4.0 * pairs + 4.0 * wl.budget * rows
    topk_gbs = topk_bytes * S / (topk_ms / 1000.0) / 1e9
    exp_bytes = 4.0 * wl.budget * rows * (1 + wl.kpool)
    exp_gbs = exp_bytes * S / (exp_ms / 1000.0) / 1e9 if exp_ms > 0 else 0.0
    # keys (and, for the gated pooling, gate scores) read once, pooled keys written once
    pool_bytes = (4.0 if wl.pooling == "gated" else 2.0) * wl.T * wl.D + 2.0 * sel.P_tot * wl.D
    pool_gbs = pool_bytes * S / (pool_ms / 1000.0) / 1e9 if pool_ms > 0 else 0.0

    cnt = committed_counters(wl.name)
    chunk_rows = sel.chunk_rows()
    nbuf = sel.chunk_buffers()
    pitch = ((sel.max_pools + 63) // 64) * 64    # (the fp32 score row pitch, for the byte counts)
    score_launch_ms = score_ms / max(1, score_n)
    topk_launch_ms = topk_ms / max(1, topk_n)
    topk = {"ms_per_step": topk_ms / S, "launches_per_step": topk_n // S,
            "avg_launch_ms": topk_launch_ms,
            # 4 B per visible pair plus the ids, over the top-k time: the rate of a full
            # scan.  The group-pruned kernel skips most of those bytes, so this is not an
            # HBM rate and may exceed the peak.
            "gbs_if_every_score_were_read": topk_gbs,
            "frac_if_every_score_were_read": topk_gbs / PEAK_HBM_GBS}
    if cnt is not None and "topk_fetch_bytes_per_launch" in cnt:
        tb = cnt["topk_fetch_bytes_per_launch"] + cnt["topk_write_bytes_per_launch"]
        topk.update({"traffic_bytes": tb,
                     "traffic_read": cnt["topk_fetch_bytes_per_launch"],
                     "traffic_write": cnt["topk_write_bytes_per_launch"],
                     "achieved_GBs": tb / (topk_launch_ms / 1000.0) / 1e9,
                     "peak_GBs": PEAK_HBM_GBS,
                     "frac": tb / (topk_launch_ms / 1000.0) / 1e9 / PEAK_HBM_GBS,
                     "how": ("HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE in the "
                             f"committed profiles/counters_{wl.name}.md (copy-calibrated, sources "
                             "hash-checked), over this run's average top-k launch time")})
    else:
        topk.update({"traffic_bytes": None, "achieved_GBs": None, "frac": None,
                     "how": f"no current counter summary for {wl.name} (profiles/counters_{wl.name}.md)"})
    score_traffic = None
    if cnt is not None and "score_fetch_bytes_per_launch" in cnt:
        score_traffic = (cnt["score_fetch_bytes_per_launch"], cnt["score_write_bytes_per_launch"])
    result = {
        "metric": "query-pool scores/s + selection wall time at 512k tokens, % MFMA/HBM peak",
        "value": pairs / (ms_step / 1000.0),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: {len(cu) - 1} sequence(s), {wl.T} tokens, rows [{q_lo}, {q_hi}), "
                         f"H={wl.H}, D={wl.D}, kpool={wl.kpool}, budget={wl.budget} pools, causal, "
                         f"{wl.pooling} pooling"),
            "tokens": wl.T, "rows": rows, "H": wl.H, "D": wl.D, "kpool": wl.kpool,
            "budget": wl.budget, "visible_pairs": pairs, "seed": args.seed, "pooling": wl.pooling,
            "score_chunk_rows": chunk_rows,
            "chunk_overlap": args.overlap,
            "workspace_bytes": sel.workspace_bytes,
            "chunk_buffers": nbuf,
            "score_bytes_per_chunk_buffer": chunk_rows * pitch * 4,
            "score_bytes_in_flight": nbuf * chunk_rows * pitch * 4,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "score_kernel<32,128>",
            "achieved": score_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": score_tflops / PEAK_BF16_TFLOPS,
            "traffic": None if score_traffic is None else sum(score_traffic),
            "traffic_unit": ("HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated), taken "
                             f"from the committed profiles/counters_{wl.name}.md, not measured in this "
                             "run; null when the sources changed since"),
            "traffic_read": None if score_traffic is None else score_traffic[0],
            "traffic_write": None if score_traffic is None else score_traffic[1],
            "mfma_busy_frac": None if cnt is None else cnt.get("score_mfma_busy_frac"),
            "mfma_busy_how": ("SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles the chip was active "
                              "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) during the score launches, from "
                              "the same committed counter summary"),
            "launches_per_step": score_n // S,
            "flops_per_launch": flops / max(1, score_n // S),
            "avg_launch_ms": score_launch_ms,
            "measured": ("HIP events around each launch on its stream, kernel pass of the same "
                         "steps with flags = 0 (every launch alone on one stream)"),
        },
        "step_ms": {"median": float(np.median(step_ms)), "min": float(min(step_ms)),
                    "max": float(max(step_ms)), "how": "HIP events between the timed steps"},
        "kernel_pass_ms_per_step": ms_serial,
        "kernels": {
            "score": {"ms_per_step": score_ms / S, "tflops": score_tflops,
                      "mfma_frac": score_tflops / PEAK_BF16_TFLOPS},
            "topk": topk,
            "pool_keys": {"ms_per_step": pool_ms / S, "gbs": pool_gbs},
            "expand": {"ms_per_step": exp_ms / S, "gbs": exp_gbs},
        },
        "pages_context": {
            "b200_selection_s": PAGES_B200_SELECTION_S.get(wl.name),
            "ratio_b200_time_over_ours": (PAGES_B200_SELECTION_S[wl.name] / (ms_step / 1000.0)
                                          if wl.name in PAGES_B200_SELECTION_S else None),
        },
    }
    pk = probe_peaks()
    pk["score_frac_of_gemm"] = score_tflops / pk["bf16_gemm_TFLOPs"]
    if topk.get("achieved_GBs"):
        pk["topk_frac_of_copy"] = topk["achieved_GBs"] / pk["hbm_copy_GBs"]
    result["probe_peaks"] = pk
    log(f"[bench] probes: copy {pk['hbm_copy_GBs']:.0f} GB/s, bf16 GEMM {pk['bf16_gemm_TFLOPs']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        result["cpu_baseline"] = cpu_baseline(wl, inp, pairs, args.seed, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

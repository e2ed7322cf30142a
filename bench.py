"""Benchmark of the verify-and-sample hot path on one MI355X.

Default workload: greedy verify + MTP shift/insert at B=256
sequences, n=4 drafts, V=128256 bf16 logits, hidden size 8192.  One step =
spec_verify_greedy_mtp(): the verification of the [256, 5, 128256] target
logits with the shift/insert of the [256, 5] token buffer and the carry of the
[256, 5, 8192] hidden states fused in (--unfused: spec_verify_greedy() then
mtp_shift_insert(), two launches).  Inputs are synthetic (seeded), resident in HBM, and rotate over
several independent copies so that no step finds its inputs in the 256 MB
last-level cache.

Prints one JSON line: verified vocab rows/s (value), HBM GB/s and % of the
8 TB/s peak, a roofline entry for the dominant kernel (the verify kernel,
timed with HIP events on its stream), and the CPU oracle timed on host cores.

    python bench.py [--steps K] [--warmup W] [--config {1,...,6}] [--no-cpu] [--unfused]
    python bench.py --lmhead [--steps K]   # greedy verify fused with the logit projection
    python bench.py --tree | --tree-sample  # greedy / sampling tree verification
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "draft_token_verification_08_amd", "csrc", "sv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--seed", type=int, default=303)
    ap.add_argument("--draft-stats", action="store_true",
                    help="sampling configs: feed the draft rows' statistics from the draft's sampling step "
                         "(spec_verify_sample_ex) instead of streaming the draft rows")
    ap.add_argument("--unfused", action="store_true",
                    help="separate verify and mtp_shift_insert calls instead of the fused call")
    ap.add_argument("--graph", action="store_true",
                    help="capture each input copy's step into a HIP graph and time graph replays")
    ap.add_argument("--draft-step", action="store_true",
                    help="the draft loop's per-step sampling (sv_sample_rows with row statistics): one token per "
                         "sequence from logits [256, 128256] bf16 at T=0.7")
    ap.add_argument("--tree", action="store_true",
                    help="greedy tree verification (spec_verify_tree_greedy): 64 sequences with a 26-node top-k "
                         "draft tree over V=128256 bf16 logits")
    ap.add_argument("--tree-sample", action="store_true",
                    help="sampling tree verification (spec_verify_tree_sample): 64 sequences with a 26-node top-k "
                         "draft tree over V=128256 bf16 target and draft logits, T=0.7")
    ap.add_argument("--lmhead", action="store_true",
                    help="greedy verify fused with the target's logit projection (spec_verify_greedy_lmhead): "
                         "hidden states [256, 5, 8192] and a [128256, 8192] projection instead of logits")
    return ap.parse_args()


LMHEAD_SRC = os.path.join(ROOT, "draft_token_verification_08_amd", "csrc", "sv_lmhead.hip")


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, src: str = KERNEL_SRC):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    only if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{kernel}|{workload}")
    if not e or e.get("source_sha256_16") != kernel_source_hash(src):
        return None
    return e.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sequences shard "
              "across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_token_verification_08_amd as sv
    from draft_token_verification_08_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.lmhead:
        bench_lmhead(args, dev)
        return
    if args.draft_step:
        bench_draft_step(args, dev)
        return
    if args.tree:
        bench_tree(args, dev)
        return
    if args.tree_sample:
        bench_tree_sample(args, dev)
        return
    cfg = synth.CONFIGS[args.config]
    greedy = cfg.mode == "greedy"
    es = 2 if cfg.dtype == torch.bfloat16 else 4

    # ---------------------------------------------------------------- inputs
    one = cfg.B * (cfg.n + 1) * cfg.V * es * (1 if greedy else 2) + 2 * cfg.B * (cfg.n + 1) * cfg.H * 2
    sets = args.sets or max(2, min(8, int(np.ceil(1.2e9 / one))))
    data = []
    for i in range(sets):
        d = synth.make(args.config, args.seed + i, device=dev)
        d["hidden_dst"] = torch.empty_like(d["hidden"]) if cfg.H else None
        d["tokens0"] = d["tokens"].clone()
        d["acc"] = torch.empty(cfg.B, dtype=torch.int32, device=dev)
        d["emi"] = torch.empty((cfg.B, cfg.n + 1), dtype=torch.int32, device=dev)
        data.append(d)
    torch.cuda.synchronize()
    ws = sv.Workspace(dev)
    wsbuf = ws.get(sv.sv_workspace_bytes(cfg.B, cfg.n, cfg.V, sv.SV_BF16 if es == 2 else sv.SV_F32))
    stream = torch.cuda.current_stream(dev)

    # calls marshalled once per input copy (the C entry points are re-issued as is);
    # with --graph they are bound to the capture stream and captured below
    cap = torch.cuda.Stream(dev) if args.graph else None
    fused = bool(cfg.H) and not args.unfused
    dstats = args.draft_stats and not greedy
    for d in data:
        if dstats:
            # the draft's sampling step computes these; it is not part of the timed step
            d["dstats"] = sv.draft_row_stats(d["draft"], d["temperature"])
            d["verify"] = sv.prepare_spec_verify_sample_ex(
                d["target"], d["draft"], d["draft_tokens"], d["draft_lens"], d["temperature"], d["uniforms"],
                d["acc"], d["emi"], wsbuf, draft_stats=d["dstats"], tokens=d["tokens"] if fused else None,
                hidden_src=d["hidden"] if fused else None, hidden_dst=d["hidden_dst"] if fused else None,
                stream=cap)
            d["mtp"] = (lambda: None) if fused or not cfg.H else sv.prepare_mtp_shift_insert(
                d["tokens"], d["hidden"], d["hidden_dst"], d["acc"], d["emi"], stream=cap)
            continue
        if fused:
            if greedy:
                d["verify"] = sv.prepare_spec_verify_greedy_mtp(d["target"], d["draft_tokens"], d["draft_lens"],
                                                                d["acc"], d["emi"], d["tokens"], d["hidden"],
                                                                d["hidden_dst"], wsbuf, stream=cap)
            else:
                d["verify"] = sv.prepare_spec_verify_sample_mtp(d["target"], d["draft"], d["draft_tokens"],
                                                                d["draft_lens"], d["temperature"], d["uniforms"],
                                                                d["acc"], d["emi"], d["tokens"], d["hidden"],
                                                                d["hidden_dst"], wsbuf, stream=cap)
            d["mtp"] = lambda: None
            continue
        if greedy:
            d["verify"] = sv.prepare_spec_verify_greedy(d["target"], d["draft_tokens"], d["draft_lens"], d["acc"],
                                                        d["emi"], wsbuf, stream=cap)
        else:
            d["verify"] = sv.prepare_spec_verify_sample(d["target"], d["draft"], d["draft_tokens"], d["draft_lens"],
                                                        d["temperature"], d["uniforms"], d["acc"], d["emi"], wsbuf,
                                                        stream=cap)
        d["mtp"] = (sv.prepare_mtp_shift_insert(d["tokens"], d["hidden"], d["hidden_dst"], d["acc"], d["emi"],
                                                stream=cap)
                    if cfg.H else (lambda: None))

    if args.graph:
        # one graph per input copy holding the whole step; replays run on the
        # launch stream
        cap.wait_stream(stream)
        for d in data:
            d["verify"]()
            d["mtp"]()
        torch.cuda.synchronize()
        for d in data:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                d["verify"]()
                d["mtp"]()
            d["graph"] = g
            d["verify"] = g.replay
            d["mtp"] = lambda: None
        torch.cuda.synchronize()

    def verify(d):
        d["verify"]()

    def mtp(d):
        d["mtp"]()

    # algorithmic bytes per step (each required row counted once)
    lens = [d["draft_lens"].clamp(0, cfg.n).to(torch.int64) for d in data]
    temps = [d["temperature"] for d in data]
    rows_t = [int((L + 1).sum()) for L in lens]
    rows_d = [0 if greedy else int((L * (t > 0).to(torch.int64)).sum()) for L, t in zip(lens, temps)]
    side = cfg.B * cfg.n * 4 + cfg.B * 4 + cfg.B * 4 + cfg.B * (cfg.n + 1) * 4
    if not greedy:
        side += cfg.B * 4 + cfg.B * (cfg.n + 1) * 4
    rows_verified = [rt + rd for rt, rd in zip(rows_t, rows_d)]
    if dstats:
        # draft rows are not streamed: their statistics (8 B per row) and one
        # gathered logit per test are read instead
        side += cfg.B * cfg.n * 8
        verify_bytes_extra = [rd * es for rd in rows_d]
        rows_d = [0 for _ in rows_d]
    else:
        verify_bytes_extra = [0 for _ in rows_d]
    verify_bytes = [(rt + rd) * cfg.V * es + side + x for rt, rd, x in zip(rows_t, rows_d, verify_bytes_extra)]
    mtp_bytes = (2 * cfg.B * (cfg.n + 1) * cfg.H * 2 + 2 * cfg.B * (cfg.n + 1) * 4 + cfg.B * 4
                 + cfg.B * (cfg.n + 1) * 4) if cfg.H else 0
    # rows streamed by the step (with the draft's statistics the draft rows are not)
    rows_per_step = rows_t if dstats else rows_verified

    # ---------------------------------------------------------------- warmup
    for i in range(args.warmup):
        d = data[i % sets]
        verify(d)
        mtp(d)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # HIP events on the launch stream.  An event pair costs a few microseconds of
    # queue time, so when the step is one call (the fused step, or a verify with
    # no MTP), one pair brackets RUN consecutive steps in every 2*RUN and the
    # launch time is the bracket over RUN; with a separate MTP call, pairs bracket
    # the verify launch of every 8th step and the MTP launch of every 8th step
    # (offset 4).
    K = args.steps
    EVERY = 8
    single = args.graph or not (cfg.H and not fused)
    RUN = 8 if single and K >= 8 else 1
    starts = range(0, K - RUN + 1, 2 * RUN) if single else range(0, K, EVERY)
    ev_v = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in starts}
    ends = {i + RUN - 1: i for i in ev_v}
    ev_m = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for i in range(EVERY // 2, K, EVERY)} if not single else {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        d = data[i % sets]
        e = ev_v.get(i)
        if e:
            e[0].record(stream)
        verify(d)
        if i in ends:
            ev_v[ends[i]][1].record(stream)
        e = ev_m.get(i)
        if e:
            e[0].record(stream)
        mtp(d)
        if e:
            e[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    verify_ms = [a.elapsed_time(b) / RUN for a, b in ev_v.values()]
    mtp_ms = [a.elapsed_time(b) for a, b in ev_m.values()] or [0.0]
    ms_per_step = elapsed * 1e3 / K
    rows_total = sum(rows_per_step[i % sets] for i in range(K))
    step_mtp_bytes = (2 * cfg.B * (cfg.n + 1) * cfg.H * 2 + 2 * cfg.B * (cfg.n + 1) * 4) if fused else mtp_bytes
    bytes_total = sum(verify_bytes[i % sets] + step_mtp_bytes for i in range(K))
    value = rows_total / elapsed
    gbps = bytes_total / elapsed / 1e9
    v_avg_ms = statistics.fmean(verify_ms)
    # fused: the hidden states and the token buffer cross HBM once each way (the
    # verify outputs are not read back)
    fused_mtp_bytes = 2 * cfg.B * (cfg.n + 1) * cfg.H * 2 + 2 * cfg.B * (cfg.n + 1) * 4
    # a graph of an unfused step holds the MTP launch too
    step_extra = fused_mtp_bytes if fused else (mtp_bytes if args.graph else 0)
    v_bytes = statistics.fmean(verify_bytes[(i + r) % sets] + step_extra for i in ev_v for r in range(RUN))
    v_gbps = v_bytes / (v_avg_ms * 1e-3) / 1e9
    m_avg_ms = statistics.fmean(mtp_ms) if cfg.H and not fused else 0.0
    mean_acc = float(torch.stack([d["acc"].float().mean() for d in data]).mean())

    # a bare event pair on the same stream: the queue time an event pair adds to
    # each bracketed launch (reported, not subtracted)
    bare = []
    for _ in range(20):
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b2.record(stream)
        bare.append((a, b2))
    torch.cuda.synchronize()
    event_pair_us = statistics.median(a.elapsed_time(b2) for a, b2 in bare) * 1e3

    # attainable-bandwidth reference on the same box: a 1 GiB device-to-device
    # copy (read + write bytes over its event time, median of 10)
    src_c = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst_c = torch.empty_like(src_c)
    dst_c.copy_(src_c)
    torch.cuda.synchronize()
    cps = []
    for _ in range(10):
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst_c.copy_(src_c)
        b2.record(stream)
        torch.cuda.synchronize()
        cps.append(2 * (1 << 30) / (a.elapsed_time(b2) * 1e-3) / 1e9)
    copy_gbps = statistics.median(cps)
    del src_c, dst_c

    kernel = (("k_stats_greedy" if greedy else "k_stats_sample+k_draw") + ("+draft_stats" if dstats else "")
              + ("+mtp_fused" if fused else ""))
    workload = cfg.name
    traffic = measured_traffic(kernel, workload) if not (args.graph and cfg.H and not fused) else None

    out = {
        "metric": "verified vocab rows/s + HBM GB/s (% of peak), V=128256 bf16, B=256, n=4",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if es == 2 else "f32",
        "data": "synthetic (seeded; inputs resident in HBM, rotated over %d copies)" % sets,
        "config": {"workload": ("greedy verify" if greedy else "sampling verify")
                   + (" with the draft's row statistics" if dstats else "")
                   + (" + MTP shift/insert" + (" (fused call)" if fused else " (two calls)") if cfg.H else "")
                   + (", replayed from a HIP graph" if args.graph else "")
                   + f" ({cfg.name})", "B": cfg.B, "n": cfg.n, "V": cfg.V, "H": cfg.H,
                   "logits": "bf16" if es == 2 else "f32", "parallelism": "none (1 GPU)"},
        "hbm_gbps": round(gbps, 1),
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "verify_us": round(v_avg_ms * 1e3, 2),
        "mtp_us": round(m_avg_ms * 1e3, 2),
        "mean_accepted": round(mean_acc, 4),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(v_gbps, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(v_gbps / PEAK_GBPS, 4),
                     "bytes_per_launch": int(v_bytes), "avg_launch_us": round(v_avg_ms * 1e3, 2),
                     "timed_launches": len(verify_ms) * RUN,
                     "timing": (f"HIP event pair around {RUN} consecutive launches, every {2 * RUN} steps"
                                if RUN > 1 else "HIP event pair around the launch of every 8th step"),
                     "bare_event_pair_us": round(event_pair_us, 2),
                     "copy_1gib_gbps": round(copy_gbps, 1),
                     "traffic": traffic},
    }

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(data[0], cfg, greedy)
        out["oracle_parity"] = out["cpu_baseline"].pop("oracle_parity")
    print(json.dumps(out), flush=True)


NEAR_TIE = 1e-5  # decisions whose oracle margin is below this may differ (never greedy ones)


def parity_report(gpu_acc, gpu_emi, ora, L, T, n):
    """The GPU's decisions against the oracle's on the same inputs, sequence by
    sequence: tests 0..k in order, then the final token.  The first difference is
    allowed only at an oracle margin below NEAR_TIE (|u - p/q| for a test, the
    distance to the nearest CDF boundary over the mass for the draw) and is then
    counted as exempt; any other difference is a hard mismatch.  Sequences with
    T <= 0 are decided by the greedy rule and have no exemption."""
    import numpy as np

    am, dm = ora.get("accept_margin"), ora.get("draw_margin")
    r = {"sequences": int(len(gpu_acc)), "decisions": 0, "near_ties": 0, "exempt": 0, "hard_mismatches": 0}
    for b in range(len(gpu_acc)):
        Lb = int(min(max(int(L[b]), 0), n))
        greedy = not (T is not None and float(T[b]) > 0)
        kg, ko = int(gpu_acc[b]), int(ora["accepted_len"][b])
        tests = min(kg, ko) + (1 if min(kg, ko) < Lb else 0)
        r["decisions"] += tests + 1
        if not greedy and am is not None:
            r["near_ties"] += int((am[b, :min(tests, n)] < NEAR_TIE).sum()) + int(dm[b] < NEAR_TIE)
        if kg != ko:
            ok = not greedy and am is not None and am[b, min(kg, ko)] < NEAR_TIE
        elif not (np.array_equal(gpu_emi[b, :ko], ora["emitted"][b, :ko]) and (gpu_emi[b, ko + 1:] == -1).all()):
            ok = False
        elif gpu_emi[b, ko] != ora["emitted"][b, ko]:
            ok = not greedy and dm is not None and dm[b] < NEAR_TIE
        else:
            continue
        r["exempt" if ok else "hard_mismatches"] += 1
    return r


def cpu_baseline(d, cfg, greedy):
    """The oracle (plain C, double precision, untuned) on one full step of the same
    workload, on the host cores: single-threaded and with one thread per core of
    this process's CPU share (sequences split evenly)."""
    import numpy as np

    import oracle
    from draft_token_verification_08_amd import synth

    orc = oracle.Oracle()
    host = dict(target=synth.host_logits(d["target"]),
                draft=None if greedy else synth.host_logits(d["draft"]),
                x=d["draft_tokens"].cpu().numpy(), L=d["draft_lens"].cpu().numpy(),
                T=d["temperature"].cpu().numpy(), u=d["uniforms"].cpu().numpy(),
                tok=d["tokens0"].cpu().numpy(),
                hid=d["hidden"].cpu().view(__import__("torch").int16).numpy() if cfg.H else None)
    rows = int((np.clip(host["L"], 0, cfg.n) + 1).sum())
    if not greedy:
        rows += int((np.clip(host["L"], 0, cfg.n) * (host["T"] > 0)).sum())
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))

    def step(th):
        if greedy:
            o = orc.verify_greedy(host["target"], host["x"], host["L"], threads=th)
        else:
            o = orc.verify_sample(host["target"], host["draft"], host["x"], host["L"], host["T"], host["u"],
                                  threads=th)
        if cfg.H:
            orc.mtp_shift_insert(host["tok"], host["hid"], o["accepted_len"], o["emitted"])

    def timed(th, budget_s):
        # whole steps repeated until the wall-clock budget is used (at least 3)
        done, t0 = 0, time.perf_counter()
        while done < 3 or time.perf_counter() - t0 < budget_s:
            step(th)
            done += 1
        return (time.perf_counter() - t0) / done, done

    t1, n1 = timed(1, 2.0)
    tn, nn = timed(threads, 1.0)
    # the GPU's outputs for this input copy (left by the timed steps) against the oracle's
    if greedy:
        o = orc.verify_greedy(host["target"], host["x"], host["L"], threads=threads)
    else:
        o = orc.verify_sample(host["target"], host["draft"], host["x"], host["L"], host["T"], host["u"],
                              threads=threads)
    parity = parity_report(d["acc"].cpu().numpy(), d["emi"].cpu().numpy(), o, host["L"],
                           None if greedy else host["T"], cfg.n)
    parity["inputs"] = "the first input copy of the timed workload, whole batch"
    # the greedy oracle stops at a sequence's first mismatch: it reads acc + 1 of
    # the L + 1 rows the step verifies (the GPU reads all of them, in parallel)
    read = int((o["accepted_len"] + 1).sum()) if greedy else rows
    return {"value": round(rows / tn, 1), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "oracle_parity": parity,
            "sample": f"{nn} full steps ({cfg.B} sequences, {rows} rows of V={cfg.V} each"
                      + (", + MTP shift/hidden copy" if cfg.H else "") + f") on {threads} threads "
                      f"(this process's CPU share, at most 16), mean time per step over a 1 s budget, "
                      f"about {nn * tn * threads:.0f} s of CPU work; single thread: {n1} steps over 2 s"
                      + (f"; the oracle stops at each sequence's first mismatch and reads {read} of the "
                         f"{rows} rows (value = the step's rows / its time)" if greedy else ""),
            "rows_read_by_oracle": read,
            "single_thread_rows_per_s": round(rows / t1, 1), "seconds_per_step": round(tn, 4),
            "cpu_model": cpu_model()}


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def bench_lmhead(args, dev):
    """The greedy verify step on hidden states instead of logits: the projection
    hidden [B, n+1, H] x weight[V, H]^T runs on the matrix cores and each tile of
    logits is reduced to per-row argmax keys in registers; the decision and the
    MTP shift/insert (tokens and hidden-state carry) follow in the same call.
    Reported against the dense bf16 matrix-core peak, beside the library path
    (torch.matmul to bf16 logits, then spec_verify_greedy_mtp)."""
    import torch

    import draft_token_verification_08_amd as sv
    from draft_token_verification_08_amd import synth

    B, n, V, H = 256, 4, 128256, 8192
    M = B * (n + 1)
    d = synth.make_lmhead(args.seed, device=dev, B=B, n=n, V=V, H=H, exact=False)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    emi = torch.empty((B, n + 1), dtype=torch.int32, device=dev)
    tokens = d["tokens"].clone()
    hdst = torch.empty_like(d["hidden"])
    wsbuf = sv.Workspace(dev).get(sv.sv_workspace_bytes(B, n, V, sv.SV_BF16))
    stream = torch.cuda.current_stream(dev)
    call = sv.prepare_spec_verify_greedy_lmhead(d["hidden"], d["weight"], d["draft_tokens"], d["draft_lens"], acc,
                                                emi, wsbuf, tokens=tokens, hidden_dst=hdst)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in evs]
    avg_ms = statistics.fmean(step_ms)
    flops = 2.0 * M * V * H
    achieved = flops / (avg_ms * 1e-3) / 1e12

    # the library path on the same inputs: bf16 logits from the library GEMM,
    # then the fused logits verify + MTP call
    h2 = d["hidden"].view(M, H)
    wt = d["weight"]
    tok2 = d["tokens"].clone()
    hdst2 = torch.empty_like(d["hidden"])
    acc2 = torch.empty_like(acc)
    emi2 = torch.empty_like(emi)

    def library_step():
        z = torch.matmul(h2, wt.t())
        sv.spec_verify_greedy_mtp(z.view(B, n + 1, V), d["draft_tokens"], d["draft_lens"], tok2, d["hidden"], hdst2,
                                  accepted_len=acc2, emitted=emi2, workspace=wsbuf)

    for _ in range(3):
        library_step()
    torch.cuda.synchronize()
    lib_ms = []
    for _ in range(max(5, min(20, K))):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        library_step()
        b.record(stream)
        torch.cuda.synchronize()
        lib_ms.append(a.elapsed_time(b))
    lib_avg = statistics.fmean(lib_ms)
    # the library path decides on bf16-rounded logits, this one on the binary32
    # sums: they can differ where two top logits round to the same bf16 value
    same_seq = ((acc == acc2) & (emi == emi2).all(dim=1)).float().mean()

    out = {
        "metric": "verified vocab rows/s, V=128256 bf16, B=256, n=4 (greedy, logits from the lm_head projection)",
        "value": round(M * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 normals; hidden states and projection resident in HBM)",
        "config": {"workload": "greedy verify fused with the lm_head projection + MTP shift/insert "
                               f"(hidden [{B}, {n + 1}, {H}] x projection [{V}, {H}] bf16)",
                   "B": B, "n": n, "V": V, "H": H, "parallelism": "none (1 GPU)"},
        "step_us": round(avg_ms * 1e3, 1),
        "library_path_us": round(lib_avg * 1e3, 1),
        "library_path": "torch.matmul to bf16 logits + spec_verify_greedy_mtp",
        "speedup_vs_library_path": round(lib_avg / avg_ms, 4),
        "library_path_same_decisions_frac": round(float(same_seq), 4),
        "mean_accepted": round(float(acc.float().mean()), 4),
        "roofline": {"bound": "mfma", "kernel": "k_lmhead (+ k_decide_greedy)", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "flops_per_launch": flops, "avg_launch_us": round(avg_ms * 1e3, 1),
                     "timed_launches": K,
                     "timing": "HIP event pair around every step (the projection launch and the per-sequence "
                               "decision launch, about 3 us)",
                     "traffic": measured_traffic("k_lmhead", "greedy_lmhead_projection", LMHEAD_SRC),
                     "traffic_note": "HBM bytes per launch; the algorithmic minimum is the projection read "
                                     "once plus the hidden states (read, and written by the carry)"},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_lmhead(d, B, n, V, H)
    print(json.dumps(out), flush=True)


def bench_draft_step(args, dev):
    """The draft loop's per-step sampling: one token per sequence from its logits
    row at temperature T (sv_sample_rows), keeping the row statistics {max, sum}
    that the verify later takes instead of streaming the draft rows.  Inputs: the
    llama-vocab sampling recipe with no drafts, B=256, V=128256 bf16, T=0.7,
    resident in HBM and rotated over input copies larger than the MALL together."""
    import numpy as np
    import torch

    import draft_token_verification_08_amd as sv
    from draft_token_verification_08_amd import synth

    B, V = 256, 128256
    sets = args.sets or 8
    wsbuf = sv.Workspace(dev).get(sv.sv_workspace_bytes(B, 0, V, sv.SV_BF16))
    stream = torch.cuda.current_stream(dev)
    data, calls = [], []
    for i in range(sets):
        d = synth.make(6, args.seed + i, device=dev, n=0)
        d["u"] = d["uniforms"][:, 0].contiguous()
        d["tok"] = torch.empty(B, dtype=torch.int32, device=dev)
        d["stats"] = torch.empty((B, 2), dtype=torch.float32, device=dev)
        data.append(d)
        calls.append(sv.prepare_sv_sample_rows(d["target"], d["temperature"], d["u"], d["tok"], wsbuf,
                                               row_stats=d["stats"]))
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    for i in range(W):
        calls[i % sets]()
    torch.cuda.synchronize()
    # one event pair around 8 consecutive calls in every 16 steps
    brackets = []
    t0 = time.perf_counter()
    i = 0
    while i < K:
        if i % 16 == 0 and i + 8 <= K:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for j in range(8):
                calls[(i + j) % sets]()
            b.record(stream)
            brackets.append((a, b))
            i += 8
        else:
            calls[i % sets]()
            i += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_ms = statistics.fmean(a.elapsed_time(b) for a, b in brackets) / 8 if brackets else elapsed * 1e3 / K
    nbytes = B * V * 2 + B * (4 + 4 + 4 + 8)  # rows read once; temperature, uniform, token, statistics
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    out = {
        "metric": "sampled vocab rows/s + HBM GB/s (% of peak), V=128256 bf16, B=256 (draft-step sampling)",
        "value": round(B * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; inputs resident in HBM, rotated over {sets} copies)",
        "config": {"workload": "draft-step sampling with row statistics (sv_sample_rows), logits [256, 128256] "
                               "bf16, T=0.7 (draft_step_sampling)", "B": B, "V": V, "parallelism": "none (1 GPU)"},
        "hbm_gbps": round(nbytes * K / elapsed / 1e9, 1),
        "pct_of_peak": round(nbytes * K / elapsed / 1e9 / PEAK_GBPS * 100, 2),
        "roofline": {"bound": "hbm", "kernel": "k_stats_sample+k_draw (no drafts)", "achieved": round(achieved, 1),
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "bytes_per_launch": nbytes, "avg_launch_us": round(avg_ms * 1e3, 2),
                     "timed_launches": 8 * len(brackets),
                     "timing": "HIP event pair around 8 consecutive calls, every 16 steps",
                     "traffic": measured_traffic("k_stats_sample+k_draw", "draft_step_sampling")},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_draft_step(data[0], B, V)
        out["oracle_parity"] = out["cpu_baseline"].pop("oracle_parity")
    print(json.dumps(out), flush=True)


def bench_tree(args, dev):
    """Greedy tree verification: every sequence's target rows (one per tree node)
    reduced to argmax keys, then the tree walk.  64 sequences, each a 26-node
    top-k tree (3 children at the root, 2 below each of those, then chains) over
    V=128256 bf16 rows of the greedy logits recipe, resident in HBM and rotated
    over input copies."""
    import numpy as np
    import torch

    import draft_token_verification_08_amd as sv
    from draft_token_verification_08_amd import synth

    B, n, V = 64, 25, 128256
    sets = args.sets or 4
    wsbuf = sv.Workspace(dev).get(sv.sv_workspace_bytes(B, n, V, sv.SV_BF16))
    stream = torch.cuda.current_stream(dev)
    data = []
    for i in range(sets):
        d = synth.make_tree(args.seed + i, device=dev, B=B, n=n, V=V)
        d["acc"] = torch.empty(B, dtype=torch.int32, device=dev)
        d["emi"] = torch.empty((B, n + 1), dtype=torch.int32, device=dev)
        d["path"] = torch.empty((B, n), dtype=torch.int32, device=dev)
        data.append(d)
    torch.cuda.synchronize()

    for d in data:
        d["call"] = sv.prepare_spec_verify_tree_greedy(d["target"], d["draft_tokens"], d["draft_parents"],
                                                       d["draft_lens"], d["acc"], d["emi"], d["path"], wsbuf)

    def call(d):
        d["call"]()

    K, W = args.steps, args.warmup
    for i in range(W):
        call(data[i % sets])
    torch.cuda.synchronize()
    brackets = []
    t0 = time.perf_counter()
    i = 0
    while i < K:
        if i % 16 == 0 and i + 8 <= K:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for j in range(8):
                call(data[(i + j) % sets])
            b.record(stream)
            brackets.append((a, b))
            i += 8
        else:
            call(data[i % sets])
            i += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_ms = statistics.fmean(a.elapsed_time(b) for a, b in brackets) / 8 if brackets else elapsed * 1e3 / K
    rows = B * (n + 1)
    nbytes = rows * V * 2 + B * n * 8 + B * 4 + B * (n + 1) * 4 + B * n * 4 + B * 4
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    out = {
        "metric": "verified vocab rows/s + HBM GB/s (% of peak), V=128256 bf16, B=64 (greedy tree of 26 nodes)",
        "value": round(rows * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; inputs resident in HBM, rotated over {sets} copies)",
        "config": {"workload": "greedy tree verification, 64 sequences x 26-node top-k tree, V=128256 bf16 "
                               "(greedy_tree_verify)", "B": B, "nodes": n + 1, "V": V, "parallelism": "none (1 GPU)"},
        "hbm_gbps": round(nbytes * K / elapsed / 1e9, 1),
        "pct_of_peak": round(nbytes * K / elapsed / 1e9 / PEAK_GBPS * 100, 2),
        "mean_accepted": round(float(data[0]["acc"].float().mean()), 4),
        "roofline": {"bound": "hbm", "kernel": "k_stats_tree", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "bytes_per_launch": nbytes,
                     "avg_launch_us": round(avg_ms * 1e3, 2), "timed_launches": 8 * len(brackets),
                     "timing": "HIP event pair around 8 consecutive calls, every 16 steps",
                     "traffic": measured_traffic("k_stats_tree", "greedy_tree_verify")},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_tree(data[0], B, n, V)
        out["oracle_parity"] = out["cpu_baseline"].pop("oracle_parity")
    print(json.dumps(out), flush=True)


def bench_tree_sample(args, dev):
    """Sampling tree verification: the statistics pass over every node's target
    row and every inner node's draft row with the walks from the root, the round
    kernels (3 for this tree: one residual mass per pending walk each) and the
    draw pass.  64 sequences, each the 26-node top-k tree (3 children at the
    root, 2 below each of those, then chains; 20 inner nodes), V=128256 bf16
    rows of the llama-vocab sampling recipe, children drawn from the draft at
    their parent, T=0.7; inputs resident in HBM, rotated over input copies."""
    import numpy as np
    import torch

    import draft_token_verification_08_amd as sv
    from draft_token_verification_08_amd import synth

    B, n, V = 64, 25, 128256
    sets = args.sets or 3
    wsbuf = sv.Workspace(dev).get(sv.sv_workspace_bytes(B, n, V, sv.SV_BF16))
    stream = torch.cuda.current_stream(dev)
    par = synth.tree_parents(n)
    R = sv.sv_tree_rounds(par)
    inner = len(set(par))
    data = []
    for i in range(sets):
        d = synth.make_tree_sample(args.seed + i, device=dev, B=B, n=n, V=V)
        d["acc"] = torch.empty(B, dtype=torch.int32, device=dev)
        d["emi"] = torch.empty((B, n + 1), dtype=torch.int32, device=dev)
        d["path"] = torch.empty((B, n), dtype=torch.int32, device=dev)
        data.append(d)
    torch.cuda.synchronize()
    for d in data:
        d["call"] = sv.prepare_spec_verify_tree_sample(d["target"], d["draft"], d["draft_tokens"],
                                                       d["draft_parents"], d["draft_lens"], d["temperature"],
                                                       d["uniforms"], R, d["acc"], d["emi"], d["path"], wsbuf)

    K, W = args.steps, args.warmup
    for i in range(W):
        data[i % sets]["call"]()
    torch.cuda.synchronize()
    brackets = []
    t0 = time.perf_counter()
    i = 0
    while i < K:
        if i % 16 == 0 and i + 8 <= K:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for j in range(8):
                data[(i + j) % sets]["call"]()
            b.record(stream)
            brackets.append((a, b))
            i += 8
        else:
            data[i % sets]["call"]()
            i += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_ms = statistics.fmean(a.elapsed_time(b) for a, b in brackets) / 8 if brackets else elapsed * 1e3 / K
    # every row the rule needs, counted once: all node target rows, inner node draft rows
    rows = B * (n + 1 + inner)
    side = B * n * 8 + B * 4 * 2 + B * (n + 1) * 4 * 2 + B * n * 4
    nbytes = rows * V * 2 + side
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    kernel = f"k_stats_tree_sample+{R}xk_tree_round+k_draw"
    out = {
        "metric": "verified vocab rows/s + HBM GB/s (% of peak), V=128256 bf16, B=64 (sampling tree of 26 nodes)",
        "value": round(rows * K / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; inputs resident in HBM, rotated over {sets} copies)",
        "config": {"workload": "sampling tree verification, 64 sequences x 26-node top-k tree, V=128256 bf16, "
                               "T=0.7 (sampling_tree_verify)", "B": B, "nodes": n + 1, "inner_nodes": inner,
                   "rounds": R, "V": V, "parallelism": "none (1 GPU)"},
        "hbm_gbps": round(nbytes * K / elapsed / 1e9, 1),
        "pct_of_peak": round(nbytes * K / elapsed / 1e9 / PEAK_GBPS * 100, 2),
        "mean_accepted": round(float(torch.stack([d["acc"].float().mean() for d in data]).mean()), 4),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "bytes_per_launch": nbytes,
                     "avg_launch_us": round(avg_ms * 1e3, 2), "timed_launches": 8 * len(brackets),
                     "timing": "HIP event pair around 8 consecutive calls, every 16 steps",
                     "traffic": measured_traffic(kernel, "sampling_tree_verify")},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_tree_sample(data[0], B, n, V, rows)
        out["oracle_parity"] = out["cpu_baseline"].pop("oracle_parity")
    print(json.dumps(out), flush=True)


def cpu_baseline_tree_sample(d, B, n, V, rows):
    """The oracle (untuned, one thread) on whole steps of the same workload for
    about 10-20 s of CPU work; then the GPU's outputs for this input copy against
    the oracle's, sequence by sequence (a difference is exempt only where one of
    the oracle's decision margins is below 1e-5)."""
    import numpy as np

    import oracle
    from draft_token_verification_08_amd import synth

    orc = oracle.Oracle()
    zt, zd = synth.host_logits(d["target"]), synth.host_logits(d["draft"])
    args = (d["draft_tokens"].cpu().numpy(), d["draft_parents"].cpu().numpy(), d["draft_lens"].cpu().numpy(),
            d["temperature"].cpu().numpy(), d["uniforms"].cpu().numpy())
    calls, t0 = 0, time.perf_counter()
    while calls < 1 or (time.perf_counter() - t0 < 12.0 and calls < 100):
        o = orc.verify_tree_sample(zt, zd, *args)
        calls += 1
    el = time.perf_counter() - t0
    acc, emi, path = d["acc"].cpu().numpy(), d["emi"].cpu().numpy(), d["path"].cpu().numpy()
    diff = (acc != o["accepted_len"]) | (emi != o["emitted"]).any(1) | (path != o["path"]).any(1)
    tie = (o["accept_margin"] < NEAR_TIE).any(1) | (o["draw_margin"] < NEAR_TIE)
    return {"value": round(calls * rows / el, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full steps ({B} sequences, {rows} needed rows of V={V}) on 1 thread, about "
                      f"{el:.0f} s of CPU work", "cpu_model": cpu_model(),
            "oracle_parity": {"sequences": B, "exempt": int((diff & tie).sum()),
                              "hard_mismatches": int((diff & ~tie).sum()),
                              "inputs": "the first input copy of the timed workload, whole batch"}}


def cpu_baseline_tree(d, B, n, V):
    """The oracle (untuned, one thread) on whole steps of the same workload for
    about 10-20 s of CPU work; then the GPU's outputs for this input copy against
    the oracle's, exactly (greedy decisions have no near-tie exemption)."""
    import numpy as np

    import oracle
    from draft_token_verification_08_amd import synth

    orc = oracle.Oracle()
    z = synth.host_logits(d["target"])
    x, par, L = d["draft_tokens"].cpu().numpy(), d["draft_parents"].cpu().numpy(), d["draft_lens"].cpu().numpy()
    calls, t0 = 0, time.perf_counter()
    while calls < 1 or (time.perf_counter() - t0 < 15.0 and calls < 100):
        o = orc.verify_tree_greedy(z, x, par, L)
        calls += 1
    el = time.perf_counter() - t0
    acc, emi, path = d["acc"].cpu().numpy(), d["emi"].cpu().numpy(), d["path"].cpu().numpy()
    bad = int(((acc != o["accepted_len"]) | (emi != o["emitted"]).any(1) | (path != o["path"]).any(1)).sum())
    return {"value": round(calls * B * (n + 1) / el, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full steps ({B} sequences, {B * (n + 1)} rows of V={V}) on 1 thread, about "
                      f"{el:.0f} s of CPU work", "cpu_model": cpu_model(),
            "oracle_parity": {"sequences": B, "decisions": int(B + acc.sum()), "exempt": 0, "hard_mismatches": bad,
                              "inputs": "the first input copy of the timed workload, whole batch"}}


def cpu_baseline_draft_step(d, B, V):
    """The oracle (untuned) drawing one token per row on a bounded sample: whole
    batches of the same rows, as many as fit about 10-20 s of CPU work."""
    import numpy as np

    import oracle
    from draft_token_verification_08_amd import synth

    orc = oracle.Oracle()
    z = synth.host_logits(d["target"])
    T = d["temperature"].cpu().numpy()
    u = d["u"].cpu().numpy()
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))
    calls, t0 = 0, time.perf_counter()
    while calls < 1 or (time.perf_counter() - t0 < 20.0 / threads and calls < 200):
        orc.sample_rows(z, T, u, threads=threads)
        calls += 1
    el = time.perf_counter() - t0
    # the GPU's tokens for this input copy (left by the timed calls) against the oracle's; a
    # differing draw is exempt only at a CDF boundary closer than NEAR_TIE of the row's mass
    o = orc.sample_rows(z, T, u, threads=threads)
    got = d["tok"].cpu().numpy()
    diff = np.nonzero(got != o["tokens"])[0]
    parity = {"sequences": B, "decisions": B, "exempt": 0, "hard_mismatches": 0,
              "inputs": "the first input copy of the timed workload, whole batch"}
    if diff.size:
        v = orc.verify_sample(z[diff], None, np.zeros((diff.size, 0), np.int32), np.zeros(diff.size, np.int32),
                              T[diff], u[diff].reshape(-1, 1), threads=threads)
        for i, b in enumerate(diff):
            near = T[b] > 0 and v["draw_margin"][i] < NEAR_TIE
            parity["exempt" if near else "hard_mismatches"] += 1
    return {"value": round(calls * B / el, 1), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} full steps ({B} rows of V={V}) on {threads} threads, about {el * threads:.0f} s "
                      f"of CPU work", "cpu_model": cpu_model(), "oracle_parity": parity}


def cpu_baseline_lmhead(d, B, n, V, H):
    """The oracle (plain C double projection + greedy rule, untuned) on a bounded
    sample: the rows of whole sequences, as many as fit about 10 s of CPU work."""
    import numpy as np

    import oracle
    from draft_token_verification_08_amd import synth

    orc = oracle.Oracle()
    h = synth.bf16_bits(d["hidden"]).reshape(-1, H)
    w = synth.bf16_bits(d["weight"])
    x = d["draft_tokens"].cpu().numpy()
    L = d["draft_lens"].cpu().numpy()
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))
    seqs, t0 = 0, time.perf_counter()
    while seqs < 1 or (time.perf_counter() - t0 < 10.0 / threads * 2 and seqs < B):
        rows = np.arange(seqs * (n + 1), (seqs + 1) * (n + 1), dtype=np.int32)
        z = orc.lmhead_logits(h, w, rows=rows, threads=threads).reshape(1, n + 1, V)
        orc.verify_greedy(z, x[seqs:seqs + 1], L[seqs:seqs + 1])
        seqs += 1
    el = time.perf_counter() - t0
    return {"value": round(seqs * (n + 1) / el, 3), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{seqs} sequences ({seqs * (n + 1)} projected rows of V={V}, H={H}) on {threads} threads, "
                      f"about {el * threads:.0f} s of CPU work", "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()

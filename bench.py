#!/usr/bin/env python3
"""Throughput of the Markov-head draft round on one MI355X, with its roofline and a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]

A step is one draft round of the serving workload: B=128 rows, K=16 positions, vocabulary V=151936, rank
r=256, bf16 W1/W2 (W2 held transposed, [V, r]), fp32 base logits, sampling at T=1 (block-race draw from
softmax) with log-probabilities, i.e. one dspark_markov_draft call: a single persistent launch that, for
every position, gathers the predecessor rows, runs the fused bias contraction / calibration / pick and the
cross-workgroup reduction.  Inputs are synthetic (the seeded generator) and are resident in HBM before timing
starts.  Before every timed round a 1 GiB read evicts the L2 and the 256 MB last-level cache, so the round
starts with nothing of W2 or U cached; the read is outside the event pair.  (A read leaves the caches clean.
A 1 GiB write fill would leave them full of dirty lines whose write-back then competes with the timed round's
reads; that variant is reported as an extra.)  The printed line is one JSON object:

    value          B*K / mean round time (draft tokens per second), from HIP events around each round
    roofline       the round kernel against HBM bandwidth: algorithmic bytes of one launch (16 positions of
                   W2 + U_k + gathered W1 rows + predecessors + outputs) over the kernel's mean duration,
                   timed with HIP events on the library's stream around each launch; traffic = the
                   counter-measured bytes per launch recorded for the current kernel source
    cpu_baseline   the fp64 CPU oracle on a bounded sample of the same workload, on this host's cores (model,
                   sockets and SMT stated), run along the GPU's drafted tokens so that the same run gives the
                   parity counts of the measured round (flagged positions, differing tokens); plus one
                   single-thread batch-1 round
    extras         the back-to-back (no eviction), write-fill, graph-replay and cooperative-launch rates, the
                   practical streaming ceiling of the round's bytes (read_ceiling), and the other measured shapes
                   (greedy, confidence head, prefix scheduler, top-16 Selector and its top-k sweep on three input
                   recipes, gated head and its top-16 Selector form, batch 1, the tiny workload's latency)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "calibrated draft tokens/s at B=128,K=16,V=151936,r=256; % of HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "markov_round_serving_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "rank_markov_draft_amd", "csrc", "markov_round.hip")


def markov_bytes_per_position(B, V, r, gated=False):
    """Algorithmic bytes of one position: W2 (bf16) + U_k (fp32) + gathered W1 rows (bf16) + predecessors
    (int32) + token and log-probability outputs (+ gate rows, fp32)."""
    return 2 * r * V + 4 * B * V + 2 * B * r + 4 * B + 8 * B + (4 * B * r if gated else 0)


def selector_bytes_per_round(B, K, V, r, topk=16):
    """U read once + gathered A/Bemb rows + candidate ids and values."""
    return 4 * B * K * V + 2 * r * B * (K * topk + (K - 1) * topk + 1) + 8 * B * K * topk


def source_hash():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def traffic_entry():
    """Counter-measured HBM bytes per launch of the step kernel, if taken on the current kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash():
        return None
    return t


def write_traffic(fetch_csv, write_csv):
    """Counter-measured bytes per launch of the round kernel, from two rocprofv3 --pmc passes (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) over `bench.py --no-extras --copy-calibration`.  Each counter is scaled by
    what it reads for the 1 GiB device copy in the same run (1 GiB read, 1 GiB written)."""
    import csv

    def per_kernel(path, counter):
        out = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] == counter:
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return out

    gib_kib = float(1 << 20)
    rec = {"kernel": "markov_round_kernel<16, sample> (serving workload)", "kernel_source_sha256_16": source_hash()}
    total = 0.0
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        d = per_kernel(path, counter)
        copy = max(d["__amd_rocclr_copyBuffer"])
        kern = [v for k, v in d.items() if "markov_round_kernel<16, 1, false, 16, false>" in k][0]
        mean = sum(kern) / len(kern)
        scale = gib_kib / copy
        rec[key] = {"counter": counter, "kib_per_launch": round(mean, 1), "launches": len(kern),
                    "copy_kib_for_1gib": round(copy, 1), "scale": round(scale, 5),
                    "bytes_per_launch": int(round(mean * 1024 * scale))}
        total += mean * 1024 * scale
    rec["bytes_per_launch"] = int(round(total))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def host_cpu():
    """Model, sockets, threads per core and the CPUs this process may use."""
    model, sockets, threads_per_core = None, None, None
    try:
        ids = set()
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name") and model is None:
                model = line.split(":", 1)[1].strip()
            if line.startswith("physical id"):
                ids.add(line.split(":", 1)[1].strip())
        sockets = len(ids) or None
    except OSError:
        pass
    try:
        smt = open("/sys/devices/system/cpu/smt/active").read().strip()
        threads_per_core = 2 if smt == "1" else 1
    except OSError:
        pass
    return {"model": model, "sockets": sockets, "smt_threads_per_core": threads_per_core,
            "usable_cpus": len(os.sched_getaffinity(0)), "logical_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-baseline duration")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference kernel for the HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter-measured traffic record from two rocprofv3 --pmc counter_collection.csv "
                         "files and exit (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_markov_draft_amd as D
    import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    def evict():
        flush_buf.sum()  # reads 1 GiB

    def evict_dirty():
        flush_buf.fill_(1.0)  # writes 1 GiB

    def to_w(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def timed_rounds(fn, n, flush=True):
        """Mean / p10 / p90 of n event-timed calls, each preceded by an (untimed) cache eviction."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if flush:
                evict()
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        return ms, wall

    # ------------------------------------------------------------------ serving workload (the metric)
    w = S.workload("serving")
    B, K, V, r = w.B, w.K, w.V, w.r
    U = torch.from_numpy(w.U).to(dev)
    W1 = to_w(w.W1)
    W2T = to_w(w.W2T)
    anchor = torch.from_numpy(w.anchor).to(dev)
    tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    logprobs = torch.empty((B, K), dtype=torch.float32, device=dev)
    ws = torch.empty(D.dspark_markov_workspace_bytes(B, K, V, r, D.DSPARK_BF16, D.DSPARK_W2_VR), dtype=torch.uint8,
                     device=dev)

    def serving_round():
        D.dspark_markov_draft(U, W1, W2T, anchor, w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_SAMPLE, seed=w.noise_seed,
                              temperature=w.temperature, tokens=tokens, logprobs=logprobs, workspace=ws)

    # Device warm-up before the W warm-up steps: the first rounds on a fresh device run up to 8% slower and
    # settle after about eight (kernel trace); these untimed rounds bring it to the steady state a serving loop
    # runs in.  The timed region is exactly the K rounds below.
    device_warmup = 12
    for _ in range(device_warmup + args.warmup):
        evict()
        serving_round()
    torch.cuda.synchronize()
    ms, wall = timed_rounds(serving_round, args.steps)
    ms_per_step = float(ms.mean())
    serving_tokens = tokens.cpu().numpy()  # the drafted tokens, for the CPU leg's parity counts
    value = B * K / (ms_per_step / 1e3)
    bytes_pos = markov_bytes_per_position(B, V, r)
    roof_round_ms = K * bytes_pos / (HBM_PEAK_GBS * 1e9) * 1e3
    roof_tok_s = B * K / (roof_round_ms / 1e3)

    # duration of the contraction kernel launches (events around each launch, on the library's stream)
    kern_total, kern_launches, round_ms_timed = 0.0, 0, []
    n_timed = max(3, min(args.steps, 10))
    for _ in range(n_timed):
        evict()
        _, _, kms, nl, rms = D.dspark_markov_draft_timed(U, W1, W2T, anchor, w2_layout=D.DSPARK_W2_VR,
                                                         mode=D.DSPARK_SAMPLE, seed=w.noise_seed,
                                                         temperature=w.temperature, tokens=tokens, logprobs=logprobs,
                                                         workspace=ws)
        kern_total += kms
        kern_launches += nl
        round_ms_timed.append(rms)
    kern_ms = kern_total / kern_launches
    positions_per_launch = K * n_timed // kern_launches
    bytes_launch = bytes_pos * positions_per_launch
    achieved = bytes_launch / (kern_ms / 1e3) / 1e9
    tr = traffic_entry()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if tr is None else tr["bytes_per_launch"],
                "kernel": "markov_round_kernel<16, sample>" if positions_per_launch > 1 else "markov_step_mfma<16, sample>",
                "bytes_per_launch": bytes_launch, "positions_per_launch": positions_per_launch,
                "bytes_per_position": bytes_pos, "launch_ms_mean": round(kern_ms, 5)}

    # back-to-back rounds without eviction (W2 may stay in the last-level cache across rounds)
    ms_b2b, _ = timed_rounds(serving_round, args.steps, flush=False)

    # rounds after a 1 GiB write fill instead of a read (its dirty lines are written back during the round)
    ms_dirty = []
    for _ in range(max(3, min(args.steps, 10))):
        evict_dirty()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        serving_round()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_dirty.append(e0.elapsed_time(e1))

    # The same round captured once in a graph and replayed, the same round with the runtime's cooperative launch,
    # and the streaming ceiling: extras (a counter or trace run with --no-extras launches only the plain rounds).
    ms_graph = ms_coop = rd_ms = None
    read_bytes = 0
    if not args.no_extras:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(graph, stream=side):
            serving_round()
        torch.cuda.synchronize()
        ms_graph, _ = timed_rounds(graph.replay, args.steps)
        del graph

        # the cooperative launch guarantees co-residency; the default ordinary launch relies on one workgroup per CU
        D.dspark_set_cooperative_launch(True)
        serving_round()
        ms_coop, _ = timed_rounds(serving_round, max(3, min(args.steps, 10)))
        D.dspark_set_cooperative_launch(False)

        # Practical streaming ceiling: the round's operand bytes (W2 and each position's base logits, here as 16
        # contiguous regions of U) read once per position by a plain streaming kernel, 16 launches replayed from
        # a HIP graph after the same eviction.  Reported beside the nominal peak; the round is not held to it.
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        u_flat = U.view(-1)
        per_pos = B * V

        def read_round():
            for k in range(K):
                D.dspark_stream_read(W2T, u_flat[k * per_pos:(k + 1) * per_pos], sink)

        read_round()
        torch.cuda.synchronize()
        read_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(read_graph):
            read_round()
        rd_ms, _ = timed_rounds(read_graph.replay, max(3, min(args.steps, 10)))
        read_bytes = K * (W2T.numel() * W2T.element_size() + per_pos * 4)
        del read_graph

    extras = {
        "round_ms_p10": round(float(np.percentile(ms, 10)), 4), "round_ms_p90": round(float(np.percentile(ms, 90)), 4),
        "device_warmup_rounds": device_warmup,
        "pct_of_hbm_roofline": round(100.0 * roof_round_ms / ms_per_step, 2),
        "roofline_tokens_per_s": round(roof_tok_s, 1), "roofline_round_ms": round(roof_round_ms, 4),
        "back_to_back_round_ms": round(float(ms_b2b.mean()), 4),
        "back_to_back_tokens_per_s": round(B * K / (float(ms_b2b.mean()) / 1e3), 1),
        "after_write_fill_round_ms": round(float(np.mean(ms_dirty)), 4),
        "timed_wall_s": round(wall, 4),
    }
    if ms_graph is not None:
        extras.update({
            "graph_replay_round_ms": round(float(ms_graph.mean()), 4),
            "graph_replay_tokens_per_s": round(B * K / (float(ms_graph.mean()) / 1e3), 1),
            "cooperative_launch_round_ms": round(float(ms_coop.mean()), 4),
            "read_ceiling": {"what": "the round's W2 and base-logit bytes read once per position by a plain "
                                     "streaming kernel (dspark_stream_read, 16 launches from a HIP graph), evicted "
                                     "like a round",
                             "round_ms": round(float(rd_ms.mean()), 4), "bytes": int(read_bytes),
                             "GB_per_s": round(read_bytes / (float(rd_ms.mean()) / 1e3) / 1e9, 1),
                             "serving_round_fraction": round(float(rd_ms.mean()) / ms_per_step, 4)}})
    if not args.no_extras:
        # the same sampling round with the confidence head and prefix survival (synthetic hidden states, D = 4096,
        # as the gated workload's): computed by the round kernel's finalizer waves, one position behind
        gen = torch.Generator(device=dev).manual_seed(0xC0F)
        hconf = torch.randn((B, K, 4096), generator=gen, device=dev).to(torch.bfloat16)
        wconf = torch.randn((4096 + r,), generator=gen, device=dev) * 0.02

        def conf_round():
            D.dspark_markov_draft_confidence(U, W1, W2T, anchor, hconf, wconf, w2_layout=D.DSPARK_W2_VR,
                                             mode=D.DSPARK_SAMPLE, seed=w.noise_seed, temperature=w.temperature,
                                             workspace=ws)

        conf_round()
        cms, _ = timed_rounds(conf_round, 10)
        extras["serving_with_confidence"] = {"round_ms": round(float(cms.mean()), 4),
                                             "overhead_ms": round(float(cms.mean()) - ms_per_step, 4),
                                             "hidden_bytes": int(hconf.numel() * 2)}
        # verify lengths from the block's survival: greedy load-aware prefix scheduling over a synthetic
        # steps-per-second curve (flat up to a knee, then falling as 1/B)
        _, _, _, surv = D.dspark_markov_draft_confidence(U, W1, W2T, anchor, hconf, wconf, w2_layout=D.DSPARK_W2_VR,
                                                         mode=D.DSPARK_SAMPLE, seed=w.noise_seed,
                                                         temperature=w.temperature, workspace=ws)
        bsz = torch.arange(B * (K + 1) + 1, device=dev, dtype=torch.float32)
        knee = float(B * 4)
        sps = torch.where(bsz <= knee, torch.full_like(bsz, 40.0), 40.0 * knee / bsz.clamp(min=1.0))
        lengths, theta = D.dspark_schedule_prefixes(surv, sps)
        sched_ms, _ = timed_rounds(lambda: D.dspark_schedule_prefixes(surv, sps), 20, flush=False)
        extras["prefix_schedule"] = {"R": B, "K": K, "call_ms": round(float(sched_ms.mean()), 4),
                                     "verified_tokens": int(lengths.sum().item()), "theta": round(float(theta.item()), 2)}
        del hconf, wconf
    del U
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------------------------- other shapes
    if not args.no_extras:
        # greedy on the same serving shape
        w = S.workload("serving", mode=S.GREEDY)
        U = torch.from_numpy(w.U).to(dev)

        def greedy_round():
            D.dspark_markov_draft(U, W1, W2T, anchor, w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_GREEDY, tokens=tokens,
                                  logprobs=logprobs, workspace=ws)

        greedy_round()
        gms, _ = timed_rounds(greedy_round, 10)
        extras["serving_greedy"] = {"round_ms": round(float(gms.mean()), 4),
                                    "tokens_per_s": round(B * K / (gms.mean() / 1e3), 1),
                                    "pct_of_hbm_roofline": round(100.0 * roof_round_ms / float(gms.mean()), 2)}
        del U
        torch.cuda.empty_cache()

        # top-16 Selector, ungated, greedy walk
        w = S.workload("selector")
        U = torch.from_numpy(w.U).to(dev)
        A, Bemb = to_w(w.W1), to_w(w.W2T)
        anc = torch.from_numpy(w.anchor).to(dev)
        sws = torch.empty(D.dspark_selector_workspace_bytes(w.B, w.K, w.V, w.r, 16), dtype=torch.uint8, device=dev)

        def sel_round():
            D.dspark_selector_draft(U, A, Bemb, anc, topk=16, workspace=sws)

        sel_round()
        sms_, _ = timed_rounds(sel_round, 10)
        sb = selector_bytes_per_round(w.B, w.K, w.V, w.r)
        extras["selector_top16"] = {"round_ms": round(float(sms_.mean()), 4),
                                    "tokens_per_s": round(w.B * w.K / (sms_.mean() / 1e3), 1),
                                    "bytes_per_round": sb,
                                    "pct_of_hbm_roofline": round(100.0 * sb / (HBM_PEAK_GBS * 1e9) * 1e3 / float(sms_.mean()), 2)}
        # the practical ceiling of the Selector's dominant stream: the same base logits read once by the plain
        # streaming kernel (16-byte non-temporal loads, as the top-k reads them), after the same eviction
        sel_sink = torch.zeros(1, dtype=torch.int32, device=dev)
        sel_pad = torch.zeros(4, dtype=torch.float32, device=dev)
        u_all = U.view(-1)

        def base_logits_read():
            D.dspark_stream_read(sel_pad, u_all, sel_sink)

        base_logits_read()
        urd, _ = timed_rounds(base_logits_read, 10)
        u_bytes = u_all.numel() * u_all.element_size()
        extras["selector_top16"]["base_logits_read"] = {
            "what": "the Selector's base logits read once by a plain streaming kernel, evicted like a round",
            "ms": round(float(urd.mean()), 4), "bytes": u_bytes,
            "GB_per_s": round(u_bytes / (float(urd.mean()) * 1e-3) / 1e9, 1),
            "selector_round_fraction": round(float(urd.mean()) / float(sms_.mean()), 3)}
        del u_all

        # top-k sweep: the Selector execution of the Markov rule (W1 = A, W2 = Bemb^T) restricted to the
        # top-k candidates, against the full-vocabulary greedy head on the same inputs: token agreement (and the
        # longest agreeing prefix) for three recipes, and the round time (the same bytes for every recipe).  The
        # serving recipe's bias (std 0.006) is far below its hot-token boost, so there the truncation never binds;
        # the moderate (bias std 0.3) and strong (1.0) recipes use U = z + 2 on the hot ids.
        sweep = {}
        for label in ("serving_recipe", "moderate_bias", "strong_bias"):
            del U, A, Bemb
            torch.cuda.empty_cache()
            if label == "serving_recipe":
                wk = S.workload("selector")
            else:
                bias_sd = 0.3 if label == "moderate_bias" else 1.0
                wk = S.workload("selector", sigma_w=float(np.sqrt(bias_sd / np.sqrt(256))), u_scale=1.0, u_boost=2.0)
            U = torch.from_numpy(wk.U).to(dev)
            A, Bemb = to_w(wk.W1), to_w(wk.W2T)
            anc = torch.from_numpy(wk.anchor).to(dev)
            full, _ = D.dspark_markov_draft(U, A, Bemb, anc, w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_GREEDY)
            fh = full.cpu().numpy()
            row = {}
            for kk in (4, 8, 16, 32, 64):
                kws = torch.empty(D.dspark_selector_workspace_bytes(wk.B, wk.K, wk.V, wk.r, kk), dtype=torch.uint8,
                                  device=dev)
                res = D.dspark_selector_draft(U, A, Bemb, anc, topk=kk, workspace=kws)
                th = res["tokens"].cpu().numpy()
                same = th == fh
                prefix = np.where(same.all(axis=1), wk.K, np.argmin(same, axis=1))
                ent = {"agreement": round(float(same.mean()), 4), "mean_agreeing_prefix": round(float(prefix.mean()), 3)}
                if label == "serving_recipe":
                    kms, _ = timed_rounds(lambda: D.dspark_selector_draft(U, A, Bemb, anc, topk=kk, workspace=kws), 5)
                    ent["round_ms"] = round(float(kms.mean()), 4)
                row["k%d" % kk] = ent
            sweep[label] = row
        extras["topk_sweep"] = sweep
        del U, A, Bemb
        torch.cuda.empty_cache()

        # gated head: gate GEMM for the block + gated full-vocabulary draft
        w = S.workload("gated")
        U = torch.from_numpy(w.U).to(dev)
        W1g, W2g = to_w(w.W1), to_w(w.W2T)
        h, Wg = to_w(w.h), to_w(w.Wg)
        anc = torch.from_numpy(w.anchor).to(dev)
        Hbuf = torch.empty((w.B, w.K, w.r), dtype=torch.float32, device=dev)
        gws = torch.empty(max(D.dspark_gate_workspace_bytes(w.B * w.K, w.D, w.r), 1), dtype=torch.uint8, device=dev)
        tok_g = torch.empty((w.B, w.K), dtype=torch.int32, device=dev)
        lp_g = torch.empty((w.B, w.K), dtype=torch.float32, device=dev)
        gws = torch.empty(D.dspark_markov_workspace_bytes(w.B, w.K, w.V, w.r, 1, 1), dtype=torch.uint8, device=dev)

        def gated_round():
            D.dspark_gate(h, Wg, out=Hbuf, workspace=gws)
            D.dspark_markov_draft(U, W1g, W2g, anc, H=Hbuf, tokens=tok_g, logprobs=lp_g, workspace=gws)

        gated_round()
        gms_, _ = timed_rounds(gated_round, 10)
        gb = w.K * markov_bytes_per_position(w.B, w.V, w.r, gated=True) + 2 * w.B * w.K * w.D + 2 * w.D * w.r + 4 * w.B * w.K * w.r
        # the gated round keeps W2 on chip (matrix-core resident round): also held to W2 read once per round
        gcomp = gb - (w.K - 1) * 2 * w.r * w.V
        extras["gated"] = {"round_ms": round(float(gms_.mean()), 4),
                           "tokens_per_s": round(w.B * w.K / (gms_.mean() / 1e3), 1), "bytes_per_round": gb,
                           "pct_of_hbm_roofline": round(100.0 * gb / (HBM_PEAK_GBS * 1e9) * 1e3 / float(gms_.mean()), 2),
                           "kernel": "gate GEMM + matrix-core resident round (W2 read once per round)",
                           "compulsory_bytes_per_round": gcomp,
                           "pct_of_compulsory_roofline": round(100.0 * gcomp / (HBM_PEAK_GBS * 1e9) * 1e3 / float(gms_.mean()), 2)}

        # its top-16 Selector form: the gate GEMM, then top-16, the gated pair tables and the walk
        gsws = torch.empty(D.dspark_selector_workspace_bytes(w.B, w.K, w.V, w.r, 16), dtype=torch.uint8, device=dev)

        def gated_sel_round():
            D.dspark_gate(h, Wg, out=Hbuf, workspace=gws)
            D.dspark_selector_draft(U, W1g, W2g, anc, H=Hbuf, topk=16, workspace=gsws)

        gated_sel_round()
        gsms, _ = timed_rounds(gated_sel_round, 10)
        gsb = (selector_bytes_per_round(w.B, w.K, w.V, w.r) + 2 * w.B * w.K * w.D + 2 * w.D * w.r
               + 2 * 4 * w.B * w.K * w.r)
        extras["gated_selector_top16"] = {
            "round_ms": round(float(gsms.mean()), 4), "tokens_per_s": round(w.B * w.K / (gsms.mean() / 1e3), 1),
            "bytes_per_round": gsb,
            "pct_of_hbm_roofline": round(100.0 * gsb / (HBM_PEAK_GBS * 1e9) * 1e3 / float(gsms.mean()), 2)}
        del U, W1g, W2g, h, Wg
        torch.cuda.empty_cache()

        # batch 1, greedy
        w = S.workload("batch1")
        U = torch.from_numpy(w.U).to(dev)
        W1b, W2b = to_w(w.W1), to_w(w.W2T)
        anc = torch.from_numpy(w.anchor).to(dev)
        tok_b = torch.empty((1, w.K), dtype=torch.int32, device=dev)
        lp_b = torch.empty((1, w.K), dtype=torch.float32, device=dev)
        bws = torch.empty(D.dspark_markov_workspace_bytes(1, w.K, w.V, w.r, 1, 1), dtype=torch.uint8, device=dev)

        def b1_round():
            D.dspark_markov_draft(U, W1b, W2b, anc, tokens=tok_b, logprobs=lp_b, workspace=bws)

        b1_round()
        bms, _ = timed_rounds(b1_round, 10)
        bb = w.K * markov_bytes_per_position(1, w.V, w.r)
        # the single-row round keeps W2 on chip (read once per round, not once per position), so it is held to the
        # compulsory bytes as well: W2 once plus every position's other bytes
        bcomp = bb - (w.K - 1) * 2 * w.r * w.V
        extras["batch1"] = {"round_ms": round(float(bms.mean()), 4),
                            "tokens_per_s": round(w.K / (bms.mean() / 1e3), 1), "bytes_per_round": bb,
                            "pct_of_hbm_roofline": round(100.0 * bb / (HBM_PEAK_GBS * 1e9) * 1e3 / float(bms.mean()), 2),
                            "kernel": "resident round (W2 read once per round)", "compulsory_bytes_per_round": bcomp,
                            "pct_of_compulsory_roofline": round(100.0 * bcomp / (HBM_PEAK_GBS * 1e9) * 1e3 / float(bms.mean()), 2)}
        del U, W1b, W2b
        torch.cuda.empty_cache()

        # the tiny workload (B=1, K=4, V=512, r=16, fp32 weights, greedy): launch-bound latency of one draft, of
        # the full head and of its top-k = V Selector form (no eviction: the operands are 74 KB)
        w = S.workload("tiny")
        U = torch.from_numpy(w.U).to(dev)
        W1t, W2t = torch.from_numpy(w.W1).to(dev), torch.from_numpy(w.W2).to(dev)
        W2tT = torch.from_numpy(np.ascontiguousarray(w.W2.T)).to(dev)
        anc = torch.from_numpy(w.anchor).to(dev)
        tws = torch.empty(D.dspark_markov_workspace_bytes(1, w.K, w.V, w.r, 0, 0), dtype=torch.uint8, device=dev)
        sws_t = torch.empty(D.dspark_selector_workspace_bytes(1, w.K, w.V, w.r, w.V), dtype=torch.uint8, device=dev)
        tiny_head = lambda: D.dspark_markov_draft(U, W1t, W2t, anc, w2_layout=D.DSPARK_W2_RV, workspace=tws)
        tiny_sel = lambda: D.dspark_selector_draft(U, W1t, W2tT, anc, topk=w.V, workspace=sws_t)
        tiny_head(), tiny_sel()
        tms, _ = timed_rounds(tiny_head, 20, flush=False)
        tsms, _ = timed_rounds(tiny_sel, 20, flush=False)
        _, _, _, nl, _ = D.dspark_markov_draft_timed(U, W1t, W2t, anc, w2_layout=D.DSPARK_W2_RV, workspace=tws)
        extras["tiny_latency"] = {"workload": "B=1, K=4, V=512, r=16, fp32, greedy",
                                  "markov_draft_us": round(1e3 * float(tms.mean()), 1),
                                  "selector_topk_V_us": round(1e3 * float(tsms.mean()), 1),
                                  "kernel_launches": {"markov_draft": nl, "selector": 3}}
        del U
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle as O

        w = S.workload("serving")
        W2Th = w.W2T
        t0 = time.perf_counter()
        O.markov_draft(w.U, w.W1, W2Th, w.anchor, w2_layout=O.W2_VR, mode=O.SAMPLE, seed=w.noise_seed, rows=[0])
        one = time.perf_counter() - t0
        threads = O.num_threads()
        nrows = int(max(1, min(w.B, round(args.cpu_seconds / max(one, 1e-3) * threads * 0.8))))
        nrows = max(threads, nrows) if nrows < w.B else w.B
        nrows = min(nrows, w.B)
        rows = list(range(nrows))
        # the oracle runs along the GPU's drafted tokens (teacher forcing), so the same timed run also gives the
        # parity counts of the measured round on these rows
        t0 = time.perf_counter()
        ref = O.markov_draft(w.U, w.W1, W2Th, w.anchor, w2_layout=O.W2_VR, mode=O.SAMPLE, seed=w.noise_seed,
                             follow=serving_tokens, rows=rows)
        dt = time.perf_counter() - t0
        agree = serving_tokens[rows] == ref["tokens"][rows]
        parity = {"rows": nrows, "positions": int(agree.size),
                  "flagged_margin_below_2e-2": int((ref["margins"][rows] < 2e-2).sum()),
                  "tokens_differing": int((~agree).sum()),
                  "differing_and_unreachable": int((~agree & (ref["reach"][rows] != 1)).sum())}
        # one single-thread batch-1 round (per-core scale)
        wb = S.workload("batch1")
        O.set_num_threads(1)
        t1 = time.perf_counter()
        O.markov_draft(wb.U, wb.W1, wb.W2T, wb.anchor, w2_layout=O.W2_VR)
        dt1 = time.perf_counter() - t1
        O.set_num_threads(threads)
        cpu = {"value": round(nrows * w.K / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"serving workload rows 0..{nrows - 1} of {w.B}, all {w.K} positions, sampling T=1 "
                         f"({nrows * w.K} draft tokens, fp64, {dt:.1f} s)",
               "host": host_cpu(), "parity_of_measured_round": parity,
               "batch1_single_thread": {"tokens_per_s": round(wb.K / dt1, 3), "round_s": round(dt1, 2),
                                        "workload": "B=1, K=16, V=151936, r=256, greedy, one thread"}}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "pct_of_roofline": extras["pct_of_hbm_roofline"], "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "serving: Markov-head draft round, sampling T=1, with log-probabilities",
                   "B": B, "K": K, "V": V, "r": r, "weights": "bf16 (W2 stored [V, r])", "base_logits": "fp32",
                   "accumulate": "fp32", "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "extras": extras,
    }
    print(json.dumps(out), flush=True)
    # orderly teardown: wait for the device, then release torch's cached blocks while the runtime is up
    torch.cuda.synchronize()
    del flush_buf, ws, tokens, logprobs, W1, W2T
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()

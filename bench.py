"""DSA decode step benchmark on one MI355X.

A step is one decode token for every sequence of the batch through the whole
hot path: dsa_index_scores -> dsa_topk_pools_expand (the top-k selection and
its expansion to token ids in one launch: both outputs are written) ->
dsa_sparse_mla_decode, on the long-context workload (4 sequences of 262144
tokens, kpool 4 -> 65536 pools each, 32 index heads x 128, select_k 512 pools =
2048 tokens, 64-head absorbed MLA over a 512-wide latent, bf16).  The pooled-key
cache comes from an untimed dsa_kpool_compress over synthetic tokens.

Inputs are resident in HBM before the timed region.  Eight replicas of the
pool cache and of the latent cache (about 8.5 GiB) rotate from step to step, so
the 256 MB last-level cache cannot serve a step from the previous one.  Each
step launches the three calls from argument tuples bound once per replica
(``--mode graph`` replays HIP graphs captured per replica instead); HIP events
on the launch stream bracket the score kernel of every timed step, which gives
that kernel's per-launch time for the roofline line.  They are timing-only
events (no system-scope fence at record), so that measuring does not add cache
flushes to the step.  The roofline's traffic
figure comes from the committed counter summary of the same kernel source.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode steps/s (indexer+top-k+sparse MLA) @262K ctx; % HBM roofline"
HBM_PEAK_GBS = 8000.0
REPLICAS = 8
RUNS = 5  # timed runs per mode; the reported figure is their median
# The score-kernel launches of every EVENT_STRIDE-th step are event-timed for
# the roofline (5 is coprime with REPLICAS, so the timed launches rotate
# through the input replicas).  A pair of events around every launch cost
# ~2.1 us per step here: 28 220-28 280 against 30 010-30 060 steps/s untimed.
EVENT_STRIDE = 5


class TimingEvents:
    """HIP events for timing only, created through the HIP runtime that torch
    uses, with hipEventDisableSystemFence: recording them performs no
    system-scope cache writeback and invalidation (HIP's documented flag for
    events that only measure time), so they neither pad the measured launch
    nor slow the work that follows."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n: int):
        import ctypes
        self._c = ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            st = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS)
            if st != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
            self.ev.append(e)

    def record(self, i: int, stream_handle: int) -> None:
        self.hip.hipEventRecord(self.ev[i], stream_handle)

    def elapsed_us(self, i: int, j: int) -> float:
        ms = self._c.c_float()
        st = self.hip.hipEventElapsedTime(self._c.byref(ms), self.ev[i], self.ev[j])
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value * 1e3

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["graph", "eager"], default="eager")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 64 MiB device copy first (a known-size kernel for counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the extra timing of the sparse MLA over a paged (bf16, fp8) latent cache")
    ap.add_argument("--workload", choices=["long", "prefill"], default="long",
                    help="long: the decode step (the headline line); prefill: the 4096-row prefill chunk's "
                         "scores + top-k + expand, reported against the MFMA roofline")
    ap.add_argument("--split-topk-expand", action="store_true",
                    help="run dsa_topk_pools and dsa_expand_selection as two calls instead of the fused call")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the oracle's timed CPU work")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_scores_traffic.txt")
SCORE_SOURCES = [os.path.join(ROOT, "dsa_decode_amd", "csrc", f)
                 for f in ("index_scores.hip", "dsa_common.hpp", "dsa_select.hpp")]


def score_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per score-kernel launch from the committed counter summary, or
    None when it is missing or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != score_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def step_algorithmic_bytes(Q: int, P: int, K: int, W: int, Hm: int, Dl: int, score_bytes: int) -> int:
    """Bytes one decode step must move at least: the score launch's bytes, the
    top-k reading the scores and writing pool ids and token ids, the sparse MLA
    reading each listed latent row once plus q_lat and writing out and lse
    (bf16 activations, 4-byte scores, ids and lse)."""
    topk = Q * P * 4 + Q * K * 4 + Q * W * 4
    mla = Q * W * Dl * 2 + Q * Hm * Dl * 2 + Q * Hm * Dl * 2 + Q * Hm * 4 + Q * W * 4
    return score_bytes + topk + mla


def score_bytes_per_pool() -> int:
    # key row (128 bf16) + pool_valid (u8) read, score (fp32) written
    return 128 * 2 + 1 + 4


def main() -> int:
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path is not "
              "sharded across GPUs", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from dsa_decode_amd import _lib, ops, synth

    _lib.load()
    torch.cuda.set_device(0)
    dev = lambda t: t.contiguous().cuda()
    if args.copy_probe:
        a = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.workload == "prefill":
        return bench_prefill(args)

    wl = synth.workload("long")
    Q, P, K, W = wl.Q, wl.P_max, wl.K, wl.W
    ti = synth.token_inputs(wl)
    ip = synth.index_params(wl)
    mi = synth.mla_inputs(wl)

    # pool cache: one compress on the GPU, then replicas
    tok_dev = dict(k=dev(ti["k"]), gate=dev(ti["gate"]), valid=dev(ti["valid"]), ape=dev(ti["ape"]),
                   seq_len=dev(ti["seq_len"]))
    comp = ops.dsa_kpool_compress(tok_dev["k"], tok_dev["gate"], tok_dev["valid"], tok_dev["ape"],
                                  tok_dev["seq_len"], wl.kp, P)
    del ti
    kv0 = dev(mi["kv"])
    reps = []
    for i in range(REPLICAS):
        reps.append(dict(k_pool=comp["k_pool"].clone(), pool_start=comp["pool_start"].clone(),
                         pool_valid=comp["pool_valid"].clone(), kv=kv0 if i == 0 else kv0.clone(),
                         scores=torch.empty((Q, P), dtype=torch.float32, device="cuda"),
                         ids=torch.empty((Q, K), dtype=torch.int32, device="cuda"),
                         tok=torch.empty((Q, W), dtype=torch.int32, device="cuda"),
                         out=torch.empty((Q, wl.Hm, wl.Dl), dtype=torch.bfloat16, device="cuda"),
                         lse=torch.empty((Q, wl.Hm), dtype=torch.float32, device="cuda")))
    q, w, gamma, beta = dev(ip["q"]), dev(ip["w"]), dev(ip["gamma"]), dev(ip["beta"])
    row_seq, row_pos = dev(ip["row_seq"]), dev(ip["row_pos"])
    q_lat = dev(mi["q_lat"])
    tk_ws = ops.topk_workspace(ops.dsa_topk_workspace_bytes(Q, P, K))
    mla_ws = torch.empty(max(1, ops.dsa_sparse_mla_workspace_bytes(Q, wl.Hm, wl.Dl, W, ops.DSA_BF16)),
                         dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    # every launch argument marshalled once per replica (plain ctypes calls in the loop)
    with torch.cuda.stream(stream):
        bound = []
        for r in reps:
            bound.append(dict(
                scores=ops.bind_index_scores(q, w, ip["scale"], r["k_pool"], r["pool_start"], r["pool_valid"],
                                             gamma, beta, ip["eps"], row_seq, row_pos, wl.kp, r["scores"]),
                rest=([ops.bind_topk_pools(r["scores"], K, r["ids"], tk_ws),
                       ops.bind_expand_selection(r["ids"], row_seq, r["pool_start"], wl.kp, r["tok"])]
                      if args.split_topk_expand else
                      [ops.bind_topk_pools_expand(r["scores"], K, r["ids"], row_seq, r["pool_start"], wl.kp,
                                                  r["tok"], tk_ws)]) + [
                      ops.bind_sparse_mla_decode(q_lat, r["kv"], row_seq, r["tok"], mi["sm_scale"], r["out"],
                                                 r["lse"], mla_ws)]))

    def scores_stage(i):
        bound[i]["scores"]()

    def rest_stages(i):
        for c in bound[i]["rest"]:
            c()

    torch.cuda.synchronize()

    def timed_runs(run_step, with_events: bool):
        """RUNS timed runs of args.steps steps each (after the warm-up), each
        bracketed by a device synchronisation; -> (ms per step of every run,
        event-timed score-kernel launches in us or [])."""
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                run_step(i % REPLICAS, None)
            stream.synchronize()
            torch.cuda.synchronize()
            ms, score_us = [], []
            for _ in range(RUNS):
                tev = TimingEvents(2 * args.steps) if with_events else None
                t0 = time.perf_counter()
                for i in range(args.steps):
                    run_step(i % REPLICAS, (tev, i) if with_events else None)
                stream.synchronize()
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                ms.append((t1 - t0) * 1e3 / args.steps)
                if with_events:
                    score_us += [tev.elapsed_us(2 * i, 2 * i + 1) for i in range(0, args.steps, EVENT_STRIDE)]
                    tev.close()
        return ms, score_us

    sh = stream.cuda_stream

    def eager_step(j, ev):
        timed = ev is not None and ev[1] % EVENT_STRIDE == 0
        if timed:
            ev[0].record(2 * ev[1], sh)
        scores_stage(j)
        if timed:
            ev[0].record(2 * ev[1] + 1, sh)
        rest_stages(j)

    # eager launches (the headline): score-kernel launches of every EVENT_STRIDE-th
    # step event-timed for the roofline
    eager_ms, score_us = timed_runs(eager_step, True)

    # the same step replayed from HIP graphs (one graph per replica: all launches of the step)
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(REPLICAS):
            scores_stage(i)
            rest_stages(i)
        stream.synchronize()
        for i in range(REPLICAS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                scores_stage(i)
                rest_stages(i)
            graphs.append(g)
    graph_ms, _ = timed_runs(lambda j, ev: graphs[j].replay(), False)
    del graphs

    ms_runs = graph_ms if args.mode == "graph" else eager_ms
    ms_per_step = float(np.median(ms_runs))
    score_us_mean = float(np.mean(score_us))
    # per-stage breakdown (separate instrumented pass, eager launches, events around each stage)
    stage_names = (["index_scores", "topk_pools", "expand_selection", "sparse_mla_decode"] if args.split_topk_expand
                   else ["index_scores", "topk_pools_expand", "sparse_mla_decode"])
    stage_t = {n: [] for n in stage_names}
    with torch.cuda.stream(stream):
        for i in range(min(64, args.steps)):
            b = bound[i % REPLICAS]
            calls = [b["scores"]] + b["rest"]
            e = TimingEvents(len(stage_names) + 1)
            e.record(0, stream.cuda_stream)
            for k, c in enumerate(calls):
                c()
                e.record(k + 1, stream.cuda_stream)
            stream.synchronize()
            for k, n in enumerate(stage_names):
                stage_t[n].append(e.elapsed_us(k, k + 1))
            e.close()
    stages_us = {n: round(float(np.median(v)), 2) for n, v in stage_t.items()}

    bytes_per_launch = score_bytes_per_pool() * Q * P + q.numel() * 2 + w.numel() * 4 + 2 * 128 * 4
    ceiling = read_stream_ceiling(reps, stream)
    achieved = bytes_per_launch / (score_us_mean * 1e-6) / 1e9
    steps_per_s = 1e3 / ms_per_step
    step_bytes = step_algorithmic_bytes(Q, P, K, W, wl.Hm, wl.Dl, bytes_per_launch)

    paged = None if args.no_paged else paged_mla_stages(wl, mi, q_lat, row_seq, reps[0]["tok"], stream)
    append_us = append_stage_us(wl, tok_dev, comp, stream)
    with_append = step_with_append_us(wl, tok_dev, comp, bound, scores_stage, rest_stages, stream, args.steps)
    del tok_dev

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ip, mi, comp, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "runs": {"count": RUNS, "steps_per_s": [round(1e3 / m, 1) for m in ms_runs],
                 "statistic": "median of the runs' steps/s"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long-context decode: batch 4 x 262144 tokens, kpool 4 (65536 pools/seq), "
                               "32 index heads x 128, select_k 512 pools (2048 tokens), absorbed NoPE MLA "
                               "64 heads x 512 latent, bf16",
                   "batch": Q, "context": wl.T_max, "kpool": wl.kp, "select_k": K, "mode": args.mode,
                   "replicas": REPLICAS},
        "tokens_per_s": round(steps_per_s * Q, 1),
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "graph_steps_per_s": round(1e3 / float(np.median(graph_ms)), 1),
        "eager_steps_per_s": round(1e3 / float(np.median(eager_ms)), 1),
        "step_with_append": with_append,
        "stages_us": stages_us,
        "paged_mla_us": paged,
        "kpool_append_us": append_us,
        "roofline": {"bound": "hbm", "kernel": "index_scores_stream", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "launch_us": round(score_us_mean, 3),
                     "timed_launches": len(score_us), "timed_every_nth_step": EVENT_STRIDE,
                     "algorithmic_bytes": bytes_per_launch, "bytes_per_pool": score_bytes_per_pool(),
                     "stream_ceiling": ceiling},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def read_stream_ceiling(reps, stream, calls: int = 64) -> dict:
    """The plain read-stream reference kernel (libdsa_probe.so) over the same
    64 MiB pool-cache buffers the score kernel reads, rotating through the
    replicas, each wave reading 32 KiB: the HBM bandwidth this machine delivers to
    a pure streaming read of that size, event-timed per launch."""
    import ctypes
    import torch
    from dsa_decode_amd import build_lib

    lib = ctypes.CDLL(build_lib.PROBE_LIB)
    lib.dsa_probe_read_stream.restype = ctypes.c_int
    lib.dsa_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_long, ctypes.c_void_p]
    bufs = [r["k_pool"] for r in reps]
    nbytes = bufs[0].numel() * bufs[0].element_size()
    ev = TimingEvents(2 * calls)
    with torch.cuda.stream(stream):
        for k in range(2 * len(bufs)):
            assert lib.dsa_probe_read_stream(bufs[k % len(bufs)].data_ptr(), nbytes, 32768, stream.cuda_stream) == 0
        stream.synchronize()
        for k in range(calls):
            ev.record(2 * k, stream.cuda_stream)
            lib.dsa_probe_read_stream(bufs[k % len(bufs)].data_ptr(), nbytes, 32768, stream.cuda_stream)
            ev.record(2 * k + 1, stream.cuda_stream)
        stream.synchronize()
    us = float(np.mean([ev.elapsed_us(2 * k, 2 * k + 1) for k in range(calls)]))
    ev.close()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "read_stream (plain 16-byte non-temporal loads, 32 KiB per wave)", "bytes": nbytes,
            "launch_us": round(us, 3), "achieved": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def step_with_append_us(wl, tok_dev, comp, bound, scores_stage, rest_stages, stream, steps: int) -> dict:
    """The decode step with the indexer-state update in front of it
    (dsa_kpool_append -> scores -> top-k + expand -> sparse MLA), event-timed
    per step.  With kpool 4, three decode tokens in four complete no pool (the
    append only reads the state) and the fourth completes one pool in every
    sequence; both kinds are timed (the state is rewound by one pool, outside
    the events, before each pool-forming step) and weighted 3:1."""
    import torch
    from dsa_decode_amd import ops

    st = {k: comp[k].clone() for k in ("k_pool", "pool_start", "pool_valid", "n_pools", "first_valid")}
    n_full = st["n_pools"].clone()
    n_back = (n_full - 1).clamp_min(0)
    res = {}
    with torch.cuda.stream(stream):
        # bound inside the stream context: a bound call launches on the stream current at bind time
        app = ops.bind_kpool_append(tok_dev["k"], tok_dev["gate"], tok_dev["valid"], tok_dev["ape"],
                                    tok_dev["seq_len"], wl.kp, st, 1)
        for name, rewind in (("no_new_pool_us", False), ("new_pool_us", True)):
            ev = TimingEvents(2 * steps)
            for i in range(steps):
                j = i % REPLICAS
                if rewind:
                    st["n_pools"].copy_(n_back)
                ev.record(2 * i, stream.cuda_stream)
                app()
                scores_stage(j)
                rest_stages(j)
                ev.record(2 * i + 1, stream.cuda_stream)
            stream.synchronize()
            res[name] = round(float(np.median([ev.elapsed_us(2 * i, 2 * i + 1) for i in range(steps)])), 2)
            ev.close()
    assert torch.equal(st["n_pools"], n_full)
    per_token = (3 * res["no_new_pool_us"] + res["new_pool_us"]) / 4
    res["mean_us_per_step"] = round(per_token, 2)
    res["steps_per_s"] = round(1e6 / per_token, 1)
    res["note"] = ("event-timed per step (median of each kind), weighted 3:1; the append updates its own copy "
                   "of the indexer state in front of the step's launches on the same stream")
    return res


def append_stage_us(wl, tok_dev, comp, stream, calls: int = 64) -> float:
    """Event-timed dsa_kpool_append for one decode token of every sequence that
    completes a pool: the state is rewound by one pool per sequence before each
    call (outside the timed events), so each call forms the newest pool of all
    4 sequences again, as the step that fills a pool would."""
    import torch
    from dsa_decode_amd import ops

    st = {k: comp[k].clone() for k in ("k_pool", "pool_start", "pool_valid", "n_pools", "first_valid")}
    n_full = st["n_pools"].clone()
    n_back = (n_full - 1).clamp_min(0)
    ev = TimingEvents(2 * calls)
    with torch.cuda.stream(stream):
        # bound inside the stream context: a bound call launches on the stream current at bind time
        call = ops.bind_kpool_append(tok_dev["k"], tok_dev["gate"], tok_dev["valid"], tok_dev["ape"],
                                     tok_dev["seq_len"], wl.kp, st, 1)
        for k in range(calls):
            st["n_pools"].copy_(n_back)
            ev.record(2 * k, stream.cuda_stream)
            call()
            ev.record(2 * k + 1, stream.cuda_stream)
        stream.synchronize()
    assert torch.equal(st["n_pools"], n_full)
    us = sorted(ev.elapsed_us(2 * k, 2 * k + 1) for k in range(calls))[calls // 2]
    ev.close()
    return round(float(us), 2)


def paged_mla_stages(wl, mi, q_lat, row_seq, tok, stream, calls: int = 64) -> dict:
    """Event-timed dsa_sparse_mla_decode_paged (main + combine launches) on the
    step's token ids, over the same latent cache laid out in 64-token pages:
    bf16 pages (1 KiB gathered per token) and fp8 E4M3 pages with a per-row
    scale (512 B + 4 B).  Eight shifted copies of the id lists rotate so that
    the gathered rows do not stay in the last-level cache between calls."""
    import torch
    from dsa_decode_amd import ops, synth

    res = {}
    Q, W = tok.shape
    toks = [((tok.long() + k * 8192) % wl.T_max).to(torch.int32).contiguous() for k in range(8)]
    toks = [torch.where(tok >= 0, t, tok) for t in toks]
    for name, fp8 in (("bf16_pages", False), ("fp8_pages", True)):
        pg = synth.paged_latent(mi["kv"], 64, seed=64, fp8=fp8)
        kvp = pg["kv_pages"].cuda()
        sc = pg["kv_scale"].cuda() if fp8 else None
        bt = pg["block_table"].cuda()
        del pg
        out = torch.empty((Q, wl.Hm, wl.Dl), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((Q, wl.Hm), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, ops.dsa_sparse_mla_paged_workspace_bytes(Q, wl.Hm, wl.Dl, W)), dtype=torch.uint8,
                         device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            # arguments marshalled once per id list (plain ctypes calls in the loop)
            bound = [ops.bind_sparse_mla_decode_paged(q_lat, kvp, sc, bt, 64, row_seq, toks[k], mi["sm_scale"],
                                                      out, lse, ws) for k in range(8)]
            run = lambda k: bound[k % 8]()
            for k in range(8):
                run(k)
            stream.synchronize()
            torch.cuda._sleep(2_000_000)  # the device starts behind the host: no launch gap is timed
            ev = TimingEvents(2 * calls)
            for k in range(calls):
                ev.record(2 * k, stream.cuda_stream)
                run(k)
                ev.record(2 * k + 1, stream.cuda_stream)
            stream.synchronize()
        res[name] = round(float(sorted(ev.elapsed_us(2 * k, 2 * k + 1) for k in range(calls))[calls // 2]), 2)
        ev.close()
        del kvp, sc, bt
        torch.cuda.synchronize()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def _timed_oracle(step_row, n_rows_per_unit: int, budget_s: float, threads: int | None):
    """Rows through step_row until about budget_s of CPU work -> (units/s,
    rows, seconds); threads limits the BLAS pool (None: as configured)."""
    from contextlib import nullcontext
    ctx = nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads)
    rows_done = 0
    with ctx:
        t0 = time.perf_counter()
        while True:
            step_row(rows_done)
            rows_done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
    return rows_done / n_rows_per_unit / el, rows_done, el


def cpu_baseline(wl, ip, mi, comp, budget_s: float) -> dict:
    """The oracle (as it is) on a bounded sample of the same step: decode rows of
    the same workload, each through scores -> top-k -> expand -> sparse MLA,
    repeated until about budget_s of CPU work; scaled to steps/s (4 rows/step).
    Timed on all the BLAS threads, then on one thread for a third of the budget."""
    from oracle import dsa_oracle as O
    from dsa_decode_amd.layout import untile_pool_cache

    cores = _oracle_threads()
    pc = dict(k_pool=untile_pool_cache(comp["k_pool"].cpu(), wl.P_max), pool_start=comp["pool_start"].cpu(),
              pool_valid=comp["pool_valid"].cpu())

    def step_row(i):
        r = i % wl.Q
        s = O.index_scores(ip["q"], ip["w"], ip["scale"], pc["k_pool"], pc["pool_start"], pc["pool_valid"],
                           ip["gamma"], ip["beta"], ip["eps"], ip["row_seq"], ip["row_pos"], wl.kp, rows=[r])
        ids = O.topk_pools(s, wl.K)
        tok = O.expand_selection(ids, ip["row_seq"].numpy()[[r]], pc["pool_start"].numpy(), wl.kp, wl.W)
        O.sparse_mla_decode(mi["q_lat"][[r]], mi["kv"], ip["row_seq"][[r]], tok, mi["sm_scale"])

    v, rows, el = _timed_oracle(step_row, wl.Q, budget_s, None)
    v1, rows1, el1 = _timed_oracle(step_row, wl.Q, budget_s / 3, 1)
    return {"value": round(v, 4), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "value_1_thread": round(v1, 4),
            "sample": f"{rows} decode rows of the same workload (scores over 65536 pools, top-k, expand, sparse "
                      f"MLA per row) in {el:.1f} s on {cores} threads, {rows1} rows in {el1:.1f} s on 1 thread; "
                      f"4 rows = 1 step"}


def cpu_baseline_prefill(wl, ip, mi, comp, k_pool, budget_s: float) -> dict:
    """The oracle (as it is) on a bounded sample of the prefill chunk: rows of the
    chunk, each through scores over the 32768 pools -> top-k -> expand -> sparse
    MLA, until about budget_s of CPU work; scaled to chunks/s (4096 rows/chunk)."""
    from oracle import dsa_oracle as O
    from dsa_decode_amd.layout import untile_pool_cache

    cores = _oracle_threads()
    kp_host = untile_pool_cache(k_pool.cpu(), wl.P_max)
    ps, pv = comp["pool_start"].cpu(), comp["pool_valid"].cpu()

    def step_row(i):
        r = (i * 997) % wl.Q
        s = O.index_scores(ip["q"], ip["w"], ip["scale"], kp_host, ps, pv, ip["gamma"], ip["beta"], ip["eps"],
                           ip["row_seq"], ip["row_pos"], wl.kp, rows=[r])
        ids = O.topk_pools(s, wl.K)
        tok = O.expand_selection(ids, ip["row_seq"].numpy()[[r]], ps.numpy(), wl.kp, wl.W)
        O.sparse_mla_decode(mi["q_lat"][[r]], mi["kv"], ip["row_seq"][[r]], tok, mi["sm_scale"])

    v, rows, el = _timed_oracle(step_row, wl.Q, budget_s, None)
    v1, rows1, el1 = _timed_oracle(step_row, wl.Q, budget_s / 3, 1)
    return {"value": round(v, 6), "unit": "chunks/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "value_1_thread": round(v1, 6),
            "sample": f"{rows} rows of the prefill chunk (scores over 32768 pools, top-k, expand, sparse MLA per "
                      f"row) in {el:.1f} s on {cores} threads, {rows1} rows in {el1:.1f} s on 1 thread; "
                      f"4096 rows = 1 chunk"}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def bench_prefill(args) -> int:
    """The prefill chunk (4096 query rows at the end of a 131072-token sequence,
    32768 pools).  A step is dsa_index_topk_pools_expand (index scores over
    every (row, pool) pair on the matrix cores, each row's candidates kept in a
    list instead of a score tensor, then top-k and expansion over the lists)
    followed by dsa_sparse_mla_decode over the selected tokens (the many-rows
    path).  The unfused dsa_index_scores + dsa_topk_pools_expand (same outputs,
    bit for bit) are timed beside it.  Inputs follow the workload recipe: q on
    the 1/8 grid, pooled keys from a 256-row codebook on the 1/8 grid (exact
    score ties straddle the cut), pool metadata from dsa_kpool_compress over
    the synthetic tokens.  Stages are timed per launch with events; the
    rooflines use the algorithmic flops (2*H*D per candidate pair for the
    scores, 4*Hm*Dl per listed id for the MLA)."""
    import numpy as np
    import torch

    from dsa_decode_amd import ops, synth
    from dsa_decode_amd.layout import tile_pool_cache

    dev = lambda t: t.contiguous().cuda()
    wl = synth.workload("prefill")
    Q, P, K, W = wl.Q, wl.P_max, wl.K, wl.W
    ti = synth.token_inputs(wl)
    comp = ops.dsa_kpool_compress(dev(ti["k"]), dev(ti["gate"]), dev(ti["valid"]), dev(ti["ape"]),
                                  dev(ti["seq_len"]), wl.kp, P)
    del ti
    ip = synth.index_params(wl)
    k_pool = dev(tile_pool_cache(synth.codebook_keys(wl)))
    q, w, gamma, beta = dev(ip["q"]), dev(ip["w"]), dev(ip["gamma"]), dev(ip["beta"])
    row_seq, row_pos = dev(ip["row_seq"]), dev(ip["row_pos"])
    scores = torch.empty((Q, P), dtype=torch.float32, device="cuda")
    ids = torch.empty((Q, K), dtype=torch.int32, device="cuda")
    tok = torch.empty((Q, W), dtype=torch.int32, device="cuda")
    tk_ws = ops.topk_workspace(ops.dsa_topk_workspace_bytes(Q, P, K))
    mi = synth.mla_inputs(wl)
    q_lat, kv = dev(mi["q_lat"]), dev(mi["kv"])
    out = torch.empty((Q, wl.Hm, wl.Dl), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Q, wl.Hm), dtype=torch.float32, device="cuda")
    mla_ws = torch.empty(max(1, ops.dsa_sparse_mla_workspace_bytes(Q, wl.Hm, wl.Dl, W, ops.DSA_BF16)),
                         dtype=torch.uint8, device="cuda")
    # candidate pairs: valid pools whose last token is at or before the row's position
    ps = comp["pool_start"][0].cpu().numpy().astype(np.int64)
    pv = comp["pool_valid"][0].cpu().numpy() != 0
    last = np.sort(ps[pv] + wl.kp - 1)
    pairs = int(np.searchsorted(last, ip["row_pos"].numpy().astype(np.int64), side="right").sum())
    flops = 2 * wl.H * wl.D * pairs
    st_ws = ops.topk_workspace(ops.dsa_index_topk_workspace_bytes(Q, P, K))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    with torch.cuda.stream(stream):
        stc = ops.bind_index_topk_pools_expand(q, w, ip["scale"], k_pool, comp["pool_start"], comp["pool_valid"],
                                               gamma, beta, ip["eps"], row_seq, row_pos, wl.kp, K, ids, tok, st_ws)
        ml = ops.bind_sparse_mla_decode(q_lat, kv, row_seq, tok, mi["sm_scale"], out, lse, mla_ws)
        for _ in range(args.warmup):
            stc()
            ml()
        stream.synchronize()
        tev = TimingEvents(3 * args.steps)
        t0 = time.perf_counter()
        for i in range(args.steps):
            tev.record(3 * i, sh)
            stc()
            tev.record(3 * i + 1, sh)
            ml()
            tev.record(3 * i + 2, sh)
        stream.synchronize()
        t1 = time.perf_counter()
    fused_us = float(np.mean([tev.elapsed_us(3 * i, 3 * i + 1) for i in range(args.steps)]))
    mla_us = float(np.mean([tev.elapsed_us(3 * i + 1, 3 * i + 2) for i in range(args.steps)]))
    tev.close()
    # the unfused stages on the same inputs: dsa_index_scores into a [Q, P]
    # tensor, then dsa_topk_pools_expand; their pool ids must be the step's
    u_ids = torch.empty_like(ids)
    u_tok = torch.empty_like(tok)
    with torch.cuda.stream(stream):
        sc = ops.bind_index_scores(q, w, ip["scale"], k_pool, comp["pool_start"], comp["pool_valid"], gamma, beta,
                                   ip["eps"], row_seq, row_pos, wl.kp, scores)
        tk = ops.bind_topk_pools_expand(scores, K, u_ids, row_seq, comp["pool_start"], wl.kp, u_tok, tk_ws)
        sc()
        tk()
        stream.synchronize()
        uev = TimingEvents(3 * args.steps)
        for i in range(args.steps):
            uev.record(3 * i, sh)
            sc()
            uev.record(3 * i + 1, sh)
            tk()
            uev.record(3 * i + 2, sh)
        stream.synchronize()
    if not (torch.equal(u_ids, ids) and torch.equal(u_tok, tok)):
        raise RuntimeError("the fused and the unfused scores -> top-k disagree")
    score_us = float(np.mean([uev.elapsed_us(3 * i, 3 * i + 1) for i in range(args.steps)]))
    topk_us = float(np.mean([uev.elapsed_us(3 * i + 1, 3 * i + 2) for i in range(args.steps)]))
    uev.close()
    ms = (t1 - t0) * 1e3 / args.steps
    achieved = flops / (score_us * 1e-6) / 1e12
    fused_achieved = flops / (fused_us * 1e-6) / 1e12
    topk_bytes = Q * P * 4 + Q * K * 4 + Q * W * 4
    # sparse MLA: per (row, listed id) 2*Hm*Dl flops for the logits and as many for the values
    listed = int((tok >= 0).sum().item())
    mla_flops = 4 * wl.Hm * wl.Dl * listed
    mla_achieved = mla_flops / (mla_us * 1e-6) / 1e12
    kernels = {
        # the step's two stages: the filtering score kernel + the top-k over
        # its lists (one entry point, timed together), and the sparse MLA
        "index_topk_pools_expand": {"launch_us": round(fused_us, 2), "achieved": round(fused_achieved, 1),
                                    "frac": round(fused_achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "algorithmic_flops": flops,
                                    "kernels": "index_scores_gemm<2, true> + topk_kernel<512, 4, false, true>"},
        "mla_rows64_pipe": {"launch_us": round(mla_us, 2), "achieved": round(mla_achieved, 1),
                              "frac": round(mla_achieved / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": mla_flops,
                              "listed_ids": listed},
        # the unfused score kernel (reference, not in the step)
        "index_scores_gemm": {"launch_us": round(score_us, 2), "achieved": round(achieved, 1),
                              "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops},
        # the unfused top-k + expand (reference): it reads the [Q, P] fp32 scores and writes the
        # pool ids and token ids, against the HBM peak
        "topk_pools_expand": {"launch_us": round(topk_us, 2), "algorithmic_bytes": topk_bytes,
                              "achieved": round(topk_bytes / (topk_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s",
                              "frac": round(topk_bytes / (topk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    dom = "index_topk_pools_expand" if fused_us >= mla_us else "mla_rows64_pipe"
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(wl, ip, mi, comp, k_pool, args.cpu_seconds)
    line = {
        "metric": "DSA prefill chunk (index_scores + top-k + expand + sparse MLA) chunks/s; % MFMA roofline",
        "value": round(1e3 / ms, 2), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill chunk: 4096 rows at positions 126976..131071 of a 131072-token "
                               "sequence, kpool 4 (32768 pools), 32 index heads x 128, select_k 512, bf16, "
                               "q and keys on the 1/8 grid (forced ties)",
                   "rows": Q, "pools": P, "select_k": K},
        "stages_us": {"index_topk_pools_expand": round(fused_us, 2), "sparse_mla_decode": round(mla_us, 2)},
        "unfused_stages_us": {"index_scores": round(score_us, 2), "topk_pools_expand": round(topk_us, 2)},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["achieved"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
                     "traffic": None, "launch_us": kernels[dom]["launch_us"],
                     "algorithmic_flops": kernels[dom]["algorithmic_flops"], "candidate_pairs": pairs},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

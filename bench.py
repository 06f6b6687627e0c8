#!/usr/bin/env python3
"""Throughput of the SMC-SD round on one MI355X.

One step = one full round (logits pass, finalize, page-table remap) over all R requests of
the workload, inputs resident in HBM. The log-weights and refcounts carry over from round
to round, and the two page-table buffers swap after each round (pointer exchange), so no
state is reset inside the timed region.

Prints one JSON line with:
  * value: rounds/s;
  * roofline of the dominant kernel (the logits pass): algorithmic bytes per launch, divided
    by its mean duration from HIP events the library records around that launch on the
    round's stream;
  * cpu_baseline: the CPU oracle timed on a bounded sample of the same workload.

Other paths (--path): sd_verify and gumbel_topk time those entry points on the same logits;
driver times the multi-round driver: an ESS-adaptive round followed by the page lifecycle
(release, copy-on-write of shared tail pages across every KV tensor, appends), with a
paged KV cache of --kv-tensors tensors and --kv-page-bytes per page in HBM.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# The sources each measured kernel is built from: stored counter results (HBM traffic) are
# reported only while these still hash to the value recorded with them.
KERNEL_SOURCES = {
    "k_logits_tv": ["k_logits_tv.hip", "logits_common.h", "smcsd_device.h", "smcsd_internal.h"],
    "k_logits_stream": ["k_logits_stream.hip", "logits_common.h", "smcsd_device.h",
                        "smcsd_internal.h"],
    "k_topk_slice": ["k_topk.hip", "smcsd_device.h", "smcsd_internal.h"],
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "smc_particle_resampling_amd", "csrc", p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles for timing kernels on a given stream (plumbing over libamdhip64)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def record(self, e, stream: int):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def read_roofline(smcsd, torch, dev, gib=4):
    """Attainable HBM read GB/s: plain streaming read of `gib` GiB (best of 3)."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    best = 0.0
    for _ in range(4):
        torch.cuda.synchronize()
        t = time.perf_counter()
        smcsd.smcsd_bench_stream_read(buf, sink, 2048)
        torch.cuda.synchronize()
        best = max(best, n / (time.perf_counter() - t) / 1e9)
    del buf
    return best


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    p = os.path.join(PROFILES, "traffic_k_logits_%s.json" % workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if kernel not in KERNEL_SOURCES:
        return None
    hashes = d.get("kernel_source_sha256_16")
    if not isinstance(hashes, dict) or hashes.get(kernel) != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch_by_kernel", {}).get(kernel)


def flush_caches(buf):
    """Overwrite a buffer larger than the L2s and the Infinity Cache together, so that the
    next round finds none of its inputs on chip."""
    buf.add_(1)


def cpu_model() -> str:
    """The host CPU's model name (for the CPU baseline's record), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_driver(w, pool_args, target_s=12.0, sample_requests=2):
    """The oracle's round plus its page lifecycle on a bounded sample: the first requests of
    the workload with a page pool of the same geometry (KV tensors zero-filled), each pass
    timed with a wall clock; driver steps/s = 1 / (R * seconds per request)."""
    import numpy as np

    import oracle
    from smc_particle_resampling_amd import synth
    rs = min(w.R, sample_requests)
    small = w.scaled(R=rs)
    host = synth.to_host(synth.make_inputs(small, 11, device="cpu", pages=False))
    ps, P, kv_tensors, page_bytes, token_rows = pool_args
    pool = synth.make_page_pool(rs, w.N, P, ps, 11, steps=w.K + 1, spare=256)
    num_pages = pool["refcount"].numel()
    kv = np.zeros((kv_tensors, num_pages, page_bytes), np.uint8)
    host.update(page_table=pool["page_table"].numpy(), refcount=pool["refcount"].numpy())
    times = []
    while not times or (sum(times) < target_s and len(times) < 1000):
        t = time.perf_counter()
        ora = oracle.round(host, V=w.V, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv)
        oracle.pages_advance(ora["page_table"], ora["refcount"], pool["free_ids"].numpy(),
                             pool["n_free"], pool["len_before"].numpy(),
                             pool["len_after"].numpy(), ps, kv, kv_inplace=True,
                             token_rows=token_rows)
        times.append(time.perf_counter() - t)
    per_request = sum(times) / (len(times) * rs)
    return {"value": 1.0 / (w.R * per_request), "unit": "driver steps/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": "%d of %d requests (N=%d, K=%d, V=%d, TV %s, %s resampling) with a pool of "
                      "%d pages x %d KV tensors x %d B: fp64 oracle round then the oracle's "
                      "page lifecycle (its KV copies included), repeated %d times (%.1f s in "
                      "all), %.4f s per request; driver steps/s = 1/(%d * that)" % (
                          rs, w.R, w.N, w.K, w.V, "on" if w.tv else "off", w.mode, num_pages,
                          kv_tensors, page_bytes, len(times), sum(times), per_request, w.R)}


def cpu_baseline(w, target_s=12.0, sample_requests=4, path="round", k=8):
    """The oracle (as it is) on a bounded sample of the workload: the first few requests
    (all N particles, K positions, V logits each), timed with a wall clock around
    oracle.round and repeated until ~target_s of CPU work; rounds/s = 1 / (R * seconds per
    request)."""
    import numpy as np

    import oracle
    from smc_particle_resampling_amd import synth
    rs = min(w.R, sample_requests)
    small = w.scaled(R=rs)
    inputs = synth.make_inputs(small, 11, device="cpu", pages=path == "round")
    if path == "sd_verify":
        inputs.update(synth.make_verify_uniforms(rs, w.N, w.K, 11, device="cpu"))
    host = synth.to_host(inputs)
    if path == "gumbel_topk":
        tz, tT, tG = (np.ascontiguousarray(x) for x in (
            host["target"][:, :, 0].reshape(rs * w.N, -1),
            np.repeat(host["temperature"], w.N), host["gumbel"].reshape(rs * w.N, -1)))
    times = []
    while not times or (sum(times) < target_s and len(times) < 1000):
        t = time.perf_counter()
        if path == "gumbel_topk":
            oracle.gumbel_topk(tz, tT, tG, k, V=w.V)
        elif path == "sd_verify":
            oracle.sd_verify(host, V=w.V)
        else:
            oracle.round(host, V=w.V, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv)
        times.append(time.perf_counter() - t)
    per_request = sum(times) / (len(times) * rs)
    unit = "rounds/s" if path == "round" else "passes/s"
    what = {"round": "round", "sd_verify": "SD verification",
            "gumbel_topk": "Gumbel-Top-K (k=%d) of every particle row" % k}[path]
    return {"value": 1.0 / (w.R * per_request), "unit": unit, "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": "%d of %d requests (N=%d, K=%d, V=%d, TV %s), fp64 oracle %s over them "
                      "repeated %d times (%.1f s in all), %.4f s per request; %s = "
                      "1/(%d * that)" % (rs, w.R, w.N, w.K, w.V, "on" if w.tv else "off", what,
                                         len(times), sum(times), per_request, unit, w.R)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 20 for --path driver, whose page pool "
                         "grows with the run)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 5; 3)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-roofline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run N launches of a plain 1 GiB copy (for counter scaling)")
    ap.add_argument("--flush", action="store_true",
                    help="write a 1 GiB buffer before every timed round (evicts the L2s and the "
                         "Infinity Cache) and time each round alone with events around all its "
                         "launches; value is then 1 / mean round time")
    ap.add_argument("--path", choices=("round", "sd_verify", "gumbel_topk", "driver"),
                    default="round",
                    help="round: one SMC-SD round (smcsd_round, the headline); sd_verify: "
                         "standard speculative-decoding verification of the same blocks "
                         "(smcsd_sd_verify); gumbel_topk: Gumbel-Top-K drafting of k tokens "
                         "per particle row (smcsd_gumbel_topk); driver: an ESS-adaptive round "
                         "then the page lifecycle (smcsd_round + smcsd_pages_advance)")
    ap.add_argument("--topk", type=int, default=8, help="k of --path gumbel_topk")
    ap.add_argument("--bonus", choices=("pass", "after"), default="pass",
                    help="round / driver: draw the bonus inside the logits pass per original "
                         "particle (pass), or after resampling per new slot with fresh noise "
                         "(after: smcsd_round without noise, then smcsd_bonus_resampled)")
    ap.add_argument("--vocab-shards", type=int, default=1,
                    help="round: run one GPU's share of a vocabulary-sharded target, V/G "
                         "columns per row (the cross-GPU combine of the partials is not built)")
    ap.add_argument("--kv-tensors", type=int, default=64,
                    help="driver: KV tensors sharing the page ids (32 layers x K and V)")
    ap.add_argument("--kv-token-rows", action="store_true",
                    help="driver: token-major KV pages (a token pool's layout); copy-on-write "
                         "moves only the tail's filled token rows")
    ap.add_argument("--kv-page-bytes", type=int, default=32768,
                    help="driver: bytes of one page in one KV tensor (16 tokens x 8 KV heads x "
                         "128 dims x bf16)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 20 if args.path == "driver" else 50
    if args.warmup is None:
        args.warmup = 3 if args.path == "driver" else 5

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the round shards by request with no "
              "communication, so N GPUs run N independent copies of this line.", file=sys.stderr)
        sys.exit(2)

    import torch
    from smc_particle_resampling_amd import smcsd, synth

    name = args.workload or synth.HEADLINE
    w = synth.WORKLOADS[name]
    if args.vocab_shards > 1:
        share = -(-w.V // args.vocab_shards)
        share = -(-share // 8) * 8            # whole 16-byte rows
        w = w.scaled(V=share, name="%s-vshard1of%d" % (name, args.vocab_shards))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("# building inputs for %s" % name, file=sys.stderr, flush=True)
    verify = args.path == "sd_verify"
    topk = args.path == "gumbel_topk"
    driver = args.path == "driver"
    if driver:
        w = w.scaled(mode="ess")
    inp = synth.make_inputs(w, 0, device=dev, pages=args.path == "round")
    after = args.bonus == "after" and args.path in ("round", "driver")
    bonus_noise = synth.make_gumbel(w, 1, device=dev) if after else None
    ev = HipEvents()
    # per timed step: (begin, split, end) around the logits pass; split separates the bonus-row
    # kernel of a TV pass from the row-pair kernel after it (else it is recorded with end)
    pairs = [(ev.create(), ev.create(), ev.create()) for _ in range(args.steps)]
    rounds = [(ev.create(), ev.create()) for _ in range(args.steps)] if args.flush else None
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush else None
    calls = None            # the round's marshalled calls (round path only)
    if topk:
        tz, tT, tG = synth.topk_rows(inp)
        out = smcsd.gumbel_topk(tz, tT, tG, args.topk, V=w.V)
        out["error_flags"] = torch.zeros((1,), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream(dev).cuda_stream

        def step(t, timing=None):
            if timing is not None:
                ev.record(timing[0], cur)
            smcsd.gumbel_topk(tz, tT, tG, args.topk, V=w.V, outputs=out)
            if timing is not None:
                ev.record(timing[1], cur)
                ev.record(timing[2], cur)
    elif verify:
        inp.update(synth.make_verify_uniforms(w.R, w.N, w.K, 0, device=dev))
        out = smcsd.run_sd_verify(inp)          # allocates the outputs once
        torch.cuda.synchronize()

        def step(t, timing=None):
            smcsd.run_sd_verify(inp, outputs=out,
                                timing_events=None if timing is None else (timing[0], timing[2]))
            if timing is not None:
                ev.record(timing[1], torch.cuda.current_stream(dev).cuda_stream)
    elif driver:
        # Page pool: every particle's length grows K + 1 tokens a step; the table holds a
        # context of up to 256 tokens before the first step plus what the run appends, and
        # the free list starts with enough pages for every append even if nothing is
        # released.
        ps = 16
        total = args.warmup + 2 * args.steps      # the timed pass and the event pass
        grow = -(-(total * (w.K + 1)) // ps) + 1       # columns the run appends, at most
        P = 16 + grow
        pool = synth.make_page_pool(w.R, w.N, P, ps, 0, steps=total * (w.K + 1),
                                    spare=w.R * w.N * grow)
        num_pages = pool["refcount"].numel()
        pool_gib = num_pages * args.kv_tensors * args.kv_page_bytes / 2**30
        if pool_gib > 160:
            raise SystemExit("page pool of %.0f GiB for %d steps does not fit beside the logits; "
                             "use fewer --steps or smaller --kv-tensors / --kv-page-bytes"
                             % (pool_gib, total))
        print("# page pool: %d pages x %d KV tensors x %d B = %.1f GiB" % (
            num_pages, args.kv_tensors, args.kv_page_bytes,
            num_pages * args.kv_tensors * args.kv_page_bytes / 2**30), file=sys.stderr, flush=True)
        kv = torch.zeros((args.kv_tensors, num_pages, args.kv_page_bytes), dtype=torch.uint8,
                         device=dev)
        inp["page_table"] = pool["page_table"].to(dev)
        inp["refcount"] = pool["refcount"].to(dev)
        free_ids = pool["free_ids"].to(dev)
        n_free = torch.tensor([pool["n_free"]], dtype=torch.int32, device=dev)
        lens = torch.stack([pool["len_before"] + t * (w.K + 1) for t in range(total + 1)])
        lens = lens.to(torch.int32).to(dev)
        stats = torch.zeros((total, 5), dtype=torch.int32, device=dev)
        pws = torch.empty(smcsd.smcsd_pages_workspace_size(w.R, w.N, P, num_pages),
                          dtype=torch.uint8, device=dev)
        out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=w.tv, V=w.V,
                                  dtype=smcsd.BF16 if w.dtype == "bf16" else smcsd.F32)
        tables = [inp["page_table"], torch.empty_like(inp["page_table"])]
        life = [(ev.create(), ev.create()) for _ in range(args.steps)]
        cur = torch.cuda.current_stream(dev).cuda_stream
        torch.cuda.synchronize()

        def step(t, timing=None):
            out["page_table_out"] = tables[(t + 1) % 2]
            inp["page_table"] = tables[t % 2]
            smcsd.run_round(inp, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv, outputs=out,
                            timing_events=timing, bonus_noise=bonus_noise)
            lt = life[t - args.warmup - args.steps] if timing is not None else None
            if lt:
                ev.record(lt[0], cur)
            smcsd.smcsd_pages_advance(len_before=lens[t], len_after=lens[t + 1],
                                      page_table=out["page_table_out"],
                                      refcount=inp["refcount"], free_ids=free_ids,
                                      n_free=n_free, page_size=ps, workspace=pws, kv=kv,
                                      token_rows=args.kv_token_rows, stats=stats[t],
                                      error_flags=out["error_flags"])
            if lt:
                ev.record(lt[1], cur)
    elif after:
        torch.cuda.synchronize()
        out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=w.tv, V=w.V,
                                  dtype=smcsd.BF16 if w.dtype == "bf16" else smcsd.F32)
        tables = [inp["page_table"], torch.empty_like(inp["page_table"])]

        def step(t, timing=None):
            out["page_table_out"] = tables[(t + 1) % 2]
            inp["page_table"] = tables[t % 2]
            smcsd.run_round(inp, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv, outputs=out,
                            timing_events=timing, bonus_noise=bonus_noise)
    else:
        # The round's arguments are marshalled once per page-table parity (the tables swap
        # every round, as a caller's pointer exchange would); each step enqueues a whole
        # round, so no per-call Python work sits between the GPU's rounds.
        torch.cuda.synchronize()
        out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=w.tv, V=w.V,
                                  dtype=smcsd.BF16 if w.dtype == "bf16" else smcsd.F32)
        tables = [inp["page_table"], torch.empty_like(inp["page_table"])]
        calls = [smcsd.RoundCall(
            target_logits=inp["target"], draft_logits=inp["draft"], draft_tokens=inp["tokens"],
            temperature=inp["temperature"], gumbel=inp["gumbel"], uniform=inp["uniform"],
            log_weights=inp["log_weights"], log_w_incr=out["log_w_incr"],
            log_norm=out["log_norm"], ess=out["ess"], resampled=out["resampled"],
            ancestors=out["ancestors"], bonus=out["bonus"], out_tokens=out["out_tokens"],
            tv=out["tv"], page_table_in=tables[p], page_table_out=tables[1 - p],
            refcount=inp["refcount"], error_flags=out["error_flags"], workspace=out["workspace"],
            V=w.V, mode=w.mode, ess_frac=w.ess_frac) for p in (0, 1)]

        def step(t, timing=None):
            calls[t % 2].launch(timing_events=timing)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    cur_stream = torch.cuda.current_stream(dev).cuda_stream
    # Timed steps: whole rounds back to back (or, with --flush, each after the cache flush,
    # timed by events around all of its launches). No event sits inside a round here: each
    # costs a few microseconds of queue time, which a small round would pay several times.
    t0 = time.perf_counter()
    for t in range(args.steps):
        if args.flush:
            flush_caches(flush_buf)
            ev.record(rounds[t][0], cur_stream)
        step(args.warmup + t)
        if args.flush:
            ev.record(rounds[t][1], cur_stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Kernel times: the same number of rounds again, with HIP events recorded by the library
    # on the round's stream around the logits pass and between its two kernels.
    for t in range(args.steps):
        if args.flush:
            flush_caches(flush_buf)
        step(args.warmup + args.steps + t, timing=pairs[t])
    torch.cuda.synchronize()
    flags = int(out["error_flags"].item())
    if flags:
        raise SystemExit("device error flags %d" % flags)
    kms = [ev.elapsed_ms(a, e) for a, _, e in pairs]
    first_ms = [ev.elapsed_ms(a, sp) for a, sp, _ in pairs]     # TV pass: the bonus rows
    second_ms = [ev.elapsed_ms(sp, e) for _, sp, e in pairs]    # TV pass: the row pairs
    for trio in pairs:
        for x in trio:
            ev.destroy(x)
    k_mean_ms = sum(kms) / len(kms)
    # The pass alone, `steps` times back to back between one pair of events
    # (smcsd_bench_logits_pass): its time without an event around each launch. An event costs
    # microseconds of queue time, which a short single-kernel pass would otherwise carry.
    batch_ms = None
    if calls is not None and not args.flush:
        b0, b1 = ev.create(), ev.create()
        ev.record(b0, cur_stream)
        calls[0].bench_pass(args.steps)
        ev.record(b1, cur_stream)
        torch.cuda.synchronize()
        batch_ms = ev.elapsed_ms(b0, b1) / args.steps
        ev.destroy(b0)
        ev.destroy(b1)
    if args.flush:
        rms = [ev.elapsed_ms(a, b) for a, b in rounds]
        ms_per_step = sum(rms) / len(rms)
    else:
        ms_per_step = elapsed * 1e3 / args.steps
    alg = w.algorithmic_bytes()
    logits_bytes = alg["target"] + alg["draft"] + alg["noise"]
    if after:       # the timed pass reads the row pairs only; the bonus is drawn afterwards
        logits_bytes = alg["target"] * w.K // (w.K + 1) + alg["draft"]
    if topk:        # one logits row and one noise row per particle
        e = 2 if w.dtype == "bf16" else 4
        logits_bytes = w.R * w.N * w.V * (e + 4)
    # The dominant kernel: with TV on and the bonus drawn in the pass, the row-pair kernel
    # (k_logits_tv, timed split..end) reads every drafted position's target and draft row;
    # otherwise one kernel is the whole pass.
    split = w.tv and not after and args.path in ("round", "driver")
    if batch_ms is not None:
        k_mean_ms = batch_ms
    if split:
        dom_bytes = alg["target"] * w.K // (w.K + 1) + alg["draft"]
        dom_ms = sum(second_ms) / len(second_ms)
        dom_kernel = "k_logits_tv"
    else:
        dom_bytes, dom_ms = logits_bytes, k_mean_ms
        dom_kernel = ("k_topk_slice+k_topk_merge" if topk else
                      "k_logits_tv+k_topk_slice (bonus rows)" if verify else
                      "k_logits_tv" if w.tv else "k_logits_stream")
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    pass_achieved = logits_bytes / (k_mean_ms * 1e-3) / 1e9
    print("# %s %.3f ms, logits pass %.3f ms (min %.3f max %.3f), %s %.3f ms" % (
        args.path, ms_per_step, k_mean_ms, min(kms), max(kms), dom_kernel, dom_ms),
        file=sys.stderr, flush=True)

    lifecycle = None
    if driver:
        lms = [ev.elapsed_ms(a, b) for a, b in life]
        st = stats[args.warmup:].cpu().numpy()
        copied = float(st[:, 2].mean())
        # read + write of every copied token row in every tensor
        moved = 2.0 * float(st[:, 4].mean()) * (args.kv_page_bytes // ps) * args.kv_tensors
        lifecycle = {"ms_mean": sum(lms) / len(lms), "ms_min": min(lms), "ms_max": max(lms),
                     "released_per_step": float(st[:, 0].mean()),
                     "pops_per_step": float(st[:, 1].mean()),
                     "pages_copied_per_step": copied,
                     "token_rows_copied_per_step": float(st[:, 4].mean()),
                     "pops_unserved": int(st[:, 3].sum()),
                     "kv_copy_bytes_per_step": moved,
                     "kv_copy_GBps_over_lifecycle": moved / (sum(lms) / len(lms) * 1e-3) / 1e9}
        if lifecycle["pops_unserved"]:
            raise SystemExit("page pool ran dry: %d pops unserved" % lifecycle["pops_unserved"])
        print("# lifecycle %.3f ms, %.1f pages copied / step" % (lifecycle["ms_mean"], copied),
              file=sys.stderr, flush=True)

    for _ in range(args.copy_calibration):
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        smcsd.smcsd_bench_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    rr = None if args.no_read_roofline else read_roofline(smcsd, torch, dev)
    if args.no_cpu_baseline:
        cpu = None
    elif driver:
        cpu = cpu_baseline_driver(w, (ps, P, args.kv_tensors, args.kv_page_bytes,
                                      args.kv_token_rows))
    else:
        cpu = cpu_baseline(w, path=args.path, k=args.topk)
    if driver:
        metric = ("SMC-SD driver steps/s (ESS-adaptive round + page lifecycle with KV "
                  "copy-on-write), N=32 K=8 V=128256 bf16")
        unit = "steps/s"
        table_bytes = alg["table"]
    elif topk:
        metric = ("Gumbel-Top-K drafting passes/s and achieved HBM GB/s (%% of peak), "
                  "%d rows V=%d bf16 k=%d" % (w.R * w.N, w.V, args.topk))
        unit = "passes/s"
        table_bytes = 0
    elif verify:
        metric = ("SD verification passes/s and achieved HBM GB/s (% of peak), "
                  "N=32 K=8 V=128256 bf16")
        unit = "passes/s"
        table_bytes = 0
    else:
        metric = "SMC-SD rounds/s and achieved HBM GB/s (% of peak), N=32 K=8 V=128256 bf16"
        if args.vocab_shards > 1:
            metric += ", one GPU's vocabulary shard (1/%d, V=%d)" % (args.vocab_shards, w.V)
        unit = "rounds/s"
        table_bytes = alg["table"]
    line = {
        "metric": metric,
        "value": (1e3 / ms_per_step) if args.flush else args.steps / elapsed,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: logits widened exactly to f32, exponentials and sums in f32, the
        # per-request weights in f64; the logits themselves are stored as config.logits_dtype
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "path": args.path, "R": w.R, "N": w.N, "K": w.K, "V": w.V,
                   "logits_dtype": w.dtype,
                   "tv": (w.tv or verify) and not topk,
                   "resample": w.mode if args.path in ("round", "driver") else None,
                   "pages_per_particle": (w.P if args.path == "round" else
                                          P if driver else None),
                   "kv_cache": ({"tensors": args.kv_tensors, "page_bytes": args.kv_page_bytes,
                                 "page_tokens": ps, "pages": num_pages,
                                 "copy": "filled token rows" if args.kv_token_rows else "whole pages"}
                                if driver else None),
                   "topk": args.topk if topk else None,
                   "vocab_shard": ("1/%d: V = %d of %d" % (args.vocab_shards, w.V,
                                                          synth.WORKLOADS[name].V)
                                   if args.vocab_shards > 1 else None),
                   "bonus": (args.bonus if args.path in ("round", "driver") else None),
                   "timing": ("each round alone (events around all its launches) after a 1 GiB "
                              "write that evicts the L2s and the Infinity Cache" if args.flush
                              else "rounds back to back, wall clock over the timed steps") +
                             "; kernel times from events in a second pass of as many rounds" +
                             ("; the pass time from the pass alone run back to back as many times "
                              "between two events" if batch_ms is not None else ""),
                   "round_GBps": (logits_bytes + table_bytes) / (ms_per_step * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": (None if (topk or verify or after or args.vocab_shards > 1)
                                 else stored_traffic(name, dom_kernel)),
                     "kernel": dom_kernel,
                     "kernel_ms": dom_ms,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "attainable_read_GBps": rr,
                     "pass": {"kernels": ("k_logits_tv+k_topk_slice (bonus rows)" if split
                                          else dom_kernel),
                              "ms": k_mean_ms, "bytes": logits_bytes, "GBps": pass_achieved,
                              "frac": pass_achieved / PEAK_HBM_GBPS,
                              "bonus_rows_ms": (sum(first_ms) / len(first_ms)) if split else None}},
        "cpu_baseline": cpu,
    }
    if driver:
        line["lifecycle"] = lifecycle
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Decode-step benchmark of retrieval-sparse paged decode attention on one GPU.

A step is one layer's decode step for the whole batch, one rkv_decode_step
call: write the token and a just-completed block's representation, score the
offload blocks (one launch), then the per-(sequence, KV head) top-k, the
merged block table and the split-K paged attention (for a batch of one the
top-k and merge run inside the attention launch; otherwise a top-k launch
precedes it), then the log-sum-exp combine.  The host tier's step is
rkv_append_select -> staging -> rkv_decode_attn, and adds the staging of kept host-resident blocks on a side
stream (rkv_stage_resident, which copies only blocks no staging slot
holds; copying every kept block, rkv_stage_blocks + rkv_merge_table, is
timed beside it).
Inputs are synthetic and already resident in HBM when timing starts.

Consecutive steps cycle over `--layers` independent copies of the layer's
KV cache (as a model's layers would), so a step never finds the previous
step's pages in the 256 MB Infinity Cache.

After the headline workload (`--config`, default the Llama-3-8B-shaped
layer) the same run measures the other workloads of the metric's 64K-128K
range and the host tier (`--also`, default 3,4,5), each in a child process
of its own (a workload measured after another in one process runs a few
percent slower): each with its own steps/s, the roofline of its attention
call and the CPU oracle on a bounded sample, under "configs" in the JSON
line.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
if "--wave-timeline" in sys.argv:
    # the per-wave timestamps need the RKV_WAVE_STAMPS build of the library
    os.environ.setdefault("RKV_LIB", os.path.join(ROOT, "sparse_retrieval_kv_amd",
                                                  "librkv_stamps.so"))

from sparse_retrieval_kv_amd import binding as B  # noqa: E402
from sparse_retrieval_kv_amd import synth  # noqa: E402
from sparse_retrieval_kv_amd.decode import DecodeSession, HostTierSession  # noqa: E402

HBM_PEAK_GBS = 8000.0

# HBM bytes moved by the timed attention call (both of its kernels:
# rkv_select_attend for a batch of one, rkv_decode_attn otherwise), from
# two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB
# per dispatch, mean over the dispatches of the timed steps).  Each counter
# is scaled by what it reads for a plain 1 GiB device-to-device copy:
# FETCH_SIZE reads 524315.6 KiB (x2.0), WRITE_SIZE 1048576 KiB (x1.0).
# A record holds only for the attention source it was taken on; after any
# change to that file the figure is reported as null until measured again.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
ATTN_SOURCE = os.path.join(ROOT, "sparse_retrieval_kv_amd", "csrc", "attn.hip")
MEASURED_TRAFFIC = {
    # config: (sha256 prefix of attn.hip, FETCH_SIZE KiB, WRITE_SIZE KiB) of
    # the attention call's kernels (split or folded kernel + combine; for the
    # host tier the calls over the whole merged table)
    2: ("82fad60adbd6b78b", 40090.5 + 646.0, 1048.9 + 16.0),
    3: ("82fad60adbd6b78b", 751662.1 + 832.0, 1302.6 + 256.0),
    4: ("82fad60adbd6b78b", 506474.3 + 1277.0, 2081.1 + 256.0),
    5: ("82fad60adbd6b78b", 474836.9 + 686.0, 1040.3 + 64.0),
}
METRIC = "decode attn steps/s and attended-KV HBM GB/s (% of peak) at 64K-128K ctx, 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def step_bytes(spec, context, t):
    """Algorithmic bytes of one step: attended K+V (bf16) per (sequence, KV
    head), the fp32 representations the scorer reads, and the K+V of the
    kept offload blocks (what the host tier stages)."""
    kv = reps = kept = 0
    for L0 in context:
        L = int(L0) + t
        nb = -(-L // 128)
        n_init = min(-(-spec.init_tokens // 128), nb)
        ls = min(max(L - spec.local_tokens, 0) // 128, nb - 1)
        n_off = max(ls - n_init, 0)
        dense = L0 < spec.dense_boundary or spec.topk_ppm >= 1_000_000
        k = n_off if dense else -(-(n_off * spec.topk_ppm) // 1_000_000)
        n_merged = n_init + k + (nb - max(ls, n_init))
        tokens = 128 * (n_merged - 1) + (L - 128 * (nb - 1))
        kv += tokens * 128 * 2 * 2
        if not dense and 0 < k < n_off:
            reps += n_off * 128 * 4
        kept += k * 128 * 128 * 2 * 2
    return kv * spec.n_kv_heads, reps * spec.n_kv_heads, kept * spec.n_kv_heads


def attn_traffic(args, config):
    """Counter-measured HBM bytes per attention call, or None when no
    record exists for this config, launch and attention source.  The records
    were taken with the default launch (MFMA, automatic split, per-head
    selection, default layer copies)."""
    if (args.impl not in ("auto", "mfma") or args.split != 0 or
            args.select != "per-head" or args.layers != 0):
        return None
    rec = MEASURED_TRAFFIC.get(config)
    if rec is None:
        return None
    with open(ATTN_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if not sha.startswith(rec[0]):
        return None
    return 1024.0 * (rec[1] * COUNTER_SCALE["FETCH_SIZE"] +
                     rec[2] * COUNTER_SCALE["WRITE_SIZE"])


def fused_select_attend(args, spec, max_blocks):
    """Whether the library folds the top-k into the attention launch for this
    launch: a batch of one, MFMA attention, per-head selection, at most 1024
    blocks per sequence."""
    return (spec.batch == 1 and args.impl != "valu" and args.select == "per-head"
            and max_blocks <= 1024)


def attn_kernel_label(impl, spec, fused=False):
    """The kernels the timed attention call launches; the split kernel is
    templated on its partition (true: a batch of one sequence)."""
    if fused:
        return "rkv_select_attend (attn_select_mfma_kernel + attn_combine_kernel)"
    strided = "true" if spec.batch == 1 else "false"
    split = (f"attn_valu_kernel<{spec.group}, {strided}>" if impl == "valu"
             else f"attn_mfma_kernel<{strided}>")
    return f"rkv_decode_attn ({split} + attn_combine_kernel)"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return None


def cpu_baseline(batch, host=None, budget_s=12.0, max_steps=100000):
    """Time the float64 oracle's decode step on the host over a bounded
    sample of the same workload (first sequence of the batch)."""
    import oracle as O
    spec = batch.spec
    prm = O.Params(spec.n_q_heads, spec.n_kv_heads, spec.init_tokens,
                   spec.local_tokens, spec.topk_ppm, spec.dense_boundary)
    b = 0
    L0 = int(batch.context[b])
    nb = -(-(L0 + spec.steps - 1) // 128)
    pages = torch.as_tensor(batch.table_np[b, :nb].astype(np.int64),
                            device=batch.k_pages.device)
    kp = batch.k_pages.index_select(0, pages).cpu().numpy().view(np.uint16)
    vp = batch.v_pages.index_select(0, pages).cpu().numpy().view(np.uint16)
    if host is not None:  # blocks kept in host memory: read the host pools
        ht = host.host_table_np[b, :nb]
        on = np.nonzero(ht >= 0)[0]
        hp = torch.as_tensor(ht[on].astype(np.int64))
        kp[on] = host.host_k.index_select(0, hp).numpy().view(np.uint16)
        vp[on] = host.host_v.index_select(0, hp).numpy().view(np.uint16)
    K, V = O.logical_kv(kp, vp, np.arange(nb), L0 + spec.steps - 1)
    reps = np.stack([O.block_reps(K[h]) for h in range(spec.n_kv_heads)])
    n = 0
    t0 = time.perf_counter()
    while n < max_steps and time.perf_counter() - t0 < budget_s:
        t = n % spec.steps
        q = O.bf16_to_f64(batch.q_bits(t)[b].cpu().numpy().view(np.uint16))
        O.decode_step(q, K, V, L0 + t, L0, prm, reps=reps)
        n += 1
    dt = time.perf_counter() - t0
    threads = blas_threads() or torch.get_num_threads()
    # one sequence of the batch per oracle step -> scale to batch steps
    seq_steps_per_s = n / dt
    return {
        "value": seq_steps_per_s / spec.batch,
        "unit": "steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} oracle decode steps of sequence 0 ({L0} tokens, "
                   f"{spec.n_q_heads}/{spec.n_kv_heads} heads, float64 NumPy, "
                   f"representations precomputed), {dt:.1f} s; value = "
                   f"sequence-steps/s / batch {spec.batch}"),
        "host": platform.processor() or platform.machine(),
        "nproc": os.cpu_count(),
    }


def measure_prefill(sess, host, lens, spec):
    """Prefill hand-over to the host tier on one layer: the representation
    build alone, the offload copies alone, both on two streams, and the
    hand-over as HostTierSession.offload_prefill runs it (build, then
    copies); each timed between HIP events on the main stream.  Leaves the
    pools filled and the reps built."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        torch.cuda.synchronize()
        ev[0].record()
        fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3

    t_reps = timed(lambda: sess.build_reps(lens))
    t_off = timed(lambda: B.offload_blocks(sess.p, sess.k_pages, sess.v_pages,
                                           sess.block_table, lens, host.host_table,
                                           host.host_k, host.host_v))
    t_conc = timed(lambda: sess.offload_prefill(host.host_k, host.host_v,
                                                host.host_table, lens, concurrent=True))
    t_both = timed(lambda: sess.offload_prefill(host.host_k, host.host_v,
                                                host.host_table, lens))
    lens_np = lens.cpu().numpy()
    complete = int(sum(int(L) // 128 for L in lens_np))
    reps_bytes = complete * spec.n_kv_heads * 128 * 128 * 2
    off_bytes = int((host.host_table_np >= 0).sum()) * spec.n_kv_heads * 128 * 128 * 2 * 2
    out = {"reps_bytes": reps_bytes, "reps_ms": t_reps * 1e3,
           "reps_gbs": reps_bytes / t_reps / 1e9,
           "offload_bytes": off_bytes, "offload_ms": t_off * 1e3,
           "offload_gbs": off_bytes / t_off / 1e9,
           "handover_ms": t_both * 1e3, "handover_two_streams_ms": t_conc * 1e3}
    log(f"prefill: reps {out['reps_gbs']:.0f} GB/s ({out['reps_ms']:.2f} ms), "
        f"offload {out['offload_gbs']:.1f} GB/s ({out['offload_ms']:.1f} ms), "
        f"hand-over {out['handover_ms']:.1f} ms (two streams: "
        f"{out['handover_two_streams_ms']:.1f} ms)")
    return out


def measure_copy_engines(sess, spec, qs, news, lens, T, t_last, kept, gather_us, dev):
    """Host tier through the copy engines (rkv_stage_*_async: coalesced
    hipMemcpy2DAsync / hipMemcpyAsync on the side stream) beside the gather
    kernel: every kept block staged per call, decode steps with residency,
    and the HBM read rate another stream gets while each mode stages; then
    the copies over four copy lanes.  Leaves the session in the
    gather-kernel mode, without lanes, with empty slots."""
    out = {}

    def full_and_resident():
        """Every kept block staged per call (wall clock: the call waits for
        the kept ids on the host, then issues the copies; the time runs until
        they are done), then decode steps with residency from empty slots,
        as the timed steps run."""
        n_st = 4
        sess.copy_mode, sess.resident = "memcpy", False
        sess.stage(lens[t_last])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_st):
            sess.stage(lens[t_last])
        torch.cuda.synchronize()
        full_us = (time.perf_counter() - t0) * 1e6 / n_st
        sess.resident = True
        sess.reset_residency()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(T):
            kn, vn = news[t]
            sess.step(qs[t], kn, vn, lens[t])
        torch.cuda.synchronize()
        step_us = (time.perf_counter() - t0) * 1e6 / T
        return ({"bytes_per_step": float(kept), "avg_us": full_us,
                 "gbs": kept / (full_us * 1e-6) / 1e9}, step_us)

    out["full"], step_us = full_and_resident()
    full_us = out["full"]["avg_us"]
    out["resident_step_us"] = step_us
    out["resident_steps_per_s"] = 1e6 / step_us
    log(f"copy engines: full staging {full_us:.0f} us ({out['full']['gbs']:.1f} GB/s); "
        f"steps with residency {step_us:.0f} us (gather kernel: full {gather_us:.0f} us)")

    # HBM readers beside staging: rkv_read_probe over 1 GiB on its own
    # stream, alone and while every kept block is staged by either mode
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    ps = torch.cuda.Stream(device=dev)

    def probe_rate(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(ps):
            e0.record()
            for _ in range(n):
                B.read_probe(buf, sink)
            e1.record()
        return n, e0, e1

    def finish(ev):
        torch.cuda.synchronize()
        n, e0, e1 = ev
        return n * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9

    torch.cuda.synchronize()
    out["read_probe_alone_gbs"] = finish(probe_rate(8))
    probe_us = (1 << 30) / (out["read_probe_alone_gbs"] * 1e9) * 1e6
    main = torch.cuda.current_stream(dev)
    for mode, mode_us in (("kernel", gather_us), ("memcpy", full_us)):
        sess.copy_mode, sess.resident = mode, False
        torch.cuda.synchronize()
        # probes first (they start at once), then the staging: probes covering
        # about half the staging time all run beside it
        ev = probe_rate(max(4, int(0.5 * mode_us / probe_us)))
        if mode == "kernel":
            sess.side.wait_stream(main)
            with torch.cuda.stream(sess.side):
                sess.stage(lens[t_last])
        else:
            sess.stage(lens[t_last])  # copies queued on the side stream
        out[f"read_probe_beside_{mode}_gbs"] = finish(ev)
    del buf
    log(f"HBM read probe: alone {out['read_probe_alone_gbs']:.0f} GB/s, beside the "
        f"gather kernel {out['read_probe_beside_kernel_gbs']:.0f} GB/s, beside the copy "
        f"engines {out['read_probe_beside_memcpy_gbs']:.0f} GB/s")

    # the copies spread over copy lanes (rkv_params.copy_lanes), measured
    # last: the lanes are streams of this process, and streams created after
    # them would share the runtime's hardware queues with them
    n_lanes = 4
    sess.p.copy_lanes = n_lanes
    try:
        lanes_full, lanes_step_us = full_and_resident()
    finally:
        sess.p.copy_lanes = 0
    out["lanes"] = {"copy_lanes": n_lanes, "full": lanes_full,
                    "resident_step_us": lanes_step_us,
                    "resident_steps_per_s": 1e6 / lanes_step_us}
    log(f"copy engines over {n_lanes} lanes: full staging {lanes_full['avg_us']:.0f} us "
        f"({lanes_full['gbs']:.1f} GB/s); steps with residency {lanes_step_us:.0f} us")
    sess.copy_mode, sess.resident = "kernel", True
    sess.reset_residency()
    torch.cuda.synchronize()
    out["path"] = ("kept ids (or the residency planner's copy list) to pinned host "
                   "memory, then one hipMemcpy2DAsync per run of consecutive blocks "
                   "and KV head (whole pages in the per-sequence mode) on the side "
                   "stream (under 'lanes': spread over that many streams forked from "
                   "and joined back to it); the main stream waits on an event")
    return out


def stream_read_probe(dev, gib=2, reps=5):
    """Achievable streaming-read bandwidth: rkv_read_probe over a buffer
    larger than the Infinity Cache, median of `reps` timed launches."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    B.read_probe(buf, sink)
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.read_probe(buf, sink)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del buf
    return (gib << 30) / (sorted(ms)[len(ms) // 2] * 1e-3) / 1e9


def measure_cascade(sessions, spec, q, lens, reps, plain_us, context, t):
    """The attention call with the shared-prefix cascade (each attended tile
    of the shared prefix read once per group of sequences) against the
    plain call over the same merged tables; tiles counted from the session's
    selections."""
    S = spec.shared_prefix_pages
    n_layers = len(sessions)
    for s_ in sessions:  # sizes each session's cascade workspace once
        s_.attend_cascade(q, lens, S)
    ev0, ev1 = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    ev0.record()
    for i in range(reps):
        sessions[i % n_layers].attend_cascade(q, lens, S)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    # attended shared tiles: per list (plain reads) and per group of 16 / G
    # sequences (cascade reads); init blocks plus kept blocks below the
    # prefix end (the window lies past it at these lengths)
    sess = sessions[0]
    sel, ns = sess.sel_ids.cpu().numpy(), sess.n_sel.cpu().numpy()
    G = spec.group
    Q = min(max(16 // G, 1), spec.batch)
    n_init = -(-spec.init_tokens // 128)
    per_list, per_group = 0, 0
    for h in range(spec.n_kv_heads):
        for g0 in range(0, spec.batch, Q):
            union = set()
            for b in range(g0, min(g0 + Q, spec.batch)):
                L = int(context[b]) + t
                se = min(S, (L - 1) // 128)
                att = set(range(min(n_init, se))) | {int(j) for j in sel[b, h, :ns[b, h]]
                                                     if j < se}
                per_list += len(att)
                union |= att
            per_group += len(union)
    tile = 2 * 128 * 128 * 2  # K and V of one (page, KV head)
    log(f"cascade: {us:.1f} us per call vs {plain_us:.1f} us plain; shared tiles "
        f"{per_group} read vs {per_list}")
    return {"call": ("rkv_decode_attn_cascade (cascade_prep_kernel, attn_mfma_kernel<false> "
                     "with cascade waves, attn_combine_kernel)"),
            "avg_us": us, "plain_avg_us": plain_us, "speedup": plain_us / us,
            "shared_blocks": S, "sequences_per_tile_read": Q,
            "shared_tiles_plain": per_list, "shared_tiles_cascade": per_group,
            "bytes_saved": (per_list - per_group) * tile}


def wave_timeline(args, dev, reps=4):
    """Per-wave timeline of the 8B layer's folded-selection attention launch
    (the RKV_WAVE_STAMPS build): the decode step runs over eight layer copies
    as in the timed run, and the stamps of the last step's launch are read
    back.  Prints percentiles of each event over the waves, in us from the
    launch's first wave start, the unit completions per microsecond and the
    finish times by unit count."""
    spec = synth.CONFIGS[2]
    base = synth.make_batch(spec, dev)
    prm = B.params(spec.n_q_heads, spec.n_kv_heads, init_tokens=spec.init_tokens,
                   local_tokens=spec.local_tokens, topk_ppm=spec.topk_ppm,
                   dense_boundary=spec.dense_boundary)
    ctx = torch.as_tensor(base.context.astype(np.int32), device=dev)
    n_layers = args.layers or 8
    sessions = []
    for layer in range(n_layers):
        kp = base.k_pages if layer == 0 else base.k_pages.clone()
        vp = base.v_pages if layer == 0 else base.v_pages.clone()
        sess = DecodeSession(prm, kp, vp, base.block_table, ctx)
        sess.build_reps(ctx - 1)
        sessions.append(sess)
    T = spec.steps
    names = ["wave start", "scores and table row arrived", "selection found",
             "first unit's V tile requested", "merged list in LDS", "wave done"]
    pct = (0, 10, 50, 90, 100)
    print(f"per-wave timeline, {spec.name}: {n_layers} layer copies, "
          f"{args.steps} steps per read-out, us from the first wave's start "
          f"(percentiles {'/'.join(map(str, pct))})", flush=True)
    for rep in range(reps):
        for i in range(args.steps):
            t = (rep * args.steps + i) % T
            kn, vn = base.new_kv_bits(t)
            sessions[i % n_layers].step(base.q_bits(t), kn, vn,
                                        torch.as_tensor(base.lens_at(t), device=dev))
        torch.cuda.synchronize()
        st = B.wave_stamps(B.WAVE_STAMP_WAVES).astype(np.int64)
        st = st[st[:, 0] > 0]
        t0 = st[:, 0].min()
        us = lambda x: (x - t0) / 100.0  # noqa: E731
        print(f"read-out {rep}: {len(st)} waves", flush=True)
        for k, name in enumerate(names):
            col = st[:, k if k < 5 else 5]
            col = col[col > 0]
            print(f"  {name:30s} " + " ".join(f"{np.percentile(us(col), p):6.2f}"
                                               for p in pct), flush=True)
        units = st[:, 7:]
        done_units = us(units[units > 0])
        n_units = (units > 0).sum(axis=1)
        hist = np.bincount(np.floor(done_units).astype(int))
        print("  unit completions per 1 us window: " +
              " ".join(f"{w}:{c}" for w, c in enumerate(hist) if c), flush=True)
        for n in sorted(set(n_units.tolist())):
            sel = n_units == n
            print(f"  waves with {n} units: {sel.sum()}, done median "
                  f"{np.median(us(st[sel, 5])):.2f} max {us(st[sel, 5]).max():.2f}",
                  flush=True)


def run_workload(args, config, steps, warmup, cpu_budget, probe_gbs, dev,
                 spread_budget=None):
    """Build one workload, time `steps` decode steps after `warmup`, the
    attention call alone, the host tier's staging (host-tier workload) and
    the CPU oracle on a bounded sample.  Returns the workload's record."""
    spec = synth.CONFIGS[config]
    log("config", config, spec.name)
    host = None
    prefill = None
    if spec.host_offload:
        max_blocks = -(-(max(spec.context) + spec.steps - 1) // 128)
        base = synth.make_batch(spec, dev, extra_pages=spec.batch * max_blocks)
    else:
        base = synth.make_batch(spec, dev)
    layer_bytes = 2 * base.k_pages.numel() * 2
    # >= 2 GiB of layers between two visits of one layer: nothing of it (pages,
    # representations, tables) is left in the 256 MB Infinity Cache, as in a
    # model with many layers (with 1 GiB, ~2% of the 8B step stayed warm)
    n_layers = args.layers or max(1, min(16, math.ceil((2 << 30) / layer_bytes)))
    impl = {"auto": B.ATTN_AUTO, "mfma": B.ATTN_MFMA, "valu": B.ATTN_VALU}[args.impl]
    prm = B.params(spec.n_q_heads, spec.n_kv_heads, init_tokens=spec.init_tokens,
                   local_tokens=spec.local_tokens, topk_ppm=spec.topk_ppm,
                   dense_boundary=spec.dense_boundary, attn_impl=impl,
                   split_waves=args.split,
                   select_mode=(B.SELECT_PER_SEQUENCE if args.select == "per-sequence"
                                else B.SELECT_PER_HEAD))
    ctx = torch.as_tensor(base.context.astype(np.int32), device=dev)
    sessions = []
    for layer in range(n_layers):
        kp = base.k_pages if layer == 0 else base.k_pages.clone()
        vp = base.v_pages if layer == 0 else base.v_pages.clone()
        if spec.host_offload:
            # prefill hand-over: the offload blocks go to pinned host memory
            # while the representations are built; then the device copies
            # are poisoned so only the host copies carry the data
            # every prompt of this workload is beyond the dense boundary, so
            # a list keeps at most ceil(ratio * max_blocks) blocks
            kept_max = -(-base.table_np.shape[1] * spec.topk_ppm // 1_000_000)
            s = HostTierSession(prm, kp, vp, base.block_table, ctx,
                                slot_cap=int(args.slots * kept_max))
            host = synth.plan_host_pools(base)
            prefill = measure_prefill(s, host, ctx - 1, spec)
            synth.poison_device_copies(base, host)
            log(f"host tier: {host.host_k.numel() * 4 / 2**30:.2f} GiB of K/V "
                "in pinned host memory")
        else:
            s = DecodeSession(prm, kp, vp, base.block_table, ctx)
            s.build_reps(ctx - 1)
        sessions.append(s)
    log(f"{n_layers} layer copies, {layer_bytes / 2**20:.0f} MiB each")

    T = spec.steps
    qs = [base.q_bits(t) for t in range(T)]
    news = [base.new_kv_bits(t) for t in range(T)]
    lens = [torch.as_tensor(base.lens_at(t), device=dev) for t in range(T)]
    torch.cuda.synchronize()

    def run(s_idx, overlap=None):
        layer = s_idx % n_layers
        t = (s_idx // n_layers) % T
        sess = sessions[layer]
        kn, vn = news[t]
        if host is not None and t == 0:
            # each pass over the workload's T steps is a fresh decode after
            # prefill: nothing staged yet (the queries repeat from pass to
            # pass, so kept staging slots would otherwise see them again)
            sess.reset_residency()
        if host is None:
            sess.step(qs[t], kn, vn, lens[t])
            return t
        if (not args.no_overlap) if overlap is None else overlap:
            # the copies overlap the attention over the blocks already in HBM
            sess.step_overlapped(qs[t], kn, vn, lens[t])
            return t
        sess.append_select(qs[t], kn, vn, lens[t])
        # stage the kept host blocks on the side stream
        main = torch.cuda.current_stream(dev)
        sess.side.wait_stream(main)
        with torch.cuda.stream(sess.side):
            sess.stage(lens[t])
        main.wait_stream(sess.side)
        sess.attend(qs[t], lens[t])
        return t

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    log(f"warmup {warmup} done; timing {steps} steps")

    # timed region: K whole steps, nothing else on the stream
    ts = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ts.append(run(warmup + i))
    t_enq = time.perf_counter()  # host side done: every step is enqueued
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    # the host's enqueue time per step; well below the step time means the
    # wall-clock figure is the GPU's
    host_us_per_step = (t_enq - t0) * 1e6 / steps

    # spread of the step time: the same steps again in chunks of 16 between
    # HIP event pairs (the pair's own cost, ~10 us, spreads over the chunk)
    chunk = 16
    n_chunks = max(1, min(16, steps // chunk, (spread_budget or steps) // chunk))
    ev_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(n_chunks)]
    base_idx = warmup + steps
    torch.cuda.synchronize()
    for c_i, (e0, e1) in enumerate(ev_pairs):
        e0.record()
        for i in range(chunk):
            run(base_idx + c_i * chunk + i)
        e1.record()
    torch.cuda.synchronize()
    chunk_us = np.array([a.elapsed_time(b) * 1e3 / chunk for a, b in ev_pairs])
    step_spread = {"chunk_steps": chunk, "chunks": n_chunks}
    if n_chunks >= 3:
        step_spread.update({"p10_us": float(np.percentile(chunk_us, 10)),
                            "p50_us": float(np.percentile(chunk_us, 50)),
                            "p90_us": float(np.percentile(chunk_us, 90))})
    else:  # percentiles of one or two chunks would say nothing
        step_spread.update({"chunk_us": [float(x) for x in chunk_us],
                            "note": f"{n_chunks} chunk(s) of {chunk} steps: too few "
                                    "for percentiles"})

    # the step's attention call alone, replayed on every layer copy between
    # one pair of HIP events on its stream (an event pair per launch would
    # add its own overhead to every launch): for a batch of one the
    # selection + attention call over the scores the last step left
    # (rkv_select_attend: one launch with the top-k folded in, + combine),
    # otherwise rkv_decode_attn over the current merged tables
    reps_attn = max(steps, 2 * n_layers)
    t_last = ts[-1]
    if host is not None and not args.no_overlap:
        # the overlapped steps leave only the resident entries in the merged
        # table: the attention replay below runs over the whole table, as the
        # plain step does (slots then hold step t_last's kept blocks)
        for s_ in sessions:
            s_.side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(s_.side):
                s_.stage(lens[t_last])
            torch.cuda.current_stream(dev).wait_stream(s_.side)
    ev0, ev1 = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    fused = host is None and fused_select_attend(args, spec, base.table_np.shape[1])
    torch.cuda.synchronize()
    ev0.record()
    for i in range(reps_attn):
        if fused:
            sessions[i % n_layers].select_attend(qs[t_last], lens[t_last])
        else:
            sessions[i % n_layers].attend(qs[t_last], lens[t_last])
    ev1.record()
    torch.cuda.synchronize()
    attn_us = ev0.elapsed_time(ev1) * 1e3 / reps_attn
    kv_attn = step_bytes(spec, base.context, t_last)[0]
    # for context beside the folded call: rkv_decode_attn alone over the
    # merged tables the replayed calls wrote (no selection work)
    attn_only = None
    if fused:
        torch.cuda.synchronize()
        ev0.record()
        for i in range(reps_attn):
            sessions[i % n_layers].attend(qs[t_last], lens[t_last])
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / reps_attn
        attn_only = {"kernel": attn_kernel_label(args.impl, spec), "avg_us": us,
                     "achieved_gbs": kv_attn / (us * 1e-6) / 1e9,
                     "frac": kv_attn / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}

    cascade = None
    if host is None and spec.shared_prefix_pages > 0 and spec.batch > 1 \
            and args.impl != "valu":
        cascade = measure_cascade(sessions, spec, qs[t_last], lens[t_last], reps_attn,
                                  attn_us, base.context, t_last)

    staging = None
    if host is not None:
        sess = sessions[0]
        kept = step_bytes(spec, base.context, t_last)[2]
        # every kept block copied (no residency), timed alone; it overwrites
        # the staging slots, so the residency state is reset afterwards
        n_st = 8
        sess.resident = False
        torch.cuda.synchronize()
        ev0.record()
        for i in range(n_st):
            sess.stage(lens[t_last])
        ev1.record()
        torch.cuda.synchronize()
        sess.resident = True
        sess.reset_residency()
        st_us = ev0.elapsed_time(ev1) * 1e3 / n_st
        # residency: blocks copied per step when the step sequence is
        # replayed from empty slots (step 0 copies every kept block)
        copied = []
        for t in range(T):
            kn, vn = news[t]
            sess.append_select(qs[t], kn, vn, lens[t])
            sess.stage(lens[t])
            sess.attend(qs[t], lens[t])
            torch.cuda.synchronize()
            copied.append(int(sess.n_staged.sum().item()))
        tile2 = 2 * 128 * 128 * 2  # K + V bytes of one block of one head
        steady = copied[1:] if len(copied) > 1 else copied
        staging = {
            "full": {"bytes_per_step": float(kept), "avg_us": st_us,
                     "gbs": kept / (st_us * 1e-6) / 1e9},
            "resident": {"slots_per_list": sess.slot_cap,
                         "blocks_copied_first_step": copied[0],
                         "blocks_copied_per_step": float(np.mean(steady)),
                         "bytes_per_step": float(np.mean(steady)) * tile2,
                         "fraction_of_full": float(np.mean(steady)) * tile2 / kept},
            "path": ("pinned host DRAM -> HBM staging slots by a gather kernel reading "
                     "host memory, side stream; timed steps use residency across steps "
                     "(first-in first-out slot reuse) and, unless --no-overlap, copy "
                     "while the blocks already in HBM are attended (step_overlapped)"),
        }
        log(f"full staging {st_us:.0f} us ({staging['full']['gbs']:.1f} GB/s); "
            f"residency copies {staging['resident']['fraction_of_full'] * 100:.0f}% "
            "of the kept bytes per step")
        staging["copy_engines"] = measure_copy_engines(sess, spec, qs, news, lens, T,
                                                       t_last, kept, st_us, dev)
        # the same steps in the other schedule: plain (staging, then the
        # attention over the whole table) or overlapped (the planner in split
        # mode, the copies on the side stream while the main stream attends
        # the blocks already in HBM, then the newly staged ones folded in)
        torch.cuda.synchronize()
        t0o = time.perf_counter()
        for i in range(steps):
            run(i * n_layers, overlap=args.no_overlap)
        torch.cuda.synchronize()
        other_us = (time.perf_counter() - t0o) * 1e6 / steps
        ovl_us = ms_per_step * 1e3 if not args.no_overlap else other_us
        plain_us = other_us if not args.no_overlap else ms_per_step * 1e3
        staging["overlapped"] = {
            "timed_steps": "plain" if args.no_overlap else "overlapped",
            "step_us": ovl_us, "plain_step_us": plain_us,
            "path": ("rkv_stage_plan (split mode) -> side stream: rkv_stage_copy; "
                     "main: rkv_decode_attn_lse over the entries already in HBM, then "
                     "over the newly staged ones with the first part folded in")}
        log(f"overlapped step: {ovl_us:.0f} us, plain step {plain_us:.0f} us")

    kv_b = np.array([step_bytes(spec, base.context, t)[0] for t in ts], dtype=np.float64)
    rep_b = np.array([step_bytes(spec, base.context, t)[1] for t in ts], dtype=np.float64)
    step_gbs = (kv_b.sum() + rep_b.sum()) / wall / 1e9
    attn_gbs = kv_attn / (attn_us * 1e-6) / 1e9
    log(f"{ms_per_step * 1e3:.1f} us/step, attention {attn_us:.1f} us avg "
        f"({attn_gbs:.0f} GB/s), step-level {step_gbs:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(base, host, budget_s=cpu_budget)

    return {
        "workload": spec.name,
        "config_id": config,
        "steps": steps,
        "warmup": warmup,
        "steps_per_s": steps / wall,
        "ms_per_step": ms_per_step,
        "batch": spec.batch,
        "context": [int(x) for x in base.context[:4]],
        "heads_q_kv": [spec.n_q_heads, spec.n_kv_heads],
        "init_local_topk_ppm": [spec.init_tokens, spec.local_tokens, spec.topk_ppm],
        "layer_copies": n_layers,
        "step_us_spread": step_spread,
        "host_enqueue_us_per_step": host_us_per_step,
        "host_staging": staging,
        "host_prefill": prefill,
        "attended_kv_gbs_step": step_gbs,
        "attended_kv_pct_peak_step": 100.0 * step_gbs / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm",
            "kernel": attn_kernel_label(args.impl, spec, fused),
            "achieved": attn_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": attn_gbs / HBM_PEAK_GBS,
            "frac_of_read_probe": attn_gbs / probe_gbs,
            "traffic": attn_traffic(args, config),
            "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per call, "
                               "scaled by a 1 GiB copy's readings"),
            "bytes_per_launch": float(kv_attn),
            "avg_launch_us": float(attn_us),
            "decode_attn_alone": attn_only,
            "cascade": cascade,
            "timing": (f"{reps_attn} back-to-back "
                       f"{'rkv_select_attend' if fused else 'rkv_decode_attn'} calls over "
                       f"the {n_layers} layer copies between one HIP event pair"),
        },
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--layers", type=int, default=0,
                    help="KV-cache copies cycled over (0: enough to exceed 1 GiB)")
    ap.add_argument("--impl", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--slots", type=float, default=2.0,
                    help="host tier: staging slots per (sequence, KV head), as a "
                         "multiple of the kept-block capacity")
    ap.add_argument("--select", default="per-head", choices=["per-head", "per-sequence"],
                    help="selection per (sequence, KV head) or once per sequence")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="host tier: time the plain step (staging, then the attention "
                         "over the whole table) instead of the one whose copies overlap "
                         "the attention over the blocks already in HBM")
    ap.add_argument("--also", default="3,4,5",
                    help="other workloads measured after the headline one in the "
                         "same run (comma-separated config ids; empty: none)")
    ap.add_argument("--record-only", action="store_true",
                    help="measure --config alone and print its record as one JSON "
                         "line (how the --also workloads are run, each in a process "
                         "of its own)")
    ap.add_argument("--probe-gbs", type=float, default=0.0,
                    help="streaming-read probe figure to report (0: measure it)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle steps for the cpu_baseline sample")
    ap.add_argument("--spread-budget", type=int, default=0,
                    help="steps timed for step_us_spread (0: up to 16 chunks of 16)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first "
                         "(a known-size reference for HBM byte counters)")
    ap.add_argument("--wave-timeline", action="store_true",
                    help="print the per-wave timeline of the 8B layer's attention "
                         "launch (librkv_stamps.so, --steps steps per read-out) "
                         "instead of timing")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.wave_timeline:
        wave_timeline(args, dev)
        return
    torch.cuda.set_device(dev)
    B.lib()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1 GiB read + 1 GiB written")

    if args.probe_gbs > 0:
        probe_gbs = args.probe_gbs
    else:
        probe_gbs = stream_read_probe(dev)
        log(f"streaming-read probe: {probe_gbs:.0f} GB/s")

    if args.record_only:
        rec = run_workload(args, args.config, args.steps, args.warmup, args.cpu_budget,
                           probe_gbs, dev, spread_budget=args.spread_budget or None)
        print(json.dumps(rec), flush=True)
        return

    head = run_workload(args, args.config, args.steps, args.warmup, args.cpu_budget,
                        probe_gbs, dev, spread_budget=args.spread_budget or None)
    gc.collect()
    torch.cuda.empty_cache()
    # each further workload in a process of its own: a workload measured
    # after another in the same process ran 3-4% slower (the batched and 70B
    # attention calls, in either order)
    others = {}
    extra = [int(x) for x in args.also.split(",") if x.strip()] if args.also else []
    for c in extra:
        if c == args.config:
            continue
        steps_c = synth.CONFIGS[c].steps * (2 if synth.CONFIGS[c].steps < 32 else 1)
        cmd = [sys.executable, os.path.abspath(__file__), "--config", str(c), "--also", "",
               "--steps", str(steps_c), "--warmup", "16", "--record-only",
               "--probe-gbs", repr(probe_gbs), "--cpu-budget", "4.0",
               "--spread-budget", str(steps_c), "--impl", args.impl,
               "--split", str(args.split), "--slots", repr(args.slots),
               "--select", args.select, "--layers", str(args.layers)]
        if args.no_cpu_baseline:
            cmd.append("--no-cpu-baseline")
        if args.no_overlap:
            cmd.append("--no-overlap")
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
        if r.returncode != 0 or not lines:
            log(f"config {c} failed (exit status {r.returncode})")
            others[str(c)] = {"error": f"exit status {r.returncode}"}
        else:
            others[str(c)] = json.loads(lines[-1])

    res = {
        "metric": METRIC,
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "bf16 K/V/q on MFMA, fp32 accumulation, softmax and output",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, planted blocks per config)",
        "config": {
            "workload": head["workload"],
            "config_id": args.config,
            "batch": head["batch"],
            "context": head["context"],
            "heads_q_kv": head["heads_q_kv"],
            "init_local_topk_ppm": head["init_local_topk_ppm"],
            "layer_copies": head["layer_copies"],
            "attn_impl": args.impl,
            "split_waves": args.split,
            "select": args.select,
        },
        "step_us_spread": head["step_us_spread"],
        "host_enqueue_us_per_step": head["host_enqueue_us_per_step"],
        "stream_read_probe_gbs": probe_gbs,
        "host_staging": head["host_staging"],
        "host_prefill": head["host_prefill"],
        "attended_kv_gbs_step": head["attended_kv_gbs_step"],
        "attended_kv_pct_peak_step": head["attended_kv_pct_peak_step"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        # the other workloads of the metric's 64K-128K range (and the host
        # tier), each measured in this same run: steps/s, roofline of its
        # attention call, CPU oracle on a bounded sample
        "configs": others,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

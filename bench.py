#!/usr/bin/env python3
"""Benchmark of the chunked causal attention prefill over a Q8_0 KV cache on one MI355X.

Prints ONE JSON line on stdout.  A step is one pass of the whole hot path over one batch of
synthetic input that is already resident in HBM: Q8_0 pack of K and V (FP32 in, 68-byte rows
out), the state (described with deferred initialisation: the first chunk call writes every row),
one attn_accumulate_chunk_final call per chunk (each writes the final out and lse of the rows
its chunk completes, and not their dead state), so no separate init or finalize launch.  The
default workload is 8 sequences x 32 heads x 2048 causal queries over 2048 keys, head_dim 64,
chunks of 512 keys (four chunk calls): the M = 2048, 32-head Q8_0 prefill.

value     = causal attention FLOPs per step (4 * 64 per visible (query, key) pair per head) /
            step time, in TFLOP/s.
value is timed over --steps steps with no instrumentation inside the timed region; a second
pass records an event at every step boundary and gives the median and minimum step.
roofline  = the accumulate kernel (the dominant one): algorithmic FLOPs per launch / its mean
            launch duration from HIP events recorded around every launch on the launch stream
            in a second, separately timed pass, against the dense FP16 MFMA peak of MI355X
            (2.5 PFLOP/s).  traffic = HBM bytes per launch from rocprofv3
            FETCH_SIZE / WRITE_SIZE counters (scaled by a plain-copy calibration), read from
            profiles/ and reported only if the kernel source is unchanged since.
cpu_baseline = the FP64 CPU oracle (pack + single-pass attention) on whole heads of the same
            workload, for about --cpu-seconds of host time; its outputs also check the GPU
            output of those heads.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attention TFLOP/s & % of MI355X FP16 MFMA peak (Q8_0 KV)"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense FP16 MFMA
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "accumulate_batch8_m2048_traffic.txt")
KERNEL_SOURCES = ["chunked_flashattention_q8_amd/csrc/attn.hip",
                  "chunked_flashattention_q8_amd/csrc/q8attn_internal.h"]


def code_tokens(src: str) -> str:
    """The source with its comments and its whitespace outside string and character literals
    removed, so that an edit of a comment or of layout leaves it unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif c.isspace():
            i += 1
        else:
            out.append(c)
            i += 1
    return "".join(out)


def kernel_source_hash() -> str:
    """SHA-256 of the accumulate kernel's code (comments and layout excluded): the key under
    which the committed HBM traffic summary is valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()


def chunk_flops(w, kv_pos0, n_kv):
    """Algorithmic FLOPs of one chunk call: 256 per visible (query, key) pair per head."""
    import numpy as np
    pos = w.q_pos0 + np.arange(w.M, dtype=np.int64)
    vis = np.clip(pos - kv_pos0 + 1, 0, n_kv)
    return int(vis.sum()) * w.B * w.H * 4 * w.D


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of `mib` MiB, for calibrating HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))


STEP_FORMS = {
    "lean": "deferred state init (no launch) + chunk calls writing the final out/lse of the "
            "rows each completes, without their dead state",
    "fused": "init launch + chunk calls writing the final rows (their state as well)",
    "plain": "init launch + plain chunk calls + a finalize launch",
}


def run_resident(w, kv_dtype, chunk, steps, warmup, inputs=None, graph=True, form="lean"):
    """Time the resident step of workload w; inputs = (q, k, v) already drawn for w, or None.
    graph=False skips the captured-graph pass and the append measurement.  form (STEP_FORMS):
    "lean" describes the state with attn_state_init_deferred and Q8A_STATE_FINAL_OUT_ONLY, and
    its chunk calls (attn_accumulate_chunk_final) write the final output of the rows each
    completes; "fused" is the same after an attn_state_init launch, keeping the completed rows'
    state; "plain" is an init launch, attn_accumulate_chunk calls and a finalize launch.  With
    lean and fused, attn_finalize runs only if some rows are left (queries past the end of the
    cache)."""
    import numpy as np
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    if inputs is None:
        q = synthetic.gen_q(w)
        k, v = synthetic.gen_kv(w)
    else:
        q, k, v = inputs
    qd = torch.from_numpy(q).view(torch.float16).to(dev)
    if kv_dtype == q8a.KV_Q8_0:
        # K and V side by side, FP32 and packed, so that one q8_0_pack call packs both (its rows
        # are independent): one launch instead of two
        kvx = torch.empty((2, w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
        kvx[0].copy_(torch.from_numpy(k))
        kvx[1].copy_(torch.from_numpy(v))
        kx, vx = kvx[0], kvx[1]
        kvd = torch.empty((2, w.B, w.H, w.N, 68), dtype=torch.uint8, device=dev)
        kd, vd = kvd[0], kvd[1]
    else:
        kd = torch.from_numpy(synthetic.to_f16_bits(k)).view(torch.float16).to(dev)
        vd = torch.from_numpy(synthetic.to_f16_bits(v)).view(torch.float16).to(dev)
    row = q8a.ROW_BYTES[kv_dtype]
    m, l, o = q8a.alloc_state(w.B, w.H, w.M, dev)
    out = torch.empty((w.B, w.H, w.M, w.D), dtype=torch.float16, device=dev)
    lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev)
    chunks = [(s, min(chunk, w.N - s)) for s in range(0, w.N, chunk)]
    acc_flops = [chunk_flops(w, s, n) for s, n in chunks]
    n_rows = w.B * w.H * w.N

    ev = {"pack": [], "init": [], "accumulate": [], "finalize": []}

    def timed(name, fn, record):
        if record:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
        else:
            fn()

    fused = form != "plain"

    def step(record):
        if kv_dtype == q8a.KV_Q8_0:
            timed("pack", lambda: q8a.q8_0_pack(kvx, kvd, 2 * n_rows, 64), record)
        st = [None]

        def init():
            st[0] = q8a.attn_state_init(m, l, o, w.B, w.H, w.M, w.D, w.q_pos0)
        if form == "lean":
            st[0] = q8a.attn_state_init_deferred(m, l, o, w.B, w.H, w.M, w.D, w.q_pos0,
                                                 q8a.STATE_FINAL_OUT_ONLY)
        else:
            timed("init", init, record)
        kp, vp = kd.data_ptr(), vd.data_ptr()
        for s, n in chunks:
            if fused:
                timed("accumulate",
                      lambda s=s, n=n: q8a.attn_accumulate_chunk_final(
                          st[0], qd, kp + s * row, vp + s * row, kv_dtype, s, n, w.N * row,
                          w.H * w.N * row, out, lse), record)
            else:
                timed("accumulate",
                      lambda s=s, n=n: q8a.attn_accumulate_chunk(
                          st[0], qd, kp + s * row, vp + s * row, kv_dtype, s, n, w.N * row,
                          w.H * w.N * row, 1), record)
        if not fused or w.q_pos0 + w.M > w.N:
            timed("finalize", lambda: q8a.attn_finalize(st[0], out, lse), record)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    # clean timing of the step
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(False)
    t1.record()
    torch.cuda.synchronize()
    ms_clean = t0.elapsed_time(t1) / steps
    # the same steps with an event at every step boundary: median and minimum of the steps
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    bounds[0].record()
    for i in range(steps):
        step(False)
        bounds[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps))
    ms_median = float(np.median(per_step))
    ms_min = per_step[0]
    # timed region with per-launch events (the roofline numbers come from here)
    for key in ev:
        ev[key].clear()
    t0.record()
    for _ in range(steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms_events = t0.elapsed_time(t1) / steps
    kern = {}
    for key, pairs in ev.items():
        if pairs:
            d = [a.elapsed_time(b) for a, b in pairs]
            kern[key] = {"launches_per_step": len(d) // steps, "mean_us": 1e3 * float(np.mean(d))}
    acc_ms = [a.elapsed_time(b) for a, b in ev["accumulate"]]
    res = dict(q=q, out=out, lse=lse, ms_clean=ms_clean, ms_events=ms_events, kernels=kern,
               ms_median=ms_median, ms_min=ms_min,
               acc_mean_ms=float(np.mean(acc_ms)), acc_flops_mean=float(np.mean(acc_flops)),
               acc_per_chunk_us=[1e3 * float(np.mean(acc_ms[i::len(chunks)]))
                                 for i in range(len(chunks))],
               acc_flops=acc_flops, k=k, v=v, chunks=chunks, append=None)
    if not graph:
        return res
    # the same step captured once into a HIP graph and replayed: a secondary, labelled number
    # (fewer launch gaps); every replay must reproduce the eager output bit for bit
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(False)
    out.zero_()
    lse.zero_()
    graph.replay()
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse))
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / steps
    graph_equal = graph_equal and bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse))
    res["ms_graph"], res["graph_equal"] = ms_graph, graph_equal
    if (kv_dtype == q8a.KV_Q8_0 and w.q_pos0 > 0 and chunks[-1][0] == w.q_pos0 and w.B == 1):
        res["append"] = measure_append(w, qd, kx, vx, kd, vd, m, l, o, out, lse, chunks, steps)
    return res


def measure_append(w, qd, kx, vx, kd, vd, m, l, o, out, lse, chunks, steps):
    """Quantise-on-append for a workload whose last chunk is the queries' own new tokens
    (positions >= q_pos0): attn_append_chunk packs them from FP32 into their cache rows and
    accumulates them.  Timed: the step init + calls over the cached tokens + the append call +
    finalize; the append call alone on the resumed state (restored before every repetition);
    and, for comparison, the same work as two q8_0_pack launches into a staging buffer plus one
    attn_accumulate_chunk."""
    import numpy as np
    import torch

    import chunked_flashattention_q8_amd as q8a

    n_new = w.N - w.q_pos0
    kn = kx[:, :, w.q_pos0:].contiguous()
    vn = vx[:, :, w.q_pos0:].contiguous()
    kp = torch.empty((w.B, w.H, n_new, 68), dtype=torch.uint8, device=kx.device)
    vp = torch.empty_like(kp)
    hs, ss = w.N * 68, w.H * w.N * 68
    koff, voff = kd.data_ptr() + w.q_pos0 * 68, vd.data_ptr() + w.q_pos0 * 68

    def cached_part():
        st = q8a.attn_state_init(m, l, o, w.B, w.H, w.M, w.D, w.q_pos0)
        for s_, n_ in chunks[:-1]:
            q8a.attn_accumulate_chunk(st, qd, kd.data_ptr() + s_ * 68, vd.data_ptr() + s_ * 68,
                                      q8a.KV_Q8_0, s_, n_, hs, ss, 1)
        return st

    def fused(st):
        q8a.attn_append_chunk(st, qd, kn, vn, koff, voff, w.q_pos0, n_new, hs, ss, 1)

    def separate(st):
        q8a.q8_0_pack(kn, kp, w.B * w.H * n_new, 64)
        q8a.q8_0_pack(vn, vp, w.B * w.H * n_new, 64)
        q8a.attn_accumulate_chunk(st, qd, kp, vp, q8a.KV_Q8_0, w.q_pos0, n_new, n_new * 68,
                                  w.H * n_new * 68, 1)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the whole step with the append call
    for _ in range(2):
        fused(cached_part())
        q8a.attn_finalize(cached_part(), out, lse)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        st = cached_part()
        fused(st)
        q8a.attn_finalize(st, out, lse)
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / steps
    # the append call alone, from the resumed state of the cached part
    st = cached_part()
    torch.cuda.synchronize()
    m0, l0, o0 = m.clone(), l.clone(), o.clone()
    times = {}
    for name, fn in (("fused", fused), ("separate", separate)):
        d = []
        for _ in range(steps + 2):
            m.copy_(m0)
            l.copy_(l0)
            o.copy_(o0)
            ev0.record()
            fn(st)
            ev1.record()
            torch.cuda.synchronize()
            d.append(ev0.elapsed_time(ev1))
        times[name] = 1e3 * float(np.mean(d[2:]))
    return {"new_tokens": n_new, "ms_per_step_with_append": round(ms_step, 4),
            "append_call_us": round(times["fused"], 2),
            "pack_pack_accumulate_us": round(times["separate"], 2),
            "note": "step = init + %d calls over the cached tokens + attn_append_chunk of the "
                    "%d new tokens from FP32 + finalize; the call alone runs on the restored "
                    "resumed state; the comparison packs into a staging buffer (two launches) "
                    "and accumulates from it" % (len(chunks) - 1, n_new)}


def build_streamed_cache(w, layer=0, resident=True):
    """Q8_0 K and V of a streamed workload (one layer), drawn and packed chunk by chunk (the FP32
    cache never exists whole): the pinned host copy [C, 1, H, chunk, 68] and, if resident, a
    device-resident copy (else None)."""
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    H, C, chunk = w.H, w.n_chunks, w.chunk
    row = q8a.ROW_BYTES[q8a.KV_Q8_0]
    kh = torch.empty((C, 1, H, chunk, row), dtype=torch.uint8, pin_memory=True)
    vh = torch.empty(kh.shape, dtype=torch.uint8, pin_memory=True)
    shape = kh.shape if resident else (1,) + kh.shape[1:]
    kd = torch.empty(shape, dtype=torch.uint8, device=dev)
    vd = torch.empty_like(kd)
    for c in range(C):
        k, v = synthetic.gen_kv_chunk(w, c, layer)
        n = k.shape[1]
        i = c if resident else 0
        # packed dense ([H, n, 68]) and then placed at the chunk's head stride (chunk rows)
        for src, dst in ((k, kd), (v, vd)):
            dense = torch.empty((H, n, row), dtype=torch.uint8, device=dev)
            q8a.q8_0_pack(torch.from_numpy(src).to(dev), dense, H * n, w.D)
            dst[i, 0, :, :n].copy_(dense)
        kh[c].copy_(kd[i])
        vh[c].copy_(vd[i])
        if c % 16 == 15:
            print("layer %d: packed chunk %d of %d" % (layer, c + 1, C), file=sys.stderr,
                  flush=True)
    return (kd, vd, kh, vh) if resident else (None, None, kh, vh)


def run_burst(w, steps, warmup, n_split):
    """Mode B burst verification: 64 queries over the whole 1M-token cache, no causal mask.
    Resident: the key range is split into n_split consecutive ranges that one state holds as
    n_split "sequences" (the same queries repeated, the sequence stride stepping from one key
    range to the next), so every chunk call works on all ranges at once; the sequence blocks are
    then merged pairwise (attn_state_merge on sub-state descriptors, log2(n_split) launches) and
    sequence 0 is finalized.  Streamed: one state fed through two device slots from pinned host
    memory, as for the prefill workload."""
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    H, C, chunk, M = w.H, w.n_chunks, w.chunk, w.M
    if C % n_split or n_split & (n_split - 1):
        raise ValueError("n_split must be a power of two dividing the chunk count")
    per = C // n_split  # chunks per key range
    row = q8a.ROW_BYTES[q8a.KV_Q8_0]
    kd, vd, kh, vh = build_streamed_cache(w)
    qd = torch.from_numpy(synthetic.gen_q(w)).view(torch.float16).to(dev)
    qrep = qd.expand(n_split, H, M, w.D).contiguous()
    chunk_bytes = H * chunk * row
    m, l, o = q8a.alloc_state(n_split, H, M, dev)
    out = torch.empty((1, H, M, w.D), dtype=torch.float16, device=dev)
    lse = torch.empty((1, H, M), dtype=torch.float32, device=dev)
    slots_k = [torch.empty(chunk_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    slots_v = [torch.empty(chunk_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    main = torch.cuda.Stream()
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def split():
        st = q8a.attn_state_init(m, l, o, n_split, H, M, w.D, w.q_pos0, main)
        for c in range(per):  # chunk c of every key range r (global chunk r * per + c)
            q8a.attn_accumulate_chunk(st, qrep, kd[c].data_ptr(), vd[c].data_ptr(),
                                      q8a.KV_Q8_0, c * chunk, chunk, chunk * row,
                                      per * chunk_bytes, 0, main)
        n = n_split
        while n > 1:
            n //= 2
            q8a.attn_state_merge(q8a.sub_state(st, 0, n), q8a.sub_state(st, n, n), main)
        q8a.attn_finalize(q8a.sub_state(st, 0, 1), out, lse, main)

    def streamed():
        st = q8a.attn_state_init(m[:1], l[:1], o[:1], 1, H, M, w.D, w.q_pos0, main)
        q8a.attn_accumulate_stream(st, qd, kh, vh, q8a.KV_Q8_0, w.N, chunk, slots_k, slots_v, 0,
                                   main, copy_stream)
        q8a.attn_finalize(st, out, lse, main)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(main)
        for _ in range(steps):
            fn()
        b.record(main)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms_split = timed(split)
    out_split = out.clone()
    ms_stream = timed(streamed)
    d = (out.float() - out_split.float()).abs().max().item()
    return dict(ms_split=ms_split, ms_stream=ms_stream, kv_bytes=2 * C * chunk_bytes,
                split_vs_streamed_max_abs=d)


def burst_line(w, args):
    n_split = 16
    r = run_burst(w, args.steps, args.warmup, n_split)
    flops = w.visible_pairs() * 4 * w.D
    kv = r["kv_bytes"]
    line = {
        "metric": "Mode B burst verification TFLOP/s (64 queries x 1M Q8_0 keys, no causal mask)",
        "value": round(flops / (r["ms_split"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms_split"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "%s: B=1 H=%d M=%d N=%d d=64 non-causal, Q8_0 KV resident in HBM "
                               "split into %d key ranges held as the sequences of one state "
                               "(chunks of %d tokens), merged pairwise with attn_state_merge; "
                               "step = init + %d chunk calls + %d merges + finalize" % (
                                   w.name, w.H, w.M, w.N, n_split, w.chunk,
                                   w.n_chunks // n_split, n_split.bit_length() - 1)},
        "kv_gbps_resident": round(kv / (r["ms_split"] * 1e-3) / 1e9, 2),
        "fraction_of_mfma_peak": round(flops / (r["ms_split"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                                       4),
        "ms_streamed_one_state": round(r["ms_stream"], 4),
        "kv_gbps_streamed": round(kv / (r["ms_stream"] * 1e-3) / 1e9, 3),
        "split_vs_streamed_output_max_abs": r["split_vs_streamed_max_abs"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = sampled_cpu_baseline(w, rows_per_head=16)
    print(json.dumps(line), flush=True)


def run_streamed(w, steps, warmup, feed_dir=None):
    """The 1M-token workload: Q8_0 K and V in pinned host memory, chunk-major, streamed through
    two device slots per tensor by attn_accumulate_stream (copies on a side stream, compute on
    the current stream).  Also timed: the same chunk calls over a device-resident copy of the
    cache (compute only) and the host-to-device copies alone (copy only)."""
    import numpy as np
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    H, C, chunk = w.H, w.n_chunks, w.chunk
    row = q8a.ROW_BYTES[q8a.KV_Q8_0]
    kd, vd, kh, vh = build_streamed_cache(w)
    qd = torch.from_numpy(synthetic.gen_q(w)).view(torch.float16).to(dev)
    m, l, o = q8a.alloc_state(1, H, w.M, dev)
    out = torch.empty((1, H, w.M, w.D), dtype=torch.float16, device=dev)
    lse = torch.empty((1, H, w.M), dtype=torch.float32, device=dev)
    chunk_bytes = H * chunk * row
    slots_k = [torch.empty(chunk_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    slots_v = [torch.empty(chunk_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    # both streams are created here (not the legacy default stream, which would serialise
    # with the copy stream); every step runs on `cur`
    copy_stream = torch.cuda.Stream()
    cur = torch.cuda.Stream()
    torch.cuda.synchronize()

    def streamed():
        st = q8a.attn_state_init(m, l, o, 1, H, w.M, w.D, w.q_pos0, cur)
        q8a.attn_accumulate_stream(st, qd, kh, vh, q8a.KV_Q8_0, w.N, chunk, slots_k, slots_v, 1,
                                   cur, copy_stream)
        q8a.attn_finalize(st, out, lse, cur)

    def resident():
        st = q8a.attn_state_init(m, l, o, 1, H, w.M, w.D, w.q_pos0, cur)
        for c, (s, n) in enumerate(w.chunks()):
            q8a.attn_accumulate_chunk(st, qd, kd[c].data_ptr(), vd[c].data_ptr(), q8a.KV_Q8_0,
                                      s, n, chunk * row, H * chunk * row, 1, cur)
        q8a.attn_finalize(st, out, lse, cur)

    def copies():
        with torch.cuda.stream(cur):
            for c in range(C):
                slots_k[c & 1].copy_(kh[c].view(-1), non_blocking=True)
                slots_v[c & 1].copy_(vh[c].view(-1), non_blocking=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cur)
        for _ in range(steps):
            fn()
        b.record(cur)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms_stream = timed(streamed)
    out_stream = out.clone()
    ms_resident = timed(resident)
    same = bool(torch.equal(out_stream, out))
    ms_copy = timed(copies)
    feed = None
    if feed_dir:
        feed = file_feed(w, feed_dir, qd, kh, vh, m, l, o, out, out_stream, slots_k, slots_v,
                         chunk_bytes, cur, copy_stream)
    return dict(ms_stream=ms_stream, ms_resident=ms_resident, ms_copy=ms_copy,
                streamed_equals_resident=same, kv_bytes=2 * C * chunk_bytes, file_feed=feed)


def file_feed(w, feed_dir, qd, kh, vh, m, l, o, out, out_stream, slots_k, slots_v, chunk_bytes,
              cur, copy_stream, steps=3):
    """The same workload fed from storage: the chunk-major K and V written to two files (then
    dropped from the page cache), read back with O_DIRECT by attn_accumulate_file into a pinned
    two-slot ring.  Timed on the host clock (the call blocks until every chunk is read).  Also
    the raw O_DIRECT read rate of the two files into the ring, without the GPU."""
    import time

    import torch

    import chunked_flashattention_q8_amd as q8a

    H, chunk = w.H, w.chunk
    paths = [os.path.join(feed_dir, "q8a_feed_%d_%s.bin" % (os.getpid(), t)) for t in "kv"]
    ring_bytes = chunk_bytes + 8192
    # direct reads cannot land in pinned memory: the ring is anonymous mmap memory
    ring_k, ring_v = q8a.alloc_ring(ring_bytes), q8a.alloc_ring(ring_bytes)
    try:
        for pth, src in zip(paths, (kh, vh)):
            with open(pth, "wb") as f:
                src.numpy().reshape(-1).tofile(f)
                f.flush()
                os.fsync(f.fileno())
            fd = os.open(pth, os.O_RDONLY)
            os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
            os.close(fd)
        fds = [os.open(pth, os.O_RDONLY | os.O_DIRECT) for pth in paths]
        try:
            # raw read rate: the files into the ring, chunk by chunk, no GPU
            t0 = time.perf_counter()
            for c in range(w.n_chunks):
                for fd, ring in zip(fds, (ring_k, ring_v)):
                    view = memoryview(ring[c & 1])[:chunk_bytes]
                    got = os.preadv(fd, [view], c * chunk_bytes)
                    assert got == chunk_bytes
            t_raw = time.perf_counter() - t0
            res = []
            for i in range(steps + 1):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                st = q8a.attn_state_init(m, l, o, 1, H, w.M, w.D, w.q_pos0, cur)
                q8a.attn_accumulate_file(st, qd, fds[0], fds[1], 0, q8a.KV_Q8_0, w.N, chunk,
                                         ring_k, ring_v, ring_bytes, slots_k, slots_v, 1, cur,
                                         copy_stream)
                q8a.attn_finalize(st, out, None, cur)
                torch.cuda.synchronize()
                if i:
                    res.append(time.perf_counter() - t0)
            same = bool(torch.equal(out, out_stream))
        finally:
            for fd in fds:
                os.close(fd)
    finally:
        for pth in paths:
            if os.path.exists(pth):
                os.unlink(pth)
    kv = 2 * w.n_chunks * chunk_bytes
    ms = 1e3 * sum(res) / len(res)
    return {"ms_per_step": round(ms, 2), "kv_gbps": round(kv / (ms * 1e-3) / 1e9, 3),
            "storage_read_gbps_odirect": round(kv / t_raw / 1e9, 3),
            "equals_streamed": same, "steps": steps,
            "note": "step = init + attn_accumulate_file + finalize, host clock; files in %s "
                    "opened with O_DIRECT, read with pread into a two-slot ring of mmap'd memory; "
                    "storage_read_gbps: the same reads without the GPU" % feed_dir}


def streamed_line(w, args):
    r = run_streamed(w, args.steps, args.warmup, args.feed_dir)
    flops = w.visible_pairs() * 4 * w.D
    kv = r["kv_bytes"]
    line = {
        "metric": "streamed KV GB/s (Q8_0 K+V from pinned host memory, double-buffered)",
        "value": round(kv / (r["ms_stream"] * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms_stream"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "%s: B=1 H=%d M=%d N=%d d=64 causal q_pos0=%d, Q8_0 KV streamed "
                               "in %d chunks of %d tokens through 2 device slots; step = init + "
                               "attn_accumulate_stream + finalize" % (
                                   w.name, w.H, w.M, w.N, w.q_pos0, w.n_chunks, w.chunk)},
        "kv_bytes_per_step": kv,
        "attention_tflops_streamed": round(flops / (r["ms_stream"] * 1e-3) / 1e12, 3),
        "ms_compute_only_resident": round(r["ms_resident"], 4),
        "attention_tflops_resident": round(flops / (r["ms_resident"] * 1e-3) / 1e12, 3),
        "ms_copy_only": round(r["ms_copy"], 4),
        "h2d_gbps_copy_only": round(kv / (r["ms_copy"] * 1e-3) / 1e9, 3),
        "overlap_efficiency": round(max(r["ms_copy"], r["ms_resident"]) / r["ms_stream"], 4),
        "streamed_equals_resident": r["streamed_equals_resident"],
        "file_feed": r["file_feed"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        base = sampled_cpu_baseline(w)
        base["extrapolated_kv_gbps"] = round(kv / base["extrapolated_full_step_s"] / 1e9, 4)
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)


def build_device_cache(w, layer):
    """Q8_0 K and V of one layer of a layered workload, packed chunk by chunk into device memory,
    chunk-major [C, 1, H, chunk, 68] (the FP32 cache never exists whole)."""
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    H, C, chunk = w.H, w.n_chunks, w.chunk
    row = q8a.ROW_BYTES[q8a.KV_Q8_0]
    kd = torch.empty((C, 1, H, chunk, row), dtype=torch.uint8, device=dev)
    vd = torch.empty_like(kd)
    for c in range(C):
        k, v = synthetic.gen_kv_chunk(w, c, layer)
        n = k.shape[1]
        for src, dst in ((k, kd), (v, vd)):
            dense = torch.empty((H, n, row), dtype=torch.uint8, device=dev)
            q8a.q8_0_pack(torch.from_numpy(src).to(dev), dense, H * n, w.D)
            dst[c, 0, :, :n].copy_(dense)
    print("layer %d packed" % layer, file=sys.stderr, flush=True)
    return kd, vd


def run_layers(w, steps, warmup):
    """The layered workload with every layer's cache resident in HBM (16 x 4.56 GB of Q8_0 K and
    V at 1M tokens fit in the 288 GB of one MI355X): each layer has its own Q, cache, state and
    output; a step runs every layer in turn: init + its chunk calls (ascending, each writing
    the final out/lse of the rows it completes; the queries sit at the end of the cache, so the
    last call completes them all)."""
    import torch

    import chunked_flashattention_q8_amd as q8a
    import synthetic

    dev = torch.device("cuda:0")
    H, chunk, L = w.H, w.chunk, w.layers
    row = q8a.ROW_BYTES[q8a.KV_Q8_0]
    if w.q_pos0 + w.M != w.N:
        raise ValueError("the layered step expects the queries at the end of the cache")
    caches = [build_device_cache(w, layer) for layer in range(L)]
    qs = [torch.from_numpy(synthetic.gen_q(w, layer)).view(torch.float16).to(dev)
          for layer in range(L)]
    states = [q8a.alloc_state(1, H, w.M, dev) for _ in range(L)]
    outs = [torch.empty((1, H, w.M, w.D), dtype=torch.float16, device=dev) for _ in range(L)]
    lses = [torch.empty((1, H, w.M), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    def step():
        for layer in range(L):
            m, l, o = states[layer]
            kd, vd = caches[layer]
            st = q8a.attn_state_init(m, l, o, 1, H, w.M, w.D, w.q_pos0)
            for c, (s0, n) in enumerate(w.chunks()):
                q8a.attn_accumulate_chunk_final(st, qs[layer], kd[c].data_ptr(),
                                                vd[c].data_ptr(), q8a.KV_Q8_0, s0, n,
                                                chunk * row, H * chunk * row, outs[layer],
                                                lses[layer])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    return dict(ms_step=a.elapsed_time(b) / steps, kv_bytes=L * 2 * w.N * H * row,
                outs=outs, lses=lses)

def layers_parity(w, res, layers):
    """Oracle check of the layered workload: the sampled rows of the given layers, the oracle
    fed from its own pack of the same draws."""
    import numpy as np

    import oracle
    import synthetic

    threads = oracle.default_threads()
    rows = synthetic.sample_rows(w)
    err = []
    t0 = time.perf_counter()
    for layer in layers:
        kb = np.empty((1, w.H, w.N, 68), dtype=np.uint8)
        vb = np.empty_like(kb)
        for c, (s0, n) in enumerate(w.chunks()):
            k, v = synthetic.gen_kv_chunk(w, c, layer)
            kb[0, :, s0:s0 + n] = oracle.q8_0_pack(k, threads)
            vb[0, :, s0:s0 + n] = oracle.q8_0_pack(v, threads)
        prob = oracle.Problem(synthetic.gen_q(w, layer), kb, vb, oracle.KV_Q8_0, w.q_pos0)
        O_ref, lse_ref = oracle.attention(prob, rows, nthreads=threads)
        out = res["outs"][layer].float().cpu().numpy().reshape(-1, w.D)[rows]
        lse = res["lses"][layer].cpu().numpy().reshape(-1)[rows]
        err.append((out.astype(np.float64) - O_ref, O_ref, lse.astype(np.float64) - lse_ref,
                    lse_ref))
        del kb, vb
    d = np.concatenate([e[0].ravel() for e in err])
    r = np.concatenate([e[1].ravel() for e in err])
    dl = np.concatenate([e[2] for e in err])
    rl = np.concatenate([e[3] for e in err])
    parity = {"layers_checked": list(layers), "rows_per_layer": int(rows.size),
              "max_abs": float(np.abs(d).max()),
              "rel_rms": float(np.sqrt((d ** 2).sum() / (r ** 2).sum())),
              "lse_rel": float((np.abs(dl) / np.maximum(1, np.abs(rl))).max()),
              "seconds": round(time.perf_counter() - t0, 1)}
    parity["ok"] = parity["max_abs"] <= 2e-3 and parity["rel_rms"] <= 1e-3 and \
        parity["lse_rel"] <= 1e-4
    return parity


def layers_line(w, args):
    r = run_layers(w, args.steps, args.warmup)
    flops = w.layers * w.visible_pairs() * 4 * w.D
    kv = r["kv_bytes"]
    value = flops / (r["ms_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "%s: %d layers, each B=1 H=%d M=%d N=%d d=64 causal q_pos0=%d "
                               "with its own Q, Q8_0 K/V cache (all %d resident in HBM, %.1f GB) "
                               "and state; step = per layer init + %d chunk calls of %d tokens, "
                               "each writing the final out/lse of the rows it completes" % (
                                   w.name, w.layers, w.H, w.M, w.N, w.q_pos0, w.layers, kv / 1e9,
                                   w.n_chunks, w.chunk)},
        "step_fraction_of_mfma_peak": round(value / PEAK_F16_TFLOPS, 4),
        "kv_bytes_per_step": kv,
        "kv_gbps_from_hbm": round(kv / (r["ms_step"] * 1e-3) / 1e9, 3),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["parity_vs_oracle"] = layers_parity(w, r, [0, w.layers - 1])
        line["cpu_baseline"] = sampled_cpu_baseline(w, rows_per_head=32)
    print(json.dumps(line), flush=True)

def secondary_points(main_w, main_res, steps, warmup):
    """The other resident points of the graded shape, each timed like the main step (labelled
    secondary numbers, not the line's value): the same step with plain chunk calls and a
    separate finalize launch, the single-sequence M=2048 prefill, the same 8 sequences with FP16
    KV (the same draws rounded to FP16, which isolates the dequantisation cost) and with the
    whole KV sequence in one chunk call (B_C = 2048, no state round trips)."""
    import chunked_flashattention_q8_amd as q8a
    import synthetic

    out = {}
    same = (main_res["q"], main_res["k"], main_res["v"])
    points = [("batch8_m2048_q8_0_bc512_init_launch", main_w, q8a.KV_Q8_0, 512, same, "fused"),
              ("batch8_m2048_q8_0_bc512_finalize_launch", main_w, q8a.KV_Q8_0, 512, same,
               "plain"),
              ("incore_m2048_q8_0_bc512", synthetic.WORKLOADS[1], q8a.KV_Q8_0, 512, None, "lean"),
              ("batch8_m2048_f16kv_bc512", main_w, q8a.KV_F16, 512, same, "lean"),
              ("batch8_m2048_q8_0_bc2048", main_w, q8a.KV_Q8_0, 2048, same, "lean")]
    for name, w, kv, chunk, inputs, form in points:
        r = run_resident(w, kv, chunk, steps, warmup, inputs=inputs, graph=False, form=form)
        flops = w.visible_pairs() * 4 * w.D
        acc = r["acc_flops_mean"] / (r["acc_mean_ms"] * 1e-3) / 1e12
        out[name] = {
            "ms_per_step": round(r["ms_clean"], 5),
            "value": round(flops / (r["ms_clean"] * 1e-3) / 1e12, 3),
            "step_fraction_of_mfma_peak": round(flops / (r["ms_clean"] * 1e-3) / 1e12 /
                                                PEAK_F16_TFLOPS, 4),
            "accumulate_mean_launch_us": round(1e3 * r["acc_mean_ms"], 3),
            "accumulate_frac": round(acc / PEAK_F16_TFLOPS, 4),
            "chunk_calls": len(r["chunks"]),
            "ms_per_step_median": round(r["ms_median"], 5),
            "step": ("pack of K and V (one call) + " if kv == q8a.KV_Q8_0 else
                     "(FP16 KV: no pack) ") + STEP_FORMS[form],
        }
    return out


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_rate(w, q, k, v, kv_dtype, head=0):
    """The oracle on one thread: pack of one head's K and V and FP64 attention over all its rows,
    in TFLOP/s of attention (the pack time included), and the seconds it took."""
    import numpy as np

    import oracle
    import synthetic

    b, h = divmod(head, w.H)
    pos = w.q_pos0 + np.arange(w.M, dtype=np.int64)
    flops = int(np.minimum(pos + 1, w.N).sum()) * 4 * w.D
    t0 = time.perf_counter()
    qh = np.ascontiguousarray(q[b:b + 1, h:h + 1])
    if kv_dtype == 0:
        prob = oracle.Problem(qh, oracle.q8_0_pack(k[b:b + 1, h:h + 1], 1),
                              oracle.q8_0_pack(v[b:b + 1, h:h + 1], 1), oracle.KV_Q8_0, w.q_pos0)
    else:
        prob = oracle.Problem(qh, synthetic.to_f16_bits(k[b:b + 1, h:h + 1]),
                              synthetic.to_f16_bits(v[b:b + 1, h:h + 1]), oracle.KV_F16, w.q_pos0)
    oracle.attention(prob, nthreads=1)
    dt = time.perf_counter() - t0
    return flops / dt / 1e12, dt


def cpu_baseline(w, res, kv_dtype, budget_s):
    """The oracle on whole heads (b, h) in order until ~budget_s of wall time has passed, on
    every host thread; then one head on one thread."""
    import numpy as np

    import oracle
    import synthetic

    threads = oracle.default_threads()
    q, k, v = res["q"], res["k"], res["v"]
    out = res["out"].float().cpu().numpy().reshape(w.B * w.H, w.M, w.D)
    lse = res["lse"].cpu().numpy().reshape(w.B * w.H, w.M)
    pos = w.q_pos0 + np.arange(w.M, dtype=np.int64)
    head_flops = int(np.minimum(pos + 1, w.N).sum()) * 4 * w.D
    done = 0
    err = []
    t0 = time.perf_counter()
    while done < w.B * w.H:
        b, h = divmod(done, w.H)
        qh = np.ascontiguousarray(q[b:b + 1, h:h + 1])
        if kv_dtype == 0:
            kb = oracle.q8_0_pack(k[b:b + 1, h:h + 1], threads)
            vb = oracle.q8_0_pack(v[b:b + 1, h:h + 1], threads)
            prob = oracle.Problem(qh, kb, vb, oracle.KV_Q8_0, w.q_pos0)
        else:
            kb = synthetic.to_f16_bits(k[b:b + 1, h:h + 1])
            vb = synthetic.to_f16_bits(v[b:b + 1, h:h + 1])
            prob = oracle.Problem(qh, kb, vb, oracle.KV_F16, w.q_pos0)
        O_ref, lse_ref = oracle.attention(prob, nthreads=threads)
        err.append((out[done].astype(np.float64) - O_ref, O_ref,
                    lse[done].astype(np.float64) - lse_ref, lse_ref))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    d = np.concatenate([e[0].ravel() for e in err])
    r = np.concatenate([e[1].ravel() for e in err])
    dl = np.concatenate([e[2] for e in err])
    rl = np.concatenate([e[3] for e in err])
    parity = {"heads_checked": done, "max_abs": float(np.abs(d).max()),
              "rel_rms": float(np.sqrt((d ** 2).sum() / (r ** 2).sum())),
              "lse_rel": float((np.abs(dl) / np.maximum(1, np.abs(rl))).max())}
    parity["ok"] = parity["max_abs"] <= 2e-3 and parity["rel_rms"] <= 1e-3 and \
        parity["lse_rel"] <= 1e-4
    st_rate, st_s = single_thread_rate(w, q, k, v, kv_dtype)
    pack = None
    if kv_dtype == 0:  # the oracle's Q8_0 pack of the whole K and V, on the same threads
        t1 = time.perf_counter()
        kb_all = oracle.q8_0_pack(k, threads)
        vb_all = oracle.q8_0_pack(v, threads)
        dp = time.perf_counter() - t1
        moved = k.nbytes + v.nbytes + kb_all.nbytes + vb_all.nbytes
        pack = {"gbps": round(moved / dp / 1e9, 3), "seconds": round(dp, 3), "threads": threads,
                "bytes": int(moved), "note": "FP32 K and V read, Q8_0 bytes written"}
        del kb_all, vb_all
    base = {"value": head_flops * done / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d (sequence, head) pairs in full (Q8_0 pack of their K and V + "
                      "FP64 single-pass causal attention over all %d rows), %.1f s" % (
                          done, w.B * w.H, w.M, dt),
            "cpu_model": cpu_model(),
            "single_thread": {"value": st_rate, "unit": "TFLOP/s", "seconds": round(st_s, 2),
                              "sample": "(sequence 0, head 0) in full on one thread"},
            "pack": pack}
    return base, parity


def sampled_cpu_baseline(w, layer=0, heads=(0,), rows_per_head=None):
    """The oracle on sampled rows of a 1M-token workload: for each sampled head, its K and V are
    drawn (the same draws, chunk by chunk) and packed by the oracle, then FP64 attention of the
    head's sampled rows over every visible key, on every host thread; one of those rows is
    timed again on one thread.  Reported in TFLOP/s of attention over the sampled rows (the pack
    of the head's cache is timed separately), with the full step's time extrapolated from both
    rates and labelled as such."""
    import numpy as np

    import oracle
    import synthetic

    threads = oracle.default_threads()
    rows_all = synthetic.sample_rows(w, rows_per_head)
    q = synthetic.gen_q(w, layer)
    t_pack = t_attn = 0.0
    flops = 0
    n_rows = 0
    st = None
    for h in heads:
        t0 = time.perf_counter()
        kb = np.empty((1, 1, w.N, 68), dtype=np.uint8)
        vb = np.empty_like(kb)
        for c, (s0, n) in enumerate(w.chunks()):
            k, v = synthetic.gen_kv_chunk_head(w, c, h, layer)
            kb[0, 0, s0:s0 + n] = oracle.q8_0_pack(k, threads)
            vb[0, 0, s0:s0 + n] = oracle.q8_0_pack(v, threads)
        t_pack += time.perf_counter() - t0
        rows = rows_all[(rows_all >= h * w.M) & (rows_all < (h + 1) * w.M)] - h * w.M
        prob = oracle.Problem(np.ascontiguousarray(q[:, h:h + 1]), kb, vb, oracle.KV_Q8_0,
                              w.q_pos0)
        prob.causal = w.causal
        pos = w.q_pos0 + rows
        vis = np.minimum(pos + 1, w.N) if w.causal else np.full(rows.size, w.N)
        t0 = time.perf_counter()
        oracle.attention(prob, rows, nthreads=threads)
        t_attn += time.perf_counter() - t0
        flops += int(vis.sum()) * 4 * w.D
        n_rows += rows.size
        if st is None:
            t0 = time.perf_counter()
            oracle.attention(prob, rows[:1], nthreads=1)
            st = (int(vis[0]) * 4 * w.D, time.perf_counter() - t0)
        del kb, vb
    full_flops = w.layers * w.visible_pairs() * 4 * w.D
    rate = flops / t_attn
    extrap_s = full_flops / rate + t_pack / len(heads) * w.H * w.layers
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d sampled query rows of head(s) %s%s over all their visible keys (FP64 "
                      "attention, %.1f s), after the oracle's pack of those heads' K and V "
                      "(%.1f s)" % (n_rows, list(heads),
                                    " of layer %d" % layer if w.layers > 1 else "", t_attn,
                                    t_pack),
            "cpu_model": cpu_model(),
            "single_thread": {"value": st[0] / st[1] / 1e12, "unit": "TFLOP/s",
                              "seconds": round(st[1], 2), "sample": "one of those rows"},
            "extrapolated_full_step_s": round(extrap_s, 1),
            "extrapolation": "full step = all heads' attention at the sampled rate + every "
                             "head's pack at the sampled pack time"}


def read_summary(path):
    """'key: value' lines of a profiles/ summary ('#' lines are comments)."""
    out = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def traffic_per_launch():
    """HBM bytes per accumulate launch from the committed counter summary, or None when there
    is none or the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = read_summary(TRAFFIC_FILE)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(t["hbm_bytes_per_launch"])


def algorithmic_bytes(w, chunk, form="lean"):
    """Algorithmic HBM bytes of each chunk call (chunks in ascending order; STEP_FORMS): the
    chunk's K and V rows (136 B per key per head); for each query row that sees the chunk its Q
    row (128 B), its state read (m, 4 B, except in the lean form's first call, whose deferred
    state is not read; l and O, 260 B, for rows that are not empty) and written (m, l, O:
    264 B); lean and fused, the final output of the rows whose position lies in the chunk (out
    128 B, lse 4 B), and lean writes no state for those rows."""
    import numpy as np
    pos = w.q_pos0 + np.arange(w.M, dtype=np.int64)
    out = []
    for s in range(0, w.N, chunk):
        n = min(chunk, w.N - s)
        touched = int((pos >= s).sum())
        nonempty = touched if s > 0 else 0  # every row sees key 0 first
        final = int(((pos >= s) & (pos < s + n)).sum()) if form != "plain" else 0
        m_read = 0 if (form == "lean" and s == 0) else 4
        state_written = touched - (final if form == "lean" else 0)
        per_head = (n * 136 + touched * (128 + m_read) + nonempty * 260 + state_written * 264 +
                    final * 132)
        out.append(per_head * w.B * w.H)
    return out


def counter_means(d, counter, name_part):
    """Mean over the dispatches whose kernel name contains name_part of the summed counter."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("no %s samples for kernels named *%s* under %s" % (counter, name_part, d))
    return sum(per.values()) / len(per), len(per)


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_mib, commands):
    """Write the HBM traffic summary of the accumulate kernel from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the default workload, and of a plain copy
    of cal_mib MiB, which scales each counter to bytes."""
    import synthetic
    w = synthetic.WORKLOADS[2]
    fetch, n_f = counter_means(fetch_dir, "FETCH_SIZE", "accumulate_kernel<0, 0, true>")
    write, n_w = counter_means(write_dir, "WRITE_SIZE", "accumulate_kernel<0, 0, true>")
    cf, _ = counter_means(cal_fetch_dir, "FETCH_SIZE", "copy")
    cw, _ = counter_means(cal_write_dir, "WRITE_SIZE", "copy")
    copy_bytes = cal_mib * (1 << 20)
    f_fac, w_fac = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    hbm = fetch * 1024 * f_fac + write * 1024 * w_fac
    alg = algorithmic_bytes(w, w.chunk)
    lines = [
        "# HBM traffic of accumulate_kernel<0, 0, true> (Q8_0 KV, the 256-row prefill form) per launch, batch8_m2048 workload:",
        "# 8 sequences x 32 heads, M = N = 2048 causal, d = 64, B_C = 512 (4 launches per step,",
        "# each also writing out and lse of the rows whose position lies in its chunk).",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch, averaged over the accumulate dispatches;",
        "# each is scaled by (bytes copied) / (counter x 1024) of a plain device copy of",
        "# %d MiB (torch copy kernel), measured the same way." % cal_mib,
        "# commands (repository root on an MI355X):",
    ] + ["#   " + c for c in commands] + [
        "#   python bench.py --traffic-summary <the four -d folders above> %d" % cal_mib,
        "kernel_source_sha256: %s" % kernel_source_hash(),
        "dispatches_fetch: %d" % n_f,
        "dispatches_write: %d" % n_w,
        "fetch_kib_per_launch: %.1f" % fetch,
        "write_kib_per_launch: %.1f" % write,
        "copy_fetch_factor: %.4f" % f_fac,
        "copy_write_factor: %.4f" % w_fac,
        "hbm_bytes_per_launch: %.0f" % hbm,
        "algorithmic_bytes_per_launch: %.0f" % (sum(alg) / len(alg)),
        "algorithmic_bytes_per_chunk_call: %s" % " ".join(str(a) for a in alg),
        "traffic_over_algorithmic: %.3f" % (hbm / (sum(alg) / len(alg))),
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the first ~50 steps of a process run slower)")
    ap.add_argument("--workload", type=int, default=2,
                    help="0-3: resident workloads; 4: the streamed 1M-token workload; "
                         "5: Mode B burst verification over the 1M-token cache; 6: the "
                         "1M-token workload for each of 16 layers")
    ap.add_argument("--chunk", type=int, default=None, help="override B_C")
    ap.add_argument("--feed-dir", default=None,
                    help="workload 4: also feed the cache from files in this directory "
                         "(attn_accumulate_file, O_DIRECT)")
    ap.add_argument("--kv", choices=["q8_0", "f16"], default="q8_0")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary points of the default line (single sequence, "
                         "FP16 KV, B_C = 2048)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--traffic-summary", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "MIB"),
                    help="write the accumulate kernel's HBM traffic summary from rocprofv3 runs")
    args = ap.parse_args()
    if args.traffic_summary:
        fd, wd, cfd, cwd, mib = args.traffic_summary
        cmds = ["rocprofv3 --pmc FETCH_SIZE -d %s -o f --output-format csv -- "
                "python bench.py --no-cpu-baseline --no-secondary --steps 3 --warmup 1" % fd,
                "rocprofv3 --pmc WRITE_SIZE -d %s -o w --output-format csv -- "
                "python bench.py --no-cpu-baseline --no-secondary --steps 3 --warmup 1" % wd,
                "rocprofv3 --pmc FETCH_SIZE -d %s -o cf --output-format csv -- "
                "python bench.py --copy-calibration %s" % (cfd, mib),
                "rocprofv3 --pmc WRITE_SIZE -d %s -o cw --output-format csv -- "
                "python bench.py --copy-calibration %s" % (cwd, mib)]
        traffic_summary(fd, wd, cfd, cwd, int(mib), cmds)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path is single-GPU by design (no collectives "
              "or sharding are built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import synthetic
    import chunked_flashattention_q8_amd as q8a

    w = synthetic.WORKLOADS[args.workload]
    if w.layers > 1:
        layers_line(w, args)
        return
    if w.streamed and not w.causal:
        burst_line(w, args)
        return
    if w.streamed:
        streamed_line(w, args)
        return
    kv_dtype = q8a.KV_Q8_0 if args.kv == "q8_0" else q8a.KV_F16
    chunk = args.chunk or w.chunk
    res = run_resident(w, kv_dtype, chunk, args.steps, args.warmup)

    flops_step = w.visible_pairs() * 4 * w.D
    ms = res["ms_clean"]  # the step without per-launch events; those only feed the roofline
    value = flops_step / (ms * 1e-3) / 1e12
    acc_achieved = res["acc_flops_mean"] / (res["acc_mean_ms"] * 1e-3) / 1e12
    kv_bytes = 2 * w.B * w.H * w.N * q8a.ROW_BYTES[kv_dtype]
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "%s: B=%d H=%d M=%d N=%d d=64 causal q_pos0=%d, %s KV, B_C=%d "
                        "(%d chunk calls); step = %s%s"
                        % (w.name, w.B, w.H, w.M, w.N, w.q_pos0, args.kv.upper(), chunk,
                           len(res["chunks"]),
                           "pack of K and V (one call) + " if kv_dtype == q8a.KV_Q8_0 else "",
                           STEP_FORMS["lean"]),
            "kv_dtype": args.kv, "chunk_tokens": chunk,
        },
        "roofline": {
            "kernel": "accumulate_kernel",
            "bound": "mfma",
            "achieved": round(acc_achieved, 3),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(acc_achieved / PEAK_F16_TFLOPS, 4),
            "traffic": traffic_per_launch() if (args.workload == 2 and chunk == 512 and
                                                kv_dtype == q8a.KV_Q8_0) else None,
            "flops_per_launch": res["acc_flops_mean"],
            "mean_launch_us": round(1e3 * res["acc_mean_ms"], 3),
        },
        "step_fraction_of_mfma_peak": round(value / PEAK_F16_TFLOPS, 4),
        "kv_gbps": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "ms_per_step_median": round(res["ms_median"], 5),
        "ms_per_step_min": round(res["ms_min"], 5),
        "ms_per_step_with_kernel_events": round(res["ms_events"], 5),
        "hip_graph": {"ms_per_step": round(res["ms_graph"], 5),
                      "value": round(flops_step / (res["ms_graph"] * 1e-3) / 1e12, 3),
                      "output_equals_eager": res["graph_equal"],
                      "note": "the same step captured once with torch.cuda.graph and replayed"},
        "kernels": res["kernels"],
        "accumulate_us_per_chunk": [round(x, 3) for x in res["acc_per_chunk_us"]],
    }
    if res["append"]:
        line["append"] = res["append"]
    if args.workload == 2 and args.chunk is None and args.kv == "q8_0" and not args.no_secondary:
        line["secondary"] = secondary_points(w, res, min(args.steps, 20), min(args.warmup, 3))
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, res, kv_dtype, args.cpu_seconds)
        line["cpu_baseline"] = base
        line["parity_vs_oracle"] = parity
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
